"""C ABI checks that need no GPU: exports, struct layout, host-side validation.

On a machine without a GPU every call that passes validation stops at the
device check with MFA_E_NO_DEVICE; nothing is launched.
"""

import ctypes as C
import os
import re
import subprocess

import pytest

from masked_flash_attention_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_ffi.LIB_PATH):
        from masked_flash_attention_amd import build
        build.build(verbose=False)
    return _ffi.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mfa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", _ffi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mfa_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(_ffi.SIGNATURES), "binding signatures and header disagree"


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.cpp"
    src.write_text(r'''
#include <cstdio>
#include <cstddef>
#include "mfa.h"
#define P(s, f) printf(#s "." #f " %zu\n", offsetof(s, f))
int main() {
  printf("mfa_attn_args %zu\nmfa_mask %zu\nmfa_attn_bwd_args %zu\n",
         sizeof(mfa_attn_args), sizeof(mfa_mask), sizeof(mfa_attn_bwd_args));
  P(mfa_attn_args, q); P(mfa_attn_args, lse); P(mfa_attn_args, o_stride); P(mfa_attn_args, alibi_slopes);
  P(mfa_attn_args, softcap);
  P(mfa_mask, tile_kind); P(mfa_mask, q_block); P(mfa_mask, cu_q); P(mfa_mask, err); P(mfa_mask, win_right); P(mfa_mask, nseq); P(mfa_mask, seqused_k); P(mfa_mask, n_pages);
  P(mfa_attn_bwd_args, dout); P(mfa_attn_bwd_args, dv_stride); P(mfa_attn_bwd_args, workspace);
  P(mfa_attn_bwd_args, workspace_bytes);
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.run(["g++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True,
                                                               text=True).stdout.split("\n") if line)
    got = {k: int(v) for k, v in got.items()}
    assert got["mfa_attn_args"] == C.sizeof(_ffi.AttnArgs)
    assert got["mfa_mask"] == C.sizeof(_ffi.Mask)
    assert got["mfa_attn_bwd_args"] == C.sizeof(_ffi.BwdArgs)
    for cls, cname in ((_ffi.AttnArgs, "mfa_attn_args"), (_ffi.Mask, "mfa_mask"), (_ffi.BwdArgs, "mfa_attn_bwd_args")):
        for key, off in got.items():
            if key.startswith(cname + "."):
                assert getattr(cls, key.split(".", 1)[1]).offset == off, key


def _args(**kw):
    a = _ffi.AttnArgs()
    a.dtype, a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.D = 0, 1, 128, 128, 4, 2, 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _status(lib, code):
    return lib.mfa_status_name(code).decode()


@pytest.mark.parametrize("kw,want", [
    (dict(Hq=3, Hkv=2), "MFA_E_SHAPE"),
    (dict(Hkv=0), "MFA_E_SHAPE"),
    (dict(Sq=-1), "MFA_E_SHAPE"),
    (dict(D=96), "MFA_E_UNSUPPORTED"),
    (dict(softcap=-1.0), "MFA_E_ARG"),
    (dict(softcap=float("nan")), "MFA_E_ARG"),
    (dict(softcap=float("inf")), "MFA_E_ARG"),
    (dict(dtype=7), "MFA_E_DTYPE"),
])
def test_attn_fwd_rejects_before_any_device_call(lib, kw, want):
    m = _ffi.Mask()
    s = lib.mfa_attn_fwd(C.byref(_args(**kw)), C.byref(m), 0.125, None)
    assert _status(lib, s) == want
    assert lib.mfa_last_error().decode()


@pytest.mark.parametrize("scale", [0.0, -0.125, float("nan"), float("inf")])
def test_scale_must_be_finite_and_positive(lib, scale):
    m = _ffi.Mask()
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args()), C.byref(m), scale, None)) == "MFA_E_ARG"
    assert "scale" in lib.mfa_last_error().decode()


def test_attn_fwd_null_and_mask_errors(lib):
    assert _status(lib, lib.mfa_attn_fwd(None, None, 0.1, None)) == "MFA_E_ARG"
    m = _ffi.Mask()
    m.kind = 9
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args()), C.byref(m), 0.1, None)) == "MFA_E_ARG"
    m = _ffi.Mask()
    m.kind, m.q_block, m.kv_block = _ffi.MASK_BSR, 32, 64
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args()), C.byref(m), 0.1, None)) == "MFA_E_UNSUPPORTED"
    m = _ffi.Mask()
    m.kind = _ffi.MASK_VARLEN
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args(B=2)), C.byref(m), 0.1, None)) == "MFA_E_SHAPE"
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args()), C.byref(_ffi.Mask()), float("nan"), None)) == "MFA_E_ARG"


def test_maskrep_validation(lib):
    st = lib.mfa_make_block_ids(None, None, 1, 8, 2, None, None, None, None, None, None)
    assert _status(lib, st) == "MFA_E_ARG" and "cross_pad" in lib.mfa_last_error().decode()
    st = lib.mfa_compact_dense_mask(None, 10, 10, 32, 64, None, None, None, None, None, None)
    assert _status(lib, st) == "MFA_E_UNSUPPORTED"
    st = lib.mfa_tile_counts(None, -1, None, None)
    assert _status(lib, st) == "MFA_E_SHAPE"
    st = lib.mfa_tile_map_coarsen(None, -1, 10, None, None, None, None, None)
    assert _status(lib, st) == "MFA_E_SHAPE"
    st = lib.mfa_varlen_schedule(None, None, 2, 64, 64, 1, -1, -1, None, None, None, None, 4, None, None)
    assert _status(lib, st) == "MFA_E_UNSUPPORTED"
    st = lib.mfa_varlen_schedule(None, None, 2, 128, 64, 1, -2, -1, None, None, None, None, 4, None, None)
    assert _status(lib, st) == "MFA_E_ARG"
    st = lib.mfa_bsr_validate(None, None, 1, 1, 4, 4, 0, None, None)
    assert _status(lib, st) == "MFA_E_ARG"
    st = lib.mfa_bsr_prepare(None, None, 1, 1, 3, 4, 0, 64, 64, 256, 256, 1, None, None, None, None, None)
    assert _status(lib, st) == "MFA_E_SHAPE"
    st = lib.mfa_bsr_from_bitmask(None, 1, -1, 4, 4, None, None, 0, None)
    assert _status(lib, st) == "MFA_E_SHAPE"
    st = lib.mfa_bsr_from_bitmask(None, 1, 1, 1 << 16, 1 << 16, None, None, 0, None)
    assert _status(lib, st) == "MFA_E_UNSUPPORTED"
    st = lib.mfa_blockid_tile_summary(None, None, None, None, 1, 8, 8, 128, 32, None, None, None, None)
    assert _status(lib, st) == "MFA_E_UNSUPPORTED"


def test_paged_varlen_validation(lib):
    """Page sizes that are not multiples of the 64-key tile, and paged k / v in
    the backward, are refused before any device call."""
    a = _args(B=1)
    for ps, mp, npg, want in ((48, 4, 8, "MFA_E_ARG"), (0, 4, 8, "MFA_E_ARG"), (64, 0, 8, "MFA_E_ARG"),
                              (128, 4, 0, "MFA_E_ARG")):
        m = _ffi.Mask()
        m.kind, m.block_table, m.page_size, m.max_pages, m.n_pages = _ffi.MASK_VARLEN, 16, ps, mp, npg
        assert _status(lib, lib.mfa_attn_fwd(C.byref(a), C.byref(m), 0.1, None)) == want
    m = _ffi.Mask()
    m.kind, m.block_table, m.page_size, m.max_pages, m.n_pages = _ffi.MASK_VARLEN, 16, 64, 4, 8
    b = _ffi.BwdArgs()
    b.fwd = _args(B=1)
    b.fwd.dtype = _ffi.MFA_BF16
    # the backward accepts paged k / v too (here it stops at the device check)
    st = lib.mfa_attn_bwd_dq(C.byref(b), C.byref(m), 0.1, None)
    assert _status(lib, st) == "MFA_E_NO_DEVICE"


def test_predicate_validation_and_composition(lib):
    p = _ffi.Predicate()
    p.n_terms = 5
    assert _status(lib, lib.mfa_predicate_tiles(C.byref(p), 16, 16, None, None, None, None, None, None)) == "MFA_E_ARG"
    p.n_terms, p.n_atoms[0] = 1, 7
    assert _status(lib, lib.mfa_predicate_tiles(C.byref(p), 16, 16, None, None, None, None, None, None)) == "MFA_E_ARG"
    assert _status(lib, lib.mfa_predicate_tiles(None, 16, 16, None, None, None, None, None, None)) == "MFA_E_ARG"
    p.n_atoms[0] = 0
    assert _status(lib, lib.mfa_predicate_tiles(C.byref(p), -1, 16, None, None, None, None, None, None)) == "MFA_E_SHAPE"
    import masked_flash_attention_amd as mfa
    # and_ distributes over the disjunctions; or_ concatenates them
    a = mfa.Pred.causal().or_(mfa.Pred.prefix(3))
    b = a.and_(mfa.Pred.past_window(5))
    assert b.terms == (((1, -1, 0), (-1, 1, 4)), ((0, -1, 2), (-1, 1, 4)))
    assert mfa.Pred.noop().and_(a).terms == a.terms
    assert mfa.Pred.never().or_(a).terms == a.terms and mfa.Pred.never().and_(a).terms == ()
    with pytest.raises(ValueError):
        mfa.Pred(tuple(((1, 0, 0),) for _ in range(5))).to_c()


def test_empty_problems_are_noops(lib):
    m = _ffi.Mask()
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args(Sq=0)), C.byref(m), 0.1, None)) == "MFA_OK"
    assert _status(lib, lib.mfa_attn_fwd(C.byref(_args(B=0)), C.byref(m), 0.1, None)) == "MFA_OK"
    st = lib.mfa_make_block_ids(None, None, 0, 8, 0, None, None, None, None, None, None)
    assert _status(lib, st) == "MFA_OK"


def test_no_device_here_is_reported(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.mfa_is_available() == 0
    assert "device" in lib.mfa_last_error().decode().lower()
    m = _ffi.Mask()
    st = lib.mfa_attn_fwd(C.byref(_args()), C.byref(m), 0.1, None)
    assert _status(lib, st) == "MFA_E_NO_DEVICE"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_ffi, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_ffi, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        _ffi.load()
    import masked_flash_attention_amd as mfa
    assert mfa.is_available() is False
    assert "not built" in mfa.load_error()


def test_tile_height_model_and_choice(lib):
    """Host-only dispatch model: the causal N=8192 map keeps 128-row tiles;
    a map whose 128-row tiles are all half empty (64 x 64 blocks) picks 64."""
    import masked_flash_attention_amd as mfa
    causal64, causal128 = (8128, 128, 8128), (4032, 128, 4032)
    blocks64, blocks128 = (15384, 0, 1000), (7192, 1000, 0)
    for D in (64, 128):
        assert mfa.choose_tile_m(causal64, causal128, 8192, D) == 128
        assert mfa.choose_tile_m(blocks64, blocks128, 8192, D) == 64
    t = (C.c_int64 * 3)(0, 10, 20)
    t2 = (C.c_int64 * 3)(0, 10, 21)
    assert lib.mfa_model_tile_time(t2, 1000, 128, 128) > lib.mfa_model_tile_time(t, 1000, 128, 128) > 0
    assert lib.mfa_choose_tile_m(None, None, 10, 128) == 128
    # near ties keep 128-row tiles: 64 only with a modelled gain of 5 % or more
    # (at D = 128 a full 64-row tile models as 0.663 of a full 128-row one)
    c128 = (0, 0, 100)
    assert mfa.choose_tile_m((0, 0, 148), c128, 0, 128) == 128   # 2 % below
    assert mfa.choose_tile_m((0, 0, 140), c128, 0, 128) == 64    # 7 % below


def test_dkdv_head_split_model(lib):
    """Host-only split model of the dK/dV pass: the smallest divisor S of the
    GQA group with key_blocks * S >= 2 * CUs * (2 at D=128, 4 at D=64)."""
    import masked_flash_attention_amd as mfa
    cs = mfa.choose_dkdv_split
    # block-id GQA with cross columns: 8 * 2 * 20 = 320 key blocks, G = 8, 256 CUs
    assert cs(320, 8, 128, 256) == 4      # 1280 >= 1024; 2 would give 640
    assert cs(320, 8, 64, 256) == 8       # target 2048: no divisor below 8 reaches it
    assert cs(100, 6, 128, 256) == 6      # 2 and 3 fall short: the whole group
    assert cs(1024, 8, 128, 256) == 1     # enough key blocks already
    assert cs(1023, 3, 128, 256) == 3
    assert cs(600, 4, 128, 256) == 2
    assert cs(320, 1, 128, 256) == 1      # no GQA
    assert cs(0, 8, 128, 256) == 1
    assert cs(320, 8, 128, 0) == 1        # no device information
    assert cs(10, 8, 128, 1) == 1         # 10 >= 4
    assert cs(3, 8, 128, 1) == 2          # 6 >= 4


def test_host_code_under_sanitizers(tmp_path):
    """The C ABI's host code (api.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host side only, linked with the
    kernels' objects and driven by tests/c_abi/mfa_host_checks.cpp (every
    entry point with NULL pointers, bad shapes and enums, non-finite scales;
    the dispatch model; per-thread error messages). Any sanitizer report or
    failed check makes the driver exit non-zero."""
    from masked_flash_attention_amd import build as B
    objs = [os.path.join(B.BUILD, f) for f in ("maskrep.o", "attn_fwd.o", "attn_bwd.o")]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    hipcc = B.hipcc()
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    api_o, drv_o, exe = tmp_path / "api_san.o", tmp_path / "driver.o", tmp_path / "host_checks"
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined"]
    steps = [
        [hipcc] + B.COMMON + ["-g", "-O1"] + san_host +
        ["-x", "hip", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", str(api_o)],
        [clangxx, "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
         "-I", "/opt/rocm/include", "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
         "-c", os.path.join(ROOT, "tests", "c_abi", "mfa_host_checks.cpp"), "-o", str(drv_o)],
        [hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         str(drv_o), str(api_o)] + objs + ["-o", str(exe)],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-2000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
