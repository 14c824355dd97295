"""Attention forward on the GPU against the fp64 oracle.

bf16: out max-abs <= 2e-2, LSE max-abs <= 1e-3; fp32 test mode: out <= 1e-4.
Rows with no allowed key must be exactly 0 / -inf. Outputs are NaN-filled
before each call so unwritten rows show up.
"""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, DEV, F32_OUT_TOL, LSE_TOL, bsr_row_mask, compare_attention, f64,
                            nan_like, note, tile_rows, to_dev)

pytestmark = pytest.mark.gpu


def _bshd(x, layout):
    """numpy fp64 (B, S, H, D) view of a tensor in `layout`."""
    a = f64(x)
    return a.transpose(0, 2, 1, 3) if layout == "bhsd" else a


def _run(q, k, v, rep, scale, layout, dtype):
    qd, kd, vd = (to_dev(t, dtype) for t in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    if layout == "thd":
        lse = torch.full((qd.shape[1], qd.shape[0]), float("nan"), device=DEV)
    else:
        B, Hq, Sq = (qd.shape[0], qd.shape[2], qd.shape[1]) if layout == "bshd" else qd.shape[:3]
        lse = torch.full((B, Hq, Sq), float("nan"), device=DEV)
    mfa.attn_fwd(qd, kd, vd, rep, scale, layout, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _tol(dtype):
    return BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL


def _inputs(shape_q, shape_k, seed, dtype):
    q, k, v = W.tensors(seed, [shape_q, shape_k, shape_k], torch.bfloat16)
    return q, k, v


# --- dense-mask tiles (BinFlash) ------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("maskcase", ["random", "causal", "all_true", "all_false"])
def test_tiles_small(dtype, layout, D, maskcase):
    note(f"tiles small {dtype} {layout} D={D} {maskcase}")
    B, H, Sq, Sk = 2, 3, 300, 333
    if maskcase == "random":
        m = W.random_dense_mask(Sq, Sk, 0.4, seed=D)
    elif maskcase == "causal":
        m = np.tri(Sq, Sk, dtype=bool)
    elif maskcase == "all_true":
        m = np.ones((Sq, Sk), bool)
    else:
        m = np.zeros((Sq, Sk), bool)
    shp_q = (B, Sq, H, D) if layout == "bshd" else (B, H, Sq, D)
    shp_k = (B, Sk, H, D) if layout == "bshd" else (B, H, Sk, D)
    q, k, v = _inputs(shp_q, shp_k, 100 + D, dtype)
    comp = mfa.compact_dense_mask(to_dev(m))
    out, lse = _run(q, k, v, mfa.MaskRep.tiles(comp), D ** -0.5, layout, dtype)
    ro, rl = A.attention_fwd(_bshd(q, layout), _bshd(k, layout), _bshd(v, layout), m[None, None], D ** -0.5)
    compare_attention(_bshd(out, layout), f64(lse), ro, rl, _tol(dtype))


@pytest.mark.parametrize("maskcase", ["random", "causal", "late_start"])
def test_tiles_peaked_scores(maskcase):
    """q and k scaled by 6 (score spread ~36x the unit case): the running max
    moves by far more than the lazy-rescale margin on many tiles, so the
    rescale path and the first-key threshold of each row are exercised.
    late_start: half of the rows see no key in their first key tiles."""
    note(f"tiles peaked {maskcase}")
    B, H, Sq, Sk, D = 1, 2, 300, 700, 128
    if maskcase == "random":
        m = W.random_dense_mask(Sq, Sk, 0.3, seed=9)
    elif maskcase == "causal":
        m = np.tri(Sq, Sk, k=Sk - Sq, dtype=bool)
    else:
        m = np.ones((Sq, Sk), bool)
        m[::2, :400] = False
    q, k, v = _inputs((B, H, Sq, D), (B, H, Sk, D), 31, torch.bfloat16)
    q, k = (q * 6).to(torch.bfloat16), (k * 6).to(torch.bfloat16)
    out, lse = _run(q, k, v, mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m))), D ** -0.5, "bhsd",
                    torch.bfloat16)
    ro, rl = A.attention_fwd(_bshd(q, "bhsd"), _bshd(k, "bhsd"), _bshd(v, "bhsd"), m[None, None], D ** -0.5)
    compare_attention(_bshd(out, "bhsd"), f64(lse), ro, rl, BF16_OUT_TOL)


def test_tiles_causal_1024_and_none_mask():
    note("tiles causal 1024 + none")
    B, H, N, D = 1, 2, 1024, 128
    q, k, v = _inputs((B, H, N, D), (B, H, N, D), 7, torch.bfloat16)
    m = np.tril(np.ones((N, N), bool))
    out, lse = _run(q, k, v, mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m))), D ** -0.5, "bhsd",
                    torch.bfloat16)
    ro, rl = A.attention_fwd(_bshd(q, "bhsd"), _bshd(k, "bhsd"), _bshd(v, "bhsd"), m[None, None], D ** -0.5)
    compare_attention(_bshd(out, "bhsd"), f64(lse), ro, rl, BF16_OUT_TOL)
    out, lse = _run(q, k, v, mfa.MaskRep.none(), D ** -0.5, "bhsd", torch.bfloat16)
    ro, rl = A.attention_fwd(_bshd(q, "bhsd"), _bshd(k, "bhsd"), _bshd(v, "bhsd"),
                             np.ones((1, 1, N, N), bool), D ** -0.5)
    compare_attention(_bshd(out, "bhsd"), f64(lse), ro, rl, BF16_OUT_TOL)


def test_cfg2_causal_8192_every_tile():
    """Causal dense mask, B=4, H=32, N=8192, D=128 bf16 in (B, H, N, D): the
    benchmark's launch, into NaN-filled out / lse. One row of every 128-row
    query tile of every (b, h) (8192 rows) against the oracle, plus the tile
    edges of a few slices; then the whole output must be finite."""
    note("cfg2 full size, every query tile of every (b, h)")
    w = W.causal_dense()
    B, H, N, D = w["q"].shape
    comp = mfa.compact_dense_mask(to_dev(w["mask"]))
    qd, kd, vd = (to_dev(w[x]) for x in "qkv")
    out = nan_like(qd)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    mfa.attn_fwd(qd, kd, vd, mfa.MaskRep.tiles(comp), w["scale"], "bhsd", out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    tri = w["mask"]
    allowed = lambda b, h, rr: tri[rr]  # noqa: E731
    allowed.heads = 1
    edges = np.array([0, 1, 63, 64, 127, 128, 129, 2047, 4095, 4096, 6000, 8190, 8191])
    worst = (0.0, 0.0)
    for b in range(B):
        for h in range(H):
            rows = tile_rows(N, 128, 7 * b + 3 * h)
            if (b, h) in ((0, 0), (1, 7), (2, 31), (3, 16)):
                rows = np.unique(np.concatenate([rows, edges]))
            sl = [w[x][b, h].double().numpy()[None, :, None, :] for x in "qkv"]
            ro, rl = A.attention_fwd(*sl, allowed, w["scale"], rows=rows)
            go = f64(out[b, h, rows])[None, :, None, :]
            gl = f64(lse[b, h, rows])[None, None, :]
            e = compare_attention(go, gl, ro, rl, BF16_OUT_TOL)
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    print(f"cfg2 every tile: out max-abs {worst[0]:.2e}, lse max-abs {worst[1]:.2e}")


# --- block ids (opentau) -----------------------------------------------------------

def _blockid_case(name):
    if name == "cfg1":
        w = W.blockcausal_tiny()
        return w, None, None
    if name == "cfg4":
        w = W.blockcausal_gqa_cross()
        return w, w["n_cross"], w["cross_pad"]
    w = W.blockcausal_gqa_cross(B=3, N=333, Hq=4, Hkv=2, D=64, Nc=37, prefix=100, blk_lo=5, blk_hi=40,
                                pad_hi=60, seed=21)
    return w, w["n_cross"], w["cross_pad"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("name", ["cfg1", "small_gqa_cross", "cfg4"])
def test_blockid(name, dtype):
    note(f"blockid {name} {dtype}")
    w, nc, cross = _blockid_case(name)
    ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), nc, None if cross is None else to_dev(cross))
    rep = mfa.MaskRep.blockid(*ids)
    out, lse = _run(w["q"], w["k"], w["v"], rep, w["scale"], "bshd", dtype)
    ref_ids = M.make_att_block_ids(w["pad"], w["att"], nc, cross)
    allowed = M.blockid_mask(*ref_ids)[:, None]
    ro, rl = A.attention_fwd(f64(w["q"]), f64(w["k"]), f64(w["v"]), allowed, w["scale"])
    compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))


def test_blockid_arbitrary_ids():
    note("blockid arbitrary ids")
    rng = np.random.default_rng(2)
    B, Sq, Sk, H, D = 2, 200, 150, 2, 128
    ids = (rng.integers(-3, 4, (B, Sq)).astype(np.int32), rng.integers(-3, 4, (B, Sk)).astype(np.int32),
           rng.random((B, Sq)) < 0.8, rng.random((B, Sk)) < 0.8)
    q, k, v = _inputs((B, Sq, H, D), (B, Sk, H, D), 3, torch.bfloat16)
    rep = mfa.MaskRep.blockid(*[to_dev(x) for x in ids])
    out, lse = _run(q, k, v, rep, 0.1, "bshd", torch.bfloat16)
    ro, rl = A.attention_fwd(f64(q), f64(k), f64(v), M.blockid_mask(*ids)[:, None], 0.1)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)


# --- BSR (flashinfer block_sparse_attention) -------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_bsr_small(dtype, causal, D):
    note(f"bsr small {dtype} causal={causal} D={D}")
    N, H = 1000, 3
    w = W.bsr_random(B=2, N=N, H=H, D=D, block=64, frac_den=3, seed=D + causal)
    ip, ix = w["indptr"], w["indices"]
    kind, _, _ = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, causal)
    rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=causal)
    out, lse = _run(w["q"], w["k"], w["v"], rep, w["scale"], "bshd", dtype)
    allowed = M.bsr_mask(ip, ix, 64, 64, N, N, causal)
    ro, rl = A.attention_fwd(f64(w["q"]), f64(w["k"]), f64(w["v"]), allowed, w["scale"])
    compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))


def test_cfg5_bsr_forward_every_block():
    """BSR, B=2, N=16384, H=16, D=128, 64x64 blocks, causal inside blocks,
    into NaN-filled out / lse: one row of every 64-row block of every (b, h)
    (8192 rows) against the oracle; the whole output must be finite."""
    note("cfg5 bsr forward full size, every block of every (b, h)")
    w = W.bsr_random()
    B, N, H, D = w["q"].shape
    blk = 64
    ip, ix = w["indptr"], w["indices"]
    kind, _, _ = mfa.bsr_prepare(to_dev(ip), to_dev(ix), blk, blk, N, N, True)
    rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=True)
    qd, kd, vd = (to_dev(w[x]) for x in "qkv")
    out = nan_like(qd)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "bshd", out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    edges = np.array([0, 5, 63, 64, 640, 5000, 9999, 16383])
    for b in range(B):
        for h in range(H):
            rows = tile_rows(N, blk, 5 * b + 11 * h)
            if (b, h) in ((0, 0), (1, 15), (0, 9)):
                rows = np.unique(np.concatenate([rows, edges]))
            allowed = lambda bb, hm, rr, b=b, h=h: bsr_row_mask(ip[b, h], ix, blk, N, rr)  # noqa: E731
            allowed.heads = 1
            sl = [w[x][b, :, h].double().numpy()[None, :, None, :] for x in "qkv"]
            ro, rl = A.attention_fwd(*sl, allowed, w["scale"], rows=rows)
            compare_attention(f64(out[b, rows, h])[None, :, None], f64(lse[b, h, rows])[None, None], ro, rl,
                              BF16_OUT_TOL)


# --- varlen (tensorplay varlen) -----------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("win", [(100, 0), (-1, -1), (511, 0)])
def test_varlen_small(dtype, win):
    note(f"varlen small {dtype} {win}")
    L = np.array([1, 128, 129, 0, 700, 300, 7, 64], np.int32)
    T = int(L.sum())
    H, D = 4, 64
    q, k, v = _inputs((T, H, D), (T, 2, D), 31, torch.bfloat16)
    causal = True
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=causal, window=win)
    out, lse = _run(q, k, v, rep, D ** -0.5, "thd", dtype)
    cu = M.cu_seqlens(L)
    ro, rl = A.varlen_attention_fwd(f64(q), f64(k), f64(v), cu, cu, D ** -0.5, causal, win[0], win[1])
    compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))


def test_cfg3_varlen_every_tile():
    """Varlen, 32 packed sequences, causal + 512-key window, (T, 16, 64) bf16,
    into NaN-filled out / lse: one row of every 128-row query tile of every
    sequence, all 16 heads, plus each sequence's first and last rows, against
    the oracle; the whole output must be finite."""
    note("cfg3 varlen full size, every query tile")
    w = W.varlen_window()
    L = w["lengths"]
    T = int(L.sum())
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=(511, 0), work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=True, window=(511, 0))
    qd, kd, vd = (to_dev(w[x]) for x in "qkv")
    out = nan_like(qd)
    lse = torch.full((qd.shape[1], T), float("nan"), device=DEV)
    mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "thd", out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    cu = M.cu_seqlens(L)
    per_seq = [cu[i] + tile_rows(int(L[i]), 128, 13 * i) for i in range(L.size)]
    rows = np.unique(np.concatenate(per_seq + [cu[:-1], cu[1:] - 1, cu[:-1] + 600]))
    rows = rows[(rows >= 0) & (rows < T)]
    ro, rl = A.varlen_attention_fwd(f64(w["q"]), f64(w["k"]), f64(w["v"]), cu, cu, w["scale"], True, 511, 0,
                                    rows=rows)
    compare_attention(f64(out[rows]), f64(lse[:, rows]), ro, rl, BF16_OUT_TOL)


def test_varlen_understated_max_is_an_error():
    note("varlen understated max")
    L = np.array([300, 100], np.int32)
    T = int(L.sum())
    q, k, v = _inputs((T, 2, 64), (T, 2, 64), 5, torch.bfloat16)
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=(-1, -1), work_cap=T // 128 + 2)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rep = mfa.MaskRep.varlen(s, 200, 200, causal=True, err=err)
    out, lse = mfa.attn_fwd(*(to_dev(t) for t in (q, k, v)), rep, None, "thd")
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert torch.isnan(out[:300].float()).all() and torch.isfinite(out[300:].float()).all()


# --- properties ---------------------------------------------------------------------

def test_deterministic_and_all_false_is_empty():
    note("determinism")
    w = W.blockcausal_tiny()
    ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]))
    rep = mfa.MaskRep.blockid(*ids)
    o1, l1 = _run(w["q"], w["k"], w["v"], rep, w["scale"], "bshd", torch.bfloat16)
    o2, l2 = _run(w["q"], w["k"], w["v"], rep, w["scale"], "bshd", torch.bfloat16)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    padded = f64(o1)[0, -16:]
    assert np.all(padded == 0.0) and np.all(np.signbit(padded) == False)  # noqa: E712
    assert torch.isneginf(l1[0, :, -16:]).all()


def test_error_paths_on_device():
    note("error paths")
    q = torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 64, 3, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mfa.MfaError) as e:
        mfa.attn_fwd(q, k, k, mfa.MaskRep.none())
    assert e.value.status_name == "MFA_E_SHAPE"
    with pytest.raises(mfa.MfaError) as e:
        mfa.attn_fwd(q.cpu(), q.cpu(), q.cpu(), mfa.MaskRep.none(), out=q.clone())
    assert e.value.status_name == "MFA_E_NOT_DEVICE"
    q96 = torch.zeros(1, 64, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mfa.MfaError) as e:
        mfa.attn_fwd(q96, q96, q96, mfa.MaskRep.none())
    assert e.value.status_name == "MFA_E_UNSUPPORTED"
    with pytest.raises(mfa.MfaError) as e:
        mfa.attn_fwd(q.half(), q.half(), q.half(), mfa.MaskRep.none())
    assert e.value.status_name == "MFA_E_DTYPE"


def test_key_span_over_4gib():
    """K and V rows 256 KiB apart (views into larger buffers), 20037 keys: one
    (batch, head)'s keys span 5.25 GB, past the 32-bit range of a buffer load
    counted from the first key. Forward and backward against the oracle."""
    Sq, Sk, D, RS = 64, 20037, 128, 1 << 17
    note(f"key span over 4 GiB: Sk={Sk} row stride {RS} elements")
    q, k, v, do = W.tensors(77, [(1, Sq, 1, D), (1, Sk, 1, D), (1, Sk, 1, D), (1, Sq, 1, D)])
    views = []
    for t in (k, v):
        buf = torch.empty(Sk * RS, dtype=torch.bfloat16, device=DEV)
        view = buf.as_strided((1, Sk, 1, D), (Sk * RS, RS, D, 1))
        view.copy_(t.to(DEV))
        views.append(view)
    kd, vd = views
    qd, dod = to_dev(q), to_dev(do)
    allowed = np.ones((1, 1, Sq, Sk), bool)
    scale = D ** -0.5
    out, lse = mfa.attn_fwd(qd, kd, vd, mfa.MaskRep.none(), scale, "bshd")
    dq, dk, dv = mfa.attn_bwd(qd, kd, vd, out, lse, dod, mfa.MaskRep.none(), scale, "bshd")
    torch.cuda.synchronize()
    kb, vb = (f64(x) for x in views)  # the bf16 values the kernels read
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(f64(qd), kb, vb, f64(dod), allowed, scale)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        err = float(np.abs(f64(g) - r).max())
        assert err <= BF16_OUT_TOL, f"{name} max-abs {err:.3e}"
    del views, kd, vd
    with pytest.raises(mfa.MfaError) as e:
        big = torch.empty((1 << 24) + 64, dtype=torch.bfloat16, device=DEV)
        qs = big.as_strided((1, 2, 1, 64), ((1 << 24) + 64, 1 << 24, 64, 1))
        mfa.attn_fwd(qs, qs, qs, mfa.MaskRep.none())
    assert e.value.status_name == "MFA_E_UNSUPPORTED"


# --- edge cases ----------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_no_keys_gives_empty_rows(dtype):
    note(f"edge Sk=0 {dtype}")
    q = to_dev(W.tensors(60, [(2, 5, 2, 64)])[0], dtype)
    k = torch.zeros(2, 0, 2, 64, dtype=dtype, device=DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, 2, 5), float("nan"), device=DEV)
    mfa.attn_fwd(q, k, k, mfa.MaskRep.none(), 0.125, "bshd", out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0) and torch.isneginf(lse).all()


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 1, 1, 65), (3, 129, 2, 1), (1, 63, 1, 64), (2, 200, 3, 300)])
def test_odd_sizes_none_and_tiles(shape):
    B, Sq, H, Sk = shape
    note(f"edge odd sizes {shape}")
    D = 128
    q, k, v = _inputs((B, Sq, H, D), (B, Sk, H, D), 61 + Sq, torch.bfloat16)
    for rep, m in ((mfa.MaskRep.none(), np.ones((Sq, Sk), bool)),
                   (None, W.random_dense_mask(Sq, Sk, 0.5, seed=Sq))):
        if rep is None:
            rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
        out, lse = _run(q, k, v, rep, 0.09, "bshd", torch.bfloat16)
        ro, rl = A.attention_fwd(f64(q), f64(k), f64(v), m[None, None], 0.09)
        compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)


def test_strided_views():
    """q/k/v/out as non-contiguous views (head-dim contiguous): a slice of a
    larger head axis and a permuted (B, H, S, D) tensor read as (B, S, H, D)."""
    note("edge strided views")
    B, S, H, D = 2, 190, 3, 64
    big = W.tensors(62, [(B, S, 2 * H, D)])[0].to(DEV)
    q = big[:, :, 1::2]  # every other head
    k, v = (W.tensors(63, [(B, H, S, D)])[0].to(DEV).permute(0, 2, 1, 3) for _ in range(2))
    out = torch.full((B, S, 2 * H, D), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :, ::2]
    lse = torch.empty(B, H, S, device=DEV)
    m = np.tri(S, S, dtype=bool)
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
    mfa.attn_fwd(q, k, v, rep, 0.125, "bshd", out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = A.attention_fwd(f64(q), f64(k), f64(v), m[None, None], 0.125)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)


def test_varlen_all_empty_sequences_and_single_tokens():
    note("edge varlen zeros and ones")
    L = np.array([0, 1, 0, 1, 2, 0], np.int32)
    T = int(L.sum())
    q, k, v = _inputs((T, 2, 64), (T, 2, 64), 64, torch.bfloat16)
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=(-1, -1), work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, 2, 2, causal=True)
    out, lse = _run(q, k, v, rep, 0.125, "thd", torch.bfloat16)
    cu = M.cu_seqlens(L)
    ro, rl = A.varlen_attention_fwd(f64(q), f64(k), f64(v), cu, cu, 0.125, True, -1, -1)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)
