"""BSR backward on the GPU (preprocess, dK/dV over key blocks, dQ over query
blocks) against the fp64 oracle: max-abs error of dQ, dK, dV <= 2e-2 (bf16).
delta = sum_d dO*O is formed from the stored bf16 output; it is checked
against that definition at fp32-accumulation tolerance."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import BF16_OUT_TOL, DEV, bsr_row_mask, compare_attention, f64, nan_like, note, tile_rows, to_dev

pytestmark = pytest.mark.gpu


def _bsr_run(w, N, causal, Hq=None):
    ip, ix = w["indptr"], w["indices"]
    ipd, ixd = to_dev(ip), to_dev(ix)
    kind, cp, ci = mfa.bsr_prepare(ipd, ixd, 64, 64, N, N, causal)
    rep = mfa.MaskRep.bsr(ipd, ixd, kind, causal=causal, csc_ptr=cp, csc_idx=ci)
    q, k, v, do = (to_dev(w[x]) for x in ("q", "k", "v", "do"))
    out, lse = mfa.attn_fwd(q, k, v, rep, w["scale"], "bshd")
    dq, dk, dv = mfa.attn_bwd(q, k, v, out, lse, do, rep, w["scale"], "bshd")
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _small(N, H, Hkv, D, seed):
    w = W.bsr_random(B=2, N=N, H=Hkv, D=D, block=64, frac_den=3, seed=seed)
    if H != Hkv:
        q, do = W.tensors(seed + 100, [(2, N, H, D), (2, N, H, D)])
        w["q"], w["do"] = q, do
    return w


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("gqa", [False, True])
def test_bsr_backward_small(D, causal, gqa):
    note(f"bsr bwd small D={D} causal={causal} gqa={gqa}")
    N = 700
    H, Hkv = (4, 2) if gqa else (3, 3)
    w = _small(N, H, Hkv, D, seed=D + 2 * causal + gqa)
    out, lse, dq, dk, dv = _bsr_run(w, N, causal)
    allowed = M.bsr_mask(w["indptr"], w["indices"], 64, 64, N, N, causal)
    rdq, rdk, rdv, ro, rl, rdelta = A.attention_bwd(w["q"], w["k"], w["v"], w["do"], allowed, w["scale"])
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        err = float(np.abs(f64(g) - r).max())
        rel = float(np.linalg.norm(f64(g) - r) / max(np.linalg.norm(r), 1e-30))
        assert err <= BF16_OUT_TOL, f"{name} max-abs {err:.3e} (rel L2 {rel:.2e})"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_bsr_key_tail_short_of_half_block(D, causal):
    """N = 520 = 8*64 + 8: the last 64-key block holds 8 keys, so with 32-key
    steps one step is partly past the end and the next wholly past it."""
    note(f"bsr fwd+bwd N=520 D={D} causal={causal}")
    N = 520
    w = _small(N, 3, 3, D, seed=40 + D + causal)
    out, lse, dq, dk, dv = _bsr_run(w, N, causal)
    allowed = M.bsr_mask(w["indptr"], w["indices"], 64, 64, N, N, causal)
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(w["q"], w["k"], w["v"], w["do"], allowed, w["scale"])
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        err = float(np.abs(f64(g) - r).max())
        assert err <= BF16_OUT_TOL, f"{name} max-abs {err:.3e}"


def test_bsr_backward_deterministic():
    note("bsr bwd determinism")
    w = _small(520, 2, 2, 128, seed=3)
    a = _bsr_run(w, 520, True)
    b = _bsr_run(w, 520, True)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bsr_delta_matches_oracle():
    note("bsr delta")
    N, D = 300, 64
    w = _small(N, 2, 2, D, seed=8)
    ipd, ixd = to_dev(w["indptr"]), to_dev(w["indices"])
    kind, cp, ci = mfa.bsr_prepare(ipd, ixd, 64, 64, N, N, True)
    rep = mfa.MaskRep.bsr(ipd, ixd, kind, causal=True, csc_ptr=cp, csc_idx=ci)
    q, k, v, do = (to_dev(w[x]) for x in ("q", "k", "v", "do"))
    out, lse = mfa.attn_fwd(q, k, v, rep, w["scale"], "bshd")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.full((2, 2, N), float("nan"), device=DEV)
    args = mfa._bwd_args(q, k, v, out, lse, do, dq, dk, dv, delta, "bshd")
    mfa.attn_bwd_preprocess(args)
    torch.cuda.synchronize()
    # delta is formed from the stored bf16 output: compare with that definition
    # exactly (fp32 accumulation), and loosely with the exact oracle output
    want = np.einsum("bshd,bshd->bhs", f64(do), f64(out))
    assert float(np.abs(f64(delta) - want).max()) <= 1e-4
    allowed = M.bsr_mask(w["indptr"], w["indices"], 64, 64, N, N, True)
    *_, rdelta = A.attention_bwd(w["q"], w["k"], w["v"], w["do"], allowed, w["scale"])
    assert float(np.abs(f64(delta) - rdelta).max()) <= 5e-2


def test_cfg5_backward_every_block():
    """B=2, N=16384, H=16, D=128, 64x64 BSR blocks, causal inside blocks:
    forward + two-pass backward at full size into NaN-filled dq / dk / dv.
    One dQ row of every 64-row query block of every (b, h) against the
    oracle's row-local gradient; one dK/dV column of every 64-key block of
    three (b, h) slices; every gradient must be finite."""
    note("cfg5 bwd full size, every block")
    w = W.bsr_random()
    B, N, H, D = w["q"].shape
    blk = 64
    ip, ix = w["indptr"], w["indices"]
    ipd, ixd = to_dev(ip), to_dev(ix)
    kind, cp, ci = mfa.bsr_prepare(ipd, ixd, blk, blk, N, N, True)
    rep = mfa.MaskRep.bsr(ipd, ixd, kind, causal=True, csc_ptr=cp, csc_idx=ci)
    q, k, v, do = (to_dev(w[x]) for x in ("q", "k", "v", "do"))
    out, lse = mfa.attn_fwd(q, k, v, rep, w["scale"], "bshd")
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    mfa.attn_bwd(q, k, v, out, lse, do, rep, w["scale"], "bshd", dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b in range(B):
        for h in range(H):
            rows = tile_rows(N, blk, 3 * b + 17 * h)
            allowed = lambda bb, hm, rr, b=b, h=h: bsr_row_mask(ip[b, h], ix, blk, N, rr)  # noqa: E731
            allowed.heads = 1
            sl = [w[x][b, :, h].double().numpy()[None, :, None, :] for x in ("q", "k", "v", "do")]
            rq = A.attention_bwd_dq_rows(*sl, allowed, w["scale"], rows)
            err = float(np.abs(f64(dq[b, rows, h]) - rq[0, :, 0]).max())
            assert err <= BF16_OUT_TOL, f"dq (b={b}, h={h}) max-abs {err:.3e}"
    cols_fixed = np.array([0, 1, 64, 9000, 16383])
    for b, h in [(0, 3), (1, 15), (1, 0)]:
        cols = np.unique(np.concatenate([tile_rows(N, blk, 29 * b + h), cols_fixed]))
        allowed = lambda bb, hm, rr, b=b, h=h: bsr_row_mask(ip[b, h], ix, blk, N, rr)  # noqa: E731
        allowed.heads = 1
        sl = [w[x][b, :, h].double().numpy()[None, :, None, :] for x in ("q", "k", "v", "do")]
        rq, rk, rv = A.attention_bwd_sampled(*sl, allowed, w["scale"], 0, 0, cols_fixed, cols, chunk=2048)
        for name, g, r in (("dq", f64(dq[b, cols_fixed, h]), rq[0]), ("dk", f64(dk[b, cols, h]), rk),
                           ("dv", f64(dv[b, cols, h]), rv)):
            err = float(np.abs(g - r).max())
            assert err <= BF16_OUT_TOL, f"{name} (b={b}, h={h}) max-abs {err:.3e}"
