"""Positional bias slope[h] * (kv_idx - q_idx) on the scaled scores (the
distance-decay score_mod of tensorplay omni_attention, intro, with one slope
per query head) through every mask kind, forward and backward, against the
oracle's score_mod path. Bounds as for the unbiased tests: bf16 out 2e-2, LSE
1e-3, fp32 test mode 1e-4; gradients 2e-2 plus one bf16 ULP of the exact value."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, DEV, F32_OUT_TOL, compare_attention, f64, grad_tolerance,
                            grad_tolerance_terms, note, to_dev)

pytestmark = pytest.mark.gpu


def geometric_slopes(H):
    """The usual ALiBi head slopes 2^(-8 (h + 1) / H)."""
    return 2.0 ** (-8.0 * (np.arange(H) + 1) / H)


def _slopes_dev(sl):
    return torch.tensor(np.asarray(sl, np.float32), device=DEV)


def _case(kind, D):
    """(q, k, v, do, rep, allowed, scale, layout, Hq) for a small case of each mask kind."""
    if kind == "tiles":
        Sq, Sk, Hq, Hkv = 300, 333, 4, 2
        mask = W.random_dense_mask(Sq, Sk, 0.3, 5) | np.eye(Sq, Sk, dtype=bool)
        q, k, v, do = W.tensors(90 + D, [(2, Sq, Hq, D), (2, Sk, Hkv, D), (2, Sk, Hkv, D), (2, Sq, Hq, D)])
        rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask)))
        return q, k, v, do, rep, mask[None, None], D ** -0.5, "bshd", Hq
    if kind == "none":
        Sq, Sk, Hq, Hkv = 200, 333, 4, 2
        q, k, v, do = W.tensors(91 + D, [(2, Sq, Hq, D), (2, Sk, Hkv, D), (2, Sk, Hkv, D), (2, Sq, Hq, D)])
        return q, k, v, do, mfa.MaskRep.none(), np.ones((1, 1, Sq, Sk), bool), D ** -0.5, "bshd", Hq
    if kind == "blockid":
        w = W.blockcausal_gqa_cross(B=3, N=333, Hq=4, Hkv=2, D=D, Nc=37, prefix=100, blk_lo=5, blk_hi=40,
                                    pad_hi=60, seed=22)
        ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), w["n_cross"], to_dev(w["cross_pad"]))
        allowed = M.blockid_mask(*M.make_att_block_ids(w["pad"], w["att"], w["n_cross"], w["cross_pad"]))[:, None]
        do = W.tensors(903, [tuple(w["q"].shape)])[0]
        return w["q"], w["k"], w["v"], do, mfa.MaskRep.blockid(*ids), allowed, w["scale"], "bshd", 4
    if kind == "bsr":
        N, H = 1000, 3
        w = W.bsr_random(B=2, N=N, H=H, D=D, block=64, frac_den=3, seed=7 + D)
        ip, ix = w["indptr"], w["indices"]
        bk, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, True)
        rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), bk, causal=True, csc_ptr=cp, csc_idx=ci)
        allowed = M.bsr_mask(ip, ix, 64, 64, N, N, True)
        do = W.tensors(904, [tuple(w["q"].shape)])[0]
        return w["q"], w["k"], w["v"], do, rep, allowed, w["scale"], "bshd", H
    raise ValueError(kind)


def _fwd(q, k, v, rep, scale, layout, dtype, slopes):
    qd, kd, vd = (to_dev(t, dtype) for t in (q, k, v))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout, alibi_slopes=_slopes_dev(slopes))
    torch.cuda.synchronize()
    return out, lse


def _check_grads(got, ref, tag, terms=(None, None, None)):
    for name, g, r, t in zip(("dq", "dk", "dv"), got, ref, terms):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite gradient"
        excess = np.abs(g - r) - (grad_tolerance(r) if t is None else grad_tolerance_terms(r, t))
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        assert excess[i] <= 0, f"{tag} {name}: |{g[i]:.5f} - {r[i]:.5f}| over the bound at {i}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["tiles", "none", "blockid", "bsr"])
def test_alibi_forward(kind, D, dtype):
    note(f"alibi fwd {kind} D={D} {dtype}")
    q, k, v, _, rep, allowed, scale, layout, Hq = _case(kind, D)
    sl = geometric_slopes(Hq)
    out, lse = _fwd(q, k, v, rep, scale, layout, dtype, sl)
    ro, rl = A.attention_fwd(q, k, v, allowed, scale, score_mod=A.alibi(sl.astype(np.float32)))
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_alibi_page_example(dtype):
    """The page's example, score - (q_idx - kv_idx), on q = k = v of shape
    (1, 2 heads, 16, D): slope 1 on both heads, no mask (head dim 64 here: the
    kernels are built for 64 and 128)."""
    note(f"alibi page example {dtype}")
    x = W.tensors(95, [(1, 2, 16, 64)])[0]
    out, lse = _fwd(x, x, x, mfa.MaskRep.none(), 64 ** -0.5, "bhsd", dtype, [1.0, 1.0])
    t = x.transpose(1, 2).contiguous()
    ro, rl = A.attention_fwd(t, t, t, np.ones((1, 1, 16, 16), bool), 64 ** -0.5, score_mod=A.alibi([1.0, 1.0]))
    compare_attention(f64(out).transpose(0, 2, 1, 3), f64(lse), ro, rl,
                      BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal,win", [(True, (100, 0)), (False, (50, 30)), (False, (-1, -1))])
def test_alibi_varlen_forward_uses_local_positions(causal, win, dtype):
    note(f"alibi varlen fwd causal={causal} win={win} {dtype}")
    L = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
    T = int(L.sum())
    Hq, Hkv, D = 4, 2, 64
    q, k, v = W.tensors(96, [(T, Hq, D), (T, Hkv, D), (T, Hkv, D)])
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=causal, window=win)
    sl = geometric_slopes(Hq) * 4
    out, lse = _fwd(q, k, v, rep, D ** -0.5, "thd", dtype, sl)
    cu = M.cu_seqlens(L)
    ro, rl = A.varlen_attention_fwd(q, k, v, cu, cu, D ** -0.5, causal, win[0], win[1],
                                    score_mod=A.alibi(sl.astype(np.float32)))
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["tiles", "none", "blockid", "bsr"])
def test_alibi_backward(kind, D):
    note(f"alibi bwd {kind} D={D}")
    q, k, v, do, rep, allowed, scale, layout, Hq = _case(kind, D)
    sl = geometric_slopes(Hq)
    slopes = _slopes_dev(sl)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout, alibi_slopes=slopes)
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, scale, layout, alibi_slopes=slopes)
    torch.cuda.synchronize()
    r = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=A.alibi(sl.astype(np.float32)), term_sums=True)
    _check_grads(got, r[:3], f"alibi {kind}", r[6])


@pytest.mark.parametrize("causal,win", [(True, (100, 0)), (False, (50, 30))])
def test_alibi_varlen_backward(causal, win):
    note(f"alibi varlen bwd causal={causal} win={win}")
    L = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
    T = int(L.sum())
    Hq, Hkv, D = 4, 2, 64
    q, k, v, do = W.tensors(97, [(T, Hq, D), (T, Hkv, D), (T, Hkv, D), (T, Hq, D)])
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=causal, window=win)
    sl = geometric_slopes(Hq) * 4
    slopes = _slopes_dev(sl)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, D ** -0.5, "thd", alibi_slopes=slopes)
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, D ** -0.5, "thd", alibi_slopes=slopes)
    torch.cuda.synchronize()
    # the bias uses positions local to each sequence: per-sequence dense oracle
    cu = M.cu_seqlens(L)
    ref = [np.zeros((T, Hq, D)), np.zeros((T, Hkv, D)), np.zeros((T, Hkv, D))]
    terms = [np.zeros_like(x) for x in ref]
    for si, n in enumerate(L):
        if n == 0:
            continue
        a, b = int(cu[si]), int(cu[si + 1])
        allowed = M.varlen_mask(np.array([0, n]), np.array([0, n]), causal, win[0], win[1])[None, None]
        g = A.attention_bwd(q[None, a:b], k[None, a:b], v[None, a:b], do[None, a:b], allowed, D ** -0.5,
                            score_mod=A.alibi(sl.astype(np.float32)), term_sums=True)
        for r, x in zip(ref, g[:3]):
            r[a:b] = x[0]
        for r, x in zip(terms, g[6]):
            r[a:b] = x[0]
    _check_grads(got, ref, "alibi varlen", terms)


def test_alibi_autograd_and_unbiased_path_unchanged():
    note("alibi autograd")
    B, N, H, D = 2, 190, 2, 128
    mask = np.tril(np.ones((N, N), bool))
    q, k, v, do = W.tensors(98, [(B, N, H, D)] * 4)
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask)))
    sl = np.array([0.5, 0.03125])
    qd, kd, vd = (to_dev(t).requires_grad_() for t in (q, k, v))
    out = mfa.masked_attention(qd, kd, vd, rep, 0.1, alibi_slopes=_slopes_dev(sl))
    out.backward(to_dev(do))
    torch.cuda.synchronize()
    mod = A.alibi(sl)
    ro = A.attention_fwd(q, k, v, mask[None, None], 0.1, score_mod=mod)[0]
    assert float(np.abs(f64(out) - ro).max()) <= BF16_OUT_TOL
    r = A.attention_bwd(q, k, v, do, mask[None, None], 0.1, score_mod=mod, term_sums=True)
    _check_grads([qd.grad, kd.grad, vd.grad], r[:3], "alibi autograd", r[6])
    # zero slopes run the biased kernels and must match the unbiased kernels bit for bit
    x = [to_dev(t) for t in (q, k, v)]
    o0, l0 = mfa.attn_fwd(*x, rep, 0.1)
    o1, l1 = mfa.attn_fwd(*x, rep, 0.1, alibi_slopes=_slopes_dev([0.0, 0.0]))
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)


def test_alibi_rejects_bad_slopes():
    note("alibi slope validation")
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device=DEV)
    for bad in (torch.ones(3, device=DEV), torch.ones(2, dtype=torch.float64, device=DEV), torch.ones(2)):
        with pytest.raises(ValueError):
            mfa.attn_fwd(q, q, q, mfa.MaskRep.none(), alibi_slopes=bad)


def test_alibi_causal_8192_sampled():
    """The causal dense-mask workload (B=4, H=32, N=8192, D=128) with the
    geometric slopes: sampled rows of two (batch, head) slices forward, and dQ
    rows / dK, dV columns of one slice."""
    note("alibi causal 8192 full size")
    w = W.causal_dense()
    B, H, N, D = w["q"].shape
    mask = w["mask"]
    sl = geometric_slopes(H)
    slopes = _slopes_dev(sl)
    do = W.tensors(2003, [(B, H, N, D)])[0]
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask)))
    qd, kd, vd, dod = (to_dev(t) for t in (w["q"], w["k"], w["v"], do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "bhsd", alibi_slopes=slopes)
    dq, dk, dv = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, w["scale"], "bhsd", alibi_slopes=slopes)
    torch.cuda.synchronize()

    def allowed(bb, hm, rr):
        return mask[np.asarray(rr)]
    allowed.heads = 1
    sl32 = sl.astype(np.float32)
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    cols = np.array([0, 63, 64, 4095, 8190, 8191])
    cut = lambda t, b, h: t[b:b + 1, h:h + 1].transpose(1, 2)  # noqa: E731  -> (1, N, 1, D)
    for b, h in ((0, 0), (3, 31)):
        mod = lambda s, bb, hh, qi, kj, h=h: s + sl32[h] * (np.asarray(kj, float) - np.asarray(qi, float))  # noqa: E731
        ro, rl = A.attention_fwd(cut(w["q"], b, h), cut(w["k"], b, h), cut(w["v"], b, h), allowed, w["scale"],
                                 rows=rows, score_mod=mod)
        compare_attention(f64(out[b, h, rows])[None, :, None], f64(lse[b, h, rows])[None, None], ro, rl,
                          BF16_OUT_TOL)
        if (b, h) == (3, 31):
            rq, rk, rv = A.attention_bwd_sampled(cut(w["q"], b, h), cut(w["k"], b, h), cut(w["v"], b, h),
                                                 cut(do, b, h), allowed, w["scale"], 0, 0, rows, cols,
                                                 chunk=2048, score_mod=mod)
            _check_grads([dq[b, h, rows], dk[b, h, cols], dv[b, h, cols]], [rq[0], rk, rv], "alibi cfg2")
    for t in (out, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
