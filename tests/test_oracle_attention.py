"""Pins for the oracle's fp64 attention (CPU only).

Library cross-checks use torch's CPU float64 scaled_dot_product_attention and
autograd; the rest are closed forms, invariants and finite differences.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import masks as M
import workloads as W


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask, scale, gqa=False):
    """torch CPU float64 SDPA in (B, H, S, D); q/k/v given as (B, S, H, D) numpy."""
    t = [torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=m, scale=scale, enable_gqa=gqa)
    return o.numpy().transpose(0, 2, 1, 3)


def test_all_true_equals_sdpa():
    q, k, v = _rand((2, 37, 3, 16), 1), _rand((2, 53, 3, 16), 2), _rand((2, 53, 3, 16), 3)
    allowed = np.ones((1, 1, 37, 53), bool)
    out, lse = A.attention_fwd(q, k, v, allowed, 0.3)
    np.testing.assert_allclose(out, _sdpa(q, k, v, None, 0.3), rtol=1e-12, atol=1e-12)
    assert lse.shape == (2, 3, 37)


def test_masked_equals_sdpa_with_bool_mask():
    rng = np.random.default_rng(4)
    q, k, v = _rand((2, 40, 4, 8), 5), _rand((2, 31, 4, 8), 6), _rand((2, 31, 4, 8), 7)
    mask = rng.random((2, 4, 40, 31)) < 0.3
    mask[..., 0] = True  # no empty rows (SDPA returns NaN for them)
    out, _ = A.attention_fwd(q, k, v, mask, 0.25)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask, 0.25), rtol=1e-12, atol=1e-12)


def test_gqa_equals_sdpa_enable_gqa_and_repeat_interleave():
    rng = np.random.default_rng(8)
    q, k, v = _rand((1, 20, 6, 8), 9), _rand((1, 24, 2, 8), 10), _rand((1, 24, 2, 8), 11)
    mask = rng.random((1, 1, 20, 24)) < 0.5
    mask[..., 3] = True
    out, lse = A.attention_fwd(q, k, v, mask, 0.5)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask, 0.5, gqa=True), rtol=1e-12, atol=1e-12)
    out2, lse2 = A.attention_fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), mask, 0.5)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_single_allowed_key_and_zero_query():
    q, k, v = _rand((1, 6, 1, 4), 12), _rand((1, 9, 1, 4), 13), _rand((1, 9, 1, 4), 14)
    mask = np.zeros((1, 1, 6, 9), bool)
    for i in range(6):
        mask[0, 0, i, (2 * i + 1) % 9] = True
    out, lse = A.attention_fwd(q, k, v, mask, 0.7)
    for i in range(6):
        j = (2 * i + 1) % 9
        np.testing.assert_array_equal(out[0, i, 0], v[0, j, 0])
        assert lse[0, 0, i] == pytest.approx(0.7 * q[0, i, 0] @ k[0, j, 0], rel=1e-14)
    q0 = np.zeros_like(q)
    mask2 = np.random.default_rng(15).random((1, 1, 6, 9)) < 0.5
    mask2[..., 0] = True
    out, lse = A.attention_fwd(q0, k, v, mask2, 0.7)
    for i in range(6):
        sel = mask2[0, 0, i]
        np.testing.assert_allclose(out[0, i, 0], v[0, sel, 0].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert lse[0, 0, i] == pytest.approx(np.log(sel.sum()), abs=1e-14)


def test_two_keys_sigmoid_weights():
    q, k, v = _rand((1, 1, 1, 5), 16), _rand((1, 2, 1, 5), 17), _rand((1, 2, 1, 5), 18)
    s = 0.4 * (k[0, :, 0] @ q[0, 0, 0])
    w0 = 1.0 / (1.0 + np.exp(s[1] - s[0]))
    out, lse = A.attention_fwd(q, k, v, np.ones((1, 1, 1, 2), bool), 0.4)
    np.testing.assert_allclose(out[0, 0, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], rtol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(s[0] + np.log1p(np.exp(s[1] - s[0])), rel=1e-13)


def test_fully_masked_rows_convention():
    q, k, v = _rand((1, 4, 2, 4), 19), _rand((1, 5, 2, 4), 20), _rand((1, 5, 2, 4), 21)
    mask = np.ones((1, 1, 4, 5), bool)
    mask[0, 0, 2] = False
    out, lse = A.attention_fwd(q, k, v, mask, 1.0)
    assert np.all(out[0, 2] == 0.0) and np.all(np.isneginf(lse[0, :, 2]))
    assert np.all(np.isfinite(lse[0, :, [0, 1, 3]]))


def test_lse_identity_and_masked_keys_do_not_matter():
    q, k, v = _rand((1, 8, 1, 6), 22), _rand((1, 10, 1, 6), 23), _rand((1, 10, 1, 6), 24)
    mask = np.random.default_rng(25).random((1, 1, 8, 10)) < 0.6
    mask[..., 9] = True
    out, lse = A.attention_fwd(q, k, v, mask, 0.5)
    s = 0.5 * (q[0, :, 0] @ k[0, :, 0].T)
    p = np.where(mask[0, 0], np.exp(s - lse[0, 0][:, None]), 0.0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(p @ v[0, :, 0], out[0, :, 0], rtol=1e-12, atol=1e-14)
    k2 = np.concatenate([k, 100 * _rand((1, 4, 1, 6), 26)], axis=1)
    v2 = np.concatenate([v, _rand((1, 4, 1, 6), 27)], axis=1)
    m2 = np.concatenate([mask, np.zeros((1, 1, 8, 4), bool)], axis=3)
    out2, lse2 = A.attention_fwd(q, k2, v2, m2, 0.5)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_row_sampling_matches_full():
    q, k, v = _rand((2, 30, 2, 4), 28), _rand((2, 30, 2, 4), 29), _rand((2, 30, 2, 4), 30)
    mask = np.random.default_rng(31).random((2, 2, 30, 30)) < 0.5
    out, lse = A.attention_fwd(q, k, v, mask, 0.5)
    rows = np.array([0, 7, 29])
    o2, l2 = A.attention_fwd(q, k, v, mask, 0.5, rows=rows, chunk=2)
    np.testing.assert_allclose(o2, out[:, rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, lse[:, :, rows], rtol=1e-13)


def test_varlen_equals_per_sequence():
    lengths = [5, 17, 1, 9]
    cu = M.cu_seqlens(lengths)
    T = int(cu[-1])
    q, k, v = _rand((T, 3, 4), 32), _rand((T, 3, 4), 33), _rand((T, 3, 4), 34)
    out, lse = A.varlen_attention_fwd(q, k, v, cu, cu, 0.5, True, 3, 0)
    for s, L in enumerate(lengths):
        sl = slice(cu[s], cu[s + 1])
        i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
        m = (j <= i) & (i - j < 4)
        o_s, l_s = A.attention_fwd(q[None, sl], k[None, sl], v[None, sl], m[None, None], 0.5)
        np.testing.assert_allclose(out[sl], o_s[0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[:, sl], l_s[0], rtol=1e-13)


def test_varlen_with_workload_recipe_small():
    w = W.varlen_window(nseq=3, lo=10, hi=40, H=2, D=8, window=8, seed=35, dtype=torch.float64)
    cu = M.cu_seqlens(w["lengths"])
    out, _ = A.varlen_attention_fwd(w["q"], w["k"], w["v"], cu, cu, w["scale"], True, 7, 0)
    m = M.varlen_mask(cu, cu, True, 7, 0)
    o2, _ = A.attention_fwd(w["q"][None], w["k"][None], w["v"][None], m[None, None], w["scale"])
    np.testing.assert_allclose(out, o2[0], rtol=1e-13, atol=1e-15)


# --- backward -----------------------------------------------------------------

def _loss(q, k, v, do, mask, scale):
    return float((A.attention_fwd(q, k, v, mask, scale)[0] * do).sum())


def test_backward_finite_differences():
    q, k, v = _rand((1, 5, 4, 3), 40), _rand((1, 6, 2, 3), 41), _rand((1, 6, 2, 3), 42)
    do = _rand((1, 5, 4, 3), 43)
    mask = np.random.default_rng(44).random((1, 2, 5, 6)) < 0.6
    mask[0, 0, 1] = False  # an empty row in one head group
    dq, dk, dv, out, lse, delta = A.attention_bwd(q, k, v, do, mask, 0.6)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (_loss(*args_p, do, mask, 0.6) - _loss(*args_m, do, mask, 0.6)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(delta, np.einsum("bshd,bshd->bhs", do, out), rtol=1e-12, atol=1e-14)
    assert np.all(dq[0, 1, :2] == 0.0)  # heads 0, 1 share mask head 0, whose row 1 is empty


def test_backward_equals_torch_autograd_sdpa():
    rng = np.random.default_rng(45)
    q, k, v = _rand((2, 24, 4, 8), 46), _rand((2, 30, 2, 8), 47), _rand((2, 30, 2, 8), 48)
    do = _rand((2, 24, 4, 8), 49)
    mask = rng.random((2, 1, 24, 30)) < 0.4
    mask[..., 5] = True
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.35)
    t = [torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v)]
    o = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(mask), scale=0.35, enable_gqa=True)
    o.backward(torch.from_numpy(do.transpose(0, 2, 1, 3).copy()))
    for g, tt in zip((dq, dk, dv), t):
        np.testing.assert_allclose(g, tt.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)


def test_sampled_backward_equals_dense_backward():
    rng = np.random.default_rng(50)
    B, Sq, Sk, Hq, Hkv, D = 2, 40, 36, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, D), 51), _rand((B, Sk, Hkv, D), 52), _rand((B, Sk, Hkv, D), 53)
    do = _rand((B, Sq, Hq, D), 54)
    mask = rng.random((B, Hkv, Sq, Sk)) < 0.5
    mask[:, :, 7] = False  # empty rows
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.3)

    def allowed(b, hm, rr):
        return mask[b, hm][rr]
    allowed.heads = Hkv
    rows, cols = np.array([0, 7, 39]), np.array([1, 17, 35])
    for b in range(B):
        for hk in range(Hkv):
            sq, sk, sv = A.attention_bwd_sampled(q, k, v, do, allowed, 0.3, b, hk, rows, cols, chunk=16)
            np.testing.assert_allclose(sq, dq[b][rows][:, hk * 2:hk * 2 + 2].transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(sk, dk[b, cols, hk], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(sv, dv[b, cols, hk], rtol=1e-10, atol=1e-12)


def test_dq_rows_equal_torch_autograd():
    """Row-local dQ against torch autograd through float64 SDPA (a library
    routine), with GQA, empty rows and a row subset."""
    rng = np.random.default_rng(55)
    B, Sq, Sk, Hq, Hkv, D = 2, 30, 26, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, D), 56), _rand((B, Sk, Hkv, D), 57), _rand((B, Sk, Hkv, D), 58)
    do = _rand((B, Sq, Hq, D), 59)
    mask = rng.random((B, 1, Sq, Sk)) < 0.4
    mask[:, :, 3] = False  # empty rows: SDPA gives NaN there, the convention gives 0
    t = [torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v)]
    o = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(mask), scale=0.45, enable_gqa=True)
    g = torch.from_numpy(do.transpose(0, 2, 1, 3).copy())
    g[:, :, 3] = 0.0
    o = torch.where(torch.from_numpy(mask.any(-1, keepdims=True)), o, torch.zeros_like(o))
    o.backward(g)
    ref = t[0].grad.numpy().transpose(0, 2, 1, 3)
    rows = np.array([0, 3, 7, 29])
    got = A.attention_bwd_dq_rows(q, k, v, do, mask, 0.45, rows)
    np.testing.assert_allclose(got, ref[:, rows], rtol=1e-11, atol=1e-12)
    assert np.all(got[:, 1] == 0.0)


# --- score_mod (tensorplay omni_attention, intro) -------------------------------------

def _small_qkv(seed, B=1, S=40, H=2, D=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, H, D)), rng.standard_normal((B, S, H, D)),
            rng.standard_normal((B, S, H, D)), rng.standard_normal((B, S, H, D)))


def test_score_mod_row_bias_only_shifts_lse():
    """A term that depends on the query row only cancels in the softmax: the
    output is unchanged and the log-sum-exp moves by exactly that term. An
    implementation that applied the term along the key axis would change the
    output."""
    q, k, v, _ = _small_qkv(1)
    allowed = np.tril(np.ones((40, 40), bool))[None, None]
    mod = lambda s, b, h, qi, kj: s + 0.37 * qi + 0.0 * kj  # noqa: E731
    o0, l0 = A.attention_fwd(q, k, v, allowed, 0.25)
    o1, l1 = A.attention_fwd(q, k, v, allowed, 0.25, score_mod=mod)
    assert np.allclose(o1, o0, atol=1e-12)
    assert np.allclose(l1 - l0, 0.37 * np.arange(40)[None, None, :], atol=1e-12)


def test_alibi_equals_an_extra_key_feature():
    """ALiBi by construction without score_mod: slope*(kv - q) = slope*kv - slope*q;
    the kv part is an extra dimension (q' = [q, slope/scale], k' = [k, kv_idx]) and
    the q part is a row constant. So outputs and dQ, dK (first D columns), dV
    equal plain attention on the augmented inputs, and LSE differs by slope*q."""
    q, k, v, do = _small_qkv(2, S=33)
    slopes = np.array([0.5, 1.0])
    scale = 0.3
    allowed = np.tril(np.ones((33, 33), bool))[None, None]
    B, S, H, D = q.shape
    qa = np.concatenate([q, np.broadcast_to((slopes / scale)[None, None, :, None], (B, S, H, 1))], axis=3)
    ka = np.concatenate([k, np.broadcast_to(np.arange(S, dtype=float)[None, :, None, None], (B, S, H, 1))], axis=3)
    o_ref, l_ref = A.attention_fwd(qa, ka, v, allowed, scale)
    o, l = A.attention_fwd(q, k, v, allowed, scale, score_mod=A.alibi(slopes))
    assert np.allclose(o, o_ref, atol=1e-12)
    assert np.allclose(l, l_ref - slopes[None, :, None] * np.arange(S)[None, None, :], atol=1e-10)
    g = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=A.alibi(slopes))
    ga = A.attention_bwd(qa, ka, v, do, allowed, scale)
    assert np.allclose(g[0], ga[0][..., :D], atol=1e-10)
    assert np.allclose(g[1], ga[1][..., :D], atol=1e-10)
    assert np.allclose(g[2], ga[2], atol=1e-10)


def test_alibi_large_slope_picks_the_nearest_allowed_key():
    """With a large positive slope the latest allowed key dominates: under a
    causal mask row i attends to key i alone (output -> v_i, LSE -> scale q.k_i)."""
    q, k, v, _ = _small_qkv(3, S=20)
    allowed = np.tril(np.ones((20, 20), bool))[None, None]
    o, l = A.attention_fwd(q, k, v, allowed, 0.2, score_mod=A.alibi([200.0, 200.0]))
    assert np.allclose(o, v, atol=1e-9)
    want = 0.2 * np.einsum("bshd,bshd->bhs", q, k)
    assert np.allclose(l, want, atol=1e-9)


def test_alibi_equals_sdpa_with_an_additive_float_mask():
    """torch's SDPA adds a float attn_mask to the scaled scores; the ALiBi term
    slope[h] * (j - i) plus -inf on disallowed entries must give the same
    output and gradients (GQA, ragged Sq != Sk)."""
    rng = np.random.default_rng(60)
    B, Sq, Sk, Hq, Hkv, D = 2, 21, 30, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, D), 61), _rand((B, Sk, Hkv, D), 62), _rand((B, Sk, Hkv, D), 63)
    do = _rand((B, Sq, Hq, D), 64)
    mask = rng.random((B, 1, Sq, Sk)) < 0.5
    mask[..., 3] = True
    slopes = np.array([0.25, -0.5, 1.0, 0.0625])
    mod = A.alibi(slopes)
    out, _ = A.attention_fwd(q, k, v, mask, 0.4, score_mod=mod)
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.4, score_mod=mod)
    bias = slopes[None, :, None, None] * (np.arange(Sk)[None, :] - np.arange(Sq)[:, None])[None, None]
    fmask = np.where(mask, bias, -np.inf)
    t = [torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v)]
    o = F.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(fmask), scale=0.4, enable_gqa=True)
    np.testing.assert_allclose(out, o.detach().numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    o.backward(torch.from_numpy(do.transpose(0, 2, 1, 3).copy()))
    for g, tt in zip((dq, dk, dv), t):
        np.testing.assert_allclose(g, tt.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)


def test_score_mod_sampled_and_varlen_agree_with_dense():
    rng = np.random.default_rng(70)
    B, S, Hq, Hkv, D = 1, 36, 4, 2, 8
    q, k, v = _rand((B, S, Hq, D), 71), _rand((B, S, Hkv, D), 72), _rand((B, S, Hkv, D), 73)
    do = _rand((B, S, Hq, D), 74)
    mask = np.tril(np.ones((S, S), bool))[None, None] & (rng.random((1, 1, S, S)) < 0.7)
    mod = A.alibi([0.5, 1.0, 2.0, 0.125])
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.3, score_mod=mod)

    def allowed(b, hm, rr):
        return mask[0, 0][rr]
    allowed.heads = 1
    rows, cols = np.array([0, 9, 35]), np.array([0, 20, 35])
    for hk in range(Hkv):
        sq, sk, sv = A.attention_bwd_sampled(q, k, v, do, allowed, 0.3, 0, hk, rows, cols, chunk=8, score_mod=mod)
        np.testing.assert_allclose(sq, dq[0][rows][:, hk * 2:hk * 2 + 2].transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sk, dk[0, cols, hk], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sv, dv[0, cols, hk], rtol=1e-10, atol=1e-12)
    # varlen: the bias uses positions local to each sequence
    lengths = [7, 1, 12]
    cu = M.cu_seqlens(lengths)
    T = int(cu[-1])
    qv, kv, vv = _rand((T, 2, 4), 75), _rand((T, 2, 4), 76), _rand((T, 2, 4), 77)
    mod2 = A.alibi([0.75, 1.5])
    out, lse = A.varlen_attention_fwd(qv, kv, vv, cu, cu, 0.5, True, -1, 0, score_mod=mod2)
    for s, L in enumerate(lengths):
        sl = slice(cu[s], cu[s + 1])
        m = np.tril(np.ones((L, L), bool))
        o_s, l_s = A.attention_fwd(qv[None, sl], kv[None, sl], vv[None, sl], m[None, None], 0.5, score_mod=mod2)
        np.testing.assert_allclose(out[sl], o_s[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[:, sl], l_s[0], rtol=1e-12)


def test_term_sums_bound_the_gradients():
    """The rounding magnitudes bound each gradient (|sum| <= sum |.|, and
    |dS_ij| <= E_ij), with equality for dV where every term has one sign (a
    single allowed key per row makes dS zero and dV_j = sum_i |dO_i| when
    dO > 0)."""
    q, k, v = _rand((1, 12, 2, 4), 80), _rand((1, 12, 2, 4), 81), _rand((1, 12, 2, 4), 82)
    do = _rand((1, 12, 2, 4), 83)
    mask = np.random.default_rng(84).random((1, 1, 12, 12)) < 0.5
    r = A.attention_bwd(q, k, v, do, mask, 0.5, score_mod=A.alibi([0.5, 2.0]), term_sums=True)
    for g, t in zip(r[:3], r[6]):
        assert np.all(np.abs(g) <= t + 1e-12)
    eye = np.eye(12, dtype=bool)[None, None]
    pos = np.abs(do)
    dq, dk, dv, *_, (tq, tk, tv) = A.attention_bwd(q, k, v, pos, eye, 0.5, term_sums=True)
    np.testing.assert_allclose(dv, tv, rtol=1e-13)
    np.testing.assert_allclose(dv, pos, rtol=1e-13)
    assert np.all(dq == 0) and np.all(dk == 0)
    # E_ii = |dP_ii| + |Delta_i| + B_i with B_i = sum|dO_i||v_i| + |dP_ii|
    dP = np.einsum("bshd,bshd->bsh", pos, v)
    B_ = np.einsum("bshd,bshd->bsh", pos, np.abs(v)) + np.abs(dP)
    E = 2 * np.abs(dP) + B_
    np.testing.assert_allclose(tq, 0.5 * E[..., None] * np.abs(k), rtol=1e-12)


# --- soft cap score_mod -----------------------------------------------------------------------

def _torch_softcap_attention(q, k, v, mask, scale, cap, slopes=None):
    """Independent torch float64 reference: scores scale q.k (+ slope (j - i)),
    then cap * tanh(. / cap), then the mask, softmax and the value sum; GQA
    by repeating k / v heads. Inputs numpy (B, S, H, D); returns tensors with
    requires_grad for q, k, v and the output (B, H, Sq, D)."""
    G = q.shape[2] // k.shape[2]
    t = [torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v)]
    kk = t[1].repeat_interleave(G, dim=1)
    vv = t[2].repeat_interleave(G, dim=1)
    s = scale * (t[0] @ kk.transpose(-1, -2))
    if slopes is not None:
        Sq, Sk = q.shape[1], k.shape[1]
        pos = torch.arange(Sk, dtype=torch.float64)[None, :] - torch.arange(Sq, dtype=torch.float64)[:, None]
        s = s + torch.tensor(slopes)[None, :, None, None] * pos
    s = cap * torch.tanh(s / cap)
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    return t, o


@pytest.mark.parametrize("with_alibi", [False, True])
def test_softcap_equals_torch_autograd(with_alibi):
    rng = np.random.default_rng(80)
    B, Sq, Sk, Hq, Hkv, D = 2, 19, 27, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, D), 81) * 2.0, _rand((B, Sk, Hkv, D), 82) * 2.0, _rand((B, Sk, Hkv, D), 83)
    do = _rand((B, Sq, Hq, D), 84)
    mask = rng.random((B, 1, Sq, Sk)) < 0.6
    mask[..., 2] = True
    slopes = np.array([0.25, -0.5, 1.0, 0.0625]) if with_alibi else None
    mod = A.softcap(1.5, A.alibi(slopes) if with_alibi else None)
    out, lse = A.attention_fwd(q, k, v, mask, 0.7, score_mod=mod)
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.7, score_mod=mod)
    t, o = _torch_softcap_attention(q, k, v, np.ascontiguousarray(np.broadcast_to(mask, (B, Hq, Sq, Sk))), 0.7, 1.5,
                                    slopes)
    np.testing.assert_allclose(out, o.detach().numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    o.backward(torch.from_numpy(do.transpose(0, 2, 1, 3).copy()))
    for g, tt in zip((dq, dk, dv), t):
        np.testing.assert_allclose(g, tt.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)


def test_softcap_finite_differences_and_limits():
    q, k, v = _rand((1, 4, 2, 3), 85) * 3.0, _rand((1, 5, 1, 3), 86) * 3.0, _rand((1, 5, 1, 3), 87)
    do = _rand((1, 4, 2, 3), 88)
    mask = np.random.default_rng(89).random((1, 1, 4, 5)) < 0.7
    mask[..., 0] = True
    mod = A.softcap(0.8)
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.5, score_mod=mod)

    def loss(qq, kk, vv):
        o, _ = A.attention_fwd(qq, kk, vv, mask, 0.5, score_mod=mod)
        return float((o * do).sum())
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (loss(*[xp if y is x else y for y in (q, k, v)]) -
                        loss(*[xm if y is x else y for y in (q, k, v)])) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)
    # a cap far above every score changes nothing; a tiny cap flattens the
    # weights to the plain mean of the allowed values
    o_big, l_big = A.attention_fwd(q, k, v, mask, 0.5, score_mod=A.softcap(1e9))
    o_ref, l_ref = A.attention_fwd(q, k, v, mask, 0.5)
    np.testing.assert_allclose(o_big, o_ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(l_big, l_ref, rtol=1e-9, atol=1e-12)
    o_small, _ = A.attention_fwd(q, k, v, mask, 0.5, score_mod=A.softcap(1e-9))
    for hq in range(2):
        for i in range(4):
            m = mask[0, 0, i]
            np.testing.assert_allclose(o_small[0, i, hq], v[0, m, 0].mean(axis=0), rtol=1e-7, atol=1e-8)


def test_softcap_sampled_and_row_backward_agree_with_dense():
    rng = np.random.default_rng(90)
    B, S, Hq, Hkv, D = 1, 33, 4, 2, 8
    q, k, v = _rand((B, S, Hq, D), 91) * 2.0, _rand((B, S, Hkv, D), 92) * 2.0, _rand((B, S, Hkv, D), 93)
    do = _rand((B, S, Hq, D), 94)
    mask = np.tril(np.ones((S, S), bool))[None, None] & (rng.random((1, 1, S, S)) < 0.8)
    mask[..., 0] = True
    mod = A.softcap(2.0, A.alibi([0.5, 1.0, 0.25, 0.125]))
    dq, dk, dv, *_ = A.attention_bwd(q, k, v, do, mask, 0.3, score_mod=mod)

    def allowed(b, hm, rr):
        return mask[0, 0][rr]
    allowed.heads = 1
    rows, cols = np.array([0, 7, 32]), np.array([0, 16, 32])
    for hk in range(Hkv):
        sq, sk, sv = A.attention_bwd_sampled(q, k, v, do, allowed, 0.3, 0, hk, rows, cols, chunk=8, score_mod=mod)
        np.testing.assert_allclose(sq, dq[0][rows][:, hk * 2:hk * 2 + 2].transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sk, dk[0, cols, hk], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sv, dv[0, cols, hk], rtol=1e-10, atol=1e-12)
    rq = A.attention_bwd_dq_rows(q, k, v, do, allowed, 0.3, rows, score_mod=mod)
    np.testing.assert_allclose(rq[0], dq[0][rows], rtol=1e-10, atol=1e-12)
