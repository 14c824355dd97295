"""Features used together: the positional bias with varlen seqused_k and
paged k / v, with BSR token validity, with 64-row dense-mask tiles and with
predicate tile maps, forward and backward against the oracle (bounds as in
the single-feature tests)."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, DEV, F32_OUT_TOL, compare_attention, f64, grad_tolerance_terms, note,
                            to_dev)

pytestmark = pytest.mark.gpu


def _slopes(H, mult=1.0):
    return (mult * 2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def _check(got, r, tag):
    for name, g, ref, t in zip(("dq", "dk", "dv"), got, r[:3], r[6]):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite"
        ex = np.abs(g - ref) - grad_tolerance_terms(ref, t)
        i = np.unravel_index(int(np.argmax(ex)), ex.shape)
        assert ex[i] <= 0, f"{tag} {name}: |{g[i]:.5f} - {ref[i]:.5f}| over the bound at {i}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_alibi_varlen_seqused_paged(dtype):
    note(f"combo alibi+varlen seqused paged {dtype}")
    Lq = np.array([64, 1, 200, 130, 0, 77], np.int32)
    Lk = np.array([64, 30, 256, 129, 9, 200], np.int32)
    used = np.array([64, 7, 180, 129, 9, 0], np.int32)
    Tq, Tk = int(Lq.sum()), int(Lk.sum())
    H, D, page = 4, 64, 128
    q, k, v = W.tensors(120, [(Tq, H, D), (Tk, 2, D), (Tk, 2, D)])
    npg = [(int(L) + page - 1) // page for L in Lk]
    n_pages = sum(npg) + 2
    perm = np.random.default_rng(121).permutation(n_pages)
    kp = torch.zeros(n_pages, page, 2, D, dtype=k.dtype)
    vp = torch.zeros_like(kp)
    table = np.zeros((Lk.size, max(npg)), np.int32)
    nxt, off = 0, 0
    for s, L in enumerate(Lk):
        for pi in range(npg[s]):
            table[s, pi] = perm[nxt]
            nxt += 1
        for j in range(int(L)):
            kp[table[s, j // page], j % page] = k[off + j]
            vp[table[s, j // page], j % page] = v[off + j]
        off += int(L)
    sl = _slopes(H, 4.0)
    sch = mfa.varlen_schedule(to_dev(Lq), to_dev(Lk), causal=True, window=(100, 0), work_cap=Tq // 128 + Lq.size)
    rep = mfa.MaskRep.varlen(sch, int(Lq.max()), int(Lk.max()), causal=True, window=(100, 0),
                             seqused_k=to_dev(used), block_table=to_dev(table), page_size=page, n_pages=n_pages)
    out, lse = mfa.attn_fwd(to_dev(q, dtype), to_dev(kp, dtype), to_dev(vp, dtype), rep, 0.125, "thd",
                            alibi_slopes=torch.tensor(sl, device=DEV))
    torch.cuda.synchronize()
    ro, rl = A.varlen_attention_fwd(q, k, v, M.cu_seqlens(Lq), M.cu_seqlens(Lk), 0.125, True, 100, 0,
                                    score_mod=A.alibi(sl), seqused_k=used)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL)


def test_alibi_bsr_kv_valid_forward_backward():
    note("combo alibi+bsr kv_valid")
    N, H, D = 700, 2, 128
    w = W.bsr_random(B=2, N=N, H=H, D=D, block=64, frac_den=2, seed=122)
    ip, ix = w["indptr"], w["indices"]
    rng = np.random.default_rng(123)
    valid = rng.random((2, N)) < 0.75
    bits_d = to_dev(M.pack_bits_rows(valid).view(np.int32))
    kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, True, kv_valid_bits=bits_d)
    rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=True, csc_ptr=cp, csc_idx=ci, kv_valid_bits=bits_d)
    sl = _slopes(H)
    slopes = torch.tensor(sl, device=DEV)
    do = W.tensors(124, [tuple(w["q"].shape)])[0]
    qd, kd, vd, dod = (to_dev(t) for t in (w["q"], w["k"], w["v"], do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "bshd", alibi_slopes=slopes)
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, w["scale"], "bshd", alibi_slopes=slopes)
    torch.cuda.synchronize()
    allowed = M.bsr_mask(ip, ix, 64, 64, N, N, True, kv_valid=valid)
    ro, rl = A.attention_fwd(w["q"], w["k"], w["v"], allowed, w["scale"], score_mod=A.alibi(sl))
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)
    r = A.attention_bwd(w["q"], w["k"], w["v"], do, allowed, w["scale"], score_mod=A.alibi(sl), term_sums=True)
    _check(got, r, "alibi bsr kv_valid")


@pytest.mark.parametrize("src", ["dense64", "predicate"])
def test_alibi_on_64_row_and_predicate_maps(src):
    note(f"combo alibi on {src} map")
    Sq = Sk = 333
    H, D = 4, 128
    if src == "dense64":
        mask = W.random_dense_mask(Sq, Sk, 0.4, 125) | np.eye(Sq, dtype=bool)
        rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask), BM=64))
    else:
        gp = mfa.Pred.causal().and_(mfa.Pred.past_window(77)).or_(mfa.Pred.prefix(5))
        mask = M.create_mask(M.or_masks(M.and_masks(M.causal, M.past_window(77)), lambda b, h, qi, kj: kj < 5),
                             1, 1, Sq, Sk)[0, 0]
        rep = mfa.MaskRep.tiles(mfa.predicate_tiles(gp, Sq, Sk))
    q, k, v, do = W.tensors(126, [(2, Sq, H, D), (2, Sk, 2, D), (2, Sk, 2, D), (2, Sq, H, D)])
    sl = _slopes(H)
    slopes = torch.tensor(sl, device=DEV)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, D ** -0.5, "bshd", alibi_slopes=slopes)
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, D ** -0.5, "bshd", alibi_slopes=slopes)
    torch.cuda.synchronize()
    ro, rl = A.attention_fwd(q, k, v, mask[None, None], D ** -0.5, score_mod=A.alibi(sl))
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)
    r = A.attention_bwd(q, k, v, do, mask[None, None], D ** -0.5, score_mod=A.alibi(sl), term_sums=True)
    _check(got, r, f"alibi {src}")
