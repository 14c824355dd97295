"""Alternate inputs to the same attention loop: BSR token validity
(kv_valid_bits) and the bitmask sparse format (exact_block_bits) of flashinfer
block_sparse_attention (Parameters), and seqused_k and paged k / v
(block_table) of tensorplay varlen (intro). Mask-side outputs must be
bit-exact against the oracle; attention within the usual bounds (bf16 out
2e-2, LSE 1e-3, fp32 test mode 1e-4, gradients 2e-2 + one bf16 ULP)."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, DEV, F32_OUT_TOL, compare_attention, f64, grad_tolerance, nan_like,
                            note, to_dev)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def _tol(dtype):
    return BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL


def _check_grads(got, ref, tag):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite gradient"
        excess = np.abs(g - r) - grad_tolerance(r)
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        assert excess[i] <= 0, f"{tag} {name}: |{g[i]:.5f} - {r[i]:.5f}| over the bound at {i}"


# --- BSR with kv_valid_bits ------------------------------------------------------------

def _valid(B, N, seed):
    rng = np.random.default_rng(seed)
    v = rng.random((B, N)) < 0.8
    v[0, 128:192] = False          # a whole 64-key block invalid
    v[-1, N - 40:] = False         # invalid tail
    return v


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_bsr_kv_valid_bits(D, causal):
    note(f"bsr kv_valid D={D} causal={causal}")
    N, H = 1000, 3
    w = W.bsr_random(B=2, N=N, H=H, D=D, block=64, frac_den=3, seed=30 + D + causal)
    ip, ix = w["indptr"], w["indices"]
    valid = _valid(2, N, 31)
    bits = M.pack_bits_rows(valid)
    bits_d = to_dev(bits.view(np.int32))
    kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, causal, kv_valid_bits=bits_d)
    torch.cuda.synchronize()
    want = M.bsr_col_kind(ip, ix, 64, 64, N, N, causal, kv_valid=valid)
    assert np.array_equal(_np(kind), want)
    rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=causal, csc_ptr=cp, csc_idx=ci,
                          kv_valid_bits=bits_d)
    allowed = M.bsr_mask(ip, ix, 64, 64, N, N, causal, kv_valid=valid)
    do = W.tensors(905, [tuple(w["q"].shape)])[0]
    for dtype in (torch.bfloat16, torch.float32):
        qd, kd, vd = (to_dev(w[x], dtype) for x in "qkv")
        out, lse = mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "bshd")
        torch.cuda.synchronize()
        ro, rl = A.attention_fwd(w["q"], w["k"], w["v"], allowed, w["scale"])
        compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))
    qd, kd, vd, dod = (to_dev(t) for t in (w["q"], w["k"], w["v"], do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, w["scale"], "bshd")
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, w["scale"], "bshd")
    torch.cuda.synchronize()
    ref = A.attention_bwd(w["q"], w["k"], w["v"], do, allowed, w["scale"])[:3]
    _check_grads(got, ref, "bsr kv_valid")
    # invalid keys get exactly zero dK / dV
    inv = ~valid
    assert np.all(f64(got[1])[inv] == 0) and np.all(f64(got[2])[inv] == 0)


# --- bitmask sparse format -------------------------------------------------------------

@pytest.mark.parametrize("nKb", [16, 40, 70])
def test_bitmask_to_bsr_bit_exact_and_attention(nKb):
    note(f"bitmask -> bsr nKb={nKb}")
    rng = np.random.default_rng(40 + nKb)
    B, H, N = 2, 2, 64 * nKb - 17
    R = (N + 63) // 64
    sel = rng.random((B, H, R, nKb)) < 0.25
    sel[:, :, np.arange(R), np.arange(R)] = True
    sel[0, 1, 3] = False
    Wd = (nKb + 31) // 32
    bits = np.zeros((B, H, R, Wd), np.uint32)
    for b, h, r, c in zip(*np.nonzero(sel)):
        bits[b, h, r, c // 32] |= np.uint32(1 << (c % 32))
    bits[:, :, :, -1] |= np.uint32(0xFFFFFFFF) << np.uint32(nKb % 32) if nKb % 32 else np.uint32(0)  # junk past nKb
    ip_d, ix_d = mfa.bsr_from_bitmask(to_dev(bits.view(np.int32)), nKb)
    torch.cuda.synchronize()
    ip, ix = M.bsr_from_bitmask(bits, nKb)
    nnz = int(ip[-1, -1, -1])
    assert np.array_equal(_np(ip_d), ip) and np.array_equal(_np(ix_d)[:nnz], ix)
    assert mfa.bsr_validate(ip_d, ix_d[:nnz], nKb) == int(sel.sum(axis=3).max())
    q, k, v = W.tensors(41, [(B, N, H, 64)] * 3)
    kind, _, _ = mfa.bsr_prepare(ip_d, ix_d[:nnz], 64, 64, N, N, False)
    rep = mfa.MaskRep.bsr(ip_d, ix_d[:nnz], kind, causal=False)
    out, lse = mfa.attn_fwd(*(to_dev(t) for t in (q, k, v)), rep, 0.125, "bshd")
    torch.cuda.synchronize()
    ro, rl = A.attention_fwd(q, k, v, M.bsr_mask(ip, ix, 64, 64, N, N, False), 0.125)
    compare_attention(f64(out), f64(lse), ro, rl, BF16_OUT_TOL)


# --- varlen seqused_k ---------------------------------------------------------------------

L_Q = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
L_K = np.array([3, 128, 200, 5, 300, 70, 64, 250], np.int32)
USED = np.array([3, 0, 150, 5, 257, -4, 64, 1], np.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal,win", [(False, (-1, -1)), (True, (100, 0)), (False, (50, 30))])
def test_varlen_seqused_k_forward(causal, win, dtype):
    note(f"varlen seqused fwd causal={causal} win={win} {dtype}")
    Tq, Tk = int(L_Q.sum()), int(L_K.sum())
    q, k, v = W.tensors(50, [(Tq, 4, 64), (Tk, 2, 64), (Tk, 2, 64)])
    s = mfa.varlen_schedule(to_dev(L_Q), to_dev(L_K), causal=causal, window=win, work_cap=Tq // 128 + L_Q.size)
    rep = mfa.MaskRep.varlen(s, int(L_Q.max()), int(L_K.max()), causal=causal, window=win,
                             seqused_k=to_dev(USED))
    qd, kd, vd = (to_dev(t, dtype) for t in (q, k, v))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, 0.125, "thd")
    torch.cuda.synchronize()
    ro, rl = A.varlen_attention_fwd(q, k, v, M.cu_seqlens(L_Q), M.cu_seqlens(L_K), 0.125, causal, win[0], win[1],
                                    seqused_k=USED)
    compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))


@pytest.mark.parametrize("causal,win", [(False, (-1, -1)), (True, (100, 0))])
def test_varlen_seqused_k_backward(causal, win):
    note(f"varlen seqused bwd causal={causal} win={win}")
    Tq, Tk = int(L_Q.sum()), int(L_K.sum())
    q, k, v, do = W.tensors(51, [(Tq, 4, 64), (Tk, 2, 64), (Tk, 2, 64), (Tq, 4, 64)])
    s = mfa.varlen_schedule(to_dev(L_Q), to_dev(L_K), causal=causal, window=win, work_cap=Tq // 128 + L_Q.size)
    rep = mfa.MaskRep.varlen(s, int(L_Q.max()), int(L_K.max()), causal=causal, window=win,
                             seqused_k=to_dev(USED))
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, 0.125, "thd")
    dq, dk, dv = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, 0.125, "thd")
    torch.cuda.synchronize()
    allowed = M.varlen_mask(M.cu_seqlens(L_Q), M.cu_seqlens(L_K), causal, win[0], win[1], seqused_k=USED)
    ref = A.attention_bwd(q[None], k[None], v[None], do[None], allowed[None, None], 0.125)[:3]
    _check_grads([dq, dk, dv], [r[0] for r in ref], "seqused")
    unused = ~allowed.any(axis=0)
    assert unused.sum() > 100
    assert np.all(f64(dk)[unused] == 0) and np.all(f64(dv)[unused] == 0)


# --- varlen with paged k / v ----------------------------------------------------------------

def _paged(k, v, lengths, page, seed, spare=3):
    """Scatter packed k / v into shuffled pages; returns (k_pages, v_pages, table, n_pages)."""
    rng = np.random.default_rng(seed)
    npg = [(int(L) + page - 1) // page for L in lengths]
    n_pages = sum(npg) + spare
    perm = rng.permutation(n_pages)
    H, D = k.shape[1], k.shape[2]
    kp = torch.zeros(n_pages, page, H, D, dtype=k.dtype)
    vp = torch.zeros(n_pages, page, H, D, dtype=v.dtype)
    table = np.full((len(lengths), max(max(npg), 1) + 1), -7, np.int32)
    nxt, off = 0, 0
    for s_, L in enumerate(lengths):
        for pi in range(npg[s_]):
            table[s_, pi] = perm[nxt]
            nxt += 1
        for j in range(int(L)):
            kp[table[s_, j // page], j % page] = k[off + j]
            vp[table[s_, j // page], j % page] = v[off + j]
        off += int(L)
    return kp, vp, table, n_pages


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("page", [64, 128])
@pytest.mark.parametrize("causal,win", [(False, (-1, -1)), (True, (100, 0))])
def test_varlen_paged_forward(page, causal, win, dtype):
    note(f"varlen paged page={page} causal={causal} win={win} {dtype}")
    Tq, Tk = int(L_Q.sum()), int(L_K.sum())
    q, k, v = W.tensors(52, [(Tq, 4, 64), (Tk, 2, 64), (Tk, 2, 64)])
    kp, vp, table, n_pages = _paged(k, v, L_K, page, seed=page)
    assert np.array_equal(M.paged_to_packed(f64(kp), table, L_K, page), f64(k))
    s = mfa.varlen_schedule(to_dev(L_Q), to_dev(L_K), causal=causal, window=win, work_cap=Tq // 128 + L_Q.size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rep = mfa.MaskRep.varlen(s, int(L_Q.max()), int(L_K.max()), causal=causal, window=win, err=err,
                             seqused_k=to_dev(USED), block_table=to_dev(table), page_size=page, n_pages=n_pages)
    qd, kd, vd = to_dev(q, dtype), to_dev(kp, dtype), to_dev(vp, dtype)
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, 0.125, "thd")
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ro, rl = A.varlen_attention_fwd(q, k, v, M.cu_seqlens(L_Q), M.cu_seqlens(L_K), 0.125, causal, win[0], win[1],
                                    seqused_k=USED)
    compare_attention(f64(out), f64(lse), ro, rl, _tol(dtype))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("page", [64, 128])
@pytest.mark.parametrize("causal,win", [(False, (-1, -1)), (True, (100, 0))])
def test_varlen_paged_backward(page, causal, win, dtype):
    """Backward over paged k / v (with seqused_k): dq equals the packed run's
    bit for bit, and dk / dv, read back through the table, equal the packed
    run's rows (keys past the used length zero); rows of the spare pages stay
    as they were (NaN). fp32 is also checked against the oracle at 1e-4."""
    note(f"varlen paged bwd page={page} causal={causal} win={win} {dtype}")
    Tq, Tk = int(L_Q.sum()), int(L_K.sum())
    q, k, v, do = W.tensors(54, [(Tq, 4, 64), (Tk, 2, 64), (Tk, 2, 64), (Tq, 4, 64)])
    kp, vp, table, n_pages = _paged(k, v, L_K, page, seed=page + 11)
    s = mfa.varlen_schedule(to_dev(L_Q), to_dev(L_K), causal=causal, window=win, work_cap=Tq // 128 + L_Q.size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    common = dict(causal=causal, window=win, err=err, seqused_k=to_dev(USED))
    rep_p = mfa.MaskRep.varlen(s, int(L_Q.max()), int(L_K.max()), block_table=to_dev(table), page_size=page,
                               n_pages=n_pages, **common)
    rep_c = mfa.MaskRep.varlen(s, int(L_Q.max()), int(L_K.max()), **common)
    qd, dod = to_dev(q, dtype), to_dev(do, dtype)
    runs = {}
    for name, kk, vv, rep in (("paged", kp, vp, rep_p), ("packed", k, v, rep_c)):
        kd, vd = to_dev(kk, dtype), to_dev(vv, dtype)
        out, lse = mfa.attn_fwd(qd, kd, vd, rep, 0.125, "thd")
        g = (nan_like(qd), nan_like(kd), nan_like(vd))
        mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, 0.125, "thd", dq=g[0], dk=g[1], dv=g[2])
        torch.cuda.synchronize()
        runs[name] = [x.cpu() for x in g]
    assert int(err.item()) == 0
    (dq_p, dk_p, dv_p), (dq_c, dk_c, dv_c) = runs["paged"], runs["packed"]
    bits = (lambda t: t.view(torch.int16)) if dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(dq_p), bits(dq_c))
    used_pages = set()
    off = 0
    for s_, Lk in enumerate(L_K.tolist()):
        for j in range(Lk):
            pg, r = int(table[s_, j // page]), j % page
            used_pages.add(pg)
            assert torch.equal(bits(dk_p[pg, r]), bits(dk_c[off + j])), (s_, j)
            assert torch.equal(bits(dv_p[pg, r]), bits(dv_c[off + j])), (s_, j)
        off += Lk
    spare = [pg for pg in range(n_pages) if pg not in used_pages]
    assert spare and torch.isnan(dk_p[spare].float()).all() and torch.isnan(dv_p[spare].float()).all()
    if dtype == torch.float32:
        allowed = M.varlen_mask(M.cu_seqlens(L_Q), M.cu_seqlens(L_K), causal, win[0], win[1], seqused_k=USED)
        ref = A.attention_bwd(q[None], k[None], v[None], do[None], allowed[None, None], 0.125)
        for name, got, r in (("dq", dq_c, ref[0][0]), ("dk", dk_c, ref[1][0]), ("dv", dv_c, ref[2][0])):
            e = float(np.abs(got.double().numpy() - r).max())
            assert e <= F32_OUT_TOL, f"{name} max-abs {e:.2e}"


def test_varlen_paged_bad_table_is_an_error():
    """A page id outside the pool, or a sequence longer than its table row,
    gives NaN rows for that sequence and sets the error word; the other
    sequences are computed normally."""
    note("varlen paged bad table")
    L = np.array([100, 200, 70], np.int32)
    T = int(L.sum())
    q, k, v = W.tensors(53, [(T, 2, 64)] * 3)
    kp, vp, table, n_pages = _paged(k, v, L, 64, seed=5)
    table[1, 2] = n_pages + 4                      # sequence 1: bad page id
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=(-1, -1), work_cap=T // 128 + L.size)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rep = mfa.MaskRep.varlen(s, 200, 200, causal=True, err=err, block_table=to_dev(table[:, :3]), page_size=64,
                             n_pages=n_pages)      # max_pages 3: sequence 1 needs 4 pages
    out, lse = mfa.attn_fwd(to_dev(q), to_dev(kp), to_dev(vp), rep, 0.125, "thd")
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    cu = M.cu_seqlens(L)
    o = out.float().cpu()
    assert torch.isnan(o[cu[1]:cu[2]]).all()
    ro, rl = A.varlen_attention_fwd(q, k, v, cu, cu, 0.125, True, -1, -1)
    keep = np.r_[cu[0]:cu[1], cu[2]:cu[3]]
    compare_attention(f64(out)[keep], f64(lse)[:, keep], ro[keep], rl[:, keep], BF16_OUT_TOL)
