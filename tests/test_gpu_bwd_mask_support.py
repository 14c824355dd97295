"""Exact support of the dK/dV pass's masks, for every mask kind.

With dO zero except one query row r per (batch, head), the dV row of key j
is P(r, j) dO(r): nonzero exactly where the mask allows (r, j), since a
masked score's P is exp2(-inf) = 0, and exactly zero elsewhere, since every
other query row contributes P * 0. dK of key j is scale * dS(r, j) q(r) with
dS(r, j) = P(r, j) (dP - delta), which is zero wherever P is. So the set of
keys with a nonzero dV row must equal the oracle's allowed row, key for key,
and dK must vanish outside it: a test of every transposed mask bit of the
chosen rows, where the parity tests only bound the gradients' values. The
rows sit on the edges of 32- and 64-query blocks (where partial blocks
split), and each head has its own kv head (Hq = Hkv), or, in the GQA case,
only one query head of each group carries a row. bf16 and the fp32 test
mode, D = 64 and 128."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import masks as M
import workloads as W
from tests.gpu_util import DEV, f64, nan_like, note, to_dev

pytestmark = pytest.mark.gpu

EDGES = (0, 1, 31, 32, 33, 63)  # offsets within a 64-query block


def _rows(n_rows, count, seed):
    """count query rows in [0, n_rows): block edges first, then random ones."""
    rng = np.random.default_rng(seed)
    cand = [b * 64 + e for b in range(-(-n_rows // 64)) for e in EDGES if b * 64 + e < n_rows]
    rng.shuffle(cand)
    out = cand[:count]
    while len(out) < count:
        out.append(int(rng.integers(0, n_rows)))
    return np.array(out[:count])


def _run(q, k, v, do, rep, scale, layout, dtype):
    qd, kd, vd, dod = (to_dev(t, dtype) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout)
    g = (nan_like(qd), nan_like(kd), nan_like(vd))
    mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, scale, layout, dq=g[0], dk=g[1], dv=g[2])
    torch.cuda.synchronize()
    return f64(g[1]), f64(g[2])


def _check_support(dk, dv, allowed_row, tag):
    """dk, dv: (Sk, D) of one kv head; allowed_row: (Sk,) bool."""
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv)), f"{tag}: non-finite gradient"
    nz = np.any(dv != 0.0, axis=-1)
    wrong = np.flatnonzero(nz != allowed_row)
    assert wrong.size == 0, (f"{tag}: dv support differs from the mask at keys {wrong[:8].tolist()} "
                             f"(allowed {allowed_row[wrong[:8]].tolist()})")
    leak = np.flatnonzero(np.any(dk != 0.0, axis=-1) & ~allowed_row)
    assert leak.size == 0, f"{tag}: dk nonzero at disallowed keys {leak[:8].tolist()}"


def _dense_do(shape, rows, seed):
    """(B, S, H, D) zeros but row rows[b, h] of each (b, h), scaled up."""
    B, S, H, D = shape
    do = torch.zeros(shape, dtype=torch.float32)
    vals = W.tensors(seed, [(B, H, D)], dtype=torch.float32)[0] * 8.0
    for b in range(B):
        for h in range(H):
            do[b, rows[b, h], h] = vals[b, h]
    return do


def _dense_case(kind, D):
    """(q, k, v, rep, allowed (B, H, Sq, Sk) bool, scale) with Hq = Hkv."""
    if kind == "tiles":
        B, Sq, Sk, H = 2, 300, 333, 4
        mask = W.random_dense_mask(Sq, Sk, 0.3, 11) | np.eye(Sq, Sk, dtype=bool)
        q, k, v = W.tensors(300 + D, [(B, Sq, H, D), (B, Sk, H, D), (B, Sk, H, D)])
        rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask)))
        return q, k, v, rep, np.broadcast_to(mask, (B, H, Sq, Sk)), D ** -0.5
    if kind in ("bsr_causal", "bsr_full", "bsr_kv_valid"):
        N, H, B = 520, 4, 2
        causal = kind != "bsr_full"
        w = W.bsr_random(B=B, N=N, H=H, D=D, block=64, frac_den=2, seed=301 + D)
        ip, ix = w["indptr"], w["indices"]
        valid, bits = None, None
        if kind == "bsr_kv_valid":
            valid = np.random.default_rng(302).random((B, N)) < 0.7
            bits = to_dev(M.pack_bits_rows(valid).view(np.int32))
        bk, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, causal, kv_valid_bits=bits)
        rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), bk, causal=causal, csc_ptr=cp, csc_idx=ci, kv_valid_bits=bits)
        allowed = M.bsr_mask(ip, ix, 64, 64, N, N, causal, kv_valid=valid)
        return w["q"], w["k"], w["v"], rep, allowed, w["scale"]
    if kind == "blockid":
        w = W.blockcausal_gqa_cross(B=3, N=333, Hq=2, Hkv=2, D=D, Nc=37, prefix=100, blk_lo=5, blk_hi=40,
                                    pad_hi=60, seed=303)
        ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), w["n_cross"], to_dev(w["cross_pad"]))
        allowed = M.blockid_mask(*M.make_att_block_ids(w["pad"], w["att"], w["n_cross"], w["cross_pad"]))
        B, Sq, Sk = allowed.shape
        return w["q"], w["k"], w["v"], mfa.MaskRep.blockid(*ids), np.broadcast_to(allowed[:, None], (B, 2, Sq, Sk)), \
            w["scale"]
    raise ValueError(kind)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["tiles", "bsr_causal", "bsr_full", "bsr_kv_valid", "blockid"])
def test_dense_layout_support(kind, D, dtype):
    note(f"bwd mask support {kind} D={D} {dtype}")
    q, k, v, rep, allowed, scale = _dense_case(kind, D)
    B, Sq, H, _ = q.shape
    rows = np.stack([_rows(Sq, H, 310 + b) for b in range(B)])
    do = _dense_do(tuple(q.shape), rows, 311)
    dk, dv = _run(q, k, v, do, rep, scale, "bshd", dtype)
    for b in range(B):
        for h in range(H):
            _check_support(dk[b, :, h], dv[b, :, h], allowed[b, h, rows[b, h]], f"{kind} b={b} h={h} row={rows[b, h]}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,win", [(True, (100, 0)), (True, (-1, -1)), (False, (50, 30)), (False, (-1, 5)),
                                        (True, (0, 0))])
def test_varlen_support(causal, win, D, dtype):
    note(f"bwd mask support varlen causal={causal} win={win} D={D} {dtype}")
    L = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
    T, H = int(L.sum()), 16
    q, k, v = W.tensors(320 + D, [(T, H, D), (T, H, D), (T, H, D)])
    cu = M.cu_seqlens(L)
    # one row per head, at block edges of the sequences
    rng = np.random.default_rng(321)
    cand = [int(cu[s]) + o for s in range(L.size) for o in range(int(L[s])) if o % 64 in EDGES or o == L[s] - 1]
    rows = rng.choice(cand, size=H, replace=False)
    do = torch.zeros(T, H, D)
    vals = W.tensors(322, [(H, D)], dtype=torch.float32)[0] * 8.0
    for h in range(H):
        do[rows[h], h] = vals[h]
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=causal, window=win)
    dk, dv = _run(q, k, v, do, rep, D ** -0.5, "thd", dtype)
    allowed = M.varlen_mask(cu, cu, causal, win[0], win[1])
    for h in range(H):
        _check_support(dk[:, h], dv[:, h], allowed[rows[h]], f"varlen h={h} row={rows[h]}")


@pytest.mark.parametrize("D", [64, 128])
def test_gqa_split_support(D):
    """GQA (G = 4) with the dK/dV head split: one query head per group carries
    a row; the split partial sums of the others are exact zeros."""
    note(f"bwd mask support GQA split D={D}")
    B, Sq, Sk, Hq, Hkv = 2, 300, 333, 8, 2
    mask = W.random_dense_mask(Sq, Sk, 0.3, 12) | np.eye(Sq, Sk, dtype=bool)
    q, k, v = W.tensors(330 + D, [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D)])
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask)))
    rows = np.stack([_rows(Sq, Hq, 331 + b) for b in range(B)])
    do = _dense_do((B, Sq, Hq, D), rows, 332)
    carrier = [3, 6]  # the one query head of each group with a nonzero row
    for h in range(Hq):
        if h not in carrier:
            do[:, :, h] = 0.0
    dk, dv = _run(q, k, v, do, rep, D ** -0.5, "bshd", torch.bfloat16)
    for b in range(B):
        for g, h in enumerate(carrier):
            _check_support(dk[b, :, g], dv[b, :, g], mask[rows[b, h]], f"gqa b={b} group={g} row={rows[b, h]}")
