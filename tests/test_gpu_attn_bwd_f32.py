"""fp32 test mode of the two-pass backward, every mask kind, against the fp64
oracle at max-abs 1e-4 for dQ, dK and dV.

The fp32 passes walk the same query-block lists (dK/dV pass) and key-tile
schedule (dQ pass) with the same mask predicates as the bf16 MFMA passes, so
this pins the backward masking (transposed allowed bits, block kinds, window
ranges, ragged tails, cross columns, empty rows) far below the bf16 bound.
Outputs are NaN-filled before each call so unwritten entries show up."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import DEV, F32_OUT_TOL, compare_attention, f64, nan_like, note, to_dev

pytestmark = pytest.mark.gpu

F32 = torch.float32


def _run(q, k, v, do, rep, scale, layout, slopes=None):
    qd, kd, vd, dod = (to_dev(t, F32) for t in (q, k, v, do))
    sd = None if slopes is None else to_dev(np.asarray(slopes, np.float32))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout, alibi_slopes=sd)
    dq, dk, dv = nan_like(qd), nan_like(kd), nan_like(vd)
    mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, scale, layout, alibi_slopes=sd, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out, lse, (dq, dk, dv)


def _check(got, ref, tag):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite (unwritten) gradient"
        err = float(np.abs(g - r).max()) if g.size else 0.0
        assert err <= F32_OUT_TOL, f"{tag} {name}: max-abs {err:.3e} > {F32_OUT_TOL}"


# --- dense-mask tiles, 128- and 64-row maps --------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("maskcase", ["random", "causal", "empty_rows"])
@pytest.mark.parametrize("tile_m", [128, 64])
def test_f32_tiles(D, maskcase, tile_m):
    note(f"f32 bwd tiles D={D} {maskcase} tile_m={tile_m}")
    B, Hq, Hkv, Sq, Sk = 2, 4, 2, 300, 333  # Sk mod 64 = 13: a ragged last key tile
    if maskcase == "causal":
        m = np.tri(Sq, Sk, dtype=bool)
    else:
        m = W.random_dense_mask(Sq, Sk, 0.35, seed=D + tile_m)
        if maskcase == "empty_rows":
            m[40:90] = False
            m[:, 200:260] = False
    q, k, v, do = W.tensors(700 + D, [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)])
    comp = mfa.compact_dense_mask(to_dev(m), BM=tile_m)
    rep = mfa.MaskRep.tiles(comp)
    scale = D ** -0.5
    out, lse, got = _run(q, k, v, do, rep, scale, "bshd")
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(q, k, v, do, m[None, None], scale)
    compare_attention(f64(out), f64(lse), ro, rl, F32_OUT_TOL)
    _check(got, (rdq, rdk, rdv), f"tiles {maskcase} {tile_m}")


def test_f32_tiles_peaked_scores():
    """q and k scaled by 4 (nearly one-hot rows; the recomputed P subtracts
    large LSE values): the fp32 passes still meet 1e-4."""
    note("f32 bwd peaked")
    Sq, Sk, D = 300, 333, 128
    m = W.random_dense_mask(Sq, Sk, 0.35, seed=5)
    q, k, v, do = W.tensors(720, [(1, Sq, 2, D), (1, Sk, 2, D), (1, Sk, 2, D), (1, Sq, 2, D)])
    q, k = (q * 4).to(torch.bfloat16), (k * 4).to(torch.bfloat16)
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
    scale = D ** -0.5
    out, lse, got = _run(q, k, v, do, rep, scale, "bshd")
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(q, k, v, do, m[None, None], scale)
    compare_attention(f64(out), f64(lse), ro, rl, F32_OUT_TOL)
    _check(got, (rdq, rdk, rdv), "peaked")


def test_f32_tiles_bhsd_and_none():
    note("f32 bwd bhsd tiles + none")
    B, H, N, D = 1, 2, 200, 64
    q, k, v, do = W.tensors(710, [(B, H, N, D)] * 4)
    m = np.tril(np.ones((N, N), bool))
    qs, ks, vs, ds = (t.transpose(1, 2) for t in (q, k, v, do))
    for rep, mk in ((mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m))), m),
                    (mfa.MaskRep.none(), np.ones((N, N), bool))):
        out, lse, got = _run(q, k, v, do, rep, 0.2, "bhsd")
        ref = A.attention_bwd(qs, ks, vs, ds, mk[None, None], 0.2)[:3]
        _check([g.transpose(1, 2) for g in got], ref, "bhsd")


# --- block ids with cross columns and padded rows ----------------------------------------------

@pytest.mark.parametrize("name", ["cfg1", "small_gqa_cross"])
def test_f32_blockid(name):
    note(f"f32 bwd blockid {name}")
    if name == "cfg1":
        w = W.blockcausal_tiny()
        nc, cross = None, None
    else:
        w = W.blockcausal_gqa_cross(B=3, N=333, Hq=4, Hkv=2, D=64, Nc=37, prefix=100, blk_lo=5, blk_hi=40,
                                    pad_hi=60, seed=21)
        nc, cross = w["n_cross"], w["cross_pad"]
    ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), nc, None if cross is None else to_dev(cross))
    rep = mfa.MaskRep.blockid(*ids)
    do = W.tensors(720, [tuple(w["q"].shape)])[0]
    out, lse, got = _run(w["q"], w["k"], w["v"], do, rep, w["scale"], "bshd")
    allowed = M.blockid_mask(*M.make_att_block_ids(w["pad"], w["att"], nc, cross))[:, None]
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(w["q"], w["k"], w["v"], do, allowed, w["scale"])
    compare_attention(f64(out), f64(lse), ro, rl, F32_OUT_TOL)
    _check(got, (rdq, rdk, rdv), f"blockid {name}")


# --- BSR, with and without kv_valid_bits --------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kv_valid", [False, True])
def test_f32_bsr(D, causal, kv_valid):
    note(f"f32 bwd bsr D={D} causal={causal} kv_valid={kv_valid}")
    N = 520  # the last 64-key block holds 8 keys
    w = W.bsr_random(B=2, N=N, H=2, D=D, block=64, frac_den=3, seed=730 + D + causal)
    q, do = W.tensors(731, [(2, N, 4, D), (2, N, 4, D)])  # GQA: 4 query heads over 2 kv heads
    ip, ix = w["indptr"], w["indices"]
    bits_d, valid = None, None
    if kv_valid:
        rng = np.random.default_rng(732)
        valid = rng.random((2, N)) < 0.8
        valid[0, 128:192] = False
        bits_d = to_dev(M.pack_bits_rows(valid).view(np.int32))
    kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, causal, kv_valid_bits=bits_d)
    rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=causal, csc_ptr=cp, csc_idx=ci,
                          kv_valid_bits=bits_d)
    out, lse, got = _run(q, w["k"], w["v"], do, rep, w["scale"], "bshd")
    allowed = M.bsr_mask(ip, ix, 64, 64, N, N, causal, kv_valid=valid)
    rdq, rdk, rdv, ro, rl, _ = A.attention_bwd(q, w["k"], w["v"], do, allowed, w["scale"])
    compare_attention(f64(out), f64(lse), ro, rl, F32_OUT_TOL)
    _check(got, (rdq, rdk, rdv), "bsr")


# --- varlen: windows, empty and single-token sequences, seqused_k ------------------------------

@pytest.mark.parametrize("causal,win", [(True, (100, 0)), (True, (-1, -1)), (False, (50, 30))])
@pytest.mark.parametrize("used", [False, True])
def test_f32_varlen(causal, win, used):
    note(f"f32 bwd varlen causal={causal} win={win} seqused={used}")
    L = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
    T = int(L.sum())
    q, k, v, do = W.tensors(740, [(T, 4, 64), (T, 2, 64), (T, 2, 64), (T, 4, 64)])
    USED = np.array([1, 0, 150, 0, 257, -4, 64, 180], np.int32) if used else None
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=causal, window=win,
                             seqused_k=None if USED is None else to_dev(USED))
    out, lse, got = _run(q, k, v, do, rep, 0.125, "thd")
    cu = M.cu_seqlens(L)
    allowed = M.varlen_mask(cu, cu, causal, win[0], win[1], seqused_k=USED)
    ref = A.attention_bwd(q[None], k[None], v[None], do[None], allowed[None, None], 0.125)
    compare_attention(f64(out)[None], f64(lse)[None], ref[3], ref[4], F32_OUT_TOL)
    _check(got, [r[0] for r in ref[:3]], "varlen")


# --- positional bias (ALiBi score_mod) --------------------------------------------------------

def test_f32_alibi_tiles():
    note("f32 bwd alibi")
    B, Hq, Hkv, S, D = 1, 4, 2, 260, 64
    slopes = np.array([2.0 ** (-8 * (h + 1) / Hq) for h in range(Hq)], np.float32)
    q, k, v, do = W.tensors(750, [(B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D), (B, S, Hq, D)])
    m = np.tri(S, S, dtype=bool)
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
    out, lse, got = _run(q, k, v, do, rep, 0.125, "bshd", slopes=slopes)
    mod = A.alibi(slopes.astype(np.float64))
    ref = A.attention_bwd(q, k, v, do, m[None, None], 0.125, score_mod=mod)[:3]
    _check(got, ref, "alibi tiles")


def test_f32_zero_keys_and_rows_past_end():
    """Sk = 0: every row empty (dQ = 0); a 1-row query tile."""
    note("f32 bwd Sk=0 and Sq=1")
    q, do = W.tensors(760, [(2, 5, 2, 64), (2, 5, 2, 64)])
    qd, dod = to_dev(q, F32), to_dev(do, F32)
    k = torch.zeros(2, 0, 2, 64, dtype=F32, device=DEV)
    out, lse = mfa.attn_fwd(qd, k, k, mfa.MaskRep.none(), 0.125, "bshd")
    dq = nan_like(qd)
    mfa.attn_bwd(qd, k, k, out, lse, dod, mfa.MaskRep.none(), 0.125, "bshd", dq=dq, dk=torch.empty_like(k),
                 dv=torch.empty_like(k))
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    q1, k1, v1, d1 = W.tensors(761, [(1, 1, 1, 128), (1, 70, 1, 128), (1, 70, 1, 128), (1, 1, 1, 128)])
    out, lse, got = _run(q1, k1, v1, d1, mfa.MaskRep.none(), 0.09, "bshd")
    ref = A.attention_bwd(q1, k1, v1, d1, np.ones((1, 1, 1, 70), bool), 0.09)[:3]
    _check(got, ref, "Sq=1")


@pytest.mark.parametrize("dtype", [torch.bfloat16, F32])
def test_no_query_rows_give_zero_dk_dv(dtype):
    """Sq = 0 with keys present: dK = dV = 0 for every key (written, not left
    as they were), for plain attention and for varlen sequences with no
    query tokens; dq is empty."""
    note(f"bwd with no query rows {dtype}")
    k, v = W.tensors(770, [(2, 70, 2, 64), (2, 70, 2, 64)])
    kd, vd = to_dev(k, dtype), to_dev(v, dtype)
    q = torch.zeros(2, 0, 4, 64, dtype=dtype, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.zeros(2, 4, 0, device=DEV)
    dk, dv = nan_like(kd), nan_like(vd)
    mfa.attn_bwd(q, kd, vd, out, lse, out, mfa.MaskRep.none(), 0.125, "bshd", dq=torch.empty_like(q), dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    # varlen: three sequences with keys and no query tokens
    Lq = np.array([0, 0, 0], np.int32)
    Lk = np.array([5, 64, 31], np.int32)
    kv = W.tensors(771, [(100, 2, 64), (100, 2, 64)])
    kd, vd = to_dev(kv[0], dtype), to_dev(kv[1], dtype)
    s = mfa.varlen_schedule(to_dev(Lq), to_dev(Lk), causal=False, window=(-1, -1), work_cap=4)
    rep = mfa.MaskRep.varlen(s, 0, int(Lk.max()), causal=False)
    q = torch.zeros(0, 4, 64, dtype=dtype, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.zeros(4, 0, device=DEV)
    dk, dv = nan_like(kd), nan_like(vd)
    mfa.attn_bwd(q, kd, vd, out, lse, out, rep, 0.125, "thd", dq=torch.empty_like(q), dk=dk, dv=dv,
                 delta=torch.empty(4, 0, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
