"""Query-head split of the dK/dV pass (GQA and MQA): with few key blocks the
pass spreads the query heads of a group over several workgroups, which write
fp32 partial sums into a caller workspace that a reduce pass adds in order.

Checked against the fp64 oracle (2e-2 plus one bf16 ULP per element), against
the same pass without a workspace (no split: the two differ only in the order
of fp32 additions, so by at most one bf16 ULP of the value plus a few fp32
epsilons where the sum cancels to near zero), for bitwise
determinism, with a workspace too small for the preferred split (a smaller
split is taken), and at the full block-id GQA workload with cross columns
(B=8, N=1024, Hq=16, Hkv=2, D=128). Outputs are NaN-filled before each call."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import DEV, f64, grad_tolerance, grad_tolerance_terms, nan_like, note, to_dev

pytestmark = pytest.mark.gpu

ULP = 2.0 ** -7  # one bf16 step relative to the value's leading bit, at most


def _n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _grads(q, k, v, do, rep, scale, layout, ws_splits="preferred", slopes=None):
    """Forward, then preprocess / dK/dV / dQ through the C ABI. ws_splits:
    'preferred' (the workspace the library asks for), None (no workspace) or
    an int (a workspace for that many splits)."""
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    sd = None if slopes is None else to_dev(np.asarray(slopes, np.float32))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout, alibi_slopes=sd)
    B, Sq, Sk, Hq, Hkv, D = mfa._dims(qd, kd, layout)
    dq, dk, dv = nan_like(qd), nan_like(kd), nan_like(vd)
    delta = torch.empty(B, Hq, Sq, dtype=torch.float32, device=DEV)
    a = mfa._bwd_args(qd, kd, vd, out, lse, dod, dq, dk, dv, delta, layout, alibi_slopes=sd)
    mfa.attn_bwd_preprocess(a)
    nbytes, splits = mfa.attn_bwd_dkdv_workspace(a, rep)
    ws = None
    if ws_splits == "preferred" and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    elif isinstance(ws_splits, int) and splits > 1:
        ws = torch.empty(nbytes // splits * ws_splits, dtype=torch.uint8, device=DEV)
    mfa.attn_bwd_dkdv(a, rep, scale, workspace=ws)
    mfa.attn_bwd_dq(a, rep, scale)
    torch.cuda.synchronize()
    return (dq, dk, dv), splits, (B, Sk, Hkv, D, Hq // Hkv)


def _expect_split(dims, splits):
    B, Sk, Hkv, D, G = dims
    want = mfa.choose_dkdv_split(B * Hkv * -(-Sk // 64), G, D, _n_cu())
    assert splits == want and splits > 1, f"split {splits}, model {want}"


def _check_oracle(got, ref, tag, terms=(None, None, None)):
    """terms: the oracle's term sums where a positional bias makes rows put
    nearly all their weight on one key (bound of the bf16 storage of P, dS, O)."""
    for name, g, r, t in zip(("dq", "dk", "dv"), got, ref, terms):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite (unwritten) gradient"
        excess = np.abs(g - r) - (grad_tolerance(r) if t is None else grad_tolerance_terms(r, t))
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        assert excess[i] <= 0, f"{tag} {name}: |{g[i]:.5f} - {r[i]:.5f}| over the bound at {i}"


def _check_vs_unsplit(split, plain, tag):
    assert torch.equal(split[0].view(torch.int16), plain[0].view(torch.int16)), f"{tag}: dq differs"
    for name, a, b in (("dk", split[1], plain[1]), ("dv", split[2], plain[2])):
        x, y = f64(a), f64(b)
        # one bf16 step of the value, plus the fp32 reordering error of sums
        # that cancel to near zero (terms are O(1): a few fp32 epsilons)
        bound = ULP * np.maximum(np.abs(x), np.abs(y)) + 1e-5
        worst = float((np.abs(x - y) - bound).max())
        assert worst <= 0, f"{tag} {name}: split and unsplit differ by more than one bf16 step"


def _case(name, D):
    """(q, k, v, do, rep, allowed, scale, layout, slopes) for a few small GQA cases."""
    if name == "tiles_random":
        B, Sq, Sk, Hq, Hkv = 2, 300, 333, 8, 2
        m = W.random_dense_mask(Sq, Sk, 0.3, seed=D)
        q, k, v, do = W.tensors(900 + D, [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)])
        rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
        return q, k, v, do, rep, m[None, None], D ** -0.5, "bshd", None
    if name == "blockid_cross":
        w = W.blockcausal_gqa_cross(B=3, N=333, Hq=4, Hkv=2, D=D, Nc=37, prefix=100, blk_lo=5, blk_hi=40,
                                    pad_hi=60, seed=31)
        ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), w["n_cross"], to_dev(w["cross_pad"]))
        rep = mfa.MaskRep.blockid(*ids)
        allowed = M.blockid_mask(*M.make_att_block_ids(w["pad"], w["att"], w["n_cross"], w["cross_pad"]))[:, None]
        do = W.tensors(901, [tuple(w["q"].shape)])[0]
        return w["q"], w["k"], w["v"], do, rep, allowed, w["scale"], "bshd", None
    if name == "bsr_kv_valid":
        N = 520
        w = W.bsr_random(B=2, N=N, H=2, D=D, block=64, frac_den=3, seed=902 + D)
        q, do = W.tensors(903, [(2, N, 8, D), (2, N, 8, D)])
        rng = np.random.default_rng(904)
        valid = rng.random((2, N)) < 0.8
        bits = to_dev(M.pack_bits_rows(valid).view(np.int32))
        ip, ix = w["indptr"], w["indices"]
        kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), 64, 64, N, N, True, kv_valid_bits=bits)
        rep = mfa.MaskRep.bsr(to_dev(ip), to_dev(ix), kind, causal=True, csc_ptr=cp, csc_idx=ci, kv_valid_bits=bits)
        allowed = M.bsr_mask(ip, ix, 64, 64, N, N, True, kv_valid=valid)
        return q, w["k"], w["v"], do, rep, allowed, w["scale"], "bshd", None
    if name == "mqa_alibi_bhsd":
        B, H, Sq, Sk = 1, 8, 200, 259
        q, k, v, do = W.tensors(905 + D, [(B, H, Sq, D), (B, 1, Sk, D), (B, 1, Sk, D), (B, H, Sq, D)])
        slopes = np.array([2.0 ** (-8 * (h + 1) / H) for h in range(H)], np.float32)
        return q, k, v, do, mfa.MaskRep.none(), np.ones((1, 1, Sq, Sk), bool), 0.1, "bhsd", slopes
    raise ValueError(name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("name", ["tiles_random", "blockid_cross", "bsr_kv_valid", "mqa_alibi_bhsd"])
def test_split_matches_oracle_and_unsplit(name, D):
    note(f"dkdv head split {name} D={D}")
    q, k, v, do, rep, allowed, scale, layout, slopes = _case(name, D)
    got, splits, dims = _grads(q, k, v, do, rep, scale, layout, slopes=slopes)
    _expect_split(dims, splits)
    plain, _, _ = _grads(q, k, v, do, rep, scale, layout, ws_splits=None, slopes=slopes)
    _check_vs_unsplit(got, plain, name)
    if layout == "bhsd":
        q, k, v, do = (t.transpose(1, 2) for t in (q, k, v, do))
        got = [g.transpose(1, 2) for g in got]
    if slopes is None:
        _check_oracle(got, A.attention_bwd(q, k, v, do, allowed, scale)[:3], name)
    else:
        r = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=A.alibi(slopes), term_sums=True)
        _check_oracle(got, r[:3], name, r[6])


def test_split_deterministic_and_partial_workspace():
    note("dkdv head split determinism, short workspace")
    q, k, v, do, rep, allowed, scale, layout, _ = _case("tiles_random", 128)
    a, splits, _ = _grads(q, k, v, do, rep, scale, layout)
    b, _, _ = _grads(q, k, v, do, rep, scale, layout)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert splits == 4  # G = 4 over 24 key blocks
    # room for 3 of the 4 splits' sums: the pass takes the largest split that
    # fits and divides G (2)
    c, _, _ = _grads(q, k, v, do, rep, scale, layout, ws_splits=3)
    _check_vs_unsplit(c, a, "short workspace")
    ref = A.attention_bwd(q, k, v, do, allowed, scale)[:3]
    _check_oracle(c, ref, "short workspace")


def test_split_full_blockid_gqa_cross():
    """B=8, N=1024, Hq=16, Hkv=2, D=128 with 256 cross columns: 320 key
    blocks, split over the 8 heads of each group; every gradient finite, and
    batch entries 0 and 7 element-wise against the oracle."""
    note("dkdv head split, full block-id GQA with cross columns")
    w = W.blockcausal_gqa_cross()
    ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), w["n_cross"], to_dev(w["cross_pad"]))
    rep = mfa.MaskRep.blockid(*ids, summary=mfa.blockid_tile_summary(*ids))
    do = W.tensors(910, [tuple(w["q"].shape)])[0]
    got, splits, dims = _grads(w["q"], w["k"], w["v"], do, rep, w["scale"], "bshd")
    _expect_split(dims, splits)
    for t in got:
        assert torch.isfinite(t.float()).all()
    allowed = M.blockid_mask(*M.make_att_block_ids(w["pad"], w["att"], w["n_cross"], w["cross_pad"]))
    for b in (0, 7):
        sl = [x[b:b + 1] for x in (w["q"], w["k"], w["v"], do)]
        ref = A.attention_bwd(*sl, allowed[b:b + 1, None], w["scale"])[:3]
        _check_oracle([g[b:b + 1] for g in got], ref, f"gqa cross b={b}")
