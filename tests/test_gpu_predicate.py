"""Predicate masks built on the GPU (mfa_predicate_tiles) against the oracle:
the oracle materialises the same predicate with create_mask (tensorplay
omni_attention, "Block masks") and compacts it; every output must be
bit-exact. Then attention forward and backward on a predicate's tiles."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import BF16_OUT_TOL, LSE_TOL, f64, grad_tolerance, note, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def _linear(a, b, c):
    """Oracle predicate for the atom a*q_idx + b*kv_idx + c >= 0."""
    def pred(bb, hh, q_idx, kv_idx):
        return a * np.asarray(q_idx, np.int64) + b * np.asarray(kv_idx, np.int64) + c >= 0
    return pred


# (name, GPU predicate, oracle predicate, Nq, Nk)
CASES = [
    ("page_causal_window4", mfa.Pred.causal().and_(mfa.Pred.past_window(4)),
     M.and_masks(M.causal, M.past_window(4)), 16, 16),
    ("causal_window_1000", mfa.Pred.causal().and_(mfa.Pred.past_window(300)),
     M.and_masks(M.causal, M.past_window(300)), 1000, 1000),
    ("prefix_lm", mfa.Pred.causal().or_(mfa.Pred.prefix(100)),
     M.or_masks(M.causal, lambda b, h, q, kv: kv < 100), 300, 517),
    ("bidirectional_window", mfa.Pred.past_window(50).and_(mfa.Pred.atom(1, -1, 49)),
     M.and_masks(M.past_window(50), lambda b, h, q, kv: kv - q < 50), 700, 650),
    ("noop", mfa.Pred.noop(), M.noop_mask, 200, 129),
    ("never", mfa.Pred.never(), lambda b, h, q, kv: np.zeros(np.broadcast(q, kv).shape, bool), 130, 300),
    ("odd_coefficients", mfa.Pred.atom(2, -3, 5).or_(mfa.Pred.atom(-1, 2, -7)),
     M.or_masks(_linear(2, -3, 5), _linear(-1, 2, -7)), 257, 300),
    ("empty_and_full_mix", mfa.Pred.atom(0, 1, -200).and_(mfa.Pred.atom(-1, 0, 150)),
     M.and_masks(_linear(0, 1, -200), _linear(-1, 0, 150)), 400, 400),
    ("causal_2048", mfa.Pred.causal(), M.causal, 2048, 2048),
]


@pytest.mark.parametrize("name,gp,op,Nq,Nk", CASES, ids=[c[0] for c in CASES])
def test_predicate_tiles_bit_exact(name, gp, op, Nq, Nk):
    note(f"predicate tiles {name}")
    dense = M.create_mask(op, 1, 1, Nq, Nk)[0, 0]
    ref = M.compact_dense_mask(dense, 128, 64)
    got = mfa.predicate_tiles(gp, Nq, Nk)
    torch.cuda.synchronize()
    nnz = int(ref["row_ptr"][-1])
    assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"])
    assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"])
    assert np.array_equal(_np(got["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(_np(got["col_idx"])[:nnz], ref["col_idx"])
    assert np.array_equal(_np(got["col_kind"])[:nnz], ref["col_kind"])


def test_predicate_page_example_pattern():
    """The page's 16 x 16 example: causal AND at most 4 past keys gives a band
    of width 4 on and below the diagonal."""
    note("predicate page example")
    got = mfa.predicate_tiles(mfa.Pred.causal().and_(mfa.Pred.past_window(4)), 16, 16)
    bits = _np(got["fine_bits"]).view(np.uint32)[:, 0]
    i = np.arange(16)
    want = np.array([sum(1 << j for j in range(max(0, r - 3), r + 1)) for r in i], np.uint32)
    assert np.array_equal(bits, want)


def test_attention_on_predicate_tiles():
    note("attention on predicate tiles")
    B, N, Hq, Hkv, D = 2, 333, 4, 2, 128
    gp = mfa.Pred.causal().and_(mfa.Pred.past_window(100)).or_(mfa.Pred.prefix(16))
    op = M.or_masks(M.and_masks(M.causal, M.past_window(100)), lambda b, h, q, kv: kv < 16)
    allowed = M.create_mask(op, 1, 1, N, N)
    q, k, v, do = W.tensors(81, [(B, N, Hq, D), (B, N, Hkv, D), (B, N, Hkv, D), (B, N, Hq, D)])
    rep = mfa.MaskRep.tiles(mfa.predicate_tiles(gp, N, N))
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, D ** -0.5, "bshd")
    dq, dk, dv = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, D ** -0.5, "bshd")
    torch.cuda.synchronize()
    ro, rl = A.attention_fwd(q, k, v, allowed, D ** -0.5)
    assert float(np.abs(f64(out) - ro).max()) <= BF16_OUT_TOL
    assert float(np.abs(f64(lse) - rl).max()) <= LSE_TOL
    ref = A.attention_bwd(q, k, v, do, allowed, D ** -0.5)[:3]
    for g, r in zip((dq, dk, dv), ref):
        assert np.all(np.abs(f64(g) - r) <= grad_tolerance(r))
