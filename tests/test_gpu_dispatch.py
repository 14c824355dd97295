"""Density-aware tile dispatch (BinFlash README, "Efficiently Dispatching
..."): 64-row dense-mask tile maps (bit-exact against the oracle's
compaction at BM = 64), the 128-row map derived from them (bit-exact against
a direct 128-row compaction), tile counts, attention forward and backward on
64-row maps, and the dispatcher's choice."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, F32_OUT_TOL, compare_attention, f64, grad_tolerance, note, to_dev)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def _blocks64(N, density, seed):
    """Random 64 x 64 blocks plus the diagonal: most 128-row tiles are half empty."""
    rng = np.random.default_rng(seed)
    nb = (N + 63) // 64
    sel = rng.random((nb, nb)) < density
    np.fill_diagonal(sel, True)
    return np.kron(sel, np.ones((64, 64), bool))[:N, :N]


MASKS = [
    ("random30_ragged", lambda: W.random_dense_mask(300, 333, 0.3, 1)),
    ("causal_1000", lambda: np.tril(np.ones((1000, 1000), bool))),
    ("blocks64_700", lambda: _blocks64(700, 0.15, 2)),
    ("sparse_65x129", lambda: W.random_dense_mask(65, 129, 0.02, 3)),
    ("all_true_130x64", lambda: np.ones((130, 64), bool)),
]


@pytest.mark.parametrize("name,mk", MASKS, ids=[m[0] for m in MASKS])
def test_bm64_compaction_coarsening_and_counts(name, mk):
    note(f"dispatch maps {name}")
    mask = mk()
    Nq, Nk = mask.shape
    c64 = mfa.compact_dense_mask(to_dev(mask), BM=64)
    c128 = mfa.coarsen_tile_map(c64, Nq, Nk)
    n64 = _np(mfa.tile_counts(c64["tile_kind"]))
    torch.cuda.synchronize()
    for got, BM in ((c64, 64), (c128, 128)):
        ref = M.compact_dense_mask(mask, BM, 64)
        nnz = int(ref["row_ptr"][-1])
        assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"]), BM
        assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"]), BM
        assert np.array_equal(_np(got["row_ptr"]), ref["row_ptr"]), BM
        assert np.array_equal(_np(got["col_idx"])[:nnz], ref["col_idx"]), BM
        assert np.array_equal(_np(got["col_kind"])[:nnz], ref["col_kind"]), BM
    k = M.compact_dense_mask(mask, 64, 64)["tile_kind"]
    assert n64.tolist() == [int((k == 0).sum()), int((k == 1).sum()), int((k == 2).sum())]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("name", ["random30_ragged", "blocks64_700"])
def test_attention_on_64_row_tiles(name, D):
    note(f"attention tile_m=64 {name} D={D}")
    mask = dict((m[0], m[1]) for m in MASKS)[name]()
    Sq, Sk = mask.shape
    q, k, v, do = W.tensors(60 + D, [(2, Sq, 4, D), (2, Sk, 2, D), (2, Sk, 2, D), (2, Sq, 4, D)])
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(mask), BM=64))
    ro, rl = A.attention_fwd(q, k, v, mask[None, None], D ** -0.5)
    for dtype, tol in ((torch.bfloat16, BF16_OUT_TOL), (torch.float32, F32_OUT_TOL)):
        out, lse = mfa.attn_fwd(*(to_dev(t, dtype) for t in (q, k, v)), rep, D ** -0.5, "bshd")
        torch.cuda.synchronize()
        compare_attention(f64(out), f64(lse), ro, rl, tol)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, D ** -0.5, "bshd")
    got = mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, D ** -0.5, "bshd")
    torch.cuda.synchronize()
    ref = A.attention_bwd(q, k, v, do, mask[None, None], D ** -0.5)[:3]
    for g, r in zip(got, ref):
        assert np.all(np.abs(f64(g) - r) <= grad_tolerance(r))


def test_dispatcher_choices():
    """64 x 64 block masks go to 64-row tiles, causal stays at 128; both
    results drive the attention kernels correctly."""
    note("dispatcher choices")
    for mask, want in ((_blocks64(2048, 0.1, 5), 64), (np.tril(np.ones((2048, 2048), bool)), 128)):
        c = mfa.compact_dense_mask_auto(to_dev(mask))
        assert c["tile_m"] == want, c["counts"]
        N = mask.shape[0]
        q, k, v = W.tensors(70, [(1, N, 2, 128)] * 3)
        out, lse = mfa.attn_fwd(*(to_dev(t) for t in (q, k, v)), mfa.MaskRep.tiles(c), 0.1, "bshd")
        torch.cuda.synchronize()
        rows = np.array([0, 1, 63, 64, 127, 128, 1000, N - 1])

        def allowed(bb, hm, rr, mask=mask):
            return mask[np.asarray(rr)]
        allowed.heads = 1
        ro, rl = A.attention_fwd(q, k, v, allowed, 0.1, rows=rows)
        compare_attention(f64(out[:, rows]), f64(lse[:, :, rows]), ro, rl, BF16_OUT_TOL)
