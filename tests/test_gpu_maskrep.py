"""Mask representations on the GPU: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from oracle import masks as M
import workloads as W
from tests.gpu_util import DEV, note, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("case", ["cfg1", "cfg4", "tiny", "no_opener", "N1"])
def test_block_ids_bit_exact(case):
    note(f"block ids {case}")
    if case == "cfg1":
        w = W.blockcausal_tiny()
        pad, att, nc, cross = w["pad"], w["att"], None, None
    elif case == "cfg4":
        w = W.blockcausal_gqa_cross()
        pad, att, nc, cross = w["pad"], w["att"], w["n_cross"], w["cross_pad"]
    elif case == "tiny":
        rng = np.random.default_rng(7)
        pad = rng.random((3, 700)) < 0.8
        att = (rng.random((3, 700)) < 0.2).astype(np.int32) * rng.integers(1, 5, (3, 700))
        nc, cross = 5, rng.random((3, 5)) < 0.5
    elif case == "no_opener":
        pad = np.ones((2, 300), bool)
        att = np.zeros((2, 300), np.int32)
        nc, cross = None, None
    else:
        pad = np.ones((1, 1), bool)
        att = np.ones((1, 1), np.int32)
        nc, cross = 1, np.zeros((1, 1), bool)
    ref = M.make_att_block_ids(pad, att, nc, cross)
    got = mfa.make_block_ids(to_dev(pad), to_dev(att), nc, None if cross is None else to_dev(cross))
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert np.array_equal(_np(g), r)


@pytest.mark.parametrize("case", ["cfg1", "cfg4", "random_ids"])
def test_blockid_tile_summary_bit_exact(case):
    note(f"blockid summary {case}")
    if case == "cfg1":
        w = W.blockcausal_tiny()
        ids = M.make_att_block_ids(w["pad"], w["att"])
    elif case == "cfg4":
        w = W.blockcausal_gqa_cross()
        ids = M.make_att_block_ids(w["pad"], w["att"], w["n_cross"], w["cross_pad"])
    else:
        rng = np.random.default_rng(3)
        ids = (rng.integers(-9, 9, (2, 333)).astype(np.int32), rng.integers(-9, 9, (2, 199)).astype(np.int32),
               rng.random((2, 333)) < 0.7, rng.random((2, 199)) < 0.7)
    for BM in (128, 64):
        ref = M.blockid_tile_summary(*ids, BM, 64)
        got = mfa.blockid_tile_summary(*[to_dev(x) for x in ids], BM=BM, BN=64)
        torch.cuda.synchronize()
        assert np.array_equal(_np(got[0]), ref[0])
        assert np.array_equal(_np(got[1]), ref[1])
        assert np.array_equal(_np(got[2]).view(np.uint32), ref[2])


def _check_compaction(m):
    ref = M.compact_dense_mask(m, 128, 64)
    got = mfa.compact_dense_mask(to_dev(m))
    torch.cuda.synchronize()
    nnz = int(ref["row_ptr"][-1])
    assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"])
    assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"])
    assert np.array_equal(_np(got["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(_np(got["col_idx"])[:nnz], ref["col_idx"])
    assert np.array_equal(_np(got["col_kind"])[:nnz], ref["col_kind"])


@pytest.mark.parametrize("case", ["causal8192", "random_vec", "random_ragged", "all_true", "all_false",
                                  "one_col", "one_row", "tall"])
def test_compact_dense_mask_bit_exact(case):
    note(f"compaction {case}")
    rng = np.random.default_rng(11)
    if case == "causal8192":
        m = np.tril(np.ones((8192, 8192), bool))
    elif case == "random_vec":
        m = W.random_dense_mask(640, 1024, 0.05, seed=1)
    elif case == "random_ragged":
        m = W.random_dense_mask(301, 333, 0.3, seed=2)
    elif case == "all_true":
        m = np.ones((512, 768), bool)
    elif case == "all_false":
        m = np.zeros((512, 768), bool)
    elif case == "one_col":
        m = rng.random((200, 1)) < 0.5
    elif case == "one_row":
        m = rng.random((1, 4096)) < 0.5
    else:
        m = rng.random((2000, 48)) < 0.9
    _check_compaction(m)


def test_compact_nonbool_bytes_count_as_true():
    note("compaction nonzero bytes")
    rng = np.random.default_rng(5)
    m = rng.integers(0, 4, (256, 512)).astype(np.uint8)
    ref = M.compact_dense_mask(m != 0, 128, 64)
    got = mfa.compact_dense_mask(to_dev(m))
    torch.cuda.synchronize()
    assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"])
    assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"])


@pytest.mark.parametrize("case", ["cfg5", "small_ragged"])
def test_bsr_prepare_bit_exact(case):
    note(f"bsr prepare {case}")
    if case == "cfg5":
        w = W.bsr_random(D=8)
        N, blk = 16384, 64
    else:
        w = W.bsr_random(B=2, N=1000, H=3, D=8, block=64, frac_den=3, seed=9)
        N, blk = 1000, 64
    ip, ix = w["indptr"], w["indices"]
    nb = -(-N // blk)
    assert mfa.bsr_validate(to_dev(ip), to_dev(ix), nb) == M.bsr_validate(ip, ix, nb)
    kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), blk, blk, N, N, True)
    torch.cuda.synchronize()
    assert np.array_equal(_np(kind), M.bsr_col_kind(ip, ix, blk, blk, N, N, True))
    rp, ri = M.bsr_to_csc(ip, ix, nb)
    assert np.array_equal(_np(cp), rp)
    assert np.array_equal(_np(ci), ri)


def test_bsr_validate_rejects_noncanonical():
    note("bsr validate rejects")
    w = W.bsr_random(B=1, N=640, H=2, D=8, block=64, frac_den=2, seed=1)
    ip, ix = w["indptr"].copy(), w["indices"].copy()
    s = ip[0, 0, 5]
    ix[s], ix[s + 1] = ix[s + 1], ix[s]
    with pytest.raises(mfa.MfaError) as e:
        mfa.bsr_validate(to_dev(ip), to_dev(ix), 10)
    assert e.value.status_name == "MFA_E_NONCANONICAL"


@pytest.mark.parametrize("case", ["cfg3", "mixed", "tiny"])
def test_varlen_schedule_bit_exact(case):
    note(f"varlen schedule {case}")
    if case == "cfg3":
        L = W.varlen_window(H=1, D=8)["lengths"]
        win = (511, 0)
    elif case == "mixed":
        L = np.array([1, 128, 129, 0, 4000, 300, 7], np.int32)
        win = (200, 0)
    else:
        L = np.array([5, 11], np.int32)
        win = (-1, -1)
    cap = int(L.sum()) // 128 + L.size
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=win, work_cap=cap)
    torch.cuda.synchronize()
    cu_q, cu_k, mq, mk, work = M.varlen_schedule(L, L, 128, 64, True, win[0], win[1])
    assert np.array_equal(_np(s["cu_q"]), cu_q) and np.array_equal(_np(s["cu_k"]), cu_k)
    assert _np(s["max_len"]).tolist() == [mq, mk]
    n = int(_np(s["n_work"])[0])
    assert n == len(work)
    assert np.array_equal(_np(s["work"])[:n], work)
    assert np.all(_np(s["work"])[n:] == -1)
