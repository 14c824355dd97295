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


def _check_compaction(m, BM=128):
    ref = M.compact_dense_mask(m, BM, 64)
    got = mfa.compact_dense_mask(to_dev(m), BM=BM)
    torch.cuda.synchronize()
    nnz = int(ref["row_ptr"][-1])
    assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"])
    assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"])
    assert np.array_equal(_np(got["row_ptr"]), ref["row_ptr"])
    assert np.array_equal(_np(got["col_idx"])[:nnz], ref["col_idx"])
    assert np.array_equal(_np(got["col_kind"])[:nnz], ref["col_kind"])


@pytest.mark.parametrize("case", ["causal8192", "random_vec", "random_ragged", "all_true", "all_false",
                                  "one_col", "one_row", "tall", "rows65536", "ragged_wide", "ragged_wide_small"])
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
    elif case == "tall":
        m = rng.random((2000, 48)) < 0.9
    elif case in ("ragged_wide", "ragged_wide_small"):
        # row length a multiple of 16 but not of 1024 (lanes past the end of a
        # row re-read its start and are zeroed) and a row count that ends
        # inside a wave's 16 rows (rows past the end re-read the last row)
        m = W.random_dense_mask(1000, 8000, 0.3, seed=4) if case == "ragged_wide" else rng.random((17, 1040)) < 0.5
        _check_compaction(m, BM=64)
    else:
        # 65,536 query rows (512 tile rows x 16 key tiles): the CSR takes the
        # linear count / scan / fill path
        m = W.random_dense_mask(65536, 1024, 0.02, seed=3)
        _check_compaction(m, BM=64)
    _check_compaction(m)


@pytest.mark.parametrize("case", ["dense_values", "sparse_values"])
def test_compact_nonbool_bytes_count_as_true(case):
    """Any nonzero byte attends. dense_values: every wave sees bytes above 1;
    sparse_values: a 0/1 mask with a few bytes of 2..255, so that only the
    waves that read one of them repack their rows with the exact test."""
    note(f"compaction nonzero bytes {case}")
    rng = np.random.default_rng(5)
    if case == "dense_values":
        m = rng.integers(0, 4, (256, 512)).astype(np.uint8)
    else:
        m = (rng.random((1000, 2048)) < 0.4).astype(np.uint8)
        idx = rng.integers(0, m.size, 12)
        m.flat[idx] = rng.integers(2, 256, 12).astype(np.uint8)
        m.flat[idx[:4]] = 0
    for BM in (128, 64):
        ref = M.compact_dense_mask(m != 0, BM, 64)
        got = mfa.compact_dense_mask(to_dev(m), BM=BM)
        torch.cuda.synchronize()
        assert np.array_equal(_np(got["fine_bits"]).view(np.uint32), ref["fine_bits"])
        assert np.array_equal(_np(got["tile_kind"]), ref["tile_kind"])


@pytest.mark.parametrize("case", ["cfg5", "small_ragged", "wide_rows", "many_kv_blocks"])
def test_bsr_prepare_bit_exact(case):
    note(f"bsr prepare {case}")
    causal = True
    if case == "cfg5":
        w = W.bsr_random(D=8)
        Sq = Skv = 16384
    elif case == "small_ragged":
        w = W.bsr_random(B=2, N=1000, H=3, D=8, block=64, frac_den=3, seed=9)
        Sq = Skv = 1000
    elif case == "wide_rows":
        # every earlier block listed: up to 64 entries per row, columns shared by many rows
        w = W.bsr_random(B=1, N=4096, H=2, D=8, block=64, frac_den=1, seed=10)
        Sq = Skv = 4096
    else:
        # 8 query-block rows over 16,384 key blocks (the most the column pass holds), non-causal
        rng = np.random.default_rng(11)
        B, H, nq, nk = 1, 2, 8, 16384
        rows = [np.sort(rng.choice(nk, int(rng.integers(0, 400)), replace=False)) for _ in range(B * H * nq)]
        counts = np.array([len(r) for r in rows])
        indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        w = {"indptr": np.stack([indptr[i * nq:(i + 1) * nq + 1] for i in range(B * H)]).reshape(B, H, nq + 1),
             "indices": np.concatenate(rows).astype(np.int32)}
        Sq, Skv, causal = nq * 64, nk * 64, False
    blk = 64
    ip, ix = w["indptr"], w["indices"]
    nb = -(-Skv // blk)
    assert mfa.bsr_validate(to_dev(ip), to_dev(ix), nb) == M.bsr_validate(ip, ix, nb)
    kind, cp, ci = mfa.bsr_prepare(to_dev(ip), to_dev(ix), blk, blk, Sq, Skv, causal)
    torch.cuda.synchronize()
    assert np.array_equal(_np(kind), M.bsr_col_kind(ip, ix, blk, blk, Sq, Skv, causal))
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


def _varlen_case(case):
    """(len_q, causal, window) of a schedule-only case (no q/k/v needed)."""
    rng = np.random.default_rng(7)
    if case == "cfg3":
        return W.varlen_window(H=1, D=8)["lengths"], True, (511, 0)
    if case == "mixed":
        return np.array([1, 128, 129, 0, 4000, 300, 7], np.int32), True, (200, 0)
    if case == "tiny":
        return np.array([5, 11], np.int32), True, (-1, -1)
    if case == "long_causal_open":
        # tiles past 262,080 keys visit 4096+ key tiles (two high digits)
        return np.array([600_000, 3000, 128, 270_000], np.int32), True, (-1, -1)
    if case == "long_noncausal_ties":
        # every tile of a sequence has the same cost: ties ordered by (seq, q0)
        return np.array([300_000, 5, 300_000, 262_145], np.int32), False, (-1, -1)
    if case == "two_sided_window":
        return rng.integers(0, 5000, 40).astype(np.int32), False, (700, 300)
    if case == "many_sequences":
        # more sequences than one 1024-thread group
        return rng.integers(0, 400, 2500).astype(np.int32), True, (255, 0)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["cfg3", "mixed", "tiny", "long_causal_open", "long_noncausal_ties",
                                  "two_sided_window", "many_sequences"])
def test_varlen_schedule_bit_exact(case):
    L, causal, win = _varlen_case(case)
    note(f"varlen schedule {case}: nseq={L.size} max_len={int(L.max())} causal={causal} window={win}")
    cap = int(L.sum()) // 128 + L.size
    s = mfa.varlen_schedule(to_dev(L), causal=causal, window=win, work_cap=cap)
    torch.cuda.synchronize()
    cu_q, cu_k, mq, mk, work = M.varlen_schedule(L, L, 128, 64, causal, win[0], win[1])
    assert np.array_equal(_np(s["cu_q"]), cu_q) and np.array_equal(_np(s["cu_k"]), cu_k)
    assert _np(s["max_len"]).tolist() == [mq, mk]
    n = int(_np(s["n_work"])[0])
    assert n == len(work)
    assert np.array_equal(_np(s["work"])[:n], work)
    assert np.all(_np(s["work"])[n:] == -1)


def test_varlen_schedule_limits():
    """Too small a work_cap gives n_work = -1; more than 16,384 tiles in one
    group of equal cost >> 12 gives n_work = -2; both leave every entry -1."""
    L = np.array([1000, 1000], np.int32)
    note("varlen schedule: work_cap too small")
    s = mfa.varlen_schedule(to_dev(L), causal=True, work_cap=10)
    torch.cuda.synchronize()
    assert int(_np(s["n_work"])[0]) == -1 and np.all(_np(s["work"]) == -1)
    L = np.array([16_385 * 128], np.int32)  # non-causal: every tile visits 32,770 key tiles
    note("varlen schedule: over-full long-cost group")
    s = mfa.varlen_schedule(to_dev(L), causal=False, work_cap=16_385)
    torch.cuda.synchronize()
    assert int(_np(s["n_work"])[0]) == -2 and np.all(_np(s["work"]) == -1)
