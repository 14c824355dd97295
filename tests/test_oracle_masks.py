"""Pins for the oracle's mask builders (CPU only).

Each test ties an oracle function to something other than itself: a worked
example from the pages, a closed form, an exhaustive brute force over tiny
inputs, or an independently written loop.
"""

import itertools

import numpy as np
import pytest

from oracle import masks as M
from tests.conftest import read_golden
import workloads as W


# --- block ids reproduce the dense mask exactly (opentau flash_attn_cuda) -------

def _all_patterns(N):
    bits = np.array(list(itertools.product([0, 1], repeat=N)), dtype=np.int32)
    pad = np.repeat(bits, len(bits), axis=0).astype(bool)
    att = np.tile(bits, (len(bits), 1))
    return pad, att


@pytest.mark.parametrize("N", [1, 2, 5, 7])
def test_blockid_rule_equals_bruteforce_exhaustive(N):
    pad, att = _all_patterns(N)
    dense = M.make_att_2d_masks(pad, att)
    qb, kb, qv, kv = M.make_att_block_ids(pad, att)
    assert np.array_equal(M.blockid_mask(qb, kb, qv, kv), dense)
    assert np.all(np.diff(qb, axis=1) >= 0)
    assert np.array_equal(qv, pad) and np.array_equal(kb, qb)


@pytest.mark.parametrize("N,Nc", [(4, 1), (5, 2), (3, 3)])
def test_blockid_rule_with_cross_columns_exhaustive(N, Nc):
    pad, att = _all_patterns(N)
    crosses = np.array(list(itertools.product([0, 1], repeat=Nc)), dtype=bool)
    for cp in crosses:
        cross = np.broadcast_to(cp, (pad.shape[0], Nc))
        dense = M.make_att_2d_masks(pad, att, cross)
        qb, kb, qv, kv = M.make_att_block_ids(pad, att, Nc, cross)
        assert np.array_equal(M.blockid_mask(qb, kb, qv, kv), dense)
        assert np.all(kb[:, :Nc] == np.iinfo(np.int32).min)
        assert np.array_equal(kv[:, :Nc], cross) and np.array_equal(kv[:, Nc:], pad)


def test_blockid_worked_example():
    g = read_golden("blockcausal_example.txt")
    att = np.array([g["att"]])
    pad = np.array([g["pad"]], dtype=bool)
    want = np.array([g[f"mask_row{i}"] for i in range(8)], dtype=bool)
    assert np.array_equal(M.make_att_2d_masks(pad, att)[0], want)
    qb, kb, qv, kv = M.make_att_block_ids(pad, att)
    assert np.array_equal(M.blockid_mask(qb, kb, qv, kv)[0], want)
    assert qb.dtype == np.int32 and qb.tolist() == [[1, 1, 1, 2, 2, 3, 3, 3]]


def test_cross_pad_required_iff_cross_tokens():
    pad = np.ones((1, 4), bool)
    att = np.ones((1, 4), np.int32)
    with pytest.raises(ValueError):
        M.make_att_block_ids(pad, att, 2, None)
    with pytest.raises(ValueError):
        M.make_att_block_ids(pad, att, None, np.ones((1, 2), bool))


def test_cross_columns_always_attended_subject_to_padding():
    w = W.blockcausal_gqa_cross(B=3, N=200, Nc=40, prefix=64, seed=11)
    dense = M.make_att_2d_masks(w["pad"], w["att"], w["cross_pad"])
    for b in range(3):
        valid_q = w["pad"][b]
        for c in range(40):
            col = dense[b, :, c]
            if w["cross_pad"][b, c]:
                assert np.array_equal(col, valid_q)
            else:
                assert not col.any()


# --- tile summaries of the block-id representation ----------------------------

@pytest.mark.parametrize("seed", range(6))
def test_blockid_tile_classification_exact(seed):
    rng = np.random.default_rng(100 + seed)
    B, Sq, Sk = 2, int(rng.integers(1, 300)), int(rng.integers(1, 300))
    BM, BN = [(128, 64), (64, 64), (32, 16)][seed % 3]
    if seed % 2:
        # arbitrary (non-monotone) ids and validity
        qb = rng.integers(-5, 6, (B, Sq)).astype(np.int32)
        kb = rng.integers(-5, 6, (B, Sk)).astype(np.int32)
        qv = rng.random((B, Sq)) < 0.8
        kv = rng.random((B, Sk)) < 0.8
    else:
        N = Sq
        att = (rng.random((B, N)) < 0.05).astype(np.int32)
        pad = np.ones((B, N), bool)
        pad[:, N - int(rng.integers(0, N // 2 + 1)):] = False
        qb, kb, qv, kv = M.make_att_block_ids(pad, att)
        Sk = N
    qsum, ksum, kv_bits = M.blockid_tile_summary(qb, kb, qv, kv, BM, BN)
    kinds = M.classify_from_summary(qsum, ksum)
    dense = M.blockid_mask(qb, kb, qv, kv)
    for b in range(B):
        assert np.array_equal(kinds[b], M.tile_kinds(dense[b], BM, BN))
        assert np.array_equal(M.unpack_bits_rows(kv_bits[b][None], Sk)[0], np.asarray(kv[b], bool))


# --- packed fine mask and tile map (BinFlash "Efficiently Dispatching ...") ----

def test_pack_bits_known_words():
    m = np.zeros((2, 40), bool)
    m[0, [0, 2, 3]] = True          # word 0 = 0b1101
    m[1, [31, 33]] = True           # word 0 bit 31, word 1 bit 1
    bits = M.pack_bits_rows(m)
    assert bits.dtype == np.uint32 and bits.shape == (2, 2)
    assert bits.tolist() == [[13, 0], [2 ** 31, 2]]


def test_pack_unpack_roundtrip_random():
    m = W.random_dense_mask(77, 301, 0.3, seed=5)
    bits = M.pack_bits_rows(m)
    assert np.array_equal(M.unpack_bits_rows(bits, 301), m)
    assert np.all(bits[:, -1] >> (301 - 32 * 9) == 0)  # pad bits are zero


def test_causal_closed_form_8192():
    g = read_golden("causal_tiles_8192.txt")
    N, BM, BN = g["N"][0], g["BM"][0], g["BN"][0]
    m = np.tril(np.ones((N, N), bool))
    c = M.compact_dense_mask(m, BM, BN)
    counts = np.bincount(c["tile_kind"].ravel(), minlength=3)
    assert counts.tolist() == [g["empty"][0], g["partial"][0], g["full"][0]]
    assert c["col_idx"].size == g["nnz"][0] == c["row_ptr"][-1]
    pc = np.unpackbits(c["fine_bits"].view(np.uint8)).sum()
    assert pc == g["popcount"][0] == N * (N + 1) // 2
    for qb in range(N // BM):
        lo, hi = c["row_ptr"][qb], c["row_ptr"][qb + 1]
        assert lo == qb * (qb + 1)
        assert c["col_idx"][lo:hi].tolist() == list(range(2 * qb + 2))
        assert c["col_kind"][lo:hi].tolist() == [2] * (2 * qb) + [1, 1]


def test_all_true_all_false_and_ragged():
    c = M.compact_dense_mask(np.ones((256, 256), bool), 128, 64)
    assert np.all(c["tile_kind"] == 2) and c["row_ptr"].tolist() == [0, 4, 8]
    c = M.compact_dense_mask(np.zeros((256, 256), bool), 128, 64)
    assert c["row_ptr"].tolist() == [0, 0, 0] and c["col_idx"].size == 0
    c = M.compact_dense_mask(np.ones((300, 130), bool), 128, 64)
    assert c["tile_kind"].tolist() == [[2, 2, 1], [2, 2, 1], [1, 1, 1]]


@pytest.mark.parametrize("seed", range(4))
def test_tile_kinds_match_loop_bruteforce(seed):
    rng = np.random.default_rng(seed)
    Nq, Nk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
    m = W.random_dense_mask(Nq, Nk, [0.0, 0.02, 0.5, 1.0][seed], seed)
    c = M.compact_dense_mask(m, 128, 64)
    k = c["tile_kind"]
    for qb in range(k.shape[0]):
        for kb in range(k.shape[1]):
            tile = np.zeros((128, 64), bool)
            sub = m[qb * 128:(qb + 1) * 128, kb * 64:(kb + 1) * 64]
            tile[:sub.shape[0], :sub.shape[1]] = sub
            want = 2 if tile.all() else (1 if tile.any() else 0)
            assert k[qb, kb] == want
    listed = [(r, c_) for r in range(k.shape[0])
              for c_ in c["col_idx"][c["row_ptr"][r]:c["row_ptr"][r + 1]]]
    assert listed == [tuple(x) for x in np.argwhere(k != 0)]


# --- BSR (flashinfer block_sparse_attention) -------------------------------------

def _small_bsr(seed=0, B=2, H=3, N=320, block=32):
    w = W.bsr_random(B=B, N=N, H=H, D=8, block=block, frac_den=3, seed=seed)
    return w["indptr"], w["indices"], N // block


def test_bsr_validate_accepts_and_reports_width():
    ip, ix, nb = _small_bsr()
    widest = M.bsr_validate(ip, ix, nb)
    rows = np.diff(ip, axis=2)
    assert widest == rows.max() == (nb - 1) // 3 + 1


@pytest.mark.parametrize("breakage", ["desc_ptr", "dup", "desc_idx", "oob", "neg", "ptr_past_end"])
def test_bsr_validate_rejects(breakage):
    ip, ix, nb = _small_bsr()
    ip, ix = ip.copy(), ix.copy()
    r = 5  # row (0, 0, 5) holds 2 entries: [x, 5]
    s = ip[0, 0, r]
    if breakage == "desc_ptr":
        ip[0, 0, r + 1] = ip[0, 0, r] - 1
    elif breakage == "dup":
        ix[s + 1] = ix[s]
    elif breakage == "desc_idx":
        ix[s], ix[s + 1] = ix[s + 1], ix[s]
    elif breakage == "oob":
        ix[s + 1] = nb
    elif breakage == "neg":
        ix[s] = -1
    elif breakage == "ptr_past_end":
        ip[-1, -1, -1] = ix.size + 1
    with pytest.raises(M.NonCanonicalBSR):
        M.bsr_validate(ip, ix, nb)


def test_bsr_full_lower_listing_with_causal_is_causal_mask():
    nb, blk = 6, 16
    rows = [list(range(r + 1)) for r in range(nb)]
    indptr = np.array([[[0] + list(np.cumsum([len(r) for r in rows]))]], np.int32)
    indices = np.concatenate([np.array(r, np.int32) for r in rows])
    m = M.bsr_mask(indptr, indices, blk, blk, nb * blk, nb * blk, causal=True)
    assert np.array_equal(m[0, 0], np.tril(np.ones((nb * blk, nb * blk), bool)))


def test_bsr_expanded_equals_listed_blocks_and_kinds():
    ip, ix, nb = _small_bsr(seed=3)
    blk = 32
    N = nb * blk
    m = M.bsr_mask(ip, ix, blk, blk, N, N, causal=True)
    kinds = M.bsr_col_kind(ip, ix, blk, blk, N, N, causal=True)
    for b in range(ip.shape[0]):
        for h in range(ip.shape[1]):
            tk = M.tile_kinds(m[b, h], blk, blk)
            listed = np.zeros((nb, nb), bool)
            for r in range(nb):
                for e in range(ip[b, h, r], ip[b, h, r + 1]):
                    listed[r, ix[e]] = True
                    assert kinds[e] == tk[r, ix[e]]
            assert np.all(tk[~listed] == 0)


def test_bsr_csc_roundtrip():
    ip, ix, nb = _small_bsr(seed=7)
    cp, ci = M.bsr_to_csc(ip, ix, nb)
    for b in range(ip.shape[0]):
        for h in range(ip.shape[1]):
            assert cp[b, h, 0] == ip[b, h, 0] and cp[b, h, -1] == ip[b, h, -1]
            rebuilt = [[] for _ in range(ip.shape[2] - 1)]
            for c in range(nb):
                col = ci[cp[b, h, c]:cp[b, h, c + 1]].tolist()
                assert col == sorted(col)
                for r in col:
                    rebuilt[r].append(c)
            for r in range(ip.shape[2] - 1):
                assert rebuilt[r] == ix[ip[b, h, r]:ip[b, h, r + 1]].tolist()


def _valid_keys(B, Skv, seed):
    rng = np.random.default_rng(seed)
    v = rng.random((B, Skv)) < 0.7
    v[0, 64:128] = False     # one whole 64-key block invalid in batch entry 0
    return v


def test_kv_valid_bits_roundtrip_and_kinds_against_bruteforce():
    """kv_valid_bits (flashinfer, Parameters): bits decode to the packing of
    pack_bits_rows; the per-entry kinds equal a brute-force classification of
    the dense mask, which is itself checked element by element against the
    definition (listed block, j <= i, valid key)."""
    ip, ix, nb = _small_bsr(seed=4, N=320, block=32)
    blk, N = 32, 320
    valid = _valid_keys(ip.shape[0], N, 5)
    bits = M.pack_bits_rows(valid)
    assert np.array_equal(M.kv_valid_from_bits(bits, N), valid)
    m = M.bsr_mask(ip, ix, blk, blk, N, N, causal=True, kv_valid=valid)
    kinds = M.bsr_col_kind(ip, ix, blk, blk, N, N, causal=True, kv_valid=valid)
    for b in range(ip.shape[0]):
        for h in range(ip.shape[1]):
            tk = M.tile_kinds(m[b, h], blk, blk)
            for r in range(nb):
                listed = set(ix[ip[b, h, r]:ip[b, h, r + 1]].tolist())
                for e in range(ip[b, h, r], ip[b, h, r + 1]):
                    assert kinds[e] == tk[r, ix[e]]
                for i in range(r * blk, (r + 1) * blk, 7):
                    for j in range(0, N, 5):
                        want = (j // blk) in listed and j <= i and bool(valid[b, j])
                        assert m[b, h, i, j] == want
    # the all-invalid block is never kept as partial or full
    sel = [e for e in range(ip[0, 0, -1]) if ix[e] in (2, 3)]
    assert sel and all(kinds[e] == M.EMPTY for e in range(ip[0, 0, 0], ip[0, 0, -1]) if ix[e] in (2, 3))


def test_bitmask_format_to_bsr_against_selection():
    """exact_block_bits (flashinfer, Parameters; sparse_format "bitmask"): a
    random block selection written as LSB-first words comes back as canonical
    BSR rows whose expansion at block size 1 is the selection itself."""
    rng = np.random.default_rng(11)
    B, H, R, nKb = 2, 3, 9, 70
    sel = rng.random((B, H, R, nKb)) < 0.2
    sel[0, 0, 0] = False
    sel[1, 2, 8] = True
    W_ = (nKb + 31) // 32
    bits = np.zeros((B, H, R, W_), np.uint32)
    for b, h, r, c in zip(*np.nonzero(sel)):
        bits[b, h, r, c // 32] |= np.uint32(1 << (c % 32))
    ip, ix = M.bsr_from_bitmask(bits, nKb)
    assert M.bsr_validate(ip, ix, nKb) == sel.sum(axis=3).max()
    assert np.array_equal(M.bsr_mask(ip, ix, 1, 1, R, nKb, causal=False), sel)
    assert ip[0, 0, 0] == 0 and ip[-1, -1, -1] == sel.sum()


# --- varlen packing (tensorplay varlen "Packed layout") ---------------------------

def test_cu_seqlens_worked_example():
    g = read_golden("cu_seqlens_example.txt")
    cu = M.cu_seqlens(g["lengths"])
    assert cu.dtype == np.int32 and cu.tolist() == g["cu_seqlens"]


def test_window_example_16():
    g = read_golden("causal_window_16.txt")
    m = M.create_mask(M.and_masks(M.causal, M.past_window(4)), 1, 1, 16, 16)[0, 0]
    assert m.sum(axis=1).tolist() == g["row_counts"] and m.sum() == g["total"][0]
    i, j = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    assert np.array_equal(M.window_allows(i, j, True, 3, -1), m)
    assert np.array_equal(M.window_allows(i, j, True, 3, 0), m)


def test_predicate_combinators():
    full = M.create_mask(M.noop_mask, 2, 3, 5, 7)
    assert full.all() and full.shape == (2, 3, 5, 7)
    c = M.create_mask(M.causal, 1, 1, 6, 6)[0, 0]
    assert np.array_equal(c, np.tril(np.ones((6, 6), bool)))
    either = M.create_mask(M.or_masks(M.causal, M.past_window(-100)), 1, 1, 6, 6)[0, 0]
    assert np.array_equal(either, c)
    neither = M.create_mask(M.and_masks(M.causal, M.past_window(-100)), 1, 1, 6, 6)[0, 0]
    assert not neither.any()


def test_window_wider_than_sequence_is_causal():
    cu = M.cu_seqlens([7, 3, 12])
    m_win = M.varlen_mask(cu, cu, True, 50, 0)
    m_c = M.varlen_mask(cu, cu, True, -1, -1)
    assert np.array_equal(m_win, m_c)
    for s in range(3):
        blk = m_c[cu[s]:cu[s + 1], cu[s]:cu[s + 1]]
        assert np.array_equal(blk, np.tril(np.ones_like(blk)))
    assert m_c.sum() == sum(L * (L + 1) // 2 for L in (7, 3, 12))


def test_varlen_schedule_costs_and_order():
    lengths = np.array([5, 300, 129, 1000, 64], np.int32)
    BM, BN, left = 128, 64, 200
    cu_q, cu_k, mq, mk, work = M.varlen_schedule(lengths, lengths, BM, BN, True, left, 0)
    assert mq == mk == 1000
    assert sorted(map(tuple, work.tolist())) == sorted(
        (s, q0) for s, L in enumerate(lengths) for q0 in range(0, L, BM))
    mask = M.varlen_mask(cu_q, cu_k, True, left, 0)
    costs = []
    for s, q0 in work.tolist():
        L = lengths[s]
        rows = mask[cu_q[s] + q0:cu_q[s] + min(q0 + BM, L), cu_k[s]:cu_k[s + 1]]
        touched = sum(rows[:, t * BN:(t + 1) * BN].any() for t in range(-(-L // BN)))
        costs.append(touched)
        assert touched == M.varlen_tile_cost(L, L, q0, BM, BN, True, left, 0)
    assert costs == sorted(costs, reverse=True)


def test_seqused_k_equals_dropping_the_unused_keys():
    """seqused_k (tensorplay varlen, intro): attention with the first
    seqused_k[s] keys of each sequence equals attention on a packed K/V from
    which the other keys were removed."""
    from oracle import attention as A
    rng = np.random.default_rng(12)
    Lq = np.array([5, 0, 17, 9])
    Lk = np.array([8, 3, 20, 9])
    used = np.array([3, 0, 20, 1])
    cq, ck = M.cu_seqlens(Lq), M.cu_seqlens(Lk)
    q = rng.standard_normal((int(cq[-1]), 2, 4))
    k = rng.standard_normal((int(ck[-1]), 2, 4))
    v = rng.standard_normal((int(ck[-1]), 2, 4))
    for causal, win in ((False, (-1, -1)), (True, (-1, -1)), (False, (2, 1))):
        out, lse = A.varlen_attention_fwd(q, k, v, cq, ck, 0.5, causal, win[0], win[1], seqused_k=used)
        keep = np.concatenate([np.arange(ck[s], ck[s] + used[s]) for s in range(4)])
        o2, l2 = A.varlen_attention_fwd(q, k[keep], v[keep], cq, M.cu_seqlens(used), 0.5, causal, win[0], win[1])
        np.testing.assert_allclose(out, o2, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse, l2, rtol=1e-13)
        m = M.varlen_mask(cq, ck, causal, win[0], win[1], seqused_k=used)
        m2 = M.varlen_mask(cq, M.cu_seqlens(used), causal, win[0], win[1])
        assert np.array_equal(m[:, keep], m2) and not m[:, np.setdiff1d(np.arange(int(ck[-1])), keep)].any()


def test_paged_gather_inverts_a_scatter_into_shuffled_pages():
    """block_table (tensorplay varlen, intro): scattering a packed K into pages
    in a random order and gathering through the table gives K back."""
    rng = np.random.default_rng(13)
    lengths = np.array([130, 1, 0, 64, 200])
    page, H, D = 64, 2, 3
    T = int(lengths.sum())
    k = rng.standard_normal((T, H, D))
    npg = [(int(L) + page - 1) // page for L in lengths]
    n_pages = sum(npg) + 3
    perm = rng.permutation(n_pages)
    pages = np.full((n_pages, page, H, D), np.nan)
    table = np.full((lengths.size, max(npg)), -1, np.int32)
    nxt, off = 0, 0
    for s, L in enumerate(lengths):
        for pi in range(npg[s]):
            table[s, pi] = perm[nxt]
            nxt += 1
        for j in range(int(L)):
            pages[table[s, j // page], j % page] = k[off + j]
        off += int(L)
    assert np.array_equal(M.paged_to_packed(pages, table, lengths, page), k)


def test_splitmix64_published_vector():
    """The input generator shared with the C client: SplitMix64 from seed
    1234567 gives the reference implementation's first five outputs."""
    from workloads.splitmix import splitmix64
    z, st = splitmix64(1234567, 5)
    assert [int(x) for x in z] == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                                   4593380528125082431, 16408922859458223821]
    z2, _ = splitmix64(st, 1)
    z3, _ = splitmix64(1234567, 6)
    assert int(z2[0]) == int(z3[5])
