"""Brute-force mask builders and mask-representation outputs (fp-free, exact).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Every builder here is written from the plain definition on the pages, with
NumPy loops or broadcasting; none of them reuses the GPU library's layout code.
Conventions fixed here (readings where the pages are silent):

* block ids are the inclusive prefix sum of the block-opening flags (int32);
* cross-attention key columns are prepended and carry block id -2**31;
* a tile is "full" only if every in-range and out-of-range position of it is
  allowed; out-of-range positions count as not allowed, so a ragged edge tile is
  never full;
* packed bits are LSB-first 32-bit words per row, pad bits zero;
* tile-kind codes: 0 empty, 1 partial, 2 full.
"""

from __future__ import annotations

import numpy as np

INT32_MIN = np.int32(-(2 ** 31))
INT32_MAX = np.int32(2 ** 31 - 1)
EMPTY, PARTIAL, FULL = 0, 1, 2


# ---------------------------------------------------------------------------
# Block-causal masks from pad/att flags
# (opentau.policies.flash_attn_cuda: module description and make_att_block_ids)
# ---------------------------------------------------------------------------

def make_att_2d_masks(pad_masks, att_masks, cross_att_pad_masks=None):
    """Dense (B, N, Nc+N) attend mask built WITHOUT prefix sums.

    Follows the convention the opentau page states for ``make_att_2d_masks``
    (parameters of ``make_att_block_ids``): a nonzero att flag opens a new
    attention block, zero continues the current one; True = attend; padded
    tokens neither attend nor are attended; prepended cross-attention columns
    are attended by every real query, subject to their own padding.

    Pairwise reading used here: query i may see self key j iff both are real
    and either j <= i (same or earlier block: blocks only open going forward)
    or no block opens at any position t with i < t <= j (same block).
    """
    pad = np.asarray(pad_masks).astype(bool)
    opener = np.asarray(att_masks) != 0
    B, N = pad.shape
    nc = 0 if cross_att_pad_masks is None else np.asarray(cross_att_pad_masks).shape[1]
    out = np.zeros((B, N, nc + N), dtype=bool)
    j = np.arange(N)
    for b in range(B):
        # next_open[i] = first position t > i that opens a block (N if none)
        next_open = np.full(N, N, dtype=np.int64)
        nxt = N
        for i in range(N - 1, -1, -1):
            next_open[i] = nxt
            if opener[b, i]:
                nxt = i
        for i in range(N):
            if not pad[b, i]:
                continue
            see = pad[b] & ((j <= i) | (j < next_open[i]))
            out[b, i, nc:] = see
            if nc:
                out[b, i, :nc] = np.asarray(cross_att_pad_masks)[b].astype(bool)
    return out


def make_att_block_ids(pad_masks, att_masks, n_cross_att_tokens=None, cross_att_pad_masks=None):
    """(q_blk, k_blk, q_valid, k_valid) per the opentau ``make_att_block_ids`` docs.

    q_blk is the inclusive running count of block openers (int32; a flag of
    1 starts a new attention block); k_blk prepends ``n_cross_att_tokens``
    columns of INT32_MIN to q_blk; q_valid = pad; k_valid = [cross pad ; pad].
    ``cross_att_pad_masks`` is required iff ``n_cross_att_tokens`` is set.
    """
    if (n_cross_att_tokens is None) != (cross_att_pad_masks is None):
        raise ValueError("cross_att_pad_masks is required iff n_cross_att_tokens is set")
    pad = np.asarray(pad_masks).astype(bool)
    att = np.asarray(att_masks)
    B, N = pad.shape
    q_blk = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        run = 0
        for i in range(N):
            if att[b, i] != 0:
                run += 1
            q_blk[b, i] = run
    nc = 0 if n_cross_att_tokens is None else int(n_cross_att_tokens)
    cross = np.zeros((B, nc), dtype=bool) if nc == 0 else np.asarray(cross_att_pad_masks).astype(bool)
    if cross.shape != (B, nc):
        raise ValueError("cross_att_pad_masks must be (B, n_cross_att_tokens)")
    k_blk = np.concatenate([np.full((B, nc), INT32_MIN, dtype=np.int32), q_blk], axis=1)
    k_valid = np.concatenate([cross, pad], axis=1)
    return q_blk, k_blk, pad.copy(), k_valid


def blockid_mask(q_blk, k_blk, q_valid, k_valid):
    """attend(i, j) = q_valid[i] & k_valid[j] & (k_blk[j] <= q_blk[i]), (B, Sq, Sk).

    The reconstruction rule quoted for ``make_att_block_ids`` / ``flash_attn_blockmask``.
    """
    qb = np.asarray(q_blk).astype(np.int64)
    kb = np.asarray(k_blk).astype(np.int64)
    return (np.asarray(q_valid).astype(bool)[:, :, None]
            & np.asarray(k_valid).astype(bool)[:, None, :]
            & (kb[:, None, :] <= qb[:, :, None]))


# ---------------------------------------------------------------------------
# Tile classification
# ---------------------------------------------------------------------------

def tile_kinds(mask2d, BM, BN):
    """Kind of every BM x BN tile of one (Nq, Nk) bool mask, (nQt, nKt) uint8.

    BinFlash, "Efficiently Dispatching ...": all-True tiles run without mask
    loads, all-False tiles are skipped, the rest use the fine mask. Positions
    outside the mask count as False (reading for ragged edges).
    """
    m = np.asarray(mask2d).astype(bool)
    Nq, Nk = m.shape
    nQt, nKt = -(-Nq // BM), -(-Nk // BN)
    padded = np.zeros((nQt * BM, nKt * BN), dtype=bool)
    padded[:Nq, :Nk] = m
    t = padded.reshape(nQt, BM, nKt, BN)
    anyv = t.any(axis=(1, 3))
    allv = t.all(axis=(1, 3))
    kinds = np.where(allv, FULL, np.where(anyv, PARTIAL, EMPTY)).astype(np.uint8)
    return kinds


def blockid_tile_summary(q_blk, k_blk, q_valid, k_valid, BM, BN):
    """Per-tile summaries of the block-id representation.

    Returns qsum (B, nQt, 4) and ksum (B, nKt, 4) int32 rows
    {min id over valid tokens, max id over valid tokens, any valid, all valid}
    (min = INT32_MAX / max = INT32_MIN when no token is valid; out-of-range
    positions are not valid), and kv_bits (B, ceil(Sk/32)) uint32, the key
    validity packed LSB-first like the flashinfer page's ``kv_valid_bits``.
    """
    def summarise(ids, valid, T):
        ids = np.asarray(ids).astype(np.int64)
        valid = np.asarray(valid).astype(bool)
        B, S = ids.shape
        n = -(-S // T)
        res = np.zeros((B, n, 4), dtype=np.int32)
        for b in range(B):
            for t in range(n):
                lo, hi = t * T, min((t + 1) * T, S)
                vv = valid[b, lo:hi]
                sel = ids[b, lo:hi][vv]
                res[b, t, 0] = sel.min() if sel.size else INT32_MAX
                res[b, t, 1] = sel.max() if sel.size else INT32_MIN
                res[b, t, 2] = 1 if vv.any() else 0
                res[b, t, 3] = 1 if (hi - lo == T and vv.all()) else 0
        return res

    qsum = summarise(q_blk, q_valid, BM)
    ksum = summarise(k_blk, k_valid, BN)
    kv = np.asarray(k_valid).astype(bool)
    kv_bits = np.stack([pack_bits_rows(kv[b][None, :])[0] for b in range(kv.shape[0])])
    return qsum, ksum, kv_bits


def classify_from_summary(qsum, ksum):
    """Tile kinds (B, nQt, nKt) from the block-id summaries.

    Empty iff no valid query, no valid key, or the smallest valid key id
    exceeds the largest valid query id; full iff every query and key of the
    tile is valid and the largest key id is <= the smallest query id; else
    partial. Pinned against ``tile_kinds(blockid_mask(...))``.
    """
    q = np.asarray(qsum).astype(np.int64)
    k = np.asarray(ksum).astype(np.int64)
    qmin, qmax, qany, qall = (q[:, :, None, c] for c in range(4))
    kmin, kmax, kany, kall = (k[:, None, :, c] for c in range(4))
    empty = (qany == 0) | (kany == 0) | (kmin > qmax)
    full = (qall == 1) & (kall == 1) & (kmax <= qmin)
    return np.where(empty, EMPTY, np.where(full, FULL, PARTIAL)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Dense (N, N) bool mask -> coarse tile map + packed fine mask + sorted lists
# (BinFlash, "Efficiently Dispatching FlashAttention For Partially Filled
#  Attention Masks")
# ---------------------------------------------------------------------------

def pack_bits_rows(mask2d):
    """(Nq, Nk) bool -> (Nq, ceil(Nk/32)) uint32, bit b of word w = mask[i, 32w+b]."""
    m = np.asarray(mask2d).astype(bool)
    Nq, Nk = m.shape
    W = -(-Nk // 32)
    padded = np.zeros((Nq, W * 32), dtype=bool)
    padded[:, :Nk] = m
    by = np.packbits(padded, axis=1, bitorder="little")  # (Nq, 4W) bytes, LSB-first
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32).reshape(Nq, W)


def unpack_bits_rows(bits, Nk):
    b = np.ascontiguousarray(np.asarray(bits, dtype="<u4"))
    by = b.view(np.uint8).reshape(b.shape[0], -1)
    return np.unpackbits(by, axis=1, bitorder="little")[:, :Nk].astype(bool)


def compact_dense_mask(mask2d, BM, BN):
    """Coarse tile map, packed fine mask and per-Q-tile ascending non-empty K-tile list.

    Output dict: tile_kind (nQt, nKt) u8; fine_bits (Nq, ceil(Nk/32)) u32;
    row_ptr (nQt+1,) i32; col_idx (nnz,) i32 ascending within each row;
    col_kind (nnz,) u8 (1 partial, 2 full).
    """
    kinds = tile_kinds(mask2d, BM, BN)
    rows, cols = np.nonzero(kinds != EMPTY)  # row-major, ascending columns per row
    nQt = kinds.shape[0]
    counts = np.bincount(rows, minlength=nQt)
    row_ptr = np.zeros(nQt + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    return {
        "tile_kind": kinds,
        "fine_bits": pack_bits_rows(mask2d),
        "row_ptr": row_ptr,
        "col_idx": cols.astype(np.int32),
        "col_kind": kinds[rows, cols].astype(np.uint8),
    }


# ---------------------------------------------------------------------------
# BSR block sparsity (flashinfer.attention.prims_ts.block_sparse_attention)
# ---------------------------------------------------------------------------

class NonCanonicalBSR(ValueError):
    pass


def bsr_validate(block_indptr, block_indices, n_kv_blocks):
    """Check canonical rows and return the widest row.

    indptr (B, Hkv, nQb+1) holds offsets into the one flat ``indices`` array;
    a row must have non-decreasing offsets within [0, len(indices)] and
    strictly ascending KV-block ids in [0, n_kv_blocks).
    """
    ip = np.asarray(block_indptr).astype(np.int64)
    ix = np.asarray(block_indices).astype(np.int64)
    if ip.ndim != 3 or ip.shape[2] < 1:
        raise NonCanonicalBSR("indptr must be (B, Hkv, nQb+1)")
    widest = 0
    for b in range(ip.shape[0]):
        for h in range(ip.shape[1]):
            p = ip[b, h]
            if p[0] < 0 or p[-1] > ix.size or np.any(np.diff(p) < 0):
                raise NonCanonicalBSR(f"row offsets of (b={b}, h={h}) are not non-decreasing within range")
            for r in range(p.size - 1):
                row = ix[p[r]:p[r + 1]]
                if row.size and (row.min() < 0 or row.max() >= n_kv_blocks):
                    raise NonCanonicalBSR(f"block id out of range in (b={b}, h={h}, r={r})")
                if np.any(np.diff(row) <= 0):
                    raise NonCanonicalBSR(f"block ids not strictly ascending in (b={b}, h={h}, r={r})")
                widest = max(widest, row.size)
    return widest


def bsr_entry_kind(r, c, q_block, kv_block, Sq, Skv, causal):
    """Kind of listed block (r, c): token-level causal j <= i on global positions."""
    i0, i1 = r * q_block, min((r + 1) * q_block, Sq) - 1
    j0, j1 = c * kv_block, min((c + 1) * kv_block, Skv) - 1
    ragged = (i1 - i0 + 1 != q_block) or (j1 - j0 + 1 != kv_block)
    if i1 < i0 or j1 < j0:
        return EMPTY
    if not causal:
        return PARTIAL if ragged else FULL
    if j0 > i1:
        return EMPTY
    if j1 <= i0 and not ragged:
        return FULL
    return PARTIAL


def kv_valid_from_bits(kv_valid_bits, Skv):
    """(B, Skv) bool from the (B, ceil(Skv/32)) u32 token-validity bitmap
    (flashinfer block_sparse_attention, Parameters: kv_valid_bits), LSB-first."""
    w = np.asarray(kv_valid_bits).astype(np.uint64)
    out = np.zeros((w.shape[0], Skv), dtype=bool)
    for b in range(w.shape[0]):
        for j in range(Skv):
            out[b, j] = (int(w[b, j // 32]) >> (j % 32)) & 1 == 1
    return out


def bsr_entry_kind_valid(r, c, q_block, kv_block, Sq, Skv, causal, kv_valid_row):
    """Kind of listed block (r, c) when only the keys with kv_valid_row[j] may be
    attended: no valid key in the block makes it empty, an invalid key makes a
    full block partial."""
    kind = bsr_entry_kind(r, c, q_block, kv_block, Sq, Skv, causal)
    if kind == EMPTY or kv_valid_row is None:
        return kind
    seg = np.asarray(kv_valid_row)[c * kv_block:min((c + 1) * kv_block, Skv)]
    if not seg.any():
        return EMPTY
    if kind == FULL and not seg.all():
        return PARTIAL
    return kind


def bsr_col_kind(block_indptr, block_indices, q_block, kv_block, Sq, Skv, causal, kv_valid=None):
    ip = np.asarray(block_indptr).astype(np.int64)
    ix = np.asarray(block_indices).astype(np.int64)
    kind = np.zeros(ix.size, dtype=np.uint8)
    for b in range(ip.shape[0]):
        for h in range(ip.shape[1]):
            for r in range(ip.shape[2] - 1):
                for e in range(ip[b, h, r], ip[b, h, r + 1]):
                    kind[e] = bsr_entry_kind_valid(r, int(ix[e]), q_block, kv_block, Sq, Skv, causal,
                                                   None if kv_valid is None else kv_valid[b])
    return kind


def bsr_to_csc(block_indptr, block_indices, n_kv_blocks):
    """Column-major copy of each (b, h) row list, for the dK/dV pass over K blocks.

    csc_ptr (B, Hkv, nKb+1): offsets into csc_idx, the (b, h) segment starting
    where its CSR segment starts (indptr[b, h, 0]); csc_idx lists, per KV
    block, the query-block rows that reference it, ascending.
    """
    ip = np.asarray(block_indptr).astype(np.int64)
    ix = np.asarray(block_indices).astype(np.int64)
    B, H, R1 = ip.shape
    csc_ptr = np.zeros((B, H, n_kv_blocks + 1), dtype=np.int32)
    csc_idx = np.zeros(ix.size, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            cols = [[] for _ in range(n_kv_blocks)]
            for r in range(R1 - 1):
                for e in range(ip[b, h, r], ip[b, h, r + 1]):
                    cols[int(ix[e])].append(r)
            pos = int(ip[b, h, 0])
            for c in range(n_kv_blocks):
                csc_ptr[b, h, c] = pos
                for r in cols[c]:
                    csc_idx[pos] = r
                    pos += 1
            csc_ptr[b, h, n_kv_blocks] = pos
    return csc_ptr, csc_idx


def bsr_mask(block_indptr, block_indices, q_block, kv_block, Sq, Skv, causal, kv_valid=None):
    """Dense (B, Hkv, Sq, Skv) mask: listed blocks, intersected with j <= i if
    causal and with the valid keys (kv_valid (B, Skv) bool) if given."""
    ip = np.asarray(block_indptr).astype(np.int64)
    ix = np.asarray(block_indices).astype(np.int64)
    B, H, R1 = ip.shape
    m = np.zeros((B, H, Sq, Skv), dtype=bool)
    for b in range(B):
        for h in range(H):
            for r in range(R1 - 1):
                for e in range(ip[b, h, r], ip[b, h, r + 1]):
                    c = int(ix[e])
                    m[b, h, r * q_block:(r + 1) * q_block, c * kv_block:(c + 1) * kv_block] = True
    if causal:
        m &= np.tri(Sq, Skv, dtype=bool)[None, None]
    if kv_valid is not None:
        m &= np.asarray(kv_valid, dtype=bool)[:, None, None, :]
    return m


def bsr_from_bitmask(bits, n_kv_blocks):
    """BSR rows from the exact-block bitmap of the bitmask sparse format
    (flashinfer block_sparse_attention, Parameters: exact_block_bits,
    sparse_format): bits (B, Hkv, nQb, ceil(nKb/32)) u32, LSB-first; bit c of
    row r selects KV block c. Returns indptr (B, Hkv, nQb+1) with one running
    offset over all rows, and the ascending block ids."""
    w = np.asarray(bits).astype(np.uint64)
    B, H, R = w.shape[:3]
    indptr = np.zeros((B, H, R + 1), dtype=np.int64)
    ids = []
    run = 0
    for b in range(B):
        for h in range(H):
            indptr[b, h, 0] = run
            for r in range(R):
                for c in range(n_kv_blocks):
                    if (int(w[b, h, r, c // 32]) >> (c % 32)) & 1:
                        ids.append(c)
                        run += 1
                indptr[b, h, r + 1] = run
    return indptr.astype(np.int32), np.asarray(ids, dtype=np.int32)


# ---------------------------------------------------------------------------
# Variable-length packing (tensorplay.nn.attention.varlen, "Packed layout")
# ---------------------------------------------------------------------------

def cu_seqlens(lengths):
    """Cumulative lengths starting at 0, int32 (worked example: 5, 11 -> 0, 5, 16)."""
    L = np.asarray(lengths).astype(np.int64)
    out = np.zeros(L.size + 1, dtype=np.int64)
    for s in range(L.size):
        out[s + 1] = out[s] + L[s]
    return out.astype(np.int32)


def window_allows(i, j, causal, left, right):
    """Sliding-window predicate on sequence-local positions; -1 = unbounded side.

    (-1, -1) disables the window (varlen page); a window of the previous W
    keys means i - j < W, i.e. left = W - 1 (omni_attention "Block masks" example).
    """
    i = np.asarray(i)
    j = np.asarray(j)
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        ok &= j <= i
    if left >= 0:
        ok &= (i - j) <= left
    if right >= 0:
        ok &= (j - i) <= right
    return ok


def varlen_mask(cu_q, cu_k, causal, left, right, seqused_k=None):
    """Packed (Tq, Tk) mask: same sequence and window predicate on local
    positions; with ``seqused_k`` only the first seqused_k[s] keys of sequence s
    may be attended (tensorplay varlen, intro: seqused_k bounds the usable key
    length)."""
    cq = np.asarray(cu_q).astype(np.int64)
    ck = np.asarray(cu_k).astype(np.int64)
    Tq, Tk = int(cq[-1]), int(ck[-1])
    m = np.zeros((Tq, Tk), dtype=bool)
    for s in range(cq.size - 1):
        qi = np.arange(cq[s + 1] - cq[s])
        kj = np.arange(ck[s + 1] - ck[s])
        ok = window_allows(qi[:, None], kj[None, :], causal, left, right)
        if seqused_k is not None:
            ok &= kj[None, :] < int(seqused_k[s])
        m[cq[s]:cq[s + 1], ck[s]:ck[s + 1]] = ok
    return m


def paged_to_packed(pages, block_table, lengths, page_size):
    """Gather paged key/value storage into the packed layout (tensorplay
    varlen, intro: block_table points at paged key/value blocks). pages
    (n_pages, page_size, H, D); block_table (nseq, max_pages) page ids; key j
    of sequence s sits at row j % page_size of page block_table[s, j //
    page_size]. Returns (sum(lengths), H, D)."""
    out = []
    for s, L in enumerate(np.asarray(lengths).astype(np.int64)):
        for j in range(int(L)):
            out.append(np.asarray(pages[int(block_table[s][j // page_size]), j % page_size]))
    if not out:
        return np.zeros((0,) + tuple(np.asarray(pages).shape[2:]))
    return np.stack(out)


def varlen_tile_cost(Lq, Lk, q0, BM, BN, causal, left, right):
    """Number of BN-key tiles (aligned to the sequence start) a BM-query tile at q0 visits."""
    q1 = min(q0 + BM, Lq) - 1
    lo = max(0, q0 - left) if left >= 0 else 0
    hi = Lk - 1
    if right >= 0:
        hi = min(hi, q1 + right)
    if causal:
        hi = min(hi, q1)
    if hi < lo:
        return 0
    return hi // BN - lo // BN + 1


def varlen_schedule(lengths_q, lengths_k, BM, BN, causal, left, right):
    """Work list of (seq, q0) query tiles, most key tiles first.

    Order: descending number of visited key tiles, ties by ascending (seq, q0).
    Returns cu_q, cu_k, max_q, max_k and work (n, 2) int32.
    """
    Lq = np.asarray(lengths_q).astype(np.int64)
    Lk = np.asarray(lengths_k).astype(np.int64)
    items = []
    for s in range(Lq.size):
        for q0 in range(0, int(Lq[s]), BM):
            cost = varlen_tile_cost(int(Lq[s]), int(Lk[s]), q0, BM, BN, causal, left, right)
            items.append((-cost, s, q0))
    items.sort()
    work = np.array([[s, q0] for _, s, q0 in items], dtype=np.int32).reshape(-1, 2)
    return (cu_seqlens(Lq), cu_seqlens(Lk), int(Lq.max(initial=0)), int(Lk.max(initial=0)), work)


# ---------------------------------------------------------------------------
# Predicates (tensorplay.nn.attention.omni_attention, "Block masks")
# ---------------------------------------------------------------------------

def causal(b, h, q_idx, kv_idx):
    """Key at or before the query: the causal window with both sides open."""
    return window_allows(q_idx, kv_idx, True, -1, -1)


def past_window(w):
    """Keys less than w positions back from the query (w of them including
    the query's own position); keys after the query are not restricted here,
    so it is combined with ``causal`` for a causal sliding window."""
    def pred(b, h, q_idx, kv_idx):
        if w <= 0:  # the key must then lie at least 1 - w positions after the query
            return np.asarray(kv_idx) - np.asarray(q_idx) >= 1 - w
        return window_allows(q_idx, kv_idx, False, w - 1, -1)
    return pred


def noop_mask(b, h, q_idx, kv_idx):
    return np.ones(np.broadcast(b, h, q_idx, kv_idx).shape, dtype=bool)


def and_masks(*preds):
    def pred(b, h, q_idx, kv_idx):
        out = noop_mask(b, h, q_idx, kv_idx)
        for p in preds:
            out = out & p(b, h, q_idx, kv_idx)
        return out
    return pred


def or_masks(*preds):
    def pred(b, h, q_idx, kv_idx):
        out = ~noop_mask(b, h, q_idx, kv_idx)
        for p in preds:
            out = out | p(b, h, q_idx, kv_idx)
        return out
    return pred


def create_mask(pred, B, H, Q_LEN, KV_LEN):
    """Materialise a predicate as a dense (B, H, Q_LEN, KV_LEN) bool array."""
    b = np.arange(B)[:, None, None, None]
    h = np.arange(H)[None, :, None, None]
    qi = np.arange(Q_LEN)[None, None, :, None]
    kj = np.arange(KV_LEN)[None, None, None, :]
    return np.broadcast_to(pred(b, h, qi, kj), (B, H, Q_LEN, KV_LEN)).copy()
