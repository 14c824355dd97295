// Per-workgroup tile schedule and per-element mask predicates, shared by the
// bf16 MFMA forward kernel, the fp32 test-mode kernel and the backward dQ
// pass (which walks the same key tiles as the forward).
//
// A workgroup owns one query tile of BM rows of one (batch, query head) (or of
// one varlen sequence). It walks only the key tiles that can hold an allowed
// entry: the CSR list of non-empty tiles (dense-mask tiles, as in the BinFlash
// method's sorted per-query-tile list of non-empty key tiles), the BSR row
// (flashinfer block_sparse_attention), the key-tile range of the sliding
// window (varlen), or every key tile classified from block-id summaries
// (opentau block ids). Full tiles skip the mask entirely; partial tiles
// evaluate the predicate per element.
#pragma once

#include "common.hpp"

namespace mfa {

constexpr int kBN = 64;  // key-tile width of every forward kernel

struct TileRange {
    int b, hq, hk;
    int qt;         // query-tile index in the representation's tile grid
    int q_row0;     // first query row of the tile (row index along Sq)
    int q_rows;     // rows of the tile that exist (<= BM)
    int q_base;     // varlen: cu_q[seq]; local query index = row - q_base
    int k_base;     // varlen: cu_k[seq]; key rows are k_base + local key index
    int k_len;      // keys that exist (Sk or the sequence's key length)
    int begin, end; // iteration range
    int seq;        // varlen sequence (-1 otherwise)
    bool active;
    bool len_error; // varlen: sequence longer than the stated max_q / max_k
};

// BN is the key-tile width the caller walks: kBN, or 32 for BSR rows, whose
// 64-key blocks are then visited as two 32-key tiles each.
template <int KIND, int BM, int BN = kBN>
__device__ __forceinline__ TileRange make_range(const FwdDev& p, const MaskDev& m, int logical) {
    static_assert(BN == kBN || (BN == 32 && (KIND == MFA_MASK_BSR || KIND == MFA_MASK_TILES)),
                  "32-key tiles are built for BSR rows and dense-mask tile lists only");
    TileRange t;
    t.seq = -1;
    t.active = true;
    t.len_error = false;
    t.q_base = 0;
    t.k_base = 0;
    t.k_len = p.Sk;
    if constexpr (KIND == MFA_MASK_VARLEN) {
        const int wi = logical / p.Hq;
        t.hq = logical - wi * p.Hq;
        t.b = 0;
        t.hk = t.hq / p.G;
        int s = -1, q0 = 0;
        if (wi < m.work_cap) {
            s = m.work[2 * wi];
            q0 = m.work[2 * wi + 1];
        }
        if (s < 0) {
            t.active = false;
            t.begin = t.end = 0;
            t.q_rows = 0;
            t.q_row0 = 0;
            t.qt = 0;
            return t;
        }
        t.seq = s;
        const int cq0 = m.cu_q[s], cq1 = m.cu_q[s + 1];
        const int ck0 = m.cu_k[s], ck1 = m.cu_k[s + 1];
        const int Lq = cq1 - cq0, Lk_alloc = ck1 - ck0;
        const int Lk = m.seqused_k ? min(Lk_alloc, max(m.seqused_k[s], 0)) : Lk_alloc;
        t.q_base = cq0;
        t.k_base = m.block_table ? 0 : ck0;  // paged keys are addressed through the block table
        t.k_len = m.block_table ? min(Lk, m.max_pages * m.page_size) : Lk;
        t.qt = q0 / BM;
        t.q_row0 = cq0 + q0;
        t.q_rows = min(BM, Lq - q0);
        const int i1 = q0 + t.q_rows - 1;
        int lo = 0, hi = t.k_len - 1;
        if (m.win_left >= 0) lo = max(0, q0 - m.win_left);
        if (m.win_right >= 0) hi = min(hi, i1 + m.win_right);
        if (m.causal) hi = min(hi, i1);
        if (hi < lo) {
            t.begin = t.end = 0;
        } else {
            t.begin = lo / kBN;
            t.end = hi / kBN + 1;
        }
        bool bad = Lq > m.max_q || Lk_alloc > m.max_k;
        if (m.block_table) {
            // a sequence that needs more pages than a table row holds, or
            // whose used pages include an id outside [0, n_pages), is an error
            bad = bad || Lk > m.max_pages * m.page_size;
            const int32_t* tb = m.block_table + (int64_t)s * m.max_pages;
            const int npg = (t.k_len + m.page_size - 1) / m.page_size;
            for (int pi = 0; pi < npg; ++pi) bad = bad || tb[pi] < 0 || tb[pi] >= m.n_pages;
        }
        if (bad) {
            t.len_error = true;
            if (m.err) *m.err = 1;
        }
        return t;
    } else {
        int bh, lvl;  // lvl: query tiles from the last one, heaviest first
        if (p.lpt_group > 0) {
            const int run = p.lpt_group * p.nQt;
            const int c = logical / run, i = logical - c * run;
            lvl = i / p.lpt_group;
            bh = c * p.lpt_group + (i - lvl * p.lpt_group);
        } else {
            bh = logical / p.nQt;
            lvl = logical - bh * p.nQt;
        }
        t.qt = p.nQt - 1 - lvl;
        t.b = bh / p.Hq;
        t.hq = bh - t.b * p.Hq;
        t.hk = t.hq / p.G;
        t.q_row0 = t.qt * BM;
        t.q_rows = min(BM, p.Sq - t.q_row0);
        if constexpr (KIND == MFA_MASK_TILES) {
            t.begin = m.row_ptr[t.qt] * (kBN / BN);
            t.end = m.row_ptr[t.qt + 1] * (kBN / BN);
        } else if constexpr (KIND == MFA_MASK_BSR) {
            const int* ip = m.indptr + ((int64_t)t.b * p.Hkv + t.hk) * (m.nQb + 1);
            t.begin = ip[t.qt] * (kBN / BN);
            t.end = ip[t.qt + 1] * (kBN / BN);
        } else {
            t.begin = 0;
            t.end = p.nKt;
        }
        return t;
    }
}

// Positional bias slope * (kv_idx - q_idx) (the distance-decay score_mod of
// tensorplay omni_attention, intro, with a slope per query head) in raw score
// units, sl = slope / scale, written into a pair of score accumulators before
// the q.k contraction adds onto them. Register r of half h holds the element at
// offset h*32 + (r>>2)*8 + (r&3) along the accumulator's row axis; d0 is
// kv_idx - q_idx of offset 0 and `step` the bias change per unit offset (sl
// when the row axis runs over keys, -sl when it runs over queries).
template <int NB>
__device__ __forceinline__ void alibi_fill(f32x16 (&s)[NB], float sl, int d0, float step) {
    const float base = sl * (float)d0;
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[h][r] = fmaf(step, (float)(h * 32 + (r >> 2) * 8 + (r & 3)), base);
}

// Paged keys (varlen with a block table): the page holding local key `key`
// of sequence `seq` (-1 when the table's id is not a page) and the key's row
// in it. k / v are then addressed as (page, row, head). Pages hold page_size
// rows, a multiple of the 64-key tile, so a tile never straddles two pages.
__device__ __forceinline__ int page_of(const MaskDev& m, int seq, int key, int& row) {
    const int pg = m.block_table[(int64_t)seq * m.max_pages + key / m.page_size];
    row = key % m.page_size;
    return (pg >= 0 && pg < m.n_pages) ? pg : -1;
}

// Kind of a listed BSR block (r, c) with qb x kb blocks: token-level causal
// j <= i on global positions inside the block when `causal` (mask_type
// "causal" of flashinfer block_sparse_attention); out-of-range positions are
// not allowed, so a ragged block is never full.
__host__ __device__ __forceinline__ int bsr_kind_of(int r, int c, int qb, int kb, int Sq, int Skv, int causal) {
    const int i0 = r * qb, i1 = min((r + 1) * qb, Sq) - 1;
    const int j0 = c * kb, j1 = min((c + 1) * kb, Skv) - 1;
    if (i1 < i0 || j1 < j0) return kTileEmpty;
    const bool ragged = (i1 - i0 + 1 != qb) || (j1 - j0 + 1 != kb);
    if (!causal) return ragged ? kTilePartial : kTileFull;
    if (j0 > i1) return kTileEmpty;
    if (j1 <= i0 && !ragged) return kTileFull;
    return kTilePartial;
}

// Block-id tile classification from the per-tile summaries {min, max, any, all}.
__device__ __forceinline__ int classify_blockid(const int32_t* qs, const int32_t* ks) {
    const int qmin = qs[0], qmax = qs[1], qany = qs[2], qall = qs[3];
    const int kmin = ks[0], kmax = ks[1], kany = ks[2], kall = ks[3];
    if (!qany || !kany || kmin > qmax) return kTileEmpty;
    if (qall && kall && kmax <= qmin) return kTileFull;
    return kTilePartial;
}

// Key tile and kind of iteration `it`. Kind 0 means skip.
template <int KIND, int BM, int BN = kBN>
__device__ __forceinline__ void tile_at(const FwdDev& p, const MaskDev& m, const TileRange& t, int it,
                                        int& kt, int& kind) {
    if constexpr (KIND == MFA_MASK_TILES) {
        constexpr int SUB = kBN / BN;  // key tiles per listed 64-key tile
        const int e = it / SUB;
        kt = m.col_idx[e] * SUB + (it - e * SUB);
        kind = m.col_kind[e];
        // a 32-key half that starts at or past the last key holds no key
        if (SUB > 1 && kt * BN >= t.k_len) kind = kTileEmpty;
    } else if constexpr (KIND == MFA_MASK_BSR) {
        constexpr int SUB = kBN / BN;  // key tiles per listed block
        const int e = it / SUB;
        kt = m.indices[e] * SUB + (it - e * SUB);
        kind = m.bsr_kind[e];
        if (SUB > 1 && kt * BN >= t.k_len) kind = kTileEmpty;
    } else if constexpr (KIND == MFA_MASK_BLOCKID) {
        kt = it;
        const int nQt = p.nQt, nKt = p.nKt;
        kind = classify_blockid(m.qsum + ((int64_t)t.b * nQt + t.qt) * 4,
                                m.ksum + ((int64_t)t.b * nKt + kt) * 4);
    } else if constexpr (KIND == MFA_MASK_VARLEN) {
        kt = it;
        const int i0 = t.q_row0 - t.q_base, i1 = i0 + t.q_rows - 1;
        const int j0 = kt * kBN, j1 = min(j0 + kBN, t.k_len) - 1;
        bool full = (j1 - j0 + 1 == kBN);
        if (m.causal) full = full && (j1 <= i0);
        if (m.win_left >= 0) full = full && (i1 - j0 <= m.win_left);
        if (m.win_right >= 0) full = full && (j1 - i0 <= m.win_right);
        kind = full ? kTileFull : kTilePartial;
    } else {
        kt = it;
        kind = kTileFull;
    }
}

// Walks the non-empty key tiles of a query tile 64 list entries at a time.
// Lane l of the wave holds entry (base + l) packed as kt | kind << 28, and a
// ballot marks the non-empty lanes, so stepping to the next tile is a bit
// scan plus v_readlane rather than a dependent global load per tile. The
// window after the current one is requested when the current one is entered,
// so its latency overlaps at least one tile of work. All members are
// wave-uniform except the two packed entry registers.
template <int KIND, int BM, int BN = kBN>
struct TileCursor {
    int base;       // list position held by lane 0 of `cur`
    uint32_t cur;   // this lane's entry of the current window
    uint32_t nxt;   // this lane's entry of the following window
    uint64_t nz;    // lanes of `cur` holding a non-empty tile

    __device__ static __forceinline__ uint32_t fetch(const FwdDev& p, const MaskDev& m, const TileRange& t,
                                                     int pos) {
        if (pos >= t.end) return 0u;
        int kt, kind;
        tile_at<KIND, BM, BN>(p, m, t, pos, kt, kind);
        return (uint32_t)kt | ((uint32_t)kind << 28);
    }

    __device__ __forceinline__ void init(const FwdDev& p, const MaskDev& m, const TileRange& t, int lane) {
        base = t.begin;
        cur = fetch(p, m, t, base + lane);
        nxt = fetch(p, m, t, base + 64 + lane);
        nz = __builtin_amdgcn_ballot_w64((cur >> 28) != 0u);
    }

    // First non-empty tile at list position >= it; it >= t.end when none.
    // The common case, a later entry of the current window, takes one
    // (rarely taken) branch.
    __device__ __forceinline__ void seek(const FwdDev& p, const MaskDev& m, const TileRange& t, int lane, int& it,
                                         int& kt, int& kind) {
        const int idx = it - base;
        const uint64_t rest = idx < 64 ? (nz >> idx) : 0ull;
        if (__builtin_expect(rest != 0ull, 1)) {
            it += (int)__builtin_ctzll(rest);
            const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)cur, it - base);
            kt = (int)(e & 0x0FFFFFFFu);
            kind = (int)(e >> 28);
            return;
        }
        seek_slow(p, m, t, lane, it, kt, kind);
    }

    __device__ void seek_slow(const FwdDev& p, const MaskDev& m, const TileRange& t, int lane, int& it, int& kt,
                              int& kind) {
        while (it < t.end) {
            const int idx = it - base;
            if (idx < 64) {
                const uint64_t rest = nz >> idx;
                if (rest) {
                    it += (int)__builtin_ctzll(rest);
                    const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)cur, it - base);
                    kt = (int)(e & 0x0FFFFFFFu);
                    kind = (int)(e >> 28);
                    return;
                }
                it = base + 64;
                continue;
            }
            base += 64;
            cur = nxt;
            nxt = fetch(p, m, t, base + 64 + lane);
            nz = __builtin_amdgcn_ballot_w64((cur >> 28) != 0u);
        }
    }
};

// Per-row mask state for one query row (one lane's query in the MFMA kernel).
template <int KIND>
struct RowMask {
    int qi;        // query row along Sq (global packed row for varlen)
    int qi_local;  // varlen local index; otherwise == qi
    int qblk;      // BLOCKID
    int qvalid;    // BLOCKID
    int row_ok;    // the row exists (inside Sq, or inside its varlen sequence)
    __device__ __forceinline__ void init(const FwdDev& p, const MaskDev& m, const TileRange& t, int row) {
        qi = row;
        qi_local = row - t.q_base;
        qblk = 0;
        qvalid = 1;
        row_ok = (row - t.q_row0) < t.q_rows;
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (row < p.Sq) {
                qblk = m.q_blk[(int64_t)t.b * p.Sq + row];
                qvalid = m.q_valid[(int64_t)t.b * p.Sq + row] != 0;
            } else {
                qvalid = 0;
            }
        }
    }
};

// Generic per-element predicate (used by the fp32 test kernel and for
// reference reasoning; the MFMA kernel has a vectorised version of each).
// key is the sequence-local key index.
template <int KIND>
__device__ __forceinline__ bool allowed(const FwdDev& p, const MaskDev& m, const TileRange& t,
                                        const RowMask<KIND>& r, int key) {
    if (key >= t.k_len || !r.row_ok) return false;
    if constexpr (KIND == MFA_MASK_TILES) {
        const uint32_t w = m.fine_bits[(int64_t)r.qi * m.fine_words + (key >> 5)];
        return (w >> (key & 31)) & 1u;
    } else if constexpr (KIND == MFA_MASK_BLOCKID) {
        const uint32_t w = m.kv_bits[(int64_t)t.b * m.kv_words + (key >> 5)];
        const int kb = m.k_blk[(int64_t)t.b * p.Sk + key];
        return r.qvalid && ((w >> (key & 31)) & 1u) && kb <= r.qblk;
    } else if constexpr (KIND == MFA_MASK_BSR) {
        if (m.kv_bits && !((m.kv_bits[(int64_t)t.b * m.kv_words + (key >> 5)] >> (key & 31)) & 1u)) return false;
        return !m.causal || key <= r.qi;
    } else if constexpr (KIND == MFA_MASK_VARLEN) {
        const int i = r.qi_local, j = key;
        if (m.causal && j > i) return false;
        if (m.win_left >= 0 && i - j > m.win_left) return false;
        if (m.win_right >= 0 && j - i > m.win_right) return false;
        return true;
    } else {
        return true;
    }
}

// Bits [0, n) set (n clamped to [0, 32]).
__device__ __forceinline__ uint32_t below(int n) {
    return n <= 0 ? 0u : (n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u));
}

// The 32-bit mask words a partial (or ragged) key tile kt of NB 32-key
// blocks needs, loaded one tile ahead with the tile's K/V so that the mask
// never waits on a load of its own: the row's fine bits (dense-mask tiles),
// or the tile's key validity bits (block ids; BSR with kv_valid_bits, all
// ones without). Words past the row's end read as 0.
template <int KIND, int NB>
__device__ __forceinline__ void tile_mask_words(const MaskDev& m, const TileRange& t, const RowMask<KIND>& rm,
                                                int row, int kt, int kind, uint32_t (&w)[2]) {
    w[0] = w[1] = 0u;
    if (!(kind == kTilePartial || (kt + 1) * (NB * 32) > t.k_len)) return;
    if constexpr (KIND == MFA_MASK_TILES) {
        if (rm.row_ok) {
            const uint32_t* fb = m.fine_bits + (int64_t)row * m.fine_words + NB * kt;
            if (NB * kt < m.fine_words) w[0] = fb[0];
            if (NB == 2 && NB * kt + 1 < m.fine_words) w[1] = fb[1];
        }
    } else if constexpr (KIND == MFA_MASK_BLOCKID || KIND == MFA_MASK_BSR) {
        if (KIND == MFA_MASK_BSR && !m.kv_bits) {
            w[0] = w[1] = 0xFFFFFFFFu;
        } else {
            const uint32_t* kw = m.kv_bits + (int64_t)t.b * m.kv_words + NB * kt;
            if (NB * kt < m.kv_words) w[0] = kw[0];
            if (NB == 2 && NB * kt + 1 < m.kv_words) w[1] = kw[1];
        }
    }
}

// Block-id masks: the key block id that the mask of a partial (or ragged)
// key tile compares against, for key kt*BN + lane of the tile. raw is the
// key's k_blk entry (loaded with blockid_key_raw), w the tile's key validity
// words (tile_mask_words): keys that are invalid or past k_len fold to
// INT32_MAX, which no row block id below INT32_MAX reaches.
template <int BN>
__device__ __forceinline__ int blockid_key_raw(const FwdDev& p, const MaskDev& m, const TileRange& t, int kt,
                                               int lane) {
    const int j = kt * BN + lane;
    return (lane < BN && j < t.k_len) ? m.k_blk[(int64_t)t.b * p.Sk + j] : INT32_MAX;
}
template <int BN>
__device__ __forceinline__ int blockid_key_fold(const TileRange& t, int kt, int raw, const uint32_t (&w)[2],
                                                int lane) {
    const int j = kt * BN + lane;
    const bool ok = lane < BN && j < t.k_len && ((w[(lane >> 5) & 1] >> (lane & 31)) & 1u);
    return ok ? raw : INT32_MAX;
}

// Sets the scores of disallowed keys of key tile kt to -inf. Register r of
// s[kb] holds key kb*32 + (r>>2)*8 + 4*hh + (r&3) of the tile (query = this
// lane's row); okw[kb] collects, at bit (r>>2)*8 + (r&3), whether that key is
// allowed. fw: the tile's mask words from tile_mask_words (the row's fine
// bits for dense-tile masks, the key validity bits for block ids and BSR).
// kblk: the tile's folded key block ids staged in LDS (block-id masks,
// blockid_key_fold; entry j for key kt*NB*32 + j), or null to read the raw
// ids and validity bits from global memory.
template <int KIND, int NB = 2>
__device__ __forceinline__ void mask_scores(const FwdDev& p, const MaskDev& m, const TileRange& t,
                                            const RowMask<KIND>& rm, int row, int hh, int kt,
                                            const uint32_t (&fw)[2], f32x16 (&s)[NB],
                                            const int32_t* kblk = nullptr) {
    if constexpr (KIND == MFA_MASK_BLOCKID) {
        // Folded ids: one compare per score (a key is allowed iff its folded id
        // is at most the row's block id), exact unless a valid row's block id
        // is INT32_MAX, which takes the general path below. Rows that are
        // invalid or past the end are cleared afterwards.
        const bool row_bad = !rm.qvalid || !rm.row_ok;
        if (kblk && __builtin_amdgcn_ballot_w64(!row_bad && rm.qblk == INT32_MAX) == 0ull) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const i32x4 k4 = *(const i32x4*)(kblk + 4 * hh + kb * 32 + g * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[kb][g * 4 + e] = k4[e] <= rm.qblk ? s[kb][g * 4 + e] : -INFINITY;
                }
            if (__builtin_amdgcn_ballot_w64(row_bad) != 0ull) {
#pragma unroll
                for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = row_bad ? -INFINITY : s[kb][r];
            }
            return;
        }
    }
    uint32_t okw[NB];
    const int base_off = kt * (NB * 32) + 4 * hh;  // tile key index of bit 0 of okw[0]
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) okw[kb] = below(t.k_len - base_off - kb * 32);
    if constexpr (KIND == MFA_MASK_TILES) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) okw[kb] &= fw[kb] >> (4 * hh);
    } else if constexpr (KIND == MFA_MASK_BLOCKID) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) okw[kb] &= fw[kb] >> (4 * hh);
        const int32_t* kbp = m.k_blk + (int64_t)t.b * p.Sk;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            uint32_t cmp = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = base_off + kb * 32 + g * 8 + e;
                    // keys past k_len are cleared by okw's range bits either way
                    const int kbk = key < t.k_len ? kbp[key] : INT32_MAX;
                    cmp |= (kbk <= rm.qblk ? 1u : 0u) << (g * 8 + e);
                }
            }
            okw[kb] &= rm.qvalid ? cmp : 0u;
        }
    } else if constexpr (KIND == MFA_MASK_BSR) {
        if (m.causal) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) okw[kb] &= below(row - base_off - kb * 32 + 1);
        }
        // token validity (kv_valid_bits; all ones without)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) okw[kb] &= fw[kb] >> (4 * hh);
    } else if constexpr (KIND == MFA_MASK_VARLEN) {
        const int i = rm.qi_local;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const int o = base_off + kb * 32;
            if (m.causal) okw[kb] &= below(i - o + 1);
            if (m.win_left >= 0) okw[kb] &= ~below(i - m.win_left - o);
            if (m.win_right >= 0) okw[kb] &= below(i + m.win_right - o + 1);
        }
    }
    if (!rm.row_ok) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) okw[kb] = 0u;
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int bit = (r >> 2) * 8 + (r & 3);
            if constexpr (KIND == MFA_MASK_BSR || KIND == MFA_MASK_VARLEN) {
                // the bit as an all-ones / all-zeros mask (a sign-extending
                // bit-field extract), then a bit-field select of the score or
                // -inf: two VALU instructions per score instead of a test, a
                // compare and a select. Faster in the 2-wave BSR kernels
                // (3-4 %) and the varlen ones (3 %, many partial tiles); in
                // the dense-tile kernels the compiler then allocates the main
                // loop differently and the causal forward was 4 % slower, so
                // they keep the compare and select.
                const int keep = __builtin_amdgcn_sbfe((int)okw[kb], bit, 1);
                s[kb][r] = __int_as_float((__float_as_int(s[kb][r]) & keep) | (int)(0xFF800000u & ~(uint32_t)keep));
            } else {
                s[kb][r] = ((okw[kb] >> bit) & 1u) ? s[kb][r] : -INFINITY;
            }
        }
}

}  // namespace mfa
