// Backward of masked attention on gfx950, for every mask representation.
//
// The split follows the BinFlash method (two passes with the forward's
// dispatch: dK/dV over key blocks, dQ over query blocks):
//   preprocess  delta_i = sum_d dO_id * O_id                       (fp32)
//   dK/dV pass  one workgroup per (batch or varlen sequence, kv head, 64-key
//               block); it walks the query blocks that can attend to the
//               block, for every query head of the GQA group, and
//               accumulates dV += P^T dO and dK += scale * dS^T Q in
//               registers;
//   dQ pass     one workgroup per forward query tile; it walks the forward's
//               key tiles and accumulates dQ += scale * dS K.
// P = exp2(s * scale*log2e - LSE*log2e) is recomputed from the forward's LSE,
// dS = P o (dP - delta), dP = dO V^T; disallowed entries have P = 0. No
// atomics: every output element is written by exactly one workgroup, so
// results are deterministic.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16): in the dK/dV pass scores are
// computed as S = Q K^T so that a lane owns one key and 16 of the queries; the
// bf16 P and dS are then directly the B operands of dV^T = dO^T P and
// dK^T = Q^T dS, whose A operands are transposed reads (ds_read_b64_tr_b16) of
// the Q / dO tiles. The dQ pass uses the forward's S^T = K Q^T layout (a lane
// owns one query) and reads K^T transposed for dQ^T = K^T dS^T.
// Q, dO (dK/dV pass) and K (dQ pass) tiles are read both row-wise and
// transposed; their LDS swizzle is conflict-free for both patterns. Both
// passes run a step as 32-wide halves whose LDS operand reads are issued a
// few MFMA groups ahead; the dK/dV grid puts a head's key blocks on one XCD,
// and 64-row dQ tiles walk 32-key tiles (two waves per SIMD).

#include <mutex>
#include "sched.hpp"

namespace mfa {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ bf16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(__attribute__((address_space(3))) char*)(p));
}

__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte chunk swizzle of a 64 x D bf16 tile that keeps both the row-wise
// operand reads (32 consecutive rows, one chunk) and the transposed reads
// (4 consecutive rows x 4 chunks per half wave) free of bank conflicts.
template <int D>
__device__ __forceinline__ int tswz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int row_off(int r, int lc) {
    return r * (2 * D) + ((lc ^ tswz<D>(r)) << 4);
}

// Byte offset of lane `lane`'s 8-byte transposed read: rows r0 + (lane&15)/4,
// columns db*32 + 16*((lane>>4)&1) + 4*(lane&3).
template <int D>
__device__ __forceinline__ int tr_off(int r0, int db, int lane) {
    const int r = r0 + ((lane & 15) >> 2);
    const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return r * (2 * D) + (((col >> 3) ^ tswz<D>(r)) << 4) + ((col >> 2) & 1) * 8;
}

// Stage a 64-row x D bf16 tile from rows [row0, row0 + 64) of a strided
// tensor into LDS with the tswz layout, using direct-to-LDS buffer loads
// (rows at or past `rows` read as zeros). `nw` waves share the work.
template <int D, int NROWS = 64>
__device__ __forceinline__ void stage_tile(const char* base, int64_t row_bytes, int row0, int rows, char* lds,
                                           int wave, int nw, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int ROWB = 2 * D, RPI = 1024 / ROWB, CPR = D / 8, NINST = NROWS / RPI;
    const int64_t start = (int64_t)row0 * row_bytes;
    // the range ends at the tile's last row or at row `rows`, whichever comes
    // first (32 bits: the host requires 128 rows to span under 2 GiB)
    const int rem = min(NROWS, rows - row0);
    const int nrec = rem > 0 ? (rem - 1) * (int)row_bytes + ROWB : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + start), 0, nrec, 0x00020000);
    for (int i = wave; i < NINST; i += nw) {
        const int r = i * RPI + lane / CPR;
        const int pc = lane % CPR;
        const int go = (int)(r * row_bytes) + ((pc ^ tswz<D>(r)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + i * 1024), 16, go, 0, 0, 0);
    }
#endif
}

// The same staging split into a descriptor and single instructions, so that
// the instructions can be spread over a compute phase: each moves 1 KB
// (RPI rows), instruction i filling LDS bytes [1024 i, 1024 i + 1024) of an
// NROWS-row tile. Instruction i reads row i*RPI + lane/CPR, chunk lane%CPR
// swizzled by the row; the swizzle depends on i only through i mod 4
// (D = 128) or i mod 2 (D = 64). A wave of NW >= 2 issues instructions
// wave + NW*k, so two lane offsets (k even, k odd) plus the wave-uniform
// i*RPI rows give every offset: one add per instruction instead of a
// 64-bit multiply-add.
template <int D, int NROWS = 64>
struct TileDma {
    static constexpr int ROWB = 2 * D, RPI = 1024 / ROWB, CPR = D / 8, NINST = NROWS / RPI;
    __amdgpu_buffer_rsrc_t rs;
    int row_bytes;  // 32 bits: the host requires 128 rows to span under 2 GiB
    __device__ __forceinline__ void init(const char* base, int64_t rb, int row0, int rows) {
#if defined(__HIP_DEVICE_COMPILE__)
        row_bytes = (int)rb;
        const int64_t start = (int64_t)row0 * rb;
        const int rem = min(NROWS, rows - row0);  // as in stage_tile
        const int nrec = rem > 0 ? (rem - 1) * (int)rb + ROWB : 0;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + start), 0, nrec, 0x00020000);
#endif
    }
    // The lane's part of instruction i's byte offset: its row within the
    // instruction's RPI rows, and its swizzled chunk.
    static __device__ __forceinline__ int lane_off(int i, int lane, int64_t rb) {
        const int r = i * RPI + lane / CPR;
        return (lane / CPR) * (int)rb + (((lane % CPR) ^ tswz<D>(r)) << 4);
    }
    // Instruction i, with loff = lane_off(i', lane, row bytes) for an i' that
    // has the same swizzle (i' = i mod 4).
    __device__ __forceinline__ void issue(char* lds, int i, int loff) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const int go = loff + i * RPI * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + i * 1024), 16, go, 0, 0, 0);
#endif
    }
};

// Stage 64 consecutive fp32 values (positions [i0, i0+64) of a row of length n).
__device__ __forceinline__ void stage_vec64(const float* base, int i0, int n, float* lds, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int nrec = n > i0 ? min(n - i0, 64) * 4 : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + i0), 0, nrec, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 4, lane * 4, 0, 0, 0);
#endif
}



__device__ __forceinline__ float lse_log2(float lse) {
    // exponent offset in log2 units; +inf for empty rows so that P = 0 there
    return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

}  // namespace

// ---------------------------------------------------------------------------
// preprocess: delta = rowsum(dO * O)
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(BwdDev p) {
    constexpr int LPR = D / 8;
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rows = (int64_t)p.f.B * p.f.Sq * p.f.Hq;
    const int64_t r = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
    float acc = 0.f;
    int b = 0, i = 0, h = 0;
    if (r < rows) {
        h = (int)(r % p.f.Hq);
        const int64_t bi = r / p.f.Hq;
        i = (int)(bi % p.f.Sq);
        b = (int)(bi / p.f.Sq);
        const bf16* o = (const bf16*)p.f.o + (int64_t)b * p.f.os0 + (int64_t)i * p.f.os1 + (int64_t)h * p.f.os2;
        const bf16* d = (const bf16*)p.dout + (int64_t)b * p.dos0 + (int64_t)i * p.dos1 + (int64_t)h * p.dos2;
        const bf16x8 ov = *(const bf16x8*)(o + (lane % LPR) * 8);
        const bf16x8 dv = *(const bf16x8*)(d + (lane % LPR) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)ov[e], (float)dv[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (r < rows && (lane % LPR) == 0) p.delta[((int64_t)b * p.f.Hq + h) * p.f.Sq + i] = acc;
}

// ---------------------------------------------------------------------------
// dK / dV pass
// ---------------------------------------------------------------------------

// Whether query i (index within the batch entry or the varlen sequence) may
// attend to key key_l, from the key side: kblk / kval are the key's block id
// and validity (BLOCKID), kval its kv_valid_bits bit (BSR). Evaluated only on
// partial blocks; full blocks need no test, empty blocks are never visited.
template <int KIND>
__device__ __forceinline__ bool allowed_qk(const FwdDev& f, const MaskDev& m, int b, int q_len, int k_len, int key_l,
                                           int i, int kblk, bool kval) {
    bool ok = i < q_len && key_l < k_len;
    if constexpr (KIND == MFA_MASK_BSR) {
        ok = ok && kval && (!m.causal || key_l <= i);
    } else if constexpr (KIND == MFA_MASK_TILES) {
        if (ok) ok = (m.fine_bits[(int64_t)i * m.fine_words + (key_l >> 5)] >> (key_l & 31)) & 1u;
    } else if constexpr (KIND == MFA_MASK_BLOCKID) {
        if (ok) {
            const int64_t qi = (int64_t)b * f.Sq + i;
            ok = kval && m.q_valid[qi] && kblk <= m.q_blk[qi];
        }
    } else if constexpr (KIND == MFA_MASK_VARLEN) {
        ok = ok && (!m.causal || key_l <= i) && (m.win_left < 0 || i - key_l <= m.win_left) &&
             (m.win_right < 0 || key_l - i <= m.win_right);
    }
    return ok;
}

// Allowed bits of one 32-query half in the dK/dV layout: bit rr says whether
// query qi0 + (rr>>2)*8 + 4*hh + (rr&3) may attend to this lane's key key_l.
// Varlen windows and BSR blocks (causal or not) allow, for one key, the
// queries whose distance query - key lies in one interval, below q_len: the
// half's 32 query offsets form one run of bits [a, e], built as a mask, and
// the lane's 16 offsets are four nibbles of it (a few instructions instead
// of the per-element tests).
template <int KIND>
__device__ __forceinline__ uint32_t allowed_bits_T(const FwdDev& f, const MaskDev& m, int b, int q_len, int k_len,
                                                   int key_l, int qi0, int hh, int kblk, bool kval) {
    if constexpr (KIND == MFA_MASK_VARLEN || KIND == MFA_MASK_BSR) {
        if (!(key_l < k_len) || (KIND == MFA_MASK_BSR && !kval)) return 0u;
        const int64_t d0 = (int64_t)qi0 - key_l;  // query offset 0 minus the key
        int64_t a = 0, e = 31;                    // allowed offsets within the half
        if (m.causal) a = max(a, -d0);
        if constexpr (KIND == MFA_MASK_VARLEN) {
            if (m.win_right >= 0) a = max(a, -(int64_t)m.win_right - d0);
            if (m.win_left >= 0) e = min(e, (int64_t)m.win_left - d0);
        }
        e = min(e, (int64_t)q_len - 1 - qi0);
        if (e < a) return 0u;
        const int w = (int)(e - a + 1);  // 1..32 offsets from a (0..31)
        const uint32_t run = w >= 32 ? 0xFFFFFFFFu : ((1u << w) - 1u) << (int)a;
        const uint32_t t = run >> (4 * hh);
        return (t & 0xFu) | ((t >> 4) & 0xF0u) | ((t >> 8) & 0xF00u) | ((t >> 12) & 0xF000u);
    } else {
        uint32_t bits = 0;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int i = qi0 + (rr >> 2) * 8 + 4 * hh + (rr & 3);
            bits |= (allowed_qk<KIND>(f, m, b, q_len, k_len, key_l, i, kblk, kval) ? 1u : 0u) << rr;
        }
        return bits;
    }
}

// Workgroup w runs on XCD w % 8. This numbering puts runs of C consecutive
// logical ids on one XCD and deals the runs round-robin over the XCDs:
// neighbours share an L2 while each XCD still gets every eighth run. Ids
// past the last whole round of 8 runs keep their plain number.
__device__ __forceinline__ int xcd_runs(int w, int total, int C) {
    const int span = 8 * C;
    if (w >= total / span * span) return w;
    const int r = w >> 3;
    return ((r / C) * 8 + (w & 7)) * C + r % C;
}

// The 64-key block of one dK/dV workgroup: (batch or varlen sequence, kv
// head, key block) and the query / key extents it works in.
struct KeyBlock {
    int b, hk, kbk;
    int q_base, q_len;  // query rows [q_base, q_base + q_len) (varlen: the sequence)
    int k_base, k_len;  // key rows k_base + [0, k_len) are attended
    int k_alloc;        // keys whose gradient rows are written (k_len of them attended)
    bool len_error;     // varlen: sequence longer than the stated max_q / max_k
    bool active;        // false: the block lies past its sequence's keys
    int split;          // query-head split of the block (0 without one)
    int g0, g1;         // the split's query heads within the GQA group: [g0, g1)
    int seq;            // varlen sequence (-1 otherwise)
};

// Where key key_l's rows of k, v, dk, dv sit: (outer, row) indices for the
// (stride 0, stride 1) pair of those tensors: (batch, k_base + key_l), or,
// with a block table, (page, row in page). false: a paged key whose page is
// past the table row or outside the pool (nothing is read or written).
__device__ __forceinline__ bool key_rows(const MaskDev& m, const KeyBlock& kb, int key_l, int64_t& outer,
                                         int64_t& row) {
    if (m.block_table && kb.seq >= 0) {
        int r = 0;
        if (key_l / m.page_size >= m.max_pages) return false;
        const int pg = page_of(m, kb.seq, key_l, r);
        outer = pg;
        row = r;
        return pg >= 0;
    }
    outer = kb.b;
    row = kb.k_base + key_l;
    return true;
}

template <int KIND>
__device__ __forceinline__ KeyBlock key_block(const BwdDev& p, const MaskDev& m, int wg_id, int n_wg, bool remap) {
    const FwdDev& f = p.f;
    KeyBlock kb;
    kb.b = 0;
    kb.hk = 0;
    kb.kbk = 0;
    kb.q_base = 0;
    kb.q_len = f.Sq;
    kb.k_base = 0;
    kb.k_len = f.Sk;
    kb.k_alloc = f.Sk;
    kb.len_error = false;
    kb.active = true;
    kb.split = 0;
    kb.g0 = 0;
    kb.g1 = f.G;
    kb.seq = -1;
    if constexpr (KIND == MFA_MASK_VARLEN) {
        const int nKbm = (m.max_k + 63) / 64;
        // runs of 8 consecutive key blocks of a (sequence, kv head) on one
        // XCD (they share most of their window's Q and dO in that XCD's
        // L2), the runs round-robin over the XCDs, so that long sequences
        // still spread over all of them
        const int wg = xcd_runs(wg_id, n_wg, 8);
        kb.kbk = wg % nKbm;
        const int sh = wg / nKbm;
        kb.hk = sh % f.Hkv;
        const int seq = sh / f.Hkv;
        kb.q_base = m.cu_q[seq];
        kb.q_len = m.cu_q[seq + 1] - kb.q_base;
        kb.seq = seq;
        kb.k_base = m.cu_k[seq];
        kb.k_alloc = m.cu_k[seq + 1] - kb.k_base;
        kb.k_len = m.seqused_k ? min(kb.k_alloc, max(m.seqused_k[seq], 0)) : kb.k_alloc;
        if (kb.kbk * 64 >= kb.k_alloc) kb.active = false;
        kb.len_error = kb.q_len > m.max_q || kb.k_alloc > m.max_k;
        if (m.block_table) {
            // paged keys (as in the forward): the used keys must fit the
            // table row, and their pages must lie in the pool
            kb.k_base = 0;
            const int cap = m.max_pages * m.page_size;
            bool bad = kb.k_len > cap;
            const int used = min(kb.k_len, cap);
            const int32_t* tb = m.block_table + (int64_t)seq * m.max_pages;
            for (int pi = 0; pi < (used + m.page_size - 1) / m.page_size; ++pi)
                bad = bad || tb[pi] < 0 || tb[pi] >= m.n_pages;
            kb.k_len = used;
            kb.len_error = kb.len_error || bad;
        }
    } else {
        const int nKb = (f.Sk + 63) / 64;
        // consecutive key blocks of one (batch, kv head, head split) on one
        // XCD, so that they share that XCD's L2 copy of the heads' Q and dO
        const int wg = xcd_logical(wg_id, n_wg, remap && (n_wg & 7) == 0);
        const int bhs = wg / nKb;
        kb.kbk = wg - bhs * nKb;
        const int S = p.gsplit > 1 ? p.gsplit : 1;
        const int bh = bhs / S;
        kb.split = bhs - bh * S;
        kb.g0 = kb.split * (f.G / S);
        kb.g1 = kb.g0 + f.G / S;
        kb.b = bh / f.Hkv;
        kb.hk = bh - kb.b * f.Hkv;
    }
    return kb;
}

// The query blocks (64 rows) that can attend to a key block, as entries
// qb | kind << 28 (kind 0: skip) at list positions [pbeg, pend): the CSC list
// (BSR), the dense tile map or the block-id summaries (both at 128-row
// granularity: a 64-row block takes its tile's kind), the window arithmetic
// (varlen) or every block (no mask).
template <int KIND>
struct QueryBlocks {
    int pbeg, pend, e0;
    bool blk_all_valid;  // BSR with kv_valid_bits: every key of the block valid
    __device__ __forceinline__ void init(const FwdDev& f, const MaskDev& m, const KeyBlock& kb) {
        pbeg = 0;
        pend = (kb.q_len + 63) / 64;
        e0 = 0;
        blk_all_valid = true;
        if constexpr (KIND == MFA_MASK_BSR) {
            bool any_valid = true;
            if (m.kv_bits) {
                const uint32_t* kw = m.kv_bits + (int64_t)kb.b * m.kv_words + 2 * kb.kbk;
                const uint32_t w0 = kw[0], w1 = (2 * kb.kbk + 1 < m.kv_words) ? kw[1] : 0u;
                blk_all_valid = w0 == 0xFFFFFFFFu && w1 == 0xFFFFFFFFu;
                any_valid = (w0 | w1) != 0u;
            }
            const int nKb = (f.Sk + 63) / 64;
            const int* cp = m.csc_ptr + ((int64_t)kb.b * f.Hkv + kb.hk) * (nKb + 1);
            e0 = cp[kb.kbk];
            pend = any_valid ? cp[kb.kbk + 1] - e0 : 0;
        } else if constexpr (KIND == MFA_MASK_VARLEN) {
            const int j0 = kb.kbk * 64, j1 = min(j0 + 63, kb.k_len - 1);
            int lo = 0, hi = j1 >= j0 ? kb.q_len - 1 : -1;  // no used key in the block: no query block
            if (m.causal) lo = max(lo, j0);
            if (m.win_right >= 0) lo = max(lo, j0 - m.win_right);
            if (m.win_left >= 0) hi = min(hi, j1 + m.win_left);
            pbeg = lo / 64;
            pend = hi >= lo ? hi / 64 + 1 : pbeg;
        }
    }
    __device__ __forceinline__ uint32_t fetch(const FwdDev& f, const MaskDev& m, const KeyBlock& kb, int pos) const {
        if (pos >= pend) return 0u;
        int qb = pos, kind = kTileFull;
        if constexpr (KIND == MFA_MASK_BSR) {
            qb = m.csc_idx[e0 + pos];
            kind = bsr_kind_of(qb, kb.kbk, 64, 64, f.Sq, f.Sk, m.causal);
            if (kind == kTileFull && !blk_all_valid) kind = kTilePartial;
        } else if constexpr (KIND == MFA_MASK_TILES) {
            kind = m.tile_kind[(int64_t)(qb >> m.tile_shift) * f.nKt + kb.kbk];
        } else if constexpr (KIND == MFA_MASK_BLOCKID) {
            kind = classify_blockid(m.qsum + ((int64_t)kb.b * f.nQt + (qb >> 1)) * 4,
                                    m.ksum + ((int64_t)kb.b * f.nKt + kb.kbk) * 4);
        } else if constexpr (KIND == MFA_MASK_VARLEN) {
            const int i0 = qb * 64, i1 = min(i0 + 63, kb.q_len - 1);
            const int j0 = kb.kbk * 64, j1 = min(j0 + 63, kb.k_len - 1);
            bool full = (i1 - i0 == 63) && (j1 - j0 == 63);
            if (m.causal) full = full && j1 <= i0;
            if (m.win_left >= 0) full = full && i1 - j0 <= m.win_left;
            if (m.win_right >= 0) full = full && j1 - i0 <= m.win_right;
            kind = full ? kTileFull : kTilePartial;
        }
        return (uint32_t)qb | ((uint32_t)kind << 28);
    }
};

// Key-side mask values of key key_l: block id and validity (BLOCKID), the
// kv_valid_bits bit (BSR; true without the bitmap).
template <int KIND>
__device__ __forceinline__ void key_side(const FwdDev& f, const MaskDev& m, const KeyBlock& kb, int key_l, bool key_ok,
                                         int& kblk, bool& kval) {
    kblk = INT32_MAX;
    kval = false;
    if constexpr (KIND == MFA_MASK_BLOCKID) {
        if (key_ok) {
            kblk = m.k_blk[(int64_t)kb.b * f.Sk + key_l];
            kval = (m.kv_bits[(int64_t)kb.b * m.kv_words + (key_l >> 5)] >> (key_l & 31)) & 1u;
        }
    } else if constexpr (KIND == MFA_MASK_BSR) {
        kval = true;
        if (m.kv_bits) kval = key_ok && ((m.kv_bits[(int64_t)kb.b * m.kv_words + (key_l >> 5)] >> (key_l & 31)) & 1u);
    }
}

// One workgroup (2 waves, 64 keys) per (batch or varlen sequence, kv head,
// 64-key block). The query blocks that can attend to the key block come from
// the CSC list (BSR), the dense tile map or the block-id summaries (both at
// 128-row granularity: a 64-row block takes its tile's kind), the window
// arithmetic (varlen) or all blocks (no mask); they are walked through a
// ScanWindow, once per query head of the GQA group. With a head split
// (p.gsplit > 1) there are gsplit workgroups per key block, each over its
// share of the group's heads, writing fp32 partial sums for the reduce pass.
// MOD: score modifications compiled in (kModBias, kModCap).
template <int D, int KIND, int MOD>
__global__ __launch_bounds__(128, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdDev p, MaskDev m) {
    constexpr bool BIAS = (MOD & kModBias) != 0, CAP = (MOD & kModCap) != 0;
    constexpr int ROWB = 2 * D, TILEB = 64 * ROWB, NKC = D / 16, NDB = D / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sQ = smem;                                   // [2][64 x D] Q
    char* sO = smem + 2 * TILEB;                       // [2][64 x D] dO
    float* sL = (float*)(smem + 4 * TILEB);            // [2][64] -LSE * log2(e)
    float* sDl = sL + 128;                             // [2][64] delta
    // query-side mask data of a partial block, staged with its Q / dO:
    int32_t* sQb = (int32_t*)(sDl + 128);              // [2][64] query block ids (block-id masks)
    uint32_t* sQv = (uint32_t*)(sQb + 128);            // [2][2] query validity bits (block-id masks)
    uint32_t* sFb = sQv + 4;                           // [2][2][64] fine-mask words per 32-key half (dense tiles)

    const FwdDev& f = p.f;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hh = lane >> 5, c = lane & 31;

    const KeyBlock kblock = key_block<KIND>(p, m, blockIdx.x, gridDim.x, true);
    if (!kblock.active) return;
    if (KIND == MFA_MASK_VARLEN && kblock.len_error && m.err && threadIdx.x == 0) *m.err = 1;
    const int b = kblock.b, hk = kblock.hk, kbk = kblock.kbk;
    const int q_base = kblock.q_base, q_len = kblock.q_len, k_len = kblock.k_len, k_alloc = kblock.k_alloc;
    const bool len_error = kblock.len_error;
    const int key_l = kbk * 64 + wave * 32 + c;  // key within the batch entry / sequence
    int64_t ko = 0, kr = 0;                      // (batch or page, row) of k, v, dk, dv
    const bool key_addr = key_rows(m, kblock, key_l, ko, kr);
    const bool key_ok = key_l < k_len && key_addr;

    // stationary K and V fragments (B operands: K^T, V^T with lane = key)
    bf16x8 kf[NKC], vf[NKC];
    {
        const bf16* kp = (const bf16*)f.k + ko * f.ks0 + kr * f.ks1 + (int64_t)hk * f.ks2 + hh * 8;
        const bf16* vp = (const bf16*)f.v + ko * f.vs0 + kr * f.vs1 + (int64_t)hk * f.vs2 + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            kf[kc] = key_ok ? *(const bf16x8*)(kp + kc * 16) : bf16x8{};
            vf[kc] = key_ok ? *(const bf16x8*)(vp + kc * 16) : bf16x8{};
        }
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    int kblk;
    bool kval;
    key_side<KIND>(f, m, kblock, key_l, key_ok, kblk, kval);

    // ---- the query blocks of this key block ----
    QueryBlocks<KIND> qbl;
    qbl.init(f, m, kblock);
    const int pbeg = qbl.pbeg, pend = qbl.pend;
    auto fetch = [&](int pos) -> uint32_t { return qbl.fetch(f, m, kblock, pos); };
    ScanWindow win;
    win.init(fetch, pbeg, lane);
    const int g_end = kblock.g1;
    int g = kblock.g0, pos = pbeg;
    uint32_t ent = 0;
    bool have = win.seek(fetch, pos, pend, lane, ent);
    auto next_step = [&](int& g_, int& pos_, uint32_t& ent_) -> bool {
        ++pos_;
        if (win.seek(fetch, pos_, pend, lane, ent_)) return true;
        if (++g_ >= g_end) return false;
        pos_ = pbeg;
        return win.seek(fetch, pos_, pend, lane, ent_);
    };

    const float c2 = f.c2;
    int qrow_off[NKC];  // A operand rows of S / dP for query block 0: row c, chunk kc*2 + hh
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qrow_off[kc] = row_off<D>(c, kc * 2 + hh);
    int trq[2][NDB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db) trq[j][db] = tr_off<D>(8 * j + 4 * hh, db, lane);

    // Lane offsets of this wave's spread Q / dO staging instructions
    // (D = 128): the wave issues instructions wave + 2k, whose residue mod 4
    // is wave + 2 (k & 1).
    int q_loff[2] = {0, 0}, o_loff[2] = {0, 0};
    if constexpr (D == 128) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            q_loff[j] = TileDma<128>::lane_off(wave + 2 * j, lane, 2 * f.qs1);
            o_loff[j] = TileDma<128>::lane_off(wave + 2 * j, lane, 2 * p.dos1);
        }
    }
    auto stage_to = [&](int g_, uint32_t ent_, char* dq_, char* do_, float* dd_) {
        const int hq = hk * f.G + g_;
        const int qb = (int)(ent_ & 0x0FFFFFFFu);
        const char* qbp = (const char*)f.q + 2 * ((int64_t)b * f.qs0 + (int64_t)hq * f.qs2);
        const char* obp = (const char*)p.dout + 2 * ((int64_t)b * p.dos0 + (int64_t)hq * p.dos2);
        const int r0 = q_base + qb * 64, rend = q_base + q_len;
        stage_tile<D>(qbp, 2 * f.qs1, r0, rend, dq_, wave, 2, lane);
        stage_tile<D>(obp, 2 * p.dos1, r0, rend, do_, wave, 2, lane);
        const int64_t lrow = ((int64_t)b * f.Hq + hq) * f.Sq;
        if (wave == 1) stage_vec64(p.delta + lrow, r0, rend, dd_, lane);
    };
    // Block-id masks: the 64 query block ids of a partial block, by wave 1
    // into LDS with the block's Q / dO (rows past the end read as 0; their
    // validity bit is 0).
    auto stage_qblk = [&](uint32_t ent_, int32_t* dst) {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (wave == 1 && (int)(ent_ >> 28) == kTilePartial)
                stage_vec64((const float*)(m.q_blk + (int64_t)b * f.Sq), (int)(ent_ & 0x0FFFFFFFu) * 64, q_len,
                            (float*)dst, lane);
        }
    };
    auto stage = [&](int g_, uint32_t ent_, int buf) {
        stage_to(g_, ent_, sQ + buf * TILEB, sO + buf * TILEB, sDl + buf * 64);
        stage_qblk(ent_, sQb + buf * 64);
    };
    // Wave 0 loads the LSE of the staged rows into a register and stores it
    // to LDS, as the exponent offset in log2 units, at the end of the step
    // (before the barrier that publishes the buffer): the per-element
    // conversion then costs nothing in the step that reads it.
    auto lse_fetch = [&](int g_, uint32_t ent_) -> float {
        const int hq = hk * f.G + g_;
        const int r = q_base + (int)(ent_ & 0x0FFFFFFFu) * 64 + lane;
        return r < q_base + q_len ? f.lse[((int64_t)b * f.Hq + hq) * f.Sq + r] : -INFINITY;
    };
    auto lse_store = [&](float lse, int buf) {
        // -lse*log2(e); -inf for empty rows (and rows past the end) so that P = 0 there
        sL[buf * 64 + lane] = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
    };
    // Row-side mask values of a partial block, row = this lane, loaded into
    // registers with the block's staging and stored to LDS at the end of the
    // step: the validity of the row (block ids, wave 0) and this wave's fine
    // word of the row (dense tiles: wave w's keys are word 2*kbk + w).
    auto side_fetch = [&](uint32_t ent_) -> uint32_t {
        uint32_t v = 0u;
        if ((int)(ent_ >> 28) != kTilePartial) return v;
        const int i = (int)(ent_ & 0x0FFFFFFFu) * 64 + lane;  // query index within the batch entry
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (wave == 0 && i < q_len) v = m.q_valid[(int64_t)b * f.Sq + i] != 0;
        } else if constexpr (KIND == MFA_MASK_TILES) {
            const int wd = 2 * kbk + wave;
            if (i < q_len && wd < m.fine_words) v = m.fine_bits[(int64_t)i * m.fine_words + wd];
        }
        return v;
    };
    auto side_store = [&](uint32_t v, int buf) {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (wave == 0) {
                const uint64_t vm = __builtin_amdgcn_ballot_w64(v != 0u);
                if (lane < 2) sQv[buf * 2 + lane] = (uint32_t)(lane ? vm >> 32 : vm);
            }
        } else if constexpr (KIND == MFA_MASK_TILES) {
            sFb[buf * 128 + wave * 64 + lane] = v;
        }
    };

    if (have) {
        stage(g, ent, 0);
        if (wave == 0) lse_store(lse_fetch(g, ent), 0);
        side_store(side_fetch(ent), 0);
    }
    vm_wait();
    __syncthreads();
    int buf = 0;
    while (have) {
        const int qb = (int)(ent & 0x0FFFFFFFu);
        const int kind = (int)(ent >> 28);
        int g_n = g, pos_n = pos;
        uint32_t ent_n = 0;
        const bool have_n = next_step(g_n, pos_n, ent_n);
        float lse_n = 0.f;
        uint32_t side_n = 0u;
        const int32_t* qbs = sQb + buf * 64;    // this block's staged query-side mask data
        const uint32_t* fbs = sFb + buf * 128 + wave * 64;
        const uint64_t qvm = KIND == MFA_MASK_BLOCKID
                                 ? ((uint64_t)sQv[buf * 2 + 1] << 32) | sQv[buf * 2]
                                 : 0ull;
        // The step works on restrict-qualified views of the two buffers: the
        // reads of this step's buffer then carry alias scopes that tell the
        // compiler they do not overlap the DMA into the other buffer, so it
        // does not make them wait for that DMA.
        auto body = [&](const char* __restrict__ q_, const char* __restrict__ o_, const float* __restrict__ l_,
                        const float* __restrict__ d_, char* __restrict__ nq_, char* __restrict__ no_,
                        float* __restrict__ nd_) {
            // The next block's Q and dO tiles. At D = 128 this wave's NPW
            // instructions of each are issued one per operand group below,
            // interleaved with the MFMAs, rather than all at the start of the
            // step (a burst of them stalls the wave on the vector memory
            // queue); at D = 64 (two waves per SIMD, no registers to spare)
            // they are issued here.
            constexpr bool SPREAD = D == 128;
            constexpr int NPW = SPREAD ? TileDma<128>::NINST / 2 : 0;
            // Without a next block the spread instructions are still issued,
            // with an empty range (they write zeros into the free buffer), so
            // that the MFMA phase below carries no branch per instruction.
            TileDma<128> dmq, dmo;  // used at D = 128 only
            if constexpr (SPREAD) {
                const int hq = hk * f.G + (have_n ? g_n : g);
                const int qbn = have_n ? (int)(ent_n & 0x0FFFFFFFu) : 0;
                const char* qbp = (const char*)f.q + 2 * ((int64_t)b * f.qs0 + (int64_t)hq * f.qs2);
                const char* obp = (const char*)p.dout + 2 * ((int64_t)b * p.dos0 + (int64_t)hq * p.dos2);
                const int r0 = q_base + qbn * 64, rend = have_n ? q_base + q_len : r0;
                dmq.init(qbp, 2 * f.qs1, r0, rend);
                dmo.init(obp, 2 * p.dos1, r0, rend);
            }
            if (have_n) {
                if constexpr (SPREAD) {
                    const int hq = hk * f.G + g_n;
                    const int r0 = q_base + (int)(ent_n & 0x0FFFFFFFu) * 64, rend = q_base + q_len;
                    const int64_t lrow = ((int64_t)b * f.Hq + hq) * f.Sq;
                    if (wave == 1) stage_vec64(p.delta + lrow, r0, rend, nd_, lane);
                } else {
                    stage_to(g_n, ent_n, nq_, no_, nd_);
                }
                stage_qblk(ent_n, sQb + (buf ^ 1) * 64);
                if (wave == 0) lse_n = lse_fetch(g_n, ent_n);
                side_n = side_fetch(ent_n);
            }

            // The two 32-query halves one after the other: S = Q K^T and
            // dP = dO V^T (G1 operand groups), then P and dS, then
            // dV^T += dO^T P and dK^T += Q^T dS (G2 groups). The LDS operand
            // reads of all 2 * (G1 + G2) groups form one stream issued PF groups
            // ahead of the MFMAs that consume them (a ring of PF + 1 slots), so
            // that with one wave per SIMD the read latency is not exposed.
            constexpr int G1 = NKC, G2 = 2 * NDB, GH = G1 + G2, GT = 2 * GH, PF = 3, RING = PF + 1;
            bf16x8 ra[RING], rb[RING];
            auto load_group = [&](int i) {
                const int h = i / GH, j = i % GH, slot = i % RING;
                if (j < G1) {
                    ra[slot] = *(const bf16x8*)(q_ + h * 32 * ROWB + qrow_off[j]);
                    rb[slot] = *(const bf16x8*)(o_ + h * 32 * ROWB + qrow_off[j]);
                } else {
                    const int jj = j - G1, k2 = jj / NDB, db = jj % NDB;
                    const int o0 = (h * 2 + k2) * 16 * ROWB;
                    const bf16x4 olo = tr_read(o_ + o0 + trq[0][db]);
                    const bf16x4 ohi = tr_read(o_ + o0 + trq[1][db]);
                    const bf16x4 qlo = tr_read(q_ + o0 + trq[0][db]);
                    const bf16x4 qhi = tr_read(q_ + o0 + trq[1][db]);
                    ra[slot] = __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7);
                    rb[slot] = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            };
            f32x16 s, dp;
            f32x4 NL[4], DL[4];
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int i = 0; i < PF; ++i) load_group(i);
#pragma clang loop unroll(full)
            for (int i = 0; i < GT; ++i) {
                const int h = i / GH, j = i % GH, slot = i % RING;
                if (j == 0) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        NL[gq] = *(const f32x4*)(l_ + h * 32 + gq * 8 + 4 * hh);
                        DL[gq] = *(const f32x4*)(d_ + h * 32 + gq * 8 + 4 * hh);
                    }
                    if constexpr (BIAS) {
                        f32x16 t2[2];
                        const float sl = f.alibi[hk * f.G + g] / f.scale;
                        alibi_fill(t2, sl, key_l - qb * 64 - 4 * hh, -sl);
                        s = t2[h];
                    } else {
                        s = f32x16{};
                    }
                    dp = f32x16{};
                }
                if (i + PF < GT) load_group(i + PF);
                if (SPREAD && i < 2 * NPW) {
                    const int ii = wave + 2 * (i >> 1);  // instruction index within the tile
                    if (i & 1) dmo.issue(no_, ii, o_loff[(i >> 1) & 1]);
                    else dmq.issue(nq_, ii, q_loff[(i >> 1) & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (j < G1) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot], kf[j], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[slot], vf[j], dp, 0, 0, 0);
                } else {
                    const int jj = j - G1, k2 = jj / NDB, db = jj % NDB;
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot], pb[k2], dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[slot], sb[k2], dk[db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (j == G1 - 1) {
                    // soft cap before the mask (masked scores stay -inf)
                    if constexpr (CAP) {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) s[rr] = softcap_raw(s[rr], f);
                    }
                    // partial blocks: disallowed scores become -inf (P = 0 there);
                    // register r is query h*32 + (r>>2)*8 + 4*hh + (r&3)
                    if (__builtin_expect(kind == kTilePartial, 0)) {
                        uint32_t okb = 0u;
                        if constexpr (KIND == MFA_MASK_BLOCKID) {
                            // staged block ids and validity of the half's rows
                            const uint32_t vw = (uint32_t)(qvm >> (h * 32));
                            uint32_t cmp = 0u, vb = 0u;
#pragma unroll
                            for (int gq = 0; gq < 4; ++gq) {
                                const i32x4 q4 = *(const i32x4*)(qbs + h * 32 + gq * 8 + 4 * hh);
#pragma unroll
                                for (int e = 0; e < 4; ++e) cmp |= (kblk <= q4[e] ? 1u : 0u) << (gq * 4 + e);
                                vb |= ((vw >> (gq * 8 + 4 * hh)) & 0xFu) << (gq * 4);
                            }
                            okb = kval ? (cmp & vb) : 0u;
                        } else if constexpr (KIND == MFA_MASK_TILES) {
                            // staged fine words of the half's rows, bit c = this lane's key
                            uint32_t bits = 0u;
#pragma unroll
                            for (int gq = 0; gq < 4; ++gq) {
                                const u32x4 w4 = *(const u32x4*)(fbs + h * 32 + gq * 8 + 4 * hh);
#pragma unroll
                                for (int e = 0; e < 4; ++e) bits |= ((w4[e] >> c) & 1u) << (gq * 4 + e);
                            }
                            okb = key_ok ? bits : 0u;
                        } else {
                            okb = allowed_bits_T<KIND>(f, m, b, q_len, k_len, key_l, qb * 64 + h * 32, hh, kblk, kval);
                        }
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr)
                            if (!((okb >> rr) & 1u)) s[rr] = -INFINITY;
                    }
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = gq * 4 + e;
                            const float pv = fast_exp2(fmaf(s[rr], c2, NL[gq][e]));
                            float ds = pv * (dp[rr] - DL[gq][e]);
                            if constexpr (CAP) ds *= softcap_grad(s[rr], f);
                            pb[gq >> 1][(gq & 1) * 4 + e] = (bf16)pv;
                            sb[gq >> 1][(gq & 1) * 4 + e] = (bf16)ds;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        body(sQ + buf * TILEB, sO + buf * TILEB, sL + buf * 64, sDl + buf * 64, sQ + (buf ^ 1) * TILEB,
             sO + (buf ^ 1) * TILEB, sDl + (buf ^ 1) * 64);
        if (wave == 0 && have_n) lse_store(lse_n, buf ^ 1);
        if (have_n) side_store(side_n, buf ^ 1);
        vm_wait();
        __syncthreads();
        buf ^= 1;
        have = have_n;
        g = g_n;
        pos = pos_n;
        ent = ent_n;
    }

    // keys past the used length get zero gradients; paged keys outside the
    // table or the pool are not written
    if (key_l >= k_alloc || !key_addr) return;
    if (p.gsplit > 1) {
        // this split's sums over its query heads, fp32 and unscaled; the
        // reduce pass adds the splits in order and writes dk / dv
        const int64_t ri = (((int64_t)kblock.split * f.B + b) * f.Sk + kr) * f.Hkv + hk;
        float* wk = p.ws + ri * D;
        float* wv = p.ws + ((int64_t)p.gsplit * f.B * f.Sk * f.Hkv + ri) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int o = db * 32 + gq * 8 + 4 * hh;
                *(f32x4*)(wk + o) = f32x4{dk[db][gq * 4], dk[db][gq * 4 + 1], dk[db][gq * 4 + 2], dk[db][gq * 4 + 3]};
                *(f32x4*)(wv + o) = f32x4{dv[db][gq * 4], dv[db][gq * 4 + 1], dv[db][gq * 4 + 2], dv[db][gq * 4 + 3]};
            }
        return;
    }
    const float nanv = __builtin_nanf("");
    bf16* dkp = (bf16*)p.dk + ko * p.dks0 + kr * p.dks1 + (int64_t)hk * p.dks2;
    bf16* dvp = (bf16*)p.dv + ko * p.dvs0 + kr * p.dvs1 + (int64_t)hk * p.dvs2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 wk, wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wk[e] = (bf16)(len_error ? nanv : dk[db][gq * 4 + e] * f.scale);
                wv[e] = (bf16)(len_error ? nanv : dv[db][gq * 4 + e]);
            }
            *(bf16x4*)(dkp + db * 32 + gq * 8 + 4 * hh) = wk;
            *(bf16x4*)(dvp + db * 32 + gq * 8 + 4 * hh) = wv;
        }
    }
}

// Sum of the query-head splits of the dK/dV pass: for every (batch, key,
// kv head) row, dk = scale * sum_s wk[s] and dv = sum_s wv[s], the splits
// added in order (the result does not depend on which split ran first).
// Eight values of a row per thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdDev p) {
    constexpr int TPR = D / 8;
    const FwdDev& f = p.f;
    const int64_t rows = (int64_t)f.B * f.Sk * f.Hkv;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = t / TPR;
    if (r >= rows) return;
    const int d = (int)(t - r * TPR) * 8;
    const int hk = (int)(r % f.Hkv);
    const int64_t bk = r / f.Hkv;
    const int key = (int)(bk % f.Sk);
    const int b = (int)(bk / f.Sk);
    const int64_t sstride = rows * D;  // floats per split of one tensor
    const float* wk = p.ws + r * D + d;
    const float* wv = wk + (int64_t)p.gsplit * sstride;
    f32x4 k0 = *(const f32x4*)wk, k1 = *(const f32x4*)(wk + 4);
    f32x4 v0 = *(const f32x4*)wv, v1 = *(const f32x4*)(wv + 4);
    for (int s = 1; s < p.gsplit; ++s) {
        k0 += *(const f32x4*)(wk + s * sstride);
        k1 += *(const f32x4*)(wk + s * sstride + 4);
        v0 += *(const f32x4*)(wv + s * sstride);
        v1 += *(const f32x4*)(wv + s * sstride + 4);
    }
    bf16* dkp = (bf16*)p.dk + (int64_t)b * p.dks0 + (int64_t)key * p.dks1 + (int64_t)hk * p.dks2 + d;
    bf16* dvp = (bf16*)p.dv + (int64_t)b * p.dvs0 + (int64_t)key * p.dvs1 + (int64_t)hk * p.dvs2 + d;
    bf16x4 a, c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (bf16)(k0[e] * f.scale);
        c[e] = (bf16)v0[e];
    }
    *(bf16x4*)dkp = a;
    *(bf16x4*)dvp = c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (bf16)(k1[e] * f.scale);
        c[e] = (bf16)v1[e];
    }
    *(bf16x4*)(dkp + 4) = a;
    *(bf16x4*)(dvp + 4) = c;
}

// ---------------------------------------------------------------------------
// dQ pass: one workgroup per forward query tile (BM = 32 * NW rows; 64 for
// BSR, 128 otherwise), walking the forward's key tiles with the same tile
// cursor and the same per-element masks.
// ---------------------------------------------------------------------------

template <int D, int NW, int KIND, int MOD, int BN = kBN>
// Two waves per SIMD except for 2-wave workgroups over 64-key tiles. (The
// block-id variant once ran one wave per SIMD to avoid spills; with its key
// block ids staged in LDS it spills at most 4 VGPRs at two waves, and the
// block-id GQA dQ pass runs 0.164 -> 0.115 ms.)
__global__ __launch_bounds__(NW * 64, (BN == 32 || NW != 2) ? 2 : 1) void bwd_dq_kernel(BwdDev p, MaskDev m) {
    constexpr bool BIAS = (MOD & kModBias) != 0, CAP = (MOD & kModCap) != 0;
    constexpr int BM = NW * 32;
    constexpr int ROWB = 2 * D, TILEB = BN * ROWB, NKC = D / 16, NDB = D / 32;
    constexpr int NH = BN / 32;  // 32-key halves per key tile
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sK = smem;                 // [2][64 x D]
    char* sV = smem + 2 * TILEB;     // [2][64 x D]
    int32_t* sKB = (int32_t*)(smem + 4 * TILEB);  // [2][BN] key block ids (block-id masks)

    const FwdDev& f = p.f;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hh = lane >> 5, c = lane & 31;

    const int logical = xcd_logical(blockIdx.x, f.total, f.xcd_remap);
    const TileRange t = make_range<KIND, BM, BN>(f, m, logical);
    if (!t.active) return;
    const int row = t.q_row0 + wave * 32 + c;
    RowMask<KIND> rm;
    rm.init(f, m, t, row);

    bf16x8 qf[NKC], of[NKC];
    {
        const bf16* qp = (const bf16*)f.q + (int64_t)t.b * f.qs0 + (int64_t)row * f.qs1 + (int64_t)t.hq * f.qs2 + hh * 8;
        const bf16* op = (const bf16*)p.dout + (int64_t)t.b * p.dos0 + (int64_t)row * p.dos1 +
                         (int64_t)t.hq * p.dos2 + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            qf[kc] = rm.row_ok ? *(const bf16x8*)(qp + kc * 16) : bf16x8{};
            of[kc] = rm.row_ok ? *(const bf16x8*)(op + kc * 16) : bf16x8{};
        }
    }
    const int64_t lrow = ((int64_t)t.b * f.Hq + t.hq) * f.Sq + row;
    const float l2 = rm.row_ok ? lse_log2(f.lse[lrow]) : INFINITY;
    const float dl = rm.row_ok ? p.delta[lrow] : 0.f;
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

    const char* kbase = (const char*)f.k + 2 * ((int64_t)t.b * f.ks0 + (int64_t)t.hk * f.ks2 + (int64_t)t.k_base * f.ks1);
    const char* vbase = (const char*)f.v + 2 * ((int64_t)t.b * f.vs0 + (int64_t)t.hk * f.vs2 + (int64_t)t.k_base * f.vs1);
    const float c2 = f.c2;

    int krow_off[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) krow_off[kc] = row_off<D>(c, kc * 2 + hh);
    int trk[2][NDB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db) trk[j][db] = tr_off<D>(8 * j + 4 * hh, db, lane);

    TileCursor<KIND, BM, BN> cursor;
    cursor.init(f, m, t, lane);
    auto fine_words = [&](int kt_, int kind_, uint32_t (&w)[2]) {
        tile_mask_words<KIND, NH>(m, t, rm, row, kt_, kind_, w);
    };
    // Where key tile kt_ lies: K and V bases and the row range [r0, rend).
    auto tile_src = [&](int kt_, const char*& kb_, const char*& vb_, int& r0, int& rend) {
        kb_ = kbase;
        vb_ = vbase;
        r0 = kt_ * BN;
        rend = t.k_len;
        if constexpr (KIND == MFA_MASK_VARLEN) {
            if (m.block_table) {
                // paged keys: the tile lies inside one page (page_size is a
                // multiple of 64); a bad page id reads as zeros (the
                // sequence's rows are NaN)
                int r = 0;
                const int pg = page_of(m, t.seq, kt_ * BN, r);
                const int n = pg >= 0 ? min(BN, t.k_len - kt_ * BN) : 0;
                kb_ = (const char*)f.k + 2 * ((int64_t)max(pg, 0) * f.ks0 + (int64_t)t.hk * f.ks2);
                vb_ = (const char*)f.v + 2 * ((int64_t)max(pg, 0) * f.vs0 + (int64_t)t.hk * f.vs2);
                r0 = r;
                rend = r + n;
            }
        }
    };
    auto stage = [&](int kt_, int buf) {
        const char *kb_, *vb_;
        int r0, rend;
        tile_src(kt_, kb_, vb_, r0, rend);
        stage_tile<D, BN>(kb_, 2 * f.ks1, r0, rend, sK + buf * TILEB, wave, NW, lane);
        stage_tile<D, BN>(vb_, 2 * f.vs1, r0, rend, sV + buf * TILEB, wave, NW, lane);
    };
    // The next tile's K and V are staged by single instructions spread over
    // the step's first operand groups (TileDma); lane offsets of this wave's
    // instructions wave + NW*k, by k & 1.
    using Dma = TileDma<D, BN>;
    constexpr int NPW = Dma::NINST / NW;  // instructions per wave and tensor
    static_assert(NPW * NW == Dma::NINST && NW >= 2, "tile rows must split evenly over the waves");
    int k_loff[2], v_loff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        k_loff[j] = Dma::lane_off(wave + NW * j, lane, 2 * f.ks1);
        v_loff[j] = Dma::lane_off(wave + NW * j, lane, 2 * f.vs1);
    }
    // Block-id masks: wave 0 loads the raw key block ids of a partial (or
    // ragged) tile into a register (lane = key) with the tile's K/V, and at
    // the end of the step stores them, folded with the key validity bits,
    // into the tile's LDS slot.
    auto kblk_raw = [&](int kt_, int kind_) -> int {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            static_assert(BN == 64, "block-id masks walk 64-key tiles");
            if (wave == 0 && (kind_ == kTilePartial || (kt_ + 1) * BN > t.k_len))
                return blockid_key_raw<BN>(f, m, t, kt_, lane);
        }
        return INT32_MAX;
    };
    auto kblk_store = [&](int kt_, int raw, const uint32_t (&w)[2], int32_t* dst) {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (wave == 0) dst[lane] = blockid_key_fold<BN>(t, kt_, raw, w, lane);
        }
    };

    float sl = 0.f;  // bias slope in raw score units
    int d_row = 0;   // 4*hh - this lane's query position (local to the sequence)
    if constexpr (BIAS) {
        sl = f.alibi[t.hq] / f.scale;
        d_row = 4 * hh - (row - t.q_base);
    }

    int it = t.begin, kt = 0, kind = kTileEmpty;
    cursor.seek(f, m, t, lane, it, kt, kind);
    uint32_t fw[2];
    fine_words(kt, kind, fw);
    if (it < t.end) {
        stage(kt, 0);
        kblk_store(kt, kblk_raw(kt, kind), fw, sKB);
    }
    vm_wait();
    __syncthreads();
    int buf = 0;
    while (it < t.end) {
        int it_n = it + 1, kt_n = kt, kind_n = kTileEmpty;
        cursor.seek(f, m, t, lane, it_n, kt_n, kind_n);
        const bool has_next = it_n < t.end;
        uint32_t fw_n[2];
        fine_words(kt_n, has_next ? kind_n : kTileEmpty, fw_n);
        // restrict-qualified views of the two buffers: the reads of this
        // tile carry alias scopes that keep the compiler from making them
        // wait for the loads into the other buffer
        auto step = [&](const char* __restrict__ k_, const char* __restrict__ v_, char* __restrict__ nk_,
                        char* __restrict__ nv_, const int32_t* __restrict__ kb_, int32_t* __restrict__ nkb_) {
            // Without a next tile the instructions are still issued, with an
            // empty range (they write zeros into the free buffer), so that
            // the MFMA phase carries no branch per instruction.
            Dma dmk, dmv;
            {
                const char *kb_, *vb_;
                int r0, rend;
                tile_src(has_next ? kt_n : kt, kb_, vb_, r0, rend);
                if (!has_next) rend = r0;
                dmk.init(kb_, 2 * f.ks1, r0, rend);
                dmv.init(vb_, 2 * f.vs1, r0, rend);
            }
            const int kraw_n = kblk_raw(kt_n, has_next ? kind_n : kTileEmpty);
            // The two 32-key halves one after the other: S^T = K Q^T and
            // dP^T = V dO^T (G1 operand groups, two MFMAs each), then dS,
            // then dQ^T += K^T dS^T over the half's two 16-key chunks (G2
            // groups). The LDS operand reads of all groups form one stream
            // issued PF groups ahead of their MFMAs (a ring of PF + 1 slots).
            constexpr int G1 = NKC, G2 = 2 * NDB, GH = G1 + G2, GT = NH * GH, PF = 3, RING = PF + 1;
            static_assert(2 * NPW <= GT, "one staging instruction per operand group");
            bf16x8 ra[RING], rb[RING];
            auto load_group = [&](int i) {
                const int h = i / GH, j = i % GH, slot = i % RING;
                if (j < G1) {
                    ra[slot] = *(const bf16x8*)(k_ + h * 32 * ROWB + krow_off[j]);
                    rb[slot] = *(const bf16x8*)(v_ + h * 32 * ROWB + krow_off[j]);
                } else {
                    const int jj = j - G1, k2 = jj / NDB, db = jj % NDB;
                    const int o0 = (h * 2 + k2) * 16 * ROWB;
                    const bf16x4 lo = tr_read(k_ + o0 + trk[0][db]);
                    const bf16x4 hi = tr_read(k_ + o0 + trk[1][db]);
                    ra[slot] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            };
            f32x16 sh, dph;
            bf16x8 sb[2];
#pragma unroll
            for (int i = 0; i < PF; ++i) load_group(i);
#pragma clang loop unroll(full)
            for (int i = 0; i < GT; ++i) {
                const int h = i / GH, j = i % GH, slot = i % RING;
                if (j == 0) {
                    if constexpr (BIAS) {
                        f32x16 t2[NH];
                        alibi_fill(t2, sl, kt * BN + d_row, sl);
                        sh = t2[h];
                    } else {
                        sh = f32x16{};
                    }
                    dph = f32x16{};
                }
                if (i + PF < GT) load_group(i + PF);
                if (i < 2 * NPW) {
                    const int k = i >> 1, ii = wave + NW * k;
                    if (i & 1) dmv.issue(nv_, ii, v_loff[k & 1]);
                    else dmk.issue(nk_, ii, k_loff[k & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (j < G1) {
                    sh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot], qf[j], sh, 0, 0, 0);
                    dph = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[slot], of[j], dph, 0, 0, 0);
                } else {
                    const int jj = j - G1, k2 = jj / NDB, db = jj % NDB;
                    dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot], sb[k2], dq[db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (j == G1 - 1) {
                    if constexpr (CAP) {  // soft cap before the mask
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) sh[rr] = softcap_raw(sh[rr], f);
                    }
                    if (__builtin_expect(kind == kTilePartial || (kt + 1) * BN > t.k_len, 0)) {
                        f32x16 s2[NH];
#pragma unroll
                        for (int x = 0; x < NH; ++x) s2[x] = x == h ? sh : f32x16{};
                        mask_scores<KIND, NH>(f, m, t, rm, row, hh, kt, fw, s2,
                                              KIND == MFA_MASK_BLOCKID ? kb_ : nullptr);
                        sh = s2[h];
                    }
                    // register r is key kt*64 + h*32 + (r>>2)*8 + 4*hh + (r&3)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const float pv = fast_exp2(fmaf(sh[rr], c2, -l2));
                        float ds = pv * (dph[rr] - dl);
                        if constexpr (CAP) ds *= softcap_grad(sh[rr], f);
                        sb[rr >> 3][rr & 7] = (bf16)ds;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            kblk_store(kt_n, kraw_n, fw_n, nkb_);
        };
        step(sK + buf * TILEB, sV + buf * TILEB, sK + (buf ^ 1) * TILEB, sV + (buf ^ 1) * TILEB, sKB + buf * BN,
             sKB + (buf ^ 1) * BN);
        vm_wait();
        __syncthreads();
        buf ^= 1;
        it = it_n;
        kt = kt_n;
        kind = kind_n;
        fw[0] = fw_n[0];
        fw[1] = fw_n[1];
    }

    if (!rm.row_ok) return;
    const float nanv = __builtin_nanf("");
    bf16* dqp = (bf16*)p.dq + (int64_t)t.b * p.dqs0 + (int64_t)row * p.dqs1 + (int64_t)t.hq * p.dqs2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 w;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) w[e4] = (bf16)(t.len_error ? nanv : dq[db][gq * 4 + e4] * f.scale);
            *(bf16x4*)(dqp + db * 32 + gq * 8 + 4 * hh) = w;
        }
}

// ---------------------------------------------------------------------------
// fp32 test mode: scalar kernels that walk the same lists with the same
// predicates as the bf16 passes (the dK/dV pass the key block's query-block
// list and allowed_qk, the dQ pass the forward's tile schedule and the
// per-element predicate of sched.hpp), in fp32 arithmetic with libm exp, so
// that the mask logic of both passes is checked at tight tolerance.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_f32_kernel(BwdDev p) {
    const int64_t rows = (int64_t)p.f.B * p.f.Sq * p.f.Hq;
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const int h = (int)(r % p.f.Hq);
    const int64_t bi = r / p.f.Hq;
    const int i = (int)(bi % p.f.Sq);
    const int b = (int)(bi / p.f.Sq);
    const float* o = (const float*)p.f.o + (int64_t)b * p.f.os0 + (int64_t)i * p.f.os1 + (int64_t)h * p.f.os2;
    const float* d = (const float*)p.dout + (int64_t)b * p.dos0 + (int64_t)i * p.dos1 + (int64_t)h * p.dos2;
    float acc = 0.f;
    for (int e = 0; e < D; ++e) acc = fmaf(o[e], d[e], acc);
    p.delta[((int64_t)b * p.f.Hq + h) * p.f.Sq + i] = acc;
}

// One thread per key: 64-key blocks as in the bf16 pass (one 64-thread
// workgroup each), summing over the query rows of the listed query blocks
// of every query head of the group.
template <int D, int KIND>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(BwdDev p, MaskDev m) {
    const FwdDev& f = p.f;
    const KeyBlock kb = key_block<KIND>(p, m, blockIdx.x, gridDim.x, false);
    if (!kb.active) return;
    if (KIND == MFA_MASK_VARLEN && kb.len_error && m.err && threadIdx.x == 0) *m.err = 1;
    const int key_l = kb.kbk * 64 + threadIdx.x;
    int64_t ko = 0, kr = 0;  // (batch or page, row) of k, v, dk, dv
    const bool key_addr = key_rows(m, kb, key_l, ko, kr);
    const bool key_ok = key_l < kb.k_len && key_addr;
    int kblk;
    bool kval;
    key_side<KIND>(f, m, kb, key_l, key_ok, kblk, kval);
    QueryBlocks<KIND> qbl;
    qbl.init(f, m, kb);
    const float* kp = (const float*)f.k + ko * f.ks0 + kr * f.ks1 + (int64_t)kb.hk * f.ks2;
    const float* vp = (const float*)f.v + ko * f.vs0 + kr * f.vs1 + (int64_t)kb.hk * f.vs2;
    float dk[D], dv[D];
    for (int e = 0; e < D; ++e) dk[e] = dv[e] = 0.f;
    if (key_ok) {
        for (int g = 0; g < f.G; ++g) {
            const int hq = kb.hk * f.G + g;
            const float slope = f.alibi ? f.alibi[hq] : 0.f;
            for (int pos = qbl.pbeg; pos < qbl.pend; ++pos) {
                const uint32_t ent = qbl.fetch(f, m, kb, pos);
                const int kind = (int)(ent >> 28);
                if (kind == kTileEmpty) continue;
                const int qb = (int)(ent & 0x0FFFFFFFu);
                for (int r = 0; r < 64; ++r) {
                    const int i = qb * 64 + r;
                    if (i >= kb.q_len) break;
                    if (kind == kTilePartial && !allowed_qk<KIND>(f, m, kb.b, kb.q_len, kb.k_len, key_l, i, kblk, kval))
                        continue;
                    const int qrow = kb.q_base + i;
                    const float lse = f.lse[((int64_t)kb.b * f.Hq + hq) * f.Sq + qrow];
                    if (lse == -INFINITY) continue;  // a row with no allowed key
                    const float* qp = (const float*)f.q + (int64_t)kb.b * f.qs0 + (int64_t)qrow * f.qs1 + (int64_t)hq * f.qs2;
                    const float* dp = (const float*)p.dout + (int64_t)kb.b * p.dos0 + (int64_t)qrow * p.dos1 +
                                      (int64_t)hq * p.dos2;
                    float sc = 0.f, dpv = 0.f;
                    for (int e = 0; e < D; ++e) {
                        sc = fmaf(qp[e], kp[e], sc);
                        dpv = fmaf(dp[e], vp[e], dpv);
                    }
                    sc = sc * f.scale + slope * (float)(key_l - i);
                    float gcap = 1.f;  // derivative of the soft cap
                    if (f.cap > 0.f) {
                        const float th = tanhf(sc / f.cap);
                        sc = f.cap * th;
                        gcap = 1.f - th * th;
                    }
                    const float pr = expf(sc - lse);
                    const float ds = pr * (dpv - p.delta[((int64_t)kb.b * f.Hq + hq) * f.Sq + qrow]) * gcap;
                    for (int e = 0; e < D; ++e) {
                        dv[e] = fmaf(pr, dp[e], dv[e]);
                        dk[e] = fmaf(ds, qp[e], dk[e]);
                    }
                }
            }
        }
    }
    // keys past the used length get zero gradients; paged keys outside the
    // table or the pool are not written
    if (key_l >= kb.k_alloc || !key_addr) return;
    float* dkp = (float*)p.dk + ko * p.dks0 + kr * p.dks1 + (int64_t)kb.hk * p.dks2;
    float* dvp = (float*)p.dv + ko * p.dvs0 + kr * p.dvs1 + (int64_t)kb.hk * p.dvs2;
    const float nanv = __builtin_nanf("");
    for (int e = 0; e < D; ++e) {
        dkp[e] = kb.len_error ? nanv : dk[e] * f.scale;
        dvp[e] = kb.len_error ? nanv : dv[e];
    }
}

// One thread per query row of the forward's query tile, walking the
// forward's key tiles (tile_at) with the per-element predicate.
template <int D, int BM, int KIND>
__global__ __launch_bounds__(BM) void bwd_dq_f32_kernel(BwdDev p, MaskDev m) {
    const FwdDev& f = p.f;
    const TileRange t = make_range<KIND, BM>(f, m, blockIdx.x);
    if (!t.active) return;
    const int row = t.q_row0 + threadIdx.x;
    RowMask<KIND> rm;
    rm.init(f, m, t, row);
    if (!rm.row_ok) return;
    const float* qp = (const float*)f.q + (int64_t)t.b * f.qs0 + (int64_t)row * f.qs1 + (int64_t)t.hq * f.qs2;
    const float* dp = (const float*)p.dout + (int64_t)t.b * p.dos0 + (int64_t)row * p.dos1 + (int64_t)t.hq * p.dos2;
    const float* K = (const float*)f.k + (int64_t)t.b * f.ks0 + (int64_t)t.hk * f.ks2 + (int64_t)t.k_base * f.ks1;
    const float* V = (const float*)f.v + (int64_t)t.b * f.vs0 + (int64_t)t.hk * f.vs2 + (int64_t)t.k_base * f.vs1;
    const int64_t lrow = ((int64_t)t.b * f.Hq + t.hq) * f.Sq + row;
    const float lse = f.lse[lrow], dl = p.delta[lrow];
    const float slope = f.alibi ? f.alibi[t.hq] : 0.f;
    float q[D], dq[D];
    for (int e = 0; e < D; ++e) {
        q[e] = qp[e];
        dq[e] = 0.f;
    }
    if (lse != -INFINITY) {
        for (int it = t.begin; it < t.end; ++it) {
            int kt, kind;
            tile_at<KIND, BM>(f, m, t, it, kt, kind);
            if (kind == kTileEmpty) continue;
            for (int j = 0; j < kBN; ++j) {
                const int key = kt * kBN + j;
                if (key >= t.k_len) break;
                if (kind == kTilePartial && !allowed<KIND>(f, m, t, rm, key)) continue;
                const float* kr = K + (int64_t)key * f.ks1;
                const float* vr = V + (int64_t)key * f.vs1;
                if constexpr (KIND == MFA_MASK_VARLEN) {
                    if (m.block_table) {  // paged keys: (page, row in page)
                        int r = 0;
                        const int pg = page_of(m, t.seq, key, r);
                        if (pg < 0) continue;  // the sequence's rows are NaN (len_error)
                        kr = (const float*)f.k + (int64_t)pg * f.ks0 + (int64_t)r * f.ks1 + (int64_t)t.hk * f.ks2;
                        vr = (const float*)f.v + (int64_t)pg * f.vs0 + (int64_t)r * f.vs1 + (int64_t)t.hk * f.vs2;
                    }
                }
                float sc = 0.f, dpv = 0.f;
                for (int e = 0; e < D; ++e) {
                    sc = fmaf(q[e], kr[e], sc);
                    dpv = fmaf(dp[e], vr[e], dpv);
                }
                sc = sc * f.scale + slope * (float)(key - (row - t.q_base));
                float gcap = 1.f;  // derivative of the soft cap
                if (f.cap > 0.f) {
                    const float th = tanhf(sc / f.cap);
                    sc = f.cap * th;
                    gcap = 1.f - th * th;
                }
                const float ds = expf(sc - lse) * (dpv - dl) * gcap;
                for (int e = 0; e < D; ++e) dq[e] = fmaf(ds, kr[e], dq[e]);
            }
        }
    }
    float* dqp = (float*)p.dq + (int64_t)t.b * p.dqs0 + (int64_t)row * p.dqs1 + (int64_t)t.hq * p.dqs2;
    for (int e = 0; e < D; ++e) dqp[e] = t.len_error ? __builtin_nanf("") : dq[e] * f.scale;
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------

static hipError_t launch_bwd_preprocess_f32(const BwdDev& p, int D, hipStream_t s) {
    const int64_t rows = (int64_t)p.f.B * p.f.Sq * p.f.Hq;
    const int grid = (int)((rows + 255) / 256);
    if (grid == 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(bwd_preprocess_f32_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bwd_preprocess_f32_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const BwdDev& p, int D, int dtype, hipStream_t s) {
    if (dtype == MFA_F32) return launch_bwd_preprocess_f32(p, D, s);
    const int64_t rows = (int64_t)p.f.B * p.f.Sq * p.f.Hq;
    const int per_wg = 4 * (64 / (D / 8));
    const int grid = (int)((rows + per_wg - 1) / per_wg);
    if (grid == 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

// The score modifications of the call as the kernels' template bits.
static int mod_bits(const FwdDev& f) { return (f.alibi ? kModBias : 0) | (f.cap > 0.f ? kModCap : 0); }

template <int D, int KIND, int MOD>
static hipError_t dkdv_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    // Q / dO double buffers, LSE and delta, query block ids, validity bits, fine words
    const size_t lds = 4 * 64 * 2 * D + 4 * 64 * sizeof(float) + 2 * 64 * 4 + 16 + 2 * 2 * 64 * 4;
    hipError_t e = hipFuncSetAttribute((const void*)&bwd_dkdv_kernel<D, KIND, MOD>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int S = p.gsplit > 1 ? p.gsplit : 1;
    const int64_t grid = KIND == MFA_MASK_VARLEN
                             ? (int64_t)m.nseq * p.f.Hkv * ((m.max_k + 63) / 64)
                             : (int64_t)p.f.B * p.f.Hkv * S * ((p.f.Sk + 63) / 64);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, KIND, MOD>), dim3((unsigned)grid), dim3(128), lds, s, p, m);
    if (S > 1) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t threads = (int64_t)p.f.B * p.f.Sk * p.f.Hkv * (D / 8);
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <int D, int KIND>
static hipError_t dkdv_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (mod_bits(p.f)) {
        case 0: return dkdv_launch<D, KIND, 0>(p, m, s);
        case kModBias: return dkdv_launch<D, KIND, kModBias>(p, m, s);
        case kModCap: return dkdv_launch<D, KIND, kModCap>(p, m, s);
        default: return dkdv_launch<D, KIND, kModBias | kModCap>(p, m, s);
    }
}

template <int D, int NW, int KIND, int MOD>
static hipError_t dq_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    // 64-row query tiles walk 32-key tiles, as in the forward
    constexpr int BN = (NW == 2 && (KIND == MFA_MASK_BSR || KIND == MFA_MASK_TILES)) ? 32 : kBN;
    // K / V double buffers, and the key block ids of block-id masks
    const size_t lds = 4 * (size_t)BN * 2 * D + (KIND == MFA_MASK_BLOCKID ? 2 * BN * sizeof(int32_t) : 0);
    if (p.f.total == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void*)&bwd_dq_kernel<D, NW, KIND, MOD, BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, KIND, MOD, BN>), dim3(p.f.total), dim3(NW * 64), lds, s, p, m);
    return hipGetLastError();
}

// 64-row query tiles (BSR blocks, 64-row dense-tile maps) run 2 waves, 128-row ones 4.
template <int D, int NW, int KIND>
static hipError_t dq_launch_mod(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (mod_bits(p.f)) {
        case 0: return dq_launch<D, NW, KIND, 0>(p, m, s);
        case kModBias: return dq_launch<D, NW, KIND, kModBias>(p, m, s);
        case kModCap: return dq_launch<D, NW, KIND, kModCap>(p, m, s);
        default: return dq_launch<D, NW, KIND, kModBias | kModCap>(p, m, s);
    }
}

template <int D, int KIND>
static hipError_t dq_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    if constexpr (KIND == MFA_MASK_BSR) {
        return dq_launch_mod<D, 2, KIND>(p, m, s);
    } else if constexpr (KIND == MFA_MASK_TILES) {
        if (m.tile_shift == 0) return dq_launch_mod<D, 2, KIND>(p, m, s);
        return dq_launch_mod<D, 4, KIND>(p, m, s);
    } else {
        return dq_launch_mod<D, 4, KIND>(p, m, s);
    }
}

template <int D, int KIND>
static hipError_t dkdv_f32_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    const int64_t grid = KIND == MFA_MASK_VARLEN
                             ? (int64_t)m.nseq * p.f.Hkv * ((m.max_k + 63) / 64)
                             : (int64_t)p.f.B * p.f.Hkv * ((p.f.Sk + 63) / 64);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, KIND>), dim3((unsigned)grid), dim3(64), 0, s, p, m);
    return hipGetLastError();
}

template <int D, int KIND>
static hipError_t dq_f32_launch(const BwdDev& p, const MaskDev& m, int BM, hipStream_t s) {
    if (p.f.total == 0) return hipSuccess;
    if (BM == 64) hipLaunchKernelGGL((bwd_dq_f32_kernel<D, 64, KIND>), dim3(p.f.total), dim3(64), 0, s, p, m);
    else hipLaunchKernelGGL((bwd_dq_f32_kernel<D, 128, KIND>), dim3(p.f.total), dim3(128), 0, s, p, m);
    return hipGetLastError();
}

template <int D>
static hipError_t dkdv_f32_kind(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (m.kind) {
        case MFA_MASK_NONE: return dkdv_f32_launch<D, MFA_MASK_NONE>(p, m, s);
        case MFA_MASK_BLOCKID: return dkdv_f32_launch<D, MFA_MASK_BLOCKID>(p, m, s);
        case MFA_MASK_TILES: return dkdv_f32_launch<D, MFA_MASK_TILES>(p, m, s);
        case MFA_MASK_BSR: return dkdv_f32_launch<D, MFA_MASK_BSR>(p, m, s);
        case MFA_MASK_VARLEN: return dkdv_f32_launch<D, MFA_MASK_VARLEN>(p, m, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t dq_f32_kind(const BwdDev& p, const MaskDev& m, int BM, hipStream_t s) {
    switch (m.kind) {
        case MFA_MASK_NONE: return dq_f32_launch<D, MFA_MASK_NONE>(p, m, BM, s);
        case MFA_MASK_BLOCKID: return dq_f32_launch<D, MFA_MASK_BLOCKID>(p, m, BM, s);
        case MFA_MASK_TILES: return dq_f32_launch<D, MFA_MASK_TILES>(p, m, BM, s);
        case MFA_MASK_BSR: return dq_f32_launch<D, MFA_MASK_BSR>(p, m, BM, s);
        case MFA_MASK_VARLEN: return dq_f32_launch<D, MFA_MASK_VARLEN>(p, m, BM, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t dkdv_kind(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (m.kind) {
        case MFA_MASK_NONE: return dkdv_launch<D, MFA_MASK_NONE>(p, m, s);
        case MFA_MASK_BLOCKID: return dkdv_launch<D, MFA_MASK_BLOCKID>(p, m, s);
        case MFA_MASK_TILES: return dkdv_launch<D, MFA_MASK_TILES>(p, m, s);
        case MFA_MASK_BSR: return dkdv_launch<D, MFA_MASK_BSR>(p, m, s);
        case MFA_MASK_VARLEN: return dkdv_launch<D, MFA_MASK_VARLEN>(p, m, s);
    }
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t dq_kind(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (m.kind) {
        case MFA_MASK_NONE: return dq_launch<D, MFA_MASK_NONE>(p, m, s);
        case MFA_MASK_BLOCKID: return dq_launch<D, MFA_MASK_BLOCKID>(p, m, s);
        case MFA_MASK_TILES: return dq_launch<D, MFA_MASK_TILES>(p, m, s);
        case MFA_MASK_BSR: return dq_launch<D, MFA_MASK_BSR>(p, m, s);
        case MFA_MASK_VARLEN: return dq_launch<D, MFA_MASK_VARLEN>(p, m, s);
    }
    return hipErrorInvalidValue;
}

// Static device scratch of the no-allocation dK/dV entry point: the fp32
// partial sums of the query-head split live here instead of in a caller
// workspace. Each device holds its own copy from module load to process
// exit; calls on one device share it (overlapping calls race). Every byte a
// split reads is written by the same call's dK/dV kernel first, so nothing
// is cleared between calls.
static __device__ __align__(256) char scratch[kBwdScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device, once known
}  // namespace

// The device address of this device's scratch array (host code must pass
// this, never the array's name, to kernels). Looked up once per device, with
// that device current.
hipError_t bwd_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = q;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_bwd_dkdv(const BwdDev& p, const MaskDev& m, int D, int dtype, hipStream_t s) {
    if (dtype == MFA_F32) return D == 128 ? dkdv_f32_kind<128>(p, m, s) : dkdv_f32_kind<64>(p, m, s);
    return D == 128 ? dkdv_kind<128>(p, m, s) : dkdv_kind<64>(p, m, s);
}

hipError_t launch_bwd_dq(const BwdDev& p, const MaskDev& m, int D, int dtype, int BM, hipStream_t s) {
    if (dtype == MFA_F32) return D == 128 ? dq_f32_kind<128>(p, m, BM, s) : dq_f32_kind<64>(p, m, BM, s);
    return D == 128 ? dq_kind<128>(p, m, s) : dq_kind<64>(p, m, s);
}

}  // namespace mfa
