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
// (RPI rows), instruction i filling LDS bytes [1024 i, 1024 i + 1024).
template <int D>
struct TileDma {
    static constexpr int ROWB = 2 * D, RPI = 1024 / ROWB, CPR = D / 8, NINST = 64 / RPI;
    __amdgpu_buffer_rsrc_t rs;
    int64_t row_bytes;
    __device__ __forceinline__ void init(const char* base, int64_t rb, int row0, int rows) {
#if defined(__HIP_DEVICE_COMPILE__)
        row_bytes = rb;
        const int64_t start = (int64_t)row0 * rb;
        const int rem = min(64, rows - row0);  // as in stage_tile
        const int nrec = rem > 0 ? (rem - 1) * (int)rb + ROWB : 0;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + start), 0, nrec, 0x00020000);
#endif
    }
    __device__ __forceinline__ void issue(char* lds, int i, int lane) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const int r = i * RPI + lane / CPR;
        const int pc = lane % CPR;
        const int go = (int)(r * row_bytes) + ((pc ^ tswz<D>(r)) << 4);
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

// Allowed bits of one 32-query half in the dK/dV layout: bit rr says whether
// query qi0 + (rr>>2)*8 + 4*hh + (rr&3) (index within the batch entry or the
// varlen sequence) may attend to this lane's key key_l. Used on partial
// blocks only; full blocks need none, empty blocks are never visited.
template <int KIND>
__device__ __forceinline__ uint32_t allowed_bits_T(const FwdDev& f, const MaskDev& m, int b, int q_len, int k_len,
                                                   int key_l, int qi0, int hh, int kblk, bool kval) {
    uint32_t bits = 0;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int i = qi0 + (rr >> 2) * 8 + 4 * hh + (rr & 3);
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
        bits |= (ok ? 1u : 0u) << rr;
    }
    return bits;
}

// One workgroup (2 waves, 64 keys) per (batch or varlen sequence, kv head,
// 64-key block). The query blocks that can attend to the key block come from
// the CSC list (BSR), the dense tile map or the block-id summaries (both at
// 128-row granularity: a 64-row block takes its tile's kind), the window
// arithmetic (varlen) or all blocks (no mask); they are walked through a
// ScanWindow, once per query head of the GQA group.
template <int D, int KIND, bool BIAS>
__global__ __launch_bounds__(128, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdDev p, MaskDev m) {
    constexpr int ROWB = 2 * D, TILEB = 64 * ROWB, NKC = D / 16, NDB = D / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sQ = smem;                                   // [2][64 x D] Q
    char* sO = smem + 2 * TILEB;                       // [2][64 x D] dO
    float* sL = (float*)(smem + 4 * TILEB);            // [2][64] -LSE * log2(e)
    float* sDl = sL + 128;                             // [2][64] delta

    const FwdDev& f = p.f;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hh = lane >> 5, c = lane & 31;

    int b = 0, hk = 0, kbk = 0;
    int q_base = 0, q_len = f.Sq, k_base = 0, k_len = f.Sk;
    int k_alloc = f.Sk;  // keys whose gradient rows are written (k_len of them are attended)
    bool len_error = false;
    if constexpr (KIND == MFA_MASK_VARLEN) {
        const int nKbm = (m.max_k + 63) / 64;
        // plain numbering: sequences differ in length, and round-robin over
        // the XCDs keeps their work balanced
        kbk = blockIdx.x % nKbm;
        const int sh = blockIdx.x / nKbm;
        hk = sh % f.Hkv;
        const int seq = sh / f.Hkv;
        q_base = m.cu_q[seq];
        q_len = m.cu_q[seq + 1] - q_base;
        k_base = m.cu_k[seq];
        k_alloc = m.cu_k[seq + 1] - k_base;
        k_len = m.seqused_k ? min(k_alloc, max(m.seqused_k[seq], 0)) : k_alloc;
        if (kbk * 64 >= k_alloc) return;
        if (q_len > m.max_q || k_alloc > m.max_k) {
            len_error = true;
            if (m.err && threadIdx.x == 0) *m.err = 1;
        }
    } else {
        const int nKb = (f.Sk + 63) / 64;
        // consecutive key blocks of one (batch, head) on one XCD, so that
        // they share that XCD's L2 copy of the head's Q and dO
        const int wg = xcd_logical(blockIdx.x, gridDim.x, (gridDim.x & 7) == 0);
        const int bh = wg / nKb;
        kbk = wg - bh * nKb;
        b = bh / f.Hkv;
        hk = bh - b * f.Hkv;
    }
    const int key_l = kbk * 64 + wave * 32 + c;  // key within the batch entry / sequence
    const bool key_ok = key_l < k_len;
    const int key = k_base + key_l;              // row of k, v, dk, dv

    // stationary K and V fragments (B operands: K^T, V^T with lane = key)
    bf16x8 kf[NKC], vf[NKC];
    {
        const bf16* kp = (const bf16*)f.k + (int64_t)b * f.ks0 + (int64_t)key * f.ks1 + (int64_t)hk * f.ks2 + hh * 8;
        const bf16* vp = (const bf16*)f.v + (int64_t)b * f.vs0 + (int64_t)key * f.vs1 + (int64_t)hk * f.vs2 + hh * 8;
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
    // key-side mask values
    int kblk = INT32_MAX;
    bool kval = false;
    if constexpr (KIND == MFA_MASK_BLOCKID) {
        if (key_ok) {
            kblk = m.k_blk[(int64_t)b * f.Sk + key_l];
            kval = (m.kv_bits[(int64_t)b * m.kv_words + (key_l >> 5)] >> (key_l & 31)) & 1u;
        }
    }
    // BSR token validity: whole-block state from the block's two words
    bool blk_all_valid = true, blk_any_valid = true;
    if constexpr (KIND == MFA_MASK_BSR) {
        kval = true;
        if (m.kv_bits) {
            const uint32_t* kw = m.kv_bits + (int64_t)b * m.kv_words + 2 * kbk;
            const uint32_t w0 = kw[0], w1 = (2 * kbk + 1 < m.kv_words) ? kw[1] : 0u;
            blk_all_valid = w0 == 0xFFFFFFFFu && w1 == 0xFFFFFFFFu;
            blk_any_valid = (w0 | w1) != 0u;
            kval = key_ok && (((key_l < 32 + kbk * 64 ? w0 : w1) >> (key_l & 31)) & 1u);
        }
    }

    // ---- the query blocks of this key block ----
    const int nQb = (q_len + 63) / 64;
    int pbeg = 0, pend = nQb, e0 = 0;
    if constexpr (KIND == MFA_MASK_BSR) {
        const int nKb = (f.Sk + 63) / 64;
        const int* cp = m.csc_ptr + ((int64_t)b * f.Hkv + hk) * (nKb + 1);
        e0 = cp[kbk];
        pend = blk_any_valid ? cp[kbk + 1] - e0 : 0;
    } else if constexpr (KIND == MFA_MASK_VARLEN) {
        const int j0 = kbk * 64, j1 = min(j0 + 63, k_len - 1);
        int lo = 0, hi = j1 >= j0 ? q_len - 1 : -1;  // no used key in the block: no query block
        if (m.causal) lo = max(lo, j0);
        if (m.win_right >= 0) lo = max(lo, j0 - m.win_right);
        if (m.win_left >= 0) hi = min(hi, j1 + m.win_left);
        pbeg = lo / 64;
        pend = hi >= lo ? hi / 64 + 1 : pbeg;
    }
    auto fetch = [&](int pos) -> uint32_t {
        if (pos >= pend) return 0u;
        int qb = pos, kind = kTileFull;
        if constexpr (KIND == MFA_MASK_BSR) {
            qb = m.csc_idx[e0 + pos];
            kind = bsr_kind_of(qb, kbk, 64, 64, f.Sq, f.Sk, m.causal);
            if (kind == kTileFull && !blk_all_valid) kind = kTilePartial;
        } else if constexpr (KIND == MFA_MASK_TILES) {
            kind = m.tile_kind[(int64_t)(qb >> m.tile_shift) * f.nKt + kbk];
        } else if constexpr (KIND == MFA_MASK_BLOCKID) {
            kind = classify_blockid(m.qsum + ((int64_t)b * f.nQt + (qb >> 1)) * 4,
                                    m.ksum + ((int64_t)b * f.nKt + kbk) * 4);
        } else if constexpr (KIND == MFA_MASK_VARLEN) {
            const int i0 = qb * 64, i1 = min(i0 + 63, q_len - 1);
            const int j0 = kbk * 64, j1 = min(j0 + 63, k_len - 1);
            bool full = (i1 - i0 == 63) && (j1 - j0 == 63);
            if (m.causal) full = full && j1 <= i0;
            if (m.win_left >= 0) full = full && i1 - j0 <= m.win_left;
            if (m.win_right >= 0) full = full && j1 - i0 <= m.win_right;
            kind = full ? kTileFull : kTilePartial;
        }
        return (uint32_t)qb | ((uint32_t)kind << 28);
    };
    ScanWindow win;
    win.init(fetch, pbeg, lane);
    int g = 0, pos = pbeg;
    uint32_t ent = 0;
    bool have = win.seek(fetch, pos, pend, lane, ent);
    auto next_step = [&](int& g_, int& pos_, uint32_t& ent_) -> bool {
        ++pos_;
        if (win.seek(fetch, pos_, pend, lane, ent_)) return true;
        if (++g_ >= f.G) return false;
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
    auto stage = [&](int g_, uint32_t ent_, int buf) {
        stage_to(g_, ent_, sQ + buf * TILEB, sO + buf * TILEB, sDl + buf * 64);
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

    if (have) {
        stage(g, ent, 0);
        if (wave == 0) lse_store(lse_fetch(g, ent), 0);
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
            constexpr int NPW = TileDma<D>::NINST / 2;
            TileDma<D> dmq, dmo;
            if (have_n) {
                if constexpr (SPREAD) {
                    const int hq = hk * f.G + g_n;
                    const int qbn = (int)(ent_n & 0x0FFFFFFFu);
                    const char* qbp = (const char*)f.q + 2 * ((int64_t)b * f.qs0 + (int64_t)hq * f.qs2);
                    const char* obp = (const char*)p.dout + 2 * ((int64_t)b * p.dos0 + (int64_t)hq * p.dos2);
                    const int r0 = q_base + qbn * 64, rend = q_base + q_len;
                    dmq.init(qbp, 2 * f.qs1, r0, rend);
                    dmo.init(obp, 2 * p.dos1, r0, rend);
                    const int64_t lrow = ((int64_t)b * f.Hq + hq) * f.Sq;
                    if (wave == 1) stage_vec64(p.delta + lrow, r0, rend, nd_, lane);
                } else {
                    stage_to(g_n, ent_n, nq_, no_, nd_);
                }
                if (wave == 0) lse_n = lse_fetch(g_n, ent_n);
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
                if (SPREAD && i < 2 * NPW && have_n) {
                    const int ii = wave + 2 * (i >> 1);  // instruction index within the tile
                    if (i & 1) dmo.issue(no_, ii, lane);
                    else dmq.issue(nq_, ii, lane);
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
                    // partial blocks: disallowed scores become -inf (P = 0 there);
                    // register r is query h*32 + (r>>2)*8 + 4*hh + (r&3)
                    if (__builtin_expect(kind == kTilePartial, 0)) {
                        const uint32_t okb =
                            allowed_bits_T<KIND>(f, m, b, q_len, k_len, key_l, qb * 64 + h * 32, hh, kblk, kval);
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
                            const float ds = pv * (dp[rr] - DL[gq][e]);
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
        vm_wait();
        __syncthreads();
        buf ^= 1;
        have = have_n;
        g = g_n;
        pos = pos_n;
        ent = ent_n;
    }

    if (key_l >= k_alloc) return;  // keys past the used length get zero gradients
    const float nanv = __builtin_nanf("");
    bf16* dkp = (bf16*)p.dk + (int64_t)b * p.dks0 + (int64_t)key * p.dks1 + (int64_t)hk * p.dks2;
    bf16* dvp = (bf16*)p.dv + (int64_t)b * p.dvs0 + (int64_t)key * p.dvs1 + (int64_t)hk * p.dvs2;
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

// ---------------------------------------------------------------------------
// dQ pass: one workgroup per forward query tile (BM = 32 * NW rows; 64 for
// BSR, 128 otherwise), walking the forward's key tiles with the same tile
// cursor and the same per-element masks.
// ---------------------------------------------------------------------------

template <int D, int NW, int KIND, bool BIAS, int BN = kBN>
__global__ __launch_bounds__(NW * 64, (BN == 32 || (NW != 2 && KIND != MFA_MASK_BLOCKID)) ? 2 : 1) void bwd_dq_kernel(BwdDev p, MaskDev m) {
    constexpr int BM = NW * 32;
    constexpr int ROWB = 2 * D, TILEB = BN * ROWB, NKC = D / 16, NDB = D / 32;
    constexpr int NH = BN / 32;  // 32-key halves per key tile
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sK = smem;                 // [2][64 x D]
    char* sV = smem + 2 * TILEB;     // [2][64 x D]

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
        w[0] = w[1] = 0u;
        if constexpr (KIND == MFA_MASK_TILES) {
            if (rm.row_ok && (kind_ == kTilePartial || (kt_ + 1) * BN > t.k_len)) {
                const uint32_t* fb = m.fine_bits + (int64_t)row * m.fine_words + NH * kt_;
                w[0] = fb[0];
                if (NH == 2 && 2 * kt_ + 1 < m.fine_words) w[1] = fb[1];
            }
        }
    };
    auto stage_to = [&](int kt_, char* dk_, char* dv_) {
        stage_tile<D, BN>(kbase, 2 * f.ks1, kt_ * BN, t.k_len, dk_, wave, NW, lane);
        stage_tile<D, BN>(vbase, 2 * f.vs1, kt_ * BN, t.k_len, dv_, wave, NW, lane);
    };
    auto stage = [&](int kt_, int buf) { stage_to(kt_, sK + buf * TILEB, sV + buf * TILEB); };

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
    if (it < t.end) stage(kt, 0);
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
                        char* __restrict__ nv_) {
            if (has_next) stage_to(kt_n, nk_, nv_);
            // The two 32-key halves one after the other: S^T = K Q^T and
            // dP^T = V dO^T (G1 operand groups, two MFMAs each), then dS,
            // then dQ^T += K^T dS^T over the half's two 16-key chunks (G2
            // groups). The LDS operand reads of all groups form one stream
            // issued PF groups ahead of their MFMAs (a ring of PF + 1 slots).
            constexpr int G1 = NKC, G2 = 2 * NDB, GH = G1 + G2, GT = NH * GH, PF = 3, RING = PF + 1;
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
                    if (__builtin_expect(kind == kTilePartial || (kt + 1) * BN > t.k_len, 0)) {
                        f32x16 s2[NH];
#pragma unroll
                        for (int x = 0; x < NH; ++x) s2[x] = x == h ? sh : f32x16{};
                        mask_scores<KIND, NH>(f, m, t, rm, row, hh, kt, fw, s2);
                        sh = s2[h];
                    }
                    // register r is key kt*64 + h*32 + (r>>2)*8 + 4*hh + (r&3)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const float pv = fast_exp2(fmaf(sh[rr], c2, -l2));
                        sb[rr >> 3][rr & 7] = (bf16)(pv * (dph[rr] - dl));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        step(sK + buf * TILEB, sV + buf * TILEB, sK + (buf ^ 1) * TILEB, sV + (buf ^ 1) * TILEB);
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
// Host launch
// ---------------------------------------------------------------------------

hipError_t launch_bwd_preprocess(const BwdDev& p, int D, hipStream_t s) {
    const int64_t rows = (int64_t)p.f.B * p.f.Sq * p.f.Hq;
    const int per_wg = 4 * (64 / (D / 8));
    const int grid = (int)((rows + per_wg - 1) / per_wg);
    if (grid == 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D, int KIND, bool BIAS>
static hipError_t dkdv_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    const size_t lds = 4 * 64 * 2 * D + 4 * 64 * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void*)&bwd_dkdv_kernel<D, KIND, BIAS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t grid = KIND == MFA_MASK_VARLEN
                             ? (int64_t)m.nseq * p.f.Hkv * ((m.max_k + 63) / 64)
                             : (int64_t)p.f.B * p.f.Hkv * ((p.f.Sk + 63) / 64);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, KIND, BIAS>), dim3((unsigned)grid), dim3(128), lds, s, p, m);
    return hipGetLastError();
}

template <int D, int KIND>
static hipError_t dkdv_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    return p.f.alibi ? dkdv_launch<D, KIND, true>(p, m, s) : dkdv_launch<D, KIND, false>(p, m, s);
}

template <int D, int NW, int KIND, bool BIAS>
static hipError_t dq_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    // 64-row query tiles walk 32-key tiles, as in the forward
    constexpr int BN = (NW == 2 && (KIND == MFA_MASK_BSR || KIND == MFA_MASK_TILES)) ? 32 : kBN;
    const size_t lds = 4 * (size_t)BN * 2 * D;
    if (p.f.total == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, KIND, BIAS, BN>), dim3(p.f.total), dim3(NW * 64), lds, s, p, m);
    return hipGetLastError();
}

// 64-row query tiles (BSR blocks, 64-row dense-tile maps) run 2 waves, 128-row ones 4.
template <int D, int KIND>
static hipError_t dq_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    if constexpr (KIND == MFA_MASK_BSR) {
        return p.f.alibi ? dq_launch<D, 2, KIND, true>(p, m, s) : dq_launch<D, 2, KIND, false>(p, m, s);
    } else if constexpr (KIND == MFA_MASK_TILES) {
        if (m.tile_shift == 0)
            return p.f.alibi ? dq_launch<D, 2, KIND, true>(p, m, s) : dq_launch<D, 2, KIND, false>(p, m, s);
        return p.f.alibi ? dq_launch<D, 4, KIND, true>(p, m, s) : dq_launch<D, 4, KIND, false>(p, m, s);
    } else {
        return p.f.alibi ? dq_launch<D, 4, KIND, true>(p, m, s) : dq_launch<D, 4, KIND, false>(p, m, s);
    }
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

hipError_t launch_bwd_dkdv(const BwdDev& p, const MaskDev& m, int D, hipStream_t s) {
    return D == 128 ? dkdv_kind<128>(p, m, s) : dkdv_kind<64>(p, m, s);
}

hipError_t launch_bwd_dq(const BwdDev& p, const MaskDev& m, int D, hipStream_t s) {
    return D == 128 ? dq_kind<128>(p, m, s) : dq_kind<64>(p, m, s);
}

}  // namespace mfa
