// Fused masked attention forward for gfx950.
//
// out = softmax(scale * q k^T restricted to allowed keys) v, with the mask
// applied per 64-key tile and never materialised as a dense score matrix
// (the shared method of the opentau flash_attn_cuda, BinFlash, flashinfer
// block_sparse_attention and tensorplay varlen pages). Empty tiles are never
// visited, full tiles run with no mask work, partial tiles evaluate the
// representation's predicate per element.
//
// bf16 kernel, one workgroup = NW waves = BM = 32*NW query rows of one
// (batch, query head):
//  * Each wave owns 32 queries. Scores are computed transposed,
//    S^T (64 keys x 32 queries) = K Q^T, with v_mfma_f32_32x32x16_bf16: the
//    accumulator then holds one query per lane (lane & 31) and 16 of its keys
//    per 32-key block, so the row max needs one cross-half exchange
//    (v_permlane32_swap) and the probabilities are already laid out as the
//    B operand of O^T (D x 32 queries) += V^T P^T. Both contractions run over
//    the same permutation of keys, which is free since keys are summed over.
//  * K and V tiles (64 x D bf16; 32 x D for 64-row query tiles, so that two
//    or more of their 2-wave workgroups fit on a CU) are double-buffered in
//    LDS, XOR-swizzled so that the K operand reads (ds_read_b128) and the
//    transposed V operand reads (ds_read_b64_tr_b16) are bank-conflict free.
//    The next tile's loads go straight from memory to LDS, a few between the
//    S MFMAs; block-id masks stage the tile's key block ids alongside.
//  * Online softmax in fp32 with exp2: c = scale*log2(e) is applied to the
//    fp32 scores after the matmul. The running max is only moved when the
//    tile max exceeds it by more than kTau (log2 units), which bounds P by
//    2^kTau and removes nearly all O rescales. The row sum adds the fp32 P
//    (the bf16 rounding of a dominant P, up to 2^-8 relative, would otherwise
//    show up in the log-sum-exp); P.V uses P rounded to bf16.
//  * Epilogue: O / l rounded to bf16 (RNE), LSE = scale*m + ln l in fp32;
//    rows with no allowed key write +0 and -inf.
//  * Workgroup ids are remapped so that the query tiles of one (batch, head)
//    run on one XCD (its L2 holds that head's K/V), heaviest tiles first.
//
// fp32 test-mode kernel: same schedule and predicates, one thread per query
// row, fp32 arithmetic with libm exp/log, used to check the tiling and masking
// logic at tight tolerance.

#include <type_traits>

#include "sched.hpp"

namespace mfa {

constexpr float kTau = 8.0f;

template <int D>
struct KV {
    static constexpr int ROWB = D * 2;
    static constexpr int CPR = D / 8;  // 16-byte chunks per row
    static constexpr int TILEB = kBN * ROWB;
    // Physical 16-byte chunk of logical chunk lc in row r.
    __device__ static __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static __forceinline__ int v_swz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Wait for every vector-memory operation of this wave (the K/V tile loads
// into LDS included).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bf16x4 ds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(__attribute__((address_space(3))) char*)(p));
}

// BN: key-tile width, kBN or 32 (BSR rows with 64-row query blocks: a 2-wave
// workgroup then needs 32 KB of LDS instead of 64, so four fit on a CU and
// each SIMD runs two waves, which hide each other's wait for the next tile).
// MOD: score modifications compiled in (kModBias: per-head slope bias,
// kModCap: soft cap); the unmodified variant pays for neither.
template <int D, int NW, int KIND, int MOD, int BN = kBN>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_bf16_kernel(FwdDev p, MaskDev m) {
    constexpr bool BIAS = (MOD & kModBias) != 0, CAP = (MOD & kModCap) != 0;
    constexpr int BM = NW * 32;
    constexpr int NT = NW * 64;
    constexpr int ROWB = KV<D>::ROWB;
    constexpr int CPR = KV<D>::CPR;
    constexpr int TILEB = BN * ROWB;
    constexpr int NB = BN / 32;              // 32-key blocks of S^T per tile
    constexpr int NK16 = BN / 16;            // 16-key chunks of the P V contraction
    constexpr int NKC = D / 16;              // 16-wide d chunks of q.k
    constexpr int NDB = D / 32;              // 32-wide d blocks of O^T

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sK = smem;
    char* sV = smem + 2 * TILEB;
    // block-id masks: the k_blk values of the K/V tile, staged with it ([2][64])
    int32_t* sKB = (int32_t*)(smem + 4 * TILEB);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases scalar
    const int hh = lane >> 5;
    const int c = lane & 31;

    const int logical = xcd_logical(blockIdx.x, p.total, p.xcd_remap);
    const TileRange t = make_range<KIND, BM, BN>(p, m, logical);
    if (!t.active) return;

    const int row = t.q_row0 + wave * 32 + c;
    RowMask<KIND> rm;
    rm.init(p, m, t, row);

    const bf16* Q = (const bf16*)p.q;
    const bf16* K = (const bf16*)p.k;
    const bf16* V = (const bf16*)p.v;

    bf16x8 qf[NKC];
    {
        const bf16* qp = Q + (int64_t)t.b * p.qs0 + (int64_t)row * p.qs1 + (int64_t)t.hq * p.qs2 + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            if (rm.row_ok) qf[kc] = *(const bf16x8*)(qp + kc * 16);
            else qf[kc] = bf16x8{};
        }
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float M = 0.f;  // scaled running max (log2 units); 0 until the row has seen an allowed key
    // threshold of the shifted tile max that moves M: -inf until the row has
    // seen an allowed key (its first finite max sets M), kTau after that
    float thr = -INFINITY;
    float l_part = 0.f;

    // ---- staging of K/V tiles: direct global->LDS buffer loads ----
    // One wave instruction moves 1 KB = RPI rows into a contiguous LDS block;
    // lane l lands at byte 16*l of it, i.e. row RPI*i + l/CPR, physical chunk
    // l%CPR, so it fetches the logical chunk that the swizzle puts there.
    // Rows past the key length read as zeros (buffer range check).
    constexpr int RPI = 1024 / ROWB;             // rows per wave instruction
    constexpr int NI = BN / RPI / NW;            // instructions per wave per tile (each of K, V)
    static_assert(NI * RPI * NW == BN, "tile rows must split evenly over the waves");
    const char* Kbh = (const char*)K + 2 * ((int64_t)t.b * p.ks0 + (int64_t)t.hk * p.ks2 + (int64_t)t.k_base * p.ks1);
    const char* Vbh = (const char*)V + 2 * ((int64_t)t.b * p.vs0 + (int64_t)t.hk * p.vs2 + (int64_t)t.k_base * p.vs1);
    const int64_t krow = 2 * p.ks1, vrow = 2 * p.vs1;
    // 32-bit row strides: the host requires 128 rows to span under 2 GiB
    const int krow32 = (int)krow, vrow32 = (int)vrow;
    int kgo[NI], vgo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (wave * NI + i) * RPI + lane / CPR;
        const int pc = lane % CPR;
        kgo[i] = (int)(r * krow) + ((pc ^ KV<D>::k_swz(r)) << 4);
        vgo[i] = (int)(r * vrow) + ((pc ^ KV<D>::v_swz(r)) << 4);
    }
    // `live` false issues the same loads with an empty range (they write
    // zeros into the free buffer), which keeps the loop free of a branch.
    // Paged keys (varlen with a block table): each tile lies inside one page,
    // found through the table (the tile range checked every page id; a bad
    // one turned the rows into NaN, and its tiles read as zeros here).
    auto tile_base = [&](int kt, bool live, const char*& kp, const char*& vp, int& kn, int& vn) {
        const int64_t k0 = (int64_t)kt * BN * krow, v0 = (int64_t)kt * BN * vrow;
        kp = Kbh + k0;
        vp = Vbh + v0;
        // the range ends at the tile's last row or at the last key, whichever
        // comes first, so it fits 32 bits however long the sequence is
        const int rem = live ? min(BN, t.k_len - kt * BN) : 0;
        kn = rem > 0 ? (rem - 1) * krow32 + ROWB : 0;
        vn = rem > 0 ? (rem - 1) * vrow32 + ROWB : 0;
        if constexpr (KIND == MFA_MASK_VARLEN) {
            if (m.block_table) {
                int r = 0;
                const int pg = page_of(m, t.seq, kt * kBN, r);
                const bool ok = pg >= 0;
                const int rows = min(kBN, t.k_len - kt * kBN);
                kp = Kbh + 2 * ((int64_t)max(pg, 0) * p.ks0 + (int64_t)r * p.ks1);
                vp = Vbh + 2 * ((int64_t)max(pg, 0) * p.vs0 + (int64_t)r * p.vs1);
                kn = (live && ok && rows > 0) ? (int)((rows - 1) * krow + ROWB) : 0;
                vn = (live && ok && rows > 0) ? (int)((rows - 1) * vrow + ROWB) : 0;
            }
        }
    };
    auto load_tile_to = [&](int kt, char* dk, char* dv, bool live) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource builtins exist only in the device pass
        const char *kp, *vp;
        int kn, vn;
        tile_base(kt, live, kp, vp, kn, vn);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, kn, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, vn, 0x00020000);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int blk = (wave * NI + i) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dk + blk), 16, kgo[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dv + blk), 16, vgo[i], 0, 0, 0);
        }
#endif
    };
    auto load_tile = [&](int kt, int buf, bool live) { load_tile_to(kt, sK + buf * TILEB, sV + buf * TILEB, live); };
    // Block-id masks: wave 0 loads the raw key block ids of a partial (or
    // ragged) tile into a register (lane = key) with the tile's K/V, and at
    // the end of the step stores them, folded with the key validity bits,
    // into the tile's LDS slot.
    auto kblk_raw = [&](int kt_, int kind_) -> int {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            static_assert(BN == 64, "block-id masks walk 64-key tiles");
            if (wave == 0 && (kind_ == kTilePartial || (kt_ + 1) * BN > t.k_len))
                return blockid_key_raw<BN>(p, m, t, kt_, lane);
        }
        return INT32_MAX;
    };
    auto kblk_store = [&](int kt_, int raw, const uint32_t (&w)[2], int32_t* dst) {
        if constexpr (KIND == MFA_MASK_BLOCKID) {
            if (wave == 0) dst[lane] = blockid_key_fold<BN>(t, kt_, raw, w, lane);
        }
    };

    // Per-lane LDS offsets of the operand reads.
    // K operand: row kb*32 + c, logical chunk kc*2 + hh.
    int koff[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) koff[kc] = c * ROWB + (((kc * 2 + hh) ^ KV<D>::k_swz(c)) << 4);
    // V operand (transposed read): row kc2*16 + 8j + 4hh + rq, column
    // db*32 + 16*((lane>>4)&1) + 4*(lane&3).
    const int rq = (lane & 15) >> 2;
    int voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int vr0 = 4 * hh + rq;
        voff[db] = vr0 * ROWB + (((col >> 3) ^ KV<D>::v_swz(vr0)) << 4) + ((col >> 2) & 1) * 8;
    }

    TileCursor<KIND, BM, BN> cursor;
    cursor.init(p, m, t, lane);
    auto advance = [&](int& it, int& kt, int& kind) { cursor.seek(p, m, t, lane, it, kt, kind); };

    // The mask words of a partial (or ragged) tile, loaded one tile ahead
    // together with that tile's K/V.
    auto fine_words = [&](int kt_, int kind_, uint32_t (&w)[2]) {
        tile_mask_words<KIND, NB>(m, t, rm, row, kt_, kind_, w);
    };

    int it = t.begin, kt = 0, kind = 0;
    advance(it, kt, kind);
    uint32_t fw[2];
    fine_words(kt, kind, fw);
    if (it < t.end) {
        load_tile(kt, 0, true);
        kblk_store(kt, kblk_raw(kt, kind), fw, sKB);
    }
    wait_vmem();
    __syncthreads();

    const float c2 = p.c2;
    float sl = 0.f;  // bias slope in raw score units
    int d_row = 0;   // 4*hh - this lane's query position (local to the sequence)
    if constexpr (BIAS) {
        sl = p.alibi[t.hq] / p.scale;
        d_row = 4 * hh - (row - t.q_base);
    }
    // One tile with the buffer parity BUF known at compile time, so that
    // every LDS operand read and DMA target is a per-lane base plus an
    // immediate offset; the loop below runs it for buffers 0 and 1 in turn.
    auto iter = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        int it_n = it + 1, kt_n = kt, kind_n = kTileEmpty;
        advance(it_n, kt_n, kind_n);
        const bool has_next = it_n < t.end;
        if (!has_next) kt_n = kt, kind_n = kTileEmpty;
        uint32_t fw_n[2];
        fine_words(kt_n, kind_n, fw_n);
        // restrict-qualified views of the two buffers: the reads of this
        // tile carry alias scopes that keep the compiler from making them
        // wait for the loads into the other buffer
        auto step = [&](const char* __restrict__ ck_, const char* __restrict__ cv_, char* __restrict__ nk_,
                        char* __restrict__ nv_, const int32_t* __restrict__ ckb_, int32_t* __restrict__ nkb_) {
            const int kraw_n = kblk_raw(kt_n, kind_n);
            // The next tile's K and V loads (into buf^1, released by the last
            // barrier) are issued a few at a time between the S MFMAs below
            // rather than as one burst, which would stall the wave on the
            // vector memory queue.
            constexpr int NDMA = 2 * NI, DPK = (NDMA + NKC - 1) / NKC;  // loads per d chunk
#if defined(__HIP_DEVICE_COMPILE__)
            const char *kp_, *vp_;
            int kn_, vn_;
            tile_base(kt_n, has_next, kp_, vp_, kn_, vn_);
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kp_, 0, kn_, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vp_, 0, vn_, 0x00020000);
#endif
            auto dma = [&](int j) {
#if defined(__HIP_DEVICE_COMPILE__)
                const int i = j >> 1, blk = (wave * NI + i) * 1024;
                if (j & 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(nv_ + blk), 16, vgo[i], 0, 0, 0);
                else __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(nk_ + blk), 16, kgo[i], 0, 0, 0);
#endif
            };

            // ---- S^T = K Q^T ----
            f32x16 s[NB];
            if constexpr (BIAS) {
                alibi_fill(s, sl, kt * BN + d_row, sl);
            } else {
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) s[kb] = f32x16{};
            }
            const char* kb_ = ck_;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) {
                    const bf16x8 a = *(const bf16x8*)(kb_ + kb * 32 * ROWB + koff[kc]);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[kb], 0, 0, 0);
                }
#pragma unroll
                for (int d = 0; d < DPK; ++d)
                    if (kc * DPK + d < NDMA) dma(kc * DPK + d);
            }
            // keep the loads spread: per d chunk, NB operand reads, NB MFMAs, DPK loads
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
                if (kc * DPK < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, DPK, 0);
            }
            // ---- soft cap (before the mask: masked scores stay -inf) ----
            if constexpr (CAP) {
#pragma unroll
                for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = softcap_raw(s[kb][r], p);
            }

            // ---- mask on partial or ragged tiles ----
            if (__builtin_expect(kind == kTilePartial || (kt + 1) * BN > t.k_len, 0))
                mask_scores<KIND, NB>(p, m, t, rm, row, hh, kt, fw, s, KIND == MFA_MASK_BLOCKID ? ckb_ : nullptr);

            // ---- online softmax ----
            // Scores are scaled and shifted first, t = s*c - M (M: the scaled
            // running max, 0 until the row has seen a key), and the tile max
            // is taken over t: t comes out of an FMA, so the max needs no
            // NaN canonicalisation, and the exponent argument is ready. M is
            // only moved when the tile max exceeds it by more than kTau.
            // Row max and row sum as 4 independent chains each (short
            // dependency chains: a single wave issues them back to back).
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c2, -M);
            float mx4[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], s[kb][r]);
            float T = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
            T = max_both_halves(T);
            // T = -inf: no allowed key of this row in the tile, M stays
            const bool need = T > thr;
            if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
                const float sh = need ? T : 0.f;
                const float alpha = (need && thr == kTau) ? fast_exp2(-T) : 1.f;
                M += sh;
                thr = need ? kTau : thr;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
                for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] -= sh;
            }
            bf16x8 pb[NK16];
            float rs4[4];
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int gp = 0; gp < 2; ++gp)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pv = fast_exp2(s[kb][gp * 8 + e]);
                        if (kb == 0 && gp == 0 && e < 4) rs4[e] = pv;
                        else rs4[e & 3] += pv;
                        pb[kb * 2 + gp][e] = (bf16)pv;
                    }
            l_part += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);

            // ---- O^T += V^T P^T ----
            const char* vb_ = cv_;
#pragma unroll
            for (int kc2 = 0; kc2 < NK16; ++kc2) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x4 lo = ds_read_tr(vb_ + kc2 * 16 * ROWB + voff[db]);
                    const bf16x4 hi = ds_read_tr(vb_ + (kc2 * 16 + 8) * ROWB + voff[db]);
                    const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], o[db], 0, 0, 0);
                }
            }
            kblk_store(kt_n, kraw_n, fw_n, nkb_);
        };
        step(sK + buf * TILEB, sV + buf * TILEB, sK + (buf ^ 1) * TILEB, sV + (buf ^ 1) * TILEB, sKB + buf * 64,
             sKB + (buf ^ 1) * 64);

        wait_vmem();  // this wave's tile loads have landed in LDS
        __syncthreads();
        it = it_n;
        kt = kt_n;
        kind = kind_n;
        fw[0] = fw_n[0];
        fw[1] = fw_n[1];
    };
    while (it < t.end) {
        iter(std::integral_constant<int, 0>{});
        if (it >= t.end) break;
        iter(std::integral_constant<int, 1>{});
    }

    // ---- epilogue ----
    const float l_tot = sum_both_halves(l_part);
    if (!rm.row_ok) return;
    const bool empty = !(l_tot > 0.f);
    float inv = empty ? 0.f : 1.f / l_tot;
    if (t.len_error) inv = __builtin_nanf("");
    bf16* op = (bf16*)p.o + (int64_t)t.b * p.os0 + (int64_t)row * p.os1 + (int64_t)t.hq * p.os2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = empty && !t.len_error ? (bf16)0.f : (bf16)(o[db][g * 4 + e] * inv);
            *(bf16x4*)(op + db * 32 + g * 8 + 4 * hh) = w;
        }
    }
    if (p.lse && hh == 0) {
        float L = empty ? -INFINITY : (M + fast_log2(l_tot)) * kLn2;
        if (t.len_error) L = __builtin_nanf("");
        p.lse[((int64_t)t.b * p.Hq + t.hq) * p.Sq + row] = L;
    }
}

// fp32 test mode: one thread per query row, scalar fp32 arithmetic.
template <int D, int BM, int KIND>
__global__ __launch_bounds__(BM) void attn_fwd_f32_kernel(FwdDev p, MaskDev m) {
    const TileRange t = make_range<KIND, BM>(p, m, blockIdx.x);
    if (!t.active) return;
    const int row = t.q_row0 + threadIdx.x;
    RowMask<KIND> rm;
    rm.init(p, m, t, row);
    const float* Q = (const float*)p.q;
    const float* K = (const float*)p.k + (int64_t)t.b * p.ks0 + (int64_t)t.hk * p.ks2 + (int64_t)t.k_base * p.ks1;
    const float* V = (const float*)p.v + (int64_t)t.b * p.vs0 + (int64_t)t.hk * p.vs2 + (int64_t)t.k_base * p.vs1;
    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = rm.row_ok ? Q[(int64_t)t.b * p.qs0 + (int64_t)row * p.qs1 + (int64_t)t.hq * p.qs2 + d] : 0.f;
        o[d] = 0.f;
    }
    float mrun = -INFINITY, l = 0.f;
    for (int it = t.begin; it < t.end; ++it) {
        int kt, kind;
        tile_at<KIND, BM>(p, m, t, it, kt, kind);
        if (kind == kTileEmpty || !rm.row_ok) continue;
        for (int j = 0; j < kBN; ++j) {
            const int key = kt * kBN + j;
            if (key >= t.k_len) break;
            if (kind == kTilePartial && !allowed<KIND>(p, m, t, rm, key)) continue;
            const float* kp = K + (int64_t)key * p.ks1;
            const float* vp = V + (int64_t)key * p.vs1;
            if constexpr (KIND == MFA_MASK_VARLEN) {
                if (m.block_table) {
                    int r = 0;
                    const int pg = page_of(m, t.seq, key, r);
                    if (pg < 0) continue;  // the tile range flagged this sequence
                    kp = K + (int64_t)pg * p.ks0 + (int64_t)r * p.ks1;
                    vp = V + (int64_t)pg * p.vs0 + (int64_t)r * p.vs1;
                }
            }
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) s = fmaf(q[d], kp[d], s);
            s *= p.scale;
            if (p.alibi) s += p.alibi[t.hq] * (float)(key - (row - t.q_base));
            if (p.cap > 0.f) s = p.cap * tanhf(s / p.cap);
            const float mn = fmaxf(mrun, s);
            const float corr = expf(mrun - mn);
            const float pe = expf(s - mn);
            l = l * corr + pe;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(pe, vp[d], o[d] * corr);
            mrun = mn;
        }
    }
    if (!rm.row_ok) return;
    const bool empty = !(l > 0.f);
    float* op = (float*)p.o + (int64_t)t.b * p.os0 + (int64_t)row * p.os1 + (int64_t)t.hq * p.os2;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = t.len_error ? __builtin_nanf("") : (empty ? 0.f : o[d] / l);
    if (p.lse) p.lse[((int64_t)t.b * p.Hq + t.hq) * p.Sq + row] =
        t.len_error ? __builtin_nanf("") : (empty ? -INFINITY : mrun + logf(l));
}

// ---------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------

template <int D, int NW, int KIND>
static hipError_t launch_bf16(const FwdDev& p, const MaskDev& m, hipStream_t s) {
    // 64-row BSR blocks walk 32-key tiles (two waves per SIMD); everything else 64-key tiles
    constexpr int BN = ((KIND == MFA_MASK_BSR || KIND == MFA_MASK_TILES) && NW == 2) ? 32 : kBN;
    const size_t lds = 4 * (size_t)BN * KV<D>::ROWB + (KIND == MFA_MASK_BLOCKID ? 2 * 64 * 4 : 0);
    const dim3 grid(p.total), block(NW * 64);
    switch ((p.alibi ? kModBias : 0) | (p.cap > 0.f ? kModCap : 0)) {
        case 0: hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, KIND, 0, BN>), grid, block, lds, s, p, m); break;
        case kModBias:
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, KIND, kModBias, BN>), grid, block, lds, s, p, m);
            break;
        case kModCap:
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, KIND, kModCap, BN>), grid, block, lds, s, p, m);
            break;
        default:
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, KIND, kModBias | kModCap, BN>), grid, block, lds, s, p,
                               m);
    }
    return hipGetLastError();
}

template <int D, int BM, int KIND>
static hipError_t launch_f32(const FwdDev& p, const MaskDev& m, hipStream_t s) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BM, KIND>), dim3(p.total), dim3(BM), 0, s, p, m);
    return hipGetLastError();
}

template <int KIND>
static hipError_t dispatch_kind(int dtype, int D, int BM, const FwdDev& p, const MaskDev& m, hipStream_t s) {
    if (dtype == MFA_BF16) {
        if (BM == 128) return D == 128 ? launch_bf16<128, 4, KIND>(p, m, s) : launch_bf16<64, 4, KIND>(p, m, s);
        return D == 128 ? launch_bf16<128, 2, KIND>(p, m, s) : launch_bf16<64, 2, KIND>(p, m, s);
    }
    if (BM == 128) return D == 128 ? launch_f32<128, 128, KIND>(p, m, s) : launch_f32<64, 128, KIND>(p, m, s);
    return D == 128 ? launch_f32<128, 64, KIND>(p, m, s) : launch_f32<64, 64, KIND>(p, m, s);
}

hipError_t launch_attn_fwd(int dtype, int D, int BM, const FwdDev& p, const MaskDev& m, hipStream_t s) {
    switch (m.kind) {
        case MFA_MASK_NONE: return dispatch_kind<MFA_MASK_NONE>(dtype, D, BM, p, m, s);
        case MFA_MASK_BLOCKID: return dispatch_kind<MFA_MASK_BLOCKID>(dtype, D, BM, p, m, s);
        case MFA_MASK_TILES: return dispatch_kind<MFA_MASK_TILES>(dtype, D, BM, p, m, s);
        case MFA_MASK_BSR: return dispatch_kind<MFA_MASK_BSR>(dtype, D, BM, p, m, s);
        case MFA_MASK_VARLEN: return dispatch_kind<MFA_MASK_VARLEN>(dtype, D, BM, p, m, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mfa
