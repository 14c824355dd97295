// Backward of masked attention for BSR block-sparse masks on gfx950.
//
// The split follows the BinFlash method ("Backward uses two passes: dKdV over
// K-blocks, dQ over Q-blocks, with the same gathered dispatch"), here over the
// flashinfer-style BSR rows and their column-major copy:
//   preprocess  delta_i = sum_d dO_id * O_id                       (fp32)
//   dK/dV pass  one workgroup per (batch, kv head, 64-key block); it walks
//               the query blocks that list this key block (CSC), for every
//               query head of the GQA group, and accumulates
//               dV += P^T dO and dK += scale * dS^T Q in registers;
//   dQ pass     one workgroup per (batch, query head, 64-query block); it walks
//               the row's key blocks (CSR) and accumulates dQ += scale * dS K.
// P = exp2(s * scale*log2e - LSE*log2e) is recomputed from the forward's LSE,
// dS = P o (dP - delta), dP = dO V^T. No atomics: every output element is
// written by exactly one workgroup, so results are deterministic.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16): in the dK/dV pass scores are
// computed as S = Q K^T so that a lane owns one key and 16 of the queries; the
// bf16 P and dS are then directly the B operands of dV^T = dO^T P and
// dK^T = Q^T dS, whose A operands are transposed reads (ds_read_b64_tr_b16) of
// the Q / dO tiles. The dQ pass uses the forward's S^T = K Q^T layout (a lane
// owns one query) and reads K^T transposed for dQ^T = K^T dS^T.
// Q, dO (dK/dV pass) and K (dQ pass) tiles are read both row-wise and
// transposed; their LDS swizzle is conflict-free for both patterns.

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
template <int D>
__device__ __forceinline__ void stage_tile(const char* base, int64_t row_bytes, int row0, int rows, char* lds,
                                           int wave, int nw, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int ROWB = 2 * D, RPI = 1024 / ROWB, CPR = D / 8, NINST = 64 / RPI;
    const int64_t start = (int64_t)row0 * row_bytes;
    const int64_t total = rows > 0 ? (int64_t)(rows - 1) * row_bytes + ROWB : 0;
    const int nrec = (int)(total > start ? total - start : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + start), 0, nrec, 0x00020000);
    for (int i = wave; i < NINST; i += nw) {
        const int r = i * RPI + lane / CPR;
        const int pc = lane % CPR;
        const int go = (int)(r * row_bytes) + ((pc ^ tswz<D>(r)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + i * 1024), 16, go, 0, 0, 0);
    }
#endif
}

// Stage 64 consecutive fp32 values (positions [i0, i0+64) of a row of length n).
__device__ __forceinline__ void stage_vec64(const float* base, int i0, int n, float* lds, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int nrec = n > i0 ? (n - i0) * 4 : 0;
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

template <int D>
__global__ __launch_bounds__(128, 1) void bwd_dkdv_kernel(BwdDev p, MaskDev m) {
    constexpr int ROWB = 2 * D, TILEB = 64 * ROWB, NKC = D / 16, NDB = D / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sQ = smem;                                   // [2][64 x D] Q
    char* sO = smem + 2 * TILEB;                       // [2][64 x D] dO
    float* sL = (float*)(smem + 4 * TILEB);            // [2][64] LSE
    float* sDl = sL + 128;                             // [2][64] delta

    const FwdDev& f = p.f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int nKb = (f.Sk + 63) / 64;
    const int bh = blockIdx.x / nKb;
    const int kbk = blockIdx.x - bh * nKb;
    const int b = bh / f.Hkv, hk = bh - b * f.Hkv;
    const int key = kbk * 64 + wave * 32 + c;
    const bool key_ok = key < f.Sk;

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

    const int* cp = m.csc_ptr + (int64_t)bh * (nKb + 1);
    const int e0 = cp[kbk], len = cp[kbk + 1] - e0;
    const int total = len * f.G;
    const float c2 = f.c2;

    // per-lane operand offsets
    int qrow_off[NKC];  // A operand rows of S / dP for query block 0: row c, chunk kc*2 + hh
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qrow_off[kc] = row_off<D>(c, kc * 2 + hh);
    // transposed reads: rows kq*16 + 8j + 4hh + (lane&15)/4; the swizzle depends on (8j + 4hh) & 15
    int trq[2][NDB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db) trq[j][db] = tr_off<D>(8 * j + 4 * hh, db, lane);

    // CSC entries of this key block, read through a register window
    auto fetch_r = [&](int i) { return i < len ? (uint32_t)m.csc_idx[e0 + i] : 0u; };
    ListWindow win;
    win.init(fetch_r, 0, lane);
    auto item = [&](int it, int& hq, int& r) {
        const int g = it / len;
        hq = hk * f.G + g;
        r = (int)win.get(fetch_r, it - g * len, lane);
    };
    auto stage = [&](int it, int buf) {
        int hq, r;
        item(it, hq, r);
        const char* qb = (const char*)f.q + 2 * ((int64_t)b * f.qs0 + (int64_t)hq * f.qs2);
        const char* ob = (const char*)p.dout + 2 * ((int64_t)b * p.dos0 + (int64_t)hq * p.dos2);
        stage_tile<D>(qb, 2 * f.qs1, r * 64, f.Sq, sQ + buf * TILEB, wave, 2, lane);
        stage_tile<D>(ob, 2 * p.dos1, r * 64, f.Sq, sO + buf * TILEB, wave, 2, lane);
        const int64_t row = ((int64_t)b * f.Hq + hq) * f.Sq;
        if (wave == 0) stage_vec64(f.lse + row, r * 64, f.Sq, sL + buf * 64, lane);
        else stage_vec64(p.delta + row, r * 64, f.Sq, sDl + buf * 64, lane);
    };

    if (total > 0) stage(0, 0);
    vm_wait();
    __syncthreads();
    int buf = 0;
    for (int it = 0; it < total; ++it) {
        int hq, r;
        item(it, hq, r);
        if (it + 1 < total) stage(it + 1, buf ^ 1);
        const char* q_ = sQ + buf * TILEB;
        const char* o_ = sO + buf * TILEB;
        const float* l_ = sL + buf * 64;
        const float* d_ = sDl + buf * 64;

        // S = Q K^T and dP = dO V^T for the two 32-query halves
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            s[qb] = f32x16{};
            dp[qb] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 aq = *(const bf16x8*)(q_ + qb * 32 * ROWB + qrow_off[kc]);
                const bf16x8 ao = *(const bf16x8*)(o_ + qb * 32 * ROWB + qrow_off[kc]);
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kc], s[qb], 0, 0, 0);
                dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kc], dp[qb], 0, 0, 0);
            }
        }
        // P and dS; register r of half qb is query qb*32 + (r>>2)*8 + 4*hh + (r&3)
        const int kind = bsr_kind_of(r, kbk, 64, 64, f.Sq, f.Sk, m.causal);
        const bool diag = m.causal && kind == kTilePartial;
        bf16x8 pb[4], sb[4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 L = *(const f32x4*)(l_ + qb * 32 + g * 8 + 4 * hh);
                const f32x4 Dl = *(const f32x4*)(d_ + qb * 32 + g * 8 + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = g * 4 + e;
                    const int qi = r * 64 + qb * 32 + g * 8 + 4 * hh + e;
                    float pv = fast_exp2(fmaf(s[qb][rr], c2, -lse_log2(L[e])));
                    if (diag && key > qi) pv = 0.f;
                    const float ds = pv * (dp[qb][rr] - Dl[e]);
                    pb[qb * 2 + (g >> 1)][(g & 1) * 4 + e] = (bf16)pv;
                    sb[qb * 2 + (g >> 1)][(g & 1) * 4 + e] = (bf16)ds;
                }
            }
        }
        // dV^T += dO^T P ; dK^T += Q^T dS  (k = 16-query chunks)
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int o0 = kq * 16 * ROWB;
                const bf16x4 olo = tr_read(o_ + o0 + trq[0][db]);
                const bf16x4 ohi = tr_read(o_ + o0 + trq[1][db]);
                const bf16x4 qlo = tr_read(q_ + o0 + trq[0][db]);
                const bf16x4 qhi = tr_read(q_ + o0 + trq[1][db]);
                const bf16x8 ao = __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 aq = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[kq], dv[db], 0, 0, 0);
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[kq], dk[db], 0, 0, 0);
            }
        }
        vm_wait();
        __syncthreads();
        buf ^= 1;
    }

    if (!key_ok) return;
    bf16* dkp = (bf16*)p.dk + (int64_t)b * p.dks0 + (int64_t)key * p.dks1 + (int64_t)hk * p.dks2;
    bf16* dvp = (bf16*)p.dv + (int64_t)b * p.dvs0 + (int64_t)key * p.dvs1 + (int64_t)hk * p.dvs2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 wk, wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wk[e] = (bf16)(dk[db][g * 4 + e] * f.scale);
                wv[e] = (bf16)dv[db][g * 4 + e];
            }
            *(bf16x4*)(dkp + db * 32 + g * 8 + 4 * hh) = wk;
            *(bf16x4*)(dvp + db * 32 + g * 8 + 4 * hh) = wv;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ pass
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(128, 2) void bwd_dq_kernel(BwdDev p, MaskDev m) {
    constexpr int ROWB = 2 * D, TILEB = 64 * ROWB, NKC = D / 16, NDB = D / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* sK = smem;                 // [2][64 x D]
    char* sV = smem + 2 * TILEB;     // [2][64 x D]

    const FwdDev& f = p.f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = lane >> 5, c = lane & 31;
    const int nQb = m.nQb;
    const int bh = blockIdx.x / nQb;
    const int r = nQb - 1 - (blockIdx.x - bh * nQb);  // longest rows first
    const int b = bh / f.Hq, hq = bh - b * f.Hq, hk = hq / f.G;
    const int qi = r * 64 + wave * 32 + c;
    const bool q_ok = qi < f.Sq;

    bf16x8 qf[NKC], of[NKC];
    {
        const bf16* qp = (const bf16*)f.q + (int64_t)b * f.qs0 + (int64_t)qi * f.qs1 + (int64_t)hq * f.qs2 + hh * 8;
        const bf16* op = (const bf16*)p.dout + (int64_t)b * p.dos0 + (int64_t)qi * p.dos1 + (int64_t)hq * p.dos2 + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            qf[kc] = q_ok ? *(const bf16x8*)(qp + kc * 16) : bf16x8{};
            of[kc] = q_ok ? *(const bf16x8*)(op + kc * 16) : bf16x8{};
        }
    }
    const int64_t lrow = ((int64_t)b * f.Hq + hq) * f.Sq + qi;
    const float l2 = q_ok ? lse_log2(f.lse[lrow]) : INFINITY;
    const float dl = q_ok ? p.delta[lrow] : 0.f;
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

    const int* ip = m.indptr + ((int64_t)b * f.Hkv + hk) * (nQb + 1);
    const int beg = ip[r], end = ip[r + 1];
    const char* kbase = (const char*)f.k + 2 * ((int64_t)b * f.ks0 + (int64_t)hk * f.ks2);
    const char* vbase = (const char*)f.v + 2 * ((int64_t)b * f.vs0 + (int64_t)hk * f.vs2);
    const float c2 = f.c2;

    int krow_off[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) krow_off[kc] = row_off<D>(c, kc * 2 + hh);
    int trk[2][NDB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db) trk[j][db] = tr_off<D>(8 * j + 4 * hh, db, lane);

    // BSR row entries (block index | kind << 28), read through a register window
    auto fetch_e = [&](int e) {
        return e < end ? (uint32_t)m.indices[e] | ((uint32_t)m.bsr_kind[e] << 28) : 0u;
    };
    ListWindow win;
    win.init(fetch_e, beg, lane);
    auto next = [&](int e) {
        while (e < end && (win.get(fetch_e, e, lane) >> 28) == (uint32_t)kTileEmpty) ++e;
        return e;
    };
    auto stage = [&](int e, int buf) {
        const int kb = (int)(win.get(fetch_e, e, lane) & 0x0FFFFFFFu);
        stage_tile<D>(kbase, 2 * f.ks1, kb * 64, f.Sk, sK + buf * TILEB, wave, 2, lane);
        stage_tile<D>(vbase, 2 * f.vs1, kb * 64, f.Sk, sV + buf * TILEB, wave, 2, lane);
    };

    int e = next(beg);
    if (e < end) stage(e, 0);
    vm_wait();
    __syncthreads();
    int buf = 0;
    while (e < end) {
        const uint32_t ent = win.get(fetch_e, e, lane);  // before next() moves the window on
        const int kb = (int)(ent & 0x0FFFFFFFu);
        const bool diag = m.causal && (int)(ent >> 28) == kTilePartial;
        const int en = next(e + 1);
        if (en < end) stage(en, buf ^ 1);
        const char* k_ = sK + buf * TILEB;
        const char* v_ = sV + buf * TILEB;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            s[h2] = f32x16{};
            dp[h2] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 ak = *(const bf16x8*)(k_ + h2 * 32 * ROWB + krow_off[kc]);
                const bf16x8 av = *(const bf16x8*)(v_ + h2 * 32 * ROWB + krow_off[kc]);
                s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[kc], s[h2], 0, 0, 0);
                dp[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[kc], dp[h2], 0, 0, 0);
            }
        }
        // register r of key half h2 is key kb*64 + h2*32 + (r>>2)*8 + 4*hh + (r&3)
        bf16x8 sb[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int key = kb * 64 + h2 * 32 + (rr >> 2) * 8 + 4 * hh + (rr & 3);
                float pv = fast_exp2(fmaf(s[h2][rr], c2, -l2));
                if (diag && key > qi) pv = 0.f;
                sb[h2 * 2 + (rr >> 3)][rr & 7] = (bf16)(pv * (dp[h2][rr] - dl));
            }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int kc2 = 0; kc2 < 4; ++kc2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int o0 = kc2 * 16 * ROWB;
                const bf16x4 lo = tr_read(k_ + o0 + trk[0][db]);
                const bf16x4 hi = tr_read(k_ + o0 + trk[1][db]);
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[kc2], dq[db], 0, 0, 0);
            }
        }
        vm_wait();
        __syncthreads();
        buf ^= 1;
        e = en;
    }

    if (!q_ok) return;
    bf16* dqp = (bf16*)p.dq + (int64_t)b * p.dqs0 + (int64_t)qi * p.dqs1 + (int64_t)hq * p.dqs2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) w[e4] = (bf16)(dq[db][g * 4 + e4] * f.scale);
            *(bf16x4*)(dqp + db * 32 + g * 8 + 4 * hh) = w;
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

template <int D>
static hipError_t dkdv_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    const size_t lds = 4 * 64 * 2 * D + 4 * 64 * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void*)&bwd_dkdv_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int grid = p.f.B * p.f.Hkv * ((p.f.Sk + 63) / 64);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(grid), dim3(128), lds, s, p, m);
    return hipGetLastError();
}

template <int D>
static hipError_t dq_launch(const BwdDev& p, const MaskDev& m, hipStream_t s) {
    const size_t lds = 4 * 64 * 2 * D;
    const int grid = p.f.B * p.f.Hq * m.nQb;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(grid), dim3(128), lds, s, p, m);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdDev& p, const MaskDev& m, int D, hipStream_t s) {
    return D == 128 ? dkdv_launch<128>(p, m, s) : dkdv_launch<64>(p, m, s);
}

hipError_t launch_bwd_dq(const BwdDev& p, const MaskDev& m, int D, hipStream_t s) {
    return D == 128 ? dq_launch<128>(p, m, s) : dq_launch<64>(p, m, s);
}

}  // namespace mfa
