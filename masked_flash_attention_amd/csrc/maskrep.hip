// Mask-representation kernels for gfx950: block ids, block-id tile
// summaries, dense-mask compaction, BSR kinds and CSC, varlen schedule.
// All outputs are deterministic (no order-dependent atomics): prefix counts
// come from wave ballots (v_mbcnt) and LDS block scans.

#include <algorithm>

#include <type_traits>

#include "sched.hpp"

namespace mfa {

// ---------------------------------------------------------------------------
// Block-wide helpers (blockDim.x multiple of 64, <= 1024)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_prefix(uint64_t ballot) {
    // number of set bits in lanes below this one
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0));
}

// Exclusive prefix count of `flag` over the block; returns the block total in *total.
__device__ __forceinline__ int block_exclusive_count(bool flag, int* total, int* lds16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint64_t b = __builtin_amdgcn_ballot_w64(flag);
    const int in_wave = lane_prefix(b);
    if (lane == 0) lds16[wave] = __builtin_popcountll(b);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int cnt = lds16[w];
        before += (w < wave) ? cnt : 0;
        tot += cnt;
    }
    __syncthreads();
    *total = tot;
    return before + in_wave;
}

// Exclusive prefix sum of small non-negative ints over the block: a
// shuffle scan inside each wavefront, then one over the wave totals, with
// three barriers (the block size is a multiple of 64, at most 1024; lds
// needs 128 ints). Every thread gets the block total.
__device__ __forceinline__ int block_exclusive_sum(int v, int* total, int* lds) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds[w] = x;
    __syncthreads();
    if (w == 0) {
        int c = lane < nw ? lds[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(c, off, 64);
            if (lane >= off) c += y;
        }
        if (lane < nw) lds[64 + lane] = c;  // inclusive sums of the wave totals
    }
    __syncthreads();
    const int before = w > 0 ? lds[64 + w - 1] : 0;
    *total = lds[64 + nw - 1];
    __syncthreads();  // lds may be reused by the next call
    return before + x - v;
}

// ---------------------------------------------------------------------------
// Block ids ("opentau.policies.flash_attn_cuda", make_att_block_ids)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void block_ids_kernel(const uint8_t* pad, const int32_t* att, int N, int nc,
                                                        const uint8_t* cross_pad, int32_t* q_blk, int32_t* k_blk,
                                                        uint8_t* q_valid, uint8_t* k_valid) {
    __shared__ int lds[16];
    const int b = blockIdx.x;
    const int Sk = nc + N;
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        k_blk[(int64_t)b * Sk + c] = MFA_BLK_CROSS;
        k_valid[(int64_t)b * Sk + c] = cross_pad[(int64_t)b * nc + c] != 0;
    }
    int carry = 0;
    for (int base = 0; base < N; base += blockDim.x) {
        const int i = base + threadIdx.x;
        const bool in = i < N;
        const bool open = in && att[(int64_t)b * N + i] != 0;
        int total;
        const int before = block_exclusive_count(open, &total, lds);
        if (in) {
            const int id = carry + before + (open ? 1 : 0);  // inclusive running count
            const uint8_t v = pad[(int64_t)b * N + i] != 0;
            q_blk[(int64_t)b * N + i] = id;
            q_valid[(int64_t)b * N + i] = v;
            k_blk[(int64_t)b * Sk + nc + i] = id;
            k_valid[(int64_t)b * Sk + nc + i] = v;
        }
        carry += total;
    }
}

// ---------------------------------------------------------------------------
// Block-id tile summaries: one wave per tile
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(64) void blockid_summary_kernel(const int32_t* q_blk, const int32_t* k_blk,
                                                             const uint8_t* q_valid, const uint8_t* k_valid,
                                                             int Sq, int Sk, int BM, int BN, int nQt, int nKt,
                                                             int32_t* qsum, int32_t* ksum, uint32_t* kv_bits) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x;
    const bool isq = tile < nQt;
    const int T = isq ? BM : BN;
    const int S = isq ? Sq : Sk;
    const int t0 = (isq ? tile : tile - nQt) * T;
    const int32_t* ids = isq ? q_blk + (int64_t)b * Sq : k_blk + (int64_t)b * Sk;
    const uint8_t* val = isq ? q_valid + (int64_t)b * Sq : k_valid + (int64_t)b * Sk;
    int mn = INT32_MAX, mx = INT32_MIN;
    bool any = false, all = true;
    for (int j = threadIdx.x; j < T; j += 64) {
        const int pos = t0 + j;
        const bool in = pos < S;
        const bool v = in && val[pos] != 0;
        if (v) {
            const int id = ids[pos];
            mn = min(mn, id);
            mx = max(mx, id);
        }
        any = any || v;
        all = all && v;
    }
    for (int off = 32; off >= 1; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off));
        mx = max(mx, __shfl_xor(mx, off));
    }
    const bool any_w = __builtin_amdgcn_ballot_w64(any) != 0;
    const bool all_w = __builtin_amdgcn_ballot_w64(!all) == 0;
    if (threadIdx.x == 0) {
        int32_t* out = isq ? qsum + ((int64_t)b * nQt + tile) * 4 : ksum + ((int64_t)b * nKt + tile - nQt) * 4;
        out[0] = mn;
        out[1] = mx;
        out[2] = any_w;
        out[3] = all_w;
    }
    if (!isq) {
        // key validity bits of this BN = 64 key tile: words 2*kt, 2*kt+1
        const int pos = t0 + threadIdx.x;
        const bool v = pos < Sk && val[pos] != 0;
        const uint64_t bits = __builtin_amdgcn_ballot_w64(v);
        const int W = (Sk + 31) / 32;
        const int w0 = t0 / 32;
        if (threadIdx.x == 0 && w0 < W) kv_bits[(int64_t)b * W + w0] = (uint32_t)bits;
        if (threadIdx.x == 0 && w0 + 1 < W) kv_bits[(int64_t)b * W + w0 + 1] = (uint32_t)(bits >> 32);
    }
}

// ---------------------------------------------------------------------------
// Dense (Nq, Nk) bool mask -> tile kinds + packed fine bits
// (BinFlash, "Efficiently Dispatching ..."). HBM-bound: each thread reads
// 16 mask bytes of a row per step (dwordx4), packs them into 16 bits and
// folds them into its key tile's any/all flags.
// Workgroup = 256 threads = 128 rows x 256 columns (4 key tiles of 64).
// ---------------------------------------------------------------------------

constexpr int kCmpRows = 128;   // rows per workgroup strip (one 128-row tile or two 64-row ones)
constexpr int kCmpCols = 256;   // 4 key tiles of 64 per workgroup
constexpr int kCmpPasses = kCmpRows / 16;

__device__ __forceinline__ uint32_t pack4(uint32_t w) {
    // 4 mask bytes -> 4 bits (bit k = byte k != 0). nz keeps bit 7 of each
    // byte; the high half of nz * (2^25 + 2^18 + 2^11 + 2^4) moves bits 7, 15,
    // 23, 31 to 32..35, and none of the other partial products reaches or
    // carries into those four bits.
    const uint32_t nz = (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
    return __umulhi(nz, 0x02040810u) & 0xFu;
}

// Body shared by the dense-mask and the predicate tile builders: one
// workgroup = 128 rows x 256 columns (4 key tiles); thread t covers a 16-column
// segment (t & 15) of row (t >> 4) + 16*pass. bits16(r, col) returns the
// allowed bits of row r, columns [col, col + 16) (0 past Nk). The tile kinds
// are written for 128-row tiles, or with bm64 for each 64-row half.
template <class Bits16>
__device__ __forceinline__ void tile_strip(const Bits16& bits16, int Nq, int Nk, int nKt, bool bm64,
                                           uint8_t* tile_kind, uint32_t* fine_bits) {
    __shared__ uint32_t s_any[8], s_all[8];  // [half][key tile]
    const int qt = blockIdx.y;
    const int col0 = blockIdx.x * kCmpCols;
    const int t = threadIdx.x, lane = t & 63;
    const int seg = t & 15;            // 16-column segment in the 256-column strip
    const int rsub = t >> 4;           // row within a 16-row pass
    const int col = col0 + seg * 16;
    const int W = (Nk + 31) / 32;
    if (t < 8) {
        s_any[t] = 0;
        s_all[t] = 1;
    }
    uint32_t words[kCmpPasses];
    // every load (or evaluation) of the strip first
#pragma unroll
    for (int ps = 0; ps < kCmpPasses; ++ps) {
        const int r = qt * kCmpRows + ps * 16 + rsub;
        words[ps] = r < Nq ? bits16(r, col) : 0u;
    }
    bool any[2] = {false, false}, all[2] = {true, true};  // per 64-row half
    // columns of this thread that exist
    const int ncol = max(0, min(16, Nk - col));
    const uint32_t full16 = ncol >= 16 ? 0xFFFFu : ((1u << ncol) - 1u);
#pragma unroll
    for (int ps = 0; ps < kCmpPasses; ++ps) {
        const int h = ps / (kCmpPasses / 2);
        const int r = qt * kCmpRows + ps * 16 + rsub;
        const uint32_t bits = words[ps];
        any[h] = any[h] || bits != 0;
        all[h] = all[h] && (r < Nq) && ncol == 16 && bits == full16;
        // pair lanes (even, odd) form one 32-bit word of the row
        const uint32_t hi = __shfl_xor(bits, 1);
        if (r < Nq && (seg & 1) == 0) {
            const int wi = col / 32;
            if (wi < W) fine_bits[(int64_t)r * W + wi] = bits | (hi << 16);
        }
    }
    // key tile of this thread: seg / 4; fold any/all over the wave, then the block
    uint64_t ba[2], bl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ba[h] = __builtin_amdgcn_ballot_w64(any[h]);
        bl[h] = __builtin_amdgcn_ballot_w64(all[h]);
    }
    __syncthreads();
    if (lane < 4) {
        const uint64_t sel = 0x000F000F000F000Full << (4 * lane);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (ba[h] & sel) atomicOr(&s_any[h * 4 + lane], 1u);
            if ((bl[h] & sel) != sel) atomicAnd(&s_all[h * 4 + lane], 0u);
        }
    }
    __syncthreads();
    if (t < 8) {
        const int h = t >> 2, kt = col0 / 64 + (t & 3);
        if (kt < nKt) {
            if (bm64) {
                const int q64 = 2 * qt + h;
                if (q64 * 64 < Nq) {
                    const uint8_t k = s_all[t] ? kTileFull : (s_any[t] ? kTilePartial : kTileEmpty);
                    tile_kind[(int64_t)q64 * nKt + kt] = k;
                }
            } else if (h == 0) {
                const bool a = s_any[t] || s_any[t + 4], f = s_all[t] && s_all[t + 4];
                tile_kind[(int64_t)qt * nKt + kt] = f ? kTileFull : (a ? kTilePartial : kTileEmpty);
            }
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void compact_tiles_kernel(const uint8_t* mask, int Nq, int Nk, int nKt, bool bm64,
                                                            uint8_t* tile_kind, uint32_t* fine_bits) {
    auto bits16 = [&](int r, int col) -> uint32_t {
        const uint8_t* rp = mask + (int64_t)r * Nk;
        uint32_t bits = 0;
        if (VEC && col + 16 <= Nk) {
            const u32x4 v = *(const u32x4*)(rp + col);
            bits = pack4(v[0]) | (pack4(v[1]) << 4) | (pack4(v[2]) << 8) | (pack4(v[3]) << 12);
        } else {
            for (int e = 0; e < 16; ++e)
                if (col + e < Nk && rp[col + e] != 0) bits |= 1u << e;
        }
        return bits;
    };
    tile_strip(bits16, Nq, Nk, nKt, bm64, tile_kind, fine_bits);
}

// Dense masks whose row length is a multiple of 16 bytes: one workgroup of
// 8 waves covers 128 rows x 1024 columns (16 key tiles). Wave w reads rows
// w*16 .. w*16+15, one 1 KB row segment per instruction (lane l: columns
// 16l .. 16l+15), so every load is a fully used 1 KB run and every row's
// fine words leave as one 128-byte store.
constexpr int kWideCols = 1024;
constexpr int kCmpRPW = 16;

template <int RPW>  // rows per wave; the workgroup's kCmpRows / RPW waves cover the strip
__global__ __launch_bounds__(64 * (kCmpRows / RPW)) void compact_tiles_wide_kernel(const uint8_t* mask, int Nq, int Nk,
                                                                                   int nKt, bool bm64,
                                                                                   uint8_t* tile_kind,
                                                                                   uint32_t* fine_bits) {
    constexpr int NWV = kCmpRows / RPW;
    __shared__ uint64_t s_any[NWV], s_all[NWV];
    const int qt = blockIdx.y;
    const int col0 = blockIdx.x * kWideCols;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: row tests stay scalar
    const int col = col0 + 16 * lane;
    const int W = (Nk + 31) / 32;
    const bool col_ok = col + 16 <= Nk;  // Nk is a multiple of 16 here
    const int r0 = qt * kCmpRows + wave * RPW;
    // Every load is issued unconditionally, so that each row's packing can
    // start as soon as that row has landed (a load under a branch would make
    // the compiler wait for all sixteen first): rows past Nq re-read row
    // Nq - 1 and columns past Nk re-read column 0 of the row, and their bits
    // are zeroed after packing.
    const int rc0 = min(r0, Nq - 1);
    const int n_in = min(RPW, Nq - rc0);  // rows of the wave that exist (>= 1)
    const uint8_t* p = mask + (int64_t)rc0 * Nk + (col_ok ? col : 0);
    u32x4 v[RPW];
#pragma unroll
    for (int ps = 0; ps < RPW; ++ps) {
        v[ps] = __builtin_nontemporal_load((const u32x4*)p);
        if (ps + 1 < n_in) p += Nk;
    }
    // the even lane of each pair stores the pair's 32-bit word, one row apart
    const int wi = col0 / 32 + (lane >> 1);
    uint32_t* const fb0 = fine_bits + (int64_t)rc0 * W + wi;
    const bool store_lane = (lane & 1) == 0 && wi < W;
    // OR and AND of the lane's row bits over the wave's rows: the tile
    // flags are ballots of these at the end (bits is 0 where !ok)
    uint32_t or_bits = 0u, and_bits = 0xFFFFu;
    // Folds a row's 16 bits into the flags and stores its fine words.
    auto emit = [&](uint32_t bits, int r, uint32_t*& fb, int ps) {
        or_bits |= bits;
        and_bits &= bits;
        // lane pairs (even, odd) form one 32-bit word of the row; the
        // partner's bits come through a DPP quad permutation [1, 0, 3, 2]
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0xB1, 0xF, 0xF, false);
        if (r < Nq && store_lane) fb[0] = bits | (hi << 16);
        if (ps + 1 < n_in) fb += W;
    };
    // First pass, for bytes of 0 or 1 (a bool mask): the byte-wise dot
    // product with weights 1, 2, 4, 8 (16, 32, 64, 128 for the second dword)
    // is the row's bits. `seen` ORs every byte read, so bits 1..7 of its bytes
    // stay clear unless some byte is above 1.
    uint32_t seen = 0u;
    {
        uint32_t* fb = fb0;
#pragma unroll
        for (int ps = 0; ps < RPW; ++ps) {
            const int r = r0 + ps;
            const bool ok = r < Nq && col_ok;
            const u32x4 x = v[ps];
            // a use the optimiser cannot see through, so that the load stays
            // where it was issued instead of being sunk into a branch
            asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
            seen |= x[0] | x[1] | x[2] | x[3];
            const uint32_t lo =
                __builtin_amdgcn_udot4(x[0], 0x08040201u, __builtin_amdgcn_udot4(x[1], 0x80402010u, 0u, false), false);
            const uint32_t hb =
                __builtin_amdgcn_udot4(x[2], 0x08040201u, __builtin_amdgcn_udot4(x[3], 0x80402010u, 0u, false), false);
            emit(ok ? lo | (hb << 8) : 0u, r, fb, ps);
        }
    }
    // A wave that read any byte above 1 (in its rows, the clamped re-reads
    // included) packs its rows again with a nonzero test per byte and stores
    // again: nz keeps bit 7 of each byte (set iff the byte is nonzero); the
    // high half of nz * (2^25 + 2^18 + 2^11 + 2^4) holds bits 7, 15, 23, 31
    // at 0..3, the multiplier shifted by 4 puts them at 4..7, and no other
    // partial product lands in (or carries into) the kept bits.
    if (__builtin_amdgcn_ballot_w64((seen & 0xFEFEFEFEu) != 0u) != 0) {
        or_bits = 0u;
        and_bits = 0xFFFFu;
        uint32_t* fb = fb0;
#pragma unroll
        for (int ps = 0; ps < RPW; ++ps) {
            const int r = r0 + ps;
            const bool ok = r < Nq && col_ok;
            uint32_t nz[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) nz[d] = (((v[ps][d] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | v[ps][d]) & 0x80808080u;
            const uint32_t lo = (__umulhi(nz[0], 0x02040810u) & 0xFu) | (__umulhi(nz[1], 0x20408100u) & 0xF0u);
            const uint32_t hb = (__umulhi(nz[2], 0x02040810u) & 0xFu) | (__umulhi(nz[3], 0x20408100u) & 0xF0u);
            emit(ok ? lo | (hb << 8) : 0u, r, fb, ps);
        }
    }
    const uint64_t any = __builtin_amdgcn_ballot_w64(or_bits != 0u);
    const uint64_t all = __builtin_amdgcn_ballot_w64(and_bits == 0xFFFFu);
    if (lane == 0) {
        s_any[wave] = any;
        s_all[wave] = all;
    }
    __syncthreads();
    // thread t < 32: half h = t / 16 (the strip's 64-row half h, waves h*NWV/2 ..), key tile j = t % 16
    // (lanes 4j .. 4j+3)
    const int t = threadIdx.x;
    if (t < 32) {
        const int h = t >> 4, j = t & 15, kt = col0 / 64 + j;
        bool a[2] = {false, false}, f[2] = {true, true};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int w = 0; w < NWV / 2; ++w) {
                a[hh] = a[hh] || ((s_any[hh * (NWV / 2) + w] >> (4 * j)) & 0xFull) != 0;
                f[hh] = f[hh] && ((s_all[hh * (NWV / 2) + w] >> (4 * j)) & 0xFull) == 0xFull;
            }
        if (kt < nKt) {
            if (bm64) {
                const int q64 = 2 * qt + h;
                if (q64 * 64 < Nq) tile_kind[(int64_t)q64 * nKt + kt] = f[h] ? kTileFull : (a[h] ? kTilePartial : kTileEmpty);
            } else if (h == 0) {
                const bool aa = a[0] || a[1], ff = f[0] && f[1];
                tile_kind[(int64_t)qt * nKt + kt] = ff ? kTileFull : (aa ? kTilePartial : kTileEmpty);
            }
        }
    }
}

// floor(n / d) and ceil(n / d) for d > 0
__device__ __forceinline__ int64_t floor_div(int64_t n, int64_t d) { return n >= 0 ? n / d : -((-n + d - 1) / d); }
__device__ __forceinline__ int64_t ceil_div(int64_t n, int64_t d) { return -floor_div(-n, d); }

// Bits e in [0, 16) with e >= d, and with e <= d.
__device__ __forceinline__ uint32_t ge16(int64_t d) { return d <= 0 ? 0xFFFFu : (d >= 16 ? 0u : (0xFFFFu & ~((1u << d) - 1u))); }
__device__ __forceinline__ uint32_t le16(int64_t d) { return d < 0 ? 0u : (d >= 15 ? 0xFFFFu : ((2u << d) - 1u)); }

// Allowed bits of row i, columns [j0, j0 + 16): OR over the conjunctions of
// the AND of their linear atoms a*i + b*j + c >= 0. Along a row each atom is
// monotone in j, so it contributes a prefix or suffix of the 16 columns.
__device__ __forceinline__ uint32_t predicate_bits16(const mfa_predicate& P, int64_t i, int64_t j0) {
    uint32_t out = 0;
    for (int tm = 0; tm < P.n_terms; ++tm) {
        uint32_t m = 0xFFFFu;
        for (int at = 0; at < P.n_atoms[tm]; ++at) {
            const mfa_pred_atom A = P.atoms[tm][at];
            const int64_t base = A.a * i + A.c;  // value at kv_idx = 0
            // unit coefficients (causal, windows, prefixes) need no division;
            // the coefficients are the same for every lane, so these branches are uniform
            if (A.b == 0) m &= base >= 0 ? 0xFFFFu : 0u;
            else if (A.b == 1) m &= ge16(-base - j0);                  // j >= -base
            else if (A.b == -1) m &= le16(base - j0);                  // j <= base
            else if (A.b > 0) m &= ge16(ceil_div(-base, A.b) - j0);   // j >= ceil(-base / b)
            else m &= le16(floor_div(base, -A.b) - j0);                // j <= floor(base / -b)
        }
        out |= m;
    }
    return out;
}

__global__ __launch_bounds__(256) void predicate_tiles_kernel(mfa_predicate P, int Nq, int Nk, int nKt, bool bm64,
                                                              uint8_t* tile_kind, uint32_t* fine_bits) {
    auto bits16 = [&](int r, int col) -> uint32_t {
        const int ncol = max(0, min(16, Nk - col));
        const uint32_t exist = ncol >= 16 ? 0xFFFFu : ((1u << ncol) - 1u);
        return predicate_bits16(P, r, col) & exist;
    };
    tile_strip(bits16, Nq, Nk, nKt, bm64, tile_kind, fine_bits);
}

// CSR of non-empty tiles: one workgroup per query-tile row. The row offset is
// the count of non-empty tiles in all earlier rows, recounted here from the
// tile map (16 kinds per load), so no workspace and no inter-workgroup
// ordering is needed.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
    return __builtin_popcount((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u);
}

__device__ __forceinline__ int block_sum(int v, int* lds16) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 0) lds16[wave] = v;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += lds16[w];
    __syncthreads();
    return tot;
}

__global__ __launch_bounds__(256) void compact_csr_kernel(const uint8_t* tile_kind, int nQt, int nKt,
                                                          int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind) {
    __shared__ int lds[16];
    const int qt = blockIdx.x;
    const int64_t nbytes = (int64_t)qt * nKt;
    int cnt = 0;
    const bool vec = (((uintptr_t)tile_kind) & 15) == 0;
    int64_t done = 0;
    if (vec) {
        const int64_t nvec = nbytes >> 4;
        const u32x4* p4 = (const u32x4*)tile_kind;
        for (int64_t i = threadIdx.x; i < nvec; i += blockDim.x) {
            const u32x4 w = p4[i];
            cnt += nonzero_bytes(w[0]) + nonzero_bytes(w[1]) + nonzero_bytes(w[2]) + nonzero_bytes(w[3]);
        }
        done = nvec << 4;
    }
    for (int64_t i = done + threadIdx.x; i < nbytes; i += blockDim.x) cnt += tile_kind[i] != 0;
    const int base = block_sum(cnt, lds);
    if (threadIdx.x == 0) row_ptr[qt] = base;
    int carry = 0;
    const uint8_t* rowk = tile_kind + nbytes;
    for (int k0 = 0; k0 < nKt; k0 += blockDim.x) {
        const int kt = k0 + threadIdx.x;
        const uint8_t k = kt < nKt ? rowk[kt] : 0;
        int n;
        const int pos = block_exclusive_count(k != 0, &n, lds);
        if (k != 0) {
            col_idx[base + carry + pos] = kt;
            col_kind[base + carry + pos] = k;
        }
        carry += n;
    }
    if (qt == nQt - 1 && threadIdx.x == 0) row_ptr[nQt] = base + carry;
}

// The same CSR in linear work for large maps: each tile row's count of
// non-empty tiles goes to row_ptr[qt + 1], one workgroup scans row_ptr in
// place, then each row writes its entries at row_ptr[qt]. (The single kernel
// above recounts every earlier row: quadratic in the number of tile rows.)
__global__ __launch_bounds__(256) void csr_count_kernel(const uint8_t* tile_kind, int nKt, int32_t* row_ptr) {
    __shared__ int lds[16];
    const int qt = blockIdx.x;
    const uint8_t* rowk = tile_kind + (int64_t)qt * nKt;
    int cnt = 0;
    for (int kt = threadIdx.x; kt < nKt; kt += blockDim.x) cnt += rowk[kt] != 0;
    const int tot = block_sum(cnt, lds);
    if (threadIdx.x == 0) {
        row_ptr[qt + 1] = tot;
        if (qt == 0) row_ptr[0] = 0;
    }
}

__global__ __launch_bounds__(1024) void csr_scan_kernel(int nQt, int32_t* row_ptr) {
    __shared__ int scan[128];
    int carry = 0;
    for (int i0 = 1; i0 <= nQt; i0 += blockDim.x) {
        const int i = i0 + threadIdx.x;
        const int v = i <= nQt ? row_ptr[i] : 0;
        int tot;
        const int ex = block_exclusive_sum(v, &tot, scan);
        if (i <= nQt) row_ptr[i] = carry + ex + v;
        carry += tot;
    }
}

__global__ __launch_bounds__(256) void csr_fill_kernel(const uint8_t* tile_kind, int nKt, const int32_t* row_ptr,
                                                       int32_t* col_idx, uint8_t* col_kind) {
    __shared__ int lds[16];
    const int qt = blockIdx.x;
    const int base = row_ptr[qt];
    const uint8_t* rowk = tile_kind + (int64_t)qt * nKt;
    int carry = 0;
    for (int k0 = 0; k0 < nKt; k0 += blockDim.x) {
        const int kt = k0 + threadIdx.x;
        const uint8_t k = kt < nKt ? rowk[kt] : 0;
        int n;
        const int pos = block_exclusive_count(k != 0, &n, lds);
        if (k != 0) {
            col_idx[base + carry + pos] = kt;
            col_kind[base + carry + pos] = k;
        }
        carry += n;
    }
}

// CSR of a tile map: the single quadratic-recount kernel for small maps
// (one launch), the linear three-kernel form for large ones.
static hipError_t launch_csr(const uint8_t* tile_kind, int nQt, int nKt, int32_t* row_ptr, int32_t* col_idx,
                             uint8_t* col_kind, hipStream_t s) {
    if ((int64_t)nQt * nQt * nKt <= (int64_t)(1 << 22)) {
        hipLaunchKernelGGL(compact_csr_kernel, dim3(nQt), dim3(256), 0, s, tile_kind, nQt, nKt, row_ptr, col_idx,
                           col_kind);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(csr_count_kernel, dim3(nQt), dim3(256), 0, s, tile_kind, nKt, row_ptr);
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, nQt, row_ptr);
    hipLaunchKernelGGL(csr_fill_kernel, dim3(nQt), dim3(256), 0, s, tile_kind, nKt, row_ptr, col_idx, col_kind);
    return hipGetLastError();
}

// 128-row tile map from a 64-row one: a 128-row tile is empty iff both halves
// are, full iff both halves exist and are full, else partial (a half past Nq
// makes the tile ragged, so never full).
__global__ __launch_bounds__(256) void coarsen_tiles_kernel(const uint8_t* kind64, int nQt64, int nKt, int nQt128,
                                                            uint8_t* kind128) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nQt128 * nKt) return;
    const int r = (int)(i / nKt), c = (int)(i - (int64_t)r * nKt);
    const int a = kind64[(int64_t)(2 * r) * nKt + c];
    const int b = 2 * r + 1 < nQt64 ? kind64[(int64_t)(2 * r + 1) * nKt + c] : -1;
    int k;
    if (b < 0) k = a == kTileEmpty ? kTileEmpty : kTilePartial;
    else if (a == kTileEmpty && b == kTileEmpty) k = kTileEmpty;
    else if (a == kTileFull && b == kTileFull) k = kTileFull;
    else k = kTilePartial;
    kind128[i] = (uint8_t)k;
}

// Counts of empty, partial and full tiles of a tile map.
__global__ __launch_bounds__(256) void tile_counts_kernel(const uint8_t* kind, int64_t n, int64_t* counts) {
    __shared__ int lds[16];
    int c1 = 0, c2 = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int k = kind[i];
        c1 += k == kTilePartial;
        c2 += k == kTileFull;
    }
    c1 = block_sum(c1, lds);
    c2 = block_sum(c2, lds);
    if (threadIdx.x == 0) {
        atomicAdd((unsigned long long*)&counts[1], (unsigned long long)c1);
        atomicAdd((unsigned long long*)&counts[2], (unsigned long long)c2);
    }
}

__global__ void tile_counts_finish_kernel(int64_t n, int64_t* counts) {
    if (threadIdx.x == 0) counts[0] = n - counts[1] - counts[2];
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// Zero n int32 words with a kernel rather than hipMemsetAsync, so that the
// call stays a kernel node when a caller captures it in a graph.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

static hipError_t zero_i32(int32_t* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// BSR (flashinfer block_sparse_attention): entry kinds and CSC. One workgroup
// per (b, h); rows are visited in ascending order, the entries of one row in
// parallel (a canonical row has distinct columns), so the CSC lists come out
// ascending without atomics on the output.
// ---------------------------------------------------------------------------

// Validity of keys [j0, j1] in one batch entry's LSB-first bitmap: bit 0 =
// some key valid, bit 1 = every key valid.
__device__ __forceinline__ int key_range_validity(const uint32_t* words, int j0, int j1) {
    bool any = false, all = true;
    for (int w = j0 >> 5; w <= (j1 >> 5); ++w) {
        const int lo = max(j0 - w * 32, 0), hi = min(j1 - w * 32, 31);
        const uint32_t span = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
        const uint32_t v = words[w] & span;
        any = any || v != 0u;
        all = all && v == span;
    }
    return (any ? 1 : 0) | (all ? 2 : 0);
}

// Row of flat entry e: the last r with ip[r] <= e (ip non-decreasing,
// ip[0] <= e < ip[nQb]).
__device__ __forceinline__ int bsr_row_of(const int* ip, int nQb, int e) {
    int lo = 0, hi = nQb;  // ip[lo] <= e < ip[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ip[mid] <= e) lo = mid;
        else hi = mid;
    }
    return lo;
}

constexpr int kBsrColBits = 14;  // column ids below 16384 (the host enforces nKb <= 16384)

// One 1024-thread workgroup per (batch, kv head). Entries are processed in
// row-major chunks of 1024: first every entry's kind and its column's count
// (LDS atomics, order-free), then a scan of the counts into csc_ptr, then a
// stable scatter: lanes of a wave with the same column are matched with
// ballots over the column's bits and the 16 waves take their positions one
// after the other, so each column lists its rows in ascending order.
__global__ __launch_bounds__(1024) void bsr_prepare_kernel(const int32_t* indptr, const int32_t* indices, int nQb,
                                                           int nKb, int64_t nnz, int qb, int kb, int Sq, int Skv,
                                                           int causal, const uint32_t* kv_valid, int Hkv,
                                                           uint8_t* col_kind, int32_t* csc_ptr, int32_t* csc_idx) {
    extern __shared__ int cnt[];  // nKb ints, then 1024 scan scratch
    int* scan = cnt + nKb;
    const int bh = blockIdx.x;
    const int t = threadIdx.x, n = blockDim.x, lane = t & 63, wv = t >> 6, nwv = n >> 6;
    const int* ip = indptr + (int64_t)bh * (nQb + 1);
    int32_t* cp = csc_ptr + (int64_t)bh * (nKb + 1);
    for (int c = t; c < nKb; c += n) cnt[c] = 0;
    __syncthreads();
    // Rows are expected canonical (mfa_bsr_validate); ids out of range are
    // skipped and every write is bounded, so malformed input cannot write
    // out of bounds.
    const int e_begin = max(ip[0], 0), e_end = (int)min((int64_t)ip[nQb], nnz);
    const uint32_t* kvw = kv_valid ? kv_valid + (int64_t)(bh / Hkv) * ((Skv + 31) >> 5) : nullptr;
    for (int e0 = e_begin; e0 < e_end; e0 += n) {
        const int e = e0 + t;
        if (e >= e_end) continue;
        const int c = indices[e];
        if (c < 0 || c >= nKb) continue;
        const int r = bsr_row_of(ip, nQb, e);
        int kind = bsr_kind_of(r, c, qb, kb, Sq, Skv, causal);
        if (kvw && kind != kTileEmpty) {
            // token validity (kv_valid_bits): no valid key -> empty, an invalid key -> not full
            const int v = key_range_validity(kvw, c * kb, min((c + 1) * kb, Skv) - 1);
            if (!(v & 1)) kind = kTileEmpty;
            else if (kind == kTileFull && !(v & 2)) kind = kTilePartial;
        }
        col_kind[e] = (uint8_t)kind;
        atomicAdd(&cnt[c], 1);
    }
    __syncthreads();
    // exclusive scan of column counts, in chunks of blockDim
    int carry = ip[0];
    for (int c0 = 0; c0 < nKb; c0 += n) {
        const int c = c0 + t;
        const int v = c < nKb ? cnt[c] : 0;
        int tot;
        const int ex = block_exclusive_sum(v, &tot, scan);
        if (c < nKb) {
            cp[c] = carry + ex;
            cnt[c] = carry + ex;  // becomes the write cursor
        }
        carry += tot;
        __syncthreads();
    }
    if (t == 0) cp[nKb] = carry;
    __syncthreads();
    for (int e0 = e_begin; e0 < e_end; e0 += n) {
        const int e = e0 + t;
        int c = -1, r = 0;
        if (e < e_end) {
            c = indices[e];
            if (c < 0 || c >= nKb) c = -1;
            else r = bsr_row_of(ip, nQb, e);
        }
        const bool valid = c >= 0;
        uint64_t same = __builtin_amdgcn_ballot_w64(valid);
        if (!valid) same = 0;
#pragma unroll
        for (int bit = 0; bit < kBsrColBits; ++bit) {
            const bool on = valid && ((c >> bit) & 1);
            const uint64_t bo = __builtin_amdgcn_ballot_w64(on);
            same &= on ? bo : ~bo;
        }
        const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
        const int rank = __builtin_popcountll(same & below);
        for (int w = 0; w < nwv; ++w) {
            if (wv == w && valid) {
                const int pos = cnt[c] + rank;
                if (pos >= 0 && pos < nnz) csc_idx[pos] = r;
                __builtin_amdgcn_wave_barrier();
                if (rank == 0) cnt[c] += __builtin_popcountll(same);
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Bitmask sparse format -> BSR rows (flashinfer block_sparse_attention,
// Parameters: exact_block_bits). One workgroup scans the per-row counts into
// the running offsets; then one thread per row writes its ascending ids.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t row_word(const uint32_t* bits, int64_t row, int W, int w, int nKb) {
    const uint32_t x = bits[row * W + w];
    const int valid = nKb - w * 32;
    return valid >= 32 ? x : (x & ((1u << valid) - 1u));
}

__global__ __launch_bounds__(1024) void bitmask_count_kernel(const uint32_t* bits, int n_bh, int nQb, int nKb,
                                                             int32_t* indptr) {
    __shared__ int scan[1024];
    const int W = (nKb + 31) >> 5;
    const int64_t rows = (int64_t)n_bh * nQb;
    int carry = 0;
    for (int64_t g0 = 0; g0 < rows; g0 += blockDim.x) {
        const int64_t g = g0 + threadIdx.x;
        int cnt = 0;
        if (g < rows)
            for (int w = 0; w < W; ++w) cnt += __builtin_popcount(row_word(bits, g, W, w, nKb));
        int tot;
        const int ex = block_exclusive_sum(cnt, &tot, scan);
        if (g < rows) {
            const int64_t bh = g / nQb, r = g - bh * nQb;
            indptr[bh * (nQb + 1) + r] = carry + ex;
            if (r == nQb - 1) indptr[bh * (nQb + 1) + nQb] = carry + ex + cnt;
        }
        carry += tot;
    }
}

__global__ __launch_bounds__(256) void bitmask_fill_kernel(const uint32_t* bits, int n_bh, int nQb, int nKb,
                                                           const int32_t* indptr, int32_t* indices, int64_t cap) {
    const int W = (nKb + 31) >> 5;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= (int64_t)n_bh * nQb) return;
    const int64_t bh = g / nQb, r = g - bh * nQb;
    int64_t pos = indptr[bh * (nQb + 1) + r];
    for (int w = 0; w < W; ++w) {
        uint32_t x = row_word(bits, g, W, w, nKb);
        while (x) {
            const int c = __builtin_ctz(x);
            x &= x - 1u;
            if (pos < cap) indices[pos] = w * 32 + c;
            ++pos;
        }
    }
}

// ---------------------------------------------------------------------------
// Varlen packing and schedule ("tensorplay.nn.attention.varlen", Packed
// layout). One workgroup of 1024 threads. The work list holds every BM-row
// query tile (seq, q0), ordered by descending number of visited key tiles,
// ties by ascending (seq, q0): a stable counting sort with exact costs.
//  * Costs below kLoCost are counted per value in LDS. Longer tiles (over
//    262,080 keys with the window open) are counted by their high digit
//    (cost >> 12); they all precede the short ones, each high bucket is
//    placed stably and then ranked exactly by cost inside the bucket.
//  * Tiles are enumerated in (seq, q0) order 1024 at a time across
//    sequence boundaries (a binary search over the tile offsets of a group
//    of up to 1024 sequences held in LDS).
//  * Stable placement: lanes of a wave with the same bucket are found with
//    ballots over the bucket's bits, and the 16 waves take their positions
//    one after the other, so equal costs keep the enumeration order.
// ---------------------------------------------------------------------------

constexpr int kLoCost = 4096;      // costs [0, kLoCost) counted exactly
constexpr int kHiDigits = 8192;    // high digits 1..8192 of longer costs (a cost is at most 2^25)
constexpr int kBucketBits = 14;    // bucket ids: cost for short tiles, kLoCost + digit - 1 for long ones
constexpr int kMaxLongBucket = 16 * 1024;  // tiles per high digit that the exact ranking holds in registers

__device__ __forceinline__ int64_t varlen_cost(int64_t Lq, int64_t Lk, int64_t q0, int BM, int BN, int causal,
                                               int left, int right) {
    const int64_t q1 = min(q0 + BM, Lq) - 1;
    const int64_t lo = left >= 0 ? max((int64_t)0, q0 - left) : 0;
    int64_t hi = Lk - 1;
    if (right >= 0) hi = min(hi, q1 + right);
    if (causal) hi = min(hi, q1);
    if (hi < lo) return 0;
    return hi / BN - lo / BN + 1;
}

// Sequence of tile `i` of a group: the last s with tp[s] <= i (tp ascending,
// tp[0] = 0, n + 1 entries).
__device__ __forceinline__ int tile_seq(const int* tp, int n, int i) {
    int lo = 0, hi = n;  // tp[lo] <= i < tp[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tp[mid] <= i) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(1024) void varlen_schedule_kernel(const int32_t* len_q, const int32_t* len_k, int nseq,
                                                               int BM, int BN, int causal, int left, int right,
                                                               int32_t* cu_q, int32_t* cu_k, int32_t* max_len,
                                                               int32_t* work, int work_cap, int32_t* n_work) {
    __shared__ int scan[1024];
    __shared__ int hist_lo[kLoCost];     // counts, then write cursors
    __shared__ int hist_hi[kHiDigits];   // counts, then write cursors
    __shared__ int tp[1025];             // tile offsets of the current sequence group
    __shared__ int s_max[2];
    __shared__ int s_bad;
    const int t = threadIdx.x, n = blockDim.x;
    const int lane = t & 63, wv = t >> 6, nwv = n >> 6;
    for (int i = t; i < kLoCost; i += n) hist_lo[i] = 0;
    for (int i = t; i < kHiDigits; i += n) hist_hi[i] = 0;
    if (t == 0) {
        s_max[0] = 0;
        s_max[1] = 0;
        s_bad = 0;
        cu_q[0] = 0;
        cu_k[0] = 0;
    }
    __syncthreads();

    // Walks the tiles of every sequence group in (seq, q0) order, 1024 per
    // call of f(valid, seq, q0, cost); every thread calls it the same number
    // of times (f may hold barriers). With `cum`, also writes the cumulative
    // lengths and maxima (first walk only). Returns the tile count.
    auto walk = [&](bool cum, auto&& f) -> int {
        int cq = 0, ck = 0, all = 0;
        for (int g0 = 0; g0 < nseq; g0 += n) {
            const int s = g0 + t;
            const int gn = min(n, nseq - g0);
            const int lq = s < nseq ? len_q[s] : 0;
            const int lk = s < nseq ? len_k[s] : 0;
            int tot, tq, tk;
            const int ex = block_exclusive_sum(s < nseq ? (lq + BM - 1) / BM : 0, &tot, scan);
            if (cum) {
                const int eq = block_exclusive_sum(lq, &tq, scan);
                const int ek = block_exclusive_sum(lk, &tk, scan);
                if (s < nseq) {
                    cu_q[s + 1] = cq + eq + lq;
                    cu_k[s + 1] = ck + ek + lk;
                    atomicMax(&s_max[0], lq);
                    atomicMax(&s_max[1], lk);
                }
                cq += tq;
                ck += tk;
            }
            if (t < gn) tp[t] = ex;
            if (t == 0) tp[gn] = tot;
            __syncthreads();
            for (int c0 = 0; c0 < tot; c0 += n) {
                const int i = c0 + t;
                const bool valid = i < tot;
                int sg = 0, q0 = 0;
                int64_t cost = -1;
                if (valid) {
                    const int sl = tile_seq(tp, gn, i);
                    sg = g0 + sl;
                    q0 = (i - tp[sl]) * BM;
                    cost = varlen_cost(len_q[sg], len_k[sg], q0, BM, BN, causal, left, right);
                }
                f(valid, sg, q0, cost);
            }
            all += tot;
            __syncthreads();  // tp is rewritten for the next group
        }
        return all;
    };

    // Pass 1: cumulative lengths, maxima and the cost histograms.
    const int ctile = walk(true, [&](bool valid, int, int, int64_t cost) {
        if (!valid) return;
        if (cost < kLoCost) atomicAdd(&hist_lo[cost], 1);
        else atomicAdd(&hist_hi[(int)(cost >> 12) - 1], 1);
    });
    __syncthreads();
    if (t == 0) {
        max_len[0] = s_max[0];
        max_len[1] = s_max[1];
    }
    for (int i = t; i < work_cap; i += n) {
        work[2 * i] = -1;
        work[2 * i + 1] = -1;
    }
    for (int i = t; i < kHiDigits; i += n)
        if (hist_hi[i] > kMaxLongBucket) s_bad = 1;
    __syncthreads();
    if (ctile > work_cap || s_bad) {
        if (t == 0) n_work[0] = ctile > work_cap ? -1 : -2;
        return;
    }
    if (t == 0) n_work[0] = ctile;

    // Write cursors. Long tiles first, by descending high digit; then the
    // short ones by descending cost.
    int n_long;
    {
        int h[8], sum = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = hist_hi[kHiDigits - 1 - (8 * t + e)];
            sum += h[e];
        }
        int run = block_exclusive_sum(sum, &n_long, scan);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hist_hi[kHiDigits - 1 - (8 * t + e)] = run;
            run += h[e];
        }
    }
    {
        int h[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = hist_lo[kLoCost - 1 - (4 * t + e)];
            sum += h[e];
        }
        int tot;
        int run = n_long + block_exclusive_sum(sum, &tot, scan);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hist_lo[kLoCost - 1 - (4 * t + e)] = run;
            run += h[e];
        }
    }
    __syncthreads();

    // Pass 2: stable placement. Lanes of one wave with the same bucket are
    // found with ballots over the bucket id's bits; waves then take their
    // positions in order.
    walk(false, [&](bool valid, int sg, int q0, int64_t cost) {
        const int bucket = !valid ? -1 : (cost < kLoCost ? (int)cost : kLoCost + (int)(cost >> 12) - 1);
        uint64_t same = __builtin_amdgcn_ballot_w64(valid);
        if (!valid) same = 0;
#pragma unroll
        for (int bit = 0; bit < kBucketBits; ++bit) {
            const bool on = valid && ((bucket >> bit) & 1);
            const uint64_t bo = __builtin_amdgcn_ballot_w64(on);
            same &= on ? bo : ~bo;
        }
        const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
        const int rank = __builtin_popcountll(same & below);
        const bool leader = valid && rank == 0;
        int* cursor = !valid ? nullptr : (bucket < kLoCost ? &hist_lo[bucket] : &hist_hi[bucket - kLoCost]);
        for (int w = 0; w < nwv; ++w) {
            if (wv == w && valid) {
                const int pos = *cursor + rank;
                work[2 * pos] = sg;
                work[2 * pos + 1] = q0;
                __builtin_amdgcn_wave_barrier();
                if (leader) *cursor = pos + __builtin_popcountll(same);
            }
            __syncthreads();
        }
    });

    // Pass 3: inside each high-digit bucket (placed in (seq, q0) order), rank
    // every tile by (cost descending, position ascending) and move it there.
    if (n_long == 0) return;
    __syncthreads();
    for (int dg = kHiDigits - 1; dg >= 0; --dg) {
        // cursor after pass 2 = bucket end; the next higher digit's end is its start
        const int end = hist_hi[dg];
        const int start = dg + 1 < kHiDigits ? hist_hi[dg + 1] : 0;
        const int k = end - start;
        if (k < 2) continue;  // uniform: LDS values read by every thread
        constexpr int J = kMaxLongBucket / 1024;
        int it_s[J], it_q[J], it_r[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int u = t + j * n;
            it_r[j] = -1;
            if (u < k) {
                it_s[j] = work[2 * (start + u)];
                it_q[j] = work[2 * (start + u) + 1];
            }
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int u = t + j * n;
            if (u >= k) continue;
            const int64_t cu = varlen_cost(len_q[it_s[j]], len_k[it_s[j]], it_q[j], BM, BN, causal, left, right);
            int r = 0;
            for (int x = 0; x < k; ++x) {
                const int sx = work[2 * (start + x)], qx = work[2 * (start + x) + 1];
                const int64_t cx = varlen_cost(len_q[sx], len_k[sx], qx, BM, BN, causal, left, right);
                r += (cx > cu || (cx == cu && x < u)) ? 1 : 0;
            }
            it_r[j] = r;
        }
        __syncthreads();  // every read of the bucket precedes the moves
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (it_r[j] < 0) continue;
            work[2 * (start + it_r[j])] = it_s[j];
            work[2 * (start + it_r[j]) + 1] = it_q[j];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

hipError_t launch_block_ids(const uint8_t* pad, const int32_t* att, int B, int N, int nc, const uint8_t* cross_pad,
                            int32_t* q_blk, int32_t* k_blk, uint8_t* q_valid, uint8_t* k_valid, hipStream_t s) {
    hipLaunchKernelGGL(block_ids_kernel, dim3(B), dim3(256), 0, s, pad, att, N, nc, cross_pad, q_blk, k_blk, q_valid,
                       k_valid);
    return hipGetLastError();
}

hipError_t launch_blockid_summary(const int32_t* q_blk, const int32_t* k_blk, const uint8_t* q_valid,
                                  const uint8_t* k_valid, int B, int Sq, int Sk, int BM, int BN, int32_t* qsum,
                                  int32_t* ksum, uint32_t* kv_bits, hipStream_t s) {
    const int nQt = (Sq + BM - 1) / BM, nKt = (Sk + BN - 1) / BN;
    if (nQt + nKt == 0) return hipSuccess;
    hipLaunchKernelGGL(blockid_summary_kernel, dim3(nQt + nKt, B), dim3(64), 0, s, q_blk, k_blk, q_valid, k_valid, Sq,
                       Sk, BM, BN, nQt, nKt, qsum, ksum, kv_bits);
    return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, int Nq, int Nk, int BM, uint8_t* tile_kind, uint32_t* fine_bits,
                          int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind, hipStream_t s) {
    const int nStrips = (Nq + kCmpRows - 1) / kCmpRows, nKt = (Nk + 63) / 64;
    const int nQt = (Nq + BM - 1) / BM;
    const bool bm64 = BM == 64;
    if (nQt == 0) {
        return zero_i32(row_ptr, 1, s);
    }
    if (nKt > 0) {
        const dim3 grid((Nk + kCmpCols - 1) / kCmpCols, nStrips);
        const bool vec = (Nk % 16 == 0) && (((uintptr_t)mask & 15) == 0);
        if (vec)
            hipLaunchKernelGGL(compact_tiles_wide_kernel<kCmpRPW>, dim3((Nk + kWideCols - 1) / kWideCols, nStrips),
                               dim3(64 * (kCmpRows / kCmpRPW)),
                               0, s, mask, Nq, Nk, nKt, bm64, tile_kind, fine_bits);
        else
            hipLaunchKernelGGL(compact_tiles_kernel<false>, grid, dim3(256), 0, s, mask, Nq, Nk, nKt, bm64,
                               tile_kind, fine_bits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_csr(tile_kind, nQt, nKt, row_ptr, col_idx, col_kind, s);
}

hipError_t launch_coarsen_tiles(const uint8_t* kind64, int Nq, int Nk, uint8_t* kind128, int32_t* row_ptr,
                                int32_t* col_idx, uint8_t* col_kind, hipStream_t s) {
    const int nQt64 = (Nq + 63) / 64, nQt = (Nq + 127) / 128, nKt = (Nk + 63) / 64;
    if (nQt == 0) return zero_i32(row_ptr, 1, s);
    const int64_t n = (int64_t)nQt * nKt;
    if (n > 0) {
        hipLaunchKernelGGL(coarsen_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kind64, nQt64,
                           nKt, nQt, kind128);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_csr(kind128, nQt, nKt, row_ptr, col_idx, col_kind, s);
}

hipError_t launch_tile_counts(const uint8_t* kind, int64_t n, int64_t* counts, hipStream_t s) {
    hipLaunchKernelGGL(zero_i64_kernel, dim3(1), dim3(64), 0, s, counts, 3);
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    if (blocks > 0) hipLaunchKernelGGL(tile_counts_kernel, dim3((unsigned)blocks), dim3(256), 0, s, kind, n, counts);
    hipLaunchKernelGGL(tile_counts_finish_kernel, dim3(1), dim3(64), 0, s, n, counts);
    return hipGetLastError();
}

hipError_t launch_predicate_tiles(const mfa_predicate& pred, int Nq, int Nk, int BM, uint8_t* tile_kind,
                                  uint32_t* fine_bits, int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind,
                                  hipStream_t s) {
    const int nStrips = (Nq + kCmpRows - 1) / kCmpRows, nKt = (Nk + 63) / 64;
    const int nQt = (Nq + BM - 1) / BM;
    if (nQt == 0) {
        return zero_i32(row_ptr, 1, s);
    }
    if (nKt > 0) {
        const dim3 grid((Nk + kCmpCols - 1) / kCmpCols, nStrips);
        hipLaunchKernelGGL(predicate_tiles_kernel, grid, dim3(256), 0, s, pred, Nq, Nk, nKt, BM == 64, tile_kind,
                           fine_bits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_csr(tile_kind, nQt, nKt, row_ptr, col_idx, col_kind, s);
}

hipError_t launch_bsr_prepare(const int32_t* indptr, const int32_t* indices, int B, int Hkv, int nQb, int nKb,
                              int64_t nnz, int qb, int kb, int Sq, int Skv, int causal, const uint32_t* kv_valid,
                              uint8_t* col_kind, int32_t* csc_ptr, int32_t* csc_idx, hipStream_t s) {
    const size_t lds = (size_t)(nKb + 1024) * sizeof(int);  // at most 68 KB (nKb <= 16384)
    hipError_t e = hipFuncSetAttribute((const void*)&bsr_prepare_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bsr_prepare_kernel, dim3(B * Hkv), dim3(1024), lds, s, indptr, indices, nQb, nKb, nnz, qb, kb, Sq,
                       Skv, causal, kv_valid, Hkv, col_kind, csc_ptr, csc_idx);
    return hipGetLastError();
}

hipError_t launch_bsr_from_bitmask(const uint32_t* bits, int B, int Hkv, int nQb, int nKb, int32_t* indptr,
                                   int32_t* indices, int64_t cap, hipStream_t s) {
    const int n_bh = B * Hkv;
    if (nQb == 0) return zero_i32(indptr, n_bh, s);
    if (nKb == 0) {
        return zero_i32(indptr, (int64_t)n_bh * (nQb + 1), s);
    }
    hipLaunchKernelGGL(bitmask_count_kernel, dim3(1), dim3(1024), 0, s, bits, n_bh, nQb, nKb, indptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)n_bh * nQb;
    hipLaunchKernelGGL(bitmask_fill_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, bits, n_bh, nQb,
                       nKb, indptr, indices, cap);
    return hipGetLastError();
}

hipError_t launch_varlen_schedule(const int32_t* len_q, const int32_t* len_k, int nseq, int BM, int BN, int causal,
                                  int left, int right, int32_t* cu_q, int32_t* cu_k, int32_t* max_len,
                                  int32_t* work, int work_cap, int32_t* n_work, hipStream_t s) {
    hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(1024), 0, s, len_q, len_k, nseq, BM, BN, causal, left,
                       right, cu_q, cu_k, max_len, work, work_cap, n_work);
    return hipGetLastError();
}

}  // namespace mfa
