// Shared device/host helpers for libmfa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfa.h"

namespace mfa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTileEmpty = MFA_TILE_EMPTY;
constexpr int kTilePartial = MFA_TILE_PARTIAL;
constexpr int kTileFull = MFA_TILE_FULL;

// Device copy of mfa_mask plus derived sizes. Passed by value to kernels.
struct MaskDev {
    int kind;
    const int32_t* q_blk;
    const int32_t* k_blk;
    const uint8_t* q_valid;
    const int32_t* qsum;
    const int32_t* ksum;
    const uint32_t* kv_bits;
    const uint32_t* fine_bits;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint8_t* col_kind;
    const int32_t* indptr;
    const int32_t* indices;
    const uint8_t* bsr_kind;
    const int32_t* csc_ptr;
    const int32_t* csc_idx;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* work;
    int32_t* err;
    int work_cap;
    int max_q, max_k;
    int causal, win_left, win_right;
    const uint8_t* tile_kind;  // TILES: (ceil(Sq/128), ceil(Sk/64)) kinds (dK/dV pass)
    int fine_words;   // ceil(Sk / 32)
    int kv_words;     // ceil(Sk / 32)
    int nQb;          // BSR query-block rows per (b, h)
    int nseq;         // VARLEN sequences
    const int32_t* seqused_k;    // VARLEN: keys used per sequence, or null
    const int32_t* block_table;  // VARLEN: (nseq, max_pages) pages of k / v, or null
    int max_pages, page_size, n_pages;
    int tile_shift;   // TILES: log2(map rows per tile / 64) (1 for 128-row maps, 0 for 64)
};

// Problem description shared by the forward kernels.
struct FwdDev {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t qs0, qs1, qs2;
    int64_t ks0, ks1, ks2;
    int64_t vs0, vs1, vs2;
    int64_t os0, os1, os2;
    int B, Sq, Sk, Hq, Hkv, G;
    int nQt, nKt;
    float scale, c2;  // c2 = scale * log2(e)
    const float* alibi;  // per query head slopes of the bias slope * (kv - q), or null
    // soft cap cap * tanh(x / cap) of the scaled scores x (0: none), with
    // cap_raw = cap / scale, cap_k2 = 2 * scale * log2(e) / cap and
    // cap_tinv = scale / cap for the raw-score form used by the MFMA kernels
    float cap, cap_raw, cap_k2, cap_tinv;
    int total;        // workgroups launched
    int xcd_remap;    // 1: logical id = (w % 8) * (total / 8) + w / 8
    // Order of the query tiles over the logical ids (dense-tile, block-id,
    // BSR and unmasked layouts). 0: (batch, head) major, each head's tiles
    // heaviest (last) first. lpt_group > 0: runs of lpt_group * nQt ids cover
    // lpt_group consecutive (batch, head) pairs, level by level from the last
    // query tile to the first, so that the heaviest tiles of the run start
    // before any lighter one (for grids of a few workgroups per slot).
    int lpt_group;
};

// Backward problem: the forward's tensors plus dO, dQ, dK, dV and delta.
// Size of the static device scratch of mfa_attn_bwd_dkdv_noalloc (96 MiB):
// the dK/dV query-head split's partial sums of a GQA problem with up to
// 12 Mi (batch, key, kv head, d) elements, e.g. B=8, Sk=1280, Hkv=2, D=128
// split four ways (80 MiB).
constexpr int64_t kBwdScratchBytes = int64_t(96) << 20;

struct BwdDev {
    FwdDev f;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;
    int64_t dos0, dos1, dos2;
    int64_t dqs0, dqs1, dqs2;
    int64_t dks0, dks1, dks2;
    int64_t dvs0, dvs1, dvs2;
    // dK/dV query-head split (GQA): gsplit workgroups per key block, each
    // over G / gsplit query heads, writing fp32 partial sums to ws
    // ([2][gsplit][B][Sk][Hkv][D]: dK, then dV) for the reduce pass; 1: no split
    float* ws;
    int gsplit;
};

__device__ __forceinline__ int xcd_logical(int w, int total, int remap) {
    if (!remap) return w;
    return (w & 7) * (total >> 3) + (w >> 3);
}

// 64 consecutive entries of a device list held one per lane of the wave,
// with the following 64 already requested: get(pos) for a non-decreasing
// wave-uniform pos is a v_readlane instead of a dependent global load.
// fetch(pos) loads entry pos (or returns 0 past the end); moving backwards
// or past the requested window reloads.
struct ListWindow {
    int base;
    uint32_t cur, nxt;

    template <class F>
    __device__ __forceinline__ void init(const F& fetch, int pos, int lane) {
        base = pos;
        cur = fetch(pos + lane);
        nxt = fetch(pos + 64 + lane);
    }

    template <class F>
    __device__ __forceinline__ uint32_t get(const F& fetch, int pos, int lane) {
        if (__builtin_expect(pos < base || pos - base >= 64, 0)) {
            if (pos - base >= 64 && pos - base < 128) {
                base += 64;
                cur = nxt;
                nxt = fetch(base + 64 + lane);
            } else {
                init(fetch, pos, lane);
            }
        }
        return (uint32_t)__builtin_amdgcn_readlane((int)cur, pos - base);
    }
};

// As ListWindow, for entries packed as value | kind << 28 where kind 0 means
// "skip": seek() moves to the next entry with a nonzero kind using a ballot
// of the window, so runs of skipped entries cost a bit scan, not a load each.
struct ScanWindow {
    int base;
    uint32_t cur, nxt;
    uint64_t nz;

    template <class F>
    __device__ __forceinline__ void init(const F& fetch, int pos, int lane) {
        base = pos;
        cur = fetch(pos + lane);
        nxt = fetch(pos + 64 + lane);
        nz = __builtin_amdgcn_ballot_w64((cur >> 28) != 0u);
    }

    // First position >= pos (and < end) whose entry has a nonzero kind;
    // false when there is none. A pos before the window restarts it.
    template <class F>
    __device__ bool seek(const F& fetch, int& pos, int end, int lane, uint32_t& entry) {
        while (pos < end) {
            if (pos < base) init(fetch, pos, lane);
            const int idx = pos - base;
            if (idx < 64) {
                const uint64_t rest = nz >> idx;
                if (rest) {
                    pos += (int)__builtin_ctzll(rest);
                    entry = (uint32_t)__builtin_amdgcn_readlane((int)cur, pos - base);
                    return true;
                }
                pos = base + 64;
                continue;
            }
            base += 64;
            cur = nxt;
            nxt = fetch(base + 64 + lane);
            nz = __builtin_amdgcn_ballot_w64((cur >> 28) != 0u);
        }
        return false;
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Score modifications compiled into a kernel variant (template bit set).
constexpr int kModBias = 1;  // per-head slope * (kv - q)
constexpr int kModCap = 2;   // soft cap

// Soft cap of a raw score s (q.k plus any bias, in units of 1 / scale):
// cap * tanh(scale * s / cap), returned in the same raw units. Uses
// tanh(y) = 1 - 2 / (exp(2y) + 1): one exp2 and one reciprocal, and it
// saturates to -+cap_raw where exp2 underflows or overflows.
__device__ __forceinline__ float softcap_raw(float s, const FwdDev& p) {
    const float e = fast_exp2(s * p.cap_k2);
    return fmaf(__builtin_amdgcn_rcpf(e + 1.f), -2.f * p.cap_raw, p.cap_raw);
}

// Derivative 1 - tanh^2 of the soft cap at a capped raw score sc; 0 for a
// masked score (-inf), so that a zero probability times it stays 0.
__device__ __forceinline__ float softcap_grad(float sc, const FwdDev& p) {
    const float t = sc * p.cap_tinv;
    return fmaxf(fmaf(-t, t, 1.f), 0.f);
}

// Value of `x` held by lane (lane ^ 32), via the gfx950 cross-half swap.
__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    // lanes 0..31: r[1] holds lane+32's value; lanes 32..63: r[0] holds lane-32's value
    return __int_as_float((__lane_id() < 32) ? r[1] : r[0]);
}

__device__ __forceinline__ float max_both_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    // one v_max_f32: fmaxf would first quiet both operands (the compiler
    // cannot tell that integer-typed lane data holds no signalling NaN)
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__int_as_float(r[0])), "v"(__int_as_float(r[1])));
    return m;
}

__device__ __forceinline__ float sum_both_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

}  // namespace mfa
