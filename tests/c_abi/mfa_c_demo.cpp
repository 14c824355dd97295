// Calls libmfa through its C ABI alone (no Python, no torch): dense mask ->
// tile compaction -> bf16 attention forward, then writes out and lse to a
// file for the test to compare with the oracle. Inputs come from SplitMix64
// (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// 2014), which the test reimplements to rebuild the same inputs.
//
// usage: mfa_c_demo OUTFILE
// q, k, v: (1, N=300, H=2, D=128) bf16, BSHD contiguous, uniform [-1, 1);
// mask (N, N): causal and at most 100 past keys (i - j < 100); scale 1/sqrt(D).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mfa.h"

static uint64_t splitmix64(uint64_t& s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint16_t to_bf16(float x) {  // round to nearest even (inputs are finite)
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 2; } } while (0)
#define CHECK_MFA(x) do { mfa_status s_ = (x); if (s_ != MFA_OK) { \
    std::fprintf(stderr, "%s: %s (line %d)\n", mfa_status_name(s_), mfa_last_error(), __LINE__); return 3; } } while (0)

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s OUTFILE\n", argv[0]);
        return 1;
    }
    const int N = 300, H = 2, D = 128;
    const size_t n = (size_t)N * H * D;
    std::vector<uint16_t> hq(n), hk(n), hv(n);
    uint64_t st = 20261203;
    for (auto* t : {&hq, &hk, &hv})
        for (size_t i = 0; i < n; ++i) (*t)[i] = to_bf16((float)((splitmix64(st) >> 40) * 0x1p-24) * 2.f - 1.f);
    std::vector<uint8_t> hm((size_t)N * N);
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) hm[(size_t)i * N + j] = (j <= i && i - j < 100) ? 1 : 0;

    const int nQt = (N + 127) / 128, nKt = (N + 63) / 64, W = (N + 31) / 32;
    void *q, *k, *v, *o, *mask, *tk, *fb, *rp, *ci, *ck;
    float* lse;
    HIP_OK(hipMalloc(&q, n * 2));
    HIP_OK(hipMalloc(&k, n * 2));
    HIP_OK(hipMalloc(&v, n * 2));
    HIP_OK(hipMalloc(&o, n * 2));
    HIP_OK(hipMalloc((void**)&lse, (size_t)H * N * 4));
    HIP_OK(hipMalloc(&mask, (size_t)N * N));
    HIP_OK(hipMalloc(&tk, (size_t)nQt * nKt));
    HIP_OK(hipMalloc(&fb, (size_t)N * W * 4));
    HIP_OK(hipMalloc(&rp, (size_t)(nQt + 1) * 4));
    HIP_OK(hipMalloc(&ci, (size_t)nQt * nKt * 4));
    HIP_OK(hipMalloc(&ck, (size_t)nQt * nKt));
    HIP_OK(hipMemcpy(q, hq.data(), n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk.data(), n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv.data(), n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(mask, hm.data(), (size_t)N * N, hipMemcpyHostToDevice));

    CHECK_MFA(mfa_compact_dense_mask((const uint8_t*)mask, N, N, 128, 64, (uint8_t*)tk, (uint32_t*)fb, (int32_t*)rp,
                                  (int32_t*)ci, (uint8_t*)ck, nullptr));
    mfa_attn_args a;
    std::memset(&a, 0, sizeof(a));
    a.dtype = MFA_BF16;
    a.B = 1; a.Sq = N; a.Sk = N; a.Hq = H; a.Hkv = H; a.D = D;
    a.q = q; a.k = k; a.v = v; a.out = o; a.lse = lse;
    const int64_t st3[3] = {(int64_t)N * H * D, (int64_t)H * D, D};  // (batch, seq, head) element strides
    std::memcpy(a.q_stride, st3, sizeof(st3));
    std::memcpy(a.k_stride, st3, sizeof(st3));
    std::memcpy(a.v_stride, st3, sizeof(st3));
    std::memcpy(a.o_stride, st3, sizeof(st3));
    mfa_mask m;
    std::memset(&m, 0, sizeof(m));
    m.kind = MFA_MASK_TILES;
    m.tile_kind = (const uint8_t*)tk;
    m.fine_bits = (const uint32_t*)fb;
    m.row_ptr = (const int32_t*)rp;
    m.col_idx = (const int32_t*)ci;
    m.col_kind = (const uint8_t*)ck;
    CHECK_MFA(mfa_attn_fwd(&a, &m, 1.f / std::sqrt((float)D), nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<uint16_t> ho(n);
    std::vector<float> hl((size_t)H * N);
    HIP_OK(hipMemcpy(ho.data(), o, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl.data(), lse, hl.size() * 4, hipMemcpyDeviceToHost));
    FILE* f = std::fopen(argv[1], "wb");
    if (!f) return 4;
    std::fwrite(ho.data(), 2, n, f);
    std::fwrite(hl.data(), 4, hl.size(), f);
    std::fclose(f);
    std::printf("ok\n");
    return 0;
}
