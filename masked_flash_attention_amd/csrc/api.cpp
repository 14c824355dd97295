// C ABI of libmfa: host-side validation, then kernel launches.
// Every entry point validates its arguments before touching the device and
// reports failures through a status code plus a thread-local message.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "common.hpp"

namespace mfa {
hipError_t launch_attn_fwd(int dtype, int D, int BM, const FwdDev& p, const MaskDev& m, hipStream_t s);
hipError_t launch_block_ids(const uint8_t*, const int32_t*, int, int, int, const uint8_t*, int32_t*, int32_t*,
                            uint8_t*, uint8_t*, hipStream_t);
hipError_t launch_blockid_summary(const int32_t*, const int32_t*, const uint8_t*, const uint8_t*, int, int, int, int,
                                  int, int32_t*, int32_t*, uint32_t*, hipStream_t);
hipError_t launch_compact(const uint8_t*, int, int, int, uint8_t*, uint32_t*, int32_t*, int32_t*, uint8_t*,
                          hipStream_t);
hipError_t launch_predicate_tiles(const mfa_predicate&, int, int, int, uint8_t*, uint32_t*, int32_t*, int32_t*,
                                  uint8_t*, hipStream_t);
hipError_t launch_bsr_prepare(const int32_t*, const int32_t*, int, int, int, int, int64_t, int, int, int, int, int,
                              const uint32_t*, uint8_t*, int32_t*, int32_t*, hipStream_t);
hipError_t launch_coarsen_tiles(const uint8_t*, int, int, uint8_t*, int32_t*, int32_t*, uint8_t*, hipStream_t);
hipError_t launch_tile_counts(const uint8_t*, int64_t, int64_t*, hipStream_t);
hipError_t launch_bsr_from_bitmask(const uint32_t*, int, int, int, int, int32_t*, int32_t*, int64_t, hipStream_t);
hipError_t launch_varlen_schedule(const int32_t*, const int32_t*, int, int, int, int, int, int, int32_t*, int32_t*,
                                  int32_t*, int32_t*, int, int32_t*, hipStream_t);
hipError_t launch_bwd_preprocess(const BwdDev& p, int D, int dtype, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdDev& p, const MaskDev& m, int D, int dtype, hipStream_t s);
hipError_t launch_bwd_dq(const BwdDev& p, const MaskDev& m, int D, int dtype, int BM, hipStream_t s);
hipError_t bwd_scratch(void** ptr);
}  // namespace mfa

using namespace mfa;

namespace {

thread_local std::string g_err;

mfa_status fail(mfa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

mfa_status ok() { return MFA_OK; }

// Launch log: with MFA_LOG set (and not "0") in the environment, every
// launching call prints its kernel variant and grid to stderr.
bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("MFA_LOG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

void log_launch(const char* fmt, ...) {
    if (!log_enabled()) return;
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "[mfa] %s\n", buf);
}

const char* kind_name(int k) {
    switch (k) {
        case MFA_MASK_NONE: return "none";
        case MFA_MASK_BLOCKID: return "blockid";
        case MFA_MASK_TILES: return "tiles";
        case MFA_MASK_BSR: return "bsr";
        case MFA_MASK_VARLEN: return "varlen";
    }
    return "?";
}

#define MFA_TRY(expr)                      \
    do {                                   \
        mfa_status _s = (expr);            \
        if (_s != MFA_OK) return _s;       \
    } while (0)

// Per-device result of the architecture check (0 unknown, 1 gfx950, 2 other),
// so that each call costs one hipGetDevice after the first.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

mfa_status ensure_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        int n = 0;
        hipError_t e = hipGetDeviceCount(&n);
        (void)hipGetLastError();
        return fail(MFA_E_NO_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
    }
    const int cached = dev < kMaxDevices ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
    if (cached == 1) return ok();
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n == 0) {
        (void)hipGetLastError();
        return fail(MFA_E_NO_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MFA_E_NO_DEVICE, "hipGetDeviceProperties failed");
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(good ? 1 : 2, std::memory_order_relaxed);
    if (!good)
        return fail(MFA_E_NO_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    return ok();
}

mfa_status dev_ptr(const void* p, const char* name, bool nullable = false) {
    if (!p) return nullable ? ok() : fail(MFA_E_ARG, "%s is NULL", name);
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MFA_E_NOT_DEVICE, "%s (%p) is not device memory", name, p);
    }
    if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
        return fail(MFA_E_NOT_DEVICE, "%s (%p) is host memory; device memory is required", name, p);
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (a.device != dev)
        return fail(MFA_E_NOT_DEVICE, "%s lives on device %d but the current device is %d", name, a.device, dev);
    return ok();
}

mfa_status hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MFA_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

int device_cus();

// Heaviest-first order over a run of (batch, head) pairs (FwdDev::lpt_group)
// when the grid is at most four workgroups per slot of the device (slots:
// two resident 128-row workgroups per CU, four 64-row ones): with so few
// rounds, a heavy tile that starts last sets the end of the launch. Each
// XCD's share of the logical ids (total / 8 with the XCD remap) is one run,
// so every XCD gets the same mix of levels and its heads stay in its L2.
// Larger grids keep the (batch, head)-major order, whose working set per XCD
// is one or two heads.
int lpt_group_for(const FwdDev& p, int BM) {
    if (p.nQt <= 1 || p.total <= 0) return 0;
    const int slots = device_cus() * (BM >= 128 ? 2 : 4);
    if (slots <= 0 || p.total > 4 * slots) return 0;
    const int chunk = p.xcd_remap ? p.total / 8 : p.total;
    if (chunk % p.nQt != 0) return 0;
    return chunk / p.nQt;
}

// Compute units of the current device (cached per device).
std::atomic<int> g_n_cu[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    const int cached = dev < kMaxDevices ? g_n_cu[dev].load(std::memory_order_relaxed) : 0;
    if (cached > 0) return cached;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < kMaxDevices) g_n_cu[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

const char* mfa_last_error(void) { return g_err.c_str(); }

const char* mfa_status_name(mfa_status s) {
    switch (s) {
        case MFA_OK: return "MFA_OK";
        case MFA_E_ARG: return "MFA_E_ARG";
        case MFA_E_SHAPE: return "MFA_E_SHAPE";
        case MFA_E_DTYPE: return "MFA_E_DTYPE";
        case MFA_E_UNSUPPORTED: return "MFA_E_UNSUPPORTED";
        case MFA_E_NOT_DEVICE: return "MFA_E_NOT_DEVICE";
        case MFA_E_NONCANONICAL: return "MFA_E_NONCANONICAL";
        case MFA_E_HIP: return "MFA_E_HIP";
        case MFA_E_NO_DEVICE: return "MFA_E_NO_DEVICE";
    }
    return "MFA_E_UNKNOWN";
}

int mfa_is_available(void) { return ensure_device() == MFA_OK ? 1 : 0; }

mfa_status mfa_make_block_ids(const uint8_t* pad, const int32_t* att, int B, int N, int n_cross,
                              const uint8_t* cross_pad, int32_t* q_blk, int32_t* k_blk, uint8_t* q_valid,
                              uint8_t* k_valid, hipStream_t stream) {
    if (B < 0 || N < 0 || n_cross < 0) return fail(MFA_E_SHAPE, "negative size (B=%d, N=%d, n_cross=%d)", B, N, n_cross);
    if ((n_cross > 0) != (cross_pad != nullptr))
        return fail(MFA_E_ARG, "cross_pad is required iff n_cross > 0 (n_cross=%d, cross_pad=%p)", n_cross, cross_pad);
    if (B == 0 || (N == 0 && n_cross == 0)) return ok();
    MFA_TRY(ensure_device());
    if (N > 0) {
        MFA_TRY(dev_ptr(pad, "pad"));
        MFA_TRY(dev_ptr(att, "att"));
        MFA_TRY(dev_ptr(q_blk, "q_blk"));
        MFA_TRY(dev_ptr(q_valid, "q_valid"));
    }
    MFA_TRY(dev_ptr(k_blk, "k_blk"));
    MFA_TRY(dev_ptr(k_valid, "k_valid"));
    if (n_cross > 0) MFA_TRY(dev_ptr(cross_pad, "cross_pad"));
    return hip_ok(launch_block_ids(pad, att, B, N, n_cross, cross_pad, q_blk, k_blk, q_valid, k_valid, stream),
                  "block_ids launch");
}

mfa_status mfa_blockid_tile_summary(const int32_t* q_blk, const int32_t* k_blk, const uint8_t* q_valid,
                                    const uint8_t* k_valid, int B, int Sq, int Sk, int BM, int BN, int32_t* qsum,
                                    int32_t* ksum, uint32_t* kv_bits, hipStream_t stream) {
    if (B < 0 || Sq < 0 || Sk < 0) return fail(MFA_E_SHAPE, "negative size");
    if (!(BM == 64 || BM == 128) || BN != 64)
        return fail(MFA_E_UNSUPPORTED, "summaries are built for BM in {64, 128} and BN = 64 (got %d, %d)", BM, BN);
    if (B == 0 || (Sq == 0 && Sk == 0)) return ok();
    MFA_TRY(ensure_device());
    if (Sq > 0) {
        MFA_TRY(dev_ptr(q_blk, "q_blk"));
        MFA_TRY(dev_ptr(q_valid, "q_valid"));
        MFA_TRY(dev_ptr(qsum, "qsum"));
    }
    if (Sk > 0) {
        MFA_TRY(dev_ptr(k_blk, "k_blk"));
        MFA_TRY(dev_ptr(k_valid, "k_valid"));
        MFA_TRY(dev_ptr(ksum, "ksum"));
        MFA_TRY(dev_ptr(kv_bits, "kv_bits"));
    }
    return hip_ok(launch_blockid_summary(q_blk, k_blk, q_valid, k_valid, B, Sq, Sk, BM, BN, qsum, ksum, kv_bits, stream),
                  "tile summary launch");
}

mfa_status mfa_compact_dense_mask(const uint8_t* mask, int Nq, int Nk, int BM, int BN, uint8_t* tile_kind,
                                  uint32_t* fine_bits, int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind,
                                  hipStream_t stream) {
    if (Nq < 0 || Nk < 0) return fail(MFA_E_SHAPE, "negative size (Nq=%d, Nk=%d)", Nq, Nk);
    if ((BM != 128 && BM != 64) || BN != 64)
        return fail(MFA_E_UNSUPPORTED, "dense-mask tiles are built for BM=128 or 64, BN=64 (got %d, %d)", BM, BN);
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(row_ptr, "row_ptr"));
    if (Nq > 0 && Nk > 0) {
        MFA_TRY(dev_ptr(mask, "mask"));
        MFA_TRY(dev_ptr(tile_kind, "tile_kind"));
        MFA_TRY(dev_ptr(fine_bits, "fine_bits"));
        MFA_TRY(dev_ptr(col_idx, "col_idx"));
        MFA_TRY(dev_ptr(col_kind, "col_kind"));
    }
    log_launch("compact_dense_mask Nq=%d Nk=%d BM=%d BN=%d", Nq, Nk, BM, BN);
    return hip_ok(launch_compact(mask, Nq, Nk, BM, tile_kind, fine_bits, row_ptr, col_idx, col_kind, stream),
                  "compaction launch");
}

mfa_status mfa_tile_map_coarsen(const uint8_t* kind64, int Nq, int Nk, uint8_t* kind128, int32_t* row_ptr,
                                int32_t* col_idx, uint8_t* col_kind, hipStream_t stream) {
    if (Nq < 0 || Nk < 0) return fail(MFA_E_SHAPE, "negative size (Nq=%d, Nk=%d)", Nq, Nk);
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(row_ptr, "row_ptr"));
    if (Nq > 0 && Nk > 0) {
        MFA_TRY(dev_ptr(kind64, "kind64"));
        MFA_TRY(dev_ptr(kind128, "kind128"));
        MFA_TRY(dev_ptr(col_idx, "col_idx"));
        MFA_TRY(dev_ptr(col_kind, "col_kind"));
    }
    return hip_ok(launch_coarsen_tiles(kind64, Nq, Nk, kind128, row_ptr, col_idx, col_kind, stream),
                  "tile map coarsening launch");
}

mfa_status mfa_tile_counts(const uint8_t* tile_kind, int64_t n, int64_t* counts, hipStream_t stream) {
    if (n < 0) return fail(MFA_E_SHAPE, "negative size");
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(counts, "counts"));
    if (n > 0) MFA_TRY(dev_ptr(tile_kind, "tile_kind"));
    return hip_ok(launch_tile_counts(tile_kind, n, counts, stream), "tile count launch");
}

// Modelled forward time of a tile map, in units of one full 128 x 64 tile:
// setup per query tile plus a cost per partial and per full tile, for each
// head dim and tile height. Least-squares fit (relative error) of MI355X
// forward times at B = 4, H = 32, N = 4096 and 8192, per head dim, over
// eight masks (all-True, all-False, a 50 %-dense random mask whose tiles are
// all partial, causal, causal documents of 32-200 tokens, a 96-wide band,
// 10 % of 64 x 64 blocks, 30 % of 128 x 128 blocks); the fit is within 18 %
// of every measured time. A 64-row tile costs 0.63-0.66 (full) to
// 0.84 (partial) of a full 128-row one, so 64-row tiles pay off only when
// many 128-row tiles are half empty; near ties keep 128 rows, and on those
// sixteen cases per head dim the choice is never more than 6 % slower than
// the faster height.
static const double kTileCost[2][2][3] = {
    // setup per query tile, partial tile, full tile
    {{1.807, 0.844, 0.633}, {3.475, 1.320, 1.000}},  // D = 64: 64-row, 128-row tiles
    {{2.196, 0.835, 0.663}, {4.287, 1.236, 1.000}},  // D = 128
};

double mfa_model_tile_time(const int64_t counts[3], int Nq, int tile_m, int D) {
    if (!counts || Nq < 0) return 0.0;
    const int d = D == 64 ? 0 : 1, h = tile_m == 64 ? 0 : 1;
    const int64_t rows = tile_m == 64 ? cdiv(Nq, 64) : cdiv(Nq, 128);
    return kTileCost[d][h][0] * (double)rows + kTileCost[d][h][1] * (double)counts[1] +
           kTileCost[d][h][2] * (double)counts[2];
}

int mfa_choose_tile_m(const int64_t counts64[3], const int64_t counts128[3], int Nq, int D) {
    if (!counts64 || !counts128 || Nq < 0) return 128;
    return mfa_model_tile_time(counts64, Nq, 64, D) < 0.95 * mfa_model_tile_time(counts128, Nq, 128, D) ? 64 : 128;
}

mfa_status mfa_predicate_tiles(const mfa_predicate* pred, int Nq, int Nk, uint8_t* tile_kind, uint32_t* fine_bits,
                               int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind, hipStream_t stream) {
    if (!pred) return fail(MFA_E_ARG, "pred is NULL");
    if (Nq < 0 || Nk < 0) return fail(MFA_E_SHAPE, "negative size (Nq=%d, Nk=%d)", Nq, Nk);
    if (pred->n_terms < 0 || pred->n_terms > MFA_PRED_MAX_TERMS)
        return fail(MFA_E_ARG, "n_terms=%d outside [0, %d]", pred->n_terms, MFA_PRED_MAX_TERMS);
    for (int t = 0; t < pred->n_terms; ++t)
        if (pred->n_atoms[t] < 0 || pred->n_atoms[t] > MFA_PRED_MAX_ATOMS)
            return fail(MFA_E_ARG, "n_atoms[%d]=%d outside [0, %d]", t, pred->n_atoms[t], MFA_PRED_MAX_ATOMS);
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(row_ptr, "row_ptr"));
    if (Nq > 0 && Nk > 0) {
        MFA_TRY(dev_ptr(tile_kind, "tile_kind"));
        MFA_TRY(dev_ptr(fine_bits, "fine_bits"));
        MFA_TRY(dev_ptr(col_idx, "col_idx"));
        MFA_TRY(dev_ptr(col_kind, "col_kind"));
    }
    mfa_predicate p = *pred;
    for (int t = p.n_terms; t < MFA_PRED_MAX_TERMS; ++t) p.n_atoms[t] = 0;
    return hip_ok(launch_predicate_tiles(p, Nq, Nk, 128, tile_kind, fine_bits, row_ptr, col_idx, col_kind, stream),
                  "predicate tiles launch");
}

mfa_status mfa_bsr_validate(const int32_t* indptr, const int32_t* indices, int B, int Hkv, int nQb, int nKb,
                            int64_t nnz, int* max_row_width, hipStream_t stream) {
    if (B < 0 || Hkv < 0 || nQb < 0 || nKb < 0 || nnz < 0) return fail(MFA_E_SHAPE, "negative size");
    if (!max_row_width) return fail(MFA_E_ARG, "max_row_width is NULL");
    *max_row_width = 0;
    const size_t np = (size_t)B * Hkv * (nQb + 1);
    if (np == 0) return ok();
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(indptr, "indptr"));
    if (nnz > 0) MFA_TRY(dev_ptr(indices, "indices"));
    std::vector<int32_t> ip(np), ix((size_t)nnz);
    MFA_TRY(hip_ok(hipMemcpyAsync(ip.data(), indptr, np * 4, hipMemcpyDeviceToHost, stream), "copy indptr"));
    if (nnz > 0)
        MFA_TRY(hip_ok(hipMemcpyAsync(ix.data(), indices, (size_t)nnz * 4, hipMemcpyDeviceToHost, stream),
                       "copy indices"));
    MFA_TRY(hip_ok(hipStreamSynchronize(stream), "stream sync"));
    int widest = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            const int32_t* p = ip.data() + ((size_t)b * Hkv + h) * (nQb + 1);
            if (p[0] < 0 || p[nQb] > nnz)
                return fail(MFA_E_NONCANONICAL, "row offsets of (b=%d, h=%d) leave [0, %lld]", b, h, (long long)nnz);
            for (int r = 0; r < nQb; ++r) {
                if (p[r + 1] < p[r])
                    return fail(MFA_E_NONCANONICAL, "row offsets of (b=%d, h=%d) decrease at row %d", b, h, r);
                for (int e = p[r]; e < p[r + 1]; ++e) {
                    if (ix[e] < 0 || ix[e] >= nKb)
                        return fail(MFA_E_NONCANONICAL, "block id %d out of [0, %d) in (b=%d, h=%d, r=%d)", ix[e], nKb,
                                    b, h, r);
                    if (e > p[r] && ix[e] <= ix[e - 1])
                        return fail(MFA_E_NONCANONICAL, "block ids not strictly ascending in (b=%d, h=%d, r=%d)", b,
                                    h, r);
                }
                widest = std::max(widest, p[r + 1] - p[r]);
            }
        }
    *max_row_width = widest;
    return ok();
}

mfa_status mfa_bsr_prepare(const int32_t* indptr, const int32_t* indices, int B, int Hkv, int nQb, int nKb,
                           int64_t nnz, int q_block, int kv_block, int Sq, int Skv, int causal,
                           const uint32_t* kv_valid_bits, uint8_t* col_kind, int32_t* csc_ptr, int32_t* csc_idx,
                           hipStream_t stream) {
    if (B < 0 || Hkv < 0 || nQb < 0 || nKb < 0 || nnz < 0 || Sq < 0 || Skv < 0)
        return fail(MFA_E_SHAPE, "negative size");
    if (q_block <= 0 || kv_block <= 0) return fail(MFA_E_ARG, "block sizes must be positive");
    if (nQb != cdiv(Sq, q_block) || nKb != cdiv(Skv, kv_block))
        return fail(MFA_E_SHAPE, "nQb=%d / nKb=%d do not match ceil(Sq/q_block)=%d / ceil(Skv/kv_block)=%d", nQb, nKb,
                    cdiv(Sq, q_block), cdiv(Skv, kv_block));
    if (nKb > 16384) return fail(MFA_E_UNSUPPORTED, "nKb=%d exceeds the 16384 KV blocks the CSC pass holds in LDS", nKb);
    if ((size_t)B * Hkv == 0) return ok();
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(indptr, "indptr"));
    MFA_TRY(dev_ptr(csc_ptr, "csc_ptr"));
    MFA_TRY(dev_ptr(kv_valid_bits, "kv_valid_bits", true));
    if (nnz > 0) {
        MFA_TRY(dev_ptr(indices, "indices"));
        MFA_TRY(dev_ptr(col_kind, "col_kind"));
        MFA_TRY(dev_ptr(csc_idx, "csc_idx"));
    }
    log_launch("bsr_prepare B=%d Hkv=%d nQb=%d nKb=%d nnz=%lld causal=%d kv_valid=%d", B, Hkv, nQb, nKb,
               (long long)nnz, causal ? 1 : 0, kv_valid_bits != nullptr);
    return hip_ok(launch_bsr_prepare(indptr, indices, B, Hkv, nQb, nKb, nnz, q_block, kv_block, Sq, Skv, causal ? 1 : 0,
                                     kv_valid_bits, col_kind, csc_ptr, csc_idx, stream),
                  "bsr prepare launch");
}

mfa_status mfa_bsr_from_bitmask(const uint32_t* bits, int B, int Hkv, int nQb, int nKb, int32_t* indptr,
                                int32_t* indices, int64_t cap, hipStream_t stream) {
    if (B < 0 || Hkv < 0 || nQb < 0 || nKb < 0 || cap < 0) return fail(MFA_E_SHAPE, "negative size");
    const int64_t rows = (int64_t)B * Hkv * nQb;
    if (rows * nKb > INT32_MAX) return fail(MFA_E_UNSUPPORTED, "more than 2^31 - 1 possible blocks");
    if ((int64_t)B * Hkv == 0) return ok();
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(indptr, "indptr"));
    if (rows > 0 && nKb > 0) MFA_TRY(dev_ptr(bits, "bits"));
    if (cap > 0) MFA_TRY(dev_ptr(indices, "indices"));
    return hip_ok(launch_bsr_from_bitmask(bits, B, Hkv, nQb, nKb, indptr, indices, cap, stream),
                  "bsr from bitmask launch");
}

mfa_status mfa_varlen_schedule(const int32_t* len_q, const int32_t* len_k, int nseq, int BM, int BN, int causal,
                               int win_left, int win_right, int32_t* cu_q, int32_t* cu_k, int32_t* max_len,
                               int32_t* work, int work_cap, int32_t* n_work, hipStream_t stream) {
    if (nseq < 0 || work_cap < 0) return fail(MFA_E_SHAPE, "negative size");
    if (BM != 128 || BN != 64) return fail(MFA_E_UNSUPPORTED, "varlen tiles are built for BM=128, BN=64");
    if (win_left < -1 || win_right < -1) return fail(MFA_E_ARG, "window sides must be >= -1");
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(cu_q, "cu_q"));
    MFA_TRY(dev_ptr(cu_k, "cu_k"));
    MFA_TRY(dev_ptr(max_len, "max_len"));
    MFA_TRY(dev_ptr(n_work, "n_work"));
    if (nseq > 0) {
        MFA_TRY(dev_ptr(len_q, "len_q"));
        MFA_TRY(dev_ptr(len_k, "len_k"));
    }
    if (work_cap > 0) MFA_TRY(dev_ptr(work, "work"));
    log_launch("varlen_schedule nseq=%d work_cap=%d causal=%d window=(%d, %d)", nseq, work_cap, causal ? 1 : 0,
               win_left, win_right);
    return hip_ok(launch_varlen_schedule(len_q, len_k, nseq, BM, BN, causal ? 1 : 0, win_left, win_right, cu_q, cu_k,
                                         max_len, work, work_cap, n_work, stream),
                  "varlen schedule launch");
}

static mfa_status check_attn_shapes(const mfa_attn_args* a) {
    if (a->dtype != MFA_BF16 && a->dtype != MFA_F32) return fail(MFA_E_DTYPE, "unknown dtype code %d", a->dtype);
    if (a->B < 0 || a->Sq < 0 || a->Sk < 0 || a->Hq < 1 || a->Hkv < 1)
        return fail(MFA_E_SHAPE, "bad sizes B=%d Sq=%d Sk=%d Hq=%d Hkv=%d", a->B, a->Sq, a->Sk, a->Hq, a->Hkv);
    if (a->Hq % a->Hkv != 0) return fail(MFA_E_SHAPE, "Hq=%d is not a multiple of Hkv=%d", a->Hq, a->Hkv);
    if (a->D != 64 && a->D != 128) return fail(MFA_E_UNSUPPORTED, "head dim %d not built (64, 128 are)", a->D);
    if (!(a->softcap >= 0.f && a->softcap <= FLT_MAX))
        return fail(MFA_E_ARG, "softcap must be finite and >= 0 (0: none)");
    return ok();
}

static mfa_status fill_mask(const mfa_attn_args* a, const mfa_mask* mk, MaskDev& m, int& BM) {
    std::memset(&m, 0, sizeof(m));
    m.kind = mk->kind;
    m.fine_words = cdiv(a->Sk, 32);
    m.kv_words = cdiv(a->Sk, 32);
    BM = 128;
    switch (mk->kind) {
        case MFA_MASK_NONE: break;
        case MFA_MASK_BLOCKID:
            m.q_blk = mk->q_blk;
            m.k_blk = mk->k_blk;
            m.q_valid = mk->q_valid;
            m.qsum = mk->qsum;
            m.ksum = mk->ksum;
            m.kv_bits = mk->kv_bits;
            break;
        case MFA_MASK_TILES:
            if (mk->tile_m != 0 && mk->tile_m != 64 && mk->tile_m != 128)
                return fail(MFA_E_UNSUPPORTED, "tile_m=%d: dense-mask tile maps have 128 or 64 rows", mk->tile_m);
            BM = mk->tile_m == 64 ? 64 : 128;
            m.tile_shift = BM == 128 ? 1 : 0;
            m.fine_bits = mk->fine_bits;
            m.row_ptr = mk->row_ptr;
            m.col_idx = mk->col_idx;
            m.col_kind = mk->col_kind;
            break;
        case MFA_MASK_BSR:
            if (mk->q_block != 64 || mk->kv_block != 64)
                return fail(MFA_E_UNSUPPORTED, "BSR block sizes %d x %d not built (64 x 64 is)", mk->q_block,
                            mk->kv_block);
            BM = 64;
            m.indptr = mk->indptr;
            m.indices = mk->indices;
            m.bsr_kind = mk->bsr_kind;
            m.csc_ptr = mk->csc_ptr;
            m.csc_idx = mk->csc_idx;
            m.causal = mk->causal ? 1 : 0;
            m.nQb = cdiv(a->Sq, 64);
            m.kv_bits = mk->kv_bits;  // optional kv_valid_bits
            break;
        case MFA_MASK_VARLEN:
            if (a->B != 1) return fail(MFA_E_SHAPE, "varlen attention takes packed (T, H, D) tensors with B = 1");
            if (mk->work_cap < 0 || mk->max_q < 0 || mk->max_k < 0)
                return fail(MFA_E_ARG, "negative work_cap / max_q / max_k");
            if (mk->win_left < -1 || mk->win_right < -1) return fail(MFA_E_ARG, "window sides must be >= -1");
            m.cu_q = mk->cu_q;
            m.cu_k = mk->cu_k;
            m.work = mk->work;
            m.work_cap = mk->work_cap;
            m.max_q = mk->max_q;
            m.max_k = mk->max_k;
            m.err = mk->err;
            m.causal = mk->causal ? 1 : 0;
            m.win_left = mk->win_left;
            m.win_right = mk->win_right;
            m.seqused_k = mk->seqused_k;
            m.block_table = mk->block_table;
            if (mk->block_table) {
                if (mk->page_size <= 0 || mk->page_size % 64 != 0)
                    return fail(MFA_E_ARG, "page_size must be a positive multiple of 64 (got %d)", mk->page_size);
                if (mk->max_pages <= 0 || mk->n_pages <= 0)
                    return fail(MFA_E_ARG, "max_pages and n_pages must be positive with a block table");
                m.max_pages = mk->max_pages;
                m.page_size = mk->page_size;
                m.n_pages = mk->n_pages;
            }
            break;
        default: return fail(MFA_E_ARG, "unknown mask kind %d", mk->kind);
    }
    return ok();
}

static mfa_status check_mask_ptrs(const mfa_mask* mk) {
    switch (mk->kind) {
        case MFA_MASK_BLOCKID:
            MFA_TRY(dev_ptr(mk->q_blk, "q_blk"));
            MFA_TRY(dev_ptr(mk->k_blk, "k_blk"));
            MFA_TRY(dev_ptr(mk->q_valid, "q_valid"));
            MFA_TRY(dev_ptr(mk->qsum, "qsum"));
            MFA_TRY(dev_ptr(mk->ksum, "ksum"));
            MFA_TRY(dev_ptr(mk->kv_bits, "kv_bits"));
            break;
        case MFA_MASK_TILES:
            MFA_TRY(dev_ptr(mk->row_ptr, "row_ptr"));
            MFA_TRY(dev_ptr(mk->fine_bits, "fine_bits"));
            MFA_TRY(dev_ptr(mk->col_idx, "col_idx"));
            MFA_TRY(dev_ptr(mk->col_kind, "col_kind"));
            break;
        case MFA_MASK_BSR:
            MFA_TRY(dev_ptr(mk->indptr, "indptr"));
            MFA_TRY(dev_ptr(mk->indices, "indices"));
            MFA_TRY(dev_ptr(mk->bsr_kind, "bsr_kind"));
            MFA_TRY(dev_ptr(mk->kv_bits, "kv_bits", true));
            break;
        case MFA_MASK_VARLEN:
            MFA_TRY(dev_ptr(mk->cu_q, "cu_q"));
            MFA_TRY(dev_ptr(mk->cu_k, "cu_k"));
            if (mk->work_cap > 0) MFA_TRY(dev_ptr(mk->work, "work"));
            MFA_TRY(dev_ptr(mk->err, "err", true));
            MFA_TRY(dev_ptr(mk->seqused_k, "seqused_k", true));
            MFA_TRY(dev_ptr(mk->block_table, "block_table", true));
            break;
        default: break;
    }
    return ok();
}

static void fill_fwd(const mfa_attn_args* a, float scale, FwdDev& p) {
    std::memset(&p, 0, sizeof(p));
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.o = a->out;
    p.lse = a->lse;
    p.qs0 = a->q_stride[0]; p.qs1 = a->q_stride[1]; p.qs2 = a->q_stride[2];
    p.ks0 = a->k_stride[0]; p.ks1 = a->k_stride[1]; p.ks2 = a->k_stride[2];
    p.vs0 = a->v_stride[0]; p.vs1 = a->v_stride[1]; p.vs2 = a->v_stride[2];
    p.os0 = a->o_stride[0]; p.os1 = a->o_stride[1]; p.os2 = a->o_stride[2];
    p.B = a->B; p.Sq = a->Sq; p.Sk = a->Sk; p.Hq = a->Hq; p.Hkv = a->Hkv; p.G = a->Hq / a->Hkv;
    p.scale = scale;
    p.c2 = scale * kLog2e;
    p.alibi = a->alibi_slopes;
    p.cap = a->softcap;
    if (a->softcap > 0.f) {
        p.cap_raw = a->softcap / scale;
        p.cap_k2 = 2.f * scale * kLog2e / a->softcap;
        p.cap_tinv = scale / a->softcap;
    }
}

static mfa_status check_strides(const char* name, const void* ptr, const int64_t* st, int dtype) {
    if (dtype == MFA_BF16) {
        if (!aligned16(ptr)) return fail(MFA_E_ARG, "%s must be 16-byte aligned", name);
        for (int i = 0; i < 3; ++i)
            if (st[i] % 8 != 0) return fail(MFA_E_ARG, "%s strides must be multiples of 8 elements", name);
    }
    for (int i = 0; i < 3; ++i)
        if (st[i] < 0) return fail(MFA_E_ARG, "%s strides must be non-negative", name);
    // Kernels address the rows of one 128-row tile with 32-bit byte offsets
    // from the tile's first row (buffer loads); the tensor itself may be
    // larger. Rows under 16 MiB apart keep 128 of them under 2 GiB.
    const int64_t esize = dtype == MFA_BF16 ? 2 : 4;
    if (st[1] >= (int64_t(1) << 24) / esize)
        return fail(MFA_E_UNSUPPORTED, "%s sequence stride %lld elements: 128 rows must span under 2 GiB", name,
                    (long long)st[1]);
    return ok();
}

mfa_status mfa_attn_fwd(const mfa_attn_args* a, const mfa_mask* mk, float scale, hipStream_t stream) {
    if (!a || !mk) return fail(MFA_E_ARG, "args or mask is NULL");
    MFA_TRY(check_attn_shapes(a));
    if (!(scale > 0.f && scale <= FLT_MAX)) return fail(MFA_E_ARG, "scale must be finite and positive");
    MaskDev m;
    int BM = 128;
    MFA_TRY(fill_mask(a, mk, m, BM));
    if (a->B == 0 || a->Sq == 0) return ok();
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(a->q, "q"));
    MFA_TRY(dev_ptr(a->out, "out"));
    MFA_TRY(dev_ptr(a->lse, "lse", true));
    MFA_TRY(dev_ptr(a->alibi_slopes, "alibi_slopes", true));
    if (a->Sk > 0) {
        MFA_TRY(dev_ptr(a->k, "k"));
        MFA_TRY(dev_ptr(a->v, "v"));
    }
    MFA_TRY(check_strides("q", a->q, a->q_stride, a->dtype));
    MFA_TRY(check_strides("k", a->k, a->k_stride, a->dtype));
    MFA_TRY(check_strides("v", a->v, a->v_stride, a->dtype));
    MFA_TRY(check_strides("out", a->out, a->o_stride, a->dtype));
    MFA_TRY(check_mask_ptrs(mk));
    FwdDev p;
    fill_fwd(a, scale, p);
    p.nQt = cdiv(a->Sq, BM);
    p.nKt = cdiv(a->Sk, 64);  // key-tile width of the forward kernels
    if (mk->kind == MFA_MASK_VARLEN) {
        p.total = mk->work_cap * a->Hq;
        p.nQt = 0;
    } else {
        p.total = a->B * a->Hq * p.nQt;
    }
    if (p.total == 0) return ok();
    // XCD-aware numbering groups consecutive logical tiles on one XCD. The
    // varlen work list is sorted heaviest first, so that grouping would give
    // the first XCD all the heaviest tiles: varlen keeps the hardware's
    // round-robin, which spreads the list over the XCDs in order (and puts
    // each query head on the same XCD when Hq is a multiple of 8).
    p.xcd_remap = (a->dtype == MFA_BF16) && (p.total % 8 == 0) && mk->kind != MFA_MASK_VARLEN ? 1 : 0;
    if (mk->kind != MFA_MASK_VARLEN) p.lpt_group = lpt_group_for(p, BM);
    log_launch("attn_fwd %s D=%d mask=%s BM=%d grid=%d x %d threads xcd_remap=%d lpt_group=%d bias=%d softcap=%g",
               a->dtype == MFA_BF16 ? "bf16" : "f32", a->D, kind_name(mk->kind), BM, p.total,
               a->dtype == MFA_BF16 ? BM / 32 * 64 : BM, p.xcd_remap, p.lpt_group, a->alibi_slopes != nullptr,
               (double)a->softcap);
    return hip_ok(launch_attn_fwd(a->dtype, a->D, BM, p, m, stream), "attention forward launch");
}

// ---- backward ----

static mfa_status check_bwd(const mfa_attn_bwd_args* a, bool need_tensors) {
    if (!a) return fail(MFA_E_ARG, "args is NULL");
    MFA_TRY(check_attn_shapes(&a->fwd));
    if (a->fwd.B == 0 || a->fwd.Sq == 0 || !need_tensors) return ok();
    MFA_TRY(ensure_device());
    MFA_TRY(dev_ptr(a->fwd.out, "out"));
    MFA_TRY(dev_ptr(a->dout, "dout"));
    MFA_TRY(dev_ptr(a->delta, "delta"));
    MFA_TRY(check_strides("out", a->fwd.out, a->fwd.o_stride, a->fwd.dtype));
    MFA_TRY(check_strides("dout", a->dout, a->do_stride, a->fwd.dtype));
    return ok();
}

static void fill_bwd(const mfa_attn_bwd_args* a, float scale, BwdDev& p) {
    std::memset(&p, 0, sizeof(p));
    fill_fwd(&a->fwd, scale, p.f);
    p.dout = a->dout;
    p.dq = a->dq;
    p.dk = a->dk;
    p.dv = a->dv;
    p.delta = a->delta;
    p.dos0 = a->do_stride[0]; p.dos1 = a->do_stride[1]; p.dos2 = a->do_stride[2];
    p.dqs0 = a->dq_stride[0]; p.dqs1 = a->dq_stride[1]; p.dqs2 = a->dq_stride[2];
    p.dks0 = a->dk_stride[0]; p.dks1 = a->dk_stride[1]; p.dks2 = a->dk_stride[2];
    p.dvs0 = a->dv_stride[0]; p.dvs1 = a->dv_stride[1]; p.dvs2 = a->dv_stride[2];
}

// Mask fields each backward pass reads (see mfa.h) and the derived sizes.
static mfa_status check_bwd_mask(const mfa_attn_bwd_args* a, const mfa_mask* mk, bool dkdv, MaskDev& m,
                                 int& BM) {
    if (!mk) return fail(MFA_E_ARG, "mask is NULL");
    MFA_TRY(fill_mask(&a->fwd, mk, m, BM));
    m.tile_kind = mk->tile_kind;
    m.nseq = mk->nseq;
    switch (mk->kind) {
        case MFA_MASK_NONE: break;
        case MFA_MASK_BLOCKID:
            MFA_TRY(dev_ptr(mk->q_blk, "q_blk"));
            MFA_TRY(dev_ptr(mk->k_blk, "k_blk"));
            MFA_TRY(dev_ptr(mk->q_valid, "q_valid"));
            MFA_TRY(dev_ptr(mk->qsum, "qsum"));
            MFA_TRY(dev_ptr(mk->ksum, "ksum"));
            MFA_TRY(dev_ptr(mk->kv_bits, "kv_bits"));
            break;
        case MFA_MASK_TILES:
            MFA_TRY(dev_ptr(mk->fine_bits, "fine_bits"));
            if (dkdv) {
                MFA_TRY(dev_ptr(mk->tile_kind, "tile_kind"));
            } else {
                MFA_TRY(dev_ptr(mk->row_ptr, "row_ptr"));
                MFA_TRY(dev_ptr(mk->col_idx, "col_idx"));
                MFA_TRY(dev_ptr(mk->col_kind, "col_kind"));
            }
            break;
        case MFA_MASK_BSR:
            MFA_TRY(dev_ptr(mk->kv_bits, "kv_bits", true));
            if (dkdv) {
                MFA_TRY(dev_ptr(mk->csc_ptr, "csc_ptr"));
                MFA_TRY(dev_ptr(mk->csc_idx, "csc_idx"));
            } else {
                MFA_TRY(dev_ptr(mk->indptr, "indptr"));
                MFA_TRY(dev_ptr(mk->indices, "indices"));
                MFA_TRY(dev_ptr(mk->bsr_kind, "bsr_kind"));
            }
            break;
        case MFA_MASK_VARLEN:
            MFA_TRY(dev_ptr(mk->cu_q, "cu_q"));
            MFA_TRY(dev_ptr(mk->cu_k, "cu_k"));
            MFA_TRY(dev_ptr(mk->err, "err", true));
            MFA_TRY(dev_ptr(mk->seqused_k, "seqused_k", true));
            if (dkdv) {
                if (mk->nseq < 0) return fail(MFA_E_ARG, "negative nseq");
            } else if (mk->work_cap > 0) {
                MFA_TRY(dev_ptr(mk->work, "work"));
            }
            break;
        default: return fail(MFA_E_ARG, "unknown mask kind %d", mk->kind);
    }
    return ok();
}

mfa_status mfa_attn_bwd_preprocess(const mfa_attn_bwd_args* a, hipStream_t stream) {
    MFA_TRY(check_bwd(a, true));
    if (a->fwd.B == 0 || a->fwd.Sq == 0) return ok();
    BwdDev p;
    fill_bwd(a, 1.f, p);
    return hip_ok(launch_bwd_preprocess(p, a->fwd.D, a->fwd.dtype, stream), "backward preprocess launch");
}

static mfa_status bwd_common(const mfa_attn_bwd_args* a, const mfa_mask* mk, float scale, bool dkdv, BwdDev& p,
                             MaskDev& m, int& BM) {
    MFA_TRY(check_bwd(a, true));
    if (!(scale > 0.f && scale <= FLT_MAX)) return fail(MFA_E_ARG, "scale must be finite and positive");
    // No query rows: the dQ pass has nothing to do, while the dK/dV pass
    // still runs, to write dK = dV = 0 (its key blocks list no query block).
    if (a->fwd.B == 0 || (a->fwd.Sq == 0 && (!dkdv || a->fwd.Sk == 0))) return ok();
    MFA_TRY(ensure_device());
    if (a->fwd.Sq > 0) {
        MFA_TRY(dev_ptr(a->fwd.q, "q"));
        MFA_TRY(dev_ptr(a->fwd.lse, "lse"));
    }
    MFA_TRY(dev_ptr(a->fwd.alibi_slopes, "alibi_slopes", true));
    if (a->fwd.Sk > 0) {
        MFA_TRY(dev_ptr(a->fwd.k, "k"));
        MFA_TRY(dev_ptr(a->fwd.v, "v"));
    }
    MFA_TRY(check_strides("q", a->fwd.q, a->fwd.q_stride, a->fwd.dtype));
    MFA_TRY(check_strides("k", a->fwd.k, a->fwd.k_stride, a->fwd.dtype));
    MFA_TRY(check_strides("v", a->fwd.v, a->fwd.v_stride, a->fwd.dtype));
    BM = 128;
    MFA_TRY(check_bwd_mask(a, mk, dkdv, m, BM));
    fill_bwd(a, scale, p);
    // the dQ pass runs the forward's grid; the dK/dV pass reads nQt / nKt of
    // the 128 x 64 tile map and summaries
    p.f.nQt = cdiv(a->fwd.Sq, BM);
    p.f.nKt = cdiv(a->fwd.Sk, 64);
    if (mk->kind == MFA_MASK_VARLEN) {
        p.f.total = mk->work_cap * a->fwd.Hq;
        p.f.nQt = 0;
    } else {
        p.f.total = a->fwd.B * a->fwd.Hq * p.f.nQt;
    }
    p.f.xcd_remap = (p.f.total % 8 == 0) && mk->kind != MFA_MASK_VARLEN ? 1 : 0;  // as in the forward
    if (mk->kind != MFA_MASK_VARLEN && !dkdv) p.f.lpt_group = lpt_group_for(p.f, BM);
    return ok();
}

int mfa_choose_dkdv_split(int64_t key_blocks, int group, int head_dim, int n_cu) {
    if (group <= 1 || key_blocks <= 0 || n_cu <= 0) return 1;
    const int64_t target = 2 * (int64_t)n_cu * (head_dim == 128 ? 2 : 4);
    if (key_blocks >= target) return 1;
    for (int s = 2; s < group; ++s)
        if (group % s == 0 && key_blocks * s >= target) return s;
    return group;
}

// Preferred head split of the dK/dV pass and the workspace bytes per split.
static void dkdv_split(const mfa_attn_bwd_args* a, const mfa_mask* mk, int& splits, int64_t& per_split) {
    splits = 1;
    per_split = 2 * (int64_t)a->fwd.B * a->fwd.Sk * a->fwd.Hkv * a->fwd.D * (int64_t)sizeof(float);
    if (a->fwd.dtype != MFA_BF16 || mk->kind == MFA_MASK_VARLEN || a->fwd.B == 0 || a->fwd.Sq == 0 ||
        a->fwd.Sk == 0)
        return;
    const int64_t key_blocks = (int64_t)a->fwd.B * a->fwd.Hkv * cdiv(a->fwd.Sk, 64);
    splits = mfa_choose_dkdv_split(key_blocks, a->fwd.Hq / a->fwd.Hkv, a->fwd.D, device_cus());
}

mfa_status mfa_attn_bwd_dkdv_workspace(const mfa_attn_bwd_args* a, const mfa_mask* mk, int64_t* bytes,
                                       int* splits) {
    if (!bytes || !splits) return fail(MFA_E_ARG, "bytes / splits is NULL");
    MFA_TRY(check_bwd(a, false));
    if (!mk) return fail(MFA_E_ARG, "mask is NULL");
    MFA_TRY(ensure_device());
    int S = 1;
    int64_t per = 0;
    dkdv_split(a, mk, S, per);
    *splits = S;
    *bytes = S > 1 ? S * per : 0;
    return ok();
}

// The dK/dV pass with its head-split buffer from the caller's workspace
// (use_scratch false: the largest split up to the preferred one whose sums
// fit) or from the library's static scratch (use_scratch true: the preferred
// split, an error if its sums do not fit).
static mfa_status bwd_dkdv_run(const mfa_attn_bwd_args* a, const mfa_mask* mk, float scale, hipStream_t stream,
                               bool use_scratch) {
    BwdDev p;
    MaskDev m;
    int BM = 128;
    MFA_TRY(bwd_common(a, mk, scale, true, p, m, BM));
    if (a->fwd.B == 0 || a->fwd.Sk == 0) return ok();
    MFA_TRY(dev_ptr(a->dk, "dk"));
    MFA_TRY(dev_ptr(a->dv, "dv"));
    MFA_TRY(check_strides("dk", a->dk, a->dk_stride, a->fwd.dtype));
    MFA_TRY(check_strides("dv", a->dv, a->dv_stride, a->fwd.dtype));
    int pref = 1, S = 1;
    int64_t per = 0;
    dkdv_split(a, mk, pref, per);
    const int G = a->fwd.Hq / a->fwd.Hkv;
    void* ws = nullptr;
    if (use_scratch) {
        if (pref > 1) {
            if (pref * per > kBwdScratchBytes)
                return fail(MFA_E_UNSUPPORTED,
                            "the dK/dV head split (%d ways) needs %lld bytes of scratch; the static scratch holds "
                            "%lld; call mfa_attn_bwd_dkdv with a workspace instead",
                            pref, (long long)(pref * per), (long long)kBwdScratchBytes);
            MFA_TRY(hip_ok(bwd_scratch(&ws), "static scratch lookup"));
            S = pref;
        }
    } else if (pref > 1 && a->workspace) {
        for (int s = pref; s > 1 && S == 1; --s)
            if (G % s == 0 && s * per <= a->workspace_bytes) S = s;
        if (S > 1) {
            MFA_TRY(dev_ptr(a->workspace, "workspace"));
            if (!aligned16(a->workspace)) return fail(MFA_E_ARG, "workspace must be 16-byte aligned");
            ws = a->workspace;
        }
    }
    p.gsplit = S;
    p.ws = (float*)ws;
    log_launch("attn_bwd_dkdv%s %s D=%d mask=%s B=%d Hkv=%d Sk=%d (64-key blocks) head_split=%d bias=%d",
               use_scratch ? "_noalloc" : "", a->fwd.dtype == MFA_BF16 ? "bf16" : "f32", a->fwd.D,
               kind_name(mk->kind), a->fwd.B, a->fwd.Hkv, a->fwd.Sk, S, a->fwd.alibi_slopes != nullptr);
    return hip_ok(launch_bwd_dkdv(p, m, a->fwd.D, a->fwd.dtype, stream), "backward dK/dV launch");
}

mfa_status mfa_attn_bwd_dkdv(const mfa_attn_bwd_args* a, const mfa_mask* mk, float scale, hipStream_t stream) {
    return bwd_dkdv_run(a, mk, scale, stream, false);
}

mfa_status mfa_attn_bwd_dkdv_noalloc(const mfa_attn_bwd_args* a, const mfa_mask* mk, float scale,
                                     hipStream_t stream) {
    return bwd_dkdv_run(a, mk, scale, stream, true);
}

int64_t mfa_bwd_scratch_bytes(void) { return kBwdScratchBytes; }

mfa_status mfa_attn_bwd_dq(const mfa_attn_bwd_args* a, const mfa_mask* mk, float scale, hipStream_t stream) {
    BwdDev p;
    MaskDev m;
    int BM = 128;
    MFA_TRY(bwd_common(a, mk, scale, false, p, m, BM));
    if (a->fwd.B == 0 || a->fwd.Sq == 0) return ok();
    MFA_TRY(dev_ptr(a->dq, "dq"));
    MFA_TRY(check_strides("dq", a->dq, a->dq_stride, a->fwd.dtype));
    log_launch("attn_bwd_dq %s D=%d mask=%s BM=%d grid=%d lpt_group=%d bias=%d",
               a->fwd.dtype == MFA_BF16 ? "bf16" : "f32", a->fwd.D, kind_name(mk->kind), BM, p.f.total,
               p.f.lpt_group, a->fwd.alibi_slopes != nullptr);
    return hip_ok(launch_bwd_dq(p, m, a->fwd.D, a->fwd.dtype, BM, stream), "backward dQ launch");
}

}  // extern "C"
