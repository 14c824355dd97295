// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (no device code runs): every
// entry point is called with NULL pointers, negative and oversized shapes,
// unknown enums and non-finite scales, and the status codes, the
// thread-local error message and the host-only dispatch model are checked.
// On a machine without a GPU, calls that pass validation stop at the device
// check (MFA_E_NO_DEVICE); nothing is launched. Exit status 0 = all passed.

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "mfa.h"

static int g_failed = 0;

static void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, mfa_last_error());
        ++g_failed;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A status that validation may return, or the no-device stop after it.
static bool is(mfa_status got, mfa_status want) { return got == want; }
static bool is_or_nodev(mfa_status got, mfa_status want) { return got == want || got == MFA_E_NO_DEVICE; }

static mfa_attn_args args(int dtype = MFA_BF16) {
    mfa_attn_args a;
    std::memset(&a, 0, sizeof(a));
    a.dtype = dtype;
    a.B = 1;
    a.Sq = 128;
    a.Sk = 128;
    a.Hq = 4;
    a.Hkv = 2;
    a.D = 128;
    return a;
}

static mfa_mask mask(int kind) {
    mfa_mask m;
    std::memset(&m, 0, sizeof(m));
    m.kind = kind;
    m.win_left = m.win_right = -1;
    return m;
}

static void attention_validation() {
    mfa_mask none = mask(MFA_MASK_NONE);
    mfa_attn_args a = args();
    EXPECT(is(mfa_attn_fwd(nullptr, &none, 0.1f, nullptr), MFA_E_ARG));
    EXPECT(is(mfa_attn_fwd(&a, nullptr, 0.1f, nullptr), MFA_E_ARG));
    EXPECT(std::strlen(mfa_last_error()) > 0);
    const float bad_scales[] = {0.f, -1.f, NAN, INFINITY};
    for (float sc : bad_scales) EXPECT(is(mfa_attn_fwd(&a, &none, sc, nullptr), MFA_E_ARG));
    a = args();
    a.Hq = 3;
    EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_E_SHAPE));
    a = args();
    a.D = 96;
    EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_E_UNSUPPORTED));
    const float bad_caps[] = {-1.f, NAN, INFINITY};
    for (float cap : bad_caps) {
        a = args();
        a.softcap = cap;
        EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_E_ARG));
    }
    a = args(7);
    EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_E_DTYPE));
    a = args();
    a.Sq = -5;
    EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_E_SHAPE));
    a = args();
    a.B = 0;
    EXPECT(is(mfa_attn_fwd(&a, &none, 0.1f, nullptr), MFA_OK));
    // unknown mask kind, unbuilt block sizes and tile heights, varlen layout errors
    a = args();
    mfa_mask m = mask(42);
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_ARG));
    m = mask(MFA_MASK_BSR);
    m.q_block = 32;
    m.kv_block = 64;
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_UNSUPPORTED));
    m = mask(MFA_MASK_TILES);
    m.tile_m = 96;
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_UNSUPPORTED));
    m = mask(MFA_MASK_VARLEN);
    a.B = 2;
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_SHAPE));
    a.B = 1;
    m.win_left = -3;
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_ARG));
    m = mask(MFA_MASK_VARLEN);
    m.block_table = reinterpret_cast<const int32_t*>(16);
    m.page_size = 48;
    m.max_pages = 4;
    m.n_pages = 8;
    EXPECT(is(mfa_attn_fwd(&a, &m, 0.1f, nullptr), MFA_E_ARG));
    // backward: same shape checks, fp32 test mode accepted by validation
    mfa_attn_bwd_args b;
    std::memset(&b, 0, sizeof(b));
    EXPECT(is(mfa_attn_bwd_preprocess(nullptr, nullptr), MFA_E_ARG));
    b.fwd = args();
    b.fwd.Hkv = 0;
    EXPECT(is(mfa_attn_bwd_dq(&b, &none, 0.1f, nullptr), MFA_E_SHAPE));
    b.fwd = args(MFA_F32);
    EXPECT(is_or_nodev(mfa_attn_bwd_dkdv(&b, &none, 0.1f, nullptr), MFA_E_ARG));
    EXPECT(is(mfa_attn_bwd_dq(&b, nullptr, 0.1f, nullptr), MFA_E_NO_DEVICE) ||
           is(mfa_attn_bwd_dq(&b, nullptr, 0.1f, nullptr), MFA_E_ARG));
    // workspace query of the dK/dV head split
    int64_t bytes = -1;
    int splits = -1;
    b.fwd = args();
    EXPECT(is(mfa_attn_bwd_dkdv_workspace(&b, &none, nullptr, &splits), MFA_E_ARG));
    EXPECT(is(mfa_attn_bwd_dkdv_workspace(&b, nullptr, &bytes, &splits), MFA_E_ARG));
    EXPECT(is(mfa_attn_bwd_dkdv_workspace(nullptr, &none, &bytes, &splits), MFA_E_ARG));
    b.fwd.Hq = 3;
    EXPECT(is(mfa_attn_bwd_dkdv_workspace(&b, &none, &bytes, &splits), MFA_E_SHAPE));
    b.fwd = args();
    mfa_status st = mfa_attn_bwd_dkdv_workspace(&b, &none, &bytes, &splits);
    EXPECT(is(st, MFA_E_NO_DEVICE) || (is(st, MFA_OK) && splits >= 1 && bytes >= 0));
    // the allocation-free dK/dV entry point validates like the workspace one
    EXPECT(is(mfa_attn_bwd_dkdv_noalloc(nullptr, &none, 0.1f, nullptr), MFA_E_ARG));
    EXPECT(is(mfa_attn_bwd_dkdv_noalloc(&b, nullptr, 0.1f, nullptr), MFA_E_ARG) ||
           is(mfa_attn_bwd_dkdv_noalloc(&b, nullptr, 0.1f, nullptr), MFA_E_NO_DEVICE));
    EXPECT(mfa_bwd_scratch_bytes() == (int64_t(96) << 20));
}

static void mask_representation_validation() {
    EXPECT(is(mfa_make_block_ids(nullptr, nullptr, 1, 8, 2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
              MFA_E_ARG));
    EXPECT(is(mfa_make_block_ids(nullptr, nullptr, -1, 8, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
              MFA_E_SHAPE));
    EXPECT(is(mfa_make_block_ids(nullptr, nullptr, 0, 8, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
              MFA_OK));
    EXPECT(is(mfa_compact_dense_mask(nullptr, 10, 10, 32, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
              MFA_E_UNSUPPORTED));
    EXPECT(is(mfa_compact_dense_mask(nullptr, -1, 10, 128, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
              MFA_E_SHAPE));
    EXPECT(is(mfa_tile_counts(nullptr, -1, nullptr, nullptr), MFA_E_SHAPE));
    EXPECT(is(mfa_tile_map_coarsen(nullptr, -1, 10, nullptr, nullptr, nullptr, nullptr, nullptr), MFA_E_SHAPE));
    EXPECT(is(mfa_blockid_tile_summary(nullptr, nullptr, nullptr, nullptr, 1, 8, 8, 128, 32, nullptr, nullptr,
                                       nullptr, nullptr),
              MFA_E_UNSUPPORTED));
    EXPECT(is(mfa_varlen_schedule(nullptr, nullptr, 2, 64, 64, 1, -1, -1, nullptr, nullptr, nullptr, nullptr, 4,
                                  nullptr, nullptr),
              MFA_E_UNSUPPORTED));
    EXPECT(is(mfa_varlen_schedule(nullptr, nullptr, -2, 128, 64, 1, -1, -1, nullptr, nullptr, nullptr, nullptr, 4,
                                  nullptr, nullptr),
              MFA_E_SHAPE));
    int w = 7;
    EXPECT(is(mfa_bsr_validate(nullptr, nullptr, 1, 1, 4, 4, 0, nullptr, nullptr), MFA_E_ARG));
    EXPECT(is(mfa_bsr_validate(nullptr, nullptr, 0, 1, 4, 4, 0, &w, nullptr), MFA_OK) && w == 0);
    EXPECT(is(mfa_bsr_prepare(nullptr, nullptr, 1, 1, 3, 4, 0, 64, 64, 256, 256, 1, nullptr, nullptr, nullptr,
                              nullptr, nullptr),
              MFA_E_SHAPE));
    EXPECT(is(mfa_bsr_prepare(nullptr, nullptr, 1, 1, 1, 20000, 0, 64, 64, 64, 20000 * 64, 1, nullptr, nullptr,
                              nullptr, nullptr, nullptr),
              MFA_E_UNSUPPORTED));
    EXPECT(is(mfa_bsr_from_bitmask(nullptr, 1, 1, 1 << 16, 1 << 16, nullptr, nullptr, 0, nullptr), MFA_E_UNSUPPORTED));
    mfa_predicate p;
    std::memset(&p, 0, sizeof(p));
    p.n_terms = MFA_PRED_MAX_TERMS + 1;
    EXPECT(is(mfa_predicate_tiles(&p, 16, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), MFA_E_ARG));
    p.n_terms = 1;
    p.n_atoms[0] = -1;
    EXPECT(is(mfa_predicate_tiles(&p, 16, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), MFA_E_ARG));
}

static void dispatch_model() {
    const int64_t causal64[3] = {8128, 128, 8128}, causal128[3] = {4032, 128, 4032};
    const int64_t blk64[3] = {15384, 0, 1000}, blk128[3] = {7192, 1000, 0};
    for (int D : {64, 128}) {
        EXPECT(mfa_choose_tile_m(causal64, causal128, 8192, D) == 128);
        EXPECT(mfa_choose_tile_m(blk64, blk128, 8192, D) == 64);
        EXPECT(mfa_choose_tile_m(nullptr, causal128, 8192, D) == 128);
    }
    const int64_t zero[3] = {0, 0, 0};
    EXPECT(mfa_model_tile_time(zero, 0, 128, 128) == 0.0);
    EXPECT(mfa_model_tile_time(nullptr, 10, 128, 128) == 0.0);
    EXPECT(mfa_model_tile_time(causal128, 8192, 128, 64) > mfa_model_tile_time(zero, 8192, 128, 64));
    EXPECT(mfa_choose_dkdv_split(320, 8, 128, 256) == 4);
    EXPECT(mfa_choose_dkdv_split(320, 8, 64, 256) == 8);
    EXPECT(mfa_choose_dkdv_split(1 << 20, 8, 128, 256) == 1);
    EXPECT(mfa_choose_dkdv_split(-5, 8, 128, 256) == 1);
}

static void names_and_thread_local_errors() {
    for (int s = 0; s <= 9; ++s) EXPECT(mfa_status_name((mfa_status)s) != nullptr);
    EXPECT(std::string(mfa_status_name(MFA_OK)) == "MFA_OK");
    // each thread sees its own last error
    std::string a, b;
    std::thread t1([&] {
        mfa_tile_counts(nullptr, -1, nullptr, nullptr);
        a = mfa_last_error();
    });
    t1.join();
    std::thread t2([&] {
        mfa_attn_fwd(nullptr, nullptr, 0.1f, nullptr);
        b = mfa_last_error();
    });
    t2.join();
    EXPECT(!a.empty() && !b.empty() && a != b);
}

int main() {
    attention_validation();
    mask_representation_validation();
    dispatch_model();
    names_and_thread_local_errors();
    if (g_failed) {
        std::fprintf(stderr, "%d host checks failed\n", g_failed);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
