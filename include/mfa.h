/*
 * mfa.h - C ABI of libmfa: masked flash attention for AMD MI355X (gfx950).
 *
 * The attention mask is applied per tile and is never materialised as a dense
 * (S, S) score matrix. Four mask representations feed one fused kernel:
 *
 *   BLOCKID  compact per-token block ids: attend(i, j) = q_valid[i] &
 *            k_valid[j] & (k_blk[j] <= q_blk[i])
 *            ("opentau.policies.flash_attn_cuda", make_att_block_ids /
 *            flash_attn_blockmask);
 *   TILES    a dense (Nq, Nk) bool mask reduced to a coarse tile map, a
 *            32-bit packed fine mask and a per-query-tile ascending list of
 *            non-empty key tiles ("BinFlash" README, section "Efficiently
 *            Dispatching FlashAttention For Partially Filled Attention Masks");
 *   BSR      block-sparse rows block_indptr / block_indices, optionally causal
 *            inside each block ("flashinfer.attention.prims_ts.
 *            block_sparse_attention", Parameters);
 *   VARLEN   sequences packed along the token axis with cumulative lengths,
 *            causal and/or sliding window on sequence-local positions
 *            ("tensorplay.nn.attention.varlen", Packed layout).
 *
 * Conventions for every call:
 *  - Every pointer is device memory unless the comment says "host". All
 *    buffers, outputs included, are owned by the caller; the library never
 *    allocates device memory.
 *  - Arguments are validated on the host before anything is launched. A
 *    device pointer check uses hipPointerGetAttributes; a host pointer where
 *    device memory is required gives MFA_E_NOT_DEVICE (the pages raise when
 *    given CPU tensors or tensors on different devices).
 *  - Calls are asynchronous on `stream` (0 = the null stream) except
 *    mfa_bsr_validate, which copies the BSR arrays to the host and waits.
 *  - Every call returns an mfa_status and never aborts. On failure a
 *    thread-local message is available from mfa_last_error().
 *  - Tile kinds: 0 empty (skipped), 1 partial (per-element mask), 2 full (no
 *    mask load). Out-of-range positions of a ragged edge tile count as not
 *    allowed, so such a tile is never "full".
 *  - A query row with no allowed key gets output +0 and log-sum-exp -inf.
 */
#ifndef MFA_H
#define MFA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mfa_status {
    MFA_OK = 0,
    MFA_E_ARG = 1,          /* null pointer or invalid scalar argument            */
    MFA_E_SHAPE = 2,        /* sizes inconsistent with each other                 */
    MFA_E_DTYPE = 3,        /* dtype code not recognised                          */
    MFA_E_UNSUPPORTED = 4,  /* well-formed but not built (head dim, tile size)    */
    MFA_E_NOT_DEVICE = 5,   /* pointer is not device memory of the current device */
    MFA_E_NONCANONICAL = 6, /* BSR rows not canonical                             */
    MFA_E_HIP = 7,          /* a HIP runtime call failed                          */
    MFA_E_NO_DEVICE = 8     /* no usable gfx950 device                            */
} mfa_status;

#define MFA_TILE_EMPTY 0
#define MFA_TILE_PARTIAL 1
#define MFA_TILE_FULL 2
/* Block id of prepended cross-attention key columns ("always attended,
 * subject to padding"): the most negative int32. */
#define MFA_BLK_CROSS INT32_MIN

/* 1 if a gfx950 device is present and the kernels in this library can run on
 * it, else 0 (the reason is then in mfa_last_error()). The opentau page's
 * is_available() / load_error() pair. */
int mfa_is_available(void);

/* Message of the last failed call on this thread; "" if none. Valid until the
 * next failing call on the same thread. */
const char* mfa_last_error(void);

/* Short name of a status code ("MFA_E_SHAPE", ...). */
const char* mfa_status_name(mfa_status s);

/* ------------------------------------------------------------------------ */
/* Mask representations                                                      */
/* ------------------------------------------------------------------------ */

/* Compact block ids from pad/att masks ("opentau.policies.flash_attn_cuda",
 * make_att_block_ids).
 *   pad        (B, N) u8, nonzero = real token
 *   att        (B, N) i32, nonzero opens a new attention block, 0 continues
 *   n_cross    number of prepended cross-attention key columns (>= 0)
 *   cross_pad  (B, n_cross) u8, required iff n_cross > 0, else must be NULL
 * Outputs:
 *   q_blk    (B, N) i32: inclusive running count of openers at or before i
 *   k_blk    (B, n_cross + N) i32: n_cross x MFA_BLK_CROSS, then q_blk
 *   q_valid  (B, N) u8 0/1 = pad != 0
 *   k_valid  (B, n_cross + N) u8 0/1 = [cross_pad ; pad] != 0 */
mfa_status mfa_make_block_ids(const uint8_t* pad, const int32_t* att, int B, int N,
                              int n_cross, const uint8_t* cross_pad,
                              int32_t* q_blk, int32_t* k_blk,
                              uint8_t* q_valid, uint8_t* k_valid, hipStream_t stream);

/* Per-tile summaries of a block-id representation, used by the attention
 * kernel to classify tiles exactly (same page: the mask is rebuilt inside the
 * kernel from the ids). Query tiles are BM tokens, key tiles BN tokens.
 *   qsum  (B, ceil(Sq/BM), 4) i32 and ksum (B, ceil(Sk/BN), 4) i32, each row
 *         {min id over valid tokens (INT32_MAX if none), max id over valid
 *         tokens (INT32_MIN if none), any valid (0/1), all BM (or BN)
 *         positions in range and valid (0/1)}
 *   kv_bits (B, ceil(Sk/32)) u32, bit b of word w = k_valid[32w+b], pad bits 0
 *         (the flashinfer page's kv_valid_bits layout).
 * A tile is empty iff no valid query, no valid key, or kmin > qmax; full iff
 * all queries and keys valid and kmax <= qmin; else partial. */
mfa_status mfa_blockid_tile_summary(const int32_t* q_blk, const int32_t* k_blk,
                                    const uint8_t* q_valid, const uint8_t* k_valid,
                                    int B, int Sq, int Sk, int BM, int BN,
                                    int32_t* qsum, int32_t* ksum, uint32_t* kv_bits,
                                    hipStream_t stream);

/* Dense (Nq, Nk) bool mask -> coarse tile map + packed fine mask + sorted
 * non-empty key-tile lists ("BinFlash" README, "Efficiently Dispatching ...").
 *   mask       (Nq, Nk) u8 row-major, nonzero = attend (True = attend)
 * Outputs:
 *   tile_kind  (ceil(Nq/BM), ceil(Nk/BN)) u8 kinds
 *   fine_bits  (Nq, ceil(Nk/32)) u32, bit b of word w = mask[i, 32w+b] != 0,
 *              pad bits 0
 *   row_ptr    (ceil(Nq/BM) + 1) i32 CSR offsets, row_ptr[0] = 0
 *   col_idx    (nnz) i32 non-empty key tiles, ascending within each row
 *   col_kind   (nnz) u8 kinds of those tiles (1 or 2)
 * col_idx / col_kind must hold nnz entries; nnz <= ceil(Nq/BM)*ceil(Nk/BN)
 * always suffices. BM is 128 or 64 and BN 64 (the attention kernels' tiles);
 * give the attention calls the same BM as mfa_mask.tile_m. */
mfa_status mfa_compact_dense_mask(const uint8_t* mask, int Nq, int Nk, int BM, int BN,
                                  uint8_t* tile_kind, uint32_t* fine_bits,
                                  int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind,
                                  hipStream_t stream);

/* Predicate masks (tensorplay omni_attention, "Block masks": a mask_mod
 * predicate of (b, h, q_idx, kv_idx), composed with and_masks / or_masks;
 * noop_mask allows everything). Here a predicate is an OR of up to
 * MFA_PRED_MAX_TERMS conjunctions, each an AND of up to MFA_PRED_MAX_ATOMS
 * linear atoms   a*q_idx + b*kv_idx + c >= 0   (int64 arithmetic, 0-based
 * positions, the same for every batch entry and head). Examples:
 *   causal (q_idx >= kv_idx)             {1, -1, 0}
 *   at most W past keys (q - kv < W)     {-1, 1, W - 1}
 *   a prefix of P keys (kv < P)          {0, -1, P - 1}
 * A conjunction with no atoms is always true (noop_mask); a predicate with
 * no conjunctions allows nothing. */
#define MFA_PRED_MAX_TERMS 4
#define MFA_PRED_MAX_ATOMS 4
typedef struct mfa_pred_atom {
    int64_t a, b, c;
} mfa_pred_atom;
typedef struct mfa_predicate {
    int n_terms;
    int n_atoms[MFA_PRED_MAX_TERMS];
    mfa_pred_atom atoms[MFA_PRED_MAX_TERMS][MFA_PRED_MAX_ATOMS];
} mfa_predicate;

/* Density-aware dispatch between 128-row and 64-row dense-mask tiles
 * (BinFlash README, "Efficiently Dispatching ...": the dispatcher picks the
 * tiling from statistics of the coarse block mask).
 * mfa_tile_map_coarsen: the 128-row tile map and its CSR (outputs as in
 *   mfa_compact_dense_mask with BM = 128) from a 64-row map kind64
 *   (ceil(Nq/64), ceil(Nk/64)) of the same mask, without reading the mask
 *   again; the fine bits are shared. Asynchronous.
 * mfa_tile_counts: counts[0..2] (device int64) = empty, partial and full
 *   tiles among the n kinds of a tile map. Asynchronous.
 * mfa_model_tile_time / mfa_choose_tile_m (host only, no device calls): the
 *   modelled forward time of a map with those counts at head dim D (64 or
 *   128; setup per query tile plus a cost per partial and per full tile,
 *   fitted to MI355X forward times), and the tile height to use: 64 only
 *   when its modelled time is at least 5% below the 128-row one. */
mfa_status mfa_tile_map_coarsen(const uint8_t* kind64, int Nq, int Nk, uint8_t* kind128,
                                int32_t* row_ptr, int32_t* col_idx, uint8_t* col_kind,
                                hipStream_t stream);
mfa_status mfa_tile_counts(const uint8_t* tile_kind, int64_t n, int64_t* counts, hipStream_t stream);
double mfa_model_tile_time(const int64_t counts[3], int Nq, int tile_m, int D);
int mfa_choose_tile_m(const int64_t counts64[3], const int64_t counts128[3], int Nq, int D);

/* The tile representation of a predicate mask over an (Nq, Nk) grid: the
 * same outputs, layout and meaning as mfa_compact_dense_mask (BM = 128,
 * BN = 64), computed by evaluating the predicate per element on the GPU, so
 * that no dense mask exists in memory. pred is a host pointer, read before
 * the call returns. Errors: MFA_E_ARG for counts outside [0, max] or
 * negative sizes, MFA_E_NO_DEVICE / MFA_E_HIP as elsewhere. */
mfa_status mfa_predicate_tiles(const mfa_predicate* pred, int Nq, int Nk, uint8_t* tile_kind,
                               uint32_t* fine_bits, int32_t* row_ptr, int32_t* col_idx,
                               uint8_t* col_kind, hipStream_t stream);

/* Synchronous inspection of BSR routing arrays (flashinfer
 * block_sparse_attention, description: the BSR inputs are checked on the
 * host for canonical rows, and the widest row is found).
 *   indptr   (B, Hkv, nQb + 1) i32: row (b, h, r) lists
 *            indices[indptr[b,h,r] : indptr[b,h,r+1]] (offsets into one flat
 *            array)
 *   indices  (nnz) i32 KV-block ids
 * Canonical: offsets non-decreasing within [0, nnz]; ids strictly ascending
 * within a row and in [0, nKb). Returns MFA_E_NONCANONICAL otherwise.
 *   max_row_width  host out: widest row. Waits for `stream`. */
mfa_status mfa_bsr_validate(const int32_t* indptr, const int32_t* indices, int B, int Hkv,
                            int nQb, int nKb, int64_t nnz, int* max_row_width,
                            hipStream_t stream);

/* Kinds of the listed blocks and the column-major copy used by the dK/dV
 * pass. Rows must be canonical (see mfa_bsr_validate).
 *   causal     1 = token-level j <= i inside the blocks (mask_type causal)
 *   kv_valid_bits  optional (B, ceil(Skv/32)) u32 token-validity bitmap
 *              (flashinfer block_sparse_attention, Parameters), LSB-first;
 *              NULL = every key valid. A block with no valid key becomes
 *              empty and a full block with an invalid key partial; pass the
 *              same bitmap as mfa_mask.kv_bits to the attention calls.
 *   col_kind   (nnz) u8: kind of entry e given Sq, Skv, block sizes, causal
 *   csc_ptr    (B, Hkv, nKb + 1) i32: for (b, h) the segment starts at
 *              indptr[b,h,0]; csc_idx[csc_ptr[b,h,c] : csc_ptr[b,h,c+1]] lists
 *              the query-block rows that reference block c, ascending
 *   csc_idx    (nnz) i32 */
mfa_status mfa_bsr_prepare(const int32_t* indptr, const int32_t* indices, int B, int Hkv,
                           int nQb, int nKb, int64_t nnz, int q_block, int kv_block,
                           int Sq, int Skv, int causal, const uint32_t* kv_valid_bits,
                           uint8_t* col_kind, int32_t* csc_ptr, int32_t* csc_idx,
                           hipStream_t stream);

/* BSR rows from the bitmask sparse format (flashinfer
 * block_sparse_attention, Parameters: exact_block_bits with sparse_format
 * bitmask): bit c (LSB-first) of row (b, h, r) selects KV block c.
 *   bits     (B, Hkv, nQb, ceil(nKb/32)) u32 device
 *   indptr   (B, Hkv, nQb + 1) i32 device out: one running offset over all
 *            rows, as mfa_bsr_validate expects
 *   indices  (cap) i32 device out: ascending block ids per row; entries
 *            past cap are not written (cap >= B*Hkv*nQb*nKb always holds
 *            them; indptr[B,Hkv,nQb] is the count either way)
 * Asynchronous; bits past nKb in a row's last word are ignored. */
mfa_status mfa_bsr_from_bitmask(const uint32_t* bits, int B, int Hkv, int nQb, int nKb,
                                int32_t* indptr, int32_t* indices, int64_t cap,
                                hipStream_t stream);

/* Variable-length packing and schedule ("tensorplay.nn.attention.varlen",
 * Packed layout).
 *   len_q, len_k  (nseq) i32 sequence lengths (>= 0)
 * Outputs:
 *   cu_q, cu_k    (nseq + 1) i32 cumulative lengths starting at 0
 *   max_len       (2) i32: {max len_q, max len_k}
 *   work          (work_cap, 2) i32 query tiles (seq, q0), q0 = 0, BM, ...,
 *                 ordered by descending number of BN-key tiles the tile
 *                 visits under the window, ties by ascending (seq, q0);
 *                 unused entries are set to (-1, -1)
 *   n_work        (1) i32 number of tiles written
 * Window (on sequence-local positions i, j): causal -> j <= i; left >= 0 ->
 * i - j <= left; right >= 0 -> j - i <= right; -1 leaves that side open.
 * work_cap must be >= sum_s ceil(len_q[s]/BM); BM = 128, BN = 64. If the
 * tiles do not fit, n_work is set to -1 and every work entry to (-1, -1).
 * The order uses exact costs at every length. Tiles visiting 4096 or more
 * key tiles (over 262,080 keys) are ranked in groups of equal cost >> 12;
 * if one such group holds more than 16,384 tiles, n_work is set to -2 and
 * every work entry to (-1, -1). Asynchronous. */
mfa_status mfa_varlen_schedule(const int32_t* len_q, const int32_t* len_k, int nseq, int BM, int BN,
                               int causal, int win_left, int win_right,
                               int32_t* cu_q, int32_t* cu_k, int32_t* max_len,
                               int32_t* work, int work_cap, int32_t* n_work,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

typedef enum mfa_dtype {
    MFA_BF16 = 0,  /* bf16 in/out, bf16 MFMA, fp32 softmax state            */
    MFA_F32 = 1    /* fp32 in/out and fp32 arithmetic: test mode            */
} mfa_dtype;

typedef enum mfa_mask_kind {
    MFA_MASK_NONE = 0,     /* every in-range key attended (plain SDPA)        */
    MFA_MASK_BLOCKID = 1,
    MFA_MASK_TILES = 2,
    MFA_MASK_BSR = 3,
    MFA_MASK_VARLEN = 4
} mfa_mask_kind;

/* q (B, Sq, Hq, D), k and v (B, Sk, Hkv, D), out like q, addressed through
 * element strides {batch, seq, head}; the D axis is contiguous. This covers
 * (B, S, H, D) (opentau, flashinfer) and (B, H, S, D) (BinFlash) tensors.
 * Hq % Hkv == 0; query head hq reads key/value head hq / (Hq / Hkv).
 * VARLEN: q is (Tq, Hq, D) with B = 1, Sq = Tq, Sk = Tk and batch stride 0.
 * lse: NULL (inference) or fp32 (B, Hq, Sq) contiguous; natural-log
 * log-sum-exp of scale * q.k over allowed keys, -inf for empty rows. */
typedef struct mfa_attn_args {
    int dtype;             /* mfa_dtype */
    int B, Sq, Sk, Hq, Hkv, D;
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int64_t q_stride[3];
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    /* Optional (Hq) fp32 device array, or NULL: adds slope[h] * (kv_idx -
     * q_idx) to every scaled score of query head h before the mask and the
     * softmax, the distance-decay score_mod of tensorplay omni_attention
     * (intro) with a slope per head (slopes of 1 give that example exactly).
     * Positions are indices along Sq and Sk (local to the sequence for
     * VARLEN). The log-sum-exp includes the bias. Read by the forward and
     * both backward passes, which must get the forward's slopes. Slopes must
     * be finite. */
    const float* alibi_slopes;
    /* Soft cap, or 0 for none: every score x (the scaled score plus the bias
     * above, if any) becomes softcap * tanh(x / softcap) before the mask and
     * the softmax, the soft-cap score_mod of tensorplay omni_attention
     * (intro). The log-sum-exp is of the capped scores, and the backward
     * passes (which must get the forward's value) take its derivative
     * 1 - tanh^2(x / softcap) into dS. Must be finite and >= 0. */
    float softcap;
} mfa_attn_args;

/* Mask representation for one attention call. Only the fields of `kind` are
 * read; the rest may be zero. */
typedef struct mfa_mask {
    int kind;              /* mfa_mask_kind */
    /* BLOCKID: outputs of mfa_make_block_ids (or any ids) plus the summaries
     * of mfa_blockid_tile_summary with BM = 128, BN = 64. */
    const int32_t* q_blk;
    const int32_t* k_blk;
    const uint8_t* q_valid;
    const uint8_t* k_valid;
    const int32_t* qsum;
    const int32_t* ksum;
    /* BLOCKID: key validity bits from the summary call. BSR: the optional
     * kv_valid_bits token bitmap (B, ceil(Sk/32)) u32 (NULL = all valid),
     * the same one given to mfa_bsr_prepare. */
    const uint32_t* kv_bits;
    /* TILES: outputs of mfa_compact_dense_mask for an (Sq, Sk) mask shared
     * by every batch entry and head. */
    const uint8_t* tile_kind;
    const uint32_t* fine_bits;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint8_t* col_kind;
    /* BSR: per (b, kv head) rows; q_block = kv_block = 64 are built.
     * col_kind from mfa_bsr_prepare; csc_ptr / csc_idx are read by the
     * dK/dV backward pass only. */
    const int32_t* indptr;
    const int32_t* indices;
    const uint8_t* bsr_kind;
    const int32_t* csc_ptr;
    const int32_t* csc_idx;
    int q_block;
    int kv_block;
    /* VARLEN: outputs of mfa_varlen_schedule. max_q / max_k are the largest
     * sequence lengths as the caller states them; a sequence longer than
     * stated is an error: its output rows are written as NaN and *err is set
     * to 1 (err may be NULL). */
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* work;
    int work_cap;
    int max_q;
    int max_k;
    int32_t* err;
    /* BSR and VARLEN */
    int causal;
    int win_left;          /* VARLEN only; -1 = open */
    int win_right;         /* VARLEN only; -1 = open */
    int nseq;              /* VARLEN: number of sequences (cu_q holds nseq + 1
                              entries); read by the dK/dV backward pass */
    /* VARLEN options (tensorplay varlen, intro), NULL / 0 when unused:
     * seqused_k    (nseq) i32: only the first min(seqused_k[s], len_k[s])
     *              keys of sequence s are attended (values < 0 count as 0);
     *              the other keys' dK/dV rows are written as zeros.
     * block_table  (nseq, max_pages) i32: paged k / v. k and v are then page
     *              pools (n_pages, page_size, Hkv, D) addressed through
     *              k_stride / v_stride = (page, row, head) element strides,
     *              and key j of sequence s sits at row j % page_size of page
     *              block_table[s, j / page_size]. page_size must be a
     *              positive multiple of 64. cu_k still gives the key lengths.
     *              A sequence needing more than max_pages pages, or whose
     *              pages include an id outside [0, n_pages), gets NaN rows
     *              and sets *err. In the backward, dk / dv are page pools
     *              like k / v (their strides likewise (page, row, head)):
     *              key j's gradient rows go to the same (page, row) as its
     *              k / v rows. Keys whose page lies past the table row or
     *              outside the pool are not written, nor are pages no key
     *              maps to; pages must not hold keys of two sequences
     *              (their rows would be written twice, in no fixed order). */
    const int32_t* seqused_k;
    const int32_t* block_table;
    int max_pages;
    int page_size;
    int n_pages;
    /* TILES: query rows per tile of the map (the BM it was compacted with):
     * 128 (or 0) or 64. 64-row maps run 2-wave workgroups. */
    int tile_m;
} mfa_mask;

/* Fused masked attention forward: out = softmax(scale q k^T + bias + mask) v
 * per (batch, head), with log-sum-exp. scale is explicit (callers usually
 * pass D^-0.5) and must be finite and positive (MFA_E_ARG otherwise). Head
 * dims 64 and 128 are built; others give MFA_E_UNSUPPORTED, and so does a
 * sequence stride of 2^23 elements or more (bf16; 2^22 for fp32) in any
 * tensor, here and in the backward: 128 rows must span under 2 GiB. */
mfa_status mfa_attn_fwd(const mfa_attn_args* args, const mfa_mask* mask, float scale,
                        hipStream_t stream);

/* Backward, split as in the BinFlash method ("Efficiently Dispatching ...":
 * dK/dV over key blocks, dQ over query blocks, with the same dispatch as the
 * forward): a preprocessing pass, dK/dV over 64-key blocks, then dQ over
 * query tiles. fwd holds q, k, v, out and lse (the forward's outputs; lse
 * required). dout/dq/dk/dv use the same stride convention as fwd. delta
 * (B, Hq, Sq) fp32 contiguous ((Hq, T) for VARLEN) is written by the
 * preprocess pass (delta_i = sum_d dout_id * out_id) and read by the others.
 * With no query rows (Sq = 0) and keys present, the dK/dV pass writes
 * dk = dv = 0 (q, lse, out and dout are then not read).
 * D = 128 or 64, every mask kind. dtype MFA_BF16: bf16 tensors, MFMA
 * passes. dtype MFA_F32 (test mode): fp32 q, k, v, out, dout, dq, dk, dv,
 * scalar fp32 passes that walk the same block lists with the same mask
 * predicates, so the masking of both passes can be checked at 1e-4.
 * Per kind the passes read:
 *   NONE     nothing;
 *   TILES    dQ: row_ptr, col_idx, col_kind, fine_bits; dK/dV: tile_kind,
 *            fine_bits;
 *   BLOCKID  q_blk, k_blk, q_valid, qsum, ksum, kv_bits (summaries at
 *            BM = 128, BN = 64);
 *   BSR      dQ: indptr, indices, bsr_kind; dK/dV: csc_ptr, csc_idx
 *            (q_block = kv_block = 64);
 *   VARLEN   dQ: cu_q, cu_k, work; dK/dV: cu_q, cu_k and nseq. Key blocks
 *            past max_k are not visited: a sequence longer than max_k or
 *            max_q gets NaN gradients in the blocks that are and sets *err. */
typedef struct mfa_attn_bwd_args {
    mfa_attn_args fwd;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;
    int64_t do_stride[3];
    int64_t dq_stride[3];
    int64_t dk_stride[3];
    int64_t dv_stride[3];
    void* workspace;         /* optional device scratch of the dK/dV pass (below); may be NULL */
    int64_t workspace_bytes; /* its size in bytes */
} mfa_attn_bwd_args;

mfa_status mfa_attn_bwd_preprocess(const mfa_attn_bwd_args* args, hipStream_t stream);
mfa_status mfa_attn_bwd_dkdv(const mfa_attn_bwd_args* args, const mfa_mask* mask, float scale,
                             hipStream_t stream);
mfa_status mfa_attn_bwd_dq(const mfa_attn_bwd_args* args, const mfa_mask* mask, float scale,
                           hipStream_t stream);

/* Query-head split of the dK/dV pass. dK and dV of a key block sum over the
 * query rows of every query head of its GQA group (Hq / Hkv heads). When the
 * key blocks alone (B * Hkv * ceil(Sk / 64)) give the device too few
 * workgroups, the pass splits the group's heads over S workgroups per key
 * block; they write fp32 partial sums, and a reduce pass adds the S sums in
 * order (so the result does not depend on scheduling) and writes dk / dv.
 * The sums take S * 2 * B * Sk * Hkv * D * 4 bytes of device memory, which
 * the caller passes as args->workspace / workspace_bytes (16-byte aligned,
 * device memory on the current device, owned by the caller, not to be used
 * by anything else until the pass has run on the stream). With less
 * workspace (or NULL) the pass takes the largest split that fits, down to
 * S = 1, which needs none. bf16 only: the fp32 test mode and VARLEN masks
 * never split.
 * mfa_attn_bwd_dkdv_workspace: *bytes = the workspace of the preferred
 * split on the current device, *splits = that split (1: none; bytes 0).
 * Validation errors as for mfa_attn_bwd_dkdv; MFA_E_NO_DEVICE without a
 * gfx950 device. */
mfa_status mfa_attn_bwd_dkdv_workspace(const mfa_attn_bwd_args* args, const mfa_mask* mask, int64_t* bytes,
                                       int* splits);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the dK/dV
 * pass of mfa_attn_bwd_dkdv with the head split's partial sums in a static
 * device scratch array of the library (mfa_bwd_scratch_bytes(), 96 MiB, held
 * by each device the library runs on until the process ends) instead of a
 * workspace; args->workspace is ignored. It takes the preferred split
 * (mfa_attn_bwd_dkdv_workspace) and fails with MFA_E_UNSUPPORTED, before
 * any launch, when that split's sums need more than the scratch holds. It
 * calls no allocator (the scratch's device address is looked up once per
 * device, on the first call there). All calls on one device share the
 * scratch: calls that overlap on one device (on different streams, or from
 * several threads without ordering) race and give wrong gradients. The
 * results equal mfa_attn_bwd_dkdv's with a workspace of the preferred size. */
mfa_status mfa_attn_bwd_dkdv_noalloc(const mfa_attn_bwd_args* args, const mfa_mask* mask, float scale,
                                     hipStream_t stream);
int64_t mfa_bwd_scratch_bytes(void);

/* The split model (host only, no device needed): the smallest divisor S > 1
 * of group with key_blocks * S >= 2 * n_cu * W, where W = 2 workgroups per
 * CU at head_dim 128 and 4 at 64 (the dK/dV workgroups a CU holds at once),
 * or group when none reaches it; 1 when group <= 1, key_blocks <= 0, or
 * key_blocks alone reaches it. */
int mfa_choose_dkdv_split(int64_t key_blocks, int group, int head_dim, int n_cu);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H */
