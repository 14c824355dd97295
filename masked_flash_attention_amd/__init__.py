"""masked_flash_attention_amd: masked flash attention on AMD MI355X (gfx950).

A thin Python binding over libmfa's C ABI (include/mfa.h). torch supplies
device memory and the current stream; every step of the computation runs in
the library's HIP kernels. The library must be built first
(``python -m masked_flash_attention_amd.build``); nothing here falls back to
another implementation.

Entry points mirror the C calls: ``make_block_ids``, ``blockid_tile_summary``,
``compact_dense_mask``, ``bsr_validate``, ``bsr_prepare``, ``varlen_schedule``,
``attn_fwd``, ``attn_bwd_preprocess``, ``attn_bwd_dkdv``, ``attn_bwd_dq``. Mask
representations are passed to the attention calls as ``MaskRep`` objects.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field

import torch

from . import _ffi
from ._ffi import MfaError

__all__ = ["MfaError", "MaskRep", "is_available", "load_error", "make_block_ids", "blockid_tile_summary",
           "compact_dense_mask", "bsr_validate", "bsr_prepare", "varlen_schedule", "attn_fwd",
           "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd", "TILE_M", "TILE_N"]

TILE_M, TILE_N = 128, 64  # query rows x key columns of one attention tile


def _lib():
    return _ffi.load()


def is_available() -> bool:
    """True if libmfa is built and a gfx950 device can run it."""
    try:
        return bool(_lib().mfa_is_available())
    except ImportError:
        return False


def load_error():
    """Why the library is unavailable (build/load error or device message), else None."""
    try:
        lib = _lib()
    except ImportError as e:
        return str(e)
    if lib.mfa_is_available():
        return None
    return lib.mfa_last_error().decode()


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _u8(t):
    if t.dtype == torch.uint8:
        return t
    if t.dtype == torch.bool:
        return t.view(torch.uint8)  # same bytes (0/1), no copy
    return t.to(torch.uint8)


def _i32(t):
    return t if t.dtype == torch.int32 else t.to(torch.int32)


def _cdiv(a, b):
    return -(-a // b)


# ---------------------------------------------------------------------------
# mask representations
# ---------------------------------------------------------------------------

def make_block_ids(pad_masks, att_masks, n_cross_att_tokens=None, cross_att_pad_masks=None):
    """(q_blk, k_blk, q_valid, k_valid) from pad/att masks (mfa_make_block_ids).

    q_blk int32 (B, N); k_blk int32 (B, Nc + N); q_valid / k_valid bool.
    """
    if (n_cross_att_tokens is None) != (cross_att_pad_masks is None):
        raise ValueError("cross_att_pad_masks is required iff n_cross_att_tokens is set")
    pad = _u8(pad_masks).contiguous()
    att = _i32(att_masks).contiguous()
    B, N = pad.shape
    nc = int(n_cross_att_tokens or 0)
    cross = None if cross_att_pad_masks is None else _u8(cross_att_pad_masks).contiguous()
    dev = pad.device
    q_blk = torch.empty(B, N, dtype=torch.int32, device=dev)
    k_blk = torch.empty(B, nc + N, dtype=torch.int32, device=dev)
    q_valid = torch.empty(B, N, dtype=torch.uint8, device=dev)
    k_valid = torch.empty(B, nc + N, dtype=torch.uint8, device=dev)
    _ffi.check(_lib().mfa_make_block_ids(_p(pad), _p(att), B, N, nc, _p(cross), _p(q_blk), _p(k_blk),
                                         _p(q_valid), _p(k_valid), _stream()))
    return q_blk, k_blk, q_valid.view(torch.bool), k_valid.view(torch.bool)


def blockid_tile_summary(q_blk, k_blk, q_valid, k_valid, BM=TILE_M, BN=TILE_N):
    """(qsum (B, nQt, 4), ksum (B, nKt, 4), kv_bits (B, ceil(Sk/32))) (mfa_blockid_tile_summary)."""
    q_blk, k_blk = _i32(q_blk).contiguous(), _i32(k_blk).contiguous()
    q_valid, k_valid = _u8(q_valid).contiguous(), _u8(k_valid).contiguous()
    B, Sq = q_blk.shape
    Sk = k_blk.shape[1]
    dev = q_blk.device
    qsum = torch.empty(B, _cdiv(Sq, BM), 4, dtype=torch.int32, device=dev)
    ksum = torch.empty(B, _cdiv(Sk, BN), 4, dtype=torch.int32, device=dev)
    kv_bits = torch.empty(B, _cdiv(Sk, 32), dtype=torch.int32, device=dev)
    _ffi.check(_lib().mfa_blockid_tile_summary(_p(q_blk), _p(k_blk), _p(q_valid), _p(k_valid), B, Sq, Sk, BM, BN,
                                               _p(qsum), _p(ksum), _p(kv_bits), _stream()))
    return qsum, ksum, kv_bits


def compact_dense_mask(mask, BM=TILE_M, BN=TILE_N):
    """Tile map, packed fine bits and CSR of non-empty tiles (mfa_compact_dense_mask).

    col_idx / col_kind are allocated at full capacity (nQt * nKt); the first
    row_ptr[-1] entries are meaningful (reading that count would need a sync).
    """
    m = _u8(mask).contiguous()
    Nq, Nk = m.shape
    nQt, nKt = _cdiv(Nq, BM), _cdiv(Nk, BN)
    dev = m.device
    out = {
        "tile_kind": torch.empty(nQt, nKt, dtype=torch.uint8, device=dev),
        "fine_bits": torch.empty(Nq, _cdiv(Nk, 32), dtype=torch.int32, device=dev),
        "row_ptr": torch.empty(nQt + 1, dtype=torch.int32, device=dev),
        "col_idx": torch.empty(max(1, nQt * nKt), dtype=torch.int32, device=dev),
        "col_kind": torch.empty(max(1, nQt * nKt), dtype=torch.uint8, device=dev),
    }
    _ffi.check(_lib().mfa_compact_dense_mask(_p(m), Nq, Nk, BM, BN, _p(out["tile_kind"]), _p(out["fine_bits"]),
                                             _p(out["row_ptr"]), _p(out["col_idx"]), _p(out["col_kind"]),
                                             _stream()))
    out["tile_m"] = BM
    return out


class Pred:
    """A mask predicate of (q_idx, kv_idx) in disjunctive form: a tuple of
    conjunctions, each a tuple of linear atoms (a, b, c) meaning
    a*q_idx + b*kv_idx + c >= 0. and_/or_ compose like and_masks / or_masks;
    noop() allows everything (one empty conjunction), never() nothing."""

    def __init__(self, terms):
        self.terms = tuple(tuple(tuple(int(x) for x in atom) for atom in term) for term in terms)

    @staticmethod
    def atom(a, b, c):
        return Pred(((((a, b, c),),)))

    @staticmethod
    def causal():
        return Pred.atom(1, -1, 0)                 # q_idx >= kv_idx

    @staticmethod
    def past_window(w):
        return Pred.atom(-1, 1, int(w) - 1)        # q_idx - kv_idx < w

    @staticmethod
    def prefix(p):
        return Pred.atom(0, -1, int(p) - 1)        # kv_idx < p

    @staticmethod
    def noop():
        return Pred(((),))

    @staticmethod
    def never():
        return Pred(())

    def and_(self, other):
        return Pred(tuple(x + y for x in self.terms for y in other.terms))

    def or_(self, other):
        return Pred(self.terms + other.terms)

    def to_c(self):
        if len(self.terms) > _ffi.PRED_MAX_TERMS or any(len(t) > _ffi.PRED_MAX_ATOMS for t in self.terms):
            raise ValueError(f"at most {_ffi.PRED_MAX_TERMS} conjunctions of {_ffi.PRED_MAX_ATOMS} atoms")
        p = _ffi.Predicate()
        p.n_terms = len(self.terms)
        for i, term in enumerate(self.terms):
            p.n_atoms[i] = len(term)
            for j, (a, b, c) in enumerate(term):
                p.atoms[i][j].a, p.atoms[i][j].b, p.atoms[i][j].c = a, b, c
        return p


def predicate_tiles(pred: Pred, Nq, Nk, device="cuda", BM=TILE_M, BN=TILE_N):
    """Tile map, packed fine bits and CSR of a predicate mask (mfa_predicate_tiles);
    the same outputs as compact_dense_mask, with no dense mask built."""
    nQt, nKt = _cdiv(Nq, BM), _cdiv(Nk, BN)
    out = {
        "tile_kind": torch.empty(nQt, nKt, dtype=torch.uint8, device=device),
        "fine_bits": torch.empty(Nq, _cdiv(Nk, 32), dtype=torch.int32, device=device),
        "row_ptr": torch.empty(nQt + 1, dtype=torch.int32, device=device),
        "col_idx": torch.empty(max(1, nQt * nKt), dtype=torch.int32, device=device),
        "col_kind": torch.empty(max(1, nQt * nKt), dtype=torch.uint8, device=device),
    }
    cp = pred.to_c()
    _ffi.check(_lib().mfa_predicate_tiles(C.byref(cp), Nq, Nk, _p(out["tile_kind"]), _p(out["fine_bits"]),
                                          _p(out["row_ptr"]), _p(out["col_idx"]), _p(out["col_kind"]), _stream()))
    return out


def bsr_validate(block_indptr, block_indices, n_kv_blocks):
    """Synchronously check canonical BSR rows; return the widest row (mfa_bsr_validate)."""
    ip, ix = _i32(block_indptr).contiguous(), _i32(block_indices).contiguous()
    B, H, R1 = ip.shape
    w = C.c_int(0)
    _ffi.check(_lib().mfa_bsr_validate(_p(ip), _p(ix), B, H, R1 - 1, n_kv_blocks, ix.numel(), C.byref(w), _stream()))
    return w.value


def bsr_prepare(block_indptr, block_indices, q_block, kv_block, Sq, Skv, causal, kv_valid_bits=None):
    """(col_kind (nnz,) u8, csc_ptr (B, H, nKb+1), csc_idx (nnz,)) (mfa_bsr_prepare).

    kv_valid_bits: optional (B, ceil(Skv/32)) int32/uint32 token-validity
    bitmap; give the same one to MaskRep.bsr."""
    ip, ix = _i32(block_indptr).contiguous(), _i32(block_indices).contiguous()
    B, H, R1 = ip.shape
    nKb = _cdiv(Skv, kv_block)
    nnz = ix.numel()
    dev = ip.device
    col_kind = torch.empty(max(1, nnz), dtype=torch.uint8, device=dev)
    csc_ptr = torch.empty(B, H, nKb + 1, dtype=torch.int32, device=dev)
    csc_idx = torch.empty(max(1, nnz), dtype=torch.int32, device=dev)
    kvb = None if kv_valid_bits is None else _kv_bits(kv_valid_bits, B, Skv)
    _ffi.check(_lib().mfa_bsr_prepare(_p(ip), _p(ix), B, H, R1 - 1, nKb, nnz, q_block, kv_block, Sq, Skv,
                                      int(bool(causal)), None if kvb is None else _p(kvb), _p(col_kind),
                                      _p(csc_ptr), _p(csc_idx), _stream()))
    return col_kind[:nnz], csc_ptr, csc_idx[:nnz]


def tile_counts(tile_kind):
    """(empty, partial, full) tile counts of a tile map, as a device int64 tensor (mfa_tile_counts)."""
    k = tile_kind.contiguous()
    out = torch.empty(3, dtype=torch.int64, device=k.device)
    _ffi.check(_lib().mfa_tile_counts(_p(k), k.numel(), _p(out), _stream()))
    return out


def coarsen_tile_map(compacted64, Nq, Nk):
    """128-row tile map + CSR from a 64-row compaction (mfa_tile_map_coarsen); shares its fine bits."""
    nQt, nKt = _cdiv(Nq, 128), _cdiv(Nk, 64)
    dev = compacted64["tile_kind"].device
    out = {
        "tile_kind": torch.empty(nQt, nKt, dtype=torch.uint8, device=dev),
        "fine_bits": compacted64["fine_bits"],
        "row_ptr": torch.empty(nQt + 1, dtype=torch.int32, device=dev),
        "col_idx": torch.empty(max(1, nQt * nKt), dtype=torch.int32, device=dev),
        "col_kind": torch.empty(max(1, nQt * nKt), dtype=torch.uint8, device=dev),
        "tile_m": 128,
    }
    _ffi.check(_lib().mfa_tile_map_coarsen(_p(compacted64["tile_kind"]), Nq, Nk, _p(out["tile_kind"]),
                                           _p(out["row_ptr"]), _p(out["col_idx"]), _p(out["col_kind"]), _stream()))
    return out


def choose_tile_m(counts64, counts128, Nq, head_dim=128):
    """Tile height (64 or 128) for a mask with these tile counts at this head
    dim (mfa_choose_tile_m, host only)."""
    a = (C.c_int64 * 3)(*[int(x) for x in counts64])
    b = (C.c_int64 * 3)(*[int(x) for x in counts128])
    return int(_lib().mfa_choose_tile_m(a, b, int(Nq), int(head_dim)))


def compact_dense_mask_auto(mask, head_dim=128):
    """Density-aware dispatch (BinFlash, "Efficiently Dispatching ..."): one
    pass over the mask at 64-row tiles, the 128-row map derived from it, the
    tile statistics of both read back (one sync), and the compaction whose
    modelled forward time at this head dim is smaller returned (with
    "tile_m" and "counts")."""
    m = _u8(mask).contiguous()
    Nq, Nk = m.shape
    c64 = compact_dense_mask(m, BM=64)
    c128 = coarsen_tile_map(c64, Nq, Nk)
    n64 = tile_counts(c64["tile_kind"]).cpu().tolist()
    n128 = tile_counts(c128["tile_kind"]).cpu().tolist()
    bm = choose_tile_m(n64, n128, Nq, head_dim)
    out = c64 if bm == 64 else c128
    out["counts"] = {64: n64, 128: n128}
    return out


def _kv_bits(bits, B, Skv):
    t = bits.contiguous()
    if t.dtype not in (torch.int32, torch.uint32) or tuple(t.shape) != (B, _cdiv(Skv, 32)):
        raise ValueError(f"kv_valid_bits must be a 32-bit ({B}, {_cdiv(Skv, 32)}) tensor")
    return t


def bsr_from_bitmask(bits, n_kv_blocks, cap=None):
    """BSR rows from the bitmask sparse format (mfa_bsr_from_bitmask).

    bits: (B, Hkv, nQb, ceil(nKb/32)) 32-bit words, bit c of a row selects KV
    block c. Returns (indptr (B, Hkv, nQb+1) i32, indices (cap,) i32), no
    host sync: cap defaults to the largest possible count, and only
    indices[:indptr[-1,-1,-1]] is meaningful."""
    t = bits.contiguous()
    B, H, R, W = t.shape
    if W != _cdiv(n_kv_blocks, 32):
        raise ValueError(f"last axis must hold ceil({n_kv_blocks}/32) words")
    cap = B * H * R * n_kv_blocks if cap is None else int(cap)
    indptr = torch.empty(B, H, R + 1, dtype=torch.int32, device=t.device)
    indices = torch.empty(max(1, cap), dtype=torch.int32, device=t.device)
    _ffi.check(_lib().mfa_bsr_from_bitmask(_p(t), B, H, R, n_kv_blocks, _p(indptr), _p(indices), cap, _stream()))
    return indptr, indices[:cap]


def varlen_schedule(len_q, len_k=None, causal=True, window=(-1, -1), BM=TILE_M, BN=TILE_N, work_cap=None):
    """cu_seqlens, max lengths and the longest-first tile list (mfa_varlen_schedule).

    ``work_cap`` (required, so that no host sync is needed) bounds the tile
    count: sum ceil(L/BM) <= total_q // BM + nseq always holds. The call is
    asynchronous; ``n_work`` (device) reads -1 when the tiles do not fit in
    work_cap and -2 when more than 16,384 tiles share one group of equal
    cost >> 12 (see mfa.h), and then every work entry is -1.
    """
    lq = _i32(len_q).contiguous()
    lk = lq if len_k is None else _i32(len_k).contiguous()
    nseq = lq.numel()
    dev = lq.device
    if work_cap is None:
        raise ValueError("work_cap is required (e.g. total_q // BM + nseq)")
    out = {
        "cu_q": torch.empty(nseq + 1, dtype=torch.int32, device=dev),
        "cu_k": torch.empty(nseq + 1, dtype=torch.int32, device=dev),
        "max_len": torch.empty(2, dtype=torch.int32, device=dev),
        "work": torch.empty(max(1, work_cap), 2, dtype=torch.int32, device=dev),
        "n_work": torch.empty(1, dtype=torch.int32, device=dev),
        "work_cap": work_cap,
    }
    left, right = window
    _ffi.check(_lib().mfa_varlen_schedule(_p(lq), _p(lk), nseq, BM, BN, int(bool(causal)), left, right,
                                          _p(out["cu_q"]), _p(out["cu_k"]), _p(out["max_len"]), _p(out["work"]),
                                          work_cap, _p(out["n_work"]), _stream()))
    return out


@dataclass
class MaskRep:
    """A mask representation for ``attn_fwd`` (fields as in mfa_mask)."""
    kind: int
    tensors: dict = field(default_factory=dict)
    ints: dict = field(default_factory=dict)

    @staticmethod
    def none():
        return MaskRep(_ffi.MASK_NONE)

    @staticmethod
    def tiles(compacted):
        return MaskRep(_ffi.MASK_TILES, {k: compacted[k] for k in
                                         ("tile_kind", "fine_bits", "row_ptr", "col_idx", "col_kind")},
                       {"tile_m": int(compacted.get("tile_m", TILE_M))})

    @staticmethod
    def blockid(q_blk, k_blk, q_valid, k_valid, summary=None):
        if summary is None:
            summary = blockid_tile_summary(q_blk, k_blk, q_valid, k_valid)
        qsum, ksum, kv_bits = summary
        return MaskRep(_ffi.MASK_BLOCKID, {"q_blk": _i32(q_blk).contiguous(), "k_blk": _i32(k_blk).contiguous(),
                                           "q_valid": _u8(q_valid).contiguous(),
                                           "k_valid": _u8(k_valid).contiguous(),
                                           "qsum": qsum, "ksum": ksum, "kv_bits": kv_bits})

    @staticmethod
    def bsr(block_indptr, block_indices, bsr_kind, q_block=64, kv_block=64, causal=True, csc_ptr=None,
            csc_idx=None, kv_valid_bits=None):
        t = {"indptr": _i32(block_indptr).contiguous(), "indices": _i32(block_indices).contiguous(),
             "bsr_kind": bsr_kind}
        if csc_ptr is not None:
            t["csc_ptr"], t["csc_idx"] = csc_ptr, csc_idx
        if kv_valid_bits is not None:
            t["kv_bits"] = kv_valid_bits.contiguous()
        return MaskRep(_ffi.MASK_BSR, t, {"q_block": q_block, "kv_block": kv_block, "causal": int(bool(causal))})

    @staticmethod
    def varlen(sched, max_q, max_k, causal=True, window=(-1, -1), err=None, seqused_k=None, block_table=None,
               page_size=None, n_pages=None):
        """Packed variable-length mask. seqused_k: optional (nseq,) int32 keys
        used per sequence. block_table (nseq, max_pages) int32 with page_size
        and n_pages: k / v are page pools (n_pages, page_size, Hkv, D), and
        so are dk / dv in the backward."""
        t = {"cu_q": sched["cu_q"], "cu_k": sched["cu_k"], "work": sched["work"]}
        ints = {"work_cap": sched["work_cap"], "max_q": int(max_q), "max_k": int(max_k),
                "causal": int(bool(causal)), "win_left": int(window[0]), "win_right": int(window[1]),
                "nseq": int(sched["cu_q"].numel()) - 1}
        if err is not None:
            t["err"] = err
        if seqused_k is not None:
            t["seqused_k"] = _i32(seqused_k).contiguous()
        if block_table is not None:
            bt = _i32(block_table).contiguous()
            t["block_table"] = bt
            ints.update(max_pages=int(bt.shape[1]), page_size=int(page_size), n_pages=int(n_pages))
        return MaskRep(_ffi.MASK_VARLEN, t, ints)

    def to_c(self):
        m = _ffi.Mask()
        m.kind = self.kind
        for k, v in self.tensors.items():
            setattr(m, k, v.data_ptr())
        for k, v in self.ints.items():
            setattr(m, k, v)
        if self.kind != _ffi.MASK_VARLEN:
            m.win_left = m.win_right = -1
        return m


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _bsh_strides(t, layout):
    """(batch, seq, head) element strides of a 4-D tensor or a 3-D packed one."""
    if t.stride(-1) != 1:
        raise ValueError("the head-dim axis must be contiguous")
    if layout == "bshd":
        return (t.stride(0), t.stride(1), t.stride(2))
    if layout == "bhsd":
        return (t.stride(0), t.stride(2), t.stride(1))
    if layout == "thd":
        if t.dim() == 4:  # paged k / v: (page, row, head) strides
            return (t.stride(0), t.stride(1), t.stride(2))
        return (0, t.stride(0), t.stride(1))
    raise ValueError(f"unknown layout {layout!r}")


def _dims(q, k, layout):
    if layout == "thd" and k.dim() == 4:  # paged k / v: (n_pages, page_size, Hkv, D)
        Sq, Hq, D = q.shape
        return 1, Sq, k.shape[0] * k.shape[1], Hq, k.shape[2], D
    if layout == "bshd":
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
    elif layout == "bhsd":
        B, Hq, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
    else:
        B = 1
        Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[0], k.shape[1]
    return B, Sq, Sk, Hq, Hkv, D


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _ffi.MFA_BF16
    if t.dtype == torch.float32:
        return _ffi.MFA_F32
    raise MfaError(3, f"dtype {t.dtype} not supported (bfloat16, or float32 test mode)")


def _slopes_ptr(alibi_slopes, Hq, device):
    """Device pointer of a (Hq,) fp32 slope vector for the positional bias
    slope[h] * (kv_idx - q_idx), or None."""
    if alibi_slopes is None:
        return None
    t = alibi_slopes
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device \
            or t.shape != (Hq,) or not t.is_contiguous():
        raise ValueError(f"alibi_slopes must be a contiguous float32 tensor of shape ({Hq},) on {device}")
    return t.data_ptr()


def attn_fwd(q, k, v, mask: MaskRep, scale=None, layout="bshd", out=None, return_lse=True, lse=None,
             alibi_slopes=None, softcap=None):
    """Masked attention forward (mfa_attn_fwd). Returns (out, lse or None).

    layout: "bshd" (B, S, H, D), "bhsd" (B, H, S, D) or "thd" (packed varlen).
    lse is fp32 (B, Hq, Sq) ((Hq, T) for "thd"). alibi_slopes: optional
    (Hq,) fp32 tensor; adds slope[h] * (kv_idx - q_idx) to the scaled scores
    (positions local to the sequence for "thd"). softcap: optional positive
    float; each score x (after the bias) becomes softcap * tanh(x / softcap).
    """
    B, Sq, Sk, Hq, Hkv, D = _dims(q, k, layout)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Sq) if layout == "thd" else (B, Hq, Sq), dtype=torch.float32, device=q.device)
    a = _ffi.AttnArgs()
    a.dtype = _dtype_code(q)
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.D = B, Sq, Sk, Hq, Hkv, D
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if (return_lse and lse is not None) else None
    a.q_stride = _ffi.i64x3(*_bsh_strides(q, layout))
    a.k_stride = _ffi.i64x3(*_bsh_strides(k, layout))
    a.v_stride = _ffi.i64x3(*_bsh_strides(v, layout))
    a.o_stride = _ffi.i64x3(*_bsh_strides(out, layout))
    a.alibi_slopes = _slopes_ptr(alibi_slopes, Hq, q.device)
    a.softcap = float(softcap or 0.0)
    m = mask.to_c()
    _ffi.check(_lib().mfa_attn_fwd(C.byref(a), C.byref(m), float(scale), _stream()))
    return out, (lse if return_lse else None)


def _bwd_args(q, k, v, out, lse, dout, dq, dk, dv, delta, layout, alibi_slopes=None, softcap=None):
    B, Sq, Sk, Hq, Hkv, D = _dims(q, k, layout)
    a = _ffi.BwdArgs()
    f = a.fwd
    f.dtype = _dtype_code(q)
    f.B, f.Sq, f.Sk, f.Hq, f.Hkv, f.D = B, Sq, Sk, Hq, Hkv, D
    f.q, f.k, f.v, f.out, f.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    f.q_stride = _ffi.i64x3(*_bsh_strides(q, layout))
    f.k_stride = _ffi.i64x3(*_bsh_strides(k, layout))
    f.v_stride = _ffi.i64x3(*_bsh_strides(v, layout))
    f.o_stride = _ffi.i64x3(*_bsh_strides(out, layout))
    f.alibi_slopes = _slopes_ptr(alibi_slopes, Hq, q.device)
    f.softcap = float(softcap or 0.0)
    a.dout, a.dq, a.dk, a.dv, a.delta = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), \
        delta.data_ptr()
    a.do_stride = _ffi.i64x3(*_bsh_strides(dout, layout))
    a.dq_stride = _ffi.i64x3(*_bsh_strides(dq, layout))
    a.dk_stride = _ffi.i64x3(*_bsh_strides(dk, layout))
    a.dv_stride = _ffi.i64x3(*_bsh_strides(dv, layout))
    return a


def attn_bwd_preprocess(args):
    _ffi.check(_lib().mfa_attn_bwd_preprocess(C.byref(args), _stream()))


def attn_bwd_dkdv_workspace(args, mask: MaskRep):
    """(bytes, splits): workspace of the dK/dV pass's preferred query-head
    split on the current device (mfa_attn_bwd_dkdv_workspace)."""
    m = mask.to_c()
    nb, ns = C.c_int64(0), C.c_int(0)
    _ffi.check(_lib().mfa_attn_bwd_dkdv_workspace(C.byref(args), C.byref(m), C.byref(nb), C.byref(ns)))
    return int(nb.value), int(ns.value)


def choose_dkdv_split(key_blocks, group, head_dim, n_cu):
    """Query-head split of the dK/dV pass (mfa_choose_dkdv_split, host only)."""
    return int(_lib().mfa_choose_dkdv_split(int(key_blocks), int(group), int(head_dim), int(n_cu)))


def attn_bwd_dkdv(args, mask: MaskRep, scale, workspace=None):
    """dK/dV pass. workspace: a device uint8 tensor for the query-head split
    (attn_bwd_dkdv_workspace gives its size), or None for no split."""
    if workspace is not None:
        args.workspace, args.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        args.workspace, args.workspace_bytes = None, 0
    m = mask.to_c()
    _ffi.check(_lib().mfa_attn_bwd_dkdv(C.byref(args), C.byref(m), float(scale), _stream()))


def attn_bwd_dkdv_noalloc(args, mask: MaskRep, scale):
    """dK/dV pass that allocates nothing (mfa_attn_bwd_dkdv_noalloc): the head
    split's partial sums go to the library's static device scratch
    (bwd_scratch_bytes()); calls that overlap on one device race."""
    m = mask.to_c()
    _ffi.check(_lib().mfa_attn_bwd_dkdv_noalloc(C.byref(args), C.byref(m), float(scale), _stream()))


def bwd_scratch_bytes():
    """Size of the static scratch of attn_bwd_dkdv_noalloc."""
    return int(_lib().mfa_bwd_scratch_bytes())


def attn_bwd_dq(args, mask: MaskRep, scale):
    m = mask.to_c()
    _ffi.check(_lib().mfa_attn_bwd_dq(C.byref(args), C.byref(m), float(scale), _stream()))


def attn_bwd(q, k, v, out, lse, dout, mask: MaskRep, scale=None, layout="bshd", alibi_slopes=None, dq=None,
             dk=None, dv=None, delta=None, softcap=None):
    """Two-pass backward (any mask kind): preprocess, dK/dV over key blocks,
    dQ over query tiles. Returns (dq, dk, dv) shaped like q, k, v (written
    into the given tensors when passed; delta is fp32 (B, Hq, Sq)). The
    slopes and the soft cap must be the forward's."""
    B, Sq, Sk, Hq, Hkv, D = _dims(q, k, layout)
    if scale is None:
        scale = D ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
    a = _bwd_args(q, k, v, out, lse, dout, dq, dk, dv, delta, layout, alibi_slopes, softcap)
    attn_bwd_preprocess(a)
    nbytes, _ = attn_bwd_dkdv_workspace(a, mask)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    attn_bwd_dkdv(a, mask, scale, workspace=ws)
    attn_bwd_dq(a, mask, scale)
    return dq, dk, dv


class _MaskedAttention(torch.autograd.Function):
    """Forward and backward both run the library's kernels; the mask
    representation, scale, bias slopes and soft cap are constants of the graph."""

    @staticmethod
    def forward(ctx, q, k, v, mask, scale, layout, alibi_slopes, softcap):
        out, lse = attn_fwd(q, k, v, mask, scale, layout, alibi_slopes=alibi_slopes, softcap=softcap)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.mask, ctx.scale, ctx.layout, ctx.slopes, ctx.softcap = mask, scale, layout, alibi_slopes, softcap
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        if dout.stride(-1) != 1 or dout.data_ptr() % 16:
            dout = dout.contiguous()
        dq, dk, dv = attn_bwd(q, k, v, out, lse, dout, ctx.mask, ctx.scale, ctx.layout, ctx.slopes,
                              softcap=ctx.softcap)
        return dq, dk, dv, None, None, None, None, None


def masked_attention(q, k, v, mask: MaskRep, scale=None, layout="bshd", alibi_slopes=None, softcap=None):
    """Differentiable masked attention: out = softmax(cap(scale q k^T + bias) + mask) v,
    cap(x) = softcap * tanh(x / softcap) when softcap is given, else x.

    bf16 q, k, v with requires_grad as needed; gradients come from the
    two-pass backward (mfa_attn_bwd_*). layout, alibi_slopes and softcap as
    for attn_fwd (the slopes get no gradient)."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _MaskedAttention.apply(q, k, v, mask, float(scale), layout, alibi_slopes, softcap)
