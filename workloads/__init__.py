"""Seeded synthetic inputs shaped like the pages' workloads.

This module is shared by the tests, the benchmark and the smoke check, and is
the ONLY code both the oracle side and the GPU side use. It draws random
numbers and lays out inputs; it holds none of the method's arithmetic (no
block ids, no tile maps, no prefix sums of lengths, no attention).

Recipes (config k):
* structure from ``np.random.default_rng(k)``, drawn in the order written below;
* tensors from ``torch.Generator().manual_seed(1000 + k)``, ``randn`` fp32 drawn
  in the order q, k, v, dO, each rounded to bfloat16 (round-to-nearest-even).

Each builder takes size overrides so that parity tests can run the same recipe
at sizes the fp64 oracle finishes in seconds.
"""

from __future__ import annotations

import numpy as np
import torch


def _randn(gen, shape, dtype):
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def tensors(seed, shapes, dtype=torch.bfloat16):
    """Draw one N(0,1) tensor per shape, in order, from a CPU generator."""
    g = torch.Generator().manual_seed(int(seed))
    return [_randn(g, s, dtype) for s in shapes]


# --- config 1: block-causal tiny (opentau block-id representation) -----------

def blockcausal_tiny(N=256, B=1, H=2, D=64, n_pad=16, p_open=0.1, seed=1, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    att = np.zeros((B, N), dtype=np.int32)
    pad = np.ones((B, N), dtype=bool)
    for b in range(B):
        att[b] = (rng.random(N) < p_open).astype(np.int32)
        att[b, 0] = 1
        if n_pad:
            pad[b, N - n_pad:] = False
    q, k, v = tensors(1000 + seed, [(B, N, H, D)] * 3, dtype)
    return dict(att=att, pad=pad, q=q, k=k, v=v, scale=D ** -0.5, layout="bshd")


# --- config 2: causal dense (N, N) bool mask (BinFlash "Use" example) --------

def causal_dense(N=8192, B=4, H=32, D=128, seed=2, dtype=torch.bfloat16, mask="causal"):
    """q/k/v in (B, H, N, D) like the BinFlash example; mask True = attend."""
    if mask == "causal":
        m = np.tril(np.ones((N, N), dtype=bool))
    elif mask == "all":
        m = np.ones((N, N), dtype=bool)
    elif mask == "none":
        m = np.zeros((N, N), dtype=bool)
    else:
        raise ValueError(mask)
    q, k, v = tensors(1000 + seed, [(B, H, N, D)] * 3, dtype)
    return dict(mask=m, q=q, k=k, v=v, scale=D ** -0.5, layout="bhsd")


def random_dense_mask(Nq, Nk, density, seed, structured=True):
    """Random (Nq, Nk) bool mask mixing empty, full and partial regions."""
    rng = np.random.default_rng(seed)
    m = rng.random((Nq, Nk)) < density
    if structured:
        for _ in range(max(1, (Nq * Nk) // 20000)):
            r0, c0 = rng.integers(0, Nq), rng.integers(0, Nk)
            h, w = rng.integers(1, 200), rng.integers(1, 200)
            m[r0:r0 + h, c0:c0 + w] = bool(rng.integers(0, 2))
    return m


# --- config 3: varlen packed, document-causal + sliding window ---------------

def varlen_window(nseq=32, lo=128, hi=4096, H=16, D=64, window=512, seed=3, dtype=torch.bfloat16):
    """Lengths uniform in [lo, hi]; q/k/v packed (total_tokens, H, D)."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, nseq).astype(np.int32)
    T = int(lengths.sum())
    q, k, v = tensors(1000 + seed, [(T, H, D)] * 3, dtype)
    return dict(lengths=lengths, q=q, k=k, v=v, scale=D ** -0.5, window=window, layout="thd")


# --- config 4: block-causal GQA with cross-attention columns -----------------

def blockcausal_gqa_cross(B=8, N=1024, Hq=16, Hkv=2, D=128, Nc=256, prefix=512,
                          blk_lo=32, blk_hi=128, pad_hi=128, p_cross=0.9, seed=4,
                          dtype=torch.bfloat16):
    """512-token bidirectional prefix, then random 32..128-token blocks,
    tail padding uniform in [0, 128], Bernoulli(0.9) cross padding.
    k/v are (B, Nc + N, Hkv, D) with the cross keys first."""
    rng = np.random.default_rng(seed)
    att = np.zeros((B, N), dtype=np.int32)
    pad = np.ones((B, N), dtype=bool)
    cross = np.zeros((B, Nc), dtype=bool)
    for b in range(B):
        att[b, 0] = 1
        pos = prefix
        while pos < N:
            att[b, pos] = 1
            pos += int(rng.integers(blk_lo, blk_hi + 1))
        p_b = int(rng.integers(0, pad_hi + 1))
        if p_b:
            pad[b, N - p_b:] = False
        cross[b] = rng.random(Nc) < p_cross
    q, k, v = tensors(1000 + seed, [(B, N, Hq, D), (B, Nc + N, Hkv, D), (B, Nc + N, Hkv, D)], dtype)
    return dict(att=att, pad=pad, cross_pad=cross, n_cross=Nc, q=q, k=k, v=v,
                scale=D ** -0.5, layout="bshd")


# --- config 5: BSR block sparse + backward (flashinfer block_sparse_attention) -

def bsr_random(B=2, N=16384, H=16, D=128, block=64, frac_den=10, seed=5, dtype=torch.bfloat16):
    """Each query-block row r lists floor(r / frac_den) distinct earlier KV blocks
    (uniform without replacement, ascending) plus the diagonal block r.
    block_indptr holds offsets into one flat block_indices array."""
    rng = np.random.default_rng(seed)
    nb = -(-N // block)
    indptr = np.zeros((B, H, nb + 1), dtype=np.int32)
    chunks = []
    pos = 0
    for b in range(B):
        for h in range(H):
            indptr[b, h, 0] = pos
            for r in range(nb):
                picks = sorted(rng.choice(r, r // frac_den, replace=False).tolist()) if r else []
                row = picks + [r]
                chunks.append(np.asarray(row, dtype=np.int32))
                pos += len(row)
                indptr[b, h, r + 1] = pos
    indices = np.concatenate(chunks).astype(np.int32)
    q, k, v, do = tensors(1000 + seed, [(B, N, H, D)] * 4, dtype)
    return dict(indptr=indptr, indices=indices, block=block, q=q, k=k, v=v, do=do,
                scale=D ** -0.5, layout="bshd")
