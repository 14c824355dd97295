"""Helpers shared by the GPU parity tests: device setup, oracle comparison."""

import sys

import numpy as np
import torch

DEV = "cuda:0"
BF16_OUT_TOL = 2e-2   # max-abs error of attention outputs, bf16 in/out, fp32 accumulate
F32_OUT_TOL = 1e-4    # max-abs error in fp32 test mode
LSE_TOL = 1e-3        # max-abs error of the log-sum-exp
GRAD_ULP = 2.0 ** -7  # one bf16 unit in the last place, relative to the value


def grad_tolerance(ref):
    """Per-element bound for bf16-stored gradients: the output tolerance plus
    one bf16 ULP of the exact value (gradients above ~2.5 in magnitude cannot
    meet 2e-2 once rounded to bf16)."""
    return BF16_OUT_TOL + GRAD_ULP * np.abs(ref)


def grad_tolerance_terms(ref, term_sum):
    """grad_tolerance plus the first-order bound of the bf16 storage of P, dS
    and O (unit roundoff 2^-9) that the oracle's term_sums give. It matters
    where rows put nearly all their weight on one key (a strong positional
    bias): then |O| ~ |v|, so Delta = dO.O taken from the rounded O moves by
    ~0.1, and dV_j is a small difference of large terms."""
    return grad_tolerance(ref) + 2.0 ** -9 * np.abs(term_sum)


def note(msg):
    """Name the case before each GPU step, flushed, so a fault names it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype=None):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        x = x.to(dtype)
    return x.to(DEV)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def compare_attention(out, lse, ref_out, ref_lse, out_tol, lse_tol=LSE_TOL, rows_axis_lse=-1):
    """Max-abs check of out and lse; empty rows (ref lse = -inf) must be exactly 0 / -inf.

    out / ref_out: same-shaped arrays with the query axis matching lse's last axis
    after transposition by the caller; returns (max out error, max lse error).
    """
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.all(np.isfinite(out)), "non-finite output"
    err_o = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "empty-row pattern of lse differs"
    fin = ~empty
    err_l = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert err_o <= out_tol, f"out max-abs error {err_o:.3e} > {out_tol}"
    assert err_l <= lse_tol, f"lse max-abs error {err_l:.3e} > {lse_tol}"
    return err_o, err_l


def tile_rows(n, tile, salt):
    """One index in every `tile`-sized block of [0, n): block t contributes
    t*tile + (37 t + salt) mod len(block), so different blocks (and different
    salts, e.g. per (batch, head)) land on different lanes and waves."""
    starts = np.arange(0, n, tile)
    lens = np.minimum(tile, n - starts)
    return starts + (37 * np.arange(starts.size) + salt) % lens


def nan_like(t):
    """A NaN-filled tensor like t: outputs the kernel leaves unwritten stay NaN."""
    return torch.full_like(t, float("nan"))


def bsr_row_mask(ip_bh, ix, blk, N, rows, causal=True):
    """Allowed keys (len(rows), N) of query rows under one (batch, head)'s BSR
    rows ip_bh (its nQb + 1 offsets into ix), causal inside blocks."""
    rows = np.asarray(rows)
    nKb = -(-N // blk)
    blocks = np.zeros((rows.size, nKb), bool)
    for n, r in enumerate(rows // blk):
        blocks[n, ix[ip_bh[r]:ip_bh[r + 1]]] = True
    a = np.repeat(blocks, blk, axis=1)[:, :N]
    if causal:
        a &= np.arange(N)[None, :] <= rows[:, None]
    return a
