"""Dense fp64 masked softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

This is the plain definition the pages' methods reach exactly (up to rounding
order): BinFlash (intro) replaces scaled-dot-product attention under a dense
(N, N) bool mask, and tensorplay omni_attention (intro) states that its result
equals masked softmax written out by hand. No tiles, no online softmax: per
(batch, query head) the full score rows are formed, masked, normalised and
applied.

Conventions (readings where the pages are silent):

* inputs are cast exactly to fp64 (bf16 and fp32 are exact in fp64);
* GQA/MQA: query head hq reads key/value head hq // (Hq // Hkv), i.e. groups of
  consecutive query heads share one KV head (opentau page: H % Hkv == 0);
* a query with no allowed key gets output 0 and log-sum-exp -inf, and in the
  backward contributes nothing (its dQ row is 0);
* the log-sum-exp is natural-log of sum over allowed keys of exp(scale q.k),
  layout (B, Hq, Sq) ("Outputs" section of omni_attention: log-sum-exp of the
  attention weights);
* masks are given as a bool array (Bm, Hm, Sq, Sk) with Bm in {1, B} and Hm in
  {1, Hkv, Hq} (head index hq * Hm // Hq), or as a callable
  ``allowed(b, hm, rows) -> (len(rows), Sk) bool`` for row-sampled checks at
  sizes where the dense mask does not fit in memory;
* ``score_mod(score, b, h, q_idx, kv_idx)`` (tensorplay omni_attention,
  intro: it receives the current score and its coordinates and returns the
  modified score) is applied to the scaled scores before masking. In the
  backward, dS is multiplied by the mod's derivative with respect to the
  incoming score, ``score_mod.grad(score, b, h, q_idx, kv_idx)``, when the
  mod carries one (the soft cap does); a mod without it is additive (a term
  that does not depend on the score, as positional biases are): derivative 1.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _mask_rows(allowed, b, hm, rows, Sk):
    if callable(allowed):
        m = np.asarray(allowed(b, hm, rows), dtype=bool)
    else:
        a = np.asarray(allowed)
        bb = b if a.shape[0] > 1 else 0
        m = a[bb, hm][rows]
    return np.broadcast_to(m, (len(rows), Sk))


def _mask_heads(allowed, Hq):
    if callable(allowed):
        return getattr(allowed, "heads", Hq)
    return np.asarray(allowed).shape[1]


def alibi(slopes):
    """score_mod adding slope[h] * (kv_idx - q_idx): a linear penalty on the
    distance of earlier keys; a slope of 1 on every head is the
    distance-decay example of the omni_attention intro."""
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score + sl[h] * (np.asarray(kv_idx, np.float64) - np.asarray(q_idx, np.float64))
    return mod


def softcap(cap, inner=None):
    """score_mod cap * tanh(x / cap), x the incoming score after the optional
    ``inner`` mod (e.g. ``alibi(slopes)``): a soft cap on the scores, one of
    the one-line score_mods the omni_attention intro lists. Carries
    ``.grad`` = d mod / d score = (1 - tanh(x / cap)^2) * d inner / d score."""
    cap = float(cap)

    def pre(score, b, h, q_idx, kv_idx):
        return score if inner is None else inner(score, b, h, q_idx, kv_idx)

    def mod(score, b, h, q_idx, kv_idx):
        return cap * np.tanh(pre(score, b, h, q_idx, kv_idx) / cap)

    def grad(score, b, h, q_idx, kv_idx):
        t = np.tanh(pre(score, b, h, q_idx, kv_idx) / cap)
        g = 1.0 - t * t
        if inner is not None and hasattr(inner, "grad"):
            g = g * inner.grad(score, b, h, q_idx, kv_idx)
        return g

    mod.grad = grad
    return mod


def _scores(q_rows, k_all, scale, score_mod, b, hq, rr):
    s = scale * (q_rows @ k_all.T)
    if score_mod is not None:
        s = score_mod(s, b, hq, np.asarray(rr)[:, None], np.arange(k_all.shape[0])[None, :])
    return s


def _mod_grad(q_rows, k_cols, scale, score_mod, b, hq, rr, cols=None):
    """Derivative of the score_mod at the scaled scores (1 for additive mods)."""
    if score_mod is None or not hasattr(score_mod, "grad"):
        return 1.0
    kj = np.arange(k_cols.shape[0]) if cols is None else np.asarray(cols)
    return score_mod.grad(scale * (q_rows @ k_cols.T), b, hq, np.asarray(rr)[:, None], kj[None, :])


def attention_fwd(q, k, v, allowed, scale, rows=None, chunk=1024, score_mod=None):
    """Masked softmax attention. q (B, Sq, Hq, D); k, v (B, Sk, Hkv, D).

    Returns (out (B, nrows, Hq, D) fp64, lse (B, Hq, nrows) fp64) for the query
    rows ``rows`` (default: all).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    Hm = _mask_heads(allowed, Hq)
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.zeros((B, rows.size, Hq, v.shape[3]))
    lse = np.full((B, Hq, rows.size), -np.inf)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            hm = hq * Hm // Hq
            for c0 in range(0, rows.size, chunk):
                rr = rows[c0:c0 + chunk]
                s = _scores(q[b, rr, hq, :], k[b, :, hk, :], scale, score_mod, b, hq, rr)
                a = _mask_rows(allowed, b, hm, rr, Sk)
                has = a.any(axis=1)
                sm = np.where(a, s, -np.inf)
                m = np.where(has, sm.max(axis=1, initial=-np.inf), 0.0)
                e = np.where(a, np.exp(sm - m[:, None]), 0.0)
                l = e.sum(axis=1)
                o = e @ v[b, :, hk, :]
                safe_l = np.where(has, l, 1.0)
                out[b, c0:c0 + rr.size, hq, :] = np.where(has[:, None], o / safe_l[:, None], 0.0)
                lse[b, hq, c0:c0 + rr.size] = np.where(has, m + np.log(safe_l), -np.inf)
    return out, lse


def attention_bwd(q, k, v, dout, allowed, scale, score_mod=None, term_sums=False):
    """Gradients of sum(out * dout) with respect to q, k, v (fp64, dense).

    P_ij = exp(s_ij - LSE_i) on allowed entries, 0 elsewhere;
    dV_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;  Delta_i = sum_j P_ij dP_ij;
    dS_ij = P_ij (dP_ij - Delta_i);  dQ_i = scale sum_j dS_ij k_j;
    dK_j = scale sum_i dS_ij q_i; dK/dV sum over the query heads of a group.
    The two-pass split (dK/dV over key blocks, dQ over query blocks) of the
    BinFlash method is a schedule of these same sums.
    Returns dq, dk, dv, out, lse, delta (delta (B, Hq, Sq)); with
    ``term_sums`` also (tq, tk, tv), magnitudes that bound how far a kernel
    storing P, dS and O in bf16 (unit roundoff u = 2^-9) can move each
    gradient, to first order in u:
      tv_j = sum_i P_ij |dO_i|                (P rounded for dV);
      E_ij = P_ij (|dP_ij| + |Delta_i| + B_i), with
      B_i  = sum_d |dO_id| |O_id| + sum_j P_ij |dP_ij|, which bounds the
             error of a Delta taken from the rounded O (output rounding plus
             the rounding of each P_ij, which scales a whole row v_j);
      tq_i = scale sum_j E_ij |k_j|, tk_j = scale sum_i E_ij |q_i|
    so that |error| <= u * t plus the fp32 accumulation error.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    Hm = _mask_heads(allowed, Hq)
    out, lse = attention_fwd(q, k, v, allowed, scale, score_mod=score_mod)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((B, Hq, Sq))
    if term_sums:
        tq, tk, tv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rows = np.arange(Sq)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            hm = hq * Hm // Hq
            a = _mask_rows(allowed, b, hm, rows, Sk)
            s = _scores(q[b, :, hq, :], k[b, :, hk, :], scale, score_mod, b, hq, rows)
            L = lse[b, hq]
            finite = np.isfinite(L)
            P = np.where(a & finite[:, None], np.exp(s - np.where(finite, L, 0.0)[:, None]), 0.0)
            dv[b, :, hk, :] += P.T @ do[b, :, hq, :]
            dP = do[b, :, hq, :] @ v[b, :, hk, :].T
            dl = (P * dP).sum(axis=1)
            delta[b, hq] = dl
            gm = _mod_grad(q[b, :, hq, :], k[b, :, hk, :], scale, score_mod, b, hq, rows)
            dS = P * (dP - dl[:, None]) * gm
            dq[b, :, hq, :] = scale * (dS @ k[b, :, hk, :])
            dk[b, :, hk, :] += scale * (dS.T @ q[b, :, hq, :])
            if term_sums:
                Bi = (np.abs(do[b, :, hq, :]) * np.abs(out[b, :, hq, :])).sum(axis=1) + (P * np.abs(dP)).sum(axis=1)
                E = P * np.abs(gm) * (np.abs(dP) + np.abs(dl)[:, None] + Bi[:, None])
                tq[b, :, hq, :] = scale * (E @ np.abs(k[b, :, hk, :]))
                tk[b, :, hk, :] += scale * (E.T @ np.abs(q[b, :, hq, :]))
                tv[b, :, hk, :] += P.T @ np.abs(do[b, :, hq, :])
    if term_sums:
        return dq, dk, dv, out, lse, delta, (tq, tk, tv)
    return dq, dk, dv, out, lse, delta


def varlen_attention_fwd(q, k, v, cu_q, cu_k, scale, causal, left, right, rows=None, score_mod=None,
                         seqused_k=None):
    """Packed variable-length attention (tensorplay varlen "Packed layout").

    q (Tq, Hq, D), k/v (Tk, Hkv, D); query row t of sequence s may see key u
    iff u is in sequence s and the window predicate holds on local positions.
    ``score_mod`` sees local positions too (q_idx = t - cu_q[s],
    kv_idx = u - cu_k[s]) and the sequence index as b. ``seqused_k`` keeps
    only the first seqused_k[s] keys of each sequence.
    Returns out (n, Hq, D), lse (Hq, n) for the rows ``rows`` (default all).
    """
    cq = np.asarray(cu_q).astype(np.int64)
    ck = np.asarray(cu_k).astype(np.int64)
    Tk = int(ck[-1])
    seq_of = np.searchsorted(cq, np.arange(int(cq[-1])), side="right") - 1
    kidx = np.arange(Tk)

    def allowed(b, hm, rr):
        s = seq_of[rr]
        i = rr - cq[s]
        j = kidx[None, :] - ck[s][:, None]
        klen = ck[s + 1] - ck[s]
        if seqused_k is not None:
            klen = np.minimum(klen, np.asarray(seqused_k).astype(np.int64)[s])
        in_seq = (j >= 0) & (j < klen[:, None])
        from .masks import window_allows
        return in_seq & window_allows(i[:, None], j, causal, left, right)

    allowed.heads = 1
    mod = None
    if score_mod is not None:
        def mod(score, b, h, q_idx, kv_idx):
            t = np.asarray(q_idx).reshape(-1)
            sq = seq_of[t]
            return score_mod(score, sq[:, None], h, (t - cq[sq])[:, None],
                             np.asarray(kv_idx).reshape(1, -1) - ck[sq][:, None])
    out, lse = attention_fwd(_f64(q)[None], _f64(k)[None], _f64(v)[None], allowed, scale, rows=rows,
                             score_mod=mod)
    return out[0], lse[0]


def attention_bwd_sampled(q, k, v, dout, allowed, scale, b, hk, rows, cols, chunk=1024, score_mod=None):
    """Selected rows of dQ and columns of dK/dV for one (batch, kv head), fp64.

    Same formulas as ``attention_bwd`` evaluated without the dense (Sq, Sk)
    matrices: the forward (O, LSE) of every query row of the group's heads is
    computed in row chunks, then dQ_i (for i in ``rows``) uses row i's
    P, dP and Delta, and dK_j / dV_j (for j in ``cols``) sum column j over all
    query rows and all query heads of the group. ``allowed`` is a callable
    ``allowed(b, hm, rows) -> (len(rows), Sk)`` (as for ``attention_fwd``);
    ``score_mod`` as there. Returns dq (G, len(rows), D) for the group's heads, dk (len(cols), D),
    dv (len(cols), D).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    Hm = _mask_heads(allowed, Hq)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    kk, vv = k[b, :, hk, :], v[b, :, hk, :]
    dq = np.zeros((G, rows.size, D))
    dk = np.zeros((cols.size, D))
    dv = np.zeros((cols.size, D))
    for g in range(G):
        hq = hk * G + g
        hm = hq * Hm // Hq
        mod = None if score_mod is None else (
            lambda sc, bb, h_, qi, kj, hq=hq: score_mod(sc, b, hq, qi, kj))
        out, lse = attention_fwd(q[b:b + 1, :, hq:hq + 1], k[b:b + 1, :, hk:hk + 1], v[b:b + 1, :, hk:hk + 1],
                                 lambda bb, h_, rr: allowed(b, hm, rr), scale, chunk=chunk, score_mod=mod)
        L = lse[0, 0]
        delta = (do[b, :, hq, :] * out[0, :, 0, :]).sum(axis=1)
        qq, dd = q[b, :, hq, :], do[b, :, hq, :]
        # dQ rows
        a = np.asarray(allowed(b, hm, rows), dtype=bool)
        s = _scores(qq[rows], kk, scale, score_mod, b, hq, rows)
        fin = np.isfinite(L[rows])
        P = np.where(a & fin[:, None], np.exp(s - np.where(fin, L[rows], 0.0)[:, None]), 0.0)
        dP = dd[rows] @ vv.T
        gm = _mod_grad(qq[rows], kk, scale, score_mod, b, hq, rows)
        dq[g] = scale * ((P * (dP - delta[rows][:, None]) * gm) @ kk)
        # dK / dV columns, all query rows in chunks
        for c0 in range(0, Sq, chunk):
            rr = np.arange(c0, min(c0 + chunk, Sq))
            a = np.asarray(allowed(b, hm, rr), dtype=bool)[:, cols]
            s = scale * (qq[rr] @ kk[cols].T)
            if score_mod is not None:
                s = score_mod(s, b, hq, rr[:, None], cols[None, :])
            fin = np.isfinite(L[rr])
            P = np.where(a & fin[:, None], np.exp(s - np.where(fin, L[rr], 0.0)[:, None]), 0.0)
            dP = dd[rr] @ vv[cols].T
            dS = P * (dP - delta[rr][:, None]) * _mod_grad(qq[rr], kk[cols], scale, score_mod, b, hq, rr, cols)
            dv += P.T @ dd[rr]
            dk += scale * (dS.T @ qq[rr])
    return dq, dk, dv


def attention_bwd_dq_rows(q, k, v, dout, allowed, scale, rows, score_mod=None):
    """dQ of the query rows ``rows`` for every query head, fp64.

    dQ_i depends on row i alone: its scores s_i over the allowed keys, its
    LSE_i, P_i = exp(s_i - LSE_i), O_i = P_i V, Delta_i = dO_i . O_i,
    dP_i = dO_i V^T, dS_i = P_i (dP_i - Delta_i) and dQ_i = scale dS_i K
    (the formulas of ``attention_bwd`` restricted to one row), so sampled rows
    are checked without forming any other row. A row with no allowed key has
    dQ_i = 0. ``allowed`` and ``score_mod`` as for ``attention_fwd``.
    Returns dq (B, len(rows), Hq, D).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    Hm = _mask_heads(allowed, Hq)
    rows = np.asarray(rows)
    dq = np.zeros((B, rows.size, Hq, D))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            hm = hq * Hm // Hq
            kk, vv = k[b, :, hk, :], v[b, :, hk, :]
            a = _mask_rows(allowed, b, hm, rows, Sk)
            has = a.any(axis=1)
            s = _scores(q[b, rows, hq, :], kk, scale, score_mod, b, hq, rows)
            sm = np.where(a, s, -np.inf)
            m = np.where(has, sm.max(axis=1, initial=-np.inf), 0.0)
            e = np.where(a, np.exp(sm - m[:, None]), 0.0)
            lse = m + np.log(np.where(has, e.sum(axis=1), 1.0))
            P = np.where(a, np.exp(sm - lse[:, None]), 0.0)
            o = P @ vv
            dd = do[b, rows, hq, :]
            delta = (dd * o).sum(axis=1)
            dP = dd @ vv.T
            gm = _mod_grad(q[b, rows, hq, :], kk, scale, score_mod, b, hq, rows)
            dq[b, :, hq, :] = scale * ((P * (dP - delta[:, None]) * gm) @ kk)
    return dq
