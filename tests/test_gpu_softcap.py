"""Soft-cap score_mod (softcap * tanh(x / softcap), tensorplay omni_attention,
intro) in the forward and both backward passes, for every mask kind, against
the fp64 oracle's softcap mod (whose backward multiplies dS by the cap's
derivative): bf16 outputs at 2e-2 and gradients at 2e-2 plus one bf16 ULP
plus the first-order bf16 storage bound from the oracle's term sums; the fp32
test mode at 1e-4 everywhere. Also with ALiBi slopes (bias first, then the
cap), through the autograd wrapper, and the argument check."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from masked_flash_attention_amd import _ffi
from oracle import attention as A
from oracle import masks as M
import workloads as W
from tests.gpu_util import (BF16_OUT_TOL, DEV, F32_OUT_TOL, compare_attention, f64, grad_tolerance_terms, nan_like,
                            note, to_dev)
from tests.test_gpu_alibi import _case, geometric_slopes

pytestmark = pytest.mark.gpu


def _run(q, k, v, do, rep, scale, layout, cap, dtype, slopes=None):
    qd, kd, vd, dod = (to_dev(t, dtype) for t in (q, k, v, do))
    sd = None if slopes is None else to_dev(np.asarray(slopes, np.float32))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, layout, alibi_slopes=sd, softcap=cap)
    g = (nan_like(qd), nan_like(kd), nan_like(vd))
    mfa.attn_bwd(qd, kd, vd, out, lse, dod, rep, scale, layout, alibi_slopes=sd, softcap=cap, dq=g[0], dk=g[1],
                 dv=g[2])
    torch.cuda.synchronize()
    return out, lse, g


def _check(out, lse, got, ref, dtype, tag):
    ro, rl = ref[3], ref[4]
    tol = BF16_OUT_TOL if dtype == torch.bfloat16 else F32_OUT_TOL
    compare_attention(f64(out), f64(lse), ro, rl, tol)
    for name, g, r, t in zip(("dq", "dk", "dv"), got, ref[:3], ref[6]):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite (unwritten) gradient"
        bound = grad_tolerance_terms(r, t) if dtype == torch.bfloat16 else F32_OUT_TOL
        excess = np.abs(g - r) - bound
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        assert excess[i] <= 0, f"{tag} {name}: |{g[i]:.5f} - {r[i]:.5f}| over the bound at {i}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["tiles", "none", "blockid", "bsr"])
def test_softcap_forward_backward(kind, D, dtype):
    note(f"softcap {kind} D={D} {dtype}")
    q, k, v, do, rep, allowed, scale, layout, Hq = _case(kind, D)
    q = q * 3.0  # scores of a few units: the cap of 2 bends most of them
    out, lse, got = _run(q, k, v, do, rep, scale, layout, 2.0, dtype)
    ref = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=A.softcap(2.0), term_sums=True)
    _check(out, lse, got, ref, dtype, f"softcap {kind}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["tiles", "bsr"])
def test_softcap_after_alibi(kind, dtype):
    note(f"softcap + alibi {kind} {dtype}")
    q, k, v, do, rep, allowed, scale, layout, Hq = _case(kind, 128)
    sl = geometric_slopes(Hq).astype(np.float32)
    out, lse, got = _run(q, k, v, do, rep, scale, layout, 5.0, dtype, slopes=sl)
    mod = A.softcap(5.0, A.alibi(sl.astype(np.float64)))
    ref = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=mod, term_sums=True)
    _check(out, lse, got, ref, dtype, f"softcap+alibi {kind}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_softcap_varlen(dtype):
    note(f"softcap varlen {dtype}")
    L = np.array([1, 128, 129, 0, 300, 7, 64, 200], np.int32)
    T = int(L.sum())
    q, k, v, do = W.tensors(770, [(T, 4, 64), (T, 2, 64), (T, 2, 64), (T, 4, 64)])
    q = q * 3.0
    s = mfa.varlen_schedule(to_dev(L), causal=True, window=(100, 0), work_cap=T // 128 + L.size)
    rep = mfa.MaskRep.varlen(s, int(L.max()), int(L.max()), causal=True, window=(100, 0))
    out, lse, got = _run(q, k, v, do, rep, 0.125, "thd", 1.5, dtype)
    cu = M.cu_seqlens(L)
    allowed = M.varlen_mask(cu, cu, True, 100, 0)
    ref = A.attention_bwd(q[None], k[None], v[None], do[None], allowed[None, None], 0.125,
                          score_mod=A.softcap(1.5), term_sums=True)
    _check(out[None], lse[None], [g[None] for g in got], ref, dtype, "softcap varlen")


def test_softcap_autograd_wrapper():
    note("softcap autograd wrapper")
    q, k, v, do, rep, allowed, scale, layout, Hq = _case("tiles", 64)
    q = q * 3.0
    qd, kd, vd = (to_dev(t).requires_grad_(True) for t in (q, k, v))
    out = mfa.masked_attention(qd, kd, vd, rep, scale, layout, softcap=2.5)
    out.backward(to_dev(do))
    torch.cuda.synchronize()
    ref = A.attention_bwd(q, k, v, do, allowed, scale, score_mod=A.softcap(2.5), term_sums=True)
    assert float(np.abs(f64(out.detach()) - ref[3]).max()) <= BF16_OUT_TOL
    for name, g, r, t in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref[:3], ref[6]):
        assert np.all(np.abs(f64(g) - r) <= grad_tolerance_terms(r, t)), name


@pytest.mark.parametrize("cap", [-1.0, float("nan"), float("inf")])
def test_softcap_must_be_finite_and_nonnegative(cap):
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(_ffi.MfaError) as e:
        mfa.attn_fwd(q, q, q, mfa.MaskRep.none(), 0.125, "bshd", softcap=cap)
    assert e.value.status_name == "MFA_E_ARG"
