"""The dK/dV entry point that allocates nothing (mfa_attn_bwd_dkdv_noalloc),
through the C ABI, against mfa_attn_bwd_dkdv with a workspace of the
preferred size: two calls in a row, the second on a smaller problem (the
static scratch still holds the first call's sums), each bit-identical to the
workspace path (same split, same kernels, same order of additions), plus the
rejection of a split whose sums exceed the scratch. Outputs are NaN-filled."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from masked_flash_attention_amd import _ffi
import workloads as W
from tests.gpu_util import DEV, nan_like, note, to_dev

pytestmark = pytest.mark.gpu


def _setup(q, k, v, do, rep, scale):
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    out, lse = mfa.attn_fwd(qd, kd, vd, rep, scale, "bshd")
    B, Sq, Sk, Hq, Hkv, D = mfa._dims(qd, kd, "bshd")
    delta = torch.empty(B, Hq, Sq, dtype=torch.float32, device=DEV)
    dq = torch.empty_like(qd)
    return qd, kd, vd, dod, out, lse, dq, delta


def _dkdv(state, rep, scale, noalloc):
    qd, kd, vd, dod, out, lse, dq, delta = state
    dk, dv = nan_like(kd), nan_like(vd)
    a = mfa._bwd_args(qd, kd, vd, out, lse, dod, dq, dk, dv, delta, "bshd")
    mfa.attn_bwd_preprocess(a)
    nbytes, splits = mfa.attn_bwd_dkdv_workspace(a, rep)
    if noalloc:
        mfa.attn_bwd_dkdv_noalloc(a, rep, scale)
    else:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes else None
        mfa.attn_bwd_dkdv(a, rep, scale, workspace=ws)
    torch.cuda.synchronize()
    return dk, dv, splits, nbytes


def _compare(state, rep, scale, tag):
    dk0, dv0, splits, nbytes = _dkdv(state, rep, scale, noalloc=False)
    dk1, dv1, _, _ = _dkdv(state, rep, scale, noalloc=True)
    assert splits > 1 and 0 < nbytes <= mfa.bwd_scratch_bytes(), (splits, nbytes)
    for name, x, y in (("dk", dk1, dk0), ("dv", dv1, dv0)):
        assert torch.isfinite(x.float()).all(), f"{tag} {name}: unwritten rows"
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{tag} {name}: differs from the workspace path"


def test_noalloc_matches_workspace_path_twice():
    # first call: the block-id GQA workload with cross columns (B=8, N=1024,
    # Hq=16, Hkv=2, D=128; a 4-way split, 80 MiB of sums)
    note("noalloc dkdv: block-id GQA with cross columns, full size")
    w = W.blockcausal_gqa_cross()
    ids = mfa.make_block_ids(to_dev(w["pad"]), to_dev(w["att"]), w["n_cross"], to_dev(w["cross_pad"]))
    rep = mfa.MaskRep.blockid(*ids, summary=mfa.blockid_tile_summary(*ids))
    do = W.tensors(920, [tuple(w["q"].shape)])[0]
    _compare(_setup(w["q"], w["k"], w["v"], do, rep, w["scale"]), rep, w["scale"], "gqa cross")
    # second call, smaller: dense-tile mask, B=2, Sq=300, Sk=333, Hq=8, Hkv=2, D=64
    note("noalloc dkdv: small dense-tile GQA after the large call")
    m = W.random_dense_mask(300, 333, 0.3, seed=921)
    q, k, v, do = W.tensors(922, [(2, 300, 8, 64), (2, 333, 2, 64), (2, 333, 2, 64), (2, 300, 8, 64)])
    rep = mfa.MaskRep.tiles(mfa.compact_dense_mask(to_dev(m)))
    _compare(_setup(q, k, v, do, rep, 0.125), rep, 0.125, "small tiles")


def test_noalloc_rejects_sums_larger_than_the_scratch():
    """B=1, Sk=14000, Hkv=1, Hq=8, D=128: 219 key blocks, an 8-way split whose
    sums take 8 * 2 * 14000 * 128 * 4 bytes (109 MiB) > 96 MiB: refused before
    any launch, dk untouched; the workspace path still runs it."""
    note("noalloc dkdv: split larger than the scratch")
    Sq, Sk = 64, 14000
    q, k, v, do = W.tensors(923, [(1, Sq, 8, 128), (1, Sk, 1, 128), (1, Sk, 1, 128), (1, Sq, 8, 128)])
    rep = mfa.MaskRep.none()
    state = _setup(q, k, v, do, rep, 0.088)
    qd, kd, vd, dod, out, lse, dq, delta = state
    dk, dv = nan_like(kd), nan_like(vd)
    a = mfa._bwd_args(qd, kd, vd, out, lse, dod, dq, dk, dv, delta, "bshd")
    mfa.attn_bwd_preprocess(a)
    nbytes, splits = mfa.attn_bwd_dkdv_workspace(a, rep)
    assert splits == 8 and nbytes > mfa.bwd_scratch_bytes()
    with pytest.raises(_ffi.MfaError) as e:
        mfa.attn_bwd_dkdv_noalloc(a, rep, 0.088)
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(dk.float()).all()
    dk0, dv0, _, _ = _dkdv(state, rep, 0.088, noalloc=False)
    assert torch.isfinite(dk0.float()).all() and torch.isfinite(dv0.float()).all()
