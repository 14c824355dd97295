"""The library driven from C alone (tests/c_abi/mfa_c_demo.cpp: HIP runtime
plus mfa.h, no Python or torch): dense mask -> tiles -> bf16 forward. Its
output must match the oracle on the same SplitMix64 inputs, rebuilt here."""

import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests.gpu_util import BF16_OUT_TOL, LSE_TOL, note
from workloads.splitmix import uniform_pm1

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c_abi", "mfa_c_demo")


def test_c_only_client_matches_oracle(tmp_path):
    note("C ABI client")
    assert os.path.exists(DEMO), "tests/c_abi/mfa_c_demo is not built (run __graft_entry__.build())"
    out_file = tmp_path / "out.bin"
    env = dict(os.environ, MFA_LOG="1")
    r = subprocess.run([DEMO, str(out_file)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, f"C client failed ({r.returncode}): {r.stdout} {r.stderr}"
    # MFA_LOG: each launching call names its kernel variant and grid
    assert "[mfa] compact_dense_mask Nq=300 Nk=300 BM=128 BN=64" in r.stderr, r.stderr
    assert "[mfa] attn_fwd bf16 D=128 mask=tiles BM=128 grid=6 x 256 threads" in r.stderr, r.stderr
    N, H, D = 300, 2, 128
    n = N * H * D
    raw = np.fromfile(out_file, dtype=np.uint8)
    out = torch.from_numpy(raw[:2 * n].copy().view(np.int16)).view(torch.bfloat16).double().numpy().reshape(1, N, H, D)
    lse = raw[2 * n:].copy().view(np.float32).astype(np.float64).reshape(1, H, N)
    st = 20261203
    qkv = []
    for _ in range(3):
        x, st = uniform_pm1(st, n)
        qkv.append(torch.from_numpy(x).to(torch.bfloat16).reshape(1, N, H, D))
    i = np.arange(N)
    mask = (i[None, :] <= i[:, None]) & (i[:, None] - i[None, :] < 100)
    ro, rl = A.attention_fwd(*qkv, mask[None, None], D ** -0.5)
    assert float(np.abs(out - ro).max()) <= BF16_OUT_TOL
    assert float(np.abs(lse - rl).max()) <= LSE_TOL
