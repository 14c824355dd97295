"""Degenerate sizes of the mask builders: empty query or key axes give the
empty representations (all offsets zero; they are written by a kernel, not a
memset, so that the calls stay capturable)."""

import numpy as np
import pytest
import torch

import masked_flash_attention_amd as mfa
from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(0, 10), (10, 0), (0, 0)])
@pytest.mark.parametrize("BM", [64, 128])
def test_compaction_of_empty_masks(shape, BM):
    note(f"empty compaction {shape} BM={BM}")
    c = mfa.compact_dense_mask(torch.zeros(shape, dtype=torch.bool, device=DEV), BM=BM)
    torch.cuda.synchronize()
    assert c["row_ptr"].cpu().tolist() == [0] * c["row_ptr"].numel()


def test_predicate_and_coarsening_with_no_queries():
    note("empty predicate / coarsening")
    got = mfa.predicate_tiles(mfa.Pred.causal(), 0, 64)
    c64 = mfa.compact_dense_mask(torch.ones(0, 64, dtype=torch.bool, device=DEV), BM=64)
    c128 = mfa.coarsen_tile_map(c64, 0, 64)
    torch.cuda.synchronize()
    assert got["row_ptr"].cpu().tolist() == [0]
    assert c128["row_ptr"].cpu().tolist() == [0]


@pytest.mark.parametrize("R,nKb", [(0, 5), (3, 0)])
def test_bitmask_with_no_rows_or_no_blocks(R, nKb):
    note(f"empty bitmask R={R} nKb={nKb}")
    bits = torch.zeros(2, 3, R, (nKb + 31) // 32, dtype=torch.int32, device=DEV)
    ip, ix = mfa.bsr_from_bitmask(bits, nKb)
    torch.cuda.synchronize()
    assert ip.shape == (2, 3, R + 1) and np.all(ip.cpu().numpy() == 0)
