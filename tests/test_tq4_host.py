"""Host-side TQ4 calls of the C-ABI library (no GPU needed): the library's
codebook against the oracle's Lloyd-Max iteration, and the TQ4 planner's
argument checks and sizing (num_cus given, so no device is asked)."""
import numpy as np
import pytest
import torch

from oracle import tq4 as otq


def _pk():
    import paged_kv_split_amd as pk
    return pk


@pytest.mark.parametrize("d", [1, 64, 128, 256, 300])
def test_library_codebook_equals_oracle(d):
    pk = _pk()
    c, b = pk.tq4_codebook(d)
    oc, ob = otq.codebook(d)
    assert np.array_equal(c.numpy(), oc)
    # the middle boundary is 0 up to the iteration's last bits
    assert np.allclose(b.numpy(), ob, rtol=1e-6, atol=1e-12)
    assert np.all(np.diff(c.numpy()) > 0)


def _problem(pk, B=4, Hq=32, Hkv=8, D=128, P=16, max_pages=64, num_pages=256):
    cache = torch.empty((num_pages, Hkv, P, D + 8), dtype=torch.uint8)
    bt = torch.zeros((B, max_pages), dtype=torch.int32)
    return pk.tq4_problem((B, Hq), cache, bt)


def test_tq4_plan_sizes_and_checks():
    pk = _pk()
    prob = _problem(pk)
    lens = torch.tensor([0, 17, 1000, 1024], dtype=torch.int32)
    pl = pk.tq4_plan(prob, lens, num_cus=256)
    assert pl.total_tiles == 8 * (0 + 2 + 63 + 64)
    assert pl.chunk_tiles >= 4 and pl.max_chunks == -(-64 // pl.chunk_tiles)
    G, D, pairs = 4, 128, 32
    rec = ((2 * G + 3) // 4 * 4 + G * D) * 4
    qseq = -(-(4 * 32 * D * 2) // 256) * 256
    assert pl.workspace_bytes == qseq + pl.max_chunks * pairs * rec
    forced = pk.tq4_plan(prob, lens, num_cus=256, chunk_tiles=3)
    assert forced.chunk_tiles == 3 and forced.max_chunks == 22
    with pytest.raises(pk.PdattnError):        # a length beyond the block table
        pk.tq4_plan(prob, torch.tensor([0, 0, 0, 64 * 16 + 1], dtype=torch.int32), num_cus=256)
    bad = _problem(pk)
    bad.kv_layout = pk.LAYOUT_NHD
    with pytest.raises(pk.PdattnError):
        pk.tq4_plan(bad, lens, num_cus=256)
    bad = _problem(pk)
    bad.kv_dtype = pk.KV_BF16
    with pytest.raises(pk.PdattnError):
        pk.tq4_plan(bad, lens, num_cus=256)
    bad = _problem(pk)
    bad.q_len = 4
    with pytest.raises(pk.PdattnError):
        pk.tq4_plan(bad, lens, num_cus=256)
    with pytest.raises(pk.PdattnError):        # the other planners refuse TQ4 problems
        pk.plan(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, max_pages_per_seq=64,
                num_pages=256, kv_dtype=pk.KV_TQ4, kv_layout=pk.LAYOUT_HND, context_lens_host=lens, num_cus=256)
