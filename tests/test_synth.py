"""The seeded input generator (CPU only): shapes, determinism and structure."""
import torch

import synth


def test_tiny_workload_shape_and_block_table_is_a_permutation():
    inp = synth.make_inputs("tiny")
    assert inp["q"].shape == (1, 8, 64) and inp["q"].dtype == torch.bfloat16
    assert inp["k_pages"].shape == (16, 16, 2, 64)
    assert inp["context_lens"].tolist() == [256]
    assert sorted(inp["block_table"][0].tolist()) == list(range(16))
    assert bool(torch.isfinite(inp["k_pages"].float()).all())


def test_generator_is_deterministic_per_seed():
    w = synth.WORKLOADS["llama3_8b"].with_(batch=4)
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    c = synth.make_inputs(w, seed=w.seed + 1)
    for key in ("q", "block_table", "context_lens"):
        assert torch.equal(a[key], b[key])
    assert torch.equal(a["k_pages"].view(torch.int16), b["k_pages"].view(torch.int16))
    assert not torch.equal(a["q"], c["q"])


def test_ragged_lengths_pool_and_unreferenced_pages():
    w = synth.WORKLOADS["llama3_8b"].with_(batch=6)
    inp = synth.make_inputs(w)
    lens = inp["context_lens"]
    assert bool(((lens >= 512) & (lens <= 4096)).all())
    needed = ((lens + 15) // 16).tolist()
    bt = inp["block_table"]
    assert inp["k_pages"].shape[0] == 2 * sum(needed)
    used = []
    for b, n in enumerate(needed):
        assert bool((bt[b, :n] >= 0).all()) and bool((bt[b, n:] == -1).all())
        used += bt[b, :n].tolist()
    assert len(set(used)) == len(used)                     # no page named twice
    unused = sorted(set(range(inp["k_pages"].shape[0])) - set(used))
    assert bool(torch.isnan(inp["k_pages"][unused].float()).all())
    assert bool(torch.isfinite(inp["v_pages"][used].float()).all())


def test_fp8_workload_codes_and_scales():
    w = synth.WORKLOADS["fp8_kv"].with_(batch=3)
    inp = synth.make_inputs(w)
    assert inp["k_pages"].dtype == torch.float8_e4m3fn
    assert inp["k_scale"].shape == inp["k_pages"].shape[:3]
    bt = inp["block_table"]
    used = bt[bt >= 0].long()
    k = inp["k_pages"][used].to(torch.float32)
    assert bool(torch.isfinite(k).all())
    assert float(k.abs().amax()) == 448.0
    assert bool((inp["k_scale"][used] > 0).all())


def test_kv_bytes_counts_k_v_and_fp8_scales():
    lens = torch.tensor([10, 20], dtype=torch.int32)
    w = synth.WORKLOADS["llama3_8b"]
    assert synth.kv_bytes(w, lens) == 30 * 8 * 2 * 128 * 2
    w8 = synth.WORKLOADS["fp8_kv"]
    assert synth.kv_bytes(w8, lens) == 30 * 8 * (2 * 128 + 8)
