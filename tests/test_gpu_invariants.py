"""Invariants and edge cases of the HIP path (through the C ABI), checked on
the GPU against the oracle or against the definition's own invariants
(the page permutation, NaN-poisoned unused memory, shared pages, the split
points, single tokens, empty and invalid lengths)."""
import math

import pytest
import torch

import oracle
import synth
from test_gpu_parity import assert_parity, gpu_run, oracle_run, small, to_dev, two_run_bound

pytestmark = pytest.mark.gpu


def test_bitwise_deterministic_for_a_fixed_plan():
    inp = synth.make_inputs("llama3_8b")
    a = gpu_run(inp)
    b = gpu_run(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_balanced_mode_repeats_to_rounding():
    # the split points move with timing; the result moves only by rounding
    inp = synth.make_inputs("llama3_8b")
    a = gpu_run(inp, balanced=True)
    for _ in range(3):
        b = gpu_run(inp, balanced=True)
        assert float((a[0] - b[0]).abs().max()) <= two_run_bound(inp)
        assert float((a[1] - b[1]).abs().max()) <= 1e-5


def test_result_does_not_depend_on_the_split_points():
    w = small(B=6, Hq=8, Hkv=2, D=128, P=16, lens=("uniform", 1, 2000), seed=301)
    inp = synth.make_inputs(w)
    ref = oracle_run(inp)
    outs = []
    for bal in (False, True):
        for force in (1, 2, 3, 17, 100, 500, 4000):
            out, lse = gpu_run(inp, force_workers=force, balanced=bal)
            assert_parity(out, lse, *ref, tag=f"workers={force} balanced={bal}")
            outs.append((out, lse))
    for out, lse in outs[1:]:
        assert float((out - outs[0][0]).abs().max()) <= two_run_bound(inp)
        assert float((lse - outs[0][1]).abs().max()) <= 1e-5


def test_single_token_returns_its_v_row_bitwise():
    w = small(B=9, Hq=16, Hkv=4, D=128, P=16, lens=("fixed", (1,) * 9), seed=302)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp)
    for b in range(9):
        page = int(inp["block_table"][b, 0])
        for h in range(16):
            v = inp["v_pages"][page, 0, h // 4].to(torch.float32)
            assert torch.equal(out[b, h], v), (b, h)


def test_constant_v_returns_the_constant():
    w = small(B=4, Hq=8, Hkv=2, D=64, P=8, lens=("uniform", 1, 900), seed=303)
    inp = synth.make_inputs(w)
    c = torch.linspace(-2, 2, 64).to(torch.bfloat16)
    inp["v_pages"] = c.expand_as(inp["v_pages"]).contiguous()
    out, _ = gpu_run(inp, force_workers=13)
    assert float((out - c.float()).abs().max()) <= 1e-5


def test_page_permutation_is_bitwise_invisible():
    w = small(B=5, Hq=8, Hkv=2, D=128, P=16, lens=("uniform", 100, 1500), seed=304)
    inp = synth.make_inputs(w)
    a = gpu_run(inp, force_workers=37)
    n = inp["k_pages"].shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9))
    moved = dict(inp)
    for key in ("k_pages", "v_pages"):
        dst = torch.empty_like(inp[key])
        dst[perm] = inp[key]
        moved[key] = dst
    bt = inp["block_table"].clone()
    bt[bt >= 0] = perm[bt[bt >= 0].long()].to(torch.int32)
    moved["block_table"] = bt
    b = gpu_run(moved, force_workers=37)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_nan_poison_outside_the_context_does_not_leak():
    w = small(B=4, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (3, 17, 250, 1000)), seed=305)
    clean = synth.make_inputs(w, unused="zero")
    poisoned = synth.make_inputs(w, unused="nan")
    for key in ("k_pages", "v_pages"):
        for b in range(4):
            L = int(poisoned["context_lens"][b])
            last = int(poisoned["block_table"][b, (L - 1) // 16])
            poisoned[key][last, (L - 1) % 16 + 1:] = float("nan")
    a = gpu_run(clean, force_workers=9)
    b = gpu_run(poisoned, force_workers=9)
    assert bool(torch.isfinite(b[0]).all())
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_nan_poison_outside_the_context_does_not_leak():
    w = small(B=3, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (5, 70, 333)), kv="fp8_e4m3", seed=306)
    inp = synth.make_inputs(w, unused="nan")
    out, lse = gpu_run(inp, force_workers=5)
    assert bool(torch.isfinite(out).all())
    assert_parity(out, lse, *oracle_run(inp), fp8=True, tag="fp8 poison")


def test_shared_pages_give_identical_rows():
    w = small(B=4, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (700, 700, 700, 700)), seed=307)
    inp = synth.make_inputs(w)
    for b in (1, 2, 3):
        inp["block_table"][b] = inp["block_table"][0]
        inp["q"][b] = inp["q"][0]
    out, lse = gpu_run(inp, force_workers=1)   # one worker: every pair summed in the same order
    for b in (1, 2, 3):
        assert torch.equal(out[b], out[0]) and torch.equal(lse[b], lse[0])


def test_empty_sequences_mixed_with_others():
    w = small(B=6, Hq=8, Hkv=2, D=64, P=16, lens=("fixed", (0, 40, 0, 0, 300, 0)), seed=308)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=6)
    ref_out, ref_lse = oracle_run(inp)
    assert_parity(out, lse, ref_out, ref_lse, tag="empty mix")
    for b in (0, 2, 3, 5):
        assert torch.equal(out[b], torch.zeros_like(out[b]))
        assert bool(torch.isneginf(lse[b]).all())


def test_all_sequences_empty():
    w = small(B=3, Hq=4, Hkv=1, D=128, P=16, lens=("fixed", (0, 0, 0)), seed=309)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp)
    assert torch.equal(out, torch.zeros_like(out)) and bool(torch.isneginf(lse).all())


def test_out_of_range_block_table_entry_gives_nan_for_that_pair_only():
    w = small(B=3, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (100, 200, 300)), seed=310)
    inp = synth.make_inputs(w)
    ref_out, ref_lse = oracle_run(inp)
    bad = dict(inp)
    bad["block_table"] = inp["block_table"].clone()
    bad["block_table"][1, 3] = inp["k_pages"].shape[0] + 7     # never read through
    out, lse = gpu_run(bad, force_workers=1)                    # one worker: no cut pairs
    assert bool(torch.isnan(out[1]).all())
    for b in (0, 2):
        assert float((out[b].double() - ref_out[b]).abs().max()) <= 1e-2


def test_device_length_beyond_the_block_table_gives_nan():
    w = small(B=3, Hq=8, Hkv=2, D=64, P=16, lens=("fixed", (50, 60, 70)), seed=311)
    inp = synth.make_inputs(w)
    import paged_kv_split_amd as pk
    d = to_dev(inp)
    cap = inp["block_table"].shape[1] * 16
    d["context_lens"] = torch.tensor([50, cap + 16, 70], dtype=torch.int32, device="cuda")
    out, lse = pk.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                               context_lens_host=inp["context_lens"])
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert bool(torch.isnan(out[1]).all()) and bool(torch.isnan(lse[1]).all())
    ref_out, _ = oracle_run(inp)
    for b in (0, 2):
        assert float((out[b].double() - ref_out[b]).abs().max()) <= 1e-2


def test_fp8_every_code_decodes_as_the_oracle_does():
    # K and V rows hold every finite e4m3fn code, with unit and random scales
    w = small(B=2, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (64, 64)), kv="fp8_e4m3", seed=312)
    inp = synth.make_inputs(w)
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    g = torch.Generator().manual_seed(4)
    for key in ("k_pages", "v_pages"):
        raw = inp[key].view(torch.uint8)
        used = inp["block_table"][inp["block_table"] >= 0].long()
        n = raw[used].numel()
        fill = codes[torch.randint(0, codes.numel(), (n,), generator=g)]
        raw[used] = fill.view(raw[used].shape)
    for key in ("k_scale", "v_scale"):
        inp[key] = torch.where(torch.isnan(inp[key]), inp[key],
                               torch.rand(inp[key].shape, generator=g) * 2 ** -7)
    out, lse = gpu_run(inp, force_workers=3)
    assert_parity(out, lse, *oracle_run(inp), fp8=True, tag="fp8 all codes")


def test_many_sequences_exercise_the_chunked_length_scan():
    # B > 256 workgroup threads: every scan thread owns several sequences
    w = small(B=2048, Hq=4, Hkv=2, D=64, P=8, lens=("uniform", 0, 40), seed=313)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp)
    assert_parity(out, lse, *oracle_run(inp), tag="B2048")


def test_streaming_kernel_at_its_largest_batch():
    # 512 sequences, the streaming kernel's largest batch: the tile prefix's
    # last entry (the total) is one no pair of sequences per thread reaches
    w = small(B=512, Hq=8, Hkv=2, D=64, P=16, lens=("uniform", 1, 300), seed=316)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp)
    assert_parity(out, lse, *oracle_run(inp), tag="B512")


MERGE_STRIDE = [(4500, 8, ("uniform", 0, 40), 0), (1100, 8, ("uniform", 64, 160), 30000),
                (512, 32, ("uniform", 16, 400), 30000)]


@pytest.mark.parametrize("B,Hkv,lens,force", MERGE_STRIDE,
                         ids=["pair-per-wave", "pair-per-workgroup", "pair-per-workgroup-stream"])
def test_more_pairs_than_reduce_workgroups(B, Hkv, lens, force):
    # more (sequence, kv head) pairs than the reduce launches workgroups (8192
    # at most), so its grid strides over them; short pairs are merged one per
    # wave, pairs cut into more pieces (many forced workers) one per workgroup
    w = small(B=B, Hq=Hkv, Hkv=Hkv, D=64, P=16, lens=lens, seed=315 + B)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=force)
    assert_parity(out, lse, *oracle_run(inp), tag=f"B{B} Hkv{Hkv} workers {force}")


def test_long_single_sequence_with_one_worker_crosses_page_buffer_refills():
    # one worker walks 3000 pages (more than one 256-entry page buffer)
    w = small(B=1, Hq=8, Hkv=1, D=64, P=8, lens=("fixed", (24000,)), seed=314)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=1)
    assert_parity(out, lse, *oracle_run(inp), tag="long single worker")


def test_more_workers_than_tiles():
    w = small(B=2, Hq=4, Hkv=2, D=128, P=16, lens=("fixed", (20, 90)), seed=315)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=64)
    assert_parity(out, lse, *oracle_run(inp), tag="64 workers, 16 tiles")


def test_heads_of_a_group_with_equal_q_agree():
    w = small(B=3, Hq=16, Hkv=2, D=128, P=16, lens=("uniform", 10, 900), seed=316)
    inp = synth.make_inputs(w)
    inp["q"][:, 3] = inp["q"][:, 2]
    inp["q"][:, 12] = inp["q"][:, 15]
    out, lse = gpu_run(inp, force_workers=11)
    assert torch.equal(out[:, 2], out[:, 3]) and torch.equal(out[:, 12], out[:, 15])


@pytest.mark.parametrize("layout", [0, 1], ids=["NHD", "HND"])
def test_fp8_full_grid_takes_the_weighted_split(layout):
    """An fp8 pool planned on the device at the streaming kernel's full grid
    takes the 5:4 worker weights (the first half of the grid heavier); the
    outputs match the oracle, and an equal-weight plan with the same workers
    (forced) within the two-cut bound. Ragged lengths with an empty and a
    one-token sequence; every length spans many worker ranges."""
    import paged_kv_split_amd as pk
    lens = [0, 1] + [2100 + 97 * i for i in range(14)]
    w = synth.Workload("gpu-fp8-weights", "fp8 weighted split", 16, 32, 8, 128, 16, ("fixed", tuple(lens)),
                       kv_dtype="fp8_e4m3", seed=611)
    inp = synth.make_inputs(w)
    data = synth.to_hnd(inp) if layout == pk.LAYOUT_HND else inp
    dev = to_dev(data)
    pl = pk.plan(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                 max_pages_per_seq=data["block_table"].shape[1], num_pages=data["k_pages"].shape[0],
                 kv_dtype=pk.KV_FP8_E4M3, context_lens_host=inp["context_lens"], kv_layout=layout)
    assert pl.split_weights == (5 << 16) | 4, (pl.num_workers, pl.num_workgroups)
    out, lse = gpu_run(data, dev, layout=layout)
    assert_parity(out, lse, *oracle_run(inp), fp8=True, tag=f"fp8 weighted split layout={layout}")
    out_eq, lse_eq = gpu_run(data, dev, layout=layout, force_workers=pl.num_workers)
    assert float((out - out_eq).abs().max()) <= two_run_bound(inp)
    fin = torch.isfinite(lse)
    assert torch.equal(fin, torch.isfinite(lse_eq))      # the empty sequence: -inf in both
    assert float((lse[fin] - lse_eq[fin]).abs().max()) <= 1e-5
