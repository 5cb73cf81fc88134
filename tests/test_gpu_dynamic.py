"""The balanced mode's own contract, on the GPU through the C ABI:
the workspace counters return to zero after every call, an unprepared
workspace is refused by NaN outputs, one workspace serves successive plans,
and the on-device split (static shares, claims, helper memberships, pairs
cut into several units, merges) matches the oracle for extreme worker
counts."""
import math

import pytest
import torch

import synth
from test_gpu_parity import assert_parity, gpu_run, oracle_run, small, to_dev, two_run_bound

pytestmark = pytest.mark.gpu

UNIT_TILES = 512  # tiles of one balancing unit (csrc/kernels.h)


def _pk():
    import paged_kv_split_amd as pk
    return pk


def run_with(pl, d, ws, out=None, lse=None):
    pk = _pk()
    B, Hq, D = d["q"].shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda") if lse is None else lse
    pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
              d["context_lens"], ws, out, lse)
    pk.reduce(pl, ws, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def make_plan(inp, **kw):
    pk = _pk()
    w = inp["workload"]
    kw.setdefault("balanced", True)
    return pk.plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                   page_size=w.page_size, max_pages_per_seq=inp["block_table"].shape[1],
                   num_pages=inp["k_pages"].shape[0], kv_dtype=0 if w.kv_dtype == "bf16" else 1,
                   context_lens_host=inp["context_lens"], **kw)


def counter_words(pl, inp):
    """The counter region of a balanced-mode workspace: after the 256-byte
    header, claims / records / done tiles per unit, then done units per pair."""
    w = inp["workload"]
    P = w.page_size
    max_tiles = math.ceil(inp["block_table"].shape[1] * P / 16)
    seg_max = max(1, math.ceil(max_tiles / UNIT_TILES))
    units_max = w.batch * w.num_kv_heads * seg_max
    return 64, 3 * units_max + w.batch * w.num_kv_heads


@pytest.mark.parametrize("name", ["llama3_8b", "many_short", "long_ctx"])
def test_counters_return_to_zero_after_every_call(name):
    inp = synth.make_inputs(name)
    d = to_dev(inp)
    pl = make_plan(inp)
    pk = _pk()
    ws = pk.workspace(pl, "cuda")
    first, nwords = counter_words(pl, inp)
    ref = oracle_run(inp)
    for it in range(3):
        out, lse = run_with(pl, d, ws)
        assert_parity(out, lse, *ref, tag=f"{name} call {it}")
        words = ws.view(torch.int32)[first:first + nwords].cpu()
        assert int((words != 0).sum()) == 0, f"{name} call {it}: {int((words != 0).sum())} counters left non-zero"


def test_unprepared_workspace_gives_nan():
    inp = synth.make_inputs("tiny")
    d = to_dev(inp)
    pl = make_plan(inp)
    ws = torch.zeros(int(pl.workspace_bytes), dtype=torch.uint8, device="cuda")  # no stamp
    out, lse = run_with(pl, d, ws)
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(lse).all())
    _pk().workspace_init(pl, ws)
    out, lse = run_with(pl, d, ws)
    assert_parity(out, lse, *oracle_run(inp), tag="after init")


def test_one_workspace_serves_successive_plans():
    # one counter layout (batch, kv heads, block table), different lengths
    # and worker counts; a plan with another layout is refused until the
    # workspace is prepared again
    pk = _pk()
    cases = [small(B=6, Hq=8, Hkv=2, D=128, P=16, lens=("uniform", 1, 3000), seed=401),
             small(B=6, Hq=8, Hkv=2, D=128, P=16, lens=("uniform", 0, 200), seed=402),
             small(B=6, Hq=8, Hkv=2, D=128, P=16, lens=("fixed", (3000, 1, 2999, 0, 17, 2048)), seed=403)]
    inps = [synth.make_inputs(c) for c in cases]
    width = max(i["block_table"].shape[1] for i in inps)
    for i in inps:  # one block-table width for all
        bt = torch.full((6, width), -1, dtype=torch.int32)
        bt[:, :i["block_table"].shape[1]] = i["block_table"]
        i["block_table"] = bt
    plans = [make_plan(i, force_workers=f) for i, f in zip(inps, (0, 37, 5))]
    ws = torch.empty(max(int(p.workspace_bytes) for p in plans), dtype=torch.uint8, device="cuda")
    pk.workspace_init(plans[0], ws)
    for rnd in range(2):
        for inp, pl in zip(inps, plans):
            out, lse = run_with(pl, to_dev(inp), ws)
            assert_parity(out, lse, *oracle_run(inp), tag=f"round {rnd} workers={pl.num_workers}")
    other = synth.make_inputs(small(B=64, Hq=8, Hkv=2, D=128, P=16, lens=("uniform", 0, 200), seed=404))
    pl = make_plan(other)
    big = torch.empty(max(int(pl.workspace_bytes), ws.numel()), dtype=torch.uint8, device="cuda")
    big[:ws.numel()].copy_(ws)  # prepared for the first layout
    out, lse = run_with(pl, to_dev(other), big)
    assert bool(torch.isnan(out).all())
    pk.workspace_init(pl, big)
    out, lse = run_with(pl, to_dev(other), big)
    assert_parity(out, lse, *oracle_run(other), tag="after preparing the new layout")


@pytest.mark.parametrize("force", [1, 2, 5, 33, 400, 3000])
def test_pairs_cut_into_several_units(force):
    # 1250- and 2600-tile pairs: three and six units, merged twice
    w = small(B=2, Hq=8, Hkv=2, D=64, P=32, lens=("fixed", (20000, 41600)), seed=404)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=force, balanced=True)
    assert_parity(out, lse, *oracle_run(inp), tag=f"multi-unit workers={force}")


@pytest.mark.parametrize("force", [1, 3, 16, 128, 1024, 4096])
def test_many_small_units_and_extreme_worker_counts(force):
    # units of 1..32 tiles; workers from one to more than the tiles
    w = small(B=40, Hq=16, Hkv=4, D=128, P=8, lens=("uniform", 1, 512), seed=405)
    inp = synth.make_inputs(w)
    out, lse = gpu_run(inp, force_workers=force, balanced=True)
    assert_parity(out, lse, *oracle_run(inp), tag=f"small units workers={force}")


def test_balanced_fp8_long_pairs():
    w = small(B=3, Hq=16, Hkv=2, D=128, P=64, lens=("fixed", (9000, 17000, 33000)), kv="fp8_e4m3", seed=406)
    inp = synth.make_inputs(w)
    ref = oracle_run(inp)
    for force in (0, 7, 300):
        out, lse = gpu_run(inp, force_workers=force, balanced=True)
        assert_parity(out, lse, *ref, fp8=True, tag=f"fp8 long workers={force}")


@pytest.mark.parametrize("balanced", [False, True], ids=["static", "balanced"])
def test_graph_replay_matches_eager(balanced):
    # capture decode + reduce once, replay several times with eager work in
    # between; every replay equals the eager result (to rounding when the
    # split is decided on the device)
    inp = synth.make_inputs("llama3_8b")
    d = to_dev(inp)
    pl = make_plan(inp, balanced=balanced)
    pk = _pk()
    ws = pk.workspace(pl, "cuda")
    eager_out, eager_lse = run_with(pl, d, ws)
    B, Hq, D = d["q"].shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_with(pl, d, ws, out, lse)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                  d["context_lens"], ws, out, lse)
        pk.reduce(pl, ws, out, lse)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert float((out.cpu() - eager_out).abs().max()) <= two_run_bound(inp), rep
        assert float((lse.cpu() - eager_lse).abs().max()) <= 1e-5, rep
        run_with(pl, d, ws)  # eager work between replays
