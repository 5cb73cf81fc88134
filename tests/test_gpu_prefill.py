"""Ragged paged prefill on the GPU against the CPU oracle (oracle/prefill.py),
with the decode tolerances: bf16 out max-abs 1e-2 and mean-abs 1e-3, fp8
max-abs 4e-2, lse max-abs 1e-3; rows that see nothing must be exactly
out 0, lse -inf.

Cases span several query tiles per request and a ragged tail (rows per tile
= 128 / G, or 64 / G at head_dim 256), K/V tiles with a ragged tail, every
group size class, both pool layouts, both KV dtypes, page sizes 8 to 128,
causal and not, requests with no rows, contexts shorter than their rows,
and the bench's workloads at full size on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import prefill as pf

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _run(inp, *, layout="nhd", causal=True, longest_first=True, lens=None):
    pk = _pk()
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (src[k].to(DEV) if src.get(k) is not None else None)
         for k in ("q", "qo_indptr", "k_pages", "v_pages", "k_scale", "v_scale", "block_table")}
    lens = inp["context_lens"] if lens is None else lens
    out, lse = pk.paged_prefill(d["q"], d["qo_indptr"], d["k_pages"], d["v_pages"], d["block_table"], lens.to(DEV),
                                qo_indptr_host=inp["qo_indptr"], context_lens_host=inp["context_lens"],
                                k_scale=d["k_scale"], v_scale=d["v_scale"], causal=causal,
                                layout=pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD,
                                longest_first=longest_first)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _compare(out, lse, ref_o, ref_l, fp8, tag):
    diff = (out.double() - ref_o).abs()
    assert bool(torch.isfinite(out).all()), tag
    mx = float(diff.max()) if diff.numel() else 0.0
    mean = float(diff.mean()) if diff.numel() else 0.0
    print(f"{tag}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)
    assert mx <= (4e-2 if fp8 else 1e-2) and mean <= 1e-3, (tag, mx, mean)
    empty = torch.isneginf(ref_l)
    assert torch.equal(torch.isneginf(lse.double()), empty), tag
    assert bool((out[empty] == 0).all()), tag
    fin = torch.isfinite(ref_l)
    if bool(fin.any()):
        assert float((lse.double()[fin] - ref_l[fin]).abs().max()) <= 1e-3, tag


def _check(inp, out, lse, causal, tag):
    ref_o, ref_l = pf.prefill(inp["q"], inp["qo_indptr"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                              inp["context_lens"], causal=causal, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    _compare(out, lse, ref_o, ref_l, inp["k_scale"] is not None, tag)


# q lengths with several tiles and ragged tails; prefixes before them
Q_LENS = (70, 10, 130, 1, 0, 33)
PREFIX = (0, 37, 200, 5, 9, 300)

CASES = [
    # Hq, Hkv, D, P, kv dtype
    (32, 8, 128, 16, "bf16"),   # Llama-3-8B heads, G 4: 32 rows per tile
    (32, 8, 128, 16, "fp8_e4m3"),
    (8, 2, 64, 8, "bf16"),      # d64, two pages per 16-token group
    (8, 2, 64, 16, "fp8_e4m3"),
    (8, 4, 256, 32, "bf16"),    # d256, G 2: 32 rows per tile
    (8, 1, 256, 16, "fp8_e4m3"),  # d256, G 8
    (4, 4, 128, 64, "bf16"),    # G 1: 128 rows per tile
    (16, 1, 128, 128, "bf16"),  # G 16: 8 rows per tile
    (6, 2, 128, 16, "bf16"),    # G 3: 42 rows per tile, 2 padding columns
    (12, 1, 64, 16, "bf16"),    # G 12
]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("case", CASES, ids=[f"G{c[0] // c[1]}_d{c[2]}_P{c[3]}_{c[4]}" for c in CASES])
def test_prefill_matches_oracle(case, layout):
    Hq, Hkv, D, P, kv = case
    inp = synth.make_prefill_inputs(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, q_lens=Q_LENS,
                                    prefix_lens=PREFIX, kv_dtype=kv, seed=4000 + Hq + D + P)
    out, lse = _run(inp, layout=layout)
    _check(inp, out, lse, True, f"G{Hq // Hkv} d{D} P{P} {kv} {layout}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_prefill_non_causal(kv):
    inp = synth.make_prefill_inputs(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_lens=Q_LENS,
                                    prefix_lens=PREFIX, kv_dtype=kv, seed=4100)
    out, lse = _run(inp, causal=False)
    _check(inp, out, lse, False, f"non-causal {kv}")


def test_prefill_tile_order_does_not_change_results():
    """Each tile is computed alone, so the order of the tile map changes
    nothing, bit for bit."""
    inp = synth.make_prefill_inputs(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_lens=Q_LENS,
                                    prefix_lens=PREFIX, seed=4200)
    a = _run(inp, longest_first=True)
    b = _run(inp, longest_first=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prefill_context_shorter_than_rows():
    """Rows whose own position does not exist yet see nothing (out 0,
    lse -inf); a request with no context at all gives such rows only."""
    inp = synth.make_prefill_inputs(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_lens=(40, 5, 20),
                                    prefix_lens=(0, 0, 0), seed=4300)
    inp["context_lens"] = torch.tensor([25, 0, 20], dtype=torch.int32)
    out, lse = _run(inp)
    _check(inp, out, lse, True, "short contexts")
    assert bool(torch.isneginf(lse[:15]).all()) and bool(torch.isneginf(lse[40:45]).all())


def test_prefill_bad_inputs_give_nan_rows():
    """A context length beyond the block table makes its request's rows NaN;
    a block-table entry outside the pool makes NaN the rows of the tiles that
    read it; every other row is unaffected."""
    inp = synth.make_prefill_inputs(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_lens=(70, 20, 30),
                                    prefix_lens=(0, 100, 0), seed=4400)
    ref_o, ref_l = pf.prefill(inp["q"], inp["qo_indptr"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                              inp["context_lens"])
    bad = dict(inp)
    bt = inp["block_table"].clone()
    bt[2, 1] = 1 << 30   # request 2, positions 16..31: read by every tile of request 2
    bad["block_table"] = bt
    lens = inp["context_lens"].clone()
    lens[1] = bt.shape[1] * 16 + 1
    out, lse = _run(bad, lens=lens)
    ptr = inp["qo_indptr"].tolist()
    assert bool(torch.isnan(out[ptr[1]:ptr[2]]).all()) and bool(torch.isnan(lse[ptr[1]:ptr[2]]).all())
    assert bool(torch.isnan(out[ptr[2]:ptr[3]]).all())
    _compare(out[:ptr[1]], lse[:ptr[1]], ref_o[:ptr[1]], ref_l[:ptr[1]], False, "rows of the good request")


def test_prefill_empty_calls():
    """No rows at all, and a batch whose requests have no rows: nothing is
    launched and nothing fails."""
    pk = _pk()
    inp = synth.make_prefill_inputs(num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16, q_lens=(0, 0),
                                    prefix_lens=(3, 0), seed=4500)
    tb, ti = pk.prefill_tiles(inp["qo_indptr"], 64, context_lens_host=inp["context_lens"])
    assert tb.numel() == 0 and ti.numel() == 0
    out, lse = _run(inp)
    assert out.shape == (0, 8, 64) and lse.shape == (0, 8)


def _sampled(inp, rows, causal=True):
    """Oracle values of the packed rows `rows` only: each is one decode of
    its request's pages with its visible length."""
    rows_b, rows_lim = pf.visible_lengths(inp["qo_indptr"], inp["context_lens"], causal)
    rows = np.asarray(rows)
    q = inp["q"][torch.from_numpy(rows)].contiguous()
    bt = inp["block_table"][torch.from_numpy(rows_b[rows])].contiguous()
    lens = torch.from_numpy(rows_lim[rows].astype(np.int32))
    return oracle.decode(q, inp["k_pages"], inp["v_pages"], bt, lens, k_scale=inp["k_scale"],
                         v_scale=inp["v_scale"])


@pytest.mark.parametrize("name", sorted(synth.PREFILL_WORKLOADS))
def test_prefill_full_size_sampled(name):
    """The bench's workloads at full size, through the call bench.py times
    (HND pools, longest tiles first): sampled rows (each request's first,
    last and two random rows) against the oracle, and every output finite."""
    inp = synth.prefill_workload(name)
    out, lse = _run(inp, layout="hnd")
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    ptr = inp["qo_indptr"].tolist()
    rng = np.random.default_rng(11)
    rows = []
    for b in range(len(ptr) - 1):
        if ptr[b + 1] > ptr[b]:
            rows += [ptr[b], ptr[b + 1] - 1] + rng.integers(ptr[b], ptr[b + 1], 2).tolist()
    ref_o, ref_l = _sampled(inp, rows)
    _compare(out[rows], lse[rows], ref_o, ref_l, False, name)
