"""Ragged paged prefill on the GPU against the CPU oracle (oracle/prefill.py),
with the decode tolerances: bf16 out max-abs 1e-2 and mean-abs 1e-3, fp8
max-abs 4e-2, lse max-abs 1e-3; rows that see nothing must be exactly
out 0, lse -inf.

Cases span several query tiles per request and a ragged tail (rows per tile
= 128 / G, or 64 / G at head_dim 256), K/V tiles with a ragged tail, every
group size class, both pool layouts, both KV dtypes, page sizes 8 to 128,
causal and not, requests with no rows, contexts shorter than their rows,
and the bench's workloads at full size on sampled rows; inline-scale fp8 pools
against the oracle and bit for bit against separate scales."""
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


# ---- split-KV prefill (pdattn_prefill_split_tiles + pdattn_prefill_split) ----

# longer prefixes so that tiles read up to 34 kernel tiles and are cut into
# several parts when the planner is given more slots than there is work
SPLIT_PREFIX = (0, 37, 2000, 5, 9, 700)


def _split_call(inp, *, layout="nhd", causal=True, slots=1 << 20, lens=None, ws=None, tiles=None):
    pk = _pk()
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (src[k].to(DEV) if src.get(k) is not None else None)
         for k in ("q", "qo_indptr", "k_pages", "v_pages", "k_scale", "v_scale", "block_table")}
    lay = pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD
    prob = pk._prefill_problem(d["q"], d["k_pages"], d["block_table"], lay, None)
    st = tiles if tiles is not None else pk.prefill_split_tiles(prob, inp["qo_indptr"], inp["context_lens"],
                                                                causal=causal, slots=slots)
    if ws is None:
        ws = pk.prefill_split_workspace(st, DEV)
    lens = (inp["context_lens"] if lens is None else lens).to(DEV)
    out = torch.empty(d["q"].shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=DEV)
    pk.prefill_split(prob, d["q"], d["qo_indptr"], st.tile_batch.to(DEV), st.tile_index.to(DEV), st.tile_kv.to(DEV),
                     st.num_slots, ws, d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"], lens,
                     out, lse, causal=causal)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), st, ws


def _counters(st, ws, Hkv):
    n = st.num_slots * Hkv
    return ws[:4 * n].view(torch.int32).cpu() if n else torch.zeros(0, dtype=torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[f"G{c[0] // c[1]}_d{c[2]}_P{c[3]}_{c[4]}" for c in CASES])
def test_split_prefill_matches_oracle(case):
    Hq, Hkv, D, P, kv = case
    inp = synth.make_prefill_inputs(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, q_lens=Q_LENS,
                                    prefix_lens=SPLIT_PREFIX, kv_dtype=kv, seed=4600 + Hq + D + P)
    layout = "hnd" if (Hq + D) % 2 == 0 else "nhd"
    out, lse, st, ws = _split_call(inp, layout=layout)
    parts = st.tile_kv[:, 3] >> 16
    print(f"split G{Hq // Hkv} d{D}: {st.num_tiles} entries, {st.num_slots} slots, up to {int(parts.max())} parts",
          flush=True)
    assert st.num_slots > 0
    _check(inp, out, lse, True, f"split G{Hq // Hkv} d{D} P{P} {kv} {layout}")
    assert int(_counters(st, ws, Hkv).abs().sum()) == 0


@pytest.mark.parametrize("causal", [True, False])
def test_split_prefill_is_deterministic_and_leaves_counters_zero(causal):
    """Two calls on one workspace give the same bits (the last part merges
    the records in part order, whatever order the parts finished in), leave
    every counter at zero, and agree with the unsplit kernel to the bf16
    rounding of the probabilities."""
    inp = synth.make_prefill_inputs(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_lens=Q_LENS,
                                    prefix_lens=SPLIT_PREFIX, seed=4700)
    a_o, a_l, st, ws = _split_call(inp, causal=causal)
    assert int(_counters(st, ws, 8).abs().sum()) == 0
    b_o, b_l, _, _ = _split_call(inp, causal=causal, ws=ws, tiles=st)
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
    assert int(_counters(st, ws, 8).abs().sum()) == 0
    u_o, u_l = _run(inp, causal=causal)
    # P is rounded to bf16 against each part's own running max, so the
    # outputs agree to that rounding (the parity bar), l and lse to fp32's
    diff = (a_o - u_o).abs()
    assert float(diff.max()) <= 1e-2 and float(diff.mean()) <= 1e-4
    fin = torch.isfinite(u_l)
    assert torch.equal(fin, torch.isfinite(a_l)) and float((a_l[fin] - u_l[fin]).abs().max()) <= 1e-5
    _check(inp, a_o, a_l, causal, f"split causal={causal}")


def test_split_prefill_bad_inputs_give_nan_rows():
    """A bad block-table entry read by one part of a split tile makes all of
    that tile's rows NaN (the poison travels through the counter); a map entry
    whose slots lie outside num_slots makes its tile's rows NaN without
    touching the workspace; other rows are unaffected."""
    pk = _pk()
    inp = synth.make_prefill_inputs(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_lens=(40, 20, 30),
                                    prefix_lens=(1000, 600, 0), seed=4800)
    ref_o, ref_l = pf.prefill(inp["q"], inp["qo_indptr"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                              inp["context_lens"])
    ptr = inp["qo_indptr"].tolist()
    bad = dict(inp)
    bt = inp["block_table"].clone()
    bt[0, 2] = 1 << 30   # request 0, positions 32..47: the first part of its tiles
    bad["block_table"] = bt
    out, lse, st, ws = _split_call(bad)
    assert int((st.tile_kv[:, 2] >= 0).sum()) > 0
    assert bool(torch.isnan(out[ptr[0]:ptr[1]]).all()) and bool(torch.isnan(lse[ptr[0]:ptr[1]]).all())
    _compare(out[ptr[1]:], lse[ptr[1]:], ref_o[ptr[1]:], ref_l[ptr[1]:], False, "split: rows of the good requests")
    assert int(_counters(st, ws, 2).abs().sum()) == 0
    # a part entry naming slots past num_slots (request 1's first split entry)
    tk = st.tile_kv.clone()
    t = [i for i in range(st.num_tiles) if int(st.tile_batch[i]) == 1 and int(tk[i, 2]) >= 0][0]
    tk[t, 2] = st.num_slots
    broken = pk.SplitTiles(st.tile_batch, st.tile_index, tk, st.num_slots, st.workspace_bytes)
    out2, lse2, _, _ = _split_call(inp, tiles=broken, ws=pk.prefill_split_workspace(st, DEV))
    rows = int(st.tile_index[t]) * 32
    assert bool(torch.isnan(out2[ptr[1] + rows:min(ptr[1] + rows + 32, ptr[2])]).all())
    _compare(out2[ptr[2]:], lse2[ptr[2]:], ref_o[ptr[2]:], ref_l[ptr[2]:], False, "split: other rows")


def test_split_prefill_graph_replays():
    """The split call captured in a HIP graph: every replay (with eager work
    and synchronisation between them) gives the eager call's bits; the
    counters restore themselves, no memset is recorded."""
    pk = _pk()
    inp = synth.make_prefill_inputs(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_lens=Q_LENS,
                                    prefix_lens=SPLIT_PREFIX, seed=4900)
    ref_o, ref_l, st, ws = _split_call(inp)
    d = {k: (inp[k].to(DEV) if inp.get(k) is not None else None)
         for k in ("q", "qo_indptr", "k_pages", "v_pages", "block_table", "context_lens")}
    prob = pk._prefill_problem(d["q"], d["k_pages"], d["block_table"], pk.LAYOUT_NHD, None)
    tb, ti, tk = st.tile_batch.to(DEV), st.tile_index.to(DEV), st.tile_kv.to(DEV)
    out = torch.zeros(d["q"].shape, dtype=torch.float32, device=DEV)
    lse = torch.zeros(d["q"].shape[:2], dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pk.prefill_split(prob, d["q"], d["qo_indptr"], tb, ti, tk, st.num_slots, ws, d["k_pages"], d["v_pages"],
                         None, None, d["block_table"], d["context_lens"], out, lse, stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), ref_o) and torch.equal(lse.cpu(), ref_l), rep
        assert int(_counters(st, ws, 8).abs().sum()) == 0, rep


@pytest.mark.parametrize("name", sorted(synth.PREFILL_WORKLOADS))
def test_split_prefill_full_size_sampled(name):
    """The bench's workloads at full size through the split call on this
    device's slot count (the planner cuts only what the schedule needs):
    sampled rows against the oracle, every output finite."""
    inp = synth.prefill_workload(name)
    out, lse, st, ws = _split_call(inp, layout="hnd", slots=0)
    print(f"{name}: {st.num_tiles} entries, {st.num_slots} slots", flush=True)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    ptr = inp["qo_indptr"].tolist()
    rng = np.random.default_rng(12)
    rows = []
    for b in range(len(ptr) - 1):
        if ptr[b + 1] > ptr[b]:
            rows += [ptr[b], ptr[b + 1] - 1] + rng.integers(ptr[b], ptr[b + 1], 6).tolist()
    ref_o, ref_l = _sampled(inp, rows)
    _compare(out[rows], lse[rows], ref_o, ref_l, False, name + " split")


def test_prefill_full_size_fp8_sampled():
    """The bench's ragged batch with fp8 pools at full size, through both
    calls bench.py times (HND pools): sampled rows against the oracle at the
    fp8 bar, every output finite, and the two calls within that bar of each
    other."""
    inp = synth.prefill_workload("llama3_8b_prefill", kv_dtype="fp8_e4m3")
    out, lse = _run(inp, layout="hnd")
    s_out, s_lse, st, _ = _split_call(inp, layout="hnd", slots=0)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(s_out).all())
    ptr = inp["qo_indptr"].tolist()
    rng = np.random.default_rng(13)
    rows = []
    for b in range(len(ptr) - 1):
        if ptr[b + 1] > ptr[b]:
            rows += [ptr[b], ptr[b + 1] - 1] + rng.integers(ptr[b], ptr[b + 1], 3).tolist()
    ref_o, ref_l = _sampled(inp, rows)
    _compare(out[rows], lse[rows], ref_o, ref_l, True, "fp8 ragged, unsplit")
    _compare(s_out[rows], s_lse[rows], ref_o, ref_l, True, f"fp8 ragged, split ({st.num_tiles} entries)")
    assert float((out - s_out).abs().max()) <= 4e-2


INLINE_CASES = [
    # Hq, Hkv, D, P
    (32, 8, 128, 16),
    (8, 2, 64, 8),     # two pages per 16-token group
    (8, 1, 256, 16),   # d256, G 8: two waves per 16-token group
    (8, 2, 128, 128),
]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("case", INLINE_CASES, ids=[f"G{c[0] // c[1]}_d{c[2]}_P{c[3]}" for c in INLINE_CASES])
def test_inline_fp8_prefill_matches_oracle_and_separate_scales(case, layout):
    """Pools with each row's scale after its codes (rows of d + 4 bytes,
    only 4-byte aligned): the oracle's fp8 bar, and bit for bit the result
    of the same values with separate scale arrays, unsplit and split (the
    kernel builds the same LDS image from either layout)."""
    Hq, Hkv, D, P = case
    inp = synth.make_prefill_inputs(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, q_lens=Q_LENS,
                                    prefix_lens=SPLIT_PREFIX, kv_dtype="fp8_e4m3", seed=4900 + Hq + D + P)
    il = synth.to_inline(inp)
    tag = f"inline G{Hq // Hkv} d{D} P{P} {layout}"
    out, lse = _run(inp, layout=layout)
    i_out, i_lse = _run(il, layout=layout)
    _check(inp, i_out, i_lse, True, tag)
    assert torch.equal(i_out, out) and torch.equal(i_lse, lse), tag
    s_out, s_lse, _, _ = _split_call(inp, layout=layout)
    si_out, si_lse, st, ws = _split_call(il, layout=layout)
    assert st.num_slots > 0, "the map splits the 2000-position prompt"
    _check(inp, si_out, si_lse, True, tag + " split")
    assert torch.equal(si_out, s_out) and torch.equal(si_lse, s_lse), tag
    assert not bool(_counters(st, ws, Hkv).any())


def test_inline_fp8_prefill_non_causal_and_bad_page():
    """Inline pools without the causal mask, and a block-table entry outside
    the pool: NaN rows for the tiles that read it, the rest as with
    separate scales."""
    inp = synth.make_prefill_inputs(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_lens=Q_LENS,
                                    prefix_lens=PREFIX, kv_dtype="fp8_e4m3", seed=4950)
    il = synth.to_inline(inp)
    out, lse = _run(il, causal=False)
    _check(inp, out, lse, False, "inline non-causal")
    bad = dict(il)
    bt = il["block_table"].clone()
    bt[2, 1] = 1 << 30   # request 2, positions 16..31: read by every tile of request 2
    bad["block_table"] = bt
    b_out, b_lse = _run(bad)
    ptr = inp["qo_indptr"].tolist()
    assert bool(torch.isnan(b_out[ptr[2]:ptr[3]]).all()) and bool(torch.isnan(b_lse[ptr[2]:ptr[3]]).all())
    g_out, g_lse = _run(il)
    keep = torch.ones(b_out.shape[0], dtype=torch.bool)
    keep[ptr[2]:ptr[3]] = False
    assert torch.equal(b_out[keep], g_out[keep]) and torch.equal(b_lse[keep], g_lse[keep])
