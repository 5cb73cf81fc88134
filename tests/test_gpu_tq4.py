"""TQ4 compressed cache on the GPU, through the C-ABI: pdattn_tq4_append
against the oracle's compress-and-scatter, and pdattn_tq4_decode against the
oracle's decode, the cache for the decode always written by the oracle.

Bars:
* append: every norm within 1e-5 relative of the oracle's fp64 norm (fp32
  sum of squares and square root); every code equal to the oracle's, except
  where the oracle's rotated value lies within eps of a boundary separating
  the two codes (the kernel decides in fp32, the oracle in fp64; eps =
  (d + 8) 2^-23 bounds the fp32 error of the rotated value: a d-term dot
  product of a unit vector with a unit row, plus the normalisation);
  untouched rows keep their bytes.
* decode: out within max-abs 4e-2 / mean-abs 1e-3 and lse within 2e-3 of
  the fp64 oracle: the kernel rounds the rotated q and the K centroids to
  fp16 (2^-11 relative; the scores' error grows with sqrt(d) such terms)
  and the V centroids and the probabilities to bf16 (2^-8 relative, as the
  fp8 path's elements).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import tq4 as otq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _tables(D):
    ck, bk = otq.codebook(D)
    return ck, bk, (ck * 1.25).astype(np.float32), (bk * 1.25).astype(np.float32)


def _workload(B, Hq, Hkv, D, P, lens, seed):
    return synth.WORKLOADS["tiny"].with_(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                                         lens=("fixed", tuple(lens)), pool="2x", seed=seed)


def _oracle_cache(inp, bk, bv):
    return otq.append(inp["cache"].numpy(), inp["k_new"], inp["v_new"], inp["token_seq"], inp["token_pos"],
                      inp["block_table"], inp["rotation"], bk, bv)


def _dev(x):
    return torch.as_tensor(x).contiguous().to(DEV)


def _check_codes(got_packed, want_packed, y, bnd, eps):
    g = otq.codes_of(got_packed).astype(np.int64)
    w = otq.codes_of(want_packed).astype(np.int64)
    diff = np.nonzero(g != w)
    for idx in zip(*diff):
        lo, hi = sorted((int(g[idx]), int(w[idx])))
        # every boundary between the two codes sits within eps of y
        assert all(abs(float(y[idx]) - float(bnd[k])) <= eps for k in range(lo, hi)), (idx, g[idx], w[idx], y[idx])
    return len(diff[0])


@pytest.mark.parametrize("D,P", [(64, 8), (128, 16), (128, 8), (256, 32)])
def test_tq4_append_matches_oracle(D, P):
    pk = _pk()
    inp = synth.make_tq4_inputs(_workload(3, 8, 2, D, P, (5, 37, 130), seed=8000 + D + P))
    ck, bk, cv, bv = _tables(D)
    want = _oracle_cache(inp, bk, bv)
    cache = _dev(inp["cache"])
    pk.tq4_append(_dev(inp["k_new"]), _dev(inp["v_new"]), _dev(inp["token_seq"]), _dev(inp["token_pos"]),
                  _dev(inp["block_table"]), _dev(inp["rotation"]), _dev(bk), _dev(bv), cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    # rows no token names: unchanged
    touched = np.zeros(got.shape[:3], bool)
    bt = inp["block_table"].numpy()
    for s, pos in zip(inp["token_seq"].tolist(), inp["token_pos"].tolist()):
        touched[bt[s, pos // P], :, pos % P] = True
    assert np.array_equal(got[~touched], want[~touched])
    g_kp, g_kn, g_vp, g_vn = otq.unpack_rows(got[touched])
    w_kp, w_kn, w_vp, w_vn = otq.unpack_rows(want[touched])
    assert np.allclose(g_kn, w_kn, rtol=1e-5, atol=0) and np.allclose(g_vn, w_vn, rtol=1e-5, atol=0)
    # the rotated values the oracle decided on, in the touched rows' order
    order = []
    for t, (s, pos) in enumerate(zip(inp["token_seq"].tolist(), inp["token_pos"].tolist())):
        order.append((bt[s, pos // P], pos % P, t))
    eps = (D + 8) * 2.0 ** -23
    rows_k, rows_v = {}, {}
    _, _, yk = otq.compress(inp["k_new"], inp["rotation"], bk, return_rotated=True)
    _, _, yv = otq.compress(inp["v_new"], inp["rotation"], bv, return_rotated=True)
    for page, slot, t in order:
        rows_k[(page, slot)] = yk[t]
        rows_v[(page, slot)] = yv[t]
    pages, heads, slots = np.nonzero(touched)
    yk_t = np.stack([rows_k[(p_, s_)][h_] for p_, h_, s_ in zip(pages, heads, slots)])
    yv_t = np.stack([rows_v[(p_, s_)][h_] for p_, h_, s_ in zip(pages, heads, slots)])
    n_k = _check_codes(g_kp, w_kp, yk_t, bk, eps)
    n_v = _check_codes(g_vp, w_vp, yv_t, bv, eps)
    print(f"D{D} P{P}: codes off by a boundary tie: K {n_k}, V {n_v} of {g_kp.size * 2} each")


CASES = [
    # B, Hq, Hkv, D, P, lens, chunk_tiles
    (3, 32, 8, 128, 16, (1, 300, 1000), 0),
    (4, 32, 8, 128, 16, (0, 17, 256, 999), 3),      # forced small work items: several per pair
    (3, 8, 8, 64, 8, (15, 16, 131), 4),             # G 1, P 8 (tiles over two pages)
    (2, 16, 8, 128, 32, (40, 513), 4),              # G 2
    (2, 64, 8, 128, 64, (700, 9), 0),               # G 8
    (2, 32, 2, 64, 16, (100, 333), 5),              # G 16
    (3, 16, 4, 256, 16, (33, 250, 64), 4),          # d 256
    (2, 12, 4, 128, 16, (200, 57), 4),              # G 3
]


def _run_decode(inp, cache_np, ck, cv, chunk_tiles=0, lens_dev=None):
    pk = _pk()
    out, lse = pk.paged_decode_tq4(_dev(inp["q"]), _dev(cache_np), _dev(inp["block_table"]),
                                   lens_dev if lens_dev is not None else _dev(inp["context_lens"]),
                                   _dev(inp["rotation"]), _dev(ck), _dev(cv), context_lens_host=inp["context_lens"],
                                   chunk_tiles=chunk_tiles)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _compare(out, lse, ref_o, ref_l, tag):
    fin = torch.isfinite(ref_l)
    diff = (out.double() - ref_o).abs()
    print(f"{tag}: max-abs {float(diff.max()):.2e} mean-abs {float(diff.mean()):.2e} "
          f"lse {float((lse.double()[fin] - ref_l[fin]).abs().max()) if bool(fin.any()) else 0:.2e}")
    assert bool(torch.isfinite(out).all())
    assert float(diff.max()) <= 4e-2 and float(diff.mean()) <= 1e-3
    assert torch.equal(torch.isneginf(lse.double()), torch.isneginf(ref_l))
    if bool(fin.any()):
        assert float((lse.double()[fin] - ref_l[fin]).abs().max()) <= 2e-3


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_G{c[1] // c[2]}_d{c[3]}_P{c[4]}_ct{c[6]}" for c in CASES])
def test_tq4_decode_matches_oracle(case):
    B, Hq, Hkv, D, P, lens, ct = case
    inp = synth.make_tq4_inputs(_workload(B, Hq, Hkv, D, P, lens, seed=8100 + D + Hq + P))
    ck, bk, cv, bv = _tables(D)
    cache = _oracle_cache(inp, bk, bv)
    out, lse = _run_decode(inp, cache, ck, cv, chunk_tiles=ct)
    ref_o, ref_l = otq.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    _compare(out, lse, ref_o, ref_l, str(case))
    empty = inp["context_lens"] == 0
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


def _run_decode_rotated(inp, cache_np, ck, cv, chunk_tiles=0, sample=None):
    """pdattn_tq4_decode_rotated on q_rot = fp16(R q) (the queries a caller
    with R folded into its q projection hands over); returns (q_rot, out,
    lse) on the CPU."""
    pk = _pk()
    q_rot = (inp["q"].double() @ inp["rotation"].double().T).to(torch.float16).contiguous()
    cache, bt, lens = _dev(cache_np), _dev(inp["block_table"]), _dev(inp["context_lens"])
    pl = pk.tq4_plan(pk.tq4_problem(q_rot, cache, bt), inp["context_lens"], chunk_tiles=chunk_tiles)
    ws = torch.empty(int(pl.workspace_bytes), dtype=torch.uint8, device=DEV)
    out = torch.full(q_rot.shape, 7.0, dtype=torch.float32, device=DEV)
    lse = torch.full(q_rot.shape[:2], 7.0, dtype=torch.float32, device=DEV)
    pk.tq4_decode_rotated(pl, _dev(q_rot), cache, _dev(ck), _dev(cv), bt, lens, ws, out, lse)
    torch.cuda.synchronize()
    return q_rot, out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_G{c[1] // c[2]}_d{c[3]}_P{c[4]}_ct{c[6]}" for c in CASES])
def test_tq4_decode_rotated_matches_oracle(case):
    """The fused attention's own boundary (fused_tq_attention.cu,
    Input/Output): q pre-rotated, the output left in the rotated space."""
    B, Hq, Hkv, D, P, lens, ct = case
    inp = synth.make_tq4_inputs(_workload(B, Hq, Hkv, D, P, lens, seed=8200 + D + Hq + P))
    ck, bk, cv, bv = _tables(D)
    cache = _oracle_cache(inp, bk, bv)
    q_rot, out, lse = _run_decode_rotated(inp, cache, ck, cv, chunk_tiles=ct)
    ref_o, ref_l = otq.decode_rotated(q_rot.double(), cache, inp["block_table"], inp["context_lens"], ck, cv)
    _compare(out, lse, ref_o, ref_l, "rotated " + str(case))
    empty = inp["context_lens"] == 0
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


def test_tq4_decode_rotated_full_size_sampled_sequences():
    """pdattn_tq4_decode_rotated on the Llama-3-8B-shaped workload at full
    size in the benchmark's launch configuration, three sequences checked
    against the oracle."""
    w = synth.WORKLOADS["llama3_8b"]
    inp = synth.make_tq4_inputs(w)
    ck, bk, cv, bv = _tables(w.head_dim)
    cache = _oracle_cache(inp, bk, bv)
    q_rot, out, lse = _run_decode_rotated(inp, cache, ck, cv)
    pick = [0, 13, 31]
    ref_o, ref_l = otq.decode_rotated(q_rot[pick].double(), cache, inp["block_table"][pick],
                                      inp["context_lens"][pick], ck, cv)
    _compare(out[pick], lse[pick], ref_o, ref_l, "llama3_8b tq4 rotated sampled")
    assert bool(torch.isfinite(out).all())


def test_tq4_decode_bad_page_and_overlong_give_nan():
    pk = _pk()
    inp = synth.make_tq4_inputs(_workload(3, 8, 2, 128, 16, (40, 40, 40), seed=8200))
    ck, bk, cv, bv = _tables(128)
    cache = _oracle_cache(inp, bk, bv)
    bt = inp["block_table"].clone()
    bt[1, 1] = cache.shape[0] + 5          # outside the pool
    lens = inp["context_lens"].clone()
    out, lse = pk.paged_decode_tq4(_dev(inp["q"]), _dev(cache), _dev(bt), _dev(lens), _dev(inp["rotation"]),
                                   _dev(ck), _dev(cv), context_lens_host=lens)
    lens_long = lens.clone()
    lens_long[2] = bt.shape[1] * 16 + 1    # beyond the block table
    out2, lse2 = pk.paged_decode_tq4(_dev(inp["q"]), _dev(cache), _dev(inp["block_table"]), _dev(lens_long),
                                     _dev(inp["rotation"]), _dev(ck), _dev(cv), context_lens_host=lens)
    torch.cuda.synchronize()
    out, lse, out2, lse2 = out.cpu(), lse.cpu(), out2.cpu(), lse2.cpu()
    assert bool(torch.isnan(out[1]).all()) and bool(torch.isnan(lse[1]).all())
    assert bool(torch.isfinite(out[0]).all()) and bool(torch.isfinite(out[2]).all())
    assert bool(torch.isnan(out2[2]).all()) and bool(torch.isfinite(out2[:2]).all())


def test_tq4_unsupported_calls_fail():
    pk = _pk()
    inp = synth.make_tq4_inputs(_workload(2, 8, 2, 128, 16, (20, 30), seed=8300))
    cache = _dev(inp["cache"])
    prob = pk.tq4_problem(inp["q"], cache, inp["block_table"])
    prob.kv_layout = pk.LAYOUT_NHD
    with pytest.raises(pk.PdattnError):
        pk.tq4_plan(prob, inp["context_lens"])
    prob = pk.tq4_problem(inp["q"], cache, inp["block_table"])
    with pytest.raises(pk.PdattnError):     # the other decode calls do not take TQ4 problems
        pk.plan(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                max_pages_per_seq=int(inp["block_table"].shape[1]), num_pages=int(cache.shape[0]),
                kv_dtype=pk.KV_TQ4, kv_layout=pk.LAYOUT_HND, context_lens_host=inp["context_lens"])
    with pytest.raises(pk.PdattnError):     # lengths beyond the block table at plan time
        pk.tq4_plan(prob, torch.tensor([20, 10 ** 6], dtype=torch.int32))


def test_tq4_full_size_sampled_sequences():
    """The Llama-3-8B-shaped workload at full size (B 32, 32 q / 8 kv heads,
    d 128, P 16, lengths ~U[512, 4096]) in the benchmark's launch
    configuration (adaptive plan), three sequences checked against the
    oracle."""
    w = synth.WORKLOADS["llama3_8b"]
    inp = synth.make_tq4_inputs(w)
    ck, bk, cv, bv = _tables(w.head_dim)
    cache = _oracle_cache(inp, bk, bv)
    out, lse = _run_decode(inp, cache, ck, cv)
    pick = [0, 13, 31]
    sub = dict(q=inp["q"][pick], block_table=inp["block_table"][pick], context_lens=inp["context_lens"][pick])
    ref_o, ref_l = otq.decode(sub["q"], cache, sub["block_table"], sub["context_lens"], inp["rotation"], ck, cv)
    _compare(out[pick], lse[pick], ref_o, ref_l, "llama3_8b tq4 sampled")
    assert bool(torch.isfinite(out).all())


def test_tq4_decode_captured_graph_replays_bitwise():
    """pdattn_tq4_decode (q rotation, chunk kernel, merge with back-rotation)
    captured in one HIP graph: every replay, with eager work between, equals
    the eager call bit for bit."""
    pk = _pk()
    inp = synth.make_tq4_inputs(_workload(4, 32, 8, 128, 16, (5, 260, 700, 33), seed=8400))
    ck, bk, cv, bv = _tables(128)
    cache = _dev(_oracle_cache(inp, bk, bv))
    q, bt, lens, rot = _dev(inp["q"]), _dev(inp["block_table"]), _dev(inp["context_lens"]), _dev(inp["rotation"])
    ckd, cvd = _dev(ck), _dev(cv)
    pl = pk.tq4_plan(pk.tq4_problem(q, cache, bt), inp["context_lens"], chunk_tiles=4)
    ws = torch.empty(int(pl.workspace_bytes), dtype=torch.uint8, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)

    def step():
        pk.tq4_decode(pl, q, cache, rot, ckd, cvd, bt, lens, ws, out, lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r}"
