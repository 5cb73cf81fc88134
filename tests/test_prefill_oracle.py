"""Pins of the ragged paged prefill oracle (oracle/prefill.py).

* the tile map against the worked example the pages print;
* causal prefill of whole prompts (context = the new rows) against torch's
  scaled_dot_product_attention with is_causal=True, fp64, on the gathered
  K/V (a library routine; top-left and bottom-right causal alignment agree
  when every row is new);
* non-causal prefill with cached prefixes against the same routine without
  a mask;
* the placement of new rows after a cached prefix, through an invariant
  that involves no formula of the oracle: a prompt prefilled in two chunks
  (the second chunk's context holds the first) gives the rows the
  whole-prompt prefill gives;
* fp8 pools through the same routine on the dequantised values;
* degenerate requests: no rows, and rows with no visible position.
Each pin also runs against a copy of the oracle with a planted mistake and
must fail there.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import brute
from oracle import prefill as pf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_tile_map.json")


def test_tile_map_matches_pages_worked_example():
    g = json.load(open(GOLDEN))
    ptr = np.concatenate([[0], np.cumsum(g["q_lens"])]).tolist()
    assert ptr == g["qo_indptr"]
    tb, ti = pf.tile_map(g["qo_indptr"], g["rows_per_tile"])
    assert tb == g["q_tile_to_batch"]
    assert ti == g["q_tile_to_index"]


def test_tile_map_covers_every_row_once():
    rng = np.random.default_rng(7)
    for _ in range(20):
        lens = rng.integers(0, 200, size=rng.integers(1, 9)).tolist()
        rt = int(rng.choice([1, 8, 32, 64, 128]))
        ptr = np.concatenate([[0], np.cumsum(lens)]).tolist()
        tb, ti = pf.tile_map(ptr, rt)
        seen = np.zeros(ptr[-1], dtype=int)
        for b, j in zip(tb, ti):
            lo = ptr[b] + j * rt
            hi = min(lo + rt, ptr[b + 1])
            assert lo < hi
            seen[lo:hi] += 1
        assert (seen == 1).all()


def _sdpa_rows(inp, causal_top_left, fp8=False):
    """torch SDPA (fp64) per request over the gathered K/V; returns out
    [total_q, Hq, d]."""
    q, ptr, lens = inp["q"], inp["qo_indptr"].tolist(), inp["context_lens"].tolist()
    Hq, D = q.shape[1], q.shape[2]
    Hkv = inp["k_pages"].shape[2]
    G = Hq // Hkv
    out = torch.zeros((q.shape[0], Hq, D), dtype=torch.float64)
    ks = inp["k_scale"] if fp8 else None
    vs = inp["v_scale"] if fp8 else None
    for b in range(len(lens)):
        n, L = ptr[b + 1] - ptr[b], lens[b]
        if n == 0 or L == 0:
            continue
        K = brute.gather_dense(inp["k_pages"], ks, inp["block_table"], L, b)
        V = brute.gather_dense(inp["v_pages"], vs, inp["block_table"], L, b)
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()   # [Hq, L, D]
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        qq = q[ptr[b]:ptr[b + 1]].to(torch.float64).permute(1, 0, 2).contiguous()  # [Hq, n, D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, K, V, is_causal=causal_top_left,
                                                             scale=1.0 / math.sqrt(D))
        out[ptr[b]:ptr[b + 1]] = o.permute(1, 0, 2)
    return out


def _run(inp, causal, fn=None):
    fn = fn or pf.prefill
    return fn(inp["q"], inp["qo_indptr"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"],
              causal=causal, k_scale=inp["k_scale"], v_scale=inp["v_scale"])


def _planted_off_by_one(q, qo_indptr, k_pages, v_pages, block_table, context_lens, *, causal=True, k_scale=None,
                        v_scale=None):
    """The oracle with each row seeing one position fewer (lim = L - n + i):
    every context shortened by one, the rows kept."""
    lens = (torch.as_tensor(context_lens) - 1).clamp(min=0).to(torch.int32)
    return pf.prefill(q, qo_indptr, k_pages, v_pages, block_table, lens, causal=causal, k_scale=k_scale,
                      v_scale=v_scale)


def _planted_top_left(q, qo_indptr, k_pages, v_pages, block_table, context_lens, *, causal=True, k_scale=None,
                      v_scale=None):
    """The oracle with the other causal alignment: row i sees t <= i."""
    ptr = torch.as_tensor(qo_indptr).to(torch.int64)
    lens = torch.as_tensor(context_lens).to(torch.int64)
    n = ptr[1:] - ptr[:-1]
    # a context of exactly n positions puts row i at position i
    res_o = torch.zeros((q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float64)
    res_l = torch.zeros((q.shape[0], q.shape[1]), dtype=torch.float64)
    for b in range(len(n)):
        sub_ptr = torch.tensor([0, int(n[b])], dtype=torch.int32)
        o, l = pf.prefill(q[int(ptr[b]):int(ptr[b + 1])], sub_ptr, k_pages, v_pages, block_table[b:b + 1],
                          torch.minimum(n[b:b + 1], lens[b:b + 1]).to(torch.int32), causal=causal,
                          k_scale=k_scale, v_scale=v_scale)
        res_o[int(ptr[b]):int(ptr[b + 1])] = o
        res_l[int(ptr[b]):int(ptr[b + 1])] = l
    return res_o, res_l


WHOLE = dict(num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16)


@pytest.mark.parametrize("q_lens", [(70, 10, 130), (1, 33, 0, 17)])
def test_causal_whole_prompts_match_sdpa(q_lens):
    inp = synth.make_prefill_inputs(**WHOLE, q_lens=q_lens, seed=3100 + len(q_lens))
    out, lse = _run(inp, causal=True)
    ref = _sdpa_rows(inp, causal_top_left=True)
    torch.testing.assert_close(out, ref, rtol=1e-10, atol=1e-10)
    assert torch.isfinite(lse).all()
    bad, _ = _run(inp, causal=True, fn=_planted_off_by_one)
    assert (bad - ref).abs().max() > 1e-3


@pytest.mark.parametrize("prefix", [(0, 5, 40), (100, 1, 0)])
def test_non_causal_with_prefix_matches_sdpa(prefix):
    inp = synth.make_prefill_inputs(**WHOLE, q_lens=(12, 30, 7), prefix_lens=prefix, seed=3200 + sum(prefix))
    out, _ = _run(inp, causal=False)
    ref = _sdpa_rows(inp, causal_top_left=False)
    torch.testing.assert_close(out, ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("n,cut", [(90, 37), (64, 63), (20, 1)])
def test_chunked_prefill_equals_whole_prompt(n, cut):
    """Rows cut..n-1 prefilled as a second chunk, with the first cut rows
    already in the cache, equal the same rows of the whole-prompt prefill
    (which the SDPA pin above fixes)."""
    whole = synth.make_prefill_inputs(**WHOLE, q_lens=(n,), seed=3300 + n)
    out_w, lse_w = _run(whole, causal=True)
    second = dict(whole)
    second["q"] = whole["q"][cut:].contiguous()
    second["qo_indptr"] = torch.tensor([0, n - cut], dtype=torch.int32)
    out_c, lse_c = _run(second, causal=True)
    torch.testing.assert_close(out_c, out_w[cut:], rtol=1e-12, atol=1e-12)
    torch.testing.assert_close(lse_c, lse_w[cut:], rtol=1e-12, atol=1e-12)
    bad, _ = _run(second, causal=True, fn=_planted_top_left)
    assert (bad - out_w[cut:]).abs().max() > 1e-3


def test_fp8_pools_match_sdpa_on_dequantised_values():
    inp = synth.make_prefill_inputs(**WHOLE, q_lens=(40, 3), kv_dtype="fp8_e4m3", seed=3400)
    out, _ = _run(inp, causal=True)
    ref = _sdpa_rows(inp, causal_top_left=True, fp8=True)
    torch.testing.assert_close(out, ref, rtol=1e-10, atol=1e-10)


def test_degenerate_requests():
    """A request with no rows contributes nothing; rows of a request whose
    context is shorter than its row count see nothing until their own
    position exists: out 0, lse -inf."""
    inp = synth.make_prefill_inputs(**WHOLE, q_lens=(0, 6), prefix_lens=(3, 0), seed=3500)
    short = dict(inp)
    short["context_lens"] = torch.tensor([3, 4], dtype=torch.int32)   # 6 rows, 4 positions
    out, lse = _run(short, causal=True)
    assert out.shape[0] == 6
    assert (out[:2] == 0).all() and torch.isinf(lse[:2]).all() and (lse[:2] < 0).all()
    assert torch.isfinite(lse[2:]).all()
    # row 2 (bottom-right: position 0) sees exactly position 0: its V row
    v0 = brute.gather_dense(inp["v_pages"], None, inp["block_table"], 1, 1)[0]   # [Hkv, d]
    G = WHOLE["num_q_heads"] // WHOLE["num_kv_heads"]
    torch.testing.assert_close(out[2], v0.repeat_interleave(G, dim=0), rtol=0, atol=0)
