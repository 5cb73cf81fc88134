"""Parity of the HIP partial-state merge (pdattn_merge, through the C ABI)
with the CPU oracle (oracle/merge.py), and the cascade property: decodes of
disjoint page ranges of each sequence, merged, equal the decode of the whole.

Tolerance of the merge alone, from its fp32 arithmetic: each weight
exp(lse_s - M) is an exp2 of a rounded product (relative error a few 1e-7
for the exponent differences that matter, |lse_s - M| <= ~30), the outputs
are convex combinations of at most a few pieces; so out max-abs <= 1e-5 *
max(1, max |o_s|) and lse max-abs <= 1e-5 * max(1, |lse|).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import merge as mg
from test_gpu_parity import two_run_bound

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _partials(S, R, d, seed, specials=True):
    g = torch.Generator().manual_seed(seed)
    po = torch.randn((S, R, d), generator=g)
    pl = torch.randn((S, R), generator=g) * 10
    if specials and R >= 8:
        pl[:, 0] = -float("inf")                 # every piece empty
        pl[0, 1] = -float("inf")                 # one piece empty
        pl[S - 1, 2] = float("nan")              # an invalid piece
        pl[:, 3] = pl[:, 3] + 3000.0             # large lse
        pl[:, 4] = 7.25                          # equal lse
        if S > 1:
            pl[1, 5] = float("inf")
        po[0, 6] *= 1000.0
    return po, pl


def _check(out, lse, po, pl, tag):
    ref_o, ref_l = mg.merge_states(po.numpy(), pl.numpy())
    out = out.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    nan_rows = np.isnan(ref_l)
    assert np.array_equal(np.isnan(lse), nan_rows), tag
    assert np.isnan(out[nan_rows]).all(), tag
    ok = ~nan_rows
    scale = max(1.0, float(np.abs(po.numpy()).max()))
    d_o = np.abs(out[ok] - ref_o[ok]).max() if ok.any() else 0.0
    assert d_o <= 1e-5 * scale, (tag, d_o)
    neg = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lse), neg), tag
    fin = ok & ~neg
    if fin.any():
        d_l = (np.abs(lse[fin] - ref_l[fin]) / np.maximum(1.0, np.abs(ref_l[fin]))).max()
        assert d_l <= 1e-5, (tag, d_l)
    print(f"{tag}: out max-abs {d_o:.2e}", flush=True)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("S,R", [(1, 9), (2, 1000), (3, 4099), (5, 257), (8, 1024)])
def test_merge_matches_oracle(S, R, d):
    po, pl = _partials(S, R, d, seed=S * 1000 + R + d)
    out, lse = _pk().merge(po.to(DEV), pl.to(DEV))
    torch.cuda.synchronize()
    _check(out, lse, po, pl, f"merge S{S} R{R} d{d}")


def test_merge_in_place_on_piece_zero_and_without_lse():
    pk = _pk()
    po, pl = _partials(4, 777, 128, seed=5)
    dpo, dpl = po.to(DEV), pl.to(DEV)
    ref_out, ref_lse = pk.merge(dpo, dpl)
    pk._check(pk._lib.pdattn_merge(4, 777, 128, pk._ptr(dpo), pk._ptr(dpl), pk._ptr(dpo), pk._ptr(dpl),
                                   pk._stream(None)), "merge in place")
    torch.cuda.synchronize()
    same = lambda a, b: torch.testing.assert_close(a.cpu(), b.cpu(), rtol=0, atol=0, equal_nan=True)
    same(dpo[0], ref_out)
    same(dpl[0], ref_lse)
    out = torch.empty((777, 128), device=DEV)
    pk._check(pk._lib.pdattn_merge(4, 777, 128, pk._ptr(po.to(DEV)), pk._ptr(pl.to(DEV)), pk._ptr(out), None,
                                   pk._stream(None)), "merge without lse")
    torch.cuda.synchronize()
    same(out, ref_out)


def _piece_tables(bt, lens, P, cuts):
    for a, b in zip(cuts[:-1], cuts[1:]):
        sub = torch.full_like(bt, -1)
        piece = bt[:, a:b]
        sub[:, :piece.shape[1]] = piece
        yield sub, (lens.to(torch.int64) - a * P).clamp(0, (b - a) * P).to(torch.int32)


@pytest.mark.parametrize("name,cuts", [("llama3_8b", [0, 32, 1000]),            # shared-prefix cascade
                                       ("many_short", [0, 1, 4, 1000]),
                                       ("fp8_kv", [0, 100, 250, 1000]),
                                       ("long_ctx", [0, 256, 512, 768, 1024, 1280, 1536, 1792, 5000])])
def test_cascade_merge_equals_whole_decode(name, cuts):
    """Decode each sequence's pages [cuts[i], cuts[i+1]) separately on the
    GPU into stacked partials, merge them on the GPU, and compare with the
    GPU decode of the whole context (the two runs' rounding only: the p.V
    products' two-term weights and fp32 summation order) and with the
    oracle's decode (the decode tolerances)."""
    pk = _pk()
    inp = synth.make_inputs(name)
    P = inp["k_pages"].shape[1]
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, Hq, D = inp["q"].shape
    S = len(cuts) - 1
    po = torch.empty((S, B, Hq, D), dtype=torch.float32, device=DEV)
    pl = torch.empty((S, B, Hq), dtype=torch.float32, device=DEV)
    for s, (sub, sub_lens) in enumerate(_piece_tables(inp["block_table"], inp["context_lens"], P, cuts)):
        pl_ = pk.plan(batch=B, num_q_heads=Hq, num_kv_heads=inp["k_pages"].shape[2], head_dim=D, page_size=P,
                      max_pages_per_seq=sub.shape[1], num_pages=inp["k_pages"].shape[0],
                      kv_dtype=pk.KV_FP8_E4M3 if inp["k_scale"] is not None else pk.KV_BF16,
                      context_lens_host=sub_lens)
        ws = pk.workspace(pl_, DEV)
        pk.decode(pl_, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], sub.to(DEV),
                  sub_lens.to(DEV), ws, po[s], pl[s])
        pk.reduce(pl_, ws, po[s], pl[s])
    out, lse = pk.merge(po, pl)
    whole_o, whole_l = pk.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                                       context_lens_host=inp["context_lens"], k_scale=d["k_scale"],
                                       v_scale=d["v_scale"])
    torch.cuda.synchronize()
    assert float((out - whole_o).abs().max()) <= two_run_bound(inp), name
    assert float((lse - whole_l).abs().max()) <= 1e-4, name
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"],
                                 k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    diff = (out.cpu().double() - ref_o).abs()
    mx = 4e-2 if inp["k_scale"] is not None else 1e-2
    print(f"cascade {name} S{S}: vs whole {float((out - whole_o).abs().max()):.2e}, "
          f"vs oracle max {float(diff.max()):.2e} mean {float(diff.mean()):.2e}", flush=True)
    assert float(diff.max()) <= mx and float(diff.mean()) <= 1e-3
    assert float((lse.cpu().double() - ref_l).abs().max()) <= 1e-3
