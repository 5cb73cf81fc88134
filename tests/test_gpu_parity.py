"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle.

Tolerances (stated with the operation they bound):
  * bf16 pools: out max-abs <= 1e-2 and mean-abs <= 1e-3;
  * fp8 pools: out max-abs <= 4e-2 and mean-abs <= 1e-3, the oracle being fed
    the same codes and scales (it dequantises them exactly in fp64);
  * lse (natural log) max-abs <= 1e-3: scores are fp32 sums of exact bf16
    products and lse carries no division, so its error is a few fp32 ulps of
    the score scale.
"""
import math

import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 1e-2, 1e-3
FP8_MAX, FP8_MEAN = 4e-2, 1e-3
LSE_MAX = 1e-3


def _lib():
    import paged_kv_split_amd as pk
    return pk


def to_dev(inp):
    dev = torch.device("cuda:0")
    d = {}
    for key in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens"):
        t = inp[key]
        d[key] = None if t is None else t.to(dev)
    return d


def gpu_run(inp, dev=None, **kw):
    pk = _lib()
    dev = to_dev(inp) if dev is None else dev
    out, lse = pk.paged_decode(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                               dev["context_lens"], context_lens_host=inp["context_lens"],
                               k_scale=dev["k_scale"], v_scale=dev["v_scale"], **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_run(inp, **kw):
    return oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                         inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"], **kw)


def two_run_bound(inp):
    """Bound on the output difference of two GPU decodes of the same rows
    whose KV ranges are cut differently (split points, cascades, the
    balanced mode). The p.V products take each weight as two bf16 terms,
    within 2^-18 relative of it, so each output lies within 2^-18 max |V|
    of the exact weighted sum of its own pieces and two of them within
    2^-17 max |V|; 1e-5 covers the fp32 summation order. (lse is formed
    from fp32 weights and keeps the fp32-order bound.)"""
    v = inp["v_pages"].float()
    if inp.get("v_scale") is not None:
        v = v * inp["v_scale"].float()[..., None]
    vmax = float(v[torch.isfinite(v)].abs().max())  # unreferenced pages may hold NaN
    return 2.0 ** -17 * vmax + 1e-5


def assert_parity(out, lse, ref_out, ref_lse, fp8=False, tag=""):
    mx_tol, mean_tol = (FP8_MAX, FP8_MEAN) if fp8 else (BF16_MAX, BF16_MEAN)
    diff = (out.to(torch.float64) - ref_out).abs()
    assert bool(torch.isfinite(out).all()), f"{tag}: non-finite output"
    mx, mean = float(diff.max()), float(diff.mean())
    print(f"{tag}: out max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert mx <= mx_tol and mean <= mean_tol, (tag, mx, mean)
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isneginf(lse.to(torch.float64)), torch.isneginf(ref_lse)), tag
    ldiff = float((lse.to(torch.float64)[fin] - ref_lse[fin]).abs().max()) if bool(fin.any()) else 0.0
    assert ldiff <= LSE_MAX, (tag, ldiff)


MODES = [False, True]
MODE_IDS = ["static", "balanced"]


@pytest.mark.parametrize("balanced", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "many_short", "fp8_kv", "long_ctx"])
def test_workload_matches_oracle(name, balanced):
    inp = synth.make_inputs(name)
    out, lse = gpu_run(inp, balanced=balanced)
    ref_out, ref_lse = oracle_run(inp)
    assert_parity(out, lse, ref_out, ref_lse, fp8=inp["k_pages"].dtype == torch.float8_e4m3fn,
                  tag=f"{name} balanced={balanced}")


def small(B, Hq, Hkv, D, P, lens, kv="bf16", seed=0):
    return synth.Workload("gpu-small", "small GPU parity case", B, Hq, Hkv, D, P, lens, kv_dtype=kv,
                          seed=seed)


SHAPES = [(G, D, kv) for G in (1, 2, 4, 8, 16) for D in (64, 128) for kv in ("bf16", "fp8_e4m3")]


@pytest.mark.parametrize("G,D,kv", SHAPES, ids=[f"G{g}-D{d}-{k}" for g, d, k in SHAPES])
def test_every_instantiation_matches_oracle(G, D, kv):
    # ragged lengths spanning several tiles, splits and a partial last page
    w = small(B=5, Hq=2 * G, Hkv=2, D=D, P=16, lens=("uniform", 1, 700), kv=kv, seed=100 + G + D)
    inp = synth.make_inputs(w)
    ref = oracle_run(inp)
    for bal in MODES:
        for force in (0, 1, 7, 64):
            out, lse = gpu_run(inp, force_workers=force, balanced=bal)
            assert_parity(out, lse, *ref, fp8=kv != "bf16", tag=f"G{G} D{D} {kv} workers={force} balanced={bal}")


@pytest.mark.parametrize("P", [8, 16, 32, 64, 128])
def test_page_sizes(P):
    w = small(B=4, Hq=8, Hkv=2, D=128, P=P, lens=("uniform", 1, 1500), seed=200 + P)
    inp = synth.make_inputs(w)
    ref = oracle_run(inp)
    for bal in MODES:
        for force in (0, 3, 200):
            out, lse = gpu_run(inp, force_workers=force, balanced=bal)
            assert_parity(out, lse, *ref, tag=f"P{P} workers={force} balanced={bal}")


@pytest.mark.parametrize("balanced", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "many_short", "fp8_kv", "long_ctx"])
def test_head_major_pages_match_oracle_and_token_major(name, balanced):
    """The same pools laid out [page][kv head][slot]: the oracle's values, and
    (same tiles in the same order) bitwise the token-major result."""
    pk = _lib()
    inp = synth.make_inputs(name)
    hnd = synth.to_hnd(inp)
    out_n, lse_n = gpu_run(inp, balanced=balanced)
    out, lse = gpu_run(hnd, layout=pk.LAYOUT_HND, balanced=balanced)
    ref_out, ref_lse = oracle_run(inp)
    assert_parity(out, lse, ref_out, ref_lse, fp8=inp["k_pages"].dtype == torch.float8_e4m3fn,
                  tag=f"{name} HND balanced={balanced}")
    if not balanced:
        assert torch.equal(out, out_n) and torch.equal(lse, lse_n), name
