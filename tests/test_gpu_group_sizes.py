"""Group sizes that are not powers of two (G query heads per kv head, any
G <= 16; with q_len rows, any q_len * G <= 16) against the CPU oracle with
the decode tolerances (bf16 out max-abs 1e-2 / mean-abs 1e-3, fp8 max-abs
4e-2, lse 1e-3). The kernel runs them on the next power-of-two instance,
the extra columns padding (zero q, never written)."""
import pytest
import torch

import oracle
import synth
from oracle import multi_query as mq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LENS = (0, 1, 7, 16, 17, 200, 1000, 2100)


def _run(inp, q=None, layout="nhd", force=0):
    import paged_kv_split_amd as pk
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (src[k].to(DEV) if src[k] is not None else None)
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    out, lse = pk.paged_decode(d["q"] if q is None else q.to(DEV), d["k_pages"], d["v_pages"], d["block_table"],
                               d["context_lens"], context_lens_host=inp["context_lens"], k_scale=d["k_scale"],
                               v_scale=d["v_scale"], force_workers=force,
                               layout=pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(out, lse, ref_o, ref_l, fp8, tag):
    diff = (out.double() - ref_o).abs()
    mx, mean = float(diff.max()), float(diff.mean())
    print(f"{tag}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)
    assert bool(torch.isfinite(out).all()), tag
    assert mx <= (4e-2 if fp8 else 1e-2) and mean <= 1e-3, (tag, mx, mean)
    assert torch.equal(torch.isneginf(lse.double()), torch.isneginf(ref_l)), tag
    fin = torch.isfinite(ref_l)
    if bool(fin.any()):
        assert float((lse.double()[fin] - ref_l[fin]).abs().max()) <= 1e-3, tag


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G,Hkv", [(3, 8), (5, 2), (6, 4), (7, 4), (12, 2), (15, 1)])
def test_group_size_matches_oracle(G, Hkv, kv, layout):
    w = synth.WORKLOADS["llama3_8b"].with_(batch=len(LENS), num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                           lens=("fixed", LENS), kv_dtype=kv, seed=8000 + G)
    inp = synth.make_inputs(w)
    out, lse = _run(inp, layout=layout)
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"],
                                 k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    _check(out, lse, ref_o, ref_l, kv != "bf16", f"G{G} Hkv{Hkv} {kv} {layout}")


@pytest.mark.parametrize("G,n", [(3, 5), (7, 2), (5, 3), (3, 4)])
@pytest.mark.parametrize("force", [0, 13])
def test_group_size_multi_query_matches_oracle(G, n, force):
    w = synth.WORKLOADS["llama3_8b"].with_(batch=len(LENS), num_q_heads=G * 4, num_kv_heads=4,
                                           lens=("fixed", LENS), seed=8100 + G * n)
    inp = synth.make_inputs(w)
    g = torch.Generator().manual_seed(8101)
    q4 = torch.randn((len(LENS), n, G * 4, 128), generator=g).to(torch.bfloat16)
    out, lse = _run(inp, q=q4, layout="hnd", force=force)
    ref_o, ref_l = mq.decode_multi_query(q4, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    _check(out, lse, ref_o, ref_l, False, f"G{G} n{n} workers={force}")


def test_qwen2_7b_like_full_size():
    """28 query heads over 4 kv heads (G 7) at the Llama-3-8B step's lengths."""
    w = synth.WORKLOADS["llama3_8b"].with_(num_q_heads=28, num_kv_heads=4, seed=8200)
    inp = synth.make_inputs(w)
    out, lse = _run(inp, layout="hnd")
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    _check(out, lse, ref_o, ref_l, False, "G7 full size")
