"""Prefill in serving order on the GPU: each request's new prompt rows are
first written into the paged cache by pdattn_kv_append (bf16, or fp8 with
power-of-two scales), then pdattn_prefill attends over the cache (cached
prefix + the new rows, causal). The reference applies the append oracle to
the same pools and then the prefill oracle. Also: the append + prefill step
captured in one HIP graph, each replay (with eager work between) equal to the
eager step bit for bit."""
import numpy as np
import pytest
import torch

import synth
from oracle import kv_append as oka
from oracle import prefill as opf

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(kv, seed, B=6, Hq=32, Hkv=8, D=128):
    inp = synth.make_append_inputs(batch=B, num_kv_heads=Hkv, head_dim=D, page_size=16, new_tokens=(1, 150),
                                   context=(0, 300), kv_dtype=kv, invalid=False, special_rows=False, spread=0,
                                   shuffle=False, seed=seed)
    n = (inp["new_lens"] - inp["context_lens"]).tolist()
    g = torch.Generator().manual_seed(seed + 5)
    inp["q"] = torch.randn((sum(n), Hq, D), generator=g).to(torch.bfloat16)
    inp["qo_indptr"] = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32)
    return inp


def _reference(inp, pow2):
    fp8 = inp["k_scale"] is not None
    if fp8:
        kp0, vp0 = inp["k_pages"].view(torch.uint8).numpy(), inp["v_pages"].view(torch.uint8).numpy()
        ks0, vs0 = inp["k_scale"].numpy(), inp["v_scale"].numpy()
    else:
        kp0, vp0 = inp["k_pages"].float().numpy(), inp["v_pages"].float().numpy()
        ks0 = vs0 = None
    kp, vp, ks, vs = oka.kv_append(kp0, vp0, ks0, vs0, inp["k_new"].float().numpy(), inp["v_new"].float().numpy(),
                                   inp["token_seq"].numpy(), inp["token_pos"].numpy(), inp["block_table"].numpy(),
                                   pow2=pow2)
    if fp8:
        kpt = torch.from_numpy(kp).view(torch.float8_e4m3fn)
        vpt = torch.from_numpy(vp).view(torch.float8_e4m3fn)
        kst, vst = torch.from_numpy(ks), torch.from_numpy(vs)
    else:
        kpt, vpt = torch.from_numpy(kp).to(torch.bfloat16), torch.from_numpy(vp).to(torch.bfloat16)
        kst = vst = None
    return opf.prefill(inp["q"], inp["qo_indptr"], kpt, vpt, inp["block_table"], inp["new_lens"], k_scale=kst,
                       v_scale=vst)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_append_then_prefill(kv, layout):
    import paged_kv_split_amd as pk
    inp = _inputs(kv, seed=5100 + (kv == "bf16") * 7 + (layout == "hnd"))
    fp8 = kv != "bf16"
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in src.items()}
    lay = pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD
    pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                 d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=fp8, layout=lay)
    out, lse = pk.paged_prefill(d["q"], d["qo_indptr"], d["k_pages"], d["v_pages"], d["block_table"],
                                d["new_lens"], qo_indptr_host=inp["qo_indptr"], context_lens_host=inp["new_lens"],
                                k_scale=d["k_scale"], v_scale=d["v_scale"], layout=lay)
    torch.cuda.synchronize()
    ro, rl = _reference(inp, pow2=fp8)
    diff = (out.cpu().double() - ro).abs()
    print(f"{kv} {layout}: rows {out.shape[0]}, max-abs {float(diff.max()):.2e} mean-abs {float(diff.mean()):.2e}")
    assert bool(torch.isfinite(out).all())
    assert float(diff.max()) <= (4e-2 if fp8 else 1e-2) and float(diff.mean()) <= 1e-3
    assert float((lse.cpu().double() - rl).abs().max()) <= 1e-3


def test_captured_append_and_prefill_replay_bitwise():
    import paged_kv_split_amd as pk
    inp = _inputs("fp8_e4m3", seed=5200)
    hnd = synth.to_hnd(inp)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in hnd.items()}
    prob = pk._prefill_problem(d["q"], d["k_pages"], d["block_table"], pk.LAYOUT_HND, None)
    tb, ti = pk.prefill_tiles(inp["qo_indptr"], pk.prefill_rows_per_tile(prob), context_lens_host=inp["new_lens"])
    tb, ti = tb.to(DEV), ti.to(DEV)
    out = torch.empty(d["q"].shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=DEV)

    def step():
        pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                     d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=True, layout=pk.LAYOUT_HND)
        pk.prefill(prob, d["q"], d["qo_indptr"], tb, ti, d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"],
                   d["block_table"], d["new_lens"], out, lse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, d["k_pages"].view(torch.uint8), d["v_scale"])]
    assert bool(torch.isfinite(out).all())
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out, lse, d["k_pages"].view(torch.uint8), d["v_scale"]]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {r}"
