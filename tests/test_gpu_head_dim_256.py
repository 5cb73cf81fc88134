"""head_dim 256 on the GPU: decode (every group size, bf16 and fp8 pools,
both page layouts, cut pairs) against the CPU oracle with the decode
tolerances (bf16 out max-abs 1e-2 / mean-abs 1e-3, fp8 max-abs 4e-2, lse
1e-3), multi-query rows at d 256, and the KV append at d 256 (bit-exact
against the append oracle)."""
import pytest
import torch

import oracle
import synth
from oracle import kv_append as ka
from oracle import multi_query as mq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _run(inp, layout="nhd", force=0, q=None):
    pk = _pk()
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
    fin = torch.isfinite(ref_l)
    assert torch.equal(torch.isneginf(lse.double()), torch.isneginf(ref_l)), tag
    if bool(fin.any()):
        assert float((lse.double()[fin] - ref_l[fin]).abs().max()) <= 1e-3, tag


LENS = (0, 1, 15, 16, 17, 100, 513, 1500, 3000)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_d256_matches_oracle(G, kv, layout):
    w = synth.WORKLOADS["llama3_8b"].with_(batch=len(LENS), num_q_heads=4 * G, num_kv_heads=4, head_dim=256,
                                           lens=("fixed", LENS), kv_dtype=kv, seed=7000 + G)
    inp = synth.make_inputs(w)
    out, lse = _run(inp, layout)
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"],
                                 k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    _check(out, lse, ref_o, ref_l, kv != "bf16", f"d256 G{G} {kv} {layout}")


@pytest.mark.parametrize("force", [1, 7, 100])
def test_d256_cut_pairs_match_oracle(force):
    w = synth.WORKLOADS["llama3_8b"].with_(batch=len(LENS), head_dim=256, lens=("fixed", LENS), seed=7100)
    inp = synth.make_inputs(w)
    out, lse = _run(inp, "hnd", force=force)
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    _check(out, lse, ref_o, ref_l, False, f"d256 workers={force}")


def test_d256_multi_query_matches_oracle():
    w = synth.WORKLOADS["llama3_8b"].with_(batch=len(LENS), head_dim=256, lens=("fixed", LENS), seed=7200)
    inp = synth.make_inputs(w)
    g = torch.Generator().manual_seed(7201)
    q4 = torch.randn((len(LENS), 4, 32, 256), generator=g).to(torch.bfloat16)
    out, lse = _run(inp, "hnd", q=q4)
    ref_o, ref_l = mq.decode_multi_query(q4, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    _check(out, lse, ref_o, ref_l, False, "d256 next_n 4")


def test_d256_full_size_step():
    """A Llama-3-8B-sized step with head_dim 256 (twice the KV bytes)."""
    w = synth.WORKLOADS["llama3_8b"].with_(head_dim=256)
    inp = synth.make_inputs(w)
    out, lse = _run(inp, "hnd")
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    _check(out, lse, ref_o, ref_l, False, "d256 llama3-sized step")


@pytest.mark.parametrize("mode", ["bf16", "fp8", "fp8_pow2"])
def test_d256_append_bit_exact(mode):
    pk = _pk()
    kv = "bf16" if mode == "bf16" else "fp8_e4m3"
    pow2 = mode == "fp8_pow2"
    inp = synth.make_append_inputs(batch=5, num_kv_heads=4, head_dim=256, page_size=16, new_tokens=(1, 40),
                                   context=(0, 50), kv_dtype=kv, seed=7300)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                 d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=pow2)
    torch.cuda.synchronize()
    fp8 = kv != "bf16"
    pool = (lambda t: t.view(torch.uint8).numpy()) if fp8 else (lambda t: t.float().numpy())
    kp, vp, ks, vs = ka.kv_append(pool(inp["k_pages"]).copy(), pool(inp["v_pages"]).copy(),
                                  inp["k_scale"].numpy() if fp8 else None, inp["v_scale"].numpy() if fp8 else None,
                                  inp["k_new"].float().numpy(), inp["v_new"].float().numpy(),
                                  inp["token_seq"].numpy(), inp["token_pos"].numpy(), inp["block_table"].numpy(),
                                  pow2=pow2)
    import numpy as np
    got_k, got_v = pool(d["k_pages"].cpu()), pool(d["v_pages"].cpu())
    if not fp8:
        got_k, got_v, kp, vp = (x.view(np.uint32) for x in (got_k, got_v, kp.astype(np.float32), vp.astype(np.float32)))
    assert np.array_equal(got_k, kp) and np.array_equal(got_v, vp)
    if fp8:
        assert np.array_equal(d["k_scale"].cpu().numpy().view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(d["v_scale"].cpu().numpy().view(np.uint32), vs.view(np.uint32))
