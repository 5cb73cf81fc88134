"""The inline-scale fp8 cache (PDATTN_KV_FP8_E4M3_INLINE: each pool row is
its d e4m3fn codes followed by its fp32 scale) on the GPU.

* decode and multi-query decode over inline pools (4-byte loads in
  token-major pools, raw 16-byte row blocks in head-major pools) against
  the oracle, fed the same codes and scales unpacked (fp8 tolerances:
  max-abs 4e-2, mean-abs 1e-3, lse 1e-3);
* the same calls on the separate-scale pools holding the same values give
  the same outputs bit for bit: both inline paths give the registers the
  values the separate-scale path gives them, and the arithmetic is shared;
* NaN codes and scales in the unused slots past a sequence's length (read
  raw by the head-major path) do not reach the outputs;
* the fp8 append into inline pools (plain and power-of-two scales) equals
  the append oracle's pools, packed, byte for byte; untouched rows stay;
* the calls this layout does not serve return errors.
"""
import pytest
import torch

import oracle
import synth
from oracle import kv_append as oka
from oracle import multi_query as mq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


CASES = [
    # Hq, Hkv, D, P, lens, q_len
    (32, 8, 128, 16, (1, 15, 16, 17, 300, 513, 1000, 0), 1),
    (8, 2, 64, 8, (3, 77, 256, 129), 1),
    (16, 2, 256, 32, (5, 400, 64), 1),
    (16, 4, 128, 16, (40, 200, 7), 4),      # multi-query: 4 rows x G 4 = 16 columns
    (12, 4, 128, 16, (33, 250), 1),         # G 3
]


def _inputs(case, seed):
    Hq, Hkv, D, P, lens, n = case
    w = synth.WORKLOADS["fp8_kv"].with_(batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                                        lens=("fixed", tuple(lens)), seed=seed)
    inp = synth.make_inputs(w)
    if n > 1:
        g = torch.Generator().manual_seed(seed + 3)
        inp["q"] = torch.randn((len(lens), n, Hq, D), generator=g).to(torch.bfloat16)
    return inp


def _decode(inp, layout):
    pk = _pk()
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (src[k].to(DEV) if src.get(k) is not None else None)
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    out, lse = pk.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                               context_lens_host=inp["context_lens"], k_scale=d["k_scale"], v_scale=d["v_scale"],
                               layout=pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("case", CASES, ids=[f"G{c[0] // c[1]}_d{c[2]}_P{c[3]}_n{c[5]}" for c in CASES])
def test_inline_decode_matches_oracle_and_separate_scales(case, layout):
    inp = _inputs(case, seed=6100 + case[2] + case[0])
    il = synth.to_inline(inp)
    out_i, lse_i = _decode(il, layout)
    out_s, lse_s = _decode(inp, layout)
    assert torch.equal(out_i, out_s) and torch.equal(lse_i, lse_s), "inline and separate scales differ"
    if inp["q"].dim() == 4:
        ref_o, ref_l = mq.decode_multi_query(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                             inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    else:
        ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                     inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    diff = (out_i.double() - ref_o).abs()
    print(f"{case} {layout}: max-abs {float(diff.max()):.2e} mean-abs {float(diff.mean()):.2e}")
    assert bool(torch.isfinite(out_i).all())
    assert float(diff.max()) <= 4e-2 and float(diff.mean()) <= 1e-3
    assert torch.equal(torch.isneginf(lse_i.double()), torch.isneginf(ref_l))
    fin = torch.isfinite(ref_l)
    assert float((lse_i.double()[fin] - ref_l[fin]).abs().max()) <= 1e-3


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("pow2", [False, True])
def test_inline_append_bit_exact(pow2, layout):
    pk = _pk()
    inp = synth.make_append_inputs(batch=5, num_kv_heads=4, head_dim=128, page_size=16, new_tokens=(1, 40),
                                   context=(0, 60), kv_dtype="fp8_e4m3", seed=6200 + pow2 * 3 + (layout == "hnd"))
    kp, vp, ks, vs = oka.kv_append(inp["k_pages"].view(torch.uint8).numpy(), inp["v_pages"].view(torch.uint8).numpy(),
                                   inp["k_scale"].numpy(), inp["v_scale"].numpy(), inp["k_new"].float().numpy(),
                                   inp["v_new"].float().numpy(), inp["token_seq"].numpy(), inp["token_pos"].numpy(),
                                   inp["block_table"].numpy(), pow2=pow2)
    want = synth.to_inline(dict(k_pages=torch.from_numpy(kp), v_pages=torch.from_numpy(vp),
                                k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs)))
    il = synth.to_inline(inp)
    src = synth.to_hnd(il) if layout == "hnd" else il
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in src.items()}
    lay = pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD
    pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                 d["v_pages"], None, None, pow2_scales=pow2, layout=lay)
    torch.cuda.synchronize()
    got_k, got_v = d["k_pages"].cpu(), d["v_pages"].cpu()
    if layout == "hnd":
        got_k, got_v = synth.from_hnd(got_k).contiguous(), synth.from_hnd(got_v).contiguous()
    assert torch.equal(got_k, want["k_pages"]) and torch.equal(got_v, want["v_pages"])


def test_inline_unsupported_calls_fail():
    pk = _pk()
    inp = synth.to_inline(_inputs(CASES[0], seed=6300))
    d = {k: (inp[k].to(DEV) if inp.get(k) is not None else None)
         for k in ("q", "k_pages", "v_pages", "block_table", "context_lens")}
    with pytest.raises(pk.PdattnError):      # balanced plans
        pk.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                        context_lens_host=inp["context_lens"], balanced=True)
    with pytest.raises(pk.PdattnError):      # separate scale arrays with inline pools
        sc = torch.ones(d["k_pages"].shape[:3], device=DEV)
        pk.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                        context_lens_host=inp["context_lens"], k_scale=sc, v_scale=sc)
    q = torch.zeros((4, 32, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pk.PdattnError):      # the prefill with separate scale arrays too
        pk.paged_prefill(q, torch.tensor([0, 4] + [4] * 7, dtype=torch.int32, device=DEV), d["k_pages"],
                         d["v_pages"], d["block_table"], d["context_lens"], k_scale=sc, v_scale=sc)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("P", [8, 16, 64])
def test_inline_unused_tail_slots_do_not_leak(layout, P):
    """The slots of a sequence's last page past its length hold NaN codes
    and NaN scales; head-major inline pools read those rows raw (whole
    blocks), and their zero weights must still give finite, correct
    outputs."""
    case = (32, 8, 128, P, (1, 9, 17, 100, 255, 300), 1)
    inp = _inputs(case, seed=6400 + P)
    bt, lens = inp["block_table"], inp["context_lens"]
    for b, L in enumerate(lens.tolist()):
        if L % P:
            page = int(bt[b, L // P])
            inp["k_pages"].view(torch.uint8)[page, L % P:] = 0x7F
            inp["v_pages"].view(torch.uint8)[page, L % P:] = 0x7F
            inp["k_scale"][page, L % P:] = float("nan")
            inp["v_scale"][page, L % P:] = float("nan")
    out, lse = _decode(synth.to_inline(inp), layout)
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], bt, lens, k_scale=inp["k_scale"],
                                 v_scale=inp["v_scale"])
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    diff = (out.double() - ref_o).abs()
    assert float(diff.max()) <= 4e-2 and float(diff.mean()) <= 1e-3
    assert float((lse.double() - ref_l).abs().max()) <= 1e-3
