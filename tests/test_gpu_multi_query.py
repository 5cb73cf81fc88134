"""Multi-query paged decode on the GPU (q_len = n query rows per sequence,
causal over the last n positions) against the CPU oracle
(oracle/multi_query.py), with the decode tolerances: bf16 out max-abs 1e-2
and mean-abs 1e-3, fp8 max-abs 4e-2, lse max-abs 1e-3. Also: each query row
equals the one-token decode with the row's shifted length on the GPU
(fp32 summation order only, 1e-5)."""
import pytest
import torch

import synth
from oracle import multi_query as mq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _inputs(name, lens, n, Hq=None, Hkv=None, D=None, P=None, seed=0):
    w = synth.WORKLOADS[name]
    kw = dict(batch=len(lens), lens=("fixed", tuple(lens)), seed=w.seed + 7 + seed)
    for k, v in (("num_q_heads", Hq), ("num_kv_heads", Hkv), ("head_dim", D), ("page_size", P)):
        if v is not None:
            kw[k] = v
    inp = synth.make_inputs(w.with_(**kw))
    g = torch.Generator().manual_seed(900 + seed)
    B, Hq_, D_ = inp["q"].shape
    inp["q4"] = torch.randn((B, n, Hq_, D_), generator=g).to(torch.bfloat16)
    return inp


def _run(inp, layout="nhd", force=0):
    pk = _pk()
    src = synth.to_hnd(inp) if layout == "hnd" else inp
    d = {k: (src[k].to(DEV) if src[k] is not None else None)
         for k in ("q4", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    out, lse = pk.paged_decode(d["q4"], d["k_pages"], d["v_pages"], d["block_table"], d["context_lens"],
                               context_lens_host=inp["context_lens"], k_scale=d["k_scale"], v_scale=d["v_scale"],
                               force_workers=force,
                               layout=pk.LAYOUT_HND if layout == "hnd" else pk.LAYOUT_NHD)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(out, lse, inp, tag):
    ref_o, ref_l = mq.decode_multi_query(inp["q4"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                         inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    fp8 = inp["k_scale"] is not None
    diff = (out.double() - ref_o).abs()
    assert bool(torch.isfinite(out).all()), tag
    mx, mean = float(diff.max()), float(diff.mean())
    print(f"{tag}: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)
    assert mx <= (4e-2 if fp8 else 1e-2) and mean <= 1e-3, (tag, mx, mean)
    assert torch.equal(torch.isneginf(lse.double()), torch.isneginf(ref_l)), tag
    fin = torch.isfinite(ref_l)
    if bool(fin.any()):
        assert float((lse.double()[fin] - ref_l[fin]).abs().max()) <= 1e-3, tag


LENS = (0, 1, 3, 4, 5, 16, 17, 31, 33, 250, 513, 1000)

CASES = [
    # name, Hq, Hkv, n, D, P: columns n * Hq / Hkv in {2, 4, 8, 16}
    ("tiny", 8, 2, 4, 64, 16),        # G 4 x 4 rows = 16 columns
    ("llama3_8b", 32, 8, 4, 128, 16),  # next_n 4 on the Llama-3-8B heads
    ("llama3_8b", 32, 8, 2, 128, 16),  # 8 columns
    ("long_ctx", 64, 8, 2, 128, 64),   # G 8 x 2
    ("llama3_8b", 16, 8, 8, 128, 16),  # G 2 x 8
    ("tiny", 8, 8, 16, 64, 8),         # G 1 x 16
    ("fp8_kv", 32, 8, 4, 128, 16),
    ("tiny", 8, 2, 1, 64, 16),         # one row through the four-dimensional path
]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_G{c[1] // c[2]}_n{c[3]}_d{c[4]}_P{c[5]}" for c in CASES])
def test_multi_query_matches_oracle(case, layout):
    name, Hq, Hkv, n, D, P = case
    inp = _inputs(name, LENS, n, Hq, Hkv, D, P, seed=n)
    out, lse = _run(inp, layout)
    _check(out, lse, inp, f"{name} G{Hq // Hkv} n{n} {layout}")


@pytest.mark.parametrize("force", [1, 5, 37, 300])
def test_multi_query_cut_pairs_match_oracle(force):
    """Forced worker counts cut pairs at odd tiles, so pieces meet in the
    split merge, which maps columns back to (query row, head)."""
    inp = _inputs("llama3_8b", LENS, 4, seed=11)
    out, lse = _run(inp, "hnd", force=force)
    _check(out, lse, inp, f"llama3_8b n4 workers={force}")


def test_rows_equal_one_token_decodes_with_shifted_lengths():
    """With 16 columns (4 rows x 4 heads) the kernel forms p . V on the
    matrix cores from bf16-rounded probabilities (each within 2^-9 of its
    fp32 value); the one-token decodes (4 columns) keep fp32 probabilities.
    So |difference| <= 2^-9 * sum_t p_t |V_t| / l <= 2^-9 * max |V| (plus
    fp32 summation order); lse is formed from fp32 probabilities in both."""
    pk = _pk()
    n = 4
    inp = _inputs("llama3_8b", LENS, n, seed=13)
    out, lse = _run(inp)
    d = {k: (inp[k].to(DEV) if inp[k] is not None else None)
         for k in ("k_pages", "v_pages", "k_scale", "v_scale", "block_table")}
    for i in range(n):
        lens_i = (inp["context_lens"].to(torch.int64) - (n - 1 - i)).clamp(min=0).to(torch.int32)
        o1, l1 = pk.paged_decode(inp["q4"][:, i].contiguous().to(DEV), d["k_pages"], d["v_pages"], d["block_table"],
                                 lens_i.to(DEV), context_lens_host=lens_i)
        torch.cuda.synchronize()
        vv = inp["v_pages"].float()
        vmax = float(vv[torch.isfinite(vv)].abs().max())   # unreferenced pages hold NaN
        assert float((out[:, i] - o1.cpu()).abs().max()) <= 2.0 ** -9 * vmax + 1e-5, i
        assert torch.equal(torch.isneginf(lse[:, i]), torch.isneginf(l1.cpu())), i
        fin = torch.isfinite(l1.cpu())
        assert float((lse[:, i][fin] - l1.cpu()[fin]).abs().max()) <= 1e-5, i


def test_full_size_llama3_next_n_4():
    """The Llama-3-8B step with four speculative rows per sequence."""
    inp = synth.make_inputs("llama3_8b")
    g = torch.Generator().manual_seed(4242)
    inp["q4"] = torch.randn((32, 4, 32, 128), generator=g).to(torch.bfloat16)
    out, lse = _run(inp, "hnd")
    _check(out, lse, inp, "llama3_8b full next_n=4 hnd")
