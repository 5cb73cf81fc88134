"""pdattn_decode_noalloc (decode + reduce on the library's static device
scratch) against pdattn_decode + pdattn_reduce on a caller workspace.

The two run the same kernels on the same plan, so their outputs agree to the
parity bar of the decode (out max-abs <= 1e-2, mean-abs <= 1e-3; lse max-abs
<= 1e-3) and are in fact expected to be bitwise equal. Two calls in a row, the
second on a smaller problem, show that what the first call leaves in the
scratch does not leak into the second.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _setup(name, layout):
    pk = _pk()
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(name)
    if layout == pk.LAYOUT_HND:
        inp = synth.to_hnd(inp)
    d = {k: (None if inp[k] is None else inp[k].to(dev))
         for k in ("q", "k_pages", "v_pages", "k_scale", "v_scale", "block_table", "context_lens")}
    num_pages, P, Hkv, _ = pk.pool_dims(d["k_pages"], layout)
    B, Hq, D = d["q"].shape
    pl = pk.plan(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                 max_pages_per_seq=d["block_table"].shape[1], num_pages=num_pages,
                 kv_dtype=pk.kv_kind(d["k_pages"]), context_lens_host=inp["context_lens"], kv_layout=layout)
    return pl, d


def _with_workspace(pl, d):
    pk = _pk()
    B, Hq, D = d["q"].shape
    out = torch.full((B, Hq, D), float("nan"), device=d["q"].device)
    lse = torch.full((B, Hq), float("nan"), device=d["q"].device)
    ws = pk.workspace(pl, d["q"].device)
    pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
              d["context_lens"], ws, out, lse)
    pk.reduce(pl, ws, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _noalloc(pl, d):
    pk = _pk()
    B, Hq, D = d["q"].shape
    out = torch.full((B, Hq, D), float("nan"), device=d["q"].device)
    lse = torch.full((B, Hq), float("nan"), device=d["q"].device)
    pk.decode_noalloc(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"],
                      d["context_lens"], out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(got, ref, tag):
    out, lse = got
    ref_out, ref_lse = ref
    assert bool(torch.isfinite(out).all()), tag
    diff = (out.double() - ref_out.double()).abs()
    mx, mean = float(diff.max()), float(diff.mean())
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isneginf(lse), torch.isneginf(ref_lse)), tag
    ldiff = float((lse[fin].double() - ref_lse[fin].double()).abs().max()) if bool(fin.any()) else 0.0
    print(f"{tag}: out max-abs {mx:.3e} mean-abs {mean:.3e}, lse max-abs {ldiff:.3e}, "
          f"bitwise {torch.equal(out, ref_out) and torch.equal(lse, ref_lse)}", flush=True)
    assert mx <= OUT_MAX and mean <= OUT_MEAN and ldiff <= LSE_MAX, (tag, mx, mean, ldiff)


@pytest.mark.parametrize("layout_name", ["nhd", "hnd"])
def test_noalloc_matches_workspace_path_twice(layout_name):
    pk = _pk()
    layout = pk.LAYOUT_HND if layout_name == "hnd" else pk.LAYOUT_NHD
    # first call: the Llama-3-8B-shaped step; second: a smaller problem
    for name in ("llama3_8b", "tiny"):
        pl, d = _setup(name, layout)
        assert pl.workspace_bytes <= pk.NOALLOC_SCRATCH_BYTES
        print(f"noalloc {name} {layout_name}: workers {pl.num_workers}, scratch bytes {pl.workspace_bytes}",
              flush=True)
        got = _noalloc(pl, d)
        ref = _with_workspace(pl, d)
        _check(got, ref, f"{name} {layout_name}")


def test_noalloc_fp8_pool():
    pk = _pk()
    pl, d = _setup("fp8_kv", pk.LAYOUT_NHD)
    _check(_noalloc(pl, d), _with_workspace(pl, d), "fp8_kv nhd")


def test_noalloc_rejects_oversized_and_balanced_plans():
    pk = _pk()
    pl, d = _setup("tiny", pk.LAYOUT_NHD)
    B, Hq, D = d["q"].shape
    # a worker count whose records exceed the static scratch
    big = pk.plan(batch=B, num_q_heads=Hq, num_kv_heads=d["k_pages"].shape[2], head_dim=D,
                  page_size=d["k_pages"].shape[1], max_pages_per_seq=d["block_table"].shape[1],
                  num_pages=d["k_pages"].shape[0], context_lens_host=[256], force_workers=1 << 16)
    assert big.workspace_bytes > pk.NOALLOC_SCRATCH_BYTES
    out = torch.empty(B, Hq, D, device=d["q"].device)
    with pytest.raises(pk.PdattnError, match="scratch"):
        pk.decode_noalloc(big, d["q"], d["k_pages"], d["v_pages"], None, None, d["block_table"],
                          d["context_lens"], out)
    bal = pk.plan(batch=B, num_q_heads=Hq, num_kv_heads=d["k_pages"].shape[2], head_dim=D,
                  page_size=d["k_pages"].shape[1], max_pages_per_seq=d["block_table"].shape[1],
                  num_pages=d["k_pages"].shape[0], context_lens_host=[256], balanced=True)
    with pytest.raises(pk.PdattnError, match="default-mode"):
        pk.decode_noalloc(bal, d["q"], d["k_pages"], d["v_pages"], None, None, d["block_table"],
                          d["context_lens"], out)
