"""A whole serving step captured in one HIP graph and replayed: KV append
(one new token per sequence, fp8 pool with power-of-two scales, head-major
pages), decode + reduce over the appended context, and a two-piece merge of
the decode with itself. Every call of the path allocates nothing and
enqueues no memset, so it can be captured; each replay (with eager work in
between) must equal the eager step bit for bit (all kernels of a static
plan are deterministic, and the append is idempotent)."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_captured_step_replays_bitwise():
    import paged_kv_split_amd as pk
    inp = synth.make_append_inputs(batch=16, num_kv_heads=8, head_dim=128, page_size=16, new_tokens=1,
                                   context=(100, 2000), kv_dtype="fp8_e4m3", num_q_heads=32, invalid=False,
                                   special_rows=False, spread=0, seed=9000)
    hnd = synth.to_hnd(inp)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in hnd.items()}
    lens_dev = inp["new_lens"].to(DEV)
    pl = pk.plan(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                 max_pages_per_seq=inp["block_table"].shape[1], num_pages=inp["k_pages"].shape[0],
                 kv_dtype=pk.KV_FP8_E4M3, context_lens_host=inp["new_lens"], kv_layout=pk.LAYOUT_HND)
    ws = pk.workspace(pl, DEV)
    out = torch.empty((16, 32, 128), device=DEV)
    lse = torch.empty((16, 32), device=DEV)
    parts_o = torch.empty((2, 16, 32, 128), device=DEV)
    parts_l = torch.empty((2, 16, 32), device=DEV)
    mo = torch.empty((16, 32, 128), device=DEV)
    ml = torch.empty((16, 32), device=DEV)

    def step():
        pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                     d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=True, layout=pk.LAYOUT_HND)
        pk.decode(pl, d["q"], d["k_pages"], d["v_pages"], d["k_scale"], d["v_scale"], d["block_table"], lens_dev,
                  ws, out, lse)
        pk.reduce(pl, ws, out, lse)
        parts_o[0].copy_(out)
        parts_o[1].copy_(out)
        parts_l[0].copy_(lse)
        parts_l[1].copy_(lse)
        pk.merge(parts_o, parts_l, mo, ml)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, mo, ml, d["k_pages"].view(torch.uint8), d["k_scale"])]
    assert bool(torch.isfinite(out).all())
    # merging a result with itself: same output, lse + ln 2
    assert float((mo - out).abs().max()) <= 1e-6
    assert float((ml - lse - 0.6931471805599453).abs().max()) <= 1e-5

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (out, lse, mo, ml):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = (out, lse, mo, ml, d["k_pages"].view(torch.uint8), d["k_scale"])
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
        step()  # eager work between replays
        torch.cuda.synchronize()
