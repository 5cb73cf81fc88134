"""Parity of the HIP KV append (pdattn_kv_append, through the C ABI) with the
CPU oracle (oracle/kv_append.py).

The append is byte work: the bar is bit-exact. bf16 pools must equal the
oracle's bit for bit; fp8 pools must hold the oracle's codes and fp32 scales
exactly (both sides take every rounding decision in fp32: a correctly
rounded division, then round to nearest even onto the e4m3 grid), and no
other byte of any pool may change. A decode over the appended pool is then
held to the decode tolerances against the oracle's decode of the oracle's
appended pool.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import kv_append as ka

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def _np_pool(t):
    """A pool as numpy: bf16 -> float32 values, fp8 -> uint8 codes."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    return t.to(torch.float32).numpy().copy()


def run_gpu(inp, pow2=False, hnd=False):
    """Append on the device; with hnd the pools are laid out [page][kv head]
    [slot] for the call and returned in the token-major order."""
    pk = _pk()
    src = synth.to_hnd(inp) if hnd else inp
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in src.items()}
    pk.kv_append(d["k_new"], d["v_new"], d["token_seq"], d["token_pos"], d["block_table"], d["k_pages"],
                 d["v_pages"], d["k_scale"], d["v_scale"], pow2_scales=pow2,
                 layout=pk.LAYOUT_HND if hnd else pk.LAYOUT_NHD)
    torch.cuda.synchronize()
    if hnd:
        for k in ("k_pages", "v_pages", "k_scale", "v_scale"):
            if d[k] is not None:
                d[k] = synth.from_hnd(d[k]).contiguous()
    return d


def run_oracle(inp, pow2=False):
    fp8 = inp["k_scale"] is not None
    return ka.kv_append(_np_pool(inp["k_pages"]), _np_pool(inp["v_pages"]),
                        inp["k_scale"].numpy() if fp8 else None, inp["v_scale"].numpy() if fp8 else None,
                        inp["k_new"].to(torch.float32).numpy(), inp["v_new"].to(torch.float32).numpy(),
                        inp["token_seq"].numpy(), inp["token_pos"].numpy(), inp["block_table"].numpy(),
                        pow2=pow2)


def assert_pools_equal(d, ref, tag):
    """Bit-exact comparison of the device pools with the oracle's."""
    kp, vp, ks, vs = ref
    for name, got, want in (("k_pages", d["k_pages"], kp), ("v_pages", d["v_pages"], vp)):
        g = _np_pool(got.cpu())
        if g.dtype == np.float32:
            g, want = g.view(np.uint32), want.astype(np.float32).view(np.uint32)
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"{tag} {name}: {len(bad)} elements differ, first at {bad[:4].tolist()}"
    if ks is not None:
        for name, got, want in (("k_scale", d["k_scale"], ks), ("v_scale", d["v_scale"], vs)):
            g = got.cpu().numpy().view(np.uint32)
            bad = np.argwhere(g != want.astype(np.float32).view(np.uint32))
            assert bad.size == 0, f"{tag} {name}: {len(bad)} scales differ, first at {bad[:4].tolist()}"


def test_hardware_fp8_conversion_matches_the_format_definition():
    """The append's float -> e4m3fn conversion instruction against the
    format's definition over every fp32 value with |y| <= 448 (both signs)."""
    assert _pk().fp8_conversion_check(DEV) == 0


CASES = [
    # (head_dim, page_size, Hkv, batch, new_tokens, context)
    (128, 16, 8, 6, (1, 70), (0, 100)),
    (64, 8, 2, 5, (1, 40), (0, 30)),
    (128, 128, 4, 3, (100, 300), (0, 200)),
    # a token's rows span several 1 KB steps, a partial last step, less than one step
    (128, 16, 16, 4, (1, 50), (0, 60)),
    (128, 32, 5, 4, (1, 50), (0, 60)),
    (64, 16, 1, 4, (1, 50), (0, 60)),
]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("case", CASES, ids=["d128_p16", "d64_p8", "d128_p128", "d128_hkv16", "d128_hkv5",
                                             "d64_hkv1"])
@pytest.mark.parametrize("mode", ["bf16", "fp8", "fp8_pow2"])
def test_append_matches_oracle_bit_exact(case, mode, layout):
    D, P, Hkv, B, new, ctx = case
    kv = "bf16" if mode == "bf16" else "fp8_e4m3"
    pow2 = mode == "fp8_pow2"
    inp = synth.make_append_inputs(batch=B, num_kv_heads=Hkv, head_dim=D, page_size=P, new_tokens=new,
                                   context=ctx, kv_dtype=kv, seed=3000 + D + P)
    tag = f"append {mode} {layout} d{D} P{P} Hkv{Hkv} N{inp['token_seq'].numel()}"
    print(tag, flush=True)
    d = run_gpu(inp, pow2, hnd=layout == "hnd")
    assert_pools_equal(d, run_oracle(inp, pow2), tag)


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_append_of_nothing_and_of_unresolved_tokens_changes_nothing(mode):
    kv = "bf16" if mode == "bf16" else "fp8_e4m3"
    inp = synth.make_append_inputs(batch=3, num_kv_heads=4, head_dim=128, page_size=16, new_tokens=0,
                                   context=(5, 40), kv_dtype=kv, seed=3100)
    assert inp["token_seq"].numel() == 5    # only the five tokens that do not resolve
    before = {k: inp[k].clone() for k in ("k_pages", "v_pages") }
    d = run_gpu(inp)
    for k in before:
        assert torch.equal(d[k].cpu().view(torch.uint8), before[k].view(torch.uint8)), k
    empty = dict(inp, k_new=inp["k_new"][:0], v_new=inp["v_new"][:0], token_seq=inp["token_seq"][:0],
                 token_pos=inp["token_pos"][:0])
    d = run_gpu(empty)
    for k in before:
        assert torch.equal(d[k].cpu().view(torch.uint8), before[k].view(torch.uint8)), k


def test_fp8_extremes_bit_exact():
    """Rows at the edges of the fp32 and e4m3 ranges: bf16's largest finite
    magnitude, bf16 subnormals, a lone nonzero, values that round onto ties
    at every e4m3 exponent, and rows around absmax 2^-82."""
    pk = _pk()
    Hkv, D, P = 1, 128, 16
    vals = []
    big = torch.tensor(3.3895e38).to(torch.bfloat16).float()
    vals.append(torch.full((D,), float(big)) * torch.sign(torch.randn(D, generator=torch.Generator().manual_seed(1))))
    vals.append(torch.arange(D, dtype=torch.float32) * 2.0 ** -133)        # bf16 subnormals
    one = torch.zeros(D)
    one[77] = -2.0 ** -100
    vals.append(one)
    # x / s on the midpoints between neighbouring e4m3 values (s = 2^-5 for absmax 14)
    fin = ka.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = torch.tensor(((fin[:-1] + fin[1:]) / 2) * 2.0 ** -5, dtype=torch.float32)
    mids = mids[mids.to(torch.bfloat16).float() == mids]
    row = torch.zeros(D)
    row[0] = 14.0
    row[1:1 + min(len(mids), D - 1)] = mids[:D - 1]
    vals.append(row)
    vals.append(-row)
    # rows on both sides of absmax 2^-82, where plain scales switch from the
    # refined reciprocal to a division per element
    g = torch.Generator().manual_seed(2)
    for top in (2.0 ** -82, 1.5 * 2.0 ** -83, 2.0 ** -81):
        r = torch.randn(D, generator=g) * 2.0 ** -84
        r = r.to(torch.bfloat16).float().clamp(-top, top)
        r[5] = top
        vals.append(r)
    rows = torch.stack(vals)[:, None, :].to(torch.bfloat16)           # [N, 1, D]
    N = rows.shape[0]
    for pow2 in (False, True):
        kp = torch.zeros((N, P, Hkv, D), dtype=torch.uint8).view(torch.float8_e4m3fn)
        sc = torch.zeros((N, P, Hkv), dtype=torch.float32)
        inp = dict(k_new=rows, v_new=rows.flip(0).contiguous(), token_seq=torch.arange(N, dtype=torch.int32),
                   token_pos=torch.full((N,), 3, dtype=torch.int32),
                   block_table=torch.arange(N, dtype=torch.int32)[:, None].contiguous(),
                   k_pages=kp, v_pages=kp.clone(), k_scale=sc, v_scale=sc.clone())
        d = run_gpu(inp, pow2)
        assert_pools_equal(d, run_oracle(inp, pow2), f"extremes pow2={pow2}")


@pytest.mark.parametrize("mode", ["bf16", "fp8", "fp8_pow2"])
def test_decode_after_append_matches_oracle(mode):
    """One decode step's append (one new token per sequence, at position L_b)
    followed by the decode over L_b + 1 tokens, against the oracle's append
    and the oracle's decode."""
    pk = _pk()
    kv = "bf16" if mode == "bf16" else "fp8_e4m3"
    pow2 = mode == "fp8_pow2"
    inp = synth.make_append_inputs(batch=8, num_kv_heads=8, head_dim=128, page_size=16, new_tokens=1,
                                   context=(0, 700), kv_dtype=kv, num_q_heads=32, invalid=False,
                                   special_rows=False, spread=0, seed=3200)
    d = run_gpu(inp, pow2)
    lens = inp["new_lens"]
    out, lse = pk.paged_decode(inp["q"].to(DEV), d["k_pages"], d["v_pages"], d["block_table"], lens.to(DEV),
                               context_lens_host=lens, k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    kp, vp, ks, vs = run_oracle(inp, pow2)
    if kv == "bf16":
        kpt, vpt = torch.from_numpy(kp).to(torch.bfloat16), torch.from_numpy(vp).to(torch.bfloat16)
        kst = vst = None
    else:
        kpt = torch.from_numpy(kp).view(torch.float8_e4m3fn)
        vpt = torch.from_numpy(vp).view(torch.float8_e4m3fn)
        kst, vst = torch.from_numpy(ks), torch.from_numpy(vs)
    ref_out, ref_lse = oracle.decode(inp["q"], kpt, vpt, inp["block_table"], lens, k_scale=kst, v_scale=vst)
    mx_tol = 1e-2 if kv == "bf16" else 4e-2
    diff = (out.cpu().to(torch.float64) - ref_out).abs()
    print(f"decode after append {mode}: max-abs {float(diff.max()):.3e} mean-abs {float(diff.mean()):.3e}",
          flush=True)
    assert float(diff.max()) <= mx_tol and float(diff.mean()) <= 1e-3
    assert float((lse.cpu().to(torch.float64) - ref_lse).abs().max()) <= 1e-3


@pytest.mark.parametrize("mode", ["bf16", "fp8_pow2"])
def test_prefill_sized_append_sampled(mode):
    """The append the benchmark times (16 sequences x 512 new tokens, 8 kv
    heads, d128, P16): every written row of a sample of 512 (token, kv head)
    rows against the oracle, bit-exact, and every slot no token names
    unchanged."""
    kv = "bf16" if mode == "bf16" else "fp8_e4m3"
    pow2 = mode == "fp8_pow2"
    inp = synth.make_append_inputs(batch=16, num_kv_heads=8, head_dim=128, page_size=16, new_tokens=512,
                                   context=(0, 0), kv_dtype=kv, invalid=False, special_rows=True, seed=3300)
    before_k = inp["k_pages"].clone()
    d = run_gpu(inp, pow2)
    g = torch.Generator().manual_seed(7)
    N = inp["token_seq"].numel()
    pick = torch.randperm(N, generator=g)[:64]
    sub = dict(inp, k_new=inp["k_new"][pick].contiguous(), v_new=inp["v_new"][pick].contiguous(),
               token_seq=inp["token_seq"][pick].contiguous(), token_pos=inp["token_pos"][pick].contiguous())
    kp, vp, ks, vs = run_oracle(sub, pow2)
    got_k = _np_pool(d["k_pages"].cpu())
    got_v = _np_pool(d["v_pages"].cpu())
    bt = inp["block_table"]
    P = 16
    for j in range(pick.numel()):
        b, t = int(sub["token_seq"][j]), int(sub["token_pos"][j])
        page, slot = int(bt[b, t // P]), t % P
        for got, want in ((got_k, kp), (got_v, vp)):
            a, w = got[page, slot], want[page, slot]
            if a.dtype == np.float32:
                a, w = a.view(np.uint32), w.astype(np.float32).view(np.uint32)
            assert np.array_equal(a, w), (mode, j, b, t)
        if ks is not None:
            assert np.array_equal(d["k_scale"][page, slot].cpu().numpy(), ks[page, slot])
            assert np.array_equal(d["v_scale"][page, slot].cpu().numpy(), vs[page, slot])
    # slots that no token names: pages outside every block-table row
    named = torch.zeros(before_k.shape[0], dtype=torch.bool)
    named[bt[bt >= 0].long()] = True
    assert torch.equal(d["k_pages"].cpu()[~named].view(torch.uint8), before_k[~named].view(torch.uint8))
