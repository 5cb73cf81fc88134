"""Pins for the CPU fp64 oracle (CPU only).

The oracle evaluates the definition of paged GQA decode attention directly
(FlashQuant wiki "CUDA Kernels": flash_attention.cu Online Softmax and GQA
Support, paged_decode.cu Page Table Addressing, split_k_reduce.cu Algorithm;
AstrAI "CUDA Kernels": Python Wrappers for layout and scale; OASR "Kernel
Layer": FP8 KV variants for the fp8 scale semantics). Nothing here trusts it
on its own word: it is checked against two independent dense references,
closed forms, invariants the definition fixes, a hand-solved worked example,
torch's own e4m3fn decoding, and a set of deliberately broken builds that the
pins must reject.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def small(B=3, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 0, 37), kv="bf16", seed=7, pool="2x"):
    return synth.Workload("small", "small oracle test case", B, Hq, Hkv, D, P, lens,
                          kv_dtype=kv, pool=pool, seed=seed)


def run(inp, library=None, **kw):
    return oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                         inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                         library=library, **kw)


def close(a, b, tol=1e-12):
    a = torch.as_tensor(a, dtype=torch.float64)
    b = torch.as_tensor(b, dtype=torch.float64)
    if a.shape != b.shape:
        return False
    both_inf = torch.isinf(a) & torch.isinf(b) & (torch.sign(a) == torch.sign(b))
    diff = torch.where(both_inf, torch.zeros_like(a), (a - b).abs())
    return bool(torch.isfinite(diff).all()) and float(diff.max()) <= tol if diff.numel() else True


CASES = [
    small(),
    small(B=2, Hq=4, Hkv=4, D=8, P=1, lens=("uniform", 1, 9), seed=11),            # MHA, P=1
    small(B=4, Hq=16, Hkv=2, D=64, P=16, lens=("uniform", 1, 70), seed=12),       # G=8
    small(B=2, Hq=2, Hkv=1, D=32, P=8, lens=("fixed", (0, 33)), seed=13),         # empty seq
    small(B=3, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 1, 30), kv="fp8_e4m3", seed=14),
    small(B=2, Hq=16, Hkv=1, D=64, P=16, lens=("uniform", 20, 90), kv="fp8_e4m3", seed=15),
]


# -- agreement with independent dense references ------------------------------

@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.kv_dtype}-G{w.num_q_heads // w.num_kv_heads}"
                         f"-D{w.head_dim}-P{w.page_size}-s{w.seed}")
def test_matches_numpy_bruteforce(w):
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    ref_out, ref_lse = brute.numpy_decode(inp["q"], inp["k_pages"], inp["v_pages"],
                                          inp["block_table"], inp["context_lens"],
                                          k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    assert close(out, ref_out)
    assert close(lse, ref_lse)


@pytest.mark.parametrize("w", CASES[:3] + CASES[4:], ids=lambda w: f"{w.kv_dtype}-s{w.seed}")
def test_matches_torch_sdpa(w):
    inp = synth.make_inputs(w)
    out, _ = run(inp)
    ref = brute.sdpa_decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                            inp["context_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    assert close(out, ref)


# -- hand-solved worked example -------------------------------------------------

def _golden():
    with open(os.path.join(HERE, "golden", "paged_worked_example.json")) as f:
        g = json.load(f)

    def t(x, dtype):
        return torch.tensor(np.array(x, dtype=np.float64), dtype=torch.float32).to(dtype)
    inp = dict(q=t(g["q"], torch.bfloat16), k_pages=t(g["k_pages"], torch.bfloat16),
               v_pages=t(g["v_pages"], torch.bfloat16), k_scale=None, v_scale=None,
               block_table=torch.tensor(g["block_table"], dtype=torch.int32),
               context_lens=torch.tensor(g["context_lens"], dtype=torch.int32))
    return g, inp


def test_worked_example_closed_form():
    g, inp = _golden()
    out, lse = run(inp, scale=g["problem"]["scale"])
    e = math.e
    z0 = 1 + e + e * e
    z1 = math.exp(5) + math.exp(-3) + math.exp(7)
    want_out = [[[(1 + e * e) / z0, (e + e * e) / z0],
                 [(math.exp(5) + math.exp(7)) / z1, (math.exp(-3) + math.exp(7)) / z1]]]
    want_lse = [[math.log(z0), math.log(z1)]]
    assert close(out, want_out, 1e-14)
    assert close(lse, want_lse, 1e-14)


# -- closed forms ---------------------------------------------------------------

def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def test_single_token_returns_its_v_row_exactly():
    w = small(B=4, Hq=8, Hkv=2, D=32, P=8, lens=("fixed", (1, 1, 1, 1)), seed=21)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    G = 4
    for b in range(4):
        page = int(inp["block_table"][b, 0])
        for h in range(8):
            v = inp["v_pages"][page, 0, h // G].to(torch.float64)
            k = inp["k_pages"][page, 0, h // G].to(torch.float64)
            assert torch.equal(out[b, h], v)
            s = float((inp["q"][b, h].to(torch.float64) * k).sum()) * inp["scale"]
            assert abs(float(lse[b, h]) - s) <= 1e-12


def test_two_tokens_sigmoid():
    w = small(B=1, Hq=2, Hkv=1, D=16, P=2, lens=("fixed", (2,)), seed=22)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    page = int(inp["block_table"][0, 0])
    k = inp["k_pages"][page, :, 0].to(torch.float64)
    v = inp["v_pages"][page, :, 0].to(torch.float64)
    for h in range(2):
        q = inp["q"][0, h].to(torch.float64)
        s0 = float(k[0] @ q) * inp["scale"]
        s1 = float(k[1] @ q) * inp["scale"]
        sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        want = sig * v[0] + (1.0 - sig) * v[1]
        assert close(out[0, h], want)
        assert abs(float(lse[0, h]) - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) <= 1e-12


def _gathered_mean(inp, b, kvh):
    L = int(inp["context_lens"][b])
    V = brute.gather_dense(inp["v_pages"], inp["v_scale"], inp["block_table"], L, b)
    return V[:, kvh, :].mean(0)


def test_zero_query_gives_mean_of_v():
    w = small(B=3, Hq=4, Hkv=2, D=16, P=4, lens=("uniform", 1, 40), seed=23)
    inp = synth.make_inputs(w)
    inp["q"] = torch.zeros_like(inp["q"])
    out, lse = run(inp)
    for b in range(3):
        L = int(inp["context_lens"][b])
        for h in range(4):
            assert close(out[b, h], _gathered_mean(inp, b, h // 2))
            assert abs(float(lse[b, h]) - math.log(L)) <= 1e-12


def test_zero_scale_gives_mean_of_v():
    w = small(B=2, Hq=4, Hkv=1, D=16, P=4, lens=("uniform", 1, 40), seed=24)
    inp = synth.make_inputs(w)
    out, _ = run(inp, scale=0.0)
    for b in range(2):
        for h in range(4):
            assert close(out[b, h], _gathered_mean(inp, b, 0))


def test_constant_v_returns_the_constant():
    w = small(B=2, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 1, 40), seed=25)
    inp = synth.make_inputs(w)
    c = _bf16(torch.linspace(-3, 3, 16))
    inp["v_pages"] = c.expand_as(inp["v_pages"]).contiguous()
    out, _ = run(inp)
    for b in range(2):
        for h in range(8):
            assert close(out[b, h], c.to(torch.float64), 1e-13)


def test_equal_scores_give_mean_and_lse_shift():
    w = small(B=2, Hq=4, Hkv=2, D=16, P=4, lens=("uniform", 2, 40), seed=26)
    inp = synth.make_inputs(w)
    krow = _bf16(torch.linspace(-1, 1, 16))
    inp["k_pages"] = krow.expand_as(inp["k_pages"]).contiguous()
    out, lse = run(inp)
    for b in range(2):
        L = int(inp["context_lens"][b])
        for h in range(4):
            s = float((inp["q"][b, h].to(torch.float64) * krow.to(torch.float64)).sum()) * inp["scale"]
            assert close(out[b, h], _gathered_mean(inp, b, h // 2))
            assert abs(float(lse[b, h]) - (s + math.log(L))) <= 1e-12


def test_dominant_score_returns_its_v_row():
    # token 5 of sequence 0 scores 1024 above every other token: exp(-1024)
    # underflows to zero in double, so the output is that token's V row.
    w = small(B=1, Hq=2, Hkv=1, D=4, P=4, lens=("fixed", (9,)), seed=27)
    inp = synth.make_inputs(w)
    inp["q"] = _bf16([[[1, 0, 0, 0], [1, 0, 0, 0]]])
    k = torch.zeros(inp["k_pages"].shape)
    bt = inp["block_table"][0]
    k[int(bt[5 // 4]), 5 % 4, 0, 0] = 1024.0
    inp["k_pages"] = k.to(torch.bfloat16)
    out, lse = run(inp, scale=1.0)
    v5 = inp["v_pages"][int(bt[1]), 1, 0].to(torch.float64)
    assert torch.equal(out[0, 0], v5) and torch.equal(out[0, 1], v5)
    assert abs(float(lse[0, 0]) - 1024.0) <= 1e-12


def test_empty_sequence_gives_zero_and_minus_inf():
    w = small(B=2, Hq=4, Hkv=2, D=8, P=4, lens=("fixed", (0, 5)), seed=28)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    assert torch.equal(out[0], torch.zeros(4, 8, dtype=torch.float64))
    assert bool(torch.isneginf(lse[0]).all())
    assert bool(torch.isfinite(lse[1]).all())


# -- invariants of the paged definition -------------------------------------------

def test_page_permutation_leaves_output_bitwise_unchanged():
    w = small(B=4, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 1, 60), seed=31)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    n = inp["k_pages"].shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    moved = dict(inp)
    for key in ("k_pages", "v_pages"):
        dst = torch.empty_like(inp[key])
        dst[perm] = inp[key]
        moved[key] = dst
    bt = inp["block_table"].clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].to(torch.int32)
    moved["block_table"] = bt
    out2, lse2 = run(moved)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_poison_in_unreferenced_pages_and_tail_slots_does_not_leak():
    w = small(B=3, Hq=8, Hkv=2, D=16, P=8, lens=("fixed", (3, 13, 17)), seed=32)
    clean = synth.make_inputs(w, unused="zero")
    poisoned = synth.make_inputs(w, unused="nan")
    for key in ("k_pages", "v_pages"):
        for b in range(3):
            L = int(poisoned["context_lens"][b])
            last = int(poisoned["block_table"][b, (L - 1) // 8])
            poisoned[key][last, (L - 1) % 8 + 1:] = float("nan")
    out_c, lse_c = run(clean)
    out_p, lse_p = run(poisoned)
    assert bool(torch.isfinite(out_p).all())
    assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)


def test_shared_pages_equal_duplicated_pages():
    w = small(B=2, Hq=4, Hkv=1, D=16, P=4, lens=("fixed", (10, 10)), seed=33)
    inp = synth.make_inputs(w)
    inp["q"][1] = inp["q"][0]
    shared = dict(inp)
    shared["block_table"] = inp["block_table"].clone()
    shared["block_table"][1] = inp["block_table"][0]        # both rows name the same pages
    dup = dict(inp)
    for key in ("k_pages", "v_pages"):                       # copy row 0's pages into row 1's
        t = inp[key].clone()
        for j in range(3):
            t[int(inp["block_table"][1, j])] = t[int(inp["block_table"][0, j])]
        dup[key] = t
    out_s, lse_s = run(shared)
    out_d, lse_d = run(dup)
    assert torch.equal(out_s[0], out_s[1])
    assert torch.equal(out_s, out_d) and torch.equal(lse_s, lse_d)


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = small(B=3, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 1, 40), seed=34)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    mha = dict(inp)
    for key in ("k_pages", "v_pages"):
        mha[key] = inp[key].repeat_interleave(4, dim=2).contiguous()
    out2, lse2 = run(mha)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_heads_of_a_group_with_equal_q_agree():
    w = small(B=2, Hq=8, Hkv=2, D=16, P=4, lens=("uniform", 1, 40), seed=35)
    inp = synth.make_inputs(w)
    inp["q"][:, 1] = inp["q"][:, 0]
    inp["q"][:, 5] = inp["q"][:, 4]
    out, _ = run(inp)
    assert torch.equal(out[:, 0], out[:, 1]) and torch.equal(out[:, 4], out[:, 5])
    assert not torch.equal(out[:, 0], out[:, 4])


def _merge(parts):
    """Test-only fp64 merge of per-split (out_s, lse_s), in the normalised form
    of the FlashQuant wiki "CUDA Kernels", split_k_reduce.cu Algorithm:
    weights l_s * 2^(m_s - m_final), combined and divided by their sum."""
    lses = torch.stack([p[1] for p in parts])
    outs = torch.stack([p[0] for p in parts])
    m = lses.max(dim=0).values
    wts = torch.where(torch.isneginf(lses), torch.zeros_like(lses), torch.exp(lses - m))
    tot = wts.sum(0)
    return (wts[..., None] * outs).sum(0) / tot[..., None], m + torch.log(tot)


@pytest.mark.parametrize("split_pages", [1, 2, 3, 5, 100])
def test_split_merge_equals_unsplit(split_pages):
    w = small(B=3, Hq=8, Hkv=2, D=16, P=4, lens=("fixed", (4, 37, 61)), seed=36)
    inp = synth.make_inputs(w)
    out, lse = run(inp)
    P = 4
    for b in range(3):
        L = int(inp["context_lens"][b])
        parts = []
        start = 0
        while start < L:
            stop = min(L, start + split_pages * P)
            sub = dict(inp)
            sub["q"] = inp["q"][b:b + 1]
            sub["block_table"] = inp["block_table"][b:b + 1, start // P:].contiguous()
            sub["context_lens"] = torch.tensor([stop - start], dtype=torch.int32)
            o, l = run(sub)
            parts.append((o[0], l[0]))
            start = stop
        parts.append((torch.zeros_like(parts[0][0]), torch.full_like(parts[0][1], -math.inf)))
        mo, ml = _merge(parts)
        assert close(mo, out[b]) and close(ml, lse[b])


def test_thread_count_does_not_change_bits():
    w = small(B=5, Hq=8, Hkv=2, D=32, P=8, lens=("uniform", 1, 90), seed=37)
    inp = synth.make_inputs(w)
    a = run(inp, threads=1)
    b = run(inp, threads=7)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_rejects_out_of_range_block_table_and_lengths():
    w = small(B=2, Hq=4, Hkv=2, D=8, P=4, lens=("fixed", (5, 9)), seed=38)
    inp = synth.make_inputs(w)
    bad = dict(inp)
    bad["block_table"] = inp["block_table"].clone()
    bad["block_table"][1, 0] = inp["k_pages"].shape[0]
    with pytest.raises(oracle.OracleError):
        run(bad)
    bad = dict(inp)
    bad["context_lens"] = torch.tensor([5, 9 + 4 * 99], dtype=torch.int32)
    with pytest.raises(oracle.OracleError):
        run(bad)


# -- fp8 --------------------------------------------------------------------------

def test_e4m3fn_decoder_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        mine = oracle.e4m3fn_to_float64(c)
        r = float(ref[c])
        if math.isnan(r):
            assert math.isnan(mine), c
        else:
            assert mine == r, (c, mine, r)
    assert oracle.e4m3fn_to_float64(0x7E) == 448.0 and oracle.e4m3fn_to_float64(0x01) == 2.0 ** -9


def test_fp8_quantizer_properties():
    x = torch.randn((64, 4, 2, 128), generator=torch.Generator().manual_seed(3))
    codes, scale = synth.quantize_rows_e4m3(x)
    deq = codes.to(torch.float64) * scale.to(torch.float64)[..., None]
    amax_idx = x.abs().argmax(dim=-1, keepdim=True)
    top = codes.to(torch.float32).gather(-1, amax_idx).abs()
    assert bool((top == 448.0).all())
    y = x.to(torch.float64) / scale.to(torch.float64)[..., None]
    normal = y.abs() >= 2.0 ** -6
    rel = ((x.to(torch.float64) - deq).abs() / x.to(torch.float64).abs())[normal]
    assert float(rel.max()) <= 2.0 ** -4


# -- the pins reject plausible mistakes -------------------------------------------

SOURCE = os.path.join(os.path.dirname(oracle.__file__), "ref_decode.c")

MUTANTS = {
    "gqa_uses_h_mod_hkv": ("const int64_t kvh = h / group;", "const int64_t kvh = h % p->num_kv_heads;"),
    "slot_off_by_one": ("int64_t slot = t % p->page_size;\n        int64_t page = job->block_table[b * p->max_pages_per_seq + logical];",
                        "int64_t slot = (t + 1) % p->page_size;\n        int64_t page = job->block_table[b * p->max_pages_per_seq + logical];"),
    "scale_dropped": ("scores[t] = p->scale * dot;", "scores[t] = dot;"),
    "exp_sign_flipped": ("scores[t] = exp(scores[t] - M);", "scores[t] = exp(M - scores[t]);"),
    "max_is_min": ("if (scores[t] > M) M = scores[t];", "if (scores[t] < M) M = scores[t];"),
    "lse_drops_max": ("= M + log(Z);", "= log(Z);"),
    "lse_base2": ("= M + log(Z);", "= M + log2(Z);"),
    "k_and_v_swapped": ("kv_element(p, job->k, job->k_scale,", "kv_element(p, job->v, job->v_scale,"),
    "first_v_row_dropped": ("    for (t = 0; t < L; ++t) {\n        int64_t page",
                            "    for (t = 1; t < L; ++t) {\n        int64_t page"),
    "weights_dropped": ("orow[d] += scores[t] * kv_element(", "orow[d] += kv_element("),
    "normalised_by_length": ("orow[d] /= Z;", "orow[d] /= (double)L;"),
    "q_row_of_kv_head": ("job->q + (b * p->num_q_heads + h) * D;", "job->q + (b * p->num_q_heads + kvh) * D;"),
    "bf16_wrong_shift": ("((uint32_t)bits) << 16;", "((uint32_t)bits) << 15;"),
    "fp8_scale_dropped": ("[idx]) * (double)scales[row];", "[idx]);"),
    "e4m3_bias_8": ("e - 10);", "e - 11);"),
    "e4m3_subnormal_as_normal": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)(8 + m), -10);"),
    "empty_lse_zero": ("= -INFINITY;", "= 0.0;"),
}


def _pin_battery(lib):
    """Quick pins run against one oracle build; returns the names that fail."""
    failed = []

    def check(name, fn):
        try:
            ok = fn()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    for i, w in enumerate(CASES):
        def brute_ok(w=w):
            inp = synth.make_inputs(w)
            o, l = run(inp, library=lib)
            ro, rl = brute.numpy_decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                        inp["context_lens"], k_scale=inp["k_scale"],
                                        v_scale=inp["v_scale"])
            return close(o, ro) and close(l, rl)
        check(f"brute[{i}]", brute_ok)

    def golden_ok():
        g, inp = _golden()
        o, l = run(inp, scale=1.0, library=lib)
        e = math.e
        z0 = 1 + e + e * e
        return close(o[0, 0], [(1 + e * e) / z0, (e + e * e) / z0], 1e-14) and \
            close(l[0, 0], math.log(z0), 1e-14)
    check("golden", golden_ok)

    def dominant_ok():
        w = small(B=1, Hq=2, Hkv=1, D=4, P=4, lens=("fixed", (9,)), seed=27)
        inp = synth.make_inputs(w)
        inp["q"] = _bf16([[[1, 0, 0, 0], [1, 0, 0, 0]]])
        k = torch.zeros(inp["k_pages"].shape)
        bt = inp["block_table"][0]
        k[int(bt[1]), 1, 0, 0] = 1024.0
        inp["k_pages"] = k.to(torch.bfloat16)
        o, _ = run(inp, scale=1.0, library=lib)
        return torch.equal(o[0, 0], inp["v_pages"][int(bt[1]), 1, 0].to(torch.float64))
    check("dominant", dominant_ok)

    def decoder_ok():
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
        for c in range(256):
            m = oracle.e4m3fn_to_float64(c, library=lib)
            r = float(ref[c])
            if not ((math.isnan(r) and math.isnan(m)) or m == r):
                return False
        return True
    check("e4m3_decoder", decoder_ok)
    return failed


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def test_pins_pass_on_the_oracle_and_reject_every_mutant(tmp_path):
    with open(SOURCE) as f:
        src = f.read()
    base = _build_variant(tmp_path, "unmutated", src)
    assert _pin_battery(base) == []
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, f"mutation {name} no longer matches the oracle source"
        lib = _build_variant(tmp_path, name, src.replace(old, new, 1))
        if not _pin_battery(lib):
            survivors.append(name)
    assert survivors == [], f"mutants not caught by any pin: {survivors}"
