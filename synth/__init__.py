"""Seeded synthetic decode-step inputs shared by the tests, the smoke check and
the benchmark.

This module only draws inputs. It holds none of the attention arithmetic: no
score, softmax, merge or dequantisation. The fp8 workload's quantiser lives
here because its codes and scales are inputs that both the GPU path and the
oracle consume unchanged.

Recipe (every decode workload; the append inputs have their own recipe in
``make_append_inputs``):
  * ``g = torch.Generator().manual_seed(seed)`` on the CPU.
  * context lengths: fixed, or ``torch.randint(lo, hi + 1)`` (inclusive).
  * pages needed by sequence b: ceil(L_b / P); pool = 2 x total needed pages
    (the tiny workload: exactly the needed pages).
  * ``perm = torch.randperm(pool)``; block_table rows take consecutive entries
    of ``perm`` in batch order; unused entries are -1.
  * q, then the K rows of every needed page, then the V rows: ``randn`` in
    fp32, rounded to bf16 (round to nearest even).
  * pages that no block_table row names are filled with NaN (bf16) or the
    NaN code 0x7F (fp8, with NaN scales), so that any read of them shows up.
  * fp8 workload: each (token, kv head) row of K and of V gets
    scale = absmax(row) / 448 (fp32; 1 for an all-zero row) and
    code = e4m3fn(round-to-nearest-even(x / scale)) clamped to +-448.
  * TQ4 workloads (``make_tq4_inputs``): the same lengths, block table and
    q; the K and V rows of every valid position are handed over as new
    tokens for a TQ4 append (the codec itself is not here); the cache starts
    as 0xFF bytes (NaN norms); the rotation is a Haar-random orthogonal
    matrix (``random_rotation``).
"""
from dataclasses import dataclass
import math

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "kv_bytes", "make_append_inputs", "append_bytes", "to_hnd",
           "make_prefill_inputs", "prefill_flops", "PREFILL_WORKLOADS", "prefill_workload", "to_inline", "from_inline",
           "from_hnd", "random_rotation", "make_tq4_inputs", "tq4_kv_bytes"]

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    lens: tuple            # ("fixed", (L0, L1, ...)) or ("uniform", lo, hi)
    kv_dtype: str = "bf16"  # "bf16" or "fp8_e4m3"
    pool: str = "2x"        # "2x" or "exact"
    seed: int = 1000

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload(
        "tiny", "paged GQA decode B1, 8 q / 2 kv heads, d64, L256, P16, 16-page pool",
        1, 8, 2, 64, 16, ("fixed", (256,)), pool="exact", seed=1001),
    "llama3_8b": Workload(
        "llama3_8b", "Llama-3-8B-shaped paged GQA decode B32, 32 q / 8 kv heads, d128, "
        "L~U[512,4096], P16", 32, 32, 8, 128, 16, ("uniform", 512, 4096), seed=1002),
    "long_ctx": Workload(
        "long_ctx", "long-context paged GQA decode B4, 64 q / 8 kv heads, d128, "
        "L in {32K,64K,96K,128K}, P64", 4, 64, 8, 128, 64,
        ("fixed", (32768, 65536, 98304, 131072)), seed=1003),
    "many_short": Workload(
        "many_short", "many-short-sequence paged GQA decode B256, 32 q / 8 kv heads, d128, "
        "L~U[16,512], P16", 256, 32, 8, 128, 16, ("uniform", 16, 512), seed=1004),
    "fp8_kv": Workload(
        "fp8_kv", "FP8-e4m3 KV paged GQA decode B32, 32 q / 8 kv heads, d128, "
        "L~U[1024,8192], P16, per-token fp32 scales", 32, 32, 8, 128, 16,
        ("uniform", 1024, 8192), kv_dtype="fp8_e4m3", seed=1005),
}


def _lens(w: Workload, g: torch.Generator) -> torch.Tensor:
    kind = w.lens[0]
    if kind == "fixed":
        vals = tuple(w.lens[1])
        if len(vals) != w.batch:
            raise ValueError("fixed lens must give one length per sequence")
        return torch.tensor(vals, dtype=torch.int32)
    if kind == "uniform":
        lo, hi = int(w.lens[1]), int(w.lens[2])
        return torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int64).to(torch.int32)
    raise ValueError(f"unknown lens kind {kind!r}")


def quantize_rows_e4m3(x: torch.Tensor):
    """Per-row (last axis) absmax fp8 quantiser for the fp8 workload's inputs.

    Returns (codes float8_e4m3fn, scale float32 with the last axis dropped)."""
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), scale


def make_inputs(w, *, seed=None, unused="nan"):
    """Draw one decode step's inputs on the CPU.

    Returns a dict: q [B,Hq,d] bf16; k_pages, v_pages [num_pages,P,Hkv,d]
    (bf16 or float8_e4m3fn); k_scale, v_scale [num_pages,P,Hkv] fp32 or None;
    block_table [B,max_pages] int32 (-1 where unused); context_lens [B] int32;
    workload; scale (1/sqrt(d)).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    g = torch.Generator().manual_seed(int(seed))
    B, Hq, Hkv, D, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    lens = _lens(w, g)
    needed = [(int(L) + P - 1) // P for L in lens.tolist()]
    total_needed = sum(needed)
    pool = total_needed if w.pool == "exact" else 2 * total_needed
    pool = max(pool, 1)
    max_pages = max(max(needed) if needed else 0, 1)
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    used_pages = perm[:total_needed].to(torch.int64)
    off = 0
    for b, n in enumerate(needed):
        block_table[b, :n] = perm[off:off + n]
        off += n
    q = torch.randn((B, Hq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k_rows = torch.randn((total_needed, P, Hkv, D), generator=g, dtype=torch.float32)
    v_rows = torch.randn((total_needed, P, Hkv, D), generator=g, dtype=torch.float32)
    k_scale = v_scale = None
    if w.kv_dtype == "bf16":
        fill = float("nan") if unused == "nan" else 0.0
        k_pages = torch.full((pool, P, Hkv, D), fill, dtype=torch.bfloat16)
        v_pages = torch.full((pool, P, Hkv, D), fill, dtype=torch.bfloat16)
        k_pages[used_pages] = k_rows.to(torch.bfloat16)
        v_pages[used_pages] = v_rows.to(torch.bfloat16)
    elif w.kv_dtype == "fp8_e4m3":
        kc, ks = quantize_rows_e4m3(k_rows)
        vc, vs = quantize_rows_e4m3(v_rows)
        code_fill = 0x7F if unused == "nan" else 0x00
        k_pages = torch.full((pool, P, Hkv, D), code_fill, dtype=torch.uint8).view(torch.float8_e4m3fn)
        v_pages = torch.full((pool, P, Hkv, D), code_fill, dtype=torch.uint8).view(torch.float8_e4m3fn)
        sfill = float("nan") if unused == "nan" else 1.0
        k_scale = torch.full((pool, P, Hkv), sfill, dtype=torch.float32)
        v_scale = torch.full((pool, P, Hkv), sfill, dtype=torch.float32)
        k_pages.view(torch.uint8)[used_pages] = kc.view(torch.uint8)
        v_pages.view(torch.uint8)[used_pages] = vc.view(torch.uint8)
        k_scale[used_pages] = ks
        v_scale[used_pages] = vs
    else:
        raise ValueError(f"unknown kv dtype {w.kv_dtype!r}")
    return dict(q=q, k_pages=k_pages, v_pages=v_pages, k_scale=k_scale, v_scale=v_scale,
                block_table=block_table, context_lens=lens, workload=w,
                scale=1.0 / math.sqrt(D))


def kv_bytes(w, context_lens) -> int:
    """Algorithmic KV bytes of one decode step: every K and V element of every
    valid (token, kv head) once, plus the two fp32 scales per (token, kv head)
    for an fp8 pool."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    tokens = int(torch.as_tensor(context_lens).to(torch.int64).sum())
    esize = 2 if w.kv_dtype == "bf16" else 1
    per = 2 * w.head_dim * esize + (8 if w.kv_dtype == "fp8_e4m3" else 0)
    return tokens * w.num_kv_heads * per


def make_append_inputs(*, batch, num_kv_heads, head_dim, page_size, new_tokens, context, kv_dtype="bf16",
                       num_q_heads=None, invalid=True, special_rows=True, spread=24, shuffle=True, seed=2000):
    """Draw the inputs of one KV append on the CPU.

    Recipe: ``g = torch.Generator().manual_seed(seed)``; existing context
    lengths L_b ~ U[context] (inclusive); new tokens n_b = new_tokens (an int)
    or ~ U[new_tokens] (inclusive); sequence b needs ceil((L_b + n_b) / P)
    pages, the pool holds 2x the total, block_table rows take consecutive
    entries of a random permutation of the pool and keep one extra column of
    -1. Every pool row holds randn data rounded to bf16 (fp8 pools: quantised
    per row like the fp8 decode workload), so a stray write shows. The new
    rows are randn * 2^u, u ~ U{-spread..spread} per (token, kv head, K or
    V) (spread 0: plain N(0,1) rows, as in the decode workloads);
    with ``special_rows`` about 1/16 of them are all zero, 1/16 a single
    spike, 1/16 scaled by 2^-128 (bf16 subnormals) and 1/16 hold values that
    sit exactly on e4m3 rounding ties. New token i of sequence b sits at
    position L_b + i. With ``invalid`` five tokens that do not resolve are
    added (sequence -1 and B, position -1 and max_pages * P, a position on a
    -1 block-table entry); with ``shuffle`` the token order is a random
    permutation, else sequence by sequence in position order (a prefill
    chunk as a serving engine hands it over).

    Returns a dict: k_new, v_new bf16 [N,Hkv,d]; token_seq, token_pos int32
    [N]; block_table int32 [B,max_pages]; k_pages, v_pages (bf16 or
    float8_e4m3fn) [num_pages,P,Hkv,d]; k_scale, v_scale fp32 or None;
    context_lens (before) and new_lens (after) int32 [B]; q bf16 [B,Hq,d]
    when num_q_heads is given.
    """
    g = torch.Generator().manual_seed(int(seed))
    B, Hkv, D, P = batch, num_kv_heads, head_dim, page_size
    lo, hi = context
    lens = torch.randint(int(lo), int(hi) + 1, (B,), generator=g, dtype=torch.int64)
    if isinstance(new_tokens, int):
        n_new = torch.full((B,), new_tokens, dtype=torch.int64)
    else:
        n_new = torch.randint(int(new_tokens[0]), int(new_tokens[1]) + 1, (B,), generator=g, dtype=torch.int64)
    total = lens + n_new
    needed = [(int(t) + P - 1) // P for t in total.tolist()]
    pool = max(2 * sum(needed), 1)
    max_pages = max(needed) + 1
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(needed):
        block_table[b, :n] = perm[off:off + n]
        off += n
    rows = torch.randn((pool, P, Hkv, D), generator=g, dtype=torch.float32)
    vrows = torch.randn((pool, P, Hkv, D), generator=g, dtype=torch.float32)
    k_scale = v_scale = None
    if kv_dtype == "bf16":
        k_pages, v_pages = rows.to(torch.bfloat16), vrows.to(torch.bfloat16)
    elif kv_dtype == "fp8_e4m3":
        k_pages, k_scale = quantize_rows_e4m3(rows)
        v_pages, v_scale = quantize_rows_e4m3(vrows)
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")

    N = int(n_new.sum())
    seq = torch.repeat_interleave(torch.arange(B, dtype=torch.int64), n_new)
    starts = torch.cumsum(n_new, 0) - n_new
    pos = lens[seq] + (torch.arange(N, dtype=torch.int64) - starts[seq])

    def new_rows():
        x = torch.randn((N, Hkv, D), generator=g, dtype=torch.float32)
        x = x * torch.exp2(torch.randint(-spread, spread + 1, (N, Hkv, 1), generator=g).to(torch.float32))
        if special_rows and N > 0:
            kind = torch.randint(0, 16, (N, Hkv), generator=g)
            x[kind == 0] = 0.0
            spike = torch.zeros((N, Hkv, D))
            spike[..., 0] = 3.0
            x = torch.where((kind == 1)[..., None], spike, x)
            x = torch.where((kind == 2)[..., None], x * 2.0 ** -128, x)
            # multiples of 2^-4 in a row whose absmax is 14 = 448 * 2^-5: the
            # scale is 2^-5 (plain or power of two), x / scale an even
            # integer, many of them halfway between two e4m3 values
            ties = torch.randint(-224, 225, (N, Hkv, D), generator=g).to(torch.float32) * 2.0 ** -4
            ties[..., 0] = 14.0
            x = torch.where((kind == 3)[..., None], ties, x)
        return x.to(torch.bfloat16)

    k_new, v_new = new_rows(), new_rows()
    if invalid:
        bad_seq = torch.tensor([-1, B, 0, 0, B - 1], dtype=torch.int64)
        bad_pos = torch.tensor([0, 0, -1, max_pages * P, (max_pages - 1) * P], dtype=torch.int64)
        seq = torch.cat([seq, bad_seq])
        pos = torch.cat([pos, bad_pos])
        extra = torch.randn((5, Hkv, D), generator=g).to(torch.bfloat16)
        k_new = torch.cat([k_new, extra])
        v_new = torch.cat([v_new, extra])
    order = torch.randperm(seq.numel(), generator=g) if shuffle else torch.arange(seq.numel())
    out = dict(k_new=k_new[order].contiguous(), v_new=v_new[order].contiguous(),
               token_seq=seq[order].to(torch.int32), token_pos=pos[order].to(torch.int32),
               block_table=block_table, k_pages=k_pages, v_pages=v_pages, k_scale=k_scale, v_scale=v_scale,
               context_lens=lens.to(torch.int32), new_lens=total.to(torch.int32))
    if num_q_heads is not None:
        out["q"] = torch.randn((B, num_q_heads, D), generator=g).to(torch.bfloat16)
    return out


def append_bytes(num_rows, head_dim, kv_dtype) -> int:
    """Algorithmic bytes of an append of num_rows (token, kv head) rows: the
    bf16 K and V rows read once, the K and V rows written once in the pool's
    element size, plus two fp32 scales per row for an fp8 pool."""
    write = 2 * head_dim * (2 if kv_dtype == "bf16" else 1) + (8 if kv_dtype == "fp8_e4m3" else 0)
    return num_rows * (4 * head_dim + write)


def to_hnd(inp):
    """A copy of an input dict whose pools (and fp8 scales) are re-laid from
    rows [page][slot][kv head] to rows [page][kv head][slot]: the same
    values, another order in memory."""
    out = dict(inp)
    for k in ("k_pages", "v_pages"):
        out[k] = inp[k].permute(0, 2, 1, 3).contiguous()
    for k in ("k_scale", "v_scale"):
        if inp.get(k) is not None:
            out[k] = inp[k].permute(0, 2, 1).contiguous()
    return out


def from_hnd(t):
    """A pool [page][kv head][slot][d] (or scales [page][kv head][slot]) back
    in rows [page][slot][kv head]."""
    return t.permute(0, 2, 1, 3) if t.dim() == 4 else t.permute(0, 2, 1)


def make_prefill_inputs(*, num_q_heads, num_kv_heads, head_dim, page_size, q_lens, prefix_lens=None,
                        kv_dtype="bf16", pool="2x", unused="nan", seed=3000):
    """Draw the inputs of one ragged paged prefill on the CPU.

    Recipe: request b has q_lens[b] new query rows and prefix_lens[b]
    (default 0) cached positions before them; its context is L_b = prefix_b
    + n_b positions, the new rows' keys and values already in the cache. The
    pools, block_table and K/V values follow ``make_inputs`` with those
    fixed lengths and the same seed (unused pages NaN); q is then drawn from
    ``torch.Generator().manual_seed(seed + 1)`` as randn rounded to bf16,
    packed [total_q, Hq, d] request by request, and qo_indptr is the prefix
    sum of q_lens (AstrAI "CUDA Kernels", Q Scheduling and KV Addressing).

    Returns the ``make_inputs`` dict with q replaced by the packed rows and
    qo_indptr int32 [B + 1], q_lens int32 [B] added.
    """
    q_lens = [int(x) for x in q_lens]
    B = len(q_lens)
    prefix_lens = [0] * B if prefix_lens is None else [int(x) for x in prefix_lens]
    if len(prefix_lens) != B or min(q_lens + prefix_lens, default=0) < 0:
        raise ValueError("one non-negative q length and prefix length per request")
    lens = tuple(p + n for p, n in zip(prefix_lens, q_lens))
    w = Workload("prefill", "ragged paged prefill", B, num_q_heads, num_kv_heads, head_dim, page_size,
                 ("fixed", lens), kv_dtype=kv_dtype, pool=pool, seed=seed)
    inp = make_inputs(w, unused=unused)
    g = torch.Generator().manual_seed(int(seed) + 1)
    total = sum(q_lens)
    inp["q"] = torch.randn((total, num_q_heads, head_dim), generator=g, dtype=torch.float32).to(torch.bfloat16)
    ptr = [0]
    for n in q_lens:
        ptr.append(ptr[-1] + n)
    inp["qo_indptr"] = torch.tensor(ptr, dtype=torch.int32)
    inp["q_lens"] = torch.tensor(q_lens, dtype=torch.int32)
    return inp


def prefill_flops(q_lens, context_lens, num_q_heads, head_dim, causal=True) -> int:
    """Algorithmic flops of a prefill: 4 d per (query row, head, visible
    position) (2 d for q.k, 2 d for p.v), with row i of a request of n rows
    and context L seeing L - n + i + 1 positions when causal (clamped to
    [0, L]), L otherwise."""
    pairs = 0
    for n, L in zip([int(x) for x in q_lens], [int(x) for x in context_lens]):
        for i in range(n):
            lim = L - n + i + 1 if causal else L
            pairs += min(max(lim, 0), L)
    return 4 * head_dim * num_q_heads * pairs


# Prefill workloads: name -> (description, heads/dims, q length recipe,
# prefix recipe, seed). Lengths are drawn with torch.randint (inclusive) from
# torch.Generator().manual_seed(seed + 2).
PREFILL_WORKLOADS = {
    "llama3_8b_prefill": ("Llama-3-8B-shaped ragged paged prefill: 8 prompts, q lengths ~U[512, 2048], no cached "
                          "prefix, 32 q / 8 kv heads, d128, P16, bf16, causal",
                          dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16), 8, (512, 2048), (0, 0),
                          3900),
    "llama3_8b_prefill_2048": ("one Llama-3-8B-shaped prompt, q = kv = 2048, 32 q / 8 kv heads, d128, P16, bf16, "
                               "causal", dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16), 1,
                               (2048, 2048), (0, 0), 3901),
    "llama3_8b_chunked_prefill": ("Llama-3-8B-shaped chunked prefill: 16 requests, 512-row chunks after cached "
                                  "prefixes ~U[0, 4096], 32 q / 8 kv heads, d128, P16, bf16, causal",
                                  dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16), 16, (512, 512),
                                  (0, 4096), 3902),
}


def prefill_workload(name, **overrides):
    """Draw the named prefill workload's inputs (``make_prefill_inputs``)."""
    desc, dims, batch, qr, pr, seed = PREFILL_WORKLOADS[name]
    g = torch.Generator().manual_seed(seed + 2)
    q_lens = torch.randint(qr[0], qr[1] + 1, (batch,), generator=g).tolist()
    prefix = torch.randint(pr[0], pr[1] + 1, (batch,), generator=g).tolist()
    kw = dict(dims, q_lens=q_lens, prefix_lens=prefix, seed=seed)
    kw.update(overrides)
    inp = make_prefill_inputs(**kw)
    inp["description"] = desc
    return inp


def to_inline(inp):
    """A copy of an fp8 input dict whose pools carry each row's fp32 scale
    after its codes (uint8 rows of d + 4 bytes, the scale's 4 bytes in
    memory order), and no separate scale arrays: the same values laid out
    as one byte cache. Works on either row order (NHD or HND)."""
    out = dict(inp)
    for pages, scale in (("k_pages", "k_scale"), ("v_pages", "v_scale")):
        codes = inp[pages].view(torch.uint8)
        sb = inp[scale].contiguous().view(torch.uint8).reshape(tuple(inp[scale].shape) + (4,))
        out[pages] = torch.cat([codes, sb], dim=-1).contiguous()
        out[scale] = None
    return out


def from_inline(pages):
    """(codes float8_e4m3fn [..., d], scales float32 [...]) of an inline
    pool (uint8 [..., d + 4])."""
    d = pages.shape[-1] - 4
    codes = pages[..., :d].contiguous().view(torch.float8_e4m3fn)
    scales = pages[..., d:].contiguous().view(torch.float32).reshape(pages.shape[:-1])
    return codes, scales


def random_rotation(d, seed):
    """A Haar-distributed random orthogonal d x d matrix (float32): the Q of
    the QR factorisation of a seeded standard Gaussian matrix, each column
    multiplied by the sign of R's diagonal entry. The TQ4 codec draws its
    rotation once; here the draw is an input."""
    g = torch.Generator().manual_seed(int(seed))
    a = torch.randn((d, d), generator=g, dtype=torch.float64)
    qm, r = torch.linalg.qr(a)
    qm = qm * torch.sign(torch.diagonal(r))[None, :]
    return qm.to(torch.float32).contiguous()


def make_tq4_inputs(w, *, seed=None):
    """Inputs of a TQ4 decode step on the CPU, for a workload of WORKLOADS
    (its kv_dtype is ignored): q bf16 [B,Hq,d]; k_new, v_new bf16
    [T,Hkv,d] (every valid position of every sequence, sequence by
    sequence; T = sum of the lengths), token_seq, token_pos int32 [T];
    block_table int32 [B,max_pages]; context_lens int32 [B]; cache uint8
    [num_pages,Hkv,P,d + 8] of 0xFF; rotation float32 [d,d]; scale."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    # the same generator start as make_inputs: the same lengths, block table
    # and q as the workload's bf16 / fp8 step
    g = torch.Generator().manual_seed(int(seed))
    B, Hq, Hkv, D, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    lens = _lens(w, g)
    needed = [(int(L) + P - 1) // P for L in lens.tolist()]
    total_needed = sum(needed)
    pool = max(total_needed if w.pool == "exact" else 2 * total_needed, 1)
    max_pages = max(max(needed) if needed else 0, 1)
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(needed):
        block_table[b, :n] = perm[off:off + n]
        off += n
    q = torch.randn((B, Hq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    T = int(lens.to(torch.int64).sum())
    k_new = torch.randn((T, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v_new = torch.randn((T, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    n = lens.to(torch.int64)
    token_seq = torch.repeat_interleave(torch.arange(B, dtype=torch.int64), n)
    starts = torch.cumsum(n, 0) - n
    token_pos = torch.arange(T, dtype=torch.int64) - starts[token_seq]
    cache = torch.full((pool, Hkv, P, D + 8), 0xFF, dtype=torch.uint8)
    return dict(q=q, k_new=k_new, v_new=v_new, token_seq=token_seq.to(torch.int32),
                token_pos=token_pos.to(torch.int32), block_table=block_table, context_lens=lens, cache=cache,
                rotation=random_rotation(D, int(seed) + 78), workload=w, scale=1.0 / math.sqrt(D))


def tq4_kv_bytes(w, context_lens) -> int:
    """Algorithmic bytes of a TQ4 decode step: the d + 8 cache bytes of every
    valid (token, kv head) once."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    tokens = int(torch.as_tensor(context_lens).to(torch.int64).sum())
    return tokens * w.num_kv_heads * (w.head_dim + 8)
