"""TEST INFRASTRUCTURE ONLY: fp64 oracle of the TQ4 compressed KV cache and of
paged decode attention over it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; it shares no code with the HIP library.

The codec follows the FlashQuant wiki pages ("CUDA Kernels": compress.cu,
decompress.cu, fused_tq_attention.cu, paged_decode.cu KV Cache Byte Layout):

* compress (compress.cu, What It Replaces and Algorithm): norm = ||x||_2,
  x_hat = x / (norm + 1e-10), y = x_hat R^T (R the d x d rotation),
  code_i = number of the 15 sorted boundaries b with b <= y_i (the kernel's
  predicated count; codes 0..15), and byte j of the packed row holds
  code_{2j} in its high nibble and code_{2j+1} in its low nibble.
* decompress (decompress.cu, Sequential Layout): byte j expands to element j
  (high nibble) and element d/2 + j (low nibble) of the output row, each the
  centroid of its code times the norm. The row is therefore the rotated
  vector with its coordinates permuted: element j approximates y_{2j} and
  element d/2 + j approximates y_{2j+1}. ``seq_rotation`` is R with its rows
  in that order, so a decompressed row approximates seq_rotation(R) x.
* attention (fused_tq_attention.cu, Input/Output and Decode Path): q is
  taken into the same rotated space, attention runs there on the
  decompressed rows, and the output is rotated back; since seq_rotation(R)
  is orthogonal, this equals attention in model space over the
  reconstructed rows seq_rotation(R)^T k_seq (which ``tests`` check with the
  dense reference in ``oracle.brute``).
* cache rows (paged_decode.cu, KV Cache Byte Layout): per token and kv head,
  [K codes (d/2 bytes) | K norm (fp32) | V codes (d/2 bytes) | V norm
  (fp32)], d + 8 bytes; pages hold them head-major, [page][kv head][slot].
* codebook (FlashQuant wiki index, Algorithm Deep Dive: Lloyd-Max via
  erfinv): the pages name the method, not its target distribution. Reading
  taken: a coordinate of a rotated unit vector in R^d is treated as
  N(0, 1/d), and the 16-level Lloyd-Max quantiser of that Gaussian is found
  by Lloyd's iteration from quantile (erfinv) starting points.
"""
import math

import numpy as np
import torch
from scipy import special, stats

LEVELS = 16
NORM_EPS = 1e-10


# ---- codebook -------------------------------------------------------------

def lloyd_max_gaussian(levels=LEVELS, sigma=1.0, tol=1e-13, max_iter=100000):
    """Lloyd-Max quantiser of N(0, sigma^2): (centroids [levels], boundaries
    [levels - 1]) in fp64. Start: the centroids at the quantiles
    Phi^-1((i + 1/2) / levels), through erfinv. Step: each boundary is the
    midpoint of its two centroids; each centroid is the mean of the Gaussian
    restricted to its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)) in
    standard units. Stops when no centroid moves by more than tol."""
    u = (np.arange(levels) + 0.5) / levels
    c = math.sqrt(2.0) * special.erfinv(2.0 * u - 1.0)
    for _ in range(max_iter):
        b = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate([[-np.inf], b, [np.inf]])
        mass = stats.norm.cdf(edges[1:]) - stats.norm.cdf(edges[:-1])
        new = (stats.norm.pdf(edges[:-1]) - stats.norm.pdf(edges[1:])) / mass
        done = np.max(np.abs(new - c)) <= tol
        c = new
        if done:
            break
    b = 0.5 * (c[1:] + c[:-1])
    return c * sigma, b * sigma


def codebook(head_dim):
    """The TQ4 tables for head_dim: (centroids [16], boundaries [15]) as
    float32 (the kernels' table type), for coordinates ~ N(0, 1/head_dim)."""
    c, b = lloyd_max_gaussian(LEVELS, 1.0 / math.sqrt(head_dim))
    return c.astype(np.float32), b.astype(np.float32)


# ---- codec ----------------------------------------------------------------

def _f64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def compress(x, rotation, boundaries, return_rotated=False):
    """x [..., d] -> (packed uint8 [..., d/2], norm float32 [...]); with
    return_rotated also y [..., d] (fp64, the values the codes decide on)."""
    x = _f64(x)
    R = _f64(rotation)
    bnd = _f64(boundaries)
    d = x.shape[-1]
    if d % 2 or R.shape != (d, d) or bnd.shape != (LEVELS - 1,):
        raise ValueError("shape mismatch")
    norm = np.sqrt(np.sum(x * x, axis=-1))
    xh = x / (norm[..., None] + NORM_EPS)
    y = xh @ R.T
    codes = np.searchsorted(bnd, y, side="right")          # #{b : b <= y}
    codes = np.clip(codes, 0, LEVELS - 1).astype(np.uint8)
    packed = (codes[..., 0::2] << 4) | codes[..., 1::2]
    res = (packed.astype(np.uint8), norm.astype(np.float32))
    return res + (y,) if return_rotated else res


def codes_of(packed):
    """Per-element codes in the compressed (rotated) order: [..., d]."""
    p = np.asarray(packed, dtype=np.uint8)
    c = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    c[..., 0::2] = p >> 4
    c[..., 1::2] = p & 15
    return c


def decompress_seq(packed, norm, centroids):
    """Sequential layout: [..., d] fp64 with element j = c[hi(byte j)] * norm
    and element d/2 + j = c[lo(byte j)] * norm."""
    p = np.asarray(packed, dtype=np.uint8)
    c = _f64(centroids)
    n = _f64(norm)[..., None]
    return np.concatenate([c[p >> 4] * n, c[p & 15] * n], axis=-1)


def seq_rotation(rotation):
    """Rows of R in the sequential layout's order: row j = R[2j], row d/2 + j
    = R[2j + 1]."""
    R = _f64(rotation)
    return np.concatenate([R[0::2], R[1::2]], axis=0)


# ---- paged cache ----------------------------------------------------------

def pack_rows(k_packed, k_norm, v_packed, v_norm):
    """Cache rows [..., d + 8] uint8: K codes | K norm | V codes | V norm."""
    kn = np.ascontiguousarray(np.asarray(k_norm, dtype=np.float32))[..., None].view(np.uint8)
    vn = np.ascontiguousarray(np.asarray(v_norm, dtype=np.float32))[..., None].view(np.uint8)
    return np.concatenate([np.asarray(k_packed, np.uint8), kn, np.asarray(v_packed, np.uint8), vn], axis=-1)


def unpack_rows(rows):
    """Inverse of pack_rows: (k_packed, k_norm, v_packed, v_norm)."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    h = (r.shape[-1] - 8) // 2
    kn = np.ascontiguousarray(r[..., h:h + 4]).view(np.float32)[..., 0]
    vn = np.ascontiguousarray(r[..., 2 * h + 4:]).view(np.float32)[..., 0]
    return r[..., :h], kn, r[..., h + 4:2 * h + 4], vn


def append(cache, k_new, v_new, token_seq, token_pos, block_table, rotation, k_boundaries, v_boundaries):
    """Compress each new token's K and V rows (per kv head) and write them at
    (page = block_table[seq, pos // P], slot = pos % P) of the head-major
    cache [num_pages, Hkv, P, d + 8]; returns the new cache (a copy).
    Tokens whose sequence, position or page falls outside the tables are
    skipped."""
    c = np.array(cache, dtype=np.uint8, copy=True)
    num_pages, Hkv, P, _ = c.shape
    kp, kn = compress(k_new, rotation, k_boundaries)
    vp, vn = compress(v_new, rotation, v_boundaries)
    rows = pack_rows(kp, kn, vp, vn)                            # [T, Hkv, d + 8]
    bt = np.asarray(block_table)
    for t, (s, pos) in enumerate(zip(np.asarray(token_seq).tolist(), np.asarray(token_pos).tolist())):
        if not (0 <= s < bt.shape[0]) or pos < 0 or pos // P >= bt.shape[1]:
            continue
        page = int(bt[s, pos // P])
        if not (0 <= page < num_pages):
            continue
        c[page, :, pos % P, :] = rows[t]
    return c


def _attend_seq(q_seq, cache, block_table, context_lens, k_centroids, v_centroids, scale):
    """Attention in the sequential rotated space (fused_tq_attention.cu,
    Decode Path; paged_decode.cu): q_seq [B, Hq, d] fp64 against the
    decompressed rows of every valid position. Returns (o_seq, lse) fp64
    arrays; an empty sequence gives o = 0, lse = -inf."""
    rows = np.asarray(cache.detach().cpu().numpy() if isinstance(cache, torch.Tensor) else cache, np.uint8)
    bt = np.asarray(block_table.detach().cpu().numpy() if isinstance(block_table, torch.Tensor) else block_table)
    lens = np.asarray(context_lens.detach().cpu().numpy() if isinstance(context_lens, torch.Tensor) else context_lens)
    B, Hq, d = q_seq.shape
    num_pages, Hkv, P, rb = rows.shape
    if rb != d + 8 or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o_seq = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        pages = bt[b, pos // P]
        if np.any(pages < 0) or np.any(pages >= num_pages):
            raise ValueError("block_table entry outside the pool")
        for h in range(Hkv):
            r = rows[pages, h, pos % P]                         # [L, d + 8]
            kpk, kn, vpk, vn = unpack_rows(r)
            K = decompress_seq(kpk, kn, k_centroids)
            V = decompress_seq(vpk, vn, v_centroids)
            for g in range(G):
                hq = h * G + g
                s = sc * (K @ q_seq[b, hq])
                m = s.max()
                w = np.exp(s - m)
                o_seq[b, hq] = (w[:, None] * V).sum(0) / w.sum()
                lse[b, hq] = m + math.log(w.sum())
    return o_seq, lse


def decode(q, cache, block_table, context_lens, rotation, k_centroids, v_centroids, *, scale=None,
           return_rotated=False):
    """Decode attention over a TQ4 cache, fp64.

    q: [B, Hq, d] (bf16 or float; model space). cache: uint8 [num_pages,
    Hkv, P, d + 8]. Returns (out [B, Hq, d], lse [B, Hq]) in model space as
    float64 tensors (lse = -inf and out = 0 for an empty sequence); with
    return_rotated also the output in the sequential rotated space."""
    qd = _f64(q)
    Rs = seq_rotation(rotation)
    q_seq = qd @ Rs.T                                           # [B, Hq, d]
    o_seq, lse = _attend_seq(q_seq, cache, block_table, context_lens, k_centroids, v_centroids, scale)
    out = o_seq @ Rs                                            # R_seq^T o_seq, row-wise
    res = (torch.from_numpy(out), torch.from_numpy(lse))
    return res + (torch.from_numpy(o_seq),) if return_rotated else res


def decode_rotated(q_rot, cache, block_table, context_lens, k_centroids, v_centroids, *, scale=None):
    """The fused attention's own boundary (fused_tq_attention.cu,
    Input/Output): the queries arrive already rotated, q_rot = R q in the
    rotation's natural coordinate order ([B, Hq, d], any float type), and
    the output stays in that space (the caller rotates it back). Element i
    of a decompressed row in natural order is centroid(code i) * norm, code
    i being nibble i of the row's codes (codes_of), so the sequential
    layout is only a reordering: q_seq = (q_rot[0::2], q_rot[1::2]) and
    out[2j] = o_seq[j], out[2j + 1] = o_seq[d/2 + j]. Returns (out [B, Hq,
    d], lse [B, Hq]) float64 tensors, out = 0 and lse = -inf for an empty
    sequence."""
    qr = _f64(q_rot)
    q_seq = np.concatenate([qr[..., 0::2], qr[..., 1::2]], axis=-1)
    o_seq, lse = _attend_seq(q_seq, cache, block_table, context_lens, k_centroids, v_centroids, scale)
    h = qr.shape[-1] // 2
    out = np.empty_like(o_seq)
    out[..., 0::2] = o_seq[..., :h]
    out[..., 1::2] = o_seq[..., h:]
    return torch.from_numpy(out), torch.from_numpy(lse)


def reconstruct_model(cache, rotation, k_centroids, v_centroids):
    """The rows a TQ4 cache stands for, in model space: (K, V) float64
    [num_pages, P, Hkv, d] (token-major, the dense references' order)."""
    rows = np.asarray(cache, np.uint8)
    Rs = seq_rotation(rotation)
    kpk, kn, vpk, vn = unpack_rows(rows)
    K = decompress_seq(kpk, kn, k_centroids) @ Rs
    V = decompress_seq(vpk, vn, v_centroids) @ Rs
    return (torch.from_numpy(np.ascontiguousarray(K.transpose(0, 2, 1, 3))),
            torch.from_numpy(np.ascontiguousarray(V.transpose(0, 2, 1, 3))))
