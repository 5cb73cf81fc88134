"""TEST INFRASTRUCTURE ONLY: two independent dense references for small inputs.

Both gather each sequence's K/V rows into a dense array first and then apply a
dense attention formula; neither shares code with ``ref_decode.c``. They pin
the C oracle on inputs small enough for dense numpy / torch work.

* ``numpy_decode``: a numpy fp64 softmax over the gathered rows.
* ``sdpa_decode``: torch's ``scaled_dot_product_attention`` in float64 on the
  CPU, with each kv head repeated for the query heads that share it
  (FlashQuant wiki "CUDA Kernels", GQA Support: consecutive query heads share
  one kv head).

fp8 pools are dequantised here with torch's own float8_e4m3fn conversion
(a library routine, not the oracle's decoder) times the per-(token, kv head)
fp32 scale.
"""
import math

import numpy as np
import torch


def _dequant(pages, scale):
    x = pages.detach().cpu().to(torch.float64)
    if scale is not None:
        x = x * scale.detach().cpu().to(torch.float64)[..., None]
    return x


def gather_dense(pages, scale, block_table, L, b):
    """Rows 0..L-1 of sequence b, shape [L, Hkv, d], float64."""
    num_pages, P, Hkv, D = pages.shape
    x = _dequant(pages, scale)
    pos = torch.arange(L)
    page = block_table[b].to(torch.int64)[pos // P]
    slot = pos % P
    return x[page, slot]


def numpy_decode(q, k_pages, v_pages, block_table, context_lens, *, scale=None,
                 k_scale=None, v_scale=None):
    B, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    qd = q.detach().cpu().to(torch.float64).numpy()
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            lse[b, :] = -np.inf
            continue
        K = gather_dense(k_pages, k_scale, block_table, L, b).numpy()
        V = gather_dense(v_pages, v_scale, block_table, L, b).numpy()
        for h in range(Hq):
            kvh = h // G
            s = sc * (K[:, kvh, :] @ qd[b, h])
            m = s.max()
            w = np.exp(s - m)
            out[b, h] = (w[:, None] * V[:, kvh, :]).sum(0) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return torch.from_numpy(out), torch.from_numpy(lse)


def sdpa_decode(q, k_pages, v_pages, block_table, context_lens, *, scale=None,
                k_scale=None, v_scale=None):
    """torch SDPA (float64, CPU) over GQA-expanded dense K/V; returns out only."""
    B, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_dense(k_pages, k_scale, block_table, L, b)      # [L, Hkv, D]
        V = gather_dense(v_pages, v_scale, block_table, L, b)
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()  # [Hq, L, D]
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        qq = q[b].detach().cpu().to(torch.float64)[:, None, :]          # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, K, V, scale=sc)
        out[b] = o[:, 0, :]
    return out
