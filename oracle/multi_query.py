"""TEST INFRASTRUCTURE ONLY: CPU oracle of multi-query paged decode (several
query rows per sequence, as in speculative decoding), fp64.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may use this
module; it shares no code with the HIP library.

The operation (DeepGEMM documentation, section 6.1: the paged form takes q of
shape [batch, next_n, heads, d]; the next_n new tokens are the last next_n
positions of each sequence's context): query row i (0 <= i < n) of
sequence b attends to the positions t < L_b - (n - 1 - i), i.e. causally
up to and including its own position. Written out directly: n one-token
decodes (the C oracle's definition) with the lengths shifted per row. A row
that sees no position gets out = 0 and lse = -inf, as an empty sequence does.
"""
import torch

from . import decode


def decode_multi_query(q, k_pages, v_pages, block_table, context_lens, *, scale=None, k_scale=None,
                       v_scale=None):
    """q: bf16 [B, n, Hq, d]; the rest as for ``oracle.decode``.
    Returns (out float64 [B, n, Hq, d], lse float64 [B, n, Hq])."""
    B, n, Hq, D = q.shape
    lens = torch.as_tensor(context_lens).to(torch.int64)
    outs, lses = [], []
    for i in range(n):
        lens_i = (lens - (n - 1 - i)).clamp(min=0).to(torch.int32)
        o, l = decode(q[:, i].contiguous(), k_pages, v_pages, block_table, lens_i, scale=scale, k_scale=k_scale,
                      v_scale=v_scale)
        outs.append(o)
        lses.append(l)
    return torch.stack(outs, dim=1), torch.stack(lses, dim=1)
