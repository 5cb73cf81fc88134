"""TEST INFRASTRUCTURE ONLY: CPU oracle of ragged paged prefill attention,
fp64, and of the query-tile map that schedules it.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may use this
module; it shares no code with the HIP library.

The operation (AstrAI "CUDA Kernels": the paged prefill entry, ragged batch
described by qo_indptr and the cache's own lengths, section "Q Scheduling and
KV Addressing"; attention as in the decode oracle): request b owns the packed
query rows qo_indptr[b] .. qo_indptr[b+1] - 1, n_b of them, and a paged
context of L_b positions that already holds the keys and values of those
rows. The pages leave open where the n_b new rows sit inside the context; the
reading taken here is that they are its last n_b positions (the same reading
as the multi-query decode, and the one that makes a prompt prefilled in
chunks give the rows a whole-prompt prefill gives). Query row i of request b
(0 <= i < n_b) then attends, when causal, to the positions t < L_b - n_b +
i + 1 (itself and everything before it); without the causal mask, to all
t < L_b. A row that sees no position gets out = 0 and lse = -inf.

Written out directly: every query row is one single-token decode (the C
oracle's definition) of its request's pages with its own visible length.
"""
import numpy as np
import torch

from . import decode


def tile_map(qo_indptr, rows_per_tile):
    """The O(1) tile -> request map of the paged prefill (AstrAI "CUDA
    Kernels", Q Scheduling and KV Addressing, the worked example with Q
    lengths 70, 10 and 130): the Q tiles of rows_per_tile rows each, request
    by request, and for each tile its request and its index inside that
    request. Returns (tile_batch, tile_index) as int lists."""
    ptr = [int(x) for x in qo_indptr]
    tile_batch, tile_index = [], []
    for b in range(len(ptr) - 1):
        n = ptr[b + 1] - ptr[b]
        if n < 0:
            raise ValueError("qo_indptr must be non-decreasing")
        for j in range((n + rows_per_tile - 1) // rows_per_tile):
            tile_batch.append(b)
            tile_index.append(j)
    return tile_batch, tile_index


def visible_lengths(qo_indptr, context_lens, causal=True):
    """Per packed query row: its request and the number of context positions
    it attends to (clamped to [0, L_b])."""
    ptr = np.asarray([int(x) for x in qo_indptr], dtype=np.int64)
    lens = np.asarray([int(x) for x in context_lens], dtype=np.int64)
    rows_b, rows_lim = [], []
    for b in range(len(ptr) - 1):
        n = int(ptr[b + 1] - ptr[b])
        L = int(lens[b])
        for i in range(n):
            lim = L - n + i + 1 if causal else L
            rows_b.append(b)
            rows_lim.append(min(max(lim, 0), L))
    return np.asarray(rows_b, dtype=np.int64), np.asarray(rows_lim, dtype=np.int64)


def prefill(q, qo_indptr, k_pages, v_pages, block_table, context_lens, *, causal=True, scale=None, k_scale=None,
            v_scale=None):
    """q: bf16 [total_q, Hq, d] packed by qo_indptr (int [B + 1]); pools,
    block_table [B, max_pages] and context_lens [B] as for ``oracle.decode``
    (NHD pools). Returns (out float64 [total_q, Hq, d], lse float64
    [total_q, Hq])."""
    rows_b, rows_lim = visible_lengths(qo_indptr, context_lens, causal)
    total = int(qo_indptr[-1]) - int(qo_indptr[0])
    if len(rows_b) != total or q.shape[0] < int(qo_indptr[-1]):
        raise ValueError("q rows do not match qo_indptr")
    Hq, D = q.shape[1], q.shape[2]
    if total == 0:
        return (torch.zeros((0, Hq, D), dtype=torch.float64), torch.zeros((0, Hq), dtype=torch.float64))
    q_rows = q[int(qo_indptr[0]):int(qo_indptr[-1])].contiguous()
    bt = torch.as_tensor(block_table).to(torch.int32)[torch.from_numpy(rows_b)].contiguous()
    lens = torch.from_numpy(rows_lim.astype(np.int32))
    return decode(q_rows, k_pages, v_pages, bt, lens, scale=scale, k_scale=k_scale, v_scale=v_scale)
