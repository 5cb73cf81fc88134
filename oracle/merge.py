"""TEST INFRASTRUCTURE ONLY: CPU oracle of the merge of exported partial
attention states (normalised output and natural-log log-sum-exp), fp64.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may use this
module; it shares no code with the HIP library.

The operation (FlashQuant wiki "CUDA Kernels", split_k_reduce.cu Algorithm and
Numerical Stability: the global maximum over the pieces, weights rescaled by
the exponential of each piece's maximum minus it, the weighted combination
divided by the summed weights, a guard for a zero sum), written for pieces
that export what a decode exports: for piece s of row r, the normalised
output o_s = sum_t p_t v_t / sum_t p_t and lse_s = ln sum_t exp(score_t).
Then, with M = max_s lse_s and w_s = exp(lse_s - M):

    out = sum_s w_s o_s / sum_s w_s,      lse = M + ln sum_s w_s

which is attention over the union of the pieces' keys. Readings where the
pages are silent: a piece with lse = -inf is empty and weighs nothing; a row
whose pieces are all empty gets out = 0 and lse = -inf (the decode's
convention for an empty sequence); a NaN or +inf lse in any piece makes the
row's out and lse NaN.
"""
import numpy as np


def merge_states(partial_out, partial_lse):
    """partial_out [S, R, d], partial_lse [S, R] (any float dtype) ->
    (out [R, d], lse [R]) in fp64."""
    po = np.asarray(partial_out, np.float64)
    pl = np.asarray(partial_lse, np.float64)
    S, R, d = po.shape
    out = np.zeros((R, d), np.float64)
    lse = np.full(R, -np.inf)
    for r in range(R):
        ls = pl[:, r]
        if np.isnan(ls).any() or np.isposinf(ls).any():
            out[r] = np.nan
            lse[r] = np.nan
            continue
        if np.isneginf(ls).all():
            continue
        m = ls.max()
        w = np.exp(ls - m)
        total = w.sum()
        out[r] = (w[:, None] * po[:, r, :]).sum(axis=0) / total
        lse[r] = m + np.log(total)
    return out, lse
