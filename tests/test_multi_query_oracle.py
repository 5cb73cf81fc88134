"""Pins of the multi-query decode oracle (oracle/multi_query.py) against an
independent dense formulation: every sequence's K/V gathered into dense
arrays, one score matrix for all query rows with an explicit causal mask
matrix, softmax in numpy fp64."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import multi_query as mq


def _dense(q, inp):
    """q [B, n, Hq, d]; causal mask over the last n positions of each context."""
    kp = inp["k_pages"].to(torch.float64).numpy()
    vp = inp["v_pages"].to(torch.float64).numpy()
    bt, lens = inp["block_table"].numpy(), inp["context_lens"].numpy()
    B, n, Hq, D = q.shape
    P, Hkv = kp.shape[1], kp.shape[2]
    G = Hq // Hkv
    qd = q.to(torch.float64).numpy()
    out = np.zeros((B, n, Hq, D))
    lse = np.full((B, n, Hq), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        K = kp[bt[b][pos // P], pos % P]          # [L, Hkv, D]
        V = vp[bt[b][pos // P], pos % P]
        visible = pos[None, :] < (L - (n - 1 - np.arange(n)))[:, None]     # [n, L]
        for h in range(Hq):
            s = qd[b, :, h, :] @ K[:, h // G, :].T / math.sqrt(D)         # [n, L]
            s = np.where(visible, s, -np.inf)
            for i in range(n):
                if not visible[i].any():
                    continue
                m = s[i].max()
                w = np.exp(s[i] - m)
                out[b, i, h] = w @ V[:, h // G, :] / w.sum()
                lse[b, i, h] = m + math.log(w.sum())
    return out, lse


def _inputs(lens, n, seed, Hq=8, Hkv=2):
    w = synth.WORKLOADS["tiny"].with_(batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv,
                                      lens=("fixed", tuple(lens)), pool="2x", seed=seed)
    inp = synth.make_inputs(w, unused="zero")
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn((len(lens), n, Hq, inp["q"].shape[-1]), generator=g).to(torch.bfloat16)
    return q, inp


@pytest.mark.parametrize("lens,n", [((37, 16, 5, 0, 1), 4), ((64, 3), 8), ((200,), 2), ((9, 2), 1)])
def test_multi_query_oracle_matches_dense_causal_attention(lens, n):
    q, inp = _inputs(lens, n, seed=50 + n)
    out, lse = mq.decode_multi_query(q, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    ref_o, ref_l = _dense(q, inp)
    assert np.abs(out.numpy() - ref_o).max() < 1e-12
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(lse.numpy()), np.isneginf(ref_l))
    assert np.abs(lse.numpy()[fin] - ref_l[fin]).max() < 1e-12


def test_last_row_is_the_plain_decode_and_short_contexts_are_empty():
    q, inp = _inputs((40, 3, 0), 4, seed=61)
    out, lse = mq.decode_multi_query(q, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["context_lens"])
    o1, l1 = oracle.decode(q[:, 3].contiguous(), inp["k_pages"], inp["v_pages"], inp["block_table"],
                           inp["context_lens"])
    assert torch.equal(out[:, 3], o1) and torch.equal(lse[:, 3], l1)
    # L = 3 < n = 4: row 0 sees nothing, row 1 sees one position
    assert torch.isneginf(lse[1, 0]).all() and (out[1, 0] == 0).all()
    assert torch.isfinite(lse[1, 1]).all()


def test_planted_off_by_one_is_caught(monkeypatch):
    """Row i seeing one position too few (its own) fails the dense pin."""
    real = mq.decode

    def shifted(q, kp, vp, bt, lens, **kw):
        return real(q, kp, vp, bt, (lens.to(torch.int64) - 1).clamp(min=0).to(torch.int32), **kw)
    monkeypatch.setattr(mq, "decode", shifted)
    with pytest.raises(AssertionError):
        test_multi_query_oracle_matches_dense_causal_attention((37, 16, 5, 0, 1), 4)
