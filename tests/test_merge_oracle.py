"""Pins of the partial-state merge oracle (oracle/merge.py) against things
other than itself: the C decode oracle over the union of disjoint key sets
(the defining property), closed forms and the empty / invalid conventions."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import merge as mg


def _split_decode(inp, cuts):
    """Decode each sequence's context in pieces [cuts[i], cuts[i+1]) of its
    pages with the C oracle (one block table per piece), stacked."""
    bt, lens = inp["block_table"], inp["context_lens"]
    P = inp["k_pages"].shape[1]
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        # piece = pages [a, b) of every sequence, shifted to the table's front
        sub = torch.full_like(bt, -1)
        piece = bt[:, a:b]
        sub[:, :piece.shape[1]] = piece
        sub_lens = (lens.to(torch.int64) - a * P).clamp(0, (b - a) * P).to(torch.int32)
        o, l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], sub, sub_lens)
        outs.append(o.numpy())
        lses.append(l.numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("cuts", [[0, 3, 100], [0, 1, 2, 5, 9, 100], [0, 100]])
def test_merge_of_disjoint_pieces_equals_decode_of_the_union(cuts):
    w = synth.WORKLOADS["tiny"].with_(batch=3, lens=("fixed", (256, 37, 5)), pool="2x", seed=77)
    inp = synth.make_inputs(w)
    po, pl = _split_decode(inp, cuts)
    B, Hq, d = inp["q"].shape
    out, lse = mg.merge_states(po.reshape(len(cuts) - 1, B * Hq, d), pl.reshape(len(cuts) - 1, B * Hq))
    ref_o, ref_l = oracle.decode(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                                 inp["context_lens"])
    assert np.abs(out - ref_o.numpy().reshape(B * Hq, d)).max() < 1e-12
    assert np.abs(lse - ref_l.numpy().reshape(B * Hq)).max() < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(1)
    o = rng.normal(size=(3, 4, 8))
    l = rng.normal(size=(3, 4)) * 5
    # one piece: identity
    out, lse = mg.merge_states(o[:1], l[:1])
    assert np.array_equal(out, o[0]) and np.allclose(lse, l[0], atol=0, rtol=0)
    # equal lse: the plain mean, lse + ln S
    eq = np.repeat(l[:1], 3, axis=0)
    out, lse = mg.merge_states(o, eq)
    assert np.allclose(out, o.mean(axis=0), atol=1e-15) and np.allclose(lse, l[0] + math.log(3), atol=1e-14)
    # two pieces: a sigmoid mix
    out, lse = mg.merge_states(o[:2], l[:2])
    a = 1.0 / (1.0 + np.exp(l[1] - l[0]))
    assert np.allclose(out, a[:, None] * o[0] + (1 - a[:, None]) * o[1], atol=1e-14)
    assert np.allclose(lse, np.logaddexp(l[0], l[1]), atol=1e-14)
    # large lse values: no overflow
    out, lse = mg.merge_states(o[:2], l[:2] + 5000.0)
    assert np.isfinite(out).all() and np.allclose(lse, np.logaddexp(l[0], l[1]) + 5000.0, atol=1e-9)


def test_empty_and_invalid_pieces():
    o = np.ones((2, 3, 4))
    l = np.array([[-np.inf, 1.0, -np.inf], [-np.inf, -np.inf, np.nan]])
    o[1, 0] = 7.0
    out, lse = mg.merge_states(o, l)
    assert np.array_equal(out[0], np.zeros(4)) and lse[0] == -np.inf      # all empty
    assert np.array_equal(out[1], o[0, 1]) and lse[1] == 1.0              # empty piece weighs nothing
    assert np.isnan(out[2]).all() and np.isnan(lse[2])                    # NaN poisons the row
    out, lse = mg.merge_states(o[:1], np.array([[np.inf, 0.0, 0.0]]))
    assert np.isnan(out[0]).all() and np.isnan(lse[0])


def test_planted_mistakes_are_caught(monkeypatch):
    """Plausible slips in the merge fail the pins above."""
    real_exp, real_log = np.exp, np.log

    # base-2 weights with a natural-log lse
    monkeypatch.setattr(mg.np, "exp", lambda x: np.power(2.0, x))
    with pytest.raises(AssertionError):
        test_closed_forms()
    monkeypatch.undo()
    # lse without the ln of the summed weights
    monkeypatch.setattr(mg.np, "log", lambda x: real_log(x) * 0)
    with pytest.raises(AssertionError):
        test_closed_forms()
    monkeypatch.undo()
    assert mg.np.exp is real_exp
