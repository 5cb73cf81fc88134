"""Pins of the TQ4 oracle (oracle/tq4.py) against facts outside it.

* the codebook: Max's published 16-level Gaussian quantiser (golden table),
  and the two Lloyd conditions checked by numerical integration;
* the codec: a hand-derived worked example (golden), including a tie on a
  boundary and a non-symmetric rotation that a transposed rotation fails;
* the attention: equal to a dense model-space reference (oracle.brute)
  over the rows the cache stands for, so the rotation, the nibble order and
  the sequential layout must all agree with each other;
* the distortion of compress + decompress on random vectors: the Lloyd-Max
  error of the Gaussian;
* planted mistakes (a dropped permutation, swapped nibbles, a transposed
  rotation) fail these pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy import integrate, stats

import synth
from oracle import brute
from oracle import tq4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_codebook_matches_max_table():
    g = _golden("lloyd_max_16_gaussian.json")
    c, b = tq4.lloyd_max_gaussian(16, 1.0)
    tol = g["printed_precision"]
    assert np.allclose(c[8:], g["outputs_positive"], atol=tol, rtol=0)
    assert np.allclose(-c[:8][::-1], g["outputs_positive"], atol=tol, rtol=0)
    assert np.allclose(b[7:], g["thresholds_positive"], atol=tol, rtol=0)
    edges = np.concatenate([[-np.inf], b, [np.inf]])
    mse = sum(integrate.quad(lambda x, ci=ci: (x - ci) ** 2 * stats.norm.pdf(x), lo, hi)[0]
              for ci, lo, hi in zip(c, edges[:-1], edges[1:]))
    assert abs(mse - g["mean_squared_error"]) <= 1e-5


def test_codebook_lloyd_conditions():
    """Each boundary is the midpoint of its centroids; each centroid is the
    Gaussian mean of its cell (by quadrature, not the closed form the
    iteration uses)."""
    c, b = tq4.lloyd_max_gaussian(16, 1.0)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(b, 0.5 * (c[1:] + c[:-1]), atol=1e-15, rtol=0)
    edges = np.concatenate([[-np.inf], b, [np.inf]])
    for ci, lo, hi in zip(c, edges[:-1], edges[1:]):
        mass = integrate.quad(stats.norm.pdf, lo, hi)[0]
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), lo, hi)[0] / mass
        assert abs(mean - ci) <= 1e-8


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebook_scales_with_head_dim(d):
    c, b = tq4.codebook(d)
    c1, b1 = tq4.lloyd_max_gaussian(16, 1.0)
    assert c.dtype == np.float32 and b.shape == (15,)
    assert np.allclose(c, c1 / math.sqrt(d), rtol=1e-6, atol=0)
    assert np.allclose(b[b != 0], (b1 / math.sqrt(d))[b != 0], rtol=1e-6, atol=0)


def _example_tables():
    b = np.array([(k - 8) / 8 for k in range(1, 16)])
    c = np.array([(i - 7.5) / 8 for i in range(16)])
    return c, b


@pytest.mark.parametrize("case", [0, 1])
def test_compress_decompress_worked_example(case):
    g = _golden("tq4_worked_example.json")
    cs = g["cases"][case]
    c, b = _example_tables()
    R = np.array(cs["rotation"], dtype=np.float64)
    packed, norm, y = tq4.compress(np.array(g["x"]), R, b, return_rotated=True)
    assert np.allclose(y, cs["rotated"], atol=1e-9)
    assert tq4.codes_of(packed).tolist() == cs["codes"]
    assert packed.tolist() == cs["packed"]
    assert float(norm) == cs["norm"]
    seq = tq4.decompress_seq(packed, norm, c)
    assert seq.tolist() == cs["decompressed_sequential"]
    assert np.allclose(seq @ tq4.seq_rotation(R), cs["reconstructed_model"], atol=1e-12)


def test_pack_rows_layout():
    kp = np.arange(8, dtype=np.uint8).reshape(1, 8)
    vp = (np.arange(8, dtype=np.uint8) + 100).reshape(1, 8)
    rows = tq4.pack_rows(kp, np.array([1.5], np.float32), vp, np.array([-2.0], np.float32))
    assert rows.shape == (1, 24)
    assert rows[0, :8].tolist() == list(range(8))
    assert rows[0, 8:12].tolist() == list(np.float32(1.5).tobytes())
    assert rows[0, 12:20].tolist() == list(range(100, 108))
    assert rows[0, 20:24].tolist() == list(np.float32(-2.0).tobytes())
    back = tq4.unpack_rows(rows)
    assert np.array_equal(back[0], kp) and float(back[1][0]) == 1.5
    assert np.array_equal(back[2], vp) and float(back[3][0]) == -2.0


def _small_case(seed, B=3, Hq=8, Hkv=2, D=64, P=8, lens=(1, 29, 70)):
    w = synth.WORKLOADS["tiny"].with_(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                                      lens=("fixed", tuple(lens)), seed=seed)
    inp = synth.make_tq4_inputs(w)
    ck, bk = tq4.codebook(D)
    cv, bv = ck * 1.25, bk * 1.25   # separate K and V tables
    cache = tq4.append(inp["cache"].numpy(), inp["k_new"], inp["v_new"], inp["token_seq"], inp["token_pos"],
                       inp["block_table"], inp["rotation"], bk, bv)
    return inp, cache, ck, cv


def _check_against_dense(inp, cache, ck, cv):
    out, lse = tq4.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    # the dense reference needs finite rows everywhere it gathers; unused
    # pool rows (0xFF: NaN norms) are never gathered
    K, V = tq4.reconstruct_model(cache, inp["rotation"], ck, cv)
    ref_o, ref_l = brute.numpy_decode(inp["q"], K, V, inp["block_table"], inp["context_lens"])
    return float((out - ref_o).abs().max()), float((lse - ref_l).abs().max())


def test_decode_equals_dense_model_space_attention():
    inp, cache, ck, cv = _small_case(seed=7100)
    do, dl = _check_against_dense(inp, cache, ck, cv)
    assert do <= 1e-9 and dl <= 1e-9


def test_decode_empty_sequence():
    inp, cache, ck, cv = _small_case(seed=7101, lens=(0, 5, 17))
    out, lse = tq4.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(out[1:]).all()


def test_append_places_each_token():
    inp, cache, ck, cv = _small_case(seed=7102)
    P = inp["cache"].shape[2]
    bt = inp["block_table"].numpy()
    for t in (0, 5, 40, int(inp["token_seq"].shape[0]) - 1):
        s, pos = int(inp["token_seq"][t]), int(inp["token_pos"][t])
        page = bt[s, pos // P]
        kp, kn, vp, vn = tq4.unpack_rows(cache[page, :, pos % P])
        ekp, ekn = tq4.compress(inp["k_new"][t], inp["rotation"], tq4.codebook(64)[1])
        assert np.array_equal(kp, ekp) and np.array_equal(kn, ekn)
    # rows no token reaches keep their bytes
    used = np.zeros(cache.shape[:1] + cache.shape[2:3], bool)
    for s, pos in zip(inp["token_seq"].tolist(), inp["token_pos"].tolist()):
        used[bt[s, pos // P], pos % P] = True
    assert np.all(cache.transpose(0, 2, 1, 3)[~used] == 0xFF)


def test_distortion_is_the_lloyd_max_error():
    """Mean squared error of a unit vector after compress + decompress, in
    model space: for 16 levels the Gaussian Lloyd-Max error per unit variance
    is 0.0095, and a rotated unit vector's d coordinates carry variance 1/d
    each, so the total is about 0.0095 (the coordinates are only nearly
    Gaussian: 10 % slack)."""
    D = 128
    g = torch.Generator().manual_seed(7103)
    x = torch.randn((4000, D), generator=g, dtype=torch.float64)
    R = synth.random_rotation(D, 7104)
    c, b = tq4.codebook(D)
    packed, norm = tq4.compress(x, R, b)
    rec = tq4.decompress_seq(packed, np.ones_like(norm), c) @ tq4.seq_rotation(R)
    xh = x.numpy() / np.linalg.norm(x.numpy(), axis=-1, keepdims=True)
    err = float(np.mean(np.sum((rec - xh) ** 2, axis=-1)))
    assert 0.0086 <= err <= 0.0105, err


# ---- planted mistakes: each must fail a pin above --------------------------

def _natural_rows(cache, k_centroids, v_centroids):
    """Decompressed rows in the rotation's natural order, straight from the
    per-element codes (element i = centroid(code i) * norm, compress.cu's
    packing: byte j holds codes 2j and 2j + 1): (K, V) float64
    [num_pages, P, Hkv, d]."""
    rows = np.asarray(cache, np.uint8)
    kpk, kn, vpk, vn = tq4.unpack_rows(rows)
    K = np.asarray(k_centroids, np.float64)[tq4.codes_of(kpk)] * np.asarray(kn, np.float64)[..., None]
    V = np.asarray(v_centroids, np.float64)[tq4.codes_of(vpk)] * np.asarray(vn, np.float64)[..., None]
    return (torch.from_numpy(np.ascontiguousarray(K.transpose(0, 2, 1, 3))),
            torch.from_numpy(np.ascontiguousarray(V.transpose(0, 2, 1, 3))))


def test_decode_rotated_equals_dense_rotated_space_attention():
    """fused_tq_attention.cu, Input/Output: q pre-rotated, output in the
    rotated space; against dense attention over rows rebuilt from the codes
    alone (no sequential layout, no rotation matrix)."""
    inp, cache, ck, cv = _small_case(seed=7106, lens=(0, 29, 70))
    g = torch.Generator().manual_seed(7106)
    q_rot = torch.randn(inp["q"].shape, generator=g, dtype=torch.float64) * 0.7
    out, lse = tq4.decode_rotated(q_rot, cache, inp["block_table"], inp["context_lens"], ck, cv)
    K, V = _natural_rows(cache, ck, cv)
    ref_o, ref_l = brute.numpy_decode(q_rot, K, V, inp["block_table"], inp["context_lens"])
    assert float((out - ref_o).abs().max()) <= 1e-9
    fin = torch.isfinite(ref_l)
    assert torch.equal(fin, torch.isfinite(lse)) and float((lse[fin] - ref_l[fin]).abs().max()) <= 1e-9
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_rotated_is_the_model_space_decode_rotated():
    """R orthogonal: attention on q_rot = R q gives R times the model-space
    output, and the same lse, up to the float32 rotation's own distance from
    orthogonality (R R^T - I, ~1e-7 here)."""
    inp, cache, ck, cv = _small_case(seed=7107)
    R = tq4._f64(inp["rotation"])
    defect = float(np.abs(R @ R.T - np.eye(R.shape[0])).max())
    tol = 4 * R.shape[0] * defect * 4.0 + 1e-12
    out_m, lse_m = tq4.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    q_rot = torch.from_numpy(tq4._f64(inp["q"]) @ R.T)
    out_r, lse_r = tq4.decode_rotated(q_rot, cache, inp["block_table"], inp["context_lens"], ck, cv)
    assert defect < 1e-6
    assert float((out_r - torch.from_numpy(out_m.numpy() @ R.T)).abs().max()) <= tol
    assert float((lse_r - lse_m).abs().max()) <= tol


def test_planted_mistakes_are_caught(monkeypatch):
    inp, cache, ck, cv = _small_case(seed=7105)
    orig_seq, orig_dec = tq4.seq_rotation, tq4.decompress_seq

    # 1. the sequential layout's permutation dropped in the attention only
    monkeypatch.setattr(tq4, "seq_rotation", lambda R: tq4._f64(R))
    out, _ = tq4.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    monkeypatch.setattr(tq4, "seq_rotation", orig_seq)
    ref, _ = tq4.decode(inp["q"], cache, inp["block_table"], inp["context_lens"], inp["rotation"], ck, cv)
    assert float((out - ref).abs().max()) > 1e-2

    # 2. nibbles swapped in the decompressor: the worked example fails
    def swapped(packed, norm, centroids):
        p = np.asarray(packed, np.uint8)
        return orig_dec(((p & 15) << 4) | (p >> 4), norm, centroids)
    monkeypatch.setattr(tq4, "decompress_seq", swapped)
    with pytest.raises(AssertionError):
        test_compress_decompress_worked_example(0)
    monkeypatch.setattr(tq4, "decompress_seq", orig_dec)

    # 3. the rotation applied transposed in compress: the permutation case fails
    orig_comp = tq4.compress
    monkeypatch.setattr(tq4, "compress", lambda x, R, b, **kw: orig_comp(x, np.asarray(R).T, b, **kw))
    with pytest.raises(AssertionError):
        test_compress_decompress_worked_example(1)

    # 4. nibbles swapped in the decompressor: the rotated-space decode no
    #    longer matches its dense pin (rows rebuilt from the codes alone)
    monkeypatch.setattr(tq4, "decompress_seq", swapped)
    with pytest.raises(AssertionError):
        test_decode_rotated_equals_dense_rotated_space_attention()
    monkeypatch.setattr(tq4, "decompress_seq", orig_dec)

    # 5. the sequential rotation's row order dropped: the model-space and
    #    rotated-space decodes disagree
    monkeypatch.setattr(tq4, "seq_rotation", lambda R: tq4._f64(R))
    with pytest.raises(AssertionError):
        test_decode_rotated_is_the_model_space_decode_rotated()
    monkeypatch.setattr(tq4, "seq_rotation", orig_seq)
