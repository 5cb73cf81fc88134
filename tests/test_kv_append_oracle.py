"""Pins of the KV-append oracle (oracle/kv_append.py) against things other
than itself: torch's own float -> float8_e4m3fn rounding (round to nearest
even), the C oracle's decoding of every code, the independent quantiser of
the synthetic fp8 workload, the format's closed-form facts (the row maximum
lands on +-448; a power-of-two scale is the smallest that fits) and the
e4m3 rounding-error bound."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import kv_append as ka


def _torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_value_table_matches_the_c_oracle_for_every_code():
    for c in range(256):
        mine = ka.decode_e4m3fn(np.array([c], np.uint8))[0]
        ref = oracle.e4m3fn_to_float64(c)
        assert (math.isnan(mine) and math.isnan(ref)) or mine == ref, c


def test_encoder_matches_torch_on_codes_midpoints_and_random_values():
    finite = ka.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2  # ties: exact in fp32
    rng = np.random.default_rng(3)
    ys = np.concatenate([finite, -finite, mids, -mids,
                         rng.uniform(-448, 448, 20000),
                         rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),     # subnormal region
                         np.ldexp(rng.uniform(1, 2, 2000), rng.integers(-12, 9, 2000))]).astype(np.float32)
    ys = np.clip(ys, -448, 448)
    mine = ka.encode_e4m3fn(ys)
    ref = _torch_e4m3(ys)
    # -0.0 and +0.0 may differ only in the sign bit of a zero code
    same = (mine == ref) | ((mine & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all(), ys[~same][:10]


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = ka.decode_e4m3fn(codes).astype(np.float32)
    back = ka.encode_e4m3fn(vals)
    ok = (back == codes) | ((codes & 0x7F) == 0) & ((back & 0x7F) == 0)
    assert ok.all()


def _bf16_rows(n, d, seed, spread=0.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, d, generator=g)
    if spread:
        x = x * torch.exp2(torch.randint(-20, 21, (n, 1), generator=g).float())
    return x.to(torch.bfloat16).to(torch.float32).numpy()


def test_plain_quantiser_agrees_with_the_workload_quantiser():
    rows = _bf16_rows(400, 128, 5, spread=1.0)
    codes_ref, scale_ref = synth.quantize_rows_e4m3(torch.from_numpy(rows))
    for i, row in enumerate(rows):
        codes, s = ka.quantize_row(row, pow2=False)
        assert s == np.float32(scale_ref[i].item())
        assert np.array_equal(codes, codes_ref[i].view(torch.uint8).numpy()), i


@pytest.mark.parametrize("pow2", [False, True])
def test_row_maximum_and_error_bound(pow2):
    rows = _bf16_rows(300, 64, 6, spread=1.0)
    for row in rows:
        codes, s = ka.quantize_row(row, pow2)
        amax = float(np.max(np.abs(row)))
        deq = ka.decode_e4m3fn(codes) * float(s)
        if not pow2:
            # the largest magnitude encodes to +-448
            assert (codes[np.argmax(np.abs(row))] & 0x7F) == 0x7E
        else:
            e = math.log2(float(s))
            assert e == int(e)                                        # a power of two
            assert 448.0 * float(s) >= amax > 224.0 * float(s)        # the smallest that fits
        normal = np.abs(row) / float(s) >= 2.0 ** -6
        err = np.abs(deq - row)
        assert (err[normal] <= 2.0 ** -4 * np.abs(row[normal]) + 1e-30).all()
        # below the normal range the step is 2^-9 of the scale
        assert (err[~normal] <= 2.0 ** -10 * float(s) * (1 + 1e-12)).all()


def test_zero_row_gets_unit_scale():
    for pow2 in (False, True):
        codes, s = ka.quantize_row(np.zeros(64, np.float32), pow2)
        assert s == 1.0 and not codes.any()


def test_append_writes_slots_and_skips_unresolved_tokens():
    rng = np.random.default_rng(8)
    num_pages, P, Hkv, d = 6, 4, 2, 8
    bt = np.array([[3, 1, -1], [0, 5, 2]], np.int32)
    kp = rng.normal(size=(num_pages, P, Hkv, d)).astype(np.float32)
    vp = rng.normal(size=(num_pages, P, Hkv, d)).astype(np.float32)
    seq = np.array([0, 1, 1, 0, 2, -1, 1], np.int32)
    pos = np.array([5, 0, 11, 9, 0, 0, 12], np.int32)   # 9 -> page -1, seq 2 / -1 and pos 12 out of range
    kn = rng.normal(size=(len(seq), Hkv, d)).astype(np.float32)
    vn = rng.normal(size=(len(seq), Hkv, d)).astype(np.float32)
    k2, v2, _, _ = ka.kv_append(kp, vp, None, None, kn, vn, seq, pos, bt)
    expect_k = kp.copy()
    expect_k[1, 1] = kn[0]   # seq 0, pos 5: block 1 -> page 1, slot 1
    expect_k[0, 0] = kn[1]   # seq 1, pos 0: page 0, slot 0
    expect_k[2, 3] = kn[2]   # seq 1, pos 11: block 2 -> page 2, slot 3
    assert np.array_equal(k2, expect_k)
    assert np.array_equal(v2[2, 3], vn[2]) and np.array_equal(v2[3], vp[3])


def _ties_away(y):
    y = np.asarray(y, np.float32)
    a = np.abs(y).astype(np.float64)
    fin = ka.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    hi = np.clip(np.searchsorted(fin, a), 0, len(fin) - 1)
    lo = np.clip(hi - 1, 0, len(fin) - 1)
    pick = np.where(np.abs(a - fin[lo]) < np.abs(fin[hi] - a), lo, hi)
    return (pick | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip in the oracle fails one of the pins above."""
    # ties away from zero instead of to even
    monkeypatch.setattr(ka, "encode_e4m3fn", _ties_away)
    with pytest.raises(AssertionError):
        test_encoder_matches_torch_on_codes_midpoints_and_random_values()
    monkeypatch.undo()
    # a power-of-two scale one step too large
    orig = ka.row_scale
    monkeypatch.setattr(ka, "row_scale", lambda row, pow2: np.float32(orig(row, pow2) * (2 if pow2 else 1)))
    with pytest.raises(AssertionError):
        test_row_maximum_and_error_bound(True)
    monkeypatch.undo()
    # a plain scale over 447 instead of 448
    monkeypatch.setattr(ka, "row_scale",
                        lambda row, pow2: np.float32(np.float32(np.max(np.abs(row))) / np.float32(447.0)))
    with pytest.raises(AssertionError):
        test_plain_quantiser_agrees_with_the_workload_quantiser()
