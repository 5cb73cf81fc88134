"""Host logic of the prefill boundary, on the CPU: the tile map that
pdattn_prefill_tiles builds (against the pages' worked example and the
oracle's tile map), its longest-first order, the rows-per-tile query and the
argument checks. No device call is made."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import prefill as pf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_tile_map.json")


def _pk():
    import paged_kv_split_amd as pk
    return pk


def test_tile_map_matches_pages_worked_example():
    pk = _pk()
    g = json.load(open(GOLDEN))
    tb, ti = pk.prefill_tiles(g["qo_indptr"], g["rows_per_tile"], longest_first=False)
    assert tb.tolist() == g["q_tile_to_batch"] and ti.tolist() == g["q_tile_to_index"]


@pytest.mark.parametrize("causal", [True, False])
def test_longest_first_is_a_sorted_permutation(causal):
    pk = _pk()
    rng = np.random.default_rng(5)
    for _ in range(30):
        B = int(rng.integers(1, 12))
        n = rng.integers(0, 300, B)
        L = n + rng.integers(0, 500, B)
        if rng.random() < 0.3:
            L = np.minimum(L, rng.integers(0, 300, B))   # contexts shorter than their rows
        ptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        rt = int(rng.choice([4, 8, 32, 42, 64, 128]))
        tb, ti = pk.prefill_tiles(ptr, rt, context_lens_host=L.astype(np.int32), causal=causal)
        ref_b, ref_i = pf.tile_map(ptr, rt)
        assert sorted(zip(tb.tolist(), ti.tolist())) == sorted(zip(ref_b, ref_i))
        reach = []
        for b, j in zip(tb.tolist(), ti.tolist()):
            last = min((j + 1) * rt, int(n[b])) - 1
            r = int(L[b]) - int(n[b]) + last + 1 if causal else int(L[b])
            reach.append(min(max(r, 0), int(L[b])))
        assert all(x >= y for x, y in zip(reach, reach[1:]))
        # equal reaches keep the request-by-request order
        pos = {t: k for k, t in enumerate(zip(ref_b, ref_i))}
        order = [pos[t] for t in zip(tb.tolist(), ti.tolist())]
        for k in range(len(order) - 1):
            if reach[k] == reach[k + 1]:
                assert order[k] < order[k + 1]


def test_rows_per_tile():
    pk = _pk()
    for D, cols in ((64, 128), (128, 128), (256, 64)):
        for G in (1, 2, 3, 4, 7, 8, 16):
            prob = pk.Problem(1, 2 * G, 2, D, 16, 1, 1, pk.KV_BF16, 0.0, pk.LAYOUT_NHD, 1)
            assert pk.prefill_rows_per_tile(prob) == cols // G


def test_tile_argument_checks():
    pk = _pk()
    with pytest.raises(pk.PdattnError):
        pk.prefill_tiles([0, 5, 3], 8, longest_first=False)        # decreasing
    with pytest.raises(pk.PdattnError):
        pk.prefill_tiles([0, 5], 0, longest_first=False)           # rows_per_tile 0
    with pytest.raises(pk.PdattnError):
        pk.prefill_tiles([0, 5], 8, longest_first=True)            # longest first needs lengths
    import ctypes
    ptr = torch.tensor([0, 100], dtype=torch.int32)
    tb = torch.empty(2, dtype=torch.int32)
    count = ctypes.c_int32(0)
    st = pk._lib.pdattn_prefill_tiles(pk._ptr(ptr), None, 1, 8, 1, 0, pk._ptr(tb), pk._ptr(tb), 2,
                                      ctypes.byref(count))
    assert st != 0 and count.value == 13    # too small a buffer; the count is still reported


def test_prefill_rejects_bad_arguments_before_launch():
    """Validation happens on the host: these calls return an error without
    touching a device (null device pointers would fault if launched)."""
    pk = _pk()
    import ctypes
    prob = pk.Problem(2, 8, 2, 128, 16, 4, 8, pk.KV_BF16, 0.0, pk.LAYOUT_NHD, 1)
    P = ctypes.c_void_p
    # required pointers missing
    st = pk._lib.pdattn_prefill(ctypes.byref(prob), 1, None, None, None, None, 3, None, None, None, None, None, None,
                                None, None, None)
    assert st == 1
    # causal flag outside {0, 1}
    st = pk._lib.pdattn_prefill(ctypes.byref(prob), 2, P(16), P(16), P(16), P(16), 3, P(16), P(16), None, None,
                                P(16), P(16), P(16), None, None)
    assert st == 1
    # head_dim not built
    bad = pk.Problem(2, 8, 2, 96, 16, 4, 8, pk.KV_BF16, 0.0, pk.LAYOUT_NHD, 1)
    st = pk._lib.pdattn_prefill(ctypes.byref(bad), 1, P(16), P(16), P(16), P(16), 3, P(16), P(16), None, None,
                                P(16), P(16), P(16), None, None)
    assert st == 2
    # zero tiles: nothing to do, success without any pointer
    st = pk._lib.pdattn_prefill(ctypes.byref(prob), 1, None, None, None, None, 0, None, None, None, None, None, None,
                                None, None, None)
    assert st == 0
