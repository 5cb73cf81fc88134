"""Host logic of the prefill boundary, on the CPU: the tile map that
pdattn_prefill_tiles builds (against the pages' worked example and the
oracle's tile map), its longest-first order, the split map of
pdattn_prefill_split_tiles (against the rule its header states), the
rows-per-tile query and the argument checks. No device call is made."""
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


def _reach(ptr, L, b, j, rt, causal):
    n = int(ptr[b + 1] - ptr[b])
    last = min((j + 1) * rt, n) - 1
    r = int(L[b]) - n + last + 1 if causal else int(L[b])
    return min(max(r, 0), int(L[b]))


def _split_problem(B, D=128, Hq=32, Hkv=8, P=16, max_len=1):
    mp = max(1, -(-max_len // P))
    return _pk().Problem(B, Hq, Hkv, D, P, mp, B * mp, 0, 0.0, 0, 1)


def _map_by_rule(ptr, L, rows, nt, H, slots, causal):
    """The split map as pdattn.h states the rule: for each candidate cap
    (none, then ceil(k x longest / 16) for k = 15 .. 3, at least 4), cut the
    long tiles evenly at multiples of 64 positions, list the entries by cost
    (most first, stable), simulate the list schedule on `slots` slots and
    keep the first cap that ends soonest. Returns entries as
    [b, j, kv0, kv1, base, pq] and the slot count."""
    import heapq
    min_units = -(-4 * nt // 64)
    tiles = []
    for b in range(len(ptr) - 1):
        n, Lb = int(ptr[b + 1] - ptr[b]), int(L[b])
        for j in range(-(-n // rows)):
            last = min((j + 1) * rows, n) - 1
            reach = min(max(Lb - n + last + 1 if causal else Lb, 0), Lb)
            opn = min(max(Lb - n + j * rows + 1 if causal else Lb, 0), Lb)
            tiles.append((b, j, reach, opn, -(-reach // nt)))

    def cost(t, kv0, kv1, part):
        i0, i1 = kv0 // nt, -(-kv1 // nt)
        return 4 * (i1 - i0) + max(0, i1 - max(i0, t[3] // nt)) + 20 + (12 if part else 0)

    def cut(cap):
        out, nslots = [], 0
        for t in tiles:
            units = -(-t[2] // 64)
            parts = min(-(-t[4] // cap), 16, units // min_units) if t[4] > cap else 1
            if parts < 2:
                out.append((cost(t, 0, t[2], False), [t[0], t[1], 0, t[2], -1, 1 << 16]))
                continue
            for q in range(parts):
                kv0 = q * units // parts * 64
                kv1 = t[2] if q + 1 == parts else (q + 1) * units // parts * 64
                out.append((cost(t, kv0, kv1, True), [t[0], t[1], kv0, kv1, nslots, q | (parts << 16)]))
            nslots += parts
        out.sort(key=lambda e: -e[0])
        return out, nslots

    def span(lst):
        free = [0] * min(slots, len(lst) * H)
        end = 0
        for c, _ in lst:
            for _ in range(H):
                t = heapq.heappop(free) + c
                heapq.heappush(free, t)
                end = max(end, t)
        return end
    longest = max((t[4] for t in tiles), default=0)
    best = None
    for cap in [1 << 62] + [max(4, -(-longest * k // 16)) for k in range(15, 2, -1)]:
        lst, nslots = cut(cap)
        sp = span(lst)
        if best is None or sp < best[0]:
            best = (sp, [e for _, e in lst], nslots)
    return (best[1], best[2]) if best else ([], 0)


@pytest.mark.parametrize("causal", [True, False])
def test_split_map_follows_the_rule_and_covers_every_position_once(causal):
    """pdattn_prefill_split_tiles: entries equal the rule pdattn.h states;
    every query tile appears, whole or as parts whose ranges join up to
    [0, reach) in part order at multiples of 64 (each at least 4 kernel
    tiles), the parts of a tile hold consecutive slots, no slot is shared,
    and the workspace size follows the slot count."""
    pk = _pk()
    rng = np.random.default_rng(17)
    cut_any = 0
    for trial in range(40):
        B = int(rng.integers(1, 10))
        n = rng.integers(0, 700, B)
        L = n + rng.integers(0, 3000, B)
        if rng.random() < 0.3:
            L = np.minimum(L, rng.integers(0, 300, B))
        ptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        D = int(rng.choice([64, 128, 256]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 8]))
        prob = _split_problem(B, D=D, Hq=G * Hkv, Hkv=Hkv, max_len=int(L.max()))
        slots = int(rng.choice([8, 64, 512, 4096]))
        st = pk.prefill_split_tiles(prob, ptr, L.astype(np.int32), causal=causal, slots=slots)
        rt = pk.prefill_rows_per_tile(prob)
        nt = 32 if D == 256 else 64
        want, want_slots = _map_by_rule(ptr, L, rt, nt, Hkv, slots, causal)
        got = [[b, j] + k for b, j, k in zip(st.tile_batch.tolist(), st.tile_index.tolist(), st.tile_kv.tolist())]
        assert got == want and st.num_slots == want_slots
        cut_any += st.num_slots > 0
        ref_b, ref_i = pf.tile_map(ptr, rt)
        parts_of = {}
        for e in got:
            parts_of.setdefault((e[0], e[1]), []).append(e[2:])
        assert sorted(parts_of) == sorted(zip(ref_b, ref_i))
        used = set()
        for (b, j), ents in parts_of.items():
            reach = _reach(ptr, L, b, j, rt, causal)
            if len(ents) == 1 and ents[0][2] == -1:
                assert ents[0] == [0, reach, -1, 1 << 16]
                continue
            parts = ents[0][3] >> 16
            assert 2 <= parts <= 16 and len(ents) == parts
            e = sorted(ents, key=lambda x: x[3] & 0xFFFF)
            assert [x[3] & 0xFFFF for x in e] == list(range(parts))
            assert all(x[3] >> 16 == parts and x[2] == e[0][2] for x in e)
            assert e[0][0] == 0 and e[-1][1] == reach
            for a, c in zip(e, e[1:]):
                assert a[1] == c[0] and a[1] % 64 == 0 and a[1] - a[0] >= 4 * nt
            assert e[-1][1] - e[-1][0] >= 4 * nt - 63
            here = set(range(e[0][2], e[0][2] + parts))
            assert not (here & used)
            used |= here
        assert used == set(range(st.num_slots))
        rec = (64 if D == 256 else 128) * (D + 2) * 4
        ws = 0 if st.num_slots == 0 else -(-st.num_slots * Hkv * 4 // 256) * 256 + st.num_slots * Hkv * rec
        assert st.workspace_bytes == ws
    assert cut_any >= 5


def test_split_planner_cuts_the_long_prompt_only():
    """One 2048-token causal prompt (64 tiles of 32 rows reading 1 to 32
    kernel tiles) on 512 slots: the longest tiles are cut; the ragged and
    chunked bench batches, whose tiles already spread over the slots, and a
    prompt of 4 kernel tiles are not."""
    pk = _pk()
    import synth
    prob = _split_problem(1, max_len=2048)
    st = pk.prefill_split_tiles(prob, [0, 2048], [2048], causal=True, slots=512)
    assert st.num_slots > 0 and st.num_tiles > 64
    for name in ("llama3_8b_prefill", "llama3_8b_chunked_prefill"):
        desc, dims, batch, qr, pr, seed = synth.PREFILL_WORKLOADS[name]
        g = torch.Generator().manual_seed(seed + 2)
        q = torch.randint(qr[0], qr[1] + 1, (batch,), generator=g)
        pre = torch.randint(pr[0], pr[1] + 1, (batch,), generator=g)
        lens = (q + pre).to(torch.int32)
        ptr = torch.cat([torch.zeros(1, dtype=torch.int64), q.cumsum(0)]).to(torch.int32)
        big = _split_problem(batch, max_len=int(lens.max()))
        st = pk.prefill_split_tiles(big, ptr, lens, causal=True, slots=512)
        assert st.num_slots == 0, name
    short = pk.prefill_split_tiles(_split_problem(1, max_len=400), [0, 32], [256], causal=True, slots=1 << 20)
    assert short.num_slots == 0 and short.num_tiles == 1


def test_split_argument_checks():
    pk = _pk()
    import ctypes
    prob = _split_problem(1, max_len=2048)
    with pytest.raises(pk.PdattnError):
        pk.prefill_split_tiles(prob, [0, 2048], [5000], slots=512)   # length beyond the block table
    with pytest.raises(pk.PdattnError):
        pk.prefill_split_tiles(prob, [0, 2048], [2048], slots=-1)
    P = ctypes.c_void_p
    call = pk._lib.pdattn_prefill_split
    # parts but no workspace; a workspace too small; no tile_kv
    assert call(ctypes.byref(prob), 1, P(16), P(16), P(16), P(16), P(16), 3, 2, None, 0, P(16), P(16), None, None,
                P(16), P(16), P(16), None, None) == 3
    assert call(ctypes.byref(prob), 1, P(16), P(16), P(16), P(16), P(16), 3, 2, P(256), 100, P(16), P(16), None,
                None, P(16), P(16), P(16), None, None) == 3
    assert call(ctypes.byref(prob), 1, P(16), P(16), P(16), P(16), None, 3, 0, None, 0, P(16), P(16), None, None,
                P(16), P(16), P(16), None, None) == 1
    assert call(ctypes.byref(prob), 1, None, None, None, None, None, 0, 0, None, 0, None, None, None, None, None,
                None, None, None, None) == 0


def test_prefill_scale_arguments_by_pool_dtype():
    """Argument checks before any launch: separate-scale fp8 pools need both
    scale arrays; bf16 and inline-scale fp8 pools (the scale after each
    row's codes) take none. Every failing call returns
    PDATTN_ERR_INVALID_ARGUMENT and enqueues nothing."""
    pk = _pk()
    import ctypes
    P = ctypes.c_void_p
    call = pk._lib.pdattn_prefill
    for kv, k_scale, v_scale in ((pk.KV_FP8_E4M3, None, None), (pk.KV_FP8_E4M3, P(16), None),
                                 (pk.KV_FP8_E4M3_INLINE, P(16), P(16)), (pk.KV_FP8_E4M3_INLINE, None, P(16)),
                                 (pk.KV_BF16, P(16), P(16))):
        prob = _split_problem(1, max_len=2048)
        prob.kv_dtype = kv
        st = call(ctypes.byref(prob), 1, P(16), P(16), P(16), P(16), 3, P(16), P(16), k_scale, v_scale, P(16),
                  P(16), P(16), None, None)
        assert st == 1, (kv, st)
        msg = pk._lib.pdattn_last_error().decode()
        assert "scale" in msg, msg
