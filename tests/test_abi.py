"""The C ABI of libpdattn.so on the CPU: exports, struct layout, the planner
and argument validation. Nothing here launches a kernel: every decode and
reduce call below is rejected by validation before any HIP call."""
import ctypes
import math
import os
import random
import re

import pytest
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pdattn.h")

import paged_kv_split_amd as pk

OK, INVALID, UNSUPPORTED, WORKSPACE, MISMATCH, DEVICE = range(6)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"PDATTN_API\s+[\w\s\*]+?\b(pdattn_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"pdattn_plan", "pdattn_decode", "pdattn_reduce", "pdattn_workspace_init", "pdattn_status_string",
            "pdattn_last_error"} <= set(names)
    lib = ctypes.CDLL(pk.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_binding():
    assert pk._lib.pdattn_problem_size() == ctypes.sizeof(pk.Problem) == 44
    assert pk._lib.pdattn_plan_size() == ctypes.sizeof(pk.Plan)


def test_status_strings():
    for s in range(6):
        assert pk._lib.pdattn_status_string(s).decode()
    assert pk._lib.pdattn_status_string(99).decode() == "unknown status"


def problem(**kw):
    d = dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, max_pages_per_seq=64,
             num_pages=512, kv_dtype=0, scale=0.0, kv_layout=0, q_len=0)
    d.update(kw)
    return d


def plan_raw(lens, num_cus=256, force=0, flags=0, **kw):
    p = problem(**kw)
    prob = pk.Problem(*[p[f] for f, _ in pk.Problem._fields_])
    lens_t = torch.as_tensor(lens, dtype=torch.int32).contiguous() if lens is not None else None
    out = pk.Plan()
    ptr = ctypes.c_void_p(lens_t.data_ptr()) if lens_t is not None else None
    st = pk._lib.pdattn_plan(ctypes.byref(prob), ptr, num_cus, force, flags, ctypes.byref(out))
    return st, out


def dyn_workspace_bytes(pl):
    """Balanced-mode workspace: 256-byte header, counters (claims, records,
    done tiles per unit; done units per pair), unit records (units_max + 3
    per worker), pair-level records when a pair can span several units."""
    pr = pl.problem
    G = pr.num_q_heads // pr.num_kv_heads
    rec = G * (pr.head_dim + 2) * 4
    max_tiles = -(-pr.max_pages_per_seq * pr.page_size // 16)
    seg_max = max(1, -(-max_tiles // 512))
    units = pr.batch * pr.num_kv_heads * seg_max
    up = lambda x: -(-x // 256) * 256
    ctl = 4 * (3 * units + pr.batch * pr.num_kv_heads)
    total = 256 + up(ctl) + up((units + 3 * pl.num_workers) * rec)
    if seg_max > 1:
        total += units * rec
    return total


@pytest.mark.parametrize("flags", [0, 2], ids=["static", "balanced"])
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plan_for_each_workload(name, flags):
    w = synth.WORKLOADS[name]
    g = torch.Generator().manual_seed(w.seed)
    lens = synth._lens(w, g)
    maxp = int((lens.max() + w.page_size - 1) // w.page_size)
    st, pl = plan_raw(lens, flags=flags, batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                      head_dim=w.head_dim, page_size=w.page_size, max_pages_per_seq=maxp, num_pages=10 ** 6,
                      kv_dtype=0 if w.kv_dtype == "bf16" else 1)
    assert st == OK, pk._lib.pdattn_last_error()
    assert pl.flags == flags
    tiles = w.num_kv_heads * sum((int(L) + 15) // 16 for L in lens.tolist())
    assert pl.total_tiles == tiles
    assert pl.max_context_len == int(lens.max())
    G = w.num_q_heads // w.num_kv_heads
    rec = G * (w.head_dim + 2) * 4
    if flags:
        assert pl.workspace_bytes == dyn_workspace_bytes(pl)
    else:
        # two records per worker, then the tile prefix (batch + 1 int64 words)
        assert pl.workspace_bytes == pl.num_workers * 2 * rec + (w.batch + 1) * 8
    assert 1 <= pl.num_workers <= 4 * pl.num_workgroups
    assert pl.num_workers <= max(1, tiles // 4)
    assert abs(pl.problem.scale - 1.0 / math.sqrt(w.head_dim)) < 1e-7


def test_plan_forced_workers_and_empty_batch():
    st, pl = plan_raw([100, 0, 37, 1024], force=7)
    assert st == OK and pl.num_workers == 7 and pl.num_workgroups == 2
    st, pl = plan_raw([], batch=0)
    assert st == OK and pl.num_workers == 1
    st, pl = plan_raw([0, 0, 0, 0])
    assert st == OK and pl.total_tiles == 0 and pl.num_workers == 1


@pytest.mark.parametrize("kw,lens,expect", [
    (dict(num_q_heads=12), [1, 1, 1, 1], INVALID),           # Hq not a multiple of Hkv
    (dict(num_q_heads=24, flags=2), [1, 1, 1, 1], UNSUPPORTED),   # G = 3 needs a static plan
    (dict(num_q_heads=256), [1, 1, 1, 1], UNSUPPORTED),      # G = 32
    (dict(head_dim=96), [1, 1, 1, 1], UNSUPPORTED),
    (dict(page_size=12), [1, 1, 1, 1], UNSUPPORTED),
    (dict(page_size=4), [1, 1, 1, 1], UNSUPPORTED),
    (dict(page_size=256), [1, 1, 1, 1], UNSUPPORTED),
    (dict(kv_dtype=7), [1, 1, 1, 1], UNSUPPORTED),
    (dict(kv_layout=2), [1, 1, 1, 1], UNSUPPORTED),
    (dict(q_len=8), [1, 1, 1, 1], UNSUPPORTED),              # 8 rows x 4 heads = 32 columns
    (dict(q_len=5), [1, 1, 1, 1], UNSUPPORTED),              # 20 columns
    (dict(q_len=-1), [1, 1, 1, 1], INVALID),
    (dict(q_len=2, flags=2), [1, 1, 1, 1], UNSUPPORTED),     # multi-query needs a static plan
    (dict(kv_layout=-1), [1, 1, 1, 1], UNSUPPORTED),
    (dict(scale=float("nan")), [1, 1, 1, 1], INVALID),
    (dict(batch=70000), [1] * 4, INVALID),
    (dict(num_kv_heads=0), [1, 1, 1, 1], INVALID),
    (dict(), [1, 1, 1, 64 * 16 + 1], INVALID),               # length beyond the block table
    (dict(), [1, -1, 1, 1], INVALID),
    (dict(), None, INVALID),                                 # no host lengths
    (dict(num_pages=0), [1, 1, 1, 1], INVALID),              # nothing to read from
    (dict(flags=1), [1, 1, 1, 1], INVALID),                  # unknown flag
    (dict(flags=2, batch=65535, num_q_heads=128, num_kv_heads=128, max_pages_per_seq=4096), [1] * 65535,
     UNSUPPORTED),                                           # 2^31 tiles per row set (balanced mode)
])
def test_plan_rejects(kw, lens, expect):
    st, _ = plan_raw(lens, **kw)
    assert st == expect
    assert pk._lib.pdattn_last_error().decode()


def _decode_raw(pl, q=16, k=16, v=16, ks=None, vs=None, bt=16, lens=16, ws=16, ws_bytes=None, out=16, lse=None):
    P = ctypes.c_void_p
    ws_bytes = pl.workspace_bytes if ws_bytes is None else ws_bytes
    return pk._lib.pdattn_decode(ctypes.byref(pl), P(q) if q else None, P(k) if k else None,
                                 P(v) if v else None, P(ks) if ks else None, P(vs) if vs else None,
                                 P(bt) if bt else None, P(lens) if lens else None, P(ws) if ws else None,
                                 ws_bytes, P(out) if out else None, P(lse) if lse else None, None)


def test_decode_validation_rejects_before_launch():
    st, pl = plan_raw([5, 9, 100, 33])
    assert st == OK
    assert _decode_raw(pl, q=0) == INVALID
    assert _decode_raw(pl, out=0) == INVALID
    assert _decode_raw(pl, q=0x1008) == INVALID          # not 16-byte aligned
    assert _decode_raw(pl, k=0x1004) == INVALID
    assert _decode_raw(pl, bt=0x1002) == INVALID
    assert _decode_raw(pl, ks=0x2000, vs=0x2000) == INVALID   # scales on a bf16 pool
    assert _decode_raw(pl, ws=0) == WORKSPACE
    assert _decode_raw(pl, ws_bytes=pl.workspace_bytes - 1) == WORKSPACE
    assert _decode_raw(pl, ws=0x1008) == INVALID
    st, pl8 = plan_raw([5, 9, 100, 33], kv_dtype=1)
    assert _decode_raw(pl8) == INVALID                     # fp8 pool without scales
    bad = pk.Plan.from_buffer_copy(bytes(pl))
    bad.magic = 0
    assert _decode_raw(bad) == MISMATCH
    bad = pk.Plan.from_buffer_copy(bytes(pl))
    bad.num_workers = 10 ** 7
    assert _decode_raw(bad) == MISMATCH
    bad = pk.Plan.from_buffer_copy(bytes(pl))
    bad.flags = 6
    assert _decode_raw(bad) == MISMATCH
    assert "workspace" in pk._lib.pdattn_last_error().decode() or pk._lib.pdattn_last_error()
    st, empty = plan_raw([], batch=0)
    assert _decode_raw(empty, q=0, k=0, v=0, bt=0, lens=0, out=0, ws=0) == OK   # nothing to do


def test_reduce_validation_rejects_before_launch():
    st, pl = plan_raw([5, 9, 100, 33])
    P = ctypes.c_void_p
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), None, pl.workspace_bytes, P(16), None, None) == WORKSPACE
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), P(16), pl.workspace_bytes - 4, P(16), None, None) == WORKSPACE
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), P(16), pl.workspace_bytes, None, None, None) == INVALID
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), P(16), pl.workspace_bytes, P(0x1004), None, None) == INVALID
    assert pk._lib.pdattn_reduce(None, P(16), 0, P(16), None, None) == INVALID


def _weight_before(w, NW, wa, wb):
    h = NW // 2
    return wa * w if w <= h else wa * h + wb * (w - h)


@pytest.mark.parametrize("wa,wb", [(1, 1), (5, 4), (3, 2), (2, 1), (16, 15)])
def test_worker_range_arithmetic(wa, wb):
    """The kernels place worker w on tiles [T W(w) / W(NW), T W(w+1) / W(NW))
    with W(w) the weight of workers 0 .. w-1 (the first half wa each, the
    rest wb), and find the worker holding tile C as the last w with
    W(w) <= ceil((C+1) W(NW) / T) - 1 (merge_ops.h); check that rule against
    a brute-force search over the ranges themselves."""
    rng = random.Random(5 + wa)
    for _ in range(2000):
        T = rng.randint(1, 5000)
        NW = rng.randint(1, 700)
        C = rng.randrange(T)
        om = _weight_before(NW, NW, wa, wb)
        start = lambda w: T * _weight_before(w, NW, wa, wb) // om
        c = ((C + 1) * om + T - 1) // T - 1
        h = NW // 2
        wf = min(c // wa if c < wa * h else h + (c - wa * h) // wb, NW - 1)
        brute = max(w for w in range(NW) if start(w) <= C)
        assert wf == brute
        assert start(wf) <= C < start(wf + 1)
        assert start(0) == 0 and start(NW) == T


def test_plan_split_weights():
    """Equal weights unless the plan takes the streaming kernel's full grid
    for an fp8 pool; forced worker counts, bf16 pools, balanced plans and the
    general kernel (page size 8) keep equal weights. A plan whose weights do
    not fit its kernel is refused."""
    lens = [4000] * 32
    kw = dict(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, max_pages_per_seq=256,
              num_pages=10 ** 6)
    equal = (1 << 16) | 1
    for extra in (dict(kv_dtype=0), dict(kv_dtype=1, force=2048), dict(kv_dtype=0, flags=2),
                  dict(kv_dtype=1, page_size=8, max_pages_per_seq=512)):
        st, pl = plan_raw(lens, **{**kw, **extra})
        assert st == OK, pk._lib.pdattn_last_error()
        assert pl.split_weights == equal, extra
    st, pl = plan_raw(lens, **{**kw, "kv_dtype": 1})
    assert st == OK and pl.split_weights in (equal, (5 << 16) | 4)
    st, bf = plan_raw(lens, **{**kw, "kv_dtype": 0})
    for bad_w in (0, (17 << 16) | 1, 1 << 16, 1):    # a weight of 0 or above 16
        bad = pk.Plan.from_buffer_copy(bytes(bf))
        bad.split_weights = bad_w
        assert _decode_raw(bad) == MISMATCH
    st, gen = plan_raw(lens, **{**kw, "kv_dtype": 1, "page_size": 8, "max_pages_per_seq": 512})
    bad = pk.Plan.from_buffer_copy(bytes(gen))
    bad.split_weights = (5 << 16) | 4
    assert _decode_raw(bad) == MISMATCH               # the general kernel splits equally


def test_workspace_init_validation():
    st, pl = plan_raw([5, 9, 100, 33], flags=2)
    P = ctypes.c_void_p
    assert pk._lib.pdattn_workspace_init(ctypes.byref(pl), None, pl.workspace_bytes, None) == WORKSPACE
    assert pk._lib.pdattn_workspace_init(ctypes.byref(pl), P(16), pl.workspace_bytes - 1, None) == WORKSPACE
    assert pk._lib.pdattn_workspace_init(ctypes.byref(pl), P(0x1008), pl.workspace_bytes, None) == INVALID
    assert pk._lib.pdattn_workspace_init(None, P(16), 0, None) == INVALID
    st, static = plan_raw([5, 9, 100, 33])
    assert pk._lib.pdattn_workspace_init(ctypes.byref(static), None, 0, None) == OK   # nothing to prepare


def test_balanced_reduce_is_a_validated_no_op():
    st, pl = plan_raw([5, 9, 100, 33], flags=2)
    P = ctypes.c_void_p
    # valid-looking arguments: nothing is launched for a default-mode plan
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), P(16), pl.workspace_bytes, P(16), None, None) == OK
    assert pk._lib.pdattn_reduce(ctypes.byref(pl), P(16), pl.workspace_bytes - 1, P(16), None, None) == WORKSPACE


def _append_raw(prob=None, n=4, kn=0x1000, vn=0x2000, seq=0x3000, pos=0x4000, bt=0x5000, kp=0x6000, vp=0x7000,
                ks=None, vs=None, flags=0, **kw):
    p = problem(**kw) if prob is None else prob
    pr = pk.Problem(*[p[f] for f, _ in pk.Problem._fields_])
    P = lambda a: ctypes.c_void_p(a) if a else None
    return pk._lib.pdattn_kv_append(ctypes.byref(pr), n, P(kn), P(vn), P(seq), P(pos), P(bt), P(kp), P(vp),
                                    P(ks), P(vs), flags, None)


def test_merge_validation_rejects_before_launch():
    P = ctypes.c_void_p
    m = pk._lib.pdattn_merge
    assert m(2, 10, 96, P(0x1000), P(0x2000), P(0x3000), None, None) == UNSUPPORTED
    assert m(0, 10, 128, P(0x1000), P(0x2000), P(0x3000), None, None) == INVALID
    assert m(2, -1, 128, P(0x1000), P(0x2000), P(0x3000), None, None) == INVALID
    assert m(2, 10, 128, None, P(0x2000), P(0x3000), None, None) == INVALID
    assert m(2, 10, 128, P(0x1000), P(0x2000), None, None, None) == INVALID
    assert m(2, 10, 128, P(0x1008), P(0x2000), P(0x3000), None, None) == INVALID
    assert m(2, 10, 128, P(0x1000), P(0x2002), P(0x3000), None, None) == INVALID
    assert m(2, 10, 128, P(0x1000), P(0x2000), P(0x3000), P(0x4001), None) == INVALID
    assert m(2, 0, 128, None, None, None, None, None) == OK        # nothing to do


def test_fp8_conversion_check_validation():
    assert pk._lib.pdattn_fp8_conversion_check(None, None) == INVALID
    assert pk._lib.pdattn_fp8_conversion_check(ctypes.c_void_p(0x1004), None) == INVALID


def test_kv_append_validation_rejects_before_launch():
    assert _append_raw(n=-1) == INVALID
    assert _append_raw(kn=0) == INVALID
    assert _append_raw(bt=0) == INVALID
    assert _append_raw(kn=0x1008) == INVALID                 # not 16-byte aligned
    assert _append_raw(vp=0x7004) == INVALID
    assert _append_raw(pos=0x4002) == INVALID
    assert _append_raw(ks=0x8000, vs=0x9000) == INVALID      # scales on a bf16 pool
    assert _append_raw(flags=pk.APPEND_POW2_SCALES) == INVALID   # pow2 scales on a bf16 pool
    assert _append_raw(flags=4) == INVALID
    assert _append_raw(kv_dtype=1) == INVALID                # fp8 pool without scales
    assert _append_raw(kv_dtype=1, ks=0x8000, vs=0x9002) == INVALID
    assert _append_raw(head_dim=96) == UNSUPPORTED
    assert _append_raw(page_size=24) == UNSUPPORTED
    assert _append_raw(num_kv_heads=3) == INVALID            # 32 q heads not a multiple of 3
    assert _append_raw(kv_layout=5) == UNSUPPORTED
    assert "aligned" in (_append_raw(kn=0x1008), pk._lib.pdattn_last_error().decode())[1]
    # nothing to do: no pointer is read
    assert _append_raw(n=0, kn=0, vn=0, seq=0, pos=0, bt=0, kp=0, vp=0) == OK
    assert _append_raw(batch=0, kn=0, vn=0, seq=0, pos=0, bt=0, kp=0, vp=0) == OK


def test_plan_accepts_any_group_up_to_16():
    for hq, hkv, qlen in ((24, 8, 0), (28, 4, 0), (12, 4, 5), (40, 8, 3), (15, 1, 1), (32, 8, 3)):
        st, pl = plan_raw([5, 9, 100, 33], num_q_heads=hq, num_kv_heads=hkv, q_len=qlen)
        assert st == OK, (hq, hkv, qlen, pk._lib.pdattn_last_error())
