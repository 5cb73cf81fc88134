"""Python binding of libpdattn.so: paged split-KV GQA decode attention on
MI355X (gfx950).

The functions below keep the C-ABI names (``plan``, ``decode``, ``reduce``)
and only marshal arguments: torch tensors in, device pointers and the
current HIP stream out. Every step of the computation runs in the library's
kernels; there is no other code path. Importing this module fails loudly when
the library has not been built (``python paged_kv_split_amd/build.py``).
"""
import ctypes
import os

import torch

__all__ = ["Problem", "Plan", "PdattnError", "plan", "decode", "reduce", "decode_noalloc", "NOALLOC_SCRATCH_BYTES",
           "workspace", "workspace_init",
           "paged_decode", "KV_BF16", "KV_FP8_E4M3", "PLAN_BALANCED", "library_path", "stream_read",
           "stream_read_sink", "kv_append", "APPEND_POW2_SCALES", "fp8_conversion_check", "merge", "LAYOUT_NHD", "LAYOUT_HND",
           "pool_dims", "kv_kind", "KV_FP8_E4M3_INLINE", "prefill_rows_per_tile", "prefill_tiles", "prefill", "paged_prefill", "TILES_LONGEST_FIRST",
           "SplitTiles", "prefill_split_tiles", "prefill_split", "prefill_split_workspace"]

KV_BF16 = 0
KV_FP8_E4M3 = 1
KV_FP8_E4M3_INLINE = 2   # uint8 pools, rows of d codes then the row's fp32 scale
PLAN_BALANCED = 2
LAYOUT_NHD = 0   # pool rows [page][slot][kv head]
LAYOUT_HND = 1   # pool rows [page][kv head][slot]
APPEND_POW2_SCALES = 1
TILES_LONGEST_FIRST = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpdattn.so")

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is missing: build it with `python paged_kv_split_amd/build.py`")

_lib = ctypes.CDLL(library_path)


class Problem(ctypes.Structure):
    """Mirror of ``pdattn_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("kv_layout", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    """Mirror of ``pdattn_plan_t``."""
    _fields_ = [
        ("problem", Problem),
        ("num_cus", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("total_tiles", ctypes.c_int64),
        ("max_context_len", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32),
        ("split_weights", ctypes.c_uint32),
    ]


_P = ctypes.c_void_p
_lib.pdattn_plan.restype = ctypes.c_int
_lib.pdattn_plan.argtypes = [ctypes.POINTER(Problem), _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                             ctypes.POINTER(Plan)]
_lib.pdattn_workspace_init.restype = ctypes.c_int
_lib.pdattn_workspace_init.argtypes = [ctypes.POINTER(Plan), _P, ctypes.c_uint64, _P]
_lib.pdattn_decode.restype = ctypes.c_int
_lib.pdattn_decode.argtypes = [ctypes.POINTER(Plan), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, _P, _P, _P]
_lib.pdattn_reduce.restype = ctypes.c_int
_lib.pdattn_reduce.argtypes = [ctypes.POINTER(Plan), _P, ctypes.c_uint64, _P, _P, _P]
_lib.pdattn_decode_noalloc.restype = ctypes.c_int
_lib.pdattn_decode_noalloc.argtypes = [ctypes.POINTER(Plan), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.pdattn_status_string.restype = ctypes.c_char_p
_lib.pdattn_status_string.argtypes = [ctypes.c_int]
_lib.pdattn_last_error.restype = ctypes.c_char_p
_lib.pdattn_last_error.argtypes = []
_lib.pdattn_stream_read.restype = ctypes.c_int
_lib.pdattn_stream_read.argtypes = [_P, ctypes.c_uint64, _P, ctypes.c_int32, _P]
_lib.pdattn_stream_read_sink_words.restype = ctypes.c_uint64
_lib.pdattn_stream_read_sink_words.argtypes = [ctypes.c_int32]
_lib.pdattn_kv_append.restype = ctypes.c_int
_lib.pdattn_kv_append.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_int32, _P]
_lib.pdattn_merge.restype = ctypes.c_int
_lib.pdattn_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P, _P]
_lib.pdattn_fp8_conversion_check.restype = ctypes.c_int
_lib.pdattn_fp8_conversion_check.argtypes = [_P, _P]
_lib.pdattn_prefill_rows_per_tile.restype = ctypes.c_int
_lib.pdattn_prefill_rows_per_tile.argtypes = [ctypes.POINTER(Problem), _P]
_lib.pdattn_prefill_tiles.restype = ctypes.c_int
_lib.pdattn_prefill_tiles.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                      ctypes.c_int32, _P]
_lib.pdattn_prefill.restype = ctypes.c_int
_lib.pdattn_prefill.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P]
_lib.pdattn_prefill_split_tiles.restype = ctypes.c_int
_lib.pdattn_prefill_split_tiles.argtypes = [ctypes.POINTER(Problem), _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                            _P, ctypes.c_int32, _P, _P, _P]
_lib.pdattn_prefill_split.restype = ctypes.c_int
_lib.pdattn_prefill_split.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_int32,
                                      ctypes.c_int32, _P, ctypes.c_uint64, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.pdattn_problem_size.restype = ctypes.c_uint64
_lib.pdattn_plan_size.restype = ctypes.c_uint64

if _lib.pdattn_problem_size() != ctypes.sizeof(Problem) or _lib.pdattn_plan_size() != ctypes.sizeof(Plan):
    raise ImportError("libpdattn.so struct layout does not match the binding")


class PdattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.pdattn_status_string(status).decode()
        detail = _lib.pdattn_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


def _check(status, where):
    if status != 0:
        raise PdattnError(status, where)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kv_kind(pages):
    """The kv dtype of a pool tensor: bf16; float8_e4m3fn (separate scale
    arrays); uint8 (inline-scale fp8 rows of d codes and 4 scale bytes)."""
    if pages.dtype == torch.uint8:
        return KV_FP8_E4M3_INLINE
    return KV_FP8_E4M3 if pages.dtype == torch.float8_e4m3fn else KV_BF16


def pool_dims(pages, layout=LAYOUT_NHD):
    """(num_pages, P, Hkv, d) of a pool tensor in the given layout."""
    n, a, b, d = pages.shape
    return (n, a, b, d) if layout == LAYOUT_NHD else (n, b, a, d)


def plan(*, batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_pages,
         kv_dtype=KV_BF16, scale=0.0, context_lens_host, num_cus=0, force_workers=0,
         balanced=False, kv_layout=LAYOUT_NHD, q_len=1) -> Plan:
    """``pdattn_plan``: context_lens_host is a CPU int32 tensor (or sequence)."""
    lens = torch.as_tensor(context_lens_host, dtype=torch.int32).cpu().contiguous()
    prob = Problem(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_pages,
                   kv_dtype, float(scale), kv_layout, q_len)
    out = Plan()
    flags = PLAN_BALANCED if balanced else 0
    _check(_lib.pdattn_plan(ctypes.byref(prob), _ptr(lens), int(num_cus), int(force_workers), flags,
                            ctypes.byref(out)), "pdattn_plan")
    return out


def decode(pl: Plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, workspace,
           out, lse=None, stream=None):
    """``pdattn_decode`` on device tensors (workspace: a uint8 tensor or None)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pdattn_decode(ctypes.byref(pl), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                              _ptr(v_scale), _ptr(block_table), _ptr(context_lens), _ptr(workspace),
                              ws_bytes, _ptr(out), _ptr(lse), _stream(stream)), "pdattn_decode")


def reduce(pl: Plan, workspace, out, lse=None, stream=None):
    """``pdattn_reduce`` on device tensors."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pdattn_reduce(ctypes.byref(pl), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                              _stream(stream)), "pdattn_reduce")


def decode_noalloc(pl: Plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, out, lse=None,
                   stream=None):
    """``pdattn_decode_noalloc``: decode and reduce on the library's static device scratch."""
    _check(_lib.pdattn_decode_noalloc(ctypes.byref(pl), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                      _ptr(v_scale), _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse),
                                      _stream(stream)), "pdattn_decode_noalloc")


NOALLOC_SCRATCH_BYTES = 64 << 20


def workspace_init(pl: Plan, workspace, stream=None):
    """``pdattn_workspace_init``: prepare a workspace for balanced-mode decodes."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pdattn_workspace_init(ctypes.byref(pl), _ptr(workspace), ws_bytes, _stream(stream)),
           "pdattn_workspace_init")


def workspace(pl: Plan, device, stream=None):
    """A torch-allocated workspace of the plan's size, prepared for use."""
    ws = torch.empty(int(pl.workspace_bytes), dtype=torch.uint8, device=device)
    workspace_init(pl, ws, stream)
    return ws


def stream_read(buffer, sink, num_cus, stream=None):
    """``pdattn_stream_read``: the streaming-read bandwidth reference."""
    _check(_lib.pdattn_stream_read(_ptr(buffer), buffer.numel() * buffer.element_size(), _ptr(sink),
                                   int(num_cus), _stream(stream)), "pdattn_stream_read")


def stream_read_sink(num_cus, device):
    return torch.empty(int(_lib.pdattn_stream_read_sink_words(int(num_cus))), dtype=torch.int32, device=device)


def kv_append(k_new, v_new, token_seq, token_pos, block_table, k_pages, v_pages, k_scale=None, v_scale=None,
              *, batch=None, pow2_scales=False, layout=LAYOUT_NHD, stream=None):
    """``pdattn_kv_append``: write new K/V rows into the pools in place.

    k_new/v_new: bf16 [N,Hkv,d]; token_seq/token_pos: int32 [N]; block_table
    int32 [B,max_pages]; k_pages/v_pages: bf16 or float8_e4m3fn, [num_pages,P,Hkv,d]
    (NHD) or [num_pages,Hkv,P,d] (HND), or uint8 rows of d + 4 bytes
    (inline-scale fp8); k_scale/v_scale: fp32, one per row, for float8 pools
    (None otherwise). ``batch`` defaults to the block table's row count.
    """
    N = k_new.shape[0]
    num_pages, P, Hkv, _ = pool_dims(k_pages, layout)
    D = k_new.shape[-1]
    kv = kv_kind(k_pages)
    B = block_table.shape[0] if batch is None else batch
    prob = Problem(B, Hkv, Hkv, D, P, block_table.shape[1], num_pages, kv, 0.0, layout, 1)
    flags = APPEND_POW2_SCALES if pow2_scales else 0
    _check(_lib.pdattn_kv_append(ctypes.byref(prob), int(N), _ptr(k_new), _ptr(v_new), _ptr(token_seq),
                                 _ptr(token_pos), _ptr(block_table), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                 _ptr(v_scale), flags, _stream(stream)), "pdattn_kv_append")


def merge(partial_out, partial_lse, out=None, lse=None, stream=None):
    """``pdattn_merge``: partial_out fp32 [S, ..., d], partial_lse fp32 [S, ...]
    (the same leading shape); returns (out [..., d], lse [...])."""
    S, d = partial_out.shape[0], partial_out.shape[-1]
    rows = partial_lse[0].numel() if S > 0 else 0
    if out is None:
        out = torch.empty(partial_out.shape[1:], dtype=torch.float32, device=partial_out.device)
    if lse is None:
        lse = torch.empty(partial_lse.shape[1:], dtype=torch.float32, device=partial_lse.device)
    _check(_lib.pdattn_merge(int(S), int(rows), int(d), _ptr(partial_out), _ptr(partial_lse), _ptr(out), _ptr(lse),
                             _stream(stream)), "pdattn_merge")
    return out, lse


def fp8_conversion_check(device, stream=None) -> int:
    """``pdattn_fp8_conversion_check``: mismatches of the hardware e4m3fn
    conversion against the format definition over every |y| <= 448."""
    out = torch.zeros(1, dtype=torch.int64, device=device)
    _check(_lib.pdattn_fp8_conversion_check(_ptr(out), _stream(stream)), "pdattn_fp8_conversion_check")
    return int(out.item())


def paged_decode(q, k_pages, v_pages, block_table, context_lens, *, context_lens_host=None,
                 k_scale=None, v_scale=None, scale=None, num_cus=0, force_workers=0,
                 balanced=False, return_lse=True, layout=LAYOUT_NHD):
    """Plan, allocate (torch) and run one decode step; returns (out, lse).

    q: bf16 [B,Hq,d], or [B,n,Hq,d] for multi-query decode (n query rows per
    sequence, the last n positions of its context; outputs then [B,n,Hq,d]
    and [B,n,Hq]); k_pages/v_pages: bf16 or float8_e4m3fn, [num_pages,P,Hkv,d]
    (NHD) or [num_pages,Hkv,P,d] (HND), or uint8 with rows of d + 4 bytes
    (inline-scale fp8: the codes, then the row's fp32 scale; k_scale and
    v_scale None); block_table int32 [B,max_pages]; context_lens int32 [B]
    on the device.
    """
    n = q.shape[1] if q.dim() == 4 else 1
    B, Hq, D = q.shape[0], q.shape[-2], q.shape[-1]
    num_pages, P, Hkv, _ = pool_dims(k_pages, layout)
    if context_lens_host is None:
        context_lens_host = context_lens.cpu()
    kv = kv_kind(k_pages)
    pl = plan(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
              max_pages_per_seq=block_table.shape[1], num_pages=num_pages, kv_dtype=kv,
              scale=0.0 if scale is None else scale, context_lens_host=context_lens_host,
              num_cus=num_cus, force_workers=force_workers, balanced=balanced, kv_layout=layout, q_len=n)
    dev = q.device
    lead = (B, n) if q.dim() == 4 else (B,)
    out = torch.empty(lead + (Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty(lead + (Hq,), dtype=torch.float32, device=dev) if return_lse else None
    ws = workspace(pl, dev)
    decode(pl, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, ws, out, lse)
    reduce(pl, ws, out, lse)
    return out, lse


def _prefill_problem(q, k_pages, block_table, layout, scale):
    Hq, D = q.shape[1], q.shape[2]
    num_pages, P, Hkv, _ = pool_dims(k_pages, layout)
    kv = kv_kind(k_pages)
    return Problem(block_table.shape[0], Hq, Hkv, D, P, block_table.shape[1], num_pages, kv,
                   0.0 if scale is None else float(scale), layout, 1)


def prefill_rows_per_tile(problem: Problem) -> int:
    """``pdattn_prefill_rows_per_tile``."""
    rows = ctypes.c_int32(0)
    _check(_lib.pdattn_prefill_rows_per_tile(ctypes.byref(problem), ctypes.byref(rows)),
           "pdattn_prefill_rows_per_tile")
    return int(rows.value)


def prefill_tiles(qo_indptr_host, rows_per_tile, *, context_lens_host=None, causal=True, longest_first=True):
    """``pdattn_prefill_tiles`` on host int32 arrays; returns (tile_batch,
    tile_index) as CPU int32 tensors."""
    ptr = torch.as_tensor(qo_indptr_host, dtype=torch.int32).contiguous().cpu()
    B = ptr.numel() - 1
    lens = None if context_lens_host is None else torch.as_tensor(context_lens_host, dtype=torch.int32).contiguous().cpu()
    flags = TILES_LONGEST_FIRST if longest_first else 0
    count = ctypes.c_int32(0)
    _check(_lib.pdattn_prefill_tiles(_ptr(ptr), _ptr(lens), B, int(rows_per_tile), int(bool(causal)), flags, None,
                                     None, 0, ctypes.byref(count)), "pdattn_prefill_tiles")
    tb = torch.empty(max(count.value, 1), dtype=torch.int32)
    ti = torch.empty(max(count.value, 1), dtype=torch.int32)
    _check(_lib.pdattn_prefill_tiles(_ptr(ptr), _ptr(lens), B, int(rows_per_tile), int(bool(causal)), flags,
                                     _ptr(tb), _ptr(ti), tb.numel(), ctypes.byref(count)), "pdattn_prefill_tiles")
    return tb[:count.value], ti[:count.value]


def prefill(problem: Problem, q, qo_indptr, tile_batch, tile_index, k_pages, v_pages, k_scale, v_scale, block_table,
            context_lens, out, lse=None, *, causal=True, stream=None):
    """``pdattn_prefill``: every tensor on the device, the tile map from
    ``prefill_tiles`` with ``prefill_rows_per_tile(problem)`` rows."""
    _check(_lib.pdattn_prefill(ctypes.byref(problem), int(bool(causal)), _ptr(q), _ptr(qo_indptr), _ptr(tile_batch),
                               _ptr(tile_index), int(tile_batch.numel()), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                               _ptr(v_scale), _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse),
                               _stream(stream)), "pdattn_prefill")


class SplitTiles:
    """``pdattn_prefill_split_tiles``'s outputs: CPU int32 tile_batch,
    tile_index [num_tiles] and tile_kv [num_tiles, 4], the workspace slots
    and bytes."""

    def __init__(self, tile_batch, tile_index, tile_kv, num_slots, workspace_bytes):
        self.tile_batch, self.tile_index, self.tile_kv = tile_batch, tile_index, tile_kv
        self.num_slots, self.workspace_bytes = int(num_slots), int(workspace_bytes)

    @property
    def num_tiles(self):
        return int(self.tile_batch.numel())


def prefill_split_tiles(problem: Problem, qo_indptr_host, context_lens_host, *, causal=True, slots=0) -> SplitTiles:
    """``pdattn_prefill_split_tiles`` on host int32 arrays (slots 0: the
    current device's resident prefill workgroups)."""
    ptr = torch.as_tensor(qo_indptr_host, dtype=torch.int32).contiguous().cpu()
    lens = torch.as_tensor(context_lens_host, dtype=torch.int32).contiguous().cpu()
    nt, ns, wb = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_uint64(0)
    args = (ctypes.byref(problem), _ptr(ptr), _ptr(lens), int(bool(causal)), int(slots))
    counts = (ctypes.byref(nt), ctypes.byref(ns), ctypes.byref(wb))
    _check(_lib.pdattn_prefill_split_tiles(*args, None, None, None, 0, *counts), "pdattn_prefill_split_tiles")
    cap = max(nt.value, 1)
    tb = torch.empty(cap, dtype=torch.int32)
    ti = torch.empty(cap, dtype=torch.int32)
    tk = torch.empty(cap, 4, dtype=torch.int32)
    _check(_lib.pdattn_prefill_split_tiles(*args, _ptr(tb), _ptr(ti), _ptr(tk), cap, *counts),
           "pdattn_prefill_split_tiles")
    n = nt.value
    return SplitTiles(tb[:n], ti[:n], tk[:n], ns.value, wb.value)


def prefill_split(problem: Problem, q, qo_indptr, tile_batch, tile_index, tile_kv, num_slots, workspace, k_pages,
                  v_pages, k_scale, v_scale, block_table, context_lens, out, lse=None, *, causal=True, stream=None):
    """``pdattn_prefill_split``: every tensor on the device; the map from
    ``prefill_split_tiles``; workspace a zero-initialised uint8 tensor of at
    least its workspace_bytes (None when num_slots is 0)."""
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pdattn_prefill_split(ctypes.byref(problem), int(bool(causal)), _ptr(q), _ptr(qo_indptr),
                                     _ptr(tile_batch), _ptr(tile_index), _ptr(tile_kv), int(tile_batch.numel()),
                                     int(num_slots), _ptr(workspace), wbytes, _ptr(k_pages), _ptr(v_pages),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(context_lens), _ptr(out),
                                     _ptr(lse), _stream(stream)), "pdattn_prefill_split")


def prefill_split_workspace(tiles: SplitTiles, device):
    """A zeroed workspace for ``prefill_split`` (None when nothing is split)."""
    if tiles.num_slots == 0:
        return None
    return torch.zeros(tiles.workspace_bytes, dtype=torch.uint8, device=device)


def paged_prefill(q, qo_indptr, k_pages, v_pages, block_table, context_lens, *, qo_indptr_host=None,
                  context_lens_host=None, k_scale=None, v_scale=None, scale=None, causal=True, layout=LAYOUT_NHD,
                  longest_first=True, return_lse=True, split=False, slots=0):
    """Build the tile map, allocate (torch) and run one prefill; returns
    (out fp32 [total_q, Hq, d], lse fp32 [total_q, Hq]).

    q: bf16 [total_q, Hq, d] packed by qo_indptr (int32 [B + 1], device);
    pools, block_table and context_lens as for ``paged_decode`` (device).
    split: the split-KV map and kernel (slots as for
    ``prefill_split_tiles``)."""
    prob = _prefill_problem(q, k_pages, block_table, layout, scale)
    ptr_h = qo_indptr.cpu() if qo_indptr_host is None else qo_indptr_host
    lens_h = context_lens.cpu() if context_lens_host is None else context_lens_host
    dev = q.device
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev) if return_lse else None
    if split:
        st = prefill_split_tiles(prob, ptr_h, lens_h, causal=causal, slots=slots)
        ws = prefill_split_workspace(st, dev)
        prefill_split(prob, q, qo_indptr, st.tile_batch.to(dev), st.tile_index.to(dev), st.tile_kv.to(dev),
                      st.num_slots, ws, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, out, lse,
                      causal=causal)
        return out, lse
    tb, ti = prefill_tiles(ptr_h, prefill_rows_per_tile(prob), context_lens_host=lens_h, causal=causal,
                           longest_first=longest_first)
    prefill(prob, q, qo_indptr, tb.to(dev), ti.to(dev), k_pages, v_pages, k_scale, v_scale, block_table,
            context_lens, out, lse, causal=causal)
    return out, lse


# ---- TQ4 compressed cache ---------------------------------------------------

KV_TQ4 = 3


class Tq4Plan(ctypes.Structure):
    """Mirror of ``pdattn_tq4_plan_t``."""
    _fields_ = [
        ("problem", Problem),
        ("num_cus", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("chunk_tiles", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32),
        ("total_tiles", ctypes.c_int64),
        ("max_context_len", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
        ("magic", ctypes.c_uint32),
        ("reserved1", ctypes.c_uint32),
    ]


_lib.pdattn_tq4_codebook.restype = ctypes.c_int
_lib.pdattn_tq4_codebook.argtypes = [ctypes.c_int32, _P, _P]
_lib.pdattn_tq4_append.restype = ctypes.c_int
_lib.pdattn_tq4_append.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.pdattn_tq4_plan.restype = ctypes.c_int
_lib.pdattn_tq4_plan.argtypes = [ctypes.POINTER(Problem), _P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Tq4Plan)]
_lib.pdattn_tq4_decode.restype = ctypes.c_int
_lib.pdattn_tq4_decode.argtypes = [ctypes.POINTER(Tq4Plan), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, _P, _P,
                                   _P]
_lib.pdattn_tq4_decode_rotated.restype = ctypes.c_int
_lib.pdattn_tq4_decode_rotated.argtypes = [ctypes.POINTER(Tq4Plan), _P, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, _P,
                                           _P, _P]
_lib.pdattn_tq4_plan_size.restype = ctypes.c_uint64
if _lib.pdattn_tq4_plan_size() != ctypes.sizeof(Tq4Plan):
    raise ImportError("libpdattn.so TQ4 plan layout does not match the binding")
__all__ += ["KV_TQ4", "Tq4Plan", "tq4_codebook", "tq4_problem", "tq4_append", "tq4_plan", "tq4_decode",
            "tq4_decode_rotated", "paged_decode_tq4"]


def tq4_codebook(head_dim):
    """pdattn_tq4_codebook: (centroids float32 [16], boundaries float32 [15])
    CPU tensors."""
    c = torch.empty(16, dtype=torch.float32)
    b = torch.empty(15, dtype=torch.float32)
    _check(_lib.pdattn_tq4_codebook(int(head_dim), _ptr(c), _ptr(b)), "pdattn_tq4_codebook")
    return c, b


def tq4_problem(q_or_heads, cache, block_table, scale=0.0):
    """The pdattn_problem of a TQ4 cache uint8 [num_pages, Hkv, P, d + 8] and
    q [B, Hq, d] (or (B, Hq) for an append, which needs no q)."""
    if cache.dtype != torch.uint8 or cache.dim() != 4:
        raise ValueError("a TQ4 cache is uint8 [num_pages, Hkv, P, d + 8]")
    num_pages, Hkv, P, rb = cache.shape
    B, Hq = (q_or_heads.shape[0], q_or_heads.shape[1]) if isinstance(q_or_heads, torch.Tensor) else q_or_heads
    return Problem(int(B), int(Hq), int(Hkv), int(rb - 8), int(P), int(block_table.shape[1]), int(num_pages), KV_TQ4,
                   float(scale), LAYOUT_HND, 1)


def tq4_append(k_new, v_new, token_seq, token_pos, block_table, rotation, k_boundaries, v_boundaries, cache,
               num_q_heads=None, stream=None):
    """pdattn_tq4_append: compress k_new / v_new (bf16 [T, Hkv, d]) into the
    cache rows their (sequence, position) name. All tensors on the device."""
    Hkv = cache.shape[1]
    prob = tq4_problem((block_table.shape[0], num_q_heads or Hkv), cache, block_table)
    for t in (k_new, v_new, rotation, cache, token_seq, token_pos, block_table, k_boundaries, v_boundaries):
        if not t.is_contiguous():
            raise ValueError("tq4_append takes contiguous tensors")
    _check(_lib.pdattn_tq4_append(ctypes.byref(prob), int(k_new.shape[0]), _ptr(k_new), _ptr(v_new), _ptr(token_seq),
                                  _ptr(token_pos), _ptr(block_table), _ptr(rotation), _ptr(k_boundaries),
                                  _ptr(v_boundaries), _ptr(cache), _stream(stream)), "pdattn_tq4_append")


def tq4_plan(problem, context_lens_host, num_cus=0, chunk_tiles=0):
    """pdattn_tq4_plan; context_lens_host: CPU int32 [B]."""
    lens = context_lens_host.to(torch.int32).contiguous()
    pl = Tq4Plan()
    _check(_lib.pdattn_tq4_plan(ctypes.byref(problem), _ptr(lens), int(num_cus), int(chunk_tiles), ctypes.byref(pl)),
           "pdattn_tq4_plan")
    return pl


def tq4_decode(pl, q, cache, rotation, k_centroids, v_centroids, block_table, context_lens, ws, out, lse,
               stream=None):
    """pdattn_tq4_decode with caller-owned workspace and outputs."""
    _check(_lib.pdattn_tq4_decode(ctypes.byref(pl), _ptr(q), _ptr(cache), _ptr(rotation), _ptr(k_centroids),
                                  _ptr(v_centroids), _ptr(block_table), _ptr(context_lens), _ptr(ws),
                                  int(ws.numel()), _ptr(out), _ptr(lse), _stream(stream)), "pdattn_tq4_decode")


def tq4_decode_rotated(pl, q_rot, cache, k_centroids, v_centroids, block_table, context_lens, ws, out, lse,
                       stream=None):
    """pdattn_tq4_decode_rotated: q_rot fp16 [B, Hq, d] (R q, natural order);
    out fp32 [B, Hq, d] stays in the rotated space. Caller-owned workspace
    and outputs."""
    if q_rot.dtype != torch.float16 or not q_rot.is_contiguous():
        raise ValueError("q_rot must be contiguous fp16")
    _check(_lib.pdattn_tq4_decode_rotated(ctypes.byref(pl), _ptr(q_rot), _ptr(cache), _ptr(k_centroids),
                                          _ptr(v_centroids), _ptr(block_table), _ptr(context_lens), _ptr(ws),
                                          int(ws.numel()), _ptr(out), _ptr(lse), _stream(stream)),
           "pdattn_tq4_decode_rotated")


def paged_decode_tq4(q, cache, block_table, context_lens, rotation, k_centroids, v_centroids, *,
                     context_lens_host=None, scale=0.0, chunk_tiles=0, stream=None):
    """Plan, allocate and run one TQ4 decode step; returns (out fp32
    [B, Hq, d], lse fp32 [B, Hq]) in model space."""
    lens_host = context_lens.cpu() if context_lens_host is None else context_lens_host
    prob = tq4_problem(q, cache, block_table, scale)
    pl = tq4_plan(prob, lens_host, chunk_tiles=chunk_tiles)
    ws = torch.empty(max(int(pl.workspace_bytes), 16), dtype=torch.uint8, device=q.device)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    tq4_decode(pl, q, cache, rotation, k_centroids, v_centroids, block_table, context_lens, ws, out, lse, stream)
    return out, lse
