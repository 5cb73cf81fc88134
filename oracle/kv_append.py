"""TEST INFRASTRUCTURE ONLY: CPU oracle of the KV append (the write of new
tokens' K/V rows into the paged cache), with the FP8 quantise-and-scatter.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py`` may use this
module; it shares no code with the HIP library.

What it computes (plain numpy, one token and kv head at a time):
  * the slot of new token i: page = block_table[seq_i][pos_i >> log2 P],
    slot = pos_i mod P (FlashQuant wiki "CUDA Kernels", paged_decode.cu, Page
    Table Addressing); a token whose sequence, position or page does not
    resolve inside the tables is skipped;
  * a bf16 pool receives the row unchanged (Atlas "CUDA Kernel Engineering",
    kernel inventory: per-token K/V write into the paged cache);
  * an fp8 pool receives float8_e4m3fn codes and one fp32 scale per (token,
    kv head), separately for K and V (OASR "Kernel Layer", FP8 KV variants:
    the quantise-and-scatter that writes the cache). Readings where the pages
    are silent:
      - plain scales: scale = absmax(row) / 448 in fp32 (a correctly rounded
        fp32 division; 1 for an all-zero row);
      - power-of-two scales (the variant those pages ship, so that products
        with the scale are exact): the smallest power of two s with
        448 * s >= absmax(row) (1 for an all-zero row);
      - code = the E4M3FN value nearest to y = x / scale (fp32 division,
        correctly rounded), y first clamped to [-448, 448]; a tie goes to the
        code whose last mantissa bit is 0 (round to nearest even). Both
        decisions are taken in fp32, as the kernel takes them.
The E4M3FN values come from the format definition (1 sign, 4 exponent bits
with bias 7, 3 mantissa bits; exponent 0 subnormal; 0x7F / 0xFF NaN).
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3fn_value_table() -> np.ndarray:
    """Values of the 128 non-negative codes 0x00..0x7F (0x7F: NaN), fp64."""
    vals = np.empty(128, np.float64)
    for c in range(128):
        e, m = c >> 3, c & 7
        vals[c] = np.ldexp(m, -9) if e == 0 else np.ldexp(8 + m, e - 10)
    vals[0x7F] = np.nan
    return vals


_VALS = e4m3fn_value_table()
_FINITE = _VALS[:0x7F]  # increasing: 0, 2^-9, ..., 448


def encode_e4m3fn(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of each fp32 y in [-448, 448], ties to even."""
    y = np.asarray(y, np.float32)
    a = np.abs(y).astype(np.float64)
    hi = np.clip(np.searchsorted(_FINITE, a, side="left"), 0, len(_FINITE) - 1)
    lo = np.clip(hi - 1, 0, len(_FINITE) - 1)
    dlo = np.abs(a - _FINITE[lo])
    dhi = np.abs(_FINITE[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    sign = np.signbit(y).astype(np.int64) << 7
    return (pick | sign).astype(np.uint8)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    v = _VALS[codes & 0x7F]
    return np.where(codes & 0x80, -v, v)


def row_scale(row: np.ndarray, pow2: bool) -> np.float32:
    """The fp32 scale of one row (float32 values)."""
    amax = np.float32(np.max(np.abs(row))) if row.size else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    if not pow2:
        return np.float32(amax / np.float32(E4M3_MAX))
    e = int(np.ceil(np.log2(float(amax) / E4M3_MAX)))
    # the smallest e with 448 * 2^e >= amax, checked exactly
    while E4M3_MAX * 2.0 ** (e - 1) >= float(amax):
        e -= 1
    while E4M3_MAX * 2.0 ** e < float(amax):
        e += 1
    return np.float32(2.0 ** e)


def quantize_row(row: np.ndarray, pow2: bool):
    """(codes uint8, scale fp32) of one K or V row (float32 values)."""
    s = row_scale(row, pow2)
    y = np.clip(row.astype(np.float32) / s, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3fn(y), s


def kv_append(k_pages, v_pages, k_scale, v_scale, k_new, v_new, token_seq, token_pos, block_table, *,
              pow2=False):
    """Write new rows into copies of the pools; returns the new pools.

    k_pages / v_pages: numpy [num_pages, P, Hkv, d], float32 holding bf16
    values (bf16 pool) or uint8 codes (fp8 pool); k_scale / v_scale: float32
    [num_pages, P, Hkv] for fp8 pools, else None. k_new / v_new: float32
    [N, Hkv, d] (bf16 values). token_seq / token_pos: int [N]; block_table:
    int [B, max_pages].
    """
    fp8 = k_scale is not None
    kp, vp = k_pages.copy(), v_pages.copy()
    ks = k_scale.copy() if fp8 else None
    vs = v_scale.copy() if fp8 else None
    num_pages, P, Hkv, _ = kp.shape
    B, maxp = block_table.shape
    for i in range(len(token_seq)):
        b, t = int(token_seq[i]), int(token_pos[i])
        if not (0 <= b < B and 0 <= t < maxp * P):
            continue
        page = int(block_table[b][t // P])
        if not 0 <= page < num_pages:
            continue
        slot = t % P
        for h in range(Hkv):
            if fp8:
                kp[page, slot, h], ks[page, slot, h] = quantize_row(k_new[i, h], pow2)
                vp[page, slot, h], vs[page, slot, h] = quantize_row(v_new[i, h], pow2)
            else:
                kp[page, slot, h] = k_new[i, h]
                vp[page, slot, h] = v_new[i, h]
    return kp, vp, ks, vs
