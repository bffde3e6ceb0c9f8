"""Seeded synthetic inputs for block-causal chunk attention.

This module only draws numbers: it holds none of the attention arithmetic and
is shared by the tests, the smoke check and the benchmark so that the GPU path
and the CPU oracle consume exactly the same values.

Generator (counter based, so any tensor of any chunk, layer and denoise step
can be regenerated on its own):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): ``mix(z)`` is its output function and the k-th
  draw of a stream with key ``s`` is ``mix(s + (k + 1) * GAMMA)``.
* A stream key is derived from the base seed and a tuple of integer ids
  (tensor tag, layer, chunk, step, ...) by folding each id into the key with
  ``mix``.
* Uniforms take the top 53 bits: ``u = (x >> 11) * 2**-53`` in [0, 1).
* Normal deviates by Box–Muller (cosine branch only): draw 2i gives ``u1``,
  draw 2i+1 gives ``u2``, ``z_i = sqrt(-2 ln(1 - u1)) * cos(2 pi u2)``.

Storage rounding (how a double becomes a tensor element): to fp32 by IEEE
round to nearest even, then, for bf16, fp32 -> bf16 by round to nearest even
on the bit pattern. Values are returned as float32 arrays holding the rounded
numbers, plus the raw uint16 bf16 bit patterns where asked.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
BASE_SEED = 20261202

# tensor tags folded into stream keys
TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_OUTLIER = 4
TAG_MISC = 5


def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _mix_arr(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(0xBF58476D1CE4E5B9)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def stream_key(*ids: int, seed: int = BASE_SEED) -> int:
    """Key of the stream named by ``ids`` (any number of non-negative ints)."""
    s = _mix_int(seed)
    for i in ids:
        s = _mix_int(s ^ ((int(i) + 0x632BE59BD9B4E019) & MASK64))
    return s


def raw_u64(key: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of stream ``key`` as uint64."""
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + k * np.uint64(GAMMA)
        return _mix_arr(z)


def uniform(key: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` uniforms in [0, 1) (float64) from draws start.. of stream ``key``."""
    x = raw_u64(key, start, count)
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, count: int) -> np.ndarray:
    """``count`` N(0, 1) deviates in float64 (Box–Muller, cosine branch)."""
    u = uniform(key, 2 * count)
    u1 = u[0::2]
    u2 = u[1::2]
    return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)


def round_fp32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x32)
    r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64/32 -> values representable in bf16 (returned as float32)."""
    return bf16_to_f32(bf16_bits(round_fp32(x)))


def tensor(shape, *ids: int, dtype: str = "bf16", scale: float = 1.0,
           outlier_frac: float = 0.0, outlier_sigma: float = 8.0,
           seed: int = BASE_SEED) -> np.ndarray:
    """A seeded N(0, 1) tensor (times ``scale``) rounded to ``dtype``.

    ``outlier_frac`` > 0 replaces each element independently, with that
    probability (a uniform from a second stream below the fraction), by
    ``outlier_sigma * sign(z)`` where z is the element's own N(0, 1) draw.
    Returns float32 holding the rounded values ("fp32" or "bf16").
    """
    count = int(np.prod(shape))
    key = stream_key(*ids, seed=seed)
    z = normal(key, count)
    if outlier_frac > 0.0:
        ukey = stream_key(TAG_OUTLIER, *ids, seed=seed)
        pick = uniform(ukey, count) < outlier_frac
        z = np.where(pick, outlier_sigma * np.sign(z), z)
    z = z * scale
    if dtype == "fp32":
        out = round_fp32(z)
    elif dtype == "bf16":
        out = round_bf16(z)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out.reshape(shape)


def tensor_rows(shape, rows, *ids: int, dtype: str = "bf16", seed: int = BASE_SEED) -> np.ndarray:
    """Rows ``rows`` (indices along the first axis) of ``tensor(shape, *ids)``
    without outliers, drawing only their counters: row r of a [R][...] tensor
    holds elements r*m .. r*m + m - 1 (m = product of the other axes), i.e.
    uniform draws 2 r m .. 2 (r + 1) m - 1 of the stream."""
    m = int(np.prod(shape[1:]))
    key = stream_key(*ids, seed=seed)
    out = np.empty((len(rows),) + tuple(shape[1:]), dtype=np.float32)
    for i, r in enumerate(rows):
        u = uniform(key, 2 * m, start=2 * int(r) * m)
        z = np.sqrt(-2.0 * np.log1p(-u[0::2])) * np.cos(2.0 * np.pi * u[1::2])
        x = round_fp32(z) if dtype == "fp32" else round_bf16(z)
        out[i] = x.reshape(shape[1:])
    return out


def qkv(n: int, H: int, d: int, layer: int, chunk: int, step: int, dtype: str = "bf16",
        outlier_frac: float = 0.0, seed: int = BASE_SEED):
    """Q, K, V of one chunk of one layer at one denoise step, each [n][H][d].

    K and V are what the chunk contributes as keys; a committed chunk's cache
    content is its K and V at the committed step. Outliers (if any) apply to K
    and V only.
    """
    q = tensor((n, H, d), TAG_Q, layer, chunk, step, dtype=dtype, seed=seed)
    k = tensor((n, H, d), TAG_K, layer, chunk, step, dtype=dtype,
               outlier_frac=outlier_frac, seed=seed)
    v = tensor((n, H, d), TAG_V, layer, chunk, step, dtype=dtype,
               outlier_frac=outlier_frac, seed=seed)
    return q, k, v
