"""Shared helpers of the GPU tests: seeded chunk sequences driven through the
C ABI, and the oracle run on the same rounded inputs."""
from __future__ import annotations

import math
import sys
import time

import numpy as np

import oracle
import synth

TOL = {"fp32": 1e-5, "bf16": 1e-2, "fp8": 5e-2, "fp8_block": 5e-2, "int8k_block": 5e-2}

# caches fed bf16 inputs
BF16_IN = ("bf16", "fp8", "fp8_block", "int8k_block")

# An 8-bit cache against the oracle run on what the cache holds (the kernel's
# own error): 1e-2 plus the bf16 rounding of the output, 2^-9 relative for O
# itself and 2^-9 more for a split piece's bf16-free but fp32-normalised
# partial; rows dominated by an 8-sigma value have |O| up to 8.
FP8_CACHE_ABS = 1e-2
FP8_CACHE_REL = 2.0 ** -8


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype in BF16_IN else t
    return t.cuda()


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


_E4M3 = None


def e4m3_table():
    """Value of every e4m3 code, from the oracle's decoder."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    return _E4M3


def fp8_stored(x, scales):
    """What an fp8 cache holds for x [n][H][d] (bf16 values), dequantised:
    decode(quant(x / s_h)) * s_h per head, with the oracle's quantiser."""
    tab = e4m3_table()
    out = np.empty(x.shape, dtype=np.float64)
    for h in range(x.shape[1]):
        out[:, h, :] = tab[oracle.quant_e4m3(x[:, h, :], scales[h])] * scales[h]
    return out


def int8_stored(x, scales):
    """What an int8 K block holds for x [n][H][d], dequantised: the oracle's
    int8 code times s_h per head."""
    out = np.empty(x.shape, dtype=np.float64)
    for h in range(x.shape[1]):
        out[:, h, :] = oracle.quant_int8(x[:, h, :], float(scales[h])).astype(np.float64) * \
            float(scales[h])
    return out


def block_stored(kind, k, v):
    """(K, V) as a per-block cache holds them: scales from the oracle's rule
    (K over 127 for int8 K, else 448; V over 448)."""
    if kind == "int8k_block":
        return (int8_stored(k, oracle.block_scales(k, qmax=127.0)),
                fp8_stored(v, oracle.block_scales(v)))
    return fp8_stored(k, oracle.block_scales(k)), fp8_stored(v, oracle.block_scales(v))


class Sequence:
    """Drives one cache layer through chunk steps and keeps the committed
    history the oracle needs (every chunk appended, keyed by id). With an fp8
    cache and `scales` = (k_scale[H], v_scale[H]) set, `history`/`ref` hold
    what the cache stores (dequantised) and `history_raw`/`ref_raw` the
    appended values themselves."""

    def __init__(self, cache, H, d, n, dtype, seed_layer=0, outlier_frac=0.0, scales=None):
        self.cache = cache
        self.H, self.d, self.n = H, d, n
        self.dtype = dtype  # "fp32" | "bf16" | "fp8" (bf16 inputs, fp8 cache)
        self.in_dtype = "fp32" if dtype == "fp32" else "bf16"
        self.seed_layer = seed_layer
        self.outlier_frac = outlier_frac
        self.scales = scales
        self.history = {}
        self.history_raw = {}
        self.ref = None
        self.ref_raw = None
        if scales is not None:
            cache.set_kv_scales(0, scales[0], scales[1])

    def chunk(self, t, step=0):
        return synth.qkv(self.n, self.H, self.d, self.seed_layer, t, step, dtype=self.in_dtype,
                         outlier_frac=self.outlier_frac)

    def stored(self, k, v):
        if self.dtype in ("fp8_block", "int8k_block"):
            return block_stored(self.dtype, k, v)
        if self.dtype == "fp8" and self.scales is not None:
            return fp8_stored(k, self.scales[0]), fp8_stored(v, self.scales[1])
        return k.astype(np.float64), v.astype(np.float64)

    def append(self, layer, t, k, v, is_ref=False):
        self.cache.append_chunk(layer, t, to_dev(k, self.dtype), to_dev(v, self.dtype),
                                is_ref=is_ref)
        raw = (k.astype(np.float64), v.astype(np.float64))
        if is_ref:
            self.ref, self.ref_raw = self.stored(k, v), raw
        else:
            self.history[t], self.history_raw[t] = self.stored(k, v), raw

    def attend(self, layer, t, q, k, v, W, use_ref=False, G=0, scale=None):
        spec = self.cache.spec(t, W, use_ref=use_ref, num_segments=G, scale=scale)
        o, lse = self.cache.attend(layer, to_dev(q, self.dtype), to_dev(k, self.dtype),
                                   to_dev(v, self.dtype), spec)
        return to_np(o), to_np(lse), spec

    def expected(self, t, q, k, v, W, use_ref=False, scale=None, history=None, raw=False):
        """The oracle on the same inputs. With an fp8 cache the chunk attends to
        cache-precision keys and values, its own included (the kernel
        quantises the current chunk as appending it would); raw=True uses the
        unquantised values instead."""
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if raw:
            hist = self.history_raw if history is None else history
            return oracle.attend(q, k, v, hist, t=t, W=W, scale=scale, ref=self.ref_raw,
                                 use_ref=use_ref)
        hist = self.history if history is None else history
        kk, vv = self.stored(k, v)
        return oracle.attend(q, kk, vv, hist, t=t, W=W, scale=scale, ref=self.ref,
                             use_ref=use_ref)


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"shape {a.shape} != {b.shape}")
    both_nan = np.isnan(a) & np.isnan(b)
    d = np.where(both_nan, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0


def assert_close(got_o, got_lse, exp_o, exp_lse, tol, what=""):
    eo, el = max_err(got_o, exp_o), max_err(got_lse, exp_lse)
    if what is not None:
        log(f"{what}: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e} (tol {tol})")
    assert eo <= tol and el <= tol, f"{what}: O err {eo}, LSE err {el} > {tol}"


def assert_fp8(seq, o, lse, t, q, k, v, W, use_ref=False, raw_tol=None, what="", history=None):
    """An 8-bit cache result against the oracle twice: on what the cache holds
    (the kernel's own error, FP8_CACHE_ABS + FP8_CACHE_REL |O|, LSE 1e-2), and
    on the unquantised seeded inputs. The second bar is raw_tol when given
    (5e-2, the bar for 8-bit K/V); otherwise it is the quantisation's own error (the
    oracle on the cache contents against the oracle on the raw inputs) plus the
    kernel's bar, i.e. what the first check already implies: e4m3 keeps 3
    mantissa bits, and on a few hundred keys a row dominated by one key
    inherits that key's rounding."""
    eo, el = seq.expected(t, q, k, v, W, use_ref=use_ref, history=history)
    ro, rl = seq.expected(t, q, k, v, W, use_ref=use_ref, raw=True,
                          history=None if history is None else {c: seq.history_raw[c] for c in history})
    d_cache_o = np.abs(np.asarray(o, np.float64) - eo)
    lim = FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo)
    ec, elc = max_err(o, eo), max_err(lse, el)
    quant_o, quant_l = max_err(eo, ro), max_err(el, rl)
    eraw, elraw = max_err(o, ro), max_err(lse, rl)
    bar = raw_tol if raw_tol is not None else None
    log(f"{what}: vs stored values max|dO| {ec:.3e} max|dLSE| {elc:.3e}; vs raw inputs "
        f"max|dO| {eraw:.3e} max|dLSE| {elraw:.3e}; quantisation alone {quant_o:.3e} / {quant_l:.3e}"
        f" (raw bar {'%.0e' % bar if bar is not None else 'quantisation + kernel bar'})")
    assert np.all(np.nan_to_num(d_cache_o, nan=np.inf) <= lim), f"{what}: O vs stored {ec}"
    assert elc <= FP8_CACHE_ABS, f"{what}: LSE vs stored {elc}"
    if raw_tol is not None:
        assert eraw <= raw_tol and elraw <= raw_tol, f"{what}: vs raw O {eraw}, LSE {elraw} > {raw_tol}"
    else:
        assert eraw <= quant_o + FP8_CACHE_ABS + FP8_CACHE_REL * float(np.abs(eo).max()), \
            f"{what}: vs raw O {eraw} beyond quantisation {quant_o} + kernel bar"
        assert elraw <= quant_l + FP8_CACHE_ABS, f"{what}: vs raw LSE {elraw}"
    return eraw, elraw
