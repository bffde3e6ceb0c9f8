"""ctypes wrapper of the C oracle in ``bca_oracle.c`` (test infrastructure).

Every function takes and returns numpy arrays in double precision (float32
for the e4m3 quantiser's input, as the quantiser decides codes in single
precision). The arithmetic is all in the C file; this wrapper only converts
layouts and pointers. ``OracleLib(path)`` wraps any build of that file (the
tests also build deliberately broken copies to show the pins catch them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "bca_oracle.c")
LIB_PATH = os.path.join(_HERE, "libbca_oracle.so")


def compile_oracle(src: str, out: str) -> str:
    """gcc -O2, OpenMP, no fast-math: ``src`` -> shared library ``out``."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-fopenmp", "-shared", "-fPIC", src, "-o", tmp,
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB_PATH):
        compile_oracle(SRC_PATH, LIB_PATH)
    return LIB_PATH


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleLib:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.bca_oracle_attend_masked.argtypes = [ctypes.c_int] * 4 + [P, P, P, P,
                                                                      ctypes.c_double,
                                                                      ctypes.c_int, P, P]
        lib.bca_oracle_attend_masked.restype = ctypes.c_int
        lib.bca_oracle_attend.argtypes = ([ctypes.c_int] * 4 +
                                          [P, P, P, ctypes.c_int, P, P, P, P, P,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, ctypes.c_int, P, P])
        lib.bca_oracle_attend.restype = ctypes.c_int
        lib.bca_oracle_attend_rows.argtypes = ([ctypes.c_int] * 5 +
                                               [P, P, P, ctypes.c_int, P, P, P, P, P,
                                                ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_double, ctypes.c_int, P, P])
        lib.bca_oracle_attend_rows.restype = ctypes.c_int
        lib.bca_oracle_lse_merge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P,
                                             P, P]
        lib.bca_oracle_lse_merge.restype = ctypes.c_int
        lib.bca_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.bca_oracle_e4m3_decode.restype = ctypes.c_double
        lib.bca_oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.bca_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.bca_oracle_quant_e4m3.argtypes = [P, ctypes.c_long, ctypes.c_float, P]
        lib.bca_oracle_quant_e4m3.restype = None
        lib.bca_oracle_block_scales.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_float, P]
        lib.bca_oracle_block_scales.restype = None
        lib.bca_oracle_quant_int8.argtypes = [P, ctypes.c_long, ctypes.c_float, P]
        lib.bca_oracle_quant_int8.restype = None
        lib.bca_oracle_threads.argtypes = []
        lib.bca_oracle_threads.restype = ctypes.c_int
        lib.bca_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.bca_oracle_set_threads.restype = None
        lib.bca_oracle_rope.argtypes = [ctypes.c_int] * 3 + [P, ctypes.c_int64, ctypes.c_double, P]
        lib.bca_oracle_rope.restype = ctypes.c_int
        lib.bca_oracle_attend_sequence.argtypes = [ctypes.c_int] * 6 + [P, P, P, ctypes.c_double,
                                                                         P, P]
        lib.bca_oracle_attend_sequence.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def threads(self) -> int:
        return self.lib.bca_oracle_threads()

    def set_threads(self, n: int) -> None:
        self.lib.bca_oracle_set_threads(int(n))

    def attend_masked(self, q, k, v, mask, scale: float, literal: bool = False):
        """Attention with an explicit mask shared by all heads.

        q [nq][H][d], k and v [nk][H][d], mask [nq][nk] (bool/0-1).
        Returns (o [nq][H][d], lse [H][nq]) in float64.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        nq, H, d = q.shape
        nk = k.shape[0]
        assert k.shape == (nk, H, d) and v.shape == (nk, H, d)
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        assert m.shape == (nq, nk)
        o = np.empty((nq, H, d), dtype=np.float64)
        lse = np.empty((H, nq), dtype=np.float64)
        rc = self.lib.bca_oracle_attend_masked(nq, nk, H, d, _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(m), float(scale), int(bool(literal)),
                                               _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"bca_oracle_attend_masked failed ({rc})")
        return o, lse

    def attend(self, q, k_cur, v_cur, history: dict, t: int, W: int, scale: float, ref=None,
               use_ref: bool = False, literal: bool = False, rows=None):
        """Block-causal attention of query chunk ``t``.

        history: {chunk_id: (k, v)} with every committed chunk (k, v [n][H][d]);
        ref: (k, v) of the reference chunk or None. Returns (o [n][H][d], lse [H][n]);
        with ``rows`` (indices into the chunk's n query rows) only those rows:
        (o [len(rows)][H][d], lse [H][len(rows)]).
        """
        q, k_cur, v_cur = _f64(q), _f64(k_cur), _f64(v_cur)
        n, H, d = k_cur.shape
        if rows is not None:
            q = np.ascontiguousarray(q[np.asarray(rows)])
        nq = q.shape[0]
        assert q.shape[1:] == (H, d)
        ids = sorted(history.keys())
        nh = len(ids)
        hid = np.array(ids, dtype=np.int64) if nh else np.zeros(1, dtype=np.int64)
        if nh:
            hk = _f64(np.stack([history[i][0] for i in ids]))
            hv = _f64(np.stack([history[i][1] for i in ids]))
        else:
            hk = np.zeros(1, dtype=np.float64)
            hv = np.zeros(1, dtype=np.float64)
        has_ref = ref is not None
        rk = _f64(ref[0]) if has_ref else np.zeros(1, dtype=np.float64)
        rv = _f64(ref[1]) if has_ref else np.zeros(1, dtype=np.float64)
        o = np.empty((nq, H, d), dtype=np.float64)
        lse = np.empty((H, nq), dtype=np.float64)
        rc = self.lib.bca_oracle_attend_rows(H, d, n, nq, nh, _ptr(hid), _ptr(hk), _ptr(hv),
                                             int(has_ref), _ptr(rk), _ptr(rv), _ptr(q),
                                             _ptr(k_cur), _ptr(v_cur), int(t), int(W),
                                             int(bool(use_ref)), float(scale),
                                             int(bool(literal)), _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"bca_oracle_attend failed ({rc})")
        return o, lse

    def lse_merge(self, o_parts, lse_parts):
        """o_parts [G][rows][d], lse_parts [G][rows] -> (o [rows][d], lse [rows])."""
        op, lp = _f64(o_parts), _f64(lse_parts)
        G, rows, d = op.shape
        assert lp.shape == (G, rows)
        o = np.empty((rows, d), dtype=np.float64)
        lse = np.empty((rows,), dtype=np.float64)
        rc = self.lib.bca_oracle_lse_merge(G, rows, d, _ptr(op), _ptr(lp), _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"bca_oracle_lse_merge failed ({rc})")
        return o, lse

    def e4m3_decode(self, codes) -> np.ndarray:
        c = np.asarray(codes, dtype=np.uint8)
        flat = [self.lib.bca_oracle_e4m3_decode(int(x)) for x in c.reshape(-1)]
        return np.array(flat, dtype=np.float64).reshape(c.shape)

    def e4m3_encode(self, x) -> np.ndarray:
        a = np.asarray(x, dtype=np.float32)
        flat = [self.lib.bca_oracle_e4m3_encode(float(v)) for v in a.reshape(-1)]
        return np.array(flat, dtype=np.uint8).reshape(a.shape)

    def attend_sequence(self, q, k, v, n: int, W: int, prefix: int, scale: float):
        """Training-form block-causal attention over a whole sequence: q
        [C*n][H][d], k and v [prefix + C*n][H][d]. Returns (o [C*n][H][d],
        lse [C][H][n]) in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        nq, H, d = q.shape
        assert nq % n == 0
        C = nq // n
        assert k.shape == (prefix + nq, H, d) and v.shape == k.shape
        o = np.empty((nq, H, d), dtype=np.float64)
        lse = np.empty((H, nq), dtype=np.float64)
        rc = self.lib.bca_oracle_attend_sequence(C, n, H, d, int(prefix), int(W), _ptr(q),
                                                 _ptr(k), _ptr(v), float(scale), _ptr(o),
                                                 _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"bca_oracle_attend_sequence failed ({rc})")
        return o, np.ascontiguousarray(lse.reshape(H, C, n).transpose(1, 0, 2))

    def rope(self, x, pos0: int, base: float) -> np.ndarray:
        """Rotary position embedding of x [n][H][d]; token r at position pos0 + r."""
        a = _f64(x)
        n, H, d = a.shape
        y = np.empty_like(a)
        rc = self.lib.bca_oracle_rope(n, H, d, _ptr(a), int(pos0), float(base), _ptr(y))
        if rc != 0:
            raise RuntimeError(f"bca_oracle_rope failed ({rc})")
        return y

    def quant_e4m3(self, x, scale: float) -> np.ndarray:
        """codes = encode(fp32(x / scale)) for a float32 array."""
        a = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.bca_oracle_quant_e4m3(_ptr(a), a.size, float(scale), _ptr(out))
        return out

    def block_scales(self, x, qmax: float = 448.0) -> np.ndarray:
        """Per-head scales of a cache block x [n][H][d]: fp32 max |x| / qmax
        (1 when the maximum is 0 or not finite), float32 [H]."""
        a = np.ascontiguousarray(x, dtype=np.float32)
        n, H, d = a.shape
        out = np.empty(H, dtype=np.float32)
        self.lib.bca_oracle_block_scales(_ptr(a), n, H, d, float(qmax), _ptr(out))
        return out

    def quant_int8(self, x, scale: float) -> np.ndarray:
        """int8 codes clamp(rne(fp32(x / scale)), -127, 127) for a float32 array."""
        a = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.int8)
        self.lib.bca_oracle_quant_int8(_ptr(a), a.size, float(scale), _ptr(out))
        return out


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = OracleLib(LIB_PATH)
    return _default


def threads():
    return default().threads()


def set_threads(n):
    return default().set_threads(n)


def attend_masked(*a, **k):
    return default().attend_masked(*a, **k)


def attend(*a, **k):
    return default().attend(*a, **k)


def lse_merge(*a, **k):
    return default().lse_merge(*a, **k)


def e4m3_decode(*a, **k):
    return default().e4m3_decode(*a, **k)


def e4m3_encode(*a, **k):
    return default().e4m3_encode(*a, **k)


def rope(*a, **k):
    return default().rope(*a, **k)


def attend_sequence(*a, **k):
    return default().attend_sequence(*a, **k)


def quant_e4m3(*a, **k):
    return default().quant_e4m3(*a, **k)


def block_scales(*a, **k):
    return default().block_scales(*a, **k)


def quant_int8(*a, **k):
    return default().quant_int8(*a, **k)
