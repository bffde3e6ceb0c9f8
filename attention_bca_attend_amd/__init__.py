"""Python binding of libbca.so (include/bca.h): block-causal ring-KV chunk attention.

Every computation runs in the library's HIP kernels; this module only
marshals arguments. The functions named ``bca_*`` mirror the C entry points
one to one and take raw device pointers (ints) and stream handles.
``Cache`` is a small convenience wrapper that uses torch for device memory
and the current stream.

The library must have been built (``python attention_bca_attend_amd/build.py``
or ``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "F32", "BF16", "FP8_E4M3", "FP8_E4M3_BLOCK", "INT8K_FP8V_BLOCK", "BcaError", "bca_cache_desc", "bca_window_spec",
    "bca_plan_info", "bca_cache_bytes", "bca_cache_create", "bca_cache_destroy",
    "bca_cache_set_kv_scales", "bca_append_chunk", "bca_attend_workspace_bytes", "bca_attend",
    "bca_append_chunk_rope", "bca_attend_rope_workspace_bytes", "bca_attend_rope",
    "bca_cache_slot_chunk", "bca_cache_set_slot_chunk", "bca_attend_plan", "bca_status_string",
    "bca_last_error", "bca_sequence_spec", "bca_attend_sequence_workspace_bytes",
    "bca_attend_sequence", "attend_sequence", "bca_append_chunk_dev",
    "bca_chunk_counter_advance", "bca_attend_replayable", "bca_attend_dev", "bca_attend_noalloc",
    "NOALLOC_SCRATCH_BYTES", "Cache", "LIB_PATH", "load_library",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbca.so")

F32, BF16, FP8_E4M3, FP8_E4M3_BLOCK, INT8K_FP8V_BLOCK = 0, 1, 2, 3, 4
BCA_OK = 0
STATUS = {0: "BCA_OK", -1: "BCA_ERR_INVALID_ARG", -2: "BCA_ERR_OUT_OF_ORDER",
          -3: "BCA_ERR_WORKSPACE", -4: "BCA_ERR_UNSUPPORTED", -5: "BCA_ERR_HIP"}


class bca_cache_desc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("ring_slots", ctypes.c_int32), ("has_ref", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


class bca_window_spec(ctypes.Structure):
    _fields_ = [("q_chunk_id", ctypes.c_int64), ("history", ctypes.c_int32),
                ("use_ref", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class bca_sequence_spec(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("prefix_tokens", ctypes.c_int32), ("history", ctypes.c_int32),
                ("num_segments", ctypes.c_int32), ("scale", ctypes.c_float)]


class bca_plan_info(ctypes.Structure):
    _fields_ = [("num_visible_blocks", ctypes.c_int32),
                ("visible_blocks", ctypes.c_int32 * 64),
                ("visible_chunk_ids", ctypes.c_int64 * 64),
                ("visible_keys", ctypes.c_int32), ("q_tiles", ctypes.c_int32),
                ("kv_tiles", ctypes.c_int32), ("units", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("max_pieces", ctypes.c_int32),
                ("merge", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class BcaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libbca.so once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          f"'python attention_bca_attend_amd/build.py'")
    # torch ships its own build of the HIP runtime under the same soname
    # (libamdhip64.so.7) as the system one libbca.so is linked against. Loading
    # torch first makes libbca bind to the runtime already in the process;
    # loaded the other way round the process would hold two HIP and two HSA
    # runtimes driving one GPU, and torch's first device copy crashes.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    desc_p = ctypes.POINTER(bca_cache_desc)
    spec_p = ctypes.POINTER(bca_window_spec)
    lib.bca_cache_bytes.argtypes = [desc_p]
    lib.bca_cache_bytes.restype = SZ
    lib.bca_cache_create.argtypes = [desc_p, P, SZ, ctypes.POINTER(P)]
    lib.bca_cache_create.restype = I32
    lib.bca_cache_destroy.argtypes = [P]
    lib.bca_cache_destroy.restype = I32
    lib.bca_cache_set_kv_scales.argtypes = [P, I32, P, P]
    lib.bca_cache_set_kv_scales.restype = I32
    lib.bca_append_chunk.argtypes = [P, I32, I64, I32, P, P, I32, P]
    lib.bca_append_chunk.restype = I32
    lib.bca_attend_workspace_bytes.argtypes = [P, spec_p]
    lib.bca_attend_workspace_bytes.restype = SZ
    lib.bca_attend.argtypes = [P, I32, spec_p, P, P, P, I32, P, P, P, SZ, P]
    lib.bca_attend.restype = I32
    D64 = ctypes.c_double
    lib.bca_append_chunk_rope.argtypes = [P, I32, I64, I32, P, P, I32, D64, I64, P]
    lib.bca_append_chunk_rope.restype = I32
    lib.bca_attend_rope_workspace_bytes.argtypes = [P, spec_p]
    lib.bca_attend_rope_workspace_bytes.restype = SZ
    lib.bca_attend_rope.argtypes = [P, I32, spec_p, P, P, P, I32, D64, I64, P, P, P, SZ, P]
    lib.bca_attend_rope.restype = I32
    seq_p = ctypes.POINTER(bca_sequence_spec)
    lib.bca_attend_sequence_workspace_bytes.argtypes = [seq_p, I32]
    lib.bca_attend_sequence_workspace_bytes.restype = SZ
    lib.bca_attend_sequence.argtypes = [seq_p, P, P, P, I32, P, P, P, SZ, P]
    lib.bca_attend_sequence.restype = I32
    lib.bca_append_chunk_dev.argtypes = [P, I32, P, P, P, I32, P]
    lib.bca_append_chunk_dev.restype = I32
    lib.bca_chunk_counter_advance.argtypes = [P, P]
    lib.bca_chunk_counter_advance.restype = I32
    lib.bca_attend_replayable.argtypes = [P, I32, spec_p, ctypes.POINTER(I32)]
    lib.bca_attend_replayable.restype = I32
    lib.bca_attend_dev.argtypes = [P, I32, spec_p, P, P, P, P, I32, P, P, P, SZ, P]
    lib.bca_attend_dev.restype = I32
    lib.bca_attend_noalloc.argtypes = [P, I32, spec_p, P, P, P, I32, P, P, P]
    lib.bca_attend_noalloc.restype = I32
    lib.bca_cache_slot_chunk.argtypes = [P, I32, I32, ctypes.POINTER(I64)]
    lib.bca_cache_slot_chunk.restype = I32
    lib.bca_cache_set_slot_chunk.argtypes = [P, I32, I32, I64]
    lib.bca_cache_set_slot_chunk.restype = I32
    lib.bca_attend_plan.argtypes = [P, I32, spec_p, ctypes.POINTER(bca_plan_info)]
    lib.bca_attend_plan.restype = I32
    lib.bca_status_string.argtypes = [I32]
    lib.bca_status_string.restype = ctypes.c_char_p
    lib.bca_last_error.argtypes = []
    lib.bca_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


load_library()


def _check(status: int) -> None:
    if status != BCA_OK:
        raise BcaError(status, _lib.bca_last_error().decode())


def _desc(d) -> bca_cache_desc:
    if isinstance(d, bca_cache_desc):
        return d
    return bca_cache_desc(**d)


def _spec(s) -> bca_window_spec:
    if isinstance(s, bca_window_spec):
        return s
    return bca_window_spec(**s)


def bca_status_string(status: int) -> str:
    return _lib.bca_status_string(status).decode()


def bca_last_error() -> str:
    return _lib.bca_last_error().decode()


def bca_cache_bytes(desc) -> int:
    return int(_lib.bca_cache_bytes(ctypes.byref(_desc(desc))))


def bca_cache_create(desc, dev_mem: int, nbytes: int) -> int:
    out = ctypes.c_void_p()
    _check(_lib.bca_cache_create(ctypes.byref(_desc(desc)), ctypes.c_void_p(dev_mem), nbytes,
                                 ctypes.byref(out)))
    return out.value


def bca_cache_destroy(handle: int) -> None:
    _check(_lib.bca_cache_destroy(ctypes.c_void_p(handle)))


def bca_cache_set_kv_scales(handle: int, layer: int, k_scale, v_scale) -> None:
    ks = (ctypes.c_float * len(k_scale))(*[float(x) for x in k_scale])
    vs = (ctypes.c_float * len(v_scale))(*[float(x) for x in v_scale])
    _check(_lib.bca_cache_set_kv_scales(ctypes.c_void_p(handle), layer, ks, vs))


def bca_append_chunk(handle: int, layer: int, chunk_id: int, is_ref: int, k: int, v: int,
                     in_dtype: int, stream: int = 0) -> None:
    _check(_lib.bca_append_chunk(ctypes.c_void_p(handle), layer, chunk_id, int(is_ref),
                                 ctypes.c_void_p(k), ctypes.c_void_p(v), in_dtype,
                                 ctypes.c_void_p(stream)))


def bca_attend_workspace_bytes(handle: int, spec) -> int:
    return int(_lib.bca_attend_workspace_bytes(ctypes.c_void_p(handle),
                                               ctypes.byref(_spec(spec))))


def bca_attend(handle: int, layer: int, spec, q: int, k_cur: int, v_cur: int, qkv_dtype: int,
               o: int, lse: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.bca_attend(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                           ctypes.c_void_p(q), ctypes.c_void_p(k_cur), ctypes.c_void_p(v_cur),
                           qkv_dtype, ctypes.c_void_p(o), ctypes.c_void_p(lse),
                           ctypes.c_void_p(workspace), workspace_bytes, ctypes.c_void_p(stream)))


def bca_append_chunk_rope(handle: int, layer: int, chunk_id: int, is_ref: int, k: int, v: int,
                          in_dtype: int, rope_base: float, pos0: int, stream: int = 0) -> None:
    _check(_lib.bca_append_chunk_rope(ctypes.c_void_p(handle), layer, chunk_id, int(is_ref),
                                      ctypes.c_void_p(k), ctypes.c_void_p(v), in_dtype,
                                      float(rope_base), int(pos0), ctypes.c_void_p(stream)))


def bca_attend_rope_workspace_bytes(handle: int, spec) -> int:
    return int(_lib.bca_attend_rope_workspace_bytes(ctypes.c_void_p(handle),
                                                    ctypes.byref(_spec(spec))))


def bca_attend_rope(handle: int, layer: int, spec, q: int, k_cur: int, v_cur: int,
                    qkv_dtype: int, rope_base: float, pos0: int, o: int, lse: int,
                    workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.bca_attend_rope(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                                ctypes.c_void_p(q), ctypes.c_void_p(k_cur),
                                ctypes.c_void_p(v_cur), qkv_dtype, float(rope_base), int(pos0),
                                ctypes.c_void_p(o), ctypes.c_void_p(lse),
                                ctypes.c_void_p(workspace), workspace_bytes,
                                ctypes.c_void_p(stream)))


def bca_attend_sequence_workspace_bytes(spec: bca_sequence_spec, qkv_dtype: int) -> int:
    return int(_lib.bca_attend_sequence_workspace_bytes(ctypes.byref(spec), qkv_dtype))


def bca_attend_sequence(spec: bca_sequence_spec, q: int, k: int, v: int, qkv_dtype: int, o: int,
                        lse: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.bca_attend_sequence(ctypes.byref(spec), ctypes.c_void_p(q), ctypes.c_void_p(k),
                                    ctypes.c_void_p(v), qkv_dtype, ctypes.c_void_p(o),
                                    ctypes.c_void_p(lse), ctypes.c_void_p(workspace),
                                    workspace_bytes, ctypes.c_void_p(stream)))


def attend_sequence(q, k, v, chunk_tokens: int, history: int, prefix_tokens: int = 0,
                    num_segments: int = 0, scale: float | None = None, workspace=None,
                    stream=None):
    """Training-form block-causal attention over a whole sequence of chunks
    (bca_attend_sequence) on torch device tensors: q [C*n][H][d], k and v
    [P + C*n][H][d] (memory prefix first), fp32 or bf16, contiguous. Returns
    (o [C*n][H][d], lse [C][H][n] fp32). ``workspace``, if given, is a uint8
    device tensor of at least bca_attend_sequence_workspace_bytes() bytes,
    256-byte aligned."""
    import torch
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise BcaError(-4, "q, k, v must be float32 or bfloat16")
    for t in (q, k, v):
        if not t.is_cuda or t.dtype != q.dtype or not t.is_contiguous() or t.dim() != 3:
            raise BcaError(-1, "q, k, v must be contiguous [rows][H][d] device tensors of one dtype")
    rows_q, H, d = q.shape
    n = int(chunk_tokens)
    if n <= 0 or rows_q % n != 0:
        raise BcaError(-1, f"q rows {rows_q} are not a multiple of chunk_tokens {n}")
    C = rows_q // n
    if tuple(k.shape) != (prefix_tokens + rows_q, H, d) or k.shape != v.shape:
        raise BcaError(-1, f"k and v must have shape {(prefix_tokens + rows_q, H, d)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    spec = bca_sequence_spec(H, d, n, C, int(prefix_tokens), int(history), int(num_segments),
                             float(scale))
    dt = F32 if q.dtype == torch.float32 else BF16
    need = bca_attend_sequence_workspace_bytes(spec, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((C, H, n), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    bca_attend_sequence(spec, q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, o.data_ptr(),
                        lse.data_ptr(), workspace.data_ptr() if workspace is not None else 0,
                        workspace.numel() if workspace is not None else 0, int(stream))
    return o, lse


def bca_append_chunk_dev(handle: int, layer: int, d_chunk_id: int, k: int, v: int,
                         in_dtype: int, stream: int = 0) -> None:
    _check(_lib.bca_append_chunk_dev(ctypes.c_void_p(handle), layer, ctypes.c_void_p(d_chunk_id),
                                     ctypes.c_void_p(k), ctypes.c_void_p(v), in_dtype,
                                     ctypes.c_void_p(stream)))


def bca_chunk_counter_advance(d_chunk_id: int, stream: int = 0) -> None:
    _check(_lib.bca_chunk_counter_advance(ctypes.c_void_p(d_chunk_id), ctypes.c_void_p(stream)))


def bca_attend_replayable(handle: int, layer: int, spec) -> bool:
    out = ctypes.c_int32()
    _check(_lib.bca_attend_replayable(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                                      ctypes.byref(out)))
    return bool(out.value)


def bca_attend_dev(handle: int, layer: int, spec, d_q_chunk_id: int, q: int, k_cur: int,
                   v_cur: int, qkv_dtype: int, o: int, lse: int, workspace: int,
                   workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.bca_attend_dev(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                               ctypes.c_void_p(d_q_chunk_id), ctypes.c_void_p(q),
                               ctypes.c_void_p(k_cur), ctypes.c_void_p(v_cur), qkv_dtype,
                               ctypes.c_void_p(o), ctypes.c_void_p(lse),
                               ctypes.c_void_p(workspace), workspace_bytes,
                               ctypes.c_void_p(stream)))


# Scratch bytes per GPU behind bca_attend_noalloc (BCA_NOALLOC_SCRATCH_BYTES in bca.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def bca_attend_noalloc(handle: int, layer: int, spec, q: int, k_cur: int, v_cur: int,
                       qkv_dtype: int, o: int, lse: int, stream: int = 0) -> None:
    _check(_lib.bca_attend_noalloc(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                                   ctypes.c_void_p(q), ctypes.c_void_p(k_cur),
                                   ctypes.c_void_p(v_cur), qkv_dtype, ctypes.c_void_p(o),
                                   ctypes.c_void_p(lse), ctypes.c_void_p(stream)))


def bca_cache_slot_chunk(handle: int, layer: int, slot: int) -> int:
    out = ctypes.c_int64()
    _check(_lib.bca_cache_slot_chunk(ctypes.c_void_p(handle), layer, slot, ctypes.byref(out)))
    return out.value


def bca_cache_set_slot_chunk(handle: int, layer: int, slot: int, chunk_id: int) -> None:
    _check(_lib.bca_cache_set_slot_chunk(ctypes.c_void_p(handle), layer, slot, chunk_id))


def bca_attend_plan(handle: int, layer: int, spec) -> dict:
    info = bca_plan_info()
    _check(_lib.bca_attend_plan(ctypes.c_void_p(handle), layer, ctypes.byref(_spec(spec)),
                                ctypes.byref(info)))
    nb = info.num_visible_blocks
    return {
        "visible_blocks": list(info.visible_blocks[:nb]),
        "visible_chunk_ids": list(info.visible_chunk_ids[:nb]),
        "visible_keys": info.visible_keys, "q_tiles": info.q_tiles,
        "kv_tiles": info.kv_tiles, "units": info.units, "workgroups": info.workgroups,
        "max_pieces": info.max_pieces, "merge": bool(info.merge),
        "workspace_bytes": int(info.workspace_bytes),
    }


_DT = {"fp32": F32, "f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp8_e4m3": FP8_E4M3,
       "fp8_block": FP8_E4M3_BLOCK, "int8k_block": INT8K_FP8V_BLOCK}


class Cache:
    """A ring-buffer KV cache in torch-allocated device memory.

    Layout of ``self.mem`` (uint8): [L][K|V][H][S+R][n][d] elements of the
    cache dtype; ``blocks(layer)`` returns typed views of one layer.
    """

    def __init__(self, num_layers: int, num_heads: int, head_dim: int, chunk_tokens: int,
                 ring_slots: int, has_ref: bool = False, kv_dtype: str = "bf16",
                 device="cuda"):
        import torch
        self.desc = bca_cache_desc(num_layers, num_heads, head_dim, chunk_tokens, ring_slots,
                                   int(bool(has_ref)), _DT[kv_dtype])
        self.kv_dtype = kv_dtype
        self.qkv_dtype = "fp32" if _DT[kv_dtype] == F32 else "bf16"
        nbytes = bca_cache_bytes(self.desc)
        if nbytes == 0:
            raise BcaError(-1, "invalid cache descriptor")
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = bca_cache_create(self.desc, self.mem.data_ptr(), nbytes)
        self._ws = {}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.bca_cache_destroy(ctypes.c_void_p(h))
            self.handle = None

    # -- views ------------------------------------------------------------
    def blocks(self, layer: int):
        """(K, V) views of one layer: [H][S+R][n][d] in the cache dtype."""
        import torch
        d = self.desc
        nb = d.ring_slots + d.has_ref
        tdt = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8,
               FP8_E4M3_BLOCK: torch.uint8, INT8K_FP8V_BLOCK: torch.uint8}[d.kv_dtype]
        es = {F32: 4, BF16: 2, FP8_E4M3: 1, FP8_E4M3_BLOCK: 1, INT8K_FP8V_BLOCK: 1}[d.kv_dtype]
        half = d.num_heads * nb * d.chunk_tokens * d.head_dim * es
        base = 2 * layer * half
        k = self.mem[base:base + half].view(tdt).view(d.num_heads, nb, d.chunk_tokens, d.head_dim)
        v = self.mem[base + half:base + 2 * half].view(tdt).view(d.num_heads, nb,
                                                                   d.chunk_tokens, d.head_dim)
        return k, v

    def block_scales(self, layer: int):
        """Per-block caches (FP8_E4M3_BLOCK, INT8K_FP8V_BLOCK): (K, V) scale
        views of one layer, fp32 [S+R][H] (the table after the blocks:
        [L][K|V][S+R][H])."""
        import torch
        d = self.desc
        if d.kv_dtype not in (FP8_E4M3_BLOCK, INT8K_FP8V_BLOCK):
            raise BcaError(-1, "only per-block caches keep scales per block")
        nb = d.ring_slots + d.has_ref
        base = 2 * d.num_layers * d.num_heads * nb * d.chunk_tokens * d.head_dim
        per = nb * d.num_heads * 4
        k = self.mem[base + 2 * layer * per:base + (2 * layer + 1) * per].view(torch.float32)
        v = self.mem[base + (2 * layer + 1) * per:base + (2 * layer + 2) * per].view(torch.float32)
        return k.view(nb, d.num_heads), v.view(nb, d.num_heads)

    def slot_chunk(self, layer: int, slot: int) -> int:
        return bca_cache_slot_chunk(self.handle, layer, slot)

    def set_slot_chunk(self, layer: int, slot: int, chunk_id: int) -> None:
        bca_cache_set_slot_chunk(self.handle, layer, slot, chunk_id)

    def set_kv_scales(self, layer: int, k_scale, v_scale) -> None:
        bca_cache_set_kv_scales(self.handle, layer, list(k_scale), list(v_scale))

    # -- operations -------------------------------------------------------
    def _check_qkv(self, *ts):
        import torch
        d = self.desc
        want = torch.float32 if self.qkv_dtype == "fp32" else torch.bfloat16
        for t in ts:
            if not t.is_cuda or t.dtype != want or not t.is_contiguous():
                raise BcaError(-1, f"expected contiguous {want} device tensors")
            if tuple(t.shape) != (d.chunk_tokens, d.num_heads, d.head_dim):
                raise BcaError(-1, f"expected shape {(d.chunk_tokens, d.num_heads, d.head_dim)}, "
                                   f"got {tuple(t.shape)}")

    @staticmethod
    def _stream(stream):
        import torch
        if stream is None:
            return torch.cuda.current_stream().cuda_stream
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def append_chunk(self, layer: int, chunk_id: int, k, v, is_ref: bool = False, stream=None,
                     rope=None):
        """rope = (base, pos0): K is rotated on its way in (bca_append_chunk_rope)."""
        self._check_qkv(k, v)
        if rope is None:
            bca_append_chunk(self.handle, layer, chunk_id, int(bool(is_ref)), k.data_ptr(),
                             v.data_ptr(), _DT[self.qkv_dtype], self._stream(stream))
        else:
            bca_append_chunk_rope(self.handle, layer, chunk_id, int(bool(is_ref)), k.data_ptr(),
                                  v.data_ptr(), _DT[self.qkv_dtype], rope[0], rope[1],
                                  self._stream(stream))

    def spec(self, q_chunk_id: int, history: int, use_ref: bool = False, num_segments: int = 0,
             scale: float | None = None) -> bca_window_spec:
        if scale is None:
            scale = 1.0 / math.sqrt(self.desc.head_dim)
        return bca_window_spec(q_chunk_id, history, int(bool(use_ref)), num_segments, scale)

    def workspace(self, spec, rope: bool = False):
        import torch
        key = (spec.history, spec.num_segments, bool(rope))
        nbytes = (bca_attend_rope_workspace_bytes if rope else bca_attend_workspace_bytes)(
            self.handle, spec)
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.mem.device)
            self._ws[key] = ws
        return ws

    def plan(self, layer: int, spec) -> dict:
        return bca_attend_plan(self.handle, layer, spec)

    def replayable(self, layer: int, spec) -> bool:
        return bca_attend_replayable(self.handle, layer, spec)

    def append_chunk_dev(self, layer: int, d_chunk_id, k, v, stream=None):
        """bca_append_chunk_dev: the chunk id is read from the int64 device tensor
        d_chunk_id when the kernels run (for replayed graphs)."""
        import torch
        self._check_qkv(k, v)
        if d_chunk_id.dtype != torch.int64 or not d_chunk_id.is_cuda:
            raise BcaError(-1, "d_chunk_id must be an int64 device tensor")
        bca_append_chunk_dev(self.handle, layer, d_chunk_id.data_ptr(), k.data_ptr(),
                             v.data_ptr(), _DT[self.qkv_dtype], self._stream(stream))

    def attend_dev(self, layer: int, d_q_chunk_id, q, k_cur, v_cur, spec, out, lse, workspace,
                   stream=None):
        """bca_attend_dev: the query chunk id is read from the int64 device tensor
        d_q_chunk_id when the kernel runs; spec.q_chunk_id is the chunk the call
        is made (or captured) for."""
        import torch
        self._check_qkv(q, k_cur, v_cur)
        if d_q_chunk_id.dtype != torch.int64 or not d_q_chunk_id.is_cuda:
            raise BcaError(-1, "d_q_chunk_id must be an int64 device tensor")
        bca_attend_dev(self.handle, layer, spec, d_q_chunk_id.data_ptr(), q.data_ptr(),
                       k_cur.data_ptr(), v_cur.data_ptr(), _DT[self.qkv_dtype], out.data_ptr(),
                       lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                       self._stream(stream))

    @staticmethod
    def advance_counter(d_chunk_id, stream=None):
        """bca_chunk_counter_advance on an int64 device tensor."""
        bca_chunk_counter_advance(d_chunk_id.data_ptr(), Cache._stream(stream))

    def attend(self, layer: int, q, k_cur, v_cur, spec, out=None, lse=None, workspace=None,
               stream=None, rope=None):
        """Returns (o [n][H][d], lse [H][n] fp32). rope = (base, pos0): Q and k_cur are
        rotated first (bca_attend_rope)."""
        import torch
        self._check_qkv(q, k_cur, v_cur)
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((self.desc.num_heads, self.desc.chunk_tokens), dtype=torch.float32,
                              device=q.device)
        if workspace is None:
            workspace = self.workspace(spec, rope=rope is not None)
        if rope is None:
            bca_attend(self.handle, layer, spec, q.data_ptr(), k_cur.data_ptr(), v_cur.data_ptr(),
                       _DT[self.qkv_dtype], out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                       workspace.numel(), self._stream(stream))
        else:
            bca_attend_rope(self.handle, layer, spec, q.data_ptr(), k_cur.data_ptr(),
                            v_cur.data_ptr(), _DT[self.qkv_dtype], rope[0], rope[1],
                            out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), self._stream(stream))
        return out, lse
