"""Python binding of the quantized KV-cache library (``libkvq.so``, C ABI in ``include/kvq.h``): 2-bit KIVI-style
caches and the 4-bit KVQuant-style variant (optional pre-RoPE keys and attention-sink token).

Argument marshalling only: every step of quantization, window management and attention runs in the library's HIP
kernels. PyTorch provides device memory and the current HIP stream. The library must be built
(``python -m decode_attention_quant_amd.build`` or ``__graft_entry__.build()``); importing this package without it
raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loaded first so the library binds to the HIP runtime torch already uses

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

OK = 0
E_NULL, E_SHAPE, E_BITS, E_ALIGN, E_CAPACITY, E_WORKSPACE, E_EMPTY, E_LAUNCH, E_STATE, E_SCRATCH = range(-1, -11, -1)
HEAD_DIM = 128
GROUP = 32
TILE_TOKENS = 32
RECORD_BYTES = 3072
RECORD_BYTES_SPARSE = 3840
RECORD_BYTES_4BIT = 5120
RECORD_BYTES_4BIT_SPARSE = 5888
SINK_BYTES = 512
NOALLOC_SCRATCH_BYTES = 16 << 20
FLAG_SINK = 1
FLAG_PRE_ROPE = 2
FLAG_SPARSE = 4


class KvqShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("residual_cap", ctypes.c_int32), ("flags", ctypes.c_int32), ("max_tokens", ctypes.c_int64),
                ("rope_base", ctypes.c_double)]


class KvqCache(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
                ("n_quant", ctypes.c_int64), ("n_resid", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("sink", ctypes.c_void_p)]


class KvqRagged(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
                ("sink", ctypes.c_void_p), ("lens", ctypes.c_void_p), ("sync", ctypes.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m decode_attention_quant_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    SP, CP, RP = ctypes.POINTER(KvqShape), ctypes.POINTER(KvqCache), ctypes.POINTER(KvqRagged)
    sigs = {
        "kv_quant_keys_per_channel": (ctypes.c_int, [SP, P, I64, I64, I64, I64, I64, P, P]),
        "kv_quant_values_per_token": (ctypes.c_int, [SP, P, I64, I64, I64, I64, I64, P, P]),
        "kv_append_and_flush": (ctypes.c_int, [SP, CP, P, P, I64, I64, I64, I64, P]),
        "kv_decode_attention_splits": (I32, [SP, CP]),
        "kv_decode_attention_workspace_bytes": (ctypes.c_size_t, [SP, CP]),
        "kv_decode_attention": (ctypes.c_int, [SP, CP, P, F, P, P, ctypes.c_size_t, P]),
        "kv_decode_attention_noalloc": (ctypes.c_int, [SP, CP, P, F, P, P]),
        "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kv_ragged_prefill": (ctypes.c_int, [SP, RP, I32, P, P, I64, I64, I64, P]),
        "kv_ragged_append": (ctypes.c_int, [SP, RP, P, P, I64, I64, P]),
        "kv_ragged_splits": (I32, [SP]),
        "kv_ragged_workspace_bytes": (ctypes.c_size_t, [SP]),
        "kv_ragged_sync_words": (ctypes.c_size_t, [SP]),
        "kv_ragged_decode_attention": (ctypes.c_int, [SP, RP, P, F, P, P, ctypes.c_size_t, P]),
        "kv_ragged_decode_step": (ctypes.c_int, [SP, RP, P, P, I64, I64, P, F, P, P, ctypes.c_size_t, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTS = ("kv_quant_keys_per_channel", "kv_quant_values_per_token", "kv_append_and_flush",
           "kv_decode_attention_splits", "kv_decode_attention_workspace_bytes", "kv_decode_attention",
           "kv_decode_attention_noalloc",
           "kvq_status_string", "kv_ragged_prefill", "kv_ragged_append", "kv_ragged_splits",
           "kv_ragged_workspace_bytes", "kv_ragged_sync_words", "kv_ragged_decode_attention",
           "kv_ragged_decode_step")


def library():
    """The loaded ``ctypes.CDLL`` (for tests that call the C ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.kvq_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise KvqError(fn, status)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _f16_4d(t: torch.Tensor, name: str, batch: int | None = None, heads: int | None = None):
    """[B, H, T, 128] float16 with unit channel stride -> (pointer, stride_b, stride_h, stride_t). The leading sizes
    must equal (batch, heads) when given: the library addresses every (batch row, head) slice of the cache's shape,
    so a smaller tensor would be read past its end."""
    if t.dtype != torch.float16 or t.dim() != 4 or t.shape[-1] != HEAD_DIM or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a float16 tensor [B, H, T, 128] with unit channel stride")
    if batch is not None and (t.shape[0], t.shape[1]) != (batch, heads):
        raise ValueError(f"{name} has leading sizes {tuple(t.shape[:2])}; the cache shape needs ({batch}, {heads})")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0), t.stride(1), t.stride(2)


def _sized_bytes(t: torch.Tensor, name: str, need: int):
    """A contiguous tensor of at least `need` bytes (any element type)."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < need:
        raise ValueError(f"{name} holds {have} bytes; {need} are needed")


def _same_cuda_device(device, **tensors):
    """Every tensor is a CUDA tensor on `device` (checked after the sizes, so size errors name the size)."""
    for name, t in tensors.items():
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a CUDA tensor on the cache's device ({device})")


def _tiles_bytes(shape) -> int:
    return shape.batch * shape.kv_heads * (shape.max_tokens // TILE_TOKENS) * shape.record_bytes


def _check_out(out: torch.Tensor, shape):
    """The fp32 output [B, Hq, 128], contiguous."""
    if out.dtype != torch.float32 or tuple(out.shape) != (shape.batch, shape.q_heads, HEAD_DIM) \
            or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 tensor [{shape.batch}, {shape.q_heads}, {HEAD_DIM}]")


def _check_q(q: torch.Tensor, shape):
    if q.dtype != torch.float16 or tuple(q.shape) != (shape.batch, shape.q_heads, HEAD_DIM) \
            or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous float16 tensor [{shape.batch}, {shape.q_heads}, {HEAD_DIM}]")


@dataclass
class Shape:
    batch: int
    kv_heads: int
    q_heads: int
    max_tokens: int
    residual_cap: int = 128
    bits: int = 2
    head_dim: int = HEAD_DIM
    group: int = GROUP
    flags: int = 0              # FLAG_SINK | FLAG_PRE_ROPE | FLAG_SPARSE (2-bit: FLAG_SPARSE only)
    rope_base: float = 0.0      # rotary base when FLAG_PRE_ROPE is set

    @property
    def record_bytes(self) -> int:
        if self.bits != 4:
            return RECORD_BYTES_SPARSE if self.flags & FLAG_SPARSE else RECORD_BYTES
        return RECORD_BYTES_4BIT_SPARSE if self.flags & FLAG_SPARSE else RECORD_BYTES_4BIT

    def c(self) -> KvqShape:
        return KvqShape(self.batch, self.kv_heads, self.q_heads, self.head_dim, self.bits, self.group,
                        self.residual_cap, self.flags, self.max_tokens, float(self.rope_base))


class KVCache:
    """Device buffers of one cache (allocated through torch) and the C struct that describes them."""

    def __init__(self, shape: Shape, device="cuda"):
        self.shape = shape
        self._cshape = shape.c()
        tiles = shape.max_tokens // TILE_TOKENS
        self.tiles = torch.zeros((shape.batch, shape.kv_heads, tiles, shape.record_bytes), dtype=torch.uint8,
                                 device=device)
        self.k_res = torch.zeros((shape.batch, shape.kv_heads, shape.residual_cap, HEAD_DIM), dtype=torch.float16,
                                 device=device)
        self.v_res = torch.zeros_like(self.k_res)
        self.sink = None
        if shape.flags & FLAG_SINK:
            self.sink = torch.zeros((shape.batch, shape.kv_heads, SINK_BYTES), dtype=torch.uint8, device=device)
        self.c = KvqCache(self.tiles.data_ptr(), self.k_res.data_ptr(), self.v_res.data_ptr(), 0, 0, 0,
                          self.sink.data_ptr() if self.sink is not None else None)

    @property
    def n_quant(self) -> int:
        return int(self.c.n_quant)

    @property
    def n_resid(self) -> int:
        return int(self.c.n_resid)

    @property
    def n_sink(self) -> int:
        return int(self.c.n_sink)

    @property
    def n_tokens(self) -> int:
        return self.n_sink + self.n_quant + self.n_resid


def _quant(fn: str, shape: Shape, x: torch.Tensor, name: str, tile0: int, tiles: torch.Tensor, stream):
    p, sb, sh, st = _f16_4d(x, name, shape.batch, shape.kv_heads)
    if tiles.dtype != torch.uint8:
        raise ValueError("tiles must be a uint8 tensor [B, Hkv, max_tokens / 32, record bytes]")
    _sized_bytes(tiles, "tiles", _tiles_bytes(shape))
    _same_cuda_device(tiles.device, **{name: x, "tiles": tiles})
    cs = shape.c()
    _check(fn, getattr(_lib, fn)(ctypes.byref(cs), p, sb, sh, st, x.shape[2], tile0,
                                 ctypes.c_void_p(tiles.data_ptr()), _stream(stream)))


def kv_quant_keys_per_channel(shape: Shape, k: torch.Tensor, tile0: int, tiles: torch.Tensor, stream=None):
    _quant("kv_quant_keys_per_channel", shape, k, "k", tile0, tiles, stream)


def kv_quant_values_per_token(shape: Shape, v: torch.Tensor, tile0: int, tiles: torch.Tensor, stream=None):
    _quant("kv_quant_values_per_token", shape, v, "v", tile0, tiles, stream)


def kv_append_and_flush(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
    s = cache.shape
    pk, sb, sh, st = _f16_4d(k_new, "k_new", s.batch, s.kv_heads)
    pv, sb2, sh2, st2 = _f16_4d(v_new, "v_new", s.batch, s.kv_heads)
    if (sb, sh, st) != (sb2, sh2, st2) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape and strides")
    _same_cuda_device(cache.tiles.device, k_new=k_new, v_new=v_new)
    _check("kv_append_and_flush", _lib.kv_append_and_flush(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), pk, pv, sb, sh, st, k_new.shape[2], _stream(stream)))


def kv_decode_attention_splits(cache: KVCache) -> int:
    return int(_lib.kv_decode_attention_splits(ctypes.byref(cache._cshape), ctypes.byref(cache.c)))


def kv_decode_attention_workspace_bytes(cache: KVCache) -> int:
    return int(_lib.kv_decode_attention_workspace_bytes(ctypes.byref(cache._cshape), ctypes.byref(cache.c)))


def kv_decode_attention(cache: KVCache, q: torch.Tensor, out: torch.Tensor | None = None, sm_scale: float = 0.0,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    s = cache.shape
    _check_q(q, s)
    if out is None:
        out = torch.empty((s.batch, s.q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check_out(out, s)
    need = kv_decode_attention_workspace_bytes(cache)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _sized_bytes(workspace, "workspace", need)
    _same_cuda_device(cache.tiles.device, q=q, out=out, workspace=workspace)
    _check("kv_decode_attention", _lib.kv_decode_attention(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), ctypes.c_void_p(q.data_ptr()), float(sm_scale),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kv_decode_attention_noalloc(cache: KVCache, q: torch.Tensor, out: torch.Tensor, sm_scale: float = 0.0,
                                stream=None) -> torch.Tensor:
    """kv_decode_attention with the split partials in the library's static per-GPU scratch (no workspace, no
    allocation by the library; ``out`` is the caller's). Calls that overlap on one GPU race (one stream, in order)."""
    s = cache.shape
    _check_q(q, s)
    _check_out(out, s)
    _same_cuda_device(cache.tiles.device, q=q, out=out)
    _check("kv_decode_attention_noalloc", _lib.kv_decode_attention_noalloc(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), ctypes.c_void_p(q.data_ptr()), float(sm_scale),
        ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out


# ---------------------------------------------------------------------------------------------------- ragged caches
class RaggedCache:
    """A 2-bit cache whose sequences sit at their own lengths, held on the device in ``lens`` (int32 [B, 4]:
    n_quant, n_resid, n_sink, status); every call enqueues fixed arguments, so decode steps can be graph-captured."""

    def __init__(self, shape: Shape, device="cuda"):
        if shape.bits != 2 or shape.flags:
            raise ValueError("ragged caches are 2-bit without flags")
        self.shape = shape
        self._cshape = shape.c()
        tiles = shape.max_tokens // TILE_TOKENS
        self.tiles = torch.zeros((shape.batch, shape.kv_heads, tiles, RECORD_BYTES), dtype=torch.uint8, device=device)
        self.k_res = torch.zeros((shape.batch, shape.kv_heads, shape.residual_cap, HEAD_DIM), dtype=torch.float16,
                                 device=device)
        self.v_res = torch.zeros_like(self.k_res)
        self.lens = torch.zeros((shape.batch, 4), dtype=torch.int32, device=device)
        # completion counters of the single-launch decode step (zero, and left zero by every step)
        self.sync = torch.zeros(library().kv_ragged_sync_words(ctypes.byref(self._cshape)), dtype=torch.int32,
                                device=device)
        self.c = KvqRagged(self.tiles.data_ptr(), self.k_res.data_ptr(), self.v_res.data_ptr(), None,
                           self.lens.data_ptr(), self.sync.data_ptr())

    def lengths(self):
        """Host copy of the per-sequence (n_quant, n_resid, n_sink, status) rows (synchronizes)."""
        return self.lens.cpu().tolist()


def _f16_tokens(t: torch.Tensor, name: str, shape=None, device=None):
    """One token per (sequence, KV head): [B, Hkv, 128] or [B, Hkv, 1, 128] -> (pointer, stride_b, stride_h)."""
    if t.dim() == 4:
        if t.shape[2] != 1:
            raise ValueError(f"{name}: one token per sequence")
        t = t[:, :, 0]
    if t.dtype != torch.float16 or t.dim() != 3 or t.shape[-1] != HEAD_DIM or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a float16 tensor [B, Hkv, 128] with unit channel stride")
    if shape is not None and (t.shape[0], t.shape[1]) != (shape.batch, shape.kv_heads):
        raise ValueError(f"{name} has leading sizes {tuple(t.shape[:2])}; the cache shape needs "
                         f"({shape.batch}, {shape.kv_heads})")
    if device is not None:
        _same_cuda_device(device, **{name: t})
    return ctypes.c_void_p(t.data_ptr()), t.stride(0), t.stride(1)


def kv_ragged_prefill(cache: RaggedCache, b: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    """Replace sequence b with the tokens of k, v ([Hkv, T, 128], unit channel stride)."""
    for t, nm in ((k, "k"), (v, "v")):
        if t.dtype != torch.float16 or t.dim() != 3 or t.shape[-1] != HEAD_DIM or \
                (t.numel() and t.stride(-1) != 1):
            raise ValueError(f"{nm} must be a float16 tensor [Hkv, T, 128] with unit channel stride")
        if t.shape[0] != cache.shape.kv_heads:
            raise ValueError(f"{nm} holds {t.shape[0]} KV heads; the cache has {cache.shape.kv_heads}")
    if not 0 <= int(b) < cache.shape.batch:
        raise ValueError(f"sequence index {b} outside [0, {cache.shape.batch})")
    _same_cuda_device(cache.tiles.device, k=k, v=v)
    if k.shape != v.shape or (k.numel() and k.stride() != v.stride()):
        raise ValueError("k and v must have the same shape and strides")
    n = k.shape[1]
    sh, st = (k.stride(0), k.stride(1)) if n else (0, 0)   # no token: nothing is read
    _check("kv_ragged_prefill", _lib.kv_ragged_prefill(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), int(b), ctypes.c_void_p(k.data_ptr() if n else None),
        ctypes.c_void_p(v.data_ptr() if n else None), sh, st, n, _stream(stream)))


def kv_ragged_append(cache: RaggedCache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
    pk, sb, sh = _f16_tokens(k_new, "k_new", cache.shape, cache.tiles.device)
    pv, sb2, sh2 = _f16_tokens(v_new, "v_new", cache.shape, cache.tiles.device)
    if (sb, sh) != (sb2, sh2):
        raise ValueError("k_new and v_new must have the same strides")
    _check("kv_ragged_append", _lib.kv_ragged_append(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), pk, pv, sb, sh, _stream(stream)))


def kv_ragged_workspace_bytes(cache: RaggedCache) -> int:
    return int(_lib.kv_ragged_workspace_bytes(ctypes.byref(cache._cshape)))


def kv_ragged_splits(cache: RaggedCache) -> int:
    return int(_lib.kv_ragged_splits(ctypes.byref(cache._cshape)))


def _ragged_io(cache, q, out, workspace):
    s = cache.shape
    _check_q(q, s)
    if out is None:
        out = torch.empty((s.batch, s.q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check_out(out, s)
    need = kv_ragged_workspace_bytes(cache)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _sized_bytes(workspace, "workspace", need)
    _same_cuda_device(cache.tiles.device, q=q, out=out, workspace=workspace)
    return out, workspace


def kv_ragged_decode_attention(cache: RaggedCache, q: torch.Tensor, out: torch.Tensor | None = None,
                               sm_scale: float = 0.0, workspace: torch.Tensor | None = None, stream=None):
    out, workspace = _ragged_io(cache, q, out, workspace)
    _check("kv_ragged_decode_attention", _lib.kv_ragged_decode_attention(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), ctypes.c_void_p(q.data_ptr()), float(sm_scale),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kv_ragged_decode_step(cache: RaggedCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                          out: torch.Tensor | None = None, sm_scale: float = 0.0,
                          workspace: torch.Tensor | None = None, stream=None):
    """Append one token per sequence, then attend: one launch that flushes full windows, attends, merges the splits,
    writes the new window rows and commits the lengths (no host state: graph-capturable). Needs the cache's
    ``sync`` counters (zero before and after every launch)."""
    pk, sb, sh = _f16_tokens(k_new, "k_new", cache.shape)
    pv, sb2, sh2 = _f16_tokens(v_new, "v_new", cache.shape)
    if (sb, sh) != (sb2, sh2):
        raise ValueError("k_new and v_new must have the same strides")
    out, workspace = _ragged_io(cache, q, out, workspace)
    _same_cuda_device(cache.tiles.device, k_new=k_new, v_new=v_new)
    _check("kv_ragged_decode_step", _lib.kv_ragged_decode_step(
        ctypes.byref(cache._cshape), ctypes.byref(cache.c), pk, pv, sb, sh, ctypes.c_void_p(q.data_ptr()),
        float(sm_scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out
