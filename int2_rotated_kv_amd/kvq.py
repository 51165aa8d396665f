"""Thin ctypes binding over libkvq.so (the C ABI declared in include/kvq.h).

Argument marshalling only: torch tensors are passed as device pointers and
the current torch stream as the HIP stream.  Every step of the hot path
runs in the library's HIP kernels; there is no fallback.  Loading fails
loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = 1
KVQ_ERR_UNSUPPORTED = 2
KVQ_ERR_WORKSPACE_TOO_SMALL = 3
KVQ_ERR_HIP = 4

KVQ_F16, KVQ_F32 = 0, 1
KVQ_ROT_NONE, KVQ_ROT_HADAMARD, KVQ_ROT_DENSE, KVQ_ROT_PERM_HADAMARD = 0, 1, 2, 3
_ROT = {"none": KVQ_ROT_NONE, "hadamard": KVQ_ROT_HADAMARD, "dense": KVQ_ROT_DENSE,
        "perm": KVQ_ROT_PERM_HADAMARD}

EXPORTED_SYMBOLS = ("kvq_quantize", "kvq_quantize_at", "kvq_quantize_bits", "kvq_quantize_at_bits",
                    "kvq_quantize_paged", "kvq_decode_workspace_bytes", "kvq_decode_attention",
                    "kvq_decode_attention_varlen", "kvq_decode_attention_bits",
                    "kvq_decode_attention_varlen_bits", "kvq_decode_attention_paged",
                    "kvq_status_str", "kvq_abi_version")

D_HEAD = 128
GROUP = 32


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kvq_status_str(status)} ({status})")
        self.status = status


class kvq_int2_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("T_cap", ctypes.c_int64)]


class kvq_paged_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("page_tokens", ctypes.c_int64), ("bits", ctypes.c_int32)]


class kvq_quant_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("T_cap", ctypes.c_int64), ("bits", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libkvq.so once; raise if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, i32, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    cp = ctypes.POINTER(kvq_int2_cache)
    lib.kvq_quantize.restype = i32
    lib.kvq_quantize.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                 i32, vp, i32, i64, cp, cp, vp]
    lib.kvq_quantize_at.restype = i32
    lib.kvq_quantize_at.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                    i32, vp, i32, vp, cp, cp, vp]
    lib.kvq_decode_attention_varlen.restype = i32
    lib.kvq_decode_attention_varlen.argtypes = [vp, i32, i64, i64, i64, i64, cp, cp, i64, vp, i64,
                                                i32, vp, i32, vp, vp, i64, vp, vp, i64, f32,
                                                vp, i32, vp, ctypes.c_size_t, vp]
    lib.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64]
    lib.kvq_decode_attention.restype = i32
    lib.kvq_decode_attention.argtypes = [vp, i32, i64, i64, i64, i64, cp, cp, i64, i64,
                                         i32, vp, i32, vp, vp, i64, vp, vp, i64, f32,
                                         vp, i32, vp, ctypes.c_size_t, vp]
    qp = ctypes.POINTER(kvq_quant_cache)
    lib.kvq_quantize_bits.restype = i32
    lib.kvq_quantize_bits.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                      i32, vp, i32, i64, qp, qp, vp]
    lib.kvq_decode_attention_bits.restype = i32
    lib.kvq_decode_attention_bits.argtypes = [vp, i32, i64, i64, i64, i64, qp, qp, i64, i64,
                                              i32, vp, i32, vp, vp, i64, vp, vp, i64, f32,
                                              vp, i32, vp, ctypes.c_size_t, vp]
    lib.kvq_quantize_at_bits.restype = i32
    lib.kvq_quantize_at_bits.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                         i32, vp, i32, vp, qp, qp, vp]
    lib.kvq_decode_attention_varlen_bits.restype = i32
    lib.kvq_decode_attention_varlen_bits.argtypes = [vp, i32, i64, i64, i64, i64, qp, qp, i64, vp,
                                                     i64, i32, vp, i32, vp, vp, i64, vp, vp, i64,
                                                     f32, vp, i32, vp, ctypes.c_size_t, vp]
    pp = ctypes.POINTER(kvq_paged_cache)
    lib.kvq_quantize_paged.restype = i32
    lib.kvq_quantize_paged.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                       i32, vp, i32, vp, vp, i64, pp, pp, vp]
    lib.kvq_decode_attention_paged.restype = i32
    lib.kvq_decode_attention_paged.argtypes = [vp, i32, i64, i64, i64, i64, pp, pp, i64, vp, i64,
                                               vp, i64, i32, vp, i32, vp, vp, i64, vp, vp, i64, f32,
                                               vp, i32, vp, ctypes.c_size_t, vp]
    lib.kvq_status_str.restype = ctypes.c_char_p
    lib.kvq_status_str.argtypes = [i32]
    lib.kvq_abi_version.restype = i32
    lib.kvq_abi_version.argtypes = []
    _lib = lib
    return lib


def kvq_status_str(status: int) -> str:
    return load_library().kvq_status_str(int(status)).decode()


def kvq_abi_version() -> int:
    return int(load_library().kvq_abi_version())


def _check(status: int, where: str):
    if status != KVQ_OK:
        raise KvqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Int2Cache:
    """Device buffers of one side (K or V) of a quantized cache.

    codes  uint8 [B, Hkv, T_cap, d*bits/8]; scales / zeros fp16 [B, Hkv, T_cap, d/32].
    bits = 2 (the INT2 format) unless given; 1 and 4 are the other widths.
    """

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 bits: int | None = None):
        self.codes, self.scales, self.zeros = codes, scales, zeros
        self.T_cap = codes.shape[2]
        d = scales.shape[3] * GROUP
        self.bits = bits if bits is not None else 8 * codes.shape[3] // d
        if codes.shape[3] * 8 != d * self.bits:
            raise ValueError("codes row length does not match the code width")

    @classmethod
    def empty(cls, B: int, Hkv: int, T_cap: int, device="cuda", d: int = D_HEAD, bits: int = 2):
        codes = torch.empty((B, Hkv, T_cap, d * bits // 8), dtype=torch.uint8, device=device)
        scales = torch.empty((B, Hkv, T_cap, d // GROUP), dtype=torch.float16, device=device)
        zeros = torch.empty((B, Hkv, T_cap, d // GROUP), dtype=torch.float16, device=device)
        return cls(codes, scales, zeros, bits)

    def c_struct(self) -> kvq_int2_cache:
        if self.bits != 2:
            raise ValueError("not a 2-bit cache")
        return kvq_int2_cache(self.codes.data_ptr(), self.scales.data_ptr(),
                              self.zeros.data_ptr(), self.T_cap)

    def c_quant_struct(self) -> kvq_quant_cache:
        return kvq_quant_cache(self.codes.data_ptr(), self.scales.data_ptr(),
                               self.zeros.data_ptr(), self.T_cap, self.bits)

    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes + self.zeros.nbytes


def kvq_quantize(K, V, cache_k: Int2Cache | None, cache_v: Int2Cache | None,
                 rot: str = "hadamard", R: torch.Tensor | None = None,
                 group: int = GROUP, t_offset: int = 0, stream=None,
                 t_offsets: torch.Tensor | None = None):
    """Rotate, quantize and pack K/V rows [B, T_new, Hkv, d] (channel stride 1)
    into cache slots [t_offset, t_offset + T_new).  Either side may be None.
    R: fp32 [Hkv, d, d] for rot="dense"; int32 [Hkv, d] channel permutations
    for rot="perm" (reorder, then the Hadamard transform); None otherwise.
    t_offsets: int32 [B] on the device: sequence b's rows land at slots
    [t_offsets[b], t_offsets[b] + T_new) (kvq_quantize_at); t_offset is then
    unused."""
    x = K if K is not None else V
    for t in (K, V):
        if t is not None and (t.dim() != 4 or t.stride(3) != 1):
            raise ValueError("K/V must be [B, T_new, Hkv, d] with unit channel stride")
    if K is not None and V is not None and (K.shape != V.shape or K.stride() != V.stride()
                                            or K.dtype != V.dtype):
        raise ValueError("K and V must share shape, strides and dtype")
    B, T_new, Hkv, d = x.shape
    lib = load_library()
    if t_offsets is not None and (t_offsets.dtype != torch.int32 or t_offsets.numel() != B):
        raise ValueError("t_offsets must be int32 [B]")
    if any(c is not None and c.bits != 2 for c in (cache_k, cache_v)):
        kq = cache_k.c_quant_struct() if cache_k is not None else None
        vq = cache_v.c_quant_struct() if cache_v is not None else None
        if t_offsets is not None:
            st = lib.kvq_quantize_at_bits(
                _ptr(K), _ptr(V), _dtype_code(x), B, T_new, Hkv, d,
                x.stride(0), x.stride(1), x.stride(2), _ROT[rot], _ptr(R), group,
                _ptr(t_offsets),
                ctypes.byref(kq) if kq is not None else None,
                ctypes.byref(vq) if vq is not None else None, _stream(stream))
            _check(st, "kvq_quantize_at_bits")
            return
        st = lib.kvq_quantize_bits(
            _ptr(K), _ptr(V), _dtype_code(x), B, T_new, Hkv, d,
            x.stride(0), x.stride(1), x.stride(2), _ROT[rot], _ptr(R), group, t_offset,
            ctypes.byref(kq) if kq is not None else None,
            ctypes.byref(vq) if vq is not None else None, _stream(stream))
        _check(st, "kvq_quantize_bits")
        return
    kc = cache_k.c_struct() if cache_k is not None else None
    vc = cache_v.c_struct() if cache_v is not None else None
    if t_offsets is not None:
        st = lib.kvq_quantize_at(
            _ptr(K), _ptr(V), _dtype_code(x), B, T_new, Hkv, d,
            x.stride(0), x.stride(1), x.stride(2), _ROT[rot], _ptr(R), group, _ptr(t_offsets),
            ctypes.byref(kc) if kc is not None else None,
            ctypes.byref(vc) if vc is not None else None, _stream(stream))
        _check(st, "kvq_quantize_at")
        return
    st = lib.kvq_quantize(
        _ptr(K), _ptr(V), _dtype_code(x), B, T_new, Hkv, d,
        x.stride(0), x.stride(1), x.stride(2), _ROT[rot], _ptr(R), group, t_offset,
        ctypes.byref(kc) if kc is not None else None,
        ctypes.byref(vc) if vc is not None else None, _stream(stream))
    _check(st, "kvq_quantize")


def kvq_decode_workspace_bytes(B, Hq, Hkv, d, n_int2_tokens, n_sink=0, n_res=0) -> int:
    return int(load_library().kvq_decode_workspace_bytes(B, Hq, Hkv, d, n_int2_tokens,
                                                         n_sink, n_res))


def kvq_decode_attention(q: torch.Tensor, cache_k: Int2Cache | None,
                         cache_v: Int2Cache | None, t_begin: int, t_end: int,
                         rot: str = "hadamard", R: torch.Tensor | None = None,
                         group: int = GROUP, sink_k=None, sink_v=None, res_k=None,
                         res_v=None, softmax_scale: float = 0.0,
                         out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None,
                         t_ends: torch.Tensor | None = None):
    """Decode attention for q [B, Hq, d] over INT2 tokens [t_begin, t_end)
    plus optional fp16 sink / residual tokens [B, Hkv, n, d].  Returns out
    [B, Hq, d] in q's dtype (or writes `out`).  t_ends: int32 [B] on the
    device, sequence b's own end (kvq_decode_attention_varlen); t_end is
    then the upper bound of every t_ends[b]."""
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv = (cache_k.codes.shape[1] if cache_k is not None
           else (sink_k if sink_k is not None else res_k).shape[1])
    n_sink = 0 if sink_k is None else sink_k.shape[2]
    n_res = 0 if res_k is None else res_k.shape[2]
    for t in (sink_k, sink_v, res_k, res_v):
        if t is not None and (t.dtype != torch.float16 or not t.is_contiguous()):
            raise ValueError("sink/residual tensors must be contiguous fp16 [B, Hkv, n, d]")
    if out is None:
        out = torch.empty_like(q)
    need = kvq_decode_workspace_bytes(B, Hq, Hkv, d, t_end - t_begin, n_sink, n_res)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    lib = load_library()
    if t_ends is not None and (t_ends.dtype != torch.int32 or t_ends.numel() != B):
        raise ValueError("t_ends must be int32 [B]")
    if any(c is not None and c.bits != 2 for c in (cache_k, cache_v)):
        kq = cache_k.c_quant_struct() if cache_k is not None else None
        vq = cache_v.c_quant_struct() if cache_v is not None else None
        if t_ends is not None:
            st = lib.kvq_decode_attention_varlen_bits(
                _ptr(q), _dtype_code(q), B, Hq, Hkv, d,
                ctypes.byref(kq) if kq is not None else None,
                ctypes.byref(vq) if vq is not None else None,
                t_begin, _ptr(t_ends), t_end, _ROT[rot], _ptr(R), group,
                _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(res_k), _ptr(res_v), n_res,
                float(softmax_scale), _ptr(out), _dtype_code(out),
                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
            _check(st, "kvq_decode_attention_varlen_bits")
            return out
        st = lib.kvq_decode_attention_bits(
            _ptr(q), _dtype_code(q), B, Hq, Hkv, d,
            ctypes.byref(kq) if kq is not None else None,
            ctypes.byref(vq) if vq is not None else None,
            t_begin, t_end, _ROT[rot], _ptr(R), group,
            _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(res_k), _ptr(res_v), n_res,
            float(softmax_scale), _ptr(out), _dtype_code(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "kvq_decode_attention_bits")
        return out
    kc = cache_k.c_struct() if cache_k is not None else None
    vc = cache_v.c_struct() if cache_v is not None else None
    if t_ends is not None:
        st = lib.kvq_decode_attention_varlen(
            _ptr(q), _dtype_code(q), B, Hq, Hkv, d,
            ctypes.byref(kc) if kc is not None else None,
            ctypes.byref(vc) if vc is not None else None,
            t_begin, _ptr(t_ends), t_end, _ROT[rot], _ptr(R), group,
            _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(res_k), _ptr(res_v), n_res,
            float(softmax_scale), _ptr(out), _dtype_code(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "kvq_decode_attention_varlen")
        return out
    st = lib.kvq_decode_attention(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, d,
        ctypes.byref(kc) if kc is not None else None,
        ctypes.byref(vc) if vc is not None else None,
        t_begin, t_end, _ROT[rot], _ptr(R), group,
        _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(res_k), _ptr(res_v), n_res,
        float(softmax_scale), _ptr(out), _dtype_code(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "kvq_decode_attention")
    return out


def default_softmax_scale(d: int = D_HEAD) -> float:
    return 1.0 / math.sqrt(d)


class PagedCache:
    """Device buffers of one side (K or V) of a paged cache:
    codes uint8 [n_pages, Hkv, page_tokens, d*bits/8]; scales / zeros fp16
    [n_pages, Hkv, page_tokens, d/32].  A block table int32 [B, max_pages]
    maps sequence b's token t to row t % page_tokens of page table[b, t // page_tokens].
    bits = 2 (the INT2 format) unless given; 1 and 4 are the other widths."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 bits: int | None = None):
        self.codes, self.scales, self.zeros = codes, scales, zeros
        self.n_pages, self.page_tokens = codes.shape[0], codes.shape[2]
        d = scales.shape[3] * GROUP
        self.bits = bits if bits is not None else 8 * codes.shape[3] // d
        if codes.shape[3] * 8 != d * self.bits:
            raise ValueError("codes row width does not match bits")

    @classmethod
    def empty(cls, n_pages: int, Hkv: int, page_tokens: int, device="cuda", d: int = D_HEAD,
              bits: int = 2):
        codes = torch.empty((n_pages, Hkv, page_tokens, d * bits // 8), dtype=torch.uint8,
                            device=device)
        scales = torch.empty((n_pages, Hkv, page_tokens, d // GROUP), dtype=torch.float16, device=device)
        zeros = torch.empty((n_pages, Hkv, page_tokens, d // GROUP), dtype=torch.float16, device=device)
        return cls(codes, scales, zeros, bits)

    def c_struct(self) -> kvq_paged_cache:
        return kvq_paged_cache(self.codes.data_ptr(), self.scales.data_ptr(), self.zeros.data_ptr(),
                               self.n_pages, self.page_tokens, self.bits)


def _table(block_table, B):
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    return block_table.shape[1]


def kvq_quantize_paged(K, V, cache_k: PagedCache | None, cache_v: PagedCache | None,
                       t_offsets: torch.Tensor, block_table: torch.Tensor,
                       rot: str = "hadamard", R: torch.Tensor | None = None,
                       group: int = GROUP, stream=None):
    """Rotate, quantize and pack K/V rows [B, T_new, Hkv, d] of fp16 into a
    paged cache: sequence b's rows are its tokens t_offsets[b] + i, placed
    through block_table [B, max_pages] (kvq_quantize_paged)."""
    x = K if K is not None else V
    B, T_new, Hkv, d = x.shape
    if t_offsets.dtype != torch.int32 or t_offsets.numel() != B:
        raise ValueError("t_offsets must be int32 [B]")
    max_pages = _table(block_table, B)
    kc = cache_k.c_struct() if cache_k is not None else None
    vc = cache_v.c_struct() if cache_v is not None else None
    st = load_library().kvq_quantize_paged(
        _ptr(K), _ptr(V), _dtype_code(x), B, T_new, Hkv, d,
        x.stride(0), x.stride(1), x.stride(2), _ROT[rot], _ptr(R), group, _ptr(t_offsets),
        _ptr(block_table), max_pages,
        ctypes.byref(kc) if kc is not None else None,
        ctypes.byref(vc) if vc is not None else None, _stream(stream))
    _check(st, "kvq_quantize_paged")


def kvq_decode_attention_paged(q: torch.Tensor, cache_k: PagedCache, cache_v: PagedCache,
                               t_begin: int, t_ends: torch.Tensor, t_end_max: int,
                               block_table: torch.Tensor, rot: str = "hadamard",
                               R: torch.Tensor | None = None, group: int = GROUP,
                               sink_k=None, sink_v=None, res_k=None, res_v=None,
                               softmax_scale: float = 0.0, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, stream=None):
    """Decode attention for q [B, Hq, d] over a paged cache: sequence b
    attends to its tokens [t_begin, t_ends[b]) (kvq_decode_attention_paged)."""
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv = cache_k.codes.shape[1]
    if t_ends.dtype != torch.int32 or t_ends.numel() != B:
        raise ValueError("t_ends must be int32 [B]")
    max_pages = _table(block_table, B)
    n_sink = 0 if sink_k is None else sink_k.shape[2]
    n_res = 0 if res_k is None else res_k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    need = kvq_decode_workspace_bytes(B, Hq, Hkv, d, t_end_max - t_begin, n_sink, n_res)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    kc, vc = cache_k.c_struct(), cache_v.c_struct()
    st = load_library().kvq_decode_attention_paged(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, d, ctypes.byref(kc), ctypes.byref(vc),
        t_begin, _ptr(t_ends), t_end_max, _ptr(block_table), max_pages,
        _ROT[rot], _ptr(R), group,
        _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(res_k), _ptr(res_v), n_res,
        float(softmax_scale), _ptr(out), _dtype_code(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "kvq_decode_attention_paged")
    return out
