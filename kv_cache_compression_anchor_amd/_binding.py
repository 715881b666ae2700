"""ctypes binding of libcachegen.so — argument marshalling only.

Each function has the name of the C entry point it calls (include/cachegen.h).
Tensors are torch tensors: device memory for the codec's inputs and outputs,
host (ideally pinned) memory for streamed blobs.  Streams default to torch's
current stream so the calls order with surrounding torch work.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcachegen.so")

CG_OK, CG_E_INVAL, CG_E_NOMEM, CG_E_HIP, CG_E_CORRUPT, CG_E_CAPACITY, CG_E_MISMATCH = (
    0, -1, -2, -3, -4, -5, -6)
CG_Q_H, CG_Q_M, CG_Q_L = 0, 1, 2
CG_GROUP_LAYER_CHANNEL, CG_GROUP_LAYER, CG_GROUP_CHANNEL, CG_GROUP_GLOBAL = 0, 1, 2, 3
_NAMES = {0: "CG_OK", -1: "CG_E_INVAL", -2: "CG_E_NOMEM", -3: "CG_E_HIP", -4: "CG_E_CORRUPT",
          -5: "CG_E_CAPACITY", -6: "CG_E_MISMATCH"}

EXPORTS = ["cg_build_tables", "cg_build_tables_grouped", "cg_tables_free", "cg_tables_serialize",
           "cg_tables_deserialize", "cg_tables_id", "cg_tables_params", "cg_num_chunks", "cg_encode_bound", "cg_encode",
           "cg_encode_batch", "cg_encode_batch_noalloc", "cg_chunk_info_parse", "cg_decode", "cg_decode_async", "cg_decode_paged_async",
           "cg_decode_streamed",
           "cg_plan_chunk", "cg_release_cached", "cg_last_error"]


class CgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_NAMES.get(code, code)}: {message}")
        self.code = code


class cg_params(C.Structure):
    _fields_ = [("layers", C.c_int32), ("tokens", C.c_int32), ("channels", C.c_int32),
                ("chunk_tokens", C.c_int32), ("group_tokens", C.c_int32),
                ("n_layer_groups", C.c_int32), ("layer_group_end", C.c_int32 * 3),
                ("layer_step", C.c_float * 3), ("quality_mult", C.c_float * 3),
                ("quality_mask", C.c_uint32), ("anchor_coding", C.c_int32)]


class cg_chunk_plan_in(C.Structure):
    _fields_ = [("budget_ms", C.c_double), ("bandwidth_bpms", C.c_double),
                ("bytes_left", C.c_uint64 * 3), ("decode_ms_left", C.c_double * 3)]


class cg_chunk_info(C.Structure):
    _fields_ = [("layers", C.c_int32), ("channels", C.c_int32), ("total_tokens", C.c_int32),
                ("token_offset", C.c_int32), ("chunk_tokens", C.c_int32),
                ("group_tokens", C.c_int32), ("n_groups", C.c_int32), ("quality", C.c_int32),
                ("payload_words", C.c_uint32), ("version", C.c_uint32),
                ("tables_id", C.c_uint64), ("blob_bytes", C.c_uint64)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); the codec has no CPU fallback")
        L = C.CDLL(LIB_PATH)
        P, SZ, I, I32 = C.c_void_p, C.c_size_t, C.c_int, C.c_int32
        sigs = {
            "cg_build_tables": (I, [C.POINTER(cg_params), P, P, P, C.POINTER(P)]),
            "cg_build_tables_grouped": (I, [C.POINTER(cg_params), I32, P, P, P, C.POINTER(P)]),
            "cg_tables_free": (None, [P]),
            "cg_tables_serialize": (I, [P, P, SZ, C.POINTER(SZ)]),
            "cg_tables_deserialize": (I, [P, SZ, C.POINTER(P)]),
            "cg_tables_id": (C.c_uint64, [P]),
            "cg_tables_params": (I, [P, C.POINTER(cg_params)]),
            "cg_num_chunks": (I, [P, C.POINTER(I32)]),
            "cg_encode_bound": (I, [P, I32, C.POINTER(SZ)]),
            "cg_encode": (I, [P, P, P, I32, I32, P, SZ, C.POINTER(SZ), P]),
            "cg_encode_batch": (I, [P, P, P, I32, C.POINTER(I32), C.POINTER(I32), C.POINTER(P),
                                    C.POINTER(SZ), C.POINTER(SZ), P]),
            "cg_encode_batch_noalloc": (I, [P, P, P, I32, C.POINTER(I32), C.POINTER(I32),
                                            C.POINTER(P), C.POINTER(SZ), C.POINTER(SZ), P]),
            "cg_chunk_info_parse": (I, [P, SZ, C.POINTER(cg_chunk_info)]),
            "cg_decode": (I, [P, I32, C.POINTER(P), C.POINTER(SZ), P, P, P]),
            "cg_decode_async": (I, [P, I32, C.POINTER(P), C.POINTER(cg_chunk_info), P, P, P, P]),
            "cg_decode_paged_async": (I, [P, I32, C.POINTER(P), C.POINTER(cg_chunk_info), P, P,
                                          C.c_int64, I32, P, C.c_int64, P, P]),
            "cg_decode_streamed": (I, [P, I32, C.POINTER(P), C.POINTER(cg_chunk_info), P, P, P,
                                       SZ, P, P, P]),
            "cg_plan_chunk": (I, [C.POINTER(cg_chunk_plan_in), C.POINTER(I32),
                                  C.POINTER(C.c_double)]),
            "cg_release_cached": (I, []),
            "cg_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def cg_last_error() -> str:
    return lib().cg_last_error().decode()


def _check(rc: int):
    if rc != CG_OK:
        raise CgError(rc, cg_last_error())


def _stream(stream) -> Optional[int]:
    """hipStream_t of a torch stream / int / None (None = torch's current stream)."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(t, dtype=None, what="tensor"):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}")
    return t.data_ptr()


def make_params(layers, tokens, channels, chunk_tokens=1536, group_tokens=10,
                layer_group_end=None, layer_step=(0.5, 1.0, 1.5), quality_mult=(1.0, 1.5, 2.5),
                quality_mask=1, anchor_coding=0) -> cg_params:
    p = cg_params()
    p.layers, p.tokens, p.channels = layers, tokens, channels
    p.chunk_tokens, p.group_tokens = chunk_tokens, group_tokens
    ends = tuple(layer_group_end) if layer_group_end is not None else ()
    p.n_layer_groups = len(ends)  # 0: the library's default split
    for i in range(3):
        p.layer_group_end[i] = ends[i] if i < len(ends) else 0
        p.layer_step[i] = layer_step[i] if i < len(layer_step) else 0.0
        p.quality_mult[i] = quality_mult[i]
    p.quality_mask = quality_mask
    p.anchor_coding = anchor_coding
    return p


class Tables:
    """Owner of a cg_tables handle (freed with the object)."""

    def __init__(self, handle: int):
        self.handle = handle

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.cg_tables_free(h)

    @property
    def id(self) -> int:
        return cg_tables_id(self)

    @property
    def params(self) -> cg_params:
        return cg_tables_params(self)


def cg_build_tables(params: cg_params, k, v, stream=None) -> Tables:
    import torch
    kp = _dev_ptr(k, torch.float16, "k")
    vp = _dev_ptr(v, torch.float16, "v")
    want = (params.layers, params.tokens, params.channels)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must both be {want}")
    out = C.c_void_p()
    _check(lib().cg_build_tables(C.byref(params), kp, vp, _stream(stream), C.byref(out)))
    return Tables(out.value)


def cg_build_tables_grouped(params: cg_params, grouping: int, k, v, stream=None) -> Tables:
    import torch
    kp = _dev_ptr(k, torch.float16, "k")
    vp = _dev_ptr(v, torch.float16, "v")
    want = (params.layers, params.tokens, params.channels)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k and v must both be {want}")
    out = C.c_void_p()
    _check(lib().cg_build_tables_grouped(C.byref(params), int(grouping), kp, vp, _stream(stream),
                                         C.byref(out)))
    return Tables(out.value)


def cg_tables_free(t: Tables):
    if t.handle:
        lib().cg_tables_free(t.handle)
        t.handle = None


def cg_tables_serialize(t: Tables) -> bytes:
    n = C.c_size_t(0)
    _check(lib().cg_tables_serialize(t.handle, None, 0, C.byref(n)))
    buf = (C.c_uint8 * n.value)()
    _check(lib().cg_tables_serialize(t.handle, buf, n.value, C.byref(n)))
    return bytes(buf)


def cg_tables_deserialize(data: bytes) -> Tables:
    out = C.c_void_p()
    buf = C.create_string_buffer(bytes(data), len(data))
    _check(lib().cg_tables_deserialize(buf, len(data), C.byref(out)))
    return Tables(out.value)


def cg_tables_id(t: Tables) -> int:
    return int(lib().cg_tables_id(t.handle))


def cg_tables_params(t: Tables) -> cg_params:
    p = cg_params()
    _check(lib().cg_tables_params(t.handle, C.byref(p)))
    return p


def cg_num_chunks(t: Tables) -> int:
    n = C.c_int32(0)
    _check(lib().cg_num_chunks(t.handle, C.byref(n)))
    return n.value


def cg_encode_bound(t: Tables, chunk: int) -> int:
    n = C.c_size_t(0)
    _check(lib().cg_encode_bound(t.handle, chunk, C.byref(n)))
    return n.value


def cg_encode(t: Tables, k, v, chunk: int, quality: int, out, stream=None) -> int:
    """Encodes one chunk into the uint8 device tensor `out`; returns the blob size."""
    import torch
    kp = _dev_ptr(k, torch.float16, "k")
    vp = _dev_ptr(v, torch.float16, "v")
    op = _dev_ptr(out, torch.uint8, "out")
    n = C.c_size_t(0)
    _check(lib().cg_encode(t.handle, kp, vp, chunk, quality, op, out.numel(), C.byref(n),
                           _stream(stream)))
    return n.value


def cg_encode_batch(t: Tables, k, v, chunks, qualities, outs, stream=None):
    """Encodes blob i = (chunks[i], qualities[i]) into the uint8 device tensor outs[i];
    returns the blob sizes."""
    return _encode_batch("cg_encode_batch", t, k, v, chunks, qualities, outs, stream)


def cg_encode_batch_noalloc(t: Tables, k, v, chunks, qualities, outs, stream=None):
    """cg_encode_batch through the entry point that allocates nothing (static
    device scratch); returns the blob sizes."""
    return _encode_batch("cg_encode_batch_noalloc", t, k, v, chunks, qualities, outs, stream)


def _encode_batch(name, t: Tables, k, v, chunks, qualities, outs, stream):
    import torch
    n = len(chunks)
    if len(qualities) != n or len(outs) != n:
        raise ValueError("one quality and one output per chunk")
    kp = _dev_ptr(k, torch.float16, "k")
    vp = _dev_ptr(v, torch.float16, "v")
    ops = [_dev_ptr(o, torch.uint8, "out") for o in outs]
    carr = (C.c_int32 * max(1, n))(*chunks)
    qarr = (C.c_int32 * max(1, n))(*qualities)
    caps = (C.c_size_t * max(1, n))(*[o.numel() for o in outs])
    lens = (C.c_size_t * max(1, n))()
    _check(getattr(lib(), name)(t.handle, kp, vp, n, carr, qarr, _ptr_array(ops), caps, lens,
                                _stream(stream)))
    return [int(x) for x in lens[:n]]


def cg_chunk_info_parse(blob_host) -> cg_chunk_info:
    """Header of a blob held in host memory (bytes, numpy array or CPU tensor)."""
    import numpy as np
    if hasattr(blob_host, "numpy"):
        arr = blob_host.numpy()
    else:
        arr = np.frombuffer(bytes(blob_host[:64]) if isinstance(blob_host, (bytes, bytearray))
                            else blob_host, dtype=np.uint8)
    arr = np.ascontiguousarray(arr[:64], dtype=np.uint8)
    info = cg_chunk_info()
    _check(lib().cg_chunk_info_parse(arr.ctypes.data_as(C.c_void_p), arr.size, C.byref(info)))
    return info


def _ptr_array(ptrs: Sequence[int]):
    return (C.c_void_p * max(1, len(ptrs)))(*ptrs)


def cg_decode(t: Tables, blobs, k_out, v_out, lens=None, stream=None):
    import torch
    bp = [_dev_ptr(b, torch.uint8, "blob") for b in blobs]
    ls = lens if lens is not None else [b.numel() for b in blobs]
    larr = (C.c_size_t * max(1, len(ls)))(*ls)
    _check(lib().cg_decode(t.handle, len(bp), _ptr_array(bp), larr,
                           _dev_ptr(k_out, torch.float16, "k_out"),
                           _dev_ptr(v_out, torch.float16, "v_out"), _stream(stream)))


def cg_decode_async(t: Tables, blobs, infos, k_out, v_out, status, stream=None):
    import torch
    bp = [_dev_ptr(b, torch.uint8, "blob") for b in blobs]
    if len(infos) != len(bp):
        raise ValueError("one info per blob")
    iarr = (cg_chunk_info * max(1, len(infos)))(*infos)
    _check(lib().cg_decode_async(t.handle, len(bp), _ptr_array(bp), iarr,
                                 _dev_ptr(k_out, torch.float16, "k_out"),
                                 _dev_ptr(v_out, torch.float16, "v_out"),
                                 _dev_ptr(status, torch.int32, "status"), _stream(stream)))


def cg_decode_paged_async(t: Tables, blobs, infos, k_pool, v_pool, page_tokens, block_table,
                          status, stream=None):
    """Decode into paged pools k_pool / v_pool (fp16 [L, num_pages, page_tokens,
    C] device tensors) through block_table (int32 device tensor, one entry per
    block of page_tokens context tokens)."""
    import torch
    bp = [_dev_ptr(b, torch.uint8, "blob") for b in blobs]
    if len(infos) != len(bp):
        raise ValueError("one info per blob")
    prm = t.params
    if (k_pool.dim() != 4 or k_pool.shape != v_pool.shape or k_pool.shape[2] != page_tokens
            or k_pool.shape[0] != prm.layers or k_pool.shape[3] != prm.channels):
        raise ValueError("pools must both be [layers, num_pages, page_tokens, channels] of the tables")
    iarr = (cg_chunk_info * max(1, len(infos)))(*infos)
    _check(lib().cg_decode_paged_async(t.handle, len(bp), _ptr_array(bp), iarr,
                                       _dev_ptr(k_pool, torch.float16, "k_pool"),
                                       _dev_ptr(v_pool, torch.float16, "v_pool"),
                                       int(k_pool.shape[1]), int(page_tokens),
                                       _dev_ptr(block_table, torch.int32, "block_table"),
                                       int(block_table.numel()),
                                       _dev_ptr(status, torch.int32, "status"), _stream(stream)))


def cg_decode_streamed(t: Tables, host_blobs, infos, k_out, v_out, staging, status,
                       copy_stream, compute_stream):
    import torch
    hp = []
    for b in host_blobs:
        if b.device.type != "cpu" or b.dtype != torch.uint8 or not b.is_contiguous():
            raise ValueError("host blobs must be contiguous uint8 CPU tensors")
        hp.append(b.data_ptr())
    if len(infos) != len(hp):
        raise ValueError("one info per blob")
    iarr = (cg_chunk_info * max(1, len(infos)))(*infos)
    _check(lib().cg_decode_streamed(t.handle, len(hp), _ptr_array(hp), iarr,
                                    _dev_ptr(k_out, torch.float16, "k_out"),
                                    _dev_ptr(v_out, torch.float16, "v_out"),
                                    _dev_ptr(staging, torch.uint8, "staging"), staging.numel(),
                                    _dev_ptr(status, torch.int32, "status"),
                                    _stream(copy_stream), _stream(compute_stream)))


def cg_release_cached():
    """Frees the device memory the library keeps between calls (workspaces,
    cached pool blocks) on every device it has used."""
    _check(lib().cg_release_cached())


def cg_plan_chunk(budget_ms: float, bandwidth_bpms: float, bytes_left, decode_ms_left):
    """The version (CG_Q_H / M / L) of the next chunk and the three ratios the
    library computed; bytes_left / decode_ms_left are per version (H, M, L), 0
    bytes marking a version that does not exist.  Host only."""
    p = cg_chunk_plan_in()
    p.budget_ms = float(budget_ms)
    p.bandwidth_bpms = float(bandwidth_bpms)
    for q in range(3):
        p.bytes_left[q] = int(bytes_left[q])
        p.decode_ms_left[q] = float(decode_ms_left[q])
    q = C.c_int32(-1)
    r = (C.c_double * 3)()
    _check(lib().cg_plan_chunk(C.byref(p), C.byref(q), r))
    return q.value, [r[0], r[1], r[2]]
