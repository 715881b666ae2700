"""CPU oracle of the CacheGen KV-cache codec — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``libcgoracle.so`` (plain C in
``cgoracle.c``, built with gcc, no SIMD intrinsics, no fast-math, no FMA
contraction) with numpy arrays in and out.  It shares no code with the GPU
library.

Parity of the range coder is pinned by brute force and information-theoretic
bounds, the binary16 conversions by numpy, the channel std by numpy's std, the
quantiser by its error bound and closed-form grids, and the coded size by the
analytic entropy of the synthetic source (tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes as C
import os
import struct
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cgoracle.c")
_LIB = os.path.join(_HERE, "libcgoracle.so")
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

NSYM = 64
ASYM = 256  # anchor symbols: value a in -127..127 is symbol a + 128
PROB_BITS = 15
ERRORS = {0: "ok", -1: "invalid argument", -2: "out of memory", -4: "corrupt",
          -5: "capacity", -6: "mismatch"}


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into oracle/libcgoracle.so."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({code})")
        self.code = code


class cgo_params(C.Structure):
    _fields_ = [("layers", C.c_int32), ("tokens", C.c_int32), ("channels", C.c_int32),
                ("chunk_tokens", C.c_int32), ("group_tokens", C.c_int32),
                ("n_layer_groups", C.c_int32), ("layer_group_end", C.c_int32 * 3),
                ("layer_step", C.c_float * 3), ("quality_mult", C.c_float * 3),
                ("quality_mask", C.c_uint32), ("anchor_coding", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P, SZ, I, I64, U64 = C.c_void_p, C.c_size_t, C.c_int, C.c_int64, C.c_uint64
        sigs = {
            "cgo_f16_to_f32_array": (None, [P, P, I64]),
            "cgo_f32_to_f16_array": (None, [P, P, I64]),
            "cgo_dequant_delta_array": (None, [P, P, P, P, I64]),
            "cgo_rc_bound": (SZ, [I64]),
            "cgo_rc_encode": (I, [P, I64, P, I, P, SZ, C.POINTER(SZ)]),
            "cgo_rc_decode": (I, [P, SZ, I64, P, I, P, C.POINTER(SZ), C.POINTER(I)]),
            "cgo_normalize": (None, [P, I, P]),
            "cgo_normalize_tables": (None, [P, C.c_int64, P]),
            "cgo_channel_stats": (None, [P, I, I, I, P, P, C.POINTER(I)]),
            "cgo_tables_size": (SZ, [C.POINTER(cgo_params)]),
            "cgo_build_tables": (I, [C.POINTER(cgo_params), P, P, I, P, SZ, C.POINTER(SZ), P]),
            "cgo_fnv1a64": (U64, [P, SZ]),
            "cgo_tables_id": (U64, [P, SZ]),
            "cgo_chunk_geometry": (I, [P, SZ, I, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                       C.POINTER(C.c_int32)]),
            "cgo_encode_bound": (SZ, [P, SZ, I]),
            "cgo_encode_chunk": (I, [P, SZ, P, P, I, I, I, P, SZ, C.POINTER(SZ)]),
            "cgo_chunk_symbols": (I, [P, SZ, P, P, I, I, P, P]),
            "cgo_decode_blob": (I, [P, SZ, P, SZ, P, P, I, C.POINTER(I)]),
            "cgo_decode_blob_symbols": (I, [P, SZ, P, SZ, P, C.POINTER(I)]),
            "cgo_stream_encode": (I, [P, SZ, I, I, I, I, P, I, P, P, SZ, C.POINTER(SZ)]),
            "cgo_stream_decode": (I, [P, SZ, I, I, I, I, P, I, P, SZ, P, C.POINTER(I)]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(rc, what)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------- #
# binary16                                                                    #
# --------------------------------------------------------------------------- #

def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().cgo_f16_to_f32_array(_ptr(bits), _ptr(out), bits.size)
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().cgo_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def dequant_delta(sym, step, ahat) -> np.ndarray:
    """Delta-token reconstruction: binary16 bits of the value nearest to the
    exact ahat + (sym - 32) * step, ties to even (elementwise)."""
    s, st, a = np.broadcast_arrays(np.asarray(sym, np.uint8), np.asarray(step, np.float32),
                                   np.asarray(ahat, np.float32))
    s, st, a = (np.ascontiguousarray(x) for x in (s, st, a))
    out = np.empty(s.shape, np.uint16)
    lib().cgo_dequant_delta_array(_ptr(s), _ptr(st), _ptr(a), _ptr(out), s.size)
    return out


# --------------------------------------------------------------------------- #
# range coder                                                                 #
# --------------------------------------------------------------------------- #

def rc_encode(symbols, freq) -> bytes:
    sym = np.ascontiguousarray(symbols, dtype=np.uint8)
    f = np.ascontiguousarray(freq, dtype=np.uint16)
    cap = lib().cgo_rc_bound(sym.size) + 8
    out = np.zeros(cap, np.uint8)
    n = C.c_size_t(0)
    _check(lib().cgo_rc_encode(_ptr(sym), sym.size, _ptr(f), f.size, _ptr(out), cap,
                               C.byref(n)), "rc_encode")
    return out[: n.value].tobytes()


def rc_decode(data: bytes, n: int, freq):
    """Returns (symbols, bytes consumed, corrupt flag); bytes past ``data`` read as 0."""
    f = np.ascontiguousarray(freq, dtype=np.uint16)
    buf = np.frombuffer(data, np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    sym = np.zeros(max(n, 1), np.uint8)
    used = C.c_size_t(0)
    bad = C.c_int(0)
    _check(lib().cgo_rc_decode(_ptr(buf), len(data), n, _ptr(f), f.size, _ptr(sym),
                               C.byref(used), C.byref(bad)), "rc_decode")
    return sym[:n], used.value, bool(bad.value)


def rc_bound(n: int) -> int:
    return lib().cgo_rc_bound(n)


def normalize(counts) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    f = np.zeros(c.size, np.uint16)
    lib().cgo_normalize(_ptr(c), c.size, _ptr(f))
    return f


def normalize_tables(counts) -> np.ndarray:
    """One 64-entry frequency table per row of counts [..., 64]."""
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    f = np.zeros(c.shape, np.uint16)
    lib().cgo_normalize_tables(_ptr(c), c.size // NSYM, _ptr(f))
    return f


# --------------------------------------------------------------------------- #
# statistics, tables, chunks                                                  #
# --------------------------------------------------------------------------- #

def channel_stats(x: np.ndarray):
    """(sigma float64 [L,C], absmax float32 [L,C], nonfinite) of a [L,T,C] fp16 tensor."""
    x = np.ascontiguousarray(x).view(np.uint16)
    L, T, Cc = x.shape
    sig = np.empty((L, Cc), np.float64)
    amax = np.empty((L, Cc), np.float32)
    nf = C.c_int(0)
    lib().cgo_channel_stats(_ptr(x), L, T, Cc, _ptr(sig), _ptr(amax), C.byref(nf))
    return sig, amax, bool(nf.value)


def make_params(layers, tokens, channels, chunk_tokens, group_tokens, layer_group_end,
                layer_step, quality_mult=(1.0, 1.5, 2.5), quality_mask=1,
                anchor_coding=0) -> cgo_params:
    p = cgo_params()
    p.layers, p.tokens, p.channels = layers, tokens, channels
    p.chunk_tokens, p.group_tokens = chunk_tokens, group_tokens
    p.n_layer_groups = len(layer_group_end)
    for i in range(3):
        p.layer_group_end[i] = layer_group_end[i] if i < len(layer_group_end) else 0
        p.layer_step[i] = layer_step[i] if i < len(layer_step) else 0.0
        p.quality_mult[i] = quality_mult[i]
    p.quality_mask = quality_mask
    p.anchor_coding = anchor_coding
    return p


def params_for(w, anchor_coding: int = 0) -> cgo_params:
    """Parameters of a ``synth.Workload``; anchor_coding = 1 range-codes the
    anchors with one 256-symbol table per (kv, layer)."""
    return make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask,
                       anchor_coding)


def build_tables(p: cgo_params, k: np.ndarray, v: np.ndarray, threads: Optional[int] = None,
                 with_counts: bool = False):
    k = np.ascontiguousarray(k).view(np.uint16)
    v = np.ascontiguousarray(v).view(np.uint16)
    size = lib().cgo_tables_size(C.byref(p))
    out = np.zeros(size, np.uint8)
    n = C.c_size_t(0)
    nq = bin(p.quality_mask & 7).count("1")
    counts = np.zeros((nq, 2, p.layers, p.channels, NSYM), np.uint32) if with_counts else None
    _check(lib().cgo_build_tables(C.byref(p), _ptr(k), _ptr(v), threads or default_threads(),
                                  _ptr(out), size, C.byref(n),
                                  _ptr(counts) if with_counts else None), "build_tables")
    t = out.tobytes()
    return (t, counts) if with_counts else t


GROUP_LAYER_CHANNEL, GROUP_LAYER, GROUP_CHANNEL, GROUP_GLOBAL = 0, 1, 2, 3


def pool_counts(counts: np.ndarray, grouping: int) -> np.ndarray:
    """Symbol counts [nq, 2, L, C, 64] pooled over a coarser group and handed back
    to every member: 1 sums over the channels of a layer, 2 over the layers of a
    channel, 3 over both (per kv and quality).  A pooled count must fit 32 bits."""
    c = counts.astype(np.uint64)
    if grouping == GROUP_LAYER_CHANNEL:
        pooled = c
    elif grouping == GROUP_LAYER:
        pooled = c.sum(axis=3, keepdims=True)
    elif grouping == GROUP_CHANNEL:
        pooled = c.sum(axis=2, keepdims=True)
    elif grouping == GROUP_GLOBAL:
        pooled = c.sum(axis=(2, 3), keepdims=True)
    else:
        raise ValueError("unknown grouping")
    if pooled.max(initial=0) > 0xFFFFFFFF:
        raise ValueError("a pooled symbol count does not fit 32 bits")
    return np.broadcast_to(pooled, counts.shape).astype(np.uint32)


def build_tables_grouped(p: cgo_params, k: np.ndarray, v: np.ndarray, grouping: int,
                         threads: Optional[int] = None) -> bytes:
    """Tables whose frequency tables come from counts pooled by ``grouping``
    (scales and steps stay per layer and channel): the per-(layer, channel)
    counts, pooled, each member's table normalised from the pooled counts."""
    t, counts = build_tables(p, k, v, threads=threads, with_counts=True)
    pooled = pool_counts(counts, grouping)
    buf = bytearray(t)
    tv = tables_view(buf)
    for i, q in enumerate(q for q in range(3) if (p.quality_mask >> q) & 1):
        tv.freq[q][...] = normalize_tables(pooled[i])
    return bytes(buf)


def fnv1a64(data: bytes) -> int:
    buf = np.frombuffer(data, np.uint8)
    return int(lib().cgo_fnv1a64(_ptr(buf), buf.size))


def tables_id(data: bytes) -> int:
    buf = np.frombuffer(data, np.uint8)
    return int(lib().cgo_tables_id(_ptr(buf), buf.size))


def chunk_geometry(tables: bytes, chunk: int):
    t = np.frombuffer(tables, np.uint8)
    t0, tc, ng = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().cgo_chunk_geometry(_ptr(t), t.size, chunk, C.byref(t0), C.byref(tc),
                                    C.byref(ng)), "chunk_geometry")
    return t0.value, tc.value, ng.value


def encode_chunk(tables: bytes, k, v, chunk: int, q: int, threads: Optional[int] = None) -> bytes:
    t = np.frombuffer(tables, np.uint8)
    k = np.ascontiguousarray(k).view(np.uint16)
    v = np.ascontiguousarray(v).view(np.uint16)
    cap = lib().cgo_encode_bound(_ptr(t), t.size, chunk)
    if cap == 0:
        raise OracleError(-1, "encode_bound")
    out = np.zeros(cap, np.uint8)
    n = C.c_size_t(0)
    _check(lib().cgo_encode_chunk(_ptr(t), t.size, _ptr(k), _ptr(v), chunk, q,
                                  threads or default_threads(), _ptr(out), cap, C.byref(n)),
           "encode_chunk")
    return out[: n.value].tobytes()


def encode_bound(tables: bytes, chunk: int) -> int:
    t = np.frombuffer(tables, np.uint8)
    return int(lib().cgo_encode_bound(_ptr(t), t.size, chunk))


def chunk_symbols(tables: bytes, k, v, chunk: int, q: int):
    """anchors int8 [2,L,ng,C] and per-token symbols uint8 [2,L,tc,C] (255 at anchors)."""
    t = np.frombuffer(tables, np.uint8)
    hdr = parse_tables_header(tables)
    t0, tc, ng = chunk_geometry(tables, chunk)
    k = np.ascontiguousarray(k).view(np.uint16)
    v = np.ascontiguousarray(v).view(np.uint16)
    L, Cc = hdr["layers"], hdr["channels"]
    anchors = np.zeros((2, L, ng, Cc), np.int8)
    syms = np.zeros((2, L, tc, Cc), np.uint8)
    _check(lib().cgo_chunk_symbols(_ptr(t), t.size, _ptr(k), _ptr(v), chunk, q,
                                   _ptr(anchors), _ptr(syms)), "chunk_symbols")
    return anchors, syms


def decode_blob(tables: bytes, blob: bytes, k_out: np.ndarray, v_out: np.ndarray,
                threads: Optional[int] = None) -> bool:
    """Decode one chunk blob into k_out / v_out ([L,T,C] fp16); returns the corrupt flag."""
    t = np.frombuffer(tables, np.uint8)
    b = np.frombuffer(blob, np.uint8)
    assert k_out.flags.c_contiguous and v_out.flags.c_contiguous
    bad = C.c_int(0)
    _check(lib().cgo_decode_blob(_ptr(t), t.size, _ptr(b), b.size, _ptr(k_out.view(np.uint16)),
                                 _ptr(v_out.view(np.uint16)), threads or default_threads(),
                                 C.byref(bad)), "decode_blob")
    return bool(bad.value)


def decode_blob_paged(tables: bytes, blob: bytes, k_pool: np.ndarray, v_pool: np.ndarray,
                      page_tokens: int, block_table: np.ndarray,
                      threads: Optional[int] = None):
    """Decode one chunk blob into paged K/V pools (the receiver hands the decoded
    cache to the model: gptget 方法详解, GPU decoding on the receiving end).

    Pools are fp16 [L, num_pages, page_tokens, C].  Context token t lives in
    row t % page_tokens of page block_table[t // page_tokens]; an entry outside
    [0, num_pages) is not written and is reported.  The blob is decoded into a
    plain [L, T, C] tensor first, then its tokens are placed one by one.
    Returns (corrupt, bad_page)."""
    h = parse_blob_header(blob)
    L, T, Cc = h["layers"], h["total_tokens"], h["channels"]
    num_pages = k_pool.shape[1]
    assert k_pool.shape == v_pool.shape == (L, num_pages, page_tokens, Cc)
    k = np.zeros((L, T, Cc), np.float16)
    v = np.zeros((L, T, Cc), np.float16)
    corrupt = decode_blob(tables, blob, k, v, threads)
    bad_page = False
    for t in range(h["token_offset"], h["token_offset"] + h["chunk_tokens"]):
        page = int(block_table[t // page_tokens])
        if not 0 <= page < num_pages:
            bad_page = True
            continue
        k_pool[:, page, t % page_tokens, :] = k[:, t, :]
        v_pool[:, page, t % page_tokens, :] = v[:, t, :]
    return corrupt, bad_page


def decode_blob_symbols(tables: bytes, blob: bytes):
    t = np.frombuffer(tables, np.uint8)
    b = np.frombuffer(blob, np.uint8)
    h = parse_blob_header(blob)
    syms = np.zeros((2, h["layers"], h["chunk_tokens"], h["channels"]), np.uint8)
    bad = C.c_int(0)
    _check(lib().cgo_decode_blob_symbols(_ptr(t), t.size, _ptr(b), b.size, _ptr(syms),
                                         C.byref(bad)), "decode_blob_symbols")
    return syms, bool(bad.value)


def stream_encode(tables: bytes, kv: int, l: int, c: int, q: int, x: np.ndarray):
    """One stream: (anchors int8 [ng], word-padded bytes)."""
    t = np.frombuffer(tables, np.uint8)
    x = np.ascontiguousarray(x).view(np.uint16)
    hdr = parse_tables_header(tables)
    G = hdr["group_tokens"]
    ng = -(-x.size // G)
    anchors = np.zeros(ng, np.int8)
    cap = rc_bound(x.size) + 8
    out = np.zeros(cap, np.uint8)
    n = C.c_size_t(0)
    _check(lib().cgo_stream_encode(_ptr(t), t.size, kv, l, c, q, _ptr(x), x.size,
                                   _ptr(anchors), _ptr(out), cap, C.byref(n)), "stream_encode")
    return anchors, out[: n.value].tobytes()


def stream_decode(tables: bytes, kv: int, l: int, c: int, q: int, anchors, tc: int,
                  data: bytes):
    """One stream back to fp16 [tc]; ``data`` is the stream followed by whatever bytes follow it."""
    t = np.frombuffer(tables, np.uint8)
    a = np.ascontiguousarray(anchors, dtype=np.int8)
    buf = np.frombuffer(data, np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    y = np.zeros(tc, np.uint16)
    bad = C.c_int(0)
    _check(lib().cgo_stream_decode(_ptr(t), t.size, kv, l, c, q, _ptr(a), tc, _ptr(buf),
                                   len(data), _ptr(y), C.byref(bad)), "stream_decode")
    return y.view(np.float16), bool(bad.value)


# --------------------------------------------------------------------------- #
# container formats (Python-side reading for tests)                           #
# --------------------------------------------------------------------------- #

TABLES_HEADER = struct.Struct("<4sI6i3i3f3fIII")
BLOB_HEADER = struct.Struct("<4sI8iIIQQ")


def parse_tables_header(t: bytes) -> dict:
    f = TABLES_HEADER.unpack_from(t, 0)
    return {"magic": f[0], "version": f[1], "layers": f[2], "channels": f[3],
            "tokens": f[4], "chunk_tokens": f[5], "group_tokens": f[6],
            "n_layer_groups": f[7], "layer_group_end": f[8:11], "layer_step": f[11:14],
            "quality_mult": f[14:17], "quality_mask": f[17], "prob_bits": f[18],
            "n_symbols": f[19]}


@dataclass
class TablesView:
    header: dict
    scale_a: np.ndarray      # f32 [2,L,C]
    inv_a: np.ndarray
    step: dict               # q -> f32 [2,L,C]
    inv_step: dict
    freq: dict               # q -> u16 [2,L,C,64]
    afreq: Optional[np.ndarray] = None  # u16 [2,L,256] anchor tables (tables version 2)


def tables_view(t: bytes) -> TablesView:
    h = parse_tables_header(t)
    L, Cc = h["layers"], h["channels"]
    n = 2 * L * Cc
    off = TABLES_HEADER.size
    buf = np.frombuffer(t, np.uint8)

    def take(dtype, count, shape):
        nonlocal off
        a = buf[off: off + count * np.dtype(dtype).itemsize].view(dtype).reshape(shape)
        off += count * np.dtype(dtype).itemsize
        return a

    scale_a = take(np.float32, n, (2, L, Cc))
    inv_a = take(np.float32, n, (2, L, Cc))
    step, inv_step, freq = {}, {}, {}
    for q in range(3):
        if (h["quality_mask"] >> q) & 1:
            step[q] = take(np.float32, n, (2, L, Cc))
            inv_step[q] = take(np.float32, n, (2, L, Cc))
            freq[q] = take(np.uint16, n * NSYM, (2, L, Cc, NSYM))
    afreq = take(np.uint16, 2 * L * ASYM, (2, L, ASYM)) if h["version"] == 2 else None
    assert off == len(t)
    return TablesView(h, scale_a, inv_a, step, inv_step, freq, afreq)


def parse_blob_header(b: bytes) -> dict:
    f = BLOB_HEADER.unpack_from(b, 0)
    return {"magic": f[0], "version": f[1], "layers": f[2], "channels": f[3],
            "total_tokens": f[4], "token_offset": f[5], "chunk_tokens": f[6],
            "group_tokens": f[7], "n_groups": f[8], "quality": f[9],
            "payload_words": f[10], "prob_bits": f[11], "tables_id": f[12]}


@dataclass
class BlobView:
    header: dict
    row_offset: np.ndarray   # u32 [2,L]: the delta streams' rows
    anchors: Optional[np.ndarray]  # i8 [2,L,ng,C] (raw anchors, version 2), else None
    lengths: np.ndarray      # u16 [2,L,C]  (words)
    payload: np.ndarray      # u32 [W]
    payload_offset: int
    tail: bytes              # bytes after the payload words
    anchor_row_offset: Optional[np.ndarray] = None  # u32 [2,L] (coded anchors, version 3)
    anchor_lengths: Optional[np.ndarray] = None     # u16 [2,L,C]


def blob_view(b: bytes) -> BlobView:
    """Version 2 (raw anchors): header, u32 rows[2L], i8 anchors[2,L,ng,C], u16
    lengths[2L,C], pad to 16, payload.  Version 3 (coded anchors): header, u32
    rows[4L], u16 lengths[4L,C], pad to 16, payload; rows 2L.. are the anchor
    streams' rows."""
    h = parse_blob_header(b)
    L, Cc, ng, W = h["layers"], h["channels"], h["n_groups"], h["payload_words"]
    coded = h["version"] == 3
    R = 4 * L if coded else 2 * L
    buf = np.frombuffer(b, np.uint8)
    off = 64
    rows = buf[off: off + 4 * R].view(np.uint32).reshape(R // L, L)
    off += 4 * R
    anchors = None
    if not coded:
        anchors = buf[off: off + 2 * L * ng * Cc].view(np.int8).reshape(2, L, ng, Cc)
        off += 2 * L * ng * Cc
    lengths = buf[off: off + 2 * R * Cc].view(np.uint16).reshape(R // L, L, Cc)
    off += 2 * R * Cc
    off = (off + 15) // 16 * 16
    payload = buf[off: off + 4 * W].view(np.uint32)
    return BlobView(h, rows[:2], anchors, lengths[:2], payload, off, bytes(b[off + 4 * W:]),
                    rows[2:] if coded else None, lengths[2:] if coded else None)


BLOCK_STREAMS = 64  # streams per payload block
UNIT_WORDS = 4      # words per interleaved unit


def stream_word_offsets(lengths_of_row: np.ndarray, c: int) -> np.ndarray:
    """Payload word offsets, from the row's start, of the words of stream c of a
    (kv, layer) row whose stream lengths (words) are ``lengths_of_row``: blocks
    of 64 streams one after another; inside a block, units 0 .. m-1 (m the fewest
    whole 4-word units any stream of the block has) interleaved unit by unit,
    then each stream's remaining words, stream after stream."""
    lens = lengths_of_row.astype(np.int64)
    b0 = c - c % BLOCK_STREAMS
    blk = lens[b0: b0 + BLOCK_STREAMS]
    ns, j = len(blk), c - b0
    m = int((blk // UNIT_WORDS).min())
    base = int(lens[:b0].sum())
    w = np.arange(int(lens[c]), dtype=np.int64)
    inter = base + UNIT_WORDS * ((w // UNIT_WORDS) * ns + j) + w % UNIT_WORDS
    tail0 = base + UNIT_WORDS * m * ns + int((blk[:j] - UNIT_WORDS * m).sum())
    return np.where(w < UNIT_WORDS * m, inter, tail0 + w - UNIT_WORDS * m)


def stream_bytes(bv: BlobView, kv: int, l: int, c: int, extra_words: int = 4,
                 anchors: bool = False) -> bytes:
    """Bytes of delta stream (kv, l, c), or with ``anchors`` of its anchor
    stream, followed by ``extra_words`` zero words (whatever follows a stream does
    not change what it decodes to)."""
    rows, lens = ((bv.anchor_row_offset, bv.anchor_lengths) if anchors
                  else (bv.row_offset, bv.lengths))
    at = int(rows[kv, l]) + stream_word_offsets(lens[kv, l], c)
    words = np.concatenate([bv.payload[at], np.zeros(extra_words, np.uint32)])
    return words.astype(">u4").tobytes()
