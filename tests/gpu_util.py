"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI, run the oracle on the same inputs."""
import numpy as np

import oracle
import synth


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def params_of(w, anchor_coding=0):
    import kv_cache_compression_anchor_amd as cg
    return cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                          w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask,
                          anchor_coding)


def gpu_tables(w, kd, vd, anchor_coding=0):
    import kv_cache_compression_anchor_amd as cg
    return cg.cg_build_tables(params_of(w, anchor_coding), kd, vd)


def gpu_encode(tab, kd, vd, chunk, q):
    """Blob of one chunk as (device tensor trimmed to its size, host bytes)."""
    import kv_cache_compression_anchor_amd as cg
    t = torch()
    cap = cg.cg_encode_bound(tab, chunk)
    out = t.empty(cap, dtype=t.uint8, device="cuda")
    n = cg.cg_encode(tab, kd, vd, chunk, q, out)
    blob = out[:n].clone()
    return blob, blob.cpu().numpy().tobytes()


def gpu_decode(tab, blobs, shape):
    """Decode device blobs with cg_decode_async; returns (k, v, status) on the host."""
    import kv_cache_compression_anchor_amd as cg
    t = torch()
    ko = t.zeros(shape, dtype=t.float16, device="cuda")
    vo = t.zeros(shape, dtype=t.float16, device="cuda")
    st = t.zeros(1, dtype=t.int32, device="cuda")
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in blobs]
    cg.cg_decode_async(tab, blobs, infos, ko, vo, st)
    t.cuda.synchronize()
    return ko.cpu().numpy(), vo.cpu().numpy(), int(st.item())


def oracle_decode(tables: bytes, blobs, shape):
    ko = np.zeros(shape, np.float16)
    vo = np.zeros(shape, np.float16)
    bad = False
    for b in blobs:
        bad |= oracle.decode_blob(tables, b, ko, vo)
    return ko, vo, bad


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(np.ascontiguousarray(a).view(np.uint16),
                          np.ascontiguousarray(b).view(np.uint16))


def first_difference(a: bytes, b: bytes):
    n = min(len(a), len(b))
    x = np.frombuffer(a[:n], np.uint8) != np.frombuffer(b[:n], np.uint8)
    i = int(np.argmax(x)) if x.any() else n
    return i, len(a), len(b)


def workload(**kw):
    base = dict(layers=3, tokens=1000, channels=100, seed=7, rho=0.85, outlier_frac=0.03,
                chunk_tokens=384, group_tokens=10, layer_group_end=(1, 2, 3),
                layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2))
    base.update(kw)
    return synth.Workload("test", **base)
