"""Benchmark of the KV-cache codec hot path on one MI355X.

One step = the whole hot path over one synthetic context (Mistral-7B-shape GQA,
K and V each [32 layers, 9216 tokens, 1024 channels] fp16, 6 chunks of 1536
tokens): build the per-(kv, layer, channel) tables, encode every chunk at H, M
and L (one cg_encode_batch call), and decode one mixed-quality selection
H,M,L,H,M,L with one cg_decode_async call.  Inputs are resident in HBM when the timed region starts.

`value` is the decode throughput in GB/s of fp16 KV written; the roofline entry
counts the decode kernel's algorithmic bytes (blob bytes read + fp16 written)
per launch against MI355X's 8 TB/s HBM peak, with the kernel's duration taken
from HIP events on the stream it runs on, and also against what a plain 1 GiB
device-to-device copy reaches on the same GPU.  The CPU baseline is the
oracle's decode of a bounded sample of the same selection on this host's cores
(and on one thread).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mistral7b_9k")
    ap.add_argument("--decode-reps", type=int, default=1,
                    help="timed decode launches per step (the selection is decoded this many times)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-anchor-coded", action="store_true",
                    help="skip the coded-anchor format's figures on the main workload")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the other workloads' figures (the 'workloads' key of the line)")
    ap.add_argument("--other-steps", type=int, default=3,
                    help="timed steps per other workload (after one warmup step)")
    ap.add_argument("--other-cpu-seconds", type=float, default=2.0,
                    help="the oracle's decode and encode sample per other workload, seconds each")
    ap.add_argument("--repeat-decodes", type=int, default=10,
                    help="after the timed steps, decodes of the last selection right after a decode "
                         "of it (roofline.repeat_decode_ms); 0 skips them")
    ap.add_argument("--cpu-sample-seconds", type=float, default=10.0,
                    help="the oracle decodes the selection repeatedly for about this long")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (for HBM counter scaling)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_traffic.json"))
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                          "COPY_WRITE_CSV"),
                    help="write the --workload's record of --traffic-json from rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE and WRITE_SIZE of the decoder, "
                         "then of a --copy-calibration run); no GPU work")
    ap.add_argument("--record-valu", nargs="+", metavar="CSV",
                    help="write the --workload's VALU-issue record in --traffic-json from rocprofv3 "
                         "--pmc counter_collection.csv files holding SQ_INSTS_VALU and "
                         "GRBM_GUI_ACTIVE of the decoder, then the run's agent_info.csv (last "
                         "argument); no GPU work")
    ap.add_argument("--adaptive", action="store_true",
                    help="measure the bandwidth-adaptive version choice instead: every chunk of "
                         "the workload encoded at H, M and L, streamed over a simulated "
                         "fluctuating link; SLO violation rates, adaptive vs fixed versions")
    ap.add_argument("--grouping", action="store_true",
                    help="measure what per-(layer, channel) symbol statistics are worth instead: "
                         "coded size of every chunk and quality with tables pooled per layer, "
                         "per channel and globally, and with tables profiled on another context")
    ap.add_argument("--format-study", action="store_true",
                    help="measure what a later format could save instead: the empirical entropy of "
                         "the blobs' 8-bit anchors under tables pooled per layer or per channel, "
                         "and the bytes of per-stream fields")
    ap.add_argument("--contexts", type=int, default=2000,
                    help="contexts streamed per policy in --adaptive")
    ap.add_argument("--streamed", action="store_true",
                    help="measure the chunk pipeline instead: the Llama-70B-shape 16K schedule "
                         "decoded from pinned host memory (H2D on one stream, decode on another)")
    ap.add_argument("--paged", action="store_true",
                    help="measure the decode into paged K/V pools instead: the selection decoded "
                         "through a shuffled block table of --page-tokens pages, beside the "
                         "decode into [L, T, C] and that decode followed by a copy into the pages")
    ap.add_argument("--page-tokens", type=int, default=16)
    return ap.parse_args()


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.traffic_json, args.workload, *args.record_traffic)
        return
    if args.record_valu:
        if len(args.record_valu) < 2:
            raise SystemExit("--record-valu: counter files, then the agent_info.csv")
        record_valu(args.traffic_json, args.workload, args.record_valu[:-1], args.record_valu[-1])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the codec's streams are independent, sharding is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        a = torch.empty(args.copy_calibration // 4, dtype=torch.int32, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel() * 4}), flush=True)
        return

    import kv_cache_compression_anchor_amd as cg
    import synth

    if args.adaptive:
        adaptive(args)
        return
    if args.format_study:
        print(json.dumps(format_study(args)))
        return
    if args.grouping:
        grouping(args)
        return
    if args.streamed:
        streamed(args)
        return
    if args.paged:
        paged(args)
        return

    w = synth.workload(args.workload)
    t_gen = time.time()
    k, v = synth.gen_kv(w)
    t_gen = time.time() - t_gen
    dev = torch.device("cuda:0")
    kd = torch.from_numpy(k).to(dev)
    vd = torch.from_numpy(v).to(dev)
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    sel = w.selection()
    nch = w.n_chunks
    elements = w.elements
    fp16_bytes = 2 * elements
    stream = torch.cuda.current_stream()

    step, bufs, ko, vo, status = make_stepper(w, p, kd, vd, args.decode_reps)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    results = []
    t_all = time.perf_counter()
    for _ in range(args.steps):
        results.append(step(True))
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t_all
    if int(status.item()) != 0:
        raise SystemExit("decode reported a corrupt stream")

    sizes = results[-1]["sizes"]
    sel_blob_bytes = sum(sizes[(c, q)] for c, q in enumerate(sel))
    dec_ms = [d for r in results for d in r["decode_ms"]]
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    dec_sorted = sorted(dec_ms)
    dec_median_ms = dec_sorted[len(dec_sorted) // 2]
    # Context, outside the timed steps: the same decode right after a decode of
    # the same blobs.  Inside a step the decode follows the encoder, whose
    # writes have displaced the blobs' lines from the caches, and the decoder
    # re-reads each lane's stream lines several times; right after a decode the
    # re-reads hit.
    tab_last = results[-1]["tab"]
    blobs_last = [bufs[(c, q)][: sizes[(c, q)]] for c, q in enumerate(sel)]
    infos_last = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in blobs_last]
    rep_ms = []
    for i in range(args.repeat_decodes + 1 if args.repeat_decodes > 0 else 0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, stream)
        e0.record(stream)
        cg.cg_decode_async(tab_last, blobs_last, infos_last, ko, vo, status)
        e1.record(stream)
        torch.cuda.synchronize()
        if i:
            rep_ms.append(e0.elapsed_time(e1))
    if int(status.item()) != 0:
        raise SystemExit("repeated decode reported a corrupt stream")
    rep_avg_ms = sum(rep_ms) / len(rep_ms) if rep_ms else None
    copy_gbps = copy_bandwidth(torch, dev, stream)
    value = fp16_bytes / (dec_avg_ms * 1e-3) / 1e9
    achieved = (fp16_bytes + sel_blob_bytes) / (dec_avg_ms * 1e-3) / 1e9
    enc_ms = sum(r["encode_ms"] for r in results) / len(results)
    build_ms = sum(r["build_ms"] for r in results) / len(results)
    step_ms = t_all * 1e3 / args.steps
    all_blob_bytes = sum(sizes.values())
    nq = len(w.qualities)
    tables_bytes = len(cg.cg_tables_serialize(results[-1]["tab"]))
    eight_bit = elements  # one byte per element
    ratio = eight_bit / sel_blob_bytes
    ratio_q = {("HML"[q]): eight_bit / sum(sizes[(c, q)] for c in range(nch)) for q in w.qualities}

    traffic = decode_traffic(args.traffic_json, w.name)
    # delta symbols per lane-wave of the decode launch: every chunk of the selection
    wave_symbols = 0
    for c in range(nch):
        tc = min(w.chunk_tokens, w.tokens - c * w.chunk_tokens)
        wave_symbols += 2 * w.layers * (tc - (tc + w.group_tokens - 1) // w.group_tokens) * w.channels // 64
    valu = decode_valu(args.traffic_json, w.name, wave_symbols)
    # algorithmic bytes of the other two steps: every encoded blob reads its
    # chunk's fp16 K/V once and writes the blob; building reads K/V twice
    # (statistics, then the histogram)
    chunk_elems = {c: 2 * w.layers * min(w.chunk_tokens, w.tokens - c * w.chunk_tokens) * w.channels
                   for c in range(nch)}
    enc_bytes = sum(2 * chunk_elems[c] + n for (c, q), n in sizes.items())
    enc_achieved = enc_bytes / (enc_ms * 1e-3) / 1e9
    build_achieved = 2 * fp16_bytes / (build_ms * 1e-3) / 1e9

    cpu = cpu_enc = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, k, v, results[-1]["tab"], bufs, sizes, sel, args.cpu_sample_seconds)
        cpu_enc = cpu_baseline_encode(w, k, v, results[-1]["tab"], args.cpu_sample_seconds / 2)

    line = {
        "metric": ("decode GB/s (fp16 KV out) + compress ratio vs 8-bit, Mistral-7B-shape 9K tok"
                   if w.name == "mistral7b_9k" else
                   f"decode GB/s (fp16 KV out) + compress ratio vs 8-bit, {w.name}"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic (seeded AR(1) K/V with lognormal channel scales)",
        "config": {"workload": w.name, "layers": w.layers, "tokens": w.tokens,
                   "channels": w.channels, "chunk_tokens": w.chunk_tokens,
                   "group_tokens": w.group_tokens, "chunks": nch,
                   "decode_selection": ",".join("HML"[q] for q in sel)},
        "compress_ratio_vs_8bit": round(ratio, 4),
        "compress_ratio_vs_8bit_with_tables": round(eight_bit / (sel_blob_bytes + tables_bytes), 4),
        "compress_ratio_by_quality": {q: round(r, 4) for q, r in ratio_q.items()},
        "selection_blob_bytes": sel_blob_bytes,
        "decode_ms": round(dec_avg_ms, 4),
        "decode_ms_median": round(dec_median_ms, 4),
        "decode_ms_min": round(dec_sorted[0], 4),
        "decode_GBps_algorithmic": round(achieved, 2),
        "encode_ms_all_chunks_all_qualities": round(enc_ms, 3),
        "encode_GBps_fp16_in": round(nq * fp16_bytes / (enc_ms * 1e-3) / 1e9, 2),
        "build_tables_ms": round(build_ms, 3),
        "build_tables_GBps_fp16_in": round(fp16_bytes / (build_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": decode_kernel_name(sel), "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "copy_GBps": round(copy_gbps, 1), "frac_of_copy": round(achieved / copy_gbps, 4),
                     "valu_issue": valu,
                     "repeat_decode_ms": round(rep_avg_ms, 4) if rep_avg_ms else None,
                     "repeat_frac": round((fp16_bytes + sel_blob_bytes) / (rep_avg_ms * 1e-3) / 1e9
                                          / HBM_PEAK_GBPS, 4) if rep_avg_ms else None},
        "cpu_baseline": cpu,
        "encode_roofline": {"bound": "hbm", "kernel": f"k_encode + k_pack (all {len(sizes)} blobs)",
                            "achieved": round(enc_achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(enc_achieved / HBM_PEAK_GBPS, 4)},
        "build_roofline": {"bound": "hbm", "kernel": "cg_build_tables (all kernels)",
                           "achieved": round(build_achieved, 2), "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": round(build_achieved / HBM_PEAK_GBPS, 4)},
        "cpu_baseline_encode": cpu_enc,
        "input_generation_s": round(t_gen, 2),
        "versions": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                     "device": torch.cuda.get_device_name(0)},
    }
    if not args.no_anchor_coded:
        line["anchor_coded"] = anchor_coded_figures(w, kd, vd, args.other_steps, 1, sel_blob_bytes,
                                                    dec_avg_ms, enc_ms, build_ms)
    if w.name == "mistral7b_9k" and not args.no_other_workloads:
        # the other workloads' figures, each in its own memory: the metric's
        # tensors are freed first
        del kd, vd, ko, vo, bufs, results, step, tab_last, blobs_last
        torch.cuda.empty_cache()
        line["workloads"] = {}
        for name in ("tiny", "llama7b", "llama34b_80k", "llama70b_16k"):
            print(f"bench: {name}", file=sys.stderr, flush=True)
            line["workloads"][name] = other_workload(name, args.other_steps, 1,
                                                     0.0 if args.no_cpu_baseline
                                                     else args.other_cpu_seconds)
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


def anchor_coded_figures(w, kd, vd, steps, warmup, raw_sel_bytes, raw_dec_ms, raw_enc_ms,
                         raw_build_ms):
    """The same step with coded anchors (tables version 2, blobs version 3):
    the selection's bytes and compression ratio, and the decode (anchor streams
    first, then the delta streams), encode and build times, beside the raw-anchor
    figures of the main line."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask,
                       anchor_coding=1)
    step, bufs, ko, vo, status = make_stepper(w, p, kd, vd)
    for _ in range(warmup):
        step()
    res = [step() for _ in range(steps)]
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit("coded-anchor decode reported a corrupt stream")
    sizes = res[-1]["sizes"]
    sel = w.selection()
    sel_bytes = sum(sizes[(c, q)] for c, q in enumerate(sel))
    dec = [d for r in res for d in r["decode_ms"]]
    dec_ms = sum(dec) / len(dec)
    enc_ms = sum(r["encode_ms"] for r in res) / len(res)
    build_ms = sum(r["build_ms"] for r in res) / len(res)
    fp16 = 2 * w.elements
    del bufs, ko, vo
    return {
        "format": "tables version 2, blobs version 3 (anchors range-coded per (kv, layer))",
        "selection_blob_bytes": sel_bytes,
        "bytes_vs_raw_anchors": round(sel_bytes / raw_sel_bytes, 4),
        "compress_ratio_vs_8bit": round(w.elements / sel_bytes, 4),
        "decode_ms": round(dec_ms, 4),
        "decode_ms_raw_anchors": round(raw_dec_ms, 4),
        "decode_frac": round((fp16 + sel_bytes) / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "encode_ms_all_chunks_all_qualities": round(enc_ms, 3),
        "encode_ms_raw_anchors": round(raw_enc_ms, 3),
        "build_tables_ms": round(build_ms, 3),
        "build_tables_ms_raw_anchors": round(raw_build_ms, 3),
        "steps": steps,
    }


def make_stepper(w, p, kd, vd, decode_reps=1):
    """One step of the hot path on workload w, K/V already in device memory:
    build the tables, encode every chunk at every quality the workload builds
    (one cg_encode_batch call), decode the selection (one cg_decode_async call,
    decode_reps times).  Each part is timed with HIP events on the launch
    stream; a spin kernel queued ahead of each decode makes its event pair
    bracket the launch's GPU time only.  Returns (step, blob buffers, K out,
    V out, status word)."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    dev = kd.device
    stream = torch.cuda.current_stream()
    sel = w.selection()
    nch = w.n_chunks
    # output buffers, allocated once: one blob buffer per (chunk, quality)
    tab0 = cg.cg_build_tables(p, kd, vd)
    bufs = {(c, q): torch.empty(cg.cg_encode_bound(tab0, c), dtype=torch.uint8, device=dev)
            for c in range(nch) for q in w.qualities}
    del tab0
    ko = torch.empty_like(kd)
    vo = torch.empty_like(vd)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(timed: bool = True):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 + 2 * decode_reps)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        tab = cg.cg_build_tables(p, kd, vd)
        ev[1].record(stream)
        jobs = [(c, q) for c in range(nch) for q in w.qualities]
        lens = cg.cg_encode_batch(tab, kd, vd, [j[0] for j in jobs], [j[1] for j in jobs],
                                  [bufs[j] for j in jobs])
        sizes = dict(zip(jobs, lens))
        ev[2].record(stream)
        blobs = [bufs[(c, q)][: sizes[(c, q)]] for c, q in enumerate(sel)]
        infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in blobs]
        for r in range(decode_reps):
            queue_ahead(torch, stream)
            ev[3 + 2 * r].record(stream)
            cg.cg_decode_async(tab, blobs, infos, ko, vo, status)
            ev[4 + 2 * r].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dec = [ev[3 + 2 * r].elapsed_time(ev[4 + 2 * r]) for r in range(decode_reps)]
        return dict(wall_ms=wall * 1e3, build_ms=ev[0].elapsed_time(ev[1]),
                    encode_ms=ev[1].elapsed_time(ev[2]), decode_ms=dec, sizes=sizes, tab=tab)

    return step, bufs, ko, vo, status


def chunk_elements(w, c):
    """K and V elements of chunk c."""
    return 2 * w.layers * min(w.chunk_tokens, w.tokens - c * w.chunk_tokens) * w.channels


def other_workload(name, steps, warmup, cpu_seconds):
    """The same step on another workload: decode, encode and build times and
    their fractions of the HBM roofline (algorithmic bytes: decode = selection
    blob bytes + fp16 written; encode = fp16 read per blob + blob written;
    build = two reads of K and V), the compression ratios, and the oracle on
    a bounded sample of the same blobs and chunks on this host's cores.  The
    streamed workload also times the chunk pipeline (H2D alone, decode alone,
    both overlapped on two streams)."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    w = synth.workload(name)
    t_gen = time.time()
    k, v = synth.gen_kv(w)
    t_gen = time.time() - t_gen
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    step, bufs, ko, vo, status = make_stepper(w, p, kd, vd)
    for _ in range(warmup):
        step()
    res = [step() for _ in range(steps)]
    if int(status.item()) != 0:
        raise SystemExit(f"{name}: decode reported a corrupt stream")
    sel = w.selection()
    sizes = res[-1]["sizes"]
    sel_bytes = sum(sizes[(c, q)] for c, q in enumerate(sel))
    fp16 = 2 * w.elements
    dec = sum(d for r in res for d in r["decode_ms"]) / sum(len(r["decode_ms"]) for r in res)
    enc = sum(r["encode_ms"] for r in res) / len(res)
    bld = sum(r["build_ms"] for r in res) / len(res)
    enc_bytes = sum(2 * chunk_elements(w, c) + n for (c, q), n in sizes.items())
    tables_bytes = len(cg.cg_tables_serialize(res[-1]["tab"]))
    frac = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    out = {
        "shape": [w.layers, w.tokens, w.channels], "chunks": w.n_chunks,
        "decode_selection": ",".join("HML"[q] for q in sel),
        "decode_kernel": decode_kernel_name(sel),
        "decode_ms": round(dec, 4), "decode_GBps_fp16_out": round(fp16 / (dec * 1e-3) / 1e9, 2),
        "decode_frac": frac(fp16 + sel_bytes, dec),
        "encode_ms": round(enc, 4), "encode_blobs": len(sizes), "encode_frac": frac(enc_bytes, enc),
        "build_ms": round(bld, 4), "build_frac": frac(2 * fp16, bld),
        "compress_ratio_vs_8bit": round(w.elements / sel_bytes, 4),
        "compress_ratio_vs_8bit_with_tables": round(w.elements / (sel_bytes + tables_bytes), 4),
        "input_generation_s": round(t_gen, 2),
    }
    tab_bytes = cg.cg_tables_serialize(res[-1]["tab"])
    blobs = [(c, bufs[(c, q)][: sizes[(c, q)]].cpu().numpy().tobytes()) for c, q in enumerate(sel)]
    if w.streamed:
        out["pipeline"] = pipeline_figures(w, res[-1]["tab"], [b for _, b in blobs], steps, warmup)
    del kd, vd, ko, vo, bufs, res
    torch.cuda.empty_cache()
    out["cpu_baseline"] = oracle_sample(w, k, v, tab_bytes, blobs, cpu_seconds)
    return out


def oracle_sample(w, k, v, tab_bytes, blobs, seconds):
    """The oracle decoding the selection's blobs in turn, and encoding its chunks
    in turn, each for about `seconds` (at least one chunk each) on this host's
    cores: GB/s of fp16 written, and of fp16 read."""
    import numpy as np

    import oracle
    threads, host = cpu_threads()
    ko = np.zeros_like(k)  # pages only the decoded chunks' rows touch are backed
    vo = np.zeros_like(v)
    n = elems = 0
    t0 = time.perf_counter()
    while True:
        c, b = blobs[n % len(blobs)]
        oracle.decode_blob(tab_bytes, b, ko, vo, threads=threads)
        elems += chunk_elements(w, c)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    dec = 2 * elems / dt / 1e9
    sel = w.selection()
    m = e_elems = 0
    t0 = time.perf_counter()
    while True:
        c = m % w.n_chunks
        oracle.encode_chunk(tab_bytes, k, v, c, int(sel[c]), threads=threads)
        e_elems += chunk_elements(w, c)
        m += 1
        de = time.perf_counter() - t0
        if de >= seconds:
            break
    return {"decode_GBps_fp16_out": round(dec, 4), "encode_GBps_fp16_in": round(2 * e_elems / de / 1e9, 4),
            "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle decode of {n} chunk blobs ({dt:.1f} s), encode of {m} chunks "
                      f"({de:.1f} s)", **host}


def pipeline_figures(w, tab, blobs, steps, warmup):
    """Chunk pipeline: blobs in pinned host memory copied to a 3-slot device
    staging buffer on one stream and decoded on another (cg_decode_streamed).
    Mean times (HIP events) of the copies alone, the decode of the same blobs
    from device memory, and the overlapped pipeline; PCIe-inclusive, not the
    decode throughput."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    host = [torch.frombuffer(bytearray(b), dtype=torch.uint8).pin_memory() for b in blobs]
    dev = [h.cuda() for h in host]
    infos = [cg.cg_chunk_info_parse(h[:64]) for h in host]
    ko = torch.empty((w.layers, w.tokens, w.channels), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    sizes = [h.numel() for h in host]
    slot = max((n + 255) // 256 * 256 for n in sizes)
    stage = torch.empty(3 * slot, dtype=torch.uint8, device="cuda")
    cs, ks = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn, stream_start, stream_end):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_start)
        fn()
        e1.record(stream_end)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def h2d():
        with torch.cuda.stream(cs):
            for i, h in enumerate(host):
                stage[(i % 3) * slot:(i % 3) * slot + h.numel()].copy_(h, non_blocking=True)

    def dec():
        with torch.cuda.stream(ks):
            cg.cg_decode_async(tab, dev, infos, ko, vo, st, stream=ks)

    def pipe():
        ks.wait_stream(cs)
        cg.cg_decode_streamed(tab, host, infos, ko, vo, stage, st, cs, ks)

    res = {"h2d": [], "decode": [], "pipeline": []}
    for it in range(warmup + steps):
        a = timed(h2d, cs, cs)
        b = timed(dec, ks, ks)
        c = timed(pipe, cs, ks)
        if it >= warmup:
            res["h2d"].append(a)
            res["decode"].append(b)
            res["pipeline"].append(c)
    if int(st.item()) != 0:
        raise SystemExit("streamed decode reported a corrupt stream")
    ms = {key: sum(val) / len(val) for key, val in res.items()}
    blob_bytes = sum(sizes)
    out_bytes = 2 * w.elements
    return {"blob_bytes": blob_bytes, "staging_slots": 3,
            "h2d_ms": round(ms["h2d"], 3), "h2d_GBps": round(blob_bytes / (ms["h2d"] * 1e-3) / 1e9, 2),
            "decode_only_ms": round(ms["decode"], 3),
            "overlapped_ms": round(ms["pipeline"], 3),
            "overlapped_GBps_fp16_out": round(out_bytes / (ms["pipeline"] * 1e-3) / 1e9, 2),
            "overlap": round((ms["h2d"] + ms["decode"]) / ms["pipeline"], 3)}


def stream_context_lib(sizes, decode_ms, slo_ms, send, prior_bpms, policy="adaptive"):
    """One context streamed chunk by chunk over a simulated link, each chunk's
    version chosen by the library (cg_plan_chunk) from the throughput the
    previous chunk saw.  sizes[c][q] / decode_ms[c][q]: bytes and decode time of
    chunk c at version q (H, M, L); send(nbytes) -> ms on the link (advances its
    clock).  Decoding of a chunk overlaps the transfer of the later ones.
    Returns (load time in ms, versions)."""
    import kv_cache_compression_anchor_amd as cg
    n = len(sizes)
    t = 0.0
    decoded = 0.0
    bw = prior_bpms
    versions = []
    for c in range(n):
        if policy == "adaptive":
            left = [sum(int(sizes[j][q]) for j in range(c, n)) for q in range(3)]
            dleft = [sum(float(decode_ms[j][q]) for j in range(c, n)) for q in range(3)]
            q, _ = cg.cg_plan_chunk(slo_ms - t, bw, left, dleft)
        else:
            q = "HML".index(policy)
        dt = send(int(sizes[c][q]))
        t += dt
        bw = int(sizes[c][q]) / dt
        decoded = max(decoded, t) + float(decode_ms[c][q])
        versions.append(q)
    return decoded, versions


def _entropy_bits(counts):
    """Sum over rows of a count matrix of n H(row), in bits: the code length of
    the symbols under each row's own empirical distribution."""
    import numpy as np
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(c > 0, c * np.log2(np.where(c > 0, n / c, 1.0)), 0.0)
    return float(t.sum())


def format_study(args):
    """What the format could still save (the next format variants the pages'
    pipeline suggests: entropy-coded anchors, streams over groups of channels),
    measured on the blobs the GPU codes: every chunk of the workload at quality
    H, anchors read back from the blobs.  The anchors' empirical entropy pooled
    per (kv, layer, channel), per (kv, layer) and globally is what coding them
    with a 256-symbol table of that granularity would approach (tables not
    counted); the lengths' bytes are the per-stream field that channel groups
    would divide."""
    import numpy as np
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    w = synth.workload(args.workload)
    k, v = synth.gen_kv(w)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    tab = cg.cg_build_tables(p, kd, vd)
    q = w.qualities[0]
    chunks = list(range(w.n_chunks))
    outs = [torch.empty(cg.cg_encode_bound(tab, c), dtype=torch.uint8, device="cuda") for c in chunks]
    sizes = cg.cg_encode_batch(tab, kd, vd, chunks, [q] * len(chunks), outs)
    L, C = w.layers, w.channels
    hist = np.zeros((2, L, C, 256), np.int64)
    total = anchors = lengths = streams = 0
    for o, n in zip(outs, sizes):
        b = o[:n].cpu().numpy()
        ng = cg.cg_chunk_info_parse(torch.from_numpy(b[:64].copy())).n_groups
        off_a = 64 + 8 * L
        a = b[off_a:off_a + 2 * L * ng * C].view(np.int8).reshape(2, L, ng, C).astype(np.int64) + 128
        for kv in range(2):
            for l in range(L):
                np.add.at(hist[kv, l], (np.arange(C)[None, :].repeat(ng, 0), a[kv, l]), 1)
        total += n
        anchors += a.size
        lengths += 2 * 2 * L * C
        streams += 2 * L * C
    h_lc = _entropy_bits(hist)
    h_l = _entropy_bits(hist.sum(axis=2))
    h_g = _entropy_bits(hist.sum(axis=(0, 1, 2))[None])
    elems = 2 * L * w.tokens * C
    return {
        "study": "format", "workload": w.name, "quality": "HML"[q], "blob_bytes": int(total),
        "elements": elems, "coded_bits_per_element": round(8 * total / elems, 4),
        "anchors": anchors, "anchor_bits_per_element_now": round(8 * anchors / elems, 4),
        "anchor_entropy_bits": {"per_layer_channel": round(h_lc / anchors, 3),
                                "per_layer": round(h_l / anchors, 3), "global": round(h_g / anchors, 3)},
        "anchor_saving_bits_per_element": {"per_layer_channel": round((8 * anchors - h_lc) / elems, 4),
                                           "per_layer": round((8 * anchors - h_l) / elems, 4),
                                           "global": round((8 * anchors - h_g) / elems, 4)},
        "anchor_saving_fraction_of_blobs": {"per_layer": round((8 * anchors - h_l) / 8 / total, 4)},
        "per_layer_tables_bytes": 2 * L * 256 * 2,
        "per_layer_channel_tables_bytes": 2 * L * C * 256 * 2,
        "streams": streams, "length_field_bytes": lengths,
        "length_fraction_of_blobs": round(lengths / total, 4),
    }


def grouping(args):
    """Table granularity (CacheGen blog, section 1: symbol probabilities counted
    per layer-channel combination): every chunk of the workload encoded at every
    quality with tables pooled per (layer, channel), per layer, per channel and
    globally (cg_build_tables_grouped), and with per-(layer, channel) tables
    profiled on another context of the same synthetic model (same channel
    scales, another token sequence); total coded bytes of each, on the GPU."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    w = synth.workload(args.workload)
    k, v = synth.gen_kv(w)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    jobs = [(c, q) for c in range(w.n_chunks) for q in w.qualities]
    tab0 = cg.cg_build_tables(p, kd, vd)
    outs = [torch.empty(cg.cg_encode_bound(tab0, c), dtype=torch.uint8, device="cuda")
            for c, q in jobs]
    del tab0

    def coded(tab):
        lens = cg.cg_encode_batch(tab, kd, vd, [c for c, q in jobs], [q for c, q in jobs], outs)
        by_q = {n: sum(b for (c, q), b in zip(jobs, lens) if q == i) for i, n in enumerate("HML")
                if i in w.qualities}
        return int(sum(lens)), by_q

    names = {cg.CG_GROUP_LAYER_CHANNEL: "layer_channel", cg.CG_GROUP_LAYER: "layer",
             cg.CG_GROUP_CHANNEL: "channel", cg.CG_GROUP_GLOBAL: "global"}
    res = {}
    for g, name in names.items():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tab = cg.cg_build_tables_grouped(p, g, kd, vd)
        build_ms = (time.perf_counter() - t0) * 1e3
        total, by_q = coded(tab)
        res[name] = {"bytes": total, "bytes_by_quality": by_q, "build_ms": round(build_ms, 3)}
    ko, vo = synth.gen_kv(w, context=1)
    other = cg.cg_build_tables(p, torch.from_numpy(ko).cuda(), torch.from_numpy(vo).cuda())
    total, by_q = coded(other)
    res["layer_channel_other_context"] = {"bytes": total, "bytes_by_quality": by_q}
    base = res["layer_channel"]["bytes"]
    for r in res.values():
        r["vs_layer_channel"] = round(r["bytes"] / base, 4)
        r["bits_per_element"] = round(8 * r["bytes"] / (w.elements * len(w.qualities)), 4)
    line = {
        "metric": "coded size with per-(layer, channel) tables vs pooled tables",
        "value": round(res["global"]["bytes"] / base - 1.0, 4),
        "unit": "extra coded bytes with one global table, fraction",
        "n_gpus": 1,
        "higher_is_better": None,
        "vs_baseline": None,
        "data": "synthetic K/V (synth); other context: synth context=1 (same channel scales)",
        "config": {"workload": w.name, "chunks": w.n_chunks,
                   "qualities": "".join("HML"[q] for q in w.qualities)},
        "results": res,
    }
    print(json.dumps(line), flush=True)


def adaptive(args):
    """Bandwidth-adaptive streaming (CacheGen blog 2.2) on the workload: every
    chunk encoded at H, M and L on the GPU; each blob's decode time measured
    alone (HIP events, median of 5); then --contexts contexts streamed over a
    simulated link whose bandwidth fluctuates around 3 Gbit/s (synth.netsim,
    50 ms steps), one context every 2.5 s of the trace, under the fixed
    versions and under the library's per-chunk choice.  The SLO is set from the
    context's H size: SLO = f * (H bytes at the mean bandwidth) for f in 0.9,
    1.0, 1.2.  The chosen versions of one context are then decoded together on
    the GPU and checked for a clean status."""
    import numpy as np
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    from synth.netsim import Link, bandwidth_trace
    w = synth.workload(args.workload)
    if len(w.qualities) != 3:
        raise SystemExit(f"{w.name} builds only {len(w.qualities)} qualities; --adaptive needs H, M, L")
    k, v = synth.gen_kv(w)
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    tab = cg.cg_build_tables(p, kd, vd)
    nch = w.n_chunks
    jobs = [(c, q) for c in range(nch) for q in range(3)]
    outs = [torch.empty(cg.cg_encode_bound(tab, c), dtype=torch.uint8, device="cuda")
            for c, q in jobs]
    lens = cg.cg_encode_batch(tab, kd, vd, [c for c, q in jobs], [q for c, q in jobs], outs)
    blob = {j: o[:n] for j, o, n in zip(jobs, outs, lens)}
    sizes = [[int(lens[jobs.index((c, q))]) for q in range(3)] for c in range(nch)]
    info = {j: cg.cg_chunk_info_parse(b[:64].cpu()) for j, b in blob.items()}
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    dec_ms = [[0.0] * 3 for _ in range(nch)]
    for (c, q), b in blob.items():
        ts = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, stream)
            e0.record(stream)
            cg.cg_decode_async(tab, [b], [info[(c, q)]], ko, vo, st)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        dec_ms[c][q] = sorted(ts[1:])[2]
    mean_gbps, step_ms, every_ms = 3.0, 50.0, 2500.0
    n_steps = int(args.contexts * every_ms / step_ms) + 4000
    trace = bandwidth_trace(11, n_steps, mean_gbps=mean_gbps)
    mean_bpms = mean_gbps * 1e9 / 8 / 1e3
    h_bytes = sum(sz[0] for sz in sizes)
    results = {}
    mix = None
    sample_versions = None
    for f in (0.9, 1.0, 1.2):
        slo = f * h_bytes / mean_bpms
        res = {}
        for pol in ("H", "M", "L", "adaptive"):
            viol, total, counts = 0, 0.0, [0, 0, 0]
            for i in range(args.contexts):
                link = Link(trace, step_ms, start_ms=i * every_ms)
                t, vs = stream_context_lib(sizes, dec_ms, slo, link.send, mean_bpms, pol)
                viol += t > slo
                total += t
                for q in vs:
                    counts[q] += 1
                if pol == "adaptive" and f == 1.0 and i == 7:
                    sample_versions = vs
            res[pol] = {"violation_rate": round(viol / args.contexts, 4),
                        "mean_load_ms": round(total / args.contexts, 2)}
            if pol == "adaptive":
                res[pol]["version_share"] = {n: round(c / sum(counts), 4) for n, c in zip("HML", counts)}
        results[f"slo_{f:g}x"] = {"slo_ms": round(slo, 2), **res}
    # the chosen versions of one context decode together on the GPU
    sel = [blob[(c, q)] for c, q in enumerate(sample_versions)]
    sinfo = [info[(c, q)] for c, q in enumerate(sample_versions)]
    st.zero_()
    cg.cg_decode_async(tab, sel, sinfo, ko, vo, st)
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise SystemExit("decode of an adaptive selection reported a corrupt stream")
    main = results["slo_1x"]
    line = {
        "metric": "SLO violation rate under a fluctuating 3 Gbit/s link, adaptive versions vs fixed H",
        "value": main["adaptive"]["violation_rate"],
        "unit": "fraction of contexts",
        "n_gpus": 1,
        "higher_is_better": False,
        "vs_baseline": None,
        "data": "synthetic K/V (synth) and synthetic bandwidth trace (synth.netsim, seed 11)",
        "config": {"workload": w.name, "chunks": nch, "contexts": args.contexts,
                   "link": "log-AR(1) bandwidth, mean 3 Gbit/s, 50 ms steps",
                   "bandwidth_estimate": "throughput of the previous chunk (3 Gbit/s prior)"},
        "fixed_H_violation_rate": main["H"]["violation_rate"],
        "chunk_bytes": {n: [sz[q] for sz in sizes] for q, n in enumerate("HML")},
        "decode_ms_per_chunk": {n: [round(d[q], 4) for d in dec_ms] for q, n in enumerate("HML")},
        "results": results,
        "sample_adaptive_versions": "".join("HML"[q] for q in sample_versions),
    }
    print(json.dumps(line), flush=True)


def streamed(args):
    """Chunk pipeline on the Llama-70B-shape 16K context (K, V each [80, 16384, 1024]
    fp16, 11 chunks at a seeded H/M/L schedule): blobs in pinned host memory, copied
    to a 3-slot device staging buffer on one stream and decoded on another.  Times
    (HIP events, mean of --steps runs): the copies alone, the decode of the same
    blobs from device memory, and the overlapped pipeline."""
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    w = synth.workload("llama70b_16k")
    k, v = synth.gen_kv(w)
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    tab = cg.cg_build_tables(p, kd, vd)
    sched = list(w.selection())
    outs = [torch.empty(cg.cg_encode_bound(tab, c), dtype=torch.uint8, device="cuda")
            for c in range(len(sched))]
    sizes = cg.cg_encode_batch(tab, kd, vd, list(range(len(sched))), sched, outs)
    blobs = [o[:n].cpu().numpy().tobytes() for o, n in zip(outs, sizes)]
    del outs, kd, vd
    fig = pipeline_figures(w, tab, blobs, args.steps, args.warmup)
    out_bytes = 2 * w.elements
    line = {
        "metric": "chunk pipeline: fp16 KV out GB/s with blobs starting in pinned host memory",
        "value": fig["overlapped_GBps_fp16_out"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": fig["overlapped_ms"], "higher_is_better": True,
        "config": {"workload": w.name, "layers": w.layers, "tokens": w.tokens,
                   "channels": w.channels, "chunks": len(sched),
                   "schedule": ",".join("HML"[q] for q in sched), "staging_slots": 3},
        "fp16_out_bytes": out_bytes,
        "compress_ratio_vs_8bit": round(w.elements / fig["blob_bytes"], 4),
        "decode_GBps_fp16_out": round(out_bytes / (fig["decode_only_ms"] * 1e-3) / 1e9, 2),
        **fig,
    }
    print(json.dumps(line), flush=True)


def paged(args):
    """Decode into paged pools [L, num_pages, P, C] on the --workload selection:
    pages of --page-tokens tokens named by a seeded shuffled block table with
    1/16 spare pages.  Times (HIP events on the launch stream, mean and min of
    --steps runs, each run right after an untimed run of the same variant): the
    decode into [L, T, C], the paged decode, and the [L, T, C]
    decode followed by a copy of its rows into the pages (torch index_put), what a
    caller without the paged entry point would run."""
    import numpy as np
    import torch

    import kv_cache_compression_anchor_amd as cg
    import synth
    w = synth.workload(args.workload)
    P = args.page_tokens
    if w.tokens % P:
        raise SystemExit("--page-tokens must divide the context")
    k, v = synth.gen_kv(w)
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    p = cg.make_params(w.layers, w.tokens, w.channels, w.chunk_tokens, w.group_tokens,
                       w.layer_group_end, w.layer_step, w.quality_mult, w.quality_mask)
    tab = cg.cg_build_tables(p, kd, vd)
    sel = list(w.selection())
    outs = [torch.empty(cg.cg_encode_bound(tab, c), dtype=torch.uint8, device="cuda")
            for c in range(len(sel))]
    sizes = cg.cg_encode_batch(tab, kd, vd, list(range(len(sel))), sel, outs)
    blobs = [o[:n] for o, n in zip(outs, sizes)]
    infos = [cg.cg_chunk_info_parse(b[:64].cpu()) for b in blobs]
    del kd, vd
    nb = w.tokens // P
    n_pages = nb + nb // 16
    table_h = np.random.default_rng(12345).permutation(n_pages)[:nb].astype(np.int32)
    table = torch.from_numpy(table_h).cuda()
    idx = table.long()
    ko = torch.empty((w.layers, w.tokens, w.channels), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    kp = torch.zeros((w.layers, n_pages, P, w.channels), dtype=torch.float16, device="cuda")
    vp = torch.zeros_like(kp)
    kq, vq = torch.zeros_like(kp), torch.zeros_like(vp)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, stream)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def flat():
        cg.cg_decode_async(tab, blobs, infos, ko, vo, st)

    def pg():
        cg.cg_decode_paged_async(tab, blobs, infos, kp, vp, P, table, st)

    def flat_then_copy():
        cg.cg_decode_async(tab, blobs, infos, ko, vo, st)
        kq[:, idx] = ko.view(w.layers, nb, P, w.channels)
        vq[:, idx] = vo.view(w.layers, nb, P, w.channels)

    # Each timed call follows an untimed call of the same variant: a decode runs
    # faster when the blobs' lines are still in the caches from a decode just
    # before it than after the copy's 1.2 GB of writes, so without this the
    # order of the variants would decide their comparison.
    def again(fn):
        fn()
        return timed(fn)

    res = {"flat": [], "paged": [], "flat_then_copy": []}
    for it in range(args.warmup + args.steps):
        a, b, c = again(flat), again(pg), again(flat_then_copy)
        if it >= args.warmup:
            res["flat"].append(a)
            res["paged"].append(b)
            res["flat_then_copy"].append(c)
    if int(st.item()) != 0:
        raise SystemExit(f"decode reported status {int(st.item())}")
    # the paged pools hold the [L, T, C] decode's rows where the table says
    same = bool(torch.equal(kp[:, idx].view(torch.int16), ko.view(w.layers, nb, P, w.channels).view(torch.int16))
                and torch.equal(vp[:, idx].view(torch.int16), vo.view(w.layers, nb, P, w.channels).view(torch.int16)))
    if not same:
        raise SystemExit("paged pools differ from the [L, T, C] decode")
    mean = {key: sum(x) / len(x) for key, x in res.items()}
    low = {key: min(x) for key, x in res.items()}
    out_bytes = 2 * w.elements
    alg = sum(sizes) + out_bytes
    line = {
        "metric": "paged decode: fp16 KV out GB/s (into pages through a block table)",
        "value": round(out_bytes / (mean["paged"] * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(mean["paged"], 4), "higher_is_better": True,
        "config": {"workload": w.name, "selection": ",".join("HML"[q] for q in sel),
                   "page_tokens": P, "blocks": nb, "pages": n_pages},
        "kernel": decode_kernel_name(sel) + " (paged instance)",
        "paged_ms": round(mean["paged"], 4), "paged_min_ms": round(low["paged"], 4),
        "flat_ms": round(mean["flat"], 4), "flat_min_ms": round(low["flat"], 4),
        "paged_over_flat": round(mean["paged"] / mean["flat"], 4),
        "flat_then_copy_ms": round(mean["flat_then_copy"], 4),
        "paged_roofline_frac": round(alg / (mean["paged"] * 1e-3) / 8e12, 4),
        "pools_equal_flat_decode": same,
    }
    print(json.dumps(line), flush=True)


DECODE_SOURCES = ["kv_cache_compression_anchor_amd/csrc/cg_decode.hip",
                  "kv_cache_compression_anchor_amd/csrc/cg_internal.h"]


def decode_kernel_name(sel):
    """The decoder kernel one cg_decode_async of the selection launches: the
    LDS-window kernel when some quality holds several chunks (workgroups of
    several chunks), else the register-buffer kernel."""
    return "k_decode_win" if any(sel.count(q) > 1 for q in set(sel)) else "k_decode_reg"


def decode_traffic(path, workload):
    """HBM bytes per decode launch from the committed FETCH_SIZE / WRITE_SIZE
    counter runs (scaled by the same counters on a plain copy of known size);
    None when there is no record for the workload or the decoder changed since."""
    try:
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != decoder_source_sha256():
            return None
        return int(rec["workloads"][workload]["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def _load_record(path):
    """The counter record for the decoder source as it is now (a fresh one if
    the file is missing or was taken on another version of the decoder)."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        rec = {}
    sha = decoder_source_sha256()
    if rec.get("kernel_source_sha256") != sha:
        rec = {"kernel": "k_decode_win / k_decode_reg", "kernel_source_sha256": sha, "workloads": {}}
    return rec


def record_valu(path, workload, counter_csvs, agent_csv):
    """Store the decoder's VALU issue for `workload`: SQ_INSTS_VALU and
    GRBM_GUI_ACTIVE per decoder dispatch (averaged over its dispatches; with
    SQ_INSTS_LDS and SQ_LDS_BANK_CONFLICT when the files hold them), the
    dispatch's duration from its timestamps, and the device's SIMD and XCD
    counts and peak engine clock from the agent file.  A wave64 VALU
    instruction takes 4 cycles of its SIMD, so
    busy = instructions x 4 / (SIMDs x GRBM cycles per XCD)."""
    import csv
    dec = "void cg::(anonymous namespace)::k_decode_"
    per = {}   # (dispatch, counter) -> value
    dur = {}   # dispatch -> ns
    for p in counter_csvs:
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                if not r["Kernel_Name"].startswith(dec):
                    continue
                d = int(r["Dispatch_Id"])
                key = (d, r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                dur[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])

    def mean(name):
        v = [x for (d, c), x in per.items() if c == name]
        if not v:
            raise SystemExit(f"record-valu: no {name} for the decoder in the counter files")
        return sum(v) / len(v)

    insts, grbm = mean("SQ_INSTS_VALU"), mean("GRBM_GUI_ACTIVE")
    lds = {c: mean(c) for c in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")
           if any(k[1] == c for k in per)}
    launch_ns = sum(dur.values()) / len(dur)
    agent = None
    with open(agent_csv, newline="") as f:
        for r in csv.DictReader(f):
            if int(r.get("Simd_Count") or 0) > 0:
                agent = r
                break
    if agent is None:
        raise SystemExit("record-valu: no GPU agent in the agent file")
    simds, xcc = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    peak_ghz = int(agent["Max_Engine_Clk_Fcompute"]) / 1000.0
    cycles = grbm / xcc
    rec = _load_record(path)
    rec.setdefault("workloads", {}).setdefault(workload, {})["valu"] = {
        "valu_insts_per_launch": insts,
        "launch_ns": launch_ns,
        "cycles_per_launch": cycles,
        "simds": simds,
        "busy_frac": insts * 4 / (simds * cycles),
        "clock_GHz": cycles / launch_ns,
        "peak_clock_GHz": peak_ghz,
        "issue_frac_at_peak_clock": insts * 4 / (simds * peak_ghz * launch_ns),
    }
    if lds:
        rec["workloads"][workload]["valu"]["lds_insts_per_launch"] = lds.get("SQ_INSTS_LDS")
        rec["workloads"][workload]["valu"]["lds_bank_conflict_cycles_per_launch"] = lds.get("SQ_LDS_BANK_CONFLICT")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["workloads"][workload]["valu"]))


def decode_valu(path, workload, wave_symbols):
    """The committed VALU-issue record of the decoder for `workload` (None when
    there is none or the decoder changed since), with VALU instructions per
    delta symbol of a lane for a launch of `wave_symbols` wave-symbols."""
    try:
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != decoder_source_sha256():
            return None
        v = dict(rec["workloads"][workload]["valu"])
    except (OSError, ValueError, KeyError):
        return None
    out = {k: round(v[k], 4) for k in ("busy_frac", "clock_GHz", "peak_clock_GHz", "issue_frac_at_peak_clock")}
    out["insts_per_symbol"] = round(v["valu_insts_per_launch"] / wave_symbols, 2) if wave_symbols else None
    if v.get("lds_insts_per_launch") is not None and wave_symbols:
        out["lds_insts_per_symbol"] = round(v["lds_insts_per_launch"] / wave_symbols, 2)
    if v.get("lds_bank_conflict_cycles_per_launch") is not None:
        out["lds_bank_conflict_cycles"] = v["lds_bank_conflict_cycles_per_launch"]
    return out


def decoder_source_sha256():
    import hashlib
    src = b"".join(open(os.path.join(ROOT, p), "rb").read() for p in DECODE_SOURCES)
    return hashlib.sha256(src).hexdigest()


def _counter_per_dispatch(csv_path, kernel_prefix):
    """{dispatch id: counter value summed over the rows of that dispatch} for
    the dispatches whose kernel name starts with kernel_prefix."""
    import csv
    out = {}
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Kernel_Name"].startswith(kernel_prefix):
                d = int(r["Dispatch_Id"])
                out[d] = out.get(d, 0.0) + float(r["Counter_Value"])
    return out


def record_traffic(path, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Store the decoder's HBM bytes per launch for `workload`: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, averaged over the decoder's dispatches), each
    scaled so that the same counter reads the true byte count of a plain copy
    (the largest copy dispatches of a --copy-calibration run)."""
    dec = "void cg::(anonymous namespace)::k_decode_"
    fk = list(_counter_per_dispatch(fetch_csv, dec).values())
    wk = list(_counter_per_dispatch(write_csv, dec).values())
    cf = list(_counter_per_dispatch(copy_fetch_csv, "__amd_rocclr_copyBuffer").values())
    cw = list(_counter_per_dispatch(copy_write_csv, "__amd_rocclr_copyBuffer").values())
    if not (fk and wk and cf and cw):
        raise SystemExit("record-traffic: a counter file holds no decoder or copy dispatch")
    copy_bytes = 1 << 30
    cf_kib, cw_kib = max(cf), max(cw)
    fetch_scale = copy_bytes / 1024 / cf_kib
    write_scale = copy_bytes / 1024 / cw_kib
    f_kib, w_kib = sum(fk) / len(fk), sum(wk) / len(wk)
    rec = _load_record(path)
    rec["copy_calibration"] = {"bytes": copy_bytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                               "fetch_scale": fetch_scale, "write_scale": write_scale}
    rec.setdefault("workloads", {}).setdefault(workload, {}).update({
        "dispatches": len(fk),
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "bytes_per_launch": int(round(1024 * (f_kib * fetch_scale + w_kib * write_scale))),
    })
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["workloads"][workload]))


# Spin length (GPU clock cycles) of the kernel queued ahead of a timed launch.
_SPIN_CYCLES = 400_000


def queue_ahead(torch, stream):
    """Queues a short spin kernel on stream, so that a start event recorded next
    fires just before the timed launch that follows instead of while the host is
    still preparing that launch (the stream would otherwise be idle, after a
    synchronising call): the event pair then brackets GPU time only."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(_SPIN_CYCLES)


def copy_bandwidth(torch, dev, stream, nbytes=1 << 30, reps=5):
    """HBM bandwidth a plain device-to-device copy reaches on this GPU: bytes read
    plus bytes written per second (torch copy_ of nbytes, HIP events, best of reps)."""
    a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, stream)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del a, b
    return 2 * nbytes / (best * 1e-3) / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Threads for the oracle: every core this process may run on (its CPU
    affinity), capped by OMP_NUM_THREADS where the environment sets it (the CPU
    share a job on this host is given); with the host's own counts, so the
    baseline says what it ran on."""
    host = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = host
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(allowed, int(cap)) if cap.isdigit() and int(cap) > 0 else allowed
    return max(1, threads), {"host_cores": host, "affinity_cores": allowed,
                             "omp_num_threads": int(cap) if cap.isdigit() else None}


def cpu_baseline(w, k, v, tab, bufs, sizes, sel, seconds):
    """The oracle decoding the selection (the same blobs the GPU decodes) on this
    host's cores, chunk after chunk, until about `seconds` have passed; GB/s of
    fp16 written."""
    import numpy as np

    import kv_cache_compression_anchor_amd as cg
    import oracle
    threads, host = cpu_threads()
    t = cg.cg_tables_serialize(tab)
    ko = np.zeros_like(k)
    vo = np.zeros_like(v)
    blobs = [bufs[(c, q)][: sizes[(c, q)]].cpu().numpy().tobytes() for c, q in enumerate(sel)]
    n = 0
    tok = 0
    t0 = time.perf_counter()
    while True:
        c = n % len(blobs)
        oracle.decode_blob(t, blobs[c], ko, vo, threads=threads)
        tok += min(w.chunk_tokens, w.tokens - c * w.chunk_tokens)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds and n >= len(blobs):
            break
    out_bytes = 2 * 2 * w.layers * tok * w.channels
    # one thread, on the first blob of the selection
    t1 = time.perf_counter()
    oracle.decode_blob(t, blobs[0], ko, vo, threads=1)
    dt1 = time.perf_counter() - t1
    one = 2 * 2 * w.layers * min(w.chunk_tokens, w.tokens) * w.channels / dt1 / 1e9
    return {"value": round(out_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle decode of {n} chunk blobs of the selection "
                      f"({n // len(blobs)}+ passes, {2 * w.layers * tok * w.channels} elements, "
                      f"{dt:.1f} s)",
            "value_1_thread": round(one, 4), "cpu_model": cpu_model(), **host}


def cpu_baseline_encode(w, k, v, tab, seconds):
    """The oracle encoding chunks of the workload (H, M, L in turn) on this host's
    cores until about `seconds` have passed; GB/s of fp16 read (one chunk's K/V
    per blob)."""
    import kv_cache_compression_anchor_amd as cg
    import oracle
    threads, host = cpu_threads()
    t = cg.cg_tables_serialize(tab)
    n = 0
    elems = 0
    t0 = time.perf_counter()
    while True:
        c = n % w.n_chunks
        q = w.qualities[n % len(w.qualities)]
        oracle.encode_chunk(t, k, v, c, q, threads=threads)
        elems += 2 * w.layers * min(w.chunk_tokens, w.tokens - c * w.chunk_tokens) * w.channels
        n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return {"value": round(2 * elems / dt / 1e9, 4), "unit": "GB/s of fp16 in", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle encode of {n} chunk blobs ({elems} elements, {dt:.1f} s)", **host}


if __name__ == "__main__":
    main()
