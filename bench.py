#!/usr/bin/env python3
"""Throughput of the fused KV encode + decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch: encode the KV
cache of the workload into its blob, then decode the blob back into a KV
tensor.  Inputs are resident in HBM before the timed region starts; two
buffer sets alternate between steps so that consecutive steps do not reuse
cache-resident data.  Prints ONE JSON line.

Reported, all on raw input bytes (the bf16 KV tensor) unless stated:
  value          raw bytes / (encode + decode time), GB/s (1e9)
  encode/decode  per-kernel raw GB/s and algorithmic-HBM GB/s (bytes read
                 plus bytes written) as a fraction of the 8 TB/s peak
  roofline       the dominant kernel: algorithmic bytes per launch / mean
                 launch time (HIP events on the launch stream, recorded
                 without a system-scope fence), vs 8 TB/s
  break_even     encode + decode time vs the wire time the compression saves
                 at 100 and 400 Gbit/s
  pipeline       per-layer chunked encode overlapped with the copy of each
                 chunk to pinned host memory (PCIe standing in for the link),
                 and copy-in overlapped with decode, against the raw copy and
                 the serial encode-then-copy (contiguous workloads)
  unfused        the same encode / decode run as separate kernels that pass
                 fp32 / byte intermediates through HBM (contiguous workloads):
                 times, stage bytes, and the fused kernels' speedup over them
  cpu_baseline   the CPU oracle on a bounded sample of the same workload
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


class TimingEvents:
    """Timing-only HIP events, recorded without a system-scope fence.

    torch's events use the default flags, and recording one performs a
    system-scope release that writes back and invalidates the caches.
    Between two kernels that adds several microseconds to each measured
    kernel and slows the kernel after it.  These events are created with
    hipEventDisableSystemFence (timing stays enabled) in the process's one
    HIP runtime, the one torch and the library use.  The caller synchronizes
    the device before reading them."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        from kv_cache_compression_kvc_amd import _lib
        runtimes = _lib._hip_runtimes()
        if len(runtimes) != 1:
            raise RuntimeError("expected one HIP runtime in the process, found %s" % runtimes)
        h = self._hip = ctypes.CDLL(runtimes[0])
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._check(h.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE), "create")
            self._ev.append(e)

    @staticmethod
    def _check(status, what):
        if status != 0:
            raise RuntimeError("hipEvent %s failed with status %d" % (what, status))

    def record(self, k, stream):
        self._check(self._hip.hipEventRecord(self._ev[k], ctypes.c_void_p(stream.cuda_stream)), "record")

    def ms(self, a, b):
        t = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(t), self._ev[a], self._ev[b]), "elapsed time")
        return t.value

    def close(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama3_8b_4k")
    ap.add_argument("--cpu-sample-chunks", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true", help="skip the separate-kernel comparator")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the transfer legs (they launch the fused kernels on layer chunks)")
    return ap.parse_args()


# the sources the fused encode / decode kernels are built from
FUSED_SOURCES = ["kvc_cursor.h", "kvc_device.h", "kvc_host.cpp", "kvc_inst.hip", "kvc_launch.hip", "kvc_pick.h",
                 "kvc_plan.h"]


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that
    editing a comment does not count as changing the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_compression_kvc_amd", "csrc")
    for name in FUSED_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, "counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)

def _oracle_chunk(args):
    name, layer, tokens = args
    import numpy as np
    import oracle
    from kv_cache_compression_kvc_amd import presets, inputs
    p = presets.preset(name)
    x = np.stack([inputs.as_u16(inputs.kv_chunk(p, layer, kv, (tokens,), device="cpu"))
                  for kv in (0, 1)])[None]                       # [1, 2, T, H, D]
    t0 = time.perf_counter()
    blob, _ = oracle.encode(x, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    oracle.decode(blob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    return x.size * 2, time.perf_counter() - t0


def cpu_baseline(p, chunks):
    import multiprocessing as mp
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    workers = max(1, min(16, os.cpu_count() or 1, chunks))
    tokens = max(1, (1 << 19) // (p.kv_heads * p.head_dim))  # 2 x 2^19 elements per chunk
    jobs = [(p.name, i % max(1, p.layers), tokens) for i in range(chunks)]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_chunk, jobs)
    wall = time.perf_counter() - t0
    raw = sum(r[0] for r in res)
    cpu = sum(r[1] for r in res)
    return {
        "value": raw / wall / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
        "sample": "%d chunks of [1,2,%d,%d,%d] %s (%.0f MiB raw), encode+decode, %.1f s of CPU work, "
                  "%d processes x 1 BLAS thread" % (chunks, tokens, p.kv_heads, p.head_dim, p.dtype,
                                                    raw / 2 ** 20, cpu, workers),
    }


# ---------------------------------------------------------------------------
# Separate-kernel comparator (same results, intermediates through HBM)

def unfused_leg(kvc, p, xs, outs, dsts, a, stream, t_enc, t_dec, raw_bytes):
    import torch
    L, T, H, D = p.layers, p.tokens, p.kv_heads, p.head_dim
    ws_bytes = kvc.unfused_workspace_size(L, T, H, D, p.bits_k, p.bits_v, p.group, p.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=xs[0].device)
    nsets = len(xs)

    def enc(i):
        kvc.encode_unfused(xs[i], p.bits_k, p.bits_v, p.group, seed=p.seed, out=outs[i], workspace=ws)

    def dec(i):
        kvc.decode_unfused(outs[i], xs[i].shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed,
                           out=dsts[i], workspace=ws)
    for i in range(max(1, a.warmup)):
        enc(i % nsets)
        dec(i % nsets)
    torch.cuda.synchronize()
    ev = TimingEvents(3 * a.steps)
    for i in range(a.steps):
        ev.record(3 * i, stream)
        enc(i % nsets)
        ev.record(3 * i + 1, stream)
        dec(i % nsets)
        ev.record(3 * i + 2, stream)
    torch.cuda.synchronize()
    te = sum(ev.ms(3 * i, 3 * i + 1) for i in range(a.steps)) / a.steps / 1e3
    td = sum(ev.ms(3 * i + 1, 3 * i + 2) for i in range(a.steps)) / a.steps / 1e3
    ev.close()
    del ws
    elems = raw_bytes // 2
    bk, bv, G = p.bits_k, p.bits_v, p.group
    # bytes each stage reads + writes, per element (K and V halves averaged)
    b8 = (bk + bv) / 2 / 8
    enc_b = elems * ((2 + 4) + (4 + 4 / G) + (4 + 4 / G + 1) + (1 + b8))
    dec_b = elems * ((b8 + 1) + (1 + 4 / G + 4) + (4 + 2))
    return {"encode_ms": te * 1e3, "decode_ms": td * 1e3,
            "encode_hbm_GBps": enc_b / te / 1e9, "decode_hbm_GBps": dec_b / td / 1e9,
            "encode_bytes": int(enc_b), "decode_bytes": int(dec_b),
            "fused_speedup_encode": te / t_enc, "fused_speedup_decode": td / t_dec,
            "fused_speedup_step": (te + td) / (t_enc + t_dec),
            "stages": "encode: rotate, minmax, quantize, pack, padding; decode: unpack, dequant, unrotate"}


# ---------------------------------------------------------------------------
# Encode overlapped with the transfer (PCIe to pinned host memory as the link)

def pipeline_leg(kvc, p, x, xout, stream, raw_bytes, reps=3, chunk_layers=8):
    import torch
    L, T, H, D = p.layers, p.tokens, p.kv_heads, p.head_dim
    bk, bv, G = p.bits_k, p.bits_v, p.group
    total, _ = kvc.chunked_size(L, T, H, D, bk, bv, G, chunk_layers, p.dtype)
    whole, _ = kvc.encoded_size(L, T, H, D, bk, bv, G, p.dtype)
    host_raw = torch.empty(raw_bytes, dtype=torch.uint8, pin_memory=True)
    host_blob = torch.empty(max(total, whole), dtype=torch.uint8, pin_memory=True)
    dev_blob = torch.empty(max(total, whole), dtype=torch.uint8, device=x.device)
    staging = torch.empty(total, dtype=torch.uint8, device=x.device)
    copy = torch.cuda.Stream()
    xr = x.view(torch.uint8).view(-1)

    def timed(fn, end_stream):
        ts = []
        for i in range(reps + 1):
            torch.cuda.synchronize()
            # torch's default events: the system-scope release at e1 makes the
            # interval end when the copied data is visible to the host
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            copy.wait_stream(stream)
            fn()
            end_stream.wait_stream(copy if end_stream is stream else stream)
            e1.record(end_stream)
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1) / 1e3)
        return sum(ts) / len(ts)

    def send_raw():
        with torch.cuda.stream(copy):
            host_raw.copy_(xr, non_blocking=True)

    def recv_raw():
        with torch.cuda.stream(copy):
            xout.view(torch.uint8).view(-1).copy_(host_raw, non_blocking=True)

    def send_serial():
        kvc.encode(x, bk, bv, G, seed=p.seed, out=dev_blob, stream=stream)
        copy.wait_stream(stream)
        with torch.cuda.stream(copy):
            host_blob[:whole].copy_(dev_blob[:whole], non_blocking=True)

    def recv_serial():
        with torch.cuda.stream(copy):
            dev_blob[:whole].copy_(host_blob[:whole], non_blocking=True)
        stream.wait_stream(copy)
        kvc.decode(dev_blob, x.shape, p.dtype, bk, bv, G, seed=p.seed, out=xout, stream=stream)

    def send_pipe():
        kvc.encode_send(x, bk, bv, G, chunk_layers, host_blob, seed=p.seed, out=dev_blob,
                        compute_stream=stream, copy_stream=copy)

    def recv_pipe():
        kvc.receive_decode(host_blob, x.shape, p.dtype, bk, bv, G, chunk_layers, seed=p.seed, staging=staging,
                           out=xout, compute_stream=stream, copy_stream=copy)
    t_send_raw = timed(send_raw, stream)
    t_recv_raw = timed(recv_raw, stream)
    t_send_serial = timed(send_serial, stream)   # whole blob in host_blob
    t_recv_serial = timed(recv_serial, stream)
    t_send_pipe = timed(send_pipe, stream)       # chunked blob in host_blob
    t_recv_pipe = timed(recv_pipe, stream)
    del host_raw, host_blob, dev_blob, staging

    def rate(t):
        return raw_bytes / t / 1e9
    return {
        "link": "PCIe between device memory and pinned host memory; raw and serial legs copy with "
                "hipMemcpyAsync, the overlapped legs with the library's link-copy kernel",
        "chunk_layers": chunk_layers,
        "link_GBps_d2h": raw_bytes / t_send_raw / 1e9, "link_GBps_h2d": raw_bytes / t_recv_raw / 1e9,
        "send_ms": {"raw": t_send_raw * 1e3, "encode_then_copy": t_send_serial * 1e3,
                    "overlapped": t_send_pipe * 1e3},
        "receive_ms": {"raw": t_recv_raw * 1e3, "copy_then_decode": t_recv_serial * 1e3,
                       "overlapped": t_recv_pipe * 1e3},
        "send_raw_GBps_effective": {"raw": rate(t_send_raw), "encode_then_copy": rate(t_send_serial),
                                    "overlapped": rate(t_send_pipe)},
        "receive_raw_GBps_effective": {"raw": rate(t_recv_raw), "copy_then_decode": rate(t_recv_serial),
                                       "overlapped": rate(t_recv_pipe)},
        "speedup_vs_raw": {"send": t_send_raw / t_send_pipe, "receive": t_recv_raw / t_recv_pipe},
    }


def copy_probe(kvc, dev, stream, reps=40):
    """GB/s (read + write) of a 1 GiB device copy by the library's streaming
    copy kernel, averaged over the last half of `reps` copies."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps // 2):
        kvc.probe_copy(src, dst)
    ev = TimingEvents(2)
    ev.record(0, stream)
    for _ in range(reps - reps // 2):
        kvc.probe_copy(src, dst)
    ev.record(1, stream)
    torch.cuda.synchronize()
    gbps = 2 * src.numel() * (reps - reps // 2) / (ev.ms(0, 1) / 1e3) / 1e9
    ev.close()
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path. Every head_dim "
              "vector is encoded and decoded on its own, so a cache shards by layer, head, "
              "request or token range with no exchange between GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_compression_kvc_amd as kvc
    from kv_cache_compression_kvc_amd import presets, inputs

    p = presets.preset(a.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    D, H, L = p.head_dim, p.kv_heads, p.layers
    nsets = 2

    if p.paged:
        lens = inputs.request_lengths(p)
        table, nb = inputs.block_table(p, lens)
        offs, total = kvc.paged_layout(lens, L, H, D, p.bits_k, p.bits_v, p.group, p.dtype)
        pools = [inputs.make_pool(p, nb, device=dev) for _ in range(nsets)]
        outs = [torch.empty(total, dtype=torch.uint8, device=dev) for _ in range(nsets)]
        dsts = [torch.empty_like(pools[0]) for _ in range(nsets)]
        bt = torch.from_numpy(table).to(dev)
        sl = torch.from_numpy(lens).to(dev)
        of = torch.from_numpy(offs).to(dev)
        tokens = int(lens.sum())
        raw_bytes = L * 2 * tokens * H * D * 2
        enc_bytes = total

        def enc(i):
            kvc.encode_paged(pools[i], bt, sl, of, total, p.bits_k, p.bits_v, p.group, seed=p.seed, out=outs[i])

        def dec(i):
            kvc.decode_paged(outs[i], dsts[i], bt, sl, of, p.bits_k, p.bits_v, p.group, seed=p.seed)
        workload = {"workload": p.name, "layers": L, "requests": len(lens), "tokens": tokens,
                    "kv_heads": H, "head_dim": D, "storage": p.dtype, "bits_k": p.bits_k,
                    "bits_v": p.bits_v, "group": p.group, "layout": "paged, 16-token blocks"}
    else:
        xs = [inputs.make_kv(p, device=dev) for _ in range(nsets)]
        total, _ = kvc.encoded_size(L, p.tokens, H, D, p.bits_k, p.bits_v, p.group, p.dtype)
        outs = [torch.empty(total, dtype=torch.uint8, device=dev) for _ in range(nsets)]
        dsts = [torch.empty_like(xs[0]) for _ in range(nsets)]
        raw_bytes = xs[0].numel() * 2
        enc_bytes = total

        def enc(i):
            kvc.encode(xs[i], p.bits_k, p.bits_v, p.group, seed=p.seed, out=outs[i])

        def dec(i):
            kvc.decode(outs[i], xs[i].shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed, out=dsts[i])
        workload = {"workload": p.name, "shape": [L, 2, p.tokens, H, D], "storage": p.dtype,
                    "bits_k": p.bits_k, "bits_v": p.bits_v, "group": p.group, "layout": "contiguous"}

    algo_bytes = raw_bytes + enc_bytes     # read + write of one encode (or one decode)
    stream = torch.cuda.current_stream()

    # copy probe: achievable streaming bandwidth in the same run.  It runs
    # before the warm-up steps on purpose: after an idle period the GPU needs
    # some tens of milliseconds of load to reach its steady state (the first
    # ~50 encode + decode steps run up to 10% slower), which the probe's
    # copies and the default 50 warm-up steps cover.
    copy_gbps = copy_probe(kvc, dev, stream)

    for i in range(a.warmup):
        enc(i % nsets)
        dec(i % nsets)
    torch.cuda.synchronize()

    ev = TimingEvents(3 * a.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        ev.record(3 * i, stream)
        enc(i % nsets)
        ev.record(3 * i + 1, stream)
        dec(i % nsets)
        ev.record(3 * i + 2, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = sorted(ev.ms(3 * i, 3 * i + 1) for i in range(a.steps))
    dec_ms = sorted(ev.ms(3 * i + 1, 3 * i + 2) for i in range(a.steps))
    ev.close()
    t_enc = sum(enc_ms) / a.steps / 1e3   # s per encode (mean)
    t_dec = sum(dec_ms) / a.steps / 1e3
    ms_per_step = wall / a.steps * 1e3

    unfused = pipeline = None
    if not p.paged and not a.no_unfused:
        unfused = unfused_leg(kvc, p, xs, outs, dsts, a, stream, t_enc, t_dec, raw_bytes)
    if not p.paged and not a.no_pipeline:
        pipeline = pipeline_leg(kvc, p, xs[0], dsts[0], stream, raw_bytes)

    enc_alg = algo_bytes / t_enc / 1e9
    dec_alg = algo_bytes / t_dec / 1e9
    dominant = "encode" if t_enc >= t_dec else "decode"
    t_dom = max(t_enc, t_dec)
    achieved = algo_bytes / t_dom / 1e9
    saved = raw_bytes - enc_bytes
    be = {}
    for gbit in (100, 400):
        wire_saved_s = saved * 8 / (gbit * 1e9)
        be["%dGbit" % gbit] = {"wire_time_saved_ms": wire_saved_s * 1e3,
                               "encode_plus_decode_ms": (t_enc + t_dec) * 1e3,
                               "pays": (t_enc + t_dec) < wire_saved_s,
                               "required_raw_GBps_each": 2 * gbit / 8 / (1 - enc_bytes / raw_bytes)}
    result = {
        "metric": "encode+decode throughput of raw bf16 KV input (GB/s); per-kernel % of HBM peak; "
                  "break-even at 400 Gbit",
        "value": raw_bytes / (t_enc + t_dec) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Gaussian KV with K outlier channels; no model weights)",
        "config": workload,
        "encode": {"raw_GBps": raw_bytes / t_enc / 1e9, "hbm_GBps": enc_alg,
                   "frac_hbm_peak": enc_alg / HBM_PEAK_GBPS, "frac_copy_probe": enc_alg / copy_gbps,
                   "ms": t_enc * 1e3, "ms_median": enc_ms[len(enc_ms) // 2], "ms_min": enc_ms[0]},
        "decode": {"raw_GBps": raw_bytes / t_dec / 1e9, "hbm_GBps": dec_alg,
                   "frac_hbm_peak": dec_alg / HBM_PEAK_GBPS, "frac_copy_probe": dec_alg / copy_gbps,
                   "ms": t_dec * 1e3, "ms_median": dec_ms[len(dec_ms) // 2], "ms_min": dec_ms[0]},
        "bytes": {"raw": raw_bytes, "encoded": enc_bytes, "ratio": raw_bytes / enc_bytes},
        "copy_probe_GBps": copy_gbps,
        "break_even": be,
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic(p.name, dominant),
                     "algorithmic_bytes_per_launch": algo_bytes, "launch_ms": t_dom * 1e3},
        "unfused": unfused,
        "pipeline": pipeline,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, a.cpu_sample_chunks)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
