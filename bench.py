#!/usr/bin/env python3
"""Throughput of the fused KV encode + decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path over one batch: encode the KV
cache of the workload into its blob, then decode the blob back into a KV
tensor.  Inputs are resident in HBM before the timed region starts; two
buffer sets alternate between steps so that consecutive steps do not reuse
cache-resident data.  Prints ONE JSON line.

Warm-up: after an idle period the GPU needs some hundreds of milliseconds
of load to reach its steady clocks, so before the W warm-up steps the
headline workload runs encode + decode back to back for --prewarm-s seconds
of wall time (reported as "prewarm"), whatever W is; the probes run after
the timed steps.  Python's cyclic garbage collector is off for the run and
collects at the start of every pre-warm instead: a full collection stalls
the host for tens of milliseconds, the GPU idles meanwhile, and the steps
after such a stall ran up to 35% slower while the clocks recovered.

Reported, all on raw input bytes (the bf16 KV tensor) unless stated:
  value          raw bytes per step / ms_per_step, GB/s (1e9); ms_per_step is
                 the wall time of the K timed steps / K (device synchronized
                 on both sides)
  encode/decode  per-kernel time (HIP events on the launch stream, mean,
                 median, min), raw GB/s and algorithmic-HBM GB/s (bytes read
                 plus bytes written) as a fraction of the 8 TB/s peak and of
                 the same-mix streaming probe
  probes         the library's streaming probe moving each kernel's bytes in
                 its read:write ratio: what a plain streaming kernel achieves
                 for that mix on this chip
  roofline       the dominant kernel: algorithmic bytes per launch / mean
                 launch time, vs 8 TB/s
  break_even     encode + decode time vs the wire time the compression saves
                 at 100 and 400 Gbit/s
  workloads      every other named workload (tiny as latency; the 8B-32k,
                 70B-16k and paged ones as encode / decode fractions of the
                 peak and break-even), same event protocol, fewer steps; the
                 paged pool is visited in pool order (kvc_paged_order, a host
                 prologue like the offsets), and in request order for
                 comparison
  pipeline       per-layer chunked encode overlapped with the copy of each
                 chunk to pinned host memory (PCIe standing in for the link),
                 and copy-in overlapped with decode, against the raw copy and
                 the serial encode-then-copy (contiguous workloads)
  unfused        the same encode / decode run as separate kernels that pass
                 fp32 / byte intermediates through HBM (contiguous workloads):
                 times, stage bytes, and the fused kernels' speedup over them
  cpu_baseline   the CPU oracle on a bounded sample of the same workload,
                 and the parity of the GPU's encode / decode of one sample
                 chunk against it (boundary flips counted)
"""

import argparse
import ctypes
import gc
import hashlib
import json
import os
import re
import sys
import threading
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

    def pair(self, a, b):
        """Handles of events a and b, for a library call to attach to its first
        kernel's start and its last kernel's end."""
        return self._ev[a], self._ev[b]

    def ms(self, a, b):
        t = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(t), self._ev[a], self._ev[b]), "elapsed time")
        return t.value

    def close(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


class ClockSample:
    """The GPU's clocks during the pre-warm, while back-to-back encodes and
    decodes keep it busy: the amdsmi library's GPU metrics (graphics clock
    of each XCD, memory clock, graphics activity) read from a thread at the
    given offsets in seconds.  Reading is all it does; an error text is
    reported instead if the library or the metrics are unavailable."""

    def __init__(self, offsets_s):
        self.samples, self.error, self._t, self._smi = [], None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no library or no device: report, do not fail the bench
            self.error = "%s: %s" % (type(e).__name__, str(e)[:160])
            return
        self._t = threading.Thread(target=self._run, args=(offsets_s,), daemon=True)
        self._t.start()

    def _run(self, offsets_s):
        num = lambda v: v if isinstance(v, (int, float)) else None
        t0 = time.perf_counter()
        for at in offsets_s:
            time.sleep(max(0.0, at - (time.perf_counter() - t0)))
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            except Exception as e:
                self.error = "%s: %s" % (type(e).__name__, str(e)[:160])
                return
            gfx = m.get("current_gfxclks")
            self.samples.append({
                "at_s": round(time.perf_counter() - t0, 3),
                "gfx_MHz_per_xcd": [v for v in gfx if num(v) is not None] if isinstance(gfx, list) else None,
                "mem_MHz": num(m.get("current_uclk")),
                "gfx_activity_pct": num(m.get("average_gfx_activity"))})

    def get(self, timeout=10.0):
        if self._t is not None:
            self._t.join(timeout)
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        return {"samples": self.samples, "error": self.error, "source": "amdsmi GPU metrics, device 0"}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of back-to-back encode + decode before the warm-up steps")
    ap.add_argument("--workload", default="llama3_8b_4k")
    ap.add_argument("--other-steps", type=int, default=20,
                    help="timed steps of each other workload (0: skip them)")
    ap.add_argument("--other-prewarm-s", type=float, default=0.3,
                    help="seconds of back-to-back encode + decode before each other workload's steps")
    ap.add_argument("--cpu-sample-chunks", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true", help="skip the separate-kernel comparator")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the transfer legs (they launch the fused kernels on layer chunks)")
    ap.add_argument("--no-transform", action="store_true",
                    help="skip the matrix-core / butterfly comparison (it launches the default kernels again)")
    return ap.parse_args(argv)


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
    tokens = sample_tokens(p)
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


def sample_tokens(p):
    return max(1, (1 << 19) // (p.kv_heads * p.head_dim))   # 2 x 2^19 elements per chunk


def sample_parity(kvc, p, dev, layer=0):
    """Criteria (2)-(4) of the GPU encode / decode of one oracle sample chunk
    (layer `layer`, both K and V, the chunk cpu_baseline times) against the
    oracle: meta and codes by the boundary rule, flips counted, and the
    decode's relative RMS against the oracle's decode."""
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    from kv_cache_compression_kvc_amd import inputs
    tokens = sample_tokens(p)
    x = torch.stack([inputs.kv_chunk(p, layer, kv, (tokens,), device="cpu") for kv in (0, 1)])[None]
    xg = x.to(dev)
    blob = kvc.encode(xg, p.bits_k, p.bits_v, p.group, seed=p.seed)
    xd = kvc.decode(blob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed)
    torch.cuda.synchronize()
    res = parity.check_blob(inputs.as_u16(x), blob.cpu().numpy(), p.dtype, p.bits_k, p.bits_v, p.group, p.seed)
    rr = parity.check_decode(inputs.as_u16(xd), res.reference, p.dtype)
    r = res.report.as_dict()
    r.update(decode_rrms=rr, chunk="[1,2,%d,%d,%d] of layer %d" % (tokens, p.kv_heads, p.head_dim, layer),
             rule="codes equal the nearest level except within 1e-5 of a rounding boundary (counted)")
    return r


# ---------------------------------------------------------------------------
# Separate-kernel comparator (same results, intermediates through HBM)

def unfused_leg(kvc, p, xs, outs, dsts, a, stream, t_enc, t_dec, raw_bytes):
    """The comparator timed with events around each call (its kernels and the
    gaps between them); t_enc / t_dec are the fused calls timed the same way."""
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


def mix_probe(kvc, src, read_bytes, dst, write_bytes, stream, reps=5):
    """Best GB/s (read + write) of the library's streaming probes moving the
    same bytes in the same read:write ratio: 4 KiB runs of the larger stream
    at 4, 8 and 16 waves per CU (kvc_probe_stream), and runs of 16 KiB
    issued at once (an encode tile's loads in flight) at 2, 4 and 8 waves per
    CU (kvc_probe_stream_runs).  The achievable-bandwidth yardstick for a
    kernel with that traffic mix.  It overwrites dst."""
    import torch
    rb, wb = read_bytes // 1024 * 1024, write_bytes // 1024 * 1024
    trials = [("4KiB runs", wpc, lambda w: kvc.probe_stream(src, rb, dst, wb, waves_per_cu=w)) for wpc in (4, 8, 16)]
    trials += [("16KiB runs at once", wpc, lambda w: kvc.probe_stream_runs(src, rb, dst, wb, run_kib=16,
                                                                            waves_per_cu=w)) for wpc in (2, 4, 8)]
    best = None
    for pattern, wpc, run in trials:
        for _ in range(2):
            run(wpc)
        ev = TimingEvents(2)
        ev.record(0, stream)
        for _ in range(reps):
            run(wpc)
        ev.record(1, stream)
        torch.cuda.synchronize()
        gbps = (rb + wb) * reps / (ev.ms(0, 1) / 1e3) / 1e9
        ev.close()
        if best is None or gbps > best["GBps"]:
            best = {"GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS, "waves_per_cu": wpc, "pattern": pattern}
    best.update(read_bytes=rb, write_bytes=wb)
    return best


def pool_block_list(p, table, lens, num_blocks):
    """Every pool block a paged call reads, as indices of [L * 2 * NB] blocks,
    in the order of the request-order kernels: slab by slab, request by
    request, block by block."""
    import numpy as np
    per_req = [table[r, :-(-int(n) // p.block_size)] for r, n in enumerate(lens)]
    one_slab = np.concatenate(per_req).astype(np.int64) if per_req else np.zeros(0, np.int64)
    slabs = np.arange(p.layers * 2, dtype=np.int64) * num_blocks
    return (slabs[:, None] + one_slab[None, :]).reshape(-1).astype(np.int32)


def blocks_probe(kvc, region, block_bytes, blocks, seq, stream_bytes, scatter, stream, reps=3):
    """Best GB/s of the library's block gather (scatter = 0) or scatter (1)
    probe over 4, 8 and 16 waves per CU: a plain kernel moving whole pool
    blocks in the paged kernels' order against a sequential stream."""
    import torch
    sb = stream_bytes // 1024 * 1024
    moved = blocks.numel() * block_bytes + sb
    best = None
    for wpc in (4, 8, 16):
        kvc.probe_blocks(region, block_bytes, blocks, seq, sb, scatter, waves_per_cu=wpc)
        ev = TimingEvents(2)
        ev.record(0, stream)
        for _ in range(reps):
            kvc.probe_blocks(region, block_bytes, blocks, seq, sb, scatter, waves_per_cu=wpc)
        ev.record(1, stream)
        torch.cuda.synchronize()
        gbps = moved * reps / (ev.ms(0, 1) / 1e3) / 1e9
        ev.close()
        if best is None or gbps > best["GBps"]:
            best = {"GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS, "waves_per_cu": wpc}
    best.update(block_bytes=int(block_bytes), blocks=int(blocks.numel()), stream_bytes=int(sb))
    return best


def leg_probes(kvc, leg, stream, enc, dec):
    """Same-mix yardsticks of the encode and the decode of a leg, and each
    kernel's fraction of its yardstick."""
    src = leg.src[0].view(-1).view(__import__("torch").uint8)
    dst = leg.dsts[0].view(-1).view(__import__("torch").uint8)
    pe = mix_probe(kvc, src, leg.raw_bytes, leg.outs[0], leg.enc_bytes, stream)
    pd = mix_probe(kvc, leg.outs[0], leg.enc_bytes, dst, leg.raw_bytes, stream)
    enc["frac_same_mix_probe"] = enc["hbm_GBps"] / pe["GBps"]
    dec["frac_same_mix_probe"] = dec["hbm_GBps"] / pd["GBps"]
    out = {"encode_mix": pe, "decode_mix": pd,
           "what": "library streaming probes reading and writing the kernel's bytes in its ratio, best of "
                   "4 KiB runs at 4/8/16 waves per CU and 16 KiB runs issued at once at 2/4/8"}
    if leg.p.paged:   # the same blocks in the table's order: reads scattered (encode), writes scattered (decode)
        region = leg.src[0].view(-1).view(__import__("torch").uint8)
        out["encode_blocks"] = blocks_probe(kvc, region, leg.block_bytes, leg.blocks, leg.outs[0], leg.enc_bytes,
                                            0, stream)
        out["decode_blocks"] = blocks_probe(kvc, dst, leg.block_bytes, leg.blocks, leg.outs[0], leg.enc_bytes,
                                            1, stream)
        enc["frac_block_probe"] = enc["hbm_GBps"] / out["encode_blocks"]["GBps"]
        dec["frac_block_probe"] = dec["hbm_GBps"] / out["decode_blocks"]["GBps"]
    return out


class Leg:
    """Device inputs and encode / decode closures of one workload."""

    def __init__(self, kvc, p, dev, nsets, pool_order=True):
        import torch
        from kv_cache_compression_kvc_amd import inputs
        L, H, D = p.layers, p.kv_heads, p.head_dim
        self.p, self.nsets = p, nsets
        self.order = None
        if p.paged:
            lens = inputs.request_lengths(p)
            table, nb = inputs.block_table(p, lens)
            offs, total = kvc.paged_layout(lens, L, H, D, p.bits_k, p.bits_v, p.group, p.dtype)
            if pool_order:   # host prologue: the (request, block) items sorted by pool block
                import numpy as np
                items = kvc.paged_order(table, lens, offs, p.block_size, nb)
                self.order = torch.from_numpy(items.view(np.uint8)).to(dev)
            self.src = [inputs.make_pool(p, nb, device=dev) for _ in range(nsets)]
            self.outs = [torch.empty(total, dtype=torch.uint8, device=dev) for _ in range(nsets)]
            self.dsts = [torch.empty_like(self.src[0]) for _ in range(nsets)]
            self.bt, self.sl, self.of = (torch.from_numpy(a).to(dev) for a in (table, lens, offs))
            self.blocks = torch.from_numpy(pool_block_list(p, table, lens, nb)).to(dev)
            self.block_bytes = p.block_size * H * D * 2
            self.total = total
            tokens = int(lens.sum())
            self.raw_bytes = L * 2 * tokens * H * D * 2
            self.config = {"workload": p.name, "layers": L, "requests": len(lens), "tokens": tokens,
                           "kv_heads": H, "head_dim": D, "storage": p.dtype, "bits_k": p.bits_k,
                           "bits_v": p.bits_v, "group": p.group,
                           "layout": "paged, %d-token blocks, %s" % (
                               p.block_size, "visited in pool order" if pool_order else "visited in request order")}
        else:
            self.src = [inputs.make_kv(p, device=dev) for _ in range(nsets)]
            total, _ = kvc.encoded_size(L, p.tokens, H, D, p.bits_k, p.bits_v, p.group, p.dtype)
            self.outs = [torch.empty(total, dtype=torch.uint8, device=dev) for _ in range(nsets)]
            self.dsts = [torch.empty_like(self.src[0]) for _ in range(nsets)]
            self.total = total
            self.raw_bytes = self.src[0].numel() * 2
            self.config = {"workload": p.name, "shape": [L, 2, p.tokens, H, D], "storage": p.dtype,
                           "bits_k": p.bits_k, "bits_v": p.bits_v, "group": p.group, "layout": "contiguous"}
        self.enc_bytes = self.total
        self.algo_bytes = self.raw_bytes + self.enc_bytes   # read + write of one encode (or decode)
        self.kvc = kvc
        self.transform = None   # contiguous: None runs kvc_encode / kvc_decode, else the *_with forms

    def enc(self, i, events=None):
        p, k = self.p, i % self.nsets
        if p.paged:
            self.kvc.encode_paged(self.src[k], self.bt, self.sl, self.of, self.total, p.bits_k, p.bits_v, p.group,
                                  seed=p.seed, out=self.outs[k], order=self.order, events=events)
        else:
            self.kvc.encode(self.src[k], p.bits_k, p.bits_v, p.group, seed=p.seed, out=self.outs[k],
                            transform=self.transform, events=events)

    def dec(self, i, events=None):
        p, k = self.p, i % self.nsets
        if p.paged:
            self.kvc.decode_paged(self.outs[k], self.dsts[k], self.bt, self.sl, self.of, p.bits_k, p.bits_v, p.group,
                                  seed=p.seed, order=self.order, events=events)
        else:
            self.kvc.decode(self.outs[k], self.src[k].shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed,
                            out=self.dsts[k], transform=self.transform, events=events)

    def prewarm(self, seconds):
        """Encode + decode back to back for `seconds` of wall time; returns the
        steps run.  Python's garbage is collected first, while the GPU is idle
        anyway (the collector is off for the rest of the run)."""
        import torch
        gc.collect()
        n, t0 = 0, time.perf_counter()
        while True:
            for _ in range(8):
                self.enc(n)
                self.dec(n)
                n += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n

    def timed(self, steps, stream):
        """K steps between device synchronizations: (wall s, encode ms list,
        decode ms list).  Each call's time is its kernels' own: the library
        attaches the events to the start of its first and the end of its last
        kernel dispatch."""
        import torch
        ev = TimingEvents(4 * steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.enc(i, events=ev.pair(4 * i, 4 * i + 1))
            self.dec(i, events=ev.pair(4 * i + 2, 4 * i + 3))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        enc_ms = [ev.ms(4 * i, 4 * i + 1) for i in range(steps)]
        dec_ms = [ev.ms(4 * i + 2, 4 * i + 3) for i in range(steps)]
        ev.close()
        return wall, enc_ms, dec_ms

    def bracketed(self, steps, stream):
        """(encode ms list, decode ms list) with events recorded on the stream
        around each call instead: what the separate-kernel comparator is timed
        with, gaps between calls included."""
        import torch
        ev = TimingEvents(3 * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            ev.record(3 * i, stream)
            self.enc(i)
            ev.record(3 * i + 1, stream)
            self.dec(i)
            ev.record(3 * i + 2, stream)
        torch.cuda.synchronize()
        enc_ms = [ev.ms(3 * i, 3 * i + 1) for i in range(steps)]
        dec_ms = [ev.ms(3 * i + 1, 3 * i + 2) for i in range(steps)]
        ev.close()
        return enc_ms, dec_ms

    def close(self):
        import torch
        del self.src, self.outs, self.dsts, self.order
        self.blocks = None
        torch.cuda.empty_cache()


def _stats(ms):
    srt = sorted(ms)
    return sum(ms) / len(ms), srt[len(srt) // 2], srt[0]


def kernel_summary(leg, ms):
    mean, med, mn = _stats(ms)
    t = mean / 1e3
    alg = leg.algo_bytes / t / 1e9
    return {"raw_GBps": leg.raw_bytes / t / 1e9, "hbm_GBps": alg, "frac_hbm_peak": alg / HBM_PEAK_GBPS,
            "frac_hbm_peak_median": leg.algo_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "ms": mean, "ms_median": med, "ms_min": mn}


def break_even(leg, t_enc, t_dec):
    saved = leg.raw_bytes - leg.enc_bytes
    be = {}
    for gbit in (100, 400):
        wire_saved_s = saved * 8 / (gbit * 1e9)
        be["%dGbit" % gbit] = {"wire_time_saved_ms": wire_saved_s * 1e3,
                               "encode_plus_decode_ms": (t_enc + t_dec) * 1e3,
                               "pays": (t_enc + t_dec) < wire_saved_s,
                               "required_raw_GBps_each": 2 * gbit / 8 / (1 - leg.enc_bytes / leg.raw_bytes)}
    return be


def transform_leg(leg, stream, steps, prewarm_s):
    """The same protocol with the transform forced to the matrix cores and to
    the in-register butterfly (kvc_encode_with / kvc_decode_with), everything
    else of the launches equal: the measurement behind the transform each
    kernel runs by default."""
    out = {}
    for name in ("matrix", "butterfly"):
        leg.transform = name
        leg.prewarm(prewarm_s)
        _, e, d = leg.timed(steps, stream)
        out[name] = {k: {f: s[f] for f in ("frac_hbm_peak", "frac_hbm_peak_median", "ms", "ms_median")}
                     for k, s in (("encode", kernel_summary(leg, e)), ("decode", kernel_summary(leg, d)))}
    leg.transform = None
    for k in ("encode", "decode"):
        m, b = out["matrix"][k]["ms_median"], out["butterfly"][k]["ms_median"]
        out[k + "_butterfly_over_matrix"] = b / m
    return out


def other_workload(kvc, name, dev, stream, steps, prewarm_s, with_transform=True):
    """The same protocol on another workload: a shorter pre-warm, 3 warm-up
    steps, `steps` timed steps; tiny reports latency."""
    from kv_cache_compression_kvc_amd import presets
    p = presets.preset(name)
    leg = Leg(kvc, p, dev, nsets=1)
    leg.prewarm(prewarm_s)
    for i in range(3):
        leg.enc(i)
        leg.dec(i)
    wall, enc_ms, dec_ms = leg.timed(steps, stream)
    e, d = kernel_summary(leg, enc_ms), kernel_summary(leg, dec_ms)
    out = {"config": leg.config, "steps": steps, "bytes": {"raw": leg.raw_bytes, "encoded": leg.enc_bytes}}
    if name == "tiny":   # launch-bound: latency, not a roofline figure
        us = lambda ms: dict(zip(("mean", "median", "min"), (v * 1e3 for v in _stats(ms))))
        be, bd = leg.bracketed(steps, stream)
        out.update(encode_us=us(enc_ms), decode_us=us(dec_ms),
                   encode_us_call=us(be), decode_us_call=us(bd),
                   what="kernel time (events on the dispatches) and call time (events on the stream around "
                        "each call, launch included)")
    else:
        out.update(encode=e, decode=d, ms_per_step=wall / steps * 1e3,
                   raw_GBps_step=leg.raw_bytes / (wall / steps) / 1e9,
                   traffic={"encode": counter_traffic(name, "encode"), "decode": counter_traffic(name, "decode")})
        out["probes"] = leg_probes(kvc, leg, stream, e, d)
        if not p.paged and with_transform:
            out["transform"] = transform_leg(leg, stream, steps, prewarm_s / 3)
    out["break_even"] = break_even(leg, e["ms"] / 1e3, d["ms"] / 1e3)
    if p.paged:   # the same pool visited in request order (no host prologue), for comparison
        leg.order = None
        leg.prewarm(prewarm_s / 3)
        _, e2, d2 = leg.timed(steps, stream)
        out["request_order"] = {"encode": kernel_summary(leg, e2), "decode": kernel_summary(leg, d2)}
    leg.close()
    return out


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
    from kv_cache_compression_kvc_amd import presets

    gc.disable()   # collections run at the start of each pre-warm (Leg.prewarm)
    p = presets.preset(a.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    leg = Leg(kvc, p, dev, nsets=2)

    # pre-warm to steady clocks (time-based, independent of --warmup), then
    # the warm-up steps, then the timed steps; the copy probe runs after them
    # (a 2 GiB copy right before the timed steps slowed the next ones by up
    # to 10%)
    # the pre-warm, then (2 s on) the transform comparison keep the GPU busy;
    # the driver refreshes its metrics table only every few hundred ms
    clocks = ClockSample([a.prewarm_s * f for f in (0.25, 0.5, 0.75)] + [a.prewarm_s + 1.0])
    t0 = time.perf_counter()
    prewarm_steps = leg.prewarm(a.prewarm_s)
    prewarm = {"seconds": time.perf_counter() - t0, "steps": prewarm_steps}
    for i in range(a.warmup):
        leg.enc(i)
        leg.dec(i)
    torch.cuda.synchronize()

    wall, enc_ms, dec_ms = leg.timed(a.steps, stream)
    ms_per_step = wall / a.steps * 1e3
    enc, dec = kernel_summary(leg, enc_ms), kernel_summary(leg, dec_ms)
    t_enc, t_dec = enc["ms"] / 1e3, dec["ms"] / 1e3
    probes = leg_probes(kvc, leg, stream, enc, dec)
    transform = None if (p.paged or a.no_transform) else transform_leg(leg, stream, a.steps, min(a.prewarm_s, 1.0))

    unfused = pipeline = None
    if not p.paged and not a.no_unfused:
        be, bd = leg.bracketed(a.steps, stream)
        unfused = unfused_leg(kvc, p, leg.src, leg.outs, leg.dsts, a, stream, _stats(be)[0] / 1e3,
                              _stats(bd)[0] / 1e3, leg.raw_bytes)
        unfused["fused_bracketed_ms"] = {"encode": _stats(be)[0], "decode": _stats(bd)[0]}
    if not p.paged and not a.no_pipeline:
        pipeline = pipeline_leg(kvc, p, leg.src[0], leg.dsts[0], stream, leg.raw_bytes)
    dominant = "encode" if t_enc >= t_dec else "decode"
    t_dom = max(t_enc, t_dec)
    achieved = leg.algo_bytes / t_dom / 1e9
    result = {
        "metric": "encode/decode GB/s of raw bf16 KV input, % of HBM peak; break-even at 400 Gbit",
        "value": leg.raw_bytes / (ms_per_step / 1e3) / 1e9,
        "value_is": "raw KV bytes of one step (one encode and one decode of the workload) / ms_per_step; "
                    "per-kernel GB/s and fractions of the 8 TB/s peak under encode / decode, break-even "
                    "under break_even",
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
        "config": leg.config,
        "prewarm": prewarm,
        "clocks": clocks.get(),
        "encode": enc,
        "decode": dec,
        "bytes": {"raw": leg.raw_bytes, "encoded": leg.enc_bytes, "ratio": leg.raw_bytes / leg.enc_bytes},
        "probes": probes,
        "transform": transform,
        "break_even": break_even(leg, t_enc, t_dec),
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic(p.name, dominant),
                     "algorithmic_bytes_per_launch": leg.algo_bytes, "launch_ms": t_dom * 1e3},
        "unfused": unfused,
        "pipeline": pipeline,
        "workloads": None,
        "cpu_baseline": None,
    }
    leg.close()
    if a.other_steps > 0:
        result["workloads"] = {name: other_workload(kvc, name, dev, stream, a.other_steps, a.other_prewarm_s,
                                                    not a.no_transform)
                               for name in presets.ORDER if name != p.name}
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, a.cpu_sample_chunks)
        result["cpu_baseline"]["parity_sample"] = sample_parity(kvc, p, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
