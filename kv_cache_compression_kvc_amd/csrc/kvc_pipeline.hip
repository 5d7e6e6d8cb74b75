/*
 * kvc_pipeline.hip -- chunked encode overlapped with the transfer of the
 * encoded bytes, and the matching receive-then-decode.
 *
 * The episode notes of "FastKVComp: checking whether high-throughput KV
 * compression pays off" state the break-even rule: compression pays only if
 * encode plus decode time stays below the wire time it saves.  Taken
 * serially that is a sum; cutting the cache into layer chunks lets the
 * encode of chunk c+1 run while chunk c is on the wire (and, on the
 * receiving side, the decode of chunk c run while chunk c+1 arrives), so the
 * cost becomes about max(encode, wire) plus one chunk of fill.
 *
 * Chunked blob (sizes from kvc_chunked_size, kvc_host.cpp): chunk c holds
 * layers [c*Lc, min(L, (c+1)*Lc)) encoded as a [L_c, 2, T, H, D] tensor
 * (the ordinary blob format), at byte offset c * stride, stride = the blob
 * size of Lc layers.
 *
 * Chunks cross the link by a small streaming-copy kernel on the copy
 * stream, so the far side must be device memory or pinned host memory
 * mapped into the device's address space (standing in for a NIC buffer).
 * Measured over PCIe to and from pinned host memory, 64 blocks of that
 * kernel move 56-57 GB/s each way, as fast as a DMA-engine copy
 * (hipMemcpyAsync) of the whole blob and faster than DMA copies of 4 MiB
 * chunks (45 GB/s); and a DMA copy that waits on the compute stream added
 * about 0.2 ms per chunk, which serialized the pipeline, where a kernel
 * waits on the other stream through the command processor in microseconds.
 *
 * Ordering between the two streams uses one event per (host thread,
 * device), created on first use and kept for the life of the thread; every
 * wait captures the event's latest record when it is enqueued, so one event
 * serves all chunks of a call.
 */
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/kvc.h"
#include "kvc_plan.h"

namespace kvc {
namespace {

constexpr int kMaxDevices = 64;

int stream_event(hipEvent_t* ev) {
  thread_local hipEvent_t events[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_EHIP;
  if (!events[dev] && hipEventCreateWithFlags(&events[dev], hipEventDisableTiming) != hipSuccess) {
    events[dev] = nullptr;
    return KVC_EHIP;
  }
  *ev = events[dev];
  return KVC_OK;
}

/* `waiter` waits for everything enqueued on `first` so far. */
int order_after(hipEvent_t ev, hipStream_t first, hipStream_t waiter) {
  if (hipEventRecord(ev, first) != hipSuccess) return KVC_EHIP;
  if (hipStreamWaitEvent(waiter, ev, 0) != hipSuccess) return KVC_EHIP;
  return KVC_OK;
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

/* Blocks of the link copy: enough 16-byte accesses in flight to fill the
 * link (measured over PCIe: 16 blocks 54 GB/s, 32-128 blocks 55.5-57 GB/s,
 * 256 or more 54-55 GB/s), few enough to leave the compute units to the
 * encode / decode beside it. */
constexpr int kLinkBlocks = 64;

__global__ __launch_bounds__(256) void link_copy_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                        uint64_t n) {
  for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += uint64_t(gridDim.x) * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

/* Copy `bytes` (a multiple of 16) on stream st. */
int link_copy(const void* src, void* dst, uint64_t bytes, hipStream_t st) {
  const uint64_t n = bytes / 16;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>(kLinkBlocks, (n + 255) / 256));
  if (grid == 0) return KVC_OK;
  hipLaunchKernelGGL(link_copy_kernel, dim3(grid), dim3(256), 0, st, static_cast<const v4u*>(src),
                     static_cast<v4u*>(dst), n);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

/* The device can access `p` directly: device memory, or host memory that
 * the runtime has pinned and mapped. */
bool device_accessible(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();  // clear the error of an unknown (pageable) pointer
    return false;
  }
  return at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeHost || at.type == hipMemoryTypeManaged;
}

/* desc of chunk k and its layer count */
kvc_desc chunk_desc(const kvc_desc* d, int64_t chunk_layers, int64_t k) {
  kvc_desc dc = *d;
  const int64_t l0 = k * chunk_layers;
  dc.layers = d->layers - l0 < chunk_layers ? d->layers - l0 : chunk_layers;
  return dc;
}

}  // namespace
}  // namespace kvc

extern "C" {

kvc_status kvc_encode_send(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                           int64_t chunk_layers, void* dst, uint64_t dst_bytes, void* compute_stream,
                           void* copy_stream) {
  kvc::Chunking c;
  int st = kvc::chunking(desc, chunk_layers, &c);
  if (st != KVC_OK) return static_cast<kvc_status>(st);
  if (c.total == 0) return KVC_OK;
  if (!kv || !out || !dst) return KVC_EINVAL;
  if (out_bytes < c.total || dst_bytes < c.total) return KVC_ENOSPC;
  if (reinterpret_cast<uintptr_t>(dst) & 15u) return KVC_EALIGN;
  if (!kvc::device_accessible(dst)) return KVC_EINVAL;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream), xs = static_cast<hipStream_t>(copy_stream);
  hipEvent_t ev;
  if ((st = kvc::stream_event(&ev)) != KVC_OK) return static_cast<kvc_status>(st);
  // a copy still reading `out` from an earlier call must finish before it is rewritten
  if ((st = kvc::order_after(ev, xs, cs)) != KVC_OK) return static_cast<kvc_status>(st);
  for (int64_t k = 0; k < c.n_chunks; ++k) {
    const kvc_desc dc = kvc::chunk_desc(desc, chunk_layers, k);
    uint64_t bytes = 0;
    if ((st = kvc_encoded_size(&dc, dc.tokens, &bytes, nullptr)) != KVC_OK) return static_cast<kvc_status>(st);
    const uint8_t* src = static_cast<const uint8_t*>(kv) + static_cast<uint64_t>(k * chunk_layers) * c.kv_layer;
    uint8_t* blob = static_cast<uint8_t*>(out) + static_cast<uint64_t>(k) * c.stride;
    if ((st = kvc_encode(&dc, src, blob, bytes, cs)) != KVC_OK) return static_cast<kvc_status>(st);
    if ((st = kvc::order_after(ev, cs, xs)) != KVC_OK) return static_cast<kvc_status>(st);
    // blob sizes are multiples of 256
    if ((st = kvc::link_copy(blob, static_cast<uint8_t*>(dst) + static_cast<uint64_t>(k) * c.stride, bytes, xs)) !=
        KVC_OK)
      return static_cast<kvc_status>(st);
  }
  return KVC_OK;
}

kvc_status kvc_receive_decode(const kvc_desc* desc, const void* src, uint64_t src_bytes, void* staging,
                              uint64_t staging_bytes, int64_t chunk_layers, void* kv_out, void* compute_stream,
                              void* copy_stream) {
  kvc::Chunking c;
  int st = kvc::chunking(desc, chunk_layers, &c);
  if (st != KVC_OK) return static_cast<kvc_status>(st);
  if (c.total == 0) return KVC_OK;
  if (!src || !staging || !kv_out) return KVC_EINVAL;
  if (src_bytes < c.total || staging_bytes < c.total) return KVC_ENOSPC;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return KVC_EALIGN;
  if (!kvc::device_accessible(src)) return KVC_EINVAL;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream), xs = static_cast<hipStream_t>(copy_stream);
  hipEvent_t ev;
  if ((st = kvc::stream_event(&ev)) != KVC_OK) return static_cast<kvc_status>(st);
  // a decode still reading `staging` from an earlier call must finish first
  if ((st = kvc::order_after(ev, cs, xs)) != KVC_OK) return static_cast<kvc_status>(st);
  for (int64_t k = 0; k < c.n_chunks; ++k) {
    const kvc_desc dc = kvc::chunk_desc(desc, chunk_layers, k);
    uint64_t bytes = 0;
    if ((st = kvc_encoded_size(&dc, dc.tokens, &bytes, nullptr)) != KVC_OK) return static_cast<kvc_status>(st);
    uint8_t* blob = static_cast<uint8_t*>(staging) + static_cast<uint64_t>(k) * c.stride;
    if ((st = kvc::link_copy(static_cast<const uint8_t*>(src) + static_cast<uint64_t>(k) * c.stride, blob, bytes,
                             xs)) != KVC_OK)
      return static_cast<kvc_status>(st);
    if ((st = kvc::order_after(ev, xs, cs)) != KVC_OK) return static_cast<kvc_status>(st);
    uint8_t* dstk = static_cast<uint8_t*>(kv_out) + static_cast<uint64_t>(k * chunk_layers) * c.kv_layer;
    if ((st = kvc_decode(&dc, blob, bytes, dstk, cs)) != KVC_OK) return static_cast<kvc_status>(st);
  }
  return KVC_OK;
}

}  // extern "C"
