/*
 * kvc_probe.hip -- measurement helpers of the C ABI (include/kvc.h): plain
 * streaming kernels that move known bytes in the access patterns of the
 * encode / decode kernels, as yardsticks of the bandwidth those patterns
 * can reach on the device.  They compute nothing of the method.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/kvc.h"

namespace kvc {
namespace dev {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

/* Streaming 16-byte copy: the achievable-bandwidth yardstick. */
__global__ __launch_bounds__(256) void copy_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                   uint64_t n) {
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4u a0 = __builtin_nontemporal_load(src + i);
    const v4u a1 = __builtin_nontemporal_load(src + i + stride);
    const v4u a2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u a3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a0, dst + i);
    __builtin_nontemporal_store(a1, dst + i + stride);
    __builtin_nontemporal_store(a2, dst + i + 2 * stride);
    __builtin_nontemporal_store(a3, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

/* Streaming mix of reads and writes at a fixed ratio: nr 1 KiB chunks of src
 * read and nw written to dst (a chunk: 64 lanes x 16 bytes).  The larger
 * stream is walked in runs of 4 consecutive chunks, grid-strided; the run
 * covering chunks [4u, 4u + 4) of it also moves chunks [floor(4u * ns / nl),
 * floor((4u + 4) * ns / nl)) of the smaller stream, so the two keep their
 * ratio at every point.  The stored data does not depend on the loads.  The
 * yardstick for a kernel with the same traffic mix. */
__global__ __launch_bounds__(64) void stream_kernel(const v4u* __restrict__ src, uint64_t nr, v4u* __restrict__ dst,
                                                    uint64_t nw) {
  const uint64_t nl = nr > nw ? nr : nw, ns = nr > nw ? nw : nr;
  const bool reads_lead = nr >= nw;
  const int lane = threadIdx.x;
  v4u acc = {0, 0, 0, 0};
  const uint64_t nu = (nl + 3) / 4, u0 = blockIdx.x, g = gridDim.x;
  // lo = floor(4u * ns / nl) with remainder, carried along without divisions
  uint64_t lo = 4 * u0 * ns / nl, rem = 4 * u0 * ns - lo * nl;
  const uint64_t dq = 4 * g * ns / nl, dr = 4 * g * ns - dq * nl;
  for (uint64_t u = u0; u < nu; u += g) {
    const uint64_t c0 = 4 * u;
    uint64_t hi = ns;
    if (c0 + 4 <= nl) {  // floor((4u + 4) * ns / nl) = lo + floor((rem + 4 ns) / nl), at most lo + 4
      uint64_t t = rem + 4 * ns;
      hi = lo;
      while (t >= nl) {
        t -= nl;
        ++hi;
      }
    }
    const uint64_t n_lead = nl - c0 < 4 ? nl - c0 : 4;
    for (uint64_t k = 0; k < n_lead; ++k) {
      const uint64_t c = c0 + k;
      if (reads_lead)
        acc ^= __builtin_nontemporal_load(src + c * 64 + lane);
      else
        __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, dst + c * 64 + lane);
    }
    for (uint64_t c = lo; c < hi; ++c) {
      if (reads_lead)
        __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, dst + c * 64 + lane);
      else
        acc ^= __builtin_nontemporal_load(src + c * 64 + lane);
    }
    lo += dq;
    rem += dr;
    if (rem >= nl) {
      rem -= nl;
      lo += 1;
    }
  }
  // the loaded data is consumed here, so the loads stay
  asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
}

/* The same mix with every run of the larger stream issued at once: RUN
 * consecutive 1 KiB chunks per run (RUN loads in flight per wave when reads
 * lead, like an encode tile arriving), grid-strided over the runs, and the
 * run covering chunks [RUN u, RUN u + RUN) of the larger stream also moves
 * chunks [floor(RUN u ns / nl), floor((RUN u + RUN) ns / nl)) of the smaller
 * one.  The host keeps nl * ns below 2^62. */
template <int RUN>
__global__ __launch_bounds__(64) void stream_runs_kernel(const v4u* __restrict__ src, uint64_t nr,
                                                         v4u* __restrict__ dst, uint64_t nw) {
  const uint64_t nl = nr > nw ? nr : nw, ns = nr > nw ? nw : nr;
  const bool reads_lead = nr >= nw;
  const int lane = threadIdx.x;
  v4u acc = {0, 0, 0, 0};
  const uint64_t nu = (nl + RUN - 1) / RUN;
  for (uint64_t u = blockIdx.x; u < nu; u += gridDim.x) {
    const uint64_t c0 = u * RUN;
    const uint64_t lo = c0 * ns / nl;
    const uint64_t hi = c0 + RUN <= nl ? (c0 + RUN) * ns / nl : ns;
    if (c0 + RUN <= nl) {
      if (reads_lead) {
        v4u v[RUN];
#pragma unroll
        for (int k = 0; k < RUN; ++k) v[k] = __builtin_nontemporal_load(src + (c0 + k) * 64 + lane);
        for (uint64_t c = lo; c < hi; ++c)
          __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, dst + c * 64 + lane);
#pragma unroll
        for (int k = 0; k < RUN; ++k) acc ^= v[k];
      } else {
#pragma unroll
        for (int k = 0; k < RUN; ++k)
          __builtin_nontemporal_store(v4u{uint32_t(c0 + k), uint32_t(lane), 0u, 0u}, dst + (c0 + k) * 64 + lane);
        for (uint64_t c = lo; c < hi; ++c) acc ^= __builtin_nontemporal_load(src + c * 64 + lane);
      }
    } else {  // the last, partial run
      for (uint64_t c = c0; c < nl; ++c) {
        if (reads_lead)
          acc ^= __builtin_nontemporal_load(src + c * 64 + lane);
        else
          __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, dst + c * 64 + lane);
      }
      for (uint64_t c = lo; c < hi; ++c) {
        if (reads_lead)
          __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, dst + c * 64 + lane);
        else
          acc ^= __builtin_nontemporal_load(src + c * 64 + lane);
      }
    }
  }
  // the loaded data is consumed here, so the loads stay
  asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
}

/* Block gather / scatter against a sequential stream (kvc_probe_blocks):
 * unit u moves block blocks[u] of the region (cpb 1-KiB chunks) and chunks
 * [floor(u * ns / n), floor((u + 1) * ns / n)) of the stream.  scatter = 0
 * reads the block and writes the stream, 1 the reverse.  The stored data
 * does not depend on the loads. */
__global__ __launch_bounds__(64) void blocks_kernel(v4u* __restrict__ region, int64_t region_blocks,
                                                    const int32_t* __restrict__ blocks, int64_t n, int cpb,
                                                    v4u* __restrict__ seq, uint64_t ns, int scatter) {
  const int lane = threadIdx.x;
  v4u acc = {0, 0, 0, 0};
  for (int64_t u = blockIdx.x; u < n; u += gridDim.x) {
    const int64_t b = blocks[u];
    const uint64_t lo = uint64_t(u) * ns / uint64_t(n), hi = uint64_t(u + 1) * ns / uint64_t(n);
    if (b >= 0 && b < region_blocks) {
      v4u* blk = region + b * cpb * 64;
      for (int c = 0; c < cpb; ++c) {
        if (!scatter)
          acc ^= __builtin_nontemporal_load(blk + c * 64 + lane);
        else
          __builtin_nontemporal_store(v4u{uint32_t(u), uint32_t(c), uint32_t(lane), 0u}, blk + c * 64 + lane);
      }
    }
    for (uint64_t c = lo; c < hi; ++c) {
      if (!scatter)
        __builtin_nontemporal_store(v4u{uint32_t(c), uint32_t(lane), 0u, 0u}, seq + c * 64 + lane);
      else
        acc ^= __builtin_nontemporal_load(seq + c * 64 + lane);
    }
  }
  // the loaded data is consumed here, so the loads stay
  asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
}

}  // namespace dev
}  // namespace kvc

extern "C" {

kvc_status kvc_probe_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                            int32_t waves_per_cu, void* stream) {
  if (read_bytes == 0 && write_bytes == 0) return KVC_OK;
  if ((read_bytes && !src) || (write_bytes && !dst) || waves_per_cu < 1 || waves_per_cu > 32) return KVC_EINVAL;
  if ((read_bytes & 1023u) || (write_bytes & 1023u) || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(dst) & 15u))
    return KVC_EALIGN;
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return KVC_EHIP;
  const uint64_t nr = read_bytes / 1024, nw = write_bytes / 1024;
  const uint64_t grid = std::min<uint64_t>(uint64_t(cus) * uint64_t(waves_per_cu), std::max(nr, nw));
  hipLaunchKernelGGL(kvc::dev::stream_kernel, dim3(static_cast<unsigned>(grid)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const kvc::dev::v4u*>(src), nr,
                     static_cast<kvc::dev::v4u*>(dst), nw);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

kvc_status kvc_probe_stream_runs(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                                 int32_t run_kib, int32_t waves_per_cu, void* stream) {
  if (read_bytes == 0 && write_bytes == 0) return KVC_OK;
  if ((read_bytes && !src) || (write_bytes && !dst) || waves_per_cu < 1 || waves_per_cu > 32 ||
      (run_kib != 4 && run_kib != 8 && run_kib != 16))
    return KVC_EINVAL;
  if ((read_bytes & 1023u) || (write_bytes & 1023u) || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(dst) & 15u))
    return KVC_EALIGN;
  const uint64_t nr = read_bytes / 1024, nw = write_bytes / 1024;
  const uint64_t nl = std::max(nr, nw), ns = std::min(nr, nw);
  if (ns && nl > (uint64_t(1) << 62) / ns) return KVC_EINVAL;   // (c0 + RUN) * ns stays in range
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return KVC_EHIP;
  const uint64_t runs = (nl + run_kib - 1) / run_kib;
  const dim3 grid(static_cast<unsigned>(std::min<uint64_t>(uint64_t(cus) * uint64_t(waves_per_cu), runs)));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const kvc::dev::v4u* in = static_cast<const kvc::dev::v4u*>(src);
  kvc::dev::v4u* out = static_cast<kvc::dev::v4u*>(dst);
  if (run_kib == 4)
    hipLaunchKernelGGL(kvc::dev::stream_runs_kernel<4>, grid, dim3(64), 0, s, in, nr, out, nw);
  else if (run_kib == 8)
    hipLaunchKernelGGL(kvc::dev::stream_runs_kernel<8>, grid, dim3(64), 0, s, in, nr, out, nw);
  else
    hipLaunchKernelGGL(kvc::dev::stream_runs_kernel<16>, grid, dim3(64), 0, s, in, nr, out, nw);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

kvc_status kvc_probe_blocks(void* region, int64_t region_blocks, uint32_t block_bytes, const int32_t* blocks,
                            int64_t n_blocks, void* seq, uint64_t stream_bytes, int32_t scatter,
                            int32_t waves_per_cu, void* stream) {
  if (n_blocks < 0 || region_blocks < 0 || (scatter != 0 && scatter != 1) || waves_per_cu < 1 || waves_per_cu > 32)
    return KVC_EINVAL;
  if (n_blocks == 0) return KVC_OK;
  if (!blocks || (region_blocks > 0 && !region) || (stream_bytes && !seq)) return KVC_EINVAL;
  if (block_bytes == 0 || (block_bytes & 1023u) || (stream_bytes & 1023u) ||
      (reinterpret_cast<uintptr_t>(region) & 15u) || (reinterpret_cast<uintptr_t>(seq) & 15u) ||
      (reinterpret_cast<uintptr_t>(blocks) & 3u))
    return KVC_EALIGN;
  const uint64_t ns = stream_bytes / 1024;
  if (ns && uint64_t(n_blocks) > (uint64_t(1) << 62) / ns) return KVC_EINVAL;   // u * ns stays in range
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return KVC_EHIP;
  const uint64_t grid = std::min<uint64_t>(uint64_t(cus) * uint64_t(waves_per_cu), uint64_t(n_blocks));
  hipLaunchKernelGGL(kvc::dev::blocks_kernel, dim3(static_cast<unsigned>(grid)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<kvc::dev::v4u*>(region), region_blocks, blocks,
                     n_blocks, static_cast<int>(block_bytes / 1024), static_cast<kvc::dev::v4u*>(seq), ns,
                     static_cast<int>(scatter));
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

kvc_status kvc_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (bytes == 0) return KVC_OK;
  if (!src || !dst) return KVC_EINVAL;
  if ((bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return KVC_EALIGN;
  int device = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kvc::dev::copy_kernel), 256,
                                                   0) != hipSuccess)
    return KVC_EHIP;
  const uint64_t n = bytes / 16;
  const uint64_t grid = std::min<uint64_t>(uint64_t(cus) * uint64_t(per_cu > 0 ? per_cu : 1), (n + 255) / 256);
  hipLaunchKernelGGL(kvc::dev::copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const kvc::dev::v4u*>(src), static_cast<kvc::dev::v4u*>(dst), n);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

}  // extern "C"
