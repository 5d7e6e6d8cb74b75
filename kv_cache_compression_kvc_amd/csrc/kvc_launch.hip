/*
 * kvc_launch.hip -- GPU entry points of the C ABI (include/kvc.h): pick the
 * kernel instance for a validated plan and launch it on the caller's stream
 * with a persistent grid (one or all resident waves per SIMD, per kernel).
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kvc_device.h"
#include "kvc_pick.h"
#include "kvc_plan.h"

namespace kvc {
namespace dev {

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

}  // namespace dev

namespace {

Kernel pick(Op op, int d, int dt, int b, int g, bool paged, int mode) {
  if (d == 64) return dt == KVC_BF16 ? pick_d64_t0(op, b, g, paged, mode) : pick_d64_t1(op, b, g, paged, mode);
  if (d == 128)
    return dt == KVC_BF16 ? pick_d128_t0(op, b, g, paged, mode) : pick_d128_t1(op, b, g, paged, mode);
  return nullptr;
}

/* Resident workgroups per device for a kernel (CUs x occupancy) and the
 * device's CU count, cached. */
struct GridCache {
  std::mutex mu;
  static constexpr int kMax = 512;
  int n = 0;
  int dev[kMax];
  const void* fn[kMax];
  int64_t grid[kMax];
  int cus[kMax];
};
GridCache g_grid;

int resident_groups(Kernel k, int threads, int64_t* out, int* cus_out = nullptr) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return KVC_EHIP;
  {
    std::lock_guard<std::mutex> lk(g_grid.mu);
    for (int i = 0; i < g_grid.n; ++i)
      if (g_grid.dev[i] == device && g_grid.fn[i] == reinterpret_cast<const void*>(k)) {
        *out = g_grid.grid[i];
        if (cus_out) *cus_out = g_grid.cus[i];
        return KVC_OK;
      }
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return KVC_EHIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), threads, 0) !=
      hipSuccess)
    return KVC_EHIP;
  const int64_t g = int64_t(cus) * (per_cu > 0 ? per_cu : 1);
  std::lock_guard<std::mutex> lk(g_grid.mu);
  if (g_grid.n < GridCache::kMax) {
    g_grid.dev[g_grid.n] = device;
    g_grid.fn[g_grid.n] = reinterpret_cast<const void*>(k);
    g_grid.grid[g_grid.n] = g;
    g_grid.cus[g_grid.n] = cus;
    ++g_grid.n;
  }
  *out = g;
  if (cus_out) *cus_out = cus;
  return KVC_OK;
}

constexpr int kSimdsPerCu = 4;

/* Blob sizes above which a contiguous decode launch runs in kDecodeLarge
 * mode: at head_dim 64, 3/4 of the 256 MB memory-side cache; at head_dim
 * 128, only for 4-bit codes in one group per vector, past 512 MiB. */
constexpr uint64_t kDecodeLargeBlobD64 = uint64_t(192) << 20;
constexpr uint64_t kDecodeLargeBlobD128 = uint64_t(512) << 20;

/*
 * How a launch fills the chip: waves per SIMD (0: every resident wave) and,
 * for the decode, its mode (kvc_device.h: the in-group transform and where a
 * tile waits for the last tile's stores).  Every tile is streamed once, so
 * extra waves only add independent access streams once enough bytes are in
 * flight.  Measured on 8B-shaped caches, each kernel alone and alternating
 * with the other:
 *   - encode: one wave per SIMD is as fast or faster (1-2% at 4k tokens,
 *     5-6% at 32k, about 4% at head_dim 64, 3% on the paged pool), except on
 *     a paged pool at head_dim 64, 5% slower there: 8 KiB tiles, each behind
 *     a dependent table load, keep too few bytes in flight;
 *   - contiguous decode, head_dim 64, blob above kDecodeLargeBlobD64 (the
 *     blob an encode just wrote then no longer sits in the memory-side
 *     cache): kDecodeLarge at one wave per SIMD, 1-3% faster than
 *     kDecodeWaitStores (2- and 4-bit, groups of 32 and 64, 1 GB blobs);
 *   - contiguous decode, head_dim 128: kDecodeWaitStores at every size,
 *     2-11% faster than kDecodeLarge on 0.3-2 GB blobs of 2-bit, 8-bit or
 *     grouped codes and on 4-bit G128 blobs up to 408 MiB; only 4-bit codes
 *     with G = 128 past kDecodeLargeBlobD128 keep kDecodeLarge (1.4-3.8%
 *     faster from 544 MiB up);
 *   - a smaller blob: kDecodeWaitStores at one wave per SIMD, 5.6-6.6%
 *     faster than kDecodeWaitTop at two waves (8B-4k, and head_dim 64 at 8k
 *     tokens);
 *   - paged decode: kDecodeWaitStores at one wave per SIMD at head_dim 128
 *     (1.5% faster than kDecodeWaitTop at two); kDecodeWaitTop at two waves
 *     at head_dim 64, where one wave lost 16%.
 * Grids between one and two waves per SIMD leave some SIMDs with a wave more
 * than others; with a static tile split those finish last, and such grids
 * measured slower than either.
 */
struct LaunchShape {
  int waves_per_simd;
  int mode;
};

/* Whether a contiguous decode launch of `bits`-bit codes takes kDecodeLarge. */
bool decode_large(const LaunchArgs& a, int head_dim, int bits) {
  if (head_dim == 64) return a.blob_total > kDecodeLargeBlobD64;
  return bits == 4 && a.groups == 1 && a.blob_total > kDecodeLargeBlobD128;
}

LaunchShape launch_shape(Op op, const LaunchArgs& a, int head_dim, int bits) {
  if (op == Op::Encode) return {(a.paged && head_dim == 64) ? 0 : 1, 0};
  if (op != Op::Decode) return {0, 0};
  if (a.paged) return head_dim == 64 ? LaunchShape{2, dev::kDecodeWaitTop} : LaunchShape{1, dev::kDecodeWaitStores};
  return decode_large(a, head_dim, bits) ? LaunchShape{1, dev::kDecodeLarge} : LaunchShape{1, dev::kDecodeWaitStores};
}

int run_plan(Op op, const Plan& plan, void* stream) {
  for (int i = 0; i < plan.n_launch; ++i) {
    const LaunchShape shape = launch_shape(op, plan.args[i], plan.head_dim, plan.bits[i]);
    Kernel k = pick(op, plan.head_dim, plan.dtype, plan.bits[i], plan.group, plan.args[i].paged != 0, shape.mode);
    if (!k) return KVC_ESHAPE;
    int64_t resident = 0;
    int cus = 0;
    int st = resident_groups(k, 64, &resident, &cus);
    if (st != KVC_OK) return st;
    const int64_t waves =
        shape.waves_per_simd > 0 ? std::min<int64_t>(resident, int64_t(cus) * kSimdsPerCu * shape.waves_per_simd)
                                 : resident;
    const int64_t grid = std::min<int64_t>(plan.args[i].total_items, waves);
    if (grid <= 0) continue;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(64), 0, static_cast<hipStream_t>(stream),
                       plan.args[i]);
    if (hipGetLastError() != hipSuccess) return KVC_EHIP;
  }
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

extern "C" {

kvc_status kvc_encode(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Encode, desc, kv, out, out_bytes, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Encode, plan, stream);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_decode(const kvc_desc* desc, const void* in, uint64_t in_bytes, void* kv_out, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Decode, desc, in, kv_out, in_bytes, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Decode, plan, stream);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_encode_paged(const kvc_desc* desc, const void* pool, const kvc_paged* paged, void* out,
                            uint64_t out_bytes, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_paged(kvc::Op::Encode, desc, pool, out, out_bytes, paged, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Encode, plan, stream);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_decode_paged(const kvc_desc* desc, const void* in, uint64_t in_bytes, const kvc_paged* paged,
                            void* pool, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_paged(kvc::Op::Decode, desc, in, pool, in_bytes, paged, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Decode, plan, stream);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_debug_rotate(const kvc_desc* desc, const void* kv, float* y_out, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Rotate, desc, kv, y_out, 0, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Rotate, plan, stream);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (bytes == 0) return KVC_OK;
  if (!src || !dst) return KVC_EINVAL;
  if ((bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return KVC_EALIGN;
  int64_t resident = 0;
  int st = kvc::resident_groups(reinterpret_cast<kvc::Kernel>(kvc::dev::copy_kernel), 256, &resident);
  if (st != KVC_OK) return static_cast<kvc_status>(st);
  const uint64_t n = bytes / 16;
  const uint64_t grid = std::min<uint64_t>(uint64_t(resident), (n + 255) / 256);
  hipLaunchKernelGGL(kvc::dev::copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const kvc::dev::v4u*>(src), static_cast<kvc::dev::v4u*>(dst), n);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
}

}  // extern "C"
