/*
 * kvc_launch.hip -- entry points of the fused path in the C ABI
 * (include/kvc.h: kvc_encode, kvc_decode, their paged and *_with forms,
 * kvc_debug_rotate): pick the kernel instance for a validated plan and
 * launch it on the caller's stream with a persistent grid (one or all
 * resident waves per SIMD, per kernel).  The measurement probes are in
 * kvc_probe.hip, the separate-kernel comparator in kvc_unfused.hip, the
 * chunked send / receive in kvc_pipeline.hip.
 */
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kvc_device.h"
#include "kvc_pick.h"
#include "kvc_plan.h"

namespace kvc {
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
 *     faster from 544 MiB up).  From kDecodeThreePerCuBlob of blob, three
 *     waves per CU rather than one per SIMD (below);
 *   - a smaller blob: kDecodeWaitStores at one wave per SIMD, 5.6-6.6%
 *     faster than kDecodeWaitTop at two waves (8B-4k, and head_dim 64 at 8k
 *     tokens);
 *   - paged decode: kDecodeWaitStores at one wave per SIMD at head_dim 128
 *     (1.5% faster than kDecodeWaitTop at two); kDecodeWaitTop at two waves
 *     at head_dim 64, where one wave lost 16%.
 * Grids between one and two waves per SIMD leave some SIMDs with a wave more
 * than others; with a static tile split those finish last, and such grids
 * measured slower than either -- except the write-heavy large decode, where
 * three waves per CU (fewer concurrent write streams) beat one per SIMD.
 * For scale: plain streaming kernels on this chip reach about 0.68 of the
 * 8 TB/s peak for the decode's mix of one byte read to four written, 0.78
 * for the encode's four to one, and 0.72 for writes alone.
 */
struct LaunchShape {
  int waves_per_simd;
  int mode;
  int waves_per_cu;   // when > 0, the grid is this many waves per CU instead
};

/* Blob size from which a contiguous decode in kDecodeWaitStores mode runs
 * three waves per CU instead of one per SIMD: on the 4 GiB 2-bit G32 cache
 * (1.02 GB blob) that measured 2-3% faster; at 512 MiB of input (136 MiB of
 * blob) one wave per SIMD stays the faster. */
constexpr uint64_t kDecodeThreePerCuBlob = uint64_t(384) << 20;

/* Whether a contiguous decode launch of `bits`-bit codes takes kDecodeLarge. */
bool decode_large(const LaunchArgs& a, int head_dim, int bits) {
  if (head_dim == 64) return a.blob_total > kDecodeLargeBlobD64;
  return bits == 4 && a.groups == 1 && a.blob_total > kDecodeLargeBlobD128;
}

/* `transform` (kvc_transform) overrides the transform of a contiguous
 * launch and keeps the rest of its shape: a forced matrix-core decode of a
 * kDecodeLarge-sized blob runs as kDecodeWaitStores, a forced butterfly
 * decode of a smaller one as kDecodeButterfly with the waves that
 * kDecodeWaitStores would take. */
LaunchShape launch_shape(Op op, const LaunchArgs& a, int head_dim, int bits, int transform) {
  const bool bfly = transform == KVC_TRANSFORM_BUTTERFLY;
  if (op == Op::Encode) {
    // 8-bit encodes take the butterfly by default: its error bound is
    // 2 D / log2(D) times tighter than the matrix cores', so far fewer codes
    // near a tie are decided again in float64
    const bool bfly_enc = bfly || (transform == KVC_TRANSFORM_AUTO && bits == 8);
    return {(a.paged && head_dim == 64) ? 0 : 1, bfly_enc ? dev::kEncodeButterfly : dev::kEncodeMatrix, 0};
  }
  if (op != Op::Decode) return {0, 0, 0};
  if (a.paged)
    return head_dim == 64 ? LaunchShape{2, dev::kDecodeWaitTop, 0} : LaunchShape{1, dev::kDecodeWaitStores, 0};
  if (transform != KVC_TRANSFORM_MATRIX && decode_large(a, head_dim, bits)) return {1, dev::kDecodeLarge, 0};
  return {1, bfly ? dev::kDecodeButterfly : dev::kDecodeWaitStores, a.blob_total >= kDecodeThreePerCuBlob ? 3 : 0};
}

/* A call's options: the transform (kvc_transform) and the events that take
 * the first kernel's start and the last kernel's end (either may be null). */
struct CallOpts {
  int transform = KVC_TRANSFORM_AUTO;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

int read_opts(const kvc_launch_opts* o, bool paged, CallOpts* out) {
  if (!o) return KVC_OK;
  const int tf = o->transform;
  if (o->reserved != 0 || tf < KVC_TRANSFORM_AUTO || tf > KVC_TRANSFORM_BUTTERFLY) return KVC_EINVAL;
  if (paged && tf == KVC_TRANSFORM_BUTTERFLY) return KVC_EINVAL;
  out->transform = tf;
  out->start = static_cast<hipEvent_t>(o->start_event);
  out->stop = static_cast<hipEvent_t>(o->stop_event);
  return KVC_OK;
}

/* Calls fn(kernel, grid, args) for every launch of a plan, in order;
 * stops at the first nonzero status fn returns. */
template <typename F>
int each_launch(Op op, const Plan& plan, const CallOpts& opts, F&& fn) {
  for (int i = 0; i < plan.n_launch; ++i) {
    const LaunchShape shape = launch_shape(op, plan.args[i], plan.head_dim, plan.bits[i], opts.transform);
    Kernel k = pick(op, plan.head_dim, plan.dtype, plan.bits[i], plan.group, plan.args[i].paged != 0, shape.mode);
    if (!k) return KVC_ESHAPE;
    int64_t resident = 0;
    int cus = 0;
    int st = resident_groups(k, 64, &resident, &cus);
    if (st != KVC_OK) return st;
    int64_t waves =
        shape.waves_per_simd > 0 ? std::min<int64_t>(resident, int64_t(cus) * kSimdsPerCu * shape.waves_per_simd)
                                 : resident;
    if (shape.waves_per_cu > 0) waves = std::min<int64_t>(resident, int64_t(cus) * shape.waves_per_cu);
    // a paged call runs one launch per chunk of kReqChunk requests
    const int chunks = plan.args[i].paged ? plan.req_chunks : 1;
    for (int c = 0; c < chunks; ++c) {
      LaunchArgs a = plan.args[i];
      if (a.paged) {
        a.req_first = c * kReqChunk;
        a.nreq = std::min(kReqChunk, a.num_reqs - a.req_first);
      }
      const int64_t grid = std::min<int64_t>(a.total_items, waves);
      if (grid <= 0) continue;
      if ((st = fn(k, static_cast<unsigned>(grid), a)) != KVC_OK) return st;
    }
  }
  return KVC_OK;
}

int run_plan(Op op, const Plan& plan, void* stream, const CallOpts& opts = CallOpts()) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!opts.start && !opts.stop)
    return each_launch(op, plan, opts, [&](Kernel k, unsigned grid, LaunchArgs& a) {
      hipLaunchKernelGGL(k, dim3(grid), dim3(64), 0, s, a);
      return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP;
    });
  // timed: the events ride on the dispatches themselves, the start event on
  // the first and the stop event on the last
  int64_t n = 0;
  int st = each_launch(op, plan, opts, [&](Kernel, unsigned, LaunchArgs&) {
    ++n;
    return KVC_OK;
  });
  if (st != KVC_OK) return st;
  if (n == 0) {
    if (opts.start && hipEventRecord(opts.start, s) != hipSuccess) return KVC_EHIP;
    if (opts.stop && hipEventRecord(opts.stop, s) != hipSuccess) return KVC_EHIP;
    return KVC_OK;
  }
  int64_t j = 0;
  return each_launch(op, plan, opts, [&](Kernel k, unsigned grid, LaunchArgs& a) {
    void* args[] = {&a};
    hipEvent_t e0 = j == 0 ? opts.start : nullptr;
    hipEvent_t e1 = j == n - 1 ? opts.stop : nullptr;
    ++j;
    return hipExtLaunchKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(64), args, 0, s, e0, e1, 0) ==
                   hipSuccess
               ? KVC_OK
               : KVC_EHIP;
  });
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

kvc_status kvc_encode_with(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                           const kvc_launch_opts* opts, void* stream) {
  kvc::CallOpts o;
  int st = kvc::read_opts(opts, false, &o);
  kvc::Plan plan;
  if (st == KVC_OK) st = kvc::plan_contiguous(kvc::Op::Encode, desc, kv, out, out_bytes, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Encode, plan, stream, o);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_decode_with(const kvc_desc* desc, const void* in, uint64_t in_bytes, void* kv_out,
                           const kvc_launch_opts* opts, void* stream) {
  kvc::CallOpts o;
  int st = kvc::read_opts(opts, false, &o);
  kvc::Plan plan;
  if (st == KVC_OK) st = kvc::plan_contiguous(kvc::Op::Decode, desc, in, kv_out, in_bytes, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Decode, plan, stream, o);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_encode_paged_with(const kvc_desc* desc, const void* pool, const kvc_paged* paged, void* out,
                                 uint64_t out_bytes, const kvc_launch_opts* opts, void* stream) {
  kvc::CallOpts o;
  int st = kvc::read_opts(opts, true, &o);
  kvc::Plan plan;
  if (st == KVC_OK) st = kvc::plan_paged(kvc::Op::Encode, desc, pool, out, out_bytes, paged, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Encode, plan, stream, o);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_decode_paged_with(const kvc_desc* desc, const void* in, uint64_t in_bytes, const kvc_paged* paged,
                                 void* pool, const kvc_launch_opts* opts, void* stream) {
  kvc::CallOpts o;
  int st = kvc::read_opts(opts, true, &o);
  kvc::Plan plan;
  if (st == KVC_OK) st = kvc::plan_paged(kvc::Op::Decode, desc, in, pool, in_bytes, paged, &plan);
  if (st == KVC_OK) st = kvc::run_plan(kvc::Op::Decode, plan, stream, o);
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

}  // extern "C"
