/*
 * kvc_unfused.hip -- the encode and decode of kvc_encode / kvc_decode as a
 * chain of separate kernels that hand full-size intermediates to each other
 * through HBM.  This is the comparator for the fused kernels: the arxivlens
 * summary of "Beyond Compression Ratio: High-Throughput KV Compression for
 * Disaggregated LLM Serving" (key results) credits the fused kernel with up
 * to 5.9x over separate kernels, and its abstract attributes the gain to
 * removing the intermediate tensor and the repeated memory accesses.
 *
 * Encode (contiguous [L, 2, T, H, D] tensors), per (layer, K/V) slab:
 *   E1 rotate    x (bf16 / fp16)  -> u  fp32 [rows, D]  sign flip + transform
 *   E2 minmax    u                -> meta (the blob's meta section)
 *   E3 quantize  u, meta          -> q  u8 [rows, D]
 *   E4 pack      q                -> codes (the blob's codes section, in its
 *                                     tiled order of 16-byte pieces)
 *   E5 padding   zeroes the padding after each slab's codes and meta
 * Decode:
 *   D1 unpack    codes            -> q  u8 [rows, D]
 *   D2 dequant   q, meta          -> z  fp32 [rows, D]  (1/sqrt(D) folded in)
 *   D3 unrotate  z                -> x  butterfly, sign flip, round to dtype
 *
 * The encode stages make the same binary32 decisions as the fused encode
 * (E1 is its transform code; the meta and code arithmetic are the same
 * functions), and at 8 bits E3 decides the codes near a tie exactly as the
 * fused encode does, so the blob is bit-identical to the fused one; only
 * the memory traffic differs.  The decode stages take the textbook order -- dequantize,
 * then the whole inverse transform -- where the fused decode transforms the
 * integer codes within their groups first and scales afterwards, so the two
 * decoded tensors differ in rounding only (both well inside the decode
 * criterion against the oracle).  The stages are written to run near the HBM
 * bound on their own: 256-thread blocks, vector loads and stores that are
 * contiguous across the wave, butterfly stages across lanes by shuffles.
 */
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/kvc.h"
#include "kvc_device.h"
#include "kvc_plan.h"

namespace kvc {
namespace uf {

using dev::v2u;
using dev::v4u;

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kUnroll = 4;           // independent rows / units per thread per iteration
constexpr int64_t kMaxBlocks = 8192;  // blocks per launch (all slabs together)
constexpr int64_t kRotateBlocks = 2048;  // one-wave blocks of E1: 256 CUs x 8 resident

__device__ __forceinline__ int64_t slab_of(const LaunchArgs& a) {
  return int64_t(blockIdx.y) * a.slab_step + a.slab_first;
}

/* Butterfly stages of D values spread over D/4 consecutive lanes, 4 per
 * lane (lane m holds elements 4m .. 4m+3): two stages inside the lane, then
 * one exchange per stage with the lane whose index differs in bit h.  The
 * lower element of every pair becomes a + b and the upper a - b, in the
 * same order as the fused kernels' in-register butterfly. */
template <int D>
__device__ __forceinline__ void fwht_lanes(float (&v)[4], int m) {
  float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
  v[0] = a0 + a2;
  v[2] = a0 - a2;
  v[1] = a1 + a3;
  v[3] = a1 - a3;
#pragma unroll
  for (int h = 1; h < D / 4; h <<= 1) {
    const bool upper = (m & h) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = __shfl_xor(v[i], h);
      v[i] = upper ? t - v[i] : v[i] + t;
    }
  }
}

/* ---- encode stages ---------------------------------------------------------- */

/* E1: the fused encode's own transform stage (tile DMA, matrix-core
 * Hadamard) writing u = H (s * x) in fp32, so that the later stages see
 * exactly the values the fused kernel quantizes. */
template <int D, int DT>
KVC_KERNEL void rotate_kernel(const LaunchArgs a, float* u) {
  dev::rotate_tiles<D, DT, true>(a, u);
}

/* Start of a slab's code rows and of its meta entries in the blob (each
 * slab padded to a multiple of 256 bytes). */
__device__ __forceinline__ uint8_t* codes_of(const LaunchArgs& a, uint8_t* blob, int64_t s) {
  const int64_t l = s >> 1, kv = s & 1;
  return blob + l * (a.code_slab_k + a.code_slab_v) + (kv ? a.code_slab_k : 0);
}

__device__ __forceinline__ uint8_t* meta_of(const LaunchArgs& a, uint8_t* blob, int64_t s) {
  return blob + a.meta_offset + s * a.meta_slab;
}

/* E2: min / max per group across G/4 lanes, then the meta word. */
template <int D, int B, int G>
__global__ __launch_bounds__(kThreads) void minmax_kernel(const LaunchArgs a, const float* u) {
  constexpr int LPR = D / 4, RPW = 64 / LPR, STEP = RPW * kUnroll, GL = G / 4, NG = D / G;
  const int lane = threadIdx.x & 63, m = lane % LPR, sub = lane / LPR;
  const int64_t s = slab_of(a);
  const float4* y = reinterpret_cast<const float4*>(u) + s * a.rows * LPR;
  uint32_t* meta = reinterpret_cast<uint32_t*>(meta_of(a, static_cast<uint8_t*>(a.dst), s));
  const int64_t wave = int64_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / 64;
  const int64_t stride = int64_t(gridDim.x) * kWavesPerBlock * STEP;
  for (int64_t r0 = wave * STEP; r0 < a.rows; r0 += stride) {
    float4 w[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t r = r0 + k * RPW + sub;
      w[k] = r < a.rows ? y[r * LPR + m] : float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      float mn = fminf(fminf(w[k].x, w[k].y), fminf(w[k].z, w[k].w));
      float mx = fmaxf(fmaxf(w[k].x, w[k].y), fmaxf(w[k].z, w[k].w));
#pragma unroll
      for (int h = 1; h < GL; h <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, h));
        mx = fmaxf(mx, __shfl_xor(mx, h));
      }
      const int64_t r = r0 + k * RPW + sub;
      if (r < a.rows && m % GL == 0) meta[r * NG + m / GL] = dev::group_meta_word<D, B>(mn, mx);
    }
  }
}

/* E3 at 8 bits: the codes of unit i of slab s (elements e0 .. e0+3 of row
 * r) whose binary32 t lies within the bound of a tie are decided again
 * exactly from the row of the input tensor -- the fused encode's rule
 * (kvc_device.h, refine_ties8), with S = sum |x_j| bounded from the row's
 * meta instead: S <= D max|y|, and every rotated value of a group lies in
 * [zero, zero + 255 scale]. */
template <int D, int DT, int G>
__device__ __forceinline__ uint32_t refine_unit8(const LaunchArgs& a, int64_t s, int64_t i, float4 w, uint32_t c,
                                                 const uint32_t* meta) {
#pragma clang fp contract(off)
  constexpr int NG = D / G;
  constexpr float RS = dev::Norm<D>::inv_sqrt;
  const int64_t r = i / (D / 4);
  const int e0 = static_cast<int>(i % (D / 4)) * 4;
  const uint32_t* mrow = meta + r * NG;
  float M = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float sc = dev::f16_value(mrow[g] & 0xffffu), ze = dev::f16_value(mrow[g] >> 16);
    M = fmaxf(M, fmaxf(fabsf(ze), fabsf(ze + 255.0f * sc)));
  }
  M *= 1.004f;
  const uint32_t mg = mrow[e0 / G];
  if (!(dev::f16_value(mg & 0xffffu) > 0.0f)) return c;
  float A, Bz;
  dev::code_affine<D>(mg, A, Bz);
  const float base = dev::tie_bound_base(2.0f * D * RS * (float(D) * M), mg);
  const float v[4] = {w.x, w.y, w.z, w.w};
  uint32_t fl = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = fmaf(v[e], A, Bz);
    if (dev::near_tie(t, base + dev::kTieBoundT * fabsf(t))) fl |= 1u << e;
  }
  if (fl == 0u) return c;
  const v4u* xr = reinterpret_cast<const v4u*>(static_cast<const uint8_t*>(a.src) + (s * a.rows + r) * (2 * D));
  v4u xs[D / 8];
#pragma unroll
  for (int p = 0; p < D / 8; ++p) {
    const v4u x = xr[p];
#pragma unroll
    for (int m = 0; m < 4; ++m) xs[p][m] = x[m] ^ a.sign_words[4 * p + m];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if ((fl >> e) & 1u) {
      const uint32_t q = dev::exact_code8(dev::exact_rotated<D, DT>(xs, e0 + e), mg);
      c = (c & ~(0xffu << (8 * e))) | (q << (8 * e));
    }
  }
  return c;
}

/* E3: 4 codes per unit (one fp32 float4 in, one u32 of bytes out). */
template <int D, int DT, int B, int G>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const LaunchArgs a, const float* u, uint8_t* q8) {
  constexpr float QMAX = float((1 << B) - 1);
  constexpr int NG = D / G;
  const int64_t s = slab_of(a);
  const int64_t units = a.rows * (D / 4);
  const float4* y = reinterpret_cast<const float4*>(u) + s * units;
  uint32_t* q = reinterpret_cast<uint32_t*>(q8) + s * units;
  const uint32_t* meta =
      reinterpret_cast<const uint32_t*>(meta_of(a, static_cast<uint8_t*>(a.dst), s));
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x; i0 < units; i0 += stride * kUnroll) {
    float4 w[kUnroll];
    uint32_t mw[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = i0 + k * stride;
      w[k] = i < units ? y[i] : float4(0.0f, 0.0f, 0.0f, 0.0f);
      mw[k] = i < units ? meta[i * 4 / G] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = i0 + k * stride;
      float A, Bz;
      dev::code_affine<D>(mw[k], A, Bz);
      // min(t, 2^b - 1) changes no code of an ordinary group (every t there
      // is below 2^b - 1/2) and bounds the codes of a degenerate one; the
      // conversion rounds half to even and clamps below at 0
      uint32_t c = dev::put_byte(fminf(fmaf(w[k].x, A, Bz), QMAX), 0, 0);
      c = dev::put_byte(fminf(fmaf(w[k].y, A, Bz), QMAX), 1, c);
      c = dev::put_byte(fminf(fmaf(w[k].z, A, Bz), QMAX), 2, c);
      c = dev::put_byte(fminf(fmaf(w[k].w, A, Bz), QMAX), 3, c);
      if constexpr (B == 8) {
        if (i < units) c = refine_unit8<D, DT, G>(a, s, i, w[k], c, meta);
      }
      if (i < units) q[i] = c;
    }
  }
}


/* 32/B codes (bytes) of a unit -> one packed 32-bit word, code k at bits
 * [B*k, B*k + B). */
template <int B>
__device__ __forceinline__ uint32_t pack_bytes(const uint32_t* w) {
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 32 / B; ++k) out |= ((w[k / 4] >> (8 * (k % 4))) & ((1u << B) - 1)) << (B * k);
  return out;
}

template <int B>
__device__ __forceinline__ void unpack_bytes(uint32_t p, uint32_t* w) {
#pragma unroll
  for (int j = 0; j < 8 / B; ++j) w[j] = 0;
#pragma unroll
  for (int k = 0; k < 32 / B; ++k) w[k / 4] |= ((p >> (B * k)) & ((1u << B) - 1)) << (8 * (k % 4));
}

/*
 * Pack and unpack move one 64-row code tile per block iteration through
 * LDS, so that both sides are contiguous: the code bytes of the tile's n
 * rows (n * D bytes in the byte tensor) and its packed pieces (n * RB bytes
 * in the blob, piece-major: all rows' piece 0, then piece 1, ...).  LDS rows
 * are padded by 16 bytes so that consecutive rows fall in different banks.
 */
template <int D>
struct TileStage {
  static constexpr int kRowV4 = D / 16 + 1;  // LDS row pitch in 16-byte units
  v4u rows[kTileVectors * kRowV4];
};

/* E4: code bytes -> packed pieces, one code tile per block iteration. */
template <int D, int B>
__global__ __launch_bounds__(kThreads) void pack_kernel(const LaunchArgs a, const uint8_t* q8) {
  constexpr int RB = D * B / 8, NP = RB / 16, IN = 8 / B, RV = D / 16;  // RV: 16-byte units per code row
  __shared__ TileStage<D> st;
  const int64_t s = slab_of(a);
  const v4u* q = reinterpret_cast<const v4u*>(q8 + s * a.rows * D);
  v4u* out = reinterpret_cast<v4u*>(codes_of(a, static_cast<uint8_t*>(a.dst), s));
  const int64_t tiles = (a.rows + kTileVectors - 1) / kTileVectors;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t r0 = t * kTileVectors;
    const int n = static_cast<int>(min<int64_t>(kTileVectors, a.rows - r0));
    __syncthreads();  // the previous tile's reads of LDS are done
    for (int k = threadIdx.x; k < n * RV; k += kThreads)
      st.rows[(k / RV) * TileStage<D>::kRowV4 + k % RV] = q[r0 * RV + k];
    __syncthreads();
    for (int k = threadIdx.x; k < n * NP; k += kThreads) {
      const int c = k / n, i = k - c * n;
      const v4u* src = &st.rows[i * TileStage<D>::kRowV4 + c * IN];
      uint32_t w[4 * IN];
#pragma unroll
      for (int m = 0; m < IN; ++m) {
        const v4u v = src[m];
        w[4 * m] = v.x, w[4 * m + 1] = v.y, w[4 * m + 2] = v.z, w[4 * m + 3] = v.w;
      }
      out[r0 * NP + k] =
          v4u{pack_bytes<B>(&w[0]), pack_bytes<B>(&w[IN]), pack_bytes<B>(&w[2 * IN]), pack_bytes<B>(&w[3 * IN])};
    }
  }
}

/* E5: the padding after each slab's codes and meta, one wave per slab
 * (grid-stride over the 2 * L slabs). */
__global__ __launch_bounds__(64) void padding_kernel(const LaunchArgs a) {
  uint8_t* blob = static_cast<uint8_t*>(a.dst);
  for (int64_t s = blockIdx.x; s < 2 * a.layers; s += gridDim.x) {
    const int64_t kv = s & 1;
    const int64_t row = kv ? a.row_v : a.row_k;
    dev::zero_tail(codes_of(a, blob, s) + a.rows * row, (kv ? a.code_slab_v : a.code_slab_k) - a.rows * row);
    dev::zero_tail(meta_of(a, blob, s) + a.rows * a.groups * 4, a.meta_slab - a.rows * a.groups * 4);
  }
}

/* ---- decode stages ---------------------------------------------------------- */

/* D1: packed pieces -> code bytes, one code tile per block iteration. */
template <int D, int B>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const LaunchArgs a, uint8_t* q8) {
  constexpr int RB = D * B / 8, NP = RB / 16, OUT = 8 / B, RV = D / 16;
  __shared__ TileStage<D> st;
  const int64_t s = slab_of(a);
  const v4u* in = reinterpret_cast<const v4u*>(
      codes_of(a, const_cast<uint8_t*>(static_cast<const uint8_t*>(a.src)), s));
  v4u* q = reinterpret_cast<v4u*>(q8 + s * a.rows * D);
  const int64_t tiles = (a.rows + kTileVectors - 1) / kTileVectors;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t r0 = t * kTileVectors;
    const int n = static_cast<int>(min<int64_t>(kTileVectors, a.rows - r0));
    __syncthreads();
    for (int k = threadIdx.x; k < n * NP; k += kThreads) {
      const int c = k / n, i = k - c * n;
      const v4u p = in[r0 * NP + k];
      uint32_t w[4 * OUT];
#pragma unroll
      for (int m = 0; m < 4; ++m) unpack_bytes<B>(p[m], &w[m * OUT]);
      v4u* dst = &st.rows[i * TileStage<D>::kRowV4 + c * OUT];
#pragma unroll
      for (int m = 0; m < OUT; ++m) dst[m] = v4u{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]};
    }
    __syncthreads();
    for (int k = threadIdx.x; k < n * RV; k += kThreads)
      q[r0 * RV + k] = st.rows[(k / RV) * TileStage<D>::kRowV4 + k % RV];
  }
}

/* D2: 4 codes per unit -> 4 fp32 values z = q * scale/sqrt(D) + zero/sqrt(D). */
template <int D, int G>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const LaunchArgs a, const uint8_t* q8, float* z) {
  constexpr float RS = dev::Norm<D>::inv_sqrt;
  constexpr int NG = D / G;
  const int64_t s = slab_of(a);
  const int64_t units = a.rows * (D / 4);
  const uint32_t* q = reinterpret_cast<const uint32_t*>(q8) + s * units;
  float4* out = reinterpret_cast<float4*>(z) + s * units;
  const uint32_t* meta =
      reinterpret_cast<const uint32_t*>(meta_of(a, static_cast<uint8_t*>(const_cast<void*>(a.src)), s));
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x; i0 < units; i0 += stride * kUnroll) {
    uint32_t c[kUnroll], mw[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = i0 + k * stride;
      c[k] = i < units ? q[i] : 0u;
      mw[k] = i < units ? meta[i * 4 / G] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = i0 + k * stride;
      const float sc = dev::f16_value(mw[k] & 0xffffu) * RS;
      const float ze = dev::f16_value(mw[k] >> 16) * RS;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = fmaf(static_cast<float>((c[k] >> (8 * j)) & 0xffu), sc, ze);
      if (i < units) out[i] = float4(v[0], v[1], v[2], v[3]);
    }
  }
}

/* D3: one row per D/4 lanes; butterfly, round to the storage type, sign. */
template <int D, int DT>
__global__ __launch_bounds__(kThreads) void unrotate_kernel(const LaunchArgs a, const float* z) {
  constexpr int LPR = D / 4, RPW = 64 / LPR, STEP = RPW * kUnroll;
  const int lane = threadIdx.x & 63, m = lane % LPR, sub = lane / LPR;
  const int64_t s = slab_of(a);
  const float4* y = reinterpret_cast<const float4*>(z) + s * a.rows * LPR;
  v2u* x = static_cast<v2u*>(a.dst) + s * a.rows * LPR;
  const uint32_t s0 = a.sign_words[2 * m], s1 = a.sign_words[2 * m + 1];
  const int64_t wave = int64_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / 64;
  const int64_t stride = int64_t(gridDim.x) * kWavesPerBlock * STEP;
  for (int64_t r0 = wave * STEP; r0 < a.rows; r0 += stride) {
    float4 w[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t r = r0 + k * RPW + sub;
      w[k] = r < a.rows ? y[r * LPR + m] : float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      float v[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
      fwht_lanes<D>(v, m);
      const int64_t r = r0 + k * RPW + sub;
      if (r < a.rows) x[r * LPR + m] = v2u{dev::pack_pair<DT>(v[0], v[1]) ^ s0, dev::pack_pair<DT>(v[2], v[3]) ^ s1};
    }
  }
}

/* ---- host ---------------------------------------------------------------------- */

/* Blocks in x for a slab of `work` units handled `per_block` at a time. */
unsigned blocks_x(int64_t work, int64_t per_block, int64_t n_slabs) {
  const int64_t need = (work + per_block - 1) / per_block;
  const int64_t cap = std::max<int64_t>(1, kMaxBlocks / std::max<int64_t>(1, n_slabs));
  return static_cast<unsigned>(std::max<int64_t>(1, std::min(need, cap)));
}

template <int D>
constexpr int64_t rows_per_block() {
  return int64_t(64 / (D / 4)) * kUnroll * kWavesPerBlock;
}
constexpr int64_t kUnitsPerBlock = int64_t(kThreads) * kUnroll;

/* Run `fn(args_chunk, grid_y)` over the launch's slabs in chunks of at most
 * 65535 (the grid's y limit). */
template <typename F>
int for_slab_chunks(const LaunchArgs& a, F fn) {
  for (int64_t first = 0; first < a.n_slabs; first += 65535) {
    LaunchArgs c = a;
    c.n_slabs = std::min<int64_t>(65535, a.n_slabs - first);
    c.slab_first = a.slab_first + first * a.slab_step;
    fn(c, static_cast<unsigned>(c.n_slabs));
    if (hipGetLastError() != hipSuccess) return KVC_EHIP;
  }
  return KVC_OK;
}

template <int D, int DT, int B, int G>
int encode_launch(const LaunchArgs& a, hipStream_t st, uint8_t* q8, float* u) {
  // E1 walks the launch's tiles on a persistent grid of one-wave blocks
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(a.total_items, kRotateBlocks));
  if (grid > 0) {
    hipLaunchKernelGGL((rotate_kernel<D, DT>), dim3(grid), dim3(64), 0, st, a, u);
    if (hipGetLastError() != hipSuccess) return KVC_EHIP;
  }
  return for_slab_chunks(a, [&](const LaunchArgs& c, unsigned gy) {
    const unsigned rx = blocks_x(c.rows, rows_per_block<D>(), c.n_slabs);
    const unsigned ex = blocks_x(c.rows * (D / 4), kUnitsPerBlock, c.n_slabs);
    const unsigned px = blocks_x(c.rows, kTileVectors, c.n_slabs);
    hipLaunchKernelGGL((minmax_kernel<D, B, G>), dim3(rx, gy), dim3(kThreads), 0, st, c, u);
    hipLaunchKernelGGL((quantize_kernel<D, DT, B, G>), dim3(ex, gy), dim3(kThreads), 0, st, c, u, q8);
    hipLaunchKernelGGL((pack_kernel<D, B>), dim3(px, gy), dim3(kThreads), 0, st, c, q8);
  });
}

template <int D, int DT, int B, int G>
int decode_launch(const LaunchArgs& a, hipStream_t st, uint8_t* q8, float* z) {
  return for_slab_chunks(a, [&](const LaunchArgs& c, unsigned gy) {
    const unsigned rx = blocks_x(c.rows, rows_per_block<D>(), c.n_slabs);
    const unsigned ex = blocks_x(c.rows * (D / 4), kUnitsPerBlock, c.n_slabs);
    const unsigned px = blocks_x(c.rows, kTileVectors, c.n_slabs);
    hipLaunchKernelGGL((unpack_kernel<D, B>), dim3(px, gy), dim3(kThreads), 0, st, c, q8);
    hipLaunchKernelGGL((dequant_kernel<D, G>), dim3(ex, gy), dim3(kThreads), 0, st, c, q8, z);
    hipLaunchKernelGGL((unrotate_kernel<D, DT>), dim3(rx, gy), dim3(kThreads), 0, st, c, z);
  });
}

template <bool ENC, int D, int DT, int B>
int dispatch_g(int g, const LaunchArgs& a, hipStream_t st, uint8_t* q8, float* f) {
  switch (g) {
    case 32: return ENC ? encode_launch<D, DT, B, 32>(a, st, q8, f) : decode_launch<D, DT, B, 32>(a, st, q8, f);
    case 64: return ENC ? encode_launch<D, DT, B, 64>(a, st, q8, f) : decode_launch<D, DT, B, 64>(a, st, q8, f);
    case 128:
      if constexpr (D >= 128)
        return ENC ? encode_launch<D, DT, B, 128>(a, st, q8, f) : decode_launch<D, DT, B, 128>(a, st, q8, f);
      return KVC_EGROUP;
    default: return KVC_EGROUP;
  }
}

template <bool ENC, int D, int DT>
int dispatch_b(int b, int g, const LaunchArgs& a, hipStream_t st, uint8_t* q8, float* f) {
  switch (b) {
    case 2: return dispatch_g<ENC, D, DT, 2>(g, a, st, q8, f);
    case 4: return dispatch_g<ENC, D, DT, 4>(g, a, st, q8, f);
    case 8: return dispatch_g<ENC, D, DT, 8>(g, a, st, q8, f);
    default: return KVC_EBITS;
  }
}

template <bool ENC>
int run(const Plan& plan, hipStream_t st, uint8_t* q8, float* f) {
  for (int i = 0; i < plan.n_launch; ++i) {
    const LaunchArgs& a = plan.args[i];
    const int b = plan.bits[i], g = plan.group;
    int rc;
    if (plan.head_dim == 64)
      rc = plan.dtype == KVC_BF16 ? dispatch_b<ENC, 64, 0>(b, g, a, st, q8, f) : dispatch_b<ENC, 64, 1>(b, g, a, st, q8, f);
    else
      rc = plan.dtype == KVC_BF16 ? dispatch_b<ENC, 128, 0>(b, g, a, st, q8, f)
                                  : dispatch_b<ENC, 128, 1>(b, g, a, st, q8, f);
    if (rc != KVC_OK) return rc;
  }
  if (ENC && plan.n_launch > 0) {
    const LaunchArgs& a = plan.args[0];
    const bool padded = a.code_slab_k != uint64_t(a.rows) * a.row_k || a.code_slab_v != uint64_t(a.rows) * a.row_v ||
                        a.meta_slab != uint64_t(a.rows) * a.groups * 4;
    if (padded) {
      const unsigned grid = static_cast<unsigned>(std::min<int64_t>(2 * a.layers, 1024));
      hipLaunchKernelGGL(padding_kernel, dim3(grid), dim3(64), 0, st, a);
      if (hipGetLastError() != hipSuccess) return KVC_EHIP;
    }
  }
  return KVC_OK;
}

/* Validate the workspace and split it: codes bytes first, fp32 after. */
int split_workspace(const kvc_desc* d, void* ws, uint64_t ws_bytes, uint8_t** q8, float** f) {
  uint64_t need = 0, fp_off = 0;
  int st = unfused_workspace(d, &need, &fp_off);
  if (st != KVC_OK) return st;
  if (need == 0) return KVC_OK;
  if (!ws) return KVC_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 15u) return KVC_EALIGN;
  if (ws_bytes < need) return KVC_ENOSPC;
  *q8 = static_cast<uint8_t*>(ws);
  *f = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + fp_off);
  return KVC_OK;
}

/*
 * Workspace of kvc_encode_unfused_noalloc: a static device array, so that
 * the call allocates nothing.  Every device the library runs on holds its
 * own copy for the life of the process.  In host code `scratch` names a
 * host-side stand-in, not device memory: its device address on the current
 * device comes from hipGetSymbolAddress, taken once per device and kept.
 * The encode stages write every byte of the workspace they read, so nothing
 * in it has to start at zero, and it keeps the last call's contents.
 */
constexpr uint64_t kStaticWorkspaceBytes = uint64_t(KVC_NOALLOC_WORKSPACE_BYTES);
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int static_workspace(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_EHIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVC_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace uf
}  // namespace kvc

extern "C" {

kvc_status kvc_encode_unfused_noalloc(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                                      void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Encode, desc, kv, out, out_bytes, &plan);
  uint64_t need = 0;
  if (st == KVC_OK) st = kvc::unfused_workspace(desc, &need, nullptr);
  if (st == KVC_OK && need > kvc::uf::kStaticWorkspaceBytes) st = KVC_ENOSPC;
  void* ws = nullptr;
  if (st == KVC_OK && need > 0) st = kvc::uf::static_workspace(&ws);
  uint8_t* q8 = nullptr;
  float* f = nullptr;
  if (st == KVC_OK) st = kvc::uf::split_workspace(desc, ws, kvc::uf::kStaticWorkspaceBytes, &q8, &f);
  if (st == KVC_OK) st = kvc::uf::run<true>(plan, static_cast<hipStream_t>(stream), q8, f);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_encode_unfused(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Encode, desc, kv, out, out_bytes, &plan);
  uint8_t* q8 = nullptr;
  float* f = nullptr;
  if (st == KVC_OK) st = kvc::uf::split_workspace(desc, workspace, workspace_bytes, &q8, &f);
  if (st == KVC_OK) st = kvc::uf::run<true>(plan, static_cast<hipStream_t>(stream), q8, f);
  return static_cast<kvc_status>(st);
}

kvc_status kvc_decode_unfused(const kvc_desc* desc, const void* in, uint64_t in_bytes, void* kv_out,
                              void* workspace, uint64_t workspace_bytes, void* stream) {
  kvc::Plan plan;
  int st = kvc::plan_contiguous(kvc::Op::Decode, desc, in, kv_out, in_bytes, &plan);
  uint8_t* q8 = nullptr;
  float* f = nullptr;
  if (st == KVC_OK) st = kvc::uf::split_workspace(desc, workspace, workspace_bytes, &q8, &f);
  if (st == KVC_OK) st = kvc::uf::run<false>(plan, static_cast<hipStream_t>(stream), q8, f);
  return static_cast<kvc_status>(st);
}

}  // extern "C"
