/*
 * kvc_device.h -- device code of the fused KV-cache encode / decode for
 * CDNA4 (gfx950): kernels as templates over head_dim, dtype, code width and
 * group size.  Instantiated by kvc_inst.hip, launched by kvc_launch.hip.
 *
 * What is computed follows the episode notes of "FastKVComp: checking
 * whether high-throughput KV compression pays off" (randomized Hadamard
 * transform, then low-bit quantization, then a lossless codec that is not
 * built here) and the abstract of "Beyond Compression Ratio: High-Throughput
 * KV Compression for Disaggregated LLM Serving" (the transform and the
 * quantization run fused in one tiled kernel with no full-size intermediate
 * tensor).  The encode reads each head_dim vector once from HBM, and writes
 * only its packed codes and its per-group fp16 (scale, zero); the decode
 * reads those and writes the vector once.
 *
 * Work decomposition (one wave64 per workgroup, persistent grid):
 *   - an item is a tile of up to 64 consecutive head_dim vectors of one
 *     (layer, K/V) slab, contiguous in the KV tensor or in one pool block;
 *   - the tile reaches LDS by DMA (global_load_lds_dwordx4: 1 KiB per
 *     instruction, fully coalesced, no register staging), laid out with an
 *     XOR swizzle so that the per-lane row reads are free of bank conflicts;
 *     every lane then owns one whole vector in registers;
 *   - encode: the Walsh-Hadamard transform of the tile runs on the matrix
 *     cores (exact bf16 / fp16 products against +-1, fp32 sums), after
 *     which every lane again holds its own vector -- or, when a caller asks
 *     for it, as the in-register butterfly of each lane's vector; the group
 *     min/max, the fp16 meta, the quantization and the packing run inside
 *     the lane;
 *   - decode: the codes are transformed within their groups (exactly, on
 *     the matrix cores or as a butterfly), scaled, combined across groups
 *     and rounded to the storage type inside the lane; the rows leave
 *     through LDS as coalesced stores;
 *   - no intermediate touches memory, and as soon as a tile's rows (or
 *     codes) are in registers the wave's next tile is requested, so HBM
 *     traffic overlaps the arithmetic.
 */
#ifndef KVC_DEVICE_H
#define KVC_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_plan.h"

#define KVC_CURSOR_FN __device__ __forceinline__
#include "kvc_cursor.h"

namespace kvc {
namespace dev {

/* Register budget: room for at least this many waves per SIMD (512 / N
 * registers per lane).  The launches use one or two waves per SIMD, chosen
 * per kernel and size (kvc_launch.hip); two must always fit. */
#ifndef KVC_WAVES_PER_EU
#define KVC_WAVES_PER_EU 2
#endif
#define KVC_KERNEL __global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KVC_WAVES_PER_EU)))

/* Phase boundary for the instruction scheduler: nothing moves across it, so
 * loads of a later phase are not hoisted into an earlier one (which would
 * keep their results live over the 128-register transform). */
#define KVC_PHASE() __builtin_amdgcn_sched_barrier(0)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // 16-byte chunk
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

template <int D>
struct Norm;
template <>
struct Norm<64> {
  static constexpr float inv_sqrt = 0.125f;
  static constexpr double inv_sqrt_d = 0.125;
};
template <>
struct Norm<128> {
  static constexpr float inv_sqrt = 0.088388347648318440550f;  // 1/sqrt(128)
  static constexpr double inv_sqrt_d = 0.088388347648318440550;
};

/* ---- element conversions ------------------------------------------------ */

/* Two packed storage elements (element 2m in the low half) -> fp32. */
template <int DT>
__device__ __forceinline__ void unpack_pair(uint32_t w, float& lo, float& hi) {
  if constexpr (DT == KVC_BF16) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  } else {
    half2_t h = __builtin_bit_cast(half2_t, w);
    lo = static_cast<float>(h.x);
    hi = static_cast<float>(h.y);
  }
}

/* fp32 pair -> packed storage, round to nearest even. */
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  float2_t f = {lo, hi};
  if constexpr (DT == KVC_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf162_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
  }
}

__device__ __forceinline__ uint32_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
__device__ __forceinline__ float f16_value(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

/* fp32 -> fp16 rounding toward -inf: round to nearest, then step down one
 * binary16 value if that overshot. */
__device__ __forceinline__ uint32_t rd16(float v) {
  uint32_t h = f16_bits(v);
  if (f16_value(h) > v) h = (h & 0x8000u) ? h + 1u : (h == 0u ? 0x8001u : h - 1u);
  return h;
}

/* fp32 -> fp16 rounding toward +inf. */
__device__ __forceinline__ uint32_t ru16(float v) {
  uint32_t h = f16_bits(v);
  if (f16_value(h) < v) h = (h & 0x8000u) ? (h == 0x8000u ? 1u : h - 1u) : h + 1u;
  return h;
}

/* ---- transform ------------------------------------------------------------ */

/* ---- quantization and packing ------------------------------------------ */

/* v_cvt_pk_u8_f32 rounds to nearest even and clamps to [0, 255] (checked on
 * gfx950 for ties k + 1/2, negative values and values above 255), so it both
 * rounds the code and inserts it into byte `sel` of `acc`. */
__device__ __forceinline__ uint32_t put_byte(float t, uint32_t sel, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(t, sel, acc);
}

/* One 32-bit word of packed codes from 32/B consecutive values t. */
template <int B>
__device__ __forceinline__ uint32_t pack_word(const float* t) {
  if constexpr (B == 8) {
    uint32_t w = put_byte(t[0], 0, 0);
    w = put_byte(t[1], 1, w);
    w = put_byte(t[2], 2, w);
    return put_byte(t[3], 3, w);
  } else if constexpr (B == 4) {
    uint32_t e = put_byte(t[0], 0, 0), o = put_byte(t[1], 0, 0);
    e = put_byte(t[2], 1, e);
    o = put_byte(t[3], 1, o);
    e = put_byte(t[4], 2, e);
    o = put_byte(t[5], 2, o);
    e = put_byte(t[6], 3, e);
    o = put_byte(t[7], 3, o);
    return e | (o << 4);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = put_byte(t[i], 0, 0);
      v = put_byte(t[4 + i], 1, v);
      v = put_byte(t[8 + i], 2, v);
      w[i] = put_byte(t[12 + i], 3, v);
    }
    return w[0] | (w[1] << 2) | (w[2] << 4) | (w[3] << 6);
  }
}

/* Codes of one 32-bit word -> 32/B floats. */
template <int B>
__device__ __forceinline__ void unpack_word(uint32_t u, float* q) {
  auto byte = [](uint32_t x, int k) { return static_cast<float>((x >> (8 * k)) & 0xffu); };
  if constexpr (B == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = byte(u, k);
  } else if constexpr (B == 4) {
    uint32_t e = u & 0x0f0f0f0fu, o = (u >> 4) & 0x0f0f0f0fu;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q[2 * k] = byte(e, k);
      q[2 * k + 1] = byte(o, k);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = (u >> (2 * i)) & 0x03030303u;
#pragma unroll
      for (int k = 0; k < 4; ++k) q[4 * k + i] = byte(w, k);
    }
  }
}

/* ---- work items ------------------------------------------------------------ */

/*
 * Code rows are stored in tiles of 64 rows per (layer, K/V) slab: tile k of
 * a slab starts at byte 64 * k * RB, and inside a tile of n rows the
 * 16-byte piece c of row i sits at byte (c * n + i) * 16, so a wave writes
 * (and reads back) each piece of its 64 rows as one contiguous KiB.
 *
 * A work tile covers `count` vectors; its first one is row i0 of the code
 * tile that starts at `codes` (n rows).  Contiguous work tiles are the code
 * tiles themselves (i0 = 0, n = count); a paged one (a block's rows) can
 * run into the next code tile, of n_next rows, at codes + 64 * RB.  The
 * three small numbers share one word (`geom`, 8 bits each), which keeps
 * the paged kernels' scalar registers from spilling.
 */
struct Tile {
  const uint8_t* src;  // first byte of the tile's vectors in the KV tensor / pool
  uint8_t* codes;      // start of the code tile holding the tile's first row
  uint8_t* meta;       // first meta entry of the tile in the blob
  int count;           // valid vectors, 1..64
  uint32_t geom;       // paged: i0 | n << 8 | n_next << 16
};

__device__ __forceinline__ uint32_t code_geom(int64_t i0, int64_t n, int64_t n_next) {
  return uint32_t(i0) | uint32_t(n) << 8 | uint32_t(n_next > 0 ? n_next : 0) << 16;
}

/* This lane's code row: pieces at piece_base[c * piece_stride], c < RB/16. */
template <int RB, bool PAGED>
__device__ __forceinline__ v4u* code_row(const Tile& t, int lane, int& piece_stride) {
  v4u* base = reinterpret_cast<v4u*>(t.codes);
  if constexpr (!PAGED) {
    piece_stride = t.count;
    return base + lane;
  } else {
    const int i0 = t.geom & 0xffu, n = (t.geom >> 8) & 0xffu;
    if (i0 + t.count <= kTileVectors) {  // wave-uniform: the tile stays in one code tile
      piece_stride = n;
      return base + i0 + lane;
    }
    const int i = i0 + lane;
    if (i < kTileVectors) {
      piece_stride = n;
      return base + i;
    }
    piece_stride = t.geom >> 16;
    return base + kTileVectors * (RB / 16) + (i - kTileVectors);
  }
}

/* Zero the padding after a slab's codes or meta: n < 256 bytes, a multiple
 * of 4, from a 4-byte aligned address (one dword store per lane). */
__device__ __forceinline__ void zero_tail(uint8_t* p, uint64_t n) {
  typedef __attribute__((address_space(1))) uint32_t global_u32;
  if (threadIdx.x * 4u < n) ((global_u32*)p)[threadIdx.x] = 0;
}

__device__ __forceinline__ uint64_t align256(uint64_t n) { return (n + 255u) & ~uint64_t(255); }

/* Wave-uniform read of a value that no kernel of the launch writes (block
 * table, lengths, offsets): through the constant address space, so it
 * becomes a scalar load and never joins the vector-memory wait counter. */
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

/*
 * Wave-uniform position in a launch's item space, advanced by the grid size
 * without divisions.
 *
 * Contiguous items walk the launch's slabs tile by tile (kvc_cursor.h: slab
 * offsets carried along, no products per step).
 *
 * Paged items are taken in units: unit (c, b) is item b of the launch's
 * slabs [c * R, min(n_slabs, c * R + R)), units numbered c * per_slab + b.
 * A wave resolves, checks and addresses a unit's first tile, then walks the
 * unit's other slabs by adding strides to that tile's addresses (the pool's
 * slab stride, and the request's code and meta slab sizes), so the per-item
 * work below is paid once per R tiles.  The decode walks R = a.run slabs
 * (WALK); the encode takes R = 1, with no walk state: its kernel is short
 * of scalar registers, and the walk's state cost it more than the walk
 * saved.
 *
 * Request order: a launch covers requests [req_first, req_first + nreq), at
 * most one per lane.  At its start every wave loads the lengths and blob
 * offsets of those requests into its lanes (lane r: request req_first + r),
 * checks them, and numbers the items of a slab request by request with a
 * prefix sum over the lanes: request r owns ceil(len / block_size) *
 * subtiles items, so there are no empty items.  An item's request is then
 * the number of lanes whose running total is at or below it (one ballot),
 * and its length and offset come from that lane (readlane).  The cursor runs
 * one unit ahead of the tiles it hands out: the block-table entry of the
 * next unit is loaded while the current one is worked on.
 *
 * Pool order: when the call brings a list of its (request, block) items
 * sorted by pool block (kvc_paged_item), item b of a slab is entry
 * b / subtiles of the list, and the entry carries the pool block, the
 * request's length and its blob offset; the waves then sweep the pool in
 * address order (neighbouring blocks at the same time) instead of in the
 * table's random order.  The entry of the next unit is loaded ahead, and
 * its length and offset are checked per unit.
 */
struct PagedPos {
  int64_t unit;          // unit of the launch
  int64_t i, b;          // its first slab i (of the launch) and item b of the slab
  int32_t r, j, sub;     // request, block of the request, subtile of the block
  int32_t blk;           // pool block of (r, j), loaded ahead
  int32_t len;           // tokens of request r
  int64_t off;           // blob offset of request r
};

struct Cursor {
  ContigCursor k;
  // paged: lane values (lane r = request req_first + r)
  int32_t incl;          // items of requests 0..r of this launch (one slab); past nreq: INT32_MAX
  int32_t len;           // tokens of request r, 0 when the request is invalid
  int64_t off;           // byte offset of request r's blob
  // paged: wave-uniform
  int64_t per_slab, total, di, db;
  // log2 of row_k, row_v and groups * 4: every supported (head_dim, bits,
  // group) makes them powers of two, so the per-item sizes and offsets are
  // shifts rather than 64-bit products
  int32_t sh_k, sh_v, sh_m;
  PagedPos cur, ahead;
  // paged, WALK: the current unit's slabs after the latest tile handed
  // out, and the blob bytes from one of its slabs to the next
  int32_t left;
  int64_t dcodes, dmeta;
};

__device__ __forceinline__ int32_t lane_value(int32_t v, int32_t lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ int64_t lane_value64(int64_t v, int32_t lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int32_t>(static_cast<uint64_t>(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int32_t>(static_cast<uint64_t>(v) >> 32), lane);
  return static_cast<int64_t>((uint64_t(hi) << 32) | lo);
}

/* Blob bytes of a request of `len` tokens: (code slab K, code slab V, meta
 * slab, total); every slab padded to a multiple of 256 bytes. */
struct ReqSizes {
  uint64_t ck, cv, mslab, total;
};
__device__ __forceinline__ ReqSizes req_sizes(const LaunchArgs& a, int64_t len) {
  ReqSizes z;
  const uint64_t rows = uint64_t(len) * uint64_t(a.heads);
  z.ck = align256(rows * uint64_t(a.row_k));
  z.cv = align256(rows * uint64_t(a.row_v));
  z.mslab = align256(rows * uint64_t(a.groups) * 4u);
  z.total = uint64_t(a.layers) * (z.ck + z.cv) + uint64_t(a.layers) * 2u * z.mslab;
  return z;
}

/* req_sizes with the shifts of the cursor (one 32 x 32-bit product). */
__device__ __forceinline__ ReqSizes req_sizes_sh(const LaunchArgs& a, const Cursor& c, int32_t len) {
  ReqSizes z;
  const uint64_t rows = uint64_t(uint32_t(len)) * uint64_t(uint32_t(a.heads));
  z.ck = align256(rows << c.sh_k);
  z.cv = align256(rows << c.sh_v);
  z.mslab = align256(rows << c.sh_m);
  z.total = uint64_t(a.layers) * (z.ck + z.cv) + uint64_t(a.layers) * 2u * z.mslab;
  return z;
}

/* (request, block, subtile) of item b of a slab, its pool block, and the
 * request's length and blob offset. */
__device__ __forceinline__ void paged_resolve(const LaunchArgs& a, const Cursor& c, PagedPos& p) {
  if (a.order) {  // pool order: entry b / subtiles of the list
    int64_t e = p.b;
    p.sub = 0;
    if (a.subtiles != 1) {
      e = p.b / a.subtiles;
      p.sub = static_cast<int32_t>(p.b - e * a.subtiles);
    }
    // the 32-byte entry (block, block_index, req, len, offset, reserved) as two
    // 16-byte scalar loads
    const v4u* q = reinterpret_cast<const v4u*>(a.order + e);
    const v4u w0 = ld_const(q), w1 = ld_const(q + 1);
    p.blk = static_cast<int32_t>(w0.x);
    p.j = static_cast<int32_t>(w0.y);
    p.r = static_cast<int32_t>(w0.z);
    p.len = static_cast<int32_t>(w0.w);
    p.off = static_cast<int64_t>((uint64_t(w1.y) << 32) | w1.x);
    return;
  }
  const uint64_t below = __builtin_amdgcn_ballot_w64(int64_t(c.incl) <= p.b);
  p.r = __builtin_popcountll(below);
  const int32_t first = p.r > 0 ? lane_value(c.incl, p.r - 1) : 0;
  const int32_t e = static_cast<int32_t>(p.b) - first;
  if (a.subtiles == 1) {
    p.j = e;
    p.sub = 0;
  } else {
    p.j = e / a.subtiles;
    p.sub = e - p.j * a.subtiles;
  }
  p.blk = ld_const(a.table + int64_t(a.req_first + p.r) * a.max_blocks + p.j);
  p.len = lane_value(c.len, p.r);
  p.off = lane_value64(c.off, p.r);
}

/* Slabs per unit. */
template <bool WALK>
__device__ __forceinline__ int32_t unit_slabs(const LaunchArgs& a) {
  return WALK ? a.run : 1;
}

template <bool WALK>
__device__ __forceinline__ void paged_step(const LaunchArgs& a, const Cursor& c, PagedPos& p) {
  p.unit += gridDim.x;
  p.i += c.di;
  p.b += c.db;
  if (p.b >= c.per_slab) {
    p.b -= c.per_slab;
    p.i += unit_slabs<WALK>(a);
  }
}

/* Units per item of a slab: the launch's slabs in runs of unit_slabs. */
template <bool WALK>
__device__ __forceinline__ int64_t unit_rows(const LaunchArgs& a) {
  return WALK ? (a.n_slabs + a.run - 1) / a.run : a.n_slabs;
}

/* The unit steps and the first unit's slab in slabs rather than in runs. */
template <bool WALK>
__device__ __forceinline__ void unit_scale(const LaunchArgs& a, Cursor& c) {
  if constexpr (WALK) {
    c.di *= a.run;
    c.cur.i *= a.run;
    c.left = 0;
  }
}

/* Per-wave set-up of a paged launch: the lanes' requests, checked (a length
 * outside [0, max_blocks * block_size] or a blob offset that is negative,
 * not a multiple of 16 or whose blob would end past the buffer: the request
 * is skipped and bit 0 of *err set), the item numbering, and the wave's
 * first two units. */
template <bool WALK>
__device__ __forceinline__ void paged_init(const LaunchArgs& a, Cursor& c) {
  const int lane = threadIdx.x;
  c.sh_k = __builtin_ctz(uint32_t(a.row_k));
  c.sh_v = __builtin_ctz(uint32_t(a.row_v));
  c.sh_m = __builtin_ctz(uint32_t(a.groups) * 4u);
  if (a.order) {  // pool order: the list numbers the items; nothing per lane
    c.per_slab = a.order_len * a.subtiles;
    c.total = c.per_slab * unit_rows<WALK>(a);
    c.cur.unit = blockIdx.x;
    if (c.per_slab == 0 || c.cur.unit >= c.total) {
      c.total = 0;
      return;
    }
    const int64_t step = gridDim.x;
    c.di = step / c.per_slab;
    c.db = step - c.di * c.per_slab;
    c.cur.i = c.cur.unit / c.per_slab;
    c.cur.b = c.cur.unit - c.cur.i * c.per_slab;
    unit_scale<WALK>(a, c);
    paged_resolve(a, c, c.cur);
    c.ahead = c.cur;
    paged_step<WALK>(a, c, c.ahead);
    if (c.ahead.unit < c.total) paged_resolve(a, c, c.ahead);
    return;
  }
  int32_t len = 0;
  int64_t off = 0;
  int32_t items = 0;
  if (lane < a.nreq) {
    len = a.lens[a.req_first + lane];
    off = a.offsets[a.req_first + lane];
    bool ok = len >= 0 && int64_t(len) <= int64_t(a.max_blocks) * a.block_size;
    if (ok) {
      const ReqSizes z = req_sizes(a, len);
      ok = off >= 0 && !(off & 15) && uint64_t(off) <= a.blob_bytes && z.total <= a.blob_bytes - uint64_t(off);
    }
    if (!ok) {
      if (a.err) atomicOr(a.err, 1);
      len = 0;
    }
    // at most max_blocks * subtiles, which the host keeps below INT32_MAX / 64
    items = static_cast<int32_t>((int64_t(len) + a.block_size - 1) / a.block_size * a.subtiles);
  }
  // inclusive prefix sum of the items over the lanes
  int32_t incl = items;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  c.per_slab = lane_value(incl, a.nreq - 1);
  c.incl = lane < a.nreq ? incl : INT32_MAX;
  c.len = len;
  c.off = off;
  c.total = c.per_slab * unit_rows<WALK>(a);
  c.cur.unit = blockIdx.x;
  if (c.per_slab == 0 || c.cur.unit >= c.total) {
    c.total = 0;
    return;
  }
  const int64_t step = gridDim.x;
  c.di = step / c.per_slab;
  c.db = step - c.di * c.per_slab;
  c.cur.i = c.cur.unit / c.per_slab;
  c.cur.b = c.cur.unit - c.cur.i * c.per_slab;
  unit_scale<WALK>(a, c);
  paged_resolve(a, c, c.cur);
  c.ahead = c.cur;
  paged_step<WALK>(a, c, c.ahead);
  if (c.ahead.unit < c.total) paged_resolve(a, c, c.ahead);
}

/* The ahead unit becomes the current one; the next one is resolved and its
 * table entry requested. */
template <bool WALK>
__device__ __forceinline__ void paged_advance(const LaunchArgs& a, Cursor& c) {
  c.cur = c.ahead;
  paged_step<WALK>(a, c, c.ahead);
  if (c.ahead.unit < c.total) paged_resolve(a, c, c.ahead);
}

template <bool PAGED, bool WALK>
__device__ __forceinline__ void cursor_init(const LaunchArgs& a, Cursor& c) {
  if constexpr (!PAGED) {
    contig_init(a, int64_t(blockIdx.x), int64_t(gridDim.x), c.k);
  } else {
    paged_init<WALK>(a, c);
  }
}

/*
 * The tile of the cursor's item (paged: the first tile of the cursor's
 * unit, which also sets up the walk over the unit's other slabs).  Paged
 * units whose subtile lies past the request's last token (the last block's
 * tail) are skipped (false), as are units whose table entry lies outside
 * the pool (bit 0 of *err is then set).  `tensor` is the KV side (source of
 * an encode, destination of a decode), `blob` the encoded side.  With PAD,
 * the last tile of each slab also zeroes the padding that follows the
 * slab's codes and its meta (each is padded to a multiple of 256 bytes),
 * right when it is found.
 */
template <int D, bool PAD, bool PAGED, bool WALK>
__device__ __forceinline__ bool cursor_tile(const LaunchArgs& a, Cursor& c, const uint8_t* tensor,
                                            uint8_t* blob, Tile& t) {
  constexpr int64_t vec_bytes = int64_t(D) * 2;
  if constexpr (!PAGED) {
    ContigTile ct;
    contig_tile(a, c.k, vec_bytes, ct);
    t.count = ct.count;
    t.geom = 0;
    t.src = tensor + ct.src;
    t.codes = blob + ct.codes;
    t.meta = blob + ct.meta;
    if (PAD && ct.last) {  // the slab's last tile also zeroes its padding
      zero_tail(blob + c.k.codes + a.rows * a.row, uint32_t(a.code_tail));
      zero_tail(blob + c.k.meta + a.rows * a.groups * 4, uint32_t(a.meta_tail));
    }
    return true;
  }
  const PagedPos& p = c.cur;
  const int32_t len = p.len;
  const int64_t off = p.off;
  const ReqSizes z = req_sizes_sh(a, c, len);  // meaningful once len >= 0 is checked below
  if (a.order) {  // a listed item carries its own length and offset: check them here
    const bool ok = len >= 0 && int64_t(len) <= int64_t(a.max_blocks) * a.block_size && p.j >= 0 &&
                    int64_t(p.j) * a.block_size < int64_t(len) && off >= 0 && !(off & 15) &&
                    uint64_t(off) <= a.blob_bytes && z.total <= a.blob_bytes - uint64_t(off);
    if (!ok) {
      if (a.err) atomicOr(a.err, 1);
      return false;
    }
  }
  const int32_t first_tok = p.j * a.block_size;  // < len: at most max_blocks * block_size <= INT32_MAX
  const int32_t ntok = min(a.block_size, len - first_tok);
  const int32_t v0 = p.sub * kTileVectors;
  const int32_t nvec = ntok * a.heads;
  if (v0 >= nvec) return false;
  if (p.blk < 0 || p.blk >= a.num_blocks) {
    if (a.err) atomicOr(a.err, 1);
    return false;
  }
  const int64_t rows = int64_t(len) * a.heads;
  const uint64_t meta_start = uint64_t(a.layers) * (z.ck + z.cv);
  const int64_t s = p.i * a.slab_step + a.slab_first;
  const int64_t l = s >> 1, kv = s & 1;
  const int sh = kv ? c.sh_v : c.sh_k;  // log2 of the slab's code row bytes
  const int64_t row0 = int64_t(first_tok) * a.heads + v0;  // t*H + h of the tile's first vector
  const int64_t tile0 = row0 / kTileVectors * kTileVectors;  // first row of its code tile
  t.count = min(kTileVectors, nvec - v0);
  t.geom = code_geom(row0 - tile0, min<int64_t>(kTileVectors, rows - tile0),
                     min<int64_t>(kTileVectors, rows - tile0 - kTileVectors));
  t.src = tensor + ((s * a.num_blocks + p.blk) * int64_t(a.block_size) * a.heads + v0) * vec_bytes;
  uint8_t* cs = blob + off + l * (z.ck + z.cv) + (kv ? z.ck : 0);
  uint8_t* ms = blob + off + meta_start + s * z.mslab;
  t.codes = cs + (tile0 << sh);
  t.meta = ms + (row0 << c.sh_m);
  if (PAD && row0 + t.count == rows) {  // the slab's last tile also zeroes its padding
    zero_tail(cs + (rows << sh), (kv ? z.cv : z.ck) - (uint64_t(rows) << sh));
    zero_tail(ms + (rows << c.sh_m), z.mslab - (uint64_t(rows) << c.sh_m));
  }
  if constexpr (WALK) {
    // the unit's next slab is slab_step slabs on; with slab_step 1 that is
    // the V slab after a K slab or the next layer's K slab after a V slab,
    // and the launch then holds K and V of equal code widths (ck == cv)
    c.left = static_cast<int32_t>(min<int64_t>(a.run, a.n_slabs - c.cur.i)) - 1;
    c.dcodes = static_cast<int64_t>(a.slab_step == 1 ? z.ck : z.ck + z.cv);
    c.dmeta = a.slab_step * static_cast<int64_t>(z.mslab);
  }
  return true;
}

/* The paged cursor's unit on its next slab: tile `prev` (the unit's latest
 * one) slab_step slabs on (the caller checked c.left > 0). */
__device__ __forceinline__ void walk_next(const LaunchArgs& a, Cursor& c, const Tile& prev, Tile& t) {
  --c.left;
  t = prev;
  t.src += a.src_stride;
  t.codes += c.dcodes;
  t.meta += c.dmeta;
}

/* Advance to the next item of this wave that maps to a tile (paged: the
 * current unit's next slab, else the next unit that maps to one).  `prev`
 * is the tile the previous call handed out (ignored when `first`).  WALK
 * units hold no padding: the decode walks them, the encode (PAD) does not. */
template <int D, bool PAD, bool PAGED, bool WALK>
__device__ __forceinline__ bool next_tile(const LaunchArgs& a, Cursor& c, const uint8_t* tensor, uint8_t* blob,
                                          const Tile& prev, Tile& t, bool first) {
  static_assert(!(PAD && WALK), "a walked unit does not zero padding");
  if constexpr (!PAGED) {
    if (!first) contig_next(a, int64_t(gridDim.x), c.k);
    while (c.k.item < a.total_items) {
      if (cursor_tile<D, PAD, PAGED, WALK>(a, c, tensor, blob, t)) return true;
      contig_next(a, int64_t(gridDim.x), c.k);
    }
    return false;
  } else {
    if (!first) {
      if (WALK && c.left > 0) {
        walk_next(a, c, prev, t);
        return true;
      }
      paged_advance<WALK>(a, c);
    }
    while (c.cur.unit < c.total) {
      if (cursor_tile<D, PAD, PAGED, WALK>(a, c, tensor, blob, t)) return true;
      paged_advance<WALK>(a, c);
    }
    return false;
  }
}

/* ---- LDS staging ------------------------------------------------------------- */

typedef __attribute__((address_space(3))) void lds_void;
/* A tile buffer as an LDS-space pointer.  The kernels cast their __shared__
 * array once at the call (a cast of the array itself, which folds); a cast
 * of a generic pointer inside the DMA helper would carry a null check. */
typedef __attribute__((address_space(3))) v4u lds_v4u;

/* Cache policy of the streaming accesses (the NT bit of the DMA loads and
 * the decode's output stores).  A tensor is read or written once, front to
 * back, and the NT hint keeps it from displacing other lines in L2 and the
 * memory-side cache: measured on a 0.54 GB encode + decode pair, the two
 * kernels run 15% faster back to back and the decode no longer leaves dirty
 * lines for the next kernel to write back.  The decode's stores into a
 * paged pool take the hint too (the encode after it ran 1.2% faster); the
 * encode's loads from a pool keep the default policy, which measured the
 * same there. */
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;

/*
 * Synchronization inside a one-wave workgroup.  LDS instructions of a wave
 * execute in order, so cross-lane exchange through LDS needs only that the
 * compiler keeps program order (a memory clobber) -- no workgroup barrier,
 * whose release fence would also wait for every outstanding global store.
 *
 * wait_vmem<N>: at most N of this wave's vector-memory operations still
 *   outstanding (they complete in issue order), then LDS may be read: the
 *   DMA data issued before the last N operations has landed.
 * lds_done: every LDS access issued so far has completed (before a DMA
 *   overwrites a buffer that was just read).
 */
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

/* s_waitcnt immediate for vmcnt(N) with the other counters left alone
 * (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8). */
constexpr int wait_vmem_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitVmem0 = wait_vmem_imm(0);

/* Raw buffer resource over `bytes` bytes from `base` (stride 0): a vector
 * store at a byte offset of `bytes` or more is dropped, a load there reads
 * zero.  0x00020000 in the last word is data format 32, which raw buffer
 * accesses need to be valid at all. */
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}

/* This lane's index as a value the compiler cannot see through: address
 * arithmetic derived from it stays inside the loop that uses it instead of
 * being hoisted out and held in registers (or spilled) across the loop. */
__device__ __forceinline__ int opaque_lane() {
  int v = threadIdx.x;
  asm volatile("" : "+v"(v));
  return v;
}

/*
 * Tile of `count` vectors of D 16-bit elements -> LDS by DMA
 * (global_load_lds_dwordx4, no register staging).  Instruction k copies the
 * k-th KiB of the tile; its lanes write consecutive 16-byte LDS slots, so the
 * row of vector v occupies slots [v*CH, v*CH + CH).  Lane l of instruction k
 * fetches chunk p = (l % CH) ^ (v % CH) of vector v = k*VPI + l / CH, so
 * chunk p of row v lands in column p ^ (v % CH): the later per-lane row
 * reads then hit 16 different bank groups in every 16-lane phase.
 *
 * The lane's byte offset inside instruction k's KiB is
 * (l / CH) * 16 * CH + 16 * ((l % CH) ^ (v % CH)); with v % CH =
 * ((k * VPI) % CH) | (l / CH) (no carries: VPI is a power of two and
 * l / CH < VPI) this is L0 ^ (16 * ((k * VPI) % CH)), L0 the k = 0 offset.
 */
template <int D, int AUX>
__device__ __forceinline__ void dma_rows_policy(const uint8_t* src, int count, lds_v4u* lds) {
  constexpr int CH = D / 8, VPI = 64 / CH;
  const int lane = opaque_lane();
  const int vin = lane / CH, col = lane % CH;
  const uint32_t l0 = uint32_t(vin * CH * 16 + 16 * (col ^ vin));
  if (count == kTileVectors) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const uint32_t off = l0 ^ uint32_t(16 * ((k * VPI) % CH));
      const uint8_t* bk = src + k * 1024;  // wave-uniform
      __builtin_amdgcn_global_load_lds(bk + off, (lds_void*)(lds + k * 64), 16, 0, AUX);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const uint32_t off = l0 ^ uint32_t(16 * ((k * VPI) % CH));
      if (k * VPI + vin < count)
        __builtin_amdgcn_global_load_lds(src + k * 1024 + off, (lds_void*)(lds + k * 64), 16, 0, AUX);
    }
  }
}

template <int D, bool STREAM>
__device__ __forceinline__ void dma_rows(const uint8_t* src, int count, lds_v4u* lds) {
  dma_rows_policy<D, STREAM ? kCacheStream : kCacheDefault>(src, count, lds);
}

/* Own LDS row -> its D storage elements, packed (chunk p = elements 8p ..
 * 8p+7), with the sign flip applied as an exact xor of each sign bit.
 * Chunk p of this lane's row v is at slot v * CH + (p ^ (v % CH)) = base ^ p. */
template <int D>
__device__ __forceinline__ void read_row_signed(const v4u* lds, const uint32_t* signs, v4u (&xc)[D / 8]) {
  constexpr int CH = D / 8;
  const int v = opaque_lane();
  const int base = v * CH + (v % CH);
  const v4u* sg = reinterpret_cast<const v4u*>(signs);
#pragma unroll
  for (int p = 0; p < CH; ++p) xc[p] = lds[base ^ p] ^ sg[p];
}

/* ---- transform on the matrix cores ------------------------------------------
 *
 * u = H (s * x) for the 64 vectors of a tile as a matrix product on the
 * MFMA units: U = H X, H the D x D Sylvester matrix, X the D x 64 matrix
 * whose column j is vector j (lane j's row).  Every product is exact: the
 * inputs are the stored bf16 / fp16 values and H holds +-1, both exact in
 * the MFMA operand type, and the sums are kept in fp32.
 *
 * v_mfma_f32_32x32x16_{bf16,f16} computes a 32 x 32 block of U from a 32 x
 * 16 block of H (operand A) and a 16 x 32 block of X (operand B): lane l
 * supplies A[l % 32][8*(l/32) + e] and B[8*(l/32) + e][l % 32], e < 8, and
 * receives D[8*(r/4) + 4*(l/32) + r%4][l % 32] in accumulator r < 16.
 *
 * Operand B: K-block b of X (rows 16b .. 16b+15) is the lane's chunks 2b
 * and 2b+1.  Lanes 0-31 must supply the first 8 of those rows for vectors
 * 0-31 and lanes 32-63 the last 8 of the same vectors; one
 * v_permlane32_swap per register exchanges chunk 2b+1 of vectors 0-31
 * with chunk 2b of vectors 32-63, after which chunk 2b is operand B of the
 * vectors 0-31 and chunk 2b+1 that of the vectors 32-63.
 *
 * Operand A: with output block a (rows 32a + i) and K-block b (columns
 * 16b + k, k = 8*(l/32) + e), the sign of H[32a + i][16b + k] is the parity
 * of popcount(i & k & 15) + (bit 4 of i)(bit 0 of b) + popcount(a & (b >> 1)).
 * The first term depends only on the lane and e, the second only on the
 * lane and whether b is odd, the third is one sign per (a, b): four
 * operand registers cover every block -- even / odd b, each also negated.
 *
 * Results: the accumulators of output block a for vectors 0-31 and for
 * vectors 32-63 are exchanged the same way (one swap per register), after
 * which lane j holds element 32a + 8*(r/4) + r%4 of its own vector in the
 * first and element 32a + 8*(r/4) + 4 + r%4 in the second.
 *
 * The compiler shares the partial sums that several output blocks have in
 * common (the first K-blocks of a and a+1 carry the same signs), so the
 * 2 * (D/32) * (D/16) products of a D = 128 tile issue as 44 instructions.
 *
 * With G < D the same code computes (I_{D/G} (x) H_G) x, the transform
 * within each group of G elements: H_D = H_{D/G} (x) H_G in Sylvester
 * order, and the block-diagonal part keeps only the blocks whose rows and
 * columns lie in one group (32a / G == 16b / G), with the third sign term
 * restricted to the in-group bits of a and b >> 1.  At G = 32 that is 16
 * products per D = 128 tile.
 */
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct HadamardA {
  v4u w[4];  // [even b, odd b, even b negated, odd b negated], 8 values each
};

template <int DT>
__device__ __forceinline__ void hadamard_operands(HadamardA& A) {
  const int l = threadIdx.x;
  const int i = l & 15, h = (l >> 5) & 1, i4 = (l >> 4) & 1;
  const uint32_t one = DT == KVC_BF16 ? 0x3F80u : 0x3C00u;  // +1.0 in the storage type
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t w = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int e = 2 * m + half;
      const uint32_t odd = __builtin_popcount(i & (8 * h + e)) & 1;
      w |= (one | (odd << 15)) << (16 * half);
    }
    A.w[0][m] = w;
    A.w[1][m] = w ^ (i4 ? 0x80008000u : 0u);
    A.w[2][m] = A.w[0][m] ^ 0x80008000u;
    A.w[3][m] = A.w[1][m] ^ 0x80008000u;
  }
}

template <int DT>
__device__ __forceinline__ f32x16_t mfma_32x32x16(v4u a, v4u b, f32x16_t c) {
  if constexpr (DT == KVC_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

/* Packed row chunks of every lane -> u = (I_{D/G} (x) H_G) x of the lane's
 * own vector (u = H x at G = D), D fp32 values in element order.  `xc` is
 * consumed. */
template <int D, int DT, int G = D>
__device__ __forceinline__ void hadamard_mfma(v4u (&xc)[D / 8], const HadamardA& A, float (&u)[D]) {
  constexpr int KB = D / 16, OB = D / 32;
#pragma unroll
  for (int b = 0; b < KB; ++b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const auto r = __builtin_amdgcn_permlane32_swap(xc[2 * b][m], xc[2 * b + 1][m], false, false);
      xc[2 * b][m] = r[0];
      xc[2 * b + 1][m] = r[1];
    }
  }
  f32x16_t acc[OB][2];
#pragma unroll
  for (int a = 0; a < OB; ++a) {
    acc[a][0] = f32x16_t{};
    acc[a][1] = f32x16_t{};
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      if ((32 * a) / G != (16 * b) / G) continue;  // block outside every group
      const int sel = ((__builtin_popcount(a & (b >> 1) & (G / 32 - 1)) & 1) << 1) | (b & 1);
      acc[a][0] = mfma_32x32x16<DT>(A.w[sel], xc[2 * b], acc[a][0]);
      acc[a][1] = mfma_32x32x16<DT>(A.w[sel], xc[2 * b + 1], acc[a][1]);
    }
  }
#pragma unroll
  for (int a = 0; a < OB; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto s =
          __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[a][0][r]), __float_as_uint(acc[a][1][r]), false, false);
      u[32 * a + 8 * (r / 4) + (r % 4)] = __uint_as_float(s[0]);
      u[32 * a + 8 * (r / 4) + 4 + (r % 4)] = __uint_as_float(s[1]);
    }
  }
}

/* Butterfly stages h = H0, 2 H0, ... < H1 of the in-place Sylvester
 * transform: stages below G stay inside groups of G elements, the others
 * combine groups. */
template <int D, int H0, int H1>
__device__ __forceinline__ void butterfly_stages(float (&y)[D]) {
#pragma unroll
  for (int h = H0; h < H1; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float p0 = y[j], p1 = y[j + h];
        y[j] = p0 + p1;
        y[j + h] = p0 - p1;
      }
    }
  }
}

/* Sign words into LDS (word m: bit 15 / 31 set when element 2m / 2m + 1 flips). */
__device__ __forceinline__ void load_signs(const LaunchArgs& a, uint32_t* signs) {
  signs[threadIdx.x] = a.sign_words[threadIdx.x];
}

/* ---- encode ---------------------------------------------------------------- */

/*
 * Meta of one group of the normalized values y = u / sqrt(D), from the
 * min / max of its unnormalized values u.  Every binary32 operation rounds
 * on its own (no contraction into fused multiply-adds):
 *   zero  = RD16(mn * rs)
 *   scale = RU16(((mx * rs) - zero) / (2^b - 1))
 * Returns scale | zero << 16 (the blob's little-endian meta entry).
 */
template <int D, int B>
__device__ __forceinline__ uint32_t group_meta_word(float mn, float mx) {
#pragma clang fp contract(off)
  constexpr float RS = Norm<D>::inv_sqrt;
  constexpr float QMAX = float((1 << B) - 1);
  const uint32_t zb = rd16(mn * RS);
  const float zf = f16_value(zb);
  const float mxn = mx * RS;
  const uint32_t sb = ru16((mxn - zf) / QMAX);
  return sb | (zb << 16);
}

/* Code of u is round(fma(u, A, Bz)): inv = 1 / scale (0 for scale 0),
 * A = inv * rs, Bz = -zero * inv, each rounded on its own. */
template <int D>
__device__ __forceinline__ void code_affine(uint32_t meta, float& A, float& Bz) {
#pragma clang fp contract(off)
  constexpr float RS = Norm<D>::inv_sqrt;
  const float sf = f16_value(meta & 0xffffu);
  const float zf = f16_value(meta >> 16);
  const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
  A = inv * RS;
  Bz = -zf * inv;
}

template <int B>
__device__ __forceinline__ void quantize_group(const float* y, float A, float Bz, bool clamp, uint32_t* words) {
  constexpr int VPW = 32 / B;
  constexpr float QMAX = float((1 << B) - 1);
  (void)VPW;
  float tq[VPW];
#pragma unroll
  for (int k = 0; k < VPW; ++k) {
    const float t = fmaf(y[k], A, Bz);
    tq[k] = clamp ? fminf(t, QMAX) : t;
  }
  *words = pack_word<B>(tq);
}

/* The encode's transform: kEncodeMatrix runs u = H x on the matrix cores
 * (hadamard_mfma), kEncodeButterfly as the in-register butterfly of each
 * lane's own vector in fp32.  Both are exact products with +-1 and fp32
 * sums, in different orders, so their u differ by rounding only. */
constexpr int kEncodeMatrix = 0, kEncodeButterfly = 1;

/* ---- exact 8-bit decisions near a tie ----------------------------------------
 *
 * At 8 bits t reaches 255, where one binary32 ulp is 2^-16, so the binary32
 * decision above (u from fp32 sums, t = fma(u, A, Bz)) can fall on the wrong
 * side of k + 1/2 when the exact t lies within a few 1e-5 of it.  Such
 * elements are found with a bound on the decision's error and decided again
 * exactly: y_i summed in fp64 from the lane's own signed row (the stored
 * values are exact in fp64, as is their sum unless their exponents span more
 * than about 35 binades), t = (y - zero) / scale in fp64, rounded half to
 * even.  Every other element provably has the code of its exact t.
 *
 * Bound of |t32 - t| against the exact t of the same meta (w = 2^-24):
 *   w (2 D rs S / scale + 4 |zero| / scale + 3 (|t32| + 1)),
 * S = sum_j |x_j| of the vector.  Each element of u comes out of D - 1 fp32
 * additions whose partial sums are bounded by S; taking each addition's
 * relative error below 2w, whatever order or rounding the matrix cores use,
 * gives |u - u_exact| <= 2 D w S.  A = fl(fl(1 / scale) rs) and Bz =
 * fl(-zero fl(1 / scale)) carry 2w each, the fused multiply-add w; the rest
 * are second-order terms, covered with the binary32 evaluation of the bound
 * itself by a 5% slack. */

/* y_i = (H (s * x))_i / sqrt(D) in fp64 from the signed row xs (chunk p =
 * elements 8p .. 8p+7, element 2m of a chunk in the low half of word m);
 * i may differ per lane.  Row i of H has the sign (-1)^popcount(i & j). */
template <int D, int DT>
__device__ __forceinline__ double exact_rotated(const v4u (&xs)[D / 8], int i) {
  uint32_t base = 0;  // bit j: parity of popcount(i & j), j < 32
  if (i & 1) base ^= 0xAAAAAAAAu;
  if (i & 2) base ^= 0xCCCCCCCCu;
  if (i & 4) base ^= 0xF0F0F0F0u;
  if (i & 8) base ^= 0xFF00FF00u;
  if (i & 16) base ^= 0xFFFF0000u;
  double sum = 0.0;
#pragma unroll
  for (int p = 0; p < D / 8; ++p) {
    const uint32_t w = (__builtin_popcount((i >> 5) & (p >> 2)) & 1) ? ~base : base;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int sh = (8 * p + 2 * m) & 31;
      const uint32_t flip = (((w >> sh) & 1u) << 15) | (((w >> (sh + 1)) & 1u) << 31);
      float lo, hi;
      unpack_pair<DT>(xs[p][m] ^ flip, lo, hi);
      sum += static_cast<double>(lo);
      sum += static_cast<double>(hi);
    }
  }
  return sum * Norm<D>::inv_sqrt_d;
}

/* The 8-bit code of y against a meta word, in fp64: round half to even of
 * (y - zero) / scale, within [0, 255]; 0 for a constant group. */
__device__ __forceinline__ uint32_t exact_code8(double y, uint32_t meta) {
  const double sc = f16_value(meta & 0xffffu), ze = f16_value(meta >> 16);
  if (!(sc > 0.0)) return 0u;
  const double t = __builtin_rint((y - ze) / sc);
  return static_cast<uint32_t>(__builtin_fmin(__builtin_fmax(t, 0.0), 255.0));
}

/* Whether a binary32 t lies within `bound` of a tie k + 1/2 (t - floor(t) is
 * exact for t >= 0, and the distance is taken on |t| otherwise). */
__device__ __forceinline__ bool near_tie(float t, float bound) {
  const float a = fabsf(t);
  return fabsf((a - floorf(a)) - 0.5f) <= bound;
}

/* Bound of |t32 - t| for the elements of one group, without its |t32| term:
 * w (c_u rs S / scale + 4 |zero| / scale + 3) with 5% slack; c_u rs S bounds
 * the fp32 error of u in units of y (c_u = 2 D with S = sum |x_j|). */
__device__ __forceinline__ float tie_bound_base(float err_u_y, uint32_t meta) {
  constexpr float W = 5.9604644775390625e-8f;  // 2^-24
  const float sc = f16_value(meta & 0xffffu), ze = f16_value(meta >> 16);
  return 1.05f * W * ((err_u_y + 4.0f * fabsf(ze)) / sc + 3.0f);
}
constexpr float kTieBoundT = 1.05f * 3.0f * 5.9604644775390625e-8f;  // per |t32|

/* Flags (bit j % 32 of word j / 32) of the elements whose binary32 t lies
 * within the bound of a tie; err_u_y bounds the error of u in units of y
 * divided by w (c_u rs S). */
template <int D, int G>
__device__ __forceinline__ void ties8_flags(const float (&u)[D], float err_u_y, const uint32_t* meta,
                                            uint32_t (&flags)[D / 32]) {
#pragma clang fp contract(off)
  constexpr int NG = D / G, NW = D / 32;
#pragma unroll
  for (int w = 0; w < NW; ++w) flags[w] = 0u;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (!(f16_value(meta[g] & 0xffffu) > 0.0f)) continue;  // constant group: every code 0, exactly
    float A, Bz;
    code_affine<D>(meta[g], A, Bz);
    const float base = tie_bound_base(err_u_y, meta[g]);
#pragma unroll
    for (int j = g * G; j < (g + 1) * G; ++j) {
      const float t = fmaf(u[j], A, Bz);
      if (near_tie(t, base + kTieBoundT * fabsf(t))) flags[j / 32] |= 1u << (j % 32);
    }
  }
}

/* Decide every flagged element again exactly from the signed row xs and
 * patch its code into words (code k at byte k % 4 of word k / 4).  The
 * wave repeats until no lane has a flag left. */
template <int D, int DT, int G>
__device__ __forceinline__ void ties8_resolve(const v4u (&xs)[D / 8], const uint32_t* meta, uint32_t (&flags)[D / 32],
                                              uint32_t* words) {
  constexpr int NG = D / G, NW = D / 32;
  for (;;) {
    uint32_t any = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= flags[w];
    if (__builtin_amdgcn_ballot_w64(any != 0u) == 0) break;
    if (any != 0u) {
      int wsel = 0;
      uint32_t fw = 0u;
#pragma unroll
      for (int w = NW - 1; w >= 0; --w) {
        if (flags[w] != 0u) {
          wsel = w;
          fw = flags[w];
        }
      }
      const int k = 32 * wsel + __builtin_ctz(fw);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (w == wsel) flags[w] = fw & (fw - 1u);
      uint32_t mg = meta[0];
#pragma unroll
      for (int g = 1; g < NG; ++g)
        if (k / G == g) mg = meta[g];
      const uint32_t q = exact_code8(exact_rotated<D, DT>(xs, k), mg);
      const int wk = k >> 2;
      const uint32_t sh = 8u * static_cast<uint32_t>(k & 3);
#pragma unroll
      for (int w = 0; w < D / 4; ++w)
        if (w == wk) words[w] = (words[w] & ~(0xffu << sh)) | (q << sh);
    }
  }
}

/* Re-decide exactly the 8-bit codes of this lane's vector whose binary32 t
 * lies within the bound of a tie, u from the matrix cores (2 D additions'
 * worth of error, each at most 2w, whatever their order and rounding).
 * u: the unnormalized rotated values; xs: the signed row they came from;
 * words: the packed codes, patched in place. */
template <int D, int DT, int G>
__device__ __forceinline__ void refine_ties8(const float (&u)[D], const v4u (&xs)[D / 8], const uint32_t* meta,
                                             uint32_t* words) {
  // one body on purpose: built from ties8_flags and ties8_resolve, this
  // kernel's register allocation spilled several times more and ran at
  // half the speed
#pragma clang fp contract(off)
  constexpr int NG = D / G, NW = D / 32;
  constexpr float RS = Norm<D>::inv_sqrt;
  float S = 0.0f;
#pragma unroll
  for (int p = 0; p < D / 8; ++p) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float lo, hi;
      unpack_pair<DT>(xs[p][m], lo, hi);
      S += fabsf(lo);
      S += fabsf(hi);
    }
  }
  uint32_t flags[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) flags[w] = 0u;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (!(f16_value(meta[g] & 0xffffu) > 0.0f)) continue;  // constant group: every code 0, exactly
    float A, Bz;
    code_affine<D>(meta[g], A, Bz);
    const float base = tie_bound_base(2.0f * D * RS * S, meta[g]);
#pragma unroll
    for (int j = g * G; j < (g + 1) * G; ++j) {
      const float t = fmaf(u[j], A, Bz);
      if (near_tie(t, base + kTieBoundT * fabsf(t))) flags[j / 32] |= 1u << (j % 32);
    }
  }
  for (;;) {
    uint32_t any = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= flags[w];
    if (__builtin_amdgcn_ballot_w64(any != 0u) == 0) break;
    if (any != 0u) {
      int wsel = 0;
      uint32_t fw = 0u;
#pragma unroll
      for (int w = NW - 1; w >= 0; --w) {
        if (flags[w] != 0u) {
          wsel = w;
          fw = flags[w];
        }
      }
      const int k = 32 * wsel + __builtin_ctz(fw);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (w == wsel) flags[w] = fw & (fw - 1u);
      uint32_t mg = meta[0];
#pragma unroll
      for (int g = 1; g < NG; ++g)
        if (k / G == g) mg = meta[g];
      const uint32_t q = exact_code8(exact_rotated<D, DT>(xs, k), mg);
      const int wk = k >> 2;
      const uint32_t sh = 8u * static_cast<uint32_t>(k & 3);
#pragma unroll
      for (int w = 0; w < D / 4; ++w)
        if (w == wk) words[w] = (words[w] & ~(0xffu << sh)) | (q << sh);
    }
  }
}

/* The same for u from the in-register butterfly: log2 D stages of IEEE
 * binary32 additions, round to nearest.  Element i's value at stage k is the
 * sum of one of the D / 2^k disjoint blocks of the signed row, so the
 * additions of stage k err by at most w times that block's sum of |x_j|
 * (times (1 + w)^k), and the stages together by log2(D) w S to first order
 * -- 2D / log2(D) times less than the matrix-core bound, and so that many
 * times fewer elements to decide again.  S is given (summed from the row
 * before the butterfly); the row itself is read back from `stash` (this
 * lane's LDS copy, chunk p at slot index base ^ p) only when some lane of
 * the wave has an element to decide. */
template <int D, int DT, int G>
__device__ __forceinline__ void refine_ties8_stash(const float (&u)[D], float S, const v4u* stash,
                                                   const uint32_t* meta, uint32_t* words) {
  constexpr float RS = Norm<D>::inv_sqrt;
  constexpr int LOG2D = D == 64 ? 6 : 7;
  static_assert(D == 64 || D == 128, "head_dim");
  uint32_t flags[D / 32];
  ties8_flags<D, G>(u, float(LOG2D) * RS * S, meta, flags);
  uint32_t any = 0u;
#pragma unroll
  for (int w = 0; w < D / 32; ++w) any |= flags[w];
  if (__builtin_amdgcn_ballot_w64(any != 0u) == 0) return;
  constexpr int CH = D / 8;
  const int v = static_cast<int>(threadIdx.x);
  const int base = v * CH + (v % CH);
  v4u xs[D / 8];
#pragma unroll
  for (int p = 0; p < CH; ++p) xs[p] = stash[base ^ p];
  ties8_resolve<D, DT, G>(xs, meta, flags, words);
}

/* Meta, codes and stores of one vector from its unnormalized rotated values
 * u; at 8 bits the codes near a tie are decided again exactly from the
 * signed row: xs in registers after the matrix cores, or the lane's LDS
 * copy in `stash` with S8 = sum |x_j| after the butterfly (all unused at 2
 * and 4 bits). */
template <int D, int DT, int B, int G, bool PAGED, int XF>
__device__ __forceinline__ void encode_vector(float (&y)[D], const Tile& t, const v4u (&xs)[D / 8], float S8,
                                              const v4u* stash) {
  constexpr int NG = D / G;
  constexpr float QMAX = float((1 << B) - 1);
  constexpr int WPG = G * B / 32;  // code words per group
  constexpr int VPW = 32 / B;      // values per code word
  uint32_t meta[NG];
  uint32_t words[D * B / 32];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float mn = y[g * G], mx = y[g * G];
#pragma unroll
    for (int j = 1; j < G; ++j) {
      mn = fminf(mn, y[g * G + j]);
      mx = fmaxf(mx, y[g * G + j]);
    }
    meta[g] = group_meta_word<D, B>(mn, mx);
    float A, Bz;
    code_affine<D>(meta[g], A, Bz);
    // t = fma(u, A, Bz) is monotone in u (A >= 0), so the group's largest
    // t is the one of its maximum: below 2^b - 1/2 no code can exceed
    // 2^b - 1 and the clamp min(t, 2^b - 1) cannot change any code.  Only a
    // degenerate group (huge offset, tiny range) takes the clamping path.
    const bool clamp = !(fmaf(mx, A, Bz) < QMAX + 0.5f);
    if (!clamp) {
#pragma unroll
      for (int w = 0; w < WPG; ++w) quantize_group<B>(&y[g * G + w * VPW], A, Bz, false, &words[g * WPG + w]);
    } else {
#pragma unroll
      for (int w = 0; w < WPG; ++w) quantize_group<B>(&y[g * G + w * VPW], A, Bz, true, &words[g * WPG + w]);
    }
    KVC_PHASE();
  }
  if constexpr (B == 8) {
    if constexpr (XF == kEncodeButterfly)
      refine_ties8_stash<D, DT, G>(y, S8, stash, meta, words);
    else
      refine_ties8<D, DT, G>(y, xs, meta, words);
  }
  if (static_cast<int>(threadIdx.x) < t.count) {
    constexpr int RB = D * B / 8;
    int stride;
    v4u* crow = code_row<RB, PAGED>(t, threadIdx.x, stride);
#pragma unroll
    for (int c = 0; c < RB / 16; ++c)
      crow[c * stride] = v4u{words[4 * c], words[4 * c + 1], words[4 * c + 2], words[4 * c + 3]};
    uint32_t* mrow = reinterpret_cast<uint32_t*>(t.meta) + threadIdx.x * NG;
    if constexpr (NG == 1) {
      mrow[0] = meta[0];
    } else if constexpr (NG == 2) {
      *reinterpret_cast<v2u*>(mrow) = v2u{meta[0], meta[1]};
    } else {
      *reinterpret_cast<v4u*>(mrow) = v4u{meta[0], meta[1], meta[2], meta[3]};
    }
  }
}


/*
 * Encode: per tile, the rows arrive in LDS by DMA; each lane reads its own
 * row into registers, the wave then starts the DMA of its next tile into the
 * same buffer and computes the current one while that load is in flight.
 */
template <int D, int DT, int B, int G, bool PAGED, int XF = kEncodeMatrix>
KVC_KERNEL void encode_kernel(const LaunchArgs a) {
  constexpr int CH = D / 8;
  // the 8-bit butterfly encode keeps each lane's signed row in LDS for the
  // exact decisions instead of in registers
  constexpr bool STASH = B == 8 && XF == kEncodeButterfly;
  __shared__ v4u lds[kTileVectors * CH];
  __shared__ v4u stash[STASH ? kTileVectors * CH : 1];
  __shared__ uint32_t signs[64];
  const uint8_t* tensor = static_cast<const uint8_t*>(a.src);
  uint8_t* blob = static_cast<uint8_t*>(a.dst);
  load_signs(a, signs);
  Cursor c;
  cursor_init<PAGED, false>(a, c);
  Tile cur;
  if (!next_tile<D, true, PAGED, false>(a, c, tensor, blob, cur, cur, true)) return;
  dma_rows<D, !PAGED>(cur.src, cur.count, (lds_v4u*)lds);
  wait_vmem<0>();
  lds_order();
  HadamardA had;
  if constexpr (XF == kEncodeMatrix) hadamard_operands<DT>(had);
  for (;;) {
    v4u xc[D / 8];
    read_row_signed<D>(lds, signs, xc);
    if constexpr (STASH) {
      const int v = static_cast<int>(threadIdx.x);
      const int base = v * CH + (v % CH);
#pragma unroll
      for (int p = 0; p < CH; ++p) stash[base ^ p] = xc[p];
    }
    KVC_PHASE();
    lds_done();  // every lane's row is in registers: the buffer is free
    Tile nxt;
    const bool more = next_tile<D, true, PAGED, false>(a, c, tensor, blob, cur, nxt, false);
    if (more) dma_rows<D, !PAGED>(nxt.src, nxt.count, (lds_v4u*)lds);
    KVC_PHASE();
    v4u xs[D / 8];  // the signed row, kept for the exact 8-bit decisions
    if constexpr (B == 8 && !STASH) {
#pragma unroll
      for (int p = 0; p < D / 8; ++p) xs[p] = xc[p];
    }
    float y[D];
    float S8 = 0.0f;
    if constexpr (XF == kEncodeButterfly) {
#pragma unroll
      for (int p = 0; p < D / 8; ++p) {
#pragma unroll
        for (int m = 0; m < 4; ++m) unpack_pair<DT>(xc[p][m], y[8 * p + 2 * m], y[8 * p + 2 * m + 1]);
      }
      if constexpr (STASH) {
#pragma unroll
        for (int j = 0; j < D; ++j) S8 += fabsf(y[j]);
      }
      butterfly_stages<D, 1, D>(y);
    } else {
      hadamard_mfma<D, DT>(xc, had, y);
    }
    KVC_PHASE();
    encode_vector<D, DT, B, G, PAGED, XF>(y, cur, xs, S8, stash);
    if (!more) break;
    // outstanding: the next tile's DMA, then this tile's code and meta
    // stores (RB / 16 + 1 instructions, issued by the lanes < count)
    wait_vmem<D * B / 128 + 1>();
    lds_order();
    cur = nxt;
  }
}

/* ---- decode ---------------------------------------------------------------- */

/* A tile's codes and meta for one lane (its own row), held in registers:
 * RB / 16 16-byte chunks and D / G meta words. */
template <int D, int B, int G>
struct CodeRegs {
  v4u codes[D * B / 128];
  uint32_t meta[D / G];
};

/* Prefetch of this lane's code row and meta entries (lanes past the tile's
 * count load nothing).  Plain vector loads: their wait counts are tracked per
 * register, so the compiler waits for them only where they are used. */
template <int D, int B, int G, bool PAGED>
__device__ __forceinline__ void load_codes(const Tile& t, CodeRegs<D, B, G>& r) {
  constexpr int RB = D * B / 8, NG = D / G;
  const int lane = threadIdx.x;
  if (lane < t.count) {
    int stride;
    const v4u* crow = code_row<RB, PAGED>(t, lane, stride);
#pragma unroll
    for (int p = 0; p < RB / 16; ++p) r.codes[p] = __builtin_nontemporal_load(crow + p * stride);
    const uint32_t* mrow = reinterpret_cast<const uint32_t*>(t.meta) + lane * NG;
    if constexpr (NG == 1) {
      r.meta[0] = __builtin_nontemporal_load(mrow);
    } else if constexpr (NG == 2) {
      const v2u m = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(mrow));
      r.meta[0] = m.x;
      r.meta[1] = m.y;
    } else {
      const v4u m = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(mrow));
#pragma unroll
      for (int g = 0; g < 4; ++g) r.meta[g] = m[g];
    }
  } else {
#pragma unroll
    for (int p = 0; p < RB / 16; ++p) r.codes[p] = v4u{0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < NG; ++g) r.meta[g] = 0;
  }
}

/* Chunk p (elements 8p .. 8p+7) of a lane's codes as fp16 pairs 1024 + q,
 * element 2m in the low half: exact for every code (q < 1024, and fp16 has
 * unit spacing on [1024, 2048)), at one byte permute and one or per pair.
 * `w` holds the lane's D * B / 32 code words. */
template <int B, int NW>
__device__ __forceinline__ v4u code_chunk_f16(const uint32_t (&w)[NW], int p) {
  constexpr uint32_t kBias = 0x64006400u;  // fp16 1024.0 in both halves
  v4u r;
  if constexpr (B == 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = w[2 * p + h];
      r[2 * h] = __builtin_amdgcn_perm(x, x, 0x0C010C00u) | kBias;
      r[2 * h + 1] = __builtin_amdgcn_perm(x, x, 0x0C030C02u) | kBias;
    }
  } else if constexpr (B == 4) {
    // codes 2m and 2m+1 are the low and high nibble of byte m
    const uint32_t x = w[p];
    const uint32_t e = x & 0x0F0F0F0Fu, o = (x >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int m = 0; m < 4; ++m) r[m] = __builtin_amdgcn_perm(o, e, 0x0C000C00u | m | ((4 + m) << 16)) | kBias;
  } else {
    // the chunk is half a word; codes 2k and 2k+1 are the two halves of nibble k
    const uint32_t x = w[p / 2];
    const int h = p & 1;
    const uint32_t e = x & 0x33333333u, o = (x >> 2) & 0x33333333u;
    const uint32_t ee = e & 0x0F0F0F0Fu, eo = (e >> 4) & 0x0F0F0F0Fu;  // even / odd nibbles to bytes
    const uint32_t oe = o & 0x0F0F0F0Fu, oo = (o >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t sel = 0x0C000C00u | uint32_t(2 * h + m / 2) | (uint32_t(4 + 2 * h + m / 2) << 16);
      r[m] = ((m & 1) ? __builtin_amdgcn_perm(oo, eo, sel) : __builtin_amdgcn_perm(oe, ee, sel)) | kBias;
    }
  }
  return r;
}

/*
 * Decode.  With q the codes of a vector, group g holding elements
 * [gG, gG + G), and H_D = H_{D/G} (x) H_G in Sylvester order:
 *   H_D yhat = (H_{D/G} (x) I_G) (I_{D/G} (x) H_G) yhat,
 *   H_G (zero_g 1 + scale_g q_g) = scale_g (H_G q_g) + zero_g G e_0.
 * So each lane first transforms its integer codes within each group, which
 * is exact (integers below 2^24 in fp32), then scales every element and adds
 * the zero term at each group's first element (one rounding each), runs the
 * log2(D/G) butterfly stages across groups in fp32, and packs to the storage
 * type with the sign flip: x = s * (H_D yhat) / sqrt(D), 1/sqrt(D) folded
 * into scale and zero.
 *
 * The in-group transform runs either on the matrix cores (the codes enter as
 * fp16 1024 + q; the bias adds exactly 1024 G to each group's first element,
 * which is subtracted exactly) or as the in-register butterfly on the codes
 * as fp32.  Both give the same integers, so every kind of decode agrees to
 * the bit; which one runs is part of the launch shape (MODE, below).
 *
 * Each lane's row goes to LDS one 128-byte line (8 chunks) at a time; the
 * wave then stores those lines with coalesced 16-byte stores, every store
 * instruction covering 8 whole lines (a pass that wrote half lines, as half
 * rows of a D = 64 tile are, left each line to be finished by a later
 * instruction and ran 1.4x slower).  The next tile's codes are loaded into
 * registers while the current one is computed.
 *
 * The stores go through a buffer resource that spans the tile's `count`
 * rows, so the stores of rows past the count are dropped by the hardware
 * instead of being skipped by a branch around each store (those branches,
 * with their exec-mask saves and restores, cost 3% at 16k-32k tokens).
 *
 * MODE, with the number of waves per SIMD it runs at (kvc_launch.hip):
 *   kDecodeWaitTop (two waves): matrix cores; a tile starts once the last
 *     tile's stores have completed, while the other wave computes.
 *   kDecodeWaitStores (one wave): matrix cores; the tile's compute overlaps
 *     the last tile's stores, which must complete before this tile's are
 *     issued.  At most one tile of stores per wave is then in flight: with
 *     two (the compiler's own waits allow that) the wider window of writes
 *     ran 12-13% slower.
 *   kDecodeLarge (one wave; large blobs at head_dim 64, and 4-bit codes in
 *     one group per vector past 512 MiB at head_dim 128): the butterfly,
 *     stores overlapped with no extra wait; its arithmetic spaces the stores
 *     by itself, and it measured 1-4% faster there than the matrix cores.
 *   kDecodeButterfly (contiguous, on request only): the butterfly with the
 *     waits of kDecodeWaitStores, so that the two in-group transforms can be
 *     timed against each other with everything else equal.
 */
constexpr int kDecodeWaitTop = 0, kDecodeWaitStores = 1, kDecodeLarge = 2, kDecodeButterfly = 3;

template <int D, int DT, int B, int G, bool PAGED, int MODE>
KVC_KERNEL void decode_kernel(const LaunchArgs a) {
  constexpr bool BFLY = MODE == kDecodeLarge || MODE == kDecodeButterfly;  // in-group transform: butterfly
  constexpr bool WAIT_STORES = MODE == kDecodeWaitStores || MODE == kDecodeButterfly;
  constexpr int CH = D / 8, NG = D / G, NW = D * B / 32, VPW = 32 / B;
  constexpr float RS = Norm<D>::inv_sqrt;
  constexpr int HALF = 8;                         // chunks per row staged at a time: one line
  constexpr int NPASS = CH / HALF;
  __shared__ v4u lds_out[kTileVectors * HALF];    // one line of every row of the tile
  __shared__ uint32_t signs[64];
  uint8_t* tensor = static_cast<uint8_t*>(a.dst);
  uint8_t* blob = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.src));
  const int lane = threadIdx.x;
  load_signs(a, signs);
  HadamardA had;
  if constexpr (!BFLY) hadamard_operands<KVC_FP16>(had);
  Cursor c;
  cursor_init<PAGED, true>(a, c);
  Tile cur;
  if (!next_tile<D, false, PAGED, true>(a, c, tensor, blob, cur, cur, true)) return;
  CodeRegs<D, B, G> cr;
  load_codes<D, B, G, PAGED>(cur, cr);
  // nothing outstanding on entry, so inside the loop the compiler's own wait
  // for the codes counts the loop's loads and stores only
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  for (;;) {
    if constexpr (MODE == kDecodeWaitTop) __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // the last tile's stores too
    float sc[NG], ze[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      sc[g] = f16_value(cr.meta[g] & 0xffffu) * RS;
      ze[g] = f16_value(cr.meta[g] >> 16) * RS;
    }
    float y[D];
    v4u xq[BFLY ? 1 : CH];
    if constexpr (BFLY) {
#pragma unroll
      for (int wi = 0; wi < NW; ++wi) unpack_word<B>(cr.codes[wi / 4][wi % 4], y + wi * VPW);
    } else {
      uint32_t wds[NW];
#pragma unroll
      for (int wi = 0; wi < NW; ++wi) wds[wi] = cr.codes[wi / 4][wi % 4];
#pragma unroll
      for (int p = 0; p < CH; ++p) xq[p] = code_chunk_f16<B, NW>(wds, p);
    }
    KVC_PHASE();
    Tile nxt;
    const bool more = next_tile<D, false, PAGED, true>(a, c, tensor, blob, cur, nxt, false);
    if (more) load_codes<D, B, G, PAGED>(nxt, cr);
    KVC_PHASE();
    if constexpr (BFLY) {
      butterfly_stages<D, 1, G>(y);
    } else {
      hadamard_mfma<D, KVC_FP16, G>(xq, had, y);
#pragma unroll
      for (int g = 0; g < NG; ++g) y[g * G] -= 1024.0f * G;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      y[g * G] = fmaf(y[g * G], sc[g], ze[g] * G);
#pragma unroll
      for (int j = 1; j < G; ++j) y[g * G + j] *= sc[g];
    }
    butterfly_stages<D, G, D>(y);
    KVC_PHASE();
    if constexpr (WAIT_STORES) {
      // outstanding: the last tile's stores, then the next tile's code and
      // meta loads (NL instructions, none after the last tile)
      constexpr int NL = D * B / 128 + 1;
      static_assert(NL < 64, "vmcnt range");
      if (more)
        __builtin_amdgcn_s_waitcnt(wait_vmem_imm(NL));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    }
    const v4u* sg = reinterpret_cast<const v4u*>(signs);
    const __amdgpu_buffer_rsrc_t out = tile_rsrc(cur.src, cur.count * CH * 16);
#pragma unroll
    for (int h = 0; h < NPASS; ++h) {
      // chunks [h*HALF, h*HALF + HALF) of every row through LDS; chunk q of
      // line h of row v sits in column q ^ (v % HALF)
      lds_order();
#pragma unroll
      for (int q = 0; q < HALF; ++q) {
        const int p = h * HALF + q;
        const v4u s = sg[p];
        v4u w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_pair<DT>(y[8 * p + 2 * i], y[8 * p + 2 * i + 1]) ^ s[i];
        lds_out[(lane * HALF) + (q ^ (lane % HALF))] = w;
        KVC_PHASE();
      }
      lds_order();
#pragma unroll
      for (int k = 0; k < HALF; ++k) {
        const int slot = k * 64 + lane;
        const int v = slot / HALF;
        const int q = (slot % HALF) ^ (v % HALF);
        __builtin_amdgcn_raw_buffer_store_b128(lds_out[slot], out, uint32_t((v * CH + h * HALF + q) * 16), 0,
                                               kCacheStream);
      }
    }
    if (!more) break;
    cur = nxt;
  }
}

/* ---- rotate ------------------------------------------------------------------ */

/*
 * The transform of the encode alone: per tile the same DMA, row read and
 * MFMA transform, then the D fp32 values of every vector to `out`
 * ([vectors, D], the tensor's vector order): u = H (s * x) when RAW, else
 * the rotated values y = u / sqrt(D).  The tile's rows go out through LDS
 * one 128-byte line (32 values) of every row at a time (in the tile buffer,
 * free once the rows are in registers), as coalesced 16-byte stores that
 * each cover 8 whole lines.
 */
template <int D, int DT, bool RAW>
__device__ __forceinline__ void rotate_tiles(const LaunchArgs& a, float* out) {
  constexpr int CH = D / 8;
  constexpr int QC = 8;       // 16-byte chunks of fp32 per line
  constexpr int NPASS = D / 32;
  constexpr float RS = Norm<D>::inv_sqrt;
  __shared__ v4u lds[kTileVectors * CH];
  __shared__ uint32_t signs[64];
  const uint8_t* tensor = static_cast<const uint8_t*>(a.src);
  const int lane = threadIdx.x;
  load_signs(a, signs);
  HadamardA had;
  hadamard_operands<DT>(had);
  Cursor c;
  cursor_init<false, false>(a, c);
  Tile t;
  for (bool ok = next_tile<D, false, false, false>(a, c, tensor, nullptr, t, t, true); ok;
       ok = next_tile<D, false, false, false>(a, c, tensor, nullptr, t, t, false)) {
    lds_done();
    dma_rows<D, false>(t.src, t.count, (lds_v4u*)lds);
    wait_vmem<0>();
    lds_order();
    v4u xc[CH];
    read_row_signed<D>(lds, signs, xc);
    float u[D];
    hadamard_mfma<D, DT>(xc, had, u);
    const int64_t vec0 = (t.src - tensor) / (2 * D);
    v4u* dst = reinterpret_cast<v4u*>(out + vec0 * D);
#pragma unroll
    for (int h = 0; h < NPASS; ++h) {
      // chunk q of this lane's line h goes to LDS column q ^ (lane % QC)
      lds_done();
      lds_order();
#pragma unroll
      for (int q = 0; q < QC; ++q) {
        const int e = h * 32 + 4 * q;
        v4u w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = __float_as_uint(RAW ? u[e + k] : u[e + k] * RS);
        lds[lane * QC + (q ^ (lane % QC))] = w;
      }
      lds_order();
#pragma unroll
      for (int k = 0; k < QC; ++k) {
        const int slot = k * 64 + lane;
        const int v = slot / QC;
        const int q = (slot % QC) ^ (v % QC);
        if (v < t.count) dst[v * (D / 4) + h * QC + q] = lds[slot];
      }
    }
  }
}

template <int D, int DT>
KVC_KERNEL void rotate_kernel(const LaunchArgs a) {
  rotate_tiles<D, DT, false>(a, static_cast<float*>(a.dst));
}

}  // namespace dev

}  // namespace kvc

#endif
