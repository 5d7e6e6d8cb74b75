/*
 * kvc_plan.h -- launch plans shared by the host half (kvc_host.cpp, plain
 * C++) and the device half (kvc_device.h, kvc_cursor.h and the .hip files).
 * No HIP types: the host half builds with g++ and is unit-tested without a
 * GPU.
 *
 * A plan describes one kernel launch over "items".  Each item is a tile of
 * at most 64 consecutive head_dim vectors of one (layer, K/V) slab; every
 * vector of a tile is contiguous in the KV tensor (or in one pool block)
 * and its code rows and meta entries are contiguous in the blob.
 */
#ifndef KVC_PLAN_H
#define KVC_PLAN_H

#include <stddef.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kTileVectors = 64;   // one vector per lane of a wave64
constexpr int kReqChunk = 64;      // requests of one paged launch: one per lane of a wave64
constexpr int kPagedRun = 2;       // slabs a paged decode wave walks per item before it resolves the next

/* Arguments of one encode / decode / rotate launch (passed by value). */
struct LaunchArgs {
  const void* src;        // encode: KV tensor or pool; decode: blob
  void* dst;              // encode: blob; decode: KV tensor or pool; rotate: fp32 y
  uint64_t blob_bytes;    // size of the blob buffer (bounds checks)

  // slab s = i * slab_step + slab_first, i in [0, n_slabs); s = l * 2 + kv
  int64_t n_slabs;
  int64_t slab_step;
  int64_t slab_first;
  int64_t layers;         // L of the whole tensor
  int32_t row_k;          // code bytes per K vector (D * bits_k / 8)
  int32_t row_v;          // code bytes per V vector
  int32_t groups;         // D / group
  int32_t paged;          // 0: contiguous, 1: paged

  // contiguous layout
  int64_t rows;           // T * H vectors per slab
  int64_t tiles_per_slab; // ceil(rows / 64)
  uint64_t code_slab_k;   // bytes of one K code slab (rows * row_k rounded up to 256)
  uint64_t code_slab_v;   // bytes of one V code slab
  uint64_t meta_slab;     // bytes of one meta slab (rows * groups * 4 rounded up to 256)
  uint64_t meta_offset;   // byte offset of the meta section in the blob
  uint64_t blob_total;    // bytes of the blob
  // slab i of this launch (s = i * slab_step + slab_first) starts at byte
  // src_first + i * src_stride of the tensor, its codes at codes_first +
  // i * codes_stride and its meta at meta_first + i * meta_stride of the blob
  // (paged: src_stride is the pool's byte stride between the launch's
  // consecutive slabs, slab_step slabs of num_blocks blocks)
  int64_t src_first, src_stride;
  int64_t codes_first, codes_stride;
  int64_t meta_first, meta_stride;
  int32_t row;            // code bytes per vector in this launch (row_k or row_v)
  int32_t code_tail;      // zero bytes after a code slab's rows * row bytes (< 256)
  int32_t meta_tail;      // zero bytes after a meta slab's rows * groups * 4 bytes (< 256)
  int32_t pad1;

  // paged layout: an item is (slab, request, block, subtile).  In request
  // order this launch covers requests [req_first, req_first + nreq), nreq <=
  // kReqChunk, and the items of a slab are numbered request by request with
  // no gaps (the kernel numbers them from the lengths); in pool order
  // (order != NULL) the items of a slab are the order_len listed entries,
  // each split into its subtiles.  A decode wave takes an item in `run`
  // consecutive slabs of the launch at a time (a unit of work; 1 for the
  // encode)
  int64_t num_blocks;
  int32_t block_size;
  int32_t heads;
  int32_t num_reqs;       // all requests of the call
  int32_t max_blocks;
  int32_t subtiles;       // ceil(block_size * H / 64)
  int32_t req_first;
  int32_t nreq;
  int32_t run;            // slabs per unit, 1..n_slabs
  const int32_t* table;
  const int32_t* lens;
  const int64_t* offsets;
  int32_t* err;
  // pool order: the call's items sorted by pool block (NULL: request order)
  const kvc_paged_item* order;
  int64_t order_len;

  int64_t total_items;    // items of this launch (paged: units, an upper bound, for the grid size)
  uint32_t sign_words[64];// bit 15 / bit 31 of word m: sign of element 2m / 2m+1
};

static_assert(sizeof(kvc_paged_item) == 32 && offsetof(kvc_paged_item, offset) == 16,
              "the kernels read a paged item as two 16-byte words");

enum class Op { Encode, Decode, Rotate };

/* Up to two launches: K and V run together when their code widths match. */
struct Plan {
  int n_launch;
  int req_chunks;         // paged: launches per entry of args, one per kReqChunk requests
  int bits[2];
  int head_dim;
  int dtype;
  int group;
  LaunchArgs args[2];
};

/* Host half: validate and fill a plan.  Returns a kvc_status. */
int plan_contiguous(Op op, const kvc_desc* d, const void* src, void* dst,
                    uint64_t blob_bytes, Plan* plan);
int plan_paged(Op op, const kvc_desc* d, const void* src, void* dst,
               uint64_t blob_bytes, const kvc_paged* pg, Plan* plan);

/* Sizes of a blob for T tokens (no validation beyond overflow).  Each
 * (layer, K/V) slab of codes and of meta is padded to a multiple of 256
 * bytes; the codes section holds the code slabs (l, K), (l, V) for l = 0..L-1,
 * the meta section the meta slabs in the same order. */
struct BlobSizes {
  uint64_t code_slab_k; // bytes of one K code slab, padding included
  uint64_t code_slab_v; // bytes of one V code slab, padding included
  uint64_t meta_slab;   // bytes of one meta slab, padding included
  uint64_t meta_offset; // start of the meta section (= bytes of the codes section)
  uint64_t total;
};
int blob_sizes(const kvc_desc* d, int64_t tokens, BlobSizes* out);

/* Layer chunks of a chunked blob: chunk k holds layers [k*chunk_layers,
 * min(L, (k+1)*chunk_layers)) as an ordinary blob at byte k * stride. */
struct Chunking {
  int64_t n_chunks;
  uint64_t stride;    // bytes between chunk starts (blob size of chunk_layers layers)
  uint64_t total;     // bytes of the chunked blob
  uint64_t kv_layer;  // bytes of one layer of the KV tensor
};
int chunking(const kvc_desc* d, int64_t chunk_layers, Chunking* c);

/* Workspace of the separate-kernel comparator for the contiguous shape in
 * d: one byte per element (codes), then four per element (fp32) at byte
 * *fp32_offset.  *bytes is 0 for an empty tensor. */
int unfused_workspace(const kvc_desc* d, uint64_t* bytes, uint64_t* fp32_offset);

}  // namespace kvc

#endif
