/*
 * kvc_host.cpp -- host half of the C ABI: argument validation, blob sizes,
 * the sign generator and launch plans.  Plain C++ with no HIP dependency,
 * so it also builds with g++ for unit tests and sanitizers.
 *
 * The sign vector of the randomized Hadamard transform (episode notes of
 * "FastKVComp: checking whether high-throughput KV compression pays off":
 * randomized Hadamard transform, then low-bit quantization) is drawn from
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): state += 0x9E3779B97F4A7C15,
 * then two xor-shift-multiply rounds and a final xor-shift; s_j = -1 iff bit
 * 63 of the (j+1)-th output is set.
 */
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "kvc_plan.h"

namespace kvc {
namespace {

constexpr uint64_t kAlign = 256;

bool mul_ok(uint64_t a, uint64_t b, uint64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(uint64_t a, uint64_t b, uint64_t* r) { return !__builtin_add_overflow(a, b, r); }

bool align_up(uint64_t n, uint64_t* r) {
  uint64_t t;
  if (!add_ok(n, kAlign - 1, &t)) return false;
  *r = t / kAlign * kAlign;
  return true;
}

uint64_t splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const kvc_desc* d) {
  if (!d) return KVC_EINVAL;
  if (d->layers < 0 || d->tokens < 0 || d->kv_heads < 0) return KVC_EINVAL;
  if (d->head_dim != 64 && d->head_dim != 128) return KVC_ESHAPE;
  if (d->dtype != KVC_BF16 && d->dtype != KVC_FP16) return KVC_EDTYPE;
  const int32_t widths[2] = {d->bits_k, d->bits_v};
  for (int32_t b : widths)
    if (b != 2 && b != 4 && b != 8) return KVC_EBITS;
  if (d->group != 32 && d->group != 64 && d->group != 128) return KVC_EGROUP;
  if (d->group > d->head_dim) return KVC_EGROUP;
  return KVC_OK;
}

void fill_signs(const kvc_desc* d, LaunchArgs* a) {
  uint64_t st = d->seed;
  memset(a->sign_words, 0, sizeof(a->sign_words));
  for (int j = 0; j < d->head_dim; ++j) {
    uint64_t z = splitmix64_next(&st);
    if (z >> 63) a->sign_words[j / 2] |= (j & 1) ? 0x80000000u : 0x00008000u;
  }
}

void common_args(const kvc_desc* d, LaunchArgs* a) {
  memset(a, 0, sizeof(*a));
  a->layers = d->layers;
  a->row_k = static_cast<int32_t>(d->head_dim * d->bits_k / 8);
  a->row_v = static_cast<int32_t>(d->head_dim * d->bits_v / 8);
  a->groups = static_cast<int32_t>(d->head_dim / d->group);
  fill_signs(d, a);
}

/* K and V together when their widths match (or for the rotate hook). */
void split_slabs(Op op, const kvc_desc* d, Plan* plan, const LaunchArgs& base) {
  if (op == Op::Rotate || d->bits_k == d->bits_v) {
    plan->n_launch = 1;
    plan->bits[0] = d->bits_k;
    plan->args[0] = base;
    plan->args[0].n_slabs = 2 * d->layers;
    plan->args[0].slab_step = 1;
    plan->args[0].slab_first = 0;
  } else {
    plan->n_launch = 2;
    for (int kv = 0; kv < 2; ++kv) {
      plan->bits[kv] = kv ? d->bits_v : d->bits_k;
      plan->args[kv] = base;
      plan->args[kv].n_slabs = d->layers;
      plan->args[kv].slab_step = 2;
      plan->args[kv].slab_first = kv;
    }
  }
}

}  // namespace

int blob_sizes(const kvc_desc* d, int64_t tokens, BlobSizes* out) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (tokens < 0 || !out) return KVC_EINVAL;
  const uint64_t layers = static_cast<uint64_t>(d->layers);
  const uint64_t row_k = static_cast<uint64_t>(d->head_dim) * d->bits_k / 8;
  const uint64_t row_v = static_cast<uint64_t>(d->head_dim) * d->bits_v / 8;
  const uint64_t meta_row = static_cast<uint64_t>(d->head_dim / d->group) * 4;
  uint64_t rows, ck, cv, m, pair, codes, metas, total;
  if (!mul_ok(static_cast<uint64_t>(tokens), static_cast<uint64_t>(d->kv_heads), &rows)) return KVC_ESHAPE;
  if (!mul_ok(rows, row_k, &ck) || !align_up(ck, &ck) || !mul_ok(rows, row_v, &cv) || !align_up(cv, &cv) ||
      !mul_ok(rows, meta_row, &m) || !align_up(m, &m))
    return KVC_ESHAPE;
  if (!add_ok(ck, cv, &pair) || !mul_ok(pair, layers, &codes) || !mul_ok(2 * layers, m, &metas) ||
      !add_ok(codes, metas, &total))
    return KVC_ESHAPE;
  if (total > static_cast<uint64_t>(INT64_MAX)) return KVC_ESHAPE;
  out->code_slab_k = ck;
  out->code_slab_v = cv;
  out->meta_slab = m;
  out->meta_offset = codes;
  out->total = total;
  return KVC_OK;
}

int chunking(const kvc_desc* d, int64_t chunk_layers, Chunking* c) {
  if (!d || !c || chunk_layers <= 0) return KVC_EINVAL;
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  kvc_desc dc = *d;
  dc.layers = d->layers < chunk_layers ? d->layers : chunk_layers;
  BlobSizes one, last;
  if ((st = blob_sizes(&dc, d->tokens, &one)) != KVC_OK) return st;
  c->n_chunks = d->layers == 0 ? 0 : (d->layers - 1) / chunk_layers + 1;
  c->stride = one.total;
  c->total = 0;
  if (c->n_chunks > 0) {
    dc.layers = d->layers - (c->n_chunks - 1) * chunk_layers;
    if ((st = blob_sizes(&dc, d->tokens, &last)) != KVC_OK) return st;
    uint64_t body;
    if (!mul_ok(static_cast<uint64_t>(c->n_chunks - 1), one.total, &body) || !add_ok(body, last.total, &c->total) ||
        c->total > static_cast<uint64_t>(INT64_MAX))
      return KVC_ESHAPE;
  }
  uint64_t kv;
  if (!mul_ok(static_cast<uint64_t>(d->tokens), static_cast<uint64_t>(d->kv_heads), &kv) ||
      !mul_ok(kv, static_cast<uint64_t>(d->head_dim) * 4, &kv))
    return KVC_ESHAPE;
  c->kv_layer = kv;
  return KVC_OK;
}

int unfused_workspace(const kvc_desc* d, uint64_t* bytes, uint64_t* fp32_offset) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (!bytes) return KVC_EINVAL;
  uint64_t rows, elems, off, fp, total;
  if (!mul_ok(static_cast<uint64_t>(d->tokens), static_cast<uint64_t>(d->kv_heads), &rows) ||
      !mul_ok(rows, 2ull * static_cast<uint64_t>(d->layers), &rows) ||
      !mul_ok(rows, static_cast<uint64_t>(d->head_dim), &elems) || !align_up(elems, &off) ||
      !mul_ok(elems, 4, &fp) || !add_ok(off, fp, &total) || total > static_cast<uint64_t>(INT64_MAX))
    return KVC_ESHAPE;
  *bytes = total;
  if (fp32_offset) *fp32_offset = off;
  return KVC_OK;
}

int plan_contiguous(Op op, const kvc_desc* d, const void* src, void* dst,
                    uint64_t blob_bytes, Plan* plan) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (!plan) return KVC_EINVAL;
  memset(plan, 0, sizeof(*plan));
  plan->head_dim = static_cast<int>(d->head_dim);
  plan->dtype = d->dtype;
  plan->group = d->group;
  BlobSizes sz;
  st = blob_sizes(d, d->tokens, &sz);
  if (st != KVC_OK) return st;
  uint64_t rows = static_cast<uint64_t>(d->tokens) * static_cast<uint64_t>(d->kv_heads);
  uint64_t elems;
  if (!mul_ok(rows, 2ull * d->layers * d->head_dim, &elems)) return KVC_ESHAPE;
  if (op != Op::Rotate && blob_bytes < sz.total) return KVC_ENOSPC;
  if (elems == 0) {  // nothing to read or write
    plan->n_launch = 0;
    return KVC_OK;
  }
  if (!src || !dst) return KVC_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return KVC_EALIGN;
  LaunchArgs base;
  common_args(d, &base);
  base.src = src;
  base.dst = dst;
  base.blob_bytes = blob_bytes;
  base.paged = 0;
  base.rows = static_cast<int64_t>(rows);
  base.tiles_per_slab = static_cast<int64_t>((rows + kTileVectors - 1) / kTileVectors);
  base.code_slab_k = sz.code_slab_k;
  base.code_slab_v = sz.code_slab_v;
  base.meta_slab = sz.meta_slab;
  base.meta_offset = sz.meta_offset;
  base.blob_total = sz.total;
  split_slabs(op, d, plan, base);
  // Every offset below is at most the tensor's or the blob's size, both of
  // which were computed without overflow above.
  const int64_t slab_bytes = static_cast<int64_t>(rows) * 2 * d->head_dim;
  for (int i = 0; i < plan->n_launch; ++i) {
    LaunchArgs& a = plan->args[i];
    uint64_t items;
    if (!mul_ok(static_cast<uint64_t>(a.n_slabs), static_cast<uint64_t>(a.tiles_per_slab), &items))
      return KVC_ESHAPE;
    a.total_items = static_cast<int64_t>(items);
    const bool v = a.slab_first == 1;  // a launch of V slabs only (K and V widths differ)
    a.src_first = a.slab_first * slab_bytes;
    a.src_stride = a.slab_step * slab_bytes;
    a.codes_first = v ? static_cast<int64_t>(sz.code_slab_k) : 0;
    a.codes_stride = a.slab_step == 1 ? static_cast<int64_t>(sz.code_slab_k)
                                      : static_cast<int64_t>(sz.code_slab_k + sz.code_slab_v);
    a.meta_first = static_cast<int64_t>(sz.meta_offset + a.slab_first * sz.meta_slab);
    a.meta_stride = a.slab_step * static_cast<int64_t>(sz.meta_slab);
    a.row = v ? a.row_v : a.row_k;
    a.code_tail = static_cast<int32_t>((v ? sz.code_slab_v : sz.code_slab_k) - rows * a.row);
    a.meta_tail = static_cast<int32_t>(sz.meta_slab - rows * a.groups * 4);
  }
  return KVC_OK;
}

int plan_paged(Op op, const kvc_desc* d, const void* src, void* dst,
               uint64_t blob_bytes, const kvc_paged* pg, Plan* plan) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (!plan || !pg || op == Op::Rotate) return KVC_EINVAL;
  memset(plan, 0, sizeof(*plan));
  plan->head_dim = static_cast<int>(d->head_dim);
  plan->dtype = d->dtype;
  plan->group = d->group;
  if (pg->block_size < 1 || pg->block_size > 1024) return KVC_ERANGE;
  if (pg->num_reqs < 0 || pg->max_blocks < 0 || pg->num_blocks < 0 || pg->reserved != 0)
    return KVC_ERANGE;
  // the paged kernels size a request's slabs by shifts: code rows and meta
  // rows must be powers of two (every supported head_dim / bits / group is)
  {
    const uint32_t widths[3] = {uint32_t(d->head_dim * d->bits_k / 8), uint32_t(d->head_dim * d->bits_v / 8),
                                uint32_t(d->head_dim / d->group * 4)};
    for (uint32_t w : widths)
      if (w == 0 || (w & (w - 1))) return KVC_ESHAPE;
  }
  // token positions (j * block_size, lengths) are 32-bit in the kernels
  if (static_cast<int64_t>(pg->max_blocks) * pg->block_size > INT32_MAX) return KVC_ERANGE;
  uint64_t vecs_per_block;
  if (!mul_ok(static_cast<uint64_t>(pg->block_size), static_cast<uint64_t>(d->kv_heads), &vecs_per_block) ||
      vecs_per_block > (1ull << 30))
    return KVC_ESHAPE;
  uint64_t subtiles = (vecs_per_block + kTileVectors - 1) / kTileVectors;
  const bool ordered = pg->order != nullptr;
  if (pg->order_len < 0 || (!ordered && pg->order_len != 0)) return KVC_EINVAL;
  uint64_t per_slab, items;
  if (ordered) {
    // one launch per code width over the listed items
    if (!mul_ok(static_cast<uint64_t>(pg->order_len), subtiles, &per_slab) || per_slab > (1ull << 40) ||
        !mul_ok(per_slab, 2ull * static_cast<uint64_t>(d->layers), &items) || items > (1ull << 62))
      return KVC_ESHAPE;
    plan->req_chunks = 1;
  } else {
    // item counts of one request chunk are 32-bit in the kernels
    if (static_cast<uint64_t>(pg->max_blocks) * subtiles * kReqChunk > static_cast<uint64_t>(INT32_MAX))
      return KVC_ERANGE;
    const uint64_t chunk = pg->num_reqs < kReqChunk ? static_cast<uint64_t>(pg->num_reqs) : kReqChunk;
    if (!mul_ok(chunk, static_cast<uint64_t>(pg->max_blocks), &per_slab) || !mul_ok(per_slab, subtiles, &per_slab) ||
        !mul_ok(per_slab, 2ull * static_cast<uint64_t>(d->layers), &items) || items > (1ull << 62))
      return KVC_ESHAPE;
    plan->req_chunks = (pg->num_reqs + kReqChunk - 1) / kReqChunk;
  }
  if (items == 0) {
    plan->n_launch = 0;
    return KVC_OK;
  }
  if (!src || !dst) return KVC_EINVAL;
  if (!ordered && (!pg->block_table || !pg->seq_lens || !pg->out_offsets)) return KVC_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return KVC_EALIGN;
  if ((reinterpret_cast<uintptr_t>(pg->out_offsets) & 7u) ||
      (reinterpret_cast<uintptr_t>(pg->block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(pg->seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(pg->err_flag) & 3u) ||
      (reinterpret_cast<uintptr_t>(pg->order) & 15u))
    return KVC_EALIGN;
  LaunchArgs base;
  common_args(d, &base);
  base.src = src;
  base.dst = dst;
  base.blob_bytes = blob_bytes;
  base.paged = 1;
  base.num_blocks = pg->num_blocks;
  base.block_size = pg->block_size;
  base.heads = static_cast<int32_t>(d->kv_heads);
  base.num_reqs = pg->num_reqs;
  base.max_blocks = pg->max_blocks;
  base.subtiles = static_cast<int32_t>(subtiles);
  base.table = pg->block_table;
  base.lens = pg->seq_lens;
  base.offsets = pg->out_offsets;
  base.err = pg->err_flag;
  base.order = pg->order;
  base.order_len = pg->order_len;
  // the pool's bytes per slab: num_blocks blocks of block_size * H vectors
  uint64_t pool_slab, pool_bytes;
  if (!mul_ok(static_cast<uint64_t>(pg->num_blocks), vecs_per_block, &pool_slab) ||
      !mul_ok(pool_slab, 2ull * static_cast<uint64_t>(d->head_dim), &pool_slab) ||
      !mul_ok(pool_slab, 2ull * static_cast<uint64_t>(d->layers), &pool_bytes) || pool_bytes > (1ull << 62))
    return KVC_ESHAPE;
  split_slabs(op, d, plan, base);
  for (int i = 0; i < plan->n_launch; ++i) {  // per request chunk; run_plan sets req_first / nreq
    LaunchArgs& a = plan->args[i];
    a.src_stride = a.slab_step * static_cast<int64_t>(pool_slab);
    // the decode kernel walks units of kPagedRun slabs, the encode kernel
    // units of one slab
    a.run = op == Op::Decode ? static_cast<int32_t>(a.n_slabs < kPagedRun ? a.n_slabs : kPagedRun) : 1;
    a.total_items = static_cast<int64_t>(per_slab) * ((a.n_slabs + a.run - 1) / a.run);
  }
  return KVC_OK;
}

}  // namespace kvc

extern "C" {

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_strerror(int32_t s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_EINVAL: return "invalid argument (null pointer or negative size)";
    case KVC_ESHAPE: return "unsupported shape or size overflow";
    case KVC_EBITS: return "bits must be 2, 4 or 8";
    case KVC_EGROUP: return "group must be 32, 64 or 128 and at most head_dim";
    case KVC_EDTYPE: return "dtype must be bf16 or fp16";
    case KVC_EALIGN: return "device pointer not suitably aligned";
    case KVC_ENOSPC: return "output buffer too small for the blob";
    case KVC_EHIP: return "HIP runtime error";
    case KVC_ERANGE: return "paged argument out of range";
    default: return "unknown status";
  }
}

kvc_status kvc_encoded_size(const kvc_desc* desc, int64_t tokens, uint64_t* total,
                            uint64_t* meta_offset) {
  if (!total) return KVC_EINVAL;
  kvc::BlobSizes sz;
  int st = kvc::blob_sizes(desc, tokens, &sz);
  if (st != KVC_OK) return static_cast<kvc_status>(st);
  *total = sz.total;
  if (meta_offset) *meta_offset = sz.meta_offset;
  return KVC_OK;
}

kvc_status kvc_sign_mask(uint64_t seed, int64_t head_dim, uint64_t* mask_words) {
  if (!mask_words || head_dim <= 0 || head_dim > 4096) return KVC_EINVAL;
  uint64_t st = seed;
  for (int64_t w = 0; w < (head_dim + 63) / 64; ++w) mask_words[w] = 0;
  for (int64_t j = 0; j < head_dim; ++j)
    if (kvc::splitmix64_next(&st) >> 63) mask_words[j / 64] |= 1ull << (j % 64);
  return KVC_OK;
}

kvc_status kvc_chunked_size(const kvc_desc* desc, int64_t chunk_layers, uint64_t* total, uint64_t* stride) {
  if (!total) return KVC_EINVAL;
  kvc::Chunking c;
  int st = kvc::chunking(desc, chunk_layers, &c);
  if (st != KVC_OK) return static_cast<kvc_status>(st);
  *total = c.total;
  if (stride) *stride = c.stride;
  return KVC_OK;
}

kvc_status kvc_unfused_workspace_size(const kvc_desc* desc, uint64_t* bytes) {
  return static_cast<kvc_status>(kvc::unfused_workspace(desc, bytes, nullptr));
}

kvc_status kvc_paged_order(const int32_t* block_table_host, int32_t num_reqs, int32_t max_blocks,
                           const int32_t* seq_lens_host, const int64_t* offsets_host, int32_t block_size,
                           int64_t num_blocks, kvc_paged_item* items_host, int64_t* n_items) {
  if (!n_items || num_reqs < 0 || max_blocks < 0 || num_blocks < 0) return KVC_EINVAL;
  if (block_size < 1 || block_size > 1024) return KVC_ERANGE;
  if (num_reqs > 0 && (!block_table_host || !seq_lens_host || !offsets_host)) return KVC_EINVAL;
  int64_t n = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int32_t len = seq_lens_host[r];
    if (len < 0) return KVC_EINVAL;
    if (static_cast<int64_t>(len) > static_cast<int64_t>(max_blocks) * block_size) return KVC_ERANGE;
    const int32_t nb = static_cast<int32_t>((static_cast<int64_t>(len) + block_size - 1) / block_size);
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t blk = block_table_host[static_cast<int64_t>(r) * max_blocks + j];
      if (blk < 0 || blk >= num_blocks) return KVC_ERANGE;
      if (items_host) {
        kvc_paged_item& it = items_host[n];
        it.block = blk;
        it.block_index = j;
        it.req = r;
        it.len = len;
        it.offset = offsets_host[r];
        it.reserved = 0;
      }
      ++n;
    }
  }
  if (items_host)
    std::sort(items_host, items_host + n, [](const kvc_paged_item& a, const kvc_paged_item& b) {
      if (a.block != b.block) return a.block < b.block;
      if (a.req != b.req) return a.req < b.req;
      return a.block_index < b.block_index;
    });
  *n_items = n;
  return KVC_OK;
}

kvc_status kvc_paged_layout(const kvc_desc* desc, const int32_t* seq_lens_host,
                            int32_t num_reqs, int64_t* offsets_host, uint64_t* total) {
  if (!total || num_reqs < 0) return KVC_EINVAL;
  if (num_reqs > 0 && (!seq_lens_host || !offsets_host)) return KVC_EINVAL;
  uint64_t acc = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (seq_lens_host[r] < 0) return KVC_EINVAL;
    kvc::BlobSizes sz;
    int st = kvc::blob_sizes(desc, seq_lens_host[r], &sz);
    if (st != KVC_OK) return static_cast<kvc_status>(st);
    offsets_host[r] = static_cast<int64_t>(acc);
    if (__builtin_add_overflow(acc, sz.total, &acc) || acc > static_cast<uint64_t>(INT64_MAX))
      return KVC_ESHAPE;
  }
  if (num_reqs == 0) {  // still validate the descriptor
    kvc::BlobSizes sz;
    int st = kvc::blob_sizes(desc, 0, &sz);
    if (st != KVC_OK) return static_cast<kvc_status>(st);
  }
  *total = acc;
  return KVC_OK;
}

}  // extern "C"
