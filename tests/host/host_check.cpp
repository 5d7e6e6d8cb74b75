// Exercises the host half of the C ABI (validation, sizes, plans, signs)
// under AddressSanitizer / UndefinedBehaviorSanitizer.  Built with g++ by
// tests/test_host_abi.py; prints "ok" and exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../kv_cache_compression_kvc_amd/csrc/kvc_plan.h"

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "%s:%d check failed: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

static uint64_t rng_state = 42;
static uint64_t rnd() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

int main() {
  const int dims[] = {64, 128, 96, 0};
  const int bits[] = {2, 4, 8, 3};
  const int groups[] = {32, 64, 128, 16};
  for (int it = 0; it < 20000; ++it) {
    kvc_desc d;
    d.layers = (int64_t)(rnd() % 90) - 2;
    d.tokens = (int64_t)(rnd() % 70000) - 2;
    d.kv_heads = (int64_t)(rnd() % 10);
    d.head_dim = dims[rnd() % 4];
    d.dtype = (int32_t)(rnd() % 3);
    d.bits_k = bits[rnd() % 4];
    d.bits_v = bits[rnd() % 4];
    d.group = groups[rnd() % 4];
    d.seed = rnd();
    uint64_t total = 0, meta = 0;
    int st = kvc_encoded_size(&d, d.tokens, &total, &meta);
    if (st == KVC_OK) {
      CHECK(total % 256 == 0 && meta % 256 == 0 && meta <= total);
      uint64_t rows = (uint64_t)d.tokens * d.kv_heads * d.layers;
      CHECK(meta >= rows * d.head_dim * (d.bits_k + d.bits_v) / 8);
      CHECK(total - meta >= rows * 2 * (d.head_dim / d.group) * 4);
      kvc::Plan plan;
      alignas(16) static char buf[32];
      int ps = kvc::plan_contiguous(kvc::Op::Encode, &d, buf, buf, total, &plan);
      CHECK(ps == KVC_OK);
      if (ps == KVC_OK && plan.n_launch) {
        int64_t items = 0;
        for (int i = 0; i < plan.n_launch; ++i) items += plan.args[i].total_items;
        CHECK(items == 2 * d.layers * ((d.tokens * d.kv_heads + 63) / 64));
        CHECK(plan.n_launch == (d.bits_k == d.bits_v ? 1 : 2));
      }
      if (total > 0) CHECK(kvc::plan_contiguous(kvc::Op::Encode, &d, buf, buf, total - 1, &plan) == KVC_ENOSPC);
      if (rows > 0 && d.head_dim > 0)
        CHECK(kvc::plan_contiguous(kvc::Op::Encode, &d, buf + 1, buf, total, &plan) == KVC_EALIGN);
    } else {
      CHECK(st < 0);
    }
  }
  // paged layout: prefix sums of 256-aligned sizes
  kvc_desc d = {28, 0, 4, 128, KVC_BF16, 2, 4, 64, 0};
  int32_t lens[64];
  int64_t offs[64];
  for (int i = 0; i < 64; ++i) lens[i] = (int32_t)(rnd() % 8192);
  uint64_t total = 0;
  CHECK(kvc_paged_layout(&d, lens, 64, offs, &total) == KVC_OK);
  for (int i = 1; i < 64; ++i) CHECK(offs[i] >= offs[i - 1] && offs[i] % 256 == 0);
  lens[5] = -1;
  CHECK(kvc_paged_layout(&d, lens, 64, offs, &total) == KVC_EINVAL);
  CHECK(kvc_paged_layout(&d, nullptr, 0, nullptr, &total) == KVC_OK && total == 0);
  // paged plans: a table row whose token span overflows 32 bits is refused
  {
    alignas(16) static char pbuf[64];
    int32_t table[1] = {0}, plen[1] = {16};
    int64_t poff[1] = {0};
    kvc_paged pg = {8, 16, 1, 1, 0, table, plen, poff, nullptr};
    kvc::Plan plan;
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    // one head, 1024-token blocks: 16 subtiles per block; both the token span
    // (max_blocks * 1024) and a 64-request chunk's items (max_blocks * 16 * 64)
    // reach INT32_MAX at the same row length
    kvc_desc d1 = d;
    d1.kv_heads = 1;
    pg.block_size = 1024;
    pg.max_blocks = (int32_t)(INT32_MAX / 1024);
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d1, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    pg.max_blocks += 1;
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d1, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_ERANGE);
    CHECK(kvc::plan_paged(kvc::Op::Decode, &d1, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_ERANGE);
    // 16-token blocks of 4 heads: one subtile per block; the chunk's items bound the row
    pg.block_size = 16;
    pg.max_blocks = (int32_t)(INT32_MAX / 64);
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    CHECK(plan.req_chunks == 1);
    pg.max_blocks += 1;
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_ERANGE);
    // 130 requests: three launches of at most 64 requests per code width
    pg.max_blocks = 4;
    pg.num_reqs = 130;
    CHECK(kvc::plan_paged(kvc::Op::Encode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    CHECK(plan.req_chunks == 3 && plan.n_launch == 2);
    // the encode takes an item one slab at a time: 64 requests x 4 blocks per
    // slab, 28 slabs per code width; the pool's slab stride spans K and V
    // slabs (2 x 8 blocks x 16 tokens x 4 heads x 256 bytes)
    for (int i = 0; i < 2; ++i) {
      CHECK(plan.args[i].run == 1 && plan.args[i].total_items == 256 * 28);
      CHECK(plan.args[i].slab_step == 2 && plan.args[i].src_stride == 2 * 8 * 16 * 4 * 256);
    }
    // the decode walks kPagedRun slabs per item
    CHECK(kvc::plan_paged(kvc::Op::Decode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    for (int i = 0; i < 2; ++i)
      CHECK(plan.args[i].run == kvc::kPagedRun && plan.args[i].total_items == 256 * (28 / kvc::kPagedRun));
    // equal code widths: one launch over the 10 slabs of 5 layers, K and V alternating
    kvc_desc d5 = d;
    d5.layers = 5;
    d5.bits_k = d5.bits_v = 4;
    CHECK(kvc::plan_paged(kvc::Op::Decode, &d5, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_OK);
    CHECK(plan.n_launch == 1 && plan.args[0].slab_step == 1 && plan.args[0].n_slabs == 10);
    CHECK(plan.args[0].src_stride == 8 * 16 * 4 * 256);
    CHECK(plan.args[0].total_items == 256 * ((10 + kvc::kPagedRun - 1) / kvc::kPagedRun));
    // a pool whose bytes pass 2^62 is refused
    pg.num_blocks = int64_t(1) << 50;
    CHECK(kvc::plan_paged(kvc::Op::Decode, &d, pbuf, pbuf, 1 << 20, &pg, &plan) == KVC_ESHAPE);
  }
  // sign mask: 128 bits, the first 64 equal for head_dim 64
  uint64_t m128[2], m64[1];
  CHECK(kvc_sign_mask(7, 128, m128) == KVC_OK && kvc_sign_mask(7, 64, m64) == KVC_OK);
  CHECK(m128[0] == m64[0]);
  CHECK(kvc_sign_mask(7, 0, m64) == KVC_EINVAL);
  for (int s = -12; s <= 1; ++s) CHECK(kvc_strerror(s) != nullptr && strlen(kvc_strerror(s)) > 0);
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
