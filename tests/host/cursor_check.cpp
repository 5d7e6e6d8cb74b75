// Walks the contiguous cursor (kvc_cursor.h) of every wave of many launches
// on the host and checks each tile against the direct formulas of the blob
// layout: slab s = l * 2 + kv of T*H rows, its vectors at (s * rows + v) *
// 2D in the tensor, its code slab at l * (ck + cv) + kv * ck, its meta slab
// at meta_offset + s * ms, every slab padded to 256 bytes.  Every item must
// be visited exactly once.  Built with g++ by tests/test_host_abi.py; prints
// "ok" and exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../kv_cache_compression_kvc_amd/csrc/kvc_plan.h"
#define KVC_CURSOR_FN inline
#include "../../kv_cache_compression_kvc_amd/csrc/kvc_cursor.h"

static int fails = 0;
#define CHECK(c)                                                                \
  do {                                                                          \
    if (!(c)) {                                                                 \
      if (fails < 20) fprintf(stderr, "%s:%d check failed: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                                                  \
    }                                                                           \
  } while (0)

static uint64_t rng_state = 7;
static uint64_t rnd() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

static int64_t up256(int64_t n) { return (n + 255) / 256 * 256; }

int main() {
  const int dims[] = {64, 128};
  const int bits[] = {2, 4, 8};
  const int groups[] = {32, 64, 128};
  int launches = 0;
  for (int it = 0; it < 2000; ++it) {
    kvc_desc d;
    d.layers = 1 + (int64_t)(rnd() % 6);
    d.tokens = 1 + (int64_t)(rnd() % (it % 4 == 0 ? 3000 : 300));
    d.kv_heads = 1 + (int64_t)(rnd() % 5);
    d.head_dim = dims[rnd() % 2];
    d.dtype = KVC_BF16;
    d.bits_k = bits[rnd() % 3];
    d.bits_v = it % 3 == 0 ? d.bits_k : bits[rnd() % 3];
    d.group = groups[rnd() % 3];
    if (d.group > d.head_dim) d.group = 32;
    d.seed = 1;
    uint64_t total = 0, meta_offset = 0;
    CHECK(kvc_encoded_size(&d, d.tokens, &total, &meta_offset) == KVC_OK);
    kvc::Plan plan;
    alignas(16) static char buf[32];
    CHECK(kvc::plan_contiguous(kvc::Op::Encode, &d, buf, buf, total, &plan) == KVC_OK);
    const int64_t rows = d.tokens * d.kv_heads;
    const int64_t D = d.head_dim, ng = D / d.group;
    const int64_t rk = D * d.bits_k / 8, rv = D * d.bits_v / 8;
    const int64_t ck = up256(rows * rk), cv = up256(rows * rv), ms = up256(rows * ng * 4);
    CHECK((int64_t)meta_offset == d.layers * (ck + cv));
    CHECK((int64_t)total == (int64_t)meta_offset + 2 * d.layers * ms);
    for (int li = 0; li < plan.n_launch; ++li) {
      const kvc::LaunchArgs& a = plan.args[li];
      ++launches;
      const int64_t n_items = a.total_items;
      const int64_t grids[] = {1, 2, 3, 7, 64, 1000, 1024, n_items, n_items + 5};
      for (int64_t grid : grids) {
        if (grid < 1) continue;
        std::vector<int> seen(n_items, 0);
        for (int64_t w = 0; w < grid && w < n_items; ++w) {
          kvc::ContigCursor c;
          kvc::contig_init(a, w, grid, c);
          int guard = 0;
          while (c.item < n_items && guard++ < 1000000) {
            kvc::ContigTile t;
            kvc::contig_tile(a, c, 2 * D, t);
            const int64_t s = (c.item / a.tiles_per_slab) * a.slab_step + a.slab_first;
            const int64_t tile = c.item % a.tiles_per_slab;
            const int64_t v0 = tile * 64, l = s >> 1, kv = s & 1;
            const int64_t row = kv ? rv : rk;
            const int64_t cslab = l * (ck + cv) + kv * ck;
            const int64_t mslab = (int64_t)meta_offset + s * ms;
            CHECK(c.tile == tile);
            CHECK(t.src == (s * rows + v0) * 2 * D);
            CHECK(t.codes == cslab + v0 * row);
            CHECK(t.meta == mslab + v0 * ng * 4);
            CHECK(t.count == (rows - v0 < 64 ? rows - v0 : 64));
            CHECK(t.last == (v0 + t.count == rows));
            CHECK(c.codes == cslab && c.meta == mslab);
            CHECK(a.row == row);
            CHECK(a.code_tail == (kv ? cv : ck) - rows * row);
            CHECK(a.meta_tail == ms - rows * ng * 4);
            // everything the tile touches lies inside the tensor and the blob
            CHECK(t.src >= 0 && t.src + t.count * 2 * D <= 2 * d.layers * rows * 2 * D);
            CHECK(t.codes + t.count * row <= (int64_t)meta_offset);
            CHECK(t.meta + t.count * ng * 4 <= (int64_t)total);
            ++seen[c.item];
            kvc::contig_next(a, grid, c);
          }
        }
        for (int64_t k = 0; k < n_items; ++k) CHECK(seen[k] == 1);
      }
    }
  }
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("ok: %d launches\n", launches);
  return 0;
}
