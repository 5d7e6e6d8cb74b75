/*
 * kvc_cursor.h -- the walk of a contiguous launch over its tiles, as plain
 * integer arithmetic shared by the kernels (kvc_device.h) and a host test
 * that checks it against the direct formulas.  The includer defines
 * KVC_CURSOR_FN (the kernels: __device__ __forceinline__; the host test:
 * inline) before including this header.
 *
 * Wave w of a grid of n handles items w, w + n, w + 2n, ... of the launch;
 * item k is tile k % tiles_per_slab of the launch's slab k / tiles_per_slab.
 * The cursor keeps the current slab's byte offsets in the tensor, the codes
 * and the meta, and advances them by per-launch constants, so a step costs
 * additions only: no product of a slab index with a stride.
 */
#ifndef KVC_CURSOR_H
#define KVC_CURSOR_H

#include <stdint.h>

#include "kvc_plan.h"

#ifndef KVC_CURSOR_FN
#error "define KVC_CURSOR_FN before including kvc_cursor.h"
#endif

namespace kvc {

struct ContigCursor {
  int64_t item;                // the wave's current item
  int64_t tile;                // its tile inside the current slab
  int64_t src, codes, meta;    // byte offsets of the current slab (tensor, code slab, meta slab)
  int64_t dtile;               // tiles advanced per step, below tiles_per_slab
  int64_t dsrc, dcodes, dmeta; // slab offsets advanced per step (whole slabs of the step)
};

/* The current tile: byte offsets of its first vector in the tensor, of the
 * start of its 64-row code tile, and of its first meta entry. */
struct ContigTile {
  int64_t src, codes, meta;
  int count;  // vectors, 1..64
  bool last;  // the slab's last tile
};

KVC_CURSOR_FN void contig_init(const LaunchArgs& a, int64_t start, int64_t step, ContigCursor& c) {
  const int64_t i = start / a.tiles_per_slab;
  const int64_t di = step / a.tiles_per_slab;
  c.item = start;
  c.tile = start - i * a.tiles_per_slab;
  c.src = a.src_first + i * a.src_stride;
  c.codes = a.codes_first + i * a.codes_stride;
  c.meta = a.meta_first + i * a.meta_stride;
  c.dtile = step - di * a.tiles_per_slab;
  c.dsrc = di * a.src_stride;
  c.dcodes = di * a.codes_stride;
  c.dmeta = di * a.meta_stride;
}

KVC_CURSOR_FN void contig_next(const LaunchArgs& a, int64_t step, ContigCursor& c) {
  c.item += step;
  c.tile += c.dtile;
  c.src += c.dsrc;
  c.codes += c.dcodes;
  c.meta += c.dmeta;
  if (c.tile >= a.tiles_per_slab) {
    c.tile -= a.tiles_per_slab;
    c.src += a.src_stride;
    c.codes += a.codes_stride;
    c.meta += a.meta_stride;
  }
}

KVC_CURSOR_FN void contig_tile(const LaunchArgs& a, const ContigCursor& c, int64_t vec_bytes, ContigTile& t) {
  const int64_t v0 = c.tile * kTileVectors;
  const int64_t left = a.rows - v0;
  t.count = static_cast<int>(left < kTileVectors ? left : kTileVectors);
  t.src = c.src + v0 * vec_bytes;
  t.codes = c.codes + v0 * a.row;
  t.meta = c.meta + v0 * (a.groups * 4);
  t.last = c.tile == a.tiles_per_slab - 1;
}

}  // namespace kvc

#endif
