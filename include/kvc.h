/*
 * kvc.h -- fused KV-cache encode / decode on AMD CDNA4 (gfx950).
 *
 * The operation is the first two stages of the KV compression data path
 * described in "Beyond Compression Ratio: High-Throughput KV Compression
 * for Disaggregated LLM Serving" (abstract: the distribution transformation
 * and low-bit quantization are fused into one kernel with no full-size
 * intermediate tensor) and in the episode notes of "FastKVComp: checking
 * whether high-throughput KV compression pays off" (the transformation is
 * a randomized Hadamard transform, followed by low-bit quantization; only
 * quantization loses information; encode plus decode time must stay below
 * the wire time saved).  The lossless third stage is not part of this
 * library.
 *
 * Encode, per head_dim vector x of a [layers, 2, tokens, kv_heads, head_dim]
 * bf16 / fp16 KV tensor (axis 1: K then V):
 *   1. y = H (s * x) / sqrt(D): s in {-1,+1}^D drawn from SplitMix64 seeded
 *      with desc->seed (s_j = -1 iff bit 63 of the (j+1)-th output is set),
 *      H the Sylvester Hadamard matrix H[i][j] = (-1)^popcount(i & j);
 *   2. per group of `group` consecutive y: zero = fp16 round-down(min y),
 *      scale = fp16 round-up((max y - zero) / (2^b - 1)), b = bits_k for K
 *      and bits_v for V;
 *   3. q = round-half-even((y - zero) / scale) in [0, 2^b - 1] (0 if
 *      scale == 0), packed LSB-first: code j at bits [b*j, b*j + b) of the
 *      vector's D*b/8 bytes.
 * Decode: yhat = zero + q * scale, x = s * (H yhat) / sqrt(D), rounded to
 * nearest even in the tensor's dtype.  Computed as H = H_{D/G} (x) H_G: the
 * integer codes are transformed within each group exactly, then scaled (the
 * zero term reaches each group's first element only, as zero * G), then
 * combined across groups in binary32; the result does not depend on the
 * launch (kvc_decode, kvc_decode_paged and the chunked receive agree to the
 * bit on every vector).
 *
 * Blob layout (for T tokens):
 *   codes: for l in [0, L), for kv in (K, V): a code slab of T*H rows,
 *          (t, h) order, RB = D*b_kv/8 bytes each, stored in tiles of 64
 *          rows: tile k starts at byte 64*k*RB of the slab, and inside a
 *          tile of n rows (64, or fewer for the last) the 16-byte piece c
 *          of row i is at byte (c*n + i)*16 of the tile; then zero padding
 *          to a multiple of 256 bytes;
 *   meta:  for l in [0, L), for kv in (K, V): a meta slab of T*H*(D/group)
 *          entries of 4 bytes in (t, h, group) order -- fp16 scale, then
 *          fp16 zero, little endian; then zero padding to a multiple of 256.
 *   Every slab starts on a 256-byte boundary, so every full tile of 64 rows
 *   (codes and meta) covers whole 128-byte lines; where T*H*RB and
 *   T*H*(D/group)*4 are multiples of 256 there is no padding at all.
 *
 * Conventions for every call:
 *   - the caller allocates and owns all buffers; the library allocates no
 *     memory and keeps no state beyond a per-device occupancy cache (and
 *     the stream-ordering event of the chunked calls below);
 *   - device pointers must be 16-byte aligned and must not overlap;
 *   - GPU work is enqueued on `stream` (a hipStream_t passed as void*,
 *     NULL = the default stream) and the call returns without waiting;
 *     buffers must stay alive until the stream has passed the work;
 *   - arguments are validated on the host before anything is enqueued; a
 *     negative kvc_status is returned and nothing runs on the GPU;
 *   - launch failures are reported as KVC_EHIP;
 *   - kvc_encode, kvc_decode and their paged forms enqueue kernel launches
 *     only, so they may be captured into a HIP graph and replayed; make one
 *     call of the same kind on the device first, outside the capture (it
 *     fills the occupancy cache).  The chunked send / receive calls record
 *     events and are not meant for capture.
 *
 * Supported: head_dim 64 or 128; bits 2, 4 or 8; group 32, 64 or 128 with
 * group <= head_dim; dtype bf16 or fp16.  Input values must be finite, and
 * the rotated values y must fit the fp16 range of the meta (|y| <= 65504);
 * a group that breaks this gets unspecified meta and codes (nothing is read
 * or written out of bounds).  Subnormal inputs are handled exactly.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: every code and meta slab of the blob padded to a multiple of 256 bytes. */
#define KVC_ABI_VERSION 2

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_EINVAL = -1,  /* null descriptor or pointer, negative size          */
  KVC_ESHAPE = -2,  /* unsupported head_dim, or a size that overflows      */
  KVC_EBITS = -3,   /* bits not in {2, 4, 8}                               */
  KVC_EGROUP = -4,  /* group not in {32, 64, 128} or larger than head_dim  */
  KVC_EDTYPE = -5,  /* dtype not KVC_BF16 / KVC_FP16                       */
  KVC_EALIGN = -6,  /* a device pointer is not 16-byte aligned             */
  KVC_ENOSPC = -7,  /* output buffer smaller than the layout requires      */
  KVC_EHIP = -8,    /* the HIP runtime reported an error                   */
  KVC_ERANGE = -9   /* paged: block size or table shape out of range       */
} kvc_status;

typedef enum kvc_dtype { KVC_BF16 = 0, KVC_FP16 = 1 } kvc_dtype;

/* Shape and quantization parameters of one call. */
typedef struct kvc_desc {
  int64_t layers;    /* L >= 0                                        */
  int64_t tokens;    /* T >= 0 (contiguous calls; ignored when paged) */
  int64_t kv_heads;  /* H >= 0                                        */
  int64_t head_dim;  /* D: 64 or 128                                  */
  int32_t dtype;     /* kvc_dtype                                     */
  int32_t bits_k;    /* code width of K: 2, 4 or 8                    */
  int32_t bits_v;    /* code width of V: 2, 4 or 8                    */
  int32_t group;     /* group size along head_dim: 32, 64 or 128      */
  uint64_t seed;     /* sign seed of the randomized Hadamard transform */
} kvc_desc;

/*
 * Paged KV: a pool [L, 2, num_blocks, block_size, H, D] in which the
 * logical block j of request r (tokens [j*block_size, (j+1)*block_size))
 * is the physical block block_table[r*max_blocks + j].  Request r holds
 * seq_lens[r] tokens and its blob (the layout above with T = seq_lens[r])
 * starts at byte out_offsets[r] of the output; kvc_paged_layout computes
 * those offsets.  All three arrays live in device memory.
 *
 * Device-side checks: an entry of block_table outside [0, num_blocks), a
 * length above max_blocks*block_size or below 0, or a request blob that
 * would end past the output buffer makes the kernel skip that work and
 * set bit 0 of *err_flag (if err_flag is not NULL); such work is never
 * read or written out of bounds.
 */
typedef struct kvc_paged {
  int64_t num_blocks;          /* physical blocks in the pool               */
  int32_t block_size;          /* tokens per block, 1..1024                 */
  int32_t num_reqs;            /* R >= 0                                    */
  int32_t max_blocks;          /* row length of block_table, >= 0           */
  int32_t reserved;            /* must be 0                                 */
  const int32_t* block_table;  /* device, [num_reqs][max_blocks]            */
  const int32_t* seq_lens;     /* device, [num_reqs]                        */
  const int64_t* out_offsets;  /* device, [num_reqs]; multiples of 16       */
  int32_t* err_flag;           /* device, optional: bit 0 set on bad input  */
} kvc_paged;

/* KVC_ABI_VERSION of the built library. */
int32_t kvc_abi_version(void);

/* Static English text for a kvc_status value (never NULL). */
const char* kvc_strerror(int32_t status);

/*
 * Blob size for `tokens` tokens of the shape in `desc` (desc->tokens is
 * ignored).  *total receives the size in bytes, *meta_offset (may be
 * NULL) the byte offset of the meta section.  Host only.
 */
kvc_status kvc_encoded_size(const kvc_desc* desc, int64_t tokens,
                            uint64_t* total, uint64_t* meta_offset);

/*
 * The D signs of the transform as a bit mask: bit j of mask_words[j / 64]
 * is set iff s_j = -1.  mask_words holds (head_dim + 63) / 64 words.  Host
 * only; the same generator the kernels use.
 */
kvc_status kvc_sign_mask(uint64_t seed, int64_t head_dim, uint64_t* mask_words);

/*
 * Encode a contiguous KV tensor.  kv: device [L, 2, T, H, D] of desc->dtype.
 * out: device buffer of out_bytes >= kvc_encoded_size(desc, T); the blob is
 * written to its first `total` bytes (padding bytes are written as zero).
 */
kvc_status kvc_encode(const kvc_desc* desc, const void* kv, void* out,
                      uint64_t out_bytes, void* stream);

/*
 * Decode a blob written by kvc_encode (same desc) into a contiguous
 * device tensor kv_out [L, 2, T, H, D] of desc->dtype.  Its size is not
 * passed: the caller guarantees L*2*T*H*D elements of desc->dtype, all of
 * which are written.
 */
kvc_status kvc_decode(const kvc_desc* desc, const void* in, uint64_t in_bytes,
                      void* kv_out, void* stream);

/*
 * Host prologue of the paged calls: offsets_host[r] = sum of the blob
 * sizes of requests 0..r-1 (each a multiple of 256), *total = the sum of
 * all of them.  seq_lens_host and offsets_host are host arrays of
 * num_reqs entries.
 */
kvc_status kvc_paged_layout(const kvc_desc* desc, const int32_t* seq_lens_host,
                            int32_t num_reqs, int64_t* offsets_host, uint64_t* total);

/*
 * Encode every request of a paged pool.  pool: device
 * [L, 2, num_blocks, block_size, H, D] of desc->dtype; out: device buffer
 * of out_bytes; request r's blob at out + out_offsets[r].  Only the first
 * seq_lens[r] tokens of each request are read.
 */
kvc_status kvc_encode_paged(const kvc_desc* desc, const void* pool,
                            const kvc_paged* paged, void* out, uint64_t out_bytes,
                            void* stream);

/*
 * Decode every request's blob back into the pool slots named by the block
 * table; slots past seq_lens[r] and blocks no request names are left
 * untouched.
 */
kvc_status kvc_decode_paged(const kvc_desc* desc, const void* in, uint64_t in_bytes,
                            const kvc_paged* paged, void* pool, void* stream);

/*
 * Test hook: the rotated values y = H (s * x) / sqrt(D) of a contiguous KV
 * tensor, computed by the same device code as kvc_encode, written as fp32
 * to y_out (device, [L, 2, T, H, D]).
 */
kvc_status kvc_debug_rotate(const kvc_desc* desc, const void* kv, float* y_out,
                            void* stream);

/*
 * Comparator for the fused kernels: the same encode / decode as kvc_encode
 * and kvc_decode, computed by separate kernels -- rotate, group min/max,
 * quantize, pack (decode: unpack, dequantize, inverse rotate) -- that pass
 * fp32 and byte intermediates through `workspace`.  The blob is bit-identical
 * to kvc_encode's; the decoded tensor differs from kvc_decode's in rounding
 * only (this one dequantizes before the whole inverse transform, kvc_decode
 * transforms the integer codes within their groups first).  The arxivlens summary of "Beyond Compression Ratio:
 * High-Throughput KV Compression for Disaggregated LLM Serving" (key
 * results) compares its fused kernel with such separate kernels; its
 * abstract names the intermediate tensor and the repeated memory accesses
 * as what fusion removes.  Contiguous tensors only.
 *
 * kvc_unfused_workspace_size: bytes of device workspace both calls need
 * for desc's shape (5 bytes per element plus alignment; 0 for an empty
 * tensor).  Host only.
 * kvc_encode_unfused / kvc_decode_unfused: arguments as kvc_encode /
 * kvc_decode, plus a caller-owned device workspace (16-byte aligned,
 * workspace_bytes >= the size above, else KVC_ENOSPC) whose contents are
 * overwritten.  Calls that share a workspace must be ordered on one stream.
 */
kvc_status kvc_unfused_workspace_size(const kvc_desc* desc, uint64_t* bytes);
kvc_status kvc_encode_unfused(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                              void* workspace, uint64_t workspace_bytes, void* stream);
kvc_status kvc_decode_unfused(const kvc_desc* desc, const void* in, uint64_t in_bytes, void* kv_out,
                              void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * Chunked encode overlapped with the transfer of its output, and the
 * receiving side.  The episode notes of "FastKVComp: checking whether
 * high-throughput KV compression pays off" give the break-even rule
 * (encode plus decode time below the wire time saved); cutting the cache
 * into layer chunks lets the encode of one chunk run while the previous one
 * is on the wire, so the encode hides behind the transfer.
 *
 * Chunked blob: the layers are cut into chunks of chunk_layers layers (the
 * last may be shorter); chunk k is the ordinary blob of layers
 * [k*chunk_layers, ...) as a [L_k, 2, T, H, D] tensor, at byte offset
 * k * stride.  kvc_chunked_size (host only) gives *total bytes and the
 * *stride (may be NULL); chunk_layers must be >= 1.
 *
 * Chunks cross the link by a streaming-copy kernel on copy_stream, so the
 * far buffer (dst / src, >= total bytes, 16-byte aligned) must be device
 * memory or pinned, mapped host memory (hipHostMalloc; it stands in for a
 * NIC buffer); pageable host memory is rejected with KVC_EINVAL.
 *
 * kvc_encode_send: encodes chunk by chunk on compute_stream into `out`
 * (device, >= total bytes) and, after each chunk, copies it to the same
 * offset of `dst` on copy_stream.  Starts only after the work already
 * enqueued on copy_stream (an earlier call's copies out of `out`).  When
 * copy_stream has passed the work, dst holds the chunked blob.
 *
 * kvc_receive_decode: copies chunk k from `src` into the same offset of
 * `staging` (device, >= total bytes) on copy_stream, then decodes it into
 * kv_out [L, 2, T, H, D] on compute_stream, so the decode of chunk k
 * overlaps the copy of chunk k+1.  Starts only after the work already
 * enqueued on compute_stream (an earlier call's decodes out of `staging`).
 *
 * Both streams must have the default priority.  The two calls keep one
 * HIP event per (host thread, device) to order the streams.
 */
kvc_status kvc_chunked_size(const kvc_desc* desc, int64_t chunk_layers, uint64_t* total, uint64_t* stride);
kvc_status kvc_encode_send(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                           int64_t chunk_layers, void* dst, uint64_t dst_bytes, void* compute_stream,
                           void* copy_stream);
kvc_status kvc_receive_decode(const kvc_desc* desc, const void* src, uint64_t src_bytes, void* staging,
                              uint64_t staging_bytes, int64_t chunk_layers, void* kv_out,
                              void* compute_stream, void* copy_stream);

/*
 * Measurement helper: copy `bytes` (a multiple of 16) from src to dst with
 * 16-byte streaming loads and stores, to measure the achievable HBM
 * bandwidth next to the encode / decode kernels.
 */
kvc_status kvc_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
