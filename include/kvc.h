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
 *     device memory in any call and keeps no state beyond a per-device
 *     occupancy cache, the stream-ordering event of the chunked calls
 *     below, and the static workspace array of kvc_encode_unfused_noalloc
 *     (part of the loaded code object, one per device);
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
 *     fills the occupancy cache).  The same holds for the *_with forms
 *     called without timing events.  The chunked send / receive calls, and
 *     *_with calls given events, set events and are not meant for capture.
 *
 * Supported: head_dim 64 or 128; bits 2, 4 or 8; group 32, 64 or 128 with
 * group <= head_dim; dtype bf16 or fp16.  Input values must be finite, and
 * the rotated values y must fit the fp16 range of the meta (|y| <= 65504);
 * a group that breaks this gets unspecified meta and codes (nothing is read
 * or written out of bounds).  Subnormal inputs are handled exactly.
 *
 * Precision.  The transform's sums are binary32, and the meta and the codes
 * are decided in binary32 (1/sqrt(D) folded into the meta, t = fma(u, A, B)
 * with A = rs / scale and B = -zero / scale, each rounded once).  A stored
 * zero or scale is then within one fp16 step of the definition above, and a
 * 2- or 4-bit code is the nearest level of the stored meta except where the
 * exact t lies within a few 2^-24 of (|y| + |zero|) / scale of a rounding
 * boundary k + 1/2 (within 1e-5 for ordinary data).  8-bit codes, whose t
 * reaches 255 where binary32 cannot resolve 1e-5, are the nearest level of
 * the stored meta to float64 accuracy: every element whose binary32 t lies
 * within a proven bound of a boundary is decided again from its input row
 * in float64.  8-bit encodes therefore rotate with the in-register
 * butterfly by default (KVC_TRANSFORM_AUTO below): its IEEE
 * additions admit a bound 2D / log2(D) times tighter than the matrix cores'
 * and leave that many times fewer elements to decide again.  The 8-bit
 * encode is still the slowest width.  In a 2- or 4-bit group whose range is comparable with
 * the binary32 resolution of its values (a huge offset with a tiny range)
 * the codes are only as good as that resolution.  Codes always stay within
 * [0, 2^b - 1].
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: every code and meta slab of the blob padded to a multiple of 256 bytes.
 * 3: kvc_paged carries an optional pool-order item list (kvc_paged_order).
 * 4: the *_with calls, whose kvc_launch_opts carries the transform and kernel timing events.
 * 5: kvc_probe_stream_runs. */
#define KVC_ABI_VERSION 5

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
 * length above max_blocks*block_size or below 0, or a request blob offset
 * that is negative, not a multiple of 16 or whose blob would end past the
 * output buffer makes the kernel skip that work (the block, or the whole
 * request) and set bit 0 of *err_flag (if err_flag is not NULL); such work
 * is never read or written out of bounds.  Overlap between request blobs
 * is not checked (the caller's guarantee).
 */
/*
 * One work item of a paged call in pool order: logical block block_index
 * of request req lives in pool block `block`; the request holds len tokens
 * and its blob starts at byte offset of the output.  32 bytes.
 */
typedef struct kvc_paged_item {
  int32_t block;        /* pool block                                     */
  int32_t block_index;  /* logical block j of the request                 */
  int32_t req;          /* request r                                      */
  int32_t len;          /* seq_lens[r]                                    */
  int64_t offset;       /* out_offsets[r]                                 */
  int64_t reserved;     /* 0                                              */
} kvc_paged_item;

typedef struct kvc_paged {
  int64_t num_blocks;          /* physical blocks in the pool               */
  int32_t block_size;          /* tokens per block, 1..1024                 */
  int32_t num_reqs;            /* R >= 0                                    */
  int32_t max_blocks;          /* row length of block_table, >= 0;
                                  max_blocks * block_size <= INT32_MAX      */
  int32_t reserved;            /* must be 0                                 */
  const int32_t* block_table;  /* device, [num_reqs][max_blocks]            */
  const int32_t* seq_lens;     /* device, [num_reqs]                        */
  const int64_t* out_offsets;  /* device, [num_reqs]; multiples of 16, the
                                  request blobs disjoint                    */
  int32_t* err_flag;           /* device, optional: bit 0 set on bad input  */
  const kvc_paged_item* order; /* device, optional: the call's items sorted
                                  by pool block (kvc_paged_order); the
                                  kernels then visit the pool in address
                                  order and read the request's length and
                                  offset from the item; NULL: request order */
  int64_t order_len;           /* items in order (0 when order is NULL)     */
} kvc_paged;

/* KVC_ABI_VERSION of the built library. */
int32_t kvc_abi_version(void);

/* Static English text for a kvc_status value (never NULL). */
const char* kvc_strerror(int32_t status);

/*
 * Blob size for `tokens` tokens of the shape in `desc` (desc->tokens is
 * ignored).  *total receives the size in bytes, *meta_offset (may be
 * NULL) the byte offset of the meta section.  Host only.  The byte format
 * is this library's own (the layout above): the pages describe compressing
 * the KV cache before it crosses the prefill-to-decode link but define no
 * format.  Errors: KVC_EINVAL (null total), the descriptor's errors,
 * KVC_ESHAPE when a size overflows.
 */
kvc_status kvc_encoded_size(const kvc_desc* desc, int64_t tokens,
                            uint64_t* total, uint64_t* meta_offset);

/*
 * The D signs of the transform as a bit mask: bit j of mask_words[j / 64]
 * is set iff s_j = -1.  mask_words holds (head_dim + 63) / 64 words.  Host
 * only; the same generator the kernels use.  The signs are the "randomized"
 * part of the randomized Hadamard transform of the episode notes of
 * "FastKVComp: checking whether high-throughput KV compression pays off";
 * the pages do not say how they are drawn (SplitMix64 is this library's
 * reading).  Errors: KVC_EINVAL (null mask, head_dim outside 1..4096).
 */
kvc_status kvc_sign_mask(uint64_t seed, int64_t head_dim, uint64_t* mask_words);

/*
 * Encode a contiguous KV tensor: the randomized Hadamard transform and the
 * low-bit quantization of the episode notes of "FastKVComp: checking
 * whether high-throughput KV compression pays off", fused in one pass with
 * no full-size intermediate as the abstract of "Beyond Compression Ratio:
 * High-Throughput KV Compression for Disaggregated LLM Serving" describes.
 * kv: device [L, 2, T, H, D] of desc->dtype (read only).  out: device buffer
 * of out_bytes >= kvc_encoded_size(desc, T), owned by the caller; the blob
 * is written to its first `total` bytes (padding bytes as zero), nothing
 * past them.  Errors: the descriptor's, KVC_EINVAL (null pointer with a
 * nonempty tensor), KVC_EALIGN, KVC_ENOSPC, KVC_EHIP.
 */
kvc_status kvc_encode(const kvc_desc* desc, const void* kv, void* out,
                      uint64_t out_bytes, void* stream);

/*
 * Decode a blob written by kvc_encode (same desc) into a contiguous
 * device tensor kv_out [L, 2, T, H, D] of desc->dtype: unpack, dequantize,
 * inverse transform -- the receiving side whose time the episode notes of
 * "FastKVComp: checking whether high-throughput KV compression pays off"
 * add to the encode's in the break-even.  in: in_bytes >= the blob size
 * (read only).  kv_out's size is not passed: the caller guarantees
 * L*2*T*H*D elements of desc->dtype, all of which are written.  Errors as
 * kvc_encode (KVC_ENOSPC: in_bytes too small).
 */
kvc_status kvc_decode(const kvc_desc* desc, const void* in, uint64_t in_bytes,
                      void* kv_out, void* stream);

/*
 * How the contiguous kernels compute the Walsh-Hadamard transform of the
 * episode notes of "FastKVComp: checking whether high-throughput KV
 * compression pays off": KVC_TRANSFORM_MATRIX as exact products with +-1 on
 * the matrix cores (a GEMM against H), KVC_TRANSFORM_BUTTERFLY as the
 * log2(D)-stage butterfly in each lane's registers, KVC_TRANSFORM_AUTO the
 * one kvc_encode / kvc_decode run for that shape (the faster one measured).
 */
typedef enum kvc_transform {
  KVC_TRANSFORM_AUTO = 0,
  KVC_TRANSFORM_MATRIX = 1,
  KVC_TRANSFORM_BUTTERFLY = 2
} kvc_transform;

/*
 * Options of the *_with calls (a NULL pointer means all defaults).
 *   transform: a kvc_transform value.  Paged calls accept AUTO and MATRIX
 *     (their kernels run on the matrix cores, except the 8-bit encode, which
 *     AUTO runs on the butterfly as for contiguous calls).
 *   start_event, stop_event: hipEvent_t handles created by the caller on the
 *     current device, or NULL.  start_event takes the time the call's first
 *     kernel starts, stop_event the time its last kernel ends (a call runs
 *     one kernel, or one per code width and per group of 64 requests), so
 *     that their elapsed time is the call's kernel time without the gaps of
 *     events recorded on the stream around it.  A call that launches nothing
 *     records both on the stream.  The events must not be recorded elsewhere
 *     until the call's work has completed.
 */
typedef struct kvc_launch_opts {
  int32_t transform;
  int32_t reserved;     /* 0 */
  void* start_event;
  void* stop_event;
} kvc_launch_opts;

/*
 * kvc_encode / kvc_decode with options: the transform chosen, everything
 * else of the launch as the automatic choice makes it (the pair the choice
 * of the transform is measured with), and kernel timing events.  The
 * butterfly and matrix-core encodes sum the same +-1 products in different
 * orders, so their blobs may differ where a rotated value rounds across a
 * code or meta boundary (both meet the oracle's criteria); every decode
 * transforms integer codes within groups exactly, so decodes of one blob
 * are bit-identical whichever transform runs.  Arguments and errors as
 * kvc_encode / kvc_decode, plus KVC_EINVAL for a transform outside the enum
 * or a nonzero reserved field, and KVC_EHIP if an event cannot be used.
 */
kvc_status kvc_encode_with(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                           const kvc_launch_opts* opts, void* stream);
kvc_status kvc_decode_with(const kvc_desc* desc, const void* in, uint64_t in_bytes, void* kv_out,
                           const kvc_launch_opts* opts, void* stream);

/*
 * Host prologue of the paged calls: offsets_host[r] = sum of the blob
 * sizes of requests 0..r-1 (each a multiple of 256), *total = the sum of
 * all of them; these offsets are disjoint by construction.  seq_lens_host
 * and offsets_host are host arrays of num_reqs entries owned by the caller.
 * Errors: KVC_EINVAL (null pointer, negative length), the descriptor's,
 * KVC_ESHAPE on overflow.
 */
kvc_status kvc_paged_layout(const kvc_desc* desc, const int32_t* seq_lens_host,
                            int32_t num_reqs, int64_t* offsets_host, uint64_t* total);

/*
 * Host prologue of the pool-order paged calls: every (request, logical
 * block) item of the call -- blocks 0 .. ceil(seq_lens[r] / block_size) - 1
 * of each request -- with its pool block, length and blob offset, sorted by
 * pool block (then request, then logical block), so that the kernels sweep
 * the pool in address order instead of in the block table's random order.
 * A block that several requests name appears once per request.  Host
 * arrays: block_table_host [num_reqs][max_blocks], seq_lens_host and
 * offsets_host [num_reqs] (kvc_paged_layout's offsets).  *n_items receives
 * the item count; items_host (may be NULL to query it) receives the items.
 * Errors: KVC_EINVAL (null pointer, negative length or count), KVC_ERANGE
 * (block_size outside 1..1024, a length above max_blocks * block_size, a
 * table entry outside [0, num_blocks)).
 */
kvc_status kvc_paged_order(const int32_t* block_table_host, int32_t num_reqs, int32_t max_blocks,
                           const int32_t* seq_lens_host, const int64_t* offsets_host, int32_t block_size,
                           int64_t num_blocks, kvc_paged_item* items_host, int64_t* n_items);

/*
 * Encode every request of a paged pool -- the KV cache as a serving engine
 * holds it, in blocks, compressed per request before it crosses the
 * prefill-to-decode link (abstract of "Beyond Compression Ratio:
 * High-Throughput KV Compression for Disaggregated LLM Serving").  pool:
 * device [L, 2, num_blocks, block_size, H, D] of desc->dtype (read only);
 * out: device buffer of out_bytes; request r's blob (the contiguous layout
 * with T = seq_lens[r]) at out + out_offsets[r].  Only the first
 * seq_lens[r] tokens of each request are read.  The request blobs
 * [out_offsets[r], out_offsets[r] + size_r) must be disjoint (the caller's
 * guarantee; kvc_paged_layout's offsets are): overlapping blobs race.
 * Without an order list, requests are processed in launches of at most 64
 * and each request's blocks in table order; with one (paged->order), one
 * launch per code width visits the items in the list's order, and the
 * list's lengths and offsets are used (they must match seq_lens and
 * out_offsets for the blobs to be those of the layout).  Errors (host): the
 * descriptor's, KVC_EINVAL, KVC_EALIGN, KVC_ERANGE (block_size outside
 * 1..1024, max_blocks * block_size above INT32_MAX, or more than INT32_MAX
 * items of 64 vectors in a 64-request launch), KVC_EHIP; on the device,
 * the checks of struct kvc_paged set *err_flag.
 */
kvc_status kvc_encode_paged(const kvc_desc* desc, const void* pool,
                            const kvc_paged* paged, void* out, uint64_t out_bytes,
                            void* stream);

/*
 * Decode every request's blob back into the pool slots named by the block
 * table (in: in_bytes, read only; pool written); slots past seq_lens[r]
 * and blocks no request names are left untouched.  Two requests must not
 * name the same pool slot.  Arguments and errors as kvc_encode_paged.
 */
kvc_status kvc_decode_paged(const kvc_desc* desc, const void* in, uint64_t in_bytes,
                            const kvc_paged* paged, void* pool, void* stream);

/*
 * kvc_encode_paged / kvc_decode_paged with the options of kvc_launch_opts
 * (transform AUTO or MATRIX, else KVC_EINVAL).  Results are those of the
 * calls without options.
 */
kvc_status kvc_encode_paged_with(const kvc_desc* desc, const void* pool, const kvc_paged* paged,
                                 void* out, uint64_t out_bytes, const kvc_launch_opts* opts,
                                 void* stream);
kvc_status kvc_decode_paged_with(const kvc_desc* desc, const void* in, uint64_t in_bytes,
                                 const kvc_paged* paged, void* pool, const kvc_launch_opts* opts,
                                 void* stream);

/*
 * Test hook: the rotated values y = H (s * x) / sqrt(D) of a contiguous KV
 * tensor -- the randomized Hadamard transform of the episode notes of
 * "FastKVComp: checking whether high-throughput KV compression pays off" --
 * computed by the same device code as kvc_encode, written as fp32 to y_out
 * (device, [L, 2, T, H, D], caller-owned; its size is the caller's
 * guarantee).  desc's bits and group are validated but unused.  Errors as
 * kvc_encode.
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
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * encode of kvc_encode_unfused with its workspace taken from a static
 * device array of KVC_NOALLOC_WORKSPACE_BYTES that the library holds on
 * every device it runs on until the process ends.  Arguments as kvc_encode;
 * the blob is bit-identical to kvc_encode_unfused's (and kvc_encode's).
 * A shape whose workspace (kvc_unfused_workspace_size) exceeds the array
 * returns KVC_ENOSPC before anything is enqueued -- 5 bytes per element, so
 * up to about 13.4 million elements.  The call allocates nothing; it needs
 * no zeroed memory (every workspace byte it reads it has written), and the
 * array keeps the last call's contents.  All calls on one device share the
 * one array: calls that overlap on a device (other streams, other host
 * threads) race and must be ordered by the caller.
 */
#define KVC_NOALLOC_WORKSPACE_BYTES (64ull << 20)
kvc_status kvc_encode_unfused_noalloc(const kvc_desc* desc, const void* kv, void* out, uint64_t out_bytes,
                                      void* stream);

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
 * copy_stream has passed the work, dst holds the chunked blob; until then
 * the copies still read `out`, so other work that writes or frees `out`
 * must first wait for copy_stream.
 *
 * kvc_receive_decode: copies chunk k from `src` into the same offset of
 * `staging` (device, >= total bytes) on copy_stream, then decodes it into
 * kv_out [L, 2, T, H, D] on compute_stream, so the decode of chunk k
 * overlaps the copy of chunk k+1.  Starts only after the work already
 * enqueued on compute_stream (an earlier call's decodes out of `staging`).
 * When compute_stream has passed the work, kv_out holds the decode; until
 * then the decodes still read `staging`, so other work that writes or frees
 * `staging` must first wait for compute_stream.
 *
 * Both streams must have the default priority (they may be the same
 * stream: the work then runs in order, without overlap).  The two calls
 * keep one HIP event per (host thread, device) to order the streams.
 * Arguments are checked before anything is enqueued; a launch failure
 * (KVC_EHIP) after the first chunk leaves the earlier chunks' work
 * enqueued.
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

/*
 * Measurement helper: read `read_bytes` of src and write `write_bytes` of
 * dst (both multiples of 1024; pointers 16-byte aligned; src and dst must
 * not overlap) with 16-byte streaming accesses, the two streams interleaved
 * at their ratio (4 KiB runs of the larger one, grid-strided) across
 * waves_per_cu (1..32) one-wave workgroups per CU.  With the read and write sizes of an encode or a
 * decode it is the achievable-bandwidth yardstick for that traffic mix.
 * dst receives unspecified bytes.  Errors: KVC_EINVAL (null pointer with a
 * nonzero size, waves_per_cu out of range), KVC_EALIGN.
 */
kvc_status kvc_probe_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                            int32_t waves_per_cu, void* stream);

/*
 * Measurement helper: the mix of kvc_probe_stream with each run of the
 * larger stream issued at once -- run_kib (4, 8 or 16) consecutive 1 KiB
 * chunks per run, so a wave has a whole run of loads in flight when reads
 * lead (16 KiB: one encode tile at head_dim 128) -- grid-strided over the
 * runs across waves_per_cu (1..32) one-wave workgroups per CU, each run
 * also moving its share of the smaller stream.  Sizes and pointers as for
 * kvc_probe_stream; dst receives unspecified bytes.  Errors: KVC_EINVAL
 * (null pointer with a nonzero size, run_kib or waves_per_cu out of range,
 * the larger size in KiB times the smaller past 2^62), KVC_EALIGN.
 */
kvc_status kvc_probe_stream_runs(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                                 int32_t run_kib, int32_t waves_per_cu, void* stream);

/*
 * Measurement helper with the access pattern of the paged kernels: a block
 * region of region_blocks blocks of block_bytes (a multiple of 1024) and a
 * sequential stream of stream_bytes (a multiple of 1024).  For each of the
 * n_blocks entries of the device array `blocks` (int32, in list order)
 * whole block blocks[i] of the region is moved, and the stream advances by
 * its share, so the two keep the ratio n_blocks * block_bytes :
 * stream_bytes.  scatter = 0 reads the listed blocks of `region` and writes
 * the stream to `seq` (the encode of a pool in table order); scatter = 1
 * reads the stream from `seq` and writes the listed blocks of `region` (the
 * decode).  Entries outside [0, region_blocks) move no block.  Written
 * bytes are unspecified.  Grid: waves_per_cu (1..32) one-wave workgroups
 * per CU, grid-strided over the list.  Errors: KVC_EINVAL (null pointer
 * with a nonzero size, negative counts, scatter not 0 or 1, waves_per_cu
 * out of range, n_blocks * stream_bytes / 1024 past 2^62), KVC_EALIGN.
 */
kvc_status kvc_probe_blocks(void* region, int64_t region_blocks, uint32_t block_bytes, const int32_t* blocks,
                            int64_t n_blocks, void* seq, uint64_t stream_bytes, int32_t scatter,
                            int32_t waves_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
