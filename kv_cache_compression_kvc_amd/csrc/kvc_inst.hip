/*
 * kvc_inst.hip -- instantiates the encode / decode / rotate kernels for one
 * (head_dim, dtype) pair, chosen with -DKVC_D=<64|128> -DKVC_DT=<0|1>, and
 * exports a picker that maps (op, code width, group size, layout, decode
 * variant) to a kernel.
 * Building the four pairs as separate objects lets them compile in parallel.
 */
#include "kvc_device.h"
#include "kvc_pick.h"

#ifndef KVC_D
#error "define KVC_D"
#endif
#ifndef KVC_DT
#error "define KVC_DT"
#endif

namespace kvc {
namespace {

template <int D, int DT, int B, int G, bool PAGED>
Kernel pick_op(Op op, int mode) {
  if (op == Op::Encode) {
    if (mode == dev::kEncodeMatrix) return dev::encode_kernel<D, DT, B, G, PAGED, dev::kEncodeMatrix>;
    // paged butterfly encodes exist at 8 bits only, where they are the
    // default; at 2 and 4 bits the butterfly is a contiguous comparator
    if constexpr (!PAGED || B == 8)
      if (mode == dev::kEncodeButterfly) return dev::encode_kernel<D, DT, B, G, PAGED, dev::kEncodeButterfly>;
    return nullptr;
  }
  if constexpr (!PAGED) {
    // kDecodeLarge is picked at head_dim 64, and for 4-bit codes in one
    // group per vector at head_dim 128 (the launch rule in kvc_launch.hip)
    if constexpr (D == 64 || (B == 4 && G == D))
      if (mode == dev::kDecodeLarge) return dev::decode_kernel<D, DT, B, G, false, dev::kDecodeLarge>;
    if (mode == dev::kDecodeWaitStores) return dev::decode_kernel<D, DT, B, G, false, dev::kDecodeWaitStores>;
    if (mode == dev::kDecodeButterfly) return dev::decode_kernel<D, DT, B, G, false, dev::kDecodeButterfly>;
  } else {
    constexpr int M = D == 64 ? dev::kDecodeWaitTop : dev::kDecodeWaitStores;
    if (mode == M) return dev::decode_kernel<D, DT, B, G, true, M>;
  }
  return nullptr;
}

template <int D, int DT, int B, bool PAGED>
Kernel pick_g(Op op, int g, int mode) {
  switch (g) {
    case 32:
      return pick_op<D, DT, B, 32, PAGED>(op, mode);
    case 64:
      return pick_op<D, DT, B, 64, PAGED>(op, mode);
    case 128:
      if constexpr (D >= 128) return pick_op<D, DT, B, 128, PAGED>(op, mode);
      return nullptr;
    default:
      return nullptr;
  }
}

template <int D, int DT, bool PAGED>
Kernel pick_b(Op op, int b, int g, int mode) {
  switch (b) {
    case 2: return pick_g<D, DT, 2, PAGED>(op, g, mode);
    case 4: return pick_g<D, DT, 4, PAGED>(op, g, mode);
    case 8: return pick_g<D, DT, 8, PAGED>(op, g, mode);
    default: return nullptr;
  }
}

}  // namespace

Kernel KVC_PICK_NAME(KVC_D, KVC_DT)(Op op, int b, int g, bool paged, int mode) {
  if (op == Op::Rotate) return paged ? nullptr : dev::rotate_kernel<KVC_D, KVC_DT>;
  return paged ? pick_b<KVC_D, KVC_DT, true>(op, b, g, mode) : pick_b<KVC_D, KVC_DT, false>(op, b, g, mode);
}

}  // namespace kvc
