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
Kernel pick_op(Op op, bool large) {
  if (op == Op::Encode) return dev::encode_kernel<D, DT, B, G, PAGED>;
  if constexpr (!PAGED)
    if (large) return dev::decode_kernel<D, DT, B, G, false, true>;
  return dev::decode_kernel<D, DT, B, G, PAGED, false>;
}

template <int D, int DT, int B, bool PAGED>
Kernel pick_g(Op op, int g, bool large) {
  switch (g) {
    case 32:
      return pick_op<D, DT, B, 32, PAGED>(op, large);
    case 64:
      return pick_op<D, DT, B, 64, PAGED>(op, large);
    case 128:
      if constexpr (D >= 128) return pick_op<D, DT, B, 128, PAGED>(op, large);
      return nullptr;
    default:
      return nullptr;
  }
}

template <int D, int DT, bool PAGED>
Kernel pick_b(Op op, int b, int g, bool large) {
  switch (b) {
    case 2: return pick_g<D, DT, 2, PAGED>(op, g, large);
    case 4: return pick_g<D, DT, 4, PAGED>(op, g, large);
    case 8: return pick_g<D, DT, 8, PAGED>(op, g, large);
    default: return nullptr;
  }
}

}  // namespace

Kernel KVC_PICK_NAME(KVC_D, KVC_DT)(Op op, int b, int g, bool paged, bool large) {
  if (op == Op::Rotate) return paged ? nullptr : dev::rotate_kernel<KVC_D, KVC_DT>;
  return paged ? pick_b<KVC_D, KVC_DT, true>(op, b, g, false) : pick_b<KVC_D, KVC_DT, false>(op, b, g, large);
}

}  // namespace kvc
