/*
 * kvc_inst.hip -- instantiates the encode / decode / rotate kernels for one
 * (head_dim, dtype) pair, chosen with -DKVC_D=<64|128> -DKVC_DT=<0|1>, and
 * exports a picker that maps (op, code width, group size, layout) to a kernel.
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

template <int D, int DT, int B, bool PAGED>
Kernel pick_g(Op op, int g) {
  switch (g) {
    case 32:
      return op == Op::Encode ? dev::encode_kernel<D, DT, B, 32, PAGED> : dev::decode_kernel<D, DT, B, 32, PAGED>;
    case 64:
      return op == Op::Encode ? dev::encode_kernel<D, DT, B, 64, PAGED> : dev::decode_kernel<D, DT, B, 64, PAGED>;
    case 128:
      if constexpr (D >= 128)
        return op == Op::Encode ? dev::encode_kernel<D, DT, B, 128, PAGED>
                                : dev::decode_kernel<D, DT, B, 128, PAGED>;
      return nullptr;
    default:
      return nullptr;
  }
}

template <int D, int DT, bool PAGED>
Kernel pick_b(Op op, int b, int g) {
  switch (b) {
    case 2: return pick_g<D, DT, 2, PAGED>(op, g);
    case 4: return pick_g<D, DT, 4, PAGED>(op, g);
    case 8: return pick_g<D, DT, 8, PAGED>(op, g);
    default: return nullptr;
  }
}

}  // namespace

Kernel KVC_PICK_NAME(KVC_D, KVC_DT)(Op op, int b, int g, bool paged) {
  if (op == Op::Rotate) return paged ? nullptr : dev::rotate_kernel<KVC_D, KVC_DT>;
  return paged ? pick_b<KVC_D, KVC_DT, true>(op, b, g) : pick_b<KVC_D, KVC_DT, false>(op, b, g);
}

}  // namespace kvc
