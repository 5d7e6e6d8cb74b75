/*
 * kvc_inst.hip -- instantiates the encode / decode / rotate kernels for one
 * (head_dim, dtype) pair, chosen with -DKVC_D=<64|128> -DKVC_DT=<0|1>, and
 * exports a picker that maps (op, code width, group size) to a kernel.
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

template <int D, int DT, int B>
Kernel pick_g(Op op, int g) {
  switch (g) {
    case 32:
      return op == Op::Encode ? dev::encode_kernel<D, DT, B, 32> : dev::decode_kernel<D, DT, B, 32>;
    case 64:
      return op == Op::Encode ? dev::encode_kernel<D, DT, B, 64> : dev::decode_kernel<D, DT, B, 64>;
    case 128:
      if constexpr (D >= 128)
        return op == Op::Encode ? dev::encode_kernel<D, DT, B, 128> : dev::decode_kernel<D, DT, B, 128>;
      return nullptr;
    default:
      return nullptr;
  }
}

}  // namespace

Kernel KVC_PICK_NAME(KVC_D, KVC_DT)(Op op, int b, int g) {
  if (op == Op::Rotate) return dev::rotate_kernel<KVC_D, KVC_DT>;
  switch (b) {
    case 2: return pick_g<KVC_D, KVC_DT, 2>(op, g);
    case 4: return pick_g<KVC_D, KVC_DT, 4>(op, g);
    case 8: return pick_g<KVC_D, KVC_DT, 8>(op, g);
    default: return nullptr;
  }
}

}  // namespace kvc
