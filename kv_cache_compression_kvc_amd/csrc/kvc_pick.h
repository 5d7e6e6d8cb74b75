/* kvc_pick.h -- kernel pickers exported by the kvc_inst.hip objects. */
#ifndef KVC_PICK_H
#define KVC_PICK_H

#include "kvc_plan.h"

namespace kvc {

using Kernel = void (*)(LaunchArgs);

#define KVC_PICK_CAT(D, DT) pick_d##D##_t##DT
#define KVC_PICK_NAME(D, DT) KVC_PICK_CAT(D, DT)

/* `mode`: the decode kernel's mode (kDecodeWaitTop / kDecodeWaitStores /
 * kDecodeLarge in kvc_device.h; ignored for other kernels).  Only the modes
 * the launcher uses are instantiated: contiguous WaitStores and Large, paged
 * WaitTop at head_dim 64 and WaitStores at 128; others return nullptr. */
Kernel pick_d64_t0(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d64_t1(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d128_t0(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d128_t1(Op op, int bits, int group, bool paged, int mode);

}  // namespace kvc

#endif
