/* kvc_pick.h -- kernel pickers exported by the kvc_inst.hip objects. */
#ifndef KVC_PICK_H
#define KVC_PICK_H

#include "kvc_plan.h"

namespace kvc {

using Kernel = void (*)(LaunchArgs);

#define KVC_PICK_CAT(D, DT) pick_d##D##_t##DT
#define KVC_PICK_NAME(D, DT) KVC_PICK_CAT(D, DT)

/* `mode`: the encode's transform (kEncodeMatrix / kEncodeButterfly) or the
 * decode kernel's mode (kDecodeWaitTop / kDecodeWaitStores / kDecodeLarge /
 * kDecodeButterfly), both in kvc_device.h; ignored for the rotate kernel.
 * Only what the launcher uses is instantiated: the butterfly encode and
 * kDecodeButterfly for contiguous tensors, kDecodeLarge where the launch
 * rule picks it, paged WaitTop at head_dim 64 and WaitStores at 128; other
 * combinations return nullptr. */
Kernel pick_d64_t0(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d64_t1(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d128_t0(Op op, int bits, int group, bool paged, int mode);
Kernel pick_d128_t1(Op op, int bits, int group, bool paged, int mode);

}  // namespace kvc

#endif
