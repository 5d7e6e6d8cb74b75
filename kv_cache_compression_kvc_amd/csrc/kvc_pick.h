/* kvc_pick.h -- kernel pickers exported by the kvc_inst.hip objects. */
#ifndef KVC_PICK_H
#define KVC_PICK_H

#include "kvc_plan.h"

namespace kvc {

using Kernel = void (*)(LaunchArgs);

#define KVC_PICK_CAT(D, DT) pick_d##D##_t##DT
#define KVC_PICK_NAME(D, DT) KVC_PICK_CAT(D, DT)

/* `large`: the decode variant for a contiguous blob larger than the
 * memory-side cache (one wave per SIMD; ignored for other kernels). */
Kernel pick_d64_t0(Op op, int bits, int group, bool paged, bool large);
Kernel pick_d64_t1(Op op, int bits, int group, bool paged, bool large);
Kernel pick_d128_t0(Op op, int bits, int group, bool paged, bool large);
Kernel pick_d128_t1(Op op, int bits, int group, bool paged, bool large);

}  // namespace kvc

#endif
