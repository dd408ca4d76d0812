// Stand-in for the split-KV launcher in the host-sanitizer build of the library,
// which carries the host code the CPU tests of the C ABI reach (argument checks,
// planning, workspace sizing, the allocation-free entry's fit) but not the split-KV
// kernels: those tests never get as far as a launch, and a call that did would get
// VA_EHIP here instead of a kernel.
#include "va_internal.h"

namespace va {

int launch_splitkv_fwd(const verify_attn_args*, const Plan&, hipStream_t) { return VA_EHIP; }

}  // namespace va
