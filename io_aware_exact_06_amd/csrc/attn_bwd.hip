// attn_bwd.hip -- recompute backward (placeholder until the kernels land).
#include "attn_launch.h"

namespace attn {

hipError_t launch_bwd(const BwdParams&) { return hipErrorNotSupported; }

}  // namespace attn
