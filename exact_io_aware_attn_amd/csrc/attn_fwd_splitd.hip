// attn_fwd_splitd.hip -- placeholder translation unit for the split-D kernels
// (bf16, 256 < D <= 1024).
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {

LaunchFn splitd_launcher(int, int) { return nullptr; }

}  // namespace attn
