// obs_inst_bf16_d128.hip -- instantiations of the scoring kernel for bfloat16 keys, head size 128.
#include "obs_score_kernel.h"

namespace snapkv {

const void *obs_kernel_bf16_d128(int mode, bool keep, int ctw) { return pick<__bf16, 128>(mode, keep, ctw); }

}  // namespace snapkv
