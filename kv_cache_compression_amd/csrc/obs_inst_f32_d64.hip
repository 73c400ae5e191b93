// obs_inst_f32_d64.hip -- instantiations of the scoring kernel for float32 keys, head size 64.
#include "obs_score_kernel.h"

namespace snapkv {

const void *obs_kernel_f32_d64(int mode, bool keep, int ctw) { return pick<float, 64>(mode, keep, ctw); }

}  // namespace snapkv
