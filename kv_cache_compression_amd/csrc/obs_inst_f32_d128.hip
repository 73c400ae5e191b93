// obs_inst_f32_d128.hip -- instantiations of the scoring kernel for float32 keys, head size 128.
#include "obs_score_kernel.h"

namespace snapkv {

const void *obs_kernel_f32_d128(int mode, bool keep, int ctw) { return pick<float, 128>(mode, keep, ctw); }

}  // namespace snapkv
