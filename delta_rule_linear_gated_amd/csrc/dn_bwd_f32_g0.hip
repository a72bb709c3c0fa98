// dn_bwd_f32_g0.hip -- bwd kernels for f32 I/O, gate 0
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(bwd, f32, float, 0)
}  // namespace dn
