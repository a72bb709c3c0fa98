// dn_bwd_f32_g1.hip -- bwd kernels for f32 I/O, gate 1
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(bwd, f32, float, 1)
}  // namespace dn
