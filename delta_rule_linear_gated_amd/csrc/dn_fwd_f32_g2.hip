// dn_fwd_f32_g2.hip -- fwd kernels for f32 I/O, gate 2
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(fwd, f32, float, 2)
}  // namespace dn
