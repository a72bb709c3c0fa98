// dn_fwd_f32_g1.hip -- fwd kernels for f32 I/O, gate 1
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(fwd, f32, float, 1)
}  // namespace dn
