// dn_fwd_bf16_g2.hip -- fwd kernels for bf16 I/O, gate 2
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(fwd, bf16, bf16, 2)
}  // namespace dn
