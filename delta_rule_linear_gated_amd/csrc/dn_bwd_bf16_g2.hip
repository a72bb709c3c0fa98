// dn_bwd_bf16_g2.hip -- bwd kernels for bf16 I/O, gate 2
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(bwd, bf16, bf16, 2)
}  // namespace dn
