// dn_bwd_bf16_g0.hip -- bwd kernels for bf16 I/O, gate 0
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(bwd, bf16, bf16, 0)
}  // namespace dn
