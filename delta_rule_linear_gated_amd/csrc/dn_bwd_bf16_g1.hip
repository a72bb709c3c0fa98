// dn_bwd_bf16_g1.hip -- bwd kernels for bf16 I/O, gate 1
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(bwd, bf16, bf16, 1)
}  // namespace dn
