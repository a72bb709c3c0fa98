// dn_fwd_bf16_g1.hip -- fwd kernels for bf16 I/O, gate 1
#include "dn_launch.h"

namespace dn {
DN_DEFINE_VARIANT(fwd, bf16, bf16, 1)
}  // namespace dn
