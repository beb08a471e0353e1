// Kernel instances for key dimension 32.
#include "gdn_launch_impl.h"
namespace gdn {
GDN_INSTANTIATE(32)
}  // namespace gdn
