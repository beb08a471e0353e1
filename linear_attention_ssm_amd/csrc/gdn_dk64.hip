// Kernel instances for key dimension 64.
#include "gdn_launch_impl.h"
namespace gdn {
GDN_INSTANTIATE(64)
}  // namespace gdn
