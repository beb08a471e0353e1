// Kernel instances for key dimension 256.
#include "gdn_launch_impl.h"
namespace gdn {
GDN_INSTANTIATE(256)
}  // namespace gdn
