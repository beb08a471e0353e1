// Kernel instances for key dimension 128.
#include "gdn_launch_impl.h"
namespace gdn {
GDN_INSTANTIATE(128)
}  // namespace gdn
