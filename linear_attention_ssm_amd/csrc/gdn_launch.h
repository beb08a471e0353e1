// gdn_launch.h -- typed launchers, one explicit instantiation per key
// dimension (gdn_dk*.hip), so the template instances compile in parallel.
#pragma once

#include "gdn_device.h"

namespace gdn {

// kg: 0 = one decay per value head (GDN), 1 = one per key channel (KDA)
template <int DK>
hipError_t launch_packed(const DecodeArgs& a, int qkv, int sd, int kg, dim3 grid, dim3 block,
                         size_t smem, hipStream_t stream);
template <int DK>
hipError_t launch_replay(const DecodeArgs& a, int qkv, int ring, int sd, int kg, dim3 grid,
                         dim3 block, size_t smem, hipStream_t stream);
template <int DK>
hipError_t launch_fold(const FoldArgs& a, int ring, int sd, int kg, dim3 grid, dim3 block,
                       size_t smem, hipStream_t stream);

hipError_t launch_reset(const CursorArgs& a, hipStream_t stream);
hipError_t launch_advance(const CursorArgs& a, hipStream_t stream);
hipError_t launch_commit(const CursorArgs& a, hipStream_t stream);
hipError_t launch_zero(int32_t* p, int n, hipStream_t stream);

}  // namespace gdn
