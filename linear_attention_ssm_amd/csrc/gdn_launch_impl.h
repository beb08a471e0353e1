// gdn_launch_impl.h -- definitions of the typed launchers (included by the
// per-key-dimension translation units only).
#pragma once

#include "gdn_kernels.h"
#include "gdn_launch.h"

namespace gdn {

template <typename K, typename A>
static hipError_t launch(K kernel, const A& a, dim3 grid, dim3 block, size_t smem,
                         hipStream_t stream) {
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, smem, stream, a);
  return hipGetLastError();
}

template <int DK, int QKV, int KG>
static hipError_t launch_packed_q(const DecodeArgs& a, int sd, dim3 grid, dim3 block, size_t smem,
                                  hipStream_t stream) {
  switch (sd) {
    case DT_F32: return launch(packed_decode_kernel<DK, QKV, DT_F32, KG>, a, grid, block, smem, stream);
    case DT_BF16: return launch(packed_decode_kernel<DK, QKV, DT_BF16, KG>, a, grid, block, smem, stream);
    case DT_F16: return launch(packed_decode_kernel<DK, QKV, DT_F16, KG>, a, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK, int KG>
static hipError_t launch_packed_g(const DecodeArgs& a, int qkv, int sd, dim3 grid, dim3 block,
                                  size_t smem, hipStream_t stream) {
  switch (qkv) {
    case DT_F32: return launch_packed_q<DK, DT_F32, KG>(a, sd, grid, block, smem, stream);
    case DT_BF16: return launch_packed_q<DK, DT_BF16, KG>(a, sd, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK>
hipError_t launch_packed(const DecodeArgs& a, int qkv, int sd, int kg, dim3 grid, dim3 block,
                         size_t smem, hipStream_t stream) {
  return kg ? launch_packed_g<DK, 1>(a, qkv, sd, grid, block, smem, stream)
            : launch_packed_g<DK, 0>(a, qkv, sd, grid, block, smem, stream);
}

template <int DK, int QKV, int RING, int SD>
static hipError_t launch_replay_s(const DecodeArgs& a, int kg, dim3 grid, dim3 block, size_t smem,
                                  hipStream_t stream) {
  // a single-token instance for T = 1 (decode steps, one-token windows)
  // (gate, in-kernel q/k normalisation) select the instance
  if (a.qk_norm) {
    if (kg) {
      if (a.T == 1) return launch(replay_decode_kernel<DK, QKV, RING, SD, 1, 1, 1>, a, grid, block, smem, stream);
      return launch(replay_decode_kernel<DK, QKV, RING, SD, 0, 1, 1>, a, grid, block, smem, stream);
    }
    if (a.T == 1) return launch(replay_decode_kernel<DK, QKV, RING, SD, 1, 0, 1>, a, grid, block, smem, stream);
    return launch(replay_decode_kernel<DK, QKV, RING, SD, 0, 0, 1>, a, grid, block, smem, stream);
  }
  if (kg) {
    if (a.T == 1) return launch(replay_decode_kernel<DK, QKV, RING, SD, 1, 1, 0>, a, grid, block, smem, stream);
    return launch(replay_decode_kernel<DK, QKV, RING, SD, 0, 1, 0>, a, grid, block, smem, stream);
  }
  if (a.T == 1) return launch(replay_decode_kernel<DK, QKV, RING, SD, 1, 0, 0>, a, grid, block, smem, stream);
  return launch(replay_decode_kernel<DK, QKV, RING, SD, 0, 0, 0>, a, grid, block, smem, stream);
}

template <int DK, int QKV, int RING>
static hipError_t launch_replay_r(const DecodeArgs& a, int sd, int kg, dim3 grid, dim3 block,
                                  size_t smem, hipStream_t stream) {
  switch (sd) {
    case DT_F32: return launch_replay_s<DK, QKV, RING, DT_F32>(a, kg, grid, block, smem, stream);
    case DT_BF16: return launch_replay_s<DK, QKV, RING, DT_BF16>(a, kg, grid, block, smem, stream);
    case DT_F16: return launch_replay_s<DK, QKV, RING, DT_F16>(a, kg, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK, int QKV>
static hipError_t launch_replay_q(const DecodeArgs& a, int ring, int sd, int kg, dim3 grid,
                                  dim3 block, size_t smem, hipStream_t stream) {
  switch (ring) {
    case DT_F32: return launch_replay_r<DK, QKV, DT_F32>(a, sd, kg, grid, block, smem, stream);
    case DT_F16: return launch_replay_r<DK, QKV, DT_F16>(a, sd, kg, grid, block, smem, stream);
    case DT_BF16: return launch_replay_r<DK, QKV, DT_BF16>(a, sd, kg, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK>
hipError_t launch_replay(const DecodeArgs& a, int qkv, int ring, int sd, int kg, dim3 grid,
                         dim3 block, size_t smem, hipStream_t stream) {
  switch (qkv) {
    case DT_F32: return launch_replay_q<DK, DT_F32>(a, ring, sd, kg, grid, block, smem, stream);
    case DT_BF16: return launch_replay_q<DK, DT_BF16>(a, ring, sd, kg, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK, int RING, int KG>
static hipError_t launch_fold_r(const FoldArgs& a, int sd, dim3 grid, dim3 block, size_t smem,
                                hipStream_t stream) {
  switch (sd) {
    case DT_F32: return launch(fold_kernel<DK, RING, DT_F32, KG>, a, grid, block, smem, stream);
    case DT_BF16: return launch(fold_kernel<DK, RING, DT_BF16, KG>, a, grid, block, smem, stream);
    case DT_F16: return launch(fold_kernel<DK, RING, DT_F16, KG>, a, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK, int KG>
static hipError_t launch_fold_g(const FoldArgs& a, int ring, int sd, dim3 grid, dim3 block,
                                size_t smem, hipStream_t stream) {
  switch (ring) {
    case DT_F32: return launch_fold_r<DK, DT_F32, KG>(a, sd, grid, block, smem, stream);
    case DT_F16: return launch_fold_r<DK, DT_F16, KG>(a, sd, grid, block, smem, stream);
    case DT_BF16: return launch_fold_r<DK, DT_BF16, KG>(a, sd, grid, block, smem, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DK>
hipError_t launch_fold(const FoldArgs& a, int ring, int sd, int kg, dim3 grid, dim3 block,
                       size_t smem, hipStream_t stream) {
  return kg ? launch_fold_g<DK, 1>(a, ring, sd, grid, block, smem, stream)
            : launch_fold_g<DK, 0>(a, ring, sd, grid, block, smem, stream);
}

#define GDN_INSTANTIATE(DK)                                                                  \
  template hipError_t launch_packed<DK>(const DecodeArgs&, int, int, int, dim3, dim3, size_t,  \
                                        hipStream_t);                                         \
  template hipError_t launch_replay<DK>(const DecodeArgs&, int, int, int, int, dim3, dim3,     \
                                        size_t, hipStream_t);                                 \
  template hipError_t launch_fold<DK>(const FoldArgs&, int, int, int, dim3, dim3, size_t,      \
                                      hipStream_t);

}  // namespace gdn
