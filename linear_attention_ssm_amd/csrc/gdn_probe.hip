// gdn_probe.hip -- the HBM probes (measurement aids): how fast this GPU
// streams a buffer in the access pattern of the decode's checkpoint reads, and
// how fast it copies one in the pattern of a checkpoint read and written back.
#include "gdn_launch.h"
#include "gdn_replay.h"

namespace gdn {
namespace {

// Each wavefront reads 8 KiB (eight 16-byte loads per lane, 1 KiB per
// instruction) with the decode's non-temporal load policy and sums a few
// words, so the loads cannot be dropped; the sum is written only if it equals
// a value no input of the probe produces.
__global__ __launch_bounds__(256) void read_probe_kernel(const char* src, float* sink) {
  const int lane = threadIdx.x & 63;
  const size_t item = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t r = brsrc(src + item * 8192, 8192);
  v4u x[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = __builtin_amdgcn_raw_buffer_load_b128(r, t * 1024 + lane * 16, 0, 2);
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc += __uint_as_float(x[t][0]) + __uint_as_float(x[t][3]);
  if (acc == 1234.5f) sink[0] = acc;
}

// Each wavefront copies 8 KiB: eight 16-byte loads per lane with the
// non-temporal policy, then eight 16-byte stores with the policy of the
// stores that write checkpoint lines back (sc1 nt). The loads of a wavefront
// all precede its stores, so a copy onto itself is exact.
__global__ __launch_bounds__(256) void copy_probe_kernel(const char* src, char* dst) {
  const int lane = threadIdx.x & 63;
  const size_t item = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t r = brsrc(src + item * 8192, 8192);
  const __amdgpu_buffer_rsrc_t w = brsrc(dst + item * 8192, 8192);
  v4u x[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = __builtin_amdgcn_raw_buffer_load_b128(r, t * 1024 + lane * 16, 0, 2);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    __builtin_amdgcn_raw_buffer_store_b128(x[t], w, t * 1024 + lane * 16, 0, kCpolSc1Nt);
}

}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_hbm_read_probe(const void* src, size_t nbytes, float* sink,
                                         void* stream) {
  if (!src || !sink || nbytes == 0 || nbytes % 32768 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || nbytes / 32768 > 0x7fffffffu)
    return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn::read_probe_kernel, dim3(static_cast<unsigned>(nbytes / 32768)), dim3(256),
                     0, static_cast<hipStream_t>(stream), static_cast<const char*>(src), sink);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

extern "C" gdn_status gdn_hbm_copy_probe(const void* src, void* dst, size_t nbytes, void* stream) {
  if (!src || !dst || nbytes == 0 || nbytes % 32768 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0 ||
      nbytes / 32768 > 0x7fffffffu)
    return GDN_ERR_INVALID_ARG;
  // the same buffer, or two that do not overlap
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 != d0 && s0 < d0 + nbytes && d0 < s0 + nbytes) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn::copy_probe_kernel, dim3(static_cast<unsigned>(nbytes / 32768)), dim3(256),
                     0, static_cast<hipStream_t>(stream), static_cast<const char*>(src),
                     static_cast<char*>(dst));
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
