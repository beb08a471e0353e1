// gdn_gates.hip -- the gate activations in front of a per-key-gate (KDA)
// decode (SGLang PR #36821, Technical principle: g_t = l * sigma(e^A (a_t +
// b_dt)) per key channel and beta_t = sigma(b_t)).
//
// One thread per four key channels of one (row, token, value head): it reads
// the four raw gate inputs and the head's four dt_bias values (16-byte
// pieces), forms g = lower_bound * sigmoid(exp(A[h]) * (a + dt_bias)) in fp32
// and writes it; the thread of channels 0..3 also writes beta = sigmoid(b).
// HBM-bound: 8 bytes per channel (a read, g written) plus 8 per head.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_device.h"
#include "gdn_replay.h"

namespace gdn {
namespace {

struct GateArgs {
  const float* a;
  const float* b;
  const float* A;
  const float* dt_bias;
  float* g;
  float* beta;
  uint32_t n4;         // four-channel groups in total (B*T*Hv*dk/4)
  int32_t Hv, c4s;     // value heads, four-channel groups per head (dk/4)
  float lower_bound;
};

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + expf(-x)); }

__global__ __launch_bounds__(256) void kda_gates_kernel(GateArgs a) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;   // four-channel group
  if (i >= a.n4) return;
  const uint32_t head = i / a.c4s;                 // (row, token, head) index
  const int c4 = static_cast<int>(i - head * a.c4s);
  const int h = static_cast<int>(head % a.Hv);
  const float ea = expf(a.A[h]);
  const f4 x = *reinterpret_cast<const f4*>(a.a + 4 * static_cast<size_t>(i));
  const f4 bias = *reinterpret_cast<const f4*>(a.dt_bias + (static_cast<size_t>(h) * a.c4s + c4) * 4);
  f4 gv;
#pragma unroll
  for (int m = 0; m < 4; ++m) gv[m] = a.lower_bound * sigmoid(ea * (x[m] + bias[m]));
  *reinterpret_cast<f4*>(a.g + 4 * static_cast<size_t>(i)) = gv;
  if (c4 == 0) a.beta[head] = sigmoid(a.b[head]);
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_kda_gates(const gdn_gate_shape* s, const float* a, const float* b,
                                    const float* A, const float* dt_bias, float* g, float* beta,
                                    void* stream) {
  using namespace gdn;
  if (!s || s->B < 0 || s->T < 1 || s->Hv < 1) return GDN_ERR_INVALID_ARG;
  if (s->dk < 4 || s->dk % 4 != 0 || s->dk > 1024) return GDN_ERR_UNSUPPORTED;
  if (!(s->lower_bound < 0.f)) return GDN_ERR_INVALID_ARG;
  const uint64_t heads = static_cast<uint64_t>(s->B) * s->T * s->Hv;
  const uint64_t n4 = heads * (s->dk / 4);
  if (n4 >= (1ull << 32) - 256) return GDN_ERR_UNSUPPORTED;
  if (heads == 0) return GDN_OK;
  if (!a || !b || !A || !dt_bias || !g || !beta) return GDN_ERR_INVALID_ARG;
  if (!aligned_to(a, 16) || !aligned_to(dt_bias, 16) || !aligned_to(g, 16) ||
      !aligned_to(b, 4) || !aligned_to(A, 4) || !aligned_to(beta, 4))
    return GDN_ERR_INVALID_ARG;
  GateArgs ga{};
  ga.a = a; ga.b = b; ga.A = A; ga.dt_bias = dt_bias; ga.g = g; ga.beta = beta;
  ga.n4 = static_cast<uint32_t>(n4);
  ga.Hv = s->Hv;
  ga.c4s = s->dk / 4;
  ga.lower_bound = s->lower_bound;
  const dim3 block(256), grid(static_cast<unsigned>((n4 + 255) / 256));
  hipLaunchKernelGGL(kda_gates_kernel, grid, block, 0, static_cast<hipStream_t>(stream), ga);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
