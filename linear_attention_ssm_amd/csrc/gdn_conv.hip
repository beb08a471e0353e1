// gdn_conv.hip -- the causal convolution step in front of the decode
// (ReplaySSM blog, section 3.1: the decode path updates the causal
// convolution, then hands the convolved mixed_qkv row to the decode kernel;
// SGLang PR #36821, Technical principle: x_hat_t = SiLU(w * x_{t-3:t})).
//
// One thread per (row, four consecutive channels). It reads the W-1 stored
// inputs of its channels (one 8- or 16-byte piece per window row of the
// [N, W-1, C] state, so a wavefront reads whole contiguous rows), the current
// input and the 4 x W taps (W pieces of four), forms the tap sum with one fma
// per tap in tap order, applies SiLU in fp32, writes y and moves the window.
// Every value the state keeps is an input as given, so the state is copied,
// never rounded. HBM-bound: 2 W C es bytes per row plus the taps once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_device.h"
#include "gdn_replay.h"

namespace gdn {
namespace {

struct ConvArgs {
  const void* x;
  const void* w;
  void* state;
  const int32_t* slot;
  void* y;
  int32_t* err;
  int32_t N, C;
  int32_t x_rs, y_rs;  // row strides (elements)
};

template <int DT, int W>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
  const int b = blockIdx.y;
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;   // channels 4 c4 .. 4 c4 + 3
  if (4 * c4 >= a.C) return;
  const int s = ld_uniform(a.slot, b);
  const size_t yi = static_cast<size_t>(b) * a.y_rs + 4 * c4;
  if (s < 0 || s >= a.N) {
    if (s >= a.N && c4 == 0 && a.err) atomicOr(a.err, EF_SLOT);
    store4<DT>(a.y, yi, f4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  // the window, oldest first: W-1 stored inputs, then the current one
  const size_t st = static_cast<size_t>(s) * (W - 1) * a.C + 4 * c4;
  f4 z[W];
#pragma unroll
  for (int i = 0; i < W - 1; ++i) z[i] = load4<DT>(a.state, st + static_cast<size_t>(i) * a.C);
  z[W - 1] = load4<DT>(a.x, static_cast<size_t>(b) * a.x_rs + 4 * c4);
  // taps of the four channels, [channel][tap]: 4 W contiguous elements,
  // read as W four-element pieces
  float tap[4 * W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const f4 t4 = load4<DT>(a.w, static_cast<size_t>(4 * c4) * W + 4 * j);
#pragma unroll
    for (int m = 0; m < 4; ++m) tap[4 * j + m] = t4[m];
  }
  f4 yv;
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) acc = fmaf(tap[ch * W + i], z[i][ch], acc);
    yv[ch] = acc / (1.f + expf(-acc));
  }
  store4<DT>(a.y, yi, yv);
  // the window moves by one input (exact: every value is an input as given)
#pragma unroll
  for (int i = 0; i < W - 1; ++i) store4<DT>(a.state, st + static_cast<size_t>(i) * a.C, z[i + 1]);
}

template <int DT>
hipError_t launch_conv(const ConvArgs& a, int W, int B, hipStream_t stream) {
  const int groups = a.C / 4;
  const dim3 block(256), grid((groups + 255) / 256, B);
  switch (W) {
    case 2: hipLaunchKernelGGL((conv_kernel<DT, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((conv_kernel<DT, 3>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((conv_kernel<DT, 4>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

// [lo, hi) byte ranges overlap
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_conv_update(const gdn_conv_shape* s, const void* x, const void* w,
                                      void* conv_state, const int32_t* slot_idx, void* y,
                                      int32_t* err_flags, void* stream) {
  using namespace gdn;
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->B < 0 || s->N < 1) return GDN_ERR_INVALID_ARG;
  if (s->C < 4 || s->C % 4 != 0 || s->C > (1 << 20) || s->W < 2 || s->W > 4 || s->B > 65535)
    return GDN_ERR_UNSUPPORTED;
  if (s->dtype != GDN_F32 && s->dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  const int64_t xs = s->x_row_stride ? s->x_row_stride : s->C;
  const int64_t ys = s->y_row_stride ? s->y_row_stride : s->C;
  if (xs < s->C || ys < s->C) return GDN_ERR_INVALID_ARG;
  const size_t es = s->dtype == GDN_F32 ? 4 : 2;
  const size_t al = 4 * es;                        // one four-channel piece
  if ((xs * es) % al != 0 || (ys * es) % al != 0) return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  if (!x || !w || !conv_state || !slot_idx || !y) return GDN_ERR_INVALID_ARG;
  if (!aligned_to(x, al) || !aligned_to(w, al) || !aligned_to(conv_state, al) ||
      !aligned_to(y, al) || !aligned_to(slot_idx, 4) || (err_flags && !aligned_to(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  const size_t x_bytes = (static_cast<size_t>(s->B - 1) * xs + s->C) * es;
  const size_t y_bytes = (static_cast<size_t>(s->B - 1) * ys + s->C) * es;
  const size_t st_bytes = static_cast<size_t>(s->N) * (s->W - 1) * s->C * es;
  if (overlap(y, y_bytes, x, x_bytes) || overlap(y, y_bytes, conv_state, st_bytes) ||
      overlap(x, x_bytes, conv_state, st_bytes))
    return GDN_ERR_INVALID_ARG;
  ConvArgs a{};
  a.x = x; a.w = w; a.state = conv_state; a.slot = slot_idx; a.y = y; a.err = err_flags;
  a.N = s->N; a.C = s->C;
  a.x_rs = static_cast<int32_t>(xs);
  a.y_rs = static_cast<int32_t>(ys);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = s->dtype == GDN_F32 ? launch_conv<DT_F32>(a, s->W, s->B, st)
                                           : launch_conv<DT_BF16>(a, s->W, s->B, st);
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
