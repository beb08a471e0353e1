// gdn_cursor.hip -- the per-slot cursor kernels (reset, advance, commit)
// and their launchers. One thread per row; every kernel only touches
// write_pos[slot_idx[b]] of its own row.
#include "gdn_launch.h"

namespace gdn {

// ============================================================= cursors

// write_pos[s] <- 0 once every layer has folded the slot's ring (its own
// launch, stream-ordered after the folds that read the old value).
__global__ static void reset_kernel(CursorArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int s = a.slot[b];
  if (s < 0) return;
  if (s >= a.N) {
    if (a.err) atomicOr(a.err, EF_SLOT);
    return;
  }
  a.write_pos[s] = 0;
}

// Advance after a forward's decode calls (SGLang PR #28451, Design 3).
__global__ static void advance_kernel(CursorArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int s = a.slot[b];
  if (s < 0) return;
  if (s >= a.N) {
    if (a.err) atomicOr(a.err, EF_SLOT);
    return;
  }
  const int p = a.write_pos[s];
  if (p < 0 || p > a.L - 1) {
    if (a.err) atomicOr(a.err, EF_CURSOR);
    return;
  }
  const bool flush = (p == a.L - 1) || (a.force_flush != nullptr && a.force_flush[b] != 0);
  a.write_pos[s] = flush ? 0 : p + 1;
}

// Commit of a verify window's accepted prefix (vLLM PR #49887).
__global__ static void commit_kernel(CursorArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int s = a.slot[b];
  if (s < 0) return;
  if (s >= a.N) {
    if (a.err) atomicOr(a.err, EF_SLOT);
    return;
  }
  const int p = a.write_pos[s];
  const int acc = a.accepted[b];
  if (p < 0 || acc < 0 || acc > a.T || p + acc > a.L) {
    if (a.err) atomicOr(a.err, EF_ACCEPTED);
    return;
  }
  a.write_pos[s] = p + acc;
}

// n int32 zeros at p (one thread per element).
__global__ static void zero_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

static hipError_t launch_rows(void (*kernel)(CursorArgs), const CursorArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(kernel, dim3((a.B + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_reset(const CursorArgs& a, hipStream_t st) { return launch_rows(reset_kernel, a, st); }
hipError_t launch_advance(const CursorArgs& a, hipStream_t st) { return launch_rows(advance_kernel, a, st); }
hipError_t launch_commit(const CursorArgs& a, hipStream_t st) { return launch_rows(commit_kernel, a, st); }

hipError_t launch_zero(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace gdn
