// gdn_api.hip -- the C ABI (include/gdn_replay.h): host-side validation,
// launch geometry and dispatch to the typed kernel instances. No call here
// synchronises, allocates or frees.
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gdn_launch.h"
#include "gdn_replay.h"

using namespace gdn;

namespace {

constexpr int kAbiVersion = 12;
static_assert(kArriveStride == GDN_ARRIVE_STRIDE, "arrival counter stride");

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t elem_size(int dt) { return dt == GDN_F32 ? 4 : 2; }

bool dk_supported(int dk) { return dk == 32 || dk == 64 || dk == 128 || dk == 256; }

// Waves per packed-decode workgroup.
constexpr int kPackedWaves = 8;

// Value rows per head per workgroup: the largest multiple of 16 dividing dv
// with G * VB / 16 <= target waves (at least 16, so at most 16 waves).
int pick_vb(int dv, int G) {
  const int tw = kPackedWaves;
  int best = 16;
  for (int vb = 16; vb <= dv; vb += 16)
    if (dv % vb == 0 && G * (vb / 16) <= (tw > G ? tw : G)) best = vb;
  return best;
}

gdn_status check_shape(const gdn_shape* s, bool need_ring) {
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->B < 0 || s->T < 1 || s->T > 16 || s->N < 1) return GDN_ERR_INVALID_ARG;
  if (s->Hv < 1 || s->Hk < 1 || s->Hv % s->Hk != 0 || s->Hv / s->Hk > 16)
    return GDN_ERR_INVALID_ARG;
  if (!dk_supported(s->dk)) return GDN_ERR_UNSUPPORTED;
  if (s->dv < 16 || s->dv > 512 || s->dv % 16 != 0) return GDN_ERR_UNSUPPORTED;
  if (s->qkv_dtype != GDN_F32 && s->qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (s->state_dtype != GDN_F32 && s->state_dtype != GDN_BF16 && s->state_dtype != GDN_F16)
    return GDN_ERR_UNSUPPORTED;
  if (s->gate != GDN_GATE_HEAD && s->gate != GDN_GATE_KEY) return GDN_ERR_INVALID_ARG;
  if (s->qk_norm != 0 && s->qk_norm != 1) return GDN_ERR_INVALID_ARG;
  {
    // input row strides: 0 = dense; else at least the dense width, and q/k
    // rows 16-byte aligned
    const int64_t es = s->qkv_dtype == GDN_F32 ? 4 : 2;
    if (s->qk_row_stride != 0 &&
        (s->qk_row_stride < static_cast<int64_t>(s->Hk) * s->dk || (s->qk_row_stride * es) % 16 != 0))
      return GDN_ERR_INVALID_ARG;
    if (s->v_row_stride != 0 && s->v_row_stride < static_cast<int64_t>(s->Hv) * s->dv)
      return GDN_ERR_INVALID_ARG;
  }
  if (need_ring) {
    if (s->L < 1 || s->L > 64) return GDN_ERR_INVALID_ARG;
    if (s->ring_dtype != GDN_F32 && s->ring_dtype != GDN_F16 && s->ring_dtype != GDN_BF16)
      return GDN_ERR_UNSUPPORTED;
  }
  return GDN_OK;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// The input row strides and the front-end switch of a decode call.
void fill_inputs(const gdn_shape* s, DecodeArgs& a) {
  a.qk_rs = s->qk_row_stride ? s->qk_row_stride : s->Hk * s->dk;
  a.v_rs = s->v_row_stride ? s->v_row_stride : s->Hv * s->dv;
  a.qk_norm = s->qk_norm;
}

// ceil(2^32 / d) for the device's udiv (0 encodes d = 1).
uint32_t recip(int d) {
  return d <= 1 ? 0u : static_cast<uint32_t>(((1ull << 32) + static_cast<uint64_t>(d) - 1) / d);
}

hipError_t dispatch_packed(int dk, const DecodeArgs& a, int qkv, int sd, int kg, dim3 g, dim3 b,
                           size_t sm, hipStream_t st) {
  switch (dk) {
    case 32: return launch_packed<32>(a, qkv, sd, kg, g, b, sm, st);
    case 64: return launch_packed<64>(a, qkv, sd, kg, g, b, sm, st);
    case 128: return launch_packed<128>(a, qkv, sd, kg, g, b, sm, st);
    case 256: return launch_packed<256>(a, qkv, sd, kg, g, b, sm, st);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_replay(int dk, const DecodeArgs& a, int qkv, int ring, int sd, int kg,
                           dim3 g, dim3 b, size_t sm, hipStream_t st) {
  switch (dk) {
    case 32: return launch_replay<32>(a, qkv, ring, sd, kg, g, b, sm, st);
    case 64: return launch_replay<64>(a, qkv, ring, sd, kg, g, b, sm, st);
    case 128: return launch_replay<128>(a, qkv, ring, sd, kg, g, b, sm, st);
    case 256: return launch_replay<256>(a, qkv, ring, sd, kg, g, b, sm, st);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_fold(int dk, const FoldArgs& a, int ring, int sd, int kg, dim3 g, dim3 b,
                         size_t sm, hipStream_t st) {
  switch (dk) {
    case 32: return launch_fold<32>(a, ring, sd, kg, g, b, sm, st);
    case 64: return launch_fold<64>(a, ring, sd, kg, g, b, sm, st);
    case 128: return launch_fold<128>(a, ring, sd, kg, g, b, sm, st);
    case 256: return launch_fold<256>(a, ring, sd, kg, g, b, sm, st);
  }
  return hipErrorInvalidValue;
}

void fill_decode_geometry(const gdn_shape* s, DecodeArgs& a, dim3& grid, dim3& block) {
  a.B = s->B; a.T = s->T; a.N = s->N; a.Hv = s->Hv; a.Hk = s->Hk; a.dv = s->dv; a.L = s->L;
  a.G = s->Hv / s->Hk;
  a.GH = a.G;
  a.nhc = 1;
  a.VB = pick_vb(s->dv, a.G);
  a.nvb = s->dv / a.VB;
  grid = dim3(static_cast<unsigned>(s->B) * s->Hk * a.nvb);
  block = dim3(64u * a.G * (a.VB / 16));
}

// Work-item geometry of the replay kernel: GH value heads (a divisor of G)
// times VB value rows per item, one wavefront per 16 rows of one head, at
// most kReplayWaves wavefronts. Wavefront 0 stages the gates of the item's GH
// heads and T tokens, one (head, token) pair per lane, so GH * T <= 64.
constexpr int kReplayWaves = 4;

void fill_replay_geometry(const gdn_shape* s, DecodeArgs& a, dim3& block, int& n_items) {
  const int tw = kReplayWaves;
  a.B = s->B; a.T = s->T; a.N = s->N; a.Hv = s->Hv; a.Hk = s->Hk; a.dv = s->dv; a.L = s->L;
  a.G = s->Hv / s->Hk;
  // value heads per workgroup: with a per-head gate, as many as fit (they
  // share the staged key ring); with the per-key gate one, since each head
  // brings a dk-wide log-decay per ring entry, which every workgroup of the
  // head re-reads and weights
  int gh = 1;
  for (int d = 1; d <= a.G && s->gate != GDN_GATE_KEY; ++d)
    if (a.G % d == 0 && d <= tw && d * s->T <= 64) gh = d;
  a.GH = gh;
  a.nhc = a.G / gh;
  int vb = 16;
  for (int v = 16; v <= s->dv; v += 16)
    if (s->dv % v == 0 && gh * (v / 16) <= tw) vb = v;
  a.VB = vb;
  a.nvb = s->dv / vb;
  block = dim3(64u * gh * (vb / 16));
  n_items = s->B * s->Hk * a.nhc * a.nvb;
  a.gsz = a.nhc * a.nvb;
  const int n_groups = n_items / a.gsz;
  a.full_blocks = (n_groups / 8 * 8) * a.gsz;
  a.m_gsz = recip(a.gsz);
  a.m_hk = recip(s->Hk);
  a.m_nvb = recip(a.nvb);
  a.m_wph = recip(vb / 16);
}

}  // namespace

extern "C" {

gdn_status gdn_packed_decode(const gdn_shape* s, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const int32_t* slot_idx,
                             void* state, void* o, int32_t* err_flags, void* stream) {
  const gdn_status st = check_shape(s, false);
  if (st != GDN_OK) return st;
  if (s->T != 1 || s->window != 0) return GDN_ERR_INVALID_ARG;
  if (!q || !k || !v || !g || !beta || !slot_idx || !state || !o) return GDN_ERR_INVALID_ARG;
  const size_t es = elem_size(s->qkv_dtype);
  const size_t ga = s->gate == GDN_GATE_KEY ? 16 : 4;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state, 16) || !aligned(v, es) ||
      !aligned(o, es) || !aligned(g, ga) || !aligned(beta, 4) || !aligned(slot_idx, 4) ||
      (err_flags && !aligned(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.slot = slot_idx; a.state = state;
  a.o = o; a.err = err_flags;
  fill_inputs(s, a);
  dim3 grid, block;
  fill_decode_geometry(s, a, grid, block);
  a.L = 1;
  a.dump_off = static_cast<int32_t>((2u * s->dk + 4) * sizeof(float));   // q, k, k^T q
  // per-key gate: [G][4][dk] floats of staged gates after the write sink
  a.kg_off = a.dump_off + static_cast<int32_t>(64 * 8 * sizeof(float));
  const size_t kg_bytes =
      s->gate == GDN_GATE_KEY ? static_cast<size_t>(a.G) * 4 * s->dk * sizeof(float) : 0;
  const size_t smem = a.kg_off + kg_bytes;
  return from_hip(dispatch_packed(s->dk, a, s->qkv_dtype, s->state_dtype, s->gate, grid, block,
                                  smem, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

gdn_status static_scratch(int32_t** out, hipStream_t stream);

// gdn_replay_decode, gdn_replay_decode_advance and
// gdn_replay_decode_advance_noalloc: arrive == nullptr and !use_scratch is the
// plain decode (write_pos only read); otherwise the cursor advance is fused,
// counting in the caller's arrive workspace or (use_scratch) in the library's
// static scratch.
gdn_status replay_decode(const gdn_shape* s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* slot_idx,
                         void* ckpt, void* ring_d, void* ring_k, float* ring_g,
                         const int32_t* write_pos, const int32_t* force_flush, void* o,
                         int32_t* arrive, int32_t* err_flags, void* stream,
                         bool use_scratch = false) {
  const gdn_status st = check_shape(s, true);
  if (st != GDN_OK) return st;
  if (s->window != 0 && s->window != 1) return GDN_ERR_INVALID_ARG;
  if (s->window == 0 && s->T != 1) return GDN_ERR_INVALID_ARG;
  if (s->window == 1 && force_flush) return GDN_ERR_INVALID_ARG;
  if (s->step_rounding != 0 && (s->step_rounding != 1 || s->window != 1)) return GDN_ERR_INVALID_ARG;
  if (s->T > s->L) return GDN_ERR_INVALID_ARG;
  if (!q || !k || !v || !g || !beta || !slot_idx || !ckpt || !ring_d || !ring_k || !ring_g ||
      !write_pos || !o)
    return GDN_ERR_INVALID_ARG;
  const size_t es = elem_size(s->qkv_dtype), rs = elem_size(s->ring_dtype);
  const size_t ga = s->gate == GDN_GATE_KEY ? 16 : 4;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(ckpt, 16) || !aligned(ring_k, 16) ||
      !aligned(ring_d, rs) || !aligned(v, es) || !aligned(o, es) || !aligned(g, ga) ||
      !aligned(beta, 4) || !aligned(ring_g, ga) || !aligned(write_pos, 4) ||
      !aligned(slot_idx, 4) || (err_flags && !aligned(err_flags, 4)) ||
      (force_flush && !aligned(force_flush, 4)))
    return GDN_ERR_INVALID_ARG;
  if (arrive && (s->window != 0 || !aligned(arrive, 128))) return GDN_ERR_INVALID_ARG;
  if (use_scratch && (s->window != 0 || s->B > GDN_SCRATCH_MAX_ROWS)) return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.slot = slot_idx; a.state = ckpt;
  a.ring_d = ring_d; a.ring_k = ring_k; a.ring_g = ring_g; a.write_pos = write_pos;
  a.arrive = arrive;
  a.write_pos_w = const_cast<int32_t*>(write_pos);   // written only when arrive != null
  a.force_flush = force_flush; a.o = o; a.err = err_flags; a.window = s->window;
  fill_inputs(s, a);
  a.step_round = s->step_rounding;
  // windows over a 16-bit ring are read out in chunked form (products on the
  // MFMA units); an fp32 ring keeps the token-by-token update, whose rounding
  // matches the packed decode bit for bit (lossless verify)
  a.win_mfma = (s->window == 1 && s->T >= 2 && s->T <= 8 && s->gate == GDN_GATE_HEAD &&
                s->step_rounding == 0 && s->ring_dtype != GDN_F32) ? 1 : 0;
  // the kernel reads one flag per row unconditionally; without
  // force_flush it reads the slot array and ignores the value
  a.ff_on = force_flush != nullptr;
  a.ff_flags = force_flush ? force_flush : slot_idx;
  dim3 block;
  int n_items = 0;
  if (static_cast<uint64_t>(s->B) * s->Hv * (s->dv / 16) >= (1ull << 31))
    return GDN_ERR_UNSUPPORTED;
  fill_replay_geometry(s, a, block, n_items);
  a.wg_per_row = s->Hk * a.gsz;
  {
    // udiv() needs every numerator below 2^32 / divisor
    const uint64_t dmax = std::max({a.gsz, s->Hk, a.nvb, 16});
    if (static_cast<uint64_t>(n_items) * dmax >= (1ull << 32)) return GDN_ERR_UNSUPPORTED;
  }
  size_t kt_bytes;
  if (s->ring_dtype == GDN_F32) {
    kt_bytes = static_cast<size_t>((s->L + 3) / 4 * 4) * s->dk * sizeof(float);
    a.kts = s->dk;
  } else {
    a.kts = (s->L + 15) / 16 * 16 + 4;
    kt_bytes = static_cast<size_t>(s->dk) * a.kts * 2;
  }
  // LDS: q and k of every token (fp32), k^T q per token, the gates of the
  // workgroup's heads, the staged key ring, a [64][8] fp32 write sink
  auto up16 = [](size_t x) { return (x + 15) / 16 * 16; };
  const size_t qk_bytes = static_cast<size_t>(s->T) * 2 * s->dk * sizeof(float);
  a.kq_off = static_cast<int32_t>(qk_bytes);
  a.gate_off = static_cast<int32_t>(qk_bytes + 16 * sizeof(float));
  a.kt_off = static_cast<int32_t>(up16(a.gate_off + static_cast<size_t>(a.GH) * s->T * 3 * sizeof(float)));
  size_t end = a.kt_off + kt_bytes;
  if (s->gate == GDN_GATE_KEY) {
    // per-key gate: no shared key ring; instead the staged gates [GH][T][4][dk],
    // one weighted key ring per head (the scalar path's layout and padding) and
    // the per-channel checkpoint decays [GH][dk]
    end = a.kt_off;
    a.kg_off = static_cast<int32_t>(end);
    end = up16(end + static_cast<size_t>(a.GH) * s->T * 4 * s->dk * sizeof(float));
    a.kw_off = static_cast<int32_t>(end);
    const size_t kw_bytes = kt_bytes;
    a.kw_head = static_cast<int32_t>(kw_bytes / elem_size(s->ring_dtype));
    end = up16(end + static_cast<size_t>(a.GH) * kw_bytes);
    a.acol_off = static_cast<int32_t>(end);
    end += static_cast<size_t>(a.GH) * s->dk * sizeof(float);
    // early copy of the ring log-decays and keys (rings of at most 16
    // entries, one 32-channel group per wavefront) and of the token gates
    const int nw = static_cast<int>(block.x / 64);
    const uint64_t g_bytes = static_cast<uint64_t>(s->B) * s->T * s->Hv * s->dk * sizeof(float);
    if (s->L <= 16 && a.GH * s->dk == 32 * nw && g_bytes < 0xfffffff0ull) {
      a.kdma = 1;
      a.g_bytes = static_cast<uint32_t>(g_bytes);
      a.kraw_wave = s->ring_dtype == GDN_F32 ? 4096 : 3072;
      end = up16(end);
      a.kraw_off = static_cast<int32_t>(end);
      end += static_cast<size_t>(nw) * a.kraw_wave;
      a.tg_off = static_cast<int32_t>(end);
      const int ntg = std::min(a.GH * s->T * (s->dk / 4), static_cast<int>(block.x));
      end += static_cast<size_t>((ntg + 63) / 64) * 1024;
    }
  }
  // a window's v values, [waves][16 tokens][16 rows] floats
  a.v_off = static_cast<int32_t>(up16(end));
  if (s->T > 1) end = a.v_off + static_cast<size_t>(block.x / 64) * 16 * 16 * sizeof(float);
  // single-token steps with an fp32 checkpoint at dk = 128 over a 16-bit
  // ring with a per-head gate: rows that do not flush take the split readout
  // (the kernel checks the rest: 1..16 valid entries, no flush); it needs the
  // token's q and k in the ring's format (512 bytes) and reuses the key-ring
  // area for the ring keys in row order
  a.split_ro = (s->window == 0 && s->gate == GDN_GATE_HEAD && s->ring_dtype != GDN_F32 &&
                s->state_dtype == GDN_F32 && s->dk == 128 && block.x == 256) ? 1 : 0;
  if (a.split_ro) {
    a.qh_off = static_cast<int32_t>(up16(end));
    end = a.qh_off + static_cast<size_t>(2) * s->dk * 2;
  }
  a.dump_off = static_cast<int32_t>(up16(end));
  const size_t smem = a.dump_off + 64 * 8 * sizeof(float);
  if (smem > 160 * 1024) return GDN_ERR_UNSUPPORTED;
  if (use_scratch) {
    // every argument is valid: only now may the first call on a device set
    // up the scratch (address lookup, one clear enqueued on the stream)
    const gdn_status ss = static_scratch(&a.arrive, static_cast<hipStream_t>(stream));
    if (ss != GDN_OK) return ss;
  }
  return from_hip(dispatch_replay(s->dk, a, s->qkv_dtype, s->ring_dtype, s->state_dtype, s->gate,
                                  dim3(n_items), block,
                                  smem, static_cast<hipStream_t>(stream)));
}

}  // namespace

// ------------------------------------------------------------- static scratch
//
// The arrival counters of gdn_replay_decode_advance_noalloc: one 128-byte
// line (GDN_ARRIVE_STRIDE int32) per row for up to GDN_SCRATCH_MAX_ROWS rows,
// 512 KiB held on every device the library runs on until the process ends.
// In host code `scratch` is only a host-side stand-in for the device array:
// its device address is looked up once per device with hipGetSymbolAddress
// (that device current) and kept in scratch_ptr, which is what kernels and
// launches receive.
static __device__ __align__(256) int32_t scratch[GDN_SCRATCH_MAX_ROWS * GDN_ARRIVE_STRIDE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
int32_t* scratch_ptr[kMaxDevices];   // per device, set on its first call

// The current device's copy of the scratch. The first call on a device looks
// up its address and enqueues one clear of the whole array on `stream` (the
// counters must start at zero; every completed call leaves them zero).
gdn_status static_scratch(int32_t** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GDN_ERR_HIP;
    int32_t* sp = static_cast<int32_t*>(p);
    if (launch_zero(sp, GDN_SCRATCH_MAX_ROWS * GDN_ARRIVE_STRIDE, stream) != hipSuccess)
      return GDN_ERR_HIP;
    scratch_ptr[dev] = sp;
  }
  *out = scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_replay_decode(const gdn_shape* s, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const int32_t* slot_idx,
                             void* ckpt, void* ring_d, void* ring_k, float* ring_g,
                             const int32_t* write_pos, const int32_t* force_flush, void* o,
                             int32_t* err_flags, void* stream) {
  return replay_decode(s, q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
                       force_flush, o, nullptr, err_flags, stream);
}

gdn_status gdn_replay_decode_advance(const gdn_shape* s, const void* q, const void* k,
                                     const void* v, const float* g, const float* beta,
                                     const int32_t* slot_idx, void* ckpt, void* ring_d,
                                     void* ring_k, float* ring_g, int32_t* write_pos,
                                     const int32_t* force_flush, void* o, int32_t* arrive,
                                     int32_t* err_flags, void* stream) {
  if (!arrive) return GDN_ERR_INVALID_ARG;
  return replay_decode(s, q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
                       force_flush, o, arrive, err_flags, stream);
}

gdn_status gdn_replay_decode_advance_noalloc(const gdn_shape* s, const void* q, const void* k,
                                             const void* v, const float* g, const float* beta,
                                             const int32_t* slot_idx, void* ckpt, void* ring_d,
                                             void* ring_k, float* ring_g, int32_t* write_pos,
                                             const int32_t* force_flush, void* o,
                                             int32_t* err_flags, void* stream) {
  if (s && s->B > GDN_SCRATCH_MAX_ROWS) return GDN_ERR_SCRATCH_LIMIT;
  return replay_decode(s, q, k, v, g, beta, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos,
                       force_flush, o, nullptr, err_flags, stream, true);
}

gdn_status gdn_replay_advance(const gdn_shape* s, const int32_t* slot_idx, int32_t* write_pos,
                              const int32_t* force_flush, int32_t* err_flags, void* stream) {
  if (!s || s->B < 0 || s->N < 1 || s->L < 1 || s->L > 64) return GDN_ERR_INVALID_ARG;
  if (!slot_idx || !write_pos) return GDN_ERR_INVALID_ARG;
  if (!aligned(slot_idx, 4) || !aligned(write_pos, 4) || (err_flags && !aligned(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  CursorArgs a{};
  a.slot = slot_idx; a.force_flush = force_flush; a.write_pos = write_pos; a.err = err_flags;
  a.B = s->B; a.N = s->N; a.L = s->L; a.T = s->T;
  return from_hip(launch_advance(a, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_replay_commit(const gdn_shape* s, const int32_t* slot_idx, const int32_t* accepted,
                             int32_t* write_pos, int32_t* err_flags, void* stream) {
  if (!s || s->B < 0 || s->N < 1 || s->L < 1 || s->L > 64 || s->T < 1 || s->T > 16)
    return GDN_ERR_INVALID_ARG;
  if (!slot_idx || !accepted || !write_pos) return GDN_ERR_INVALID_ARG;
  if (!aligned(slot_idx, 4) || !aligned(accepted, 4) || !aligned(write_pos, 4) ||
      (err_flags && !aligned(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  CursorArgs a{};
  a.slot = slot_idx; a.accepted = accepted; a.write_pos = write_pos; a.err = err_flags;
  a.B = s->B; a.N = s->N; a.L = s->L; a.T = s->T;
  return from_hip(launch_commit(a, static_cast<hipStream_t>(stream)));
}

namespace {

// The fold of n layers of equal shapes, kFoldMaxLayers per launch (the layer
// in blockIdx.y). Every pointer array holds n device pointers.
gdn_status fold_layers(const gdn_shape* s, int n, const int32_t* slot_idx, void* const* ckpt,
                       const void* const* ring_d, const void* const* ring_k,
                       const float* const* ring_g, const int32_t* write_pos, int32_t* err_flags,
                       void* stream) {
  const gdn_status st = check_shape(s, true);
  if (st != GDN_OK) return st;
  if (!slot_idx || !write_pos) return GDN_ERR_INVALID_ARG;
  if (s->step_rounding != 0 && s->step_rounding != 1) return GDN_ERR_INVALID_ARG;
  const size_t ga = s->gate == GDN_GATE_KEY ? 16 : 4;
  if (!aligned(write_pos, 4) || !aligned(slot_idx, 4) || (err_flags && !aligned(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  for (int l = 0; l < n; ++l) {
    if (!ckpt[l] || !ring_d[l] || !ring_k[l] || !ring_g[l]) return GDN_ERR_INVALID_ARG;
    if (!aligned(ckpt[l], 16) || !aligned(ring_d[l], 16) || !aligned(ring_k[l], 16) ||
        !aligned(ring_g[l], ga))
      return GDN_ERR_INVALID_ARG;
  }
  if (n > 1) {
    // the launch writes every layer's checkpoint at once: they must not overlap
    const size_t bytes = static_cast<size_t>(s->N) * s->Hv * s->dv * s->dk *
                         elem_size(s->state_dtype);
    for (int l = 0; l < n; ++l)
      for (int m = l + 1; m < n; ++m) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(ckpt[l]);
        const uintptr_t y = reinterpret_cast<uintptr_t>(ckpt[m]);
        if ((x < y ? y - x : x - y) < bytes) return GDN_ERR_INVALID_ARG;
      }
  }
  if (s->B == 0) return GDN_OK;
  FoldArgs a{};
  a.slot = slot_idx;
  a.write_pos = write_pos; a.err = err_flags;
  a.B = s->B; a.N = s->N; a.Hv = s->Hv; a.Hk = s->Hk; a.dv = s->dv; a.L = s->L;
  a.G = s->Hv / s->Hk;
  a.step_round = s->step_rounding;
  // value rows per workgroup: 64 (or the largest of 32, 16 dividing dv), so
  // that the ring entries staged in LDS serve several rows per thread
  a.fv = s->dv % 64 == 0 ? 64 : (s->dv % 32 == 0 ? 32 : 16);
  const dim3 block(static_cast<unsigned>(16 * s->dk / 4));
  // LDS: the ring's keys [L][dk], d [L][fv] and decays ([L], or [L][dk] per key)
  const size_t n_al = s->gate == GDN_GATE_KEY ? static_cast<size_t>(s->dk) : 1;
  const size_t smem = static_cast<size_t>(s->L) * (n_al + a.fv + s->dk) * sizeof(float);
  if (smem > 160 * 1024) return GDN_ERR_UNSUPPORTED;
  for (int l0 = 0; l0 < n; l0 += kFoldMaxLayers) {
    const int nl = std::min(n - l0, kFoldMaxLayers);
    for (int i = 0; i < kFoldMaxLayers; ++i) {
      const int l = l0 + (i < nl ? i : 0);
      a.ckpt[i] = ckpt[l]; a.ring_d[i] = ring_d[l]; a.ring_k[i] = ring_k[l]; a.ring_g[i] = ring_g[l];
    }
    const dim3 grid(static_cast<unsigned>(s->B) * s->Hv * (s->dv / a.fv), static_cast<unsigned>(nl));
    const gdn_status r = from_hip(dispatch_fold(s->dk, a, s->ring_dtype, s->state_dtype, s->gate,
                                                grid, block, smem,
                                                static_cast<hipStream_t>(stream)));
    if (r != GDN_OK) return r;
  }
  return GDN_OK;
}

}  // namespace

gdn_status gdn_replay_fold(const gdn_shape* s, const int32_t* slot_idx, void* ckpt,
                           const void* ring_d, const void* ring_k, const float* ring_g,
                           const int32_t* write_pos, int32_t* err_flags, void* stream) {
  return fold_layers(s, 1, slot_idx, &ckpt, &ring_d, &ring_k, &ring_g, write_pos, err_flags,
                     stream);
}

gdn_status gdn_replay_fold_layers(const gdn_shape* s, int32_t n_layers, const int32_t* slot_idx,
                                  void* const* ckpt, const void* const* ring_d,
                                  const void* const* ring_k, const float* const* ring_g,
                                  const int32_t* write_pos, int32_t* err_flags, void* stream) {
  if (n_layers < 1 || n_layers > GDN_FOLD_MAX_LAYERS || !ckpt || !ring_d || !ring_k || !ring_g)
    return GDN_ERR_INVALID_ARG;
  return fold_layers(s, n_layers, slot_idx, ckpt, ring_d, ring_k, ring_g, write_pos, err_flags,
                     stream);
}

gdn_status gdn_replay_reset(const gdn_shape* s, const int32_t* slot_idx, int32_t* write_pos,
                            int32_t* err_flags, void* stream) {
  if (!s || s->B < 0 || s->N < 1) return GDN_ERR_INVALID_ARG;
  if (!slot_idx || !write_pos) return GDN_ERR_INVALID_ARG;
  if (!aligned(slot_idx, 4) || !aligned(write_pos, 4) || (err_flags && !aligned(err_flags, 4)))
    return GDN_ERR_INVALID_ARG;
  if (s->B == 0) return GDN_OK;
  CursorArgs c{};
  c.slot = slot_idx; c.write_pos = write_pos; c.err = err_flags;
  c.B = s->B; c.N = s->N; c.L = s->L; c.T = s->T;
  return from_hip(launch_reset(c, static_cast<hipStream_t>(stream)));
}

const char* gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case GDN_ERR_HIP: return "HIP launch error";
    case GDN_ERR_SCRATCH_LIMIT:
      return "more rows than the static scratch holds (GDN_SCRATCH_MAX_ROWS)";
  }
  return "unknown status";
}

int32_t gdn_abi_version(void) { return kAbiVersion; }

}  // extern "C"
