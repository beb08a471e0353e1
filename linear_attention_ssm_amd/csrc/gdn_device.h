// gdn_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Tile layout used by every decode kernel. A wavefront owns 16 consecutive
// value rows v0..v0+15 of one value head and all dk key columns. Lane l holds
// column group g = l / 16 and value row v = v0 + l % 16, and for every key
// tile t (16 keys) the four consecutive keys 16t + 4g .. 16t + 4g + 3:
//     S[t] = state[v][16t + 4g .. 16t + 4g + 3]          (one 16-byte load)
// This is exactly the accumulator layout of the 16x16 MFMA when the product is
// computed transposed (rows = keys, columns = value rows), so the checkpoint
// tile is loaded straight into the accumulator registers.
//
// The readout (Sq, Sk, k^T q, the correction d and the output o) and the
// two-instruction state update live here so that the packed decode and the
// ring-replay decode execute the same operations in the same order; with an
// empty ring the two kernels therefore produce identical bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum : int { EF_SLOT = 1, EF_CURSOR = 2, EF_WINDOW = 4, EF_ACCEPTED = 8 };

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; };
template <> struct Elem<DT_BF16> { using T = uint16_t; };
template <> struct Elem<DT_F16> { using T = _Float16; };

template <int DT>
__device__ __forceinline__ float to_f32(typename Elem<DT>::T x) {
  if constexpr (DT == DT_F32) return x;
  else if constexpr (DT == DT_BF16) return bf16_to_f32(x);
  else return static_cast<float>(x);
}

template <int DT>
__device__ __forceinline__ typename Elem<DT>::T from_f32(float x) {
  if constexpr (DT == DT_F32) return x;
  else if constexpr (DT == DT_BF16) return f32_to_bf16(x);
  else return static_cast<_Float16>(x);
}

// Four consecutive elements starting at element `idx` (a multiple of 4) of a
// 16-byte aligned array, widened to fp32.
template <int DT>
__device__ __forceinline__ f4 load4(const void* base, size_t idx) {
  if constexpr (DT == DT_F32) {
    return *reinterpret_cast<const f4*>(static_cast<const float*>(base) + idx);
  } else {
    const u16x4 r = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + idx);
    f4 out;
    if constexpr (DT == DT_BF16) {
      out.x = bf16_to_f32(r.x); out.y = bf16_to_f32(r.y);
      out.z = bf16_to_f32(r.z); out.w = bf16_to_f32(r.w);
    } else {
      out.x = static_cast<float>(__builtin_bit_cast(_Float16, r.x));
      out.y = static_cast<float>(__builtin_bit_cast(_Float16, r.y));
      out.z = static_cast<float>(__builtin_bit_cast(_Float16, r.z));
      out.w = static_cast<float>(__builtin_bit_cast(_Float16, r.w));
    }
    return out;
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  return to_f32<DT>(static_cast<const typename Elem<DT>::T*>(base)[idx]);
}

template <int DT>
__device__ __forceinline__ void store1(void* base, size_t idx, float x) {
  static_cast<typename Elem<DT>::T*>(base)[idx] = from_f32<DT>(x);
}

// Four fp32 values written as four consecutive elements (idx multiple of 4).
template <int DT>
__device__ __forceinline__ void store4(void* base, size_t idx, f4 x) {
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<f4*>(static_cast<float*>(base) + idx) = x;
  } else {
    u16x4 r;
    r.x = __builtin_bit_cast(uint16_t, from_f32<DT>(x.x));
    r.y = __builtin_bit_cast(uint16_t, from_f32<DT>(x.y));
    r.z = __builtin_bit_cast(uint16_t, from_f32<DT>(x.z));
    r.w = __builtin_bit_cast(uint16_t, from_f32<DT>(x.w));
    *reinterpret_cast<u16x4*>(static_cast<uint16_t*>(base) + idx) = r;
  }
}

// ------------------------------------------------------------- launch mapping

// Workgroups are handed to the 8 XCDs round-robin by workgroup id. Remap the
// id so that each XCD receives one contiguous range of logical blocks: the
// blocks that share a row's key ring and q/k then meet in the same L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int X = 8;
  const int xcd = i % X, local = i / X, per = n / X, rem = n % X;
  return xcd < rem ? xcd * (per + 1) + local
                   : rem * (per + 1) + (xcd - rem) * per + local;
}

// ------------------------------------------------------------- wave reductions

// Sum over the four column groups (lanes l, l^16, l^32, l^48). Every lane of
// the quartet ends with the same bits (IEEE addition commutes exactly).
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Inclusive suffix sum over the 64 lanes: lane j receives sum_{i >= j} x_i.
__device__ __forceinline__ float wave_suffix_sum(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_down(x, off, 64);
    if (lane + off < 64) x += y;
  }
  return x;
}

// ------------------------------------------------------------- readout

// Per-lane partial dot products of the 16-row slab with q and k, and of k
// with q, reduced over the four column groups. q_l / k_l point at fp32 copies
// of the token's q and k in LDS.
template <int NT>
__device__ __forceinline__ void slab_dots(const f4 (&S)[NT], const float* q_l,
                                          const float* k_l, int grp, float& sq,
                                          float& sk, float& kq) {
  float pq = 0.f, pk = 0.f, pkq = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f4 qv = *reinterpret_cast<const f4*>(q_l + 16 * t + 4 * grp);
    const f4 kv = *reinterpret_cast<const f4*>(k_l + 16 * t + 4 * grp);
    pq = __builtin_fmaf(S[t].x, qv.x, pq);
    pq = __builtin_fmaf(S[t].y, qv.y, pq);
    pq = __builtin_fmaf(S[t].z, qv.z, pq);
    pq = __builtin_fmaf(S[t].w, qv.w, pq);
    pk = __builtin_fmaf(S[t].x, kv.x, pk);
    pk = __builtin_fmaf(S[t].y, kv.y, pk);
    pk = __builtin_fmaf(S[t].z, kv.z, pk);
    pk = __builtin_fmaf(S[t].w, kv.w, pk);
    pkq = __builtin_fmaf(kv.x, qv.x, pkq);
    pkq = __builtin_fmaf(kv.y, qv.y, pkq);
    pkq = __builtin_fmaf(kv.z, qv.z, pkq);
    pkq = __builtin_fmaf(kv.w, qv.w, pkq);
  }
  sq = quad_sum(pq);
  sk = quad_sum(pk);
  kq = quad_sum(pkq);
}

// alpha = exp(g) evaluated in double and rounded once to fp32: the same value
// the checkpoint fold uses for a ring entry's decay.
__device__ __forceinline__ float decay_of(float g) {
  return static_cast<float>(exp(static_cast<double>(g)));
}

// Output-only readout of one token (GDN math of SGLang PR #28451):
//   d = beta (v - alpha Sk),   o = alpha Sq + d (k^T q).
__device__ __forceinline__ void token_out(float sq, float sk, float kq,
                                          float alpha, float beta, float v,
                                          float& d, float& o) {
#pragma clang fp contract(off)
  const float sqa = alpha * sq;
  const float ska = alpha * sk;
  d = beta * (v - ska);
  o = __builtin_fmaf(d, kq, sqa);
}

// State update S <- alpha S + d k^T with the two-instruction rounding
// fma(d, k, RN(alpha * S)) (SGLang PR #42388, "The idea").
template <int NT>
__device__ __forceinline__ void slab_update(f4 (&S)[NT], const float* k_l, int grp,
                                            float alpha, float d) {
#pragma clang fp contract(off)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f4 kv = *reinterpret_cast<const f4*>(k_l + 16 * t + 4 * grp);
    const float ax = alpha * S[t].x, ay = alpha * S[t].y;
    const float az = alpha * S[t].z, aw = alpha * S[t].w;
    S[t].x = __builtin_fmaf(d, kv.x, ax);
    S[t].y = __builtin_fmaf(d, kv.y, ay);
    S[t].z = __builtin_fmaf(d, kv.z, az);
    S[t].w = __builtin_fmaf(d, kv.w, aw);
  }
}

// ------------------------------------------------------------- kernel args

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* slot;
  float* state;            // packed: the state; replay: the checkpoint
  void* ring_d;
  void* ring_k;
  float* ring_g;
  const int32_t* write_pos;
  const uint8_t* force_flush;
  void* o;
  int32_t* err;
  int32_t B, T, N, Hv, Hk, dv, L;
  int32_t G;               // Hv / Hk
  int32_t VB;              // value rows per head per workgroup (multiple of 16)
  int32_t nvb;             // dv / VB
  int32_t window;          // 1: verify window (no flush, entries at p..p+T-1)
  int32_t kts;             // LDS row stride (elements) of the transposed key ring
};

struct CursorArgs {
  const int32_t* slot;
  const uint8_t* force_flush;
  const int32_t* accepted;
  int32_t* write_pos;
  int32_t* err;
  int32_t B, N, L, T;
};

struct FoldArgs {
  const int32_t* slot;
  float* ckpt;
  const void* ring_d;
  const void* ring_k;
  const float* ring_g;
  const int32_t* write_pos;
  int32_t* err;
  int32_t B, N, Hv, Hk, dv, L, G;
};

}  // namespace gdn
