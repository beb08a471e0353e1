// gdn_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Tile layout used by every decode kernel. A wavefront owns 16 consecutive
// value rows v0..v0+15 of one value head and all dk key columns. Lane l holds
// column group g = l / 16 and value row v = v0 + l % 16, and for every key
// tile t the four consecutive keys key_base(t, g) .. key_base(t, g) + 3 in the
// fp32 register S[t]. This is the accumulator layout of the 16x16 MFMA when
// the product is computed transposed (rows = keys, columns = value rows): row
// m of tile t stands for key key_base(t, m / 4) + m % 4, so the MFMA's key
// operand is read in that order and the state tile lands in the accumulator.
// The key order depends on the storage format of the state:
//   fp32 state:    key_base(t, g) = 16t + 4g       S[t] is one 16-byte load
//   16-bit state:  key_base(t, g) = 32(t/2) + 8g + 4(t%2)
//                  S[2u], S[2u+1] are the 8 consecutive keys 32u + 8g .. +7,
//                  one 16-byte load of eight 16-bit values
// so that every lane reads its part of a value row in 16-byte pieces.
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
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

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

// A state value rounded to its storage format, from the fp32 value as
// computed. The empty asm keeps the compiler from folding an fp32 FMA and this
// conversion into one mixed-precision FMA that rounds straight to fp16, which
// would round the exact product-sum instead of its fp32 value.
template <int DT>
__device__ __forceinline__ typename Elem<DT>::T state_round(float x) {
  if constexpr (DT == DT_F16) asm("" : "+v"(x));
  return from_f32<DT>(x);
}

// A 16-bit element's bits as its storage type. The element arrives as a
// scalar parameter: applying __builtin_bit_cast to a vector element
// expression (v.y) directly reads element 0 with this compiler.
template <int DT>
__device__ __forceinline__ typename Elem<DT>::T from_bits(uint16_t e) {
  return __builtin_bit_cast(typename Elem<DT>::T, e);
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
    out.x = to_f32<DT>(from_bits<DT>(r[0]));
    out.y = to_f32<DT>(from_bits<DT>(r[1]));
    out.z = to_f32<DT>(from_bits<DT>(r[2]));
    out.w = to_f32<DT>(from_bits<DT>(r[3]));
    return out;
  }
}

// Raw (undecoded) loads: issue the memory access now, decode later, so the
// wait for the data lands at the first use rather than at the load.
template <int DT> struct Raw4 { using T = u16x4; };
template <> struct Raw4<DT_F32> { using T = f4; };

template <int DT>
__device__ __forceinline__ typename Raw4<DT>::T load4_raw(const void* base, size_t idx) {
  using R = typename Raw4<DT>::T;
  if constexpr (DT == DT_F32)
    return *reinterpret_cast<const R*>(static_cast<const float*>(base) + idx);
  else
    return *reinterpret_cast<const R*>(static_cast<const uint16_t*>(base) + idx);
}

template <int DT>
__device__ __forceinline__ f4 decode4(typename Raw4<DT>::T r) {
  if constexpr (DT == DT_F32) {
    return r;
  } else {
    f4 out;
    out.x = to_f32<DT>(from_bits<DT>(r[0]));
    out.y = to_f32<DT>(from_bits<DT>(r[1]));
    out.z = to_f32<DT>(from_bits<DT>(r[2]));
    out.w = to_f32<DT>(from_bits<DT>(r[3]));
    return out;
  }
}

template <int DT>
__device__ __forceinline__ typename Elem<DT>::T load1_raw(const void* base, size_t idx) {
  return static_cast<const typename Elem<DT>::T*>(base)[idx];
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

// Load of a wave-uniform value that no kernel writes while it runs (slot
// indices, cursors, flags, per-head gates): through the constant address
// space it becomes a scalar-cache load, counted on lgkmcnt, so waiting for
// it never waits for the vector loads (the state stream) issued before it.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, size_t i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

// ------------------------------------------------------------- launch mapping

// n / d for a wave-uniform n < 2^32 / d, given m = ceil(2^32 / d) (m = 0 for
// d = 1): with e = m d - 2^32 < d, n m / 2^32 = n / d + n e / (d 2^32) and the
// excess stays below 1/d, so the floor is exact (Granlund and Montgomery's
// division by invariant integers, in its round-up form).
__device__ __forceinline__ uint32_t udiv(uint32_t n, uint32_t m) {
  return m ? __umulhi(n, m) : n;
}

// Workgroups are handed to the 8 XCDs round-robin by workgroup id. The work
// items come in groups of gsz consecutive items that share a row's key side
// (q, k and the key ring of one key head). Map workgroup ids so that all items
// of a group run on one XCD (they meet in its L2) and consecutive groups go to
// different XCDs: the groups of one row, and with them the checkpoint writes
// of a flushing row, spread over all eight XCDs instead of piling up on one.
// The last n_groups % 8 groups keep the identity mapping.
__device__ __forceinline__ int item_of_block(int i, int n_items, int gsz) {
  constexpr int X = 8;
  const int full = (n_items / gsz) / X * X;
  if (i >= full * gsz) return i;
  const int x = i % X, k = i / X;
  return ((k / gsz) * X + x) * gsz + (k % gsz);
}

// ------------------------------------------------------------- wave reductions

// Sum over the four column groups (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap instructions: v_permlane16_swap hands each lane the lower
// and the upper row of its row pair, v_permlane32_swap the lower and upper
// half of the wave. Both partners add the two in the same order, so every
// lane of a quartet ends with identical bits.
__device__ __forceinline__ float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sum over aligned groups of C lanes (C a power of two, at most 64) by a
// butterfly: after each step a lane and its partner hold the same two
// operands, so every lane of the group ends with identical bits.
template <int C>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < C; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// A buffer resource over `nbytes` bytes at the wave-uniform `base`. Loads
// through it at offsets past nbytes return zero without touching memory
// (raw buffer bounds check), which is how reads are limited to the valid
// ring entries and how a masked row reads nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, 0x00020000);
}

// The memory unit copies 16 bytes per active lane into LDS, lane l's at
// lds + 16 l (lds wavefront-uniform). From a bounded buffer, bytes past its
// end arrive as zeros.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds,
                                                uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds), 16, voff, 0, 0, 0);
}

// x from lane l + n of the same 16-lane row (0 past the row end), by DPP.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf,
                                                    false));
}

// Inclusive suffix sum over the 64 lanes (lane j receives sum_{i >= j} x_i)
// and the exclusive one (lane j receives sum_{i > j} x_i). Within a 16-lane
// row: four DPP row shifts; across rows (only when entries live in more than
// one row, i.e. more than 16 of them): the row totals through scalar reads.
__device__ __forceinline__ void wave_suffix_sums(float x, int lane, bool multi_row, float& incl,
                                                 float& excl) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  if (multi_row) {
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    const int row = lane >> 4;
    const float after = row == 0 ? r1 + (r2 + r3) : row == 1 ? r2 + r3 : row == 2 ? r3 : 0.f;
    x += after;
    // the first lane of the next row now holds the sum of everything after
    // this row: the exclusive sum of a row's last lane
    const float n1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float n2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float n3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    const float nxt = row == 0 ? n1 : row == 1 ? n2 : row == 2 ? n3 : 0.f;
    incl = x;
    // one DPP move, all lanes active: lane l takes lane l+1 of its row; the
    // last lane of a row has no source in the row and keeps `nxt` (bound_ctrl
    // off). A select here could turn into a divergent branch, and a DPP read
    // from a lane switched off in EXEC does not see that lane's value.
    excl = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(nxt), __float_as_int(x),
                                                      0x101, 0xf, 0xf, false));
  } else {
    incl = x;
    excl = row_shl<1>(x);
  }
}

// ------------------------------------------------------------- state slab

// First of the four keys lane group `grp` holds in tile t (layout above).
template <int SD>
__device__ __forceinline__ int key_base(int t, int grp) {
  if constexpr (SD == DT_F32) return 16 * t + 4 * grp;
  else return 32 * (t >> 1) + 8 * grp + 4 * (t & 1);
}

// The key of MFMA tile row m (0..15) in tile t.
template <int SD>
__device__ __forceinline__ int key_of_row(int t, int m) {
  return key_base<SD>(t, m >> 2) + (m & 3);
}

// A wavefront's 16-row slab as loaded, before widening: NT 16-byte pieces of
// fp32 state, or NT/2 pieces of eight 16-bit values.
template <int SD, int DK> struct SlabRaw {
  static constexpr int NP = SD == DT_F32 ? DK / 16 : DK / 32;
  v4u r[NP];
};

// Request this lane's part of the slab whose row 0 starts at `slab` (rows DK
// elements apart): row col, 16-byte pieces in the key order of key_base.
template <int SD, int DK>
__device__ __forceinline__ void slab_load(SlabRaw<SD, DK>& R, const void* slab, int col, int grp) {
  if constexpr (SD == DT_F32) {
    const float* row = static_cast<const float*>(slab) + col * DK + 4 * grp;
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) R.r[t] = *reinterpret_cast<const v4u*>(row + 16 * t);
  } else {
    const uint16_t* row = static_cast<const uint16_t*>(slab) + col * DK + 8 * grp;
#pragma unroll
    for (int u = 0; u < DK / 32; ++u) R.r[u] = *reinterpret_cast<const v4u*>(row + 32 * u);
  }
}

// Widen a loaded slab to the fp32 tile registers (exact for 16-bit formats).
template <int SD, int DK>
__device__ __forceinline__ void slab_decode(f4 (&S)[DK / 16], const SlabRaw<SD, DK>& R) {
  if constexpr (SD == DT_F32) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) S[t] = __builtin_bit_cast(f4, R.r[t]);
  } else {
#pragma unroll
    for (int u = 0; u < DK / 32; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = R.r[u][i];   // keys 2i, 2i+1 of the piece
        const float lo = to_f32<SD>(from_bits<SD>(static_cast<uint16_t>(w & 0xffffu)));
        const float hi = to_f32<SD>(from_bits<SD>(static_cast<uint16_t>(w >> 16)));
        f4& dst = S[2 * u + (i >> 1)];
        dst[2 * (i & 1)] = lo;
        dst[2 * (i & 1) + 1] = hi;
      }
    }
  }
}

// ------------------------------------------------------------- readout

// Per-lane partial dot products of the 16-row slab with q and k, and of k
// with q, reduced over the four column groups. q_l / k_l point at fp32 copies
// of the token's q and k in LDS.
template <int SD, int NT>
__device__ __forceinline__ void slab_dots(const f4 (&S)[NT], const float* q_l,
                                          const float* k_l, int grp, float& sq, float& sk) {
  float pq = 0.f, pk = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f4 qv = *reinterpret_cast<const f4*>(q_l + key_base<SD>(t, grp));
    const f4 kv = *reinterpret_cast<const f4*>(k_l + key_base<SD>(t, grp));
    pq = __builtin_fmaf(S[t].x, qv.x, pq);
    pq = __builtin_fmaf(S[t].y, qv.y, pq);
    pq = __builtin_fmaf(S[t].z, qv.z, pq);
    pq = __builtin_fmaf(S[t].w, qv.w, pq);
    pk = __builtin_fmaf(S[t].x, kv.x, pk);
    pk = __builtin_fmaf(S[t].y, kv.y, pk);
    pk = __builtin_fmaf(S[t].z, kv.z, pk);
    pk = __builtin_fmaf(S[t].w, kv.w, pk);
  }
  sq = quad_sum(pq);
  sk = quad_sum(pk);
}

// k^T q of one token, from the staging threads' four-key pieces: each of the
// DK/4 threads that stage the token's q and k forms its partial product, and
// the group of DK/4 lanes sums them. Every kernel that reads a token out uses
// this one order, so the packed and the replay decode agree bit for bit.
template <int DK>
__device__ __forceinline__ float token_kq(f4 qv, f4 kv) {
  float x = qv.x * kv.x;
  x = __builtin_fmaf(qv.y, kv.y, x);
  x = __builtin_fmaf(qv.z, kv.z, x);
  x = __builtin_fmaf(qv.w, kv.w, x);
  return group_sum<DK / 4>(x);
}

// In-kernel q/k normalisation (the decode's front end: q and k L2-normalised
// per key head, q scaled by dk^-1/2; SGLang PR #28451, Modifications). Each of
// the DK/4 staging threads of a token holds four elements of q and of k; the
// group of DK/4 lanes sums the squares (one order, shared by every kernel).
// x <- x / sqrt(sum x^2 + 1e-6); q is then multiplied by dk^-1/2.
template <int DK>
__device__ __forceinline__ void token_l2norm(f4& qv, f4& kv) {
  float sq = qv.x * qv.x, sk = kv.x * kv.x;
  sq = __builtin_fmaf(qv.y, qv.y, sq);
  sk = __builtin_fmaf(kv.y, kv.y, sk);
  sq = __builtin_fmaf(qv.z, qv.z, sq);
  sk = __builtin_fmaf(kv.z, kv.z, sk);
  sq = __builtin_fmaf(qv.w, qv.w, sq);
  sk = __builtin_fmaf(kv.w, kv.w, sk);
  sq = group_sum<DK / 4>(sq);
  sk = group_sum<DK / 4>(sk);
  constexpr float kScale = DK == 32 ? 0.17677669529663688f : DK == 64 ? 0.125f
                         : DK == 128 ? 0.08838834764831845f : 0.0625f;   // dk^-1/2
  const float rq = kScale / __builtin_sqrtf(sq + 1e-6f);
  const float rk = 1.f / __builtin_sqrtf(sk + 1e-6f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qv[i] = qv[i] * rq;
    kv[i] = kv[i] * rk;
  }
}

// alpha = exp(g) of one step, evaluated in double and rounded once to fp32.
// Every kernel that applies a step's decay to a state (packed decode, the
// replay readout and flush, the verify window, the fold) uses this one value,
// so that replaying stored (d, k, g) entries with the two-instruction update
// reproduces a sequential decode bit for bit (SGLang PR #42388, "The idea":
// the rebuild must round exactly as the verify kernel does).
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
template <int SD, int NT>
__device__ __forceinline__ void slab_update(f4 (&S)[NT], const float* k_l, int grp,
                                            float alpha, float d) {
#pragma clang fp contract(off)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f4 kv = *reinterpret_cast<const f4*>(k_l + key_base<SD>(t, grp));
    const float ax = alpha * S[t].x, ay = alpha * S[t].y;
    const float az = alpha * S[t].z, aw = alpha * S[t].w;
    S[t].x = __builtin_fmaf(d, kv.x, ax);
    S[t].y = __builtin_fmaf(d, kv.y, ay);
    S[t].z = __builtin_fmaf(d, kv.z, az);
    S[t].w = __builtin_fmaf(d, kv.w, aw);
  }
}

// The same update with a per-key gate (KDA, SGLang PR #28451 Modifications
// item 7): S <- S Diag(a) + d k^T, rounded as fma(d, k[c], RN(a[c] * S[c])).
// a_l holds the token's decays a[c] = RN_f32(exp_f64(g[c])) in LDS.
template <int SD, int NT>
__device__ __forceinline__ void slab_update_key(f4 (&S)[NT], const float* k_l, const float* a_l,
                                                int grp, float d) {
#pragma clang fp contract(off)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f4 kv = *reinterpret_cast<const f4*>(k_l + key_base<SD>(t, grp));
    const f4 av = *reinterpret_cast<const f4*>(a_l + key_base<SD>(t, grp));
    const float ax = av.x * S[t].x, ay = av.y * S[t].y;
    const float az = av.z * S[t].z, aw = av.w * S[t].w;
    S[t].x = __builtin_fmaf(d, kv.x, ax);
    S[t].y = __builtin_fmaf(d, kv.y, ay);
    S[t].z = __builtin_fmaf(d, kv.z, az);
    S[t].w = __builtin_fmaf(d, kv.w, aw);
  }
}

// A token's per-key gate for one head, staged in LDS as four rows of dk
// floats: the decays a = RN_f32(exp_f64(g)), a o q, a o k, and g itself (for
// the ring). The readout then is Sq = S (a o q), Sk = S (a o k): the token's
// decay folds into q and k (SGLang PR #28451, Modifications item 7).
// Four channels c4*4 .. +3 of the row; q and k as fp32.
__device__ __forceinline__ void stage_key_gate(float* gl, int dk, int c4, f4 g4, f4 qv, f4 kv) {
  f4 al;
  al.x = decay_of(g4.x);
  al.y = decay_of(g4.y);
  al.z = decay_of(g4.z);
  al.w = decay_of(g4.w);
  f4 aq, ak;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aq[i] = al[i] * qv[i];
    ak[i] = al[i] * kv[i];
  }
  *reinterpret_cast<f4*>(gl + 4 * c4) = al;
  *reinterpret_cast<f4*>(gl + dk + 4 * c4) = aq;
  *reinterpret_cast<f4*>(gl + 2 * dk + 4 * c4) = ak;
  *reinterpret_cast<f4*>(gl + 3 * dk + 4 * c4) = g4;
}

// The value lane `i` (wave-uniform) holds, in every lane.
__device__ __forceinline__ float lane_value(float x, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}

// Lane i of each 16-lane row receives lane i^8's value (DPP row_ror:8).
__device__ __forceinline__ f4 row_swap8(f4 x) {
  f4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[i]), 0x128, 0xf, 0xf, false));
  return r;
}

// Cache-policy bits of the gfx950 buffer stores (sc0 = 1, nt = 2, sc1 = 16).
// Measured on MI355X, per kernel:
//   sc1 nt  the packed decode's state write-back: a line goes on to memory at
//           once instead of staying dirty in L2 until the state stream evicts
//           it between other reads (49.8 us per launch, 54-56 us otherwise);
//   sc1     the replay decode's flush, whose checkpoint loads are
//           non-temporal: 0.4 us faster per launch than sc1 nt.
constexpr int kCpolSc1Nt = 16 | 2;
constexpr int kCpolSc1 = 16;

// One 16-byte store with cache policy CP through a buffer resource over
// `nbytes` bytes at the wave-uniform `base`.
template <int CP>
__device__ __forceinline__ void store16(float* base, int nbytes, int byte_off, f4 x) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), rs, byte_off, 0, CP);
}

// A 16-bit state's on-chip values rounded to the format and widened back
// (the state a step-by-step decode would hold); fp32 is left as is.
template <int SD, int NT>
__device__ __forceinline__ void slab_round(f4 (&S)[NT]) {
  if constexpr (SD != DT_F32) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] = to_f32<SD>(state_round<SD>(S[t][i]));
  }
}

// The 8-byte form of store16.
template <int CP>
__device__ __forceinline__ void store8(float* base, int nbytes, int byte_off, u16x4 x) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, x), rs, byte_off, 0, CP);
}

// Store a wavefront's 16-row slab, rounded to the state format (round to
// nearest even), so that every store instruction writes whole 128-byte lines.
// Each lane holds NP 16-byte pieces of its row (fp32: tile t = keys 16t+4g..;
// 16-bit: piece u = keys 32u+8g..). Rows col and col^8 trade the odd pieces of
// each pair (DPP row_ror:8): one instruction then writes rows 0-7 and the next
// rows 8-15, each covering the pair's 2 x 64 bytes of all eight rows. A slab
// with one piece per lane (16-bit, dk = 32) is written piece by piece.
// `slab` is the wave-uniform address of row 0; rows are DK elements apart.
// The stores carry cache policy CP. Needs all 64 lanes active.
template <int SD, int DK, int CP>
__device__ __forceinline__ void store_slab(void* slab, const f4 (&S)[DK / 16], int col, int grp) {
  constexpr int ES = SD == DT_F32 ? 4 : 2;          // bytes per element
  constexpr int NP = SlabRaw<SD, DK>::NP;
  constexpr int KP = SD == DT_F32 ? 16 : 32;        // keys between pieces of a lane
  constexpr int KG = SD == DT_F32 ? 4 : 8;          // keys between lane groups
  constexpr int NB = 16 * DK * ES;
  float* base = static_cast<float*>(slab);
  f4 X[NP];
  if constexpr (SD == DT_F32) {
#pragma unroll
    for (int t = 0; t < NP; ++t) X[t] = S[t];
  } else {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      v4u w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f4& src = S[2 * u + (i >> 1)];
        const uint32_t lo = __builtin_bit_cast(uint16_t, state_round<SD>(src[2 * (i & 1)]));
        const uint32_t hi = __builtin_bit_cast(uint16_t, state_round<SD>(src[2 * (i & 1) + 1]));
        w[i] = lo | (hi << 16);
      }
      X[u] = __builtin_bit_cast(f4, w);
    }
  }
  if constexpr (NP == 1) {
    store16<CP>(base, NB, (col * DK + KG * grp) * ES, X[0]);
  } else {
    const bool lo = col < 8;
    const int r = col & 7;
    const int k0 = (lo ? 0 : KP) + KG * grp;
#pragma unroll
    for (int u = 0; u < NP / 2; ++u) {
      const f4 x0 = X[2 * u], x1 = X[2 * u + 1];
      const f4 z = row_swap8(lo ? x1 : x0);
      store16<CP>(base, NB, (r * DK + 2 * KP * u + k0) * ES, lo ? x0 : z);
      store16<CP>(base, NB, ((r + 8) * DK + 2 * KP * u + k0) * ES, lo ? z : x1);
    }
  }
}

// ------------------------------------------------------------- kernel args

// int32 elements between two rows' arrival counters (one 128-byte line each)
constexpr int kArriveStride = 32;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* slot;
  void* state;             // packed: the state; replay: the checkpoint (state dtype)
  void* ring_d;
  void* ring_k;
  float* ring_g;
  const int32_t* write_pos;
  const int32_t* force_flush;
  const int32_t* ff_flags;  // force_flush, or any readable [B] int32 when ff_on == 0
  int32_t ff_on;
  void* o;
  int32_t* err;
  int32_t B, T, N, Hv, Hk, dv, L;
  int32_t G;               // Hv / Hk
  int32_t GH;              // value heads per work item (divides G)
  int32_t nhc;             // G / GH head chunks per key head
  int32_t VB;              // value rows per head per work item (multiple of 16)
  int32_t nvb;             // dv / VB
  int32_t window;          // 1: verify window (no flush, entries at p..p+T-1)
  int32_t win_mfma;        // window read out in chunked form (see window_chunked)
  int32_t kts;             // LDS row stride (elements) of the transposed key ring
  int32_t dump_off;        // LDS byte offset of the [64][8] fp32 write sink
  // work-item mapping of the replay kernel without runtime divisions: the
  // divisors (items per key-side group, Hk, value blocks, waves per head) come
  // with their reciprocals m = ceil(2^32 / d) (0 for d = 1), see udiv()
  int32_t gsz, full_blocks;
  uint32_t m_gsz, m_hk, m_nvb, m_wph;
  // LDS byte offsets: per-token k^T q, per (head, token) gates (alpha, beta,
  // g), the staged key ring
  int32_t kq_off, gate_off, kt_off;
  int32_t v_off;           // LDS byte offset of the window's v values ([waves][16][16] floats)
  int32_t step_round;      // round a 16-bit state after each window token
  // per-key gate (KDA) only, LDS byte offsets: the staged gates of the
  // workgroup's heads and tokens ([GH][T][4][dk] floats, see stage_key_gate),
  // the weighted key rings of the heads (kw_head elements apart) and the
  // per-channel checkpoint decays A ([GH][dk] floats)
  int32_t kg_off, kw_off, acol_off, kw_head;
  // per-key gate, early copy (kdma = 1: ring depth <= 16 and one 32-channel
  // group of the workgroup's GH*dk channels per wavefront): before the
  // checkpoint slab is requested, each wavefront has the memory unit copy the
  // ring log-decays and keys of its channels into LDS (kraw_wave bytes per
  // wavefront from kraw_off) and the first piece of each thread's token gates
  // (16 bytes per lane from tg_off), so the weighting waits on no load issued
  // after the slab; g_bytes is the size of the token gates g
  int32_t kdma, kraw_off, kraw_wave, tg_off;
  uint32_t g_bytes;
  // cursor advance fused into a decode step (gdn_replay_decode_advance): the
  // workgroups of a row count themselves in arrive[b] once every wavefront of
  // theirs has read the cursor; the last one writes the advanced cursor
  int32_t* arrive;         // [B][kArriveStride] int32, zero between calls; null: no advance
  int32_t* write_pos_w;    // write_pos, writable (the same array)
  int32_t wg_per_row;      // workgroups per row
  // input rows: elements between the q (and k) of consecutive (row, token)
  // pairs, and between their v (Hk*dk and Hv*dv for dense tensors; the width
  // of the packed mixed_qkv row when q, k, v are views into it)
  int32_t qk_rs, v_rs;
  int32_t qk_norm;         // 1: L2-normalise q and k in the kernel, scale q
  // split readout of a single-token step with an fp32 checkpoint (process(),
  // "split readout"): enabled for workgroups of 4 wavefronts at dk = 128;
  // qh_off is the LDS byte offset of the token's q and k in the ring's
  // 16-bit format ([2][dk])
  int32_t split_ro, qh_off;
};

struct CursorArgs {
  const int32_t* slot;
  const int32_t* force_flush;
  const int32_t* accepted;
  int32_t* write_pos;
  int32_t* err;
  int32_t B, N, L, T;
};

// Layers one fold launch covers at most (grid.y; their buffers travel in the
// kernel arguments).
constexpr int kFoldMaxLayers = 16;

struct FoldArgs {
  const int32_t* slot;
  const int32_t* write_pos;
  int32_t* err;
  int32_t B, N, Hv, Hk, dv, L, G;
  int32_t step_round;      // round a 16-bit state after each folded entry
  int32_t fv;              // value rows per workgroup (16, 32 or 64, divides dv)
  // layer blockIdx.y: its checkpoint and ring (same shapes for every layer)
  void* ckpt[kFoldMaxLayers];
  const void* ring_d[kFoldMaxLayers];
  const void* ring_k[kFoldMaxLayers];
  const float* ring_g[kFoldMaxLayers];
};

}  // namespace gdn
