// gdn_kernels.h -- the gfx950 kernels of the GDN decode path (templates).
//
// Workgroup = (row b, key head hk, value block vb). It holds the G = Hv/Hk
// value heads that share key head hk, and VB value rows of each of them; one
// wavefront per 16 value rows of one head. Everything a row needs from the
// key side (q, k, the key ring) is staged once per workgroup in LDS and shared
// by the G heads, so the key ring is read once per key head, as the ring
// layout intends (ReplaySSM blog, section 2.2: same-group value heads share
// the key entries).
#pragma once

#include "gdn_device.h"

namespace gdn {

// Zero the outputs of one wavefront's rows for every token of a row that is
// padding (negative slot) or in error.
template <int QKV>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, int b, int h, int vcol,
                                          int grp) {
  if (grp != 0) return;
  for (int tau = 0; tau < a.T; ++tau) {
    const size_t ih = (static_cast<size_t>(b) * a.T + tau) * a.Hv + h;
    store1<QKV>(a.o, ih * a.dv + vcol, 0.f);
  }
}

// Stage the row's q and k for all T tokens into LDS as fp32:
// lds[tau][0][:] = q, lds[tau][1][:] = k.
template <int DK, int QKV>
__device__ __forceinline__ void stage_qk(const DecodeArgs& a, float* lds, int b, int hk) {
  constexpr int C4 = DK / 4;
  const int total = a.T * C4;
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    const int tau = c / C4, e4 = (c % C4) * 4;
    const size_t src = ((static_cast<size_t>(b) * a.T + tau) * a.Hk + hk) * DK + e4;
    const f4 qv = load4<QKV>(a.q, src);
    const f4 kv = load4<QKV>(a.k, src);
    *reinterpret_cast<f4*>(lds + (tau * 2 + 0) * DK + e4) = qv;
    *reinterpret_cast<f4*>(lds + (tau * 2 + 1) * DK + e4) = kv;
  }
}

// ============================================================= packed decode
//
// The plain read-update-write step (SGLang PR #28451: the packed decode that
// reads the state, updates it and writes it back every step).
template <int DK, int QKV>
__global__ __launch_bounds__(1024) void packed_decode_kernel(DecodeArgs a) {
  constexpr int NT = DK / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  float* qk = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int vb = blk % a.nvb;
  blk /= a.nvb;
  const int hk = blk % a.Hk;
  const int b = blk / a.Hk;
  const int wph = a.VB / 16;
  const int h = hk * a.G + wave / wph;
  const int vcol = vb * a.VB + (wave % wph) * 16 + col;

  const int s = a.slot[b];
  if (s < 0 || s >= a.N) {
    if (s >= a.N && threadIdx.x == 0 && a.err) atomicOr(a.err, EF_SLOT);
    zero_rows<QKV>(a, b, h, vcol, grp);
    return;
  }

  float* st = a.state + ((static_cast<size_t>(s) * a.Hv + h) * a.dv + vcol) * DK + 4 * grp;
  f4 S[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) S[t] = *reinterpret_cast<const f4*>(st + 16 * t);

  const size_t ih = static_cast<size_t>(b) * a.Hv + h;
  const float vv = load1<QKV>(a.v, ih * a.dv + vcol);
  const float gv = a.g[ih], bt = a.beta[ih];
  stage_qk<DK, QKV>(a, qk, b, hk);
  __syncthreads();

  float sq, sk, kq, d, o;
  slab_dots<NT>(S, qk, qk + DK, grp, sq, sk, kq);
  const float alpha = decay_of(gv);
  token_out(sq, sk, kq, alpha, bt, vv, d, o);
  if (grp == 0) store1<QKV>(a.o, ih * a.dv + vcol, o);
  slab_update<NT>(S, qk + DK, grp, alpha, d);
#pragma unroll
  for (int t = 0; t < NT; ++t) *reinterpret_cast<f4*>(st + 16 * t) = S[t];
}

// ============================================================= replay decode
//
// ReplaySSM output-only decode (window == 0, T == 1) and verify window
// (window == 1). See gdn_replay.h for the contract.
//
// Steps per workgroup:
//   1. resolve the row: slot, p = write_pos[slot], flush flag;
//   2. load the checkpoint slab into registers (16-byte loads, issued early);
//   3. stage q/k of the T tokens and the key ring (positions < p, zero beyond)
//      into LDS, the key ring transposed to [key][entry] for the MFMA A operand;
//   4. per wavefront: suffix-sum the ring's log-decays with a wave scan,
//      A = exp(sum g), w_j = exp(sum_{i>j} g_i); build the B operand
//      w_j * d_j[v] in the ring dtype;
//   5. S = A * S0 (in registers), then S += K^T (w o D) on the MFMA units,
//      one 16x16 tile per 16 keys, accumulated in place;
//   6. per token: Sq, Sk, k^T q -> d, o; store o; append the ring entry
//      (non-flush) or update the slab on chip (window tokens, flush);
//   7. on a flush, write the updated slab to the checkpoint.
template <int RING> struct RingMfma;

template <> struct RingMfma<DT_F16> {
  static constexpr int CH = 16;  // ring entries per MFMA k-step (16x16x16)
  using op_t = h4;
  __device__ static f4 mma(op_t a, op_t b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};
template <> struct RingMfma<DT_BF16> {
  static constexpr int CH = 16;
  using op_t = s4;
  __device__ static f4 mma(op_t a, op_t b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};
template <> struct RingMfma<DT_F32> {
  static constexpr int CH = 4;   // 16x16x4 fp32
  using op_t = float;
  __device__ static f4 mma(op_t a, op_t b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <int DK, int QKV, int RING>
__global__ __launch_bounds__(1024) void replay_decode_kernel(DecodeArgs a) {
  constexpr int NT = DK / 16;
  constexpr int C4 = DK / 4;
  using RT = typename Elem<RING>::T;
  using MM = RingMfma<RING>;
  constexpr int CH = MM::CH;
  constexpr bool RF32 = (RING == DT_F32);

  extern __shared__ __align__(16) unsigned char smem[];
  float* qk = reinterpret_cast<float*>(smem);
  RT* kt = reinterpret_cast<RT*>(smem + static_cast<size_t>(a.T) * 2 * DK * sizeof(float));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int vb = blk % a.nvb;
  blk /= a.nvb;
  const int hk = blk % a.Hk;
  const int b = blk / a.Hk;
  const int wph = a.VB / 16;
  const int h = hk * a.G + wave / wph;
  const int vcol = vb * a.VB + (wave % wph) * 16 + col;

  // ---- 1. row resolve
  const int s = a.slot[b];
  if (s < 0 || s >= a.N) {
    if (s >= a.N && threadIdx.x == 0 && a.err) atomicOr(a.err, EF_SLOT);
    zero_rows<QKV>(a, b, h, vcol, grp);
    return;
  }
  const int p = a.write_pos[s];
  const int ef = a.window ? ((p < 0 || p + a.T > a.L) ? EF_WINDOW : 0)
                          : ((p < 0 || p > a.L - 1) ? EF_CURSOR : 0);
  if (ef) {
    if (threadIdx.x == 0 && a.err) atomicOr(a.err, ef);
    zero_rows<QKV>(a, b, h, vcol, grp);
    return;
  }
  const bool flush = !a.window &&
                     (p == a.L - 1 || (a.force_flush != nullptr && a.force_flush[b] != 0));
  const int nch = (p + CH - 1) / CH;   // MFMA k-steps over the valid entries
  const int lp = nch * CH;             // entries covered, zero-padded beyond p

  const size_t hs = static_cast<size_t>(s) * a.Hv + h;            // (slot, head)
  const size_t ks = static_cast<size_t>(s) * a.Hk + hk;           // (slot, k-head)

  // ---- per-lane ring decay input (lane j < p holds g_j)
  const float gj = (lane < p) ? a.ring_g[hs * a.L + lane] : 0.f;

  // ---- 2. checkpoint slab
  const float* ck = a.state + (hs * a.dv + vcol) * DK + 4 * grp;
  f4 S[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) S[t] = *reinterpret_cast<const f4*>(ck + 16 * t);

  // ---- 3. LDS staging: q/k of the window, the key ring
  stage_qk<DK, QKV>(a, qk, b, hk);
  {
    const int total = p * C4;
    const RT* src = static_cast<const RT*>(a.ring_k) + ks * a.L * DK;
    for (int c = threadIdx.x; c < total; c += blockDim.x) {
      const int j = c / C4, e4 = (c % C4) * 4;
      if constexpr (RF32) {
        *reinterpret_cast<f4*>(kt + j * DK + e4) =
            *reinterpret_cast<const f4*>(src + static_cast<size_t>(j) * DK + e4);
      } else {
        const u16x4 r = *reinterpret_cast<const u16x4*>(src + static_cast<size_t>(j) * DK + e4);
        uint16_t* kt16 = reinterpret_cast<uint16_t*>(kt);
        kt16[(e4 + 0) * a.kts + j] = r.x;
        kt16[(e4 + 1) * a.kts + j] = r.y;
        kt16[(e4 + 2) * a.kts + j] = r.z;
        kt16[(e4 + 3) * a.kts + j] = r.w;
      }
    }
    const int pad = lp - p;   // zero the entries between p and the k-step edge
    for (int c = threadIdx.x; c < pad * DK; c += blockDim.x) {
      const int j = p + c / DK, key = c % DK;
      if constexpr (RF32) kt[j * DK + key] = 0.f;
      else reinterpret_cast<uint16_t*>(kt)[key * a.kts + j] = 0;
    }
  }
  __syncthreads();

  // ---- 4./5. reconstruction S = A S0 + sum_j w_j d_j k_j^T
  if (p > 0) {
    // Lanes >= p hold g = 0, so W_p = 0 exactly and lane p-1 reads
    // W_{j+1} = 0 from its neighbour (p <= 63, so lane 63 never needs it).
    const float W = wave_suffix_sum(gj, lane);          // W_j = sum_{i>=j} g_i
    const float Wn = __shfl_down(W, 1, 64);             // W_{j+1}
    const float wj = (lane < p) ? expf(Wn) : 0.f;       // w_j = exp(W_{j+1})
    const float A = expf(__shfl(W, 0, 64));             // A = exp(W_0)
#pragma unroll
    for (int t = 0; t < NT; ++t) S[t] *= A;
    const RT* dsrc = static_cast<const RT*>(a.ring_d) + hs * a.L * a.dv + vcol;
    for (int c = 0; c < nch; ++c) {
      typename MM::op_t bop;
      if constexpr (RF32) {
        const int j = c * CH + grp;
        const float w = __shfl(wj, j, 64);
        bop = (j < p) ? w * dsrc[static_cast<size_t>(j) * a.dv] : 0.f;
      } else {
        u16x4 bb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = c * CH + 4 * grp + i;
          const float w = __shfl(wj, j & 63, 64);
          const float x = (j < p) ? w * to_f32<RING>(dsrc[static_cast<size_t>(j) * a.dv]) : 0.f;
          bb[i] = __builtin_bit_cast(uint16_t, from_f32<RING>(x));
        }
        bop = __builtin_bit_cast(typename MM::op_t, bb);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        typename MM::op_t aop;
        if constexpr (RF32) {
          aop = kt[(c * CH + grp) * DK + 16 * t + col];
        } else {
          aop = *reinterpret_cast<const typename MM::op_t*>(
              kt + (16 * t + col) * a.kts + c * CH + 4 * grp);
        }
        S[t] = MM::mma(aop, bop, S[t]);
      }
    }
  }

  // ---- 6. tokens
  const bool kwriter = (vb == 0) && (wave == 0);        // one key-ring writer per k-head
  const bool gwriter = (vb == 0) && (wave % wph == 0) && lane == 0;
  for (int tau = 0; tau < a.T; ++tau) {
    const float* ql = qk + tau * 2 * DK;
    const float* kl = ql + DK;
    const size_t ih = (static_cast<size_t>(b) * a.T + tau) * a.Hv + h;
    const float vv = load1<QKV>(a.v, ih * a.dv + vcol);
    const float gv = a.g[ih], bt = a.beta[ih];
    float sq, sk, kq, d, o;
    slab_dots<NT>(S, ql, kl, grp, sq, sk, kq);
    const float alpha = decay_of(gv);
    token_out(sq, sk, kq, alpha, bt, vv, d, o);
    if (grp == 0) store1<QKV>(a.o, ih * a.dv + vcol, o);
    if (!flush) {
      const int pos = p + tau;
      if (grp == 0)
        store1<RING>(a.ring_d, (hs * a.L + pos) * a.dv + vcol, d);
      if (gwriter) a.ring_g[hs * a.L + pos] = gv;
      if (kwriter && lane < C4) {
        const f4 kv = *reinterpret_cast<const f4*>(kl + 4 * lane);
        store4<RING>(a.ring_k, (ks * a.L + pos) * DK + 4 * lane, kv);
      }
    }
    if (flush || (a.window && tau + 1 < a.T)) slab_update<NT>(S, kl, grp, alpha, d);
  }

  // ---- 7. flush: the updated slab becomes the checkpoint
  if (flush) {
    float* cw = a.state + (hs * a.dv + vcol) * DK + 4 * grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f4*>(cw + 16 * t) = S[t];
  }
}

// ============================================================= fold
//
// Fold the valid ring entries into the checkpoint with the pinned two-step
// rounding (SGLang PR #42388 "The idea"; SGLang PR #36821 fold). Workgroup =
// (row, value head, 16 value rows); thread = one 16-byte group of 4 keys.
template <int DK, int RING>
__global__ __launch_bounds__(1024) void fold_kernel(FoldArgs a) {
  constexpr int C4 = DK / 4;
  constexpr int FV = 16;
  using RT = typename Elem<RING>::T;
  extern __shared__ __align__(16) unsigned char smem[];
  float* kl = reinterpret_cast<float*>(smem);        // [L][DK]  key entries (16-byte rows)
  float* dl = kl + a.L * DK;                          // [L][FV]  d entries
  float* al = dl + a.L * FV;                          // [L]      decays

  const int nvb = a.dv / FV;
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int vb = blk % nvb;
  blk /= nvb;
  const int h = blk % a.Hv;
  const int b = blk / a.Hv;
  const int s = a.slot[b];
  if (s < 0) return;
  if (s >= a.N) {
    if (threadIdx.x == 0 && a.err) atomicOr(a.err, EF_SLOT);
    return;
  }
  const int p = a.write_pos[s];
  if (p < 0 || p > a.L) {
    if (threadIdx.x == 0 && a.err) atomicOr(a.err, EF_CURSOR);
    return;
  }
  if (p == 0) return;
  const int hk = h / a.G;
  const size_t hs = static_cast<size_t>(s) * a.Hv + h;
  const size_t ks = static_cast<size_t>(s) * a.Hk + hk;
  const int tid = threadIdx.x;
  const int row = tid / C4, e4 = (tid % C4) * 4;
  const int v = vb * FV + row;

  float* xp = a.ckpt + (hs * a.dv + v) * DK + e4;
  f4 x = *reinterpret_cast<const f4*>(xp);

  if (tid < p) al[tid] = decay_of(a.ring_g[hs * a.L + tid]);
  for (int c = tid; c < p * FV; c += blockDim.x) {
    const int j = c / FV, r = c % FV;
    dl[c] = to_f32<RING>(static_cast<const RT*>(a.ring_d)[(hs * a.L + j) * a.dv + vb * FV + r]);
  }
  for (int c = tid; c < p * C4; c += blockDim.x) {
    const int j = c / C4, q4 = (c % C4) * 4;
    const RT* src = static_cast<const RT*>(a.ring_k) + (ks * a.L + j) * DK + q4;
    f4 kv;
    kv.x = to_f32<RING>(src[0]); kv.y = to_f32<RING>(src[1]);
    kv.z = to_f32<RING>(src[2]); kv.w = to_f32<RING>(src[3]);
    *reinterpret_cast<f4*>(kl + j * DK + q4) = kv;
  }
  __syncthreads();

  {
#pragma clang fp contract(off)
    for (int j = 0; j < p; ++j) {
      const float aj = al[j];
      const float dj = dl[j * FV + row];
      const f4 kv = *reinterpret_cast<const f4*>(kl + j * DK + e4);
      const float tx = aj * x.x, ty = aj * x.y, tz = aj * x.z, tw = aj * x.w;
      x.x = __builtin_fmaf(dj, kv.x, tx);
      x.y = __builtin_fmaf(dj, kv.y, ty);
      x.z = __builtin_fmaf(dj, kv.z, tz);
      x.w = __builtin_fmaf(dj, kv.w, tw);
    }
  }
  *reinterpret_cast<f4*>(xp) = x;
}

}  // namespace gdn
