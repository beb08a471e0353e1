// gdn_kernels.h -- the gfx950 kernels of the GDN decode path (templates).
//
// Workgroup = (row b, key head hk, value block vb). It holds the G = Hv/Hk
// value heads that share key head hk (the replay kernel: a chunk of GH of
// them), and VB value rows of each; one wavefront per 16 value rows of one
// head. Everything a row needs from the key side (q, k, the key ring) is
// staged once per workgroup in LDS and shared by its heads, so the key ring
// is read once per key head and chunk, as the ring layout intends (ReplaySSM
// blog, section 2.2: same-group value heads share the key entries).
#pragma once

#include <type_traits>

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

// ============================================================= packed decode
//
// The plain read-update-write step (SGLang PR #28451: the packed decode that
// reads the state, updates it and writes it back every step). KG = 1 takes
// the per-key gate (KDA): g is [B, Hv, dk] and the decay is applied per key
// channel.
template <int DK, int QKV, int SD, int KG>
__global__ __launch_bounds__(1024) void packed_decode_kernel(DecodeArgs a) {
  constexpr int NT = DK / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  float* qk = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;
  int blk = item_of_block(blockIdx.x, gridDim.x, a.nvb);
  const int vb = blk % a.nvb;
  blk /= a.nvb;
  const int hk = blk % a.Hk;
  const int b = blk / a.Hk;
  const int wph = a.VB / 16;
  const int h = hk * a.G + wave / wph;
  const int vrow0 = vb * a.VB + (wave % wph) * 16;   // the wavefront's first value row
  const int vcol = vrow0 + col;

  const int s = ld_uniform(a.slot, b);
  if (s < 0 || s >= a.N) {
    if (s >= a.N && threadIdx.x == 0 && a.err) atomicOr(a.err, EF_SLOT);
    zero_rows<QKV>(a, b, h, vcol, grp);
    return;
  }

  // small loads first (raw, unconditional), then the state stream; the
  // q/k decode and LDS staging then overlap the state loads in flight
  constexpr int C4 = DK / 4;
  const int tid = threadIdx.x;
  const int cq = tid < C4 ? tid : C4 - 1;
  const size_t qsrc = static_cast<size_t>(b) * a.qk_rs + hk * DK + cq * 4;
  const auto q_raw = load4_raw<QKV>(a.q, qsrc);
  const auto k_raw = load4_raw<QKV>(a.k, qsrc);
  const size_t ih = static_cast<size_t>(b) * a.Hv + h;
  const auto v_raw = load1_raw<QKV>(a.v, static_cast<size_t>(b) * a.v_rs + h * a.dv + vcol);
  const float gv = KG ? 0.f : ld_uniform(a.g, ih), bt = ld_uniform(a.beta, ih);

  using SE = typename Elem<SD>::T;
  SE* st = static_cast<SE*>(a.state) + ((static_cast<size_t>(s) * a.Hv + h) * a.dv + vrow0) * DK;
  SlabRaw<SD, DK> R;
  slab_load<SD, DK>(R, st, col, grp);

  {
    // unconditional writes (surplus threads into the dump area) keep the
    // early q/k loads ahead of the state loads
    float* dump = reinterpret_cast<float*>(smem + a.dump_off);
    f4 qv = decode4<QKV>(q_raw), kv = decode4<QKV>(k_raw);
    if (a.qk_norm && wave == 0) token_l2norm<DK>(qv, kv);
    float* qdst = tid < C4 ? qk + 4 * tid : dump + lane * 8;
    float* kdst = tid < C4 ? qk + DK + 4 * tid : dump + lane * 8 + 4;
    *reinterpret_cast<f4*>(qdst) = qv;
    *reinterpret_cast<f4*>(kdst) = kv;
    if (wave == 0) {
      const float kq0 = token_kq<DK>(qv, kv);
      if (lane == 0) qk[2 * DK] = kq0;
    }
  }
  float* kgl = reinterpret_cast<float*>(smem + a.kg_off);   // KG: [G][4][DK]
  if constexpr (KG) {
    // the per-key gates of the workgroup's G heads (while the state is in
    // flight), from q and k as given, or (normalised in the kernel) from
    // their staged copies
    if (a.qk_norm) __syncthreads();
    for (int i = tid; i < a.G * C4; i += blockDim.x) {
      const int hh = i / C4, c4 = i - hh * C4;
      const f4 g4 = *reinterpret_cast<const f4*>(
          a.g + (static_cast<size_t>(b) * a.Hv + hk * a.G + hh) * DK + 4 * c4);
      f4 qv, kv;
      if (a.qk_norm) {
        qv = *reinterpret_cast<const f4*>(qk + 4 * c4);
        kv = *reinterpret_cast<const f4*>(qk + DK + 4 * c4);
      } else {
        const size_t qi = static_cast<size_t>(b) * a.qk_rs + hk * DK + 4 * c4;
        qv = load4<QKV>(a.q, qi);
        kv = load4<QKV>(a.k, qi);
      }
      stage_key_gate(kgl + hh * 4 * DK, DK, c4, g4, qv, kv);
    }
  }
  const float alpha = decay_of(gv);   // while the state is in flight
  __syncthreads();
  const float vv = to_f32<QKV>(v_raw);

  f4 S[NT];
  slab_decode<SD, DK>(S, R);
  float sq, sk, d, o;
  const float kq = qk[2 * DK];
  if constexpr (KG) {
    const float* gl = kgl + (h - hk * a.G) * 4 * DK;
    slab_dots<SD>(S, gl + DK, gl + 2 * DK, grp, sq, sk);
    token_out(sq, sk, kq, 1.f, bt, vv, d, o);
  } else {
    slab_dots<SD>(S, qk, qk + DK, grp, sq, sk);
    token_out(sq, sk, kq, alpha, bt, vv, d, o);
  }
  if (grp == 0) store1<QKV>(a.o, ih * a.dv + vcol, o);
  if constexpr (KG) slab_update_key<SD>(S, qk + DK, kgl + (h - hk * a.G) * 4 * DK, grp, d);
  else slab_update<SD>(S, qk + DK, grp, alpha, d);
  store_slab<SD, DK, kCpolSc1Nt>(st, S, col, grp);
}

// ============================================================= replay decode
//
// ReplaySSM output-only decode (window == 0, T == 1) and verify window
// (window == 1). See gdn_replay.h for the contract.
//
// One workgroup per work item (row, key head, head chunk, value block); one
// wavefront per 16 value rows of one head. Per item:
//   fetch:   the cursor and the flush flag (scalar loads), the gates, q/k,
//            one key-ring piece per thread, the wave's ring d entries and g,
//            v (ring reads bounded by the cursor through buffer resources),
//            then the 16-row checkpoint slab in 16-byte loads of whole lines;
//   process: stage q/k (normalised if asked) and the key ring (transposed to
//            [key][entry] for the MFMA A operand) in LDS; suffix-sum the
//            ring's log-decays with a wave scan, A = exp(sum g),
//            w_j = exp(sum_{i>j} g_i); S = A*S0 + K^T (w o D) on the MFMA
//            units; per token Sq, Sk, k^T q -> d, o; append the ring entry
//            (non-flush) or update the slab on chip (window tokens, flush)
//            and write it to the checkpoint on a flush. With the per-key
//            gate (KG) the decays are per channel and fold onto the keys
//            (weight_keys) instead of onto d; for rings of up to 16 entries
//            the memory unit copies the ring's log-decays and keys into LDS
//            ahead of the slab (fetch_key_gate, weight_keys_lds). With a
//            fused cursor advance the row's last workgroup writes the
//            advanced cursor. A single-token row with an fp32 checkpoint
//            that does not flush skips forming S: its Sq and Sk come from
//            S0 as loaded and from the ring products k_j . q, k_j . k on the
//            MFMA units (the split readout in process()).
// The small operands are requested before the slab: vector loads retire in
// issue order, so the staging and the MFMA operand build can proceed while
// the slab is still in flight.
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

// Where a work item sits, and which head / value row this lane holds in it.
struct ItemGeo {
  int b, hk, hc, vb, h;
  int vrow0;   // the wavefront's first value row (wave-uniform: slab base addresses)
  int vcol;    // this lane's value row
};

__device__ __forceinline__ ItemGeo item_geo(const DecodeArgs& a, int wave, int col) {
  // block -> (key-side group, item within the group): the blocks of a group
  // run on one XCD, consecutive groups on different XCDs (item_of_block)
  const uint32_t i = blockIdx.x;
  uint32_t grp_i, w;
  if (static_cast<int>(i) < a.full_blocks) {
    const uint32_t kk = i >> 3, q = udiv(kk, a.m_gsz);
    w = kk - q * a.gsz;
    grp_i = q * 8 + (i & 7);
  } else {
    grp_i = udiv(i, a.m_gsz);
    w = i - grp_i * a.gsz;
  }
  ItemGeo g;
  g.b = static_cast<int>(udiv(grp_i, a.m_hk));
  g.hk = static_cast<int>(grp_i) - g.b * a.Hk;
  g.hc = static_cast<int>(udiv(w, a.m_nvb));
  g.vb = static_cast<int>(w) - g.hc * a.nvb;
  const int wph = a.VB / 16;                    // wavefronts per head
  const int wh = static_cast<int>(udiv(static_cast<uint32_t>(wave), a.m_wph));
  g.h = g.hk * a.G + g.hc * a.GH + wh;
  g.vrow0 = g.vb * a.VB + (wave - wh * wph) * 16;
  g.vcol = g.vrow0 + col;
  return g;
}

// The small operands of one item, as raw (undecoded) registers.
template <int DK, int QKV, int RING>
struct Small {
  typename Raw4<QKV>::T q_raw, k_raw;   // staging threads: four keys of q and k
  v4u kr;                               // key-ring piece of this thread (see fetch_small)
  uint32_t g_raw;                       // ring g of entry `lane` (0 past the valid entries)
  uint32_t d_raw[4];                    // this lane's ring d entries (raw bits)
  float gate_g, gate_b;                 // wave 0, lane hh*T+t: g and beta of head hh, token t
  typename Elem<QKV>::T v_raw;          // single token: this lane's v
  typename Elem<QKV>::T vt_raw[4];      // window: v of tokens grp + 4i (i < 4) for this lane's row
};

// Where a row stands: its slot, its valid ring entries and whether it flushes.
// A padding row (negative slot), a slot beyond the pool and a cursor out of
// range all run masked: p = 0, zero output, no state or ring write.
struct RowState {
  int s, sc;          // slot, and the slot clamped into the pool
  int p;              // valid ring entries read (0 for a masked row)
  int ef;             // error bits of the row
  bool slot_ok, ok, flush;
};

__device__ __forceinline__ RowState row_state(const DecodeArgs& a, int b, int T, int slot) {
  RowState r;
  r.s = slot;
  r.slot_ok = r.s >= 0 && r.s < a.N;
  r.sc = r.slot_ok ? r.s : 0;
  const int p_raw = ld_uniform(a.write_pos, r.sc);
  const int ff = ld_uniform(a.ff_flags, b);
  r.ef = r.s >= a.N ? EF_SLOT : 0;
  if (r.slot_ok)
    r.ef = a.window ? ((p_raw < 0 || p_raw + T > a.L) ? EF_WINDOW : 0)
                    : ((p_raw < 0 || p_raw > a.L - 1) ? EF_CURSOR : 0);
  r.ok = r.slot_ok && r.ef == 0;
  r.p = r.ok ? p_raw : 0;
  // bitwise, not short-circuit: no branch holds the flag load back
  r.flush = r.ok & (a.window == 0) & ((p_raw == a.L - 1) | ((a.ff_on != 0) & (ff != 0)));
  return r;
}

// Request an item's small operands. The ring reads go through buffer
// resources sized to the valid entries, so that entries at or past p read as
// zero without a memory access (they are also the MFMA's zero padding). All
// loads are unconditional (surplus lanes read a clamped address) so that they
// issue before the slab.
// Request an item's token operands: they depend on the row and head only,
// not on the slot or the cursor, so they are issued before the row's slot and
// cursor are known and their latency overlaps that scalar chain.
template <int DK, int QKV, int RING, int TT, int KG>
__device__ __forceinline__ void fetch_tokens(Small<DK, QKV, RING>& f, const DecodeArgs& a,
                                             const ItemGeo& g, int T, int tid, int lane,
                                             int grp, int wave) {
  constexpr int C4 = DK / 4;
  // wave 0: the gates of the workgroup's GH heads, lane hh*T + t
  if (wave == 0) {
    const int ng = a.GH * T;
    const int l = lane < ng ? lane : 0;
    const int hh = TT ? l : l / T, t = TT ? 0 : l - hh * T;
    const size_t gi = (static_cast<size_t>(g.b) * T + t) * a.Hv + g.hk * a.G + g.hc * a.GH + hh;
    f.gate_g = KG ? 0.f : a.g[gi];     // a per-key gate is staged in process()
    f.gate_b = a.beta[gi];
  }
  // staging threads: four keys of q and k of token c / C4 (only the
  // wavefronts that hold staging threads load them)
  const int nqk = T * C4;
  if (64 * wave < nqk) {
    const int cq = tid < nqk ? tid : nqk - 1;
    const int tq = TT ? 0 : cq / C4;
    const size_t qsrc = (static_cast<size_t>(g.b) * T + tq) * a.qk_rs + g.hk * DK + (cq - tq * C4) * 4;
    f.q_raw = load4_raw<QKV>(a.q, qsrc);
    f.k_raw = load4_raw<QKV>(a.k, qsrc);
  }
  if constexpr (TT) {
    f.v_raw = load1_raw<QKV>(a.v, static_cast<size_t>(g.b) * a.v_rs + g.h * a.dv + g.vcol);
  } else {
    // every window token's v: the token loop then reads them from LDS
    // instead of waiting for a load per token (tokens past T read the last
    // one; T <= 16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = grp + 4 * i < T ? grp + 4 * i : T - 1;
      f.vt_raw[i] = load1_raw<QKV>(a.v, (static_cast<size_t>(g.b) * T + t) * a.v_rs + g.h * a.dv + g.vcol);
    }
  }
}

template <int DK, int QKV, int RING, int TT, int KG>
__device__ __forceinline__ void fetch_small(Small<DK, QKV, RING>& f, const DecodeArgs& a,
                                            const ItemGeo& g, const RowState& r, int T,
                                            int tid, int lane, int grp, int wave) {
  constexpr int C4 = DK / 4;
  constexpr bool RF32 = (RING == DT_F32);
  constexpr int RS = RF32 ? 4 : 2;
  // the key ring of (slot, key head), the valid entries only
  const char* kbase = static_cast<const char*>(a.ring_k) +
                      (static_cast<size_t>(r.sc) * a.Hk + g.hk) * a.L * DK * RS;
  const __amdgpu_buffer_rsrc_t rk = brsrc(kbase, static_cast<uint32_t>(r.p) * DK * RS);
  if constexpr (KG) {
    f.kr = v4u{0u, 0u, 0u, 0u};   // the per-key path weights the keys in process()
  } else if constexpr (RF32) {
    f.kr = __builtin_amdgcn_raw_buffer_load_b128(rk, tid * 16, 0, 0);   // chunk tid
  } else {
    // keys 8kg + 2sub, +1 of entries 4eg .. 4eg+3
    const int pr = tid >> 2, sub = tid & 3;
    const int eg = pr / (DK / 8), kg = pr % (DK / 8);
    const int off = (4 * eg * DK + kg * 8 + 2 * sub) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.kr[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, off + i * DK * 2, 0, 0);
  }
  const size_t hs = static_cast<size_t>(r.sc) * a.Hv + g.h;
  if constexpr (KG) {
    f.g_raw = 0u;
  } else {
    const __amdgpu_buffer_rsrc_t rg = brsrc(a.ring_g + hs * a.L, static_cast<uint32_t>(r.p) * 4);
    f.g_raw = __builtin_amdgcn_raw_buffer_load_b32(rg, lane * 4, 0, 0);
  }
  // this lane's ring d entries: 16-bit rings j = 4*grp + i (one 16x16x16
  // k-step), fp32 rings j = 4*i + grp (four 16x16x4 k-steps)
  const char* dbase = static_cast<const char*>(a.ring_d) + hs * a.L * a.dv * RS;
  const __amdgpu_buffer_rsrc_t rd = brsrc(dbase, static_cast<uint32_t>(r.p) * a.dv * RS);
  if constexpr (RF32) {
    const int off = (grp * a.dv + g.vcol) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.d_raw[i] = __builtin_amdgcn_raw_buffer_load_b32(rd, off, 16 * i * a.dv, 0);
  } else {
    const int off = (4 * grp * a.dv + g.vcol) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.d_raw[i] = __builtin_amdgcn_raw_buffer_load_b16(rd, off, 2 * i * a.dv, 0);
  }
}

// Per-key gate, early copy (a.kdma != 0). Each wavefront has the memory unit
// copy the ring log-decays and keys of its 32 channels, ring entries 0..15,
// into LDS as [16 entries][32 channels] (zeros past the valid entries), and
// each gate-staging thread its first 16 bytes of token gates. Issued before
// the slab, these arrive with the other small operands, so weight_keys_lds
// and the gate staging do not wait for loads queued behind the slab.
template <int DK, int RING>
__device__ __forceinline__ void fetch_key_gate(const DecodeArgs& a, const ItemGeo& g,
                                               const RowState& r, int T, unsigned char* buf,
                                               int tid, int lane, int wave) {
  constexpr bool RF32 = (RING == DT_F32);
  constexpr int RS = RF32 ? 4 : 2;
  const uint32_t p = static_cast<uint32_t>(r.p);
  const char* kbase = static_cast<const char*>(a.ring_k) +
                      (static_cast<size_t>(r.sc) * a.Hk + g.hk) * a.L * DK * RS;
  const __amdgpu_buffer_rsrc_t rk = brsrc(kbase, p * DK * RS);
  unsigned char* d = buf + a.kraw_off + wave * a.kraw_wave;
  const int e8 = lane >> 3, q8 = 4 * (lane & 7);   // entry and channel offset of 16-byte pieces
  const int ch = wave * 32;
  const int hh = ch / DK, c0 = ch % DK;
  const size_t hsh = static_cast<size_t>(r.sc) * a.Hv + g.hk * a.G + g.hc * a.GH + hh;
  const __amdgpu_buffer_rsrc_t rg = brsrc(a.ring_g + hsh * a.L * DK, p * DK * 4);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    buffer_to_lds16(rg, d + 1024 * i, ((8 * i + e8) * DK + c0 + q8) * 4);
  if constexpr (RF32) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      buffer_to_lds16(rk, d + 2048 + 1024 * i, ((8 * i + e8) * DK + c0 + q8) * 4);
  } else {
    buffer_to_lds16(rk, d + 2048, ((lane >> 2) * DK + c0 + 8 * (lane & 3)) * 2);
  }
  // token gates: thread tid stages piece i = tid (head hh, token tau, four
  // channels from 4 c4)
  constexpr int C4 = DK / 4;
  const int nqk = T * C4;
  // (a buffer copy: lanes past the last piece read at the end of g, out of
  // range, and copy zeros, so the copy needs no lane condition)
  if (64 * wave < a.GH * nqk) {
    const int hh = tid / nqk, c = tid - hh * nqk;
    const int tau = c / C4, c4 = c - tau * C4;
    const uint32_t gi = ((static_cast<uint32_t>(g.b) * T + tau) * a.Hv + g.hk * a.G + g.hc * a.GH + hh) * DK;
    const __amdgpu_buffer_rsrc_t rt = brsrc(a.g, a.g_bytes);
    buffer_to_lds16(rt, buf + a.tg_off + wave * 1024,
                    tid < a.GH * nqk ? (gi + 4 * c4) * 4 : a.g_bytes);
  }
}

// The checkpoint slab is read once per launch and not again before the next
// layer's launches have streamed through the caches: its loads carry the
// non-temporal policy (nt), which streams them past the caches' normal
// allocation. Measured on MI355X: a plain read of 128 MiB in this pattern takes
// 20.0 us with it and 21.3 us without, and the replay decode 26.3 us instead of
// 29.1 us. (The packed decode, which writes every line it reads, gets slower
// with it and keeps the default policy.)
constexpr int kSlabLoadPolicy = 2;   // nt

// Request an item's 16-row checkpoint slab: 16-byte loads in the lane order
// of the accumulator layout (widened to fp32 in process()). A masked row
// reads nothing (zeros).
template <int SD, int DK>
__device__ __forceinline__ void fetch_slab(SlabRaw<SD, DK>& R, const DecodeArgs& a,
                                           const ItemGeo& g, const RowState& r, int col, int grp) {
  constexpr int ES = SD == DT_F32 ? 4 : 2;
  const size_t hs = static_cast<size_t>(r.sc) * a.Hv + g.h;
  const char* base = static_cast<const char*>(a.state) + (hs * a.dv + g.vrow0) * DK * ES;
  const __amdgpu_buffer_rsrc_t rs = brsrc(base, r.ok ? 16 * DK * ES : 0);
  if constexpr (SD == DT_F32) {
    // whole 128-byte lines per instruction: rows 0-7 then rows 8-15 of keys
    // 32u..32u+31; slab_decode trades the halves back
    const bool lo = col < 8;
    const int off = ((lo ? col : col - 8) * DK + (lo ? 0 : 16) + 4 * grp) * 4;
#pragma unroll
    for (int u = 0; u < DK / 32; ++u) {
      R.r[2 * u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 128 * u, 0, kSlabLoadPolicy);
      R.r[2 * u + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 128 * u, 8 * DK * 4,
                                                             kSlabLoadPolicy);
    }
  } else {
    const int off = (col * DK + 8 * grp) * ES;
#pragma unroll
    for (int t = 0; t < SlabRaw<SD, DK>::NP; ++t)
      R.r[t] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * t, 0, kSlabLoadPolicy);
  }
}

// A token's small outputs leave in as few store instructions as possible (a
// store at the end of a wavefront costs about as much as a large one): lanes
// of group 0 write o, lanes of group 1 the ring d entry, two lanes of group 2
// the ring g entry (as two halves when the others are 16-bit), all in one
// instruction when o and d have the same width.
//   oi, di, gi: element indices into o, ring_d, ring_g
template <int QKV, int RING>
__device__ __forceinline__ void small_stores(const DecodeArgs& a, size_t oi, size_t di, size_t gi,
                                             float o, float d, float gv, bool app, bool gw,
                                             int grp, int col) {
  using OT = typename Elem<QKV>::T;
  using DT = typename Elem<RING>::T;
  if constexpr (sizeof(OT) == sizeof(DT)) {
    using W = std::conditional_t<sizeof(OT) == 2, uint16_t, uint32_t>;
    W* dst = nullptr;
    W val = 0;
    if (grp == 0) {
      dst = reinterpret_cast<W*>(static_cast<OT*>(a.o) + oi);
      val = __builtin_bit_cast(W, from_f32<QKV>(o));
    } else if (grp == 1) {
      dst = app ? reinterpret_cast<W*>(static_cast<DT*>(a.ring_d) + di) : nullptr;
      val = __builtin_bit_cast(W, from_f32<RING>(d));
    } else if (grp == 2) {
      const uint32_t gb = __float_as_uint(gv);
      if constexpr (sizeof(W) == 2) {
        dst = (app && gw && col < 2) ? reinterpret_cast<W*>(a.ring_g + gi) + col : nullptr;
        val = static_cast<W>(col ? gb >> 16 : gb & 0xffffu);
      } else {
        dst = (app && gw && col == 0) ? reinterpret_cast<W*>(a.ring_g + gi) : nullptr;
        val = gb;
      }
    }
    if (dst) *dst = val;
  } else {
    // o, and ring d with ring g, in two instructions
    if (grp == 0) store1<QKV>(a.o, oi, o);
    using W = std::conditional_t<sizeof(DT) == 2, uint16_t, uint32_t>;
    W* dst = nullptr;
    W val = 0;
    if (grp == 1) {
      dst = app ? reinterpret_cast<W*>(static_cast<DT*>(a.ring_d) + di) : nullptr;
      val = __builtin_bit_cast(W, from_f32<RING>(d));
    } else if (grp == 2) {
      const uint32_t gb = __float_as_uint(gv);
      if constexpr (sizeof(W) == 2) {
        dst = (app && gw && col < 2) ? reinterpret_cast<W*>(a.ring_g + gi) + col : nullptr;
        val = static_cast<W>(col ? gb >> 16 : gb & 0xffffu);
      } else {
        dst = (app && gw && col == 0) ? reinterpret_cast<W*>(a.ring_g + gi) : nullptr;
        val = gb;
      }
    }
    if (dst) *dst = val;
  }
}

// The per-key gate (KDA) part of the reconstruction for the workgroup's GH
// heads: per head and key channel c, A[c] = exp(sum_{j<p} g_j[c]) and the
// MFMA key operand w_j[c] k_j[c] with w_j[c] = exp(sum_{j<i<p} g_i[c]): the
// decay products fold onto the stored keys instead of onto d (SGLang PR
// #28451, Modifications item 7). One thread per (head, key channel) runs the
// channel's suffix sums from the newest entry down (spreading the channels
// over every thread of the workgroup: one thread per four channels left three
// quarters of the workgroup waiting on the first wavefront). Entries at or
// past p read as g = 0, k = 0 through the bounded loads, so the padded tail of
// the last k-step comes out as zeros. The operand lands in the layout of the
// scalar gate's staged key ring: [key][entry] (row stride kts) for 16-bit
// rings, [entry][key] for fp32.
template <int DK, int RING>
__device__ __forceinline__ void weight_keys(const DecodeArgs& a, const ItemGeo& g,
                                            const RowState& r, int lp, unsigned char* buf,
                                            int tid, int nthr) {
  using RT = typename Elem<RING>::T;
  constexpr bool RF32 = (RING == DT_F32);
  constexpr int RS = RF32 ? 4 : 2;
  const int p = r.p;
  const char* kbase = static_cast<const char*>(a.ring_k) +
                      (static_cast<size_t>(r.sc) * a.Hk + g.hk) * a.L * DK * RS;
  const __amdgpu_buffer_rsrc_t rk = brsrc(kbase, static_cast<uint32_t>(p) * DK * RS);
  float* acol = reinterpret_cast<float*>(buf + a.acol_off);
  for (int i = tid; i < a.GH * DK; i += nthr) {
    const int hh = i / DK, c = i - hh * DK;
    const size_t hsh = static_cast<size_t>(r.sc) * a.Hv + g.hk * a.G + g.hc * a.GH + hh;
    const __amdgpu_buffer_rsrc_t rg =
        brsrc(a.ring_g + hsh * a.L * DK, static_cast<uint32_t>(p) * DK * 4);
    RT* kw = reinterpret_cast<RT*>(buf + a.kw_off) + hh * a.kw_head;
    float W = 0.f;                             // sum of g_i[c] over the entries after j
    for (int eg = lp / 4 - 1; eg >= 0; --eg) {
      float gq[4], kv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * eg + e;
        gq[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (j * DK + c) * 4, 0, 0));
        if constexpr (RF32)
          kv[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, (j * DK + c) * 4, 0, 0));
        else
          kv[e] = to_f32<RING>(from_bits<RING>(static_cast<uint16_t>(
              __builtin_amdgcn_raw_buffer_load_b16(rk, (j * DK + c) * 2, 0, 0))));
      }
      uint16_t o16[4];
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const float kwv = __expf(W) * kv[e];
        if constexpr (RF32) kw[(4 * eg + e) * DK + c] = kwv;
        else o16[e] = __builtin_bit_cast(uint16_t, from_f32<RING>(kwv));
        W += gq[e];
      }
      if constexpr (!RF32) {
        uint2 pk;
        pk.x = static_cast<uint32_t>(o16[0]) | (static_cast<uint32_t>(o16[1]) << 16);
        pk.y = static_cast<uint32_t>(o16[2]) | (static_cast<uint32_t>(o16[3]) << 16);
        *reinterpret_cast<uint2*>(kw + c * a.kts + 4 * eg) = pk;
      }
    }
    acol[hh * DK + c] = __expf(W);
  }
}

// weight_keys from the early copy (a.kdma != 0, entries 0..15): two lanes
// per channel, lanes 32..63 take entries 15..8 and lanes 0..31 entries 7..0.
// The lower half starts its running sum from the upper half's total, so every
// W and weight is the same float as in weight_keys' sequential sum.
// NSLAB: the vector loads of the slab, the only ones issued after the copy.
template <int DK, int RING, int NSLAB>
__device__ __forceinline__ void weight_keys_lds(const DecodeArgs& a, int lp, unsigned char* buf,
                                                int lane, int wave) {
  using RT = typename Elem<RING>::T;
  constexpr bool RF32 = (RING == DT_F32);
  // The compiler does not order LDS reads after a copy into LDS by the
  // memory unit: wait here until at most the NSLAB slab loads (issued after
  // the copy, in order) are outstanding, so the copy has landed. Encoding:
  // vmcnt in bits 3:0 and 15:14, expcnt (7) and lgkmcnt (15) left open.
  static_assert(NSLAB < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((NSLAB & 15) | (7 << 4) | (15 << 8) | ((NSLAB >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  const int cl = lane & 31, e0 = (lane >> 5) ? 8 : 0;
  float* acol = reinterpret_cast<float*>(buf + a.acol_off);
  const unsigned char* w = buf + a.kraw_off + wave * a.kraw_wave;
  {
    const int ch = wave * 32 + cl;
    const int hh = ch / DK, c = ch % DK;
    const float* gr = reinterpret_cast<const float*>(w);
    const RT* kr = reinterpret_cast<const RT*>(w + 2048);
    float gv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = gr[(e0 + e) * 32 + cl];
    float t = 0.f;                                 // the upper half's total
#pragma unroll
    for (int e = 7; e >= 0; --e) t += gv[e];
    // every lane takes part in the exchange (a shuffle under a lane condition
    // would leave the source lanes' totals uncomputed)
    const float tu = __shfl(t, cl + 32, 64);
    float W = e0 ? 0.f : tu;
    float kwv[8];
#pragma unroll
    for (int e = 7; e >= 0; --e) {
      kwv[e] = __expf(W) * to_f32<RING>(kr[(e0 + e) * 32 + cl]);
      W += gv[e];
    }
    RT* kw = reinterpret_cast<RT*>(buf + a.kw_off) + hh * a.kw_head;
    if constexpr (RF32) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e0 + e < lp) kw[(e0 + e) * DK + c] = kwv[e];
    } else if (e0 < lp) {                          // lp is 16 here (0 for an empty ring)
      uint2 pk[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pk[h].x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<RING>(kwv[4 * h]))) |
                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<RING>(kwv[4 * h + 1]))) << 16);
        pk[h].y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<RING>(kwv[4 * h + 2]))) |
                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<RING>(kwv[4 * h + 3]))) << 16);
      }
      *reinterpret_cast<uint2*>(kw + c * a.kts + e0) = pk[0];
      *reinterpret_cast<uint2*>(kw + c * a.kts + e0 + 4) = pk[1];
    }
    if (e0 == 0) acol[hh * DK + c] = __expf(W);
  }
}

// Verify window in chunked form (a.win_mfma: 16-bit ring, 2 <= T <= 8, gate
// per head, no per-step rounding). The window's tokens are read out of the
// pre-window slab S_0 without updating it token by token: the recurrence
// S_{t+1} = alpha_t S_t + d_t k_t^T gives, for any vector x,
//     S_{t+1} x = alpha_t (S_t x) + d_t (k_t . x),
// so every S_t q_t and S_t k_t follows from the products S_0 q_m, S_0 k_m of
// all window tokens m and the window's inner products k_j . q_m, k_j . k_m
// (the causal mask over the window, vLLM PR #49887, Core concept). Both sets
// of products are dense contractions and run on the MFMA units: with the
// lane's A operand the window vector x_m (m = the lane's column; q_m for
// m < 8, k_{m-8} else), P = X^T S_0^T takes the slab registers as the B
// operand, and the Gram matrix X^T X the same operand twice. Each fp32
// operand is split into two bf16 parts, v = hi + lo with hi = RN_bf16(v) and
// lo = RN_bf16(v - hi) (|v - hi - lo| <= 2^-17 |v|), and a product takes the
// three terms hi.hi + hi.lo + lo.hi on the 16x16x32 bf16 MFMA (exact products,
// fp32 accumulation): a tenth of the matrix-unit time of 16x16x4 fp32
// products. XEX: the window vectors are bf16 values as given (bf16 q and k,
// not normalised in the kernel), so their low parts are zero: P takes two
// terms, the Gram matrix one, and the vectors need no split. The per-row recurrence over the T tokens then costs O(T^2) scalar
// operations instead of two passes over the 16 x dk slab per token. The
// results differ from the token-by-token update in rounding only (relative
// 1e-5 here, against the 2e-2 of a 16-bit ring).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// v = hi + lo, both bf16 (round to nearest even).
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

template <int DK, int QKV, int RING, int SD, bool XEX>
__device__ __forceinline__ void window_chunked(const DecodeArgs& a, const ItemGeo& g,
                                               const RowState& r, int T, const f4 (&S)[DK / 16],
                                               const float* qk, const float* vl, const float* gts,
                                               size_t hs, size_t ks, bool kwriter,
                                               bool gwriter_wave, int grp, int col, int lane) {
  constexpr int NT = DK / 16;
  constexpr int C4 = DK / 4;
  // this lane's window vector (vector slots past T read q_0; their rows of
  // the products are never used)
  const int tv = col & 7;
  const float* xv = qk + (tv < T ? tv : 0) * 2 * DK + (col >= 8 ? DK : 0);
  f4 P = {0.f, 0.f, 0.f, 0.f}, Gm = {0.f, 0.f, 0.f, 0.f};
  // k-step u covers keys 32u .. 32u + 31: the lane's eight keys are the four
  // of tile 2u and the four of tile 2u + 1 it holds (key_base), in the same
  // order for the A (window vectors) and the B (slab) operand
#pragma unroll
  for (int u = 0; u < NT / 2; ++u) {
    const f4 x0 = *reinterpret_cast<const f4*>(xv + key_base<SD>(2 * u, grp));
    const f4 x1 = *reinterpret_cast<const f4*>(xv + key_base<SD>(2 * u + 1, grp));
    bf16x8 xh, xl, sh, sl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __bf16 h, l;
      if constexpr (XEX) {
        xh[j] = static_cast<__bf16>(x0[j]);            // exact
        xh[4 + j] = static_cast<__bf16>(x1[j]);
      } else {
        split_bf16(x0[j], h, l); xh[j] = h; xl[j] = l;
        split_bf16(x1[j], h, l); xh[4 + j] = h; xl[4 + j] = l;
      }
      split_bf16(S[2 * u][j], h, l); sh[j] = h; sl[j] = l;
      split_bf16(S[2 * u + 1][j], h, l); sh[4 + j] = h; sl[4 + j] = l;
    }
    P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, sh, P, 0, 0, 0);
    P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, sl, P, 0, 0, 0);
    Gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, xh, Gm, 0, 0, 0);
    if constexpr (!XEX) {
      P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, sh, P, 0, 0, 0);
      Gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, xl, Gm, 0, 0, 0);
      Gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, xh, Gm, 0, 0, 0);
    }
  }
  // P: lane (row col, group grp) holds x_m . S_0[row] for m = 4 grp + i in
  // register i. Gather all 16 into every lane of the row: v_permlane16_swap
  // pairs groups (0,1) and (2,3), v_permlane32_swap the two halves.
  float pv[16];
  {
    float e[4], o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(P[i]), __float_as_uint(P[i]),
                                                      false, false);
      e[i] = __uint_as_float(w[0]);   // from the pair's even group
      o[i] = __uint_as_float(w[1]);   // from its odd group
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto we = __builtin_amdgcn_permlane32_swap(__float_as_uint(e[i]), __float_as_uint(e[i]),
                                                       false, false);
      const auto wo = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[i]), __float_as_uint(o[i]),
                                                       false, false);
      pv[i] = __uint_as_float(we[0]);        // group 0
      pv[8 + i] = __uint_as_float(we[1]);    // group 2
      pv[4 + i] = __uint_as_float(wo[0]);    // group 1
      pv[12 + i] = __uint_as_float(wo[1]);   // group 3
    }
  }
  // Gram entry (u, v) = x_u . x_v sits in lane v + 16 (u / 4), register u % 4
  auto gram = [&](int u, int v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gm[u & 3]), v + 16 * (u >> 2)));
  };
  float pq[8], pk[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    pq[m] = pv[m];
    pk[m] = pv[8 + m];
  }
  const bool app = r.ok;                       // a window never flushes
  // Store targets of token 0, stepped once per token: with a 16-bit o the
  // lane groups write o (group 0), the ring d entry (group 1) and the two
  // halves of the ring g entry (group 2) in one instruction.
  using OT = typename Elem<QKV>::T;
  constexpr bool ONE = sizeof(OT) == 2 && RING != DT_F32;   // 16-bit o and ring
  uint16_t* sdst = nullptr;
  size_t sstep = 0;
  bool son = false;
  if constexpr (ONE) {
    if (grp == 0) {
      sdst = static_cast<uint16_t*>(a.o) + (static_cast<size_t>(g.b) * T * a.Hv + g.h) * a.dv + g.vcol;
      sstep = static_cast<size_t>(a.Hv) * a.dv;
      son = true;
    } else if (grp == 1) {
      sdst = static_cast<uint16_t*>(const_cast<void*>(a.ring_d)) + (hs * a.L + r.p) * a.dv + g.vcol;
      sstep = a.dv;
      son = app;
    } else if (grp == 2) {
      sdst = reinterpret_cast<uint16_t*>(a.ring_g + hs * a.L + r.p) + col;
      sstep = 2;
      son = app && gwriter_wave && col < 2;
    }
  }
  size_t kidx = (ks * a.L + r.p) * DK + 4 * lane;
  const bool kon = app && kwriter && lane < C4;
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    if (tau < T) {
      const float* gt = gts + 3 * tau;
      const float alpha = gt[0], bt = gt[1], gv = gt[2];
      const float vv = vl[tau * 16 + col];
      float d, o;
      token_out(pq[tau], pk[tau], gram(8 + tau, tau), alpha, bt, vv, d, o);
      if constexpr (ONE) {
        // every candidate formed on every lane, then one select (no branch
        // per lane group)
        const uint32_t gb = __float_as_uint(gv);
        const uint16_t hv = static_cast<uint16_t>(col ? gb >> 16 : gb & 0xffffu);
        const uint16_t ob = __builtin_bit_cast(uint16_t, from_f32<QKV>(r.ok ? o : 0.f));
        const uint16_t db = __builtin_bit_cast(uint16_t, from_f32<RING>(d));
        const uint16_t val = grp == 0 ? ob : (grp == 1 ? db : hv);
        if (son) *sdst = val;
        sdst += sstep;
      } else {
        const size_t ih = (static_cast<size_t>(g.b) * T + tau) * a.Hv + g.h;
        const int pos = r.p + tau;
        small_stores<QKV, RING>(a, ih * a.dv + g.vcol, (hs * a.L + pos) * a.dv + g.vcol,
                                hs * a.L + pos, r.ok ? o : 0.f, d, gv, app, gwriter_wave, grp, col);
      }
      if (kon) {
        const f4 kv = *reinterpret_cast<const f4*>(qk + tau * 2 * DK + DK + 4 * lane);
        store4<RING>(a.ring_k, kidx, kv);
      }
      kidx += DK;
      // the later tokens' products after this token's update
#pragma unroll
      for (int m = tau + 1; m < 8; ++m) {
        if (m < T) {
          pq[m] = __builtin_fmaf(d, gram(8 + tau, m), alpha * pq[m]);
          pk[m] = __builtin_fmaf(d, gram(8 + tau, 8 + m), alpha * pk[m]);
        }
      }
    }
  }
}

template <int DK, int QKV, int RING, int SD, int TT, int KG, int NRM>
__device__ __forceinline__ void process(const DecodeArgs& a, const ItemGeo& g, const RowState& r,
                                        int T, const Small<DK, QKV, RING>& f,
                                        const SlabRaw<SD, DK>& R, unsigned char* buf, float* dump,
                                        int tid, int lane, int grp, int col, int wave) {
  constexpr int NT = DK / 16;
  constexpr int C4 = DK / 4;
  using RT = typename Elem<RING>::T;
  using MM = RingMfma<RING>;
  constexpr int CH = MM::CH;
  constexpr bool RF32 = (RING == DT_F32);
  constexpr int RS = RF32 ? 4 : 2;
  const int nthr = blockDim.x;
  float* qk = reinterpret_cast<float*>(buf);                      // [T][2][DK]
  float* kq_l = reinterpret_cast<float*>(buf + a.kq_off);         // [T]
  float* gates = reinterpret_cast<float*>(buf + a.gate_off);      // [GH*T][alpha, beta, g]
  RT* kt = reinterpret_cast<RT*>(buf + a.kt_off);                 // staged key ring
  if (r.ef && tid == 0 && a.err) atomicOr(a.err, r.ef);
  const int p = r.p;
  const int nch = (p + CH - 1) / CH;   // MFMA k-steps over the valid entries
  const int lp = nch * CH;             // entries covered, zero-padded beyond p
  const int nqk = T * C4;
  // the split readout (a single-token row with 1..16 valid entries that
  // does not flush): see below
  constexpr bool SPLIT = TT && !KG && RING != DT_F32 && SD == DT_F32 && DK == 128;
  constexpr int KNS = DK + 4;          // LDS row stride (elements) of the ring keys in row order
  bool split = false;
  if constexpr (SPLIT) split = a.split_ro && !r.flush && p > 0 && p <= 16;

  // ---- LDS staging. Every thread writes (threads past the last piece into a
  // per-lane dump area) so the early loads have unconditional uses.
  if (64 * wave < nqk) {                         // waves holding staging threads
    f4 qv = decode4<QKV>(f.q_raw), kv = decode4<QKV>(f.k_raw);
    if constexpr (NRM) token_l2norm<DK>(qv, kv);
    const int tq = TT ? 0 : tid / C4;
    float* qdst = tid < nqk ? qk + tq * 2 * DK + (tid - tq * C4) * 4 : dump + lane * 8;
    float* kdst = tid < nqk ? qdst + DK : dump + lane * 8 + 4;
    *reinterpret_cast<f4*>(qdst) = qv;
    *reinterpret_cast<f4*>(kdst) = kv;
    if constexpr (SPLIT) {
      // q and k in the ring's 16-bit format: the ring products' operand
      if (a.split_ro && tid < nqk) {
        uint16_t* xh = reinterpret_cast<uint16_t*>(buf + a.qh_off) + 4 * tid;
        u16x4 hq, hk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const typename Elem<RING>::T hqi = from_f32<RING>(qv[i]), hki = from_f32<RING>(kv[i]);
          hq[i] = __builtin_bit_cast(uint16_t, hqi);
          hk[i] = __builtin_bit_cast(uint16_t, hki);
        }
        *reinterpret_cast<u16x4*>(xh) = hq;
        *reinterpret_cast<u16x4*>(xh + DK) = hk;
      }
    }
    const float kq0 = token_kq<DK>(qv, kv);
    if (tid < nqk && tid - tq * C4 == 0) kq_l[tq] = kq0;
  }
  for (int c = tid + nthr; c < nqk; c += nthr) {        // long windows only
    const int tau = c / C4, e4 = (c % C4) * 4;
    const size_t src = (static_cast<size_t>(g.b) * T + tau) * a.qk_rs + g.hk * DK + e4;
    f4 qv = load4<QKV>(a.q, src), kv = load4<QKV>(a.k, src);
    if constexpr (NRM) token_l2norm<DK>(qv, kv);
    *reinterpret_cast<f4*>(qk + (tau * 2 + 0) * DK + e4) = qv;
    *reinterpret_cast<f4*>(qk + (tau * 2 + 1) * DK + e4) = kv;
    const float kq0 = token_kq<DK>(qv, kv);   // groups of C4 lanes stay aligned
    if (e4 == 0) kq_l[tau] = kq0;
  }
  // window: each wavefront's v values [T][16 rows] in LDS
  float* vl = reinterpret_cast<float*>(buf + a.v_off) + wave * 16 * 16;
  if constexpr (!TT) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (grp + 4 * i < T) vl[(grp + 4 * i) * 16 + col] = to_f32<QKV>(f.vt_raw[i]);
  }
  // gates of the workgroup's heads (wave 0): alpha = RN_f32(exp_f64(g))
  if (wave == 0) {
    const float al = decay_of(f.gate_g);
    if (lane < a.GH * T) {
      gates[3 * lane + 0] = al;
      gates[3 * lane + 1] = f.gate_b;
      gates[3 * lane + 2] = f.gate_g;
    }
  }
  float* kgl = reinterpret_cast<float*>(buf + a.kg_off);       // KG: [GH][T][4][DK]
  if constexpr (KG) {
    if (a.kdma) weight_keys_lds<DK, RING, SlabRaw<SD, DK>::NP>(a, lp, buf, lane, wave);
    else weight_keys<DK, RING>(a, g, r, lp, buf, tid, nthr);
    // per-key gates of the workgroup's heads for every token, from the staged
    // q and k (normalised in the kernel: once every wavefront has staged;
    // as given: a thread below nqk reads back its own staging, the others
    // load them); a thread's first piece of gates comes from the early copy
    if constexpr (NRM) __syncthreads();
    for (int i = tid; i < a.GH * nqk; i += nthr) {
      const int hh = i / nqk, c = i - hh * nqk;
      const int tau = TT ? 0 : c / C4, c4 = c - tau * C4;
      const size_t gi = ((static_cast<size_t>(g.b) * T + tau) * a.Hv + g.hk * a.G + g.hc * a.GH + hh) * DK;
      const f4 g4 = (a.kdma && i == tid)
                        ? *reinterpret_cast<const f4*>(buf + a.tg_off + wave * 1024 + lane * 16)
                        : *reinterpret_cast<const f4*>(a.g + gi + 4 * c4);
      f4 qv, kv;
      if (NRM || (i == tid && tid < nqk)) {
        qv = *reinterpret_cast<const f4*>(qk + tau * 2 * DK + 4 * c4);
        kv = *reinterpret_cast<const f4*>(qk + tau * 2 * DK + DK + 4 * c4);
      } else {
        const size_t qi = (static_cast<size_t>(g.b) * T + tau) * a.qk_rs + g.hk * DK + 4 * c4;
        qv = load4<QKV>(a.q, qi);
        kv = load4<QKV>(a.k, qi);
      }
      stage_key_gate(kgl + (hh * T + tau) * 4 * DK, DK, c4, g4, qv, kv);
    }
  }
  // the key ring, entries p..lp-1 as zeros (the bounded loads read them so)
  const char* kbase = static_cast<const char*>(a.ring_k) +
                      (static_cast<size_t>(r.sc) * a.Hk + g.hk) * a.L * DK * RS;
  const __amdgpu_buffer_rsrc_t rk = brsrc(kbase, static_cast<uint32_t>(p) * DK * RS);
  if constexpr (KG) {
    // staged by weight_keys
  } else if constexpr (RF32) {
    const int nkz = lp * (DK / 4);               // 16-byte chunks up to lp
    *reinterpret_cast<v4u*>(tid < nkz ? kt + tid * 4 : reinterpret_cast<RT*>(dump + lane * 8)) = f.kr;
    for (int c = tid + nthr; c < nkz; c += nthr)
      *reinterpret_cast<v4u*>(kt + c * 4) = __builtin_amdgcn_raw_buffer_load_b128(rk, c * 16, 0, 0);
  } else {
    // transposed [key][entry] (row stride kts): a thread writes two keys x four
    // entries as two 8-byte pieces
    constexpr int NKG = DK / 8;
    auto put_kt = [&](int pr, int sub, const v4u& v) {
      const int eg = pr / NKG, kg = pr % NKG;
      const bool in = 4 * eg < lp;
      uint2 a0, a1;
      a0.x = (v[0] & 0xffffu) | (v[1] << 16);
      a0.y = (v[2] & 0xffffu) | (v[3] << 16);
      a1.x = (v[0] >> 16) | (v[1] & 0xffff0000u);
      a1.y = (v[2] >> 16) | (v[3] & 0xffff0000u);
      uint16_t* kt16 = reinterpret_cast<uint16_t*>(kt);
      const int key = kg * 8 + 2 * sub;
      uint16_t* d16 = reinterpret_cast<uint16_t*>(dump + lane * 8);
      *reinterpret_cast<uint2*>(in ? kt16 + key * a.kts + 4 * eg : d16) = a0;
      *reinterpret_cast<uint2*>(in ? kt16 + (key + 1) * a.kts + 4 * eg : d16 + 4) = a1;
    };
    if (split) {
      // row order [entry][KNS] (4 workgroup wavefronts at dk = 128 hold all
      // 16 entries): a thread writes its two keys of each of its four entries
      const int pr = tid >> 2, sub = tid & 3;
      const int eg = pr / NKG, kg = pr % NKG;
      uint32_t* kn = reinterpret_cast<uint32_t*>(kt);
#pragma unroll
      for (int i = 0; i < 4; ++i) kn[((4 * eg + i) * KNS + kg * 8 + 2 * sub) >> 1] = f.kr[i];
    } else {
      put_kt(tid >> 2, tid & 3, f.kr);
      const int npr = (lp / 4) * NKG;                    // (entry group, key group) pairs
      for (int t2 = tid + nthr; t2 < 4 * npr; t2 += nthr) {   // deep rings / small workgroups
        const int pr = t2 >> 2, sub = t2 & 3;
        const int eg = pr / NKG, kg = pr % NKG;
        const int off = (4 * eg * DK + kg * 8 + 2 * sub) * 2;
        v4u v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, off + i * DK * 2, 0, 0);
        put_kt(pr, sub, v);
      }
    }
  }

  // ---- reconstruction weights, before the barrier: the suffix sums of the
  // log-decays W_j = sum_{i>=j} g_i, A = exp(W_0), w_j = exp(W_{j+1}), and the
  // MFMA operand w o D of the first k-steps (from the entries fetched early)
  constexpr int NPRE = RF32 ? 4 : 1;                  // k-steps covered by the fetch
  float A = 1.f, wj = 0.f;
  typename MM::op_t bops[NPRE];
  float wd[4] = {0.f, 0.f, 0.f, 0.f};   // split rows: w_j d_j of this lane's entries 4 grp + i
  auto bop_of = [&](int c, const float (&dval)[4]) {
    typename MM::op_t bop;
    if constexpr (KG) {
      // per-key gate: the weights sit on the keys, d enters as stored
      if constexpr (RF32) {
        bop = dval[0];
      } else {
        u16x4 bb;
#pragma unroll
        for (int i = 0; i < 4; ++i) bb[i] = __builtin_bit_cast(uint16_t, from_f32<RING>(dval[i]));
        bop = __builtin_bit_cast(typename MM::op_t, bb);
      }
    } else if constexpr (RF32) {
      bop = __shfl(wj, (c * CH + grp) & 63, 64) * dval[0];
    } else {
      u16x4 bb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __shfl(wj, (c * CH + 4 * grp + i) & 63, 64);
        bb[i] = __builtin_bit_cast(uint16_t, from_f32<RING>(w * dval[i]));
      }
      bop = __builtin_bit_cast(typename MM::op_t, bb);
    }
    return bop;
  };
  auto dval_of = [&](uint32_t raw) {
    if constexpr (RF32) return __uint_as_float(raw);
    else return to_f32<RING>(from_bits<RING>(static_cast<uint16_t>(raw)));
  };
  if (p > 0) {
    if constexpr (!KG) {
      // entries at or past p read as g = 0: the exclusive sum of lane p-1 is
      // exactly 0 (empty product = 1)
      float W, Wn;                                      // W_j = sum_{i>=j} g_i, W_{j+1}
      wave_suffix_sums(__uint_as_float(f.g_raw), lane, p > 16, W, Wn);
      wj = (lane < p) ? __expf(Wn) : 0.f;               // w_j = exp(W_{j+1})
      A = __expf(__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(W))));
    }
#pragma unroll
    for (int c = 0; c < NPRE; ++c) {
      float dv1[4];
      if constexpr (RF32) {
        dv1[0] = dval_of(f.d_raw[c]);
        dv1[1] = dv1[2] = dv1[3] = 0.f;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dv1[i] = dval_of(f.d_raw[i]);
      }
      if (split) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = __shfl(wj, (4 * grp + i) & 63, 64) * dv1[i];
      } else {
        bops[c] = bop_of(c, dv1);
      }
    }
  }
  __syncthreads();

  // ---- fused cursor advance (decode steps only): past the barrier every
  // wavefront of this workgroup has read the row's cursor, so the workgroup
  // counts itself in; the row's last workgroup to arrive writes the advanced
  // cursor (the rule of gdn_replay_advance) and clears the counter. Each
  // row's counter has a 128-byte line of its own: device-scope atomics on one
  // line serialise, and rows sharing a line made the launch ~20 us slower.
  if constexpr (TT) {
    if (a.arrive != nullptr && r.ok && tid == 0) {
      int* cnt = a.arrive + static_cast<size_t>(g.b) * kArriveStride;
      const int n = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (n == a.wg_per_row - 1) {
        a.write_pos_w[r.s] = r.flush ? 0 : p + 1;
        __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  const int wph = a.VB / 16;
  const int wh = g.h - (g.hk * a.G + g.hc * a.GH);              // head within the workgroup
  const bool kwriter = (g.vb == 0) && (g.hc == 0) && (wave == 0);   // one key-ring writer per k-head
  const bool gwriter_wave = (g.vb == 0) && (wave % wph == 0);     // one g writer per head
  const size_t hs = static_cast<size_t>(r.sc) * a.Hv + g.h;
  const size_t ks = static_cast<size_t>(r.sc) * a.Hk + g.hk;

  // ---- split readout. A row that does not flush needs its state
  // S = A S0 + sum_j w_j d_j k_j^T only through S q and S k, and
  //   S x = A (S0 x) + sum_j (w_j d_j) (k_j . x),
  // so the state is never formed: S0 x runs over the checkpoint as loaded,
  // and the ring products k_j . q, k_j . k take one MFMA k-step per 16 keys.
  // In it lane (col, grp) supplies four keys of ring entry col and of q
  // (col even) or k (col odd), and receives k_{4 grp + i} . x_col in register
  // i: the products of exactly the entries whose weights w_j d_j it holds.
  if constexpr (SPLIT) {
    if (split) {
      const uint16_t* kn = reinterpret_cast<const uint16_t*>(kt) + col * KNS + 4 * grp;
      const uint16_t* xh = reinterpret_cast<const uint16_t*>(buf + a.qh_off) + (col & 1) * DK + 4 * grp;
      f4 ce = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 16; ++s)
        ce = MM::mma(*reinterpret_cast<const typename MM::op_t*>(kn + 16 * s),
                     *reinterpret_cast<const typename MM::op_t*>(xh + 16 * s), ce);
      float dq = 0.f, dk = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the neighbour lane (col ^ 1) holds the other vector's product
        const float nb = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(ce[i]), 0xB1, 0xf, 0xf, false));
        const float kxq = (col & 1) ? nb : ce[i];
        const float kxk = (col & 1) ? ce[i] : nb;
        dq = __builtin_fmaf(wd[i], kxq, dq);
        dk = __builtin_fmaf(wd[i], kxk, dk);
      }
      // S0 q, S0 k over this lane's part of row col. As loaded, lane col
      // holds rows col & 7 (a) and (col & 7) + 8 (b) of keys
      // 32u + 16 (col >= 8) + 4 grp .. + 3; lane col ^ 8 holds the other half
      // of those rows' keys
      const bool lo = col < 8;
      const float* ql = qk + (lo ? 0 : 16) + 4 * grp;
      float qa = 0.f, qb = 0.f, ka = 0.f, kb = 0.f;
#pragma unroll
      for (int u = 0; u < DK / 32; ++u) {
        const f4 qv = *reinterpret_cast<const f4*>(ql + 32 * u);
        const f4 kv = *reinterpret_cast<const f4*>(ql + DK + 32 * u);
        const f4 ra = __builtin_bit_cast(f4, R.r[2 * u]);
        const f4 rb = __builtin_bit_cast(f4, R.r[2 * u + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qa = __builtin_fmaf(ra[j], qv[j], qa);
          qb = __builtin_fmaf(rb[j], qv[j], qb);
          ka = __builtin_fmaf(ra[j], kv[j], ka);
          kb = __builtin_fmaf(rb[j], kv[j], kb);
        }
      }
      const float xq = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(lo ? qb : qa), 0x128, 0xf, 0xf, false));
      const float xk = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(lo ? kb : ka), 0x128, 0xf, 0xf, false));
      const float mq = (lo ? qa : qb) + xq;
      const float mk = (lo ? ka : kb) + xk;
      const float sq = quad_sum(__builtin_fmaf(A, mq, dq));
      const float sk = quad_sum(__builtin_fmaf(A, mk, dk));
      const float* gt = gates + 3 * wh;
      const float alpha = gt[0], bt = gt[1], gv = gt[2];
      float d, o;
      token_out(sq, sk, kq_l[0], alpha, bt, to_f32<QKV>(f.v_raw), d, o);
      const size_t ih = static_cast<size_t>(g.b) * a.Hv + g.h;
      small_stores<QKV, RING>(a, ih * a.dv + g.vcol, (hs * a.L + p) * a.dv + g.vcol, hs * a.L + p,
                              o, d, gv, true, gwriter_wave, grp, col);
      if (kwriter && lane < C4)
        store4<RING>(a.ring_k, (ks * a.L + p) * DK + 4 * lane,
                     *reinterpret_cast<const f4*>(qk + DK + 4 * lane));
      return;
    }
  }

  // ---- reconstruction S = A S0 + sum_j w_j d_j k_j^T
  f4 S[NT];
  slab_decode<SD, DK>(S, R);
  if constexpr (SD == DT_F32) {
    const bool lo = col < 8;
#pragma unroll
    for (int u = 0; u < NT / 2; ++u) {
      const f4 A0 = S[2 * u], B0 = S[2 * u + 1];
      const f4 z = row_swap8(lo ? B0 : A0);
      S[2 * u] = lo ? A0 : z;
      S[2 * u + 1] = lo ? z : B0;
    }
  }
  if (p > 0) {
    const int wh0 = g.h - (g.hk * a.G + g.hc * a.GH);         // head within the workgroup
    const RT* ko = KG ? reinterpret_cast<const RT*>(buf + a.kw_off) + wh0 * a.kw_head : kt;
    auto kstep = [&](int c, typename MM::op_t bop) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        typename MM::op_t aop;
        const int key = key_of_row<SD>(t, col);
        if constexpr (RF32) aop = ko[(c * CH + grp) * DK + key];
        else aop = *reinterpret_cast<const typename MM::op_t*>(ko + key * a.kts + c * CH + 4 * grp);
        S[t] = MM::mma(aop, bop, S[t]);
      }
    };
    if constexpr (KG) {
      const float* acol = reinterpret_cast<const float*>(buf + a.acol_off) + wh0 * DK;
#pragma unroll
      for (int t = 0; t < NT; ++t) S[t] *= *reinterpret_cast<const f4*>(acol + key_base<SD>(t, grp));
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) S[t] *= A;
    }
#pragma unroll
    for (int c = 0; c < NPRE; ++c)
      if (c < nch) kstep(c, bops[c]);
    if (nch > NPRE) {                                   // rings deeper than 16 entries
      const char* dbase = static_cast<const char*>(a.ring_d) + hs * a.L * a.dv * RS;
      const __amdgpu_buffer_rsrc_t rd = brsrc(dbase, static_cast<uint32_t>(p) * a.dv * RS);
      for (int c = NPRE; c < nch; ++c) {
        float dv1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (RF32) {
            dv1[i] = i == 0 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                  rd, ((c * CH + grp) * a.dv + g.vcol) * 4, 0, 0))
                            : 0.f;
          } else {
            dv1[i] = dval_of(__builtin_amdgcn_raw_buffer_load_b16(
                rd, ((c * CH + 4 * grp + i) * a.dv + g.vcol) * 2, 0, 0));
          }
        }
        kstep(c, bop_of(c, dv1));
      }
    }
  }

  // ---- tokens
  if constexpr (!TT && !KG) {
    if (a.win_mfma) {
      window_chunked<DK, QKV, RING, SD, QKV == DT_BF16 && !NRM>(a, g, r, T, S, qk, vl, gates + 3 * wh * T, hs, ks, kwriter,
                                        gwriter_wave, grp, col, lane);
      return;
    }
  }
  for (int tau = 0; tau < T; ++tau) {
    const float* ql = qk + tau * 2 * DK;
    const float* kl = ql + DK;
    const size_t ih = (static_cast<size_t>(g.b) * T + tau) * a.Hv + g.h;
    const float vv = TT ? to_f32<QKV>(f.v_raw) : vl[tau * 16 + col];
    const float* gt = gates + 3 * (wh * T + tau);
    const float alpha = gt[0], bt = gt[1], gv = gt[2];
    const float kq = kq_l[tau];
    const float* gl = kgl + (wh * T + tau) * 4 * DK;      // KG: a, a o q, a o k, g
    float sq, sk, d, o;
    if constexpr (KG) {
      slab_dots<SD>(S, gl + DK, gl + 2 * DK, grp, sq, sk);
      token_out(sq, sk, kq, 1.f, bt, vv, d, o);
    } else {
      slab_dots<SD>(S, ql, kl, grp, sq, sk);
      token_out(sq, sk, kq, alpha, bt, vv, d, o);
    }
    const bool app = r.ok && !r.flush;              // this token appends a ring entry
    const int pos = p + tau;
    small_stores<QKV, RING>(a, ih * a.dv + g.vcol, (hs * a.L + pos) * a.dv + g.vcol,
                            hs * a.L + pos, r.ok ? o : 0.f, d, gv, app,
                            KG ? false : gwriter_wave, grp, col);
    if constexpr (KG) {
      if (app && gwriter_wave && lane < C4)
        *reinterpret_cast<f4*>(a.ring_g + (hs * a.L + pos) * DK + 4 * lane) =
            *reinterpret_cast<const f4*>(gl + 3 * DK + 4 * lane);
    }
    if (app && kwriter && lane < C4) {
      const f4 kv = *reinterpret_cast<const f4*>(kl + 4 * lane);
      store4<RING>(a.ring_k, (ks * a.L + pos) * DK + 4 * lane, kv);
    }
    if (r.flush || (!TT && a.window && tau + 1 < T)) {
      if constexpr (KG) slab_update_key<SD>(S, kl, gl, grp, d);
      else slab_update<SD>(S, kl, grp, alpha, d);
      if (!TT && a.step_round) slab_round<SD>(S);
    }
  }
  if (r.flush) {
    using SE = typename Elem<SD>::T;
    store_slab<SD, DK, kCpolSc1>(static_cast<SE*>(a.state) + (hs * a.dv + g.vrow0) * DK, S, col, grp);
  }
}

// NRM = 1: q and k are L2-normalised (q scaled) in the kernel (a.qk_norm).
// Windows (TT = 0) are bound by vector issue after the checkpoint arrives;
// held to 80 VGPRs (6 wavefronts per SIMD instead of 5, no spills at dk <= 128
// without in-kernel normalisation) their launches run in fewer rounds:
// 20.4 -> 20.0 us (T = 5, B = 32), lossless 21.9 -> 20.8 us.
constexpr int window_waves_per_eu(int DK, int TT, int NRM) {
  return (TT || NRM || DK > 128) ? 1 : 6;
}

template <int DK, int QKV, int RING, int SD, int TT, int KG, int NRM>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(window_waves_per_eu(DK, TT, NRM)))) void replay_decode_kernel(
    DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* dump = reinterpret_cast<float*>(smem + a.dump_off);    // [64][8] write sink
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, col = lane & 15;
  const int T = TT ? 1 : a.T;
  // The row's metadata pointers are needed right after the work-item
  // mapping; used here, they are loaded with the mapping's arguments, so the
  // chain before the first vector load is arguments -> slot -> cursor.
  asm volatile("" ::"s"(a.slot), "s"(a.write_pos), "s"(a.ff_flags));
  const ItemGeo g = item_geo(a, wave, col);
  // the slot load first, then the token operands while it is in flight
  const int slot = ld_uniform(a.slot, g.b);
  Small<DK, QKV, RING> sm;
  fetch_tokens<DK, QKV, RING, TT, KG>(sm, a, g, T, tid, lane, grp, wave);
  const RowState r = row_state(a, g.b, T, slot);
  SlabRaw<SD, DK> R;
  fetch_small<DK, QKV, RING, TT, KG>(sm, a, g, r, T, tid, lane, grp, wave);
  if constexpr (KG) {
    if (a.kdma) fetch_key_gate<DK, RING>(a, g, r, T, smem, tid, lane, wave);
  }
  __builtin_amdgcn_sched_barrier(0);
  fetch_slab<SD, DK>(R, a, g, r, col, grp);
  process<DK, QKV, RING, SD, TT, KG, NRM>(a, g, r, T, sm, R, smem, dump, tid, lane, grp, col, wave);
}

// ============================================================= fold
//
// Fold the valid ring entries into the checkpoint with the pinned two-step
// rounding (SGLang PR #42388 "The idea"; SGLang PR #36821 fold). Workgroup =
// (layer, row, value head, FV value rows), the layer in blockIdx.y; thread =
// one 16-byte group of 4 keys in FV/16 consecutive rows (the ring entries
// staged in LDS serve all of them). One launch may fold the same rows of
// several layers: a single layer's launch at 32 rows has a fixed cost of
// about 5 us (its first workgroups' start and its last ones' tail) in 27 us,
// and the layers of a verify round are folded together anyway.
// KG = 1: per-key gate (ring_g [N, Hv, L, dk]), each channel decays by its
// own a_j[c].
// The fold reads each checkpoint line and writes it back: its stores go on
// to memory at once (sc1 nt), as the packed decode's do.
constexpr int kFoldStorePolicy = kCpolSc1Nt;

template <int DK, int RING, int SD, int KG>
__global__ __launch_bounds__(1024) void fold_kernel(FoldArgs a) {
  constexpr int C4 = DK / 4;
  constexpr int MAXR = 4;                             // rows per thread, at most
  extern __shared__ __align__(16) unsigned char smem[];
  const int FV = a.fv;                                // value rows per workgroup (16, 32 or 64)
  const int nr = FV >> 4;                             // rows per thread
  float* kl = reinterpret_cast<float*>(smem);        // [L][DK]  key entries (16-byte rows)
  float* dl = kl + a.L * DK;                          // [L][FV]  d entries
  float* al = dl + a.L * FV;                          // [L] decays ([L][DK] for KG)

  // this workgroup's layer: the launch folds gridDim.y layers of equal shapes
  const int layer = blockIdx.y;
  void* const ckpt = a.ckpt[layer];
  const void* const ring_d = a.ring_d[layer];
  const void* const ring_k = a.ring_k[layer];
  const float* const ring_g = a.ring_g[layer];
  const int nvb = a.dv / FV;
  int blk = item_of_block(blockIdx.x, gridDim.x, nvb * a.G);
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
  const int row = (tid / C4) * nr, e4 = (tid % C4) * 4;   // rows row .. row + nr - 1

  using SE = typename Elem<SD>::T;
  SE* xbase = static_cast<SE*>(ckpt) + (hs * a.dv + vb * FV) * DK;   // the block's FV rows
  const int F4 = FV >> 2;                             // four d entries per item
  // This thread's first piece of ring g, d and keys is requested before the
  // checkpoint rows, so that staging them in LDS waits only for them: vector
  // loads complete in issue order (30.5 -> 28.6 us at p = 15, B = 32). Only
  // the wavefronts that hold some of a range request it (a wave-uniform
  // branch); their surplus lanes read the range's last piece again.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lf4 = FV == 64 ? 4 : (FV == 32 ? 3 : 2);   // F4 = 2^lf4
  const int cd = tid < p * F4 ? tid : p * F4 - 1, ck = tid < p * C4 ? tid : p * C4 - 1;
  const int jd = cd >> lf4, jk = ck / C4;
  float g_raw = 0.f;
  typename Raw4<RING>::T d_raw{}, k_raw{};
  if (!KG && wave == 0) g_raw = ring_g[hs * a.L + (tid < p ? tid : p - 1)];
  if (64 * wave < p * F4)
    d_raw = load4_raw<RING>(ring_d, (hs * a.L + jd) * a.dv + vb * FV + (cd - jd * F4) * 4);
  if (64 * wave < p * C4)
    k_raw = load4_raw<RING>(ring_k, (ks * a.L + jk) * DK + (ck - jk * C4) * 4);
  // the block's checkpoint rows, read with the non-temporal policy (each line
  // is read once and written back once: 31.4 -> 30.3 us at p = 15, B = 32)
  f4 x[MAXR];
#pragma unroll
  for (int m = 0; m < MAXR; ++m)
    if (m < nr) {
      if constexpr (SD == DT_F32) {
        x[m] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(xbase + (row + m) * DK + e4));
      } else {
        const u16x4 r4 = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(xbase + (row + m) * DK + e4));
        x[m] = f4{to_f32<SD>(from_bits<SD>(r4[0])), to_f32<SD>(from_bits<SD>(r4[1])),
                  to_f32<SD>(from_bits<SD>(r4[2])), to_f32<SD>(from_bits<SD>(r4[3]))};
      }
    }

  if constexpr (KG) {
    for (int c = tid; c < p * C4; c += blockDim.x) {
      const int j = c / C4, q4 = (c % C4) * 4;
      const f4 g4 = *reinterpret_cast<const f4*>(ring_g + (hs * a.L + j) * DK + q4);
      f4 av;
      av.x = decay_of(g4.x); av.y = decay_of(g4.y); av.z = decay_of(g4.z); av.w = decay_of(g4.w);
      *reinterpret_cast<f4*>(al + j * DK + q4) = av;
    }
  } else {
    if (tid < p) al[tid] = decay_of(g_raw);
  }
  if (tid < p * F4) *reinterpret_cast<f4*>(dl + jd * FV + (cd - jd * F4) * 4) = decode4<RING>(d_raw);
  if (tid < p * C4) *reinterpret_cast<f4*>(kl + jk * DK + (ck - jk * C4) * 4) = decode4<RING>(k_raw);
  for (int c = tid + blockDim.x; c < p * F4; c += blockDim.x) {
    const int j = c / F4, r4 = (c - j * F4) * 4;
    *reinterpret_cast<f4*>(dl + j * FV + r4) =
        load4<RING>(ring_d, (hs * a.L + j) * a.dv + vb * FV + r4);
  }
  for (int c = tid + blockDim.x; c < p * C4; c += blockDim.x) {
    const int j = c / C4, q4 = (c % C4) * 4;
    *reinterpret_cast<f4*>(kl + j * DK + q4) = load4<RING>(ring_k, (ks * a.L + j) * DK + q4);
  }
  __syncthreads();

  if (SD == DT_F32 && nr == MAXR) {
    // fp32 state, four rows per thread, folded two at a time: the first pair
    // is stored while the second is folded, and the first pair's work starts
    // once its two rows have arrived (28.2 -> 26.8 us at p = 15, B = 32). One
    // row at a time reads the staged entries four times (30.0 us); the same
    // split written for every state format and row count measured 28.5 us.
    // The same operations in the same order per element as the loop below.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma clang fp contract(off)
      for (int j = 0; j < p; ++j) {
        f4 aj;
        if constexpr (KG) aj = *reinterpret_cast<const f4*>(al + j * DK + e4);
        else aj = f4{al[j], al[j], al[j], al[j]};
        const f4 kv = *reinterpret_cast<const f4*>(kl + j * DK + e4);
        const float2 d2 = *reinterpret_cast<const float2*>(dl + j * FV + row + 2 * h2);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const float dj = mm ? d2.y : d2.x;
          f4& y = x[2 * h2 + mm];
          const float tx = aj.x * y.x, ty = aj.y * y.y, tz = aj.z * y.z, tw = aj.w * y.w;
          y.x = __builtin_fmaf(dj, kv.x, tx);
          y.y = __builtin_fmaf(dj, kv.y, ty);
          y.z = __builtin_fmaf(dj, kv.z, tz);
          y.w = __builtin_fmaf(dj, kv.w, tw);
        }
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int off = (row + 2 * h2 + mm) * DK + e4;
        store16<kFoldStorePolicy>(reinterpret_cast<float*>(xbase), FV * DK * 4, off * 4, x[2 * h2 + mm]);
      }
    }
    return;
  }
  {
#pragma clang fp contract(off)
    for (int j = 0; j < p; ++j) {
      f4 aj;
      if constexpr (KG) aj = *reinterpret_cast<const f4*>(al + j * DK + e4);
      else aj = f4{al[j], al[j], al[j], al[j]};
      const f4 kv = *reinterpret_cast<const f4*>(kl + j * DK + e4);
      // the thread's nr consecutive rows: one 16-byte read of d when nr = 4
      f4 d4;
      if (nr == MAXR) {
        d4 = *reinterpret_cast<const f4*>(dl + j * FV + row);
      } else {
#pragma unroll
        for (int m = 0; m < MAXR; ++m) d4[m] = m < nr ? dl[j * FV + row + m] : 0.f;
      }
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        if (m < nr) {
          const float dj = d4[m];
          f4& y = x[m];
          const float tx = aj.x * y.x, ty = aj.y * y.y, tz = aj.z * y.z, tw = aj.w * y.w;
          y.x = __builtin_fmaf(dj, kv.x, tx);
          y.y = __builtin_fmaf(dj, kv.y, ty);
          y.z = __builtin_fmaf(dj, kv.z, tz);
          y.w = __builtin_fmaf(dj, kv.w, tw);
          if constexpr (SD != DT_F32) {
            if (a.step_round) {
              y.x = to_f32<SD>(state_round<SD>(y.x));
              y.y = to_f32<SD>(state_round<SD>(y.y));
              y.z = to_f32<SD>(state_round<SD>(y.z));
              y.w = to_f32<SD>(state_round<SD>(y.w));
            }
          }
        }
      }
    }
  }
  // fp32 result of the exact fold, rounded once to the state format
#pragma unroll
  for (int m = 0; m < MAXR; ++m) {
    if (m < nr) {
      const int off = (row + m) * DK + e4;
      if constexpr (SD == DT_F32) {
        store16<kFoldStorePolicy>(reinterpret_cast<float*>(xbase), FV * DK * 4, off * 4, x[m]);
      } else {
        u16x4 r;
        r.x = __builtin_bit_cast(uint16_t, state_round<SD>(x[m].x));
        r.y = __builtin_bit_cast(uint16_t, state_round<SD>(x[m].y));
        r.z = __builtin_bit_cast(uint16_t, state_round<SD>(x[m].z));
        r.w = __builtin_bit_cast(uint16_t, state_round<SD>(x[m].w));
        store8<kFoldStorePolicy>(reinterpret_cast<float*>(xbase), FV * DK * 2, off * 2, r);
      }
    }
  }
}

}  // namespace gdn
