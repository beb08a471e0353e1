/*
 * gdn_replay.h -- C ABI of the MI355X (gfx950) ReplaySSM Gated DeltaNet
 * decode library (libgdn_replay.so).
 *
 * The method: a slot's recurrent state is kept as one checkpoint (fp32, or a
 * 16-bit format) plus a ring holding the (d, k, g) entries of its L most
 * recent steps. A decode step rebuilds the pre-token state from them, reads
 * the output out of it, appends its own entry to the ring, and writes the
 * full state back only on a flush (ReplaySSM blog, llm.rainlin.net, sections 2-3; SGLang PR #28451,
 * Modifications and Design 1-5).
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device (HBM) pointers; the `shape` struct
 *     (and the per-layer pointer arrays of gdn_replay_fold_layers) are host
 *     memory read during the call only. `stream` is a hipStream_t (NULL =
 *     the null stream).
 *   - Every call is asynchronous on `stream`: it validates its host-side
 *     arguments, enqueues one or two kernels (gdn_replay_fold_layers: one
 *     per 16 layers), and returns. It never
 *     synchronises, never allocates and never frees. The caller owns every
 *     buffer and must keep it alive until the stream has passed the call.
 *   - On a host-side validation failure the call returns a non-zero status
 *     and enqueues nothing. A failed launch returns GDN_ERR_HIP.
 *   - Data errors that only the device can see (a slot index >= N, a cursor
 *     out of range, a verify window that does not fit the ring, an accepted
 *     count out of range) are reported by OR-ing GDN_EF_* bits into
 *     *err_flags (device int32, nullable) without a sync; the affected row is
 *     then handled as a padding row (zero output, no state or ring write).
 *   - A negative slot index marks a padding row: its outputs are written as
 *     zeros and nothing else is touched (ReplaySSM blog, section 3.1).
 *   - Within one call, the non-negative slot indices must be distinct.
 *   - Calls on one stream are ordered; calls on different streams that touch
 *     the same slots race.
 *
 * Tensor layouts (all contiguous, row-major, base pointers 16-byte aligned):
 *   q, k           [B, T, Hk, dk]   qkv_dtype; q/k already normalised, q scaled
 *   v, o           [B, T, Hv, dv]   qkv_dtype (o is written in the same dtype)
 *   g, beta        [B, T, Hv]       fp32 (per-key gate: g [B, T, Hv, dk]); g is the
 *                                  log-decay. Every kernel applies
 *                                  the decay alpha = RN_f32(exp_f64(g)), one value per
 *                                  step, so that stored steps replay exactly
 *   state / ckpt   [N, Hv, dv, dk]  state_dtype, dk fastest (ReplaySSM blog, 2.2)
 *   ring_d         [N, Hv, L, dv]   ring_dtype  (the correction vectors d)
 *   ring_k         [N, Hk, L, dk]   ring_dtype  (keys, one per k-head)
 *   ring_g         [N, Hv, L]       fp32        (log-decays; [N, Hv, L, dk] per key)
 *   write_pos      [N]              int32, number of valid ring entries
 *   slot_idx       [B]              int32, row -> slot, negative = padding
 *   force_flush    [B]              int32, nullable (nonzero = force a flush)
 *   accepted       [B]              int32
 * Value head h uses key head h / (Hv / Hk).
 *
 * Supported sizes: dk in {32, 64, 128, 256}; dv a multiple of 16, 16..512;
 * Hv % Hk == 0 with Hv / Hk <= 16; 1 <= L <= 64; 1 <= T <= 16; B >= 0.
 * qkv_dtype in {GDN_F32, GDN_BF16}; ring_dtype in {GDN_F32, GDN_F16, GDN_BF16};
 * state_dtype in {GDN_F32, GDN_BF16, GDN_F16}.
 *
 * 16-bit state (state_dtype GDN_BF16 or GDN_F16). vLLM PR #49887 (Out of
 * scope) notes that fp16 and bf16 states are supported by its decode code; its review
 * thread contrasts a decode that stores the state in 16 bits after every
 * token with ReplaySSM, which keeps the state in fp32 between checkpoint
 * writes and rounds only when the buffer is full. The library follows that
 * reading. All arithmetic is fp32; a 16-bit value is widened exactly on load,
 * and a state written to memory is rounded once, to nearest even:
 *   gdn_packed_decode  rounds the updated state every step;
 *   gdn_replay_decode  rounds the checkpoint only on a flush;
 *   gdn_replay_fold    folds in fp32 and rounds the result once.
 * At L = 1 replay and packed decode therefore still agree bit for bit.
 *
 * step_rounding = 1 (verify windows and folds only) rounds a 16-bit state
 * after every step instead: the window rounds its on-chip state after each
 * token's update and the fold after each entry, as the packed decode does.
 * A verify window from an exact checkpoint (write_pos = 0) with an fp32 ring,
 * committed and folded with step_rounding, then equals token-by-token packed
 * decode bit for bit also for a 16-bit state (SGLang PR #42388 keeps the
 * ring in fp32 for every state dtype, which is what makes this possible).
 * With an fp32 state the flag changes nothing.
 *
 * Per-key gate (gate = GDN_GATE_KEY, KDA). SGLang PR #28451 (Modifications,
 * item 7) runs KDA through the same kernels: KDA is the same delta rule with
 * the decay taken per key channel, S' = S Diag(a) + d k^T with a = exp(g) a
 * vector over the dk channels. Then
 *   g       [B, T, Hv, dk] fp32 and ring_g [N, Hv, L, dk] fp32 (both
 *           16-byte aligned), one log-decay per key channel;
 *   readout d = beta (v - S (a o k)),  o = S (a o q) + d (k^T q): the token's
 *           decays fold into q and k (a o q is the element-wise product);
 *   update  S <- S Diag(a) + d k^T, rounded fma(d[v], k[c], RN(a[c] * S[v,c]));
 *   replay  S = ckpt Diag(A) + sum_{j<p} d_j (w_j o k_j)^T with, per channel c,
 *           A[c] = exp(sum_{i<p} g_i[c]), w_j[c] = exp(sum_{j<i<p} g_i[c]):
 *           the decay products fold onto the stored keys;
 *   fold    x <- fma(d_j[v], k_j[c], RN(a_j[c] * x)) with a_j[c] = RN_f32(exp_f64(g_j[c])).
 * Everything else (ring d and k, cursors, flush, windows, state formats,
 * step_rounding) is the same as with the per-head gate. Only gdn_packed_decode,
 * gdn_replay_decode and gdn_replay_fold read the field; the cursor calls ignore it.
 *
 * Strided inputs. The decode calls read q, k and v as rows of (b, t): element
 * [b, t, h, i] of q (and k) is at q[(b*T + t) * qk_row_stride + h*dk + i], of v
 * at v[(b*T + t) * v_row_stride + h*dv + i]. With the strides 0 the tensors are
 * dense. Set both to 2*Hk*dk + Hv*dv, with k = q + Hk*dk and v = q + 2*Hk*dk,
 * to read the packed mixed_qkv row [B, T, 2*Hk*dk + Hv*dv] that the serving
 * stack hands to the decode (ReplaySSM blog, section 3.1). qk_row_stride must
 * keep every q and k row 16-byte aligned. o, g and beta stay dense.
 *
 * Front end (qk_norm = 1). The pages hand the decode q and k already
 * L2-normalised and q scaled (SGLang PR #28451, Modifications). With qk_norm
 * the kernels do it themselves: q <- q / sqrt(sum q^2 + 1e-6) * dk^-1/2 and
 * k <- k / sqrt(sum k^2 + 1e-6) per key head and token, in fp32, before the
 * readout; the ring stores the normalised k. The packed and the replay decode
 * normalise in the same order, so the L = 1 identity stays bitwise.
 */
#ifndef GDN_REPLAY_H
#define GDN_REPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size or mode    */
    GDN_ERR_UNSUPPORTED = 2, /* a size or dtype outside the compiled set        */
    GDN_ERR_HIP = 3,         /* the HIP runtime refused the launch              */
    GDN_ERR_SCRATCH_LIMIT = 4 /* B > GDN_SCRATCH_MAX_ROWS (the _noalloc call)   */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype;

/* Granularity of the decay (gdn_shape.gate). */
typedef enum {
    GDN_GATE_HEAD = 0, /* GDN: one log-decay g per value head                       */
    GDN_GATE_KEY = 1   /* KDA: one log-decay per value head and key channel          */
} gdn_gate;

/* Device-side data error bits OR-ed into *err_flags. */
enum {
    GDN_EF_SLOT_RANGE = 1,   /* slot_idx[b] >= N                                */
    GDN_EF_CURSOR_RANGE = 2, /* write_pos outside its valid range for the call  */
    GDN_EF_WINDOW = 4,       /* verify window: write_pos + T > L                */
    GDN_EF_ACCEPTED = 8      /* commit: accepted outside [0, T] or past L       */
};

typedef struct {
    int32_t B;          /* rows in the call                                      */
    int32_t T;          /* tokens per row (1 for decode; the window length)      */
    int32_t N;          /* slots in the pool                                     */
    int32_t Hv, Hk;     /* value / key heads                                     */
    int32_t dk, dv;     /* key / value head dimensions                           */
    int32_t L;          /* ring capacity (ignored by gdn_packed_decode)          */
    int32_t qkv_dtype;  /* gdn_dtype of q, k, v and o                            */
    int32_t ring_dtype; /* gdn_dtype of ring_d and ring_k                        */
    int32_t window;     /* gdn_replay_decode: 0 = decode step, 1 = verify window */
    int32_t state_dtype;/* gdn_dtype of the state / checkpoint (0 = GDN_F32)     */
    int32_t step_rounding; /* 1: round a 16-bit state after every step (verify
                              window and fold only; see below), else 0    */
    int32_t gate;       /* gdn_gate: GDN_GATE_HEAD (0) or GDN_GATE_KEY (1)       */
    int32_t qk_row_stride; /* elements between the q (and k) of consecutive (b, t)
                              rows; 0 = dense (Hk*dk). See "Strided inputs". */
    int32_t v_row_stride;  /* the same for v; 0 = dense (Hv*dv)              */
    int32_t qk_norm;    /* 1: L2-normalise q and k in the kernel and scale q by
                           dk^-1/2 (see "Front end"); 0: take them as given */
} gdn_shape;

/*
 * gdn_packed_decode -- the plain read-update-write decode step (T must be 1).
 *
 * Per row b with slot s = slot_idx[b] >= 0 and per value head h, with
 * alpha = exp(g), following SGLang PR #28451 (Modifications, the GDN math):
 *     Sq = S q,  Sk = S k                     (S = state[s, h], before the token)
 *     d  = beta (v - alpha Sk)
 *     o  = alpha Sq + d (k^T q)
 *     state[s, h] <- alpha S + d k^T          (written every step)
 * The state update is rounded in two steps, fma(d[v], k[c], RN(alpha*S[v,c])),
 * the form SGLang PR #42388 ("The idea") names for an exactly reproducible
 * replay. This is the baseline whose per-step state read+write the ReplaySSM
 * path removes (SGLang PR #28451, Motivation).
 *   state   (device) state_dtype [N, Hv, dv, dk], read and written (a 16-bit
 *           state is rounded to its format after every step).
 *   o       (device) [B, 1, Hv, dv], written for every row (zeros for padding).
 */
gdn_status gdn_packed_decode(const gdn_shape *shape, const void *q, const void *k,
                             const void *v, const float *g, const float *beta,
                             const int32_t *slot_idx, void *state, void *o,
                             int32_t *err_flags, void *stream);

/*
 * gdn_replay_decode -- the ReplaySSM output-only decode step (window = 0,
 * T = 1) or the verify window from one checkpoint (window = 1, T >= 1).
 *
 * Per row b with slot s and per value head h, with p = write_pos[s] valid ring
 * entries (only positions < p are ever read, SGLang PR #28451 Design 5):
 *   pre-token state (ReplaySSM blog, section 2.1, closed form):
 *       S = A ckpt[s,h] + sum_{j<p} w_j d_j k_j^T,
 *       A = exp(sum_{i<p} g_i),  w_j = exp(sum_{j<i<p} g_i)   (empty sum = 0)
 *   readout (SGLang PR #28451, Modifications): as for gdn_packed_decode.
 * Decode (window = 0, T = 1): the step flushes when p == L-1 or
 * force_flush[b] != 0 (SGLang PR #28451, Design 4-5). A non-flush step appends
 * (d, k, g) at ring position p (k once per key head); a flush step writes
 * ckpt[s,h] <- fma(d[v], k[c], RN(alpha*S[v,c])) and leaves the ring bytes
 * unchanged (ReplaySSM blog, section 3.3). write_pos is NOT changed: advance it
 * once per forward with gdn_replay_advance, after every layer's decode call.
 * Requires 0 <= p <= L-1, else GDN_EF_CURSOR_RANGE.
 * Verify window (window = 1): tokens t = 0..T-1 of the row are read out in
 * order from the same checkpoint + ring; token t sees window tokens < t
 * through an on-chip update of S (vLLM PR #49887, Core concept). Entries are
 * written at positions p..p+T-1; there is no flush and write_pos is NOT moved
 * (commit with gdn_replay_commit). force_flush must be NULL. Requires
 * p + T <= L, else GDN_EF_WINDOW.
 *   ckpt           (device) state_dtype [N, Hv, dv, dk]; written only on a
 *                  flush (rounded to a 16-bit state format there).
 *   ring_d/k/g     (device) read at positions < p, written as described.
 *   write_pos      (device) int32 [N], read only.
 *   force_flush    (device) int32 [B] or NULL; nonzero forces a flush.
 *   o              (device) [B, T, Hv, dv], written for every row.
 */
gdn_status gdn_replay_decode(const gdn_shape *shape, const void *q, const void *k,
                             const void *v, const float *g, const float *beta,
                             const int32_t *slot_idx, void *ckpt, void *ring_d,
                             void *ring_k, float *ring_g, const int32_t *write_pos,
                             const int32_t *force_flush, void *o, int32_t *err_flags,
                             void *stream);

/*
 * gdn_replay_decode_advance -- a decode step (window = 0, T = 1) with the
 * cursor advance of gdn_replay_advance fused into it: the forward's last
 * layer calls it instead of gdn_replay_decode followed by gdn_replay_advance
 * (SGLang PR #28451, Design 3: the cursor advances once per forward, after
 * every layer has read it). Outputs, checkpoint and ring writes are those of
 * gdn_replay_decode; afterwards write_pos[s] holds what gdn_replay_advance
 * with the same force_flush would have written. Rows that are padding or in
 * error keep their cursor (and set the error bits as gdn_replay_decode does).
 *   write_pos  (device) int32 [N], read and written.
 *   arrive     (device) int32 [B * GDN_ARRIVE_STRIDE] workspace, owned by the
 *              caller, 128-byte aligned: all zero before the call; the call
 *              leaves it all zero. Row b's workgroups count themselves in
 *              arrive[b * GDN_ARRIVE_STRIDE] after they have read the row's
 *              cursor; the last one writes the advanced cursor. (One 128-byte
 *              line per row: device-scope atomics on a shared line serialise.)
 *              Two calls that share an arrive buffer must not overlap.
 * Returns GDN_ERR_INVALID_ARG if arrive is NULL or misaligned, or if
 * shape->window != 0. Every other argument as gdn_replay_decode.
 */
#define GDN_ARRIVE_STRIDE 32
gdn_status gdn_replay_decode_advance(const gdn_shape *shape, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta,
                                     const int32_t *slot_idx, void *ckpt, void *ring_d,
                                     void *ring_k, float *ring_g, int32_t *write_pos,
                                     const int32_t *force_flush, void *o, int32_t *arrive,
                                     int32_t *err_flags, void *stream);

/*
 * gdn_replay_decode_advance_noalloc -- gdn_replay_decode_advance for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It allocates nothing, not
 * even through the caller: the arrival counters live in a static device
 * array of the library instead of the caller's `arrive` workspace.
 *   Limit: B <= GDN_SCRATCH_MAX_ROWS (4096) rows; a larger B returns
 *   GDN_ERR_SCRATCH_LIMIT before anything is enqueued. The array is 512 KiB
 *   (one 128-byte line per row) on every device the library runs on, held
 *   until the process ends.
 *   Set-up: the first call on a device (the device current at the call)
 *   looks up that device's copy of the array and enqueues one clear of it on
 *   `stream`; make that first call outside stream capture.
 *   Sharing: every call on one device uses the same array, which keeps what
 *   the last call left (all zero after every completed call). Calls that
 *   overlap on one device (different streams, or host threads racing on one
 *   stream) race on the counters; calls ordered on one stream do not.
 * Outputs, checkpoint, ring and cursor writes, error bits and every other
 * argument are those of gdn_replay_decode_advance (with window = 0, T = 1).
 */
#define GDN_SCRATCH_MAX_ROWS 4096
gdn_status gdn_replay_decode_advance_noalloc(const gdn_shape *shape, const void *q,
                                             const void *k, const void *v, const float *g,
                                             const float *beta, const int32_t *slot_idx,
                                             void *ckpt, void *ring_d, void *ring_k,
                                             float *ring_g, int32_t *write_pos,
                                             const int32_t *force_flush, void *o,
                                             int32_t *err_flags, void *stream);

/*
 * gdn_replay_advance -- the cursor advance that follows a forward's decode
 * calls (SGLang PR #28451, Design 3): for each row with slot s >= 0,
 *     write_pos[s] <- (write_pos[s] == L-1 || force_flush[b]) ? 0 : write_pos[s]+1.
 * It must see the same force_flush as the forward's decode calls.
 *   write_pos (device) int32 [N], read and written. force_flush nullable.
 * A cursor outside [0, L-1] is left as is and sets GDN_EF_CURSOR_RANGE.
 */
gdn_status gdn_replay_advance(const gdn_shape *shape, const int32_t *slot_idx,
                              int32_t *write_pos, const int32_t *force_flush,
                              int32_t *err_flags, void *stream);

/*
 * gdn_replay_commit -- keep the accepted prefix of a verify window: for each
 * row with slot s >= 0, write_pos[s] <- write_pos[s] + accepted[b] (vLLM PR
 * #49887: rollback of rejected drafts is only a cursor move). accepted[b]
 * must lie in [0, T] and write_pos[s] + accepted[b] <= L, else the cursor is
 * left as is and GDN_EF_ACCEPTED is set.
 */
gdn_status gdn_replay_commit(const gdn_shape *shape, const int32_t *slot_idx,
                             const int32_t *accepted, int32_t *write_pos,
                             int32_t *err_flags, void *stream);

/*
 * gdn_replay_fold -- fold each listed slot's p = write_pos[s] valid ring
 * entries of one layer into that layer's checkpoint (SGLang PR #36821,
 * Technical principle: at commit the kept entries are applied to the
 * checkpoint in place, replaying the recurrence with its exact operation
 * order). Per element, for j = 0..p-1:
 *     a = RN_f32(exp_f64(g_j));  x <- fma(d_j[v], k_j[c], RN(a*x))
 * with the two-instruction rounding of SGLang PR #42388 ("The idea"). The
 * result is bit-identical to that sequential recurrence on the stored entries.
 * The decays are the same values every decode and verify kernel applies, so a
 * verify window started from an exact checkpoint (write_pos = 0) with an fp32
 * ring, committed and folded, equals decoding the accepted tokens one at a
 * time with gdn_packed_decode, bit for bit (the lossless verify of SGLang PR
 * #42388).
 * write_pos is only read: the cursors are shared by every layer, so fold all
 * layers, then clear the cursors once with gdn_replay_reset.
 * Requires 0 <= p <= L, else GDN_EF_CURSOR_RANGE (the slot is not touched).
 * With a 16-bit state the fold runs in fp32 from the widened checkpoint and the
 * result is rounded once to the state format.
 *   ckpt (device) read and written; ring_d/k/g (device) read at positions < p.
 */
gdn_status gdn_replay_fold(const gdn_shape *shape, const int32_t *slot_idx,
                           void *ckpt, const void *ring_d, const void *ring_k,
                           const float *ring_g, const int32_t *write_pos,
                           int32_t *err_flags, void *stream);

/*
 * gdn_replay_fold_layers -- gdn_replay_fold of n_layers layers in one go:
 * layer l folds ring_d[l], ring_k[l], ring_g[l] into ckpt[l], with the same
 * slots, cursors, shapes and dtypes for every layer (SGLang PR #36821,
 * Technical principle: the fold runs at commit, once the verify pass has
 * gone through every layer, so all layers' entries are known together).
 * Each layer's result is bit-identical to gdn_replay_fold on that layer.
 * The layers run in launches of up to 16 layers each, so the fixed start
 * and tail cost of a launch is paid once per 16 layers instead of per layer.
 *   n_layers      1..GDN_FOLD_MAX_LAYERS;
 *   ckpt, ring_d, ring_k, ring_g
 *                 host arrays of n_layers device pointers (each with the
 *                 layout and alignment of gdn_replay_fold). The checkpoints
 *                 must not overlap one another (checked: GDN_ERR_INVALID_ARG)
 *                 nor any ring; rings may be shared between layers.
 * The host arrays are read during the call only. Errors and error bits are
 * those of gdn_replay_fold; an argument error is returned before anything is
 * launched.
 */
#define GDN_FOLD_MAX_LAYERS 1024
gdn_status gdn_replay_fold_layers(const gdn_shape *shape, int32_t n_layers,
                                  const int32_t *slot_idx, void *const *ckpt,
                                  const void *const *ring_d, const void *const *ring_k,
                                  const float *const *ring_g, const int32_t *write_pos,
                                  int32_t *err_flags, void *stream);

/*
 * gdn_replay_reset -- write_pos[s] <- 0 for each row with slot s >= 0: the
 * ring is empty again once every layer has folded it (SGLang PR #36821: after
 * the fold the checkpoint holds the committed state). A slot >= N sets
 * GDN_EF_SLOT_RANGE.
 *   write_pos (device) int32 [N], written.
 */
gdn_status gdn_replay_reset(const gdn_shape *shape, const int32_t *slot_idx,
                            int32_t *write_pos, int32_t *err_flags, void *stream);

/*
 * gdn_conv_update -- the causal convolution step in front of the decode
 * (ReplaySSM blog, section 3.1: the decode path first updates the causal
 * convolution and hands the convolved packed row to the kernel; SGLang PR
 * #36821, Technical principle: x_hat_t = SiLU(w * x_{t-3:t}), a depthwise
 * convolution over the current input and the three before it, then SiLU).
 * Per row b with slot s = slot_idx[b] >= 0 and channel c < C, with the W
 * inputs z_0..z_{W-1} of the window, oldest first,
 *     z_i = conv_state[s, i, c] (i < W-1),  z_{W-1} = x[b, c]:
 *     acc     = sum_{i<W} w[c, i] z_i      fp32, one fma per tap, i ascending
 *     y[b, c] = acc / (1 + exp(-acc))      SiLU in fp32, rounded to dtype
 *     conv_state[s, i, c] <- z_{i+1}       (i < W-1): the window moves by one
 * Tap W-1 multiplies the current input. Padding rows (s < 0) get y = 0 and
 * leave every state untouched; s >= N sets GDN_EF_SLOT_RANGE and the row is
 * handled as padding. The non-negative slots of one call must be distinct.
 * Feed y to the decode as its packed mixed_qkv row (the row strides of
 * gdn_shape, with qk_norm = 1 to normalise q and k in the kernel).
 *   x           (device) dtype [B, C], row b at x + b * x_row_stride.
 *   w           (device) dtype [C, W], the taps of channel c contiguous.
 *   conv_state  (device) dtype [N, W-1, C], read and written (rows s of live
 *               rows only).
 *   y           (device) dtype [B, C], row b at y + b * y_row_stride; written
 *               for every row. x, y and conv_state must not overlap.
 * Sizes: C a multiple of 4, 4 <= C <= 2^20; 2 <= W <= 4; B >= 0, N >= 1;
 * dtype GDN_F32 or GDN_BF16; every base pointer and row 16-byte aligned for
 * fp32, 8-byte aligned for bf16.
 */
typedef struct {
    int32_t B;            /* rows in the call                                    */
    int32_t N;            /* slots in the conv-state pool                        */
    int32_t C;            /* channels (2*Hk*dk + Hv*dv for the mixed_qkv row)    */
    int32_t W;            /* convolution width (taps), 2..4                      */
    int32_t dtype;        /* gdn_dtype of x, w, conv_state and y                 */
    int32_t x_row_stride; /* elements between rows of x; 0 = dense (C)           */
    int32_t y_row_stride; /* elements between rows of y; 0 = dense (C)           */
} gdn_conv_shape;

gdn_status gdn_conv_update(const gdn_conv_shape *shape, const void *x, const void *w,
                           void *conv_state, const int32_t *slot_idx, void *y,
                           int32_t *err_flags, void *stream);

/*
 * gdn_kda_gates -- the gate activations in front of a per-key-gate (KDA)
 * decode (SGLang PR #36821, Technical principle): from the raw projections,
 * per (row b, token t, value head h) and key channel c,
 *     g[b,t,h,c]  = lower_bound * sigmoid(exp(A[h]) * (a[b,t,h,c] + dt_bias[h,c]))
 *     beta[b,t,h] = sigmoid(b_raw[b,t,h])
 * in fp32 (sigmoid(x) = 1 / (1 + exp(-x))). g is a log-decay in
 * [lower_bound, 0] and feeds gdn_replay_decode / gdn_packed_decode with
 * gate = GDN_GATE_KEY, beta their beta.
 *   a, g     (device) fp32 [B, T, Hv, dk], 16-byte aligned.
 *   b, beta  (device) fp32 [B, T, Hv].
 *   A        (device) fp32 [Hv]; dt_bias (device) fp32 [Hv, dk], 16-byte aligned.
 * Sizes: dk a multiple of 4, 4..1024; lower_bound < 0.
 */
typedef struct {
    int32_t B, T, Hv, dk;
    float lower_bound;    /* l < 0: the log-decay's lower bound */
} gdn_gate_shape;

gdn_status gdn_kda_gates(const gdn_gate_shape *shape, const float *a, const float *b,
                         const float *A, const float *dt_bias, float *g, float *beta,
                         void *stream);

/*
 * gdn_hbm_read_probe -- a measurement aid, not a step of the method: streams
 * `nbytes` of device memory at `src` once, in the access pattern of the
 * decode's checkpoint reads (each wavefront 8 KiB in 16-byte loads, the
 * non-temporal load policy), and writes nothing (sink is written only in a
 * case that does not occur). Timed over several launches it gives the read
 * bandwidth this GPU reaches for that pattern, the measured peak the
 * decode's bandwidth is compared with beside the 8 TB/s specification.
 *   src    (device) 16-byte aligned; nbytes a positive multiple of 32 KiB.
 *   sink   (device) one float.
 * Returns GDN_ERR_INVALID_ARG for a null pointer, a bad size or alignment.
 */
gdn_status gdn_hbm_read_probe(const void *src, size_t nbytes, float *sink, void *stream);

/*
 * gdn_hbm_copy_probe -- a measurement aid, not a step of the method: copies
 * `nbytes` of device memory from `src` to `dst` in the access pattern of a
 * checkpoint block read and written back (each wavefront 8 KiB in 16-byte
 * loads with the non-temporal policy, then the same bytes stored with the
 * policy of the checkpoint write-back). Timed over several launches it gives
 * the read + write bandwidth this GPU reaches for that pattern, the measured
 * peak the fold and the packed decode are compared with. `dst` may be `src`
 * (an exact copy onto itself: each wavefront loads its 8 KiB before storing
 * them).
 *   src, dst (device) 16-byte aligned; the same buffer or non-overlapping;
 *            nbytes a positive multiple of 32 KiB.
 * Returns GDN_ERR_INVALID_ARG for a null pointer, a bad size or alignment, or
 * buffers that overlap without being the same.
 */
gdn_status gdn_hbm_copy_probe(const void *src, void *dst, size_t nbytes, void *stream);

/* Static description of a status code (never NULL). */
const char *gdn_status_string(gdn_status status);

/* Library ABI version (incremented on any signature change). */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_REPLAY_H */
