/*
 * gdn_oracle.c -- CPU oracle for the Gated DeltaNet decode path.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, sequential reference that
 * the parity tests, the smoke check and the benchmark's CPU-baseline leg call.
 * The product (the HIP library) never links, loads or calls it, and it shares
 * no code, header, table or helper with the HIP side.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -lm
 * (no contraction, no flush-to-zero: every operation below rounds exactly as
 * written, in IEEE round-to-nearest-even).
 *
 * Layouts (all row-major, contiguous):
 *   S / ckpt   [N, Hv, dv, dk]   per value head a dv x dk matrix, dk fastest
 *   q, k       [B, Hk, dk]       one token per row
 *   v, o, u    [B, Hv, dv]
 *   g, beta    [B, Hv]           (per-key gate, O6/O7: g [B, Hv, dk])
 *   ring_d     [N, Hv, L, dv]    ring_k [N, Hk, L, dk]    ring_g [N, Hv, L]
 *                                (per-key gate: ring_g [N, Hv, L, dk])
 * Value head h reads key head h / (Hv / Hk) (contiguous GQA groups).
 * A row whose slot index is negative is a padding row: its outputs are zero
 * and no state is touched.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * O1 -- one decode token of the gated delta rule, in float64.
 *
 * Follows the recurrence as the ReplaySSM blog (llm.rainlin.net, section 1,
 * "Decode state cost") defines it for one value head, with alpha = exp(g):
 *     S~  = alpha * S_{t-1}
 *     u   = beta * (v - S~ k)
 *     S_t = S~ + u k^T
 *     y   = S_t q
 * The state is materialised first and the output read from the new state, so
 * this function does not use the output-only factorisation of the decode
 * kernels; the tests check that factorisation against it.
 *
 * u_out (nullable) receives u, the correction vector the ring stores.
 */
void oracle_gdn_step_f64(int32_t B, int32_t N, int32_t Hv, int32_t Hk,
                         int32_t dk, int32_t dv, const int32_t *slot,
                         double *S, const double *q, const double *k,
                         const double *v, const double *g, const double *beta,
                         double *o, double *u_out)
{
    const int32_t G = Hv / Hk;
    /* (row, value head) pairs are independent (the slots of one call are
       distinct); a timing build with OpenMP runs them on several threads */
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t s = slot[b];
            double *ob = o + ((size_t)b * Hv + h) * dv;
            double *ub = u_out ? u_out + ((size_t)b * Hv + h) * dv : NULL;
            if (s < 0 || s >= N) {
                for (int32_t i = 0; i < dv; ++i) {
                    ob[i] = 0.0;
                    if (ub) ub[i] = 0.0;
                }
                continue;
            }
            const int32_t hk = h / G;
            double *Sh = S + ((size_t)s * Hv + h) * dv * dk;
            const double *qb = q + ((size_t)b * Hk + hk) * dk;
            const double *kb = k + ((size_t)b * Hk + hk) * dk;
            const double *vb = v + ((size_t)b * Hv + h) * dv;
            const double alpha = exp(g[(size_t)b * Hv + h]);
            const double bt = beta[(size_t)b * Hv + h];

            /* S~ = alpha * S */
            for (size_t e = 0; e < (size_t)dv * dk; ++e) Sh[e] = alpha * Sh[e];
            /* u = beta * (v - S~ k), then S = S~ + u k^T, row by row */
            for (int32_t i = 0; i < dv; ++i) {
                double *row = Sh + (size_t)i * dk;
                double sk = 0.0;
                for (int32_t j = 0; j < dk; ++j) sk += row[j] * kb[j];
                const double u = bt * (vb[i] - sk);
                if (ub) ub[i] = u;
                for (int32_t j = 0; j < dk; ++j) row[j] = row[j] + u * kb[j];
            }
            /* y = S_t q */
            for (int32_t i = 0; i < dv; ++i) {
                const double *row = Sh + (size_t)i * dk;
                double y = 0.0;
                for (int32_t j = 0; j < dk; ++j) y += row[j] * qb[j];
                ob[i] = y;
            }
        }
    }
}

/*
 * O1, fp32 instance -- the same recurrence, statement for statement, in
 * float32 (exp in double, rounded once). Used by the benchmark's CPU baseline
 * (the plain read-update-write decode a CPU would run) and for the fp32 noise
 * floor; parity is always judged against the fp64 function above.
 */
void oracle_gdn_step_f32(int32_t B, int32_t N, int32_t Hv, int32_t Hk,
                         int32_t dk, int32_t dv, const int32_t *slot,
                         float *S, const float *q, const float *k,
                         const float *v, const float *g, const float *beta,
                         float *o)
{
    const int32_t G = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t s = slot[b];
            float *ob = o + ((size_t)b * Hv + h) * dv;
            if (s < 0 || s >= N) {
                for (int32_t i = 0; i < dv; ++i) ob[i] = 0.0f;
                continue;
            }
            const int32_t hk = h / G;
            float *Sh = S + ((size_t)s * Hv + h) * dv * dk;
            const float *qb = q + ((size_t)b * Hk + hk) * dk;
            const float *kb = k + ((size_t)b * Hk + hk) * dk;
            const float *vb = v + ((size_t)b * Hv + h) * dv;
            const float alpha = (float)exp((double)g[(size_t)b * Hv + h]);
            const float bt = beta[(size_t)b * Hv + h];

            for (size_t e = 0; e < (size_t)dv * dk; ++e) Sh[e] = alpha * Sh[e];
            for (int32_t i = 0; i < dv; ++i) {
                float *row = Sh + (size_t)i * dk;
                float sk = 0.0f;
                for (int32_t j = 0; j < dk; ++j) sk += row[j] * kb[j];
                const float u = bt * (vb[i] - sk);
                for (int32_t j = 0; j < dk; ++j) row[j] = row[j] + u * kb[j];
            }
            for (int32_t i = 0; i < dv; ++i) {
                const float *row = Sh + (size_t)i * dk;
                float y = 0.0f;
                for (int32_t j = 0; j < dk; ++j) y += row[j] * qb[j];
                ob[i] = y;
            }
        }
    }
}

/* Threads of a timing build (OpenMP); the parity build has one. Returns the
   number of threads the steps will use. */
int32_t oracle_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * O3 -- fold of a slot's valid ring entries into its fp32 checkpoint, with the
 * rounding pinned.
 *
 * Per element x of the checkpoint and per ring entry j = 0 .. p-1 in order:
 *     a = RN_f32(exp_f64(g_j))         the entry's decay, rounded once to fp32
 *     t = RN_f32(a * x)                the decayed state, a separately rounded multiply
 *     x = fma_f32(d_j[v], k_j[k], t)   the rank-1 update, one fused multiply-add
 * This is the recurrence S <- alpha*S + d k^T driven by the stored entries, in
 * the two-instruction form SGLang PR #42388 ("The idea") prescribes for an exact
 * replay: the decayed state is rounded on its own and the update is a single
 * FMA. It is the checkpoint update SGLang PR #36821 (Technical principle)
 * performs at commit, where the kept entries are applied to the checkpoint in
 * place, here for the GDN (d, k, g) ring. The ring values are taken as their
 * exact fp32 upcasts.
 *
 * order = 0 is the pinned form above. order = 1 is a deliberately different
 * association, x = fma_f32(a, x, RN_f32(d*k)), kept only so that a test can
 * show the bitwise comparison detects a change of operation order.
 *
 * write_pos[s] is the number of valid entries p of slot s; after the fold the
 * slot's write_pos is reset to 0. Rows with a negative or out-of-range slot,
 * or with p outside [0, L], are skipped.
 */
void oracle_fold_f32(int32_t B, int32_t N, int32_t Hv, int32_t Hk, int32_t dk,
                     int32_t dv, int32_t L, const int32_t *slot,
                     int32_t *write_pos, float *ckpt, const float *ring_d,
                     const float *ring_k, const float *ring_g, int32_t order)
{
    const int32_t G = Hv / Hk;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slot[b];
        if (s < 0 || s >= N) continue;
        const int32_t p = write_pos[s];
        if (p < 0 || p > L) continue;
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t hk = h / G;
            float *X = ckpt + ((size_t)s * Hv + h) * dv * dk;
            for (int32_t j = 0; j < p; ++j) {
                const float a = (float)exp((double)ring_g[((size_t)s * Hv + h) * L + j]);
                const float *dj = ring_d + (((size_t)s * Hv + h) * L + j) * dv;
                const float *kj = ring_k + (((size_t)s * Hk + hk) * L + j) * dk;
                for (int32_t i = 0; i < dv; ++i) {
                    for (int32_t c = 0; c < dk; ++c) {
                        float *x = X + (size_t)i * dk + c;
                        if (order == 0) {
                            const float t = a * (*x);
                            *x = fmaf(dj[i], kj[c], t);
                        } else {
                            const float dk_ = dj[i] * kj[c];
                            *x = fmaf(a, *x, dk_);
                        }
                    }
                }
            }
        }
    }
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slot[b];
        if (s < 0 || s >= N) continue;
        const int32_t p = write_pos[s];
        if (p < 0 || p > L) continue;
        write_pos[s] = 0;
    }
}

/*
 * O6 -- one decode token of the delta rule with a per-key gate (KDA), in
 * float64.
 *
 * SGLang PR #28451 (Modifications, item 7: one kernel for GDN and KDA) states
 * that KDA is the same delta-rule decode with the decay applied per key
 * channel instead of per head: the state update is S' = S Diag(a) + d k^T with
 * a = exp(g) a vector over the dk key channels. Written out for one value head
 * in the same materialise-then-read order as O1:
 *     S~  = S_{t-1} Diag(a)       column c of the [dv x dk] state times a[c]
 *     u   = beta * (v - S~ k)
 *     S_t = S~ + u k^T
 *     y   = S_t q
 * With every a[c] equal this is O1 operation for operation.
 * g is [B, Hv, dk] (one log-decay per key channel); everything else as O1.
 */
void oracle_kda_step_f64(int32_t B, int32_t N, int32_t Hv, int32_t Hk,
                         int32_t dk, int32_t dv, const int32_t *slot,
                         double *S, const double *q, const double *k,
                         const double *v, const double *g, const double *beta,
                         double *o, double *u_out)
{
    const int32_t G = Hv / Hk;
    /* (row, value head) pairs are independent (the slots of one call are
       distinct); a timing build with OpenMP runs them on several threads */
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t s = slot[b];
            double *ob = o + ((size_t)b * Hv + h) * dv;
            double *ub = u_out ? u_out + ((size_t)b * Hv + h) * dv : NULL;
            if (s < 0 || s >= N) {
                for (int32_t i = 0; i < dv; ++i) {
                    ob[i] = 0.0;
                    if (ub) ub[i] = 0.0;
                }
                continue;
            }
            const int32_t hk = h / G;
            double *Sh = S + ((size_t)s * Hv + h) * dv * dk;
            const double *qb = q + ((size_t)b * Hk + hk) * dk;
            const double *kb = k + ((size_t)b * Hk + hk) * dk;
            const double *vb = v + ((size_t)b * Hv + h) * dv;
            const double *gb = g + ((size_t)b * Hv + h) * dk;
            const double bt = beta[(size_t)b * Hv + h];

            /* S~ = S Diag(a): every row scaled channel by channel */
            for (int32_t i = 0; i < dv; ++i)
                for (int32_t j = 0; j < dk; ++j)
                    Sh[(size_t)i * dk + j] = exp(gb[j]) * Sh[(size_t)i * dk + j];
            /* u = beta * (v - S~ k), then S = S~ + u k^T, row by row */
            for (int32_t i = 0; i < dv; ++i) {
                double *row = Sh + (size_t)i * dk;
                double sk = 0.0;
                for (int32_t j = 0; j < dk; ++j) sk += row[j] * kb[j];
                const double u = bt * (vb[i] - sk);
                if (ub) ub[i] = u;
                for (int32_t j = 0; j < dk; ++j) row[j] = row[j] + u * kb[j];
            }
            /* y = S_t q */
            for (int32_t i = 0; i < dv; ++i) {
                const double *row = Sh + (size_t)i * dk;
                double y = 0.0;
                for (int32_t j = 0; j < dk; ++j) y += row[j] * qb[j];
                ob[i] = y;
            }
        }
    }
}

/*
 * O7 -- fold of a slot's valid ring entries into its fp32 checkpoint with a
 * per-key gate, rounding pinned as in O3 but with one decay per key channel:
 * per element x = ckpt[v, c] and per entry j = 0 .. p-1 in order,
 *     a = RN_f32(exp_f64(g_j[c]))
 *     t = RN_f32(a * x)
 *     x = fma_f32(d_j[v], k_j[c], t)
 * (the KDA update S <- S Diag(a) + d k^T of SGLang PR #28451, Modifications
 * item 7, in the two-instruction form of SGLang PR #42388, "The idea").
 * ring_g is [N, Hv, L, dk]. Rows, cursors and the reset as O3.
 */
void oracle_fold_kda_f32(int32_t B, int32_t N, int32_t Hv, int32_t Hk, int32_t dk,
                         int32_t dv, int32_t L, const int32_t *slot,
                         int32_t *write_pos, float *ckpt, const float *ring_d,
                         const float *ring_k, const float *ring_g)
{
    const int32_t G = Hv / Hk;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slot[b];
        if (s < 0 || s >= N) continue;
        const int32_t p = write_pos[s];
        if (p < 0 || p > L) continue;
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t hk = h / G;
            float *X = ckpt + ((size_t)s * Hv + h) * dv * dk;
            for (int32_t j = 0; j < p; ++j) {
                const float *gj = ring_g + (((size_t)s * Hv + h) * L + j) * dk;
                const float *dj = ring_d + (((size_t)s * Hv + h) * L + j) * dv;
                const float *kj = ring_k + (((size_t)s * Hk + hk) * L + j) * dk;
                for (int32_t i = 0; i < dv; ++i) {
                    for (int32_t c = 0; c < dk; ++c) {
                        float *x = X + (size_t)i * dk + c;
                        const float a = (float)exp((double)gj[c]);
                        const float t = a * (*x);
                        *x = fmaf(dj[i], kj[c], t);
                    }
                }
            }
        }
    }
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slot[b];
        if (s < 0 || s >= N) continue;
        const int32_t p = write_pos[s];
        if (p < 0 || p > L) continue;
        write_pos[s] = 0;
    }
}

/* ABI version of this oracle library, for the loader's sanity check. */
int32_t oracle_version(void) { return 2; }
