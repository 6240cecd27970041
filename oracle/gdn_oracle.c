/*
 * Oracle for the gated delta rule forward pass — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  It shares no code, header or constant with the HIP
 * library: it is the plain definition of the method, written out as a
 * token-by-token loop in double precision, one (batch, head) pair at a time.
 *
 * What it computes (state S is dv x dk, a read is o = S q):
 *
 *   PREDICT_THEN_DECAY (order 0), the recurrence
 *       S_t = alpha_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,  o_t = S_t q_t
 *     as written in the Gated DeltaNet GPU-parallelisation blog (m.lqnn.cn),
 *     section 1.2 (formula, there in the transposed d_k x d_v orientation),
 *     and its affine form A_t = alpha_t I - beta_t k k^T of section 2.2.
 *
 *   DECAY_THEN_PREDICT (order 1): decay first, then predict with the decayed
 *     state, as in the worked GDN example of the DeltaNet illustrated notes
 *     (stay-hungry-time.github.io/deltanet), architectures section, GDN and
 *     KDA paragraphs:  Sbar = S_{t-1} D_t;  S_t = Sbar + beta_t (v_t - Sbar k_t) k_t^T.
 *
 *   Gate kinds: scalar alpha_t per token-head (D_t = alpha_t I), or a vector
 *   alpha_t in R^{dk} per token-head that scales the columns of S, i.e. the
 *   key channels (D_t = Diag(alpha_t)), as in the GLA gating section and the
 *   KDA paragraph of the DeltaNet illustrated notes.
 *
 *   The output is read AFTER the update, with the query, times `scale`
 *   (DeltaNet illustrated notes, DeltaNet section: o_t = S_t q_t).
 *
 * Layouts (row-major, contiguous):
 *   q, k   [B, T, H, dk]      v, out [B, T, H, dv]
 *   alpha  [B, T, H] (scalar gate) or [B, T, H, dk] (channel gate)
 *   beta   [B, T, H]
 *   state0, state_out [B, H, dv, dk]; state0 may be NULL (zero start)
 *
 * Parallelism: OpenMP over (batch, head) pairs only; every pair runs the
 * plain sequential loop.  Returns 0 on success, -1 on a bad argument.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void one_sequence(int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int gate, int order, double scale,
                         const double *q, const double *k, const double *v,
                         const double *alpha, const double *beta,
                         const double *s0, double *out, double *s_out,
                         int64_t b, int64_t h, double *S, double *pred)
{
    /* S is dv x dk, row r = value dimension, column c = key channel */
    if (s0)
        memcpy(S, s0, sizeof(double) * dv * dk);
    else
        memset(S, 0, sizeof(double) * dv * dk);

    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;      /* token-head index */
        const double *kt = k + row * dk;
        const double *qt = q + row * dk;
        const double *vt = v + row * dv;
        const double bt = beta[row];

        if (order == 1) {
            /* decay first: S <- S D_t */
            for (int64_t r = 0; r < dv; ++r)
                for (int64_t c = 0; c < dk; ++c)
                    S[r * dk + c] *= (gate == 0) ? alpha[row] : alpha[row * dk + c];
        }
        /* prediction p = S k_t (with the decayed state under order 1) */
        for (int64_t r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                acc += S[r * dk + c] * kt[c];
            pred[r] = acc;
        }
        if (order == 0) {
            /* decay after the prediction: S <- S D_t */
            for (int64_t r = 0; r < dv; ++r)
                for (int64_t c = 0; c < dk; ++c)
                    S[r * dk + c] *= (gate == 0) ? alpha[row] : alpha[row * dk + c];
        }
        /* correction: S <- S + beta_t (v_t - p) k_t^T */
        for (int64_t r = 0; r < dv; ++r) {
            const double e = bt * (vt[r] - pred[r]);
            for (int64_t c = 0; c < dk; ++c)
                S[r * dk + c] += e * kt[c];
        }
        /* read after the update: o_t = scale * S_t q_t */
        double *ot = out + row * dv;
        for (int64_t r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                acc += S[r * dk + c] * qt[c];
            ot[r] = scale * acc;
        }
    }
    if (s_out)
        memcpy(s_out, S, sizeof(double) * dv * dk);
}

int gdn_oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       int gate, int order, double scale,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *state0, double *out, double *state_out,
                       int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate != 0 && gate != 1) return -1;
    if (order != 0 && order != 1) return -1;
    if (B * H == 0) return 0;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return -1;

    const int64_t pairs = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t b = p / H, h = p % H;
        double *S = (double *)malloc(sizeof(double) * dv * dk);
        double *pred = (double *)malloc(sizeof(double) * dv);
        if (!S || !pred) {
            failed = 1;
        } else {
            one_sequence(T, H, dk, dv, gate, order, scale, q, k, v, alpha, beta,
                         state0 ? state0 + p * dv * dk : NULL, out,
                         state_out ? state_out + p * dv * dk : NULL, b, h, S, pred);
        }
        free(S);
        free(pred);
    }
    return failed ? -1 : 0;
}

/* Threads OpenMP would use by default (reported beside the CPU timing). */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
