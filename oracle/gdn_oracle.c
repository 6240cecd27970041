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

/*
 * Backward pass (reverse mode) of the forward above — TEST INFRASTRUCTURE ONLY.
 *
 * The pages give the forward recurrence but no gradient formulas; these are
 * the chain rule applied to one token step, written row by row (rows of S are
 * value dimensions and evolve independently given the token's k, gate, beta).
 * For token t, with the decay vector d (alpha_t in every channel for a scalar
 * gate, alpha_t itself for a channel gate) and the row r of the state before
 * the token S_r:
 *   X_r = S_r (predict-then-decay) or S_r * d (decay-then-predict, elementwise)
 *   p_r = X_r . k,   e_r = beta (v_r - p_r)
 *   S'_r = S_r * d + e_r k  (predict-then-decay)  or  X_r + e_r k  (decay-then-predict)
 *   o_r = scale (S'_r . q)
 * Given G_r = dL/dS'_r (the gradient carried back from later tokens plus
 * scale do_r q from this token's read), with gk_r = G_r . k:
 *   dq   += scale sum_r do_r S'_r
 *   dv_r  = beta gk_r
 *   dbeta = sum_r gk_r (v_r - p_r)
 *   dk    = sum_r (e_r G_r - beta gk_r X_r)
 *   predict-then-decay:  dS_r = G_r * d - beta gk_r k;   dd = sum_r G_r * S_r
 *   decay-then-predict:  dX_r = G_r - beta gk_r k;  dS_r = dX_r * d;  dd = sum_r dX_r * S_r
 *   scalar gate: dalpha_t = sum over channels of dd; channel gate: dalpha_t = dd.
 * Sweeping t = T-1 .. 0 from dL/dS_T (ds_out, or zero) leaves dL/dS_0.
 * The states S_0 .. S_{T-1} come from a forward sweep kept whole in memory
 * ((T + 1) dv dk doubles per (batch, head) in flight).
 *
 * dout [B, T, H, dv]; ds_out, ds0 [B, H, dv, dk] (either may be NULL);
 * dq, dk [B, T, H, dk]; dv [B, T, H, dv]; dalpha shaped as alpha; dbeta [B, T, H].
 */
static void one_backward(int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int gate, int order, double scale,
                         const double *q, const double *k, const double *v,
                         const double *alpha, const double *beta,
                         const double *s0, const double *dout, const double *ds_out,
                         double *dq, double *dkk, double *dvv, double *dalpha,
                         double *dbeta, double *ds0, int64_t b, int64_t h,
                         double *Sall, double *G, double *d, double *X,
                         double *pred)
{
    const int64_t DD = dv * dk;
    /* forward sweep: Sall[t] = state before token t, t = 0 .. T */
    if (s0)
        memcpy(Sall, s0, sizeof(double) * DD);
    else
        memset(Sall, 0, sizeof(double) * DD);
    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        const double *S = Sall + t * DD;
        double *Sn = Sall + (t + 1) * DD;
        const double *kt = k + row * dk;
        for (int64_t c = 0; c < dk; ++c)
            d[c] = gate == 0 ? alpha[row] : alpha[row * dk + c];
        for (int64_t r = 0; r < dv; ++r) {
            double p = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                X[c] = order == 0 ? S[r * dk + c] : S[r * dk + c] * d[c];
                p += X[c] * kt[c];
            }
            const double e = beta[row] * (v[row * dv + r] - p);
            for (int64_t c = 0; c < dk; ++c)
                Sn[r * dk + c] = (order == 0 ? S[r * dk + c] * d[c] : X[c]) + e * kt[c];
        }
    }
    /* reverse sweep */
    if (ds_out)
        memcpy(G, ds_out, sizeof(double) * DD);
    else
        memset(G, 0, sizeof(double) * DD);
    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = (b * T + t) * H + h;
        const double *S = Sall + t * DD;
        const double *Sn = Sall + (t + 1) * DD;
        const double *kt = k + row * dk;
        const double *qt = q + row * dk;
        const double bt = beta[row];
        double *dqt = dq + row * dk, *dkt = dkk + row * dk;
        for (int64_t c = 0; c < dk; ++c) {
            d[c] = gate == 0 ? alpha[row] : alpha[row * dk + c];
            dqt[c] = 0.0;
            dkt[c] = 0.0;
        }
        double db = 0.0;
        double *dd = pred;  /* dk doubles of scratch for dd */
        for (int64_t c = 0; c < dk; ++c) dd[c] = 0.0;
        for (int64_t r = 0; r < dv; ++r) {
            const double dor = dout[row * dv + r];
            double *Gr = G + r * dk;
            double p = 0.0, gk = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                X[c] = order == 0 ? S[r * dk + c] : S[r * dk + c] * d[c];
                p += X[c] * kt[c];
                Gr[c] += scale * dor * qt[c];
                dqt[c] += scale * dor * Sn[r * dk + c];
            }
            for (int64_t c = 0; c < dk; ++c) gk += Gr[c] * kt[c];
            const double e = bt * (v[row * dv + r] - p);
            dvv[row * dv + r] = bt * gk;
            db += gk * (v[row * dv + r] - p);
            for (int64_t c = 0; c < dk; ++c) {
                dkt[c] += e * Gr[c] - bt * gk * X[c];
                if (order == 0) {
                    dd[c] += Gr[c] * S[r * dk + c];
                    Gr[c] = Gr[c] * d[c] - bt * gk * kt[c];
                } else {
                    const double dx = Gr[c] - bt * gk * kt[c];
                    dd[c] += dx * S[r * dk + c];
                    Gr[c] = dx * d[c];
                }
            }
        }
        dbeta[row] = db;
        if (gate == 0) {
            double s = 0.0;
            for (int64_t c = 0; c < dk; ++c) s += dd[c];
            dalpha[row] = s;
        } else {
            for (int64_t c = 0; c < dk; ++c) dalpha[row * dk + c] = dd[c];
        }
    }
    if (ds0)
        memcpy(ds0, G, sizeof(double) * DD);
}

int gdn_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int gate, int order, double scale,
                        const double *q, const double *k, const double *v,
                        const double *alpha, const double *beta,
                        const double *state0, const double *dout, const double *ds_out,
                        double *dq, double *dkk, double *dvv, double *dalpha,
                        double *dbeta, double *ds0, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate != 0 && gate != 1) return -1;
    if (order != 0 && order != 1) return -1;
    if (B * H == 0) return 0;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !dout || !dq || !dkk || !dvv ||
                  !dalpha || !dbeta)) return -1;

    const int64_t pairs = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t b = p / H, h = p % H;
        double *Sall = (double *)malloc(sizeof(double) * (T + 1) * dv * dk);
        double *G = (double *)malloc(sizeof(double) * dv * dk);
        double *d = (double *)malloc(sizeof(double) * dk);
        double *X = (double *)malloc(sizeof(double) * dk);
        double *pred = (double *)malloc(sizeof(double) * (dk > dv ? dk : dv));
        if (!Sall || !G || !d || !X || !pred) {
            failed = 1;
        } else {
            one_backward(T, H, dk, dv, gate, order, scale, q, k, v, alpha, beta,
                         state0 ? state0 + p * dv * dk : NULL, dout,
                         ds_out ? ds_out + p * dv * dk : NULL, dq, dkk, dvv, dalpha,
                         dbeta, ds0 ? ds0 + p * dv * dk : NULL, b, h, Sall, G, d, X, pred);
        }
        free(Sall);
        free(G);
        free(d);
        free(X);
        free(pred);
    }
    return failed ? -1 : 0;
}
