/*
 * gdr_oracle.c -- fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (gated_delta_rule_44_amd) never links, imports or calls it, and it shares
 * no code, header, table or helper with the HIP kernels.
 *
 * What it computes.  "Super Apriel: One Checkpoint, Many Speeds" (arXiv
 * 2604.19877; the gist.science technical summary, section 2a "supernet
 * architecture") names two recurrent O(n) mixers: Kimi Delta Attention,
 * gated per key channel, and Gated DeltaNet, gated by one scalar per head.
 * The pages give no formula; the plain reading used here is the standard
 * gated delta rule, per (sequence, head):
 *
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t                       (state AFTER the update)
 *
 * with S in R^{Dv x Dk} (row = value index i, column = key index j), the
 * gate supplied as its logarithm g = ln a <= 0, a_t = exp(g_t) either one
 * value per (token, head) [scalar gate, GDN] or Dk values [channel gate,
 * KDA].  Expanding the product,
 *     S' = S_{t-1} Diag(a_t);   S_t = S' + beta_t (v_t - S' k_t) k_t^T,
 * which is the form evaluated below, one token at a time, in fp64.
 *
 * Inputs are float32 (bf16 and fp32 values are exactly representable) and
 * are widened to double before any arithmetic.  Nothing is chunked, fused
 * or reordered.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Run the recurrence over one (sequence, head) pair.
 *   q,k : token-major rows, row t at  q + t*qk_stride,  Dk values each
 *   v   : row t at v + t*v_stride, Dv values
 *   g   : channel gate: row t at g + t*g_stride, Dk values
 *         scalar gate : value at g[t*g_stride]
 *   beta: value at beta[t*b_stride]
 *   S   : Dv*Dk doubles, holds the initial state on entry and the final
 *         state on exit (row-major, S[i*Dk + j])
 *   o   : row t at o + t*o_stride, Dv doubles
 */
static void recur_one(int T, int Dk, int Dv, int channel_gate, double scale,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta,
                      size_t qk_stride, size_t v_stride, size_t g_stride,
                      size_t b_stride, size_t o_stride,
                      double *S, double *o, double *a, double *kt, double *qt)
{
    for (int t = 0; t < T; ++t) {
        const float *qrow = q + (size_t)t * qk_stride;
        const float *krow = k + (size_t)t * qk_stride;
        const float *vrow = v + (size_t)t * v_stride;
        const double bt = (double)beta[(size_t)t * b_stride];

        for (int j = 0; j < Dk; ++j) {
            kt[j] = (double)krow[j];
            qt[j] = (double)qrow[j];
            a[j] = channel_gate ? exp((double)g[(size_t)t * g_stride + j])
                                : exp((double)g[(size_t)t * g_stride]);
        }

        for (int i = 0; i < Dv; ++i) {
            double *Si = S + (size_t)i * Dk;
            /* S' = S Diag(a): column j scaled by a_j */
            for (int j = 0; j < Dk; ++j)
                Si[j] *= a[j];
            /* (S' k)_i */
            double y = 0.0;
            for (int j = 0; j < Dk; ++j)
                y += Si[j] * kt[j];
            /* S_i += beta (v_i - (S'k)_i) k^T */
            const double u = bt * ((double)vrow[i] - y);
            for (int j = 0; j < Dk; ++j)
                Si[j] += u * kt[j];
            /* o_i = scale * (S_t q)_i with the updated row */
            double oi = 0.0;
            for (int j = 0; j < Dk; ++j)
                oi += Si[j] * qt[j];
            o[(size_t)t * o_stride + i] = scale * oi;
        }
    }
}

/*
 * Packed-batch entry point.
 *
 *   N            number of sequences
 *   cu_seqlens   N+1 non-decreasing offsets into the packed token axis;
 *                sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1])
 *   H, Dk, Dv    heads, key width, value width
 *   channel_gate 1: g is [T_total, H, Dk];  0: g is [T_total, H]
 *   q, k         [T_total, H, Dk] float32
 *   v            [T_total, H, Dv] float32
 *   beta         [T_total, H] float32
 *   h0           [N, H, Dv, Dk] float32, or NULL for zero initial states
 *   o            [T_total, H, Dv] double (written)
 *   ht           [N, H, Dv, Dk] double (written), or NULL
 *   num_threads  OpenMP threads (<= 0: library default)
 *
 * Returns 0 on success, -1 on bad arguments, -2 if scratch allocation
 * failed.  The state is reset to h0[n] at every sequence start, so nothing
 * crosses a cu_seqlens boundary.
 */
int gdr_oracle_forward(int N, const int64_t *cu_seqlens, int H, int Dk, int Dv,
                       int channel_gate, double scale,
                       const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const float *h0,
                       double *o, double *ht, int num_threads)
{
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || !cu_seqlens)
        return -1;
    for (int n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;

    const size_t qk_stride = (size_t)H * Dk;
    const size_t v_stride = (size_t)H * Dv;
    const size_t g_stride = channel_gate ? (size_t)H * Dk : (size_t)H;
    const size_t b_stride = (size_t)H;
    const size_t o_stride = (size_t)H * Dv;
    const size_t SS = (size_t)Dv * Dk;
    const long pairs = (long)N * H;
    int failed = 0;

#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * SS);
        double *a = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *kt = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *qt = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!S || !a || !kt || !qt) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long p = 0; p < pairs; ++p) {
                const int n = (int)(p / H);
                const int h = (int)(p % H);
                const int64_t t0 = cu_seqlens[n];
                const int T = (int)(cu_seqlens[n + 1] - t0);
                const float *h0p = h0 ? h0 + ((size_t)n * H + h) * SS : NULL;
                for (size_t e = 0; e < SS; ++e)
                    S[e] = h0p ? (double)h0p[e] : 0.0;
                recur_one(T, Dk, Dv, channel_gate, scale,
                          q + (size_t)t0 * qk_stride + (size_t)h * Dk,
                          k + (size_t)t0 * qk_stride + (size_t)h * Dk,
                          v + (size_t)t0 * v_stride + (size_t)h * Dv,
                          channel_gate ? g + (size_t)t0 * g_stride + (size_t)h * Dk
                                       : g + (size_t)t0 * g_stride + h,
                          beta + (size_t)t0 * b_stride + h,
                          qk_stride, v_stride, g_stride, b_stride, o_stride,
                          S, o + (size_t)t0 * o_stride + (size_t)h * Dv, a, kt, qt);
                if (ht)
                    memcpy(ht + ((size_t)n * H + h) * SS, S, sizeof(double) * SS);
            }
        }
        free(S);
        free(a);
        free(kt);
        free(qt);
    }
    return failed ? -2 : 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int gdr_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward: the vector-Jacobian product of the recurrence above, for
 * upstream gradients dO of the outputs and dS_T of the final state (the
 * gradients a training step of the mixers needs; the summary's section 2a
 * recurrence differentiated by hand, one token at a time, in fp64).
 *
 * Write one token as  P = S_{t-1} Diag(a_t),  e = v_t - P k_t,
 * S_t = P + beta_t e k_t^T,  o_t = scale S_t q_t.  With R the gradient of
 * the loss with respect to S_t through everything after token t, the
 * gradient with respect to S_t in total is  R' = R + scale do_t q_t^T, and
 *   dq_t    = scale S_t^T do_t
 *   dv_t    = beta_t R' k_t
 *   dbeta_t = e . (R' k_t)
 *   dk_t    = beta_t (R'^T e - P^T (R' k_t))
 *   dP      = R' - beta_t (R' k_t) k_t^T
 *   dg_t[j] = sum_i dP[i][j] P[i][j]     (summed over j for a scalar gate,
 *                                         since da/dg = a)
 *   R      <- dP Diag(a_t)               (the gradient w.r.t. S_{t-1})
 * starting from R = dS_T after the last token; dS_0 is R after the first.
 * The states S_{t-1} are recomputed forward from checkpoints taken every
 * kBlock tokens, the block's states kept while it is walked backwards.
 */
enum { kBlock = 64 };

/* S <- S Diag(a); S += beta (v - S k) k^T; e (Dv) receives v - S' k */
static void fwd_token(int Dk, int Dv, const double *a, const double *kt, double bt,
                      const float *vrow, double *S, double *e)
{
    for (int i = 0; i < Dv; ++i) {
        double *Si = S + (size_t)i * Dk;
        double y = 0.0;
        for (int j = 0; j < Dk; ++j) {
            Si[j] *= a[j];
            y += Si[j] * kt[j];
        }
        e[i] = (double)vrow[i] - y;
        for (int j = 0; j < Dk; ++j)
            Si[j] += bt * e[i] * kt[j];
    }
}

static void token_inputs(int Dk, int channel_gate, const float *krow, const float *grow,
                         double *a, double *kt)
{
    for (int j = 0; j < Dk; ++j) {
        kt[j] = (double)krow[j];
        a[j] = exp((double)(channel_gate ? grow[j] : grow[0]));
    }
}

/*
 * Packed-batch backward.  Layouts as gdr_oracle_forward; do_ like v,
 * dht like h0 (NULL: zero).  Outputs (double, written): dq, dk like q,
 * dv like v, dg like g, dbeta like beta, dh0 [N, H, Dv, Dk] (or NULL).
 * Returns 0, -1 on bad arguments, -2 if scratch allocation failed.
 */
int gdr_oracle_backward(int N, const int64_t *cu_seqlens, int H, int Dk, int Dv,
                        int channel_gate, double scale,
                        const float *q, const float *k, const float *v,
                        const float *g, const float *beta, const float *h0,
                        const float *do_, const float *dht,
                        double *dq, double *dk, double *dv, double *dg, double *dbeta,
                        double *dh0, int num_threads)
{
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || !cu_seqlens)
        return -1;
    int64_t Tmax = 0;
    for (int n = 0; n < N; ++n) {
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -1;
        if (cu_seqlens[n + 1] - cu_seqlens[n] > Tmax)
            Tmax = cu_seqlens[n + 1] - cu_seqlens[n];
    }
    const size_t qk_stride = (size_t)H * Dk;
    const size_t v_stride = (size_t)H * Dv;
    const size_t g_stride = channel_gate ? (size_t)H * Dk : (size_t)H;
    const size_t SS = (size_t)Dv * Dk;
    const size_t nblk_max = (size_t)((Tmax + kBlock - 1) / kBlock);
    const long pairs = (long)N * H;
    int failed = 0;

#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif

#pragma omp parallel
    {
        double *ck = (double *)malloc(sizeof(double) * SS * (nblk_max ? nblk_max : 1));
        double *Sb = (double *)malloc(sizeof(double) * SS * (kBlock + 1));
        double *R = (double *)malloc(sizeof(double) * SS);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *rk = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *a = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *kt = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!ck || !Sb || !R || !e || !rk || !a || !kt) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long p = 0; p < pairs; ++p) {
                const int n = (int)(p / H);
                const int h = (int)(p % H);
                const int64_t t0 = cu_seqlens[n];
                const int T = (int)(cu_seqlens[n + 1] - t0);
                const int nblk = (T + kBlock - 1) / kBlock;
                const size_t pair_off = ((size_t)n * H + h) * SS;
#define ROWQK(base, t) ((base) + (size_t)(t0 + (t)) * qk_stride + (size_t)h * Dk)
#define ROWV(base, t) ((base) + (size_t)(t0 + (t)) * v_stride + (size_t)h * Dv)
#define ROWG(base, t) ((base) + (size_t)(t0 + (t)) * g_stride + (size_t)h * (channel_gate ? Dk : 1))
#define AT(base, t) ((base) + (size_t)(t0 + (t)) * H + h)
                /* forward, keeping the state that enters every block */
                double *S = Sb;
                for (size_t x = 0; x < SS; ++x)
                    S[x] = h0 ? (double)h0[pair_off + x] : 0.0;
                for (int t = 0; t < T; ++t) {
                    if (t % kBlock == 0)
                        memcpy(ck + (size_t)(t / kBlock) * SS, S, sizeof(double) * SS);
                    token_inputs(Dk, channel_gate, ROWQK(k, t), ROWG(g, t), a, kt);
                    fwd_token(Dk, Dv, a, kt, (double)*AT(beta, t), ROWV(v, t), S, e);
                }
                for (size_t x = 0; x < SS; ++x)
                    R[x] = dht ? (double)dht[pair_off + x] : 0.0;
                for (int c = nblk - 1; c >= 0; --c) {
                    const int tb = c * kBlock;
                    const int L = T - tb < kBlock ? T - tb : kBlock;
                    /* the block's states: Sb[u] enters token tb + u */
                    memcpy(Sb, ck + (size_t)c * SS, sizeof(double) * SS);
                    for (int u = 0; u < L; ++u) {
                        memcpy(Sb + (size_t)(u + 1) * SS, Sb + (size_t)u * SS, sizeof(double) * SS);
                        token_inputs(Dk, channel_gate, ROWQK(k, tb + u), ROWG(g, tb + u), a, kt);
                        fwd_token(Dk, Dv, a, kt, (double)*AT(beta, tb + u), ROWV(v, tb + u),
                                  Sb + (size_t)(u + 1) * SS, e);
                    }
                    for (int u = L - 1; u >= 0; --u) {
                        const int t = tb + u;
                        const double *Sp = Sb + (size_t)u * SS;       /* S_{t-1} */
                        const double *St = Sb + (size_t)(u + 1) * SS; /* S_t */
                        const float *qrow = ROWQK(q, t), *vrow = ROWV(v, t), *dorow = ROWV(do_, t);
                        const double bt = (double)*AT(beta, t);
                        token_inputs(Dk, channel_gate, ROWQK(k, t), ROWG(g, t), a, kt);
                        double *dqr = ROWQK(dq, t), *dkr = ROWQK(dk, t), *dvr = ROWV(dv, t);
                        double *dgr = ROWG(dg, t);
                        for (int j = 0; j < Dk; ++j) {
                            dqr[j] = 0.0;
                            dkr[j] = 0.0;
                        }
                        for (int j = 0; j < (channel_gate ? Dk : 1); ++j)
                            dgr[j] = 0.0;
                        double db = 0.0;
                        for (int i = 0; i < Dv; ++i) {
                            const double doi = (double)dorow[i];
                            double *Ri = R + (size_t)i * Dk;
                            const double *Pi_src = Sp + (size_t)i * Dk;
                            const double *Sti = St + (size_t)i * Dk;
                            double y = 0.0, r = 0.0;
                            for (int j = 0; j < Dk; ++j) {
                                Ri[j] += scale * doi * (double)qrow[j];   /* R' */
                                dqr[j] += scale * doi * Sti[j];
                                y += a[j] * Pi_src[j] * kt[j];
                                r += Ri[j] * kt[j];
                            }
                            e[i] = (double)vrow[i] - y;
                            rk[i] = r;
                            dvr[i] = bt * r;
                            db += e[i] * r;
                        }
                        *AT(dbeta, t) = db;
                        for (int i = 0; i < Dv; ++i) {
                            double *Ri = R + (size_t)i * Dk;
                            const double *Pi_src = Sp + (size_t)i * Dk;
                            for (int j = 0; j < Dk; ++j) {
                                const double P = a[j] * Pi_src[j];
                                dkr[j] += bt * (e[i] * Ri[j] - rk[i] * P);
                                const double dP = Ri[j] - bt * rk[i] * kt[j];
                                dgr[channel_gate ? j : 0] += dP * P;
                                Ri[j] = dP * a[j];
                            }
                        }
                    }
                }
                if (dh0)
                    memcpy(dh0 + pair_off, R, sizeof(double) * SS);
#undef ROWQK
#undef ROWV
#undef ROWG
#undef AT
            }
        }
        free(ck);
        free(Sb);
        free(R);
        free(e);
        free(rk);
        free(a);
        free(kt);
    }
    return failed ? -2 : 0;
}
