/*
 * ssd_oracle.c -- plain, slow, fp64 CPU reference for the Mamba-2 SSD recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path never links it.
 * It shares no code, header or constant with the GPU library.
 *
 * What it computes (one token at a time, per sequence and head):
 *
 *   a_t        = exp(dt_t * A_h)
 *   h_t[n][p]  = a_t * h_{t-1}[n][p] + dt_t * x_t[p] * B_t[n]
 *   y_t[p]     = sum_n C_t[n] * h_t[n][p] + D_h * x_t[p]
 *
 * Passages followed:
 *  - COREY: Entropy-Guided Runtime Chunk Scheduling for Selective Scan Kernels,
 *    section 3.1 (Preliminaries): the generic selective SSM update
 *    h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t + D_t x_t.
 *  - Compiler-First State Space Duality and Portable O(1) Autoregressive Caching
 *    for Inference, Abstract: in SSD the state transition of head h is a
 *    scalar, exp(dt*A_h), times the identity.
 *  - Mamba-2 SSD fused layer via VGpuWarp -- design sketch, "Lane mapping" and
 *    "S2 RESULT": each (head, head_dim) channel sweeps d_state with one exp per
 *    step; the state h is an N x P matrix per head.
 *  - Recurrence Scan (poot docs), "One equation, one packed result": the scan
 *    returns the output and the carried state, and a CPU oracle is compared on
 *    every element of both.
 * Readings where the pages are silent (documented with the build): dt is the
 * final positive step (softplus already applied by the caller), A_h is the
 * negative decay rate itself, the input term is dt*x (x) B with no zero-order-hold
 * factor, D is a per-head scalar skip, head h reads group floor(h*G/H).
 *
 * The decode-layer operations around the scan (the causal conv1d step and
 * the gated RMS norm), the Mamba-1 selective scan, the reverse-mode gradients
 * of the recurrence (the backward half of a training step) and the gated
 * delta rule are at the end of this file, with their own passages.
 *
 * Inputs are float32 (bf16 inputs are upcast exactly before the call); all
 * arithmetic and the outputs are float64.  Layouts are row-major:
 *   x [T][H][P], dt [T][H], A [H], B [T][G][N], C [T][G][N], D [H],
 *   state [nseq][H][N][P], y [T][H][P].
 * Sequences are packed along T; sequence s covers tokens cu[s] .. cu[s+1]-1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Advance one (sequence, head) state by one token and write that token's output. */
static void ssd_token(double *h, const float *x, double dt, double A,
                      const float *B, const float *C, double D, double *y,
                      int P, int N)
{
    const double a = exp(dt * A);
    for (int n = 0; n < N; ++n) {
        const double bn = (double)B[n];
        for (int p = 0; p < P; ++p)
            h[(size_t)n * P + p] = a * h[(size_t)n * P + p] + dt * (double)x[p] * bn;
    }
    for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n)
            acc += (double)C[n] * h[(size_t)n * P + p];
        y[p] = acc + D * (double)x[p];
    }
}

/*
 * Whole-sequence recurrence for every (sequence, head) pair.
 * h0 may be NULL (zero initial state).  h_out may be NULL (not written).
 * cu has nseq+1 entries, cu[0] = 0, non-decreasing.
 * Returns 0, or -1 on an invalid argument.
 */
int ssd_ref_prefill(const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D,
                    const double *h0, const int64_t *cu, int nseq,
                    int H, int P, int N, int G,
                    double *y, double *h_out, int nthreads)
{
    if (!x || !dt || !A || !B || !C || !D || !cu || !y) return -1;
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    for (int s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    const long units = (long)nseq * H;
    if (nthreads <= 0) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long u = 0; u < units; ++u) {
        const int s = (int)(u / H), hd = (int)(u % H);
        const int g = (int)(((long)hd * G) / H);
        double *h = (double *)malloc(sizeof(double) * (size_t)N * P);
        if (!h) { bad = 1; continue; }
        const size_t hoff = ((size_t)s * H + hd) * (size_t)N * P;
        if (h0) memcpy(h, h0 + hoff, sizeof(double) * (size_t)N * P);
        else memset(h, 0, sizeof(double) * (size_t)N * P);
        for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
            ssd_token(h, x + ((size_t)t * H + hd) * P, (double)dt[(size_t)t * H + hd],
                      (double)A[hd], B + ((size_t)t * G + g) * N,
                      C + ((size_t)t * G + g) * N, (double)D[hd],
                      y + ((size_t)t * H + hd) * P, P, N);
        }
        if (h_out) memcpy(h_out + hoff, h, sizeof(double) * (size_t)N * P);
        free(h);
    }
    return bad ? -1 : 0;
}

/*
 * One decode token for a batch of independent states, updated in place.
 * x [b][H][P], dt [b][H], B, C [b][G][N], h [b][H][N][P] (float64), y [b][H][P].
 */
int ssd_ref_step(const float *x, const float *dt, const float *A,
                 const float *B, const float *C, const float *D,
                 double *h, double *y, int batch, int H, int P, int N, int G,
                 int nthreads)
{
    if (!x || !dt || !A || !B || !C || !D || !h || !y) return -1;
    if (batch < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    const long units = (long)batch * H;
    if (nthreads <= 0) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long u = 0; u < units; ++u) {
        const int b = (int)(u / H), hd = (int)(u % H);
        const int g = (int)(((long)hd * G) / H);
        ssd_token(h + ((size_t)b * H + hd) * (size_t)N * P,
                  x + ((size_t)b * H + hd) * P, (double)dt[(size_t)b * H + hd],
                  (double)A[hd], B + ((size_t)b * G + g) * N,
                  C + ((size_t)b * G + g) * N, (double)D[hd],
                  y + ((size_t)b * H + hd) * P, P, N);
    }
    return 0;
}

/*
 * Decode-layer operations on either side of the scan.  Mamba-2 SSD fused
 * layer via VGpuWarp -- design sketch lists them among the layer steps to move
 * onto the device: the causal conv1d step (a per-channel FIR over d_conv taps
 * with a rolling buffer) and the gated RMS norm (y times silu(z), then the root
 * mean square over d_inner, times norm_w).
 *
 * Causal conv1d, one token, per channel c: the window win[c][0..W-1] (oldest
 * first) drops win[c][0], moves the rest down one place and takes u[c] as its
 * newest entry win[c][W-1]; the output is
 *     v = bias[c] + sum_k w[c][k] * win[c][k]          (bias NULL: 0)
 * and, when silu != 0, v * sigmoid(v).
 * Layouts: u [b][C], win [b][C][W] fp64 (updated in place), w [C][W],
 * bias [C], out [b][C] fp64.
 */
int ssd_ref_conv1d_step(const float *u, double *win, const float *w, const float *bias,
                        int silu, int batch, int channels, int width, double *out)
{
    if (batch < 0 || channels < 1 || width < 1)
        return -1;
    for (int b = 0; b < batch; ++b) {
        for (int c = 0; c < channels; ++c) {
            double *wd = win + ((size_t)b * channels + c) * width;
            for (int k = 0; k + 1 < width; ++k)
                wd[k] = wd[k + 1];
            wd[width - 1] = (double)u[(size_t)b * channels + c];
            double v = bias ? (double)bias[c] : 0.0;
            for (int k = 0; k < width; ++k)
                v += (double)w[(size_t)c * width + k] * wd[k];
            if (silu)
                v = v / (1.0 + exp(-v));
            out[(size_t)b * channels + c] = v;
        }
    }
    return 0;
}

/*
 * Gated RMS norm over the D channels of one token:
 *     g = y * silu(z),   out = g / sqrt(mean(g^2) + eps) * w
 * Layouts: y [b][D] fp64, z [b][D], w [D], out [b][D] fp64.
 */
int ssd_ref_gated_rmsnorm(const double *y, const float *z, const float *w, double eps,
                          int batch, int dim, double *out)
{
    if (batch < 0 || dim < 1 || eps < 0.0)
        return -1;
    for (int b = 0; b < batch; ++b) {
        double ss = 0.0;
        for (int d = 0; d < dim; ++d) {
            const double zz = (double)z[(size_t)b * dim + d];
            const double g = y[(size_t)b * dim + d] * (zz / (1.0 + exp(-zz)));
            out[(size_t)b * dim + d] = g;
            ss += g * g;
        }
        const double r = 1.0 / sqrt(ss / dim + eps);
        for (int d = 0; d < dim; ++d)
            out[(size_t)b * dim + d] *= r * (double)w[d];
    }
    return 0;
}

/*
 * Mamba-1 selective scan: the generic selective update of COREY: Entropy-Guided
 * Runtime Chunk Scheduling for Selective Scan Kernels, section 3.1
 * (h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t + D_t x_t) with a diagonal
 * transition per channel and state, discretised as the SSD path above:
 *
 *   h_t[d][n] = exp(dt_t[d] * A[d][n]) * h_{t-1}[d][n] + dt_t[d] * B_t[n] * x_t[d]
 *   y_t[d]    = sum_n C_t[n] * h_t[d][n] + D[d] * x_t[d]
 *
 * (the kernel that section 5.1 of that page times at batch 1, d 1024, L 4096,
 * d_state 16).  Layouts: x, dt [b][L][d]; A [d][N]; B, C [b][L][N]; D [d];
 * h0, h_out [b][d][N] (h0 NULL: zeros); y [b][L][d].
 */
int ssd_ref_selective_scan(const float *x, const float *dt, const float *A, const float *B,
                           const float *C, const float *D, const double *h0, int batch, int L,
                           int dim, int N, double *y, double *h_out, int nthreads)
{
    if (batch < 0 || L < 0 || dim < 1 || N < 1)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long u = 0; u < (long)batch * dim; ++u) {
        const int b = (int)(u / dim), d = (int)(u % dim);
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        for (int n = 0; n < N; ++n)
            h[n] = h0 ? h0[((size_t)b * dim + d) * N + n] : 0.0;
        for (int t = 0; t < L; ++t) {
            const size_t td = ((size_t)b * L + t) * dim + d;
            const double dtv = (double)dt[td], xv = (double)x[td];
            const float *Bt = B + ((size_t)b * L + t) * N;
            const float *Ct = C + ((size_t)b * L + t) * N;
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                h[n] = exp(dtv * (double)A[(size_t)d * N + n]) * h[n] + dtv * (double)Bt[n] * xv;
                acc += (double)Ct[n] * h[n];
            }
            y[td] = acc + (double)D[d] * xv;
        }
        if (h_out)
            for (int n = 0; n < N; ++n)
                h_out[((size_t)b * dim + d) * N + n] = h[n];
        free(h);
    }
    return 0;
}

/*
 * Gradients of the SSD recurrence above (reverse mode, fp64) for a scalar loss
 * L with dL/dy = dy [T][H][P] and dL/dh_out = dh_out [nseq][H][N][P] (NULL: 0).
 * Per (sequence, head) the states h_t are recomputed forward and kept; then,
 * walking the tokens backward with g_t = dL/dh_t (everything downstream of
 * h_t):
 *   g_t        = C_t (x) dy_t + a_{t+1} g_{t+1}     (g of the last token adds dh_out)
 *   dC_t[n]   += sum_p h_t[n][p] dy_t[p]
 *   dx_t[p]    = D dy_t[p] + dt_t sum_n B_t[n] g_t[n][p]
 *   dB_t[n]   += dt_t sum_p x_t[p] g_t[n][p]
 *   da_t       = sum_{n,p} g_t[n][p] h_{t-1}[n][p]          (a_t = exp(dt_t A))
 *   ddt_t      = A a_t da_t + sum_{n,p} g_t[n][p] x_t[p] B_t[n]
 *   dA        += dt_t a_t da_t;   dD += sum_p dy_t[p] x_t[p];   dh0 = a_first g_first
 * dB and dC [T][G][N] sum over the heads of a group; dA, dD [H] over every
 * sequence.  This is the chain rule through the unrolled recurrence, the
 * training-side counterpart of the forward scan (Compiler-First State Space
 * Duality and Portable O(1) Autoregressive Caching for Inference, Table 13
 * times forward plus backward steps).  Arrays as in ssd_ref_prefill; every
 * output is written (zeros where nothing flows).
 */
int ssd_ref_prefill_backward(const float *x, const float *dt, const float *A,
                             const float *B, const float *C, const float *D,
                             const double *h0, const int64_t *cu, int nseq,
                             int H, int P, int N, int G,
                             const double *dy, const double *dh_out,
                             double *dx, double *ddt, double *dA, double *dB,
                             double *dC, double *dD, double *dh0, int nthreads)
{
    if (!x || !dt || !A || !B || !C || !D || !cu || !dy) return -1;
    if (!dx || !ddt || !dA || !dB || !dC || !dD) return -1;
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    for (int s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    const int64_t T = nseq > 0 ? cu[nseq] : 0;
    const size_t NP = (size_t)N * P;
    /* per-head contributions, reduced over heads / sequences afterwards */
    double *dBh = (double *)calloc((size_t)(T > 0 ? T : 1) * H * N, sizeof(double));
    double *dCh = (double *)calloc((size_t)(T > 0 ? T : 1) * H * N, sizeof(double));
    double *dAs = (double *)calloc((size_t)(nseq > 0 ? nseq : 1) * H, sizeof(double));
    double *dDs = (double *)calloc((size_t)(nseq > 0 ? nseq : 1) * H, sizeof(double));
    if (!dBh || !dCh || !dAs || !dDs) { free(dBh); free(dCh); free(dAs); free(dDs); return -1; }
    const long units = (long)nseq * H;
    if (nthreads <= 0) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long u = 0; u < units; ++u) {
        const int s = (int)(u / H), hd = (int)(u % H);
        const int g = (int)(((long)hd * G) / H);
        const int64_t t0 = cu[s], L = cu[s + 1] - cu[s];
        const double Ah = (double)A[hd], Dh = (double)D[hd];
        const size_t hoff = ((size_t)s * H + hd) * NP;
        /* hs[k] = state after k tokens (hs[0] = h0) */
        double *hs = (double *)malloc(sizeof(double) * NP * (size_t)(L + 1));
        double *gg = (double *)malloc(sizeof(double) * NP);
        if (!hs || !gg) { bad = 1; free(hs); free(gg); continue; }
        if (h0) memcpy(hs, h0 + hoff, sizeof(double) * NP);
        else memset(hs, 0, sizeof(double) * NP);
        for (int64_t k = 0; k < L; ++k) {
            const int64_t t = t0 + k;
            const double dtv = (double)dt[(size_t)t * H + hd], a = exp(dtv * Ah);
            const float *xt = x + ((size_t)t * H + hd) * P, *Bt = B + ((size_t)t * G + g) * N;
            const double *hp = hs + NP * (size_t)k;
            double *hn = hs + NP * (size_t)(k + 1);
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p)
                    hn[(size_t)n * P + p] = a * hp[(size_t)n * P + p] + dtv * (double)xt[p] * (double)Bt[n];
        }
        if (dh_out) memcpy(gg, dh_out + hoff, sizeof(double) * NP);
        else memset(gg, 0, sizeof(double) * NP);
        double dAacc = 0.0, dDacc = 0.0, a_next = 1.0;
        for (int64_t k = L - 1; k >= 0; --k) {
            const int64_t t = t0 + k;
            const double dtv = (double)dt[(size_t)t * H + hd], a = exp(dtv * Ah);
            const float *xt = x + ((size_t)t * H + hd) * P;
            const float *Bt = B + ((size_t)t * G + g) * N, *Ct = C + ((size_t)t * G + g) * N;
            const double *dyt = dy + ((size_t)t * H + hd) * P;
            const double *ht = hs + NP * (size_t)(k + 1), *hprev = hs + NP * (size_t)k;
            /* g_t = a_{t+1} g_{t+1} + C_t (x) dy_t  (a_next = 1 for the last token) */
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p)
                    gg[(size_t)n * P + p] = a_next * gg[(size_t)n * P + p] + (double)Ct[n] * dyt[p];
            double *dxt = dx + ((size_t)t * H + hd) * P;
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += (double)Bt[n] * gg[(size_t)n * P + p];
                dxt[p] = Dh * dyt[p] + dtv * acc;
                dDacc += dyt[p] * (double)xt[p];
            }
            double da = 0.0, gxb = 0.0;
            for (int n = 0; n < N; ++n) {
                double cb = 0.0, bb = 0.0;
                for (int p = 0; p < P; ++p) {
                    const double gv = gg[(size_t)n * P + p];
                    cb += ht[(size_t)n * P + p] * dyt[p];
                    bb += (double)xt[p] * gv;
                    da += gv * hprev[(size_t)n * P + p];
                }
                dCh[((size_t)t * H + hd) * N + n] = cb;
                dBh[((size_t)t * H + hd) * N + n] = dtv * bb;
                gxb += bb * (double)Bt[n];
            }
            ddt[(size_t)t * H + hd] = Ah * a * da + gxb;
            dAacc += dtv * a * da;
            a_next = a;
        }
        if (dh0)
            for (size_t e = 0; e < NP; ++e)
                dh0[hoff + e] = a_next * gg[e];
        dAs[(size_t)s * H + hd] = dAacc;
        dDs[(size_t)s * H + hd] = dDacc;
        free(hs);
        free(gg);
    }
    /* sums over the heads of a group and over the sequences */
    for (int64_t t = 0; t < T; ++t)
        for (int g = 0; g < G; ++g)
            for (int n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int hd = 0; hd < H; ++hd)
                    if ((int)(((long)hd * G) / H) == g) {
                        sb += dBh[((size_t)t * H + hd) * N + n];
                        sc += dCh[((size_t)t * H + hd) * N + n];
                    }
                dB[((size_t)t * G + g) * N + n] = sb;
                dC[((size_t)t * G + g) * N + n] = sc;
            }
    for (int hd = 0; hd < H; ++hd) {
        double sa = 0.0, sd = 0.0;
        for (int s = 0; s < nseq; ++s) {
            sa += dAs[(size_t)s * H + hd];
            sd += dDs[(size_t)s * H + hd];
        }
        dA[hd] = sa;
        dD[hd] = sd;
    }
    free(dBh); free(dCh); free(dAs); free(dDs);
    return bad ? -1 : 0;
}

/*
 * Gated delta rule: the other scan family that Recurrence Scan covers ("One
 * equation, one packed result": a per-head matrix state that every token
 * rewrites and that the scan carries forward and returns beside the
 * output).  The page gives no
 * equation; this is the published gated delta rule, per sequence and head h
 * (q, k read group g = floor(h*G/H)), state S [V][K] (row i = value index):
 *   a_t   = exp(g_t)                                   (g_t <= 0: the gate)
 *   u     = S_{t-1} k_t                                (V vector)
 *   S_t   = a_t S_{t-1} + beta_t (v_t - a_t u) k_t^T  (delta-rule correction)
 *   o_t   = S_t q_t
 * i.e. S_t = S_{t-1} a_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.  q, k, v, g,
 * beta arrive final: any normalisation of k, scale of q, activation of beta
 * and log-gate are the caller's.  Layouts: q, k [T][G][K]; v [T][H][V];
 * g, beta [T][H]; h0, h_out [nseq][H][V][K] (h0 NULL: zeros); o [T][H][V].
 * Sequences are packed along T by cu (cu[s] .. cu[s+1]-1).
 */
int ssd_ref_gated_delta_rule(const float *q, const float *k, const float *v, const float *g,
                             const float *beta, const double *h0, const int64_t *cu, int nseq,
                             int H, int G, int K, int V, double *o, double *h_out,
                             int nthreads)
{
    if (!cu || nseq < 0 || H <= 0 || G <= 0 || K <= 0 || V <= 0 || H % G != 0) return -1;
    for (int s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    if (nseq > 0 && cu[nseq] > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    const long units = (long)nseq * H;
    const size_t VK = (size_t)V * K;
    if (nthreads <= 0) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long un = 0; un < units; ++un) {
        const int s = (int)(un / H), hd = (int)(un % H);
        const int gr = (int)(((long)hd * G) / H);
        double *S = (double *)malloc(sizeof(double) * VK);
        double *u = (double *)malloc(sizeof(double) * V);
        if (!S || !u) { bad = 1; free(S); free(u); continue; }
        const size_t soff = ((size_t)s * H + hd) * VK;
        if (h0) memcpy(S, h0 + soff, sizeof(double) * VK);
        else memset(S, 0, sizeof(double) * VK);
        for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
            const float *qt = q + ((size_t)t * G + gr) * K, *kt = k + ((size_t)t * G + gr) * K;
            const float *vt = v + ((size_t)t * H + hd) * V;
            const double a = exp((double)g[(size_t)t * H + hd]);
            const double b = (double)beta[(size_t)t * H + hd];
            for (int i = 0; i < V; ++i) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += S[(size_t)i * K + j] * (double)kt[j];
                u[i] = acc;
            }
            for (int i = 0; i < V; ++i) {
                const double c = b * ((double)vt[i] - a * u[i]);
                for (int j = 0; j < K; ++j)
                    S[(size_t)i * K + j] = a * S[(size_t)i * K + j] + c * (double)kt[j];
            }
            double *ot = o + ((size_t)t * H + hd) * V;
            for (int i = 0; i < V; ++i) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += S[(size_t)i * K + j] * (double)qt[j];
                ot[i] = acc;
            }
        }
        if (h_out) memcpy(h_out + soff, S, sizeof(double) * VK);
        free(S);
        free(u);
    }
    return bad ? -1 : 0;
}
