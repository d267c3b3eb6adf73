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
 * the gated RMS norm) and the Mamba-1 selective scan are at the end of this
 * file, with their own passages.
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
