// ssd_s6.hip -- Mamba-1 selective scan on gfx950: a diagonal transition per
// channel d and state n (the per-channel form of the selective update of
// COREY: Entropy-Guided Runtime Chunk Scheduling for Selective Scan Kernels,
// section 3.1; the kernel its section 5.1 times at batch 1, d 1024, L 4096,
// d_state 16):
//   h_t[d][n] = exp(dt_t[d] A[d][n]) h_{t-1}[d][n] + dt_t[d] B_t[n] x_t[d]
//   y_t[d]    = sum_n C_t[n] h_t[d][n] + D[d] x_t[d]
//
// A thread owns one channel and all its N (<= 16) states, in registers.  Time
// is cut into S segments so that there are enough threads: a segment's
// recurrence started from zero gives its end state hs and sum of dt; walking
// the segments in order, H_in(k+1) = exp(A sum_dt(k)) H_in(k) + hs(k) gives the
// state entering each; each segment is then replayed from that state to
// produce y.  Three launches (summary, pass, replay); the exponentials of
// the two token passes bound the run time (one transcendental per (t, d, n)
// per pass).  Segment B and C rows are staged in LDS (the same for every
// channel); x, dt and y are token-major, so a wave touches 64 consecutive
// channels of one token.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr float kS6Log2e = 1.4426950408889634f;
constexpr int kS6Threads = 256;

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const bf16 *p) { return (float)*p; }
__device__ __forceinline__ float ld1(const _Float16 *p) { return (float)*p; }

// Stage rows [t0, t0 + len) of B and C (each [b][L][N]) as float32 into LDS.
template <typename T, int N>
__device__ __forceinline__ void s6_stage_bc(float *bs, float *cs, const T *__restrict__ B,
                                            const T *__restrict__ C, size_t row0, int len) {
  for (int i = threadIdx.x; i < len * N; i += kS6Threads) {
    bs[i] = ld1(B + row0 * N + i);
    cs[i] = ld1(C + row0 * N + i);
  }
}

// Summary of segment k: the state at its end, started from zero, and sum dt.
template <typename T, int N>
__global__ __launch_bounds__(kS6Threads) void k_s6_summary(const T *__restrict__ x,
                                                           const T *__restrict__ dt,
                                                           const float *__restrict__ A,
                                                           const T *__restrict__ B, int L, int dim,
                                                           int seg, float *__restrict__ hs,
                                                           float *__restrict__ sdt) {
  extern __shared__ float sh[];
  float *bs = sh;  // [seg][N]
  const int d = blockIdx.x * kS6Threads + threadIdx.x, k = blockIdx.y, b = blockIdx.z;
  const int t0 = k * seg, len = min(seg, L - t0);
  const size_t row0 = (size_t)b * L + t0;
  for (int i = threadIdx.x; i < len * N; i += kS6Threads) bs[i] = ld1(B + row0 * N + i);
  __syncthreads();
  if (d >= dim) return;
  float a2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    a2[n] = A[(size_t)d * N + n] * kS6Log2e;
    h[n] = 0.f;
  }
  float sum = 0.f;
  const T *xp = x + row0 * dim + d, *dp = dt + row0 * dim + d;
  for (int t = 0; t < len; ++t) {
    const float dv = ld1(dp + (size_t)t * dim), dx = dv * ld1(xp + (size_t)t * dim);
    sum += dv;
#pragma unroll
    for (int n = 0; n < N; ++n)
      h[n] = __builtin_amdgcn_exp2f(fminf(dv * a2[n], 0.f)) * h[n] + dx * bs[t * N + n];
  }
  const size_t o = ((size_t)b * gridDim.y + k) * dim + d;
#pragma unroll
  for (int n = 0; n < N; ++n) hs[o * N + n] = h[n];
  sdt[o] = sum;
}

// Per (b, d, n): walk the segments in order; hs(k) is replaced by the state
// entering segment k; the final state goes to h_out.
template <int N>
__global__ __launch_bounds__(kS6Threads) void k_s6_pass(const float *__restrict__ A,
                                                        const float *h0, float *h_out,
                                                        float *__restrict__ hs,
                                                        const float *__restrict__ sdt, int batch,
                                                        int dim, int nseg) {
  const long e = (long)blockIdx.x * kS6Threads + threadIdx.x;  // (b, d, n), n fastest
  if (e >= (long)batch * dim * N) return;
  const int n = (int)(e % N), d = (int)((e / N) % dim), b = (int)(e / ((long)N * dim));
  const float a2 = A[(size_t)d * N + n] * kS6Log2e;
  float H = h0 ? h0[e] : 0.f;
  constexpr int U = 32;  // segment summaries in flight
  for (int k0 = 0; k0 < nseg; k0 += U) {
    float hv[U], sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < nseg) {
        const size_t o = ((size_t)b * nseg + k0 + u) * dim + d;
        hv[u] = hs[o * N + n];
        sv[u] = sdt[o];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < nseg) {
        const size_t o = ((size_t)b * nseg + k0 + u) * dim + d;
        hs[o * N + n] = H;
        H = __builtin_amdgcn_exp2f(fminf(a2 * sv[u], 0.f)) * H + hv[u];
      }
    }
  }
  if (h_out) h_out[e] = H;
}

// Replay segment k from the state entering it; y_t[d] for every token.
template <typename T, int N>
__global__ __launch_bounds__(kS6Threads) void k_s6_replay(const T *__restrict__ x,
                                                          const T *__restrict__ dt,
                                                          const float *__restrict__ A,
                                                          const T *__restrict__ B,
                                                          const T *__restrict__ C,
                                                          const float *__restrict__ D, int L,
                                                          int dim, int seg,
                                                          const float *__restrict__ hin,
                                                          float *__restrict__ y) {
  extern __shared__ float sh[];
  const int d = blockIdx.x * kS6Threads + threadIdx.x, k = blockIdx.y, b = blockIdx.z;
  const int t0 = k * seg, len = min(seg, L - t0);
  const size_t row0 = (size_t)b * L + t0;
  float *bs = sh, *cs = sh + seg * N;
  s6_stage_bc<T, N>(bs, cs, B, C, row0, len);
  __syncthreads();
  if (d >= dim) return;
  const size_t o = ((size_t)b * gridDim.y + k) * dim + d;
  float a2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    a2[n] = A[(size_t)d * N + n] * kS6Log2e;
    h[n] = hin[o * N + n];
  }
  const float Dv = D[d];
  const T *xp = x + row0 * dim + d, *dp = dt + row0 * dim + d;
  float *yp = y + row0 * dim + d;
  for (int t = 0; t < len; ++t) {
    const float dv = ld1(dp + (size_t)t * dim), xv = ld1(xp + (size_t)t * dim), dx = dv * xv;
    float acc = Dv * xv;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      h[n] = __builtin_amdgcn_exp2f(fminf(dv * a2[n], 0.f)) * h[n] + dx * bs[t * N + n];
      acc += cs[t * N + n] * h[n];
    }
    yp[(size_t)t * dim] = acc;
  }
}

// Segments: enough that (batch x dim x segments) threads fill the GPU twice,
// each at least 16 tokens long, at most 8192/N tokens (the staged B and C rows
// of a segment, 8N bytes per token, stay within 64 KB of LDS), and at most
// 65535 of them (the grid's y extent).
S6Plan s6_plan(int batch, int L, int dim, int N) {
  S6Plan p{};
  if (L <= 0) return p;
  const long want = 2L * 256 * 4 * 64;  // two waves per SIMD
  long nseg = (want + (long)batch * dim - 1) / ((long)batch * dim);
  const long max_seg = L / 16 > 0 ? L / 16 : 1;
  if (nseg > max_seg) nseg = max_seg;
  if (nseg < 1) nseg = 1;
  long seg = (L + nseg - 1) / nseg;
  const long cap = 8192 / N;
  if (seg > cap) seg = cap;
  if ((L + seg - 1) / seg > 65535) seg = (L + 65534) / 65535;
  p.seg = (int)seg;
  p.nseg = (int)((L + seg - 1) / seg);
  return p;
}

size_t s6_workspace(int batch, int L, int dim, int N) {
  const S6Plan p = s6_plan(batch, L, dim, N);
  const size_t units = (size_t)batch * (p.nseg > 0 ? p.nseg : 1) * dim;
  return ((units * N * 4 + 255) / 256) * 256 + ((units * 4 + 255) / 256) * 256;
}

template <typename T, int N>
static hipError_t run_s6(const S6Args &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const S6Plan p = s6_plan(a.batch, a.L, a.dim, N);
  const size_t units = (size_t)a.batch * p.nseg * a.dim;
  float *hs = static_cast<float *>(a.workspace);
  float *sdt = reinterpret_cast<float *>(static_cast<char *>(a.workspace) +
                                         ((units * N * 4 + 255) / 256) * 256);
  if (p.nseg > 0) {
    dim3 grid((a.dim + kS6Threads - 1) / kS6Threads, p.nseg, a.batch);
    hipLaunchKernelGGL((k_s6_summary<T, N>), grid, dim3(kS6Threads), (size_t)p.seg * N * 4, st,
                       (const T *)a.x, (const T *)a.dt, a.A, (const T *)a.B, a.L, a.dim, p.seg,
                       hs, sdt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long states = (long)a.batch * a.dim * N;
  if (states > 0) {
    hipLaunchKernelGGL(k_s6_pass<N>, dim3((unsigned)((states + kS6Threads - 1) / kS6Threads)),
                       dim3(kS6Threads), 0, st, a.A, a.h0, a.h_out, hs, sdt, a.batch, a.dim,
                       p.nseg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nseg > 0) {
    dim3 grid((a.dim + kS6Threads - 1) / kS6Threads, p.nseg, a.batch);
    hipLaunchKernelGGL((k_s6_replay<T, N>), grid, dim3(kS6Threads), (size_t)p.seg * N * 8, st,
                       (const T *)a.x, (const T *)a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D,
                       a.L, a.dim, p.seg, hs, a.y);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
static hipError_t s6_N(const S6Args &a) {
  switch (a.N) {
    case 1: return run_s6<T, 1>(a);
    case 2: return run_s6<T, 2>(a);
    case 4: return run_s6<T, 4>(a);
    case 8: return run_s6<T, 8>(a);
    case 16: return run_s6<T, 16>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_selective_scan(const S6Args &a) {
  if (a.batch == 0 || a.dim == 0) return hipSuccess;
  switch (a.dtype) {
    case 0: return s6_N<float>(a);
    case 1: return s6_N<bf16>(a);
    case 2: return s6_N<_Float16>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
