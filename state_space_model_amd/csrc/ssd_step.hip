// ssd_step.hip -- fused single-token SSD decode step on gfx950 (HBM-bound).
//
// Per (batch b, head h), in place:
//   a = exp(dt A_h);  h[n][p] = a h[n][p] + (dt x[p]) B[n];  y[p] = sum_n C[n] h[n][p] + D_h x[p]
// The state is [b][h][n][p] with p fastest, so a row h[n][0..P) is P*4
// contiguous bytes and consecutive lanes read consecutive 16-byte vectors:
// every state byte is read once and written once, fully coalesced.  (Mamba-2
// SSD fused layer via VGpuWarp, "S2 RESULT": a per-channel sweep over a
// channel-major h[c*d_state+n] puts consecutive lanes d_state*4 bytes apart and
// wastes most of each cache line; storing h n-major fixes it.  "Lane mapping":
// the work is one independent lane per (head, head_dim) channel folding over
// d_state; here a 256-thread block owns one head and splits both p and n.)
//
// Block = 256 threads per (b, h) -- or per (b, h, half of p) when the batch
// is too small to give every CU several blocks (PS = 2): TPR = P/PS/4 threads
// cover the block's columns of one state row with float4 vectors, RPP =
// 256/TPR rows per pass, U passes in flight; the partial y sums over rows are
// reduced through LDS at the end (y[p] sums over n only, so the halves of p
// need nothing from each other).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int P, int PS>
__global__ __launch_bounds__(256) void k_step(const T *__restrict__ x, const float *__restrict__ dt,
                                              const float *__restrict__ A,
                                              const T *__restrict__ B, const T *__restrict__ C,
                                              const float *__restrict__ D, float *__restrict__ h,
                                              float *__restrict__ y, int H, int N, int G,
                                              size_t xbs, size_t bcs) {
  constexpr int PB = P / PS;  // the block's columns
  constexpr int TPR = PB / 4;
  constexpr int RPP = 256 / TPR;
  __shared__ float Bsh[1024], Csh[1024];
  __shared__ f4 red[256];
  const int hd = blockIdx.x / PS, pc = (blockIdx.x % PS) * PB, b = blockIdx.y;
  const int g = (hd * G) / H;
  const int tid = threadIdx.x, q = tid % TPR, r0 = tid / TPR;
  const T *Bp = B + (size_t)b * bcs + (size_t)g * N;  // x, B, C rows are xbs / bcs apart
  const T *Cp = C + (size_t)b * bcs + (size_t)g * N;
  const size_t bh = (size_t)b * H + hd;
  float *hp = h + bh * (size_t)N * P + pc + 4 * q;
  // U rows per thread in flight (all of them at N = 128 with the halves of p).
  // With the columns split (few blocks, latency-bound) the first U are loaded
  // before B and C are staged, so that the two round trips overlap; with many
  // blocks that only holds registers longer (the Codestral step: 1 % slower)
  constexpr int U = PS == 1 ? 8 : 4;
  const bool first = PS > 1 && r0 + (U - 1) * RPP < N;
  f4 v0[U];
  if (first) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      v0[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(hp + (size_t)(r0 + u * RPP) * P));
  }
  for (int n = tid; n < N; n += 256) {
    Bsh[n] = to_f32(Bp[n]);
    Csh[n] = to_f32(Cp[n]);
  }
  const float dtv = dt[bh];
  const float a = expf(fminf(dtv * A[hd], 0.f));
  const f4 xv = ld4f(x + (size_t)b * xbs + (size_t)hd * P + pc + 4 * q);
  f4 dx;
#pragma unroll
  for (int e = 0; e < 4; ++e) dx[e] = dtv * xv[e];
  __syncthreads();

  f4 yacc = zero4();
  int n = r0;
  if (first) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float bn = Bsh[n + u * RPP], cn = Csh[n + u * RPP];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[u][e] = a * v0[u][e] + dx[e] * bn;
        yacc[e] += cn * v0[u][e];
      }
      __builtin_nontemporal_store(v0[u], reinterpret_cast<f4 *>(hp + (size_t)(n + u * RPP) * P));
    }
    n += U * RPP;
  }
  for (; n + (U - 1) * RPP < N; n += U * RPP) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(hp + (size_t)(n + u * RPP) * P));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float bn = Bsh[n + u * RPP], cn = Csh[n + u * RPP];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[u][e] = a * v[u][e] + dx[e] * bn;
        yacc[e] += cn * v[u][e];
      }
      __builtin_nontemporal_store(v[u], reinterpret_cast<f4 *>(hp + (size_t)(n + u * RPP) * P));
    }
  }
  for (; n < N; n += RPP) {
    f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(hp + (size_t)n * P));
    const float bn = Bsh[n], cn = Csh[n];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a * v[e] + dx[e] * bn;
      yacc[e] += cn * v[e];
    }
    __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(hp + (size_t)n * P));
  }
  red[tid] = yacc;
  __syncthreads();
  if (tid < TPR) {
    f4 s = red[tid];
    for (int r = 1; r < RPP; ++r) {
      const f4 t = red[r * TPR + tid];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += t[e];
    }
    const float dv = D[hd];
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += dv * xv[e];
    st4(y + bh * P + pc + 4 * q, s);
  }
}

// Fewer (b, h) blocks than this (four per CU) and P >= 32: each head's
// columns in two blocks.
constexpr long kStepSplitBelow = 4L * 256;

template <typename T>
static hipError_t run_step(const StepArgs &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int ps = (long)a.batch * a.H < kStepSplitBelow && a.P >= 32 ? 2 : 1;
  dim3 grid(a.H * ps, a.batch);
  const size_t xbs = a.x_bstride ? a.x_bstride : (size_t)a.H * a.P;
  const size_t bcs = a.bc_bstride ? a.bc_bstride : (size_t)a.G * a.N;
#define SSD_LAUNCH(p, s)                                                                       \
  hipLaunchKernelGGL((k_step<T, p, s>), grid, dim3(256), 0, st, (const T *)a.x, a.dt, a.A,     \
                     (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.H, a.N, a.G, xbs, bcs);
  switch (a.P * 10 + ps) {
    case 161: SSD_LAUNCH(16, 1) break;
    case 321: SSD_LAUNCH(32, 1) break;
    case 322: SSD_LAUNCH(32, 2) break;
    case 641: SSD_LAUNCH(64, 1) break;
    case 642: SSD_LAUNCH(64, 2) break;
    case 1281: SSD_LAUNCH(128, 1) break;
    case 1282: SSD_LAUNCH(128, 2) break;
    default: return hipErrorInvalidValue;
  }
#undef SSD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a) {
  if (a.batch == 0) return hipSuccess;
  return a.bf16 ? run_step<bf16>(a) : run_step<float>(a);
}

// ------------------------------------------------------------------------
// Many decode steps in one launch, over inputs staged for every step:
//   x [S][b][H][P], dt [S][b][H], B, C [S][b][G][N], y [S][b][H][P]
// equal to S successive single steps.  One wave per (b, h, 64-column part of
// p) keeps its slice of the state in registers for all S steps, so the state
// crosses HBM once (read at the start, written at the end) instead of twice per
// step; the work per step is then the 5 flops per state element of the update
// and the output (the fp32 vector units bound it).  This is the recurrence run
// as a stream over time, as Recurrence Scan does ("The schedule"); a step's
// inputs are fetched while the previous step is computed.
//
// Lane l: column group c = l % (PL/4) (4 consecutive p), row group
// r = l / (PL/4) owning rows [r RPL, (r+1) RPL); y[p] is summed over the row
// groups with xor shuffles.
template <typename T, int PL, int N>
__global__ __launch_bounds__(64) void k_step_multi(const T *__restrict__ x,
                                                   const float *__restrict__ dt,
                                                   const float *__restrict__ A,
                                                   const T *__restrict__ B, const T *__restrict__ C,
                                                   const float *__restrict__ D,
                                                   float *__restrict__ h, float *__restrict__ y,
                                                   int steps, int batch, int H, int P, int G) {
  constexpr int TPR = PL / 4;       // lanes per state row
  constexpr int RG = 64 / TPR;      // row groups
  constexpr int RPL = N / RG;       // rows per lane
  static_assert(RPL >= 1 && N % RG == 0, "rows per lane");
  __shared__ __align__(16) float bc[2 * N];  // B then C of the current step
  const int lane = threadIdx.x, c = lane % TPR, r = lane / TPR;
  const int parts = P / PL;
  const int hd = blockIdx.x / parts, part = blockIdx.x % parts, b = blockIdx.y;
  const int g = (hd * G) / H;
  const int p0 = part * PL + 4 * c;
  const size_t bh = (size_t)b * H + hd;
  const size_t xs = (size_t)batch * H * P, ds = (size_t)batch * H, bs = (size_t)batch * G * N;
  const float A2 = A[hd], dv = D[hd];

  float *hp = h + bh * (size_t)N * P + p0;
  f4 st[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) st[k] = ld4(hp + (size_t)(r * RPL + k) * P);

  // step inputs, prefetched one step ahead: lanes < N/4 carry B, the next N/4 C
  const bool bl = lane < N / 4, cl = !bl && lane < N / 2;
  const T *bsrc = B + ((size_t)b * G + g) * N + 4 * lane;
  const T *csrc = C + ((size_t)b * G + g) * N + 4 * (lane - N / 4);
  auto fetch = [&](int t, f4 &xv, float &dtv, f4 &bcv) {
    xv = ld4f(x + t * xs + bh * P + p0);
    dtv = dt[t * ds + bh];
    bcv = bl ? ld4f(bsrc + t * bs) : cl ? ld4f(csrc + t * bs) : zero4();
  };
  f4 xv, bcv;
  float dtv;
  if (steps > 0) fetch(0, xv, dtv, bcv);
  for (int t = 0; t < steps; ++t) {
    if (bl || cl) st4(bc + 4 * lane, bcv);
    __syncthreads();
    const f4 xc = xv;
    const float dtc = dtv;
    if (t + 1 < steps) fetch(t + 1, xv, dtv, bcv);
    const float a = expf(fminf(dtc * A2, 0.f));
    f4 dx, yp = zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) dx[e] = dtc * xc[e];
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      const float bn = bc[r * RPL + k], cn = bc[N + r * RPL + k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st[k][e] = a * st[k][e] + dx[e] * bn;
        yp[e] += cn * st[k][e];
      }
    }
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) yp[e] += __shfl_xor(yp[e], off, 64);
    if (r == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) yp[e] += dv * xc[e];
      st4(y + t * xs + bh * P + p0, yp);
    }
    __syncthreads();  // bc is rewritten by the next step
  }
#pragma unroll
  for (int k = 0; k < RPL; ++k) st4(hp + (size_t)(r * RPL + k) * P, st[k]);
}

template <typename T, int PL>
static hipError_t multi_N(const MultiStepArgs &a, hipStream_t st) {
  dim3 grid(a.H * (a.P / PL), a.batch);
#define SSD_LAUNCH(n)                                                                            \
  hipLaunchKernelGGL((k_step_multi<T, PL, n>), grid, dim3(64), 0, st, (const T *)a.x, a.dt, a.A, \
                     (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.steps, a.batch, a.H, a.P,  \
                     a.G);                                                                       \
  break;
  switch (a.N) {
    case 16: SSD_LAUNCH(16)
    case 32: SSD_LAUNCH(32)
    case 64: SSD_LAUNCH(64)
    case 128: SSD_LAUNCH(128)
    default: return hipErrorInvalidValue;
  }
#undef SSD_LAUNCH
  return hipGetLastError();
}

template <typename T>
static hipError_t run_multi(const MultiStepArgs &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  switch (a.P) {
    case 16: return multi_N<T, 16>(a, st);
    case 32: return multi_N<T, 32>(a, st);
    case 64: return multi_N<T, 64>(a, st);
    case 128: return multi_N<T, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_step_multi(const MultiStepArgs &a) {
  if (a.batch == 0 || a.steps == 0) return hipSuccess;
  return a.bf16 ? run_multi<bf16>(a) : run_multi<float>(a);
}

}  // namespace ssd
