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
// Block = 256 threads per (b, h): TPR = P/4 threads cover one state row with
// float4 vectors, RPP = 256/TPR rows per pass, eight passes in flight; the partial
// y sums over rows are reduced through LDS at the end.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

template <typename T, int P>
__global__ __launch_bounds__(256) void k_step(const T *__restrict__ x, const float *__restrict__ dt,
                                              const float *__restrict__ A,
                                              const T *__restrict__ B, const T *__restrict__ C,
                                              const float *__restrict__ D, float *__restrict__ h,
                                              float *__restrict__ y, int H, int N, int G) {
  constexpr int TPR = P / 4;
  constexpr int RPP = 256 / TPR;
  __shared__ float Bsh[1024], Csh[1024];
  __shared__ f4 red[256];
  const int hd = blockIdx.x, b = blockIdx.y;
  const int g = (hd * G) / H;
  const int tid = threadIdx.x, q = tid % TPR, r0 = tid / TPR;
  const T *Bp = B + ((size_t)b * G + g) * N;
  const T *Cp = C + ((size_t)b * G + g) * N;
  for (int n = tid; n < N; n += 256) {
    Bsh[n] = to_f32(Bp[n]);
    Csh[n] = to_f32(Cp[n]);
  }
  const size_t bh = (size_t)b * H + hd;
  const float dtv = dt[bh];
  const float a = expf(fminf(dtv * A[hd], 0.f));
  const f4 xv = ld4f(x + bh * P + 4 * q);
  f4 dx;
#pragma unroll
  for (int e = 0; e < 4; ++e) dx[e] = dtv * xv[e];
  __syncthreads();

  float *hp = h + bh * (size_t)N * P + 4 * q;
  f4 yacc = zero4();
  int n = r0;
  // eight rows per thread in flight
  constexpr int U = 8;
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
    st4(y + bh * P + 4 * q, s);
  }
}

template <typename T>
static hipError_t run_step(const StepArgs &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  dim3 grid(a.H, a.batch);
  switch (a.P) {
    case 16: hipLaunchKernelGGL((k_step<T, 16>), grid, dim3(256), 0, st, (const T *)a.x, a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.H, a.N, a.G); break;
    case 32: hipLaunchKernelGGL((k_step<T, 32>), grid, dim3(256), 0, st, (const T *)a.x, a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.H, a.N, a.G); break;
    case 64: hipLaunchKernelGGL((k_step<T, 64>), grid, dim3(256), 0, st, (const T *)a.x, a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.H, a.N, a.G); break;
    case 128: hipLaunchKernelGGL((k_step<T, 128>), grid, dim3(256), 0, st, (const T *)a.x, a.dt, a.A, (const T *)a.B, (const T *)a.C, a.D, a.h, a.y, a.H, a.N, a.G); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a) {
  if (a.batch == 0) return hipSuccess;
  return a.bf16 ? run_step<bf16>(a) : run_step<float>(a);
}

}  // namespace ssd
