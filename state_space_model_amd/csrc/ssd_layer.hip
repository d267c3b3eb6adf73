// ssd_layer.hip -- the decode-layer operations on either side of the scan, as
// device kernels (Mamba-2 SSD fused layer via VGpuWarp -- design sketch, the
// list of layer steps to move onto the device): the causal conv1d step over the
// in_proj channels x|B|C with a rolling window kept in device memory, and the
// gated RMS norm of the scan output.  With them the layer body runs on the
// device and the scan output never leaves it.
//
//   conv:  win[c] <- (win[c][1..W-1], u[c]);  v = bias[c] + sum_k w[c][k] win[c][k];
//          out = silu(v) = v sigmoid(v)  (or v)
//   norm:  g = y silu(z);  out = g / sqrt(mean_d(g^2) + eps) w
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// One thread per (token, channel): the window (W <= 8 floats, oldest first) is
// read, rolled and written back; the output is written as TO.
template <typename T, typename TO, int W>
__global__ __launch_bounds__(256) void k_conv1d_step(const T *__restrict__ u,
                                                     float *__restrict__ state,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ bias, int silu,
                                                     TO *__restrict__ out, int channels) {
  const int c = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (c >= channels) return;
  const size_t bc = (size_t)b * channels + c;
  float *win = state + bc * W;
  float v[W];
#pragma unroll
  for (int k = 0; k + 1 < W; ++k) v[k] = win[k + 1];
  v[W - 1] = to_f32(u[bc]);
  float acc = bias ? bias[c] : 0.f;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    win[k] = v[k];
    acc += w[(size_t)c * W + k] * v[k];
  }
  if (silu) acc = acc / (1.f + expf(-acc));
  out[bc] = from_f32<TO>(acc);
}

// One workgroup per token row: g = y silu(z) in registers (or recomputed for
// long rows), the mean square by a block reduction, then the scaled row.
template <typename T>
__global__ __launch_bounds__(1024) void k_gated_rmsnorm(const float *__restrict__ y,
                                                        const T *__restrict__ z,
                                                        const float *__restrict__ w, float eps,
                                                        float *__restrict__ out, int dim) {
  __shared__ float part[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const float *yr = y + (size_t)b * dim;
  const T *zr = z + (size_t)b * dim;
  auto gate = [&](int d) {
    const float zz = to_f32(zr[d]);
    return yr[d] * (zz / (1.f + expf(-zz)));
  };
  float ss = 0.f;
  for (int d = tid; d < dim; d += blockDim.x) {
    const float g = gate(d);
    ss += g * g;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < nw; ++i) tot += part[i];
  const float r = 1.f / sqrtf(tot / (float)dim + eps);
  float *orow = out + (size_t)b * dim;
  for (int d = tid; d < dim; d += blockDim.x) orow[d] = gate(d) * r * w[d];
}

template <typename T, typename TO>
static hipError_t conv_T(const void *u, float *state, const float *w, const float *bias, int silu,
                         void *out, int batch, int channels, int width, hipStream_t st) {
  dim3 grid((channels + 255) / 256, batch);
#define SSD_CONV(k)                                                                          \
  case k:                                                                                    \
    hipLaunchKernelGGL((k_conv1d_step<T, TO, k>), grid, dim3(256), 0, st, (const T *)u,      \
                       state, w, bias, silu, (TO *)out, channels);                           \
    break;
  switch (width) {
    SSD_CONV(1) SSD_CONV(2) SSD_CONV(3) SSD_CONV(4) SSD_CONV(5) SSD_CONV(6) SSD_CONV(7)
    SSD_CONV(8)
    default: return hipErrorInvalidValue;
  }
#undef SSD_CONV
  return hipGetLastError();
}

hipError_t launch_conv1d_step(const void *u, float *state, const float *w, const float *bias,
                              bool silu, void *out, int batch, int channels, int width,
                              bool is_bf16, bool out_f32, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  if (!is_bf16) return conv_T<float, float>(u, state, w, bias, silu, out, batch, channels, width, st);
  return out_f32 ? conv_T<bf16, float>(u, state, w, bias, silu, out, batch, channels, width, st)
                 : conv_T<bf16, bf16>(u, state, w, bias, silu, out, batch, channels, width, st);
}

hipError_t launch_gated_rmsnorm(const float *y, const void *z, const float *w, float eps,
                                float *out, int batch, int dim, bool is_bf16, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  const int threads = dim >= 1024 ? 1024 : ((dim + 63) / 64) * 64;
  if (is_bf16)
    hipLaunchKernelGGL(k_gated_rmsnorm<bf16>, dim3(batch), dim3(threads), 0, st, y,
                       (const bf16 *)z, w, eps, out, dim);
  else
    hipLaunchKernelGGL(k_gated_rmsnorm<float>, dim3(batch), dim3(threads), 0, st, y,
                       (const float *)z, w, eps, out, dim);
  return hipGetLastError();
}

}  // namespace ssd
