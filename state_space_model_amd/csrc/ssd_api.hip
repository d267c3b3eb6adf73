// ssd_api.hip -- the C ABI of libssd.so (declared in include/ssd.h).
//
// Host-side only: argument checks before anything is enqueued (shapes that
// have no compiled instance are refused up front, as the Recurrence Scan
// design note's planner refuses a state column that does not fit, "The
// schedule"), workspace sizing, and dispatch to the kernels on the caller's
// stream.  No allocation, no synchronisation, no exception across the ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "ssd.h"
#include "ssd_launch.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int check_prefill(const void *x, const float *dt, const float *A, const void *B, const void *C,
                  const float *D, float *y, int nseq, int64_t T, int H, int P, int N, int G,
                  int chunk, ssd_dtype_t dtype, const int32_t *cu) {
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (nseq < 1) return fail(SSD_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (T < 0 || T > INT32_MAX) return fail(SSD_ERR_INVALID_ARG, "total_tokens %lld out of range", (long long)T);
  if (H < 1 || G < 1) return fail(SSD_ERR_INVALID_ARG, "H and G must be >= 1 (H=%d G=%d)", H, G);
  if (H % G != 0) return fail(SSD_ERR_INVALID_ARG, "H %% G != 0 (H=%d G=%d)", H, G);
  if (!pow2_in(P, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "headdim P=%d not in {16,32,64,128}", P);
  if (!pow2_in(N, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "d_state N=%d not in {16,32,64,128}", N);
  if (!pow2_in(chunk, 32, 512))
    return fail(SSD_ERR_UNSUPPORTED, "chunk=%d not in {32,64,128,256,512}%s", chunk,
                chunk == 16 ? " (the token step of the matrix cores is 32: use chunk 32)" : "");
  if (!cu && T % nseq != 0)
    return fail(SSD_ERR_INVALID_ARG, "dense batch: total_tokens %lld not divisible by nseq %d", (long long)T, nseq);
  if (T > 0 && (!x || !dt || !B || !C || !y))
    return fail(SSD_ERR_INVALID_ARG, "null x/dt/B/C/y pointer");
  if (!A || !D) return fail(SSD_ERR_INVALID_ARG, "null A/D pointer");
  if ((int64_t)T * H > INT32_MAX * 16LL) return fail(SSD_ERR_UNSUPPORTED, "problem too large");
  // tile loads address a chunk's rows with 32-bit byte offsets
  if ((int64_t)chunk * H * P * 4 > INT32_MAX || (int64_t)chunk * G * N * 4 > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "chunk x row stride too large (H*P*chunk*4 and G*N*chunk*4 must stay below 2^31)");
  return SSD_OK;
}

int prefill_impl(unsigned stages, const void *x, const float *dt, const float *A, const void *B,
                 const void *C, const float *D, const float *h0, float *y, float *h_out,
                 const int32_t *cu, int nseq, int64_t T, int H, int P, int N, int G, int chunk,
                 ssd_dtype_t dtype, void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  int rc = check_prefill(x, dt, A, B, C, D, y, nseq, T, H, P, N, G, chunk, dtype, cu);
  if (rc) return rc;
  if (stages & ~(unsigned)(SSD_STAGE_ALL | SSD_VARIANT_MASK))
    return fail(SSD_ERR_INVALID_ARG, "unknown stage bits 0x%x", stages);
  if ((stages & SSD_VARIANT_SCAN_ROWS) && (stages & SSD_VARIANT_SCAN_HEADS))
    return fail(SSD_ERR_INVALID_ARG, "SSD_VARIANT_SCAN_ROWS and _HEADS are exclusive");
  if ((stages & SSD_VARIANT_STATE_CHUNKS) && (stages & SSD_VARIANT_STATE_WALK))
    return fail(SSD_ERR_INVALID_ARG, "SSD_VARIANT_STATE_CHUNKS and _WALK are exclusive");
  const ssd::WorkspaceLayout L =
      ssd::prefill_layout(T, nseq, H, P, N, G, chunk, dtype == SSD_BF16 ? 2 : 4);
  if (!workspace || workspace_bytes < L.total)
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  ssd::PrefillArgs a{x, dt, A, B, C, D, h0, y, h_out, cu, nseq, T, H, P, N, G, chunk,
                     dtype == SSD_BF16, workspace, stream};
  a.variant = stages & SSD_VARIANT_MASK;
  hipError_t e = ssd::launch_prefill(a, stages & SSD_STAGE_ALL);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

// Scratch of ssd_scan_prefill_noalloc(): the prefill workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate.  Each device holds its own copy from library load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up
// once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address in *out; SSD_OK or an error code.
int scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSD_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_scan_prefill_workspace(int64_t total_tokens, int nseq, int H, int P, int N, int G,
                                  int chunk, ssd_dtype_t dtype) {
  if (dtype != SSD_F32 && dtype != SSD_BF16) return 0;
  if (nseq < 1 || total_tokens < 0 || total_tokens > INT32_MAX || H < 1 || G < 1 || H % G != 0)
    return 0;
  if (!pow2_in(P, 16, 128) || !pow2_in(N, 16, 128) || !pow2_in(chunk, 32, 512)) return 0;
  // as check_prefill
  if ((int64_t)total_tokens * H > INT32_MAX * 16LL) return 0;
  if ((int64_t)chunk * H * P * 4 > INT32_MAX || (int64_t)chunk * G * N * 4 > INT32_MAX) return 0;
  return ssd::prefill_layout(total_tokens, nseq, H, P, N, G, chunk, dtype == SSD_BF16 ? 2 : 4)
      .total;
}

unsigned ssd_scan_prefill_plan(int64_t total_tokens, int nseq, int H, int P, int N, int G,
                               int chunk, ssd_dtype_t dtype, int packed) {
  if (ssd_scan_prefill_workspace(total_tokens, nseq, H, P, N, G, chunk, dtype) == 0) return 0;
  return ssd::prefill_plan(total_tokens, nseq, H, P, N, G, chunk, dtype == SSD_BF16, packed != 0,
                           0u);
}

int ssd_scan_prefill(const void *x, const float *dt, const float *A, const void *B, const void *C,
                     const float *D, const float *h0, float *y, float *h_out,
                     const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H, int P, int N,
                     int G, int chunk, ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                     void *stream) {
  return prefill_impl(SSD_STAGE_ALL, x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, nseq,
                      total_tokens, H, P, N, G, chunk, dtype, workspace, workspace_bytes, stream);
}

int ssd_scan_prefill_noalloc(const void *x, const float *dt, const float *A, const void *B,
                             const void *C, const float *D, const float *h0, float *y,
                             float *h_out, const int32_t *cu_seqlens, int nseq,
                             int64_t total_tokens, int H, int P, int N, int G, int chunk,
                             ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  int rc = check_prefill(x, dt, A, B, C, D, y, nseq, total_tokens, H, P, N, G, chunk, dtype,
                         cu_seqlens);
  if (rc) return rc;
  // the limit is checked before anything touches the device
  const size_t need =
      ssd::prefill_layout(total_tokens, nseq, H, P, N, G, chunk, dtype == SSD_BF16 ? 2 : 4).total;
  if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
    return fail(SSD_ERR_WORKSPACE,
                "these shapes need %zu bytes of workspace; the built-in scratch holds %zu "
                "(pass a workspace to ssd_scan_prefill instead)",
                need, (size_t)SSD_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  return prefill_impl(SSD_STAGE_ALL, x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, nseq,
                      total_tokens, H, P, N, G, chunk, dtype, ws, SSD_NOALLOC_SCRATCH_BYTES,
                      stream);
}

int ssd_scan_prefill_stages(unsigned stages, const void *x, const float *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *h0,
                            float *y, float *h_out, const int32_t *cu_seqlens, int nseq,
                            int64_t total_tokens, int H, int P, int N, int G, int chunk,
                            ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                            void *stream) {
  return prefill_impl(stages, x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, nseq, total_tokens, H,
                      P, N, G, chunk, dtype, workspace, workspace_bytes, stream);
}

int ssd_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
             const float *D, float *h, float *y, int batch, int H, int P, int N, int G,
             ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 0) return fail(SSD_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (H < 1 || G < 1 || H % G != 0) return fail(SSD_ERR_INVALID_ARG, "need H >= 1, G >= 1, H %% G == 0 (H=%d G=%d)", H, G);
  if (!pow2_in(P, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "headdim P=%d not in {16,32,64,128}", P);
  if (N < 1 || N > 1024) return fail(SSD_ERR_UNSUPPORTED, "d_state N=%d not in 1..1024", N);
  if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch > 0 && (!x || !dt || !A || !B || !C || !D || !h || !y))
    return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  ssd::StepArgs a{x, dt, A, B, C, D, h, y, batch, H, P, N, G, dtype == SSD_BF16, stream};
  hipError_t e = ssd::launch_step(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

int ssd_step_multi(const void *x, const float *dt, const float *A, const void *B, const void *C,
                   const float *D, float *h, float *y, int steps, int batch, int H, int P, int N,
                   int G, ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (steps < 0) return fail(SSD_ERR_INVALID_ARG, "steps must be >= 0 (got %d)", steps);
  if (batch < 0) return fail(SSD_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (H < 1 || G < 1 || H % G != 0) return fail(SSD_ERR_INVALID_ARG, "need H >= 1, G >= 1, H %% G == 0 (H=%d G=%d)", H, G);
  if (!pow2_in(P, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "headdim P=%d not in {16,32,64,128}", P);
  if (!pow2_in(N, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "d_state N=%d not in {16,32,64,128}", N);
  if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if ((long long)H * (P / (P > 64 ? 64 : P)) > 0x7fffffff) return fail(SSD_ERR_UNSUPPORTED, "too many heads");
  if (batch > 0 && (!h || (steps > 0 && (!x || !dt || !A || !B || !C || !D || !y))))
    return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  ssd::MultiStepArgs a{x, dt, A, B, C, D, h, y, steps, batch, H, P, N, G, dtype == SSD_BF16, stream};
  hipError_t e = ssd::launch_step_multi(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

int ssd_conv1d_step(const void *u, float *conv_state, const float *w, const float *bias,
                    int silu, void *out, int batch, int channels, int width, ssd_dtype_t dtype,
                    void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 0 || channels < 1) return fail(SSD_ERR_INVALID_ARG, "need batch >= 0, channels >= 1 (batch=%d channels=%d)", batch, channels);
  if (width < 1 || width > 8) return fail(SSD_ERR_UNSUPPORTED, "conv width %d not in 1..8", width);
  if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch > 0 && (!u || !conv_state || !w || !out)) return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  hipError_t e = ssd::launch_conv1d_step(u, conv_state, w, bias, silu != 0, out, batch, channels,
                                         width, dtype == SSD_BF16, false,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

int ssd_gated_rmsnorm(const float *y, const void *z, const float *w, float eps, float *out,
                      int batch, int dim, ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 0 || dim < 1) return fail(SSD_ERR_INVALID_ARG, "need batch >= 0, dim >= 1 (batch=%d dim=%d)", batch, dim);
  if (!(eps >= 0.f)) return fail(SSD_ERR_INVALID_ARG, "eps must be >= 0");
  if (batch > 0 && (!y || !z || !w || !out)) return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  hipError_t e = ssd::launch_gated_rmsnorm(y, z, w, eps, out, batch, dim, dtype == SSD_BF16,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

int ssd_decode_layer_step(const void *xbc, const void *z, const float *dt, const float *A,
                          const float *D, float *conv_state, const float *conv_w,
                          const float *conv_b, float *h, const float *norm_w, float eps,
                          float *out, float *xbc_act, float *y, int batch, int H, int P, int N,
                          int G, int width, ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 0) return fail(SSD_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (H < 1 || G < 1 || H % G != 0) return fail(SSD_ERR_INVALID_ARG, "need H >= 1, G >= 1, H %% G == 0 (H=%d G=%d)", H, G);
  if (!pow2_in(P, 16, 128)) return fail(SSD_ERR_UNSUPPORTED, "headdim P=%d not in {16,32,64,128}", P);
  if (N < 1 || N > 1024 || N % 4 != 0) return fail(SSD_ERR_UNSUPPORTED, "d_state N=%d: need 4 <= N <= 1024, N %% 4 == 0", N);
  if (width < 1 || width > 8) return fail(SSD_ERR_UNSUPPORTED, "conv width %d not in 1..8", width);
  if (!(eps >= 0.f)) return fail(SSD_ERR_INVALID_ARG, "eps must be >= 0");
  if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch > 0 && (!xbc || !z || !dt || !A || !D || !conv_state || !conv_w || !h || !norm_w ||
                    !out || !xbc_act || !y))
    return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  if (batch == 0) return SSD_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = dtype == SSD_BF16;
  const int inner = H * P, channels = inner + 2 * G * N;
  // the convolved channels stay float32 (the scan's arithmetic type), so the
  // layer adds no rounding of its own between the conv and the scan
  hipError_t e = ssd::launch_conv1d_step(xbc, conv_state, conv_w, conv_b, true, xbc_act, batch,
                                         channels, width, bf, true, st);
  if (e == hipSuccess) {
    const float *act = xbc_act;
    ssd::StepArgs a{act, dt, A, act + inner, act + inner + (size_t)G * N, D, h, y, batch, H, P, N,
                    G, false, stream, (size_t)channels, (size_t)channels};
    e = ssd::launch_step(a);
  }
  if (e == hipSuccess) e = ssd::launch_gated_rmsnorm(y, z, norm_w, eps, out, batch, inner, bf, st);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

size_t ssd_selective_scan_workspace(int batch, int L, int dim, int N) {
  if (batch < 0 || L < 0 || dim < 1 || !(N == 1 || N == 2 || N == 4 || N == 8 || N == 16)) return 0;
  return ssd::s6_workspace(batch, L, dim, N);
}

int ssd_selective_scan(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *h0, float *y, float *h_out,
                       int batch, int L, int dim, int N, ssd_dtype_t dtype, void *workspace,
                       size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16 && dtype != SSD_F16)
    return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 0 || L < 0 || dim < 1) return fail(SSD_ERR_INVALID_ARG, "need batch >= 0, L >= 0, dim >= 1 (batch=%d L=%d dim=%d)", batch, L, dim);
  if (!(N == 1 || N == 2 || N == 4 || N == 8 || N == 16)) return fail(SSD_ERR_UNSUPPORTED, "d_state N=%d not in {1,2,4,8,16}", N);
  if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if ((long long)L > 65535LL * (8192 / N)) return fail(SSD_ERR_UNSUPPORTED, "sequence length %d too long", L);
  if (batch > 0 && L > 0 && (!x || !dt || !A || !B || !C || !D || !y))
    return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  if (batch > 0 && !A) return fail(SSD_ERR_INVALID_ARG, "null pointer argument");
  const size_t need = ssd::s6_workspace(batch, L, dim, N);
  if (batch > 0 && (!workspace || workspace_bytes < need))
    return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  ssd::S6Args a{x, dt, A, B, C, D, h0, y, h_out, batch, L, dim, N, (int)dtype, workspace, stream};
  hipError_t e = ssd::launch_selective_scan(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

size_t ssd_scan_prefill_backward_workspace(int64_t total_tokens, int nseq, int H, int P, int N,
                                           int G, int chunk, ssd_dtype_t dtype) {
  if (dtype != SSD_F32 && dtype != SSD_BF16) return 0;
  if (nseq < 1 || total_tokens < 0 || total_tokens > INT32_MAX || H < 1 || G < 1 || H % G != 0)
    return 0;
  if (!pow2_in(P, 16, 128) || !pow2_in(N, 16, 128) || !pow2_in(chunk, 32, 512)) return 0;
  if ((int64_t)chunk * H * P * 4 > INT32_MAX || (int64_t)chunk * G * N * 4 > INT32_MAX) return 0;
  return ssd::bwd_layout(total_tokens, nseq, H, P, N, G, chunk, dtype == SSD_BF16 ? 2 : 4).total;
}

static int backward_impl(bool saved, const void *x, const float *dt, const float *A,
                         const void *B, const void *C, const float *D, const float *h0,
                         const void *dy, const float *dh_out, float *dx, float *ddt, float *dA,
                         float *dB, float *dC, float *dD, float *dh0, const int32_t *cu_seqlens,
                         int nseq, int64_t total_tokens, int H, int P, int N, int G, int chunk,
                         ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                         void *stream) {
  g_err[0] = 0;
  int rc = check_prefill(x, dt, A, B, C, D, dx, nseq, total_tokens, H, P, N, G, chunk, dtype,
                         cu_seqlens);
  if (rc) return rc;
  if (total_tokens > 0 && (!dy || !ddt || !dB || !dC))
    return fail(SSD_ERR_INVALID_ARG, "null dy/ddt/dB/dC pointer");
  if (!dA || !dD) return fail(SSD_ERR_INVALID_ARG, "null dA/dD pointer");
  const ssd::BwdLayout L = ssd::bwd_layout(total_tokens, nseq, H, P, N, G, chunk,
                                           dtype == SSD_BF16 ? 2 : 4);
  if (!workspace || workspace_bytes < L.total)
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  ssd::BwdArgs a{};
  a.f = ssd::PrefillArgs{x, dt, A, B, C, D, h0, nullptr, nullptr, cu_seqlens, nseq,
                         total_tokens, H, P, N, G, chunk, dtype == SSD_BF16, workspace, stream};
  a.dy = dy;
  a.dh_out = dh_out;
  a.dx = dx;
  a.ddt = ddt;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.dh0 = dh0;
  a.saved = saved;
  hipError_t e = ssd::launch_prefill_backward(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

int ssd_scan_prefill_backward(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *h0, const void *dy,
                              const float *dh_out, float *dx, float *ddt,
                              float *dA, float *dB, float *dC, float *dD, float *dh0,
                              const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H,
                              int P, int N, int G, int chunk, ssd_dtype_t dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return backward_impl(false, x, dt, A, B, C, D, h0, dy, dh_out, dx, ddt, dA, dB, dC, dD, dh0,
                       cu_seqlens, nseq, total_tokens, H, P, N, G, chunk, dtype, workspace,
                       workspace_bytes, stream);
}

int ssd_scan_prefill_backward_saved(const void *x, const float *dt, const float *A, const void *B,
                                    const void *C, const float *D, const float *h0,
                                    const void *dy, const float *dh_out, float *dx, float *ddt,
                                    float *dA, float *dB, float *dC, float *dD, float *dh0,
                                    const int32_t *cu_seqlens, int nseq, int64_t total_tokens,
                                    int H, int P, int N, int G, int chunk, ssd_dtype_t dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  return backward_impl(true, x, dt, A, B, C, D, h0, dy, dh_out, dx, ddt, dA, dB, dC, dD, dh0,
                       cu_seqlens, nseq, total_tokens, H, P, N, G, chunk, dtype, workspace,
                       workspace_bytes, stream);
}

int ssd_scan_prefill_train_forward(const void *x, const float *dt, const float *A, const void *B,
                                   const void *C, const float *D, const float *h0, float *y,
                                   float *h_out, const int32_t *cu_seqlens, int nseq,
                                   int64_t total_tokens, int H, int P, int N, int G, int chunk,
                                   ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  g_err[0] = 0;
  int rc = check_prefill(x, dt, A, B, C, D, y, nseq, total_tokens, H, P, N, G, chunk, dtype,
                         cu_seqlens);
  if (rc) return rc;
  const ssd::BwdLayout L = ssd::bwd_layout(total_tokens, nseq, H, P, N, G, chunk,
                                           dtype == SSD_BF16 ? 2 : 4);
  if (!workspace || workspace_bytes < L.total)
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  ssd::PrefillArgs a{x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, nseq, total_tokens, H, P, N, G,
                     chunk, dtype == SSD_BF16, workspace, stream};
  hipError_t e = ssd::launch_prefill_train_forward(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

static int gdn_check(const void *q, const void *k, const void *v, const float *g,
                     const float *beta, float *o, const int32_t *cu_seqlens, int nseq,
                     int64_t total_tokens, int H, int G, int K, int V, ssd_dtype_t dtype) {
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (nseq < 1) return fail(SSD_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (total_tokens < 0 || total_tokens > INT32_MAX) return fail(SSD_ERR_INVALID_ARG, "total_tokens %lld out of range", (long long)total_tokens);
  if (H < 1 || G < 1 || H % G != 0) return fail(SSD_ERR_INVALID_ARG, "need H >= 1, G >= 1, H %% G == 0 (H=%d G=%d)", H, G);
  if (!(K == 64 || K == 128 || K == 256)) return fail(SSD_ERR_UNSUPPORTED, "key dim K=%d not in {64,128,256}", K);
  if (V < 16 || V > 1024 || V % 16 != 0) return fail(SSD_ERR_UNSUPPORTED, "value dim V=%d: need 16 <= V <= 1024, V %% 16 == 0", V);
  if (H > 65535 || nseq > 65535) return fail(SSD_ERR_UNSUPPORTED, "H or nseq above 65535");
  if (!cu_seqlens && total_tokens % nseq != 0)
    return fail(SSD_ERR_INVALID_ARG, "dense batch: total_tokens %lld not divisible by nseq %d", (long long)total_tokens, nseq);
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(SSD_ERR_INVALID_ARG, "null q/k/v/g/beta/o pointer");
  return SSD_OK;
}

int ssd_gated_delta_rule(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, float *o, float *h_out,
                         const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H, int G,
                         int K, int V, ssd_dtype_t dtype, void *stream) {
  g_err[0] = 0;
  const int rc = gdn_check(q, k, v, g, beta, o, cu_seqlens, nseq, total_tokens, H, G, K, V, dtype);
  if (rc != SSD_OK) return rc;
  ssd::GdnArgs a{q, k, v, g, beta, h0, o, h_out, cu_seqlens, nseq, total_tokens, H, G, K, V,
                 dtype == SSD_BF16, stream};
  hipError_t e = ssd::launch_gated_delta_rule(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

size_t ssd_gated_delta_rule_chunked_workspace(int64_t total_tokens, int nseq, int H, int K, int V,
                                              ssd_dtype_t dtype) {
  if (total_tokens < 0 || total_tokens > INT32_MAX || nseq < 1 || H < 1) return 0;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return 0;
  if (!ssd::gdn_chunk_supported(K, V)) return 0;
  return ssd::gdn_chunk_layout(total_tokens, nseq, H, K, V, dtype == SSD_BF16 ? 2 : 4).total;
}

int ssd_gated_delta_rule_chunked(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *h0, float *o, float *h_out,
                                 const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H,
                                 int G, int K, int V, ssd_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  const int rc = gdn_check(q, k, v, g, beta, o, cu_seqlens, nseq, total_tokens, H, G, K, V, dtype);
  if (rc != SSD_OK) return rc;
  if (!ssd::gdn_chunk_supported(K, V))
    return fail(SSD_ERR_UNSUPPORTED, "chunked form: need K in {64,128}, V %% 32 == 0, V + K <= 256 (K=%d V=%d)", K, V);
  const size_t need = ssd::gdn_chunk_layout(total_tokens, nseq, H, K, V, dtype == SSD_BF16 ? 2 : 4).total;
  if (!workspace || workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  ssd::GdnArgs a{q, k, v, g, beta, h0, o, h_out, cu_seqlens, nseq, total_tokens, H, G, K, V,
                 dtype == SSD_BF16, stream, workspace};
  hipError_t e = ssd::launch_gdn_chunked(a);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return SSD_OK;
}

const char *ssd_last_error(void) { return g_err; }

}  // extern "C"
