// ssd_launch.h -- internal interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

struct PrefillArgs {
  const void *x;
  const float *dt, *A;
  const void *B, *C;
  const float *D, *h0;
  float *y, *h_out;
  const int32_t *cu;
  int nseq;
  int64_t T;
  int H, P, N, G, Q;
  bool bf16;
  void *workspace;
  void *stream;
};

// Byte offsets of the prefill workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
  int64_t nc_max;  // upper bound on the number of chunks: floor((T + nseq*(Q-1)) / Q)
  size_t info;     // int4 [max(nc_max,1)]       chunk -> {seq, t0, len, index in seq}
  size_t seq_off;  // int  [nseq+1]              first chunk of each sequence
  size_t s;        // f32  [nc_max][H][Q]        chunk-local cumsum of dt*A
  size_t dt;       // f32  [nc_max][H][Q]        dt, chunk-major (0 on padded rows)
  size_t u;        // f32  [nc_max][H][Q]        2^(s_ref(j) - s_j) dt_j, s_ref(j) = s at the
                   //                            last row of j's 32-row block (log2 units)
  size_t S;        // f32  [nc_max][H][N][P]     chunk states
  size_t hin;      // T    [nc_max][H][N][P]     state entering each chunk (operand type)
  size_t total;
};

WorkspaceLayout prefill_layout(int64_t T, int nseq, int H, int P, int N, int Q, int elem);
hipError_t launch_prefill(const PrefillArgs &a, unsigned stages);

// Stages 1-2: chunk-local cumulative decay (s, dt, u) and, if `state`, the
// chunk states S.
hipError_t launch_chunk_state(const PrefillArgs &a, const WorkspaceLayout &L, int nc, bool state,
                              hipStream_t st);

// Chunk scan with the heads of a B/C group streamed through one workgroup
// (bfloat16, selected P/N/Q).  scan_heads_choice() returns the heads per
// workgroup to use, or 0 where the row-split scan is the better (or only)
// choice; launch_scan_heads() enqueues it over the workspace written by the
// earlier stages.
int scan_heads_choice(int P, int N, int Q, bool bf16, int nc, int H, int G);
hipError_t launch_scan_heads(const PrefillArgs &a, const WorkspaceLayout &L, int nc, int HB,
                             hipStream_t st);

struct StepArgs {
  const void *x;
  const float *dt, *A;
  const void *B, *C;
  const float *D;
  float *h, *y;
  int batch, H, P, N, G;
  bool bf16;
  void *stream;
  size_t x_bstride = 0, bc_bstride = 0;  // elements between batch rows (0: packed)
};
hipError_t launch_step(const StepArgs &a);

struct MultiStepArgs {
  const void *x;
  const float *dt, *A;
  const void *B, *C;
  const float *D;
  float *h, *y;
  int steps, batch, H, P, N, G;
  bool bf16;
  void *stream;
};
hipError_t launch_step_multi(const MultiStepArgs &a);

// Mamba-1 selective scan (ssd_s6.hip).  dtype: 0 float32, 1 bfloat16, 2 float16.
struct S6Args {
  const void *x, *dt;
  const float *A;
  const void *B, *C;
  const float *D, *h0;
  float *y, *h_out;
  int batch, L, dim, N, dtype;
  void *workspace;
  void *stream;
};
struct S6Plan {
  int seg, nseg;  // tokens per segment, segments
};
S6Plan s6_plan(int batch, int L, int dim, int N);
size_t s6_workspace(int batch, int L, int dim, int N);
hipError_t launch_selective_scan(const S6Args &a);

// Decode-layer operations around the scan (ssd_layer.hip).
hipError_t launch_conv1d_step(const void *u, float *state, const float *w, const float *bias,
                              bool silu, void *out, int batch, int channels, int width,
                              bool is_bf16, bool out_f32, hipStream_t st);
hipError_t launch_gated_rmsnorm(const float *y, const void *z, const float *w, float eps,
                                float *out, int batch, int dim, bool is_bf16, hipStream_t st);

}  // namespace ssd
