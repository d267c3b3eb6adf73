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
  float *hin32 = nullptr;  // optional float32 copy of the state entering each chunk
  float *h_out2 = nullptr;  // optional second destination of the final state
  unsigned variant = 0;     // SSD_VARIANT_* bits (0: the library's choice by size)
  bool scan_follows = true; // false: no chunk scan reads this workspace (skip C.B^T)
  // bf16: chunk states from the decay-weighted operand split into two bf16
  // operands (its rounded value and the rounding's remainder), in either state
  // kernel; the training forward and the backward's recompute, whose gradients
  // amplify the states' rounding
  bool precise_states = false;
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
  // bf16 C.B^T fragments of each (chunk, group) for the row-split chunk scan,
  // [nc_max][G][Q/16][Q/32][64 lanes][8], present (has_cbg) for bf16 with
  // P 64, N 128 and chunk <= 256
  size_t cbg;
  bool has_cbg;
  // B of every (chunk, group) in MFMA fragment order for the state walk,
  // [nc_max][G][Q/32][N/16][64 lanes][8] bf16 (bf16 with P 64, N 128)
  size_t bfrag;
  bool has_bfrag;
  // the state walk writes no chunk states; walking a sequence in segments, it
  // keeps each segment's end state f32 [nseq][nseg][H][N][P] in the S region
  size_t segend;
  size_t total;
};

WorkspaceLayout prefill_layout(int64_t T, int nseq, int H, int P, int N, int G, int Q, int elem);
unsigned prefill_plan(int64_t T, int nseq, int H, int P, int N, int G, int Q, bool bf16,
                      bool packed, unsigned variant);
hipError_t launch_prefill(const PrefillArgs &a, unsigned stages);

// Stages 1-2: chunk-local cumulative decay (s, dt, u) and, if `state`, the
// chunk states S.  With `bwd` (a.x = dy, a.B = C): only the gradient chunk
// states Sb_c = sum_t 2^(s_t) C_t dy_t^T, written over S.
hipError_t launch_chunk_state(const PrefillArgs &a, const WorkspaceLayout &L, int nc, bool state,
                              hipStream_t st, bool bwd = false);

// Stages 1, 2 and 4 in one kernel for large batches (ssd_state_walk.hip): a
// workgroup per (sequence, head) walks the sequence's
// chunks in order with the state in registers, writing s, dt, u and the
// entering states (operand type) -- the chunk states never reach memory.
// walk_choice() says whether the library uses it for a call (the variant bits
// force either way); launch_state_walk() enqueues it (after the chunk map of a
// packed batch), writing h_out only when write_hout.
constexpr long kWalkMinChains = 128;
bool walk_supported(int P, int N, int Q, bool bf16);
bool walk_choice(int P, int N, int Q, bool bf16, int nseq, int H, int64_t nc, bool packed,
                 unsigned variant, bool training = false);
hipError_t launch_state_walk(const PrefillArgs &a, const WorkspaceLayout &L, int nc,
                             bool write_hout, hipStream_t st);

// Chunk scan with the heads of a B/C group streamed through one workgroup
// (bfloat16, selected P/N/Q).  scan_heads_choice() returns the heads per
// workgroup to use, or 0 where the row-split scan is the better (or only)
// choice; launch_scan_heads() enqueues it over the workspace written by the
// earlier stages.
int scan_heads_choice(int P, int N, int Q, bool bf16, int nc, int H, int G, unsigned variant);
hipError_t launch_scan_heads(const PrefillArgs &a, const WorkspaceLayout &L, int nc, int HB,
                             hipStream_t st);

// Gradients of the prefill (ssd_backward.hip).
struct BwdArgs {
  PrefillArgs f;        // the forward's inputs (f.y and f.h_out unused)
  const void *dy;       // dL/dy, operand type
  const float *dh_out;  // dL/dh_out or null
  float *dx, *ddt, *dA, *dB, *dC, *dD, *dh0;  // dh0 may be null
  bool saved = false;   // the workspace holds a training forward's states: no recompute
};
// The forward's workspace followed by the gradient pass's regions.
struct BwdLayout {
  WorkspaceLayout fwd;
  size_t hfin;    // f32 [nseq][H][N][P]  final states (the forward recompute)
  size_t hin32;   // f32 [nc][H][N][P]    state entering each chunk, float32
  size_t dHc;     // T   [nc][H][N][P]    dL/d(state leaving chunk c)
  size_t dHlo;    // bf16 [nc][H][N][P]    dL/d(state) - dHc, bfloat16 only (DX scan)
  size_t epart;   // f32 [nc][H][NP/64]   16-lane-row partials of <dH_c, H_c>
  size_t rows;             // f32 6 x [nc][H][Q]  per-row terms of dz (q, cv, r, dyx, rs x 2)
  size_t dApart, dDpart;   // f32 [nc][H]
  size_t dBh, dCh;         // f32 [T][H/hb][N]  partial dB, dC per block of hb heads
                           //                  (absent when one block holds a whole group)
  size_t total;
};
BwdLayout bwd_layout(int64_t T, int nseq, int H, int P, int N, int G, int Q, int elem);
hipError_t launch_prefill_backward(const BwdArgs &a);
// The forward of a training step: y and h_out as launch_prefill, leaving in
// the backward workspace (f.workspace) everything the backward would
// recompute (chunk map, s, dt, u, the entering states as operand type and
// float32, the final states).
hipError_t launch_prefill_train_forward(const PrefillArgs &f);

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

// Gated delta rule (ssd_gdn.hip).
struct GdnArgs {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  float *o, *h_out;
  const int32_t *cu;
  int nseq;
  int64_t T;
  int H, G, K, V;
  bool bf16;
  void *stream;
  void *workspace = nullptr;  // chunked form only
};
hipError_t launch_gated_delta_rule(const GdnArgs &a);

// Chunked gated delta rule (ssd_gdn_chunk.hip): supported shapes, workspace
// layout (byte offsets, 256-aligned) and the launch.
struct GdnLayout {
  int64_t nc_max;        // upper bound on the chunks of 64 tokens
  size_t info, seq_off;  // chunk map of a packed batch
  size_t U, W, P;        // T [T][H][V], [T][H][K], [T][H][64]
  size_t E;              // f32 [T][H][2]  gamma_t and the write scale 2^(G_C - G_t)
  size_t total;
};
bool gdn_chunk_supported(int K, int V);
GdnLayout gdn_chunk_layout(int64_t T, int nseq, int H, int K, int V, int elem);
hipError_t launch_gdn_chunked(const GdnArgs &a);

// Chunk map of a packed batch for chunk length Q (ssd_prefill.hip).
hipError_t launch_chunk_map(const int32_t *cu, int nseq, int64_t T, int Q, int nc, int4 *info,
                            int *seq_off, hipStream_t st);

// Decode-layer operations around the scan (ssd_layer.hip).
hipError_t launch_conv1d_step(const void *u, float *state, const float *w, const float *bias,
                              bool silu, void *out, int batch, int channels, int width,
                              bool is_bf16, bool out_f32, hipStream_t st);
hipError_t launch_gated_rmsnorm(const float *y, const void *z, const float *w, float eps,
                                float *out, int batch, int dim, bool is_bf16, hipStream_t st);

}  // namespace ssd
