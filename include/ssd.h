/*
 * ssd.h -- C ABI of libssd.so: the Mamba-2 SSD (state space duality) selective
 * scan on AMD Instinct MI355X (gfx950).
 *
 * The recurrence, per sequence and per head h (head h reads B/C group
 * g = floor(h*G/H)):
 *
 *     a_t       = exp(dt_t * A_h)
 *     h_t[n][p] = a_t * h_{t-1}[n][p] + dt_t * x_t[p] * B_t[n]
 *     y_t[p]    = sum_n C_t[n] * h_t[n][p] + D_h * x_t[p]
 *
 * Sources: COREY: Entropy-Guided Runtime Chunk Scheduling for Selective Scan
 * Kernels, section 3.1 (the generic selective SSM update); Compiler-First State
 * Space Duality and Portable O(1) Autoregressive Caching for Inference,
 * Abstract (one scalar decay per head, equal-length chunks whose work is dense
 * contractions, a decode cache of constant size) and Tables 7-8 (static causal mask inside a
 * chunk; decay kept in float32); Recurrence Scan (poot docs), "One equation,
 * one packed result" and "The schedule" (the scan returns the output and the
 * carried state; a long sequence may be split across launches that hand the
 * state on; shapes that do not fit are refused before any work); Mamba-2 SSD
 * fused layer via VGpuWarp, "S2 RESULT" (the decode state stored so that
 * consecutive lanes touch consecutive addresses).
 *
 * Conventions for every entry point:
 *  - Every array pointer is caller-owned DEVICE memory, row-major, contiguous.
 *    The library never allocates, frees or retains caller memory.
 *  - Work is enqueued on `stream` (hipStream_t passed as void*; NULL = the null
 *    stream) and returns without synchronising.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Return value: SSD_OK, or a negative SSD_ERR_* code.  Arguments are checked
 *    before anything is enqueued; on error nothing is launched and
 *    ssd_last_error() describes the problem.  No C++ exception crosses the ABI.
 *  - Preconditions that are NOT checked (values, not shapes): A_h <= 0,
 *    dt >= 0, all inputs finite.  Under them every exponent is <= 0.
 *  - dtype selects the element type of x, B and C (float32 or bfloat16).
 *    dt, A, D, states and y are always float32; decay math is float32 and
 *    matrix products accumulate in float32.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 } ssd_dtype_t;  /* F16: selective scan only */

enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARG = -1, /* null pointer, negative size, H % G != 0, ... */
    SSD_ERR_UNSUPPORTED = -2, /* P, N or chunk without a compiled instance    */
    SSD_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
    SSD_ERR_HIP = -4          /* a HIP runtime call or launch failed          */
};

/* Stages of the chunked prefill, for ssd_scan_prefill_stages(). */
enum {
    SSD_STAGE_CHUNK_CUMSUM = 1u, /* per-chunk cumulative log-decay s = cumsum(dt*A) */
    SSD_STAGE_CHUNK_STATE = 2u,  /* per-chunk state S_c = sum_j exp(s_end-s_j) dt_j B_j x_j^T */
    SSD_STAGE_STATE_PASS = 4u,   /* sequential carry H_c = exp(s_end) H_{c-1} + S_c     */
    SSD_STAGE_CHUNK_SCAN = 8u,   /* y = intra-chunk (masked C.B^T) x + exp(s) C.H_in + D x */
    SSD_STAGE_ALL = 15u
};

/* Kernel-variant bits, OR-ed into the `stages` mask of
 * ssd_scan_prefill_stages().  Without them the library picks each kernel by
 * problem size; a bit forces one implementation (for tests and tuning).  All
 * variants compute the same result up to floating-point reassociation.  The
 * stage calls of one split sequence must all pass the same bits. */
enum {
    SSD_VARIANT_SCAN_ROWS = 0x100u,  /* chunk scan: a workgroup per (chunk, head, half) */
    SSD_VARIANT_SCAN_HEADS = 0x200u, /* chunk scan: the heads of a B/C group streamed
                                        through one workgroup (bf16, P 64, N 128 and a
                                        few other shapes; otherwise the row split) */
    SSD_VARIANT_STATE_CHUNKS = 0x400u, /* states: every chunk state written, then passed
                                          along the chunks by a second kernel */
    SSD_VARIANT_STATE_WALK = 0x800u,   /* states: one kernel walks each sequence's chunks
                                          with the state in registers (bf16, P 64,
                                          N 128, chunk <= 256; otherwise the chunk
                                          states).  Stages 1,
                                          2 and 4 are then one kernel: each of those bits
                                          runs all three (h_out is written with bit 4) */
    SSD_VARIANT_MASK = 0xF00u
};

/*
 * Workspace bytes needed by ssd_scan_prefill() for `total_tokens` tokens in
 * `nseq` sequences of H heads in G B/C groups (chunking restarts at every
 * sequence start).  Returns 0 for arguments ssd_scan_prefill() would reject
 * (including H % G != 0 and the 2^31 row-offset limit below).  Besides the
 * per-chunk decays and states it holds, for bf16 with P 64, N 128 and
 * chunk <= 256, the intra-chunk C.B^T of every (chunk, group) as bf16
 * fragments (chunk^2 / 512 KB each): SSD_STAGE_STATE_PASS writes them when
 * the row-split chunk scan will run, and SSD_STAGE_CHUNK_SCAN reads them.
 */
size_t ssd_scan_prefill_workspace(int64_t total_tokens, int nseq, int H, int P, int N, int G,
                                  int chunk, ssd_dtype_t dtype);

/*
 * The kernels ssd_scan_prefill() would run for these shapes (packed != 0: a
 * cu_seqlens array will be passed): one SSD_VARIANT_STATE_* bit for the
 * states and one SSD_VARIANT_SCAN_* bit for the chunk scan; 0 for arguments
 * the prefill would reject.  A planning query: nothing is enqueued.
 */
unsigned ssd_scan_prefill_plan(int64_t total_tokens, int nseq, int H, int P, int N, int G,
                               int chunk, ssd_dtype_t dtype, int packed);

/*
 * Chunked SSD prefill over a packed batch of sequences.
 *
 *   x        [T][H][P]      dtype       inputs
 *   dt       [T][H]         float32     step sizes (softplus already applied)
 *   A        [H]            float32     per-head decay rate (<= 0)
 *   B, C     [T][G][N]      dtype       input / output projections
 *   D        [H]            float32     per-head skip
 *   h0       [nseq][H][N][P] float32    initial states, or NULL for zeros
 *   y        [T][H][P]      float32     output (must not alias any input)
 *   h_out    [nseq][H][N][P] float32    final states, or NULL to skip; may be
 *                                        the same pointer as h0 (read first)
 *   cu_seqlens  device int32 [nseq+1], cu[0] = 0, non-decreasing, cu[nseq] = T;
 *            or NULL for a dense batch of nseq sequences of T/nseq tokens each.
 *            The values are not checked on the host (they live on the device);
 *            the kernels give a sequence that starts below 0 or ends past T no
 *            chunks and never index past the buffers the other arguments size,
 *            but the outputs of a malformed array are unspecified
 *   chunk    chunk length Q; the result is the same for every supported Q up
 *            to floating-point reassociation
 *   workspace / workspace_bytes   device scratch of at least
 *            ssd_scan_prefill_workspace(...) bytes (256-byte aligned)
 *
 * Supported: P in {16,32,64,128}, N in {16,32,64,128}, chunk in
 * {32,64,128,256,512}, H % G == 0, and H*P*chunk*4 and G*N*chunk*4 below
 * 2^31 (a chunk's rows are addressed with 32-bit offsets; otherwise
 * SSD_ERR_UNSUPPORTED).  A chunk of 16 is refused (SSD_ERR_UNSUPPORTED): the
 * matrix-core step over tokens is 32 wide, and any chunk gives the same
 * result up to reassociation.  T = 0 copies h0 (or zeros) to h_out.
 * Splitting a sequence at any token and passing h_out of the first part as h0
 * of the second gives the same result as one call.
 */
int ssd_scan_prefill(const void *x, const float *dt, const float *A, const void *B,
                     const void *C, const float *D, const float *h0, float *y, float *h_out,
                     const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H, int P,
                     int N, int G, int chunk, ssd_dtype_t dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * ssd_scan_prefill() without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, serving loops, harnesses
 * that forbid hipMalloc): the workspace is a device array inside the library,
 * SSD_NOALLOC_SCRATCH_BYTES bytes per device, held from library load until
 * the process ends.  Arguments, results and errors as ssd_scan_prefill(), with
 * every stage and the library's kernel choice; shapes whose
 * ssd_scan_prefill_workspace() exceeds SSD_NOALLOC_SCRATCH_BYTES are refused
 * with SSD_ERR_WORKSPACE before anything touches the device.  Nothing is
 * allocated: the first call on a device only looks up the array's address.
 * Every call on one device shares that device's array and leaves its contents
 * behind (no stage reads what an earlier call left there): calls that overlap
 * on one device -- on different streams, or from different threads -- race,
 * so serialise them.
 */
#define SSD_NOALLOC_SCRATCH_BYTES (32u << 20)
int ssd_scan_prefill_noalloc(const void *x, const float *dt, const float *A, const void *B,
                             const void *C, const float *D, const float *h0, float *y,
                             float *h_out, const int32_t *cu_seqlens, int nseq,
                             int64_t total_tokens, int H, int P, int N, int G, int chunk,
                             ssd_dtype_t dtype, void *stream);

/*
 * The same computation as ssd_scan_prefill(), running only the stages in the
 * bitmask `stages` (SSD_STAGE_*, optionally with SSD_VARIANT_* bits).  Stages
 * communicate through the workspace, so running CHUNK_CUMSUM, CHUNK_STATE,
 * STATE_PASS and CHUNK_SCAN in that order, in one call or in four calls with
 * identical arguments, equals one ssd_scan_prefill() call.  Used to time and
 * test each stage, and each kernel variant, on its own.  Other bits:
 * SSD_ERR_INVALID_ARG.
 */
int ssd_scan_prefill_stages(unsigned stages, const void *x, const float *dt, const float *A,
                            const void *B, const void *C, const float *D, const float *h0,
                            float *y, float *h_out, const int32_t *cu_seqlens, int nseq,
                            int64_t total_tokens, int H, int P, int N, int G, int chunk,
                            ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * One decode token for `batch` independent states, updated in place.
 *
 *   x   [batch][H][P]  dtype;  dt [batch][H] float32;  A, D [H] float32
 *   B,C [batch][G][N]  dtype
 *   h   [batch][H][N][P] float32, read and overwritten with the new state
 *       (layout n-major, p fastest: consecutive lanes touch consecutive bytes)
 *   y   [batch][H][P]  float32 (must not alias any input)
 *
 * Supported: P in {16,32,64,128}, N in {1..1024}, H % G == 0.
 * Equal to ssd_scan_prefill() over one token with h0 = h.
 */
int ssd_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
             const float *D, float *h, float *y, int batch, int H, int P, int N, int G,
             ssd_dtype_t dtype, void *stream);

/*
 * `steps` decode tokens for `batch` independent states in one launch, over
 * inputs staged for every step; the state is updated in place.  Equal to
 * `steps` successive ssd_step() calls with the slices of step t.
 *
 *   x   [steps][batch][H][P]  dtype;  dt [steps][batch][H] float32
 *   A, D [H] float32;  B, C [steps][batch][G][N]  dtype
 *   h   [batch][H][N][P] float32, read at the start, overwritten at the end
 *   y   [steps][batch][H][P] float32 (must not alias any input)
 *
 * The state stays on chip for all steps: it crosses HBM once instead of twice
 * per step.  This is the decode loop kept on the device with one launch from
 * the host (Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference, Figure 1; the loop's throughput is its
 * Table 10), with the steps run as a stream over time as in Recurrence Scan,
 * "The schedule".
 * Supported: P in {16,32,64,128}, N in {16,32,64,128}, H % G == 0.
 * steps = 0 or batch = 0 does nothing.
 */
int ssd_step_multi(const void *x, const float *dt, const float *A, const void *B, const void *C,
                   const float *D, float *h, float *y, int steps, int batch, int H, int P, int N,
                   int G, ssd_dtype_t dtype, void *stream);

/*
 * Decode-layer operations on either side of the scan (Mamba-2 SSD fused layer
 * via VGpuWarp -- design sketch, its list of layer steps to move onto the
 * device: the causal conv1d step, a per-channel FIR over d_conv taps with a
 * rolling buffer kept in device memory, and the gated RMS norm, y times
 * silu(z), then the root mean square over d_inner, times norm_w).
 *
 * ssd_conv1d_step: one token of a causal depthwise convolution.
 *   u          [batch][channels]         dtype    this token's inputs
 *   conv_state [batch][channels][width]  float32  window, oldest tap first;
 *              rolled in place (drops the oldest, appends u)
 *   w          [channels][width] float32;  bias [channels] float32 or NULL
 *   out        [batch][channels]         dtype    bias + sum_k w[c][k] win[c][k],
 *              then v * sigmoid(v) when silu != 0 (must not alias any input)
 *   Supported: width in 1..8.
 */
int ssd_conv1d_step(const void *u, float *conv_state, const float *w, const float *bias,
                    int silu, void *out, int batch, int channels, int width, ssd_dtype_t dtype,
                    void *stream);

/*
 * ssd_gated_rmsnorm: out = g / sqrt(mean_d(g^2) + eps) * w with g = y * silu(z),
 * per token row.
 *   y [batch][dim] float32;  z [batch][dim] dtype;  w [dim] float32;  eps >= 0
 *   out [batch][dim] float32 (must not alias y or z)
 */
int ssd_gated_rmsnorm(const float *y, const void *z, const float *w, float eps, float *out,
                      int batch, int dim, ssd_dtype_t dtype, void *stream);

/*
 * ssd_decode_layer_step: the layer body around the scan for one token, all on
 * the device: conv1d step (with SiLU) over the x|B|C channels, ssd_step on
 * the convolved x, B, C, then the gated RMS norm of y.  Equal to
 * ssd_conv1d_step(silu=1) + ssd_step + ssd_gated_rmsnorm.
 *   xbc      [batch][H*P + 2*G*N]  dtype    in_proj's x | B | C channels
 *   z        [batch][H*P]          dtype    gate
 *   dt       [batch][H] float32;  A, D [H] float32
 *   conv_state [batch][H*P + 2*G*N][width] float32, rolled in place
 *   conv_w   [H*P + 2*G*N][width] float32;  conv_b [H*P + 2*G*N] float32 or NULL
 *   h        [batch][H][N][P] float32, updated in place
 *   norm_w   [H*P] float32;  eps >= 0
 *   out      [batch][H*P] float32   the normalised, gated scan output
 *   xbc_act  [batch][H*P + 2*G*N] float32, y [batch][H*P] float32: caller-owned
 *            scratch (the convolved channels, kept in the scan's float32, and
 *            the scan output)
 *   Supported: P in {16,32,64,128}, 4 <= N <= 1024 with N % 4 == 0,
 *   width in 1..8, H % G == 0.
 */
int ssd_decode_layer_step(const void *xbc, const void *z, const float *dt, const float *A,
                          const float *D, float *conv_state, const float *conv_w,
                          const float *conv_b, float *h, const float *norm_w, float eps,
                          float *out, float *xbc_act, float *y, int batch, int H, int P, int N,
                          int G, int width, ssd_dtype_t dtype, void *stream);

/*
 * Mamba-1 selective scan: a diagonal transition per channel d and state n (the
 * per-channel form of the selective update of COREY: Entropy-Guided Runtime
 * Chunk Scheduling for Selective Scan Kernels, section 3.1, discretised as the
 * SSD path; the kernel its section 5.1 times at batch 1, d 1024, L 4096,
 * d_state 16):
 *     h_t[d][n] = exp(dt_t[d] A[d][n]) h_{t-1}[d][n] + dt_t[d] B_t[n] x_t[d]
 *     y_t[d]    = sum_n C_t[n] h_t[d][n] + D[d] x_t[d]
 *
 *   x, dt   [batch][L][dim]   dtype (float32, bfloat16 or float16)
 *   A       [dim][N] float32 (<= 0);  D [dim] float32
 *   B, C    [batch][L][N]     dtype
 *   h0      [batch][dim][N] float32, or NULL for zeros
 *   y       [batch][L][dim] float32 (must not alias any input)
 *   h_out   [batch][dim][N] float32, or NULL; may be h0
 *   workspace / workspace_bytes: device scratch of at least
 *           ssd_selective_scan_workspace(batch, L, dim, N) bytes
 * Arithmetic is float32.  Supported: N in {1,2,4,8,16}.  L = 0 copies h0 (or
 * zeros) to h_out.  Splitting the sequence and passing h_out on as h0 gives
 * the same result as one call.
 */
size_t ssd_selective_scan_workspace(int batch, int L, int dim, int N);
int ssd_selective_scan(const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *h0, float *y, float *h_out,
                       int batch, int L, int dim, int N, ssd_dtype_t dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Gradients of ssd_scan_prefill() -- the backward half of a training step
 * (Compiler-First State Space Duality and Portable O(1) Autoregressive Caching
 * for Inference, Table 13: forward plus backward of the chunked scan) -- for a
 * loss L with dL/dy = dy and dL/dh_out = dh_out.
 *
 *   x, dt, A, B, C, D, h0, cu_seqlens, nseq, total_tokens, H, P, N, G, chunk,
 *   dtype      exactly as passed to ssd_scan_prefill()
 *   dy       [T][H][P]       dtype    dL/dy
 *   dh_out   [nseq][H][N][P] float32  dL/dh_out, or NULL for zeros
 * Outputs (float32; each written in full, none may alias an input or another):
 *   dx [T][H][P], ddt [T][H], dA [H], dB [T][G][N], dC [T][G][N], dD [H],
 *   dh0 [nseq][H][N][P] (or NULL to skip)
 *   workspace / workspace_bytes  device scratch of at least
 *            ssd_scan_prefill_backward_workspace(...) bytes (256-byte aligned)
 *
 * Per chunk, with G_t = dL/dh_t: dx_t = D dy_t + dt_t B_t^T G_t,
 * dB_t = dt_t G_t x_t (summed over the heads of a group), dC_t = h_t dy_t,
 * and dL/d(dt_t A) = <G_t, h_t> - dt_t x_t^T G_t^T B_t, from which ddt and dA
 * follow.  The states are recomputed from the inputs: nothing is kept from the
 * forward call.  Sums over heads, chunks and sequences run in a fixed order:
 * the result is deterministic.  Supported shapes as ssd_scan_prefill().
 * T = 0 gives dA = dD = 0 and dh0 = dh_out (or zeros).
 */
size_t ssd_scan_prefill_backward_workspace(int64_t total_tokens, int nseq, int H, int P, int N,
                                           int G, int chunk, ssd_dtype_t dtype);
int ssd_scan_prefill_backward(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *h0, const void *dy,
                              const float *dh_out, float *dx, float *ddt,
                              float *dA, float *dB, float *dC, float *dD, float *dh0,
                              const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H,
                              int P, int N, int G, int chunk, ssd_dtype_t dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * A training step without the backward's forward recompute.
 *
 * ssd_scan_prefill_train_forward() computes y and h_out exactly as
 * ssd_scan_prefill() (bitwise) and leaves in `workspace` -- sized by
 * ssd_scan_prefill_backward_workspace() for the same shapes and chunk -- the
 * chunk map, the chunk-local decays, the states entering every chunk (operand
 * type and float32) and the final states, which the backward would otherwise
 * recompute.  ssd_scan_prefill_backward_saved() then takes the same arguments
 * as ssd_scan_prefill_backward() and skips that recompute: its results are
 * bitwise those of ssd_scan_prefill_backward().  Preconditions (not checked):
 * the inputs (x, dt, A, B, C, D, h0, cu_seqlens) and shapes are the training
 * forward's, and nothing wrote the workspace in between except other
 * ssd_scan_prefill_backward_saved() calls on it (the backward leaves the
 * saved part intact, so the same forward serves several backward calls).
 * Errors as ssd_scan_prefill() / ssd_scan_prefill_backward().
 */
int ssd_scan_prefill_train_forward(const void *x, const float *dt, const float *A, const void *B,
                                   const void *C, const float *D, const float *h0, float *y,
                                   float *h_out, const int32_t *cu_seqlens, int nseq,
                                   int64_t total_tokens, int H, int P, int N, int G, int chunk,
                                   ssd_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                   void *stream);
int ssd_scan_prefill_backward_saved(const void *x, const float *dt, const float *A, const void *B,
                                    const void *C, const float *D, const float *h0,
                                    const void *dy, const float *dh_out, float *dx, float *ddt,
                                    float *dA, float *dB, float *dC, float *dD, float *dh0,
                                    const int32_t *cu_seqlens, int nseq, int64_t total_tokens,
                                    int H, int P, int N, int G, int chunk, ssd_dtype_t dtype,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gated delta rule scan: the delta-rule family of Recurrence Scan (poot docs:
 * gated delta rule layers replace attention by a per-head state matrix that
 * each token updates and that is carried from step to step; the scan returns
 * the output and the carried state, "One equation, one packed result"; "The
 * schedule": a streaming kernel with a workgroup per head and block of state
 * columns, the state on chip, a runtime loop over tokens, and a state column's
 * rows shared by several lanes that add their partial dot products each token).
 * The page writes no equation; this is the published gated delta rule, per
 * sequence and head h (q, k read group g = floor(h*G/H)), state S [V][K]:
 *
 *     a_t = exp(g_t);   S_t = a_t S_{t-1} + beta_t (v_t - a_t S_{t-1} k_t) k_t^T
 *     o_t = S_t q_t
 *
 *   q, k     [T][G][K]       dtype    query and key (already normalised/scaled:
 *                                     the library applies no L2 norm or scale)
 *   v        [T][H][V]       dtype
 *   g        [T][H]          float32  log-gate, <= 0 (not checked)
 *   beta     [T][H]          float32  write strength (after its activation)
 *   h0       [nseq][H][V][K] float32  initial states, or NULL for zeros
 *   o        [T][H][V]       float32  output (must not alias any input)
 *   h_out    [nseq][H][V][K] float32  final states, or NULL; may be h0
 *   cu_seqlens  device int32 [nseq+1] or NULL (dense: nseq sequences of T/nseq);
 *            as for the prefill (non-decreasing, cu[nseq] = T); values outside
 *            0 .. T are clamped into it, so no access leaves the buffers, but
 *            the outputs of a malformed array are unspecified
 * Supported: K in {64,128,256}, V a multiple of 16 up to 1024, H % G == 0.
 * Arithmetic and the state are float32.  No workspace.  Splitting a sequence
 * and passing h_out on as h0 gives the same result as one call.
 */
int ssd_gated_delta_rule(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, float *o, float *h_out,
                         const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H, int G,
                         int K, int V, ssd_dtype_t dtype, void *stream);

/*
 * The same gated delta rule in chunks of 64 tokens, with the work on MFMA:
 * within a chunk the recurrence is regrouped exactly into a unit
 * lower-triangular system (I + A) D = diag(beta) V - diag(beta gamma) K S_0^T
 * for the chunk's write vectors D, whose state-free part (U, W) is solved for
 * every chunk at once, and three products per chunk carry the state: D = U -
 * W S_0^T, O = diag(gamma) Q S_0^T + P D and S_C = gamma_C S_0 + D~^T K, with
 * gamma the chunk-local cumulative gate, A_tj = beta_t (gamma_t/gamma_j)
 * k_t.k_j and P_tj = (gamma_t/gamma_j) q_t.k_j (j < t, resp. j <= t).
 * Arguments as ssd_gated_delta_rule(), plus
 *   workspace / workspace_bytes   device scratch of at least
 *            ssd_gated_delta_rule_chunked_workspace(...) bytes (256-aligned)
 * Supported: K in {64,128}, V a multiple of 32 with V + K <= 256, H % G == 0
 * (the workspace query returns 0 for other shapes: use the streaming call).
 * Arithmetic float32; with bfloat16 operands the state and D enter the
 * products as bfloat16 pairs (hi + lo) and U, W, P are held in bfloat16.
 * h_out may be h0.  Errors as ssd_gated_delta_rule(), and SSD_ERR_WORKSPACE.
 */
size_t ssd_gated_delta_rule_chunked_workspace(int64_t total_tokens, int nseq, int H, int K, int V,
                                              ssd_dtype_t dtype);
int ssd_gated_delta_rule_chunked(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *h0, float *o, float *h_out,
                                 const int32_t *cu_seqlens, int nseq, int64_t total_tokens, int H,
                                 int G, int K, int V, ssd_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char *ssd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
