// ssd_prefill.hip -- chunked SSD prefill on gfx950: stage launcher, chunk map,
// state pass and the row-split chunk scan.
//
// Math (per sequence, head h, chunk c of Q tokens; all exponents <= 0):
//   s_i    = sum_{k<=i} dt_k A_h                         (chunk-local, float32)
//   S_c    = sum_j exp(s_{Q-1} - s_j) dt_j  B_j x_j^T     (N x P chunk state)
//   H_c    = exp(s_{Q-1}) H_{c-1} + S_c,   H_{-1} = h0     (state carried across chunks)
//   y_i    = sum_{j<=i} (C_i . B_j) exp(s_i - s_j) dt_j x_j   (intra-chunk, causal)
//          + exp(s_i) C_i . H_{c-1}                         (state entering the chunk)
//          + D_h x_i
// This is the unrolled recurrence regrouped into chunks of one fixed length:
// the structured-state-space-duality form of Compiler-First State Space
// Duality and Portable O(1) Autoregressive Caching for Inference (Abstract:
// each head decays by one scalar per step, the sequence is cut into equal
// chunks and the work inside a chunk is dense contractions), with the static
// lower-triangular mask of its Table 7 and the float32 decay of its Table 8;
// the state is handed from chunk to chunk as in Recurrence Scan ("One
// equation, one packed result").
//
// Kernels (one launch each, all on the caller's stream):
//   k_chunk_map        (packed batches only) chunk -> {sequence, first token, length}
//   k_chunk_state      s, dt, u and S_c^T = (w o X)^T B on MFMA     (ssd_chunk_state.hip)
//   k_state_pass       grid (NP/1024,H,nseq): sequential H_c over the chunks of a sequence
//   k_chunk_scan       y, one wave per 16-token tile: C.B^T (k = N), mask/decay,
//                      Y^T = X^T M^T (k = tokens) and 2^s H^T C^T (k = N) on MFMA
//   k_chunk_scan_heads y for large batches, heads of a group streamed  (ssd_scan_heads.hip)
// Every padded row of a partial chunk has dt = 0, x = 0, B = 0: it changes
// nothing (decay 1, no input), so the chunk-end value s_{Q-1} equals
// s_{len-1}.  The workspace holds s in base-2 units (s * log2(e)) so every
// decay is one v_exp_f32 (2^x) of a non-positive argument.
#include "ssd.h"
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

// ---------------------------------------------------------------- chunk map
// Chunks restart at every sequence start: chunk k of sequence s covers tokens
// cu[s] + kQ .. min(cu[s] + (k+1)Q, cu[s+1]) - 1.  info = {seq, t0, len, k}.

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Block-wide inclusive scan (blockDim.x a multiple of 64, <= 1024).
__device__ int block_incl_scan(int v, int *sh, int &total) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) sh[wave] = v;
  __syncthreads();
  int prefix = 0;
  total = 0;
  for (int w = 0; w < nw; ++w) {
    int s = sh[w];
    if (w < wave) prefix += s;
    total += s;
  }
  __syncthreads();
  return v + prefix;
}

// Resolve chunk c of the packed batch into {seq, t0, len, index} (block-wide;
// O(nseq / blockDim) block scans).  Block (0, 0) also writes seq_off.
__device__ int4 locate_chunk(const int32_t *__restrict__ cu, int nseq, int L_dense, int64_t T,
                             int Q, int c, int nc_max, int *__restrict__ seq_off,
                             bool write_off) {
  __shared__ int sh_scan[16];
  __shared__ int4 sh_info;
  const int tid = threadIdx.x;
  if (tid == 0) sh_info = make_int4(-1, 0, 0, 0);
  __syncthreads();
  if (cu == nullptr) {
    const int cps = (L_dense + Q - 1) / Q;
    if (tid == 0 && cps > 0) {
      const int seq = c / cps, k = c % cps;
      if (seq < nseq) sh_info = make_int4(seq, seq * L_dense + k * Q, min(Q, L_dense - k * Q), k);
    }
    if (write_off)
      for (int s = tid; s <= nseq; s += blockDim.x) seq_off[s] = s * cps;
  } else {
    int running = 0;
    for (int base = 0; base < nseq; base += blockDim.x) {
      const int s = base + tid;
      int start = 0, len = 0;
      if (s < nseq) {
        start = cu[s];
        len = max(0, cu[s + 1] - start);
        if (start < 0 || (int64_t)start + len > T) len = 0;  // malformed: no chunks
      }
      const int cnt = (len + Q - 1) / Q;
      int total;
      const int incl = block_incl_scan(cnt, sh_scan, total);
      const int excl = incl - cnt;
      if (cnt > 0 && running + excl <= c && c < running + incl) {
        const int k = c - running - excl;
        sh_info = make_int4(s, start + k * Q, min(Q, len - k * Q), k);
      }
      // chunk offsets clamped to the workspace's chunk count: overlapping
      // sequences (cu decreasing somewhere) could otherwise ask for more
      // chunks than the buffers hold
      if (write_off && s < nseq) seq_off[s] = min(running + excl, nc_max);
      running += total;
    }
    if (write_off && tid == 0) seq_off[nseq] = min(running, nc_max);
  }
  __syncthreads();
  return sh_info;
}

// Chunk map of a packed batch: grid (chunks), 256 threads; block c writes
// info[c], block 0 also the first chunk of every sequence.  (A dense batch
// needs neither: its map is arithmetic.)
__global__ __launch_bounds__(256) void k_chunk_map(const int32_t *__restrict__ cu, int nseq,
                                                   int64_t T, int Q, int nc_max,
                                                   int4 *__restrict__ info_out,
                                                   int *__restrict__ seq_off) {
  const int c = blockIdx.x;
  const int4 ci = locate_chunk(cu, nseq, 0, T, Q, c, nc_max, seq_off, blockIdx.x == 0);
  if (c < nc_max && threadIdx.x == 0) info_out[c] = ci.x < 0 ? make_int4(0, 0, 0, 0) : ci;
}

hipError_t launch_chunk_map(const int32_t *cu, int nseq, int64_t T, int Q, int nc, int4 *info,
                            int *seq_off, hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_map, dim3(nc > 0 ? nc : 1), dim3(256), 0, st, cu, nseq, T, Q, nc, info,
                     seq_off);
  return hipGetLastError();
}

// ----------------------------------------------------------- K3 state pass
// Per (sequence, head), per 4 state elements: walk the sequence's chunks in
// order, emit the state entering each chunk (as the MFMA operand type, and
// optionally as float32) and the final state (to h_out, and to h_out2 when
// given).  For the row-split scan with precomputed C.B^T, the same launch
// carries the C.B^T units (cbg_unit) in extra z-slices past the sequences.

// C.B^T for the row-split chunk scan, once per (chunk, B/C group) instead of
// once per head (bf16, N = 128): one wave per (chunk, group, 16-row output
// tile t, 32-row block k <= t/2 of source rows j) forms the pair of 16x16
// results (B_j . C_i) of the scan's block step -- the same MFMA
// sequence, rows past the chunk read as zero -- and stores them rounded to
// bf16 in that step's fragment order (lane l: column i = 16 t + l % 16, rows
// j = 32 k + 4 (l / 16) + r and 32 k + 16 + 4 (l / 16) + r): 1 KB per (t, k).
// Blocks starting past the chunk end are never read and not written.
struct CbgArgs {
  const bf16 *B, *C;
  bf16 *out;  // [nc][G][Q/16][Q/32][64][8]
  int G, nc, nz;  // nz: z-slices of the state pass proper (its sequences)
};
__device__ __forceinline__ void cbg_unit(const CbgArgs &a, ChunkMap cmap, int Q, int u) {
  constexpr int N = 128, KS = N / 32;
  const int NT = Q / 16, NKB = Q / 32;
  // unit u = (chunk * G + group) * npairs + p over the blocks the scan reads,
  // k <= t/2: tiles 2m and 2m+1 read m+1 blocks each, so the pairs of tiles
  // below m hold m (m+1) units; one 1 KB block per unit, a single round trip
  const int npairs = (NT / 2) * (NT / 2 + 1);
  const int cg = u / npairs, p = u - cg * npairs, c = cg / a.G, gr = cg - c * a.G;
  if (c >= a.nc) return;
  int m = (int)((__builtin_sqrtf(4.f * p + 1.f) - 1.f) * 0.5f);
  while (m * (m + 1) > p) --m;
  while ((m + 1) * (m + 2) <= p) ++m;
  const int r = p - m * (m + 1), hi = r > m ? 1 : 0;
  const int t = 2 * m + hi, k = r - hi * (m + 1);
  const int4 ci = cmap(c);
  const int len = ci.z;
  if (len <= 0 || 32 * k >= len) return;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const size_t bstride = (size_t)a.G * N;
  const bf16 *Cg = a.C + (size_t)ci.y * bstride + (size_t)gr * N;
  const bf16 *Bg = a.B + (size_t)ci.y * bstride + (size_t)gr * N;
  const int i = 16 * t + col;
  Frag<bf16> cf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    cf[ks] = i < len ? frag_global(Cg + (size_t)i * bstride + ks * 32 + 8 * grp) : frag_zero<bf16>();
  bf16 *out = a.out + (((size_t)cg * NT + t) * NKB + k) * 512;
  const int j0 = 32 * k + col, j1 = j0 + 16;
  Frag<bf16> b0[KS], b1[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int n8 = ks * 32 + 8 * grp;
    b0[ks] = j0 < len ? frag_global(Bg + (size_t)j0 * bstride + n8) : frag_zero<bf16>();
    b1[ks] = j1 < len ? frag_global(Bg + (size_t)j1 * bstride + n8) : frag_zero<bf16>();
  }
  f4 g0 = zero4(), g1 = zero4();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    mma(g0, b0[ks], cf[ks]);
    mma(g1, b1[ks], cf[ks]);
  }
  *reinterpret_cast<bf16x8 *>(out + lane * 8) =
      cvt_bf8(f8v{g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]});
}

template <typename T>
__global__ __launch_bounds__(256) void k_state_pass(const float *__restrict__ S,
                                                    const float *__restrict__ s_ws,
                                                    const int *__restrict__ seq_off,
                                                    ChunkMap cmap, const float *h0, float *h_out,
                                                    T *__restrict__ hin, int H, int NP, int Q,
                                                    float *__restrict__ hin32, float *h_out2,
                                                    CbgArgs cbg) {
  constexpr int BATCH = 8;  // chunk states in flight per thread
  // extra z-slices (dispatched after every block of the walk): C.B^T units,
  // four a block
  if (sizeof(T) == 2 && (int)blockIdx.z >= cbg.nz) {
    const int lb = (((int)blockIdx.z - cbg.nz) * (int)gridDim.y + (int)blockIdx.y) *
                       (int)gridDim.x + (int)blockIdx.x;
    cbg_unit(cbg, cmap, Q, lb * 4 + (int)(threadIdx.x >> 6));
    return;
  }
  const int s = blockIdx.z, hd = blockIdx.y;
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= NP) return;
  int c0, c1;  // chunks of sequence s
  if (cmap.L > 0) {
    const int cps = (cmap.L + Q - 1) / Q;
    c0 = s * cps;
    c1 = c0 + cps;
  } else {
    c0 = seq_off[s];
    c1 = seq_off[s + 1];
  }
  const size_t hofs = ((size_t)s * H + hd) * NP + e;
  f4 st = h0 ? ld4(h0 + hofs) : zero4();
  for (int cb = c0; cb < c1; cb += BATCH) {
    f4 Sb[BATCH];
    float sl[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (cb + u < c1) {
        const size_t ch = (size_t)(cb + u) * H + hd;
        Sb[u] = ld4(S + ch * NP + e);
        sl[u] = s_ws[ch * Q + Q - 1];
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (cb + u < c1) {
        st4T(hin + ((size_t)(cb + u) * H + hd) * NP + e, st);
        if (hin32) st4(hin32 + ((size_t)(cb + u) * H + hd) * NP + e, st);
        const float a = __builtin_amdgcn_exp2f(fminf(sl[u], 0.f));
#pragma unroll
        for (int q = 0; q < 4; ++q) st[q] = a * st[q] + Sb[u][q];
      }
    }
  }
  if (h_out) st4(h_out + hofs, st);
  if (h_out2) st4(h_out2 + hofs, st);
}

// ------------------------------------------------------------ K4 chunk scan
// One workgroup per (chunk, head, part z of SPLIT), one wave per 16-token
// output tile.  Q <= 128: SPLIT 1, Q/16 waves.  Q >= 256: SPLIT 2, Q/32
// waves: part z owns tiles t_k = 2k + (z ^ (k & 1)), whose causal work is k + 1
// j-blocks in both parts, and wave w takes k = w for w < NW/2, else
// k = 3NW/2 - 1 - w, so the waves sharing a SIMD carry equal work.  At Q = 256
// a part has 8 waves and stages 64 rows per phase (under 53 KB of LDS), so
// three workgroups share a CU and some load while others compute.
// Per output tile (all accumulation in float32):
//   Y^T[p][i]  = 2^(s_i) (H_in^T C^T)[p][i]             k = n    (A: H_in tile, transpose read)
//             += sum_j X^T[p][j] M^T[j][i]              k = j    (A: X tile, transpose read)
//             += D x_i                                  (while the tile's own rows are staged)
//   M^T[j][i]  = (B C^T)[j][i] 2^(s_i - s_j) dt_j  (j <= i)      k = n
// The two 16x16 results of B C^T for rows jb..jb+15 and jb+16..jb+31 are fed
// straight back as the B operand (paired k map); X^T is read with the same
// pairing.  Staging uses the direct global->LDS load (16 bytes per lane, lane
// l writing base + 16 l): H_in and the first JP rows of B and X are requested
// together with no staging registers, so each phase of JP rows costs one memory
// round trip.  With CBG (bf16, P 64, N 128, chunk <= 256, small batches) the
// B C^T pairs come precomputed per (chunk, group) from the state-pass launch
// (cbg_unit) as 1 KB fragment blocks read one block ahead: no B tile, and
// 128-row phases of X.
template <typename T, int P, int N> struct ScanCfg {
  static constexpr int NK = N < 32 ? 32 : N;  // contraction over n, padded to the k-step
  static constexpr int KS = NK / 32;
  static constexpr int VN = 16 / sizeof(T);
  static constexpr int XP = P + kTrPad, BP = NK + row_pad<T>(), HP = P + kTrPad;
  static constexpr int XS = XP / VN, BS = BP / VN, HS = HP / VN;  // 16-byte slots per row
  static constexpr int XD = P / VN, BD = N / VN;                   // data slots per row
  // bf16 with 128-byte x and H_in rows and 256-byte B rows: block-swizzled
  // tiles (whole-block loads, no padding slots) instead of padded rows
  static constexpr bool SWZ = sizeof(T) == 2 && P == 64 && N == 128;
  // one float row of q values, staged whole 1 KB requests at a time
  static constexpr size_t frow_bytes(int q) { return ((size_t)q * 4 + 1023) / 1024 * 1024; }
  // cbg: C.B^T comes precomputed (no B tile)
  static constexpr size_t lds_bytes(int jp, int q, bool cbg = false) {
    if (SWZ)
      return (size_t)(NK / 8 + jp / 8) * kBlk128 + (cbg ? 0 : (size_t)(jp / 4) * kBlk256) +
             3 * frow_bytes(q);
    return (size_t)(tile_slots(NK, HS) + tile_slots(jp, BS) + tile_slots(jp, XS)) * 16 +
           12 * (size_t)q;
  }
  // staged rows per phase for chunk length q and `threads`: up to 64 rows
  // (128 without a B tile) in blocks of at most 512 threads (under 53 KB, so
  // three workgroups share a CU and the row-split grid of a small batch is
  // resident at once), up to 256 rows otherwise, halved until the LDS fits
  static int jp(int q, int threads, bool cbg = false) {
    const int lim = threads <= 512 ? (cbg ? 128 : 64) : 256;
    int j = q < lim ? q : lim;
    const size_t cap = threads <= 512 ? 53 * 1024 : 160 * 1024;
    while (j > 32 && lds_bytes(j, q, cbg) > cap) j /= 2;
    return j;
  }
};

template <typename T, int P, int N, int SPLIT, bool CBG>
__global__ __launch_bounds__(1024) void k_chunk_scan(
    const T *__restrict__ x, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ s_ws, const float *__restrict__ dt_ws,
    const float *__restrict__ u_ws, const T *__restrict__ hin, ChunkMap cmap, int nc, int H,
    int G, int Q, int JP, float *__restrict__ y, const T *__restrict__ cbg) {
  typedef ScanCfg<T, P, N> K;
  constexpr int KS = K::KS, NK = K::NK, XP = K::XP, BP = K::BP, HP = K::HP;
  constexpr int NPT = P / 16;
  constexpr bool SWZ = K::SWZ;
  static_assert(!CBG || SWZ, "precomputed C.B^T only with the block-swizzled tiles");
  const ChunkHead ch = xcd_chunk_head(H * SPLIT);
  const int c = ch.c, hd = ch.h / SPLIT, part = ch.h % SPLIT;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  if (ci.z <= 0) return;
  const int len = ci.z;
  const int g = (hd * G) / H;
  const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;
  int tile = wave;
  if (SPLIT == 2) {
    const int k = wave < nw / 2 ? wave : 3 * nw / 2 - 1 - wave;
    tile = 2 * k + (part ^ (k & 1));
  }
  const int t0 = 16 * tile;  // first row of the wave's tile (wave-uniform)

  extern __shared__ __align__(16) char smem[];
  // padded layout: H_in [NK][HP], B [JP][BP], X [JP][XP] (elements)
  T *Hs = reinterpret_cast<T *>(smem);
  T *Bs = Hs + tile_slots(NK, K::HS) * K::VN;
  T *Xs = Bs + tile_slots(JP, K::BS) * K::VN;
  // swizzled layout: H_in NK/8 blocks, B JP/4 blocks, X JP/8 blocks
  char *Hc = smem;
  char *Bc = Hc + (NK / 8) * kBlk128;
  char *Xc = Bc + (CBG ? 0 : (JP / 4) * kBlk256);
  float *s_l = SWZ ? reinterpret_cast<float *>(Xc + (JP / 8) * kBlk128)
                   : reinterpret_cast<float *>(Xs + tile_slots(JP, K::XS) * K::VN);  // [Q]
  // [Q] each (swizzled layout: rows rounded up to 1 KB, filled by whole requests)
  const int FR = SWZ ? (int)K::frow_bytes(Q) / 4 : Q;
  float *dt_l = s_l + FR;
  float *u_l = dt_l + FR;  // 2^(s_ref(j) - s_j) dt_j, s_ref(j) = s at the end of j's 32-block

  const size_t csh = (size_t)c * H + hd;
  const T *xs = x + ((size_t)ci.y * H + hd) * P;
  const T *bs = B + ((size_t)ci.y * G + g) * N;
  const size_t xstride = (size_t)H * P, bstride = (size_t)G * N;
  // swizzled loads: byte strides, and each lane's offset into a block's rows
  const uint32_t xsb = (uint32_t)(xstride * sizeof(T)), bsb = (uint32_t)(bstride * sizeof(T));
  const int lb8 = lane >> 3, lb4 = lane >> 4;
  const uint32_t xl = lb8 * xsb + 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  const uint32_t bl = lb4 * bsb + 16 * ((lane & 15) ^ lb4);
  const uint32_t hl = lb8 * (P * sizeof(T)) + 16 * ((lane & 7) ^ (2 * swz8(lb8)));

  // ---- prologue: H_in, the first phase of B/X, C fragments and decays in flight together
  if constexpr (SWZ) {
    const int v0 = max(0, min(len, JP));
    dma_swz<kBlk128>(Hc, hin + csh * (size_t)(N * P), N * P * sizeof(T), hl, 1024, NK / 8, wave, nw);
    if (!CBG) dma_swz<kBlk256>(Bc, bs, v0 * bsb, bl, 4 * bsb, JP / 4, wave, nw);
    dma_swz<kBlk128>(Xc, xs, v0 * xsb, xl, 8 * xsb, JP / 8, wave, nw);
    // the chunk's s, dt and u rows (written by the chunk-state stage), one
    // wave each
    const uint32_t fl = 16 * lane;
    const int nr = FR / 256, w1 = (wave + nw - 1 % nw) % nw, w2 = (wave + nw - 2 % nw) % nw;
    dma_swz<1024>(reinterpret_cast<char *>(s_l), s_ws + csh * Q, Q * 4, fl, 1024, nr, wave, nw);
    dma_swz<1024>(reinterpret_cast<char *>(dt_l), dt_ws + csh * Q, Q * 4, fl, 1024, nr, w1, nw);
    dma_swz<1024>(reinterpret_cast<char *>(u_l), u_ws + csh * Q, Q * 4, fl, 1024, nr, w2, nw);
  } else {
    dma_tile<T, K::HS, K::XD>(Hs, hin + csh * (size_t)(N * P), (size_t)P, NK, N, wave, nw);
    dma_tile<T, K::BS, K::BD>(Bs, bs, bstride, JP, len, wave, nw);
    dma_tile<T, K::XS, K::XD>(Xs, xs, xstride, JP, len, wave, nw);
  }
  const T *Cg = C + ((size_t)ci.y * G + g) * N;
  Frag<T> cf[KS];
  const int i = t0 + col;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int n8 = ks * 32 + 8 * grp;
    cf[ks] = (i < len && n8 < N) ? frag_global(Cg + (size_t)i * bstride + n8) : frag_zero<T>();
  }
  const float si = s_ws[csh * Q + i];
  if (!SWZ) {
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
      s_l[j] = s_ws[csh * Q + j];
      dt_l[j] = dt_ws[csh * Q + j];
      u_l[j] = u_ws[csh * Q + j];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's direct-to-LDS loads have landed
  __syncthreads();

  // lane byte offsets into the swizzled tiles (bits 5-6 hold the segment
  // swizzle, so segment pt is reached by XOR with 32 pt):
  //  H_in rows ks*32 + 8 grp + col/4 (+4): block 4 ks + grp, row col/4 (+4)
  //  X rows jl + 4 grp + col/4 (+16): block jl/8 + grp/2 (+2), row 4 (grp&1) + col/4
  //  B rows jl + col (+16): block jl/4 + col/4 (+4), row col&3, vector 4 ks + grp
  //  D x, row r0 + col: block r0/8 + col/8, row col&7, 8 bytes at 32 pt + 8 grp
  const int c4 = col >> 2, cq = 8 * (col & 3);
  const int hlo = grp * kBlk128 + c4 * 128 + cq + 32 * swz8(c4);
  const int hhi = grp * kBlk128 + (4 + c4) * 128 + cq + 32 * swz8(4 + c4);
  const int xb = 4 * (grp & 1) + c4;
  const int xo = (grp >> 1) * kBlk128 + xb * 128 + cq + 32 * swz8(xb);
  const int bo = c4 * kBlk256 + (col & 3) * 256 + 16 * (grp ^ (col & 3));
  const int dxo = (col >> 3) * kBlk128 + (col & 7) * 128 + 8 * grp + 32 * swz8(col & 7);

  // ---- state entering the chunk: Y^T = 2^(s_i) H_in^T C^T
  const bool live = t0 < len;  // wave-uniform
  f4 acc[NPT];
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) acc[pt] = zero4();
  if (live) {
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> a;
        if constexpr (SWZ)
          a = frag_kmaj_at(Hc + ks * 4 * kBlk128, hlo ^ (32 * pt), hhi ^ (32 * pt));
        else
          a = frag_kmaj(Hs, HP, pt * 16, ks * 32 + 8 * grp, ks * 32 + 8 * grp + 4);
        mma(acc[pt], a, cf[ks]);
      }
    }
    const float ei = __builtin_amdgcn_exp2f(fminf(si, 0.f));
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[pt][r] *= ei;
  }

  const int tile_last = min(t0 + 15, len - 1);
  const float dv = D[hd];
  for (int ph = 0; ph < len; ph += JP) {  // phases past the chunk length add nothing
    if (ph > 0) {  // stage the next JP rows (one round trip)
      __syncthreads();
      if constexpr (SWZ) {
        const int vr = min(len - ph, JP);
        if (!CBG)
          dma_swz<kBlk256>(Bc, bs + (size_t)ph * bstride, vr * bsb, bl, 4 * bsb, JP / 4, wave, nw);
        dma_swz<kBlk128>(Xc, xs + (size_t)ph * xstride, vr * xsb, xl, 8 * xsb, JP / 8, wave, nw);
      } else {
        dma_tile<T, K::BS, K::BD>(Bs, bs + (size_t)ph * bstride, bstride, JP, len - ph, wave, nw);
        dma_tile<T, K::XS, K::XD>(Xs, xs + (size_t)ph * xstride, xstride, JP, len - ph, wave, nw);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    const bool mine = live && t0 >= ph && t0 < ph + JP;  // the tile's own rows are staged
    if (mine) {  // skip term D x_i
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        f4 xv;
        if constexpr (SWZ)
          xv = ld4f(reinterpret_cast<const T *>(Xc + (t0 - ph) / 8 * kBlk128 + (dxo ^ (32 * pt))));
        else
          xv = ld4f(Xs + (t0 + col - ph) * XP + pt * 16 + 4 * grp);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[pt][r] += dv * xv[r];
      }
    }
    const int jend = live ? min(ph + JP, tile_last + 1) : ph;
    // precomputed C.B^T: this tile's 1 KB fragments, one block ahead
    const T *gt =
        CBG ? cbg + ((((size_t)c * G + g) * (Q / 16) + tile) * (Q / 32)) * 512 + lane * 8 : cbg;
    typedef typename Vec16<T>::type Vg;
    Vg gnext = vzero<Vg>();
    if (CBG && ph < jend) gnext = *reinterpret_cast<const Vg *>(gt + (ph / 32) * 512);
    for (int jb = ph; jb < jend; jb += 32) {
      const int jl = jb - ph;
      f4 g0 = zero4(), g1 = zero4();  // G^T = B C^T for this j-block
      if constexpr (CBG) {
        const Vg gcur = gnext;
        if (jb + 32 < jend) gnext = *reinterpret_cast<const Vg *>(gt + (jb / 32 + 1) * 512);
        const f8v gf = cvt_f8(gcur);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g0[r] = gf[r];
          g1[r] = gf[4 + r];
        }
      }
#pragma unroll
      for (int ks = 0; ks < (CBG ? 0 : KS); ++ks) {
        Frag<T> b0, b1;
        if constexpr (SWZ) {
          const char *bb = Bc + (jl / 4) * kBlk256 + 64 * ks;
          b0 = frag_rowk_at(bb, bo);
          b1 = frag_rowk_at(bb + 4 * kBlk256, bo);
        } else {
          b0 = frag_rowk(Bs, BP, jl + col, ks * 32 + 8 * grp);
          b1 = frag_rowk(Bs, BP, jl + 16 + col, ks * 32 + 8 * grp);
        }
        mma(g0, b0, cf[ks]);
        mma(g1, b1, cf[ks]);
      }
      float m[8];
      if (jb + 31 < t0) {
        // block entirely before the tile: no mask, and the decay factors through
        // the block end, 2^(s_i - s_ref) * [2^(s_ref - s_j) dt_j], both <= 1
        const float v = __builtin_amdgcn_exp2f(fminf(si - s_l[jb + 31], 0.f));
        const f4 u0 = ld4(u_l + jb + 4 * grp), u1 = ld4(u_l + jb + 16 + 4 * grp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          m[r] = g0[r] * u0[r] * v;
          m[4 + r] = g1[r] * u1[r] * v;
        }
      } else {  // block holding the tile's rows: causal mask, exact decay
        const f4 sj0 = ld4(s_l + jb + 4 * grp), sj1 = ld4(s_l + jb + 16 + 4 * grp);
        const f4 dj0 = ld4(dt_l + jb + 4 * grp), dj1 = ld4(dt_l + jb + 16 + 4 * grp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j0 = jb + 4 * grp + r, j1 = j0 + 16;
          // every argument is clamped to <= 0, so each product is finite; the
          // mask is a select (no branch)
          const float e0 = __builtin_amdgcn_exp2f(fminf(si - sj0[r], 0.f)) * dj0[r];
          const float e1 = __builtin_amdgcn_exp2f(fminf(si - sj1[r], 0.f)) * dj1[r];
          m[r] = j0 <= i ? g0[r] * e0 : 0.f;
          m[4 + r] = j1 <= i ? g1[r] * e1 : 0.f;
        }
      }
      const Frag<T> mf = frag_from_f32(m, T());
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {  // Y^T += X^T M^T
        Frag<T> a;
        if constexpr (SWZ) {
          const char *xb_ = Xc + (jl / 8) * kBlk128;
          a = frag_kmaj_at(xb_, xo ^ (32 * pt), (xo ^ (32 * pt)) + 2 * kBlk128);
        } else {
          a = frag_kmaj(Xs, XP, pt * 16, jl + 4 * grp, jl + 16 + 4 * grp);
        }
        mma(acc[pt], a, mf);
      }
    }
    if (mine && i < len) {  // the tile has seen every j <= i: store it now
      const size_t row = ((size_t)ci.y + i) * H + hd;
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
        __builtin_nontemporal_store(acc[pt], reinterpret_cast<f4 *>(y + row * P + pt * 16 + 4 * grp));
    }
  }
}

// ------------------------------------------------------------------ launch
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

WorkspaceLayout prefill_layout(int64_t T, int nseq, int H, int P, int N, int G, int Q,
                               int elem) {
  WorkspaceLayout L{};
  const int64_t nc = (T + (int64_t)nseq * (Q - 1)) / Q;
  L.nc_max = nc;
  size_t off = 0;
  L.info = off;
  off = align_up(off + 16 * (size_t)(nc > 0 ? nc : 1), 256);
  L.seq_off = off;
  off = align_up(off + 4 * (size_t)(nseq + 1), 256);
  L.s = off;
  off = align_up(off + 4 * (size_t)nc * H * Q, 256);
  L.dt = off;
  off = align_up(off + 4 * (size_t)nc * H * Q, 256);
  L.u = off;
  off = align_up(off + 4 * (size_t)nc * H * Q, 256);
  L.S = off;
  off = align_up(off + 4 * (size_t)nc * H * N * P, 256);
  L.hin = off;
  off = align_up(off + (size_t)elem * nc * H * N * P, 256);
  L.cbg = off;
  L.has_cbg = elem == 2 && P == 64 && N == 128 && Q <= 256;
  if (L.has_cbg) off = align_up(off + (size_t)nc * G * (Q / 16) * (Q / 32) * 1024, 256);
  L.bfrag = off;
  L.has_bfrag = walk_supported(P, N, Q, elem == 2);
  if (L.has_bfrag) off = align_up(off + (size_t)nc * G * Q * N * 2, 256);
  // the walk's piece end states: one per segment of a chain, or per run piece
  // (a packed batch walked by lists), at most one per (chunk, head): fits in S,
  // which the walk leaves unused
  L.segend = L.S;
  L.total = off;
  return L;
}

// Which implementation runs each part of a call: SSD_VARIANT_STATE_* for the
// states (stages 1, 2, 4) and SSD_VARIANT_SCAN_* for the chunk scan.
unsigned prefill_plan(int64_t T, int nseq, int H, int P, int N, int G, int Q, bool bf16,
                      bool packed, unsigned variant) {
  const int64_t nc = (T + (int64_t)nseq * (Q - 1)) / Q;
  const int L_dense = packed ? 0 : (int)(T / nseq);
  const int nc_real = L_dense > 0 ? nseq * ((L_dense + Q - 1) / Q) : (int)nc;
  const bool walk = nc > 0 && walk_choice(P, N, Q, bf16, nseq, H, nc, packed, variant);
  const int HB = scan_heads_choice(P, N, Q, bf16, nc_real, H, G, variant);
  return (walk ? SSD_VARIANT_STATE_WALK : SSD_VARIANT_STATE_CHUNKS) |
         (HB > 0 ? SSD_VARIANT_SCAN_HEADS : SSD_VARIANT_SCAN_ROWS);
}

template <typename T, int P, int N>
static hipError_t run_prefill(const PrefillArgs &a, unsigned stages) {
  const WorkspaceLayout L = prefill_layout(a.T, a.nseq, a.H, P, N, a.G, a.Q, sizeof(T));
  char *ws = static_cast<char *>(a.workspace);
  int4 *info = reinterpret_cast<int4 *>(ws + L.info);
  int *seq_off = reinterpret_cast<int *>(ws + L.seq_off);
  float *s_ws = reinterpret_cast<float *>(ws + L.s);
  float *dt_ws = reinterpret_cast<float *>(ws + L.dt);
  float *u_ws = reinterpret_cast<float *>(ws + L.u);
  float *S = reinterpret_cast<float *>(ws + L.S);
  T *hin = reinterpret_cast<T *>(ws + L.hin);
  const int nc = (int)L.nc_max;
  const int L_dense = a.cu ? 0 : (int)(a.T / a.nseq);
  const ChunkMap cmap{info, L_dense, a.nseq, a.Q};
  hipStream_t st = static_cast<hipStream_t>(a.stream);

  // the state walk does stages 1, 2 and 4 in one kernel
  const bool walk =
      nc > 0 && walk_choice(P, N, a.Q, a.bf16, a.nseq, a.H, nc, a.cu != nullptr, a.variant,
                            a.hin32 != nullptr);
  if ((stages & (walk ? 7u : 3u)) && (a.cu || L_dense == 0)) {
    // packed (or empty) batch: chunk map first.  Block 0 also writes the first
    // chunk of every sequence, which the state pass reads even when there are
    // no chunks at all (then every entry is 0).
    hipLaunchKernelGGL(k_chunk_map, dim3(nc > 0 ? nc : 1), dim3(256), 0, st, a.cu, a.nseq, a.T,
                       a.Q, nc, info, seq_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (walk && (stages & 7u)) {
    hipError_t e = launch_state_walk(a, L, nc, (stages & 4u) != 0, st);
    if (e != hipSuccess) return e;
  } else if ((stages & 3u) && nc > 0) {  // cumulative decay (stage 1) and chunk states (stage 2)
    hipError_t e = launch_chunk_state(a, L, nc, (stages & 2u) != 0, st);
    if (e != hipSuccess) return e;
  }
  // the head-count choice counts the chunks exactly for a dense batch (nc is
  // an upper bound)
  const int nc_real = L_dense > 0 ? a.nseq * ((L_dense + a.Q - 1) / a.Q) : nc;
  const int HB = scan_heads_choice(P, N, a.Q, a.bf16, nc_real, a.H, a.G, a.variant);
  // the row-split scan reads C.B^T precomputed per (chunk, group) where the
  // workspace holds it; the state-pass launch forms it (stage 4), in extra
  // workgroups that run beside the latency-bound walk over the chunks, unless
  // no scan will read this workspace
  const bool use_cbg = L.has_cbg && HB == 0 && ScanCfg<T, P, N>::SWZ;
  const bool form_cbg = use_cbg && a.scan_follows;
  T *cbg = reinterpret_cast<T *>(ws + L.cbg);
  if (stages & 4u) {
    const int NP = N * P, npb = (NP + 1023) / 1024;
    CbgArgs ca{nullptr, nullptr, nullptr, a.G, nc, a.nseq};
    int gz = 0;
    if (form_cbg && nc > 0) {
      ca.B = reinterpret_cast<const bf16 *>(a.B);
      ca.C = reinterpret_cast<const bf16 *>(a.C);
      ca.out = reinterpret_cast<bf16 *>(cbg);
      const long units = (long)nc * a.G * (a.Q / 32) * (a.Q / 32 + 1);
      const long blocks = (units + 3) / 4, per_z = (long)npb * a.H;
      gz = (int)((blocks + per_z - 1) / per_z);
    }
    // with the walk, the launch carries only the C.B^T units (if any)
    if (walk) ca.nz = 0;
    const int gzs = walk ? gz : a.nseq + gz;
    if (gzs > 0) {
      hipLaunchKernelGGL(k_state_pass<T>, dim3(npb, a.H, gzs), dim3(256), 0, st, S, s_ws,
                         seq_off, cmap, a.h0, a.h_out, hin, a.H, NP, a.Q, a.hin32, a.h_out2, ca);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((stages & 8u) && nc > 0 && HB > 0) {
    hipError_t e = launch_scan_heads(a, L, nc, HB, st);
    if (e != hipSuccess) return e;
  } else if ((stages & 8u) && nc > 0) {
    // Q <= 128: one workgroup of Q/16 waves per (chunk, head); Q >= 256: two of Q/32 waves
    typedef ScanCfg<T, P, N> K;
    const int split = a.Q >= 256 ? 2 : 1;
    const int threads = 64 * (a.Q / 16) / split;
    const int jp = K::jp(a.Q, threads, use_cbg);
    const size_t lds = K::lds_bytes(jp, a.Q, use_cbg);
    if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
    const void *kern;
    if constexpr (K::SWZ) {
      if (use_cbg)
        kern = split == 1 ? (const void *)k_chunk_scan<T, P, N, 1, true>
                          : (const void *)k_chunk_scan<T, P, N, 2, true>;
      else
        kern = split == 1 ? (const void *)k_chunk_scan<T, P, N, 1, false>
                          : (const void *)k_chunk_scan<T, P, N, 2, false>;
    } else {
      kern = split == 1 ? (const void *)k_chunk_scan<T, P, N, 1, false>
                        : (const void *)k_chunk_scan<T, P, N, 2, false>;
    }
    hipError_t e = set_lds_limit(kern);
    if (e != hipSuccess) return e;
    const T *xp = (const T *)a.x, *bp = (const T *)a.B, *cp = (const T *)a.C;
    const T *hp = (const T *)hin;
    int nc_ = nc, H_ = a.H, G_ = a.G, Q_ = a.Q, jp_ = jp;
    const float *Dp = a.D;
    float *yp = a.y;
    ChunkMap cm = cmap;
    const T *gp = cbg;
    void *args[] = {&xp, &bp, &cp, &Dp, &s_ws, &dt_ws, &u_ws, &hp, &cm, &nc_, &H_, &G_, &Q_, &jp_,
                    &yp, &gp};
    e = hipLaunchKernel(kern, dim3(xcd_grid(nc, a.H * split)), dim3(threads), args, lds, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int P>
static hipError_t dispatch_N(const PrefillArgs &a, unsigned stages) {
  switch (a.N) {
    case 16: return run_prefill<T, P, 16>(a, stages);
    case 32: return run_prefill<T, P, 32>(a, stages);
    case 64: return run_prefill<T, P, 64>(a, stages);
    case 128: return run_prefill<T, P, 128>(a, stages);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_P(const PrefillArgs &a, unsigned stages) {
  switch (a.P) {
    case 16: return dispatch_N<T, 16>(a, stages);
    case 32: return dispatch_N<T, 32>(a, stages);
    case 64: return dispatch_N<T, 64>(a, stages);
    case 128: return dispatch_N<T, 128>(a, stages);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs &a, unsigned stages) {
  return a.bf16 ? dispatch_P<bf16>(a, stages) : dispatch_P<float>(a, stages);
}

}  // namespace ssd
