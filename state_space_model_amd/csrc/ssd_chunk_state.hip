// ssd_chunk_state.hip -- first stage of the chunked prefill: per (chunk, head)
// the chunk-local cumulative decay and the chunk state, in one kernel.
//
// Per chunk c and head h (s in log2 units, all exponents <= 0):
//   s_i  = log2(e) A_h sum_{k<=i} dt_k
//   S_c  = sum_j 2^(s_{Q-1} - s_j) dt_j B_j x_j^T            (N x P, float32)
// The chunk state is the part of the state at the chunk end contributed by
// the chunk's own tokens: the recurrence h_t = exp(dt_t A_h) h_{t-1} +
// dt_t x_t (x) B_t unrolled over one chunk with a zero entering state
// (Compiler-First State Space Duality and Portable O(1) Autoregressive
// Caching for Inference, Abstract; float32 decay as in its Table 8).
//
// Also written for the later stages: s, dt and u_j = 2^(s_r - s_j) dt_j (r the
// last row of j's 32-row block), each [chunk][head][Q].
//
// The gradient pass runs the same kernel with BWD set, on C and dy in place of
// B and x: Sb_c = sum_t 2^(s_t) C_t dy_t^T, the gradient that the chunk's own
// outputs send to the state entering it (y_t holds 2^(s_t) C_t . H_in).
//
// One workgroup per (chunk, head), or per (chunk, head, half of the n
// columns) when there are few chunks and heads.  Every load of a phase (x
// rows, B rows, and the strided dt column) goes straight to LDS in one batch:
// one memory round trip before the scan, the x scaling and the MFMAs.
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

template <typename T, int P, int N, int NH_> struct StateCfg {
  static constexpr int NH = NH_;              // workgroups per (chunk, head)
  static constexpr int NN = N / NH;           // n columns per workgroup
  static constexpr int VN = 16 / (int)sizeof(T);
  // pitch = width + one 16-byte slot: the transpose reads of lane groups 8
  // rows apart (one read pass) then fall on disjoint banks
  static constexpr int XP = P + VN, BP = NN + VN;
  static constexpr int XS = XP / VN, BS = BP / VN, XD = P / VN, BD = NN / VN;
  static constexpr int TILES = (P / 16) * (NN / 16);
  static constexpr int NW = TILES >= 8 ? 8 : 4;  // waves (at least 4 for the scan)
  static constexpr int TPW = (TILES + NW - 1) / NW;
  static constexpr int THREADS = 64 * NW;
  // bf16 with 128-byte x rows and 128- or 256-byte B rows: block-swizzled tiles
  static constexpr bool SWZ = sizeof(T) == 2 && P == 64 && (NN == 64 || NN == 128);
  static constexpr int B_BLK = NN == 64 ? kBlk128 : kBlk256T;  // B block pitch
  static constexpr int B_RPB = NN == 64 ? 8 : 4;               // B rows per block
  static constexpr size_t lds_bytes(int jp, int q) {
    const size_t tiles = SWZ ? (size_t)(jp / 8) * kBlk128 + (size_t)(jp / B_RPB) * B_BLK
                             : (size_t)(tile_slots(jp, XS) + tile_slots(jp, BS)) * 16;
    return tiles + 4 * (size_t)(3 * q + 64 + 16);  // dt (staged, padded), s, w, scan partials
  }
  // rows staged per phase: at most `cap`, halved until the LDS fits in 80 KB
  static int jp(int q, int cap) {
    int j = q < cap ? q : cap;
    while (j > 32 && lds_bytes(j, q) > 80 * 1024) j /= 2;
    return j;
  }
};

// Scale rows [0, rows) of a token-major LDS tile by w[r0 + r] (float32
// arithmetic, rounded back to T).
template <typename T, int PITCH, int DATA>
__device__ __forceinline__ void scale_rows(T *tile, const float *w, int r0, int rows) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::n;
  for (int idx = threadIdx.x; idx < rows * DATA; idx += blockDim.x) {
    const int r = idx / DATA, v = idx % DATA;
    V *p = reinterpret_cast<V *>(tile + r * PITCH + v * VN);
    *p = vscale(*p, w[r0 + r]);
  }
}

// scale_rows for a block-swizzled tile of 128-byte rows (a row's vectors are
// permuted within the row, which a per-row scale does not see)
template <typename T>
__device__ __forceinline__ void scale_rows_swz(char *tile, const float *w, int r0, int rows) {
  typedef typename Vec16<T>::type V;
  for (int idx = threadIdx.x; idx < rows * 8; idx += blockDim.x) {
    const int r = idx >> 3;
    V *p = reinterpret_cast<V *>(tile + (r >> 3) * kBlk128 + (r & 7) * 128 + 16 * (idx & 7));
    *p = vscale(*p, w[r0 + r]);
  }
}

// The chunk's cumulative decay from its dt column (dt_l, staged in LDS; rows
// past the chunk length hold 0): s_l = log2(e) A cumsum(dt) -- R consecutive
// rows per thread, then a block scan -- and w_l[j] = 2^(s_end - s_j) dt_j
// (with `bwd`: w_l[j] = 2^(s_j).
// With `emit`, s, dt and u_j = 2^(s_r - s_j) dt_j (r the last row of j's
// 32-row block) are written at out_off of s_out / dt_out / u_out.  Contains
// block barriers: every thread of the block calls it.  Returns s_end.
template <int THREADS>
__device__ __forceinline__ float decay_scan(const float *dt_l, float *s_l, float *w_l,
                                            float *part, int Q, float a2, bool emit, bool bwd,
                                            size_t out_off, float *__restrict__ s_out,
                                            float *__restrict__ dt_out,
                                            float *__restrict__ u_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = (Q + THREADS - 1) / THREADS;  // 1 or 2 (Q <= 512)
  float v0 = 0.f, v1 = 0.f;
  if (tid * R < Q) v0 = dt_l[tid * R] * a2;
  if (R > 1 && tid * R + 1 < Q) v1 = v0 + dt_l[tid * R + 1] * a2;
  const float tot = R > 1 ? v1 : v0;
  float incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  float pre = 0.f;
  for (int w = 0; w < wave; ++w) pre += part[w];
  const float excl = pre + incl - tot;
  if (tid * R < Q) s_l[tid * R] = excl + v0;
  if (R > 1 && tid * R + 1 < Q) s_l[tid * R + 1] = excl + v1;
  __syncthreads();
  // padded rows have dt = 0 and so weight 0
  const float s_end = s_l[Q - 1];
  for (int j = tid; j < Q; j += THREADS) {
    const float sj = s_l[j], dj = dt_l[j];
    w_l[j] = bwd ? __builtin_amdgcn_exp2f(fminf(sj, 0.f))
                 : __builtin_amdgcn_exp2f(fminf(s_end - sj, 0.f)) * dj;
    if (emit) {
      s_out[out_off + j] = sj;
      dt_out[out_off + j] = dj;
      u_out[out_off + j] = __builtin_amdgcn_exp2f(fminf(s_l[j | 31] - sj, 0.f)) * dj;
    }
  }
  return s_end;
}

// Direct loads of a chunk's dt column (rows past `len` read 0) into dt_l.
__device__ __forceinline__ void dma_dt(float *dt_l, const float *__restrict__ dt, size_t row0,
                                       int H, int hd, int Q, int len, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  for (int base = wave * 64; base < Q; base += nw * 64) {
    const int i = base + lane;
    const void *gp = i < len ? (const void *)(dt + (row0 + i) * H + hd) : (const void *)g_zero16;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gp,
                                     (__attribute__((address_space(3))) void *)(dt_l + base), 4,
                                     0, 0);
  }
}

template <typename T, int P, int N, int NH, bool BWD, bool PREC>
__global__ __launch_bounds__((StateCfg<T, P, N, NH>::THREADS)) void k_chunk_state(
    const T *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ B, ChunkMap cmap, int nc, int H, int G, int Q, int JP, int do_state,
    float *__restrict__ s_out, float *__restrict__ dt_out, float *__restrict__ u_out,
    float *__restrict__ S_out) {
  typedef StateCfg<T, P, N, NH> K;
  constexpr int NW = K::NW, TPW = K::TPW, NNT = K::NN / 16;
  const ChunkHead ch = xcd_chunk_head(H * K::NH);
  const int c = ch.c, hd = ch.h / K::NH, half = ch.h % K::NH;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  const int len = ci.z;
  if (len <= 0) return;
  const int g = (hd * G) / H;
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  constexpr bool SWZ = K::SWZ;
  extern __shared__ __align__(16) char smem[];
  T *Xs = reinterpret_cast<T *>(smem);  // padded: [JP][XP], [JP][BP]
  T *Bs = Xs + tile_slots(JP, K::XS) * K::VN;
  char *Xc = smem, *Bc = smem + (JP / 8) * kBlk128;  // swizzled: JP/8 and JP/B_RPB blocks
  float *dt_l = SWZ ? reinterpret_cast<float *>(Bc + (JP / K::B_RPB) * K::B_BLK)
                    : reinterpret_cast<float *>(Bs + tile_slots(JP, K::BS) * K::VN);  // [Q + 64]
  float *s_l = dt_l + Q + 64;                                                   // [Q]
  float *w_l = s_l + Q;                                                         // [Q]
  float *part = w_l + Q;                                                        // [16]

  const size_t xstride = (size_t)H * P, bstride = (size_t)G * N;
  const T *xs = x + (size_t)ci.y * xstride + (size_t)hd * P;
  const T *bs = B + (size_t)ci.y * bstride + (size_t)g * N + half * K::NN;

  // swizzled loads: byte strides and the lane's offset into a block's rows
  const uint32_t xsb = (uint32_t)(xstride * sizeof(T)), bsb = (uint32_t)(bstride * sizeof(T));
  const int lb8 = lane >> 3, lb4 = lane >> 4;
  const uint32_t lo8 = 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  // B: 128-byte half-rows as x; 256-byte rows 4 to a block, this wave's
  // blocks all of the parity of `wave` (NW is even)
  const uint32_t bl = K::B_RPB == 8 ? lb8 * bsb + lo8
                                    : lb4 * bsb + 16 * ((lane & 15) ^ (2 * (lb4 ^ (4 * (wave & 1)))));
  const uint32_t brow = 2 * K::NN;  // bytes of a B row in the tile

  // ---- one batch of direct loads: the dt column, first phase of x and B
  dma_dt(dt_l, dt, (size_t)ci.y, H, hd, Q, len, wave, NW);
  if (do_state) {
    if constexpr (SWZ) {
      const uint32_t v0 = (uint32_t)min(len, JP);
      dma_swz<kBlk128>(Xc, xs, v0 * xsb, lb8 * xsb + lo8, 8 * xsb, JP / 8, wave, NW);
      dma_swz<K::B_BLK>(Bc, bs, (v0 - 1) * bsb + brow, bl, K::B_RPB * bsb, JP / K::B_RPB, wave,
                        NW);
    } else {
      dma_tile<T, K::XS, K::XD>(Xs, xs, xstride, JP, len, wave, NW);
      dma_tile<T, K::BS, K::BD>(Bs, bs, bstride, JP, len, wave, NW);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  decay_scan<K::THREADS>(dt_l, s_l, w_l, part, Q, A[hd] * kLog2e, half == 0 && !BWD, BWD,
                         ((size_t)c * H + hd) * Q, s_out, dt_out, u_out);
  if (!do_state) return;
  __syncthreads();

  // ---- S^T[p][n] = sum_j (w_j x_j)[p] B[j][n]   (MFMA, k = tokens)
  f4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = zero4();
  for (int ph = 0; ph < len; ph += JP) {  // phases past the chunk length add nothing
    if (ph > 0) {
      __syncthreads();
      if constexpr (SWZ) {
        const uint32_t vr = (uint32_t)min(len - ph, JP);
        dma_swz<kBlk128>(Xc, xs + (size_t)ph * xstride, vr * xsb, lb8 * xsb + lo8, 8 * xsb,
                         JP / 8, wave, NW);
        dma_swz<K::B_BLK>(Bc, bs + (size_t)ph * bstride, (vr - 1) * bsb + brow, bl,
                          K::B_RPB * bsb, JP / K::B_RPB, wave, NW);
      } else {
        dma_tile<T, K::XS, K::XD>(Xs, xs + (size_t)ph * xstride, xstride, JP, len - ph, wave, NW);
        dma_tile<T, K::BS, K::BD>(Bs, bs + (size_t)ph * bstride, bstride, JP, len - ph, wave, NW);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if constexpr (!PREC) {
      if constexpr (SWZ)
        scale_rows_swz<T>(Xc, w_l, ph, min(JP, len - ph));
      else
        scale_rows<T, K::XP, K::XD>(Xs, w_l, ph, min(JP, len - ph));
      __syncthreads();
    }
    // swizzled transposed reads use the paired k map: rows k0 + 4 grp + col/4
    // and k0 + 16 + 4 grp + col/4 (any map works when both operands share it);
    // segment pt (or nt) by XOR with 32 pt (bits 5-6, or 5-7, of the offsets)
    //  x, and B half-rows: block k0/8 + grp/2 (+2), row 4 (grp&1) + col/4
    //  B rows of 256 bytes: block k0/4 + grp (+4), row col/4, parity grp&1
    const int c4 = col >> 2, cq = 8 * (col & 3);
    const int xb = 4 * (grp & 1) + c4;
    const int xo = (grp >> 1) * kBlk128 + xb * 128 + cq + 32 * swz8(xb);
    const int bo = K::B_RPB == 8 ? xo : grp * kBlk256T + c4 * 256 + cq + 32 * (c4 ^ (4 * (grp & 1)));
    constexpr int BHI = K::B_RPB == 8 ? 2 * kBlk128 : 4 * kBlk256T;  // +16 rows
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tile = wave + NW * t;
      if (tile < K::TILES) {
        const int pt = tile / NNT, nt = tile % NNT;
        for (int k0 = 0; k0 < JP; k0 += 32) {
          Frag<T> a, b;
          if constexpr (SWZ) {
            const char *xk = Xc + (k0 / 8) * kBlk128;
            const char *bk = Bc + (k0 / K::B_RPB) * K::B_BLK;
            a = frag_kmaj_at(xk, xo ^ (32 * pt), (xo ^ (32 * pt)) + 2 * kBlk128);
            b = frag_kmaj_at(bk, bo ^ (32 * nt), (bo ^ (32 * nt)) + BHI);
          } else {
            a = frag_kmaj(Xs, K::XP, pt * 16, k0 + 8 * grp, k0 + 8 * grp + 4);
            b = frag_kmaj(Bs, K::BP, nt * 16, k0 + 8 * grp, k0 + 8 * grp + 4);
          }
          if constexpr (PREC) {
            // w x in float32 from the unscaled tile, as two bfloat16 operands:
            // the rounded product and what the rounding dropped (rows past
            // the chunk take weight 0)
            const int ta = ph + k0 + (SWZ ? 4 * grp : 8 * grp);
            const int tb = ph + k0 + (SWZ ? 16 + 4 * grp : 8 * grp + 4);
            const f8v xv = cvt_f8(a.v);
            f8v xw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              xw[r] = ta + r < len ? xv[r] * w_l[ta + r] : 0.f;
              xw[4 + r] = tb + r < len ? xv[4 + r] * w_l[tb + r] : 0.f;
            }
            Frag<T> hi, lo;
            hi.v = cvt_bf8(xw);
            lo.v = cvt_bf8(xw - cvt_f8(hi.v));
            mma(acc[t], hi, b);
            mma(acc[t], lo, b);
          } else {
            mma(acc[t], a, b);
          }
        }
      }
    }
  }
  float *so = S_out + ((size_t)c * H + hd) * (size_t)(N * P);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + NW * t;
    if (tile < K::TILES) {
      const int pt = tile / NNT, nt = tile % NNT;
      const int n = half * K::NN + nt * 16 + col, p = pt * 16 + 4 * grp;
      st4(so + (size_t)n * P + p, acc[t]);
    }
  }
}

template <typename T, int P, int N, int NH>
static hipError_t run_state(const PrefillArgs &a, const WorkspaceLayout &L, int nc, int jp_cap,
                            bool state, bool bwd, hipStream_t st) {
  typedef StateCfg<T, P, N, NH> K;
  const int jp = K::jp(a.Q, jp_cap);
  const size_t lds = K::lds_bytes(jp, a.Q);
  if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
  const void *kern;
  if (bwd)
    kern = (const void *)k_chunk_state<T, P, N, NH, true, false>;
  else if (sizeof(T) == 2 && a.precise_states)
    kern = (const void *)k_chunk_state<T, P, N, NH, false, sizeof(T) == 2>;
  else
    kern = (const void *)k_chunk_state<T, P, N, NH, false, false>;
  hipError_t e = set_lds_limit(kern);
  if (e != hipSuccess) return e;
  char *ws = static_cast<char *>(a.workspace);
  const T *xp = (const T *)a.x, *bp = (const T *)a.B;
  const float *dtp = a.dt, *Ap = a.A;
  ChunkMap cm{reinterpret_cast<const int4 *>(ws + L.info), a.cu ? 0 : (int)(a.T / a.nseq), a.nseq,
              a.Q};
  int nc_ = nc, H_ = a.H, G_ = a.G, Q_ = a.Q, jp_ = jp, do_ = state ? 1 : 0;
  float *sp = reinterpret_cast<float *>(ws + L.s), *dp = reinterpret_cast<float *>(ws + L.dt);
  float *up = reinterpret_cast<float *>(ws + L.u), *Sp = reinterpret_cast<float *>(ws + L.S);
  void *args[] = {&xp, &dtp, &Ap, &bp, &cm, &nc_, &H_, &G_, &Q_, &jp_, &do_, &sp, &dp, &up, &Sp};
  return hipLaunchKernel(kern, dim3(xcd_grid(nc, a.H * K::NH)), dim3(K::THREADS), args, lds, st);
}

// Shape of the launch.  Few (chunk, head) units: split the n columns over two
// workgroups and stage up to 128 rows, so the whole grid is resident at once.
// Many units: one workgroup per unit and 64-row phases -- small LDS lets four
// workgroups share a CU, so some are always loading while others compute.
template <typename T, int P, int N>
static hipError_t run_state_auto(const PrefillArgs &a, const WorkspaceLayout &L, int nc,
                                 bool state, bool bwd, hipStream_t st) {
  const bool few = (long)nc * a.H < 2048;
  if constexpr (N >= 64) {
    if (few) return run_state<T, P, N, 2>(a, L, nc, 128, state, bwd, st);
  }
  return run_state<T, P, N, 1>(a, L, nc, few ? 128 : 64, state, bwd, st);
}

template <typename T, int P>
static hipError_t state_N(const PrefillArgs &a, const WorkspaceLayout &L, int nc, bool s, bool b,
                          hipStream_t st) {
  switch (a.N) {
    case 16: return run_state_auto<T, P, 16>(a, L, nc, s, b, st);
    case 32: return run_state_auto<T, P, 32>(a, L, nc, s, b, st);
    case 64: return run_state_auto<T, P, 64>(a, L, nc, s, b, st);
    case 128: return run_state_auto<T, P, 128>(a, L, nc, s, b, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t state_P(const PrefillArgs &a, const WorkspaceLayout &L, int nc, bool s, bool b,
                          hipStream_t st) {
  switch (a.P) {
    case 16: return state_N<T, 16>(a, L, nc, s, b, st);
    case 32: return state_N<T, 32>(a, L, nc, s, b, st);
    case 64: return state_N<T, 64>(a, L, nc, s, b, st);
    case 128: return state_N<T, 128>(a, L, nc, s, b, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state(const PrefillArgs &a, const WorkspaceLayout &L, int nc, bool state,
                              hipStream_t st, bool bwd) {
  return a.bf16 ? state_P<bf16>(a, L, nc, state, bwd, st)
                : state_P<float>(a, L, nc, state, bwd, st);
}

}  // namespace ssd
