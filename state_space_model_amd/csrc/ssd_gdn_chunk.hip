// ssd_gdn_chunk.hip -- the gated delta rule in chunks of 64 tokens, on MFMA.
//
// The rule, per sequence and head (q, k read group floor(h*G/H)), state S [V][K]:
//   a_t = exp(g_t);  S_t = a_t S_{t-1} + beta_t (v_t - a_t S_{t-1} k_t) k_t^T;  o_t = S_t q_t
// (the delta-rule family of Recurrence Scan, poot docs).  The page gives only
// the streaming schedule; the chunked form below is this recurrence regrouped
// exactly, the same way the structured-state-space-duality form regroups the
// SSD recurrence (Compiler-First State Space Duality ..., Abstract).
//
// Within a chunk of C tokens with entering state S_0, let G_t = sum_{i<=t} g_i
// (chunk-local) and gamma_t = exp(G_t).  Writing d_t = beta_t (v_t - a_t
// S_{t-1} k_t), the state is S_t = gamma_t S_0 + sum_{j<=t} exp(G_t - G_j)
// d_j k_j^T, and the rows d_t^T of D solve the unit lower-triangular system
//   (I + A) D = diag(beta) Vc - diag(beta gamma) Kc S_0^T,
//   A_tj = beta_t exp(G_t - G_j) (k_t . k_j)  for j < t,
// so D = U - W S_0^T with U = (I + A)^-1 diag(beta) Vc and W = (I + A)^-1
// diag(beta gamma) Kc, which do not depend on the state.  Then
//   O     = diag(gamma) Qc S_0^T + P D,   P_tj = exp(G_t - G_j) (q_t . k_j), j <= t
//   S_C   = gamma_C S_0 + (diag(exp(G_C - G_j)) D)^T Kc
//
// Two launches:
//   k_gdn_prep   one workgroup per (chunk, head), all chunks at once: K K^T
//                and Q K^T on MFMA, A and P, forward substitution of
//                (I + A) X = [diag(beta) Vc | diag(beta gamma) Kc] in float32
//                (a thread per column, the column in registers), U, W, P to
//                the workspace, indexed by token.
//   k_gdn_walk   one workgroup per (sequence, head, 16 state rows v): walks
//                the chunks with the state block in MFMA accumulators; per
//                chunk D = U - W S_0^T, O, and the state update are three
//                MFMA products.  The next chunk's U, W, P, q, k, g are
//                staged into a second LDS buffer while the current chunk is
//                computed.  For bfloat16 operands the state and D enter the
//                products as a bfloat16 pair hi + lo (x = hi + lo to 16 bits
//                of mantissa), so only U, W, P carry one bfloat16 rounding.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

constexpr int kGc = 64;   // tokens per chunk
constexpr int kGvb = 16;  // state rows v per walking workgroup

__device__ __forceinline__ void split_pair(float x, bf16 &hi, bf16 &lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// Direct loads of a strided float column (one value per row, rows >= len
// read 0) into 64 consecutive LDS floats.
__device__ __forceinline__ void dma_col64(float *dst, const float *__restrict__ src, size_t stride,
                                          int len, int wave) {
  if (wave != 0) return;
  const int lane = threadIdx.x & 63;
  const void *gp = lane < len ? (const void *)(src + (size_t)lane * stride) : (const void *)g_zero16;
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gp,
                                   (__attribute__((address_space(3))) void *)dst, 4, 0, 0);
}

// Inclusive prefix sum of 64 floats held one per lane of a wave.
__device__ __forceinline__ float wave_scan64(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// ------------------------------------------------------------------ prep
template <typename T, int K> struct GdnPrepCfg {
  static constexpr int VN = 16 / (int)sizeof(T);
  static constexpr int KP = K + VN;     // q/k row pitch (elements)
  static constexpr int AP = kGc + 4;    // A row pitch (floats)
  static constexpr size_t LDS = (size_t)2 * kGc * KP * sizeof(T) + (size_t)kGc * AP * 4 + 2 * kGc * 4;
};

template <typename T, int K>
__global__ __launch_bounds__(256) void k_gdn_prep(const T *__restrict__ q, const T *__restrict__ k,
                                                  const T *__restrict__ v,
                                                  const float *__restrict__ g,
                                                  const float *__restrict__ beta, ChunkMap cmap,
                                                  int nc, int H, int G, int V, T *__restrict__ U,
                                                  T *__restrict__ W, T *__restrict__ Pm) {
  typedef GdnPrepCfg<T, K> F;
  constexpr int KP = F::KP, AP = F::AP, VN = F::VN;
  extern __shared__ __align__(16) char smem[];
  T *Ks = reinterpret_cast<T *>(smem);  // [64][KP]
  T *Qs = Ks + kGc * KP;                // [64][KP]
  float *As = reinterpret_cast<float *>(Qs + kGc * KP);  // [64][AP]  A transposed
  float *gl = As + kGc * AP;                             // [64] cumulative log2 gate
  float *bl = gl + kGc;                                  // [64] beta

  const int c = blockIdx.x, hd = blockIdx.y;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  const int len = ci.z;
  if (len <= 0) return;
  const int t0 = ci.y, gr = (int)(((long)hd * G) / H);
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  dma_tile<T, KP / VN, K / VN>(Ks, k + ((size_t)t0 * G + gr) * K, (size_t)G * K, kGc, len, wave, 4);
  dma_tile<T, KP / VN, K / VN>(Qs, q + ((size_t)t0 * G + gr) * K, (size_t)G * K, kGc, len, wave, 4);
  if (tid < kGc) {
    const bool ok = tid < len;
    gl[tid] = ok ? fminf(g[(size_t)(t0 + tid) * H + hd], 0.f) * kLog2e : 0.f;
    bl[tid] = ok ? beta[(size_t)(t0 + tid) * H + hd] : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (wave == 0) {
    const float s = wave_scan64(gl[lane]);
    gl[lane] = s;
  }
  __syncthreads();

  // K K^T (lower tiles, 10) -> A;  Q K^T (all 16 tiles) -> P (zero above the diagonal)
  for (int tt = wave; tt < 26; tt += 4) {
    const bool isq = tt >= 10;
    int ti, tj;
    if (isq) {
      ti = (tt - 10) >> 2;
      tj = (tt - 10) & 3;
    } else {
      int idx = tt;
      ti = 0;
      while (idx > ti) {
        idx -= ti + 1;
        ++ti;
      }
      tj = idx;
    }
    f4 acc = zero4();
    const T *Ar = isq ? Qs : Ks;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const Frag<T> a = frag_rowk(Ar, KP, ti * 16 + col, k0 + 8 * grp);
      const Frag<T> b = frag_rowk(Ks, KP, tj * 16 + col, k0 + 8 * grp);
      mma(acc, a, b);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ti * 16 + 4 * grp + r, j = tj * 16 + col;
      const float e = __builtin_amdgcn_exp2f(fminf(gl[t] - gl[j], 0.f));
      if (!isq) {
        As[j * AP + t] = j < t ? bl[t] * e * acc[r] : 0.f;  // transposed: column j of A
      } else if (t < len) {
        Pm[((size_t)(t0 + t) * H + hd) * kGc + j] = from_f32<T>(j <= t ? e * acc[r] : 0.f);
      }
    }
  }
  __syncthreads();

  // (I + A) X = R by forward substitution, one column of R per thread:
  // columns [0, V) are beta_t v_t, columns [V, V + K) are beta_t gamma_t k_t
  if (tid < V + K) {
    float x[kGc];
#pragma unroll
    for (int t = 0; t < kGc; ++t) {
      float r = 0.f;
      if (t < len) {
        r = tid < V ? bl[t] * to_f32(v[((size_t)(t0 + t) * H + hd) * V + tid])
                    : bl[t] * __builtin_amdgcn_exp2f(fminf(gl[t], 0.f)) * to_f32(Ks[t * KP + tid - V]);
      }
      x[t] = r;
    }
    // column by column: once x_j is final, remove its share from every later
    // row (column j of A is row j of the transposed tile)
#pragma unroll
    for (int j = 0; j < kGc - 1; ++j) {
      const float xj = x[j];
#pragma unroll
      for (int t = (j + 1) & ~3; t < kGc; t += 4) {
        const f4 a = ld4(As + j * AP + t);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (t + u > j) x[t + u] -= a[u] * xj;
      }
      // every later row is updated now: without this the compiler defers the
      // updates to each row's last use and keeps all of A in registers
#pragma unroll
      for (int t = j + 1; t < kGc; ++t) asm volatile("" : "+v"(x[t]));
    }
#pragma unroll
    for (int t = 0; t < kGc; ++t) {
      if (t < len) {
        const size_t row = (size_t)(t0 + t) * H + hd;
        if (tid < V) U[row * V + tid] = from_f32<T>(x[t]);
        else W[row * K + tid - V] = from_f32<T>(x[t]);
      }
    }
  }
}

// ------------------------------------------------------------------ walk
template <typename T, int K> struct GdnWalkCfg {
  static constexpr int VN = 16 / (int)sizeof(T);
  static constexpr bool SPL = sizeof(T) == 2;    // bfloat16: hi + lo pairs
  static constexpr int NBUF = SPL ? 2 : 1;       // staged chunks in LDS
  static constexpr int KP = K + VN;              // W, q, k row pitch
  static constexpr int UP = kGvb + VN;           // U rows (16 columns)
  static constexpr int PP = kGc + VN;            // P rows
  static constexpr int DP = kGvb + VN;           // D [j][v] pitch
  static constexpr int SP = K + VN;              // S_0 [v][k] pitch
  // one staged chunk: W, q, k [64][KP], U [64][UP], P [64][PP] (T), g [64] (float)
  static constexpr int W_OFF = 0;
  static constexpr int Q_OFF = W_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int K_OFF = Q_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int U_OFF = K_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int P_OFF = U_OFF + kGc * UP * (int)sizeof(T);
  static constexpr int G_OFF = P_OFF + kGc * PP * (int)sizeof(T);
  static constexpr int BUF = G_OFF + kGc * 4;
  // then S_0 (hi, lo), D (hi, lo), D~ (hi, lo), gamma and the D~ row scale
  static constexpr int NS = SPL ? 2 : 1;
  static constexpr int S_OFF = NBUF * BUF;
  static constexpr int D_OFF = S_OFF + NS * kGvb * SP * (int)sizeof(T);
  static constexpr int E_OFF = D_OFF + 2 * NS * kGc * DP * (int)sizeof(T);
  static constexpr int LDS = E_OFF + 2 * kGc * 4;
  static_assert(BUF % 16 == 0 && S_OFF % 16 == 0 && D_OFF % 16 == 0 && E_OFF % 16 == 0, "align");
};

template <typename T, int K>
__global__ __launch_bounds__(256) void k_gdn_walk(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ g,
    const T *__restrict__ U, const T *__restrict__ W, const T *__restrict__ Pm, const float *h0,
    float *__restrict__ o, float *h_out, const int32_t *__restrict__ cu, int L_dense, int nseq,
    int H, int G, int V) {
  typedef GdnWalkCfg<T, K> F;
  constexpr int VN = F::VN, KP = F::KP, UP = F::UP, PP = F::PP, DP = F::DP, SP = F::SP;
  constexpr bool SPL = F::SPL;
  constexpr int KT = K / 16;        // 16-column k tiles of the state
  constexpr int KTW = KT / 4;       // per wave
  static_assert(KT % 4 == 0, "K must be a multiple of 64");

  // XCD-aware order: the v-blocks of one head share an XCD (its L2 holds the
  // chunk's U, W, P, q, k for all of them)
  const int nvb = V / kGvb;
  const int L = blockIdx.x, per = 8 * nvb;
  const int hb = L / per, rem = L - hb * per;
  const int vb = rem >> 3, hs = hb * 8 + (rem & 7);  // hs = s * H + h
  if (hs >= nseq * H) return;
  const int s = hs / H, hd = hs - s * H;
  const int gr = (int)(((long)hd * G) / H);
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int t0, t1;
  if (cu) {
    t0 = cu[s];
    t1 = cu[s + 1];
  } else {
    t0 = s * L_dense;
    t1 = t0 + L_dense;
  }

  extern __shared__ __align__(16) char smem[];
  T *Ss = reinterpret_cast<T *>(smem + F::S_OFF);                // [NS][16][SP]
  T *Ds = reinterpret_cast<T *>(smem + F::D_OFF);                // [NS][64][DP]
  T *Dt = Ds + F::NS * kGc * DP;                                 // [NS][64][DP]  scaled rows
  float *gam = reinterpret_cast<float *>(smem + F::E_OFF);       // [64]
  float *dsc = gam + kGc;                                        // [64]

  auto stage = [&](int b, int tb) {
    char *buf = smem + b * F::BUF;
    const int len = min(kGc, t1 - tb);
    dma_tile<T, KP / VN, K / VN>(reinterpret_cast<T *>(buf + F::W_OFF),
                                 W + ((size_t)tb * H + hd) * K, (size_t)H * K, kGc, len, wave, 4);
    dma_tile<T, KP / VN, K / VN>(reinterpret_cast<T *>(buf + F::Q_OFF),
                                 q + ((size_t)tb * G + gr) * K, (size_t)G * K, kGc, len, wave, 4);
    dma_tile<T, KP / VN, K / VN>(reinterpret_cast<T *>(buf + F::K_OFF),
                                 k + ((size_t)tb * G + gr) * K, (size_t)G * K, kGc, len, wave, 4);
    dma_tile<T, UP / VN, kGvb / VN>(reinterpret_cast<T *>(buf + F::U_OFF),
                                    U + ((size_t)tb * H + hd) * V + vb * kGvb, (size_t)H * V, kGc,
                                    len, wave, 4);
    dma_tile<T, PP / VN, kGc / VN>(reinterpret_cast<T *>(buf + F::P_OFF),
                                   Pm + ((size_t)tb * H + hd) * kGc, (size_t)H * kGc, kGc, len, wave,
                                   4);
    dma_col64(reinterpret_cast<float *>(buf + F::G_OFF), g + (size_t)tb * H + hd, (size_t)H, len,
              wave);
  };

  // the state block: rows v = vb*16 + 4*grp + r, columns k = kt*16 + col
  f4 st[KTW];
  const size_t sofs = ((size_t)hs * V + vb * kGvb) * K;
#pragma unroll
  for (int u = 0; u < KTW; ++u) {
    const int kc = (wave * KTW + u) * 16 + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) st[u][r] = h0 ? h0[sofs + (size_t)(4 * grp + r) * K + kc] : 0.f;
  }

  if (t0 < t1) stage(0, t0);
  int cur = 0;
  for (int tb = t0; tb < t1; tb += kGc) {
    const int len = min(kGc, t1 - tb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // chunk tb staged; the previous chunk's buffer is free
    if (F::NBUF == 2 && tb + kGc < t1) stage(cur ^ 1, tb + kGc);
    const char *buf = smem + cur * F::BUF;
    const T *Ws = reinterpret_cast<const T *>(buf + F::W_OFF);
    const T *Qs = reinterpret_cast<const T *>(buf + F::Q_OFF);
    const T *Ks = reinterpret_cast<const T *>(buf + F::K_OFF);
    const T *Us = reinterpret_cast<const T *>(buf + F::U_OFF);
    const T *Ps = reinterpret_cast<const T *>(buf + F::P_OFF);
    const float *gs = reinterpret_cast<const float *>(buf + F::G_OFF);

    // gamma_t = 2^(G_t), row scale 2^(G_C - G_j); the state block to LDS
    if (wave == 0) {
      const float Gt = wave_scan64(fminf(gs[lane], 0.f) * kLog2e);
      const float GC = __shfl(Gt, 63, 64);  // rows past the chunk add 0
      gam[lane] = __builtin_amdgcn_exp2f(fminf(Gt, 0.f));
      dsc[lane] = __builtin_amdgcn_exp2f(fminf(GC - Gt, 0.f));
    }
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
      const int kc = (wave * KTW + u) * 16 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vr = 4 * grp + r;
        if constexpr (SPL) {
          bf16 hi, lo;
          split_pair(st[u][r], hi, lo);
          Ss[vr * SP + kc] = hi;
          Ss[kGvb * SP + vr * SP + kc] = lo;
        } else {
          Ss[vr * SP + kc] = from_f32<T>(st[u][r]);
        }
      }
    }
    __syncthreads();

    // D = U - W S_0^T and Qc S_0^T for rows t of this wave's tile, 16 columns v
    f4 ws = zero4(), qs = zero4();
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const Frag<T> a = frag_rowk(Ws, KP, wave * 16 + col, k0 + 8 * grp);
      const Frag<T> aq = frag_rowk(Qs, KP, wave * 16 + col, k0 + 8 * grp);
      const Frag<T> b = frag_rowk(Ss, SP, col, k0 + 8 * grp);
      mma(ws, a, b);
      mma(qs, aq, b);
      if constexpr (SPL) {
        const Frag<T> bl = frag_rowk(Ss + kGvb * SP, SP, col, k0 + 8 * grp);
        mma(ws, a, bl);
        mma(qs, aq, bl);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = wave * 16 + 4 * grp + r;
      const float d = to_f32(Us[t * UP + col]) - ws[r];
      const float dt = d * dsc[t];
      qs[r] *= gam[t];
      if constexpr (SPL) {
        bf16 hi, lo;
        split_pair(d, hi, lo);
        Ds[t * DP + col] = hi;
        Ds[kGc * DP + t * DP + col] = lo;
        split_pair(dt, hi, lo);
        Dt[t * DP + col] = hi;
        Dt[kGc * DP + t * DP + col] = lo;
      } else {
        Ds[t * DP + col] = from_f32<T>(d);
        Dt[t * DP + col] = from_f32<T>(dt);
      }
    }
    __syncthreads();

    // O = diag(gamma) Qc S_0^T + P D   (k = j)
#pragma unroll
    for (int j0 = 0; j0 < kGc; j0 += 32) {
      const Frag<T> a = frag_rowk(Ps, PP, wave * 16 + col, j0 + 8 * grp);
      const Frag<T> b = frag_kmaj(Ds, DP, 0, j0 + 8 * grp, j0 + 8 * grp + 4);
      mma(qs, a, b);
      if constexpr (SPL) {
        const Frag<T> bl = frag_kmaj(Ds + kGc * DP, DP, 0, j0 + 8 * grp, j0 + 8 * grp + 4);
        mma(qs, a, bl);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = wave * 16 + 4 * grp + r;
      if (t < len) o[((size_t)(tb + t) * H + hd) * V + vb * kGvb + col] = qs[r];
    }
    // S <- gamma_C S_0 + D~^T Kc   (k = j)
    const float gC = gam[kGc - 1];  // rows past the chunk add 0 to G
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st[u][r] *= gC;
      const int kt = wave * KTW + u;
#pragma unroll
      for (int j0 = 0; j0 < kGc; j0 += 32) {
        const Frag<T> a = frag_kmaj(Dt, DP, 0, j0 + 8 * grp, j0 + 8 * grp + 4);
        const Frag<T> b = frag_kmaj(Ks, KP, kt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
        mma(st[u], a, b);
        if constexpr (SPL) {
          const Frag<T> al = frag_kmaj(Dt + kGc * DP, DP, 0, j0 + 8 * grp, j0 + 8 * grp + 4);
          mma(st[u], al, b);
        }
      }
    }
    if (F::NBUF == 1 && tb + kGc < t1) {
      __syncthreads();  // every read of the one buffer is done
      stage(0, tb + kGc);
    }
    cur ^= F::NBUF - 1;
  }
  if (h_out) {
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
      const int kc = (wave * KTW + u) * 16 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) h_out[sofs + (size_t)(4 * grp + r) * K + kc] = st[u][r];
    }
  }
}

// ------------------------------------------------------------------ launch
bool gdn_chunk_supported(int K, int V) {
  return (K == 64 || K == 128) && V % kGvb == 0 && V + K <= 256;
}

GdnLayout gdn_chunk_layout(int64_t T, int nseq, int H, int K, int V, int elem) {
  GdnLayout Lw{};
  const int64_t nc = (T + (int64_t)nseq * (kGc - 1)) / kGc;
  Lw.nc_max = nc;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  Lw.info = off;
  off = up(off + 16 * (size_t)(nc > 0 ? nc : 1));
  Lw.seq_off = off;
  off = up(off + 4 * (size_t)(nseq + 1));
  Lw.U = off;
  off = up(off + (size_t)elem * T * H * V);
  Lw.W = off;
  off = up(off + (size_t)elem * T * H * K);
  Lw.P = off;
  off = up(off + (size_t)elem * T * H * kGc);
  Lw.total = off;
  return Lw;
}

template <typename T, int K>
static hipError_t gdn_chunk_run(const GdnArgs &a) {
  const GdnLayout Lw = gdn_chunk_layout(a.T, a.nseq, a.H, K, a.V, sizeof(T));
  char *ws = static_cast<char *>(a.workspace);
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  int4 *info = reinterpret_cast<int4 *>(ws + Lw.info);
  int *seq_off = reinterpret_cast<int *>(ws + Lw.seq_off);
  T *Up = reinterpret_cast<T *>(ws + Lw.U), *Wp = reinterpret_cast<T *>(ws + Lw.W);
  T *Pp = reinterpret_cast<T *>(ws + Lw.P);
  const int nc = (int)Lw.nc_max;
  const int L_dense = a.cu ? 0 : (int)(a.T / a.nseq);
  if (nc > 0) {
    if (a.cu) {
      hipError_t e = launch_chunk_map(a.cu, a.nseq, a.T, kGc, nc, info, seq_off, st);
      if (e != hipSuccess) return e;
    }
    typedef GdnPrepCfg<T, K> FP;
    const void *kp = (const void *)k_gdn_prep<T, K>;
    hipError_t e = set_lds_limit(kp);
    if (e != hipSuccess) return e;
    const T *qp = (const T *)a.q, *kkp = (const T *)a.k, *vp = (const T *)a.v;
    const float *gp = a.g, *bp = a.beta;
    ChunkMap cm{info, L_dense, a.nseq, kGc};
    int nc_ = nc, H_ = a.H, G_ = a.G, V_ = a.V;
    void *args[] = {&qp, &kkp, &vp, &gp, &bp, &cm, &nc_, &H_, &G_, &V_, &Up, &Wp, &Pp};
    e = hipLaunchKernel(kp, dim3(nc, a.H), dim3(256), args, FP::LDS, st);
    if (e != hipSuccess) return e;
  }
  typedef GdnWalkCfg<T, K> FW;
  const void *kw = (const void *)k_gdn_walk<T, K>;
  hipError_t e = set_lds_limit(kw);
  if (e != hipSuccess) return e;
  const T *qp = (const T *)a.q, *kkp = (const T *)a.k;
  const float *gp = a.g, *h0p = a.h0;
  const T *Uc = Up, *Wc = Wp, *Pc = Pp;
  float *op = a.o, *hop = a.h_out;
  const int32_t *cup = a.cu;
  int Ld = L_dense, ns = a.nseq, H_ = a.H, G_ = a.G, V_ = a.V;
  void *args[] = {&qp, &kkp, &gp, &Uc, &Wc, &Pc, &h0p, &op, &hop, &cup, &Ld, &ns, &H_, &G_, &V_};
  const int heads = a.nseq * a.H;
  const unsigned grid = (unsigned)((heads + 7) / 8) * 8u * (unsigned)(a.V / kGvb);
  return hipLaunchKernel(kw, dim3(grid), dim3(256), args, FW::LDS, st);
}

hipError_t launch_gdn_chunked(const GdnArgs &a) {
  if (!gdn_chunk_supported(a.K, a.V)) return hipErrorInvalidValue;
  if (a.bf16) return a.K == 64 ? gdn_chunk_run<bf16, 64>(a) : gdn_chunk_run<bf16, 128>(a);
  return a.K == 64 ? gdn_chunk_run<float, 64>(a) : gdn_chunk_run<float, 128>(a);
}

}  // namespace ssd
