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
//   k_gdn_walk   one workgroup per (sequence, head, block of state rows v): walks
//                the chunks with the state block in MFMA accumulators; per
//                chunk D = U - W S_0^T, O, and the state update are three
//                MFMA products.  With bfloat16 operands the next chunk's U, W,
//                P, q, k, gamma are loaded into registers while the current
//                chunk is computed, and written to LDS at the chunk boundary.  For bfloat16 operands the state and D enter the
//                products as a bfloat16 pair hi + lo (x = hi + lo to 16 bits
//                of mantissa), so only U, W, P carry one bfloat16 rounding.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

constexpr int kGc = 64;   // tokens per chunk

__device__ __forceinline__ void split_pair(float x, bf16 &hi, bf16 &lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
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
                                                  T *__restrict__ W, T *__restrict__ Pm,
                                                  float *__restrict__ E) {
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
    // per token: gamma_t = 2^(G_t) and the write scale 2^(G_C - G_t) of the walk
    const float GC = __shfl(s, 63, 64);  // rows past the chunk add 0
    if (lane < len) {
      float *e = E + ((size_t)(t0 + lane) * H + hd) * 2;
      e[0] = __builtin_amdgcn_exp2f(fminf(s, 0.f));
      e[1] = __builtin_amdgcn_exp2f(fminf(GC - s, 0.f));
    }
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
    // no branch per row: every load is issued before the first is used
    // (rows past the chunk read the last row and are zeroed by beta = 0)
    float x[kGc];
    if (tid < V) {
#pragma unroll
      for (int t = 0; t < kGc; ++t) {
        const int tr = min(t, len - 1);
        x[t] = bl[t] * to_f32(v[((size_t)(t0 + tr) * H + hd) * V + tid]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kGc; ++t)
        x[t] = bl[t] * __builtin_amdgcn_exp2f(fminf(gl[t], 0.f)) * to_f32(Ks[t * KP + tid - V]);
    }
    // column by column: once x_j is final, remove its share from every later
    // row (column j of A is row j of the transposed tile)
    // column j + 1 of A is read while step j runs (the LDS latency would
    // otherwise stand between every two steps of the chain)
    f4 acur[kGc / 4], anext[kGc / 4];
#pragma unroll
    for (int q4 = 0; q4 < kGc / 4; ++q4) acur[q4] = ld4(As + q4 * 4);
#pragma unroll
    for (int j = 0; j < kGc - 1; ++j) {
      if (j + 1 < kGc - 1) {
#pragma unroll
        for (int q4 = (j + 2) / 4; q4 < kGc / 4; ++q4) anext[q4] = ld4(As + (j + 1) * AP + q4 * 4);
      }
      const float xj = x[j];
#pragma unroll
      for (int q4 = (j + 1) / 4; q4 < kGc / 4; ++q4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (q4 * 4 + u > j) x[q4 * 4 + u] -= acur[q4][u] * xj;
      }
      // every later row is updated now: without this the compiler defers the
      // updates to each row's last use and keeps all of A in registers
#pragma unroll
      for (int t = j + 1; t < kGc; ++t) asm volatile("" : "+v"(x[t]));
#pragma unroll
      for (int q4 = (j + 2) / 4; q4 < kGc / 4; ++q4) acur[q4] = anext[q4];
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
// VB state rows per workgroup, VB/4 waves: wave w owns output tile (rows
// t = 16 (w % 4) .., columns v = 16 (w / 4) ..) of D and O, and K/64 tiles of
// the state block (rows v of the same 16, columns k = 16 ((w % 4) K/64 + u)).
template <typename T, int K, int VB> struct GdnWalkCfg {
  static constexpr int VN = 16 / (int)sizeof(T);
  static constexpr bool SPL = sizeof(T) == 2;    // bfloat16: hi + lo pairs, register prefetch
  static constexpr int NW = VB / 4;              // waves
  static constexpr int NT = 64 * NW;             // threads
  static constexpr int KP = K + VN;              // W, q, k row pitch
  static constexpr int UP = VB + VN;             // U rows
  static constexpr int PP = kGc + VN;            // P rows
  static constexpr int DP = VB + VN;             // D [j][v] pitch
  static constexpr int SP = K + VN;              // S_0 [v][k] pitch
  // one staged chunk: W, q, k [64][KP], U [64][UP], P [64][PP] (T), gamma, scale [64] (float)
  static constexpr int W_OFF = 0;
  static constexpr int Q_OFF = W_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int K_OFF = Q_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int U_OFF = K_OFF + kGc * KP * (int)sizeof(T);
  static constexpr int P_OFF = U_OFF + kGc * UP * (int)sizeof(T);
  static constexpr int G_OFF = P_OFF + kGc * PP * (int)sizeof(T);
  static constexpr int BUF = G_OFF + 2 * kGc * 4;
  // then S_0 (hi, lo), D (hi, lo), D~ (hi, lo)
  static constexpr int NS = SPL ? 2 : 1;
  static constexpr int S_OFF = BUF;
  static constexpr int D_OFF = S_OFF + NS * VB * SP * (int)sizeof(T);
  static constexpr int LDS = D_OFF + 2 * NS * kGc * DP * (int)sizeof(T);
  // 16-byte pieces of one chunk's W, q, k, U, P and of the whole, per thread
  static constexpr int PW = kGc * K / VN, PU = kGc * VB / VN, PPn = kGc * kGc / VN;
  static constexpr int PIECES = 3 * PW + PU + PPn;
  static constexpr int PPT = (PIECES + NT - 1) / NT;
  static_assert(BUF % 16 == 0 && S_OFF % 16 == 0 && D_OFF % 16 == 0, "align");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <typename T, int K, int VB>
__global__ __launch_bounds__(VB * 16) void k_gdn_walk(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ E,
    const T *__restrict__ U, const T *__restrict__ W, const T *__restrict__ Pm, const float *h0,
    float *__restrict__ o, float *h_out, const int32_t *__restrict__ cu, int L_dense, int T_all,
    int nseq, int H, int G, int V) {
  typedef GdnWalkCfg<T, K, VB> F;
  constexpr int VN = F::VN, KP = F::KP, UP = F::UP, PP = F::PP, DP = F::DP, SP = F::SP;
  constexpr bool SPL = F::SPL;
  constexpr int KTW = K / 64;       // state tiles per wave
  typedef typename Vec16<T>::type Vv;

  // XCD-aware order: the v-blocks of one head share an XCD (its L2 holds the
  // chunk's W, P, q, k for all of them)
  const int nvb = V / VB;
  const int L = blockIdx.x, per = 8 * nvb;
  const int hb = L / per, rem = L - hb * per;
  const int vb = rem >> 3, hs = hb * 8 + (rem & 7);  // hs = s * H + h
  if (hs >= nseq * H) return;
  const int s = hs / H, hd = hs - s * H;
  const int gr = (int)(((long)hd * G) / H);
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tt = wave & 3, vt = wave >> 2;  // this wave's t tile and v tile
  int t0, t1;
  if (cu) {  // kept inside 0 .. T_all whatever the array holds
    t0 = min(max(cu[s], 0), T_all);
    t1 = min(max(cu[s + 1], t0), T_all);
  } else {
    t0 = s * L_dense;
    t1 = t0 + L_dense;
  }

  extern __shared__ __align__(16) char smem[];
  T *Ws = reinterpret_cast<T *>(smem + F::W_OFF);
  T *Qs = reinterpret_cast<T *>(smem + F::Q_OFF);
  T *Ks = reinterpret_cast<T *>(smem + F::K_OFF);
  T *Us = reinterpret_cast<T *>(smem + F::U_OFF);
  T *Ps = reinterpret_cast<T *>(smem + F::P_OFF);
  float *gam = reinterpret_cast<float *>(smem + F::G_OFF);  // gamma_t (0 past the chunk)
  float *dsc = gam + kGc;                                    // 2^(G_C - G_t)
  T *Ss = reinterpret_cast<T *>(smem + F::S_OFF);            // [NS][VB][SP]
  T *Ds = reinterpret_cast<T *>(smem + F::D_OFF);            // [NS][64][DP]
  T *Dt = Ds + F::NS * kGc * DP;                             // [NS][64][DP]  scaled rows

  // piece p of a chunk -> (source row pointer, row, 16-byte vector, LDS tile)
  auto piece = [&](int p, int tb, const T *&src, T *&dst) {
    int r, v;
    if (p < 3 * F::PW) {
      const int m = p / F::PW, e = p - m * F::PW;
      r = e / (K / VN);
      v = e - r * (K / VN);
      const T *base = m == 0 ? W + ((size_t)tb * H + hd) * K
                      : (m == 1 ? q : k) + ((size_t)tb * G + gr) * K;
      const size_t stride = m == 0 ? (size_t)H * K : (size_t)G * K;
      src = base + r * stride + v * VN;
      dst = (m == 0 ? Ws : m == 1 ? Qs : Ks) + r * KP + v * VN;
    } else if (p < 3 * F::PW + F::PU) {
      const int e = p - 3 * F::PW;
      r = e / (VB / VN);
      v = e - r * (VB / VN);
      src = U + ((size_t)(tb + r) * H + hd) * V + vb * VB + v * VN;
      dst = Us + r * UP + v * VN;
    } else {
      const int e = p - 3 * F::PW - F::PU;
      r = e / (kGc / VN);
      v = e - r * (kGc / VN);
      src = Pm + ((size_t)(tb + r) * H + hd) * kGc + v * VN;
      dst = Ps + r * PP + v * VN;
    }
    return r;
  };
  Vv pre[F::PPT];
  float2 epre = make_float2(0.f, 0.f);
  auto fetch = [&](int tb) {  // the chunk at tb -> registers
    const int len = min(kGc, t1 - tb);
#pragma unroll
    for (int c = 0; c < F::PPT; ++c) {
      const int p = tid + c * F::NT;
      pre[c] = vzero<Vv>();
      if (p < F::PIECES) {
        const T *src;
        T *dst;
        const int r = piece(p, tb, src, dst);
        if (r < len) pre[c] = *reinterpret_cast<const Vv *>(src);
      }
    }
    if (tid < kGc)
      epre = tid < len ? *reinterpret_cast<const float2 *>(E + ((size_t)(tb + tid) * H + hd) * 2)
                       : make_float2(0.f, 0.f);
  };
  auto commit = [&](int tb) {  // registers -> LDS
#pragma unroll
    for (int c = 0; c < F::PPT; ++c) {
      const int p = tid + c * F::NT;
      if (p < F::PIECES) {
        const T *src;
        T *dst;
        piece(p, tb, src, dst);
        *reinterpret_cast<Vv *>(dst) = pre[c];
      }
    }
    if (tid < kGc) {
      gam[tid] = epre.x;
      dsc[tid] = epre.y;
    }
  };

  // the state block: rows v = vb*VB + 16 vt + 4 grp + r, columns k = (4 (tt) KTW + u) 16 + col
  f4 st[KTW];
  const size_t sofs = ((size_t)hs * V + vb * VB + vt * 16) * K;
#pragma unroll
  for (int u = 0; u < KTW; ++u) {
    const int kc = (tt * KTW + u) * 16 + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) st[u][r] = h0 ? h0[sofs + (size_t)(4 * grp + r) * K + kc] : 0.f;
  }

  if (t0 < t1) fetch(t0);
  for (int tb = t0; tb < t1; tb += kGc) {
    const int len = min(kGc, t1 - tb);
    __syncthreads();  // every read of the previous chunk's tiles is done
    commit(tb);
    if (tb + kGc < t1) fetch(tb + kGc);  // lands while this chunk is computed

    // the state block to LDS
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
      const int kc = (tt * KTW + u) * 16 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vr = vt * 16 + 4 * grp + r;
        if constexpr (SPL) {
          bf16 hi, lo;
          split_pair(st[u][r], hi, lo);
          Ss[vr * SP + kc] = hi;
          Ss[VB * SP + vr * SP + kc] = lo;
        } else {
          Ss[vr * SP + kc] = from_f32<T>(st[u][r]);
        }
      }
    }
    __syncthreads();

    // D = U - W S_0^T and Qc S_0^T for this wave's tile
    f4 ws = zero4(), qs = zero4();
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const Frag<T> a = frag_rowk(Ws, KP, tt * 16 + col, k0 + 8 * grp);
      const Frag<T> aq = frag_rowk(Qs, KP, tt * 16 + col, k0 + 8 * grp);
      const Frag<T> b = frag_rowk(Ss, SP, vt * 16 + col, k0 + 8 * grp);
      mma(ws, a, b);
      mma(qs, aq, b);
      if constexpr (SPL) {
        const Frag<T> bl = frag_rowk(Ss + VB * SP, SP, vt * 16 + col, k0 + 8 * grp);
        mma(ws, a, bl);
        mma(qs, aq, bl);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tt * 16 + 4 * grp + r, vc = vt * 16 + col;
      const float d = to_f32(Us[t * UP + vc]) - ws[r];
      const float dt = d * dsc[t];
      qs[r] *= gam[t];
      if constexpr (SPL) {
        bf16 hi, lo;
        split_pair(d, hi, lo);
        Ds[t * DP + vc] = hi;
        Ds[kGc * DP + t * DP + vc] = lo;
        split_pair(dt, hi, lo);
        Dt[t * DP + vc] = hi;
        Dt[kGc * DP + t * DP + vc] = lo;
      } else {
        Ds[t * DP + vc] = from_f32<T>(d);
        Dt[t * DP + vc] = from_f32<T>(dt);
      }
    }
    __syncthreads();

    // O = diag(gamma) Qc S_0^T + P D   (k = j)
#pragma unroll
    for (int j0 = 0; j0 < kGc; j0 += 32) {
      const Frag<T> a = frag_rowk(Ps, PP, tt * 16 + col, j0 + 8 * grp);
      const Frag<T> b = frag_kmaj(Ds, DP, vt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
      mma(qs, a, b);
      if constexpr (SPL) {
        const Frag<T> bl = frag_kmaj(Ds + kGc * DP, DP, vt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
        mma(qs, a, bl);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tt * 16 + 4 * grp + r;
      if (t < len) o[((size_t)(tb + t) * H + hd) * V + vb * VB + vt * 16 + col] = qs[r];
    }
    // S <- gamma_C S_0 + D~^T Kc   (k = j)
    const float gC = gam[len - 1];
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st[u][r] *= gC;
      const int kt = tt * KTW + u;
#pragma unroll
      for (int j0 = 0; j0 < kGc; j0 += 32) {
        const Frag<T> a = frag_kmaj(Dt, DP, vt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
        const Frag<T> b = frag_kmaj(Ks, KP, kt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
        mma(st[u], a, b);
        if constexpr (SPL) {
          const Frag<T> al = frag_kmaj(Dt + kGc * DP, DP, vt * 16, j0 + 8 * grp, j0 + 8 * grp + 4);
          mma(st[u], al, b);
        }
      }
    }
  }
  if (h_out) {
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
      const int kc = (tt * KTW + u) * 16 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) h_out[sofs + (size_t)(4 * grp + r) * K + kc] = st[u][r];
    }
  }
}

// ------------------------------------------------------------------ launch
bool gdn_chunk_supported(int K, int V) {
  return (K == 64 || K == 128) && V % 32 == 0 && V + K <= 256;
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
  Lw.E = off;
  off = up(off + (size_t)8 * T * H);
  Lw.total = off;
  return Lw;
}

template <typename T, int K, int VB>
static hipError_t gdn_walk_launch(const GdnArgs &a, int L_dense, const float *Ec, const T *Uc,
                                  const T *Wc, const T *Pc, hipStream_t st) {
  typedef GdnWalkCfg<T, K, VB> FW;
  const void *kw = (const void *)k_gdn_walk<T, K, VB>;
  hipError_t e = set_lds_limit(kw);
  if (e != hipSuccess) return e;
  const T *qp = (const T *)a.q, *kkp = (const T *)a.k;
  const float *h0p = a.h0;
  float *op = a.o, *hop = a.h_out;
  const int32_t *cup = a.cu;
  int Ld = L_dense, Ta = (int)a.T, ns = a.nseq, H_ = a.H, G_ = a.G, V_ = a.V;
  void *args[] = {&qp, &kkp, &Ec, &Uc, &Wc, &Pc, &h0p, &op, &hop, &cup, &Ld, &Ta, &ns, &H_, &G_, &V_};
  const int heads = a.nseq * a.H;
  const unsigned grid = (unsigned)((heads + 7) / 8) * 8u * (unsigned)(a.V / VB);
  return hipLaunchKernel(kw, dim3(grid), dim3(FW::NT), args, FW::LDS, st);
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
  float *Ep = reinterpret_cast<float *>(ws + Lw.E);
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
    void *args[] = {&qp, &kkp, &vp, &gp, &bp, &cm, &nc_, &H_, &G_, &V_, &Up, &Wp, &Pp, &Ep};
    e = hipLaunchKernel(kp, dim3(nc, a.H), dim3(256), args, FP::LDS, st);
    if (e != hipSuccess) return e;
  }
  // bfloat16: 32 state rows per workgroup (64 halve the re-reads of each
  // chunk's W, P, q, k but leave three quarters of the CUs idle at 32 heads:
  // 329 against 260 us); float32: 16 (its tiles fill the LDS)
  if constexpr (sizeof(T) == 2) {
    return gdn_walk_launch<T, K, 32>(a, L_dense, Ep, Up, Wp, Pp, st);
  } else {
    return gdn_walk_launch<T, K, 16>(a, L_dense, Ep, Up, Wp, Pp, st);
  }
}

hipError_t launch_gdn_chunked(const GdnArgs &a) {
  if (!gdn_chunk_supported(a.K, a.V)) return hipErrorInvalidValue;
  if (a.bf16) return a.K == 64 ? gdn_chunk_run<bf16, 64>(a) : gdn_chunk_run<bf16, 128>(a);
  return a.K == 64 ? gdn_chunk_run<float, 64>(a) : gdn_chunk_run<float, 128>(a);
}

}  // namespace ssd
