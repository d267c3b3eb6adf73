// ssd_gdn.hip -- gated delta rule scan on gfx950: the delta-rule family of
// Recurrence Scan (poot docs, "One equation, one packed result": a per-head
// matrix state rewritten by every token), as the streaming kernel of its "The
// schedule": a workgroup per (sequence, head, block of state rows), the state
// held on chip for the whole sequence, a runtime loop over tokens, and each
// row's dot products split over several lanes that add their partial sums
// every token.
//
// Per sequence and head h (q, k read group g = floor(h*G/H)), state S [V][K]:
//   a_t = exp(g_t);  u = S_{t-1} k_t;  S_t = a_t S_{t-1} + beta_t (v_t - a_t u) k_t^T
//   o_t = S_t q_t
//
// Lanes: 16 consecutive lanes own one state row i (value index) and 1/16 of
// its K columns each, in registers; a 256-thread workgroup owns 16 rows.  Per
// token a lane does K/16 multiply-adds for S k, four xor-shuffle steps sum the
// row (DPP moves inside a 16-lane row), K/16 for the update and K/16 plus four
// steps for S q; the next token's operands are read from LDS meanwhile.  q, k, v, the gate
// and beta of the next TB tokens are fetched into registers while the current
// TB are computed from LDS; o goes out through LDS a block at a time.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int kGdnSplit = 16;                      // lanes per state row
constexpr int kGdnRows = 256 / kGdnSplit;          // rows per workgroup

// Sum over the 16 lanes of a DPP row, left in every lane: xor 1 and xor 2
// inside each quad (quad_perm [1,0,3,2], [2,3,0,1]), then lane i with 7 - i
// (row_half_mirror: quad 0 with 1, quad 2 with 3) and lane i with 15 - i
// (row_mirror: the two halves).  Four VALU ops, no LDS round trip.
__device__ __forceinline__ float gdn_row_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

template <typename T, int K>
__global__ __launch_bounds__(256) void k_gdn(const T *__restrict__ q, const T *__restrict__ k,
                                             const T *__restrict__ v,
                                             const float *__restrict__ g,
                                             const float *__restrict__ beta, const float *h0,
                                             float *__restrict__ o, float *h_out,
                                             const int32_t *__restrict__ cu, int L_dense,
                                             int T_all, int H, int G, int V) {
  constexpr int KE = K / kGdnSplit;               // columns per lane (a multiple of 4)
  static_assert(KE % 4 == 0, "K must be a multiple of 64");
  constexpr int RB = kGdnRows;
  constexpr int TB = K <= 128 ? 32 : 16;          // tokens per staged block
  constexpr int VN = 16 / (int)sizeof(T);
  constexpr int QCH = TB * K / VN;                // 16-byte pieces of q (and of k) per block
  constexpr int QPT = (QCH + 255) / 256;          // per thread
  constexpr int VPT = (TB * RB + 255) / 256;      // v values per thread per block
  typedef typename Vec16<T>::type Vv;

  __shared__ __align__(16) float qs[TB][K];
  __shared__ __align__(16) float ks[TB][K];
  __shared__ float vs[TB][RB];
  __shared__ float as_[TB], bs_[TB];
  __shared__ float os[TB][RB];

  const int s = blockIdx.z, hd = blockIdx.y, rb = blockIdx.x;
  const int gr = (int)(((long)hd * G) / H);
  const int tid = threadIdx.x, part = tid % kGdnSplit, r = tid / kGdnSplit;
  const int i = rb * RB + r;  // this lane's state row
  int t0, t1;
  if (cu) {  // kept inside 0 .. T_all whatever the array holds
    t0 = min(max(cu[s], 0), T_all);
    t1 = min(max(cu[s + 1], t0), T_all);
  } else {
    t0 = s * L_dense;
    t1 = t0 + L_dense;
  }

  float S[KE];
  const size_t srow = (((size_t)s * H + hd) * V + i) * K + part * KE;
#pragma unroll
  for (int e = 0; e < KE; e += 4) {
    const f4 h = h0 ? ld4(h0 + srow + e) : zero4();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) S[e + q4] = h[q4];
  }

  // ---- prefetch of one block of tokens into registers
  Vv qr[QPT], kr[QPT];
  float vr[VPT], ar = 0.f, br = 0.f;
  auto fetch = [&](int tb) {
#pragma unroll
    for (int c = 0; c < QPT; ++c) {
      const int ch = tid + 256 * c, tt = ch / (K / VN), col = (ch % (K / VN)) * VN;
      const bool ok = ch < QCH && tb + tt < t1;
      const size_t off = ((size_t)(tb + tt) * G + gr) * K + col;
      qr[c] = ok ? *reinterpret_cast<const Vv *>(q + off) : vzero<Vv>();
      kr[c] = ok ? *reinterpret_cast<const Vv *>(k + off) : vzero<Vv>();
    }
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
      const int e = tid + 256 * c, tt = e / RB, rr = e % RB;
      vr[c] = (e < TB * RB && tb + tt < t1)
                  ? to_f32(v[((size_t)(tb + tt) * H + hd) * V + rb * RB + rr])
                  : 0.f;
    }
    if (tid < TB && tb + tid < t1) {
      ar = __builtin_amdgcn_exp2f(fminf(g[(size_t)(tb + tid) * H + hd], 0.f) * 1.4426950408889634f);
      br = beta[(size_t)(tb + tid) * H + hd];
    } else {
      ar = 1.f;
      br = 0.f;
    }
  };
  // ---- registers -> LDS (float32)
  auto commit = [&]() {
#pragma unroll
    for (int c = 0; c < QPT; ++c) {
      const int ch = tid + 256 * c, tt = ch / (K / VN), col = (ch % (K / VN)) * VN;
      if (ch < QCH) {
        if constexpr (VN == 8) {
          const f8v qf = cvt_f8(qr[c]), kf = cvt_f8(kr[c]);
          st4(&qs[tt][col], f4{qf[0], qf[1], qf[2], qf[3]});
          st4(&qs[tt][col + 4], f4{qf[4], qf[5], qf[6], qf[7]});
          st4(&ks[tt][col], f4{kf[0], kf[1], kf[2], kf[3]});
          st4(&ks[tt][col + 4], f4{kf[4], kf[5], kf[6], kf[7]});
        } else {
          st4(&qs[tt][col], qr[c]);
          st4(&ks[tt][col], kr[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
      const int e = tid + 256 * c;
      if (e < TB * RB) vs[e / RB][e % RB] = vr[c];
    }
    if (tid < TB) {
      as_[tid] = ar;
      bs_[tid] = br;
    }
  };

  fetch(t0);
  for (int tb = t0; tb < t1; tb += TB) {
    commit();
    __syncthreads();
    if (tb + TB < t1) fetch(tb + TB);  // lands while this block is computed
    const int nt = min(TB, t1 - tb);
    // token tt's operands are read from LDS while token tt-1 is computed
    float kv[KE], qv[KE], vv, av, bv;
    auto operands = [&](int tt, float (&kk)[KE], float (&qq)[KE], float &v_, float &a_, float &b_) {
#pragma unroll
      for (int e = 0; e < KE; e += 4) {
        const f4 k4 = ld4(&ks[tt][part * KE + e]), q4 = ld4(&qs[tt][part * KE + e]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          kk[e + x] = k4[x];
          qq[e + x] = q4[x];
        }
      }
      v_ = vs[tt][r];
      a_ = as_[tt];
      b_ = bs_[tt];
    };
    operands(0, kv, qv, vv, av, bv);
    // u = S k for the block's first token; afterwards each token's pass over
    // the updated S forms S q (its output) and S k of the next token together,
    // so the two row sums run side by side
    float u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int e = 0; e < KE; e += 2) {
      u0 += S[e] * kv[e];
      u1 += S[e + 1] * kv[e + 1];
    }
    float u = gdn_row_sum(u0 + u1);
#pragma unroll 2
    for (int tt = 0; tt < nt; ++tt) {
      float kn[KE], qn[KE], vn, an, bn;
      operands(min(tt + 1, TB - 1), kn, qn, vn, an, bn);
      const float c = bv * (vv - av * u);
      float p0 = 0.f, p1 = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
      for (int e = 0; e < KE; e += 2) {
        S[e] = av * S[e] + c * kv[e];
        S[e + 1] = av * S[e + 1] + c * kv[e + 1];
        p0 += S[e] * qv[e];
        p1 += S[e + 1] * qv[e + 1];
        n0 += S[e] * kn[e];
        n1 += S[e + 1] * kn[e + 1];
      }
      const float ov = gdn_row_sum(p0 + p1);
      u = gdn_row_sum(n0 + n1);  // S k of token tt+1 (unused after the last)
      os[tt][r] = ov;  // the row's 16 lanes hold the same sum: no branch
#pragma unroll
      for (int e = 0; e < KE; ++e) {
        kv[e] = kn[e];
        qv[e] = qn[e];
      }
      vv = vn;
      av = an;
      bv = bn;
    }
    __syncthreads();
    for (int e = tid; e < nt * RB; e += 256) {
      const int tt = e / RB, rr = e % RB;
      o[((size_t)(tb + tt) * H + hd) * V + rb * RB + rr] = os[tt][rr];
    }
  }
  if (h_out) {
#pragma unroll
    for (int e = 0; e < KE; e += 4) st4(h_out + srow + e, f4{S[e], S[e + 1], S[e + 2], S[e + 3]});
  }
}

template <typename T>
static hipError_t gdn_K(const GdnArgs &a) {
  dim3 grid(a.V / kGdnRows, a.H, a.nseq);
  const int L_dense = a.cu ? 0 : (int)(a.T / a.nseq);
#define SSD_GDN(KK)                                                                            \
  case KK:                                                                                     \
    hipLaunchKernelGGL((k_gdn<T, KK>), grid, dim3(256), 0, static_cast<hipStream_t>(a.stream), \
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta, a.h0, a.o,  \
                       a.h_out, a.cu, L_dense, (int)a.T, a.H, a.G, a.V);                       \
    break;
  switch (a.K) {
    SSD_GDN(64) SSD_GDN(128) SSD_GDN(256)
    default: return hipErrorInvalidValue;
  }
#undef SSD_GDN
  return hipGetLastError();
}

hipError_t launch_gated_delta_rule(const GdnArgs &a) {
  if (a.nseq == 0) return hipSuccess;
  return a.bf16 ? gdn_K<bf16>(a) : gdn_K<float>(a);
}

}  // namespace ssd
