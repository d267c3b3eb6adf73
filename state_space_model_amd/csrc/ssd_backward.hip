// ssd_backward.hip -- gradients of the chunked SSD prefill on gfx950: the
// backward half of a training step (Compiler-First State Space Duality and
// Portable O(1) Autoregressive Caching for Inference, Table 13 times forward
// plus backward passes of the same chunked scan).
//
// For a loss L with dL/dy = dy and dL/dh_out = dh_out, per sequence, head h
// and chunk c (s chunk-local, G_t = dL/dh_t the adjoint state):
//   G_t      = sum_{t'>=t in c} e^(s_t' - s_t) C_t' dy_t'^T + e^(s_end - s_t) dH_c
//   dH_c     = dL/d(state leaving chunk c), carried backward over the chunks:
//              dH_{c-1} = e^(s_end) dH_c + Sb_c,  Sb_c = sum_t e^(s_t) C_t dy_t^T,
//              dH_last = dh_out, dh0 = dH_{first - 1}
//   dX_t     = B_t^T G_t = sum_{t'>=t} e^(s_t' - s_t) (B_t . C_t') dy_t'
//                          + e^(s_end - s_t) dH_c^T B_t
//   dx_t     = D dy_t + dt_t dX_t
//   dB_t     = dt_t G_t x_t = dt_t [sum_{t'>=t} e^(s_t' - s_t) (x_t . dy_t') C_t'
//                                  + e^(s_end - s_t) dH_c x_t]
//   dC_t     = h_t dy_t = sum_{j<=t} e^(s_t - s_j) dt_j (dy_t . x_j) B_j + e^(s_t) H_in dy_t
//   dz_i     = dL/d(dt_i A) = sum_{t>=i in c} ds_t + <dH_c, H_c>      (H_c: state leaving c)
//   ds_t     = r_t + sum_j W[t][j] - sum_j W[j][t] - v_t
//   W[t][j]  = e^(s_t - s_j) dt_j (C_t . B_j)(dy_t . x_j)  (j <= t)
//   r_t      = C_t . (e^(s_t) H_in dy_t),   v_t = dt_t x_t . (e^(s_end - s_t) dH_c^T B_t)
//   ddt_i    = A dz_i + q_i  (q_t = x_t . dX_t),   dA = sum_i dt_i dz_i,   dD = sum_t dy_t . x_t
// dz_i collects every path through the decay e^(dt_i A): the products W of
// pairs j < i <= t inside the chunk (as a suffix sum of row minus column sums),
// the state entering the chunk (r), and the chunk's end state.  W comes from
// float32 accumulators of exact products, so the cancellation between its row
// and column sums costs float32 rounding only; forms through y or q, whose
// operands are rounded to bfloat16 for the MFMA, would carry that rounding
// through the same cancellation.  For the same reason the DX scan's state
// term, from which v comes, takes dH_c as two bfloat16 operands, its rounded
// value and what the rounding dropped: with dH_c rounded once, v alone moved
// dA by about 1 % of its size on the 130M layer.
//
// Launches, all on the caller's stream:
//   forward recompute   chunk states, state pass (H_in per chunk, final state)
//   k_chunk_state<BWD>  Sb_c on MFMA (the forward chunk-state kernel on C, dy)
//   k_state_pass_bwd    dH_c per chunk, <dH_c, H_c> partials, dh0
//   k_bwd_scan<DX>      dx, q, W row/column sums, v, dy . x (reverse-time masked scan)
//   k_bwd_scan<DB>      dB per head                        (reverse-time masked scan)
//   k_bwd_scan<DC>      dC per head, r                     (forward-time masked scan)
//   k_bwd_ddt           dz by a suffix scan, ddt, per-chunk dA and dD
//   k_bwd_sums          dA, dD summed over the chunks; dB, dC over the partial
//                       rows of a group (only when heads are not all summed on chip)
// The three masked scans are one kernel: a wave owns 16 output rows i and
// sweeps 32-row source blocks j (j >= i reverse, j <= i forward):
//   M^T[j][i] = (K_j . Q_i) 2^(|s_i - s_j|) w_j, masked      k = KD  (MFMA)
//   out^T[v][i] += V^T[v][j] M^T[j][i]                        k = j   (MFMA)
//   out^T[v][i] += scale_i (state . Q_i)[v]                   k = KD  (MFMA)
// with (Q, K, V, state) = (B, C, dy, dH_c) for DX, (x, dy, C, dH_c) for DB and
// (dy, x, B, H_in) for DC.  Sums over heads and chunks are fixed-order: every
// result is deterministic.
#include <stdlib.h>

#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

enum { kBwdDX = 0, kBwdDB = 1, kBwdDC = 2 };

// Per-row terms of dz, each [chunk][head][Q] float32 (rs: one row per part of
// the DX scan's split).
struct BwdRows {
  float *q;    // x_t . dX_t
  float *cv;   // W column sum of t + v_t
  float *r;    // C_t . (2^(s_t) H_in dy_t)
  float *dyx;  // dy_t . x_t
  float *rs;   // W row sum of t, [chunk][head][part][Q]
};

template <typename T, int MODE, int KD, int VD> struct BwdScanCfg {
  static constexpr bool REV = MODE != kBwdDC;
  static constexpr bool ST_ROWS = MODE != kBwdDX;  // state [VD][KD], read along rows
  static constexpr int NK = KD < 32 ? 32 : KD;     // contraction padded to the k-step
  static constexpr int KS = NK / 32;
  static constexpr int VN = 16 / (int)sizeof(T);
  static constexpr int KP = NK + row_pad<T>();  // K rows: fragments read along a row
  static constexpr int VP = VD + kTrPad;        // V rows: transpose reads
  static constexpr int SR = ST_ROWS ? VD : NK;  // state tile rows
  static constexpr int SP = ST_ROWS ? KP : VP;  // state tile pitch
  static constexpr int SD = (ST_ROWS ? KD : VD) / VN;
  static constexpr int SS = SP / VN, KSL = KP / VN, VSL = VP / VN, KDS = KD / VN, VDS = VD / VN;
  // bf16 with P = 64, N = 128: block-swizzled tiles -- the state [N][P] in
  // 128-byte rows; K and V rows of 64 (128 bytes) or 128 (256 bytes) values
  static constexpr bool SWZ = sizeof(T) == 2 && (MODE == kBwdDX ? (KD == 128 && VD == 64)
                                                                : (KD == 64 && VD == 128));
  static constexpr size_t s_bytes() { return SWZ ? 16 * kBlk128 : tile_slots(SR, SS) * 16; }
  // DX in bf16 also stages what the bf16 state dropped (same layout)
  static constexpr bool LO = MODE == kBwdDX && sizeof(T) == 2;
  static constexpr size_t lo_bytes() { return LO ? s_bytes() : 0; }
  static constexpr size_t k_bytes(int jp) {
    return SWZ ? (KD == 128 ? (size_t)(jp / 4) * kBlk256 : (size_t)(jp / 8) * kBlk128)
               : (size_t)tile_slots(jp, KSL) * 16;
  }
  static constexpr size_t v_bytes(int jp) {
    return SWZ ? (VD == 64 ? (size_t)(jp / 8) * kBlk128 : (size_t)(jp / 4) * kBlk256T)
               : (size_t)tile_slots(jp, VSL) * 16;
  }
  // + s, dt, u rows; DX also keeps one row of W row sums per wave
  static constexpr size_t lds_bytes(int jp, int q, int nw) {
    return s_bytes() + lo_bytes() + k_bytes(jp) + v_bytes(jp) + 12 * (size_t)q +
           (MODE == kBwdDX ? 4 * (size_t)nw * q : 0);
  }
  // rows per phase: up to 64 in blocks of at most 512 threads (under 61 KB),
  // up to 256 otherwise, halved until the LDS fits
  static int jp(int q, int threads) {
    const int lim = threads <= 512 ? 64 : 256;
    int j = q < lim ? q : lim;
    const size_t cap = threads <= 512 ? 61 * 1024 : 160 * 1024;
    while (j > 32 && lds_bytes(j, q, threads / 64) > cap) j /= 2;
    return j;
  }
};

// One workgroup per (chunk, block of hb heads of one group, part of SPLIT);
// one wave per 16-row output tile, tiles dealt to the parts and waves as in
// the forward chunk scan so that the waves of a SIMD carry equal work.  DB and
// DC sum the hb heads in their accumulators (DB takes dt_i into its own-row
// operand, so no per-head factor is left), which leaves H / hb partial rows
// per token for the group sum instead of H; DX has hb = 1.  MAXT bounds the
// workgroup (512 up to Q = 256, which leaves 256 VGPRs a lane; 1024 for
// Q = 512).
template <typename T, int MODE, int P, int N, int SPLIT, int MAXT, bool MULTI>
__global__ __launch_bounds__(MAXT) void k_bwd_scan(
    const T *__restrict__ x, const T *__restrict__ dy, const T *__restrict__ B,
    const T *__restrict__ C, const float *__restrict__ D, const float *__restrict__ s_ws,
    const float *__restrict__ dt_ws, const float *__restrict__ u_ws,
    const T *__restrict__ state, const T *__restrict__ state_lo, ChunkMap cmap, int nc, int H,
    int G, int Q, int JP, int hb, float *__restrict__ out, int ostride, BwdRows rows) {
  constexpr int KD = MODE == kBwdDX ? N : P;
  constexpr int VD = MODE == kBwdDX ? P : N;
  typedef BwdScanCfg<T, MODE, KD, VD> K;
  constexpr bool REV = K::REV;
  constexpr int KS = K::KS, NVT = VD / 16;
  constexpr int KSP = (P < 32 ? 32 : P) / 32;  // k-steps of the dy . x products (DX)
  if (!MULTI) hb = 1;
  const ChunkHead chd = xcd_chunk_head((H / hb) * SPLIT);
  const int c = chd.c, blk = chd.h / SPLIT, part = chd.h % SPLIT;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  if (ci.z <= 0) return;
  const int len = ci.z;
  const int hd0 = blk * hb, g = (hd0 * G) / H;  // the block's heads share group g
  const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, col = lane & 15;
  int tile = wave;
  if (SPLIT == 2) {
    const int k = wave < nw / 2 ? wave : 3 * nw / 2 - 1 - wave;
    tile = 2 * k + (part ^ (k & 1));
  }
  const int t0 = 16 * tile;
  const int i = t0 + col;
  const bool live = t0 < len;  // wave-uniform
  const int tile_last = min(t0 + 15, len - 1);

  constexpr bool SWZ = K::SWZ;
  extern __shared__ __align__(16) char smem[];
  char *Sc = smem, *Slo = Sc + K::s_bytes(), *Kc = Slo + K::lo_bytes(),
       *Vc = Kc + K::k_bytes(JP);
  T *Ss = reinterpret_cast<T *>(Sc);  // padded: state [SR][SP]
  T *Ks = reinterpret_cast<T *>(Kc);  //         K rows [JP][KP]
  T *Vs = reinterpret_cast<T *>(Vc);  //         V rows [JP][VP]
  float *s_l = reinterpret_cast<float *>(Vc + K::v_bytes(JP));  // [Q]
  float *dt_l = s_l + Q;                                                        // [Q]
  float *u_l = dt_l + Q;                                                        // [Q]
  float *rs_l = u_l + Q;  // DX: [nw][Q] W row sums, one row per wave

  const size_t hstride = (size_t)H * P, gstride = (size_t)G * N;
  // swizzled tiles: the lane's offsets into a block's rows (x / dy rows of
  // 128 bytes, B / C rows of 256 bytes; the 256-byte V rows keep the block
  // parity of `wave`, nw being even) and into the rows it reads
  const uint32_t hsb = (uint32_t)(hstride * 2), gsb = (uint32_t)(gstride * 2);
  const int lb8 = lane >> 3, lb4 = lane >> 4;
  const uint32_t lo8 = 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  const uint32_t sl = lb8 * (P * 2) + lo8;
  const uint32_t kl = KD == 128 ? lb4 * gsb + 16 * ((lane & 15) ^ lb4) : lb8 * hsb + lo8;
  const uint32_t vl = VD == 64 ? lb8 * hsb + lo8
                               : lb4 * gsb + 16 * ((lane & 15) ^ (2 * (lb4 ^ (4 * (wave & 1)))));
  const uint32_t ksb = KD == 128 ? gsb : hsb, vsb = VD == 64 ? hsb : gsb;
  const int c4 = col >> 2, cq = 8 * (col & 3);
  //  transposed, natural k map (state, DX): rows 32 kk + 8 grp + col/4 (+4)
  const int so_lo = grp * kBlk128 + c4 * 128 + cq + 32 * swz8(c4);
  const int so_hi = grp * kBlk128 + (4 + c4) * 128 + cq + 32 * swz8(4 + c4);
  //  row reads of 128-byte rows r0 + col: block r0/8 + col/8, vector 4 kk + grp
  const int r128 = (col >> 3) * kBlk128 + (col & 7) * 128 + 16 * (grp ^ (2 * swz8(col & 7)));
  //  row reads of 256-byte rows jl + col: block jl/4 + col/4, vector 4 kk + grp
  const int r256 = c4 * kBlk256 + (col & 3) * 256 + 16 * (grp ^ (col & 3));
  //  transposed, paired k map (V): rows jl + 4 grp + col/4 (+16)
  const int xb = 4 * (grp & 1) + c4;
  const int v128 = (grp >> 1) * kBlk128 + xb * 128 + cq + 32 * swz8(xb);
  const int v256 = grp * kBlk256T + c4 * 256 + cq + 32 * (c4 ^ (4 * (grp & 1)));
  auto load_k = [&](const T *src, int rows) {
    if constexpr (KD == 128)
      dma_swz<kBlk256>(Kc, src, rows * ksb, kl, 4 * ksb, JP / 4, wave, nw);
    else
      dma_swz<kBlk128>(Kc, src, rows * ksb, kl, 8 * ksb, JP / 8, wave, nw);
  };
  auto load_v = [&](const T *src, int rows) {
    if constexpr (VD == 64)
      dma_swz<kBlk128>(Vc, src, rows * vsb, vl, 8 * vsb, JP / 8, wave, nw);
    else
      dma_swz<kBlk256T>(Vc, src, rows * vsb, vl, 4 * vsb, JP / 4, wave, nw);
  };
  const T *Bg = B + (size_t)ci.y * gstride + (size_t)g * N;
  const T *Cg = C + (size_t)ci.y * gstride + (size_t)g * N;
  f4 acc[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) acc[vt] = zero4();
  float sp = 0.f, csum = 0.f, dti = 0.f;  // DX: v_i / dt_i and W column-sum partials

  const int nheads = MULTI ? hb : 1;  // one head: no loop
  for (int hh = 0; hh < nheads; ++hh) {
    const int hd = hd0 + hh;
    const size_t csh = (size_t)c * H + hd;
    const T *xh = x + (size_t)ci.y * hstride + (size_t)hd * P;
    const T *dyh = dy + (size_t)ci.y * hstride + (size_t)hd * P;
    const T *qg = MODE == kBwdDX ? Bg : (MODE == kBwdDB ? xh : dyh);
    const T *kg = MODE == kBwdDX ? Cg : (MODE == kBwdDB ? dyh : xh);
    const T *vg = MODE == kBwdDX ? dyh : (MODE == kBwdDB ? Cg : Bg);
    const size_t qs = MODE == kBwdDX ? gstride : hstride;
    const size_t ks_ = MODE == kBwdDX ? gstride : hstride;
    const size_t vs = MODE == kBwdDX ? hstride : gstride;
    if (hh > 0) __syncthreads();  // the previous head's tiles are no longer read

    // ---- prologue: the state tile and the first phase of K/V rows in flight together
    if constexpr (SWZ) {
      const int v0 = min(len, JP);
      dma_swz<kBlk128>(Sc, state + csh * (size_t)(N * P), N * P * 2, sl, 1024, N * P * 2 / 1024,
                       wave, nw);
      if constexpr (K::LO)
        dma_swz<kBlk128>(Slo, state_lo + csh * (size_t)(N * P), N * P * 2, sl, 1024,
                         N * P * 2 / 1024, wave, nw);
      load_k(kg, v0);
      load_v(vg, v0);
    } else {
      dma_tile<T, K::SS, K::SD>(Ss, state + csh * (size_t)(N * P), (size_t)P, K::SR,
                                K::ST_ROWS ? VD : KD, wave, nw);
      if constexpr (K::LO)
        dma_tile<T, K::SS, K::SD>(reinterpret_cast<T *>(Slo), state_lo + csh * (size_t)(N * P),
                                  (size_t)P, K::SR, KD, wave, nw);
      dma_tile<T, K::KSL, K::KDS>(Ks, kg, ks_, JP, len, wave, nw);
      dma_tile<T, K::VSL, K::VDS>(Vs, vg, vs, JP, len, wave, nw);
    }
    dti = dt_ws[csh * Q + i];
    Frag<T> qf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k8 = kk * 32 + 8 * grp;
      qf[kk] = (i < len && k8 < KD) ? frag_global(qg + (size_t)i * qs + k8) : frag_zero<T>();
      if constexpr (MULTI && MODE == kBwdDB) qf[kk] = frag_scale(qf[kk], dti);  // dt_i x_i
    }
    Frag<T> xf[KSP];  // DX: the tile's own x rows, for dy_t . x_i
    if constexpr (MODE == kBwdDX) {
#pragma unroll
      for (int kk = 0; kk < KSP; ++kk) {
        const int k8 = kk * 32 + 8 * grp;
        xf[kk] = (i < len && k8 < P) ? frag_global(xh + (size_t)i * hstride + k8)
                                     : frag_zero<T>();
      }
      for (int j = threadIdx.x; j < nw * Q; j += blockDim.x) rs_l[j] = 0.f;
    }
    const float si = s_ws[csh * Q + i];
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
      const float sv = s_ws[csh * Q + j];
      s_l[j] = sv;
      dt_l[j] = dt_ws[csh * Q + j];
      if (REV) {  // u_j = 2^(s_j - s_(jb-1)), jb the first row of j's 32-row block
        const int jb = j & ~31;
        const float sprev = jb > 0 ? s_ws[csh * Q + jb - 1] : 0.f;
        u_l[j] = __builtin_amdgcn_exp2f(fminf(sv - sprev, 0.f));
      } else {  // u_j = 2^(s_r - s_j) dt_j, r the last row of j's block
        u_l[j] = u_ws[csh * Q + j];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- the state term: out^T += scale_i (state . Q_i)
    if (live) {
      const float sc = MODE == kBwdDC ? __builtin_amdgcn_exp2f(fminf(si, 0.f))
                                      : __builtin_amdgcn_exp2f(fminf(s_l[Q - 1] - si, 0.f));
      // one 16x16 tile at a time (a single temporary), with the lane partials of
      // the state-path terms: DX v_i / dt_i = x_i . st_i, DC r_i = C_i . st_i
      // (summed over the lane groups below)
      float part_sp = 0.f;
      const T *row = MODE == kBwdDX ? xh + (size_t)i * hstride : Cg + (size_t)i * gstride;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        // one head: straight into the (zero) accumulator; several: a temporary
        f4 st = MULTI ? zero4() : acc[vt];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          Frag<T> a;
          if constexpr (SWZ && K::ST_ROWS)
            a = frag_rowk_at(Sc + 2 * vt * kBlk128, r128 ^ (64 * kk));
          else if constexpr (SWZ)
            a = frag_kmaj_at(Sc + kk * 4 * kBlk128, so_lo ^ (32 * vt), so_hi ^ (32 * vt));
          else if constexpr (K::ST_ROWS)
            a = frag_rowk(Ss, K::SP, vt * 16 + col, kk * 32 + 8 * grp);
          else
            a = frag_kmaj(Ss, K::SP, vt * 16, kk * 32 + 8 * grp, kk * 32 + 8 * grp + 4);
          mma(st, a, qf[kk]);
          if constexpr (K::LO) {
            // what the bf16 copy of dH_c rounded away, from its own tile
            Frag<T> lo;
            if constexpr (SWZ)
              lo = frag_kmaj_at(Slo + kk * 4 * kBlk128, so_lo ^ (32 * vt), so_hi ^ (32 * vt));
            else
              lo = frag_kmaj(reinterpret_cast<const T *>(Slo), K::SP, vt * 16,
                             kk * 32 + 8 * grp, kk * 32 + 8 * grp + 4);
            mma(st, lo, qf[kk]);
          }
        }
        f4 w4 = zero4();
        if (MODE != kBwdDB && i < len) w4 = ld4f(row + vt * 16 + 4 * grp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = st[r] * sc;
          acc[vt][r] = MULTI ? acc[vt][r] + v : v;
          part_sp += w4[r] * v;
        }
      }
      if constexpr (MODE == kBwdDX) sp = part_sp;
      if constexpr (MODE == kBwdDC) {  // r_t of this head
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) part_sp += __shfl_xor(part_sp, off, 64);
        if (grp == 0 && i < len) rows.r[csh * Q + i] = part_sp;
      }
    }

    // ---- the masked intra-chunk terms
    for (int ph = 0; ph < len; ph += JP) {
      if (ph > 0) {
        __syncthreads();
        if constexpr (SWZ) {
          const int vr = min(len - ph, JP);
          load_k(kg + (size_t)ph * ks_, vr);
          load_v(vg + (size_t)ph * vs, vr);
        } else {
          dma_tile<T, K::KSL, K::KDS>(Ks, kg + (size_t)ph * ks_, ks_, JP, len - ph, wave, nw);
          dma_tile<T, K::VSL, K::VDS>(Vs, vg + (size_t)ph * vs, vs, JP, len - ph, wave, nw);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      int jb0, jend;
      if (REV) {
        jb0 = max(ph, t0 & ~31);
        jend = live ? min(ph + JP, len) : jb0;
      } else {
        jb0 = ph;
        jend = live ? min(ph + JP, tile_last + 1) : ph;
      }
      for (int jb = jb0; jb < jend; jb += 32) {
        const int jl = jb - ph;
        f4 g0 = zero4(), g1 = zero4();  // (K Q^T) for rows jb..jb+15 and jb+16..jb+31
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          Frag<T> k0, k1;
          if constexpr (SWZ && KD == 128) {
            const char *kb = Kc + (jl / 4) * kBlk256 + 64 * kk;
            k0 = frag_rowk_at(kb, r256);
            k1 = frag_rowk_at(kb + 4 * kBlk256, r256);
          } else if constexpr (SWZ) {
            const char *kb = Kc + (jl / 8) * kBlk128;
            k0 = frag_rowk_at(kb, r128 ^ (64 * kk));
            k1 = frag_rowk_at(kb + 2 * kBlk128, r128 ^ (64 * kk));
          } else {
            k0 = frag_rowk(Ks, K::KP, jl + col, kk * 32 + 8 * grp);
            k1 = frag_rowk(Ks, K::KP, jl + 16 + col, kk * 32 + 8 * grp);
          }
          mma(g0, k0, qf[kk]);
          mma(g1, k1, qf[kk]);
        }
        float m[8];
        const bool off = REV ? (jb > t0 + 15) : (jb + 31 < t0);
        if (off) {
          // block entirely past (reverse) or before (forward) the tile: the decay
          // factors through the block edge, both factors <= 1
          const float v = REV ? __builtin_amdgcn_exp2f(fminf(s_l[jb - 1] - si, 0.f))
                              : __builtin_amdgcn_exp2f(fminf(si - s_l[jb + 31], 0.f));
          const f4 u0 = ld4(u_l + jb + 4 * grp), u1 = ld4(u_l + jb + 16 + 4 * grp);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            m[r] = g0[r] * u0[r] * v;
            m[4 + r] = g1[r] * u1[r] * v;
          }
        } else {  // the block holding the tile's rows: causal mask, exact decay
          const f4 sj0 = ld4(s_l + jb + 4 * grp), sj1 = ld4(s_l + jb + 16 + 4 * grp);
          const f4 dj0 = ld4(dt_l + jb + 4 * grp), dj1 = ld4(dt_l + jb + 16 + 4 * grp);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j0 = jb + 4 * grp + r, j1 = j0 + 16;
            float e0, e1, k0, k1;
            if (REV) {
              e0 = __builtin_amdgcn_exp2f(fminf(sj0[r] - si, 0.f));
              e1 = __builtin_amdgcn_exp2f(fminf(sj1[r] - si, 0.f));
              k0 = j0 >= i ? 1.f : 0.f;
              k1 = j1 >= i ? 1.f : 0.f;
            } else {
              e0 = __builtin_amdgcn_exp2f(fminf(si - sj0[r], 0.f)) * dj0[r];
              e1 = __builtin_amdgcn_exp2f(fminf(si - sj1[r], 0.f)) * dj1[r];
              k0 = j0 <= i ? 1.f : 0.f;
              k1 = j1 <= i ? 1.f : 0.f;
            }
            m[r] = g0[r] * e0 * k0;
            m[4 + r] = g1[r] * e1 * k1;
          }
        }
        const Frag<T> mf = frag_from_f32(m, T());
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          Frag<T> a;
          if constexpr (SWZ && VD == 64) {
            const int o = v128 ^ (32 * vt);
            a = frag_kmaj_at(Vc + (jl / 8) * kBlk128, o, o + 2 * kBlk128);
          } else if constexpr (SWZ) {
            const int o = v256 ^ (32 * vt);
            a = frag_kmaj_at(Vc + jl * 256, o, o + 4 * kBlk256T);
          } else {
            a = frag_kmaj(Vs, K::VP, vt * 16, jl + 4 * grp, jl + 16 + 4 * grp);
          }
          mma(acc[vt], a, mf);
        }
        if constexpr (MODE == kBwdDX) {
          // W[t][i] = m dt_i (dy_t . x_i) in float32; rows t = jb + 4 grp + r (+16)
          f4 d0 = zero4(), d1 = zero4();
#pragma unroll
          for (int kk = 0; kk < KSP; ++kk) {
            Frag<T> a0, a1;
            if constexpr (SWZ) {
              const char *vb = Vc + (jl / 8) * kBlk128;
              a0 = frag_rowk_at(vb, r128 ^ (64 * kk));
              a1 = frag_rowk_at(vb + 2 * kBlk128, r128 ^ (64 * kk));
            } else {
              a0 = frag_rowk(Vs, K::VP, jl + col, kk * 32 + 8 * grp);
              a1 = frag_rowk(Vs, K::VP, jl + 16 + col, kk * 32 + 8 * grp);
            }
            mma(d0, a0, xf[kk]);
            mma(d1, a1, xf[kk]);
          }
          float w[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            w[r] = m[r] * d0[r] * dti;
            w[4 + r] = m[4 + r] * d1[r] * dti;
            csum += w[r] + w[4 + r];
          }
          // row sums over the 16 columns of the lane group: a reduce-scatter
          // with DPP moves inside the 16-lane row, pairing lane col with
          // 15 - col (row_mirror), then 7 - col within each half
          // (row_half_mirror), then col ^ 2 and col ^ 1 (quad_perm); at each
          // step the lane keeps one half of its values and adds the partner's
          // copy of that half.  Lane col ends with the total of value col >> 1.
          const bool b8 = col & 8, b4 = col & 4, b2 = col & 2;
          float w4[4], w2[2];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float snd = b8 ? w[k] : w[k + 4];
            w4[k] = (b8 ? w[k + 4] : w[k]) + dpp_mov<0x140>(snd);
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float snd = b4 ? w4[k] : w4[k + 2];
            w2[k] = (b4 ? w4[k + 2] : w4[k]) + dpp_mov<0x141>(snd);
          }
          float w1 = (b2 ? w2[1] : w2[0]) + dpp_mov<0x4E>(b2 ? w2[0] : w2[1]);
          w1 += dpp_mov<0xB1>(w1);
          if ((col & 1) == 0) {
            const int idx = col >> 1;  // value index: rows 4 grp + idx, or 16 + 4 grp + idx - 4
            const int t = jb + (idx < 4 ? 4 * grp + idx : 16 + 4 * grp + idx - 4);
            rs_l[wave * Q + t] = w1;
          }
        }
      }
    }
    if constexpr (MODE == kBwdDX) {  // W row sums of this part: fixed-order sum over the waves
      __syncthreads();
      for (int t = threadIdx.x; t < len; t += blockDim.x) {
        float sum = 0.f;
        for (int w = 0; w < nw; ++w) sum += rs_l[w * Q + t];
        rows.rs[(csh * SPLIT + part) * Q + t] = sum;
      }
    }
  }

  // ---- epilogue: lane holds column i, rows v = 16 vt + 4 grp + r
  if (!live) return;
  if constexpr (MODE == kBwdDX) {
    const int hd = hd0;
    const size_t csh = (size_t)c * H + hd;
    float qp = 0.f, dp = 0.f;
    const float Dh = D[hd];
    if (i < len) {
      const size_t row = ((size_t)ci.y + i) * H + hd;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const int v = vt * 16 + 4 * grp;
        const f4 x4 = ld4f(x + row * P + v), d4 = ld4f(dy + row * P + v);
        f4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[r] = Dh * d4[r] + dti * acc[vt][r];
          qp += x4[r] * acc[vt][r];
          dp += d4[r] * x4[r];
        }
        st4(out + row * P + v, o);
      }
    }
    // sum over the four lane groups holding column i
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      qp += __shfl_xor(qp, off, 64);
      dp += __shfl_xor(dp, off, 64);
      sp += __shfl_xor(sp, off, 64);
      csum += __shfl_xor(csum, off, 64);
    }
    if (grp == 0 && i < len) {
      rows.q[csh * Q + i] = qp;
      rows.dyx[csh * Q + i] = dp;
      rows.cv[csh * Q + i] = csum + dti * sp;  // W column sum + v_i
    }
  } else if (i < len) {
    const size_t orow = ((size_t)ci.y + i) * ostride + (ostride == G ? g : blk);
    const float sc = (MODE == kBwdDB && !MULTI) ? dti : 1.f;  // DB of one head: dt_i here
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      f4 o = acc[vt];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= sc;
      st4(out + orow * N + vt * 16 + 4 * grp, o);
    }
  }
}

// ----------------------------------------------------- backward state pass
// Per (sequence, head), per 4 state elements: walk the chunks last to first
// with g = dH_c; write dH_c (operand type), each 16-lane row's share of
// <dH_c, H_c> (H_c = the state entering chunk c+1, or the final state, both
// float32: the dot enters dz of every row of the chunk; summed in the row by
// DPP moves), then g <- 2^(s_end) g + Sb_c.  The last g is dh0.
template <typename T>
__global__ __launch_bounds__(256) void k_state_pass_bwd(
    const float *__restrict__ Sb, const float *__restrict__ s_ws, const int *__restrict__ seq_off,
    ChunkMap cmap, const float *__restrict__ dh_out, const float *__restrict__ hfin,
    const float *__restrict__ hin32, T *__restrict__ dHc, T *__restrict__ dHlo,
    float *__restrict__ epart, float *__restrict__ dh0, int H, int NP, int Q) {
  constexpr int BATCH = 8;
  const int s = blockIdx.z, hd = blockIdx.y;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int e = tid * 4;
  if (e >= NP) return;  // NP is a multiple of 256: whole waves leave
  const int npr = NP / 64, rid = tid >> 4, lane16 = threadIdx.x & 15;
  int c0, c1;
  if (cmap.L > 0) {
    const int cps = (cmap.L + Q - 1) / Q;
    c0 = s * cps;
    c1 = c0 + cps;
  } else {
    c0 = seq_off[s];
    c1 = seq_off[s + 1];
  }
  const size_t hofs = ((size_t)s * H + hd) * NP + e;
  f4 gv = dh_out ? ld4(dh_out + hofs) : zero4();
  f4 hend = ld4(hfin + hofs);
  for (int cb = c1 - 1; cb >= c0; cb -= BATCH) {
    f4 Sv[BATCH], Hv[BATCH];
    float sl[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (cb - u >= c0) {
        const size_t ch = (size_t)(cb - u) * H + hd;
        Sv[u] = ld4(Sb + ch * NP + e);
        Hv[u] = ld4(hin32 + ch * NP + e);
        sl[u] = s_ws[ch * Q + Q - 1];
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (cb - u >= c0) {  // wave-uniform
        const size_t ch = (size_t)(cb - u) * H + hd;
        float d = gv[0] * hend[0] + gv[1] * hend[1] + gv[2] * hend[2] + gv[3] * hend[3];
        d += dpp_mov<0xB1>(d);   // xor 1
        d += dpp_mov<0x4E>(d);   // xor 2
        d += dpp_mov<0x141>(d);  // lane i with 7 - i
        d += dpp_mov<0x140>(d);  // lane i with 15 - i
        if (lane16 == 0) epart[ch * npr + rid] = d;
        st4T(dHc + ch * NP + e, gv);
        if (dHlo) {  // bfloat16: what the rounding to dHc dropped, in dHc's layout
          const f4 hi = __builtin_convertvector(__builtin_convertvector(gv, bf16x4), f4);
          st4T(dHlo + ch * NP + e, gv - hi);
        }
        const float a = __builtin_amdgcn_exp2f(fminf(sl[u], 0.f));
#pragma unroll
        for (int q = 0; q < 4; ++q) gv[q] = a * gv[q] + Sv[u][q];
        hend = Hv[u];
      }
    }
  }
  if (dh0) st4(dh0 + hofs, gv);
}

// ------------------------------------------------------------ ddt, dA, dD
// One workgroup per (chunk, head), one thread per row (reversed, so that an
// inclusive scan gives the suffix sums): dz_i = sum_{t>=i} ds_t + <dH_c, H_c>.
__global__ __launch_bounds__(512) void k_bwd_ddt(BwdRows rows, int nsplit,
                                                 const float *__restrict__ dt_ws,
                                                 const float *__restrict__ epart, int npw,
                                                 const float *__restrict__ A, ChunkMap cmap,
                                                 int H, int Q, float *__restrict__ ddt,
                                                 float *__restrict__ dApart,
                                                 float *__restrict__ dDpart) {
  __shared__ float part[3][8];
  __shared__ float e_sh;
  const int c = blockIdx.x / H, hd = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int4 ci = cmap(c);
  const int len = ci.z;
  const size_t csh = (size_t)c * H + hd;
  if (wave == 0) {
    float e = 0.f;
    for (int k = lane; k < npw; k += 64) e += epart[csh * npw + k];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off, 64);
    if (lane == 0) e_sh = e;
  }
  const int i = Q - 1 - tid;  // rows in reverse
  const bool row = i >= 0 && i < len;
  float v = 0.f;
  if (row) {
    v = rows.r[csh * Q + i] - rows.cv[csh * Q + i];
    for (int k = 0; k < nsplit; ++k) v += rows.rs[(csh * nsplit + k) * Q + i];
  }
  float incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) part[0][wave] = incl;
  __syncthreads();
  float pre = 0.f;
  for (int w = 0; w < wave; ++w) pre += part[0][w];
  const float dz = pre + incl + e_sh;
  float da = 0.f, dd = 0.f;
  if (row) {
    const float dti = dt_ws[csh * Q + i];
    ddt[((size_t)ci.y + i) * H + hd] = A[hd] * dz + rows.q[csh * Q + i];
    da = dti * dz;
    dd = rows.dyx[csh * Q + i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    da += __shfl_xor(da, off, 64);
    dd += __shfl_xor(dd, off, 64);
  }
  if (lane == 0) {
    part[1][wave] = da;
    part[2][wave] = dd;
  }
  __syncthreads();
  if (tid == 0) {
    float sa = 0.f, sd = 0.f;
    for (int w = 0; w < nw; ++w) {
      sa += part[1][w];
      sd += part[2][w];
    }
    dApart[csh] = sa;
    dDpart[csh] = sd;
  }
}

// Fixed-order sums, one launch: workgroups [0, H) add the per-chunk partials
// of dA[h] and dD[h]; the rest (when parts > 1) add the `parts` partial rows of
// each group of dB and dC (partial row k of group g is row g * parts + k).
__global__ __launch_bounds__(256) void k_bwd_sums(const float *__restrict__ dApart,
                                                  const float *__restrict__ dDpart, int nc,
                                                  int H, float *__restrict__ dA,
                                                  float *__restrict__ dD,
                                                  const float *__restrict__ dBp,
                                                  const float *__restrict__ dCp,
                                                  float *__restrict__ dB, float *__restrict__ dC,
                                                  int64_t T, int G, int N, int parts) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < H) {
    __shared__ float part[2][4];
    const int hd = blockIdx.x, lane = tid & 63, wave = tid >> 6;
    float sa = 0.f, sd = 0.f;
    for (int c = tid; c < nc; c += 256) {
      sa += dApart[(size_t)c * H + hd];
      sd += dDpart[(size_t)c * H + hd];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sa += __shfl_xor(sa, off, 64);
      sd += __shfl_xor(sd, off, 64);
    }
    if (lane == 0) {
      part[0][wave] = sa;
      part[1][wave] = sd;
    }
    __syncthreads();
    if (tid == 0) {
      dA[hd] = part[0][0] + part[0][1] + part[0][2] + part[0][3];
      dD[hd] = part[1][0] + part[1][1] + part[1][2] + part[1][3];
    }
    return;
  }
  const int64_t idx = (int64_t)(blockIdx.x - H) * 256 + tid;
  const int nq = N / 4;
  if (idx >= T * G * nq) return;
  const int n = (int)(idx % nq) * 4, g = (int)((idx / nq) % G);
  const int64_t t = idx / ((int64_t)nq * G);
  f4 sb = zero4(), sc = zero4();
  for (int k = 0; k < parts; ++k) {
    const size_t o = ((size_t)t * G * parts + (size_t)g * parts + k) * N + n;
    sb += ld4(dBp + o);
    sc += ld4(dCp + o);
  }
  const size_t o = ((size_t)t * G + g) * N + n;
  st4(dB + o, sb);
  st4(dC + o, sc);
}

// ------------------------------------------------------------------ launch
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Heads per DB/DC workgroup: the largest divisor of H/G that still leaves at
// least 768 workgroups (three per CU), so few chunks keep every head apart and
// many chunks sum most heads of a group on chip.
static int bwd_heads_per_block(int64_t nc, int H, int G, int Q) {
  const int hpg = H / G, split = Q >= 256 ? 2 : 1;
  const int64_t units = nc * H * split;
  for (int d = hpg; d > 1; --d)
    if (hpg % d == 0 && units / d >= 768) return d;
  return 1;
}

BwdLayout bwd_layout(int64_t T, int nseq, int H, int P, int N, int G, int Q, int elem) {
  BwdLayout L{};
  L.fwd = prefill_layout(T, nseq, H, P, N, G, Q, elem);
  const size_t nc = (size_t)(L.fwd.nc_max > 0 ? L.fwd.nc_max : 1);
  const size_t NP = (size_t)N * P;
  size_t off = L.fwd.total;
  L.hfin = off;
  off = align_up(off + 4 * (size_t)nseq * H * NP, 256);
  L.hin32 = off;
  off = align_up(off + 4 * nc * H * NP, 256);
  L.dHc = off;
  off = align_up(off + (size_t)elem * nc * H * NP, 256);
  L.dHlo = off;  // bfloat16 only
  off = align_up(off + (elem == 2 ? 2 * nc * H * NP : 0), 256);
  L.epart = off;
  off = align_up(off + 4 * nc * H * (NP / 64), 256);
  L.rows = off;  // q, cv, r, dyx, then rs for two parts
  off = align_up(off + 4 * 6 * nc * H * Q, 256);
  L.dApart = off;
  off = align_up(off + 4 * nc * H, 256);
  L.dDpart = off;
  off = align_up(off + 4 * nc * H, 256);
  const int hb = bwd_heads_per_block(L.fwd.nc_max, H, G, Q);
  const size_t per_head = hb < H / G ? 4 * (size_t)(T > 0 ? T : 0) * (H / hb) * N : 0;
  L.dBh = off;
  off = align_up(off + per_head, 256);
  L.dCh = off;
  off = align_up(off + per_head, 256);
  L.total = off;
  return L;
}

static BwdRows bwd_rows(char *ws, const BwdLayout &L, int nc, int H, int Q) {
  float *base = reinterpret_cast<float *>(ws + L.rows);
  const size_t n = (size_t)(nc > 0 ? nc : 1) * H * Q;
  return BwdRows{base, base + n, base + 2 * n, base + 3 * n, base + 4 * n};
}

template <typename T, int MODE, int P, int N>
static hipError_t launch_bwd_scan(const BwdArgs &a, const BwdLayout &L, int nc, const T *state,
                                  const T *state_lo, float *out, int ostride, int hb,
                                  hipStream_t st) {
  constexpr int KD = MODE == kBwdDX ? N : P, VD = MODE == kBwdDX ? P : N;
  typedef BwdScanCfg<T, MODE, KD, VD> K;
  const int Q = a.f.Q;
  const int split = Q >= 256 ? 2 : 1;
  const int threads = 64 * (Q / 16) / split;
  const int jp = K::jp(Q, threads);
  const size_t lds = K::lds_bytes(jp, Q, threads / 64);
  if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
  const void *kern;
  if (hb > 1) {  // several heads per workgroup (DB and DC only)
    if constexpr (MODE != kBwdDX) {
      kern = split == 1     ? (const void *)k_bwd_scan<T, MODE, P, N, 1, 512, true>
             : threads <= 512 ? (const void *)k_bwd_scan<T, MODE, P, N, 2, 512, true>
                              : (const void *)k_bwd_scan<T, MODE, P, N, 2, 1024, true>;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    kern = split == 1     ? (const void *)k_bwd_scan<T, MODE, P, N, 1, 512, false>
           : threads <= 512 ? (const void *)k_bwd_scan<T, MODE, P, N, 2, 512, false>
                            : (const void *)k_bwd_scan<T, MODE, P, N, 2, 1024, false>;
  }
  hipError_t e = set_lds_limit(kern);
  if (e != hipSuccess) return e;
  char *ws = static_cast<char *>(a.f.workspace);
  const T *xp = (const T *)a.f.x, *dyp = (const T *)a.dy, *bp = (const T *)a.f.B,
          *cp = (const T *)a.f.C;
  const float *Dp = a.f.D;
  const float *sp = reinterpret_cast<const float *>(ws + L.fwd.s);
  const float *dtp = reinterpret_cast<const float *>(ws + L.fwd.dt);
  const float *up = reinterpret_cast<const float *>(ws + L.fwd.u);
  ChunkMap cm{reinterpret_cast<const int4 *>(ws + L.fwd.info),
              a.f.cu ? 0 : (int)(a.f.T / a.f.nseq), a.f.nseq, Q};
  int nc_ = nc, H_ = a.f.H, G_ = a.f.G, Q_ = Q, jp_ = jp, hb_ = hb, os_ = ostride;
  BwdRows rows = bwd_rows(ws, L, nc, a.f.H, Q);
  void *args[] = {&xp, &dyp, &bp, &cp, &Dp, &sp, &dtp, &up, &state, &state_lo, &cm, &nc_,
                  &H_, &G_, &Q_, &jp_, &hb_, &out, &os_, &rows};
  return hipLaunchKernel(kern, dim3(xcd_grid(nc, (a.f.H / hb) * split)), dim3(threads), args, lds,
                         st);
}

template <typename T, int P, int N>
static hipError_t run_backward(const BwdArgs &a) {
  const PrefillArgs &f = a.f;
  const BwdLayout L = bwd_layout(f.T, f.nseq, f.H, P, N, f.G, f.Q, sizeof(T));
  char *ws = static_cast<char *>(f.workspace);
  hipStream_t st = static_cast<hipStream_t>(f.stream);
  const int nc = (int)L.fwd.nc_max;
  const int NP = N * P;
  float *hfin = reinterpret_cast<float *>(ws + L.hfin);
  float *hin32 = reinterpret_cast<float *>(ws + L.hin32);
  T *dHc = reinterpret_cast<T *>(ws + L.dHc);
  T *dHlo = sizeof(T) == 2 ? reinterpret_cast<T *>(ws + L.dHlo) : nullptr;
  T *hin = reinterpret_cast<T *>(ws + L.fwd.hin);
  float *S = reinterpret_cast<float *>(ws + L.fwd.S);
  float *epart = reinterpret_cast<float *>(ws + L.epart);
  float *dApart = reinterpret_cast<float *>(ws + L.dApart);
  float *dDpart = reinterpret_cast<float *>(ws + L.dDpart);
  const ChunkMap cmap{reinterpret_cast<const int4 *>(ws + L.fwd.info),
                      f.cu ? 0 : (int)(f.T / f.nseq), f.nseq, f.Q};
  hipError_t e;

  // forward recompute: s, dt, u, chunk states, H_in per chunk and the final
  // states (skipped when a training forward left them in the workspace)
  if (!a.saved) {
    PrefillArgs fa = f;
    fa.y = nullptr;
    fa.h_out = hfin;
    fa.hin32 = hin32;
    fa.scan_follows = false;  // only the states are recomputed
    fa.precise_states = true;  // as the training forward computes them
    e = launch_prefill(fa, 7u);
    if (e != hipSuccess) return e;
  }
  if (nc > 0) {  // Sb_c over the spent chunk states
    PrefillArgs ba = f;
    ba.x = a.dy;
    ba.B = f.C;
    e = launch_chunk_state(ba, L.fwd, nc, true, st, true);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_state_pass_bwd<T>, dim3((NP + 1023) / 1024, f.H, f.nseq), dim3(256), 0, st,
                     S, reinterpret_cast<const float *>(ws + L.fwd.s),
                     reinterpret_cast<const int *>(ws + L.fwd.seq_off), cmap, a.dh_out, hfin,
                     hin32, dHc, dHlo, epart, a.dh0, f.H, NP, f.Q);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hb = bwd_heads_per_block(nc, f.H, f.G, f.Q);
  const int parts = f.H / f.G / hb;  // partial rows per group and token (1: written directly)
  float *dBo = parts == 1 ? a.dB : reinterpret_cast<float *>(ws + L.dBh);
  float *dCo = parts == 1 ? a.dC : reinterpret_cast<float *>(ws + L.dCh);
  if (nc > 0) {
    const int os = f.H / hb;
    e = launch_bwd_scan<T, kBwdDX, P, N>(a, L, nc, dHc, dHlo, a.dx, f.H, 1, st);
    if (e != hipSuccess) return e;
    e = launch_bwd_scan<T, kBwdDB, P, N>(a, L, nc, dHc, nullptr, dBo, os, hb, st);
    if (e != hipSuccess) return e;
    e = launch_bwd_scan<T, kBwdDC, P, N>(a, L, nc, hin, nullptr, dCo, os, hb, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_ddt, dim3((unsigned)nc * f.H), dim3(f.Q < 64 ? 64 : f.Q), 0, st,
                       bwd_rows(ws, L, nc, f.H, f.Q), f.Q >= 256 ? 2 : 1,
                       reinterpret_cast<const float *>(ws + L.fwd.dt), epart, NP / 64, f.A, cmap,
                       f.H, f.Q, a.ddt, dApart, dDpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t ngs = (parts > 1 && nc > 0) ? (f.T * f.G * (N / 4) + 255) / 256 : 0;
  hipLaunchKernelGGL(k_bwd_sums, dim3((unsigned)(f.H + ngs)), dim3(256), 0, st, dApart, dDpart,
                     nc, f.H, a.dA, a.dD, dBo, dCo, a.dB, a.dC, f.T, f.G, N, parts);
  return hipGetLastError();
}

template <typename T, int P>
static hipError_t bwd_N(const BwdArgs &a) {
  switch (a.f.N) {
    case 16: return run_backward<T, P, 16>(a);
    case 32: return run_backward<T, P, 32>(a);
    case 64: return run_backward<T, P, 64>(a);
    case 128: return run_backward<T, P, 128>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t bwd_P(const BwdArgs &a) {
  switch (a.f.P) {
    case 16: return bwd_N<T, 16>(a);
    case 32: return bwd_N<T, 32>(a);
    case 64: return bwd_N<T, 64>(a);
    case 128: return bwd_N<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_backward(const BwdArgs &a) {
  return a.f.bf16 ? bwd_P<bf16>(a) : bwd_P<float>(a);
}

hipError_t launch_prefill_train_forward(const PrefillArgs &f) {
  const BwdLayout L = bwd_layout(f.T, f.nseq, f.H, f.P, f.N, f.G, f.Q, f.bf16 ? 2 : 4);
  char *ws = static_cast<char *>(f.workspace);
  float *hfin = reinterpret_cast<float *>(ws + L.hfin);
  PrefillArgs fa = f;
  fa.h_out = hfin;  // the state pass writes the final state here and to the caller's h_out
  fa.h_out2 = f.h_out;
  fa.hin32 = reinterpret_cast<float *>(ws + L.hin32);
  fa.precise_states = true;  // the backward reads these states (bitwise as its recompute)
  return launch_prefill(fa, 15u);
}

}  // namespace ssd
