// ssd_scan_heads.hip -- chunk scan (the output stage of the chunked prefill)
// with the heads of one B/C group streamed through a workgroup, bfloat16.
//
// Per chunk c and head h (s in log2 units, all exponents <= 0):
//   y_i = 2^(s_i) C_i . H_in                                  state entering the chunk
//       + sum_{j<=i} (C_i . B_j) 2^(s_i - s_j) dt_j x_j          intra-chunk, causal
//       + D_h x_i
// the regrouping of the recurrence into fixed-length chunks given by
// Compiler-First State Space Duality and Portable O(1) Autoregressive Caching
// for Inference (Abstract; static causal mask of Table 7, float32 decay of
// Table 8).
//
// C.B^T does not depend on the head.  A workgroup takes one chunk and HB heads
// of one group: it computes C.B^T once, keeps it in registers (bfloat16), and
// then streams the heads: while head k is computed from one LDS buffer, the
// direct global->LDS loads of head k+1 (x, H_in, s, dt, u) fill the other.
//
// Q/32 waves, 16-row output tiles; wave w owns tiles w and Q/16-1-w, whose
// causal work is Q/32+1 blocks of 32 columns j in every wave.  Block slots of
// the upper tile sit at cb[0 .. nB-1], those of the lower tile at
// cb[NS-1 .. NS-nA] (nA + nB = NS), so every register index is a compile-time
// constant.  Each lane holds, per slot, the pair layout of two stacked 16x16
// results (rows 4g..4g+3 and 16+4g..16+4g+3 of the block, column i): after the
// decay it is the B operand of Y^T += X^T M^T as it stands.
#include <algorithm>

#include "ssd.h"
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

template <int P, int N, int Q> struct HeadsCfg {
  static constexpr int NW = Q / 32;       // waves
  static constexpr int NT = Q / 16;       // output tiles
  static constexpr int NS = Q / 32 + 1;   // j-block slots per wave
  static constexpr int KS = N / 32;       // k-steps over n
  static constexpr int NPT = P / 16;      // 16-column tiles of p
  static constexpr int VN = 8;            // bf16 per 16 bytes
  // 128-byte x / H_in rows and 256-byte B rows: block-swizzled tiles
  static constexpr bool SWZ = P == 64 && N == 128;
  static constexpr int XP = P + kTrPad, HP = P + kTrPad, BP = N + 8;  // LDS pitches (elements)
  static constexpr int XS = XP / VN, HS = HP / VN, BS = BP / VN;       // 16-byte slots per row
  static constexpr int PD = P / VN, ND = N / VN;                       // data slots per row
  static constexpr int QS = Q / 4;                                     // slots of one float row
  // one head's buffer: X, H_in, s, dt, u (bytes, 16-aligned)
  static constexpr int X_BYTES = SWZ ? Q / 8 * kBlk128 : tile_slots(Q, XS) * 16;
  static constexpr int H_BYTES = SWZ ? N / 8 * kBlk128 : tile_slots(N, HS) * 16;
  static constexpr int X_OFF = 0;
  static constexpr int H_OFF = X_OFF + X_BYTES;
  static constexpr int S_OFF = H_OFF + H_BYTES;
  static constexpr int DT_OFF = S_OFF + tile_slots(1, QS) * 16;
  static constexpr int U_OFF = DT_OFF + tile_slots(1, QS) * 16;
  static constexpr int BUF = U_OFF + tile_slots(1, QS) * 16;
  // B, only before the heads
  static constexpr int B_BYTES = SWZ ? Q / 4 * kBlk256 : tile_slots(Q, BS) * 16;
  static constexpr int LDS = BUF + (BUF > B_BYTES ? BUF : B_BYTES);
  static_assert(P % 16 == 0 && N % 32 == 0 && Q % 32 == 0, "tile shape");
};

// Issue the direct loads of one head into buffer `buf` (no wait).  Swizzled
// tiles: xl / hl are the lane's offsets into a block's x / H_in rows.
template <int P, int N, int Q>
__device__ __forceinline__ void load_head(char *buf, const bf16 *__restrict__ xs, size_t xstride,
                                          const bf16 *__restrict__ hs, const float *__restrict__ s,
                                          const float *__restrict__ dt,
                                          const float *__restrict__ u, int len, int wave,
                                          uint32_t xl, uint32_t hl) {
  typedef HeadsCfg<P, N, Q> K;
  if constexpr (K::SWZ) {
    const uint32_t xsb = (uint32_t)(xstride * sizeof(bf16));
    dma_swz<kBlk128>(buf + K::X_OFF, xs, len * xsb, xl, 8 * xsb, Q / 8, wave, K::NW);
    dma_swz<kBlk128>(buf + K::H_OFF, hs, N * P * 2, hl, 1024, N * P * 2 / 1024, wave, K::NW);
    // the three float rows, 1 KB requests from different waves
    const uint32_t fl = 16 * (threadIdx.x & 63);
    constexpr int NR = (Q * 4 + 1023) / 1024;
    const int w1 = wave >= 1 % K::NW ? wave - 1 % K::NW : wave - 1 % K::NW + K::NW;
    const int w2 = wave >= 2 % K::NW ? wave - 2 % K::NW : wave - 2 % K::NW + K::NW;
    dma_swz<1024>(buf + K::S_OFF, s, Q * 4, fl, 1024, NR, wave, K::NW);
    dma_swz<1024>(buf + K::DT_OFF, dt, Q * 4, fl, 1024, NR, w1, K::NW);
    dma_swz<1024>(buf + K::U_OFF, u, Q * 4, fl, 1024, NR, w2, K::NW);
  } else {
    dma_tile<bf16, K::XS, K::PD>(reinterpret_cast<bf16 *>(buf + K::X_OFF), xs, xstride, Q, len,
                                 wave, K::NW);
    dma_tile<bf16, K::HS, K::PD>(reinterpret_cast<bf16 *>(buf + K::H_OFF), hs, (size_t)P, N, N,
                                 wave, K::NW);
    dma_tile<float, K::QS, K::QS>(reinterpret_cast<float *>(buf + K::S_OFF), s, 0, 1, 1, wave,
                                  K::NW);
    dma_tile<float, K::QS, K::QS>(reinterpret_cast<float *>(buf + K::DT_OFF), dt, 0, 1, 1, wave,
                                  K::NW);
    dma_tile<float, K::QS, K::QS>(reinterpret_cast<float *>(buf + K::U_OFF), u, 0, 1, 1, wave,
                                  K::NW);
  }
}

// The decayed, masked block of M^T for one slot: m = (B C^T)[j][i] * 2^(s_i - s_j) dt_j
// for j <= i.  Blocks wholly before the tile factor the decay through the
// block's last row r: 2^(s_i - s_r) * u_j, u_j = 2^(s_r - s_j) dt_j (both <= 1).
__device__ __forceinline__ Frag<bf16> decay_block(bf16x8 gb, int jb, int t0, int i, float si,
                                                  const float *s_l, const float *dt_l,
                                                  const float *u_l, int grp) {
  // opaque per use: keeps the compiler from hoisting the unpacked float32
  // copy of every slot out of the head loop (which needs twice the registers)
  asm volatile("" : "+v"(gb));
  const f8v g = cvt_f8(gb);
  float m[8];
  if (jb + 32 <= t0) {
    const float v = __builtin_amdgcn_exp2f(fminf(si - s_l[jb + 31], 0.f));
    const f4 u0 = ld4(u_l + jb + 4 * grp), u1 = ld4(u_l + jb + 16 + 4 * grp);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[r] = g[r] * (u0[r] * v);
      m[4 + r] = g[4 + r] * (u1[r] * v);
    }
  } else {
    const f4 sj0 = ld4(s_l + jb + 4 * grp), sj1 = ld4(s_l + jb + 16 + 4 * grp);
    const f4 dj0 = ld4(dt_l + jb + 4 * grp), dj1 = ld4(dt_l + jb + 16 + 4 * grp);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j0 = jb + 4 * grp + r, j1 = j0 + 16;
      const float e0 = __builtin_amdgcn_exp2f(fminf(si - sj0[r], 0.f)) * dj0[r];
      const float e1 = __builtin_amdgcn_exp2f(fminf(si - sj1[r], 0.f)) * dj1[r];
      m[r] = j0 <= i ? g[r] * e0 : 0.f;
      m[4 + r] = j1 <= i ? g[4 + r] * e1 : 0.f;
    }
  }
  return frag_from_f32(m, bf16());
}

// Value of lane (l + 8) mod 16 of the lane's 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ float rot8(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

template <int P, int N, int Q>
__global__ __launch_bounds__(64 * (Q / 32)) void k_chunk_scan_heads(
    const bf16 *__restrict__ x, const bf16 *__restrict__ B, const bf16 *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ s_ws, const float *__restrict__ dt_ws,
    const float *__restrict__ u_ws, const bf16 *__restrict__ hin, ChunkMap cmap, int nc, int H,
    int G, int HB, float *__restrict__ y) {
  typedef HeadsCfg<P, N, Q> K;
  constexpr int NS = K::NS, KS = K::KS, NPT = K::NPT;
  constexpr bool SWZ = K::SWZ;
  const ChunkHead ch = xcd_chunk_head(H / HB);
  const int c = ch.c, h0 = ch.h * HB;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  const int len = ci.z;
  if (len <= 0) return;
  const int g = (h0 * G) / H;  // HB divides H / G: every head of the block reads group g
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tA = wave, tB = K::NT - 1 - wave;  // tA < tB
  const int nA = tA / 2 + 1, nB = tB / 2 + 1;  // j-blocks of each tile; nA + nB = NS
  const int iA = 16 * tA + col, iB = 16 * tB + col;

  extern __shared__ __align__(16) char smem[];
  char *buf0 = smem, *buf1 = smem + K::BUF;
  const bf16 *Bs = reinterpret_cast<const bf16 *>(buf1);  // B aliases the second buffer

  const size_t xstride = (size_t)H * P, bstride = (size_t)G * N;
  const bf16 *xc = x + (size_t)ci.y * xstride;
  const bf16 *bc = B + (size_t)ci.y * bstride + (size_t)g * N;
  const bf16 *cc = C + (size_t)ci.y * bstride + (size_t)g * N;
  auto head_ptrs = [&](int hd, const bf16 *&xs, const bf16 *&hs, size_t &o) {
    xs = xc + (size_t)hd * P;
    o = (size_t)c * H + hd;
    hs = hin + o * (size_t)(N * P);
  };
  // swizzled loads: the lane's offsets into a block's x, H_in and B rows
  const int lb8 = lane >> 3, lb4 = lane >> 4;
  const uint32_t xsb = (uint32_t)(xstride * 2), bsb = (uint32_t)(bstride * 2);
  const uint32_t xl = lb8 * xsb + 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  const uint32_t hl = lb8 * (P * 2) + 16 * ((lane & 7) ^ (2 * swz8(lb8)));

  // ---- prologue: head h0 -> buffer 0, B -> buffer 1, C^T fragments -> registers
  {
    const bf16 *xs, *hs;
    size_t o;
    head_ptrs(h0, xs, hs, o);
    load_head<P, N, Q>(buf0, xs, xstride, hs, s_ws + o * Q, dt_ws + o * Q, u_ws + o * Q, len, wave,
                       xl, hl);
  }
  if constexpr (SWZ)
    dma_swz<kBlk256>(buf1, bc, len * bsb, lb4 * bsb + 16 * ((lane & 15) ^ lb4), 4 * bsb, Q / 4,
                     wave, K::NW);
  else
    dma_tile<bf16, K::BS, K::ND>(const_cast<bf16 *>(Bs), bc, bstride, Q, len, wave, K::NW);
  Frag<bf16> cfA[KS], cfB[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int n8 = ks * 32 + 8 * grp;
    cfA[ks] = iA < len ? frag_global(cc + (size_t)iA * bstride + n8) : frag_zero<bf16>();
    cfB[ks] = iB < len ? frag_global(cc + (size_t)iB * bstride + n8) : frag_zero<bf16>();
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // lane byte offsets into the swizzled tiles (bits 5-6 hold the segment
  // swizzle, so segment pt is reached by XOR with 32 pt):
  //  H_in rows ks*32 + 8 grp + col/4 (+4): block 4 ks + grp, row col/4 (+4)
  //  X rows jb + 4 grp + col/4 (+16): block jb/8 + grp/2 (+2), row 4 (grp&1) + col/4
  //  B rows 32 k + col (+16): block 8 k + col/4 (+4), row col&3, vector 4 ks + grp
  //  D x, row 16 t + col: block 2 t + col/8, row col&7, 8 bytes at 32 pt + 8 grp
  const int c4 = col >> 2, cq = 8 * (col & 3);
  const int hlo = grp * kBlk128 + c4 * 128 + cq + 32 * swz8(c4);
  const int hhi = grp * kBlk128 + (4 + c4) * 128 + cq + 32 * swz8(4 + c4);
  const int xb = 4 * (grp & 1) + c4;
  const int xo = (grp >> 1) * kBlk128 + xb * 128 + cq + 32 * swz8(xb);
  const int bo = c4 * kBlk256 + (col & 3) * 256 + 16 * (grp ^ (col & 3));
  const int dxo = (col >> 3) * kBlk128 + (col & 7) * 128 + 8 * grp + 32 * swz8(col & 7);

  // ---- C.B^T for every slot of both tiles (k = n), kept in registers as
  // bfloat16 (the operand precision of the product it feeds)
  bf16x8 cb[NS];
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {
    if (k < nB) {
      f4 gB0 = zero4(), gB1 = zero4(), gA0 = zero4(), gA1 = zero4();
      const bool a = k < nA;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<bf16> b0, b1;
        if constexpr (SWZ) {
          const char *bb = buf1 + 8 * k * kBlk256 + 64 * ks;
          b0 = frag_rowk_at(bb, bo);
          b1 = frag_rowk_at(bb + 4 * kBlk256, bo);
        } else {
          b0 = frag_rowk(Bs, K::BP, 32 * k + col, ks * 32 + 8 * grp);
          b1 = frag_rowk(Bs, K::BP, 32 * k + 16 + col, ks * 32 + 8 * grp);
        }
        mma(gB0, b0, cfB[ks]);
        mma(gB1, b1, cfB[ks]);
        if (a) {
          mma(gA0, b0, cfA[ks]);
          mma(gA1, b1, cfA[ks]);
        }
      }
      cb[k] = cvt_bf8(f8v{gB0[0], gB0[1], gB0[2], gB0[3], gB1[0], gB1[1], gB1[2], gB1[3]});
      if (a) cb[NS - 1 - k] = cvt_bf8(f8v{gA0[0], gA0[1], gA0[2], gA0[3], gA1[0], gA1[1], gA1[2], gA1[3]});
    }
  }
  __syncthreads();  // B is no longer read: buffer 1 may be refilled

  for (int hk = 0; hk < HB; ++hk) {
    const int hd = h0 + hk;
    // buffer offset as one opaque register: every LDS access of the head is
    // then that register plus an immediate offset
    int cur_off = (hk & 1) * K::BUF;
    asm volatile("" : "+v"(cur_off));
    const char *cur = smem + cur_off;
    if (hk + 1 < HB) {  // next head's loads fly while this head is computed
      const bf16 *xs, *hs;
      size_t o;
      head_ptrs(hd + 1, xs, hs, o);
      load_head<P, N, Q>((hk & 1) ? buf0 : buf1, xs, xstride, hs, s_ws + o * Q, dt_ws + o * Q,
                         u_ws + o * Q, len, wave, xl, hl);
    }
    const bf16 *Xs = reinterpret_cast<const bf16 *>(cur + K::X_OFF);
    const bf16 *Hs = reinterpret_cast<const bf16 *>(cur + K::H_OFF);
    const float *s_l = reinterpret_cast<const float *>(cur + K::S_OFF);
    const float *dt_l = reinterpret_cast<const float *>(cur + K::DT_OFF);
    const float *u_l = reinterpret_cast<const float *>(cur + K::U_OFF);
    const float siA = s_l[iA], siB = s_l[iB];
    int iAh = iA, iBh = iB;  // opaque per head: the diagonal masks are rebuilt, not held
    asm volatile("" : "+v"(iAh), "+v"(iBh));

    // state entering the chunk: Y^T = 2^(s_i) H_in^T C^T
    f4 accA[NPT], accB[NPT];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      accA[pt] = zero4();
      accB[pt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<bf16> a;
        if constexpr (SWZ)
          a = frag_kmaj_at(cur + K::H_OFF + ks * 4 * kBlk128, hlo ^ (32 * pt), hhi ^ (32 * pt));
        else
          a = frag_kmaj(Hs, K::HP, pt * 16, ks * 32 + 8 * grp, ks * 32 + 8 * grp + 4);
        mma(accA[pt], a, cfA[ks]);
        mma(accB[pt], a, cfB[ks]);
      }
    }
    {
      const float eA = __builtin_amdgcn_exp2f(fminf(siA, 0.f));
      const float eB = __builtin_amdgcn_exp2f(fminf(siB, 0.f));
      const float dv = D[hd];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {  // + D x_i
        f4 xA, xB;
        if constexpr (SWZ) {
          const char *xc_ = cur + K::X_OFF + (dxo ^ (32 * pt));
          xA = ld4f(reinterpret_cast<const bf16 *>(xc_ + 2 * tA * kBlk128));
          xB = ld4f(reinterpret_cast<const bf16 *>(xc_ + 2 * tB * kBlk128));
        } else {
          xA = ld4f(Xs + iA * K::XP + pt * 16 + 4 * grp);
          xB = ld4f(Xs + iB * K::XP + pt * 16 + 4 * grp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          accA[pt][r] = accA[pt][r] * eA + dv * xA[r];
          accB[pt][r] = accB[pt][r] * eB + dv * xB[r];
        }
      }
    }

    // intra-chunk: Y^T += X^T M^T over the j-blocks, the X fragments shared by
    // both tiles.  Every wave runs the same straight sequence: a tile with
    // fewer blocks multiplies a zero M block (wave-uniform branches choose only
    // the M fragment, never whether an accumulator is updated).
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      const int jb = 32 * k;
      Frag<bf16> mB = frag_zero<bf16>(), mA = frag_zero<bf16>();
      if (k < nB) mB = decay_block(cb[k], jb, 16 * tB, iBh, siB, s_l, dt_l, u_l, grp);
      if (k < nA) mA = decay_block(cb[NS - 1 - k], jb, 16 * tA, iAh, siA, s_l, dt_l, u_l, grp);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        Frag<bf16> xa;
        if constexpr (SWZ) {
          const char *xb_ = cur + K::X_OFF + (jb / 8) * kBlk128;
          xa = frag_kmaj_at(xb_, xo ^ (32 * pt), (xo ^ (32 * pt)) + 2 * kBlk128);
        } else {
          xa = frag_kmaj(Xs, K::XP, pt * 16, jb + 4 * grp, jb + 16 + 4 * grp);
        }
        mma(accB[pt], xa, mB);
        mma(accA[pt], xa, mA);
      }
    }

    // the next head's loads have landed and nobody reads this buffer any more;
    // the stores go out after the wait so it never waits for them
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // y rows leave as whole 128-byte lines: lanes i and i^8 of each 16-lane
    // row swap the odd p-tile (DPP rotate by 8), so one store covers 8 rows x
    // 32 columns instead of 16 rows x 16 columns
    const bool lo = col < 8;
    auto put = [&](const f4 (&acc)[NPT], int t) {
#pragma unroll
      for (int pt = 0; pt < NPT; pt += 2) {
        // built as a whole vector from four scalar moves (element-wise
        // inserts into the vector are not lowered correctly)
        const f4 o = acc[pt + 1];
        const f4 r = f4{rot8(o[0]), rot8(o[1]), rot8(o[2]), rot8(o[3])};
        const int i1 = 16 * t + (lo ? col : col - 8), i2 = i1 + 8;
        const f4 v1 = lo ? acc[pt] : r, v2 = lo ? r : acc[pt];
        const int c1 = 16 * (lo ? pt : pt + 1) + 4 * grp, c2 = 16 * (lo ? pt + 1 : pt) + 4 * grp;
        if (i1 < len)
          __builtin_nontemporal_store(
              v1, reinterpret_cast<f4 *>(y + (((size_t)ci.y + i1) * H + hd) * P + c1));
        if (i2 < len)
          __builtin_nontemporal_store(
              v2, reinterpret_cast<f4 *>(y + (((size_t)ci.y + i2) * H + hd) * P + c2));
      }
    };
    put(accA, tA);
    put(accB, tB);
  }
}

// ------------------------------------------------------------------ launch
template <int P, int N, int Q>
static hipError_t run_heads(const PrefillArgs &a, const WorkspaceLayout &L, int nc, int HB,
                            hipStream_t st) {
  static_assert(P % 32 == 0, "stores pair p-tiles");
  typedef HeadsCfg<P, N, Q> K;
  const void *kern = (const void *)k_chunk_scan_heads<P, N, Q>;
  hipError_t e = set_lds_limit(kern);
  if (e != hipSuccess) return e;
  char *ws = static_cast<char *>(a.workspace);
  const bf16 *xp = (const bf16 *)a.x, *bp = (const bf16 *)a.B, *cp = (const bf16 *)a.C;
  const float *Dp = a.D;
  const float *sp = reinterpret_cast<const float *>(ws + L.s);
  const float *dp = reinterpret_cast<const float *>(ws + L.dt);
  const float *up = reinterpret_cast<const float *>(ws + L.u);
  const bf16 *hp = reinterpret_cast<const bf16 *>(ws + L.hin);
  ChunkMap cm{reinterpret_cast<const int4 *>(ws + L.info), a.cu ? 0 : (int)(a.T / a.nseq), a.nseq,
              a.Q};
  int nc_ = nc, H_ = a.H, G_ = a.G, HB_ = HB;
  float *yp = a.y;
  void *args[] = {&xp, &bp, &cp, &Dp, &sp, &dp, &up, &hp, &cm, &nc_, &H_, &G_, &HB_, &yp};
  return hipLaunchKernel(kern, dim3(xcd_grid(nc, a.H / HB)), dim3(64 * K::NW), args, K::LDS, st);
}

// Whether to stream heads, and how many per workgroup (0: use the row-split
// scan).  Streaming pays once there are several workgroups of heads per CU:
// a short stream spends most of its time loading B and forming C.B^T.  The
// head count d (a divisor of H/G) minimises rounds(d) * (d + 2): rounds of
// resident workgroups (`slots` of them at once) times the time of one
// workgroup, d heads plus a fixed cost (B, C.B^T, the first head's loads)
// taken as two heads' worth.  Ties go to the larger d.  The variant bits
// SSD_VARIANT_SCAN_ROWS / _HEADS of the call force either kernel.
static int pick_heads(int nc, int H, int G, long slots, unsigned variant) {
  const bool want_rows = (variant & SSD_VARIANT_SCAN_ROWS) != 0;
  const bool want_heads = (variant & SSD_VARIANT_SCAN_HEADS) != 0;
  const long units = (long)nc * H;
  if (want_rows || (!want_heads && units < 2048)) return 0;
  const int hg = H / G;
  int best = 1;
  long best_cost = -1;
  for (int d = 1; d <= hg; ++d) {
    if (hg % d) continue;
    const long wgs = units / d, rounds = (wgs + slots - 1) / slots;
    const long cost = rounds * (d + 2);
    if (best_cost < 0 || cost <= best_cost) {
      best = d;
      best_cost = cost;
    }
  }
  return best;
}

#define SSD_HEADS_CASES(X) X(64, 128, 256) X(64, 128, 128) X(64, 128, 64) X(64, 64, 256) \
  X(64, 64, 128) X(32, 128, 256) X(32, 64, 256)

// Workgroups of one instance resident on the chip at once (256 CUs): bounded
// by LDS and by the waves a CU holds at the kernel's register use (two per
// SIMD); 0 when there is no instance for the shape.
static long heads_slots(int P, int N, int Q, bool bf16) {
  if (!bf16) return 0;
#define SSD_CASE(p, n, q)                                                    \
  if (P == p && N == n && Q == q) {                                          \
    const long by_lds = (160L * 1024) / HeadsCfg<p, n, q>::LDS;              \
    const long by_waves = 8 / HeadsCfg<p, n, q>::NW;                         \
    return 256 * std::max(1L, std::min(by_lds, by_waves));                   \
  }
  SSD_HEADS_CASES(SSD_CASE)
#undef SSD_CASE
  return 0;
}

int scan_heads_choice(int P, int N, int Q, bool bf16, int nc, int H, int G, unsigned variant) {
  const long slots = heads_slots(P, N, Q, bf16);
  return slots > 0 ? pick_heads(nc, H, G, slots, variant) : 0;
}

hipError_t launch_scan_heads(const PrefillArgs &a, const WorkspaceLayout &L, int nc, int HB,
                             hipStream_t st) {
#define SSD_CASE(p, n, q) \
  if (a.P == p && a.N == n && a.Q == q) return run_heads<p, n, q>(a, L, nc, HB, st);
  SSD_HEADS_CASES(SSD_CASE)
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
