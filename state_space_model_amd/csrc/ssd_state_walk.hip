// ssd_state_walk.hip -- the state half of the chunked prefill for large
// batches in one kernel: per chunk the cumulative decay, the chunk state and
// the carried state, walking each sequence's chunks in order with the state
// held in registers, so no chunk state is written to memory and read back.
//
// Per (sequence, head) and its chunks c in order (s in log2 units, every
// exponent <= 0):
//   s_i    = log2(e) A_h sum_{k<=i} dt_k                       chunk-local
//   S_c^T  = sum_j x_j (2^(s_end - s_j) dt_j B_j)^T             P x N, MFMA over tokens
//   H_in_c = H                                                  stored for the chunk scan
//   H      = 2^(s_end) H + S_c                                  float32, in registers
// with H = h0 (or 0) before the first chunk and h_out = H after the last: the
// recurrence regrouped into fixed-length chunks (Compiler-First State Space
// Duality and Portable O(1) Autoregressive Caching for Inference, Abstract:
// one scalar decay per head, equal chunks whose work is dense contractions;
// float32 decay as in its Table 8), and the state handed from chunk to chunk
// as Recurrence Scan's schedule carries it from one launch to the next ("The
// schedule").  Also written for the chunk scan: s, dt and u_j = 2^(s_r - s_j)
// dt_j (r the last row of j's 32-row block), [chunk][head][Q].
//
// The chunk states do not depend on one another, only their sum does, so the
// walk's serial part is one multiply-add per state element per chunk; what a
// chain waits for is its loads.  A chain -- a (sequence, head), or a segment
// of its chunks -- is walked by one or two workgroups (each owning a share of
// the state's n columns) that stream its chunks with the next phase's loads in
// flight: the x rows go straight to LDS (block-swizzled, read transposed as
// the MFMA A operand), the B rows come from a copy of B already in MFMA
// fragment order (k_bfrag) straight into registers and are weighted there, so
// B, which every head of a group shares, is never staged per head.  Every
// wave computes the chunk's decay itself (a DPP scan over the wave), so no
// barrier waits for it; a wave owns one n-tile and the four p-tiles of the
// chain's P x N state.
//
// Segments: with enough room on the chip, each chain is walked in segments at
// once, each after the first from a zero state, and k_walk_fixup then adds
// the earlier segments' decayed contribution to their entering states and
// forms the final state (the recurrence is linear in the entering state).
// Some heads' chains in two segments fill the chip's slots; the rest, in
// shorter segments, fill the slots those free (SegPlan).  A packed batch,
// whose sequence lengths only the device knows, is walked by lists instead:
// every chunk of every chain in one order, cut into equal runs, one per
// resident workgroup (k_state_walk_list, k_walk_fixup_list).
#include <algorithm>

#include "ssd.h"
#include "ssd_launch.h"
#include "ssd_prefill_util.h"

namespace ssd {

// B in MFMA fragment order for the chunk-state product:
// out[chunk][group][Q/32][N/16][64 lanes][8] bf16.  Lane l of fragment (ks, nt)
// holds column n = 16 nt + l % 16 at tokens 32 ks + 4 (l / 16) + r (slots
// 0..3) and 32 ks + 16 + 4 (l / 16) + r (slots 4..7), r = 0..3 -- the paired
// token map of the x fragments read transposed from LDS -- and zero past the
// chunk's end.  One workgroup per (chunk, group, 32-token step): its 32 rows
// of B (8 KB) are read whole-row into LDS, then each wave forms two n-tiles'
// fragments with transposed LDS reads and writes them as whole 1 KB rows.
__global__ __launch_bounds__(256) void k_bfrag(const bf16 *__restrict__ B, ChunkMap cmap, int nc,
                                               int G, int Q, bf16 *__restrict__ out) {
  constexpr int N = 128, NTL = N / 16, PITCH = N + kTrPad;
  __shared__ __align__(16) bf16 rows[32 * PITCH];
  const int KS = Q / 32;
  const int u = blockIdx.x;  // (chunk, group, step), step fastest
  const int ks = u % KS, cg = u / KS;
  const int c = cg / G, g = cg - (cg / G) * G;
  if (c >= nc) return;
  const int4 ci = cmap(c);
  const int len = ci.z;
  if (len <= 0) return;
  const int tid = threadIdx.x;
  // 32 rows x 256 bytes: thread t moves 32 bytes of row t / 8 (zero past the chunk)
  {
    const int r = tid >> 3, q = (tid & 7) * 16;  // row, first column
    const int j = 32 * ks + r;
    i4v v0 = i4v{0, 0, 0, 0}, v1 = i4v{0, 0, 0, 0};
    if (j < len) {
      const i4v *src = reinterpret_cast<const i4v *>(B + ((size_t)ci.y + j) * G * N +
                                                     (size_t)g * N + q);
      v0 = src[0];
      v1 = src[1];
    }
    i4v *dst = reinterpret_cast<i4v *>(rows + r * PITCH + q);
    dst[0] = v0;
    dst[1] = v1;
  }
  __syncthreads();
  const int lane = tid & 63, grp = lane >> 4, wave = tid >> 6;
  bf16 *oc = out + (((size_t)c * G + g) * KS + ks) * (size_t)NTL * 512;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int nt = 2 * wave + k;
    const Frag<bf16> f = frag_kmaj(rows, PITCH, 16 * nt, 4 * grp, 16 + 4 * grp);
    *reinterpret_cast<bf16x8 *>(oc + (size_t)nt * 512 + lane * 8) = f.v;
  }
}

// Chunk c's map entry.  For a dense batch it is arithmetic only: a value
// loaded from memory here would make the compiler drain every outstanding
// memory operation (the previous chunk's stores included) before the loads it
// feeds could issue.
template <bool DENSE>
__device__ __forceinline__ int4 walk_map(const ChunkMap &m, int c) {
  if constexpr (DENSE) {
    const int cps = (m.L + m.Q - 1) / m.Q;
    const int seq = c / cps, k = c - seq * cps;
    return make_int4(seq, seq * m.L + k * m.Q, min(m.Q, m.L - k * m.Q), k);
  } else {
    return m(c);
  }
}

// How a walk cuts its chains into segments: the chains of heads below hsplit
// in nlo segments, those of the others in nhi (nlo = nhi = 1: whole chains).
// The first kind comes first in the launch order, the second fills the slots
// they free.
struct SegPlan {
  int nlo, nhi, hsplit;
  __host__ __device__ int nseg(int hd) const { return hd < hsplit ? nlo : nhi; }
  __host__ __device__ int maxseg() const { return nlo > nhi ? nlo : nhi; }
  __host__ __device__ long chains(int nseq, int H) const {
    return (long)nseq * (hsplit * nlo + (H - hsplit) * nhi);
  }
};

template <int Q, int NH, int JP_, int NW_> struct WalkCfg {
  static constexpr int P = 64, N = 128;
  static constexpr int NW = NW_;                // waves
  static constexpr int NT = N / 16 / NH;        // n-tiles of the chain's state block
  static constexpr int NTW = NT / NW;           // n-tiles per wave
  static constexpr int JP = JP_ < Q ? JP_ : Q;  // rows per phase
  static constexpr int NPH = Q / JP;            // phases per chunk
  static constexpr int KSP = JP / 32;           // token k-steps per phase
  static constexpr int XB = (JP / 8) * kBlk128;  // one phase's x tile
  static constexpr int DTN = Q < 64 ? 64 : Q;   // floats of a dt column buffer (whole-wave loads)
  static constexpr int OFF_DT = 2 * XB;
  static constexpr int OFF_W = OFF_DT + 2 * DTN * 4;  // a w row per wave
  // each wave's bf16 rows of the entering state, staged for whole-line stores
  // (row pitch padded by 16 bytes against bank conflicts)
  static constexpr int HST_PITCH = P * 2 + 16;
  static constexpr int HST_WAVE = NTW * 16 * HST_PITCH;
  static constexpr int OFF_HST = OFF_W + NW * DTN * 4;
  static constexpr int LDS = OFF_HST + NW * HST_WAVE;
  static_assert(NTW >= 1 && NT % NW == 0 && Q <= 256, "walk shape");
};

// One 4-byte-per-lane buffer load into LDS at lds_addr + 4 * lane, issued from
// inline assembly for the reason given at lds_load16 (the caller waits).
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr,
                                          uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr)
               : "memory");
}

// Inclusive prefix sum over the 64 lanes of a wave in registers: shifts of 1,
// 2, 4 and 8 lanes within each 16-lane row (lanes shifted in from outside the
// row add 0), then the last lane of row 0 and of row 2 added to rows 1 and 3
// (row broadcast 15) and that of row 1 to rows 2 and 3 (row broadcast 31).
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x111, 0xF, 0xF, true));  // row_shr:1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x112, 0xF, 0xF, true));  // row_shr:2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x114, 0xF, 0xF, true));  // row_shr:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x118, 0xF, 0xF, true));  // row_shr:8
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x142, 0xA, 0xF, false));  // row_bcast:15
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// The chunk's s, dt and u rows for the chunk scan, R consecutive rows per lane,
// held in registers from the decay until they are stored.
template <int Q> struct WalkRows {
  static constexpr int R = Q >= 64 ? Q / 64 : 1;
  float s[R], dt[R], u[R];
};

// The chunk's cumulative decay, computed by every wave from the chunk's dt
// column in LDS (rows past its length hold 0), R consecutive rows per lane:
// s = log2(e) A cumsum(dt), w_j = 2^(s_end - s_j) dt_j into the wave's own LDS
// row w_l (read back by the same wave only: no barrier), and s, dt and
// u_j = 2^(s_r - s_j) dt_j (r the last row of j's 32-row block) into `rows`.
// Returns s_end.
template <int Q>
__device__ __forceinline__ float walk_decay(const float *dt_l, float *w_l, float a2,
                                            WalkRows<Q> &rows) {
  constexpr int R = WalkRows<Q>::R;
  const int lane = threadIdx.x & 63;
  float run = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane * R + r;
    rows.dt[r] = i < Q ? dt_l[i] : 0.f;
    run += rows.dt[r] * a2;
    rows.s[r] = run;
  }
  const float incl = wave_incl_scan(run);
  const float excl = incl - run;
#pragma unroll
  for (int r = 0; r < R; ++r) rows.s[r] += excl;
  // row Q - 1 sits in slot R - 1 of lane (Q - 1) / R; the last row of a lane's
  // 32-row block in slot R - 1 of the block's last lane
  const float s_end = __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rows.s[R - 1]), (Q - 1) / R));
  const float s_ref = __shfl(rows.s[R - 1], lane | (32 / R - 1), 64);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane * R + r;
    if (i < Q) w_l[i] = __builtin_amdgcn_exp2f(fminf(s_end - rows.s[r], 0.f)) * rows.dt[r];
    rows.u[r] = __builtin_amdgcn_exp2f(fminf(s_ref - rows.s[r], 0.f)) * rows.dt[r];
  }
  return s_end;
}

template <int Q>
__device__ __forceinline__ void walk_store_rows(const WalkRows<Q> &rows, size_t off,
                                                float *__restrict__ s_out,
                                                float *__restrict__ dt_out,
                                                float *__restrict__ u_out) {
  constexpr int R = WalkRows<Q>::R;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane * R + r;
    if (i < Q) {
      s_out[off + i] = rows.s[r];
      dt_out[off + i] = rows.dt[r];
      u_out[off + i] = rows.u[r];
    }
  }
}

// The x rows of phase ph of chunk ci -> a block-swizzled LDS tile (rows past
// the chunk read 0).  The source address and length are made wave-uniform
// explicitly so the buffer descriptor stays in scalar registers.
template <typename K>
__device__ __forceinline__ void walk_issue_x(const bf16 *__restrict__ x, int4 ci, int ph,
                                             size_t xstride, int hd, uint32_t xl, char *tile,
                                             int wave) {
  const int t0 = __builtin_amdgcn_readfirstlane(ci.y), len = __builtin_amdgcn_readfirstlane(ci.z);
  const int r0 = ph * K::JP;
  const int vr = max(0, min(K::JP, len - r0));
  const uint32_t xsb = (uint32_t)(xstride * 2);
  const uint64_t xa =
      reinterpret_cast<uint64_t>(x + ((size_t)t0 + r0) * xstride + (size_t)hd * K::P);
  const uint64_t xu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xa) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(xa >> 32)) << 32);
  dma_swz<kBlk128>(tile, reinterpret_cast<const void *>(xu),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)vr * xsb)), xl,
                   8 * xsb, K::JP / 8, wave, K::NW);
}

// The dt column of chunk ci (rows past the chunk read 0) -> LDS at lds_addr.
template <typename K>
__device__ __forceinline__ void walk_issue_dt(const float *__restrict__ dt, int4 ci, int H, int hd,
                                              uint32_t lds_addr, int wave) {
  const int t0 = __builtin_amdgcn_readfirstlane(ci.y), len = __builtin_amdgcn_readfirstlane(ci.z);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(dt + (size_t)t0 * H + hd), (short)0, len > 0 ? (len - 1) * H * 4 + 4 : 0,
      0x00020000);
  const int lane = threadIdx.x & 63;
  for (int r = wave * 64; r < K::DTN; r += K::NW * 64)
    lds_load4(rs, lds_addr + r * 4, (uint32_t)(r + lane) * (uint32_t)H * 4);
}

// The B fragments of phase ph of a chunk (bc: the chunk's fragments at this
// wave's first n-tile and lane) for the wave's NTW n-tiles.
template <typename K>
__device__ __forceinline__ void walk_load_b(const bf16 *bc, int ph,
                                            bf16x8 (&bf)[K::NTW][K::KSP]) {
  constexpr int NTL = K::N / 16;
#pragma unroll
  for (int k = 0; k < K::KSP; ++k)
#pragma unroll
    for (int t = 0; t < K::NTW; ++t)
      bf[t][k] = *reinterpret_cast<const bf16x8 *>(
          bc + (size_t)((ph * K::KSP + k) * NTL + t) * 512);
}

template <int Q, int NH, int JP_, int NW_, bool DENSE, bool PREC>
__global__ __launch_bounds__(64 * NW_) void k_state_walk(
    const bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ bfr, const int *__restrict__ seq_off, ChunkMap cmap, int H, int G,
    int nchain, const float *h0, float *h_out, float *__restrict__ s_out,
    float *__restrict__ dt_out, float *__restrict__ u_out, bf16 *__restrict__ hin,
    float *__restrict__ hin32, float *h_out2, SegPlan sp, float *__restrict__ seg_end) {
  typedef WalkCfg<Q, NH, JP_, NW_> K;
  constexpr int P = K::P, N = K::N, NTW = K::NTW, NPT = P / 16, KSP = K::KSP, NPH = K::NPH;
  constexpr int NTL = N / 16, JP = K::JP;
  // chains in contiguous blocks per XCD (workgroup L runs on XCD L % 8), so the
  // chains of one sequence, which read the same B fragments, share an L2
  int part, hd, seg, s;
  const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
  if (sp.maxseg() == 1) {
    const int per = (nchain + 7) >> 3;
    const int chn = xcd * per + slot;
    if (chn >= nchain) return;
    // chain = (sequence, head, part), part fastest
    part = chn % NH;
    hd = (chn / NH) % H;
    seg = 0;
    s = chn / NH / H;
  } else {
    // segments (NH = 1): each XCD's block of first-kind chains, then its block
    // of second-kind ones; each kind ordered (sequence, segment, head)
    const int nseq = cmap.nseq, hs = sp.hsplit, hr = H - hs;
    const int nlong = nseq * hs * sp.nlo, nshort = nseq * hr * sp.nhi;
    const int lp = (nlong + 7) >> 3, spg = (nshort + 7) >> 3;
    part = 0;
    if (slot < lp) {
      const int i = xcd * lp + slot;
      if (i >= nlong) return;
      hd = i % hs;
      seg = (i / hs) % sp.nlo;
      s = i / hs / sp.nlo;
    } else {
      const int j = xcd * spg + (slot - lp);
      if (slot - lp >= spg || j >= nshort) return;
      hd = hs + j % hr;
      seg = (j / hr) % sp.nhi;
      s = j / hr / sp.nhi;
    }
  }
  hd = __builtin_amdgcn_readfirstlane(hd);
  seg = __builtin_amdgcn_readfirstlane(seg);
  s = __builtin_amdgcn_readfirstlane(s);
  const int nseg = sp.nseg(hd);
  int c0, c1;  // chunks of sequence s
  if constexpr (DENSE) {
    const int cps = (cmap.L + Q - 1) / Q;
    c0 = s * cps;
    c1 = c0 + cps;
  } else {
    c0 = __builtin_amdgcn_readfirstlane(seq_off[s]);
    c1 = __builtin_amdgcn_readfirstlane(seq_off[s + 1]);
  }
  {  // this chain's segment of them: segments after the first start from zero
    const int nchk = c1 - c0;
    const int a0 = c0 + (seg * nchk) / nseg, a1 = c0 + ((seg + 1) * nchk) / nseg;
    c0 = a0;
    c1 = a1;
  }
  const int g = (hd * G) / H;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  extern __shared__ __align__(16) char smem[];
  float *w_l = reinterpret_cast<float *>(smem + K::OFF_W) + wave * K::DTN;  // this wave's row
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)smem;

  // the chain's state block in the accumulator layout of S^T tiles: tile
  // (t, pt) of a lane holds H[n][p .. p+3], n = 16 (nt0 + t) + col, p = 16 pt + 4 grp
  const int nt0 = part * K::NT + wave * NTW;
  const size_t hofs = ((size_t)s * H + hd) * (size_t)(N * P);
  f4 Hs[NTW][NPT];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
      Hs[t][pt] = (h0 && seg == 0)
                      ? ld4(h0 + hofs + (size_t)(16 * (nt0 + t) + col) * P + 16 * pt + 4 * grp)
                      : zero4();

  const size_t xstride = (size_t)H * P;
  const int lb8 = lane >> 3;
  const uint32_t xl = lb8 * (uint32_t)(xstride * 2) + 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  // B fragments of this wave's n-tiles: chunk c's at bfw + c * bfc
  const bf16 *bfw = bfr + (size_t)g * ((Q / 32) * NTL) * 512 + (size_t)nt0 * 512 + lane * 8;
  const size_t bfc = (size_t)G * ((Q / 32) * NTL) * 512;
  // x fragment offsets (paired token map: rows k0 + 4 grp + col/4 and
  // k0 + 16 + 4 grp + col/4; p-tile pt by XOR with 32 pt)
  const int c4 = col >> 2, cq = 8 * (col & 3);
  const int xbk = 4 * (grp & 1) + c4;
  const int xo = (grp >> 1) * kBlk128 + xbk * 128 + cq + 32 * swz8(xbk);
  const float a2 = A[hd] * kLog2e;

  typedef bf16x8 BF[NTW][KSP];
  // B fragments of the current phase and of the next one, in alternating
  // register sets (phase ph computes from bq[ph & 1]), so none are copied
  // when a chunk has an even number of phases
  BF bq[2];
  int4 cn = make_int4(0, 0, 0, 0);  // the next chunk's map entry, read a chunk ahead
  if (c0 < c1) {
    const int4 ci = walk_map<DENSE>(cmap, c0);
    walk_issue_dt<K>(dt, ci, H, hd, lds0 + K::OFF_DT, wave);
    walk_issue_x<K>(x, ci, 0, xstride, hd, xl, smem, wave);
    walk_load_b<K>(bfw + (size_t)c0 * bfc, 0, bq[0]);
    if (c0 + 1 < c1) cn = walk_map<DENSE>(cmap, c0 + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int xbuf = 0;
  for (int c = c0; c < c1; ++c) {
    const int4 ci = walk_map<DENSE>(cmap, c);
    const int db = (c - c0) & 1;
    const int4 cnow = cn;  // chunk c + 1
    float s_end = 0.f;
    WalkRows<Q> rows;
    f4 S[NTW][NPT];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) S[t][pt] = zero4();
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      // the next phase's loads first (this chunk's next rows, or the next
      // chunk's first rows and its dt column), so nothing issued later in the
      // phase stands before them
      if (ph + 1 < NPH) {
        walk_issue_x<K>(x, ci, ph + 1, xstride, hd, xl, smem + (xbuf ^ 1) * K::XB, wave);
        walk_load_b<K>(bfw + (size_t)(c) * bfc, ph + 1, bq[(ph + 1) & 1]);
      } else if (c + 1 < c1) {
        walk_issue_x<K>(x, cnow, 0, xstride, hd, xl, smem + (xbuf ^ 1) * K::XB, wave);
        walk_issue_dt<K>(dt, cnow, H, hd, lds0 + K::OFF_DT + (db ^ 1) * K::DTN * 4, wave);
        walk_load_b<K>(bfw + (size_t)(c + 1) * bfc, 0, bq[(ph + 1) & 1]);
        if (c + 2 < c1) cn = walk_map<DENSE>(cmap, c + 2);
      }
      if (ph == 0) {
        // the chunk's decay, in every wave (wave 0 of part 0 writes s, dt, u)
        s_end = walk_decay<Q>(
            reinterpret_cast<const float *>(smem + K::OFF_DT + db * K::DTN * 4), w_l, a2, rows);
      }
      // S^T += sum over this phase's tokens of x_j (w_j B_j)^T
      const char *xt = smem + xbuf * K::XB;
#pragma unroll
      for (int k = 0; k < KSP; ++k) {
        const int j0 = ph * JP + 32 * k;
        Frag<bf16> xa[NPT];
        const char *xk = xt + 4 * k * kBlk128;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          xa[pt] = frag_kmaj_at(xk, xo ^ (32 * pt), (xo ^ (32 * pt)) + 2 * kBlk128);
        const f4 w0 = ld4(w_l + j0 + 4 * grp), w1 = ld4(w_l + j0 + 16 + 4 * grp);
        Frag<bf16> bw[NTW], bl[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const f8v bv = cvt_f8(bq[ph & 1][t][k]);
          const f8v wb = f8v{bv[0] * w0[0], bv[1] * w0[1], bv[2] * w0[2], bv[3] * w0[3],
                             bv[4] * w1[0], bv[5] * w1[1], bv[6] * w1[2], bv[7] * w1[3]};
          bw[t].v = cvt_bf8(wb);
          // PREC: also what the rounding dropped, as a second operand
          if constexpr (PREC) bl[t].v = cvt_bf8(wb - cvt_f8(bw[t].v));
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            mma(S[t][pt], xa[pt], bw[t]);
            if constexpr (PREC) mma(S[t][pt], xa[pt], bl[t]);
          }
      }
      // the next phase's loads have landed and this phase's buffers are free
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (ph == 0) {
        // the state entering chunk c, in the operand type, for the chunk scan:
        // stored after the wait, so that the stores complete under the next
        // phase's work instead of holding up this one's wait
        // The wave's rows 16 nt0 .. 16 (nt0 + NTW) - 1 of the N x P block are
        // contiguous; the accumulator layout gives each lane 8-byte pieces of
        // 16 rows, so the rows go through the wave's own LDS rows first and
        // leave as 16 bytes per lane, 8 whole 128-byte rows per store (one
        // wave writes and reads its rows: no barrier)
        const size_t hco = ((size_t)c * H + hd) * (size_t)(N * P);
        char *hst = smem + K::OFF_HST + wave * K::HST_WAVE;
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            *reinterpret_cast<bf16x4 *>(hst + (16 * t + col) * K::HST_PITCH + 32 * pt + 8 * grp) =
                __builtin_convertvector(Hs[t][pt], bf16x4);
            if (hin32)  // a training forward keeps them in float32 as well
              st4(hin32 + hco + (size_t)(16 * (nt0 + t) + col) * P + 16 * pt + 4 * grp, Hs[t][pt]);
          }
        bf16 *hrow = hin + hco + (size_t)(16 * nt0) * P;
#pragma unroll
        for (int k = 0; k < 2 * NTW; ++k) {
          const int r = 8 * k + (lane >> 3);
          *reinterpret_cast<bf16x8 *>(hrow + (size_t)r * P + 8 * (lane & 7)) =
              *reinterpret_cast<const bf16x8 *>(hst + r * K::HST_PITCH + 16 * (lane & 7));
        }
        // s, dt and u for the chunk scan, likewise after the wait (wave 0 of
        // part 0, from the registers the decay left them in: the chunk's dt
        // column in LDS may already be taking the next chunk's)
        if (part == 0 && wave == 0)
          walk_store_rows<Q>(rows, ((size_t)c * H + hd) * Q, s_out, dt_out, u_out);
      }
      if constexpr (NPH % 2 == 1) {  // the next chunk's first phase starts from bq[0]
        if (ph == NPH - 1) {
#pragma unroll
          for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int k = 0; k < KSP; ++k) bq[0][t][k] = bq[1][t][k];
        }
      }
      xbuf ^= 1;
    }
    // carry: H = 2^(s_end) H + S
    const float a = __builtin_amdgcn_exp2f(fminf(s_end, 0.f));
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
        for (int q = 0; q < 4; ++q) Hs[t][pt][q] = a * Hs[t][pt][q] + S[t][pt][q];
  }
  // the state leaving the chain: the final state, or with several segments the
  // segment's own end state (from its own entering state) for k_walk_fixup
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      const size_t e = (size_t)(16 * (nt0 + t) + col) * P + 16 * pt + 4 * grp;
      if (sp.maxseg() > 1) {
        st4(seg_end + (((size_t)s * H + hd) * sp.maxseg() + seg) * (size_t)(N * P) + e,
            Hs[t][pt]);
      } else {
        if (h_out) st4(h_out + hofs + e, Hs[t][pt]);
        if (h_out2) st4(h_out2 + hofs + e, Hs[t][pt]);
      }
    }
}

// ------------------------------------------------------------------ walk by lists
// The walk of a packed batch, whose sequences' chunk counts differ and are
// known on the device only: the work cut evenly over the workgroups the chip
// holds at once.  The chunks of all chains in one order (sequence by
// sequence, head by head, each chain's chunks in order), position f = (the
// chain's first position) + k, and workgroup l walks positions
// [l W, (l + 1) W).  Where its run begins inside a chain it starts from a zero
// state; where a piece of a run ends (its chain's end or the run's) it leaves
// the piece's state at seg_end[the piece's first position], and
// k_walk_fixup_list then adds each piece's share of the pieces before it (the
// recurrence is linear in the entering state).  Whole chains would leave the
// longest sequence's chains running alone long after the rest; here every
// workgroup has the same number of chunks.  (A dense batch's chains are cut
// at the same chunk in every head instead -- SegPlan -- which keeps the
// heads' chunk positions aligned and reads x rows and B fragments together.)

struct WalkPos {
  int s, hd, k, nchk, cs;  // sequence, head, chunk in the chain, chunks in it, first chunk
  int t0, t1;              // the sequence's tokens t0 .. t1 - 1
};

// The chain and chunk at position f (f below the total count): the last
// sequence whose positions start at or before f (an empty sequence shares its
// start with the next one, so it is never the last), then head and chunk.
__device__ __forceinline__ WalkPos walk_locate(int f, const int *__restrict__ seq_off,
                                               const int *__restrict__ cu, int H, int nseq) {
  WalkPos w;
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (H * seq_off[mid] <= f) lo = mid;
    else hi = mid - 1;
  }
  w.s = lo;
  w.cs = seq_off[lo];
  w.nchk = seq_off[lo + 1] - w.cs;
  const int r = f - H * w.cs;
  w.hd = r / w.nchk;
  w.k = r - w.hd * w.nchk;
  w.s = __builtin_amdgcn_readfirstlane(w.s);
  w.hd = __builtin_amdgcn_readfirstlane(w.hd);
  w.k = __builtin_amdgcn_readfirstlane(w.k);
  w.nchk = __builtin_amdgcn_readfirstlane(w.nchk);
  w.cs = __builtin_amdgcn_readfirstlane(w.cs);
  w.t0 = __builtin_amdgcn_readfirstlane(cu[w.s]);
  w.t1 = __builtin_amdgcn_readfirstlane(cu[w.s + 1]);
  return w;
}

// The chunk-map entry {sequence, first token, length, chunk in the sequence}
// of a position, by arithmetic (a map entry loaded inside the walk's loop
// would be waited for with nothing else in flight: a round trip per chunk).
template <int Q> __device__ __forceinline__ int4 walk_entry(const WalkPos &p) {
  const int t = p.t0 + p.k * Q;
  return make_int4(p.s, t, min(Q, p.t1 - t), p.k);
}

template <int Q, int JP_, int NW_>
__global__ __launch_bounds__(64 * NW_) void k_state_walk_list(
    const bf16 *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ bfr, const int *__restrict__ seq_off, const int *__restrict__ cu,
    int H, int G, int nseq, int F, int W, int nlist, const float *__restrict__ h0,
    float *__restrict__ s_out, float *__restrict__ dt_out, float *__restrict__ u_out,
    bf16 *__restrict__ hin, float *__restrict__ seg_end) {
  typedef WalkCfg<Q, 1, JP_, NW_> K;
  constexpr int P = K::P, N = K::N, NTW = K::NTW, NPT = P / 16, KSP = K::KSP, NPH = K::NPH;
  constexpr int NTL = N / 16, JP = K::JP;
  // runs in contiguous blocks per XCD (workgroup L runs on XCD L % 8), so the
  // runs of one sequence, which read the same B fragments, share an L2
  const int per = (nlist + 7) >> 3;
  const int li = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (li >= nlist) return;
  const int Fr = min(F, H * __builtin_amdgcn_readfirstlane(seq_off[nseq]));
  const int f0 = li * W, f1 = min(Fr, f0 + W);
  if (f0 >= f1) return;
  const int lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  extern __shared__ __align__(16) char smem[];
  float *w_l = reinterpret_cast<float *>(smem + K::OFF_W) + wave * K::DTN;  // this wave's row
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)smem;
  const int nt0 = wave * NTW;
  const size_t xstride = (size_t)H * P;
  const int lb8 = lane >> 3;
  const uint32_t xl = lb8 * (uint32_t)(xstride * 2) + 16 * ((lane & 7) ^ (2 * swz8(lb8)));
  const size_t bfc = (size_t)G * ((Q / 32) * NTL) * 512;
  auto bfw_of = [&](int hd) {  // the B fragments of head hd's group, this wave's n-tiles
    return bfr + (size_t)((hd * G) / H) * ((Q / 32) * NTL) * 512 + (size_t)nt0 * 512 + lane * 8;
  };
  const int c4 = col >> 2, cq = 8 * (col & 3);
  const int xbk = 4 * (grp & 1) + c4;
  const int xo = (grp >> 1) * kBlk128 + xbk * 128 + cq + 32 * swz8(xbk);

  WalkPos cur = walk_locate(f0, seq_off, cu, H, nseq);
  const bf16 *bfw = bfw_of(cur.hd);
  float a2 = A[cur.hd] * kLog2e;
  f4 Hs[NTW][NPT];
  auto reset_state = [&]() {  // a chain's first chunk: h0; a piece after a run's start: zero
    const size_t hofs = ((size_t)cur.s * H + cur.hd) * (size_t)(N * P);
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
        Hs[t][pt] = (h0 && cur.k == 0)
                        ? ld4(h0 + hofs + (size_t)(16 * (nt0 + t) + col) * P + 16 * pt + 4 * grp)
                        : zero4();
  };
  reset_state();
  int fp = f0;  // the current piece's first position

  typedef bf16x8 BF[NTW][KSP];
  BF bq[2];
  {
    const int4 ci = walk_entry<Q>(cur);
    walk_issue_dt<K>(dt, ci, H, cur.hd, lds0 + K::OFF_DT, wave);
    walk_issue_x<K>(x, ci, 0, xstride, cur.hd, xl, smem, wave);
    walk_load_b<K>(bfw + (size_t)(cur.cs + cur.k) * bfc, 0, bq[0]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int xbuf = 0;
  for (int f = f0; f < f1; ++f) {
    const int c = cur.cs + cur.k;
    const int4 ci = walk_entry<Q>(cur);
    const int db = (f - f0) & 1;
    const bool more = f + 1 < f1;
    // the next position: this chain's next chunk, the next head's first, or
    // (searched for, once per sequence) the next sequence's
    WalkPos nx = cur;
    if (more) {
      if (cur.k + 1 < cur.nchk) {
        nx.k = cur.k + 1;
      } else if (cur.hd + 1 < H) {
        nx.hd = cur.hd + 1;
        nx.k = 0;
      } else {
        nx = walk_locate(f + 1, seq_off, cu, H, nseq);
      }
    }
    const int cnx = nx.cs + nx.k;
    const int4 cin = walk_entry<Q>(nx);
    const bf16 *bfn = nx.hd == cur.hd ? bfw : bfw_of(nx.hd);
    float s_end = 0.f;
    WalkRows<Q> rows;
    f4 S[NTW][NPT];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) S[t][pt] = zero4();
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      // the next phase's loads first (this chunk's next rows, or the next
      // position's first rows and its dt column)
      if (ph + 1 < NPH) {
        walk_issue_x<K>(x, ci, ph + 1, xstride, cur.hd, xl, smem + (xbuf ^ 1) * K::XB, wave);
        walk_load_b<K>(bfw + (size_t)c * bfc, ph + 1, bq[(ph + 1) & 1]);
      } else if (more) {
        walk_issue_x<K>(x, cin, 0, xstride, nx.hd, xl, smem + (xbuf ^ 1) * K::XB, wave);
        walk_issue_dt<K>(dt, cin, H, nx.hd, lds0 + K::OFF_DT + (db ^ 1) * K::DTN * 4, wave);
        walk_load_b<K>(bfn + (size_t)cnx * bfc, 0, bq[(ph + 1) & 1]);
      }
      if (ph == 0)
        s_end = walk_decay<Q>(
            reinterpret_cast<const float *>(smem + K::OFF_DT + db * K::DTN * 4), w_l, a2, rows);
      // S^T += sum over this phase's tokens of x_j (w_j B_j)^T
      const char *xt = smem + xbuf * K::XB;
#pragma unroll
      for (int kk = 0; kk < KSP; ++kk) {
        const int j0 = ph * JP + 32 * kk;
        Frag<bf16> xa[NPT];
        const char *xk = xt + 4 * kk * kBlk128;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          xa[pt] = frag_kmaj_at(xk, xo ^ (32 * pt), (xo ^ (32 * pt)) + 2 * kBlk128);
        const f4 w0 = ld4(w_l + j0 + 4 * grp), w1 = ld4(w_l + j0 + 16 + 4 * grp);
        Frag<bf16> bw[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const f8v bv = cvt_f8(bq[ph & 1][t][kk]);
          bw[t].v = cvt_bf8(f8v{bv[0] * w0[0], bv[1] * w0[1], bv[2] * w0[2], bv[3] * w0[3],
                                bv[4] * w1[0], bv[5] * w1[1], bv[6] * w1[2], bv[7] * w1[3]});
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
          for (int t = 0; t < NTW; ++t) mma(S[t][pt], xa[pt], bw[t]);
      }
      // the next phase's loads have landed and this phase's buffers are free
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (ph == 0) {
        // the state entering chunk c (from the piece's start), staged per wave
        // for whole-row stores as in k_state_walk, and the s, dt, u rows
        const size_t hco = ((size_t)c * H + cur.hd) * (size_t)(N * P);
        char *hst = smem + K::OFF_HST + wave * K::HST_WAVE;
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt)
            *reinterpret_cast<bf16x4 *>(hst + (16 * t + col) * K::HST_PITCH + 32 * pt + 8 * grp) =
                __builtin_convertvector(Hs[t][pt], bf16x4);
        bf16 *hrow = hin + hco + (size_t)(16 * nt0) * P;
#pragma unroll
        for (int kk = 0; kk < 2 * NTW; ++kk) {
          const int r = 8 * kk + (lane >> 3);
          *reinterpret_cast<bf16x8 *>(hrow + (size_t)r * P + 8 * (lane & 7)) =
              *reinterpret_cast<const bf16x8 *>(hst + r * K::HST_PITCH + 16 * (lane & 7));
        }
        if (wave == 0) walk_store_rows<Q>(rows, ((size_t)c * H + cur.hd) * Q, s_out, dt_out, u_out);
      }
      if constexpr (NPH % 2 == 1) {  // the next chunk's first phase starts from bq[0]
        if (ph == NPH - 1) {
#pragma unroll
          for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int kk = 0; kk < KSP; ++kk) bq[0][t][kk] = bq[1][t][kk];
        }
      }
      xbuf ^= 1;
    }
    // carry: H = 2^(s_end) H + S
    const float a = __builtin_amdgcn_exp2f(fminf(s_end, 0.f));
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
        for (int q = 0; q < 4; ++q) Hs[t][pt][q] = a * Hs[t][pt][q] + S[t][pt][q];
    // the piece ends at its chain's last chunk or at the run's end: its state
    // goes to seg_end at the piece's first position
    if (!more || nx.k == 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          st4(seg_end + (size_t)fp * (N * P) + (size_t)(16 * (nt0 + t) + col) * P + 16 * pt +
                  4 * grp,
              Hs[t][pt]);
    }
    if (more) {
      if (nx.k == 0) {  // the next chain
        cur = nx;
        bfw = bfn;
        a2 = A[cur.hd] * kLog2e;
        reset_state();
        fp = f + 1;
      } else {
        cur.k = nx.k;
      }
    }
  }
}

// The entering states and the final state of walks by lists: per (sequence,
// head), E = the state leaving the chain's first piece (walked from h0); for
// each later piece (it starts at a run boundary, a multiple of W) the stored
// entering states of its chunks get (decay since the piece's start) E added,
// and E = (the piece's decay) E + the piece's own end state.  The last E is
// the final state.  The corrected entering states are rounded to bf16 again.
__global__ __launch_bounds__(256) void k_walk_fixup_list(
    const float *__restrict__ s_ws, const int *__restrict__ seq_off, int H, int NP, int Q, int W,
    const float *__restrict__ seg_end, const float *__restrict__ h0, bf16 *__restrict__ hin,
    float *h_out, float *h_out2) {
  const int s = blockIdx.z, hd = blockIdx.y;
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= NP) return;
  const int cs = seq_off[s], nchk = seq_off[s + 1] - cs;
  const int cf0 = H * cs + hd * nchk;  // the chain's first position
  const size_t hofs = ((size_t)s * H + hd) * (size_t)NP + e;
  f4 E;
  if (nchk == 0) {  // an empty sequence keeps its state
    E = h0 ? ld4(h0 + hofs) : zero4();
  } else {
    E = ld4(seg_end + (size_t)cf0 * NP + e);
    for (int b = (cf0 / W + 1) * W; b < cf0 + nchk; b += W) {
      const int b1 = min(b + W, cf0 + nchk);
      float dec = 1.f;  // 2^(sum of s_end over the piece's chunks so far)
      for (int f = b; f < b1; ++f) {
        const size_t ch = (size_t)(cs + f - cf0) * H + hd;
        bf16 *hp = hin + ch * (size_t)NP + e;
        const f4 hv = ld4f(hp);
        st4T(hp, hv + dec * E);
        dec *= __builtin_amdgcn_exp2f(fminf(s_ws[ch * Q + Q - 1], 0.f));
      }
      E = dec * E + ld4(seg_end + (size_t)b * NP + e);
    }
  }
  if (h_out) st4(h_out + hofs, E);
  if (h_out2) st4(h_out2 + hofs, E);
}

// The entering states of a sequence whose chains were walked in segments
// (the counts per head as the plan says), each after the first walked from a
// zero state: the recurrence is linear in the entering
// state, so segment k's true entering states are those walked plus
// (product of the decays of its chunks so far) E_k, with E_1 = the first
// segment's end state (walked from h0) and E_(k+1) = (segment k's total decay)
// E_k + segment k's own end state.  One thread per 4 state elements of a
// (sequence, head), walking the segments and their chunks in order; the last
// E is the final state.  The corrected H_in is rounded to bf16 again.
__global__ __launch_bounds__(256) void k_walk_fixup(const float *__restrict__ s_ws,
                                                    const int *__restrict__ seq_off, ChunkMap cmap,
                                                    int H, int NP, int Q, SegPlan sp,
                                                    const float *__restrict__ seg_end,
                                                    bf16 *__restrict__ hin, float *h_out,
                                                    float *h_out2) {
  const int s = blockIdx.z, hd = blockIdx.y;
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (e >= NP) return;
  int c0, c1;
  if (cmap.L > 0) {
    const int cps = (cmap.L + Q - 1) / Q;
    c0 = s * cps;
    c1 = c0 + cps;
  } else {
    c0 = seq_off[s];
    c1 = seq_off[s + 1];
  }
  const int nchk = c1 - c0;
  const int nseg = sp.nseg(hd);
  const size_t sb = ((size_t)s * H + hd) * sp.maxseg();  // the chain's segment end states
  f4 E = ld4(seg_end + sb * NP + e);  // segment 0, from h0
  for (int k = 1; k < nseg; ++k) {
    const int a0 = c0 + (k * nchk) / nseg, a1 = c0 + ((k + 1) * nchk) / nseg;
    float dec = 1.f;  // 2^(sum of s_end over the segment's chunks so far)
    for (int c = a0; c < a1; ++c) {
      const size_t ch = (size_t)c * H + hd;
      bf16 *hp = hin + ch * (size_t)NP + e;
      const f4 hv = ld4f(hp);
      st4T(hp, hv + dec * E);
      dec *= __builtin_amdgcn_exp2f(fminf(s_ws[ch * Q + Q - 1], 0.f));
    }
    const f4 own = ld4(seg_end + (sb + k) * NP + e);
    E = dec * E + own;
  }
  const size_t hofs = ((size_t)s * H + hd) * (size_t)NP + e;
  if (h_out) st4(h_out + hofs, E);
  if (h_out2) st4(h_out2 + hofs, E);
}

// ------------------------------------------------------------------ launch
bool walk_supported(int P, int N, int Q, bool bf16) {
  return bf16 && P == 64 && N == 128 && Q >= 32 && Q <= 256;
}

// The walk pays when there are enough chains to fill the chip (a packed batch
// walks by lists, which even out its sequences' lengths).  A packed batch's
// training forward keeps the chunk states: the list walk keeps no float32
// entering states; nor do the lists take 2^30 or more (chunk, head)
// positions (32-bit position arithmetic).  The variant bits force either way.
bool walk_choice(int P, int N, int Q, bool bf16, int nseq, int H, int64_t nc, bool packed,
                 unsigned variant, bool training) {
  if (!walk_supported(P, N, Q, bf16) || (variant & SSD_VARIANT_STATE_CHUNKS)) return false;
  if (variant & SSD_VARIANT_STATE_WALK) return true;
  if (packed && training) return false;
  if (packed && (int64_t)H * nc >= (int64_t(1) << 30)) return false;
  return (long)nseq * H >= kWalkMinChains;
}

// Launch shape (compile-time constants): NH workgroups of NW waves per chain
// walked whole (each owns N/NH of the state's n columns), JP rows per pipeline
// phase; one workgroup of SEG_NW waves and SEG_JP-row phases per chain segment.
#ifndef SSD_WALK_NH
#define SSD_WALK_NH 2
#endif
#ifndef SSD_WALK_JP
#define SSD_WALK_JP 128
#endif
#ifndef SSD_WALK_NW
#define SSD_WALK_NW 4
#endif

template <int Q, int NH, int JP, int NW>
static hipError_t run_walk(const PrefillArgs &a, const WorkspaceLayout &L, bool write_hout,
                           SegPlan plan, hipStream_t st) {
  typedef WalkCfg<Q, NH, JP, NW> K;
  const void *kern =
      a.precise_states
          ? (a.cu ? (const void *)k_state_walk<Q, NH, JP, NW, false, true>
                  : (const void *)k_state_walk<Q, NH, JP, NW, true, true>)
          : (a.cu ? (const void *)k_state_walk<Q, NH, JP, NW, false, false>
                  : (const void *)k_state_walk<Q, NH, JP, NW, true, false>);
  hipError_t e = set_lds_limit(kern);
  if (e != hipSuccess) return e;
  char *ws = static_cast<char *>(a.workspace);
  const bf16 *xp = (const bf16 *)a.x;
  const float *dtp = a.dt, *Ap = a.A;
  const bf16 *bp = reinterpret_cast<const bf16 *>(ws + L.bfrag);
  const int *so = reinterpret_cast<const int *>(ws + L.seq_off);
  ChunkMap cm{reinterpret_cast<const int4 *>(ws + L.info), a.cu ? 0 : (int)(a.T / a.nseq), a.nseq,
              a.Q};
  int H_ = a.H, G_ = a.G, nch = a.nseq * a.H * NH;
  SegPlan sp_ = plan;
  float *se = reinterpret_cast<float *>(ws + L.segend);
  const float *h0p = a.h0;
  float *hop = write_hout ? a.h_out : nullptr, *hop2 = write_hout ? a.h_out2 : nullptr;
  float *sp = reinterpret_cast<float *>(ws + L.s), *dp = reinterpret_cast<float *>(ws + L.dt);
  float *up = reinterpret_cast<float *>(ws + L.u);
  bf16 *hp = reinterpret_cast<bf16 *>(ws + L.hin);
  float *h32 = a.hin32;
  void *args[] = {&xp, &dtp, &Ap, &bp, &so, &cm, &H_, &G_, &nch, &h0p, &hop, &sp, &dp, &up, &hp,
                  &h32, &hop2, &sp_, &se};
  unsigned grid = 8u * (unsigned)((nch + 7) / 8);
  if (plan.maxseg() > 1) {  // each XCD's block of each kind of chain
    const long nlong = (long)a.nseq * plan.hsplit * plan.nlo;
    const long nshort = (long)a.nseq * (a.H - plan.hsplit) * plan.nhi;
    grid = 8u * (unsigned)((nlong + 7) / 8 + (nshort + 7) / 8);
  }
  return hipLaunchKernel(kern, dim3(grid), dim3(64 * K::NW), args, K::LDS, st);
}

// How the chains are cut (see SegPlan).  Whole chains for a training forward
// (its float32 entering states would need the fix-up too), for sequences of
// fewer than 8 chunks on average, and when twice the chains would exceed three
// per compute unit.  Otherwise the heads' chains in two segments while those
// fill the slots the chip holds at once (`slots` workgroups of the segment
// walk), and the remaining heads' chains in more, shorter segments, so that
// they fill the slots the first free instead of leaving a tail of long chains
// running alone: as many second-kind segments as half the slots (the slots
// free at different times; one each for every slot measured 3.5 µs slower at
// the 2.7B layer), each of at least two chunks.
static SegPlan walk_seg_plan(int nseq, int H, int64_t T, int Q, int nc, bool packed,
                             bool training, long slots) {
  const SegPlan whole{1, 1, H};
  if (training || nseq <= 0) return whole;
  if (2L * nseq * H > 3L * 256) return whole;
  const int64_t cps = packed ? nc / nseq : (T / nseq + Q - 1) / Q;
  if (cps < 8) return whole;
  const long hs = slots / (2L * nseq);
  if (hs <= 0 || hs >= H) return SegPlan{2, 2, H};
  const long hr = H - hs;
  long nhi = (slots / 2 + nseq * hr / 2) / (nseq * hr);
  nhi = std::max(2L, std::min<long>(nhi, cps / 2));
  return SegPlan{2, (int)nhi, (int)hs};
}

#ifndef SSD_WALK_SEG_NW
#define SSD_WALK_SEG_NW 8
#endif
#ifndef SSD_WALK_SEG_JP
#define SSD_WALK_SEG_JP 128
#endif

// Workgroups of the segment walk's instance the chip holds at once.
template <int Q> static long walk_seg_slots(bool dense) {
  typedef WalkCfg<Q, 1, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW> K;
  const void *kern =
      dense ? (const void *)k_state_walk<Q, 1, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW, true, false>
            : (const void *)k_state_walk<Q, 1, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW, false, false>;
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      set_lds_limit(kern) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * K::NW, K::LDS) !=
          hipSuccess)
    return 2L * 256;  // the instance's two per CU on 256 CUs
  return (long)std::max(1, ncu) * std::max(1, per_cu);
}

template <int Q>
static hipError_t run_walk_q(const PrefillArgs &a, const WorkspaceLayout &L, int nc,
                             bool write_hout, SegPlan *used, hipStream_t st) {
  const SegPlan sp = walk_seg_plan(a.nseq, a.H, a.T, a.Q, nc, a.cu != nullptr,
                                   a.hin32 != nullptr, walk_seg_slots<Q>(a.cu == nullptr));
  *used = sp;
  if (sp.maxseg() > 1)
    return run_walk<Q, 1, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW>(a, L, write_hout, sp, st);
  return run_walk<Q, SSD_WALK_NH, SSD_WALK_JP, SSD_WALK_NW>(a, L, write_hout, sp, st);
}

// The walk by lists of a packed batch: as many runs as the chip holds
// workgroups of the list kernel at once (at least 8 chunks a run), then the
// fix-up.
template <int Q>
static hipError_t run_walk_list(const PrefillArgs &a, const WorkspaceLayout &L, int nc,
                                bool write_hout, hipStream_t st) {
  typedef WalkCfg<Q, 1, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW> K;
  const void *kern = (const void *)k_state_walk_list<Q, SSD_WALK_SEG_JP, SSD_WALK_SEG_NW>;
  hipError_t e = set_lds_limit(kern);
  if (e != hipSuccess) return e;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * K::NW, K::LDS)) !=
      hipSuccess)
    return e;
  const int slots = std::max(1, ncu * std::max(1, per_cu));
  // positions: every chunk of every head (a packed batch: an upper bound, the
  // kernel takes the exact count from the chunk offsets)
  const long F = (long)a.H * nc;
  if (F <= 0 || F >= (1L << 31) / 2) return hipErrorInvalidValue;
  const int W = (int)std::max<long>(8, (F + slots - 1) / slots);
  const int nlist = (int)((F + W - 1) / W);
  char *ws = static_cast<char *>(a.workspace);
  const bf16 *xp = (const bf16 *)a.x;
  const float *dtp = a.dt, *Ap = a.A;
  const bf16 *bp = reinterpret_cast<const bf16 *>(ws + L.bfrag);
  const int *so = reinterpret_cast<const int *>(ws + L.seq_off);
  const int *cup = a.cu;
  int H_ = a.H, G_ = a.G, nseq_ = a.nseq, F_ = (int)F, W_ = W, nl_ = nlist;
  const float *h0p = a.h0;
  float *sp = reinterpret_cast<float *>(ws + L.s), *dp = reinterpret_cast<float *>(ws + L.dt);
  float *up = reinterpret_cast<float *>(ws + L.u);
  bf16 *hp = reinterpret_cast<bf16 *>(ws + L.hin);
  float *se = reinterpret_cast<float *>(ws + L.segend);
  void *args[] = {&xp, &dtp, &Ap, &bp, &so, &cup, &H_, &G_, &nseq_, &F_, &W_, &nl_, &h0p,
                  &sp, &dp, &up, &hp, &se};
  e = hipLaunchKernel(kern, dim3(8u * (unsigned)((nlist + 7) / 8)), dim3(64 * K::NW), args, K::LDS,
                      st);
  if (e != hipSuccess) return e;
  const int NP = K::N * K::P;
  hipLaunchKernelGGL(k_walk_fixup_list, dim3((NP + 1023) / 1024, a.H, a.nseq), dim3(256), 0, st,
                     (const float *)sp, so, a.H, NP, a.Q, W, (const float *)se, a.h0, hp,
                     write_hout ? a.h_out : nullptr, write_hout ? a.h_out2 : nullptr);
  return hipGetLastError();
}

hipError_t launch_state_walk(const PrefillArgs &a, const WorkspaceLayout &L, int nc,
                             bool write_hout, hipStream_t st) {
  char *ws = static_cast<char *>(a.workspace);
  const ChunkMap cm{reinterpret_cast<const int4 *>(ws + L.info), a.cu ? 0 : (int)(a.T / a.nseq),
                    a.nseq, a.Q};
  if (nc > 0) {
    hipLaunchKernelGGL(k_bfrag, dim3((unsigned)nc * a.G * (a.Q / 32)), dim3(256), 0, st,
                       (const bf16 *)a.B, cm, nc, a.G, a.Q, reinterpret_cast<bf16 *>(ws + L.bfrag));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.cu != nullptr && a.hin32 == nullptr && nc > 0) {  // a packed batch, not training
    switch (a.Q) {
      case 32: return run_walk_list<32>(a, L, nc, write_hout, st);
      case 64: return run_walk_list<64>(a, L, nc, write_hout, st);
      case 128: return run_walk_list<128>(a, L, nc, write_hout, st);
      case 256: return run_walk_list<256>(a, L, nc, write_hout, st);
    }
    return hipErrorInvalidValue;
  }
  SegPlan sp{1, 1, a.H};
  hipError_t e = hipErrorInvalidValue;
  switch (a.Q) {
    case 32: e = run_walk_q<32>(a, L, nc, write_hout, &sp, st); break;
    case 64: e = run_walk_q<64>(a, L, nc, write_hout, &sp, st); break;
    case 128: e = run_walk_q<128>(a, L, nc, write_hout, &sp, st); break;
    case 256: e = run_walk_q<256>(a, L, nc, write_hout, &sp, st); break;
  }
  if (e != hipSuccess || sp.maxseg() == 1) return e;
  const int NP = 128 * 64;
  hipLaunchKernelGGL(k_walk_fixup, dim3((NP + 1023) / 1024, a.H, a.nseq), dim3(256), 0, st,
                     reinterpret_cast<const float *>(ws + L.s),
                     reinterpret_cast<const int *>(ws + L.seq_off), cm, a.H, NP, a.Q, sp,
                     reinterpret_cast<const float *>(ws + L.segend),
                     reinterpret_cast<bf16 *>(ws + L.hin), write_hout ? a.h_out : nullptr,
                     write_hout ? a.h_out2 : nullptr);
  return hipGetLastError();
}

}  // namespace ssd
