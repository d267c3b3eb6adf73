// ssd_prefill_util.h -- helpers shared by the prefill kernels: decay units,
// LDS padding, the XCD-aware chunk order and direct global->LDS tile loads.
#pragma once
#include <mutex>
#include <set>
#include <utility>

#include "ssd_device.h"

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;

// LDS row padding.  Tiles read with the 16-lane transpose read (4 rows x 32
// bytes per lane group) use a pitch of width + 16 elements, i.e. 32 bytes (bf16)
// or 64 bytes (float) past a multiple of 128 bytes, so the rows of one
// read land on disjoint banks.  Tiles read 16 bytes per lane along a row use
// width + 16 bytes (8 consecutive rows of a lane octet then cover every bank).
constexpr int kTrPad = 16;
template <typename T> constexpr int row_pad() { return 16 / (int)sizeof(T); }

// XCD-aware (chunk, head) order for a 1-D grid of 8 * H * ceil(nc / 8)
// workgroups.  Workgroup L is dispatched to XCD L % 8; decoding
// c = 8 (q / H) + L % 8, h = q % H with q = L / 8 puts every head of chunk c on
// the same XCD, back to back, so the chunk's B (and C) rows are fetched from
// HBM once and then hit that XCD's L2 for the other heads.
struct ChunkHead {
  int c, h;
};
__device__ __forceinline__ ChunkHead xcd_chunk_head(int H) {
  const int L = blockIdx.x, q = L >> 3;
  return ChunkHead{8 * (q / H) + (L & 7), q % H};
}
static inline unsigned xcd_grid(int nc, int H) { return 8u * (unsigned)H * (unsigned)((nc + 7) / 8); }

// Chunk c of the packed batch -> {sequence, first token, length, index in
// sequence}.  A dense batch (L tokens per sequence) is pure arithmetic, so a
// workgroup needs no memory round trip before its first load; a packed batch
// reads the table written by the cumulative-sum stage.
struct ChunkMap {
  const int4 *table;  // used when L == 0
  int L, nseq, Q;
  __device__ __forceinline__ int4 operator()(int c) const {
    if (L > 0) {
      const int cps = (L + Q - 1) / Q;
      const int seq = c / cps, k = c - seq * cps;
      if (seq >= nseq) return make_int4(0, 0, 0, 0);
      return make_int4(seq, seq * L + k * Q, min(Q, L - k * Q), k);
    }
    return table[c];
  }
};

// zero source for padding slots (one copy per translation unit)
static __device__ __attribute__((aligned(16))) unsigned int g_zero16[4];

// Fill a padded LDS tile of `rows` rows: each row has DATA 16-byte vectors
// from `src` (row r at src + r * stride) followed by pad vectors up to SPR
// slots; rows at or beyond `valid` are zero.  The tile spans a whole number
// of 64-slot wave requests (the caller sizes it with tile_slots()).
template <typename T, int SPR, int DATA>
__device__ __forceinline__ void dma_tile(T *tile, const T *__restrict__ src, size_t stride,
                                         int rows, int valid, int wave, int nw) {
  constexpr int VN = 16 / sizeof(T);
  const int total = rows * SPR;
  const int lane = threadIdx.x & 63;
  // slot s = base + lane sits at row r = s / SPR, vector v = s % SPR; both are
  // advanced by the wave-uniform step instead of divided again per request
  const int step = nw * 64;
  const int dr = step / SPR, dv = step - dr * SPR;
  const int s0 = wave * 64 + lane;
  int r = s0 / SPR, v = s0 - r * SPR;
  const int lim = min(valid, rows);  // slots past the tile end have r >= rows
  const T *zero = reinterpret_cast<const T *>(g_zero16);
  for (int base = wave * 64; base < total; base += step) {
    const T *g = (r < lim && v < DATA) ? src + (size_t)r * stride + v * VN : zero;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)(tile + base * VN),
                                     16, 0, 0);
    v += dv;
    r += dr;
    if (v >= SPR) {
      v -= SPR;
      ++r;
    }
  }
}
__host__ __device__ constexpr int tile_slots(int rows, int spr) { return (rows * spr + 63) / 64 * 64; }

// Block-swizzled bf16 tiles.  A tile of 128- or 256-byte rows is held as
// 1 KB blocks (8 or 4 rows: one direct-load request each) at a pitch of
// kBlk128 = 1152 or kBlk256 = 1088 bytes.  Inside a block the 16-byte vectors
// of row b are permuted by an XOR with a function of b instead of padding
// every row, so a request is one whole block and each lane loads the same
// (row in block, vector) in every request: its source offset is a constant
// plus the request's row offset, and no slot is padding.
//  - 128-byte rows, read by the transposed 8-byte read (a 16-lane group
//    reads 4 rows x one 32-byte segment s): segment s of row b sits at
//    s ^ swz8(b).  Rows 0..7 of a block at one segment then fall on 8
//    distinct 32-byte bank groups of a 256-byte bank window (and any 4
//    aligned rows on distinct groups of a 128-byte one); the 1152-byte pitch
//    (128 mod 256) separates rows 0..3 (or 4..7) of neighbouring blocks.
//  - 256-byte rows, read 16 bytes per lane down 16 rows: vector v of row b
//    sits at v ^ b, and the 1088-byte pitch (64 mod 256) shifts each block,
//    so 16 consecutive rows at one vector hit 16 distinct 16-byte bank groups.
//  - 256-byte rows read by the transposed read at rows r0 + 4 g + (0..3) of
//    lane group g (r0 a multiple of 8, so group g reads block r0/4 + g):
//    blocks of 4 rows at a pitch of 1024 bytes, and segment s of row b of
//    block q sits at s ^ b ^ (4 (q & 1)).  A half-wave (groups 0 and 1) then
//    reads 4 distinct segments of one half of the 256-byte window per block,
//    the two blocks in opposite halves.  A wave's requests keep one block
//    parity when the workgroup has an even number of waves.
constexpr int kBlk128 = 1152, kBlk256 = 1088, kBlk256T = 1024;
__host__ __device__ constexpr int swz8(int b) { return ((b >> 1) & 3) ^ ((b & 1) << 1); }

// One 16-byte-per-lane buffer load into LDS at lds_addr + 16 * lane, issued
// from inline assembly.  The compiler then does not see a pending LDS write:
// through the builtin it would wait for every such load before the next LDS
// read anywhere in the workgroup's code, which serialises a load into one
// buffer with reads of the other.  Callers wait themselves (s_waitcnt
// vmcnt(0) and a barrier) before anything reads the loaded bytes.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr,
                                           uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds_addr)
               : "memory");
}

// Load blocks q = wave, wave + nw, ... < nreq of a swizzled tile (block q at
// lds + q * BLK) from `src`: the lane's byte offset into block 0's rows is
// lane_off and block q starts q * req_bytes further.  Only the first
// valid_bytes of `src` are read: bytes at or past it arrive as zero (the
// buffer range check), which is how rows past the end of the data are
// zero-filled.  valid_bytes and every offset must stay below 2^31.  No wait:
// the caller waits for vmcnt(0) and synchronises before reading the tile.
template <int BLK>
__device__ __forceinline__ void dma_swz(char *lds, const void *src, uint32_t valid_bytes,
                                        uint32_t lane_off, uint32_t req_bytes, int nreq,
                                        int wave, int nw) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(src), (short)0, (int)valid_bytes, 0x00020000);
  const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)lds;
  uint32_t off = lane_off + (uint32_t)wave * req_bytes;
  const uint32_t step = (uint32_t)nw * req_bytes;
  for (int q = wave; q < nreq; q += nw) {
    lds_load16(rs, base + q * BLK, off);
    off += step;
  }
}

// Allow a kernel the full 160 KB of LDS (once per kernel and device; not a
// stream operation, so calls under graph capture are unaffected after the
// first).
static inline hipError_t set_lds_limit(const void *kern) {
  static std::mutex mu;
  static std::set<std::pair<int, const void *>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kern})) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.insert({dev, kern});
  return e;
}

}  // namespace ssd
