// ssd_device.h -- gfx950 device helpers for the SSD kernels: element types,
// 16x16 MFMA fragments, LDS operand loaders.
//
// Fragment convention (one wave64, a 16x16 output tile, a k-step of 32):
//   lane l, group g = l / 16, column/row c = l % 16
//   A operand : row c of the M x K tile, 8 k-slots owned by group g
//   B operand : column c of the K x N tile, the same 8 k-slots
//   result    : column c, rows 4g .. 4g+3 (acc[0..3])
// The k-slot -> k-index map is free as long as A and B use the same one,
// because the product sums over k.  The "natural" map gives group g the
// k-indices 8g .. 8g+7.  The "paired" map gives it 4g .. 4g+3 and
// 16+4g .. 16+4g+3: that is exactly what two stacked 16x16 results hold in one
// lane, so a result tile pair can be fed back as a B operand without moving
// data between lanes.
//
// bf16 uses v_mfma_f32_16x16x32_bf16 (one instruction per k-step).  float32
// uses v_mfma_f32_16x16x4_f32 eight times per k-step: instruction e takes
// slot e of every group, i.e. the k-indices {slot e of group 0..3}.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;
typedef __attribute__((address_space(3))) short4v lds_short4v;

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f8v;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i4v;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

// bf16 vectors are always built and converted as whole vectors
// (__builtin_convertvector / bit casts), never by 16-bit element inserts.
__device__ __forceinline__ f8v cvt_f8(bf16x8 v) { return __builtin_convertvector(v, f8v); }
__device__ __forceinline__ bf16x8 cvt_bf8(f8v v) { return __builtin_convertvector(v, bf16x8); }

__device__ __forceinline__ Frag<bf16> frag_from_f32(const float (&m)[8], bf16) {
  Frag<bf16> f;
  f.v = cvt_bf8(f8v{m[0], m[1], m[2], m[3], m[4], m[5], m[6], m[7]});
  return f;
}
__device__ __forceinline__ Frag<float> frag_from_f32(const float (&m)[8], float) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = m[e];
  return f;
}
// Fragment times a scalar (float32 arithmetic, rounded back for bf16).
__device__ __forceinline__ Frag<bf16> frag_scale(const Frag<bf16> &f, float s) {
  Frag<bf16> o;
  o.v = cvt_bf8(cvt_f8(f.v) * s);
  return o;
}
__device__ __forceinline__ Frag<float> frag_scale(const Frag<float> &f, float s) {
  Frag<float> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = f.v[e] * s;
  return o;
}
template <typename T> __device__ __forceinline__ Frag<T> frag_zero() {
  const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return frag_from_f32(z, T());
}

__device__ __forceinline__ void mma(f4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// Fragment from an LDS tile stored with k contiguous: element (row, k) at
// tile[row * pitch + k].  Lane reads row `row`, k-indices k8 .. k8+7
// (the caller passes row = r0 + l%16 and k8 = k0 + 8*(l/16)).
// Alignment: (row*pitch + k8) * sizeof(T) must be a multiple of 16.
__device__ __forceinline__ Frag<bf16> frag_rowk(const bf16 *tile, int pitch, int row, int k8) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(tile + row * pitch + k8);
  return f;
}
__device__ __forceinline__ Frag<float> frag_rowk(const float *tile, int pitch, int row, int k8) {
  Frag<float> f;
  const f4 *p = reinterpret_cast<const f4 *>(tile + row * pitch + k8);
  f4 a = p[0], b = p[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
  return f;
}

// Fragment from an LDS tile stored with k as the SLOW index: element (k, m)
// at tile[k * pitch + m].  Lane gets column m0 + l%16 and the k-rows
// rlo .. rlo+3 (slots 0..3) and rhi .. rhi+3 (slots 4..7); rlo/rhi may depend
// on the lane group.  bf16 uses the gfx950 LDS transpose read
// (ds_read_b64_tr_b16): within each 16-lane group, lane j' supplies the address
// of row (base + j'/4), columns m0 + 4*(j'%4) .. +3, and lane i receives column
// m0 + i of rows base .. base+3.  Alignment: pitch and m0 multiples of 4.
__device__ __forceinline__ Frag<bf16> frag_kmaj(const bf16 *tile, int pitch, int m0, int rlo,
                                                int rhi) {
  const int j = threadIdx.x & 15;
  const bf16 *plo = tile + (rlo + (j >> 2)) * pitch + m0 + 4 * (j & 3);
  const bf16 *phi = tile + (rhi + (j >> 2)) * pitch + m0 + 4 * (j & 3);
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(plo));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(phi));
  // whole-vector casts: building the fragment element by element from 16-bit
  // lanes of the two reads is mis-lowered by the compiler
  Frag<bf16> f;
  f.v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0,
                                1, 2, 3, 4, 5, 6, 7);
  return f;
}
// frag_kmaj (bf16) with the two row-quad addresses given as byte offsets
// into an LDS tile (each lane's own address, as frag_kmaj computes them).
__device__ __forceinline__ Frag<bf16> frag_kmaj_at(const char *lds, int lo, int hi) {
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(lds + lo));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(lds + hi));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0,
                                1, 2, 3, 4, 5, 6, 7);
  return f;
}
// frag_rowk (bf16) at a byte offset: the lane's 8 k-values, 16 bytes.
__device__ __forceinline__ Frag<bf16> frag_rowk_at(const char *lds, int off) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(lds + off);
  return f;
}
__device__ __forceinline__ Frag<float> frag_kmaj(const float *tile, int pitch, int m0, int rlo,
                                                 int rhi) {
  const int c = m0 + (threadIdx.x & 15);
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = tile[(rlo + e) * pitch + c];
    f.v[4 + e] = tile[(rhi + e) * pitch + c];
  }
  return f;
}

// 16-byte vector of T (8 bf16 or 4 floats) for global <-> LDS staging.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int n = 8;
  typedef bf16x8 type;
};
template <> struct Vec16<float> {
  static constexpr int n = 4;
  typedef f4 type;
};

__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }

// Four consecutive elements of T as floats (8-byte or 16-byte load).
__device__ __forceinline__ f4 ld4f(const float *p) { return ld4(p); }
__device__ __forceinline__ f4 ld4f(const bf16 *p) {
  return __builtin_convertvector(*reinterpret_cast<const bf16x4 *>(p), f4);
}
// Store four floats as T (rounded to nearest even for bf16).
__device__ __forceinline__ void st4T(float *p, f4 v) { st4(p, v); }
__device__ __forceinline__ void st4T(bf16 *p, f4 v) {
  *reinterpret_cast<bf16x4 *>(p) = __builtin_convertvector(v, bf16x4);
}
// 16-byte vector scaled by s (computed in float32, rounded back for bf16).
__device__ __forceinline__ bf16x8 vscale(bf16x8 v, float s) { return cvt_bf8(cvt_f8(v) * s); }
__device__ __forceinline__ f4 vscale(f4 v, float s) { return v * s; }
template <typename V> __device__ __forceinline__ V vzero() { return __builtin_bit_cast(V, i4v{0, 0, 0, 0}); }

// A float from another lane of the same 16-lane DPP row (CTRL: a DPP control
// code, e.g. 0xB1 quad_perm [1,0,3,2], 0x4E quad_perm [2,3,0,1], 0x140
// row_mirror, 0x141 row_half_mirror, 0x128 row_ror:8).  One VALU move.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

}  // namespace ssd

namespace ssd {
// Eight consecutive elements from global memory as a fragment (16-byte
// aligned for bf16, 32-byte for float).
__device__ __forceinline__ Frag<bf16> frag_global(const bf16 *p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(p);
  return f;
}
__device__ __forceinline__ Frag<float> frag_global(const float *p) {
  Frag<float> f;
  const f4 a = ld4(p), b = ld4(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
  return f;
}
}  // namespace ssd
