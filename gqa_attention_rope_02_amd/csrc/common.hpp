// Shared device helpers for the gfx950 attention kernels: vector types,
// bf16 conversion, MFMA wrappers and the argument blocks the host fills in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// -------------------------------------------------------------------- bf16

// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// 8 consecutive elements starting at p (16-byte aligned for bf16, 32 for fp32)
// as bf16 operands.
__device__ __forceinline__ bf16x8 load8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// the same 8 elements as fp32
__device__ __forceinline__ void load8_f32(const __bf16* p, float* x) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void load8_f32(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[i + 4] = b[i];
  }
}
__device__ __forceinline__ bf16x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = to_bf16(a[i]);
    r[i + 4] = to_bf16(b[i]);
  }
  return r;
}

// Store 4 consecutive fp32 values as the output element type.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = to_bf16(a);
  r[1] = to_bf16(b);
  r[2] = to_bf16(c);
  r[3] = to_bf16(d);
  *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 r = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = r;
}

// -------------------------------------------------------------------- LDS

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
using lds_void = __attribute__((address_space(3))) void;
using lds_i16x4 = __attribute__((address_space(3))) i16x4;

constexpr int kRsrcWord3 = 0x00020000;   // buffer descriptor word 3 (raw, no swizzle)

// Physical 16-byte chunk of logical chunk c in row r of a tile read as rows
// (ds_read_b128 of one chunk per lane).
template <int CH>
__device__ __forceinline__ int k_chunk(int c, int r) { return c ^ (r & (CH - 1)); }
// Tiles also read with the transposing ds_read_b64_tr_b16: rows 1 apart are
// spread by 4 chunks (64 bytes), so one transposing read of 32 lanes (4
// consecutive rows x two 32-byte halves of a 32-column block) touches every
// bank of the 256-byte row once. An XOR with a row-only term is its own
// inverse, which the loaders rely on.
template <int CH>
__device__ __forceinline__ int v_chunk(int c, int r) { return c ^ (CH == 16 ? 4 * (r & 3) : 2 * (r & 3)); }

// One 16-byte-per-lane load from `base` into LDS: lane i's 16 bytes at byte
// offset `voff` land at dst + 16 i; bytes at or past `bytes_valid` read as zero.
__device__ __forceinline__ void load_lds16(const void* base, int bytes_valid, int voff, char* dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes_valid, kRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, 0, 0, 0);
}
// The same with 4 bytes per lane (lane i's dword lands at dst + 4 i).
__device__ __forceinline__ void load_lds4(const void* base, int bytes_valid, int voff, char* dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes_valid, kRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, voff, 0, 0, 0);
}

// -------------------------------------------------------------------- MFMA

// D(32x32) += A(32x16) * B(16x32). Lane l holds A[l%32][8*(l/32)+i] and
// B[8*(l/32)+i][l%32] (i = 0..7) and D[8*(j/4)+4*(l/32)+j%4][l%32] (j = 0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16). Lane l holds A[l%16][8*(l/16)+i],
// B[8*(l/16)+i][l%16] and D[4*(l/16)+j][l%16] (j = 0..3).
__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x16) * B(16x16). Lane l holds A[l%16][4*(l/16)+i],
// B[4*(l/16)+i][l%16] (i = 0..3) and D[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// First document offset <= t in row[0..n] (row non-decreasing, row[0] = 0):
// the first key visible to a query at token t.
__device__ __forceinline__ int doc_start(const int32_t* row, int n, int t) {
  int lo = 0, hi = n;  // invariant: row[lo] <= t, answer index in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= t) lo = mid; else hi = mid;
  }
  return row[lo];
}

// One past the last token of the document holding token t: the first entry of
// row[0..n] above t (row non-decreasing, row[n] > t).
__device__ __forceinline__ int doc_end(const int32_t* row, int n, int t) {
  int lo = 0, hi = n;  // invariant: row[lo] <= t < row[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= t) lo = mid; else hi = mid;
  }
  return row[hi];
}

}  // namespace la
