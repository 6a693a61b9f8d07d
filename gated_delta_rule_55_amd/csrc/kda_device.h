// kda_device.h -- device-side building blocks shared by the KDA kernels:
// storage types, conversions, and the 16x16 matrix-core (MFMA) step.
//
// MFMA operand layout used throughout (gfx950, wave64):
//   A (16 x K), B (K x 16), D (16 x 16) fp32.
//   Lane l supplies row (l % 16) of A and column (l % 16) of B.  The 64 lanes
//   form four groups g = l / 16; within a 32-wide slice of the contraction
//   index, lane group g holds eight values e = 0..7.  Which contraction index
//   (g, e) stands for is chosen by whoever fills the fragments; A and B only
//   have to agree.  D comes back with lane l holding rows 4g + i (i = 0..3)
//   of column l % 16.
//
// Two contraction orders are used:
//   kstd(g, e)  = 8g + e                       -- 8 consecutive indices per
//                                                 lane: one 16-byte load
//   kperm(g, e) = 16(e / 4) + 4g + (e % 4)     -- exactly the rows a D tile
//                                                 pair holds in lane group g,
//                                                 so a D result feeds the next
//                                                 contraction from registers
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Fragment type for one 32-wide contraction slice: 8 values per lane.
template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
  typedef bf16x8 type;
};
template <>
struct Frag<float> {
  typedef f32x8 type;
};

// D += A * B over one 32-wide contraction slice.
// bf16: one v_mfma_f32_16x16x32_bf16.  fp32: eight v_mfma_f32_16x16x4_f32, each
// pairing element e of every lane group (so the slice's index set is the same).
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}
// fp32 16x16x16 step: four 16x16x4 MFMAs; element m of lane group g is
// contraction index 4m + g for the caller's choice of ordering.
__device__ __forceinline__ f32x4 mma16_f32(const float (&a)[4], const float (&b)[4], f32x4 c) {
#pragma unroll
  for (int m = 0; m < 4; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ int kstd(int g, int e) { return 8 * g + e; }
__device__ __forceinline__ int kperm(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Fragment of 8 consecutive elements at p (16-byte aligned for bf16, 32 for f32).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag8(const T* p);
template <>
__device__ __forceinline__ bf16x8 load_frag8<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ f32x8 load_frag8<float>(const float* p) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Store 8 consecutive elements (two 16-byte halves for fp32).
__device__ __forceinline__ void store_frag8(bf16* p, bf16x8 f) { *reinterpret_cast<bf16x8*>(p) = f; }
__device__ __forceinline__ void store_frag8(float* p, f32x8 f) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// Fragment in kperm order from a row: elements p[base + 4g + 0..3] and
// p[base + 16 + 4g + 0..3] (base = 32 * slice); two 4-element loads.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag_perm(const T* row, int g);
template <>
__device__ __forceinline__ bf16x8 load_frag_perm<bf16>(const bf16* row, int g) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 4 * g);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 + 4 * g);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <>
__device__ __forceinline__ f32x8 load_frag_perm<float>(const float* row, int g) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * g);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 + 4 * g);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Fragment from two D tiles held in registers (tile 0 -> e 0..3, tile 1 ->
// e 4..7): the kperm order.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type frag_from_d(f32x4 d0, f32x4 d1) {
  typename Frag<T>::type f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = from_f32<T>(d0[i]);
    f[4 + i] = from_f32<T>(d1[i]);
  }
  return f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// eps of the in-kernel q / k L2 normalisation: x / sqrt(sum x^2 + eps).
constexpr float kQkNormEps = 1e-6f;

// The Kimi gate in base 2: g log2(e) with g = -exp(a_log) softplus(z),
// z = x + dt_bias, given ea = exp(a_log).  softplus(z) log2(e) =
// log2(1 + 2^(z log2 e)), which is z log2(e) to fp32 precision once that
// exceeds 24.  (For very negative z, 1 + 2^(z log2 e) rounds to 1 and the
// gate reads 0 instead of a value below 1e-7 of ea: no decay lost that fp32
// could hold.)
__device__ __forceinline__ float kimi_gate_log2(float z, float ea) {
  const float zl = z * kLog2e;
  return -ea * (zl > 24.f ? zl : __builtin_amdgcn_logf(1.f + fast_exp2(zl)));
}

// Four consecutive state values (fp32 or bf16 storage) as fp32, and back
// (bf16 stores round to nearest even).
__device__ __forceinline__ f32x4 load_state4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load_state4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store_state4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void store_state4(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Two values of T in one vector (4 bytes for bf16, 8 for fp32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <typename T>
struct Vec2;
template <>
struct Vec2<bf16> {
  typedef bf16x2 type;
};
template <>
struct Vec2<float> {
  typedef f32x2 type;
};

// Four values of T in one vector (8 bytes for bf16, 16 for fp32).
template <typename T>
struct Vec4;
template <>
struct Vec4<bf16> {
  typedef bf16x4 type;
};
template <>
struct Vec4<float> {
  typedef f32x4 type;
};

// Raw buffer stores: a lane whose byte offset is at or past the buffer's
// num_records has its store dropped by the hardware, so a masked store needs
// no branch.  kBufferOff is such an offset.
constexpr int kBufferOff = (int)0x80000000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_store(bf16 v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store(float v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0, 0);
}
// Raw buffer load: lanes whose offset falls outside the buffer read 0.
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buffer_store16(uint4 v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}

}  // namespace kda
