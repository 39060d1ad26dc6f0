// Device-side building blocks for the gfx950 (CDNA4) Gated DeltaNet kernels:
// element types, 16-byte LDS/global moves and 16x16 MFMA tiles.
//
// Tile convention.  mma16<K>(acc, A, lda, Bt, ldb) adds A * B to a 16x16 fp32
// tile, where A is 16 rows x K (row-major, leading dimension lda) and B is
// given as its transpose Bt: 16 rows x K, so both operands are read along
// the contraction index.  On a 64-lane wavefront, lane l holds
//     acc[e] = D[m = 4*(l/16) + e][n = l % 16],   e = 0..3,
// the accumulator layout of the gfx950 16x16 MFMA family.  For the bf16
// path each lane feeds the eight consecutive contraction indices
// 8*(l/16) .. 8*(l/16)+7 of its row (v_mfma_f32_16x16x32_bf16); the fp32
// path feeds the same indices one instruction at a time
// (v_mfma_f32_16x16x4_f32), which is a permutation of the contraction order
// applied identically to A and B.  K must be a multiple of 16; a trailing
// 16 uses v_mfma_f32_16x16x16_bf16 (bf16) or four fp32 steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Round-to-nearest-even conversion (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_elem_bf16(float x) { return (bf16)x; }

template <typename T>
__device__ __forceinline__ T from_float(float x);
template <>
__device__ __forceinline__ float from_float<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_float<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16 x) { return (float)x; }

// Elements per 16-byte granule.
template <typename T>
struct Gran {
  static constexpr int n = 16 / (int)sizeof(T);
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *(const uint4*)p; }
__device__ __forceinline__ void st16(void* p, uint4 v) { *(uint4*)p = v; }

// Four consecutive elements (8 bytes for bf16, 16 for fp32).
template <typename T>
struct Quad;
template <>
struct Quad<bf16> {
  typedef bf16x4 type;
};
template <>
struct Quad<float> {
  typedef f32x4 type;
};

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  typename Quad<T>::type v;
  v[0] = from_float<T>(a);
  v[1] = from_float<T>(b);
  v[2] = from_float<T>(c);
  v[3] = from_float<T>(d);
  *(typename Quad<T>::type*)p = v;
}

template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p) {
  typename Quad<T>::type v = *(const typename Quad<T>::type*)p;
  f32x4 r;
  r[0] = to_float(v[0]);
  r[1] = to_float(v[1]);
  r[2] = to_float(v[2]);
  r[3] = to_float(v[3]);
  return r;
}

template <int K>
__device__ __forceinline__ void mma16(f32x4& acc, const bf16* A, int lda,
                                      const bf16* Bt, int ldb, int lane) {
  static_assert(K % 16 == 0, "contraction must be a multiple of 16");
  const int r = lane & 15, q = lane >> 4;
  const bf16* a = A + r * lda;
  const bf16* b = Bt + r * ldb;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    const bf16x8 av = *(const bf16x8*)(a + k0 + q * 8);
    const bf16x8 bv = *(const bf16x8*)(b + k0 + q * 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    const bf16x4 av = *(const bf16x4*)(a + k0 + q * 4);
    const bf16x4 bv = *(const bf16x4*)(b + k0 + q * 4);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
  }
}

template <int K>
__device__ __forceinline__ void mma16(f32x4& acc, const float* A, int lda,
                                      const float* Bt, int ldb, int lane) {
  static_assert(K % 16 == 0, "contraction must be a multiple of 16");
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda;
  const float* b = Bt + r * ldb;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    const f32x4 a0 = *(const f32x4*)(a + k0 + q * 8);
    const f32x4 a1 = *(const f32x4*)(a + k0 + q * 8 + 4);
    const f32x4 b0 = *(const f32x4*)(b + k0 + q * 8);
    const f32x4 b1 = *(const f32x4*)(b + k0 + q * 8 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], b1[j], acc, 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    const f32x4 a0 = *(const f32x4*)(a + k0 + q * 4);
    const f32x4 b0 = *(const f32x4*)(b + k0 + q * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc, 0, 0, 0);
  }
}

// fp32 tile product with B given row-major (K rows x 16 columns, leading
// dimension ldb): acc += A * B.  Used for the small triangular blocks.
__device__ __forceinline__ void mma16_f32_kn(f32x4& acc, const float* A, int lda,
                                             const float* B, int ldb, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + q * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float bv = B[(q * 4 + j) * ldb + r];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], bv, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

}  // namespace gdn
