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

// Four consecutive elements exactly as stored, and their conversion.
template <typename T>
struct Raw4;
template <>
struct Raw4<bf16> {
  typedef uint2 type;
};
template <>
struct Raw4<float> {
  typedef uint4 type;
};

template <typename T>
__device__ __forceinline__ typename Raw4<T>::type load_raw4(const T* p) {
  return *(const typename Raw4<T>::type*)p;
}

template <typename T>
__device__ __forceinline__ f32x4 raw4_to_f32(typename Raw4<T>::type r) {
  const typename Quad<T>::type v = __builtin_bit_cast(typename Quad<T>::type, r);
  f32x4 o;
  o[0] = to_float(v[0]);
  o[1] = to_float(v[1]);
  o[2] = to_float(v[2]);
  o[3] = to_float(v[3]);
  return o;
}

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

// Pins an MFMA accumulator to VGPRs at this point of the program, so the
// copy out of the accumulator registers happens in the same basic block as
// the MFMAs that produced it.  The compiler inserts the wait states an
// MFMA result needs before a VALU read reliably in straight-line code; on a
// path that branches right after the MFMAs it was seen to read a stale
// element (the fourth accumulator register, before the last MFMA had
// landed).  Use it on accumulators that stay live across a branch.
__device__ __forceinline__ void settle(f32x4& acc) { asm volatile("" : "+v"(acc)); }

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

}  // namespace gdn

namespace gdn {

// ---------------------------------------------------------------------------
// Fragment order.  A 16 x K operand tile (rows m, contraction index k) is
// stored so that one wavefront reads its MFMA operand registers with
// contiguous 16-byte (or 8-byte) loads: for every 32-wide k-group g, the 64
// lanes' eight consecutive elements (lane l: row l % 16, k = 32 g + 8 (l/16)
// + j) follow each other; a trailing 16-wide group stores four elements per
// lane (k = K32 + 4 (l/16) + j).  The same order serves as the A or the B
// operand, since both take row/column l % 16 and the same k range per lane.
template <int K>
__host__ __device__ constexpr int frag_pos(int m, int k) {
  constexpr int K32 = (K / 32) * 32;
  return k < K32 ? (k / 32) * 512 + (m + 16 * ((k % 32) / 8)) * 8 + (k % 8)
                 : K32 * 16 + (m + 16 * ((k - K32) / 4)) * 4 + ((k - K32) % 4);
}

// Per-lane registers of one 16 x K fragment tile.
template <typename TI, int K>
struct Frag {
  static constexpr int NG = K / 32;                 // full 32-wide groups
  static constexpr bool TAIL = (K % 32) == 16;
  static constexpr int U4_PER_G = sizeof(TI) == 2 ? 1 : 2;   // uint4 per lane per group
  static constexpr int NV = NG * U4_PER_G + (TAIL ? 1 : 0);  // uint4 slots (tail: bf16 uses .xy)
  uint4 v[NV > 0 ? NV : 1];

  __device__ __forceinline__ void load(const TI* tile, int lane) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const TI* p = tile + g * 512 + lane * 8;
      v[g * U4_PER_G] = ld16(p);
      if constexpr (U4_PER_G == 2) v[g * U4_PER_G + 1] = ld16(p + 4);
    }
    if constexpr (TAIL) {
      const TI* p = tile + NG * 512 + lane * 4;
      if constexpr (sizeof(TI) == 2) {
        const uint2 t = *(const uint2*)p;
        v[NV - 1] = make_uint4(t.x, t.y, 0, 0);
      } else {
        v[NV - 1] = ld16(p);
      }
    }
  }
};

// acc += A * B^T with A from fragment registers and B^T rows from LDS
// (16 rows, leading dimension ldb, contraction contiguous).
template <int K>
__device__ __forceinline__ void mma_frag_lds(f32x4& acc, const Frag<bf16, K>& a,
                                             const bf16* Bt, int ldb, int lane) {
  const bf16* b = Bt + (lane & 15) * ldb + (lane >> 4) * 8;
#pragma unroll
  for (int g = 0; g < Frag<bf16, K>::NG; ++g) {
    const bf16x8 bv = *(const bf16x8*)(b + g * 32);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[g]), bv, acc, 0, 0, 0);
  }
  if constexpr (Frag<bf16, K>::TAIL) {
    constexpr int NG = Frag<bf16, K>::NG;
    const bf16x4 bv = *(const bf16x4*)(Bt + (lane & 15) * ldb + NG * 32 + (lane >> 4) * 4);
    const uint2 t = make_uint2(a.v[Frag<bf16, K>::NV - 1].x, a.v[Frag<bf16, K>::NV - 1].y);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, t), bv, acc, 0, 0, 0);
  }
}

template <int K>
__device__ __forceinline__ void mma_frag_lds(f32x4& acc, const Frag<float, K>& a,
                                             const float* Bt, int ldb, int lane) {
  const float* b = Bt + (lane & 15) * ldb + (lane >> 4) * 8;
#pragma unroll
  for (int g = 0; g < Frag<float, K>::NG; ++g) {
    const f32x4 b0 = *(const f32x4*)(b + g * 32);
    const f32x4 b1 = *(const f32x4*)(b + g * 32 + 4);
    const f32x4 a0 = __builtin_bit_cast(f32x4, a.v[2 * g]);
    const f32x4 a1 = __builtin_bit_cast(f32x4, a.v[2 * g + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], b1[j], acc, 0, 0, 0);
  }
  if constexpr (Frag<float, K>::TAIL) {
    constexpr int NG = Frag<float, K>::NG;
    const f32x4 b0 = *(const f32x4*)(Bt + (lane & 15) * ldb + NG * 32 + (lane >> 4) * 4);
    const f32x4 a0 = __builtin_bit_cast(f32x4, a.v[Frag<float, K>::NV - 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b0[j], acc, 0, 0, 0);
  }
}

// Two products sharing one LDS operand H (16 rows of H^T, contraction d_k):
//   accu += A * H^T-rows   (A from fragments: U = W H)
//   acco += H^T-rows * B   (B from fragments: O^T = H^T Q'^T)
template <int K>
__device__ __forceinline__ void mma_pair_lds(f32x4& accu, f32x4& acco, const Frag<bf16, K>& a,
                                             const Frag<bf16, K>& b, const bf16* Ht, int ldh,
                                             int lane) {
  const bf16* h = Ht + (lane & 15) * ldh + (lane >> 4) * 8;
#pragma unroll
  for (int g = 0; g < Frag<bf16, K>::NG; ++g) {
    const bf16x8 hv = *(const bf16x8*)(h + g * 32);
    accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[g]), hv, accu, 0, 0, 0);
    acco = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, __builtin_bit_cast(bf16x8, b.v[g]), acco, 0, 0, 0);
  }
  if constexpr (Frag<bf16, K>::TAIL) {
    constexpr int NG = Frag<bf16, K>::NG, NV = Frag<bf16, K>::NV;
    const bf16x4 hv = *(const bf16x4*)(Ht + (lane & 15) * ldh + NG * 32 + (lane >> 4) * 4);
    const bf16x4 av = __builtin_bit_cast(bf16x4, make_uint2(a.v[NV - 1].x, a.v[NV - 1].y));
    const bf16x4 bv = __builtin_bit_cast(bf16x4, make_uint2(b.v[NV - 1].x, b.v[NV - 1].y));
    accu = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, hv, accu, 0, 0, 0);
    acco = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hv, bv, acco, 0, 0, 0);
  }
}

template <int K>
__device__ __forceinline__ void mma_pair_lds(f32x4& accu, f32x4& acco, const Frag<float, K>& a,
                                             const Frag<float, K>& b, const float* Ht, int ldh,
                                             int lane) {
  const float* h = Ht + (lane & 15) * ldh + (lane >> 4) * 8;
#pragma unroll
  for (int g = 0; g < Frag<float, K>::NG; ++g) {
    const f32x4 h0 = *(const f32x4*)(h + g * 32);
    const f32x4 h1 = *(const f32x4*)(h + g * 32 + 4);
    const f32x4 a0 = __builtin_bit_cast(f32x4, a.v[2 * g]), a1 = __builtin_bit_cast(f32x4, a.v[2 * g + 1]);
    const f32x4 b0 = __builtin_bit_cast(f32x4, b.v[2 * g]), b1 = __builtin_bit_cast(f32x4, b.v[2 * g + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accu = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], h0[j], accu, 0, 0, 0);
      acco = __builtin_amdgcn_mfma_f32_16x16x4f32(h0[j], b0[j], acco, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accu = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], h1[j], accu, 0, 0, 0);
      acco = __builtin_amdgcn_mfma_f32_16x16x4f32(h1[j], b1[j], acco, 0, 0, 0);
    }
  }
  if constexpr (Frag<float, K>::TAIL) {
    constexpr int NG = Frag<float, K>::NG, NV = Frag<float, K>::NV;
    const f32x4 h0 = *(const f32x4*)(Ht + (lane & 15) * ldh + NG * 32 + (lane >> 4) * 4);
    const f32x4 a0 = __builtin_bit_cast(f32x4, a.v[NV - 1]), b0 = __builtin_bit_cast(f32x4, b.v[NV - 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accu = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], h0[j], accu, 0, 0, 0);
      acco = __builtin_amdgcn_mfma_f32_16x16x4f32(h0[j], b0[j], acco, 0, 0, 0);
    }
  }
}

// Accumulator tiles stored as [lane][4] (lane l holds rows 4 (l/16) + e,
// column l % 16 of a 16 x 16 tile): 256 elements per tile.
template <typename TI>
__device__ __forceinline__ void store_acc_tile(TI* tile, const f32x4& a, int lane) {
  store4<TI>(tile + lane * 4, a[0], a[1], a[2], a[3]);
}

}  // namespace gdn

namespace gdn {

// Register-blocked product: acc[i][j] += A_i * Bt_j^T for MT row tiles of A
// (16 rows each, starting at A, leading dimension lda) and NT row tiles of Bt
// (starting at Bt, leading dimension ldb), contraction K.  Each operand
// fragment is read from LDS once per k-group and feeds MT x NT MFMAs.
template <int MT, int NT, int K>
__device__ __forceinline__ void mma_block(f32x4 (&acc)[MT][NT], const bf16* A, int lda,
                                          const bf16* Bt, int ldb, int lane) {
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) a[i] = *(const bf16x8*)(A + (16 * i + r) * lda + k0 + q * 8);
#pragma unroll
    for (int j = 0; j < NT; ++j) b[j] = *(const bf16x8*)(Bt + (16 * j + r) * ldb + k0 + q * 8);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    bf16x4 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) a[i] = *(const bf16x4*)(A + (16 * i + r) * lda + k0 + q * 4);
#pragma unroll
    for (int j = 0; j < NT; ++j) b[j] = *(const bf16x4*)(Bt + (16 * j + r) * ldb + k0 + q * 4);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

template <int MT, int NT, int K>
__device__ __forceinline__ void mma_block(f32x4 (&acc)[MT][NT], const float* A, int lda,
                                          const float* Bt, int ldb, int lane) {
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 a[MT], b[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = *(const f32x4*)(A + (16 * i + r) * lda + k0 + q * 8 + 4 * half);
#pragma unroll
      for (int j = 0; j < NT; ++j) b[j] = *(const f32x4*)(Bt + (16 * j + r) * ldb + k0 + q * 8 + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    f32x4 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) a[i] = *(const f32x4*)(A + (16 * i + r) * lda + k0 + q * 4);
#pragma unroll
    for (int j = 0; j < NT; ++j) b[j] = *(const f32x4*)(Bt + (16 * j + r) * ldb + k0 + q * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
  }
}

// exp(x) through the hardware base-2 exponential: x * log2(e), then
// v_exp_f32.  Relative error grows like |x| * 2^-24 from the scaling, which
// is far below bf16 resolution and below 1e-6 for |x| < 10 (larger |x| give
// values below 5e-5 whose absolute error is then negligible).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

}  // namespace gdn

namespace gdn {

// Row-swizzled LDS matrices.  A matrix of rows of `ld` elements is stored
// without padding; the 16-byte granule g of row r lives at granule
// g ^ (r & SW).  SW = (granules per row - 1) makes the 16 rows read by one
// MFMA fragment load land on distinct banks.  SW = 0 is a plain layout
// (used with padded rows).
template <typename T, int SW>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int GE = 16 / (int)sizeof(T);
  if constexpr (SW == 0) return col;
  return ((((col / GE) ^ (row & SW))) * GE) + (col % GE);
}

// mma_block on swizzled operands: acc[i][j] += A_i * Bt_j^T, A rows start
// at row a0 of A, Bt rows at row b0 of Bt.
template <int MT, int NT, int K, int SWA, int SWB>
__device__ __forceinline__ void mma_block_sw(f32x4 (&acc)[MT][NT], const bf16* A, int lda, int a0,
                                             const bf16* Bt, int ldb, int b0, int lane) {
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = a0 + 16 * i + r;
      a[i] = *(const bf16x8*)(A + row * lda + swz<bf16, SWA>(row, k0 + q * 8));
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = b0 + 16 * j + r;
      b[j] = *(const bf16x8*)(Bt + row * ldb + swz<bf16, SWB>(row, k0 + q * 8));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    bf16x4 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = a0 + 16 * i + r;
      a[i] = *(const bf16x4*)(A + row * lda + swz<bf16, SWA>(row, k0 + q * 4));
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = b0 + 16 * j + r;
      b[j] = *(const bf16x4*)(Bt + row * ldb + swz<bf16, SWB>(row, k0 + q * 4));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

template <int MT, int NT, int K, int SWA, int SWB>
__device__ __forceinline__ void mma_block_sw(f32x4 (&acc)[MT][NT], const float* A, int lda, int a0,
                                             const float* Bt, int ldb, int b0, int lane) {
  static_assert(SWA == 0 && SWB == 0, "fp32 operands use padded rows");
  mma_block<MT, NT, K>(acc, A + a0 * lda, lda, Bt + b0 * ldb, ldb, lane);
}

// acc += A_blk * B where B is a 16 x 16 fp32 tile held in accumulator
// layout by this wave (lane (q, r) holds B[4q + e][r]); with the contraction
// order of instruction e taken as k = 4q + e this is exactly the operand
// layout of v_mfma_f32_16x16x4_f32, so no LDS round trip is needed.
__device__ __forceinline__ void mma16_f32_acc_b(f32x4& acc, const float* A, int lda, const f32x4& b,
                                                int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + q * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}

}  // namespace gdn
