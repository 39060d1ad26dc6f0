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
// k-tile order.  The scan's stored MFMA operands follow the accumulator
// layout along the contraction index: for a 16-row tile (rows m) and a
// 16-wide k-tile t, lane m + 16 g holds the four elements k = 16 t + 4 g + e
// (e = 0..3), which are the rows an accumulator tile gives that lane.  A
// product whose other operand is an accumulator (the state H, the U rows)
// then feeds its registers to the MFMA without moving data between lanes;
// the contraction order is permuted identically on both operands.  bf16
// pairs k-tiles (2u, 2u + 1) into one 16-byte unit per lane (the eight
// contraction indices of one v_mfma_f32_16x16x32_bf16); a trailing single
// bf16 k-tile is an 8-byte half unit (v_mfma_f32_16x16x16_bf16).  fp32 puts
// one k-tile in a 16-byte unit (four v_mfma_f32_16x16x4_f32, one per e).
// A full unit is 64 lanes x 16 bytes = 1 KiB.
template <typename TI, int K>
struct KTile {
  static_assert(K % 16 == 0, "contraction must be a multiple of 16");
  static constexpr int TPU = sizeof(TI) == 2 ? 2 : 1;       // k-tiles per unit
  static constexpr int NT = K / 16;                          // k-tiles
  static constexpr int NU = (NT + TPU - 1) / TPU;            // units
  static constexpr bool HALF_TAIL = TPU == 2 && (NT % 2) == 1;
  static constexpr int UNIT = 64 * 4 * TPU;                  // elements per full unit
  // Element offset of (m, k) inside one 16 x K tile (16 K elements).
  __host__ __device__ static constexpr int pos(int m, int k) {
    const int t = k / 16, g = (k % 16) / 4, e = k % 4, u = t / TPU, h = t % TPU;
    return (HALF_TAIL && u == NU - 1) ? u * UNIT + (m + 16 * g) * 4 + e
                                      : u * UNIT + (m + 16 * g) * 4 * TPU + 4 * h + e;
  }
};

// One unit's operand registers: a full bf16 unit (8 elements), a bf16 half
// unit (4; the upper half unused) or an fp32 unit (4).
template <typename TI>
struct Unit;
template <>
struct Unit<bf16> {
  typedef bf16x8 type;
};
template <>
struct Unit<float> {
  typedef f32x4 type;
};

// acc += A * B over one unit of the contraction (see KTile).
template <bool HALF>
__device__ __forceinline__ void mma_unit(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (HALF) {
    const bf16x4 a4 = __builtin_shufflevector(a, a, 0, 1, 2, 3);
    const bf16x4 b4 = __builtin_shufflevector(b, b, 0, 1, 2, 3);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
}
template <bool HALF>
__device__ __forceinline__ void mma_unit(f32x4& acc, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}

// Operand unit from accumulator tiles: k-tiles (2u, 2u + 1) for bf16 (a
// half unit takes one), k-tile u for fp32.
template <bool HALF>
__device__ __forceinline__ bf16x8 acc_unit(const f32x4& t0, const f32x4& t1, bf16) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (bf16)t0[e];
    v[4 + e] = HALF ? (bf16)0.f : (bf16)t1[e];
  }
  return v;
}
template <bool HALF>
__device__ __forceinline__ f32x4 acc_unit(const f32x4& t0, const f32x4&, float) {
  return t0;
}

// Reads one unit of a k-tile-order tile from LDS (byte address of the unit).
template <typename TI, bool HALF>
__device__ __forceinline__ typename Unit<TI>::type lds_unit(const char* unit, int lane) {
  if constexpr (sizeof(TI) == 2 && HALF) {
    const uint2 r = *(const uint2*)(unit + lane * 8);
    return __builtin_bit_cast(bf16x8, make_uint4(r.x, r.y, 0u, 0u));
  } else {
    return __builtin_bit_cast(typename Unit<TI>::type, *(const uint4*)(unit + lane * 16));
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

// The decay gate from its raw projection a for value head h (the reading
// documented at GDN_FLAG_DECAY_PROJ): g = -exp(A[h]) * softplus(a + bias[h]),
// softplus(x) = log(1 + e^x), in fp32.  For x > 20, e^-x is below half an
// fp32 ulp of x and softplus(x) rounds to x; otherwise log1p(e^x).  Null
// parameter arrays read as zeros.
__device__ __forceinline__ float decay_gate(float a, const float* a_log, const float* a_bias, int h) {
  const float x = a + (a_bias ? a_bias[h] : 0.f);
  const float sp = x > 20.f ? x : log1pf(expf(x));
  return -expf(a_log ? a_log[h] : 0.f) * sp;
}

// silu(x) = x / (1 + e^-x) in fp32 with the hardware exp2 and reciprocal
// (each within about an ulp; for x below about -88 the reciprocal of the
// overflowed 1 + e^-x is 0 and silu gives -0).
__device__ __forceinline__ float silu_f32(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + fast_exp(-x));
}

// The activation before the prefill (GDN_FLAG_QKV_SILU): silu in fp32,
// rounded to the input type TI as a separate activation pass would store it.
template <typename TI>
__device__ __forceinline__ float qkv_act(float x) {
  return to_float(from_float<TI>(silu_f32(x)));
}

// The end of the short convolution (GDN_FLAG_QKV_CONV): its fp32 sum, through
// silu when the activation is on, rounded once to the input type TI.
template <typename TI>
__device__ __forceinline__ TI conv_act(float y, int silu) {
  return from_float<TI>(silu ? silu_f32(y) : y);
}

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
// at row a0 of A, Bt rows at row b0 of Bt.  Only the tiles I0 <= i < I1,
// J0 <= j < J1 are computed (and only their fragments read); the others are
// left as they are.
template <int MT, int NT, int K, int SWA, int SWB, int I0 = 0, int I1 = MT, int J0 = 0, int J1 = NT>
__device__ __forceinline__ void mma_block_sw(f32x4 (&acc)[MT][NT], const bf16* A, int lda, int a0,
                                             const bf16* Bt, int ldb, int b0, int lane) {
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 + 32 <= K; k0 += 32) {
    bf16x8 a[MT], b[NT];
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int row = a0 + 16 * i + r;
      a[i] = *(const bf16x8*)(A + row * lda + swz<bf16, SWA>(row, k0 + q * 8));
    }
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int row = b0 + 16 * j + r;
      b[j] = *(const bf16x8*)(Bt + row * ldb + swz<bf16, SWB>(row, k0 + q * 8));
    }
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = J0; j < J1; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  if constexpr (K % 32 == 16) {
    constexpr int k0 = K - 16;
    bf16x4 a[MT], b[NT];
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int row = a0 + 16 * i + r;
      a[i] = *(const bf16x4*)(A + row * lda + swz<bf16, SWA>(row, k0 + q * 4));
    }
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int row = b0 + 16 * j + r;
      b[j] = *(const bf16x4*)(Bt + row * ldb + swz<bf16, SWB>(row, k0 + q * 4));
    }
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = J0; j < J1; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// fp32 operands: every tile is computed (the range only says which are needed).
template <int MT, int NT, int K, int SWA, int SWB, int I0 = 0, int I1 = MT, int J0 = 0, int J1 = NT>
__device__ __forceinline__ void mma_block_sw(f32x4 (&acc)[MT][NT], const float* A, int lda, int a0,
                                             const float* Bt, int ldb, int b0, int lane) {
  static_assert(SWA == 0 && SWB == 0, "fp32 operands use padded rows");
  mma_block<MT, NT, K>(acc, A + a0 * lda, lda, Bt + b0 * ldb, ldb, lane);
}

// acc += A_blk * B with both 16 x 16 fp32 operands in registers: a holds
// row lane % 16, columns 4 (lane / 16) + 0..3 of A_blk (as read by
// mma16_f32_acc_b), b a tile in accumulator layout.
__device__ __forceinline__ void mma16_f32_ab(f32x4& acc, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
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
