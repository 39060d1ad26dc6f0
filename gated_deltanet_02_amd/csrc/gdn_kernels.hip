// gfx950 (CDNA4) kernels of the chunked Gated DeltaNet prefill.
//
// The operation is the chunked Gated DeltaNet prefill that the serving pages
// run in their native backend and test against float64 references ("Cua-S1
// 4B 0.2 native text worker"; "Open-Jev-27B-v1.1 native text worker",
// section "Validation and optimization scope").  The pages print no formula;
// the recurrence taken here (state H, d_k x d_v) is
//   H_t = exp(g_t) (I - beta_t k^_t k^_t^T) H_{t-1} + beta_t k^_t v_t^T,
//   o_t = scale H_t^T q^_t,  q^, k^ the L2-normalised rows,
// evaluated chunk by chunk in its WY (compact product) form, which follows
// from summing the recurrence over a chunk.  For a chunk of n <= C
// tokens with chunk-local cumulative gate gamma_r = g_0 + ... + g_r and
// D_rs = exp(gamma_r - gamma_s) (s <= r):
//
//   A   = strictly-lower part of beta_r D_rs (k^_r . k^_s)
//   T   = (I + A)^-1                              (forward substitution)
//   W   = T diag(beta e^gamma) K^,   U~ = T diag(beta) V
//   P   = scale * D o (Q^ K^T)                    (causal, diagonal included)
//   Q'  = scale diag(e^gamma) Q^ - P W,   O_loc = P U~
//   K~_r = e^(gamma_last - gamma_r) k^_r = s_r k_r,
//   s_r = e^(gamma_last - gamma_r) / sqrt(|k_r|^2 + eps)   (k_r as passed)
// and, carried from chunk to chunk with state H (d_k x d_v, fp32):
//   U = U~ - W H,   O = Q' H + O_loc,   H <- e^gamma_last H + K~^T U.
// The state update is taken as K^T U' with U' = diag(s) U~ - diag(s) W H:
// the WY kernel stores diag(s) W and diag(s) U~, and the scan reads the
// chunk's key rows as passed, so no K~ is ever written.
//
// Kernels, launched in this order on the caller's stream:
//   table_kernel  packed batches only: sanitised sequence starts, the
//                 exclusive prefix of per-sequence chunk counts and a
//                 (sequence, first token, length) row per chunk.
//   wy_kernel     one workgroup per (chunk, key head), looping over the value
//                 heads of the group: L2 norms of q and k rows, the gate
//                 cumulative sum, K^K^T and Q^K^T (shared by the group), the
//                 blocked triangular inverse and every per-chunk matrix above.
//                 Fully parallel over chunks.
//   scan_kernel   one workgroup per (sequence, value head, one or two
//                 16-column slices of d_v): the only sequential part.  Per
//                 slice one wave runs the recurrence with the state slice in
//                 its MFMA accumulators; W and Q' are stored by the WY
//                 kernel in k-tile order (the contraction index follows the
//                 accumulator layout) and the key rows are read transposed
//                 in the same order, so the state and the U rows feed the
//                 MFMAs from the registers they were accumulated in, with no
//                 exchange through LDS; a second wave forms the slice's
//                 output.  Two more waves stream the chunks' operands (W,
//                 Q' and the key rows) into an LDS ring with LDS-direct
//                 loads, two chunks ahead.
//   scan_split_kernel, scan_fix_kernel
//                 the two-level form of the scan, on request (both halves of
//                 each sequence at once, then the second half's correction).
//   decode_kernel one token per sequence on a state in memory.
//
// bf16 inputs use bf16 MFMA operands with fp32 accumulation; the triangular
// solve and every gate exponential are fp32.  fp32 inputs use fp32 MFMA
// throughout.  All exponents are <= 0 when g <= 0: differences of gamma are
// only formed for s <= r and never factored into exp(gamma_r) exp(-gamma_s).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_cu_check.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kThreads = 256;
constexpr int kLdsLimit = 160 * 1024;

// ---------------------------------------------------------------------------
// chunk bookkeeping

__device__ __forceinline__ bool chunk_info(const ChunkMap& m, int c, int C,
                                           int& seq, int& t0, int& n) {
  if (!m.packed) {
    if (c >= m.n_seq * m.chunks_per_seq) return false;
    seq = c / m.chunks_per_seq;
    const int j = c - seq * m.chunks_per_seq;
    t0 = seq * m.seq_stride + j * C;
    n = min(C, m.seq_len - j * C);
    return true;
  }
  if (c >= m.chunk_off[m.n_seq]) return false;
  const int* row = m.table + 4 * (int64_t)c;
  seq = row[0];
  t0 = row[1];
  n = row[2];
  return true;
}

__device__ __forceinline__ void seq_range(const ChunkMap& m, int seq, int C,
                                          int& c_begin, int& c_end, int& tok0,
                                          int& tok_end) {
  if (!m.packed) {
    c_begin = seq * m.chunks_per_seq;
    c_end = c_begin + m.chunks_per_seq;
    tok0 = seq * m.seq_stride;
    tok_end = tok0 + m.seq_len;
    return;
  }
  c_begin = m.chunk_off[seq];
  c_end = m.chunk_off[seq + 1];
  tok0 = m.seq_start[seq];
  tok_end = m.seq_start[seq + 1];
}

// Single workgroup.  Sequence ends are clamped into [previous end, T] so a
// malformed cu_seqlens can only produce wrong results, never an access
// outside the tensors.
__global__ __launch_bounds__(1024) void table_kernel(TableParams p) {
  __shared__ int s_max[1024];
  __shared__ int s_sum[1024];
  __shared__ int s_carry_end, s_carry_chunks;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry_end = 0;
    s_carry_chunks = 0;
    p.seq_start[0] = 0;
    p.chunk_off[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < p.n_seq; base += 1024) {
    const int i = base + tid;
    int64_t e64 = 0;
    if (i < p.n_seq) e64 = p.cu_i64 ? ((const int64_t*)p.cu)[i + 1] : ((const int32_t*)p.cu)[i + 1];
    const int e = (int)min(max(e64, (int64_t)0), (int64_t)p.t_total);
    s_max[tid] = e;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = tid >= off ? s_max[tid - off] : 0;
      __syncthreads();
      s_max[tid] = max(s_max[tid], y);
      __syncthreads();
    }
    const int carry_end = s_carry_end;
    const int end_i = max(s_max[tid], carry_end);
    const int start_i = tid > 0 ? max(s_max[tid - 1], carry_end) : carry_end;
    const int nch = (i < p.n_seq) ? (end_i - start_i + p.chunk - 1) / p.chunk : 0;
    if (i < p.n_seq) p.seq_start[i + 1] = end_i;
    s_sum[tid] = nch;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += y;
      __syncthreads();
    }
    const int carry_chunks = s_carry_chunks;
    if (i < p.n_seq) p.chunk_off[i + 1] = carry_chunks + s_sum[tid];
    __syncthreads();
    if (tid == 1023) {
      s_carry_chunks = carry_chunks + s_sum[1023];
      s_carry_end = max(carry_end, s_max[1023]);
    }
    __syncthreads();
  }
  __threadfence();
  __syncthreads();
  const int total = min(p.chunk_off[p.n_seq], p.max_chunks);
  for (int c = tid; c < total; c += 1024) {
    int lo = 0, hi = p.n_seq - 1;  // largest i with chunk_off[i] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int j = c - p.chunk_off[lo];
    const int t0 = p.seq_start[lo] + j * p.chunk;
    int* row = p.table + 4 * (int64_t)c;
    row[0] = lo;
    row[1] = t0;
    row[2] = min(p.chunk, p.seq_start[lo + 1] - t0);
    row[3] = 0;
  }
}

// ---------------------------------------------------------------------------
// WY kernel

// Column order of the bf16 [*][C] tiles of the WY kernel (P, Tb, Tv):
// within each full 32-column block, column s = 32 u + 16 h + 4 q + e is
// stored at 32 u + 8 q + 4 h + e, so that a k-tile-order operand unit (see
// KTile: elements 32 u + 4 q + {0..3} and 32 u + 16 + 4 q + {0..3} for
// lane group q) is 16 contiguous bytes.  A trailing half block (C % 32 ==
// 16) and fp32 tiles keep the natural order.  kinv maps a stored position
// back to its column.
template <typename TI, int C>
__device__ __forceinline__ int kperm(int s) {
  if constexpr (sizeof(TI) != 2) return s;
  if (s >= C / 32 * 32) return s;
  return (s & ~31) + 8 * ((s >> 2) & 3) + 4 * ((s >> 4) & 1) + (s & 3);
}
template <typename TI, int C>
__device__ __forceinline__ int kinv(int pos) {
  if constexpr (sizeof(TI) != 2) return pos;
  if (pos >= C / 32 * 32) return pos;
  return (pos & ~31) + 16 * ((pos >> 2) & 1) + 4 * ((pos >> 3) & 3) + (pos & 3);
}

// One k-tile-order operand unit (see KTile) of row `row` of an LDS tile in
// the kperm column order: bf16 columns 32 u + 4 q + {0..3} and 32 u + 16 +
// 4 q + {0..3} (q = lane / 16; a half unit leaves the second four zero),
// fp32 columns 16 u + 4 q + {0..3}.  It pairs with an operand unit built
// from accumulator tiles (acc_unit) over the same contraction order.
template <typename TI, bool HALF, int SW>
__device__ __forceinline__ typename Unit<TI>::type row_unit(const TI* m, int ld, int row, int u,
                                                            int lane) {
  const int q = lane >> 4;
  if constexpr (sizeof(TI) == 2) {
    const TI* base = m + row * ld;
    if constexpr (HALF) {
      const uint2 lo = *(const uint2*)(base + swz<TI, SW>(row, 32 * u + 4 * q));
      return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, 0u, 0u));
    } else {
      return *(const bf16x8*)(base + swz<TI, SW>(row, 32 * u + 8 * q));
    }
  } else {
    return *(const f32x4*)(m + row * ld + 16 * u + 4 * q);
  }
}

// The same operand unit for column c0 + lane % 16 of a row-major LDS matrix,
// contracting over its rows (the matrix read transposed): the unit holds
// rows 32 u + 4 q + {0..3} and 32 u + 16 + 4 q + {0..3} (bf16), 16 u + 4 q
// + {0..3} (fp32).  bf16 uses the LDS transpose read, which gives lane j of
// each 16-lane group element j % 4 of the 8 bytes read by lane
// 4 k + j / 4 as its element k: lane 4 k + c reads row 4 q + k (+ 32 u, then
// + 16), columns c0 + 4 c .. + 3.
template <typename TI, bool HALF, int SW>
__device__ __forceinline__ typename Unit<TI>::type col_unit(const TI* m, int ld, int c0, int u,
                                                            int lane) {
  const int q = lane >> 4, j = lane & 15;
  if constexpr (sizeof(TI) == 2) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int r = 32 * u + 4 * q + (j >> 2), c = c0 + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(m + r * ld + swz<TI, SW>(r, c)));
    s16x4 hi = {0, 0, 0, 0};
    if constexpr (!HALF)
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(m + (r + 16) * ld + swz<TI, SW>(r + 16, c)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = m[(16 * u + 4 * q + e) * ld + c0 + j];
    return v;
  }
}

// The Gram tiles (kind 0: K_rt K_j^T, j >= rt, the blocks A reads), the
// (Q K^T)^T tiles (kind 1: K_j Q_rt^T, j <= rt, the blocks P reads) and the
// diagonal Q Q^T tiles (kind 2: Q_rt Q_rt^T, whose diagonal gives q's row
// norms) held by wave w of the WY kernel, slot t (kind -1: none).  With four
// row tiles the ten tiles of each of the first two kinds go three, three,
// two, two to waves 0..3 (Gram) and 4..7 (Q K^T), and the four Q Q^T tiles
// fill the third slots of waves 2..5; with fewer (one or two), wave w
// (w - 4) takes every tile of row (column) tile w (w - 4) and wave nb + rt
// the Q Q^T tile rt.
struct WyTile {
  int kind, rt, j;
};
__host__ __device__ constexpr WyTile wy_tile(int nb, int w, int t) {
  if (nb == 4) {
    if (t == 2 && w >= 2 && w <= 5) return WyTile{2, w - 2, w - 2};
    constexpr int tb[8][3][2] = {{{0, 0}, {0, 1}, {0, 2}}, {{1, 1}, {1, 2}, {1, 3}},
                                 {{2, 2}, {2, 3}, {-1, -1}}, {{3, 3}, {0, 3}, {-1, -1}},
                                 {{0, 0}, {3, 0}, {-1, -1}}, {{1, 0}, {1, 1}, {-1, -1}},
                                 {{2, 0}, {2, 1}, {2, 2}}, {{3, 1}, {3, 2}, {3, 3}}};
    if (w < 0 || w > 7 || t < 0 || t > 2 || tb[w][t][0] < 0) return WyTile{-1, 0, 0};
    return WyTile{w < 4 ? 0 : 1, tb[w][t][0], tb[w][t][1]};
  }
  if (w >= 0 && w < nb) return w + t < nb ? WyTile{0, w, w + t} : WyTile{-1, 0, 0};
  if (w >= 4 && w - 4 < nb) return t <= w - 4 ? WyTile{1, w - 4, t} : WyTile{-1, 0, 0};
  if (nb <= 2 && w >= nb && w < 2 * nb) return t == 0 ? WyTile{2, w - nb, w - nb} : WyTile{-1, 0, 0};
  return WyTile{-1, 0, 0};
}
// Each row tile's Gram diagonal and Q Q^T tile is held exactly once.
__host__ __device__ constexpr bool wy_tiles_cover(int nb) {
  for (int rt = 0; rt < nb; ++rt) {
    int kdiag = 0, qdiag = 0;
    for (int w = 0; w < 8; ++w)
      for (int t = 0; t < 3; ++t) {
        const WyTile T = wy_tile(nb, w, t);
        if (T.kind == 0 && T.rt == rt && T.j == rt) ++kdiag;
        if (T.kind == 2 && T.rt == rt) ++qdiag;
      }
    if (kdiag != 1 || qdiag != 1) return false;
  }
  return true;
}
static_assert(wy_tiles_cover(1) && wy_tiles_cover(2) && wy_tiles_cover(4), "diagonal tiles");

// A compile-time integer passed as a value, and a dispatch of a runtime
// value in [I, N) to f(IntC<value>) (f is not called for values outside).
template <int V>
struct IntC {
  static constexpr int value = V;
};
template <int I, int N, typename F>
__device__ __forceinline__ void dispatch_int(int v, F& f) {
  if constexpr (I < N) {
    if (v == I) f(IntC<I>{});
    else dispatch_int<I + 1, N>(v, f);
  }
}

// A compile-time flag passed as a value (selects a branch-free product pass).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

constexpr int kWyThreads = 512;  // 8 waves, one workgroup per CU

// LDS plan of the WY kernel (bytes).  bf16 tiles are stored unpadded with
// row-swizzled 16-byte granules; fp32 tiles (and fp32 inputs) use rows padded
// by 16 bytes.  K and V stay as the rows they arrive in: the products that
// contract over the chunk read them transposed (col_unit).  Regions are
// reused as their contents die:
//   kv  K rows [C][dk]                                       whole item
//   v   V rows [C][128]                                      per value head
//   t   T (f32)
//   x   Q rows [C][dk] -> P [C][C] beside A (f32) -> P beside Tb, Tv
template <typename TI, int C, int DK>
struct WyLayout {
  static constexpr int S = sizeof(TI);
  static constexpr bool SWIZ = S == 2;
  static constexpr int PK = SWIZ ? 0 : 16 / S;
  static constexpr int DVM = 128;  // largest d_v and d_k
  static_assert(DK <= DVM, "d_k up to 128");
  static constexpr int LK = DK + PK;
  static constexpr int LV = DVM + PK;
  static constexpr int LC = C + PK;
  static constexpr int LF = C + 4;
  static constexpr int SWK = SWIZ ? DK / 8 - 1 : 0;
  static constexpr int SWC = SWIZ ? C / 8 - 1 : 0;
  static constexpr int SWV = SWIZ ? DVM / 8 - 1 : 0;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int r_kv = 0;
  static constexpr int r_v = r_kv + C * LK * S;
  static constexpr int r_t = r_v + C * LV * S;
  static constexpr int sz_t = C * LF * 4;
  static constexpr int r_x = r_t + sz_t;
  static constexpr int sz_p = C * LC * S;  // one [C][C] tile set (P, Tb or Tv)
  static constexpr int sz_x = cmax(cmax(C * LK * S, sz_p + C * LF * 4), 3 * sz_p);
  static constexpr int r_vec = r_x + sz_x;
  static constexpr int r_gate = r_vec + 7 * C * 4;  // g, beta of the first value head
  // The short convolution (GDN_FLAG_QKV_CONV): taps (f32, flat [d][W]) and
  // up to KW - 1 history rows (unswizzled) of q and k, used before the Gram
  // products, and of one value head's v, used as its V rows are stored.
  // The q, k part sits in the V and T regions, which hold nothing until the
  // first V rows are stored and T is formed, where they are large enough.
  static constexpr int KW = kConvMaxWidth;
  static constexpr int h_qk = (KW - 1) * DK * S;  // one history block of q or k
  static constexpr int t_qk = DK * KW * 4;        // one tap block of q or k
  static constexpr int qk_need = 2 * h_qk + 2 * t_qk;
  static constexpr int h_v = (KW - 1) * DVM * S;
  static constexpr int v_need = h_v + DVM * KW * 4;
  static constexpr bool qk_in_vt = C * LV * S + sz_t >= qk_need;
  static constexpr int plain = r_gate + 2 * C * 4;  // the kernel without the convolution
  static constexpr int r_cv = plain;  // v history, then v taps
  static constexpr int r_cqk = qk_in_vt ? r_v : r_cv + v_need;  // q, k history, then q, k taps
  static constexpr int total = r_cv + v_need + (qk_in_vt ? 0 : qk_need);
};

// Issues LDS-direct copies of rows 0 .. R-1 of a row-major LDS region (row
// stride LDR elements, granule swizzle SW) from global rows src + r * st,
// D elements each: every 16-byte slot of the region fetches the global
// granule stored there, so the copy lands in the swizzled layout directly.
// Rows r >= n and slots past the data are left alone (the caller zeroes the
// rows).  The 1 KiB pieces are spread over the NW waves.
template <typename TI, int R, int LDR, int SW, int NW>
__device__ __forceinline__ void dma_rows(char* region, const TI* src, int64_t st, int D, int n,
                                         int wave, int lane) {
  constexpr int S = sizeof(TI), GE = 16 / S;
  constexpr int BYTES = R * LDR * S;
  constexpr int PIECES = (BYTES + 1023) / 1024;
  for (int pc = wave; pc < PIECES; pc += NW) {
    const int o = pc * 1024 + lane * 16;
    const int row = o / (LDR * S), ce = (o % (LDR * S)) / S;
    const int gcol = ((ce / GE) ^ (row & SW)) * GE;
    if (o < BYTES && row < n && gcol < D)
      __builtin_amdgcn_global_load_lds((const void*)(src + row * st + gcol),
                                       (__attribute__((address_space(3))) void*)(region + pc * 1024),
                                       16, 0, 0);
  }
}

// Issues LDS-direct copies of `bytes` (a multiple of 16) contiguous bytes
// from src to region, 1 KiB pieces spread over the NW waves.
template <int NW>
__device__ __forceinline__ void dma_flat(char* region, const char* src, int bytes, int wave,
                                         int lane) {
  for (int pc = wave; pc * 1024 < bytes; pc += NW) {
    const int o = pc * 1024 + lane * 16;
    if (o < bytes)
      __builtin_amdgcn_global_load_lds((const void*)(src + o),
                                       (__attribute__((address_space(3))) void*)(region + pc * 1024),
                                       16, 0, 0);
  }
}

// The short convolution's inputs beside one block of d channels: its taps
// (flat [d][W] f32) and its W - 1 history rows, from the inputs' rows before
// the chunk (src, row stride st) or, at a sequence's first chunk, from the
// history array (null: left for the caller to zero).  ch: the block's first
// channel among the D of q | k | v.
template <typename TI, int LDR, int NW>
__device__ __forceinline__ void conv_fetch(char* hist, char* taps, const WyParams& p, bool first,
                                           int seq, const TI* src, int64_t st, int ch, int d,
                                           int wave, int lane) {
  const int W = p.conv_width;
  dma_flat<NW>(taps, (const char*)(p.conv_w + (int64_t)ch * W), d * W * 4, wave, lane);
  if (W < 2) return;
  if (first) {
    if (p.conv_state)
      dma_rows<TI, 3, LDR, 0, NW>(hist, (const TI*)p.conv_state + (int64_t)seq * (W - 1) * p.conv_d + ch,
                                  p.conv_d, d, W - 1, wave, lane);
  } else {
    dma_rows<TI, 3, LDR, 0, NW>(hist, src - (int64_t)(W - 1) * st, st, d, W - 1, wave, lane);
  }
}

// The inputs of the chunk (first token t0, n tokens) for key head kh: q, k
// rows and the first value head's v rows and gates, copied straight into
// their LDS regions (no registers); with the short convolution also the
// taps and history rows of q, k and that value head's v.
template <typename TI, int C, int DK, bool CONV>
__device__ __forceinline__ void wy_fetch(char* buf, const WyParams& p, int kh, int t0, int n,
                                         bool first, int seq, int wave, int lane) {
  using L = WyLayout<TI, C, DK>;
  constexpr int NW = kWyThreads / 64;
  const int h = kh * (p.hv / p.hk);
  dma_rows<TI, C, L::LK, L::SWK, NW>(buf + L::r_kv, (const TI*)p.k + (int64_t)t0 * p.k_st + kh * p.k_sh,
                                     p.k_st, DK, n, wave, lane);
  dma_rows<TI, C, L::LK, L::SWK, NW>(buf + L::r_x, (const TI*)p.q + (int64_t)t0 * p.q_st + kh * p.q_sh,
                                     p.q_st, DK, n, wave, lane);
  if (wave == NW - 1 && lane < n) {
    __builtin_amdgcn_global_load_lds((const void*)(p.g + (int64_t)(t0 + lane) * p.g_st + h * p.g_sh),
                                     (__attribute__((address_space(3))) void*)(buf + L::r_gate), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(p.beta + (int64_t)(t0 + lane) * p.b_st + h * p.b_sh),
                                     (__attribute__((address_space(3))) void*)(buf + L::r_gate + C * 4),
                                     4, 0, 0);
  }
  if constexpr (CONV) {
    static_assert(L::KW - 1 <= 3, "history rows fit the copies below");
    char* qk = buf + L::r_cqk;
    conv_fetch<TI, DK, NW>(qk, qk + 2 * L::h_qk, p, first, seq,
                           (const TI*)p.q + (int64_t)t0 * p.q_st + kh * p.q_sh, p.q_st, kh * DK, DK,
                           wave, lane);
    conv_fetch<TI, DK, NW>(qk + L::h_qk, qk + 2 * L::h_qk + L::t_qk, p, first, seq,
                           (const TI*)p.k + (int64_t)t0 * p.k_st + kh * p.k_sh, p.k_st,
                           (p.hk + kh) * DK, DK, wave, lane);
    conv_fetch<TI, L::DVM, NW>(buf + L::r_cv, buf + L::r_cv + L::h_v, p, first, seq,
                               (const TI*)p.v + (int64_t)t0 * p.v_st + h * p.v_sh, p.v_st,
                               2 * p.hk * DK + h * p.dv, p.dv, wave, lane);
  }
}
// One workgroup per (chunk, key head) item, under 128 VGPRs and 80 KiB of
// LDS so that two workgroups share a compute unit and hide each other's
// barriers and latencies.  CONV: the short convolution is on (a separate
// build of the kernel, so that its code costs the plain kernel nothing).
template <typename TI, int C, int DK, bool CONV>
__global__ __launch_bounds__(kWyThreads, 4) void wy_kernel(WyParams p) {
  using L = WyLayout<TI, C, DK>;
  constexpr int NT = kWyThreads;
  constexpr int LK = L::LK, LV = L::LV, LC = L::LC, LF = L::LF;
  constexpr int SWK = L::SWK, SWC = L::SWC, SWV = L::SWV;
  constexpr int GR = Gran<TI>::n;
  constexpr int NB = C / 16;    // 16-row tiles along the chunk
  constexpr int NKT = DK / 16;  // 16-row tiles along d_k
  constexpr int NVG = (C * (128 / GR) + NT - 1) / NT;  // v granules per thread (d_v <= 128)
  __shared__ __attribute__((aligned(1024))) char smem[CONV ? L::total : L::plain];

  const int it = blockIdx.x;
  if (it >= p.n_items) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TI* vg = (const TI*)p.v;
  const int DV = p.dv;
  const int GPRV = DV / GR;  // granules per v row: a power of two (d_v is 16 .. 128)
  const int LGV = __builtin_ctz(GPRV);
  const int NVT = DV / 16;
  const int grp = p.hv / p.hk;
  TI* sKV = (TI*)(smem + L::r_kv);   // K rows | V^T
  TI* sVr = (TI*)(smem + L::r_v);    // V rows
  float* sT = (float*)(smem + L::r_t);
  TI* sQ = (TI*)(smem + L::r_x);     // Q rows
  TI* sP = (TI*)(smem + L::r_x);
  float* sA = (float*)(smem + L::r_x + L::sz_p);
  TI* sTb = (TI*)(smem + L::r_x + L::sz_p);
  TI* sTv = sTb + C * LC;
  float* sRq = (float*)(smem + L::r_vec);
  float* sRk = sRq + C;
  float* sGam = sRk + C;
  float* sBeta = sGam + C;
  float* sEg = sBeta + C;   // e^gamma_r
  float* sKs = sEg + C;     // rk_r e^(gamma_last - gamma_r)
  float* sCb = sKs + C;     // beta_s e^gamma_s rk_s  (column scale of Tb)
  const float* sGate = (const float*)(smem + L::r_gate);

  // Chunks are taken last first: the scan reads the first chunks first, and
  // those, written last, are the likeliest to be still in the memory-side
  // cache when the intermediates do not all fit there.
  const int c = p.n_items / p.hk - 1 - it / p.hk, kh = it % p.hk;
  int seq, t0, n;
  if (!chunk_info(p.map, c, C, seq, t0, n)) return;
  // The short convolution: a sequence's first chunk takes its history rows
  // from the history array, the others from the rows before them.
  constexpr bool conv = CONV;
  bool first = false;
  if constexpr (conv)
    first = p.map.packed ? t0 == p.map.seq_start[seq] : !p.conv_cont && t0 == seq * p.map.seq_stride;
  const bool zero_hist = conv && first && !p.conv_state && p.conv_width > 1;
  wy_fetch<TI, C, DK, CONV>(smem, p, kh, t0, n, first, seq, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n < C || zero_hist) {
    // rows past the chunk's end are zero (the copies skipped them), and so
    // is a fresh sequence's history
    for (int idx = tid; idx < (C - n) * LK; idx += NT) {
      sKV[n * LK + idx] = from_float<TI>(0.f);
      sQ[n * LK + idx] = from_float<TI>(0.f);
    }
    if (tid < C - n) {
      ((float*)sGate)[n + tid] = 0.f;
      ((float*)sGate)[C + n + tid] = 0.f;
    }
    if (zero_hist) {
      TI* hqk = (TI*)(smem + L::r_cqk);  // q and k history blocks, back to back
      for (int idx = tid; idx < 2 * L::h_qk / (int)sizeof(TI); idx += NT) hqk[idx] = from_float<TI>(0.f);
      TI* hv = (TI*)(smem + L::r_cv);
      for (int idx = tid; idx < L::h_v / (int)sizeof(TI); idx += NT) hv[idx] = from_float<TI>(0.f);
    }
    __syncthreads();
  }
  if constexpr (conv) {
    // q and k rows through the convolution (and silu), in place: each
    // thread takes RB consecutive rows of one 16-byte column of q or k,
    // walks the rows from W - 1 before them once with the column's taps in
    // registers, and stores its results after every thread has read its
    // raw rows
    auto qk_pass = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
      constexpr int GE = 16 / (int)sizeof(TI), GPR = DK / GE;
      constexpr int RB = 2 * C * GPR / NT < 1 ? 1 : 2 * C * GPR / NT;
      constexpr int NBLK = C / RB;
      static_assert(2 * GPR * NBLK <= NT && C % RB == 0, "one column block per thread");
      const int m = tid / (GPR * NBLK), gc = (tid / NBLK) % GPR, r0 = (tid % NBLK) * RB;
      const bool live = tid < 2 * GPR * NBLK && r0 < n;
      uint4 res[RB];
      if (live) {
        const TI* rows = m ? sKV : sQ;
        const TI* hist = (const TI*)(smem + L::r_cqk + m * L::h_qk) + gc * GE;
        const float* tp = (const float*)(smem + L::r_cqk + 2 * L::h_qk + m * L::t_qk) + gc * GE * W;
        float taps[GE][W], acc[RB][GE];
#pragma unroll
        for (int e = 0; e < GE; ++e)
#pragma unroll
          for (int j = 0; j < W; ++j) taps[e][j] = tp[e * W + j];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int e = 0; e < GE; ++e) acc[i][e] = 0.f;
        // window row t is row r0 - (W - 1) + t; it feeds output row i = t - j
        // with tap j (so each output sums its taps in order)
#pragma unroll
        for (int t = 0; t < RB + W - 1; ++t) {
          const int rr = r0 - (W - 1) + t;
          const uint4 raw = ld16(rr >= 0 ? rows + rr * LK + ((gc ^ (rr & SWK)) * GE) : hist + (rr + W - 1) * DK);
          TI x[GE];
          __builtin_memcpy(x, &raw, 16);
#pragma unroll
          for (int j = 0; j < W; ++j) {
            const int i = t - j;
            if (i < 0 || i >= RB) continue;
#pragma unroll
            for (int e = 0; e < GE; ++e) acc[i][e] += taps[e][j] * to_float(x[e]);
          }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          TI y[GE];
#pragma unroll
          for (int e = 0; e < GE; ++e) y[e] = conv_act<TI>(acc[i][e], p.qkv_silu);
          __builtin_memcpy(&res[i], y, 16);
        }
      }
      __syncthreads();
      if (live) {
        TI* rows = m ? sKV : sQ;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int r = r0 + i;
          if (r < n) st16(rows + r * LK + ((gc ^ (r & SWK)) * GE), res[i]);  // padded rows stay zero
        }
      }
      __syncthreads();
    };
    dispatch_int<1, L::KW + 1>(p.conv_width, qk_pass);
  } else if (p.qkv_silu) {
    // the activation on the q and k rows in place (elementwise, so the
    // granule swizzle does not matter; silu(0) = 0 keeps padded rows zero)
    constexpr int GE = 16 / (int)sizeof(TI), GPR = DK / GE;
    for (int idx = tid; idx < 2 * C * GPR; idx += NT) {
      const int m = idx / (C * GPR), r = (idx / GPR) % C, g = idx % GPR;
      TI* e = (m ? sKV : sQ) + r * LK + g * GE;
      const uint4 raw = ld16(e);
      TI x[GE];
      __builtin_memcpy(x, &raw, 16);
#pragma unroll
      for (int j = 0; j < GE; ++j) x[j] = from_float<TI>(qkv_act<TI>(to_float(x[j])));
      uint4 out;
      __builtin_memcpy(&out, x, 16);
      st16(e, out);
    }
    __syncthreads();
  }
  if (conv || p.qkv_silu) {
    // the chunk's key rows as used out for the scan, unswizzled, in the
    // token layout of a contiguous [T][Hk][dk] tensor
    constexpr int GE = 16 / (int)sizeof(TI), GPR = DK / GE;
    TI* ka = (TI*)p.k_act + ((int64_t)t0 * p.hk + kh) * DK;
    for (int idx = tid; idx < n * GPR; idx += NT) {
      const int r = idx / GPR, g = idx % GPR;
      st16(ka + (int64_t)r * p.hk * DK + ((g ^ (r & SWK)) * GE), ld16(sKV + r * LK + g * GE));
    }
  }

  uint4 vreg[NVG];
  float gv = 0.f, bv = 0.f;
  // v rows and gates of value head h (heads after the first of a group go
  // through registers, one head ahead)
  auto load_head = [&](int h, bool gates) {
    // thread indices re-read here, so the addresses are formed at the call
    // and not kept live across the value-head loop
    int tid_l;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid_l) : "v"(tid));
    const int lane = tid_l & 63;
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const int idx = tid_l + i * NT;
      const int r = idx >> LGV, gc = idx & (GPRV - 1);
      vreg[i] = make_uint4(0, 0, 0, 0);
      if (idx < C * GPRV && r < n) vreg[i] = ld16(vg + (int64_t)(t0 + r) * p.v_st + h * p.v_sh + gc * GR);
    }
    if (!gates) return;
    if (wave == 0 && lane < n) {
      gv = p.g[(int64_t)(t0 + lane) * p.g_st + h * p.g_sh];
      bv = p.beta[(int64_t)(t0 + lane) * p.b_st + h * p.b_sh];
    } else {
      gv = 0.f;
      bv = 0.f;
    }
  };
  // The short convolution of value head h's V rows, stored raw in the V
  // region: its taps and history rows (the group's first head's came with
  // the chunk's inputs), then every result from the raw rows, then stored.
  auto conv_v = [&](int gi_, int h_, int tid_s) {
    const int W = p.conv_width;
    TI* hv = (TI*)(smem + L::r_cv);
    float* tv = (float*)(smem + L::r_cv + L::h_v);
    if (gi_ > 0) {
      const int ch = 2 * p.hk * DK + h_ * DV;
      for (int idx = tid_s; idx < DV * W / 4; idx += NT)
        ((f32x4*)tv)[idx] = ((const f32x4*)(p.conv_w + (int64_t)ch * W))[idx];
      for (int idx = tid_s; idx < (W - 1) * GPRV; idx += NT) {
        const int r = idx >> LGV, gc = idx & (GPRV - 1);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (!first)
          x = ld16(vg + (int64_t)(t0 - (W - 1) + r) * p.v_st + h_ * p.v_sh + gc * GR);
        else if (p.conv_state)
          x = ld16((const TI*)p.conv_state + ((int64_t)seq * (W - 1) + r) * p.conv_d + ch + gc * GR);
        st16(hv + r * L::DVM + gc * GR, x);
      }
    }
    __syncthreads();
    // as the q, k pass: RB consecutive rows of one 16-byte column per thread
    auto v_pass = [&](auto wc) {
      constexpr int WC = decltype(wc)::value;
      constexpr int GMAX = L::DVM / GR;  // columns of the widest d_v
      constexpr int RB = C * GMAX / NT < 1 ? 1 : C * GMAX / NT;
      constexpr int NBLK = C / RB;
      static_assert(GMAX * NBLK <= NT && C % RB == 0, "one column block per thread");
      const int gc = tid_s / NBLK, r0 = (tid_s % NBLK) * RB;
      const bool live = gc < GPRV && r0 < n;
      uint4 res[RB];
      if (live) {
        const float* tp = tv + gc * GR * WC;
        float taps[GR][WC], acc[RB][GR];
#pragma unroll
        for (int e = 0; e < GR; ++e)
#pragma unroll
          for (int j = 0; j < WC; ++j) taps[e][j] = tp[e * WC + j];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int e = 0; e < GR; ++e) acc[i][e] = 0.f;
#pragma unroll
        for (int t = 0; t < RB + WC - 1; ++t) {
          const int rr = r0 - (WC - 1) + t;
          const uint4 raw = ld16(rr >= 0 ? sVr + rr * LV + swz<TI, SWV>(rr, gc * GR)
                                         : hv + (rr + WC - 1) * L::DVM + gc * GR);
          TI x[GR];
          __builtin_memcpy(x, &raw, 16);
#pragma unroll
          for (int j = 0; j < WC; ++j) {
            const int i = t - j;
            if (i < 0 || i >= RB) continue;
#pragma unroll
            for (int e = 0; e < GR; ++e) acc[i][e] += taps[e][j] * to_float(x[e]);
          }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          TI y[GR];
#pragma unroll
          for (int e = 0; e < GR; ++e) y[e] = conv_act<TI>(acc[i][e], p.qkv_silu);
          __builtin_memcpy(&res[i], y, 16);
        }
      }
      __syncthreads();
      if (live) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int r = r0 + i;
          if (r < n) st16(sVr + r * LV + swz<TI, SWV>(r, gc * GR), res[i]);  // padded rows stay zero
        }
      }
    };
    dispatch_int<1, L::KW + 1>(W, v_pass);
  };
  // V rows from the registers load_head filled (rows past the chunk's end
  // are zero) into the V region (through the convolution when it is on;
  // the caller's barrier follows)
  auto store_v = [&](int gi_, int h_) {
    int tid_s;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid_s) : "v"(tid));
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const int idx = tid_s + i * NT;
      if (idx < C * GPRV) {
        const int r = idx >> LGV, gc = idx & (GPRV - 1);
        uint4 vv = vreg[i];
        if (p.qkv_silu && !conv) {
          TI x[GR];
          __builtin_memcpy(x, &vv, 16);
#pragma unroll
          for (int j = 0; j < GR; ++j) x[j] = from_float<TI>(qkv_act<TI>(to_float(x[j])));
          __builtin_memcpy(&vv, x, 16);
        }
        st16(sVr + r * LV + swz<TI, SWV>(r, gc * GR), vv);
      }
    }
    if constexpr (conv) conv_v(gi_, h_, tid_s);
  };
  // The first value head's V rows go to registers (its gates came with the
  // q, k rows): they arrive while the Gram products, A, P and T are formed.
  // (LDS-direct copies would not do: every LDS read would wait for them.)
  load_head(kh * grp, false);

  // Raw K K^T and Q K^T tiles (the wave's slots, see wy_tile).  They stay
  // in registers for all value heads of the group; norms and gates are
  // applied when A and P are built.  The inverse row norms of k and q come
  // from the diagonals of the Gram and Q Q^T tiles.
  constexpr int NSLOT = NB == 4 ? 3 : NB;
  f32x4 acc_gs[NSLOT];
#pragma unroll
  for (int t = 0; t < NSLOT; ++t) acc_gs[t] = zero4();
  auto gram_tiles = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) {
      const WyTile T = wy_tile(NB, W, t);
      if (T.kind < 0) continue;
      f32x4 acc1[1][1] = {{zero4()}};
      if (T.kind == 0)  // K_rt K_j^T: lane holds column 16 j + lane % 16
        mma_block_sw<1, 1, DK, SWK, SWK>(acc1, sKV, LK, 16 * T.rt, sKV, LK, 16 * T.j, lane);
      else if (T.kind == 1)  // K_j Q_rt^T: lane holds query 16 rt + lane % 16, four consecutive keys
        mma_block_sw<1, 1, DK, SWK, SWK>(acc1, sKV, LK, 16 * T.j, sQ, LK, 16 * T.rt, lane);
      else  // Q_rt Q_rt^T
        mma_block_sw<1, 1, DK, SWK, SWK>(acc1, sQ, LK, 16 * T.rt, sQ, LK, 16 * T.rt, lane);
      acc_gs[t] = acc1[0][0];
    }
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) settle(acc_gs[t]);
    // a diagonal tile (rt, rt): lane m + 16 (m / 4) holds the squared norm of
    // row 16 rt + m as element m % 4
    auto diag_norms = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr WyTile T = wy_tile(NB, W, t);
      if constexpr ((T.kind == 0 && T.rt == T.j) || T.kind == 2) {
        const int m = lane & 15;
        if ((m >> 2) == (lane >> 4)) {
          float d = acc_gs[t][0];
          if ((m & 3) == 1) d = acc_gs[t][1];
          if ((m & 3) == 2) d = acc_gs[t][2];
          if ((m & 3) == 3) d = acc_gs[t][3];
          (T.kind == 0 ? sRk : sRq)[16 * T.rt + m] = 1.0f / sqrtf(d + p.eps);
        }
      }
    };
    diag_norms(IntC<0>{});
    if constexpr (NSLOT > 1) diag_norms(IntC<1>{});
    if constexpr (NSLOT > 2) diag_norms(IntC<2>{});
  };
  dispatch_int<0, kWyThreads / 64>(wave, gram_tiles);
  // The gate cumulative sum gamma, beta (sigmoid of a logit for a real
  // token; padded rows stay 0) and e^gamma of the value head whose g and
  // beta are in gv, bv (wave 0).
  auto gate_scan = [&](int h) {
    float x = gv;  // inclusive scan over the chunk
    if (p.decay_proj && lane < n) x = decay_gate(x, p.a_log, p.a_bias, h);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane < C) {
      sGam[lane] = x;
      if (p.beta_logits && lane < n) bv = 1.f / (1.f + fast_exp(-bv));
      sBeta[lane] = bv;
      sEg[lane] = fast_exp(x);
    }
  };
  if (wave == 0) {
    gv = sGate[lane < C ? lane : 0];
    bv = sGate[C + (lane < C ? lane : 0)];
    if (lane >= C) gv = bv = 0.f;
    gate_scan(kh * grp);  // the first value head's, beside the Gram products
  }
  // The q elements this wave needs for Q' (d_k tile `wave`, rows
  // 16 j + lane % 16, four columns from 4 (lane / 16)) for every value head
  // of the group, read before their LDS region is reused: q leaves HBM once.
  typename Raw4<TI>::type qraw[NB];
  if (wave < NKT) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = 16 * j + (lane & 15), dk0 = 16 * wave + (lane >> 4) * 4;
      qraw[j] = *(const typename Raw4<TI>::type*)(sQ + r * LK + swz<TI, SWK>(r, dk0));
    }
  }
  __syncthreads();

  for (int gi = 0; gi < grp; ++gi) {
    const int h = kh * grp + gi;
    const int64_t blk = (int64_t)c * p.hv + h;
    // re-read thread indices per head (see the item loop): the addresses of
    // each phase are computed where they are used, not all up front
    int tid_h;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid_h) : "v"(tid));
    const int tid = tid_h, lane = tid_h & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid_h >> 6);

    // Later value heads: v rows into the T region (the first head's are
    // there already) and the gate scan.  Then the next value head's inputs
    // are requested.
    if (gi > 0) {
      store_v(gi, h);
      if (wave == 0) gate_scan(h);
      __syncthreads();
    }

    // A from the K K^T tiles:
    // A_rs = beta_r exp(gamma_r - gamma_s) rk_r rk_s (k_r . k_s), s < r
    // (only the strictly lower part is ever read), and
    // P = scale D o (Q^K^T) from the (Q K^T)^T tiles, from each wave's slots.
    auto build_ap = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
#pragma unroll
      for (int t = 0; t < NSLOT; ++t) {
        const WyTile T = wy_tile(NB, W, t);
        if (T.kind == 0) {
          // the Gram tile (rt, j) read transposed (K K^T is symmetric): lane
          // holds row r = 16 j + lane % 16 and the four consecutive columns
          // c = 16 rt + 4 (lane / 16) + e
          const int c0 = 16 * T.rt + (lane >> 4) * 4;
          const f32x4 gc = *(const f32x4*)(sGam + c0), rkc = *(const f32x4*)(sRk + c0);
          const int r = 16 * T.j + (lane & 15);
          const float br = sBeta[r] * sRk[r], gr = sGam[r];
          f32x4 a;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a[e] = (c0 + e < r) ? br * rkc[e] * fast_exp(gr - gc[e]) * acc_gs[t][e] : 0.f;
          *(f32x4*)(sA + r * LF + c0) = a;
        } else if (T.kind == 1) {
          // lane holds query row r = 16 rt + lane % 16 and the four
          // consecutive keys s = 16 j + 4 (lane / 16) + e
          const int r = 16 * T.rt + (lane & 15);
          const float qr = p.scale * sRq[r], gr = sGam[r];
          const int s0 = 16 * T.j + (lane >> 4) * 4;
          const f32x4 gs = *(const f32x4*)(sGam + s0), rks = *(const f32x4*)(sRk + s0);
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[e] = (s0 + e <= r) ? qr * rks[e] * fast_exp(gr - gs[e]) * acc_gs[t][e] : 0.f;
          store4<TI>(sP + r * LC + swz<TI, SWC>(r, kperm<TI, C>(s0)), pv[0], pv[1], pv[2], pv[3]);
        }
      }
      constexpr WyTile T0 = wy_tile(NB, W, 0);
      if constexpr (T0.kind == 1) {
        // P is zero right of the diagonal tile of the wave's first row tile
        const int r = 16 * T0.rt + (lane & 15);
#pragma unroll
        for (int j = T0.rt + 1; j < NB; ++j) {
          const int s0 = 16 * j + (lane >> 4) * 4;
          store4<TI>(sP + r * LC + swz<TI, SWC>(r, kperm<TI, C>(s0)), 0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    dispatch_int<0, kWyThreads / 64>(wave, build_ap);
    if (wave == NB - 1 && lane < C) {
      // the row scale s_r = rk_r e^(gamma_last - gamma_r) of the stored W
      // and U~, and Tb's column scale beta_s e^gamma_s rk_s
      const float rk = sRk[lane];
      sKs[lane] = rk * fast_exp(sGam[C - 1] - sGam[lane]);
      sCb[lane] = sBeta[lane] * sEg[lane] * rk;
    }
    __syncthreads();

    // T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution, one
    // lane per column; then the blocks below the diagonal,
    //   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj   (fp32 MFMA, block column j
    // on wave j).
    if (wave == 0) {
      const int b = lane >> 4, col = lane & 15;
      if (b < NB) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
        const float* Ab = sA + (16 * b) * LF + 16 * b;
        // row r + 1's entries (16-byte reads; the block is zero on and above
        // its diagonal) are requested while row r's sums run
        f32x4 cur[4], nxt[4];
        cur[0] = *(const f32x4*)(Ab + LF);
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          if (r + 1 < 16) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (4 * v < r + 1) nxt[v] = *(const f32x4*)(Ab + (r + 1) * LF + 4 * v);
          }
          float a0 = x[r], a1 = 0.f;  // two independent partial sums
#pragma unroll
          for (int s2 = 0; s2 < r; ++s2) {
            if (s2 & 1) a1 -= cur[s2 >> 2][s2 & 3] * x[s2];
            else a0 -= cur[s2 >> 2][s2 & 3] * x[s2];
          }
          x[r] = a0 + a1;
#pragma unroll
          for (int v = 0; v < 4; ++v) cur[v] = nxt[v];
          // one row's operands in flight at a time: keeps the register
          // footprint small
          __builtin_amdgcn_sched_barrier(0);
        }
        float* Tb = sT + (16 * b) * LF + 16 * b;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * LF + col] = x[i];
      }
    }
    __syncthreads();
    // Wave j takes block column j down the rows: every T_kj its sums need
    // is one it made itself, kept in registers in the accumulator layout
    // (lane (r, q) holds rows 4 q + e of column r), which is the second
    // operand's layout for the next product, so the column needs no
    // exchange and no barrier between block rows.  All A blocks and
    // diagonal T blocks of the column are read first, and each term
    // A_ik T_kj enters its sum as soon as T_kj is known (in k order), so
    // the chain of dependent products holds only one term per block.
    auto off_diag = [&](auto bjc) {
      constexpr int BJ = decltype(bjc)::value;
      constexpr int ND = NB - BJ;  // blocks of the column, the diagonal one included
      const int r = lane & 15, q = lane >> 4;
      f32x4 ab[ND][ND], td[ND], tcol[ND], m[ND];
#pragma unroll
      for (int di = 1; di < ND; ++di) {
        const int bi = BJ + di;
        td[di] = *(const f32x4*)(sT + (16 * bi + r) * LF + 16 * bi + 4 * q);
#pragma unroll
        for (int dk = 0; dk < di; ++dk)
          ab[di][dk] = *(const f32x4*)(sA + (16 * bi + r) * LF + 16 * (BJ + dk) + 4 * q);
        m[di] = zero4();
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tcol[0][e] = sT[(16 * BJ + 4 * q + e) * LF + 16 * BJ + r];
      // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
      for (int dk = 0; dk + 1 < ND; ++dk) {
#pragma unroll
        for (int di = dk + 1; di < ND; ++di) mma16_f32_ab(m[di], ab[di][dk], tcol[dk]);
        const int di = dk + 1, bi = BJ + di;
        settle(m[di]);
        f32x4 t = zero4();
        mma16_f32_ab(t, td[di], m[di]);
        settle(t);
        float* dst = sT + (16 * bi) * LF + 16 * BJ;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tcol[di][e] = -t[e];
          dst[(4 * q + e) * LF + r] = -t[e];
        }
      }
    };
    dispatch_int<0, NB - 1>(wave, off_diag);
    __syncthreads();

    // Tb = T diag(beta e^gamma rk), Tv = T diag(beta), 8 stored positions
    // (kperm order) per item.
#pragma unroll
    for (int it = 0; it < (C * (C / 8) + NT - 1) / NT; ++it) {
      const int idx = tid + it * NT;
      if (C * (C / 8) % NT != 0 && idx >= C * (C / 8)) break;
      const int r = idx / (C / 8), s0 = (idx % (C / 8)) * 8;
      // the 8 stored positions s0 .. s0 + 7 are the columns c_lo + 0..3 and
      // c_hi + 0..3 (kperm within a full 32-column block, else natural)
      int c_lo = s0, c_hi = s0 + 4;
      if (sizeof(TI) == 2 && s0 < C / 32 * 32) {
        c_lo = (s0 & ~31) + 4 * ((s0 >> 3) & 3);
        c_hi = c_lo + 16;
      }
      const f32x4 tl = *(const f32x4*)(sT + r * LF + c_lo), th = *(const f32x4*)(sT + r * LF + c_hi);
      const f32x4 bl = *(const f32x4*)(sCb + c_lo), bh = *(const f32x4*)(sCb + c_hi);
      const f32x4 vl = *(const f32x4*)(sBeta + c_lo), vh = *(const f32x4*)(sBeta + c_hi);
      typedef TI vec8 __attribute__((ext_vector_type(8)));
      vec8 tb, tv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t0 = (c_lo + e <= r) ? tl[e] : 0.f, t1 = (c_hi + e <= r) ? th[e] : 0.f;
        tb[e] = from_float<TI>(t0 * bl[e]);
        tv[e] = from_float<TI>(t0 * vl[e]);
        tb[4 + e] = from_float<TI>(t1 * bh[e]);
        tv[4 + e] = from_float<TI>(t1 * vh[e]);
      }
      if constexpr (sizeof(TI) == 2) {
        *(vec8*)(sTb + r * LC + swz<TI, SWC>(r, s0)) = tb;
        *(vec8*)(sTv + r * LC + swz<TI, SWC>(r, s0)) = tv;
      } else {
        *(f32x4*)(sTb + r * LC + s0) = __builtin_shufflevector(tb, tb, 0, 1, 2, 3);
        *(f32x4*)(sTb + r * LC + s0 + 4) = __builtin_shufflevector(tb, tb, 4, 5, 6, 7);
        *(f32x4*)(sTv + r * LC + s0) = __builtin_shufflevector(tv, tv, 0, 1, 2, 3);
        *(f32x4*)(sTv + r * LC + s0 + 4) = __builtin_shufflevector(tv, tv, 4, 5, 6, 7);
      }
    }
    // this value head's V rows into LDS for U~ = Tv V (the first head's
    // arrive in registers here; later heads' were stored at the loop top),
    // then the next value head's inputs are requested
    if (gi == 0) store_v(gi, h);
    if (gi + 1 < grp) load_head(h + 1, true);
    __syncthreads();

    // Per wave, from the LDS tiles Tv, Tb, V, K and P:
    //  - U~ = Tv V for d_v tile `wave`: accumulator tiles to global memory
    //    (rows scaled by s_r), and kept as operand units of U~^T
    //    (contraction over the chunk);
    //  - W[r][dk] = sum_s Tb[r][s] K[s][dk] for d_k tile `wave`, twice from
    //    the same operand registers: W^T tiles (rows d_k, columns r, scaled
    //    by s_r) to global memory in k-tile order, and W tiles (rows r, columns d_k)
    //    kept as operand units of W^T (a K^T operand unit, rows d_k, holds
    //    the same registers as a K operand unit, columns d_k);
    //  - one pass over P's rows (in the same contraction order) feeding
    //    O_loc^T = U~^T P^T and Q'^T = scale (diag(e^gamma rq) Q)^T - W^T P^T.
    // Neither U~ nor W goes through LDS.
    {
      using KT = KTile<TI, C>;
      using UT = typename Unit<TI>::type;
      constexpr int NUF = KT::HALF_TAIL ? KT::NU - 1 : KT::NU;  // full units
      constexpr int T1 = KT::TPU == 2 ? 1 : 0;
      const int rr = lane & 15;
      const bool uv = wave < NVT, wq = wave < NKT;
      UT ua[KT::NU], wu[KT::NU];
      auto u_part = [&]() {
        TI* ut_g = (TI*)p.im.ut + blk * DV * C;
        f32x4 acc[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[i] = zero4();
#pragma unroll
        for (int u = 0; u < NUF; ++u) {
          const auto vb = col_unit<TI, false, SWV>(sVr, LV, 16 * wave, u, lane);
#pragma unroll
          for (int i = 0; i < NB; ++i)
            mma_unit<false>(acc[i], row_unit<TI, false, SWC>(sTv, LC, 16 * i + rr, u, lane), vb);
        }
        if constexpr (KT::HALF_TAIL) {
          constexpr int u = KT::NU - 1;
          const auto vb = col_unit<TI, true, SWV>(sVr, LV, 16 * wave, u, lane);
#pragma unroll
          for (int i = 0; i < NB; ++i)
            mma_unit<true>(acc[i], row_unit<TI, true, SWC>(sTv, LC, 16 * i + rr, u, lane), vb);
        }
        // stored with row r scaled by s_r (lane holds rows 16 i + 4 (lane / 16) + e)
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const f32x4 sr = *(const f32x4*)(sKs + 16 * i + (lane >> 4) * 4);
          store4<TI>(ut_g + (wave * NB + i) * 256 + lane * 4, acc[i][0] * sr[0], acc[i][1] * sr[1],
                     acc[i][2] * sr[2], acc[i][3] * sr[3]);
        }
#pragma unroll
        for (int u = 0; u < NUF; ++u) ua[u] = acc_unit<false>(acc[KT::TPU * u], acc[KT::TPU * u + T1], TI());
        if constexpr (KT::HALF_TAIL)
          ua[KT::NU - 1] = acc_unit<true>(acc[KT::TPU * (KT::NU - 1)], acc[KT::TPU * (KT::NU - 1)], TI());
      };
      const int dk0 = 16 * wave + (lane >> 4) * 4;
      auto w_part = [&]() {
        TI* w_g = (TI*)p.im.w + blk * C * DK;
        // K operand units for every chunk unit, then one row tile of W and
        // W^T at a time (each W^T tile is stored as soon as it is complete)
        typename Unit<TI>::type ka[KT::NU];
#pragma unroll
        for (int u = 0; u < NUF; ++u) ka[u] = col_unit<TI, false, SWK>(sKV, LK, 16 * wave, u, lane);
        if constexpr (KT::HALF_TAIL)
          ka[KT::NU - 1] = col_unit<TI, true, SWK>(sKV, LK, 16 * wave, KT::NU - 1, lane);
        f32x4 wr[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          f32x4 wt = zero4();
          wr[j] = zero4();
#pragma unroll
          for (int u = 0; u < NUF; ++u) {
            const auto tb = row_unit<TI, false, SWC>(sTb, LC, 16 * j + rr, u, lane);
            mma_unit<false>(wt, ka[u], tb);
            mma_unit<false>(wr[j], tb, ka[u]);
          }
          if constexpr (KT::HALF_TAIL) {
            constexpr int u = KT::NU - 1;
            const auto tb = row_unit<TI, true, SWC>(sTb, LC, 16 * j + rr, u, lane);
            mma_unit<true>(wt, ka[u], tb);
            mma_unit<true>(wr[j], tb, ka[u]);
          }
          // stored with row r = 16 j + lane % 16 scaled by s_r
          const float sr = sKs[16 * j + rr];
          store4<TI>(w_g + j * 16 * DK + KTile<TI, DK>::pos(rr, dk0), wt[0] * sr, wt[1] * sr,
                     wt[2] * sr, wt[3] * sr);
        }
#pragma unroll
        for (int u = 0; u < NUF; ++u) wu[u] = acc_unit<false>(wr[KT::TPU * u], wr[KT::TPU * u + T1], TI());
        if constexpr (KT::HALF_TAIL)
          wu[KT::NU - 1] = acc_unit<true>(wr[KT::TPU * (KT::NU - 1)], wr[KT::TPU * (KT::NU - 1)], TI());
      };
      // The pass over P (branch-free in the common case of both products).
      auto p_pass = [&](auto do_o, auto do_q) {
        constexpr bool DO = decltype(do_o)::value, DQ = decltype(do_q)::value;
        f32x4 ol[NB], pw[NB];
#pragma unroll
        for (int jr = 0; jr < NB; ++jr) ol[jr] = pw[jr] = zero4();
#pragma unroll
        for (int u = 0; u < NUF; ++u)
#pragma unroll
          for (int jr = 0; jr < NB; ++jr) {
            const auto pu = row_unit<TI, false, SWC>(sP, LC, 16 * jr + rr, u, lane);
            if constexpr (DO) mma_unit<false>(ol[jr], ua[u], pu);
            if constexpr (DQ) mma_unit<false>(pw[jr], wu[u], pu);
          }
        if constexpr (KT::HALF_TAIL) {
          constexpr int u = KT::NU - 1;
#pragma unroll
          for (int jr = 0; jr < NB; ++jr) {
            const auto pu = row_unit<TI, true, SWC>(sP, LC, 16 * jr + rr, u, lane);
            if constexpr (DO) mma_unit<true>(ol[jr], ua[u], pu);
            if constexpr (DQ) mma_unit<true>(pw[jr], wu[u], pu);
          }
        }
        if constexpr (DO) {
          TI* ol_g = (TI*)p.im.oloc + blk * C * DV;
#pragma unroll
          for (int jr = 0; jr < NB; ++jr) store_acc_tile<TI>(ol_g + (wave * NB + jr) * 256, ol[jr], lane);
        }
        if constexpr (DQ) {
          TI* qp_g = (TI*)p.im.qp + blk * C * DK;
#pragma unroll
          for (int jr = 0; jr < NB; ++jr) {
            const int r = 16 * jr + rr;
            const float qs = p.scale * sEg[r] * sRq[r];
            const f32x4 qv = raw4_to_f32<TI>(qraw[jr]);
            store4<TI>(qp_g + jr * 16 * DK + KTile<TI, DK>::pos(rr, dk0), qs * qv[0] - pw[jr][0],
                       qs * qv[1] - pw[jr][1], qs * qv[2] - pw[jr][2], qs * qv[3] - pw[jr][3]);
          }
        }
      };
      // both parts in one straight-line block where a wave has both (every
      // wave when d_k = d_v = 128), so their reads and products interleave
      if (uv && wq) {
        u_part();
        w_part();
        p_pass(BoolC<true>{}, BoolC<true>{});
      } else if (uv) {
        u_part();
        p_pass(BoolC<true>{}, BoolC<false>{});
      } else if (wq) {
        w_part();
        p_pass(BoolC<false>{}, BoolC<true>{});
      }
    }
    if (tid == 0) p.im.decay[blk] = sEg[C - 1];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// state scan fused with the output
//
// One workgroup per (sequence, value head, group of NSL 16-column slices of
// d_v), 2 NSL + 2 waves with fixed roles:
//   wave s < NSL       the recurrence of slice s: U = U~ - W H and
//                      H <- e^gamma_last H + K~^T U, with the state slice in
//                      its MFMA accumulators; at the start of each chunk it
//                      leaves -H (as bf16 / fp32 operand units) in LDS;
//   wave NSL + s       the output of slice s, one chunk behind:
//                      O = Q' H + O_loc from Q' held in registers since the
//                      previous chunk, off the recurrence's critical path;
//   the last two waves copy each chunk's W, Q' and key rows (one slice: also its
//                      U~ tiles and the decay) from global memory into a ring
//                      of LDS stages with LDS-direct loads (no registers),
//                      `lead` chunks ahead.
// One barrier per chunk hands a stage (and the H copies) over.  With more
// than one slice the recurrence waves take their U~ tiles and the decay into
// registers, two chunks ahead.
//
// A wave reads LDS at about half of what its SIMD's LDS port delivers, and
// the recurrence of one slice reads 32 KiB of W and key rows per chunk, so its
// chunk step is bound by that wave's reads, not by its MFMAs.  Slices of one
// workgroup share the ring's copies and run on separate SIMDs: two slices
// cost the compute unit about what one does.

constexpr int kScanCopyWaves = 2;

// The value head of the r-th (sequence, head) unit of a sequence.  Units
// land on XCD r % 8 (blockIdx % 8).  With key heads shared by grp > 1 value
// heads and a multiple of 8 key heads, the value heads of one key head are
// placed on one XCD, where they share its key rows through the L2:
// r = 8 y + x takes key head x + 8 (y / grp) and value head grp (x + 8 (y /
// grp)) + y % grp (a permutation of 0 .. hv - 1).  Otherwise r itself.
__device__ __forceinline__ int scan_head(int r, int grp, int hv) {
  if (grp <= 1 || (hv / grp) % 8 != 0) return r;
  const int x = r % 8, y = r / 8;
  return grp * (x + 8 * (y / grp)) + y % grp;
}

template <typename TI, int C, int DK, int NSL>
struct ScanRing {
  using Elem = TI;
  static constexpr int D = DK;
  static constexpr int S = sizeof(TI);
  static constexpr int BIG = C * DK * S;            // W, Q', K rows of one chunk
  static constexpr int SMALL = C * 16 * S;          // U~ tiles of one slice
  static constexpr bool UTR = NSL == 1;             // U~ and the decay staged too
  static constexpr int w = 0, qp = BIG, kr = 2 * BIG, ut = 3 * BIG;
  // the key rows [C][DK] are row-swizzled (bf16) for the transposed reads
  static constexpr int SWK = S == 2 ? DK / 8 - 1 : 0;
  static constexpr int dec = ut + SMALL;            // e^gamma_last (4 bytes)
  static constexpr int stage = UTR ? dec + 16 : 3 * BIG;
  static constexpr int HB = KTile<TI, DK>::NU * 1024;  // -H of one slice as operand units
  static constexpr int room = (kLdsLimit - 2 * NSL * HB) / stage;
  static constexpr int slots = room < 4 ? room : 4;
  static constexpr int lead = slots - 1;
  static constexpr int hbuf = slots * stage;        // two H buffers per slice
  static constexpr int total = hbuf + 2 * NSL * HB;
  // 1 KiB copies per stage (the last of a region may be 512 bytes), plus
  // one 4-byte copy of the decay
  static constexpr int PB = (BIG + 1023) / 1024, PS = (SMALL + 1023) / 1024;
  static constexpr int pieces = 3 * PB + (UTR ? PS + 1 : 0);
  static constexpr int per_wave = (pieces + kScanCopyWaves - 1) / kScanCopyWaves;
  static_assert(slots < 2 || per_wave * lead <= 63, "loads in flight exceed the wave's counter");
  // slice s's copy b of -H
  static constexpr int hcopy(int s, int b) { return hbuf + (2 * s + b) * HB; }
};

// Workgroup barrier that the compiler may not move memory accesses across;
// the waits it needs are issued explicitly before it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt <= n only; lgkmcnt == 0 only.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
__host__ __device__ constexpr int lgkmcnt0_imm() { return 15 | (3 << 14) | (7 << 4); }

// Copies chunk cc's operands into one LDS stage: copying wave CW's share of
// the stage's pieces (CW, CW + kScanCopyWaves, ...), each a coalesced 16
// bytes per lane.  Indices beyond the stage repeat its last piece (same
// bytes, same place), so that every copying wave issues exactly per_wave
// loads per stage.  All piece indices are compile-time constants.
template <typename R, int C, int CW>
__device__ __forceinline__ void ring_copy(char* stage, const ScanParams& p, int cc, int h,
                                          int ctile, int t0, int t_end, int lane) {
  constexpr int NB = C / 16;
  constexpr int GE = 16 / R::S;  // elements per 16-byte granule
  const int64_t blk = (int64_t)cc * p.hv + h;
  const int64_t big = blk * R::BIG, small = (blk * C * p.dv + (int64_t)ctile * NB * 256) * R::S;
  const char* bases[4] = {(const char*)p.im.w + big, (const char*)p.im.qp + big, nullptr,
                          (const char*)p.im.ut + small};
  // the chunk's key rows (of key head h / grp), row-swizzled like the WY
  // kernel's K rows; rows past the chunk's end repeat its last row (finite,
  // and the rows of U they meet are zero), so every copy issues the same
  // number of loads
  const int n = min(C, t_end - t0);
  using TI = typename R::Elem;
  constexpr int DK = R::D;
  const TI* krow = (const TI*)p.k + (int64_t)(h / p.grp) * p.k_sh;
#pragma unroll
  for (int j = 0; j < R::per_wave; ++j) {
    const int i = min(CW + kScanCopyWaves * j, R::pieces - 1);
    if (R::UTR && i == R::pieces - 1) {
      if (lane == 0)
        __builtin_amdgcn_global_load_lds((const void*)(p.im.decay + blk),
                                         (__attribute__((address_space(3))) void*)(stage + R::dec),
                                         4, 0, 0);
      continue;
    }
    const int r = i < 3 * R::PB ? i / R::PB : 3;
    const int k = i - r * R::PB;
    const int bytes = r < 3 ? R::BIG : R::SMALL;
    const int lds_off = r * R::BIG + k * 1024;
    const bool half = (bytes % 1024) != 0 && k == (bytes - 1) / 1024;
    if (half && lane >= 32) continue;
    const char* src;
    if (r == 2) {
      const int o = k * 1024 + lane * 16;          // byte offset in the [C][DK] rows
      const int row = o / (DK * R::S), slot = (o % (DK * R::S)) / 16;
      const int gcol = (slot ^ (row & R::SWK)) * GE;
      const int trow = t0 + (row < n ? row : n - 1);
      src = (const char*)(krow + (int64_t)trow * p.k_st + gcol);
    } else {
      src = bases[r] + k * 1024 + lane * 16;
    }
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(stage + lds_off),
                                     16, 0, 0);
  }
}

// Copying wave CW: fills the first `lead` stages, then one stage per chunk,
// and meets the other waves at one barrier per chunk once the stage they
// need next has landed.  Loads past the last chunk re-read it.
template <typename R, int C, int CW>
__device__ __forceinline__ void ring_producer(char* smem, const ScanParams& p, int c_begin,
                                              int c_end, int h, int ctile, int tok0, int tok_end,
                                              int lane) {
  const int last = c_end - 1;
  auto copy = [&](char* stage, int cc) {
    ring_copy<R, C, CW>(stage, p, cc, h, ctile, tok0 + (cc - c_begin) * C, tok_end, lane);
  };
#pragma unroll
  for (int k = 0; k < R::lead; ++k) copy(smem + k * R::stage, min(c_begin + k, last));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::per_wave * (R::lead - 1)));
  ring_barrier();
  int slot = R::lead;
  for (int cc = c_begin; cc < c_end; ++cc) {
    copy(smem + slot * R::stage, min(cc + R::lead, last));
    slot = slot + 1 == R::slots ? 0 : slot + 1;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::per_wave * (R::lead - 1)));
    ring_barrier();
  }
}

// -H as operand units (B of U = U~ + W (-H), A of -O^T = (-H)^T Q'^T) from
// the state's accumulator tiles.  Carrying the negated state lets U~ enter
// the MFMA as its accumulator input, so no subtraction follows the product.
template <typename TI, int DK, typename UT>
__device__ __forceinline__ void state_units(UT* hb, const f32x4* hacc) {
  using KD = KTile<TI, DK>;
#pragma unroll
  for (int q = 0; q < KD::NU; ++q) {
    const f32x4 a = -hacc[KD::TPU * q], b = -hacc[KD::TPU * q + KD::TPU - 1];
    hb[q] = (KD::HALF_TAIL && q == KD::NU - 1) ? acc_unit<true>(a, a, TI{})
                                               : acc_unit<false>(a, b, TI{});
  }
}

// One slice of the two-level scan (scan_split_kernel).
struct SliceJob {
  int first;  // 1: first segment, from the initial state; 0: second, from zero
  int phi;    // 1: transition columns: U~ = 0, O_loc = 0, identity start, Q' Phi out
  int ctile;  // column tile (of d_v; of d_k for transition columns)
};

// The output wave of slice s (column tile ctile), one chunk behind the
// recurrence: during chunk i it reads Q'_i (LDS) and O_loc_i (global) into
// registers and forms
//   O_{i-1}^T = O_loc^T - (-H_{i-1})^T Q'^T
// with -H_{i-1} as the recurrence wave left it in LDS during chunk i - 1.
// Lane holds row 16 rt + lane % 16, columns 16 ctile + 4 (lane / 16) + 0..3.
// In the two-level scan (SPLIT) a transition slice writes Q'_i Phi_i (all
// rows) to the workspace instead.
template <typename TI, int C, int DK, int NSL, bool SPLIT = false>
__device__ __forceinline__ void scan_output(char* smem, const ScanParams& p, int h, int s,
                                            int ctile, int c_begin, int nch, int tok0,
                                            int tok_end, int lane, SliceJob job = {}) {
  using R = ScanRing<TI, C, DK, NSL>;
  using KD = KTile<TI, DK>;
  using UT = typename Unit<TI>::type;
  typedef typename Raw4<TI>::type RT;
  constexpr int NB = C / 16;
  constexpr int S = R::S;
  const int DV = p.dv;
  TI* outg = (TI*)p.out;
  struct OBuf {
    UT q[NB][KD::NU];
    RT ol[NB];
  };
  auto fetch = [&](OBuf& o, int i, int slot) {
    const char* st = smem + slot * R::stage;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int q = 0; q < KD::NU; ++q) {
        const char* qu = st + R::qp + rt * 16 * DK * S + q * KD::UNIT * S;
        o.q[rt][q] = (KD::HALF_TAIL && q == KD::NU - 1) ? lds_unit<TI, true>(qu, lane)
                                                        : lds_unit<TI, false>(qu, lane);
      }
    const TI* src = (const TI*)p.im.oloc + ((int64_t)(c_begin + i) * p.hv + h) * C * DV +
                    (int64_t)ctile * NB * 256 + lane * 4;
    if (SPLIT && job.phi) {
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) o.ol[rt] = RT{};
    } else {
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) o.ol[rt] = load_raw4<TI>(src + rt * 256);
    }
  };
  auto emit = [&](const OBuf& o, int i) {
    const char* hsrc = smem + R::hcopy(s, i & 1);
    UT ha[KD::NU];
#pragma unroll
    for (int q = 0; q < KD::NU; ++q) ha[q] = lds_unit<TI, false>(hsrc + q * 1024, lane);
    f32x4 ao[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) ao[rt] = zero4();
#pragma unroll
    for (int q = 0; q < KD::NU; ++q)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        if (KD::HALF_TAIL && q == KD::NU - 1) mma_unit<true>(ao[rt], ha[q], o.q[rt][q]);
        else mma_unit<false>(ao[rt], ha[q], o.q[rt][q]);
      }
    const int tok = tok0 + i * C;
    if (SPLIT && job.phi) {
      TI* y = (TI*)p.sp_y + ((int64_t)(c_begin + i) * p.hv + h) * C * DK + 16 * ctile + (lane >> 4) * 4;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        settle(ao[rt]);
        const int r = 16 * rt + (lane & 15);
        store4<TI>(y + r * DK, -ao[rt][0], -ao[rt][1], -ao[rt][2], -ao[rt][3]);
      }
      return;
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      settle(ao[rt]);
      const f32x4 ol = raw4_to_f32<TI>(o.ol[rt]);
      const int r = 16 * rt + (lane & 15);
      if (r < tok_end - tok)
        store4<TI>(outg + (int64_t)(tok + r) * p.o_st + (int64_t)h * p.o_sh + 16 * ctile + (lane >> 4) * 4,
                   ol[0] - ao[rt][0], ol[1] - ao[rt][1], ol[2] - ao[rt][2], ol[3] - ao[rt][3]);
    }
  };
  auto iter = [&](OBuf& cur, const OBuf& prev, int i, int& slot) {
    fetch(cur, i, slot);
    if (i > 0) emit(prev, i - 1);
    slot = slot + 1 == R::slots ? 0 : slot + 1;
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    ring_barrier();
  };
  OBuf oa, ob;
  ring_barrier();
  int slot = 0, i = 0;
  for (; i + 1 < nch; i += 2) {
    iter(oa, ob, i, slot);
    iter(ob, oa, i + 1, slot);
  }
  if (i < nch) {
    iter(oa, ob, i, slot);
    emit(oa, nch - 1);
  } else {
    emit(ob, nch - 1);
  }
}

// The recurrence wave of slice s (column tile ctile).  hacc[t] holds rows
// 16 t + 4 (lane / 16) + e of the state slice, column 16 ctile + lane % 16.
// In the two-level scan (SPLIT) the slice starts from the initial state
// (first segment), from zero, or from identity columns (transition), and its
// end state goes to the workspace.
template <typename TI, int C, int DK, int NSL, bool SPLIT = false>
__device__ __forceinline__ void scan_recurrence(char* smem, const ScanParams& p, int seq, int h,
                                                int s, int ctile, int c_begin, int c_end,
                                                int lane, SliceJob job = {}) {
  using R = ScanRing<TI, C, DK, NSL>;
  using KD = KTile<TI, DK>;
  using KC = KTile<TI, C>;
  using UT = typename Unit<TI>::type;
  typedef typename Raw4<TI>::type RT;
  constexpr int NB = C / 16, NKT = DK / 16;
  constexpr int S = R::S;
  const int DV = p.dv;
  const int nch = c_end - c_begin;
  const int64_t sbase = ((int64_t)seq * p.hv + h) * DK * DV;
  const int col = 16 * ctile + (lane & 15);
  f32x4 hacc[NKT];
  const bool from_init = p.init && (!SPLIT || (job.first && !job.phi));
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    hacc[t] = zero4();
    const int dk0 = 16 * t + (lane >> 4) * 4;
    if (from_init) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[t][e] = p.init[sbase + (int64_t)(dk0 + e) * DV + col];
    } else if (SPLIT && job.phi) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[t][e] = dk0 + e == col ? 1.f : 0.f;
    }
  }

  if (nch > 0) {
    UT hb[KD::NU];
    state_units<TI, DK>(hb, hacc);
#pragma unroll
    for (int q = 0; q < KD::NU; ++q) *(UT*)(smem + R::hcopy(s, 0) + q * 1024 + lane * 16) = hb[q];
    int slot = 0;
    // One chunk step, given U~ (the accumulator input of U) and the decay.
    auto rstep = [&](int i, f32x4 (&au)[NB], float dec) {
      const char* st = smem + slot * R::stage;
      // U = U~ + W (-H) over the d_k units.  Row tiles are finished in
      // pairs, so that the state update for the first 32 rows can start
      // while the MFMAs for the rest run.
#pragma unroll
      for (int r0 = 0; r0 < NB; r0 += 2)
#pragma unroll
        for (int q = 0; q < KD::NU; ++q)
#pragma unroll
          for (int rt = r0; rt < r0 + 2 && rt < NB; ++rt) {
            const char* wu = st + R::w + rt * 16 * DK * S + q * KD::UNIT * S;
            if (KD::HALF_TAIL && q == KD::NU - 1)
              mma_unit<true>(au[rt], lds_unit<TI, true>(wu, lane), hb[q]);
            else
              mma_unit<false>(au[rt], lds_unit<TI, false>(wu, lane), hb[q]);
          }
      // -H_i for the output wave, which reads it after the next barrier
      // (written behind this chunk's operand reads)
      if (i > 0) {
        char* hdst = smem + R::hcopy(s, i & 1);
#pragma unroll
        for (int q = 0; q < KD::NU; ++q) *(UT*)(hdst + q * 1024 + lane * 16) = hb[q];
      }
#pragma unroll
      for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[t][e] *= dec;
      // U (accumulator tiles) as operand units over chunk rows.
      UT ub[KC::NU];
#pragma unroll
      for (int q = 0; q < KC::NU; ++q)
        ub[q] = (KC::HALF_TAIL && q == KC::NU - 1)
                    ? acc_unit<true>(au[KC::TPU * q], au[KC::TPU * q], TI{})
                    : acc_unit<false>(au[KC::TPU * q], au[KC::TPU * q + KC::TPU - 1], TI{});
      // H <- e^gamma_last H + K^T U' (U' = diag(s) U, the key rows read
      // transposed: K~^T U with K~_r = s_r k_r).
      const TI* kr = (const TI*)(st + R::kr);
#pragma unroll
      for (int q = 0; q < KC::NU; ++q)
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
          if (KC::HALF_TAIL && q == KC::NU - 1)
            mma_unit<true>(hacc[t], col_unit<TI, true, R::SWK>(kr, DK, 16 * t, q, lane), ub[q]);
          else
            mma_unit<false>(hacc[t], col_unit<TI, false, R::SWK>(kr, DK, 16 * t, q, lane), ub[q]);
        }
#pragma unroll
      for (int t = 0; t < NKT; ++t) settle(hacc[t]);
      // the next chunk's operand -H
      state_units<TI, DK>(hb, hacc);
      slot = slot + 1 == R::slots ? 0 : slot + 1;
      // every LDS access of this chunk has completed before the copying
      // waves may refill the stage
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
      ring_barrier();
    };
    if constexpr (R::UTR) {
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
      ring_barrier();
      for (int i = 0; i < nch; ++i) {
        const char* st = smem + slot * R::stage;
        f32x4 au[NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) au[rt] = load4<TI>((const TI*)(st + R::ut + rt * 256 * S) + lane * 4);
        rstep(i, au, *(const float*)(st + R::dec));
      }
    } else {
      // the slice's U~ tiles and the decay of chunk cc, requested two chunk
      // steps before their use (past the last chunk the last is read again)
      auto fetch_u = [&](RT (&un)[NB], float& dn, int cc) {
        const int64_t blk = (int64_t)cc * p.hv + h;
        const TI* src = (const TI*)p.im.ut + blk * C * DV + (int64_t)ctile * NB * 256 + lane * 4;
        if (SPLIT && job.phi) {
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) un[rt] = RT{};
        } else {
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) un[rt] = load_raw4<TI>(src + rt * 256);
        }
        dn = p.im.decay[blk];
      };
      auto take = [&](f32x4 (&au)[NB], const RT (&un)[NB]) {
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) au[rt] = raw4_to_f32<TI>(un[rt]);
      };
      RT pa[NB], pb[NB];
      float da, db;
      fetch_u(pa, da, c_begin);
      fetch_u(pb, db, min(c_begin + 1, c_end - 1));
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
      ring_barrier();
      int i = 0;
      for (; i + 1 < nch; i += 2) {
        {
          f32x4 au[NB];
          take(au, pa);
          // into a scalar register, so that the next load may reuse da's
          const float dec = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(da)));
          fetch_u(pa, da, min(c_begin + i + 2, c_end - 1));
          __builtin_amdgcn_sched_barrier(0);
          rstep(i, au, dec);
        }
        {
          f32x4 au[NB];
          take(au, pb);
          const float dec = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(db)));
          fetch_u(pb, db, min(c_begin + i + 3, c_end - 1));
          __builtin_amdgcn_sched_barrier(0);
          rstep(i + 1, au, dec);
        }
      }
      if (i < nch) {
        f32x4 au[NB];
        take(au, pa);
        rstep(i, au, da);
      }
    }
  }

  if constexpr (SPLIT) {
    // end of the first segment (fp32, and its bf16 transpose for the
    // output correction), of the second from zero, or the transition
    const int64_t u = (int64_t)seq * p.hv + h;
    float* dst = job.phi ? p.sp_phi + u * DK * DK : job.first ? p.sp_hmid + sbase : p.sp_psi + sbase;
    const int ld = job.phi ? DK : DV;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const int dk0 = 16 * t + (lane >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(int64_t)(dk0 + e) * ld + col] = hacc[t][e];
      if (job.first && !job.phi)
        store4<TI>((TI*)p.sp_hmid_t + u * DV * DK + (int64_t)col * DK + dk0, hacc[t][0], hacc[t][1],
                   hacc[t][2], hacc[t][3]);
    }
  } else if (p.final_state) {
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const int dk0 = 16 * t + (lane >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) p.final_state[sbase + (int64_t)(dk0 + e) * DV + col] = hacc[t][e];
    }
  }
}

template <int NSL>
constexpr int scan_threads() { return 64 * (2 * NSL + kScanCopyWaves); }

template <typename TI, int C, int DK, int NSL>
__global__ __launch_bounds__(scan_threads<NSL>()) void scan_kernel(ScanParams p) {
  using R = ScanRing<TI, C, DK, NSL>;
  __shared__ __attribute__((aligned(1024))) char smem[R::total];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NS = p.n_slices;
  // XCD-aware: the slice groups of one (sequence, head) share blockIdx % 8
  // and so land on the same XCD, where they share W, Q' and the key rows
  // through its L2.
  const int b = blockIdx.x;
  const int u = (b / (8 * NS)) * 8 + (b % 8);
  const int sl = (b / 8) % NS;
  if (u >= p.map.n_seq * p.hv) return;
  const int seq = u / p.hv, h = scan_head(u % p.hv, p.grp, p.hv);
  int c_begin, c_end, tok0, tok_end;
  seq_range(p.map, seq, C, c_begin, c_end, tok0, tok_end);
  const int nch = c_end - c_begin;

  if (wave >= 2 * NSL) {
    if (nch <= 0) return;
    auto produce = [&](auto cw) {
      ring_producer<R, C, decltype(cw)::value>(smem, p, c_begin, c_end, h, NSL * sl, tok0, tok_end, lane);
    };
    dispatch_int<0, kScanCopyWaves>(wave - 2 * NSL, produce);
    return;
  }
  if (wave >= NSL) {
    if (nch <= 0) return;
    const int s = wave - NSL;
    scan_output<TI, C, DK, NSL>(smem, p, h, s, NSL * sl + s, c_begin, nch, tok0, tok_end, lane);
    return;
  }
  scan_recurrence<TI, C, DK, NSL>(smem, p, seq, h, wave, NSL * sl + wave, c_begin, c_end, lane);
}

// ---------------------------------------------------------------------------
// two-level scan
//
// Each chunk maps the incoming state affinely, H' = M_c H + B_c with
// M_c = e^gamma_last I - K~^T W and B_c = K~^T U~.  A sequence is split at
// chunk `split` into two segments scanned at the same time:
//   first segment   the ordinary scan from the initial state (its outputs
//                   are final), ending in H_mid;
//   second segment  the ordinary scan from zero (local outputs O', end state
//                   Psi), and beside it the same recurrence on identity
//                   columns with U~ = 0 and O_loc = 0: Phi_i, the product of
//                   the segment's M_c before chunk i, and Q'_i Phi_i.
// Linearity in (U~, start) then gives, for second-segment chunk i,
//   O_i = O'_i + (Q'_i Phi_i) H_mid   and   H_end = Phi_end H_mid + Psi,
// which scan_fix_kernel applies.  The chain is half as long at the price of
// the transition columns (d_k more state columns in the second segment).
//
// Per (sequence, head): d_v / 16 first-segment workgroups of one slice (the
// second slice's waves leave at once; a barrier waits for live waves only),
// then (d_v + d_k) / 32 second-segment workgroups of two slices (value
// columns first, then transition columns).  A one-slice workgroup steps
// faster, so the host gives the first segment more chunks.

template <typename TI, int C, int DK>
__global__ __launch_bounds__(scan_threads<2>()) void scan_split_kernel(ScanParams p) {
  using R = ScanRing<TI, C, DK, 2>;
  __shared__ __attribute__((aligned(1024))) char smem[R::total];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NW = p.n_slices;  // workgroups per (sequence, head)
  // XCD-aware: the workgroups of one (sequence, head) share blockIdx % 8.
  const int b = blockIdx.x;
  const int u = (b / (8 * NW)) * 8 + (b % 8);
  const int wg = (b / 8) % NW;
  if (u >= p.map.n_seq * p.hv) return;
  const int seq = u / p.hv, h = scan_head(u % p.hv, p.grp, p.hv);
  int c_begin, c_end, tok0, tok_end;
  seq_range(p.map, seq, C, c_begin, c_end, tok0, tok_end);
  const int NV = p.dv / 16;  // value column tiles = first-segment workgroups
  SliceJob job;
  job.first = wg < NV;
  if (job.first && wave < 4 && (wave & 1)) return;  // one slice: waves 0, 2 and the copiers
  const int k0 = job.first ? wg : 2 * (wg - NV);  // this workgroup's first job in its segment
  job.phi = !job.first && k0 >= NV;
  const int cb = job.first ? c_begin : c_begin + p.split;
  const int ce = job.first ? c_begin + p.split : c_end;
  const int tb = tok0 + (cb - c_begin) * C;
  const int te = job.first ? tb + p.split * C : tok_end;
  if (ce <= cb) return;

  if (wave >= 4) {
    auto produce = [&](auto cw) {
      ring_producer<R, C, decltype(cw)::value>(smem, p, cb, ce, h, 0, tb, te, lane);
    };
    dispatch_int<0, kScanCopyWaves>(wave - 4, produce);
    return;
  }
  const int s = wave & 1;
  job.ctile = k0 + s - (job.phi ? NV : 0);
  if (wave >= 2)
    scan_output<TI, C, DK, 2, true>(smem, p, h, s, job.ctile, cb, ce - cb, tb, te, lane, job);
  else
    scan_recurrence<TI, C, DK, 2, true>(smem, p, seq, h, s, job.ctile, cb, ce, lane, job);
}

// Applies the second segment's correction.  Output blocks: per (sequence,
// head, kFixChunks chunks of the second segment) O^T += H_mid^T (Q' Phi)^T
// with bf16 operands (the same rounding as the scan's Q' H); each wave keeps
// H_mid^T's operand units in registers and requests the rows of all its
// (chunk, row tile) jobs before the first product, so the block waits on
// memory once.  State blocks: per (sequence, head, 16 columns)
// H_end = Phi_end H_mid + Psi in fp32 MFMA tiles: a wave takes DK / 64 row
// tiles, with Phi's rows and Psi read straight into operand and accumulator
// units and H_mid's 16 columns staged once in LDS.
constexpr int kFixThreads = 256;
constexpr int kFixChunks = 2;

__host__ __device__ constexpr int fix_groups(int l1) { return (l1 + kFixChunks - 1) / kFixChunks; }

template <int C, int DK, int DV>
__global__ __launch_bounds__(kFixThreads) void scan_fix_kernel(ScanParams p) {
  constexpr int NW = kFixThreads / 64;
  constexpr int JPW = (kFixChunks * (C / 16) + NW - 1) / NW;  // jobs per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L1 = p.map.chunks_per_seq - p.split;
  const int NG = fix_groups(L1);
  const int n_heads = p.map.n_seq * p.hv;
  const int n_out = (n_heads + 7) / 8 * 8 * NG;
  int b = blockIdx.x;
  if (b < n_out) {
    // XCD-aware: the blocks of one (sequence, head) share blockIdx % 8
    const int u = (b / (8 * NG)) * 8 + (b % 8), gi = (b / 8) % NG;
    if (u >= n_heads) return;
    const int seq = u / p.hv, h = u % p.hv;
    // every job's rows first: Q' Phi rows and the outputs they correct
    typedef typename Raw4<bf16>::type RT;
    bf16x8 yb[JPW][DK / 32];
    RT ov[JPW][DV / 16];
    int n_live[JPW], rows[JPW];
    bf16* orows[JPW];
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      const int jb = wave + NW * j;
      const int i1 = gi * kFixChunks + jb / (C / 16), rt = jb % (C / 16);
      const bool job = jb < kFixChunks * (C / 16) && i1 < L1;
      const int cc = seq * p.map.chunks_per_seq + p.split + (job ? i1 : 0);
      const int tok = seq * p.map.seq_stride + (p.split + (job ? i1 : 0)) * C;
      n_live[j] = job ? min(C, seq * p.map.seq_stride + p.map.seq_len - tok) : 0;
      const int r = 16 * rt + (lane & 15);
      rows[j] = r;
      const bf16* yrow = (const bf16*)p.sp_y + (((int64_t)cc * p.hv + h) * C + r) * DK + (lane >> 4) * 8;
#pragma unroll
      for (int q = 0; q < DK / 32; ++q) yb[j][q] = job ? *(const bf16x8*)(yrow + 32 * q) : bf16x8{};
      orows[j] = (bf16*)p.out + (int64_t)(tok + r) * p.o_st + (int64_t)h * p.o_sh + (lane >> 4) * 4;
#pragma unroll
      for (int ct = 0; ct < DV / 16; ++ct)
        ov[j][ct] = r < n_live[j] ? load_raw4<bf16>(orows[j] + 16 * ct) : RT{};
    }
    const bf16* ht = (const bf16*)p.sp_hmid_t + (int64_t)u * DV * DK + (lane & 15) * DK + (lane >> 4) * 8;
    bf16x8 ha[DV / 16][DK / 32];
#pragma unroll
    for (int ct = 0; ct < DV / 16; ++ct)
#pragma unroll
      for (int q = 0; q < DK / 32; ++q) ha[ct][q] = *(const bf16x8*)(ht + 16 * ct * DK + 32 * q);
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      if (n_live[j] <= 0) continue;
#pragma unroll
      for (int ct = 0; ct < DV / 16; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int q = 0; q < DK / 32; ++q)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[ct][q], yb[j][q], acc, 0, 0, 0);
        if (rows[j] < n_live[j]) {
          const f32x4 o = raw4_to_f32<bf16>(ov[j][ct]);
          store4<bf16>(orows[j] + 16 * ct, o[0] + acc[0], o[1] + acc[1], o[2] + acc[2], o[3] + acc[3]);
        }
      }
    }
    return;
  }
  b -= n_out;
  if (!p.final_state) return;
  constexpr int NT = DV / 16;
  const int u = b / NT, ct = b % NT;
  if (u >= n_heads) return;
  // H_mid's columns 16 ct .. + 15 as B operand units: for k-tile t, lane
  // (n, q) holds rows 16 t + 4 q + 0..3 of column n
  __shared__ f32x4 sB[DK / 16][64];
  const float* hm = p.sp_hmid + (int64_t)u * DK * DV + 16 * ct;
  for (int idx = tid; idx < (DK / 16) * 64; idx += kFixThreads) {
    const int t = idx / 64, l = idx % 64, n = l & 15, q = l >> 4;
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = hm[(int64_t)(16 * t + 4 * q + e) * DV + n];
    sB[t][l] = v;
  }
  __syncthreads();
  const int n = lane & 15, q = lane >> 4;
  for (int rt = wave; rt < DK / 16; rt += NW) {
    // Psi's tile as the accumulator: lane (n, q) holds rows 16 rt + 4 q + e
    const float* ps = p.sp_psi + ((int64_t)u * DK + 16 * rt + 4 * q) * DV + 16 * ct + n;
    f32x4 acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = ps[(int64_t)e * DV];
    // Phi's rows 16 rt + n as A operand units: k-tile t, columns 16 t + 4 q + 0..3
    const float* ph = p.sp_phi + ((int64_t)u * DK + 16 * rt + n) * DK + 4 * q;
    f32x4 a[DK / 16];
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) a[t] = *(const f32x4*)(ph + 16 * t);
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) mma16_f32_ab(acc, a[t], sB[t][lane]);
    settle(acc);
    float* dst = p.final_state + ((int64_t)u * DK + 16 * rt + 4 * q) * DV + 16 * ct + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(int64_t)e * DV] = acc[e];
  }
}

// ---------------------------------------------------------------------------
// decode: one token per sequence
//
// The same recurrence for a single token, applied to a state carried in
// memory (the step a generator runs after the prefill):
//   H <- exp(g) (I - beta k^ k^T) H + beta k^ v^T,   out = scale H^T q^.
// It reads and writes the whole fp32 state once, so it is bound by HBM: one
// workgroup per (sequence, value head); each thread holds four adjacent
// columns of a band of DK / RG rows in registers, read and written with
// 16-byte accesses (a row of the state is one coalesced run across the
// threads of a row group).  The two contractions over d_k (k^T H before the
// update, q^T H after it) are reduced across the row groups through LDS.
// Everything is fp32.

template <int DK, int DV>
struct DecodeShape {
  static constexpr int CG = DV / 4;                                    // column groups
  static constexpr int RG = (1024 / DV) < DK ? (1024 / DV) : DK;        // row groups
  static constexpr int NT = CG * RG;                                   // threads
  static constexpr int RPT = DK / RG;                                  // rows per thread
};

// Channel c of sequence i's token x through the short convolution: its
// history rows, then x with the last tap; silu when on; rounded to TI.
template <typename TI>
__device__ __forceinline__ float decode_conv(const DecodeParams& p, int i, int c, float x) {
  const int W = p.conv_width;
  const float* w = p.conv_w + (int64_t)c * W;
  const TI* hist = (const TI*)p.conv_state;
  float acc = 0.f;
  for (int j = 0; j + 1 < W; ++j)
    acc += w[j] * (hist ? to_float(hist[((int64_t)i * (W - 1) + j) * p.conv_d + c]) : 0.f);
  acc += w[W - 1] * x;
  return to_float(conv_act<TI>(acc, p.qkv_silu));
}

template <typename TI, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(DecodeParams p) {
  using D = DecodeShape<DK, DV>;
  constexpr int NT = D::NT, CG = D::CG, RG = D::RG, RPT = D::RPT;
  __shared__ float sq[DK], sk[DK], snorm[2];
  __shared__ __attribute__((aligned(16))) float sred[RG][DV];
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  if (u >= p.n * p.hv) return;
  const int i = u / p.hv, h = u % p.hv, kh = h / (p.hv / p.hk);
  const int cg = tid % CG, rg = tid / CG;
  const int c0 = 4 * cg, r0 = rg * RPT;

  // this thread's band of the state, requested first
  float* Hs = p.state + (int64_t)u * DK * DV + (int64_t)r0 * DV + c0;
  f32x4 hreg[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) hreg[r] = *(const f32x4*)(Hs + (int64_t)r * DV);

  // q and k rows and their inverse norms
  const TI* qr = (const TI*)p.q + (int64_t)i * p.q_st + (int64_t)kh * p.q_sh;
  const TI* kr = (const TI*)p.k + (int64_t)i * p.k_st + (int64_t)kh * p.k_sh;
  for (int d = tid; d < DK; d += NT) {
    sq[d] = to_float(qr[d]);
    sk[d] = to_float(kr[d]);
    if (p.conv_w) {
      sq[d] = decode_conv<TI>(p, i, kh * DK + d, sq[d]);
      sk[d] = decode_conv<TI>(p, i, (p.hk + kh) * DK + d, sk[d]);
    } else if (p.qkv_silu) {
      sq[d] = qkv_act<TI>(sq[d]);
      sk[d] = qkv_act<TI>(sk[d]);
    }
  }
  __syncthreads();
  if (tid < 64 * (NT >= 128 ? 2 : 1)) {
    const int l = tid & 63;
#pragma unroll
    for (int which = 0; which < (NT >= 128 ? 1 : 2); ++which) {
      const int sel = NT >= 128 ? (tid >> 6) : which;
      const float* src = sel == 0 ? sq : sk;
      float s2 = 0.f;
      for (int d = l; d < DK; d += 64) s2 += src[d] * src[d];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s2 += __shfl_xor(s2, off);
      if (l == 0) snorm[sel] = 1.0f / sqrtf(s2 + p.eps);
    }
  }
  float g = p.g[(int64_t)i * p.g_st + (int64_t)h * p.g_sh];
  if (p.decay_proj) g = decay_gate(g, p.a_log, p.a_bias, h);
  float beta = p.beta[(int64_t)i * p.b_st + (int64_t)h * p.b_sh];
  if (p.beta_logits) beta = 1.f / (1.f + __expf(-beta));
  const float alpha = expf(g);
  f32x4 vj = load4<TI>((const TI*)p.v + (int64_t)i * p.v_st + (int64_t)h * p.v_sh + c0);
  if (p.conv_w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vj[e] = decode_conv<TI>(p, i, 2 * p.hk * DK + h * p.dv + c0 + e, vj[e]);
  } else if (p.qkv_silu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vj[e] = qkv_act<TI>(vj[e]);
  }

  // (k^T H)_j over this band, with the raw k (the norm is applied below)
  f32x4 part = zero4();
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kv = sk[r0 + r];
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] += kv * hreg[r][e];
  }
  *(f32x4*)&sred[rg][c0] = part;
  __syncthreads();
  const float rq = snorm[0], rk = snorm[1];
  f32x4 kth = zero4();
  for (int q = 0; q < RG; ++q) {
    const f32x4 t = *(const f32x4*)&sred[q][c0];
#pragma unroll
    for (int e = 0; e < 4; ++e) kth[e] += t[e];
  }
  __syncthreads();
  // H' = alpha (H - beta k^ (k^T H)) + beta k^ v^T, and q^T H'
  part = zero4();
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kh_r = sk[r0 + r] * rk, qv = sq[r0 + r];
    f32x4 hn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hn[e] = alpha * (hreg[r][e] - beta * kh_r * (kth[e] * rk)) + beta * kh_r * vj[e];
      part[e] += qv * hn[e];
    }
    *(f32x4*)(Hs + (int64_t)r * DV) = hn;
  }
  *(f32x4*)&sred[rg][c0] = part;
  __syncthreads();
  if (rg == 0) {
    f32x4 o = zero4();
    for (int q = 0; q < RG; ++q) {
      const f32x4 t = *(const f32x4*)&sred[q][c0];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += t[e];
    }
    const float sc = p.scale * rq;
    store4<TI>((TI*)p.out + (int64_t)i * p.o_st + (int64_t)h * p.o_sh + c0, sc * o[0], sc * o[1],
               sc * o[2], sc * o[3]);
  }
}

// ---------------------------------------------------------------------------
// dispatch

// fp32 inputs are built for chunks of 16 and 32 only (their WY tiles at 64
// would exceed the LDS or the register budget).
template <typename TI, int C, int DK>
static constexpr bool fits() {
  return WyLayout<TI, C, DK>::total <= kLdsLimit && ScanRing<TI, C, DK, 1>::slots >= 2 &&
         (sizeof(TI) == 2 || C <= 32);
}

// Workgroups of two or four slices are built for bf16 inputs.
template <typename TI, int C, int DK, int NSL = 2>
static constexpr bool fits_group() {
  return fits<TI, C, DK>() && sizeof(TI) == 2 && ScanRing<TI, C, DK, NSL>::slots >= 2;
}

template <typename TI, int C, int DK>
static int launch_pair(int stage, const WyParams* wy, const ScanParams* sc,
                       dim3 grid, hipStream_t s) {
  if constexpr (fits<TI, C, DK>()) {
    if (stage == 0) {
      if (wy->conv_w)
        hipLaunchKernelGGL((wy_kernel<TI, C, DK, true>), grid, dim3(kWyThreads), 0, s, *wy);
      else
        hipLaunchKernelGGL((wy_kernel<TI, C, DK, false>), grid, dim3(kWyThreads), 0, s, *wy);
    } else if (sc->nsl == 4) {
      if constexpr (fits_group<TI, C, DK, 4>())
        hipLaunchKernelGGL((scan_kernel<TI, C, DK, 4>), grid, dim3(scan_threads<4>()), 0, s, *sc);
      else
        return -1;
    } else if (sc->nsl == 2) {
      if constexpr (fits_group<TI, C, DK>())
        hipLaunchKernelGGL((scan_kernel<TI, C, DK, 2>), grid, dim3(scan_threads<2>()), 0, s, *sc);
      else
        return -1;
    } else {
      hipLaunchKernelGGL((scan_kernel<TI, C, DK, 1>), grid, dim3(scan_threads<1>()), 0, s, *sc);
    }
    return 0;
  } else {
    return -1;
  }
}

template <typename TI, int C>
static int dispatch_dk(int dk, int stage, const WyParams* wy, const ScanParams* sc,
                       dim3 grid, hipStream_t s) {
  switch (dk) {
    case 16: return launch_pair<TI, C, 16>(stage, wy, sc, grid, s);
    case 32: return launch_pair<TI, C, 32>(stage, wy, sc, grid, s);
    case 64: return launch_pair<TI, C, 64>(stage, wy, sc, grid, s);
    case 128: return launch_pair<TI, C, 128>(stage, wy, sc, grid, s);
  }
  return -1;
}

template <typename TI>
static int dispatch_c(int chunk, int dk, int stage, const WyParams* wy,
                      const ScanParams* sc, dim3 grid, hipStream_t s) {
  switch (chunk) {
    case 16: return dispatch_dk<TI, 16>(dk, stage, wy, sc, grid, s);
    case 32: return dispatch_dk<TI, 32>(dk, stage, wy, sc, grid, s);
    case 64: return dispatch_dk<TI, 64>(dk, stage, wy, sc, grid, s);
  }
  return -1;
}

template <typename TI>
static bool fits_any(int chunk, int dk) {
#define GDN_FITS(CC, DD) if (chunk == CC && dk == DD) return fits<TI, CC, DD>();
  GDN_FITS(16, 16) GDN_FITS(16, 32) GDN_FITS(16, 64) GDN_FITS(16, 128)
  GDN_FITS(32, 16) GDN_FITS(32, 32) GDN_FITS(32, 64) GDN_FITS(32, 128)
  GDN_FITS(64, 16) GDN_FITS(64, 32) GDN_FITS(64, 64) GDN_FITS(64, 128)
#undef GDN_FITS
  return false;
}

bool kernels_available(bool bf16, int chunk, int dk) {
  return bf16 ? fits_any<gdn::bf16>(chunk, dk) : fits_any<float>(chunk, dk);
}

static bool group_available(int chunk, int dk, int nsl) {
#define GDN_FITS(CC, DD)                                                                \
  if (chunk == CC && dk == DD)                                                          \
    return nsl == 4 ? fits_group<gdn::bf16, CC, DD, 4>() : fits_group<gdn::bf16, CC, DD, 2>();
  GDN_FITS(16, 16) GDN_FITS(16, 32) GDN_FITS(16, 64) GDN_FITS(16, 128)
  GDN_FITS(32, 16) GDN_FITS(32, 32) GDN_FITS(32, 64) GDN_FITS(32, 128)
  GDN_FITS(64, 16) GDN_FITS(64, 32) GDN_FITS(64, 64) GDN_FITS(64, 128)
#undef GDN_FITS
  return false;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Slices per scan workgroup.  The scan runs one workgroup per compute unit.
// Where the 16-column slices fit the compute units at once, one slice per
// workgroup spreads the chains widest.  Where they would queue, two slices
// per workgroup share one copy of each chunk's operands and run on separate
// SIMDs, for about the time per chunk of one.  Where even four-slice
// workgroups fill every compute unit, four slices share each copy: half the
// operand traffic from L2 into the compute units, which bounds the scan once
// the chip is full (two stages of the ring instead of three).
int scan_slices_per_group(bool bf16, int chunk, int dk, int dv, int64_t seq_heads) {
  if (!bf16 || dv % 32 != 0 || !group_available(chunk, dk, 2)) return 1;
  const int64_t slices = seq_heads * (dv / 16), cus = device_cus();
  if (slices <= cus) return 1;
  if (dv % 64 == 0 && group_available(chunk, dk, 4) && slices >= 4 * cus) return 4;
  return 2;
}

// GDN_DEBUG_CHECK: one workgroup checks every entry of cu_seqlens.
template <typename I>
__global__ __launch_bounds__(256) void check_cu_kernel(const I* cu, int64_t n_seq,
                                                      int64_t t_total, int32_t* faults) {
  __shared__ int32_t s_f;
  if (threadIdx.x == 0) s_f = 0;
  __syncthreads();
  int32_t f = 0;
  for (int64_t i = threadIdx.x; i <= n_seq; i += blockDim.x) f |= cu_entry_faults(cu, i, n_seq, t_total);
  if (f) atomicOr(&s_f, f);
  __syncthreads();
  if (threadIdx.x == 0) *faults = s_f;
}

hipError_t launch_check_cu(const void* cu, bool cu_i64, int64_t n_seq, int64_t t_total,
                           int32_t* faults, hipStream_t s) {
  if (cu_i64)
    hipLaunchKernelGGL(check_cu_kernel<int64_t>, dim3(1), dim3(256), 0, s, (const int64_t*)cu, n_seq,
                       t_total, faults);
  else
    hipLaunchKernelGGL(check_cu_kernel<int32_t>, dim3(1), dim3(256), 0, s, (const int32_t*)cu, n_seq,
                       t_total, faults);
  return hipGetLastError();
}

hipError_t launch_table(const TableParams& p, hipStream_t s) {
  hipLaunchKernelGGL(table_kernel, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wy(bool bf16, int chunk, int dk, const WyParams& p, hipStream_t s) {
  const dim3 grid(p.n_items);
  const int rc = bf16 ? dispatch_c<gdn::bf16>(chunk, dk, 0, &p, nullptr, grid, s)
                      : dispatch_c<float>(chunk, dk, 0, &p, nullptr, grid, s);
  if (rc) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_scan(bool bf16, int chunk, int dk, const ScanParams& p,
                       int grid_x, hipStream_t s) {
  const dim3 grid(grid_x);
  const int rc = bf16 ? dispatch_c<gdn::bf16>(chunk, dk, 1, nullptr, &p, grid, s)
                      : dispatch_c<float>(chunk, dk, 1, nullptr, &p, grid, s);
  if (rc) return hipErrorInvalidValue;
  return hipGetLastError();
}

bool two_level_available(bool bf16, int chunk, int dk) { return bf16 && group_available(chunk, dk, 2); }

template <int C, int DK>
static hipError_t launch_two_level_dk(const ScanParams& p, hipStream_t s) {
  if constexpr (fits_group<gdn::bf16, C, DK>()) {
    const int64_t heads = (int64_t)p.map.n_seq * p.hv, heads8 = (heads + 7) / 8 * 8;
    const int64_t grid_a = heads8 * p.n_slices;
    const int64_t grid_fix = heads8 * fix_groups(p.map.chunks_per_seq - p.split) + heads * (p.dv / 16);
    hipLaunchKernelGGL((scan_split_kernel<gdn::bf16, C, DK>), dim3((unsigned)grid_a),
                       dim3(scan_threads<2>()), 0, s, p);
    switch (p.dv) {
      case 32: hipLaunchKernelGGL((scan_fix_kernel<C, DK, 32>), dim3((unsigned)grid_fix), dim3(kFixThreads), 0, s, p); break;
      case 64: hipLaunchKernelGGL((scan_fix_kernel<C, DK, 64>), dim3((unsigned)grid_fix), dim3(kFixThreads), 0, s, p); break;
      case 128: hipLaunchKernelGGL((scan_fix_kernel<C, DK, 128>), dim3((unsigned)grid_fix), dim3(kFixThreads), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_two_level(int chunk, int dk, const ScanParams& p, hipStream_t s) {
  if (chunk == 32 && dk == 32) return launch_two_level_dk<32, 32>(p, s);
  if (chunk == 32 && dk == 64) return launch_two_level_dk<32, 64>(p, s);
  if (chunk == 32 && dk == 128) return launch_two_level_dk<32, 128>(p, s);
  if (chunk == 64 && dk == 32) return launch_two_level_dk<64, 32>(p, s);
  if (chunk == 64 && dk == 64) return launch_two_level_dk<64, 64>(p, s);
  if (chunk == 64 && dk == 128) return launch_two_level_dk<64, 128>(p, s);
  return hipErrorInvalidValue;
}

template <typename TI, int DK>
static hipError_t launch_decode_dv(const DecodeParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.n * p.hv));
  switch (p.dv) {
#define GDN_DECODE(V)                                                                           \
    case V:                                                                                     \
      hipLaunchKernelGGL((decode_kernel<TI, DK, V>), grid, dim3(DecodeShape<DK, V>::NT), 0, s, p); \
      return hipGetLastError();
    GDN_DECODE(16) GDN_DECODE(32) GDN_DECODE(64) GDN_DECODE(128)
#undef GDN_DECODE
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// The gated output norm: y = x / sqrt(mean(x^2) + eps) * w * silu(z) over
// rows of DV elements (the reading at GDN_FLAG_OUTPUT_GATE in gdn.h).  A
// bandwidth-bound pass: each lane moves one 16-byte granule of x, z and y;
// DV / (granule elements) lanes hold a row and reduce its sum of squares
// with butterfly shuffles inside their lane group, so a wave covers several
// rows and every access is a full 16-byte vector access.

constexpr int kGateThreads = 256;

template <typename TI, int DV>
__global__ __launch_bounds__(kGateThreads) void output_gate_kernel(GateParams p) {
  constexpr int EPL = 16 / (int)sizeof(TI);  // elements per lane
  constexpr int LPR = DV / EPL;              // lanes per row (a power of two, <= 64)
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row width");
  constexpr int RPB = kGateThreads / LPR;    // rows per workgroup
  const int sub = threadIdx.x % LPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  bool live = r < p.rows;
  const int64_t t = live ? r / p.inner : 0, h = live ? r % p.inner : 0;
  if (live && p.t_end) live = t < (int64_t)*p.t_end;  // rows past the packed batch's end
  float x[EPL], z[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = z[e] = 0.f;
  if (live) {
    const uint4 xv = ld16((const TI*)p.x + t * p.x_st + h * p.x_sh + sub * EPL);
    const uint4 zv = ld16((const TI*)p.z + t * p.z_st + h * p.z_sh + sub * EPL);
    const TI* xe = (const TI*)&xv;
    const TI* ze = (const TI*)&zv;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = to_float(xe[e]);
      z[e] = to_float(ze[e]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float rn = 1.0f / sqrtf(ss / (float)DV + p.eps);
  if (!live) return;
  uint4 yv;
  TI* ye = (TI*)&yv;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float w = p.w ? p.w[sub * EPL + e] : 1.f;
    const float silu = z[e] / (1.f + expf(-z[e]));
    ye[e] = from_float<TI>(x[e] * rn * w * silu);
  }
  st16((TI*)p.out + t * p.o_st + h * p.o_sh + sub * EPL, yv);
}

template <typename TI>
static hipError_t launch_output_gate_t(int dv, const GateParams& p, hipStream_t s) {
  constexpr int EPL = 16 / (int)sizeof(TI);
  const int64_t rpb = kGateThreads / (dv / EPL);
  const int64_t blocks = (p.rows + rpb - 1) / rpb;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  switch (dv) {
#define GDN_GATE(V)                                                                                 \
    case V:                                                                                         \
      hipLaunchKernelGGL((output_gate_kernel<TI, V>), dim3((unsigned)blocks), dim3(kGateThreads), 0, s, p); \
      return hipGetLastError();
    GDN_GATE(16) GDN_GATE(32) GDN_GATE(64) GDN_GATE(128)
#undef GDN_GATE
  }
  return hipErrorInvalidValue;
}

hipError_t launch_output_gate(bool bf16, int dv, const GateParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  return bf16 ? launch_output_gate_t<gdn::bf16>(dv, p, s) : launch_output_gate_t<float>(dv, p, s);
}

// ---------------------------------------------------------------------------
// The short convolution's state after a call (GDN_FLAG_QKV_CONV): for
// sequence s (L rows) and channel c, row j of the new state is row L + j of
// the old history followed by the sequence, i.e. input row L + j - (W - 1)
// when that is >= 0, else history row L + j.  One thread per (sequence,
// channel) reads all of its values before it writes any, so the new state
// may overwrite the old.

constexpr int kConvStateThreads = 256;

template <typename TI>
__global__ __launch_bounds__(kConvStateThreads) void conv_state_kernel(ConvStateParams p) {
  const int64_t u = (int64_t)blockIdx.x * kConvStateThreads + threadIdx.x;
  if (u >= (int64_t)p.n_seq * p.d) return;
  const int seq = (int)(u / p.d), c = (int)(u % p.d);
  const int W = p.width;
  int64_t tok0;
  int L;
  if (p.seq_start) {
    tok0 = p.seq_start[seq];
    L = p.seq_start[seq + 1] - p.seq_start[seq];
  } else {
    tok0 = (int64_t)seq * p.seq_len;
    L = p.seq_len;
  }
  // channel c of q | k | v: its column of the token rows
  const int qk = p.hk * p.dk;
  const TI* x;
  int64_t st;
  if (c < qk) {
    x = (const TI*)p.q + (int64_t)(c / p.dk) * p.q_sh + c % p.dk;
    st = p.q_st;
  } else if (c < 2 * qk) {
    x = (const TI*)p.k + (int64_t)((c - qk) / p.dk) * p.k_sh + (c - qk) % p.dk;
    st = p.k_st;
  } else {
    x = (const TI*)p.v + (int64_t)((c - 2 * qk) / p.dv) * p.v_sh + (c - 2 * qk) % p.dv;
    st = p.v_st;
  }
  const TI* hin = (const TI*)p.state_in;
  TI vals[kConvMaxWidth - 1];
#pragma unroll
  for (int j = 0; j < kConvMaxWidth - 1; ++j) {
    if (j >= W - 1) break;
    const int r = L + j;
    if (r >= W - 1) vals[j] = x[(tok0 + r - (W - 1)) * st];
    else vals[j] = hin ? hin[((int64_t)seq * (W - 1) + r) * p.d + c] : from_float<TI>(0.f);
  }
  TI* hout = (TI*)p.state_out;
#pragma unroll
  for (int j = 0; j < kConvMaxWidth - 1; ++j)
    if (j < W - 1) hout[((int64_t)seq * (W - 1) + j) * p.d + c] = vals[j];
}

hipError_t launch_conv_state(bool bf16, const ConvStateParams& p, hipStream_t s) {
  const int64_t threads = (int64_t)p.n_seq * p.d;
  if (threads <= 0 || p.width < 2) return hipSuccess;
  const int64_t blocks = (threads + kConvStateThreads - 1) / kConvStateThreads;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL((conv_state_kernel<gdn::bf16>), dim3((unsigned)blocks), dim3(kConvStateThreads), 0, s, p);
  else
    hipLaunchKernelGGL((conv_state_kernel<float>), dim3((unsigned)blocks), dim3(kConvStateThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation prefill: the workspace as a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is what the launches receive.

}  // namespace gdn

static __device__ __align__(256) char scratch[gdn::kScratchBytes];
static __device__ int32_t debug_word;

namespace gdn {

hipError_t scratch_region(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t debug_word_region(int32_t** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_word));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = (int32_t*)p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(bool bf16, int dk, const DecodeParams& p, hipStream_t s) {
  switch (dk) {
#define GDN_DECODE(D) \
    case D: return bf16 ? launch_decode_dv<gdn::bf16, D>(p, s) : launch_decode_dv<float, D>(p, s);
    GDN_DECODE(16) GDN_DECODE(32) GDN_DECODE(64) GDN_DECODE(128)
#undef GDN_DECODE
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
