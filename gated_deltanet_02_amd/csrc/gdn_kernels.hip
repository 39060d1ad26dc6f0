// gfx950 (CDNA4) kernels of the chunked Gated DeltaNet prefill.
//
// The operation is the gated delta rule (Gated Delta Networks, Yang, Kautz,
// Hatamizadeh, ICLR 2025, section 3), evaluated chunk by chunk in its WY
// form (Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length, Yang et al., NeurIPS 2024, section 3).  For a chunk of n <= C
// tokens with chunk-local cumulative gate gamma_r = g_0 + ... + g_r and
// D_rs = exp(gamma_r - gamma_s) (s <= r):
//
//   A   = strictly-lower part of beta_r D_rs (k^_r . k^_s)
//   T   = (I + A)^-1                              (forward substitution)
//   W   = T diag(beta e^gamma) K^,   U~ = T diag(beta) V
//   P   = scale * D o (Q^ K^T)                    (causal, diagonal included)
//   Q'  = scale diag(e^gamma) Q^ - P W,   O_loc = P U~
//   K~_r = e^(gamma_last - gamma_r) k^_r
// and, carried from chunk to chunk with state H (d_k x d_v, fp32):
//   U = U~ - W H,   O = Q' H + O_loc,   H <- e^gamma_last H + K~^T U.
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
//   scan_kernel   one workgroup per (sequence, value head, 16-column slice of
//                 d_v): the only sequential part.  The state slice lives in
//                 MFMA accumulators.  W, Q' and K~^T are stored by the WY
//                 kernel in MFMA fragment order, so each wave loads its
//                 operands straight into registers, three chunks ahead; LDS
//                 only carries the two exchanges per step (H and U).  The
//                 output is produced in the same step.
//
// bf16 inputs use bf16 MFMA operands with fp32 accumulation; the triangular
// solve and every gate exponential are fp32.  fp32 inputs use fp32 MFMA
// throughout.  All exponents are <= 0 when g <= 0: differences of gamma are
// only formed for s <= r and never factored into exp(gamma_r) exp(-gamma_s).
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_internal.h"
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
    t0 = seq * m.seq_len + j * C;
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
    tok0 = seq * m.seq_len;
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
    int e = (i < p.n_seq) ? p.cu[i + 1] : 0;
    e = min(max(e, 0), p.t_total);
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
// LDS helpers (whole workgroup)

// dst[d][r] = src[r][d] for r < R (even), d < D (multiple of a granule).
// Pairs of rows are packed so each LDS write carries two elements.
template <typename TI, int NT = kThreads>
__device__ __forceinline__ void transpose_lds(const TI* src, int lds, TI* dst,
                                              int ldd, int R, int D, int tid) {
  constexpr int GR = Gran<TI>::n;
  typedef TI pair_t __attribute__((ext_vector_type(2)));
  const int npair = R / 2, ngran = D / GR;
  for (int idx = tid; idx < npair * ngran; idx += NT) {
    const int m = idx % npair, gc = idx / npair;
    const uint4 va = ld16(src + (2 * m) * lds + gc * GR);
    const uint4 vb = ld16(src + (2 * m + 1) * lds + gc * GR);
    const TI* ea = (const TI*)&va;
    const TI* eb = (const TI*)&vb;
#pragma unroll
    for (int j = 0; j < GR; ++j) {
      pair_t pr;
      pr[0] = ea[j];
      pr[1] = eb[j];
      *(pair_t*)(dst + (gc * GR + j) * ldd + 2 * m) = pr;
    }
  }
}

// out[r] = 1 / sqrt(sum_d src[r][d]^2 + eps); four lanes per row, each
// reading its quarter of the row in 16-byte pieces.
template <typename TI, int D, int NT = kThreads>
__device__ __forceinline__ void row_inv_norms(const TI* src, int lds, int R,
                                              float eps, float* out, int tid) {
  constexpr int GR = Gran<TI>::n;
  for (int base = 0; base < R * 4; base += NT) {
    const int idx = base + tid;
    const int r = idx >> 2, part = idx & 3;
    float s = 0.f;
    if (r < R) {
      const TI* row = src + r * lds + part * (D / 4);
      if constexpr ((D / 4) % GR == 0) {
#pragma unroll
        for (int g = 0; g < D / 4 / GR; ++g) {
          const uint4 v = ld16(row + g * GR);
          const TI* e = (const TI*)&v;
#pragma unroll
          for (int j = 0; j < GR; ++j) {
            const float x = to_float(e[j]);
            s += x * x;
          }
        }
      } else {
#pragma unroll
        for (int d = 0; d < D / 4; ++d) {
          const float x = to_float(row[d]);
          s += x * x;
        }
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (r < R && part == 0) out[r] = 1.0f / sqrtf(s + eps);
  }
}

// ---------------------------------------------------------------------------
// WY kernel

constexpr int kWyThreads = 512;  // 8 waves, one workgroup per CU

// LDS plan of the WY kernel (bytes).  bf16 tiles are stored unpadded with
// row-swizzled 16-byte granules; fp32 tiles (and fp32 inputs) use rows padded
// by 16 bytes.  Regions are reused as their contents die:
//   kt  K^T [dk][C]                                          whole kernel
//   kv  K rows [C][dk] -> V^T [dv][C] -> W^T [dk][C]
//   t   V rows [C][128] -> T (f32) -> U~^T [dv][C]
//   x   Q rows [C][dk] -> A (f32) -> Tb, Tv, P [C][C]
template <typename TI, int C, int DK>
struct WyLayout {
  static constexpr int S = sizeof(TI);
  static constexpr bool SWIZ = S == 2;
  static constexpr int PK = SWIZ ? 0 : 16 / S;
  static constexpr int DVM = 128;  // largest d_v
  static constexpr int LK = DK + PK;
  static constexpr int LV = DVM + PK;
  static constexpr int LC = C + PK;
  static constexpr int LF = C + 4;
  static constexpr int SWK = SWIZ ? DK / 8 - 1 : 0;
  static constexpr int SWC = SWIZ ? C / 8 - 1 : 0;
  static constexpr int SWV = SWIZ ? DVM / 8 - 1 : 0;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int r_kt = 0;
  static constexpr int r_kv = r_kt + DK * LC * S;
  static constexpr int sz_kv = cmax(cmax(C * LK, DVM * LC), DK * LC) * S;
  static constexpr int r_t = r_kv + sz_kv;
  static constexpr int sz_t = cmax(cmax(C * LF * 4, DVM * LC * S), C * LV * S);
  static constexpr int r_x = r_t + sz_t;
  static constexpr int sz_x = cmax(cmax(C * LK * S, C * LF * 4), 3 * C * LC * S);
  static constexpr int r_vec = r_x + sz_x;
  static constexpr int total = r_vec + 7 * C * 4;
};

// dst[d][r] = src[r][d] for r < R (even), d < D (whole granules), with the
// source and destination row swizzles.  Pairs of rows are packed so each LDS
// write carries two elements.
template <typename TI, int NT, int SWS, int SWD>
__device__ __forceinline__ void transpose_sw(const TI* src, int lds, TI* dst, int ldd, int R, int D,
                                             int tid) {
  constexpr int GR = Gran<TI>::n;
  typedef TI pair_t __attribute__((ext_vector_type(2)));
  const int npair = R / 2, ngran = D / GR;
  for (int idx = tid; idx < npair * ngran; idx += NT) {
    const int m = idx % npair, gc = idx / npair;
    const uint4 va = ld16(src + (2 * m) * lds + swz<TI, SWS>(2 * m, gc * GR));
    const uint4 vb = ld16(src + (2 * m + 1) * lds + swz<TI, SWS>(2 * m + 1, gc * GR));
    const TI* ea = (const TI*)&va;
    const TI* eb = (const TI*)&vb;
#pragma unroll
    for (int j = 0; j < GR; ++j) {
      pair_t pr;
      pr[0] = ea[j];
      pr[1] = eb[j];
      const int row = gc * GR + j;
      *(pair_t*)(dst + row * ldd + swz<TI, SWD>(row, 2 * m)) = pr;
    }
  }
}

template <typename TI, int C, int DK>
__global__ __launch_bounds__(kWyThreads) void wy_kernel(WyParams p) {
  using L = WyLayout<TI, C, DK>;
  constexpr int NT = kWyThreads;
  constexpr int LK = L::LK, LV = L::LV, LC = L::LC, LF = L::LF;
  constexpr int SWK = L::SWK, SWC = L::SWC, SWV = L::SWV;
  constexpr int GR = Gran<TI>::n;
  constexpr int NB = C / 16;    // 16-row tiles along the chunk
  constexpr int NKT = DK / 16;  // 16-row tiles along d_k
  constexpr int GPR = DK / GR;  // 16-byte granules per q / k row
  constexpr int NQK = (C * GPR + NT - 1) / NT;
  constexpr int NVG = (C * (128 / GR) + NT - 1) / NT;  // v granules per thread (d_v <= 128)
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  TI* sKt = (TI*)(smem + L::r_kt);
  TI* sKV = (TI*)(smem + L::r_kv);   // K rows | V^T | W^T
  TI* sVr = (TI*)(smem + L::r_t);    // V rows
  float* sT = (float*)(smem + L::r_t);
  TI* sUt = (TI*)(smem + L::r_t);    // U~^T
  TI* sQ = (TI*)(smem + L::r_x);     // Q rows
  float* sA = (float*)(smem + L::r_x);
  TI* sTb = (TI*)(smem + L::r_x);
  TI* sTv = sTb + C * LC;
  TI* sP = sTv + C * LC;
  float* sRq = (float*)(smem + L::r_vec);
  float* sRk = sRq + C;
  float* sGam = sRk + C;
  float* sBeta = sGam + C;
  float* sEg = sBeta + C;   // e^gamma_r
  float* sKs = sEg + C;     // rk_r e^(gamma_last - gamma_r)
  float* sCb = sKs + C;     // beta_s e^gamma_s rk_s  (column scale of Tb)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, kh = blockIdx.y;
  int seq, t0, n;
  if (!chunk_info(p.map, c, C, seq, t0, n)) return;
  (void)seq;
  const TI* qg = (const TI*)p.q;
  const TI* kg = (const TI*)p.k;
  const TI* vg = (const TI*)p.v;
  const int DV = p.dv;
  const int GPRV = DV / GR;
  const int NVT = DV / 16;
  const int grp = p.hv / p.hk;

  // All global inputs of the chunk are requested up front: q and k rows,
  // the v rows and gates of the first value head (zeros past the chunk end).
  uint4 kreg[NQK], qreg[NQK], vreg[NVG];
  float gv = 0.f, bv = 0.f;
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    const int idx = tid + i * NT;
    const int r = idx / GPR, gc = idx % GPR;
    kreg[i] = qreg[i] = make_uint4(0, 0, 0, 0);
    if (idx < C * GPR && r < n) {
      const int64_t t = t0 + r;
      kreg[i] = ld16(kg + t * p.k_st + kh * p.k_sh + gc * GR);
      qreg[i] = ld16(qg + t * p.q_st + kh * p.q_sh + gc * GR);
    }
  }
  auto load_head = [&](int h) {
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / GPRV, gc = idx % GPRV;
      vreg[i] = make_uint4(0, 0, 0, 0);
      if (idx < C * GPRV && r < n) vreg[i] = ld16(vg + (int64_t)(t0 + r) * p.v_st + h * p.v_sh + gc * GR);
    }
    if (wave == 0 && lane < n) {
      gv = p.g[(int64_t)(t0 + lane) * p.g_st + h * p.g_sh];
      bv = p.beta[(int64_t)(t0 + lane) * p.b_st + h * p.b_sh];
    } else {
      gv = 0.f;
      bv = 0.f;
    }
  };
  load_head(kh * grp);

#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    const int idx = tid + i * NT;
    if (idx < C * GPR) {
      const int r = idx / GPR, gc = idx % GPR;
      st16(sKV + r * LK + swz<TI, SWK>(r, gc * GR), kreg[i]);
      st16(sQ + r * LK + swz<TI, SWK>(r, gc * GR), qreg[i]);
    }
  }
  __syncthreads();
  transpose_sw<TI, NT, SWK, SWC>(sKV, LK, sKt, LC, C, DK, tid);
  row_inv_norms<TI, DK, NT>(sKV, LK, C, p.eps, sRk, tid);  // sums are order-free: the
  row_inv_norms<TI, DK, NT>(sQ, LK, C, p.eps, sRq, tid);   // swizzle only permutes a row

  // Raw K K^T (waves 0..NB-1) and Q K^T (waves 4..4+NB-1), one row tile
  // against every column tile.  The tiles stay in registers for all value
  // heads of the group; norms and gates are applied when A and P are built.
  const bool g_wave = wave < NB;
  const bool s_wave = wave >= 4 && wave - 4 < NB;
  const int rt = g_wave ? wave : wave - 4;
  f32x4 acc_gs[1][NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc_gs[0][j] = zero4();
  if (g_wave || s_wave) {
    mma_block_sw<1, NB, DK, SWK, SWK>(acc_gs, g_wave ? sKV : sQ, LK, 16 * rt, sKV, LK, 0, lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) settle(acc_gs[0][j]);
  }
  __syncthreads();

  for (int gi = 0; gi < grp; ++gi) {
    const int h = kh * grp + gi;
    const int64_t blk = (int64_t)c * p.hv + h;

    // v rows into the T region and the gate scan; then the next value
    // head's inputs are requested.
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const int idx = tid + i * NT;
      if (idx < C * GPRV) {
        const int r = idx / GPRV, gc = idx % GPRV;
        st16(sVr + r * LV + swz<TI, SWV>(r, gc * GR), vreg[i]);
      }
    }
    if (wave == 0) {
      float x = gv;  // inclusive scan over the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      const float glast = __shfl(x, C - 1);
      if (lane < C) {
        const float eg = fast_exp(x);
        sGam[lane] = x;
        sBeta[lane] = bv;
        sEg[lane] = eg;
        sKs[lane] = sRk[lane] * fast_exp(glast - x);
        sCb[lane] = bv * eg * sRk[lane];
      }
    }
    if (gi + 1 < grp) load_head(h + 1);
    __syncthreads();

    // V^T [dv][s] from the v rows, and A from the K K^T tiles:
    // A_rs = beta_r exp(gamma_r - gamma_s) rk_r rk_s (k_r . k_s), s < r
    // (only the strictly lower part is ever read).
    transpose_sw<TI, NT, SWV, SWC>(sVr, LV, sKV, LC, C, DV, tid);
    if (g_wave) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j > rt) continue;
        const int col = 16 * j + (lane & 15);
        const float gc = sGam[col], rkc = sRk[col];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + (lane >> 4) * 4 + e;
          if (col < row)
            sA[row * LF + col] = sBeta[row] * sRk[row] * rkc * fast_exp(sGam[row] - gc) * acc_gs[0][j][e];
        }
      }
    }
    __syncthreads();

    // T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution, one
    // lane per column; then block rows i = 1.. by
    //   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj   (fp32 MFMA; the inner sum
    // stays in registers as the second operand).
    if (wave == 0) {
      const int b = lane >> 4, col = lane & 15;
      if (b < NB) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
        const float* Ab = sA + (16 * b) * LF + 16 * b;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
          float acc = x[r];
#pragma unroll
          for (int s2 = 0; s2 < r; ++s2) acc -= Ab[r * LF + s2] * x[s2];
          x[r] = acc;
          // one row's operands at a time: keeps the register footprint small
          __builtin_amdgcn_sched_barrier(0);
        }
        float* Tb = sT + (16 * b) * LF + 16 * b;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * LF + col] = x[i];
      }
    }
    __syncthreads();
    for (int bi = 1; bi < NB; ++bi) {
      if (wave < bi) {
        const int bj = wave;
        f32x4 m = zero4();
        for (int bk = bj; bk < bi; ++bk)
          mma16_f32_kn(m, sA + (16 * bi) * LF + 16 * bk, LF, sT + (16 * bk) * LF + 16 * bj, LF, lane);
        settle(m);
        f32x4 t = zero4();
        mma16_f32_acc_b(t, sT + (16 * bi) * LF + 16 * bi, LF, m, lane);
        settle(t);
        float* dst = sT + (16 * bi) * LF + 16 * bj;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[((lane >> 4) * 4 + e) * LF + (lane & 15)] = -t[e];
      }
      __syncthreads();
    }

    // Tb = T diag(beta e^gamma rk), Tv = T diag(beta) (8 columns per item),
    // and P = scale D o (Q^K^T) from the Q K^T tiles.
    for (int idx = tid; idx < C * (C / 8); idx += NT) {
      const int r = idx / (C / 8), s0 = (idx % (C / 8)) * 8;
      typedef TI vec8 __attribute__((ext_vector_type(8)));
      vec8 tb, tv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = (s0 + j <= r) ? sT[r * LF + s0 + j] : 0.f;
        tb[j] = from_float<TI>(t * sCb[s0 + j]);
        tv[j] = from_float<TI>(t * sBeta[s0 + j]);
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
    if (s_wave) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = 16 * j + (lane & 15);
        const float gc = sGam[col], rkc = sRk[col];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + (lane >> 4) * 4 + e;
          const float pv = (col <= row)
              ? p.scale * sRq[row] * rkc * fast_exp(sGam[row] - gc) * acc_gs[0][j][e] : 0.f;
          sP[row * LC + swz<TI, SWC>(row, col)] = from_float<TI>(pv);
        }
      }
    }
    __syncthreads();

    // U~ = Tv V (all chunk row tiles x d_v tile `wave`): accumulator tiles
    // to global memory, U~^T [dv][r] into the T region.
    TI* ut_g = (TI*)p.im.ut + blk * DV * C;
    if (wave < NVT) {
      const int j = wave;
      f32x4 acc[NB][1];
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i][0] = zero4();
      mma_block_sw<NB, 1, C, SWC, SWC>(acc, sTv, LC, 0, sKV, LC, 16 * j, lane);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int dv = 16 * j + (lane & 15), r0 = 16 * i + (lane >> 4) * 4;
        store_acc_tile<TI>(ut_g + (i * NVT + j) * 256, acc[i][0], lane);
        store4<TI>(sUt + dv * LC + swz<TI, SWC>(dv, r0), acc[i][0][0], acc[i][0][1], acc[i][0][2],
                   acc[i][0][3]);
      }
    }
    __syncthreads();

    // W^T tiles (rows d_k, columns r): W[r][dk] = sum_s Tb[r][s] K[s][dk].
    // W in fragment order to global memory, W^T [dk][r] over the dead V^T.
    // The q rows for Q' are requested here and used after the next barrier.
    constexpr int KPW = 1;  // d_k tiles per wave
    const int i0 = wave;
    typename Raw4<TI>::type qraw[KPW][NB];
    if (i0 < NKT) {
#pragma unroll
      for (int i = 0; i < KPW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = 16 * j + (lane & 15), dk0 = 16 * (i0 + i) + (lane >> 4) * 4;
          qraw[i][j] = typename Raw4<TI>::type{};
          if (r < n) qraw[i][j] = load_raw4<TI>(qg + (int64_t)(t0 + r) * p.q_st + kh * p.q_sh + dk0);
        }
      TI* w_g = (TI*)p.im.w + blk * C * DK;
      f32x4 acc[KPW][NB];
#pragma unroll
      for (int i = 0; i < KPW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = zero4();
      mma_block_sw<KPW, NB, C, SWC, SWC>(acc, sKt, LC, 16 * i0, sTb, LC, 0, lane);
#pragma unroll
      for (int i = 0; i < KPW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = 16 * j + (lane & 15), dk0 = 16 * (i0 + i) + (lane >> 4) * 4;
          store4<TI>(w_g + j * 16 * DK + frag_pos<DK>(lane & 15, dk0), acc[i][j][0], acc[i][j][1],
                     acc[i][j][2], acc[i][j][3]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sKV[(dk0 + e) * LC + swz<TI, SWC>(dk0 + e, r)] = from_float<TI>(acc[i][j][e]);
        }
    }
    __syncthreads();

    // Q' = scale diag(e^gamma rq) Q - P W (Q'^T tiles, fragment order), and
    // O_loc = P U~ (O_loc^T tiles).
    if (i0 < NKT) {
      TI* qp_g = (TI*)p.im.qp + blk * C * DK;
      f32x4 acc[KPW][NB];
#pragma unroll
      for (int i = 0; i < KPW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = zero4();
      mma_block_sw<KPW, NB, C, SWC, SWC>(acc, sKV, LC, 16 * i0, sP, LC, 0, lane);
#pragma unroll
      for (int i = 0; i < KPW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = 16 * j + (lane & 15), dk0 = 16 * (i0 + i) + (lane >> 4) * 4;
          const float qs = p.scale * sEg[r] * sRq[r];
          const f32x4 qv = raw4_to_f32<TI>(qraw[i][j]);
          store4<TI>(qp_g + j * 16 * DK + frag_pos<DK>(lane & 15, dk0), qs * qv[0] - acc[i][j][0],
                     qs * qv[1] - acc[i][j][1], qs * qv[2] - acc[i][j][2], qs * qv[3] - acc[i][j][3]);
        }
    }
    TI* ol_g = (TI*)p.im.oloc + blk * C * DV;
    if (wave < NVT) {
      const int v0 = wave;
      f32x4 acc[1][NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[0][j] = zero4();
      mma_block_sw<1, NB, C, SWC, SWC>(acc, sUt, LC, 16 * v0, sP, LC, 0, lane);
#pragma unroll
      for (int j = 0; j < NB; ++j) store_acc_tile<TI>(ol_g + (v0 * NB + j) * 256, acc[0][j], lane);
    }
    // K~^T [dk][r] = K^T[dk][r] rk_r e^(gamma_last - gamma_r), in fragment
    // order per 16-row tile of d_k (contraction over r), four at a time.
    TI* kt_g = (TI*)p.im.kt + blk * DK * C;
    for (int idx = tid; idx < DK * (C / 4); idx += NT) {
      const int dk = idx / (C / 4), r0 = (idx % (C / 4)) * 4;
      const f32x4 kv = load4<TI>(sKt + dk * LC + swz<TI, SWC>(dk, r0));
      const f32x4 ks = *(const f32x4*)(sKs + r0);
      store4<TI>(kt_g + (dk / 16) * 16 * C + frag_pos<C>(dk % 16, r0), kv[0] * ks[0],
                 kv[1] * ks[1], kv[2] * ks[2], kv[3] * ks[3]);
    }
    if (tid == 0) p.im.decay[blk] = sEg[C - 1];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// state scan fused with the output

template <typename TI, int C, int DK>
struct ScanLayout {
  static constexpr int S = sizeof(TI);
  static constexpr int PADE = 16 / S;
  static constexpr int LK = DK + PADE;
  static constexpr int LC = C + PADE;
  static constexpr int r_ht = 0;                   // H^T slice [16][LK]
  static constexpr int r_ut = 16 * LK * S;         // U^T slice [16][LC]
  static constexpr int total = r_ut + 16 * LC * S;
};

// Everything one wave needs from global memory for one chunk step.  The
// values are kept exactly as loaded (no conversion) so that issuing the loads
// never waits for them; they are consumed a few steps later.
template <typename TI, int C, int DK>
struct ScanStage {
  static constexpr int NHW = (DK / 16 + 3) / 4;
  Frag<TI, DK> w, q;                 // this wave's 16 rows of W and Q'
  Frag<TI, C> kt[NHW];               // this wave's 16-row tiles of K~^T
  typename Raw4<TI>::type ut, ol;    // U~ (U layout) and O_loc (O^T layout)
  float dec;                         // e^gamma_last
};

// Every wave issues the same loads whatever its share of the work (tile
// indices are clamped; a clamped tile is loaded but not used), so the
// number of loads in flight is fixed and the compiler can wait for exactly
// the stage it needs.
template <typename TI, int C, int DK>
__device__ __forceinline__ void scan_load(ScanStage<TI, C, DK>& st, const ScanParams& p,
                                          int cc, int h, int sl, int wave, int lane) {
  constexpr int NB = C / 16, NKT = DK / 16;
  const int64_t blk = (int64_t)cc * p.hv + h;
  const int NVT = p.dv / 16;
  const int wt = NB >= 4 ? wave : min(wave, NB - 1);
  st.w.load((const TI*)p.im.w + blk * C * DK + wt * 16 * DK, lane);
  st.q.load((const TI*)p.im.qp + blk * C * DK + wt * 16 * DK, lane);
  st.ut = load_raw4<TI>((const TI*)p.im.ut + blk * C * p.dv + (wt * NVT + sl) * 256 + lane * 4);
  st.ol = load_raw4<TI>((const TI*)p.im.oloc + blk * C * p.dv + (sl * NB + wt) * 256 + lane * 4);
#pragma unroll
  for (int j = 0; j < ScanStage<TI, C, DK>::NHW; ++j) {
    const int ti = min(wave + 4 * j, NKT - 1);
    st.kt[j].load((const TI*)p.im.kt + blk * DK * C + ti * 16 * C, lane);
  }
  st.dec = p.im.decay[blk];
}

template <typename TI, int C, int DK>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanParams p) {
  using L = ScanLayout<TI, C, DK>;
  using Stage = ScanStage<TI, C, DK>;
  constexpr int LK = L::LK, LC = L::LC;
  constexpr int NB = C / 16;
  constexpr int NKT = DK / 16;
  constexpr int NHW = Stage::NHW;
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  TI* sHt = (TI*)(smem + L::r_ht);
  TI* sUt = (TI*)(smem + L::r_ut);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NS = p.n_slices;
  // XCD-aware: the slices of one (sequence, head) share blockIdx % 8 and so
  // land on the same XCD, where they share W, Q' and K~^T through its L2.
  const int b = blockIdx.x;
  const int u = (b / (8 * NS)) * 8 + (b % 8);
  const int sl = (b / 8) % NS;
  if (u >= p.map.n_seq * p.hv) return;
  const int seq = u / p.hv, h = u % p.hv;
  const int DV = p.dv;
  const int dv0 = 16 * sl;
  int c_begin, c_end, tok0, tok_end;
  seq_range(p.map, seq, C, c_begin, c_end, tok0, tok_end);

  const int64_t sbase = ((int64_t)seq * p.hv + h) * DK * DV;
  f32x4 hacc[NHW];
#pragma unroll
  for (int j = 0; j < NHW; ++j) {
    hacc[j] = zero4();
    const int ti = wave + 4 * j;
    if (ti < NKT && p.init) {
      const int dk0 = 16 * ti + (lane >> 4) * 4, dv = dv0 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[j][e] = p.init[sbase + (int64_t)(dk0 + e) * DV + dv];
    }
  }
  TI* outg = (TI*)p.out;

  // One chunk step: H -> LDS; U = U~ - W H and O = Q' H + O_loc; U -> LDS;
  // H <- e^gamma_last H + K~^T U.
  auto step = [&](const Stage& st, int cc) {
#pragma unroll
    for (int j = 0; j < NHW; ++j) {
      const int ti = wave + 4 * j;
      if (ti < NKT)
        store4<TI>(sHt + (lane & 15) * LK + 16 * ti + (lane >> 4) * 4, hacc[j][0], hacc[j][1],
                   hacc[j][2], hacc[j][3]);
    }
    __syncthreads();
    if (NB >= 4 || wave < NB) {
      f32x4 au = zero4(), ao = zero4();
      mma_pair_lds<DK>(au, ao, st.w, st.q, sHt, LK, lane);
      settle(au);
      settle(ao);
      const f32x4 ut = raw4_to_f32<TI>(st.ut), ol = raw4_to_f32<TI>(st.ol);
      store4<TI>(sUt + (lane & 15) * LC + 16 * wave + (lane >> 4) * 4, ut[0] - au[0],
                 ut[1] - au[1], ut[2] - au[2], ut[3] - au[3]);
      const int tok = tok0 + (cc - c_begin) * C;
      const int r = 16 * wave + (lane & 15);
      if (r < tok_end - tok)
        store4<TI>(outg + (int64_t)(tok + r) * p.o_st + (int64_t)h * p.o_sh + dv0 + (lane >> 4) * 4,
                   ao[0] + ol[0], ao[1] + ol[1], ao[2] + ol[2], ao[3] + ol[3]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NHW; ++j) {
      const int ti = wave + 4 * j;
      if (ti < NKT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[j][e] *= st.dec;
        mma_frag_lds<C>(hacc[j], st.kt[j], sUt, LC, lane);
        settle(hacc[j]);
      }
    }
  };

  // Three stages in flight: the loads for chunk c + 3 are issued as soon as
  // chunk c's registers are consumed.  Loads past the last chunk re-read it
  // (clamped) so that every iteration issues the same loads.
  if (c_begin < c_end) {
    const int last = c_end - 1;
    Stage s0, s1, s2;
    scan_load(s0, p, c_begin, h, sl, wave, lane);
    scan_load(s1, p, min(c_begin + 1, last), h, sl, wave, lane);
    scan_load(s2, p, min(c_begin + 2, last), h, sl, wave, lane);
    for (int cc = c_begin; cc < c_end; cc += 3) {
      step(s0, cc);
      scan_load(s0, p, min(cc + 3, last), h, sl, wave, lane);
      if (cc + 1 < c_end) step(s1, cc + 1);
      scan_load(s1, p, min(cc + 4, last), h, sl, wave, lane);
      if (cc + 2 < c_end) step(s2, cc + 2);
      scan_load(s2, p, min(cc + 5, last), h, sl, wave, lane);
    }
  }

  if (p.final_state) {
#pragma unroll
    for (int j = 0; j < NHW; ++j) {
      const int ti = wave + 4 * j;
      if (ti < NKT) {
        const int dk0 = 16 * ti + (lane >> 4) * 4, dv = dv0 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) p.final_state[sbase + (int64_t)(dk0 + e) * DV + dv] = hacc[j][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch

// fp32 inputs are built for chunks of 16 and 32 only (their WY tiles at 64
// would exceed the LDS or the register budget).
template <typename TI, int C, int DK>
static constexpr bool fits() {
  return WyLayout<TI, C, DK>::total <= kLdsLimit && ScanLayout<TI, C, DK>::total <= kLdsLimit &&
         (sizeof(TI) == 2 || C <= 32);
}

template <typename TI, int C, int DK>
static int launch_pair(int stage, const WyParams* wy, const ScanParams* sc,
                       dim3 grid, hipStream_t s) {
  if constexpr (fits<TI, C, DK>()) {
    if (stage == 0) hipLaunchKernelGGL((wy_kernel<TI, C, DK>), grid, dim3(kWyThreads), 0, s, *wy);
    else hipLaunchKernelGGL((scan_kernel<TI, C, DK>), grid, dim3(kThreads), 0, s, *sc);
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

hipError_t launch_table(const TableParams& p, hipStream_t s) {
  hipLaunchKernelGGL(table_kernel, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wy(bool bf16, int chunk, int dk, const WyParams& p,
                     int grid_x, int grid_y, hipStream_t s) {
  const dim3 grid(grid_x, grid_y);
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

}  // namespace gdn
