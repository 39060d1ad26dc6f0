// Parameter blocks shared by the host launcher and the gfx950 kernels of the
// chunked Gated DeltaNet prefill.  Plain structs passed by value as kernel
// arguments.
#pragma once

#include <stdint.h>

namespace gdn {

// Widest short convolution (GDN_FLAG_QKV_CONV) the kernels take.
constexpr int kConvMaxWidth = 4;

// How a global chunk id maps to (sequence, first token, length).
//   uniform: n_seq sequences of seq_len tokens each, seq_stride tokens
//            apart (seq_len, or more for a segment of longer sequences),
//            chunk ids in sequence order; no table is read.
//   packed:  the chunk table built on the device from cu_seqlens.
struct ChunkMap {
  int32_t packed;        // 0 = uniform, 1 = packed
  int32_t n_seq;
  int32_t seq_len;       // uniform mode: tokens per sequence
  int32_t seq_stride;    // uniform mode: tokens from one sequence's first token to the next's
  int32_t chunks_per_seq;// uniform mode
  const int32_t* table;      // packed: int32[max_chunks][4]
  const int32_t* chunk_off;  // packed: int32[n_seq + 1]
  const int32_t* seq_start;  // packed: sanitised cu_seqlens, int32[n_seq + 1]
};

struct TableParams {
  const void* cu;        // caller's cu_seqlens, [n_seq + 1] int32 or int64 (cu_i64)
  int32_t cu_i64;
  int32_t* seq_start;    // out: sanitised copy
  int32_t* chunk_off;    // out: exclusive prefix of chunk counts
  int32_t* table;        // out: per chunk (seq, t0, n, 0)
  int32_t n_seq;
  int32_t t_total;
  int32_t chunk;
  int32_t max_chunks;
};

// Per-(chunk, value head) intermediates, all in the input element type.
// W and U~ are stored with row r scaled by s_r = e^(gamma_last - gamma_r)
// / |k_r|, so that the state update takes k's own rows: K~^T U = K^T diag(s) U.
struct Intermediates {
  void* w;       // [C][dk]  diag(s) W
  void* qp;      // [C][dk]
  void* ut;      // [dv][C]  diag(s) U~
  void* oloc;    // [C][dv]
  float* decay;  // [chunk][Hv]
};

struct WyParams {
  const void* q;  // [T, Hk, dk] with token stride q_st, head stride q_sh
  const void* k;
  const void* v;  // [T, Hv, dv]
  const float* g;     // [T, Hv] strides g_st, g_sh
  const float* beta;  // [T, Hv] strides b_st, b_sh
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  int64_t g_st, g_sh, b_st, b_sh;
  int32_t hk, hv, dv;
  int32_t n_items;    // (chunk, key head) work items: max_chunks * hk
  int32_t beta_logits;  // 1: beta holds logits b, the kernel takes sigmoid(b)
  int32_t decay_proj;   // 1: g holds the projection a, the kernel takes decay_gate(a)
  const float* a_log;   // [Hv] or null (zeros), with decay_proj
  const float* a_bias;  // [Hv] or null (zeros), with decay_proj
  int32_t qkv_silu;     // 1: q, k, v hold pre-activation values, the kernel takes silu
  void* k_act;          // with qkv_silu or the convolution: key rows as used, [T][Hk][dk] contiguous
  // the short convolution before the activation (conv_w null: none)
  const float* conv_w;      // taps [conv_d][conv_width] f32
  const void* conv_state;   // raw rows before each sequence [N][conv_width - 1][conv_d], or null (zeros)
  int32_t conv_width;       // 1 .. 4
  int32_t conv_d;           // channels: 2 hk dk + hv dv (q | k | v)
  int32_t conv_cont;        // 1: the first chunk of a sequence here continues it (a later
                            // segment): its history rows are the input rows before it
  float scale, eps;
  ChunkMap map;
  Intermediates im;
};

struct ScanParams {
  void* out;             // [T, Hv, dv] strides o_st, o_sh
  int64_t o_st, o_sh;
  const void* k;         // [T, Hk, dk] strides k_st, k_sh: the state update's K rows
  int64_t k_st, k_sh;
  int32_t grp;           // value heads per key head
  const float* init;     // [N, Hv, dk, dv] or null
  float* final_state;    // [N, Hv, dk, dv] or null
  int32_t hv, dv;
  int32_t nsl;           // 16-column slices per workgroup (1, 2 or 4)
  int32_t n_slices;      // workgroups per (sequence, head): dv / (16 nsl)
  ChunkMap map;
  Intermediates im;
  // two-level scan (uniform sequences only): chunks in the first segment,
  // 0 for the one-pass scan, and its workspace
  int32_t split;
  void* sp_y;            // Q'_c Phi_c of second-segment chunks [chunk][Hv][C][dk]
  float* sp_hmid;        // state after the first segment [N][Hv][dk][dv]
  void* sp_hmid_t;       // its bf16 transpose [N][Hv][dv][dk]
  float* sp_psi;         // second segment's end state from zero [N][Hv][dk][dv]
  float* sp_phi;         // second segment's transition [N][Hv][dk][dk]
};

// One recurrent step per sequence (decode).
struct DecodeParams {
  const void* q;         // [N, Hk, dk] strides q_st, q_sh
  const void* k;
  const void* v;         // [N, Hv, dv]
  const float* g;        // [N, Hv] strides g_st, g_sh
  const float* beta;
  float* state;          // [N, Hv, dk, dv], read and written in place
  void* out;             // [N, Hv, dv] strides o_st, o_sh
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int64_t g_st, g_sh, b_st, b_sh;
  int32_t n, hk, hv, dv;
  int32_t beta_logits;   // 1: beta holds logits b, the kernel takes sigmoid(b)
  int32_t decay_proj;    // 1: g holds the projection a, the kernel takes decay_gate(a)
  const float* a_log;    // [Hv] or null (zeros), with decay_proj
  const float* a_bias;   // [Hv] or null (zeros), with decay_proj
  int32_t qkv_silu;      // 1: q, k, v hold pre-activation values, the kernel takes silu
  const float* conv_w;   // the short convolution's taps [conv_d][conv_width], or null (none)
  const void* conv_state;// history rows [N][conv_width - 1][conv_d], or null (zeros)
  int32_t conv_width, conv_d;
  float scale, eps;
};

// The short convolution's state after a call: for every sequence and
// channel, the last width - 1 raw rows of its history followed by its rows.
// Sequences as in ChunkMap (uniform: seq_len tokens seq_len apart; packed:
// the sanitised starts).
struct ConvStateParams {
  const void* q;         // token rows, strides as the inputs'
  const void* k;
  const void* v;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  const void* state_in;  // [N][width - 1][D] or null (zeros)
  void* state_out;       // [N][width - 1][D]; may be state_in
  const int32_t* seq_start;  // packed: int32[n_seq + 1], else null
  int32_t n_seq, seq_len, width, d;
  int32_t hk, dk, dv;
};

// The gated output norm over rows of dv elements: row r is (r / inner,
// r % inner) of a [outer, inner, dv] view with the given strides.
struct GateParams {
  const void* x;
  const void* z;
  void* out;
  const float* w;        // [dv] or null (ones)
  const int32_t* t_end;  // rows of tokens at or after *t_end are left alone (null: none)
  int64_t rows, inner;
  int64_t x_st, x_sh, z_st, z_sh, o_st, o_sh;
  float eps;
};

}  // namespace gdn
