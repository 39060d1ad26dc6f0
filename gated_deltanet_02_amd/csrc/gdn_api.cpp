// C ABI of the chunked Gated DeltaNet prefill (declared in include/gdn.h).
//
// Host side only: argument validation (no HIP call and no device read before
// it passes), workspace layout, and the launch sequence on the caller's
// stream.  Invalid input is rejected before any work is enqueued, as the
// serving pages require of oversize prompts ("Open-Jev-27B-v1.1 native text
// worker", section "Prepare the checkpoint").
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <cstring>
#include <algorithm>
#include <list>
#include <mutex>
#include <string>

#include "gdn.h"
#include "gdn_cu_check.h"
#include "gdn_internal.h"
#include "gdn_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// A token-major view: [T, H, D] (or [B, Tb, H, D] flattened to T = B * Tb).
struct View {
  int64_t T = 0, H = 0, D = 0;
  int64_t st = 0, sh = 0;  // token and head strides (elements)
  int64_t B = 1;           // leading batch of a 4-D view
};

// 3-D/4-D per-head vectors (q, k, v, out).
int parse_vec_tensor(const gdn_tensor* t, const char* name, View* v) {
  if (t->ndim == 3) {
    v->B = 1;
    v->T = t->shape[0];
    v->H = t->shape[1];
    v->D = t->shape[2];
    v->st = t->stride[0];
    v->sh = t->stride[1];
  } else if (t->ndim == 4) {
    v->B = t->shape[0];
    v->T = t->shape[0] * t->shape[1];
    v->H = t->shape[2];
    v->D = t->shape[3];
    v->st = t->stride[1];
    v->sh = t->stride[2];
  } else {
    return fail(GDN_ERR_SHAPE, "%s: expected 3 or 4 dimensions, got %d", name, t->ndim);
  }
  int64_t numel = 1;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] < 0) return fail(GDN_ERR_SHAPE, "%s: negative size", name);
    numel *= t->shape[i];
  }
  if (numel == 0) return GDN_OK;  // strides of an empty tensor carry no layout
  for (int i = 0; i < t->ndim; ++i)
    if (t->stride[i] < 0) return fail(GDN_ERR_LAYOUT, "%s: negative stride", name);
  if (t->stride[t->ndim - 1] != 1) return fail(GDN_ERR_LAYOUT, "%s: last dimension must have unit stride", name);
  if (t->ndim == 4 && t->shape[0] > 1 && t->stride[0] != t->shape[1] * t->stride[1])
    return fail(GDN_ERR_LAYOUT, "%s: batch stride must equal seq_len * token stride", name);
  return GDN_OK;
}

// 2-D/3-D per-head scalars (g, beta).
int parse_scalar_tensor(const gdn_tensor* t, const char* name, View* v) {
  if (t->ndim == 2) {
    v->B = 1;
    v->T = t->shape[0];
    v->H = t->shape[1];
    v->st = t->stride[0];
    v->sh = t->stride[1];
  } else if (t->ndim == 3) {
    v->B = t->shape[0];
    v->T = t->shape[0] * t->shape[1];
    v->H = t->shape[2];
    v->st = t->stride[1];
    v->sh = t->stride[2];
  } else {
    return fail(GDN_ERR_SHAPE, "%s: expected 2 or 3 dimensions, got %d", name, t->ndim);
  }
  int64_t numel = 1;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] < 0) return fail(GDN_ERR_SHAPE, "%s: negative size", name);
    numel *= t->shape[i];
  }
  if (numel == 0) return GDN_OK;
  for (int i = 0; i < t->ndim; ++i)
    if (t->stride[i] < 0) return fail(GDN_ERR_LAYOUT, "%s: negative stride", name);
  if (t->ndim == 3 && t->shape[0] > 1 && t->stride[0] != t->shape[1] * t->stride[1])
    return fail(GDN_ERR_LAYOUT, "%s: batch stride must equal seq_len * token stride", name);
  return GDN_OK;
}

bool supported_head_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Problem {
  bool bf16 = true;
  int chunk = 64;
  int dk = 0, dv = 0, hk = 0, hv = 0;
  int64_t T = 0;
  int n_seq = 1;
  bool packed = false;
  int seq_len = 0, chunks_per_seq = 0;
  int64_t max_chunks = 0;
  View q, k, v, o, g, b;
  float scale = 1.f, eps = 1e-6f;
  uint32_t stages = GDN_STAGE_ALL;
  int scan_split = GDN_SCAN_AUTO;
  bool beta_logits = false;
  bool decay_proj = false;   // GDN_FLAG_DECAY_PROJ
  bool out_gate = false;     // GDN_FLAG_OUTPUT_GATE
  bool qkv_silu = false;     // GDN_FLAG_QKV_SILU
  bool qkv_conv = false;     // GDN_FLAG_QKV_CONV
  const float* conv_w = nullptr;
  int conv_width = 0;
  const void* conv_in = nullptr;
  void* conv_out = nullptr;
  const float* a_log = nullptr;
  const float* a_bias = nullptr;
  const void* gate_z = nullptr;
  const float* norm_w = nullptr;
  float norm_eps = 1e-6f;
  int split = 0;  // two-level scan: chunks in the first segment (0: one pass)
  int seg_opt = 0;           // gdn_options.segment_chunks
  int64_t seg_chunks = 0;    // chunks per segment (0: one pass over all chunks)
};

constexpr uint32_t kKnownFlags =
    GDN_FLAG_BETA_LOGITS | GDN_FLAG_DECAY_PROJ | GDN_FLAG_OUTPUT_GATE | GDN_FLAG_QKV_SILU |
    GDN_FLAG_QKV_CONV;

// Checks of the gate fields of gdn_options that need no shapes.
int check_gate_options(const gdn_options& o) {
  if (o.flags & ~kKnownFlags) return fail(GDN_ERR_SHAPE, "unknown flag bits 0x%x", o.flags);
  if (!(o.norm_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "norm_eps must be >= 0");
  if ((uintptr_t)o.decay_a_log % 4 || (uintptr_t)o.decay_bias % 4 || (uintptr_t)o.norm_weight % 4)
    return fail(GDN_ERR_LAYOUT, "decay_a_log, decay_bias and norm_weight must be 4-byte aligned");
  if (o.flags & GDN_FLAG_QKV_CONV) {
    if (o.conv_width < 1 || o.conv_width > gdn::kConvMaxWidth)
      return fail(GDN_ERR_SHAPE, "conv_width must be 1 .. %d (got %d)", gdn::kConvMaxWidth, o.conv_width);
    if ((uintptr_t)o.conv_weight % 16 || (uintptr_t)o.conv_state_in % 16 ||
        (uintptr_t)o.conv_state_out % 16)
      return fail(GDN_ERR_LAYOUT, "conv_weight, conv_state_in and conv_state_out must be 16-byte aligned");
  }
  return GDN_OK;
}

struct Layout {
  size_t table = 0, chunk_off = 0, seq_start = 0, decay = 0;
  size_t w = 0, qp = 0, ut = 0, oloc = 0;
  size_t y = 0, hmid = 0, hmid_t = 0, psi = 0, phi = 0, carry = 0, kact = 0, total = 0;
};

// Bytes of the intermediates of one (chunk, value head): W, Q', U~, O_loc
// and the decay.
size_t block_bytes(const Problem& P) {
  const size_t es = P.bf16 ? 2 : 4;
  return (size_t)P.chunk * (2 * P.dk + 2 * P.dv) * es + 4;
}

Layout make_layout(const Problem& P) {
  Layout L;
  const size_t es = P.bf16 ? 2 : 4;
  const size_t blocks = (size_t)P.max_chunks * P.hv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.table = take(P.packed ? (size_t)P.max_chunks * 16 : 0);
  L.chunk_off = take(P.packed ? (size_t)(P.n_seq + 1) * 4 : 0);
  L.seq_start = take(P.packed ? (size_t)(P.n_seq + 1) * 4 : 0);
  L.decay = take(blocks * 4);
  L.w = take(blocks * P.chunk * P.dk * es);
  L.qp = take(blocks * P.chunk * P.dk * es);
  L.ut = take(blocks * P.chunk * P.dv * es);
  L.oloc = take(blocks * P.chunk * P.dv * es);
  if (P.split > 0) {
    const size_t heads = (size_t)P.n_seq * P.hv;
    L.y = take(blocks * P.chunk * P.dk * 2);
    L.hmid = take(heads * P.dk * P.dv * 4);
    L.hmid_t = take(heads * P.dv * P.dk * 2);
    L.psi = take(heads * P.dk * P.dv * 4);
    L.phi = take(heads * P.dk * P.dk * 4);
  }
  if (P.seg_chunks > 0) L.carry = take((size_t)P.n_seq * P.hv * P.dk * P.dv * 4);
  if (P.qkv_silu || P.qkv_conv) L.kact = take((size_t)P.T * P.hk * P.dk * es);
  L.total = off;
  return L;
}

int resolve_options(const gdn_options* opts, bool bf16, Problem* P) {
  gdn_options o;
  gdn_default_options(&o);
  if (opts) o = *opts;
  int chunk = o.chunk;
  if (chunk == 0) chunk = bf16 ? 64 : 32;
  if (chunk != 16 && chunk != 32 && chunk != 64)
    return fail(GDN_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", chunk);
  if (!(o.l2_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "l2_eps must be >= 0");
  if ((o.stages & ~GDN_STAGE_ALL) != 0) return fail(GDN_ERR_SHAPE, "unknown stage bits 0x%x", o.stages);
  if (o.scan_split < GDN_SCAN_AUTO || o.scan_split > GDN_SCAN_TWO_LEVEL)
    return fail(GDN_ERR_SHAPE, "unknown scan_split %d", o.scan_split);
  if (o.segment_chunks < -1) return fail(GDN_ERR_SHAPE, "segment_chunks must be >= -1 (got %d)", o.segment_chunks);
  int rc;
  if ((rc = check_gate_options(o))) return rc;
  P->chunk = chunk;
  P->scale = o.scale;
  P->eps = o.l2_eps;
  P->stages = o.stages;
  P->scan_split = o.scan_split;
  P->beta_logits = (o.flags & GDN_FLAG_BETA_LOGITS) != 0;
  P->decay_proj = (o.flags & GDN_FLAG_DECAY_PROJ) != 0;
  P->out_gate = (o.flags & GDN_FLAG_OUTPUT_GATE) != 0;
  P->qkv_silu = (o.flags & GDN_FLAG_QKV_SILU) != 0;
  P->qkv_conv = (o.flags & GDN_FLAG_QKV_CONV) != 0;
  P->conv_w = P->qkv_conv ? o.conv_weight : nullptr;
  P->conv_width = P->qkv_conv ? o.conv_width : 0;
  P->conv_in = P->qkv_conv ? o.conv_state_in : nullptr;
  P->conv_out = P->qkv_conv ? o.conv_state_out : nullptr;
  P->a_log = P->decay_proj ? o.decay_a_log : nullptr;
  P->a_bias = P->decay_proj ? o.decay_bias : nullptr;
  P->gate_z = P->out_gate ? o.gate_z : nullptr;
  P->norm_w = P->out_gate ? o.norm_weight : nullptr;
  P->norm_eps = o.norm_eps;
  P->seg_opt = o.segment_chunks;
  return GDN_OK;
}

// Intermediates the automatic choice keeps per segment (W, Q', U~ and O_loc
// of every sequence and value head; the decays are not counted): half of the 256 MiB
// memory-side cache, the rest left to the inputs and outputs the two
// launches touch.  Measured on MI355X (whole calls): a 16384-token prompt
// with 16 heads (256 MiB of intermediates) takes 323 us in one pass, 281 us
// in segments of 128 chunks (the automatic choice), 278 us in segments of
// 64 and 307 us in segments of 32; with 16 key and 48 value heads 586 us in
// one pass, 554 us in segments of 32 chunks (the automatic choice), 586 us
// in segments of 64 and 689 us in segments of 16.
constexpr size_t kSegmentBytes = (size_t)128 << 20;
constexpr int64_t kMinAutoSegment = 8;
// WY workgroups resident at once on MI355X: 256 compute units, two each.
constexpr int64_t kWySlots = 512;

// Chunks per segment (gdn_options.segment_chunks), 0 for one pass.
void choose_segments(Problem* P) {
  P->seg_chunks = 0;
  if (P->packed || P->split > 0 || P->stages != GDN_STAGE_ALL || P->seg_opt < 0 ||
      P->chunks_per_seq < 2)
    return;
  int64_t seg = P->seg_opt;
  if (seg == 0) {
    const size_t per_chunk = (size_t)P->n_seq * P->hv * (block_bytes(*P) - 4);
    if ((size_t)P->chunks_per_seq * per_chunk <= kSegmentBytes) return;
    const int64_t most = (int64_t)(kSegmentBytes / per_chunk);
    if (most < kMinAutoSegment) return;
    // the longest segment within the budget whose WY work items fill whole
    // rounds of the workgroup slots; else the fewest segments of equal length
    const int64_t items = (int64_t)P->n_seq * P->hk;  // WY work items per chunk position
    const int64_t round = kWySlots / std::gcd(kWySlots, items);
    if (round <= most) {
      seg = most / round * round;
    } else {
      const int64_t n = (P->chunks_per_seq + most - 1) / most;
      seg = (P->chunks_per_seq + n - 1) / n;
    }
  }
  if (seg < P->chunks_per_seq) P->seg_chunks = seg;
}

// The two-level scan's split point (see GDN_SCAN_TWO_LEVEL), 0 for one pass.
// Only on request: measured on MI355X at the 4096-token, 16-head prompt, its
// two launches take longer than the one-pass scan.
int choose_split(Problem* P) {
  P->split = 0;
  if (P->scan_split != GDN_SCAN_TWO_LEVEL) return GDN_OK;
  const bool ok = P->bf16 && !P->packed && P->dk % 32 == 0 && P->dv % 32 == 0 &&
                  P->chunk >= 32 && P->chunks_per_seq >= 2 &&
                  gdn::two_level_available(P->bf16, P->chunk, P->dk);
  if (!ok)
    return fail(GDN_ERR_UNSUPPORTED, "the two-level scan needs bf16 uniform sequences of 2 or more "
                "chunks of 32 or 64, d_k and d_v multiples of 32");
  // about 17/32 of the chunks to the first segment: the first segment's
  // one-slice workgroups step in about 0.88 of the time of the second's
  // two-slice ones (measured 755 and 861 ns per chunk at 128 columns)
  const int64_t heads8 = ((int64_t)P->n_seq * P->hv + 7) / 8 * 8;
  if (heads8 * (P->dv / 16 + (P->dv + P->dk) / 32) >= ((int64_t)1 << 31) ||
      heads8 * P->chunks_per_seq + heads8 * (P->dv / 16) >= ((int64_t)1 << 31))
    return fail(GDN_ERR_SHAPE, "too many (sequence, head) pairs for the two-level scan");
  P->split = std::min(std::max((17 * P->chunks_per_seq + 16) / 32, 1), P->chunks_per_seq - 1);
  return GDN_OK;
}

// Shape/dtype/layout checks shared by every entry point.  When `full` is
// false only the tensors that determine the workspace are examined.
int validate(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
             const gdn_tensor* g, const gdn_tensor* beta, const gdn_tensor* cu,
             const gdn_tensor* init, const gdn_tensor* out,
             const gdn_tensor* fin, const gdn_options* opts, bool full,
             Problem* P) {
  if (!q || !k || !v) return fail(GDN_ERR_NULL_ARG, "q, k and v are required");
  if (full && (!g || !beta || !out)) return fail(GDN_ERR_NULL_ARG, "g, beta and out are required");
  if (q->dtype != GDN_DTYPE_BF16 && q->dtype != GDN_DTYPE_F32)
    return fail(GDN_ERR_DTYPE, "q must be bf16 or f32");
  if (k->dtype != q->dtype || v->dtype != q->dtype || (full && out->dtype != q->dtype))
    return fail(GDN_ERR_DTYPE, "q, k, v and out must share one dtype");
  P->bf16 = q->dtype == GDN_DTYPE_BF16;
  int rc;
  if ((rc = resolve_options(opts, P->bf16, P))) return rc;
  if ((rc = parse_vec_tensor(q, "q", &P->q))) return rc;
  if ((rc = parse_vec_tensor(k, "k", &P->k))) return rc;
  if ((rc = parse_vec_tensor(v, "v", &P->v))) return rc;
  if (q->ndim != k->ndim || q->ndim != v->ndim) return fail(GDN_ERR_SHAPE, "q, k and v must have the same rank");
  if (P->q.T != P->k.T || P->q.H != P->k.H || P->q.D != P->k.D || P->q.B != P->k.B)
    return fail(GDN_ERR_SHAPE, "q and k shapes differ");
  if (P->v.T != P->q.T || P->v.B != P->q.B) return fail(GDN_ERR_SHAPE, "v token count differs from q");
  if (!supported_head_dim(P->q.D) || !supported_head_dim(P->v.D))
    return fail(GDN_ERR_UNSUPPORTED, "d_k and d_v must be 16, 32, 64 or 128 (got %lld, %lld)",
                (long long)P->q.D, (long long)P->v.D);
  if (P->q.H < 1 || P->v.H < 1 || P->v.H % P->q.H)
    return fail(GDN_ERR_SHAPE, "value heads (%lld) must be a positive multiple of key heads (%lld)",
                (long long)P->v.H, (long long)P->q.H);
  if (P->q.H > 65535) return fail(GDN_ERR_UNSUPPORTED, "at most 65535 key heads");
  if (P->q.T >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "T must be < 2^31");
  P->dk = (int)P->q.D;
  P->dv = (int)P->v.D;
  P->hk = (int)P->q.H;
  P->hv = (int)P->v.H;
  P->T = P->q.T;
  if (!gdn::kernels_available(P->bf16, P->chunk, P->dk))
    return fail(GDN_ERR_UNSUPPORTED, "no %s kernel for chunk %d with d_k %d (LDS limit)",
                P->bf16 ? "bf16" : "f32", P->chunk, P->dk);

  // Sequences.
  if (cu) {
    if (cu->dtype != GDN_DTYPE_I32 && cu->dtype != GDN_DTYPE_I64)
      return fail(GDN_ERR_DTYPE, "cu_seqlens must be int32 or int64");
    if (cu->ndim != 1 || cu->shape[0] < 2) return fail(GDN_ERR_SHAPE, "cu_seqlens must be 1-D with N+1 >= 2 entries");
    if (cu->stride[0] != 1) return fail(GDN_ERR_LAYOUT, "cu_seqlens must be contiguous");
    if (!cu->data) return fail(GDN_ERR_NULL_ARG, "cu_seqlens data is NULL");
    if (P->q.B != 1) return fail(GDN_ERR_SHAPE, "with cu_seqlens the batch dimension must be 1");
    if (cu->shape[0] - 1 >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "too many sequences");
    P->n_seq = (int)(cu->shape[0] - 1);
    // the sequence bounds are read on the device from cu_seqlens, also for
    // one sequence (cu = [0, L] with L < T covers L tokens only)
    P->packed = true;
    P->seq_len = 0;
  } else {
    P->n_seq = (int)P->q.B;
    P->packed = false;
    P->seq_len = P->n_seq > 0 ? (int)(P->T / P->n_seq) : 0;
  }
  if (P->n_seq < 1) return fail(GDN_ERR_SHAPE, "at least one sequence is required");
  if (P->packed) {
    P->max_chunks = P->T / P->chunk + P->n_seq;
  } else {
    P->chunks_per_seq = (P->seq_len + P->chunk - 1) / P->chunk;
    P->max_chunks = (int64_t)P->n_seq * P->chunks_per_seq;
  }
  if (P->max_chunks * P->hk >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "too many chunks");
  const int64_t n_slices = P->dv / 16;
  const int64_t scan_blocks = ((int64_t)P->n_seq * P->hv + 7) / 8 * 8 * n_slices;
  if (scan_blocks >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "too many (sequence, head) pairs");
  if ((rc = choose_split(P))) return rc;
  choose_segments(P);
  if (!full) return GDN_OK;

  // The remaining tensors.
  int gr = P->bf16 ? 8 : 4;  // elements per 16 bytes
  if ((rc = parse_vec_tensor(out, "out", &P->o))) return rc;
  if (P->o.T != P->T || P->o.H != P->hv || P->o.D != P->dv) return fail(GDN_ERR_SHAPE, "out must match v");
  if (g->dtype != GDN_DTYPE_F32 || beta->dtype != GDN_DTYPE_F32) return fail(GDN_ERR_DTYPE, "g and beta must be f32");
  if ((rc = parse_scalar_tensor(g, "g", &P->g))) return rc;
  if ((rc = parse_scalar_tensor(beta, "beta", &P->b))) return rc;
  if (P->g.T != P->T || P->g.H != P->hv || P->b.T != P->T || P->b.H != P->hv)
    return fail(GDN_ERR_SHAPE, "g and beta must be [T, Hv]");
  const struct { const gdn_tensor* t; const View* v; const char* n; } vecs[] = {
      {q, &P->q, "q"}, {k, &P->k, "k"}, {v, &P->v, "v"}, {out, &P->o, "out"}};
  for (const auto& x : vecs) {
    if (P->T == 0) break;  // nothing is read or written
    if (!x.t->data) return fail(GDN_ERR_NULL_ARG, "%s data is NULL", x.n);
    if ((uintptr_t)x.t->data % 16) return fail(GDN_ERR_LAYOUT, "%s must be 16-byte aligned", x.n);
    if (x.v->st % gr || x.v->sh % gr)
      return fail(GDN_ERR_LAYOUT, "%s: token/head strides must be multiples of %d elements", x.n, gr);
  }
  if (P->T > 0 && (!g->data || !beta->data)) return fail(GDN_ERR_NULL_ARG, "g/beta data is NULL");
  if (P->qkv_conv && P->T > 0 && !P->conv_w)
    return fail(GDN_ERR_NULL_ARG, "GDN_FLAG_QKV_CONV needs conv_weight");
  if (P->out_gate && P->T > 0) {
    if (!P->gate_z) return fail(GDN_ERR_NULL_ARG, "GDN_FLAG_OUTPUT_GATE needs gate_z");
    if ((uintptr_t)P->gate_z % 16) return fail(GDN_ERR_LAYOUT, "gate_z must be 16-byte aligned");
  }
  if (P->T > 0 && ((uintptr_t)g->data % 4 || (uintptr_t)beta->data % 4))
    return fail(GDN_ERR_LAYOUT, "g/beta must be 4-byte aligned");
  const gdn_tensor* states[2] = {init, fin};
  const char* snames[2] = {"init_state", "final_state"};
  for (int i = 0; i < 2; ++i) {
    const gdn_tensor* s = states[i];
    if (!s) continue;
    if (s->dtype != GDN_DTYPE_F32) return fail(GDN_ERR_DTYPE, "%s must be f32", snames[i]);
    if (s->ndim != 4 || s->shape[0] != P->n_seq || s->shape[1] != P->hv || s->shape[2] != P->dk ||
        s->shape[3] != P->dv)
      return fail(GDN_ERR_SHAPE, "%s must be [N=%d, Hv=%d, dk=%d, dv=%d]", snames[i], P->n_seq, P->hv,
                  P->dk, P->dv);
    if (s->stride[3] != 1 || s->stride[2] != P->dv || s->stride[1] != (int64_t)P->dk * P->dv ||
        s->stride[0] != (int64_t)P->hv * P->dk * P->dv)
      return fail(GDN_ERR_LAYOUT, "%s must be contiguous", snames[i]);
    if (!s->data) return fail(GDN_ERR_NULL_ARG, "%s data is NULL", snames[i]);
    if ((uintptr_t)s->data % 16) return fail(GDN_ERR_LAYOUT, "%s must be 16-byte aligned", snames[i]);
  }
  return GDN_OK;
}

// Decode: one token per sequence.  q, k [N, Hk, dk]; v, out [N, Hv, dv];
// g, beta [N, Hv] f32; state [N, Hv, dk, dv] f32 contiguous.
int validate_decode(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                    const gdn_tensor* g, const gdn_tensor* beta, const gdn_tensor* state,
                    const gdn_tensor* out, const gdn_options* opts, gdn::DecodeParams* d,
                    bool* bf16, int* dk) {
  if (!q || !k || !v || !g || !beta || !state || !out)
    return fail(GDN_ERR_NULL_ARG, "q, k, v, g, beta, state and out are required");
  if (q->dtype != GDN_DTYPE_BF16 && q->dtype != GDN_DTYPE_F32)
    return fail(GDN_ERR_DTYPE, "q must be bf16 or f32");
  if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
    return fail(GDN_ERR_DTYPE, "q, k, v and out must share one dtype");
  if (g->dtype != GDN_DTYPE_F32 || beta->dtype != GDN_DTYPE_F32 || state->dtype != GDN_DTYPE_F32)
    return fail(GDN_ERR_DTYPE, "g, beta and state must be f32");
  const gdn_tensor* vecs[4] = {q, k, v, out};
  const char* names[4] = {"q", "k", "v", "out"};
  for (int i = 0; i < 4; ++i)
    if (vecs[i]->ndim != 3) return fail(GDN_ERR_SHAPE, "%s must be [N, H, D]", names[i]);
  if (g->ndim != 2 || beta->ndim != 2) return fail(GDN_ERR_SHAPE, "g and beta must be [N, Hv]");
  const int64_t N = q->shape[0], hk = q->shape[1], dkk = q->shape[2];
  const int64_t hv = v->shape[1], dv = v->shape[2];
  if (N < 0 || hk < 1 || hv < 1) return fail(GDN_ERR_SHAPE, "bad sizes");
  if (k->shape[0] != N || k->shape[1] != hk || k->shape[2] != dkk) return fail(GDN_ERR_SHAPE, "q and k shapes differ");
  if (v->shape[0] != N || out->shape[0] != N || out->shape[1] != hv || out->shape[2] != dv)
    return fail(GDN_ERR_SHAPE, "v and out must be [N, Hv, dv]");
  if (g->shape[0] != N || g->shape[1] != hv || beta->shape[0] != N || beta->shape[1] != hv)
    return fail(GDN_ERR_SHAPE, "g and beta must be [N, Hv]");
  if (!supported_head_dim(dkk) || !supported_head_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "d_k and d_v must be 16, 32, 64 or 128");
  if (hv % hk) return fail(GDN_ERR_SHAPE, "value heads must be a multiple of key heads");
  if (state->ndim != 4 || state->shape[0] != N || state->shape[1] != hv || state->shape[2] != dkk ||
      state->shape[3] != dv)
    return fail(GDN_ERR_SHAPE, "state must be [N, Hv, dk, dv]");
  if (N * hv >= ((int64_t)1 << 31)) return fail(GDN_ERR_SHAPE, "too many (sequence, head) pairs");
  if (N > 0) {
    for (int i = 0; i < 4; ++i) {
      if (!vecs[i]->data) return fail(GDN_ERR_NULL_ARG, "%s data is NULL", names[i]);
      if (vecs[i]->stride[2] != 1 || vecs[i]->stride[0] < 0 || vecs[i]->stride[1] < 0)
        return fail(GDN_ERR_LAYOUT, "%s: last dimension must have unit stride", names[i]);
    }
    if (!g->data || !beta->data || !state->data) return fail(GDN_ERR_NULL_ARG, "g, beta or state data is NULL");
    if (g->stride[0] < 0 || g->stride[1] < 0 || beta->stride[0] < 0 || beta->stride[1] < 0)
      return fail(GDN_ERR_LAYOUT, "negative stride");
    if (state->stride[3] != 1 || state->stride[2] != dv || state->stride[1] != dkk * dv ||
        state->stride[0] != hv * dkk * dv)
      return fail(GDN_ERR_LAYOUT, "state must be contiguous");
    // v and out are accessed four elements at a time, the state 16 bytes at a time
    const int64_t es = q->dtype == GDN_DTYPE_BF16 ? 2 : 4;
    for (const gdn_tensor* t : {v, out})
      if ((uintptr_t)t->data % (4 * es) || t->stride[0] % 4 || t->stride[1] % 4)
        return fail(GDN_ERR_LAYOUT, "v and out rows must start on 4-element boundaries");
    if ((uintptr_t)state->data % 16) return fail(GDN_ERR_LAYOUT, "state must be 16-byte aligned");
  }
  gdn_options o;
  gdn_default_options(&o);
  if (opts) o = *opts;
  if (!(o.l2_eps >= 0.f)) return fail(GDN_ERR_SHAPE, "l2_eps must be >= 0");
  int rc;
  if ((rc = check_gate_options(o))) return rc;
  if ((o.flags & GDN_FLAG_OUTPUT_GATE) && N > 0) {
    // the gate moves 16-byte granules of out and z (z laid out as out)
    const int64_t epg = q->dtype == GDN_DTYPE_BF16 ? 8 : 4;
    if (!o.gate_z) return fail(GDN_ERR_NULL_ARG, "GDN_FLAG_OUTPUT_GATE needs gate_z");
    if ((uintptr_t)o.gate_z % 16 || (uintptr_t)out->data % 16 || out->stride[0] % epg ||
        out->stride[1] % epg)
      return fail(GDN_ERR_LAYOUT, "with GDN_FLAG_OUTPUT_GATE, out and gate_z rows must start on "
                  "16-byte boundaries");
  }
  d->q = q->data; d->k = k->data; d->v = v->data; d->out = out->data;
  d->g = (const float*)g->data; d->beta = (const float*)beta->data; d->state = (float*)state->data;
  d->q_st = q->stride[0]; d->q_sh = q->stride[1];
  d->k_st = k->stride[0]; d->k_sh = k->stride[1];
  d->v_st = v->stride[0]; d->v_sh = v->stride[1];
  d->o_st = out->stride[0]; d->o_sh = out->stride[1];
  d->g_st = g->stride[0]; d->g_sh = g->stride[1];
  d->b_st = beta->stride[0]; d->b_sh = beta->stride[1];
  d->n = (int32_t)N; d->hk = (int32_t)hk; d->hv = (int32_t)hv; d->dv = (int32_t)dv;
  d->scale = o.scale; d->eps = o.l2_eps;
  d->beta_logits = (o.flags & GDN_FLAG_BETA_LOGITS) ? 1 : 0;
  d->decay_proj = (o.flags & GDN_FLAG_DECAY_PROJ) ? 1 : 0;
  d->qkv_silu = (o.flags & GDN_FLAG_QKV_SILU) ? 1 : 0;
  if (o.flags & GDN_FLAG_QKV_CONV) {
    if (N > 0 && !o.conv_weight) return fail(GDN_ERR_NULL_ARG, "GDN_FLAG_QKV_CONV needs conv_weight");
    d->conv_w = o.conv_weight;
    d->conv_state = o.conv_state_in;
    d->conv_width = o.conv_width;
    d->conv_d = (int32_t)(2 * hk * dkk + hv * dv);
  }
  d->a_log = d->decay_proj ? o.decay_a_log : nullptr;
  d->a_bias = d->decay_proj ? o.decay_bias : nullptr;
  *bf16 = q->dtype == GDN_DTYPE_BF16;
  *dk = (int)dkk;
  return GDN_OK;
}

// Names the fault bits of a cu_seqlens table.
const char* cu_fault_text(int32_t f) {
  if (f & gdn::kCuFirstNonzero) return "cu[0] != 0";
  if (f & gdn::kCuDecreasing) return "entries decrease";
  if (f & gdn::kCuPastEnd) return "cu[N] > T";
  return "malformed";
}

bool debug_check_enabled() {
  const char* e = getenv("GDN_DEBUG_CHECK");
  return e && e[0] == '1' && e[1] == 0;
}

// GDN_DEBUG_CHECK=1: the device table is checked before anything else is
// enqueued (skipped while the stream is being captured).
int debug_check_cu(const Problem& P, const gdn_tensor* cu, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return fail(GDN_ERR_HIP, "hipStreamIsCapturing failed");
  if (cs != hipStreamCaptureStatusNone) return GDN_OK;
  int32_t* word = nullptr;
  hipError_t e = gdn::debug_word_region(&word);
  if (e == hipSuccess)
    e = gdn::launch_check_cu(cu->data, cu->dtype == GDN_DTYPE_I64, P.n_seq, P.T, word, s);
  int32_t faults = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&faults, word, sizeof faults, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "cu_seqlens check: %s", hipGetErrorString(e));
  if (faults) return fail(GDN_ERR_INPUT, "cu_seqlens is malformed (%s; GDN_DEBUG_CHECK)", cu_fault_text(faults));
  return GDN_OK;
}

int run(const Problem& P, const gdn_tensor* q, const gdn_tensor* k,
        const gdn_tensor* v, const gdn_tensor* g, const gdn_tensor* beta,
        const gdn_tensor* cu, const gdn_tensor* init, gdn_tensor* out,
        gdn_tensor* fin, void* ws, hipStream_t s) {
  const Layout L = make_layout(P);
  char* base = (char*)ws;
  gdn::ChunkMap map{};
  map.packed = P.packed ? 1 : 0;
  map.n_seq = P.n_seq;
  map.seq_len = P.seq_len;
  map.seq_stride = P.seq_len;
  map.chunks_per_seq = P.chunks_per_seq;
  map.table = (const int32_t*)(base + L.table);
  map.chunk_off = (const int32_t*)(base + L.chunk_off);
  map.seq_start = (const int32_t*)(base + L.seq_start);
  gdn::Intermediates im{};
  im.w = base + L.w;
  im.qp = base + L.qp;
  im.ut = base + L.ut;
  im.oloc = base + L.oloc;
  im.decay = (float*)(base + L.decay);

  hipError_t e;
  if (P.packed && (P.stages & GDN_STAGE_TABLE) && debug_check_enabled()) {
    const int rc = debug_check_cu(P, cu, s);
    if (rc) return rc;
  }
  if (P.packed && (P.stages & GDN_STAGE_TABLE)) {
    gdn::TableParams tp{};
    tp.cu = cu->data;
    tp.cu_i64 = cu->dtype == GDN_DTYPE_I64 ? 1 : 0;
    tp.seq_start = (int32_t*)(base + L.seq_start);
    tp.chunk_off = (int32_t*)(base + L.chunk_off);
    tp.table = (int32_t*)(base + L.table);
    tp.n_seq = P.n_seq;
    tp.t_total = (int32_t)P.T;
    tp.chunk = P.chunk;
    tp.max_chunks = (int32_t)P.max_chunks;
    if ((e = gdn::launch_table(tp, s)) != hipSuccess)
      return fail(GDN_ERR_HIP, "chunk table launch: %s", hipGetErrorString(e));
  }
  // Byte offsets of token t0 in the token-indexed tensors (a segment's
  // views: its first token, the same strides).
  const size_t es = P.bf16 ? 2 : 4;
  auto at = [](const void* base, int64_t t0, int64_t st, size_t bytes) {
    return (const char*)base + t0 * st * (int64_t)bytes;
  };
  // The WY transform of the chunks `m` maps, inputs from token t0 on.
  auto wy = [&](const gdn::ChunkMap& m, int64_t n_chunks, int64_t t0) -> int {
    gdn::WyParams wp{};
    wp.q = at(q->data, t0, P.q.st, es);
    wp.k = at(k->data, t0, P.k.st, es);
    wp.v = at(v->data, t0, P.v.st, es);
    wp.g = (const float*)at(g->data, t0, P.g.st, 4);
    wp.beta = (const float*)at(beta->data, t0, P.b.st, 4);
    wp.q_st = P.q.st; wp.q_sh = P.q.sh;
    wp.k_st = P.k.st; wp.k_sh = P.k.sh;
    wp.v_st = P.v.st; wp.v_sh = P.v.sh;
    wp.g_st = P.g.st; wp.g_sh = P.g.sh;
    wp.b_st = P.b.st; wp.b_sh = P.b.sh;
    wp.hk = P.hk;
    wp.hv = P.hv;
    wp.dv = P.dv;
    wp.scale = P.scale;
    wp.eps = P.eps;
    wp.map = m;
    wp.im = im;
    wp.n_items = (int32_t)(n_chunks * P.hk);
    wp.beta_logits = P.beta_logits ? 1 : 0;
    wp.decay_proj = P.decay_proj ? 1 : 0;
    wp.a_log = P.a_log;
    wp.a_bias = P.a_bias;
    wp.qkv_silu = P.qkv_silu ? 1 : 0;
    wp.k_act = L.kact ? base + L.kact + t0 * P.hk * P.dk * (int64_t)es : nullptr;
    if (P.qkv_conv) {
      wp.conv_w = P.conv_w;
      wp.conv_state = P.conv_in;
      wp.conv_width = P.conv_width;
      wp.conv_d = 2 * P.hk * P.dk + P.hv * P.dv;
      wp.conv_cont = t0 > 0 ? 1 : 0;  // a later segment continues its sequences
    }
    const hipError_t e = gdn::launch_wy(P.bf16, P.chunk, P.dk, wp, s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "WY launch: %s", hipGetErrorString(e));
    return GDN_OK;
  };
  // The scan of the chunks `m` maps from state `h0` (null: zeros) to `h1`
  // (null: not stored), outputs from token t0 on.
  auto scan = [&](const gdn::ChunkMap& m, int64_t t0, const float* h0, float* h1) -> int {
    gdn::ScanParams sp{};
    sp.out = (void*)at(out->data, t0, P.o.st, es);
    sp.o_st = P.o.st;
    sp.o_sh = P.o.sh;
    sp.init = h0;
    sp.final_state = h1;
    if (L.kact) {  // the WY kernel's key rows as used, [T][Hk][dk] contiguous
      sp.k = base + L.kact + t0 * P.hk * P.dk * (int64_t)es;
      sp.k_st = (int64_t)P.hk * P.dk;
      sp.k_sh = P.dk;
    } else {
      sp.k = at(k->data, t0, P.k.st, es);
      sp.k_st = P.k.st;
      sp.k_sh = P.k.sh;
    }
    sp.grp = P.hv / P.hk;
    sp.hv = P.hv;
    sp.dv = P.dv;
    sp.map = m;
    sp.im = im;
    const int64_t heads8 = ((int64_t)P.n_seq * P.hv + 7) / 8 * 8;
    hipError_t e;
    if (P.split > 0) {
      sp.split = P.split;
      sp.sp_y = base + L.y;
      sp.sp_hmid = (float*)(base + L.hmid);
      sp.sp_hmid_t = base + L.hmid_t;
      sp.sp_psi = (float*)(base + L.psi);
      sp.sp_phi = (float*)(base + L.phi);
      sp.nsl = 2;
      sp.n_slices = P.dv / 16 + (P.dv + P.dk) / 32;  // workgroups per (sequence, head)
      if ((e = gdn::launch_scan_two_level(P.chunk, P.dk, sp, s)) != hipSuccess)
        return fail(GDN_ERR_HIP, "two-level scan launch: %s", hipGetErrorString(e));
    } else {
      sp.nsl = gdn::scan_slices_per_group(P.bf16, P.chunk, P.dk, P.dv, (int64_t)P.n_seq * P.hv);
      sp.n_slices = P.dv / (16 * sp.nsl);
      const int64_t blocks = heads8 * sp.n_slices;
      if ((e = gdn::launch_scan(P.bf16, P.chunk, P.dk, sp, (int)blocks, s)) != hipSuccess)
        return fail(GDN_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
    }
    return GDN_OK;
  };
  const float* h_init = init ? (const float*)init->data : nullptr;
  float* h_fin = fin ? (float*)fin->data : nullptr;
  int rc;
  if (P.seg_chunks > 0) {
    // Segments of whole chunks of every sequence: tokens [t0, t0 + len) of
    // each, the state carried in f32 through the workspace (read and
    // written in place, each element by the lane that owns it).
    float* carry = (float*)(base + L.carry);
    for (int64_t c0 = 0; c0 < P.chunks_per_seq; c0 += P.seg_chunks) {
      const int64_t nc = std::min<int64_t>(P.seg_chunks, P.chunks_per_seq - c0);
      const int64_t t0 = c0 * P.chunk;
      const bool last = c0 + nc >= P.chunks_per_seq;
      gdn::ChunkMap m = map;
      m.seq_len = (int32_t)std::min<int64_t>(P.seq_len - t0, nc * P.chunk);
      m.chunks_per_seq = (int32_t)nc;
      if ((rc = wy(m, (int64_t)P.n_seq * nc, t0))) return rc;
      if ((rc = scan(m, t0, c0 == 0 ? h_init : carry, last ? h_fin : carry))) return rc;
    }
  } else {
    if ((P.stages & GDN_STAGE_WY) && P.max_chunks > 0 && (rc = wy(map, P.max_chunks, 0))) return rc;
    if ((P.stages & GDN_STAGE_SCAN) && (rc = scan(map, 0, h_init, h_fin))) return rc;
  }
  if (P.qkv_conv && P.conv_out && (P.stages & GDN_STAGE_WY)) {
    // the short convolution's history for a later call: after every WY
    // launch has read the old one (it may be the same memory)
    gdn::ConvStateParams cp{};
    cp.q = q->data; cp.k = k->data; cp.v = v->data;
    cp.q_st = P.q.st; cp.q_sh = P.q.sh;
    cp.k_st = P.k.st; cp.k_sh = P.k.sh;
    cp.v_st = P.v.st; cp.v_sh = P.v.sh;
    cp.state_in = P.conv_in;
    cp.state_out = P.conv_out;
    cp.seq_start = P.packed ? (const int32_t*)(base + L.seq_start) : nullptr;
    cp.n_seq = P.n_seq;
    cp.seq_len = P.seq_len;
    cp.width = P.conv_width;
    cp.d = 2 * P.hk * P.dk + P.hv * P.dv;
    cp.hk = P.hk; cp.dk = P.dk; cp.dv = P.dv;
    if ((e = gdn::launch_conv_state(P.bf16, cp, s)) != hipSuccess)
      return fail(GDN_ERR_HIP, "convolution state launch: %s", hipGetErrorString(e));
  }
  if (P.stages & GDN_STAGE_SCAN) {
    if (P.out_gate && P.T > 0) {
      // the gated output norm over the stored rows (packed: up to cu[N])
      gdn::GateParams gp{};
      gp.x = out->data;
      gp.z = P.gate_z;
      gp.out = out->data;
      gp.w = P.norm_w;
      // (the sanitised end the chunk table kept: cu[N] clamped into [0, T])
      gp.t_end = P.packed ? (const int32_t*)(base + L.seq_start) + P.n_seq : nullptr;
      gp.rows = P.T * P.hv;
      gp.inner = P.hv;
      gp.x_st = gp.z_st = gp.o_st = P.o.st;
      gp.x_sh = gp.z_sh = gp.o_sh = P.o.sh;
      gp.eps = P.norm_eps;
      if ((e = gdn::launch_output_gate(P.bf16, P.dv, gp, s)) != hipSuccess)
        return fail(GDN_ERR_HIP, "output gate launch: %s", hipGetErrorString(e));
    }
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

void gdn_default_options(gdn_options* opts) {
  if (!opts) return;
  opts->chunk = 0;  // 64 for bf16, 32 for f32
  opts->scale = 1.0f;
  opts->l2_eps = 1e-6f;
  opts->stages = GDN_STAGE_ALL;
  opts->scan_split = GDN_SCAN_AUTO;
  opts->flags = 0;
  opts->decay_a_log = nullptr;
  opts->decay_bias = nullptr;
  opts->gate_z = nullptr;
  opts->norm_weight = nullptr;
  opts->norm_eps = 1e-6f;
  opts->segment_chunks = 0;
  opts->conv_weight = nullptr;
  opts->conv_width = 4;
  opts->conv_state_in = nullptr;
  opts->conv_state_out = nullptr;
}

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_ARG: return "null argument";
    case GDN_ERR_DTYPE: return "unsupported or mismatched dtype";
    case GDN_ERR_SHAPE: return "inconsistent or out-of-range shape";
    case GDN_ERR_LAYOUT: return "unsupported strides or alignment";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case GDN_ERR_HIP: return "HIP error";
    case GDN_ERR_INPUT: return "malformed input values";
  }
  return "unknown status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_workspace_size(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                       const gdn_tensor* cu_seqlens, const gdn_options* opts, size_t* bytes) {
  if (!bytes) return fail(GDN_ERR_NULL_ARG, "bytes is NULL");
  Problem P;
  const int rc = validate(q, k, v, nullptr, nullptr, cu_seqlens, nullptr, nullptr, nullptr, opts, false, &P);
  if (rc) return rc;
  *bytes = make_layout(P).total;
  return GDN_OK;
}

int gdn_get_workspace_layout(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                             const gdn_tensor* cu_seqlens, const gdn_options* opts,
                             gdn_workspace_layout* layout) {
  if (!layout) return fail(GDN_ERR_NULL_ARG, "layout is NULL");
  Problem P;
  const int rc = validate(q, k, v, nullptr, nullptr, cu_seqlens, nullptr, nullptr, nullptr, opts, false, &P);
  if (rc) return rc;
  const Layout L = make_layout(P);
  layout->total_bytes = L.total;
  layout->max_chunks = P.max_chunks;
  layout->chunk_table = L.table;
  layout->chunk_offsets = L.chunk_off;
  layout->seq_starts = L.seq_start;
  layout->decay = L.decay;
  layout->w = L.w;
  layout->qp = L.qp;
  layout->ut = L.ut;
  layout->oloc = L.oloc;
  layout->split_chunks = P.split;
  layout->split_y = L.y;
  layout->split_hmid = L.hmid;
  layout->split_hmid_t = L.hmid_t;
  layout->split_psi = L.psi;
  layout->split_phi = L.phi;
  layout->segment_chunks = (int32_t)P.seg_chunks;
  layout->segment_state = L.carry;
  layout->k_act = L.kact;
  return GDN_OK;
}

int gdn_prefill_ex(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                   const gdn_tensor* g, const gdn_tensor* beta, const gdn_tensor* cu_seqlens,
                   const gdn_tensor* init_state, gdn_tensor* out, gdn_tensor* final_state,
                   const gdn_options* opts, void* workspace, size_t workspace_bytes, void* stream) {
  Problem P;
  int rc = validate(q, k, v, g, beta, cu_seqlens, init_state, out, final_state, opts, true, &P);
  if (rc) return rc;
  const size_t need = make_layout(P).total;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if ((uintptr_t)workspace % kAlign) return fail(GDN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  g_last_error.clear();
  return run(P, q, k, v, g, beta, cu_seqlens, init_state, out, final_state, workspace,
             (hipStream_t)stream);
}

int gdn_prefill(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                const gdn_tensor* g, const gdn_tensor* beta, const gdn_tensor* cu_seqlens,
                const gdn_tensor* init_state, gdn_tensor* out, gdn_tensor* final_state,
                void* stream) {
  Problem P;
  int rc = validate(q, k, v, g, beta, cu_seqlens, init_state, out, final_state, nullptr, true, &P);
  if (rc) return rc;
  const size_t need = make_layout(P).total;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = hipMallocAsync(&ws, need, s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "workspace allocation of %zu bytes: %s", need, hipGetErrorString(e));
  }
  g_last_error.clear();
  rc = run(P, q, k, v, g, beta, cu_seqlens, init_state, out, final_state, ws, s);
  if (ws) {
    const hipError_t e = hipFreeAsync(ws, s);
    if (rc == GDN_OK && e != hipSuccess) rc = fail(GDN_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
  }
  return rc;
}

int gdn_prefill_noalloc(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                        const gdn_tensor* g, const gdn_tensor* beta,
                        const gdn_tensor* cu_seqlens, const gdn_tensor* init_state,
                        gdn_tensor* out, gdn_tensor* final_state, const gdn_options* opts,
                        void* stream) {
  static_assert(gdn::kScratchBytes == GDN_NOALLOC_SCRATCH_BYTES, "scratch size in gdn.h");
  Problem P;
  int rc = validate(q, k, v, g, beta, cu_seqlens, init_state, out, final_state, opts, true, &P);
  if (rc) return rc;
  const size_t need = make_layout(P).total;
  if (need > gdn::kScratchBytes)
    return fail(GDN_ERR_WORKSPACE,
                "these sizes need a workspace of %zu bytes; the no-allocation prefill's scratch "
                "holds %zu (use gdn_prefill_ex with a larger workspace)",
                need, gdn::kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = gdn::scratch_region(&ws);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "scratch lookup: %s", hipGetErrorString(e));
  g_last_error.clear();
  return run(P, q, k, v, g, beta, cu_seqlens, init_state, out, final_state, ws,
             (hipStream_t)stream);
}

int gdn_decode(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
               const gdn_tensor* g, const gdn_tensor* beta, gdn_tensor* state,
               gdn_tensor* out, const gdn_options* opts, void* stream) {
  gdn::DecodeParams d{};
  bool bf16 = true;
  int dk = 0;
  const int rc = validate_decode(q, k, v, g, beta, state, out, opts, &d, &bf16, &dk);
  if (rc) return rc;
  g_last_error.clear();
  if (d.n == 0) return GDN_OK;
  hipError_t e = gdn::launch_decode(bf16, dk, d, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  if (d.conv_w && opts->conv_state_out) {
    // the step's raw rows shifted into the history, after the step read it
    gdn::ConvStateParams cp{};
    cp.q = q->data; cp.k = k->data; cp.v = v->data;
    cp.q_st = q->stride[0]; cp.q_sh = q->stride[1];
    cp.k_st = k->stride[0]; cp.k_sh = k->stride[1];
    cp.v_st = v->stride[0]; cp.v_sh = v->stride[1];
    cp.state_in = opts->conv_state_in;
    cp.state_out = opts->conv_state_out;
    cp.n_seq = d.n;
    cp.seq_len = 1;
    cp.width = d.conv_width;
    cp.d = d.conv_d;
    cp.hk = d.hk; cp.dk = dk; cp.dv = d.dv;
    if ((e = gdn::launch_conv_state(bf16, cp, (hipStream_t)stream)) != hipSuccess)
      return fail(GDN_ERR_HIP, "convolution state launch: %s", hipGetErrorString(e));
  }
  if (opts && (opts->flags & GDN_FLAG_OUTPUT_GATE)) {
    gdn::GateParams gp{};
    gp.x = out->data;
    gp.z = opts->gate_z;
    gp.out = out->data;
    gp.w = opts->norm_weight;
    gp.rows = (int64_t)d.n * d.hv;
    gp.inner = d.hv;
    gp.x_st = gp.z_st = gp.o_st = out->stride[0];
    gp.x_sh = gp.z_sh = gp.o_sh = out->stride[1];
    gp.eps = opts->norm_eps;
    if ((e = gdn::launch_output_gate(bf16, d.dv, gp, (hipStream_t)stream)) != hipSuccess)
      return fail(GDN_ERR_HIP, "output gate launch: %s", hipGetErrorString(e));
  }
  return GDN_OK;
}

int gdn_check_cu_seqlens(const int32_t* cu_host, int64_t n_seq, int64_t t_total) {
  if (!cu_host) return fail(GDN_ERR_NULL_ARG, "cu_host is NULL");
  if (n_seq < 1 || t_total < 0) return fail(GDN_ERR_SHAPE, "n_seq must be >= 1 and t_total >= 0");
  for (int64_t i = 0; i <= n_seq; ++i) {
    const int32_t f = gdn::cu_entry_faults(cu_host, i, n_seq, t_total);
    if (f) return fail(GDN_ERR_INPUT, "cu_seqlens[%lld] = %d: %s", (long long)i, cu_host[i], cu_fault_text(f));
  }
  g_last_error.clear();
  return GDN_OK;
}

int gdn_output_gate(const gdn_tensor* x, const gdn_tensor* z, const float* weight, float eps,
                    gdn_tensor* out, void* stream) {
  if (!x || !z || !out) return fail(GDN_ERR_NULL_ARG, "x, z and out are required");
  if (x->dtype != GDN_DTYPE_BF16 && x->dtype != GDN_DTYPE_F32) return fail(GDN_ERR_DTYPE, "x must be bf16 or f32");
  if (z->dtype != x->dtype || out->dtype != x->dtype) return fail(GDN_ERR_DTYPE, "x, z and out must share one dtype");
  if (x->ndim != 2 && x->ndim != 3) return fail(GDN_ERR_SHAPE, "x must be [R, dv] or [T, H, dv]");
  if (z->ndim != x->ndim || out->ndim != x->ndim) return fail(GDN_ERR_SHAPE, "x, z and out must have one rank");
  for (int i = 0; i < x->ndim; ++i) {
    if (x->shape[i] < 0) return fail(GDN_ERR_SHAPE, "negative size");
    if (z->shape[i] != x->shape[i] || out->shape[i] != x->shape[i])
      return fail(GDN_ERR_SHAPE, "x, z and out shapes differ");
  }
  const int64_t dv = x->shape[x->ndim - 1];
  if (!supported_head_dim(dv)) return fail(GDN_ERR_UNSUPPORTED, "dv must be 16, 32, 64 or 128");
  if (!(eps >= 0.f)) return fail(GDN_ERR_SHAPE, "eps must be >= 0");
  if ((uintptr_t)weight % 4) return fail(GDN_ERR_LAYOUT, "weight must be 4-byte aligned");
  const bool three = x->ndim == 3;
  const int64_t outer = x->shape[0], inner = three ? x->shape[1] : 1;
  const int64_t rows = outer * inner;
  if (rows == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const int64_t epg = x->dtype == GDN_DTYPE_BF16 ? 8 : 4;
  const gdn_tensor* ts[3] = {x, z, out};
  const char* names[3] = {"x", "z", "out"};
  for (int i = 0; i < 3; ++i) {
    const gdn_tensor* t = ts[i];
    if (!t->data) return fail(GDN_ERR_NULL_ARG, "%s data is NULL", names[i]);
    if ((uintptr_t)t->data % 16) return fail(GDN_ERR_LAYOUT, "%s must be 16-byte aligned", names[i]);
    if (t->stride[t->ndim - 1] != 1) return fail(GDN_ERR_LAYOUT, "%s: last dimension must have unit stride", names[i]);
    for (int d = 0; d + 1 < t->ndim; ++d)
      if (t->stride[d] < 0 || t->stride[d] % epg)
        return fail(GDN_ERR_LAYOUT, "%s: strides must be non-negative multiples of %lld elements", names[i],
                    (long long)epg);
  }
  gdn::GateParams gp{};
  gp.x = x->data;
  gp.z = z->data;
  gp.out = out->data;
  gp.w = weight;
  gp.rows = rows;
  gp.inner = inner;
  gp.x_st = x->stride[0];
  gp.z_st = z->stride[0];
  gp.o_st = out->stride[0];
  gp.x_sh = three ? x->stride[1] : 0;
  gp.z_sh = three ? z->stride[1] : 0;
  gp.o_sh = three ? out->stride[1] : 0;
  gp.eps = eps;
  g_last_error.clear();
  const hipError_t e = gdn::launch_output_gate(x->dtype == GDN_DTYPE_BF16, (int)dv, gp, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "output gate launch: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Captured replays (HIP graphs) of gdn_prefill_ex.

namespace {

// An entry is found by its shape key (everything but the data pointers,
// including which optional pointers are NULL) and its pointer key (the data
// pointers): the launches' grids and kernels depend only on the first.
struct GraphEntry {
  std::string shape_key, ptr_key;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

// Pointer variants of one shape kept side by side before a new variant
// updates the least recently used of them in place.
constexpr int kVariantsPerShape = 4;

void release(GraphEntry& e) {
  if (e.exec) (void)hipGraphExecDestroy(e.exec);
  if (e.graph) (void)hipGraphDestroy(e.graph);
  e.exec = nullptr;
  e.graph = nullptr;
}

void append(std::string& k, const void* p, size_t n) { k.append((const char*)p, n); }

// A tensor's shape-key part (presence, dtype, shape, strides) and its data
// pointer in the pointer key.
void append_tensor(std::string& k, std::string& kp, const gdn_tensor* t) {
  const int32_t none = -1;
  if (!t) {
    append(k, &none, sizeof none);
    return;
  }
  const int32_t null_data = t->data == nullptr;
  append(k, &null_data, sizeof null_data);
  append(kp, &t->data, sizeof t->data);
  append(k, &t->dtype, sizeof t->dtype);
  append(k, &t->ndim, sizeof t->ndim);
  append(k, t->shape, sizeof(int64_t) * (size_t)(t->ndim > 0 && t->ndim <= 4 ? t->ndim : 0));
  append(k, t->stride, sizeof(int64_t) * (size_t)(t->ndim > 0 && t->ndim <= 4 ? t->ndim : 0));
}

}  // namespace

struct gdn_graph_cache {
  std::mutex mu;
  int capacity = 64;
  std::list<GraphEntry> entries;  // most recently used first
  int64_t hits = 0, misses = 0, updates = 0, fallbacks = 0;
};

extern "C" {

int gdn_graph_cache_create(int capacity, gdn_graph_cache** cache) {
  if (!cache) return fail(GDN_ERR_NULL_ARG, "cache pointer is NULL");
  if (capacity < 1 || capacity > 4096) return fail(GDN_ERR_SHAPE, "capacity must be 1..4096");
  gdn_graph_cache* c = new (std::nothrow) gdn_graph_cache;
  if (!c) return fail(GDN_ERR_HIP, "out of host memory");
  c->capacity = capacity;
  *cache = c;
  return GDN_OK;
}

void gdn_graph_cache_destroy(gdn_graph_cache* cache) {
  if (!cache) return;
  for (auto& e : cache->entries) release(e);
  delete cache;
}

void gdn_graph_cache_clear(gdn_graph_cache* cache) {
  if (!cache) return;
  std::lock_guard<std::mutex> lock(cache->mu);
  for (auto& e : cache->entries) release(e);
  cache->entries.clear();
}

int gdn_graph_cache_stats(gdn_graph_cache* cache, int* entries, int64_t* hits,
                          int64_t* misses, int64_t* updates, int64_t* fallbacks) {
  if (!cache) return fail(GDN_ERR_NULL_ARG, "cache is NULL");
  std::lock_guard<std::mutex> lock(cache->mu);
  if (entries) *entries = (int)cache->entries.size();
  if (hits) *hits = cache->hits;
  if (misses) *misses = cache->misses;
  if (updates) *updates = cache->updates;
  if (fallbacks) *fallbacks = cache->fallbacks;
  return GDN_OK;
}

int gdn_prefill_graph(gdn_graph_cache* cache, const gdn_tensor* q, const gdn_tensor* k,
                      const gdn_tensor* v, const gdn_tensor* g, const gdn_tensor* beta,
                      const gdn_tensor* cu_seqlens, const gdn_tensor* init_state,
                      gdn_tensor* out, gdn_tensor* final_state, const gdn_options* opts,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache) return fail(GDN_ERR_NULL_ARG, "cache is NULL");
  Problem P;
  int rc = validate(q, k, v, g, beta, cu_seqlens, init_state, out, final_state, opts, true, &P);
  if (rc) return rc;
  const size_t need = make_layout(P).total;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if ((uintptr_t)workspace % kAlign) return fail(GDN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  g_last_error.clear();
  hipStream_t s = (hipStream_t)stream;

  // The keys: every argument the launches depend on.  The kernels read the
  // sequence lengths from device memory, so a capture stays valid for any
  // lengths with the same shapes and buffers; the buffers themselves enter
  // the launches only as kernel arguments.
  std::string key, kp;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  append(key, &dev, sizeof dev);
  const gdn_tensor* ts[9] = {q, k, v, g, beta, cu_seqlens, init_state, out, final_state};
  for (const gdn_tensor* t : ts) append_tensor(key, kp, t);
  gdn_options o;
  gdn_default_options(&o);
  if (opts) o = *opts;
  // field by field (the struct's padding carries no value); pointers by
  // presence in the shape key and by value in the pointer key
  auto ptr = [&](const void* p) {
    const int32_t present = p != nullptr;
    append(key, &present, sizeof present);
    append(kp, &p, sizeof p);
  };
  append(key, &o.chunk, sizeof o.chunk);
  append(key, &o.scale, sizeof o.scale);
  append(key, &o.l2_eps, sizeof o.l2_eps);
  append(key, &o.stages, sizeof o.stages);
  append(key, &o.scan_split, sizeof o.scan_split);
  append(key, &o.flags, sizeof o.flags);
  ptr(o.decay_a_log);
  ptr(o.decay_bias);
  ptr(o.gate_z);
  ptr(o.norm_weight);
  append(key, &o.norm_eps, sizeof o.norm_eps);
  append(key, &o.segment_chunks, sizeof o.segment_chunks);
  ptr(o.conv_weight);
  append(key, &o.conv_width, sizeof o.conv_width);
  ptr(o.conv_state_in);
  ptr(o.conv_state_out);
  ptr(workspace);
  append(key, &workspace_bytes, sizeof workspace_bytes);

  std::lock_guard<std::mutex> lock(cache->mu);
  auto launch_front = [&]() {
    const hipError_t e = hipGraphLaunch(cache->entries.front().exec, s);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
    return (int)GDN_OK;
  };
  int variants = 0;
  auto oldest = cache->entries.end();
  for (auto it = cache->entries.begin(); it != cache->entries.end(); ++it) {
    if (it->shape_key != key) continue;
    if (it->ptr_key == kp) {
      cache->entries.splice(cache->entries.begin(), cache->entries, it);
      ++cache->hits;
      return launch_front();
    }
    ++variants;
    oldest = it;
  }
  // Record the launches on a private stream (the caller's may be the null
  // stream, which cannot be captured).
  hipGraph_t graph = nullptr;
  hipStream_t cs = nullptr;
  bool ok = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) == hipSuccess;
  if (ok) ok = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) == hipSuccess;
  if (ok) {
    const int rrc = run(P, q, k, v, g, beta, cu_seqlens, init_state, out, final_state, workspace, cs);
    const hipError_t ec = hipStreamEndCapture(cs, &graph);
    ok = rrc == GDN_OK && ec == hipSuccess && graph != nullptr;
  }
  if (cs) (void)hipStreamDestroy(cs);
  if (ok && variants >= kVariantsPerShape) {
    // Same launches on other buffers: update the least recently used
    // variant's executable graph in place (no instantiation).  Launches of
    // it already enqueued keep the arguments they were enqueued with.
    hipGraphNode_t bad = nullptr;
    hipGraphExecUpdateResult res = hipGraphExecUpdateError;
    if (hipGraphExecUpdate(oldest->exec, graph, &bad, &res) == hipSuccess &&
        res == hipGraphExecUpdateSuccess) {
      (void)hipGraphDestroy(oldest->graph);
      oldest->graph = graph;
      oldest->ptr_key = kp;
      cache->entries.splice(cache->entries.begin(), cache->entries, oldest);
      ++cache->updates;
      return launch_front();
    }
    (void)hipGetLastError();
    // refused: the variant is replaced by a new instantiation below
    release(*oldest);
    cache->entries.erase(oldest);
  }
  ++cache->misses;
  GraphEntry ent;
  ent.shape_key = key;
  ent.ptr_key = kp;
  ent.graph = graph;
  if (ok) ok = hipGraphInstantiate(&ent.exec, ent.graph, nullptr, nullptr, 0) == hipSuccess;
  if (!ok) {
    // fall back to the eager launches
    release(ent);
    (void)hipGetLastError();
    ++cache->fallbacks;
    g_last_error.clear();
    return run(P, q, k, v, g, beta, cu_seqlens, init_state, out, final_state, workspace, s);
  }
  cache->entries.push_front(ent);
  while ((int)cache->entries.size() > cache->capacity) {
    release(cache->entries.back());
    cache->entries.pop_back();
  }
  return launch_front();
}

}  // extern "C"
