/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked Gated DeltaNet prefill.
 *
 * The operation.  For every sequence i (tokens cu[i] .. cu[i+1]-1 of a packed
 * batch) and every value head h (reading key head h / (Hv/Hk)), starting from
 * the d_k x d_v state H = init_state[i, h] (or zeros):
 *
 *     q^ = q_t / sqrt(|q_t|^2 + eps),  k^ = k_t / sqrt(|k_t|^2 + eps)
 *     H  = exp(g_t) (I - beta_t k^ k^T) H + beta_t k^ v_t^T
 *     out[t, h] = scale * H^T q^
 *
 * and final_state[i, h] = H after the sequence's last token: the gated
 * delta rule, with the state stored as d_k x d_v.  The serving pages name
 * the operation as the chunked Gated DeltaNet prefill of their native
 * Qwen3.5 backend ("Cua-S1 4B 0.2 native text worker"; "Open-Jev-27B-v1.1
 * native text worker", section "Validation and optimization scope") and
 * test it against float64 references, as this library's tests do; they
 * print no formula, so the recurrence above is the definition this library
 * takes.
 *
 * The library evaluates it chunk by chunk (chunk C in {16, 32, 64}, default
 * 64) on the caller's HIP stream with three kernels: a chunk table, a fused
 * L2-norm / gate-prep / intra-chunk WY kernel, and a fused inter-chunk
 * state-scan / output kernel (two with GDN_SCAN_TWO_LEVEL).
 *
 * Conventions taken from the pages:
 *   - a versioned ABI that callers are rebuilt against ("Cua-S1 4B 0.2
 *     native text worker"; "Open-Jev-27B-v1.1 native text worker", section
 *     "Build and serve");
 *   - invalid or oversize inputs are rejected before any work starts
 *     (same page, section "Prepare the checkpoint");
 *   - vector memory paths only where width, stride and pointers permit
 *     (same page, section "Validation and optimization scope"); here
 *     layouts that do not permit them are rejected with GDN_ERR_LAYOUT.
 *
 * Error behaviour (all entry points): arguments are validated on the host
 * before any HIP call; a failed validation returns a negative status and
 * enqueues nothing.  No exception crosses the ABI.  gdn_last_error() gives a
 * message for the calling thread's last failure.  The contents of
 * cu_seqlens are a precondition (cu[0] = 0, non-decreasing, cu[N] <= T);
 * by default the library does not read device memory on the host, so it
 * does not check them, but the kernels clamp them so that a bad table
 * cannot make them access memory outside the tensors.  gdn_check_cu_seqlens
 * checks a host copy.  With the environment variable GDN_DEBUG_CHECK=1, a
 * packed prefill first checks the device table in a one-workgroup kernel,
 * waits for it (a stream synchronisation) and, if the table is malformed,
 * returns GDN_ERR_INPUT with nothing else enqueued (the pages reject bad
 * input before any work starts: "Open-Jev-27B-v1.1 native text worker",
 * section "Prepare the checkpoint").  The check is skipped while the stream
 * is being captured into a graph (a capture cannot wait).  Faults of
 * enqueued work surface at the caller's next synchronisation of the
 * stream.  Apart from GDN_DEBUG_CHECK, no call synchronises the device.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 9

/* Status codes. */
#define GDN_OK 0
#define GDN_ERR_NULL_ARG (-1)    /* a required tensor or pointer is NULL      */
#define GDN_ERR_DTYPE (-2)       /* unsupported or mismatched element types   */
#define GDN_ERR_SHAPE (-3)       /* inconsistent or out-of-range sizes        */
#define GDN_ERR_LAYOUT (-4)      /* strides / alignment the kernels cannot use */
#define GDN_ERR_UNSUPPORTED (-5) /* valid but not built: head size, chunk ... */
#define GDN_ERR_WORKSPACE (-6)   /* workspace missing, too small or misaligned */
#define GDN_ERR_HIP (-7)         /* a HIP call or kernel launch failed        */
#define GDN_ERR_INPUT (-8)       /* malformed input values (cu_seqlens)       */

/* Element types. */
#define GDN_DTYPE_BF16 1
#define GDN_DTYPE_F32 2
#define GDN_DTYPE_I32 3
#define GDN_DTYPE_I64 4

/* A strided view of caller-owned memory (device memory for every tensor
 * argument).  shape/stride have ndim valid entries, outermost first; strides
 * are in elements.  The library never frees, retains or reallocates it. */
typedef struct gdn_tensor {
  void* data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} gdn_tensor;

/* Stage mask bits for gdn_options.stages.  A full call runs all of them; a
 * caller-owned workspace keeps the intermediates between partial calls so a
 * caller may run (and time) the stages one at a time, in order. */
#define GDN_STAGE_TABLE 1u /* chunk table from cu_seqlens                   */
#define GDN_STAGE_WY 2u    /* L2 norms, gate cumsum, (I+A)^-1, W, U~, Q', O_loc */
#define GDN_STAGE_SCAN 4u  /* sequential state scan fused with the output   */
#define GDN_STAGE_ALL 7u

typedef struct gdn_options {
  int32_t chunk;      /* 16, 32 or 64 (default 64)                          */
  float scale;        /* output multiplier (default 1.0)                     */
  float l2_eps;       /* epsilon inside the L2 norm's square root (1e-6)     */
  uint32_t stages;    /* GDN_STAGE_* mask (default GDN_STAGE_ALL)            */
  int32_t scan_split; /* GDN_SCAN_* (default GDN_SCAN_AUTO)                  */
  uint32_t flags;     /* GDN_FLAG_* (default 0)                              */
  /* GDN_FLAG_DECAY_PROJ: per value head f32 [Hv] device arrays A and bias
   * (NULL reads as zeros; default NULL)                                     */
  const float* decay_a_log;
  const float* decay_bias;
  /* GDN_FLAG_OUTPUT_GATE: the gate projection z, device memory laid out
   * exactly as `out` (same shape, dtype and strides); the weight, f32 [dv]
   * device array (NULL reads as ones); the epsilon inside the root (1e-6) */
  const void* gate_z;
  const float* norm_weight;
  float norm_eps;
  /* Segments (uniform sequences, all stages, one-pass scan; ignored
   * otherwise): the sequences run as consecutive segments of whole chunks,
   * each the WY transform and then the scan from the previous segment's
   * state (carried in f32 in the workspace), so that a segment's
   * intermediates stay in the GPU's 256 MiB memory-side cache between the
   * two launches.  The results are bit-identical to one pass.  0 (default):
   * automatic, when the intermediates of the whole call (W, Q', U~ and
   * O_loc over all sequences and value heads) exceed 128 MiB: segments
   * within 128 MiB each, at least 8 chunks long, the longest whose WY work
   * items (sequences x key heads x chunks) fill whole rounds of the 512
   * WY workgroups an MI355X holds at once, else the fewest of equal
   * length; -1: never; n > 0: segments of n chunks.                      */
  int32_t segment_chunks;
  /* GDN_FLAG_QKV_CONV: the short convolution's taps, an f32 device array
   * [D][conv_width] (channel-major, the last tap multiplies the current
   * token) over D = 2 Hk dk + Hv dv channels in the order q | k | v, each
   * part in its tensor's [H][d] order, 16-byte aligned; its width, 1 .. 4
   * (default 4); the raw rows before each sequence, a contiguous device
   * array [N][conv_width - 1][D] of the input dtype, 16-byte aligned, or
   * NULL for zeros (fresh sequences); and where the last conv_width - 1 raw
   * rows of each sequence go, the same layout, or NULL (not written).
   * conv_state_out may be conv_state_in.  Sizes are not checked: the arrays
   * must hold what these shapes name.                                     */
  const float* conv_weight;
  int32_t conv_width;
  const void* conv_state_in;
  void* conv_state_out;
} gdn_options;

/*
 * GDN_FLAG_BETA_LOGITS: `beta` holds the write gate's raw projection b, and
 * the kernels use beta = sigmoid(b) = 1 / (1 + e^-b), computed in fp32 as the
 * gate is loaded (beta in (0, 1) is a sigmoid of a projection), so
 * no separate activation pass over [T, Hv] runs before the prefill or the
 * decode step.  b = +-inf give beta = 1 / 0.
 */
#define GDN_FLAG_BETA_LOGITS 1u

/*
 * The gates on either side of the prefill.  The serving pages run "fused
 * norm, activation" operations around the chunked Gated DeltaNet and keep
 * the bf16 rounding points of the unfused sequence when they fuse a gate
 * into an epilogue ("Open-Jev-27B-v1.1 native text worker", section
 * "Validation and optimization scope"); they print no formula for either,
 * so the two below are this library's reading.
 *
 * GDN_FLAG_DECAY_PROJ: `g` holds the decay gate's raw projection a, and the
 * kernels take
 *     g = -exp(A[h]) * softplus(a + bias[h]),   softplus(x) = log(1 + e^x)
 * in fp32 as they load it (A = decay_a_log, bias = decay_bias, per value
 * head), so every g is <= 0 for any a and no activation pass over [T, Hv]
 * runs first.  (A = bias = 0 with -a in place of a gives log sigmoid(a).)
 *
 * GDN_FLAG_OUTPUT_GATE: after the outputs are stored (rounded to the output
 * type, as an unfused norm would read them), each (token, value head) row o
 * of d_v outputs is replaced, in one pass, by
 *     y = o / sqrt(mean(o^2) + norm_eps) * w * silu(z),  silu(z) = z / (1 + e^-z)
 * computed in fp32 from the stored o and rounded once.  The norm spans the
 * whole row, which the state scan writes in 16-column slices from separate
 * workgroups, so it runs as its own bandwidth-bound kernel at the end of the
 * call (the same kernel as gdn_output_gate).  z is read with out's strides.
 */
#define GDN_FLAG_DECAY_PROJ 2u
#define GDN_FLAG_OUTPUT_GATE 4u

/*
 * GDN_FLAG_QKV_SILU: q, k and v hold the values before the activation that
 * precedes the layer, and the kernels (prefill and decode) take
 *     silu(x) = x / (1 + e^-x)
 * elementwise in fp32 as they load them, each result rounded to the input
 * dtype as a separate activation pass would store it (so the L2 norms of q
 * and k are taken of the activated rows).  The same reading as the gates
 * above: the pages run "fused norm, activation" operations around the
 * chunked Gated DeltaNet and name SiLU as the activation they check
 * ("Open-Jev-27B-v1.1 native text worker", section "Validation and
 * optimization scope").  Alone it applies no convolution (see
 * GDN_FLAG_QKV_CONV).  In the prefill the WY kernel writes the activated key rows to the workspace
 * (the `k_act` region, laid out as a contiguous [T][Hk][dk] tensor of the
 * input dtype) for the scan.
 */
#define GDN_FLAG_QKV_SILU 8u

/*
 * GDN_FLAG_QKV_CONV: before the activation, every channel c of q, k and v
 * passes through a causal depthwise convolution of width W = conv_width
 * along the tokens of its own sequence:
 *     y[t, c] = sum_{j=0}^{W-1} conv_weight[c][j] * e[t + j, c],
 * e being the sequence's W - 1 history rows (conv_state_in, or zeros)
 * followed by its raw rows.  y then goes through silu when
 * GDN_FLAG_QKV_SILU is also set, and is rounded once to the input dtype;
 * the L2 norms of q and k are taken of the result.  Computed in fp32 as the
 * rows are loaded: the WY kernel reads W - 1 rows before each chunk (from
 * the inputs, or from conv_state_in at a sequence's first chunk) and writes
 * the chunk's key rows as used to the `k_act` workspace region for the
 * scan.  With conv_state_out the last W - 1 raw rows of each sequence (the
 * history a later call continues from; fewer rows than that shift in the
 * tail of conv_state_in) are written after the WY stage.  The decode step
 * does the same per token and shifts its row into conv_state_out.
 * Reading: the pages name "fused norm, activation" operations around the
 * chunked Gated DeltaNet ("Open-Jev-27B-v1.1 native text worker", section
 * "Validation and optimization scope") and name no convolution; this is the
 * short convolution a Gated DeltaNet layer runs on its q, k, v projections
 * before the SiLU, for callers that fuse it here.
 */
#define GDN_FLAG_QKV_CONV 16u

/*
 * The state scan's schedule.  Each chunk maps its incoming state affinely
 * (the recurrence above summed over a chunk): H' = M H + B with
 * M = e^{gamma_last} I - K~^T W and B = K~^T U~.
 * GDN_SCAN_TWO_LEVEL splits every sequence (at about 17/32 of its chunks) and scans
 * both halves at once: the second from zero, beside the product of its M
 * (d_k more state columns), then adds M-product x (state at the split) to
 * its outputs and final state.  The chain of dependent chunk steps shortens
 * to about 17/32 of the chunks; the arithmetic differs from the one-pass scan only
 * in rounding.  Offered
 * for bf16 inputs without cu_seqlens (uniform sequences), d_k and d_v
 * multiples of 32 and chunks of 32 or 64; GDN_SCAN_TWO_LEVEL elsewhere is
 * GDN_ERR_UNSUPPORTED.  GDN_SCAN_AUTO is the one-pass scan (on MI355X the
 * two-level scan's two launches take longer at the sizes measured).
 */
#define GDN_SCAN_AUTO 0
#define GDN_SCAN_ONE_PASS 1
#define GDN_SCAN_TWO_LEVEL 2

/* Returns GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

/* Fills *opts with the defaults listed in gdn_options. */
void gdn_default_options(gdn_options* opts);

/*
 * gdn_prefill -- the whole prefill on `stream` (a hipStream_t; NULL = the
 * null stream), with default options and a workspace the library allocates
 * and frees stream-ordered (hipMallocAsync / hipFreeAsync on `stream`).
 *
 *   q, k        [T, Hk, dk] or [B, T/B, Hk, dk]; bf16 or f32
 *   v, out      [T, Hv, dv] (or 4-D like q); same dtype as q
 *   g, beta     [T, Hv] (or [B, T/B, Hv]) f32: g is the log-decay (<= 0,
 *               alpha = exp(g)), beta the write strength in [0, 1] (already
 *               passed through the sigmoid).  These ranges are
 *               preconditions, not checked (see GDN_FLAG_DECAY_PROJ and
 *               GDN_FLAG_BETA_LOGITS for raw projections).
 *   cu_seqlens  int32 or int64 [N+1] device array of sequence starts
 *               (entries below 2^31), or NULL: one
 *               sequence of T tokens (3-D inputs) or B sequences of T/B
 *               tokens each (4-D inputs).  With cu_seqlens, 4-D inputs need
 *               B == 1, and the bounds are read from it also for N = 1:
 *               rows at or after cu[N] are not written.
 *   init_state  f32 [N, Hv, dk, dv] contiguous, or NULL for zeros
 *   final_state f32 [N, Hv, dk, dv] contiguous, or NULL (not written); it
 *               may be the same memory as init_state.
 * Sizes: dk, dv in {16, 32, 64, 128}; Hv a multiple of Hk; N, T < 2^31.
 * Layout: unit stride in the last dimension; other strides multiples of 8
 * elements (bf16) or 4 (f32); 16-byte aligned data pointers; for 4-D
 * tensors stride[0] == shape[1] * stride[1].  Otherwise GDN_ERR_LAYOUT.
 * All tensors are caller-owned device memory that must stay valid until
 * the stream reaches the end of the enqueued work.  Returns a GDN_* status.
 */
int gdn_prefill(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
                const gdn_tensor* g, const gdn_tensor* beta,
                const gdn_tensor* cu_seqlens, const gdn_tensor* init_state,
                gdn_tensor* out, gdn_tensor* final_state, void* stream);

/*
 * gdn_prefill_ex -- as gdn_prefill, with options (NULL = defaults) and a
 * caller-owned device workspace of at least gdn_workspace_size() bytes,
 * 256-byte aligned.  It allocates nothing.  The workspace must not be used
 * by another call that overlaps on the device.
 */
int gdn_prefill_ex(const gdn_tensor* q, const gdn_tensor* k,
                   const gdn_tensor* v, const gdn_tensor* g,
                   const gdn_tensor* beta, const gdn_tensor* cu_seqlens,
                   const gdn_tensor* init_state, gdn_tensor* out,
                   gdn_tensor* final_state, const gdn_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_noalloc -- gdn_prefill_ex without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Its workspace is a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES held by the library on every GPU it runs on
 * until the process ends (looked up on the first call on each device).  The
 * caller still passes every input and output; `opts` may be NULL.  Sizes
 * whose workspace (gdn_workspace_size) exceeds the scratch are rejected with
 * GDN_ERR_WORKSPACE before anything is enqueued (96 MiB covers, e.g., 4096
 * tokens x 16 heads at d = 128 in bf16, which needs 64 MiB).  No part of the
 * scratch has to start at zero: each call writes everything it reads.  All
 * calls on one GPU share its scratch, which keeps the last call's contents:
 * calls that overlap on one GPU (different streams or threads) race, and
 * must be serialised by the caller.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int gdn_prefill_noalloc(const gdn_tensor* q, const gdn_tensor* k,
                        const gdn_tensor* v, const gdn_tensor* g,
                        const gdn_tensor* beta, const gdn_tensor* cu_seqlens,
                        const gdn_tensor* init_state, gdn_tensor* out,
                        gdn_tensor* final_state, const gdn_options* opts,
                        void* stream);

/* Byte offsets of the intermediates inside the workspace (for inspection and
 * tests).  Per (chunk c, value head h) block, all in the input dtype:
 *   w     diag(s) W,  W = T diag(beta e^gamma) K^     C x dk, k-tile order
 *   qp    Q' = scale diag(e^gamma) Q^ - P W             C x dk, k-tile order
 *   ut    diag(s) U~, U~ = T diag(beta) V              C x dv, accumulator tiles
 *   oloc  O_loc = P U~                                  C x dv, transposed tiles
 * with the row scale s_r = e^(gamma_last - gamma_r) / sqrt(|k_r|^2 + eps)
 * (k_r the key row as passed), and f32 decay[c][h] = e^(gamma_last).  With
 * U' = diag(s) U~ - diag(s) W H the state update is H' = e^(gamma_last) H +
 * K^T U' with K the chunk's key rows as passed, equal to K~^T U for
 * K~_r = e^(gamma_last - gamma_r) k^_r.  A block starts at
 * offset + (c * Hv + h) * (its element count) * element_size.
 * "k-tile order": 16-row tiles one after another; inside a tile, for the
 * 16-wide k-tile t of the second index, lane l = m + 16 ((k % 16) / 4)
 * holds the 4 elements k % 4 = 0..3.  bf16 pairs k-tiles 2u and 2u+1 into
 * one unit of 8 elements per lane (4 of k-tile 2u, then 4 of 2u+1; a
 * trailing single k-tile has 4); f32 has one k-tile (4 elements) per unit.
 * Units follow each other, lanes in order inside a unit.
 * "Accumulator tiles": 16 x 16 tiles, column-tile major (tile (ct, rt) at
 * ct * C/16 + rt), of 64 lanes x 4, lane l holding rows 4 (l / 16) .. +3 of
 * column l % 16; "transposed tiles" hold the same tiles with lane l holding
 * columns 4 (l / 16) .. +3 of row l % 16.  Rows past the end of a short
 * chunk are zero.  chunk_table is int32 [max_chunks][4] = (sequence, first
 * token, length, 0) in packed mode. */
typedef struct gdn_workspace_layout {
  size_t total_bytes;
  int64_t max_chunks;
  size_t chunk_table, chunk_offsets, seq_starts, decay, w, qp, ut, oloc;
  /* two-level scan (split_chunks > 0: chunks in the first segment), else 0:
   *   split_y      bf16 [chunk][Hv][C][dk]  Q' x M-product, second segment
   *   split_hmid   f32 [N][Hv][dk][dv]      state at the split
   *   split_hmid_t bf16 [N][Hv][dv][dk]     its transpose
   *   split_psi    f32 [N][Hv][dk][dv]      second segment's end from zero
   *   split_phi    f32 [N][Hv][dk][dk]      second segment's M-product   */
  int32_t split_chunks;
  size_t split_y, split_hmid, split_hmid_t, split_psi, split_phi;
  /* segments (gdn_options.segment_chunks): chunks per segment, 0 for one
   * pass, and the state carried between segments, f32 [N][Hv][dk][dv]    */
  int32_t segment_chunks;
  size_t segment_state;
  /* GDN_FLAG_QKV_SILU or GDN_FLAG_QKV_CONV: the key rows as the
   * recurrence uses them (activated, convolved), a contiguous [T][Hk][dk]
   * tensor of the input dtype (0 without either flag)                    */
  size_t k_act;
} gdn_workspace_layout;

/* Computes the workspace size / layout for the given tensors and options
 * (host only; data pointers are not read). */
int gdn_workspace_size(const gdn_tensor* q, const gdn_tensor* k,
                       const gdn_tensor* v, const gdn_tensor* cu_seqlens,
                       const gdn_options* opts, size_t* bytes);
int gdn_get_workspace_layout(const gdn_tensor* q, const gdn_tensor* k,
                             const gdn_tensor* v, const gdn_tensor* cu_seqlens,
                             const gdn_options* opts,
                             gdn_workspace_layout* layout);

/*
 * gdn_decode -- one recurrent step per sequence: the single-token form of
 * the same gated delta rule, as a
 * generator runs it after the prefill, on the state the prefill returned.
 * For every sequence i and value head h (key head h / (Hv/Hk)):
 *     H = state[i, h];  H <- exp(g) (I - beta k^ k^T) H + beta k^ v^T;
 *     out[i, h] = scale * H^T q^;  state[i, h] = H (in place)
 * with q^, k^ L2-normalised as in gdn_prefill.  Computed in fp32.
 *   q, k     [N, Hk, dk]; v, out [N, Hv, dv]; one dtype, bf16 or f32; unit
 *            stride in the last dimension
 *   g, beta  [N, Hv] f32 (same preconditions as gdn_prefill)
 *   state    f32 [N, Hv, dk, dv] contiguous and 16-byte aligned, read and
 *            written in place; v and out rows start on 4-element
 *            boundaries (address and strides)
 *   opts     NULL or options; scale, l2_eps, flags and the gate fields are
 *            used (with GDN_FLAG_OUTPUT_GATE, gate_z is laid out as out;
 *            with GDN_FLAG_QKV_CONV the convolution fields, N sequences of
 *            one token each: the history is read from conv_state_in and
 *            the step's raw row shifted into conv_state_out, which may be
 *            conv_state_in)
 * dk, dv in {16, 32, 64, 128}.  N = 0 enqueues nothing.  Allocates nothing.
 * Returns a GDN_* status; validation errors enqueue nothing.
 */
int gdn_decode(const gdn_tensor* q, const gdn_tensor* k, const gdn_tensor* v,
               const gdn_tensor* g, const gdn_tensor* beta, gdn_tensor* state,
               gdn_tensor* out, const gdn_options* opts, void* stream);

/*
 * Captured replays.  gdn_prefill_graph behaves as gdn_prefill_ex, but keeps
 * a HIP graph of the launches in `cache`.  A graph is found by every
 * argument the launches depend on: device, tensor descriptors (which
 * optional tensors and options pointers are NULL, dtypes, shapes, strides),
 * option values and workspace size (the shape key), and the data, options
 * and workspace pointers (the pointer key).  A hit (both keys stored) only
 * launches the stored graph, which removes the per-kernel launch cost.
 * Otherwise the launches are recorded on a private stream (stream capture):
 * while fewer than 4 graphs of the same shape key are stored, the recording
 * is instantiated as a new graph (a miss); from then on the least recently
 * used graph of that shape key is updated in place to the new pointers
 * (hipGraphExecUpdate: an update, no instantiation; launches of it already
 * enqueued keep their arguments), or replaced by a new instantiation if the
 * update is refused.  If capture or instantiation fails the call runs the
 * launches eagerly (and counts a fallback).  The sequence lengths are read from cu_seqlens on the device by
 * the kernels themselves, so one capture stays valid for any lengths with
 * the same shapes and buffers (the serving pages key their captures by the
 * length tuple: "Cua-S1 4B 0.2 native text worker"; "Open-Jev-27B-v1.1
 * native text worker", section "Build and serve").  The cache holds at most
 * `capacity` graphs and drops the least recently used.  Buffers named by a
 * stored graph must stay allocated while it may be replayed: call
 * gdn_graph_cache_clear after freeing or growing any of them.  A cache may be
 * shared by threads (calls are serialised); entries of one cache must not be
 * replayed on overlapping streams with the same workspace.
 */
typedef struct gdn_graph_cache gdn_graph_cache;

int gdn_graph_cache_create(int capacity, gdn_graph_cache** cache);
void gdn_graph_cache_destroy(gdn_graph_cache* cache);
void gdn_graph_cache_clear(gdn_graph_cache* cache);
int gdn_graph_cache_stats(gdn_graph_cache* cache, int* entries, int64_t* hits,
                          int64_t* misses, int64_t* updates, int64_t* fallbacks);
int gdn_prefill_graph(gdn_graph_cache* cache, const gdn_tensor* q,
                      const gdn_tensor* k, const gdn_tensor* v,
                      const gdn_tensor* g, const gdn_tensor* beta,
                      const gdn_tensor* cu_seqlens, const gdn_tensor* init_state,
                      gdn_tensor* out, gdn_tensor* final_state,
                      const gdn_options* opts, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * gdn_output_gate -- the gated output norm of GDN_FLAG_OUTPUT_GATE on its
 * own, for outputs already in memory:
 *     out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w * silu(z[r])
 * for every row r of d_v elements, computed in fp32, rounded once.
 *   x, z, out  [R, dv] or [T, H, dv]; one dtype, bf16 or f32; unit stride
 *              in the last dimension; other strides multiples of 8 (bf16)
 *              or 4 (f32) elements; 16-byte aligned data.  out may be x
 *              (in place).
 *   weight     f32 [dv] device array (4-byte aligned), or NULL for ones
 *   eps        >= 0
 * dv in {16, 32, 64, 128}.  No rows enqueues nothing.  Allocates nothing.
 * The reading and its citation are at GDN_FLAG_OUTPUT_GATE.  Returns a
 * GDN_* status; validation errors enqueue nothing.
 */
int gdn_output_gate(const gdn_tensor* x, const gdn_tensor* z, const float* weight,
                    float eps, gdn_tensor* out, void* stream);

/*
 * gdn_check_cu_seqlens -- checks a host copy of a cu_seqlens table of
 * n_seq + 1 entries for t_total tokens against the preconditions above
 * (cu[0] = 0, non-decreasing, cu[n_seq] <= t_total) with the predicate the
 * GDN_DEBUG_CHECK device check uses.  cu_host is host memory.  Returns
 * GDN_OK, GDN_ERR_INPUT (the message names the first bad entry), or
 * GDN_ERR_NULL_ARG / GDN_ERR_SHAPE for a NULL table or n_seq < 1.
 */
int gdn_check_cu_seqlens(const int32_t* cu_host, int64_t n_seq, int64_t t_total);

/* Short description of a status code (static storage). */
const char* gdn_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
