/*
 * libgdn: packed (varlen) gated-delta-rule prefill with prefix-cache
 * checkpoints, a one-token decode step, the short convolution ahead of them
 * and a checkpoint copy on its own stream, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes
 *   Per prompt s and value head h (qk head j = h / (Hv / Hqk)), starting from
 *   S = init_state[s, h] (zeros when init_state is NULL), for every token t
 *   of the prompt in order, with alpha_t = exp(g_t):
 *       S   <- alpha_t * S (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T
 *       o_t  = scale * S q^_t
 *   S is head_v_dim x head_k_dim.  k^ and q^ are k and q divided by
 *   sqrt(sum x^2 + l2_eps) when GDN_QK_L2NORM is set.  This is the gated
 *   delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks", ICLR 2025).
 *
 *   Several prompts share one packed pass and each keeps its own state, so a
 *   prompt's outputs, checkpoints and final state are bit-identical whether it
 *   runs alone or packed (sparkinfer release v0.6.28: packed prompt passes;
 *   "Measured": checkpoints identical alone or packed).
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major with the innermost dimension contiguous.  Device
 *     pointers are HIP device memory (or, where stated, device-mapped pinned
 *     host memory).  The caller owns every buffer; no call allocates memory.
 *   - All arguments are validated on the host before anything is enqueued.
 *     A call that returns an error has enqueued no work (GDN_ERR_HIP: the
 *     library synchronised the stream it used before returning, so nothing it
 *     launched is still in flight).
 *   - Work is asynchronous on the given stream (a hipStream_t passed as
 *     void*; NULL = the null stream).  The library keeps no global mutable
 *     state and shares no scratch memory between calls or streams.
 *   - Each (prompt, head)'s arithmetic depends only on that prompt's own
 *     inputs, initial state and checkpoint positions: never on the grid, the
 *     other prompts of the pack or their order (the launch grid itself does
 *     depend on the number of prompts).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  GDN_ERR_SHAPE = 2,       /* negative count, bad stride or inconsistent sizes            */
  GDN_ERR_UNSUPPORTED = 3, /* head dims, chunk, dtype, flags or head ratio not built      */
  GDN_ERR_SEQLENS = 4,     /* cu_seqlens not 0-based, non-decreasing, ending at n_tokens  */
  GDN_ERR_CKPT = 5,        /* checkpoints not strictly increasing, or outside every prompt */
  GDN_ERR_CAPACITY = 6,    /* an output list is too short, or a slot outside the pool      */
  GDN_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed                  */
} gdn_status;

typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* shape.flags */
#define GDN_QK_L2NORM 1u

/* Layer geometry and numeric options, passed by pointer to every call.
 *   num_qk_heads, num_v_heads: Hqk and Hv, Hv a multiple of Hqk.
 *   head_k_dim, head_v_dim:    dk and dv, each one of 32, 64, 128.
 *   chunk:                     the most tokens one chunk of the chunked scan
 *                              holds, one of 16, 32, 64.  The scans run chunks
 *                              of min(chunk, 32) tokens from each prompt's first
 *                              token (a 64-token chunk's end state is the same
 *                              quantity as two 32-token chunks'), and a chunk
 *                              also ends at every checkpoint.
 *   io_dtype:                  gdn_dtype of q, k, v, out, x, y, conv states.
 *   flags:                     GDN_QK_L2NORM or 0.
 *   scale:                     factor on the outputs (1.0 for none).
 *   l2_eps:                    added to sum x^2 before the square root.
 *   q/k/v_tok_stride:          elements between consecutive tokens of q, k, v
 *                              (0 = dense: Hqk*dk, Hqk*dk, Hv*dv), so q, k and
 *                              v may be column views of one [T, conv_dim] row;
 *                              every token stride (given or dense, also x/y
 *                              of the conv) is below 2^23 elements. */
typedef struct gdn_shape {
  int32_t num_qk_heads;
  int32_t num_v_heads;
  int32_t head_k_dim;
  int32_t head_v_dim;
  int32_t chunk;
  int32_t io_dtype;
  uint32_t flags;
  float scale;
  float l2_eps;
  int32_t reserved;
  int64_t q_tok_stride;
  int64_t k_tok_stride;
  int64_t v_tok_stride;
} gdn_shape;

/* Human-readable name of a status code (static string, never NULL). */
GDN_API const char* gdn_status_string(int32_t status);

/* Checkpoint planner (host only, no HIP call).
 * Source: sparkinfer release v0.6.28, the bullet on checkpoints that fall in
 * a prompt's last 16 tokens moving back one block so the prompt stays in the
 * pack.  For prompt s (length L = cu[s+1]-cu[s], absolute first position
 * p0[s], 0 when p0_host is NULL) every multiple c of `block` with
 * p0 < c <= p0 + L is taken; if p0 + L - c < tail it moves back to c - block;
 * it is kept when still > p0 and not already taken.  Writes the global pack
 * offsets cu[s] + (c - p0), ascending, to out_pos[0 .. *n_out).
 *   cu_host:   host int32 [n_seqs + 1], validated like gdn_prefill_packed's.
 *   block:     >= 1.  tail: >= 0 (16 on the page).
 *   out_pos:   host int32 [cap]; may be NULL when cap == 0 (count only).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE (n_seqs < 0, block < 1, tail < 0,
 * p0 < 0), GDN_ERR_SEQLENS, GDN_ERR_CAPACITY (more than cap positions;
 * *n_out still receives the full count). */
GDN_API gdn_status gdn_plan_checkpoints(const int32_t* cu_host, int32_t n_seqs, const int32_t* p0_host,
                                int32_t block, int32_t tail, int32_t* out_pos, int32_t cap,
                                int32_t* n_out);

/* Width-4 causal depthwise conv + SiLU over a pack, never reading across a
 * prompt boundary (the short convolution ahead of q, k, v in Gated Delta
 * Networks' block design).  For channel c and token p of prompt s:
 *     y[p, c] = silu( sum_{j=0..3} w[c, j] * xs[p - 3 + j, c] )
 * where xs is the prompt's own inputs and, before its first token, its conv
 * state (zeros when conv_state_in is NULL).
 *   conv_dim = 2*Hqk*dk + Hv*dv, channels ordered [q | k | v].
 *   cu_seqlens / cu_seqlens_host: device / host int32 [n_seqs + 1].
 *   x, y:            device [n_tokens, conv_dim] io_dtype, token strides in
 *                    elements (0 = conv_dim); y must not overlap x.
 *   weight:          device fp32 [conv_dim, 4], tap 3 on the current token.
 *   conv_state_in:   device io_dtype [n_seqs, 3, conv_dim] oldest first, or NULL.
 *   conv_state_out:  device io_dtype [n_seqs, 3, conv_dim] or NULL: each
 *                    prompt's last three inputs (reaching into its history
 *                    when shorter than 3).  May equal conv_state_in.
 *   ckpt_positions(_host), n_ckpt: as in gdn_prefill_packed; when conv_ckpt
 *                    is non-NULL it receives, per checkpoint, the three
 *                    inputs before it: io_dtype [n_ckpt, 3, conv_dim].
 * Errors: as gdn_prefill_packed. */
GDN_API gdn_status gdn_conv1d_silu_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t n_seqs,
                                  int32_t n_tokens, const void* x, int64_t x_tok_stride,
                                  const float* weight, const void* conv_state_in, void* y,
                                  int64_t y_tok_stride, void* conv_state_out,
                                  const int32_t* ckpt_positions,
                                  const int32_t* ckpt_positions_host, int32_t n_ckpt,
                                  void* conv_ckpt, void* stream);

/* Packed prefill: the chunked gated-delta-rule scan over every prompt of a
 * pack, writing outputs, the state at each checkpoint and each prompt's
 * final state (sparkinfer release v0.6.28: packed passes and prefix-cache
 * checkpoints of the linear-attention state).
 *   cu_seqlens:       device int32 [n_seqs + 1]; cu_seqlens_host its host
 *                     mirror (validated: cu[0] = 0, non-decreasing,
 *                     cu[n_seqs] = n_tokens).  Empty prompts are allowed
 *                     (their final state is their initial state).
 *   q, k:             device io_dtype [n_tokens, Hqk, dk] (token stride from
 *                     shape); v: [n_tokens, Hv, dv].
 *   g, beta:          device fp32 [n_tokens, Hv]: log-gate (alpha = exp g)
 *                     and write strength.
 *   init_state:       device fp32 [n_seqs, Hv, dv, dk] or NULL (zeros).
 *   ckpt_positions:   device int32 [n_ckpt] global pack offsets, strictly
 *                     increasing; ckpt_positions_host its host mirror.  A
 *                     position p belongs to the prompt with cu[s] < p <=
 *                     cu[s+1]; the checkpoint is the state after the
 *                     prompt's first p - cu[s] tokens.  Any such position
 *                     works: the scan ends a chunk there and starts the
 *                     next one at p, so a prompt resumed from a checkpoint
 *                     (init_state = that checkpoint, the prompt's later
 *                     tokens, the later checkpoints) gives the unbroken run's
 *                     outputs, checkpoints and final state bit for bit.
 *                     gdn_plan_checkpoints makes such lists, also for
 *                     prompts resumed at an absolute position p0.
 *   out:              device io_dtype [n_tokens, Hv, dv] (dense).
 *   final_state:      device fp32 [n_seqs, Hv, dv, dk] or NULL (not written).
 *   ckpt_buf:         device fp32 [n_ckpt, Hv, dv, dk]; may be NULL iff n_ckpt = 0.
 * Arithmetic: states are carried and accumulated in fp32.  With bf16 io the
 * scan's products run on fp16 matrix-core operands: q/k rows convert to fp16
 * exactly while their sum of squares lies in [2^-4, 2^20], other rows are
 * scaled by a power of two first (the factor folded into the row's norm);
 * the state is held per 32 state columns as 2^E S, E chosen per chunk from
 * the largest |S| entry and the chunk's largest |v| (0 while both lie in
 * [2^-6, 2^7)); the fp32 values entering a product (state, T, P, Y, U) are
 * rounded to fp16 once.  This holds states to about 4e-4 relative Frobenius
 * against exact arithmetic at any input scale inside fp32's range, as long
 * as the |v| rows of one 32-token chunk lie within about 2^14 of each other
 * (rows far below the chunk's largest reach fp16's subnormal range).  With
 * fp32 io a token-recurrent fp32 kernel runs instead.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS,
 * GDN_ERR_CKPT, GDN_ERR_HIP.  init_state may alias final_state. */
GDN_API gdn_status gdn_prefill_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t n_tokens,
                              const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* init_state,
                              const int32_t* ckpt_positions, const int32_t* ckpt_positions_host,
                              int32_t n_ckpt, void* out, float* final_state, float* ckpt_buf,
                              void* stream);

/* Packed prefill with the short convolution fused into the scan's loads:
 * the scan reads the pre-conv rows x and applies the width-4 causal conv +
 * SiLU to q, k and v itself, so the conv output never goes through HBM (the
 * in_proj -> GDN path is bandwidth-bound: vllm.cpp docs, "vLLM, online
 * serving", ModelOpt table, the "Lever 2, GDN fp8 in_proj" row).  Results
 * equal gdn_conv1d_silu_packed (x -> y, with the same conv states,
 * checkpoints and windows) followed by gdn_prefill_packed on the column
 * views q = y[:, :Hqk*dk], k = y[:, Hqk*dk:2*Hqk*dk], v = y[:, 2*Hqk*dk:],
 * bit for bit: the conv runs in conv1d_silu's operation order and its bf16
 * outputs are converted for the products exactly as loaded ones are.
 * Performance: the conv's arithmetic runs on the workgroups of the scan, one
 * per (prompt, value head).  On MI355X this is the faster path when those
 * fill the 256 CUs several times over (32 x 1,024 tokens, 32 value heads:
 * 13% below the two launches); with fewer (prompt, head) pairs than CUs
 * (4 prompts x 32 heads) the two launches are faster, since the separate
 * conv uses the whole chip.
 *   shape:           bf16 io, dk = dv = 128, chunk 32 or 64 (the scan's
 *                    32-token tiles); other shapes: GDN_ERR_UNSUPPORTED.
 *                    q/k/v_tok_stride are not used.
 *   x:               device bf16 [n_tokens, conv_dim], conv_dim = 2*Hqk*dk +
 *                    Hv*dv, channels [q | k | v], token stride x_tok_stride
 *                    in elements (0 = conv_dim).
 *   conv_weight:     device fp32 [conv_dim, 4], tap 3 on the current token.
 *   conv_state_in:   device bf16 [n_seqs, 3, conv_dim] (oldest first) or
 *                    NULL (zeros).
 *   conv_state_out:  device bf16 [n_seqs, 3, conv_dim] or NULL: each
 *                    prompt's last three inputs.  May equal conv_state_in
 *                    (the windows are then written by a second launch after
 *                    the scan); must not overlap it otherwise.
 *   conv_ckpt:       device bf16 [n_ckpt, 3, conv_dim] or NULL: the three
 *                    inputs before each checkpoint.
 *   the rest:        as gdn_prefill_packed.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE (also when out overlaps x),
 * GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS, GDN_ERR_CKPT, GDN_ERR_HIP. */
GDN_API gdn_status gdn_prefill_conv_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t n_seqs,
                                   int32_t n_tokens, const void* x, int64_t x_tok_stride,
                                   const float* conv_weight, const void* conv_state_in,
                                   void* conv_state_out, const float* g, const float* beta,
                                   const float* init_state, const int32_t* ckpt_positions,
                                   const int32_t* ckpt_positions_host, int32_t n_ckpt,
                                   void* conv_ckpt, void* out, float* final_state,
                                   float* ckpt_buf, void* stream);

/* One recurrent step for each of `batch` decoding sequences, in place on a
 * state pool (one forward pass carries decodes beside a packed prefill:
 * sparkinfer release v0.6.4, "What changed"; packed GDN decode: vllm.cpp
 * docs, "vLLM, online serving", lever 2b).
 *   q, k:       device io_dtype [batch, Hqk, dk] (token stride from shape);
 *   v:          [batch, Hv, dv];  g, beta: device fp32 [batch, Hv].
 *   state:      device fp32 [pool_slots, Hv, dv, dk], updated in place.
 *   slot:       device int32 [batch] pool rows, or NULL for rows 0..batch-1;
 *               slot_host its host mirror (required with slot): every entry
 *               in [0, pool_slots) and all distinct.
 *   out:        device io_dtype [batch, Hv, dv].
 *   conv_w:     device fp32 [conv_dim, 4] or NULL; conv_state: device io_dtype
 *               [pool_slots, 3, conv_dim] or NULL (both or neither;
 *               conv_dim = 2*Hqk*dk + Hv*dv, channels [q | k | v]).  With
 *               them, q, k and v are the inputs of the short convolution
 *               (gdn_conv1d_silu_packed's x): each channel's value is the
 *               width-4 conv + SiLU over its last three inputs (the slot's
 *               conv_state, oldest first) and the current one, rounded to
 *               io_dtype as a stored conv output is, in the same operation
 *               order, so the results equal gdn_conv1d_silu_packed followed
 *               by this call without the conv, bit for bit.  The slot's
 *               conv_state then holds its last three inputs.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_CAPACITY
 * (slot outside the pool, repeated, or batch > pool_slots without slots),
 * GDN_ERR_HIP. */
GDN_API gdn_status gdn_decode_step(const gdn_shape* shape, int32_t batch, const void* q, const void* k,
                           const void* v, const float* g, const float* beta, float* state,
                           int64_t pool_slots, const int32_t* slot, const int32_t* slot_host,
                           void* out, const float* conv_w, void* conv_state, void* stream);

/* n_tok recurrent steps for each of `batch` decoding sequences, in place on
 * the state pool, keeping the state after every token: the verification pass
 * of speculative or multi-token-prediction decoding, where a rejected suffix
 * is rolled back by restoring a kept state (vllm-ascend tutorial,
 * Qwen3.6-35B-A3B, section 9.3 "Model-Specific Optimizations": MTP
 * speculative decoding).  gdn_decode_step is the n_tok = 1 case.
 *   n_tok:      tokens per sequence, >= 1.
 *   q, k:       device io_dtype [batch * n_tok, Hqk, dk], sequence-major (row
 *               b * n_tok + i is token i of sequence b; token stride from
 *               shape);  v: [batch * n_tok, Hv, dv];
 *   g, beta:    device fp32 [batch * n_tok, Hv].
 *   state:      device fp32 [pool_slots, Hv, dv, dk]; the addressed rows end
 *               at the state after the sequence's last token.
 *   slot, slot_host, pool_slots: as in gdn_decode_step.
 *   out:        device io_dtype [batch * n_tok, Hv, dv].
 *   snapshots:  device fp32 [batch, n_tok, Hv, dv, dk] (entry i: the state
 *               after token i of the sequence), or NULL.
 *   conv_w, conv_state: as in gdn_decode_step; token i's window reaches back
 *               into the sequence's earlier tokens of this call, then into
 *               the slot's conv state, which ends at the last three inputs.
 *               (A rollback restores it from the call's own inputs.)
 * The arithmetic per token is gdn_decode_step's, so n_tok calls of it give
 * the same bits.  Errors: as gdn_decode_step (n_tok < 1: GDN_ERR_SHAPE). */
GDN_API gdn_status gdn_decode_tokens(const gdn_shape* shape, int32_t batch, int32_t n_tok, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             float* state, int64_t pool_slots, const int32_t* slot,
                             const int32_t* slot_host, void* out, float* snapshots,
                             const float* conv_w, void* conv_state, void* stream);

/* Checkpoint copy on its own stream (sparkinfer release v0.6.28: the scan and
 * the checkpoint copy of checkpointing prompts run on their own streams, and
 * pinned host buffers for checkpoints are allocated when the prefix cache
 * starts, never mid-pass).  copy_stream first waits on wait_event (when
 * non-NULL, typically recorded after gdn_prefill_packed), then a gather
 * kernel copies item i (bytes_each bytes at ckpt_buf + i * bytes_each) to
 * dst_pool + dst_slot[i] * bytes_each, then done_event (when non-NULL) is
 * recorded on copy_stream.
 *   ckpt_buf:      device memory, n * bytes_each bytes.
 *   bytes_each:    > 0 and a multiple of 16; both pointers 16-byte aligned.
 *   dst_pool:      device memory or device-mapped pinned host memory (e.g.
 *                  from hipHostMalloc), pool_slots * bytes_each bytes.  Into
 *                  host memory (hipPointerGetAttributes) the gather runs on
 *                  one workgroup per item: the host link bounds it, so few
 *                  CUs are held while it runs.
 *   dst_slot:      device int64 [n]; dst_slot_host its host mirror, each in
 *                  [0, pool_slots) and all distinct.
 *   wait_event, done_event: hipEvent_t as void*, or NULL.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_CAPACITY, GDN_ERR_HIP. */
GDN_API gdn_status gdn_snapshot_copy(const void* ckpt_buf, int32_t n, int64_t bytes_each, void* dst_pool,
                             int64_t pool_slots, const int64_t* dst_slot,
                             const int64_t* dst_slot_host, void* wait_event, void* copy_stream,
                             void* done_event);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
