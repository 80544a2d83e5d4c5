// C-ABI entry points of libgdn: host-side validation, the checkpoint planner
// and kernel dispatch.  No HIP call is made before a call is fully validated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

bool supported_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }
bool supported_chunk(int32_t c) { return c == 16 || c == 32 || c == 64; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks common to every call that takes a gdn_shape.
gdn_status check_shape(const gdn_shape* s) {
  if (!s) return GDN_ERR_NULL;
  if (s->num_qk_heads < 1 || s->num_v_heads < 1) return GDN_ERR_SHAPE;
  if (s->num_v_heads % s->num_qk_heads != 0) return GDN_ERR_UNSUPPORTED;
  if (!supported_dim(s->head_k_dim) || !supported_dim(s->head_v_dim)) return GDN_ERR_UNSUPPORTED;
  if (!supported_chunk(s->chunk)) return GDN_ERR_UNSUPPORTED;
  if (s->io_dtype != GDN_BF16 && s->io_dtype != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (s->flags & ~GDN_QK_L2NORM) return GDN_ERR_UNSUPPORTED;
  if (!std::isfinite(s->scale) || !std::isfinite(s->l2_eps) || s->l2_eps < 0.f) return GDN_ERR_SHAPE;
  if (s->q_tok_stride < 0 || s->k_tok_stride < 0 || s->v_tok_stride < 0) return GDN_ERR_SHAPE;
  return GDN_OK;
}

int64_t elem_bytes(const gdn_shape* s) { return s->io_dtype == GDN_BF16 ? 2 : 4; }

// Resolve a token stride (0 = dense) and check that it fits the row, stays
// below 2^23 elements (the kernels address the rows of a chunk with 32-bit
// offsets) and keeps 16-byte alignment of every row.
gdn_status resolve_stride(const gdn_shape* s, int64_t given, int64_t dense, int64_t* out) {
  const int64_t st = given == 0 ? dense : given;
  if (st < dense || st >= (int64_t(1) << 23)) return GDN_ERR_SHAPE;
  if ((st * elem_bytes(s)) % 16 != 0) return GDN_ERR_SHAPE;
  *out = st;
  return GDN_OK;
}

gdn_status check_seqlens(const int32_t* cu, int32_t n_seqs, int32_t n_tokens) {
  if (n_seqs < 0 || n_tokens < 0) return GDN_ERR_SHAPE;
  if (!cu) return GDN_ERR_NULL;
  if (cu[0] != 0) return GDN_ERR_SEQLENS;
  for (int32_t s = 0; s < n_seqs; ++s)
    if (cu[s + 1] < cu[s]) return GDN_ERR_SEQLENS;
  if (cu[n_seqs] != n_tokens) return GDN_ERR_SEQLENS;
  return GDN_OK;
}

// Checkpoints: strictly increasing, each inside a prompt (cu[s] < p <= cu[s+1]).
// Any position works: the scan also ends a chunk at every checkpoint.
gdn_status check_ckpts(const int32_t* cu, int32_t n_seqs, const int32_t* pos, int32_t n) {
  if (n < 0) return GDN_ERR_SHAPE;
  if (n == 0) return GDN_OK;
  if (!pos) return GDN_ERR_NULL;
  int32_t s = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pos[i];
    if (i > 0 && p <= pos[i - 1]) return GDN_ERR_CKPT;
    while (s < n_seqs && cu[s + 1] < p) ++s;
    // skip empty prompts that end exactly at p-1 ... the owner has cu[s] < p
    while (s < n_seqs && !(cu[s] < p && p <= cu[s + 1])) ++s;
    if (s >= n_seqs) return GDN_ERR_CKPT;
  }
  return GDN_OK;
}

// Every slot in [0, pool_slots) and no slot twice; the check sorts a copy
// of the n slots, so its host memory is O(n) whatever the pool's size.
template <typename T>
gdn_status check_slots(const T* slots, int64_t n, int64_t pool_slots) {
  std::vector<int64_t> v(slots, slots + n);
  std::sort(v.begin(), v.end());
  for (int64_t i = 0; i < n; ++i)
    if (v[i] < 0 || v[i] >= pool_slots || (i > 0 && v[i] == v[i - 1])) return GDN_ERR_CAPACITY;
  return GDN_OK;
}

gdn_status finish_launch(hipError_t e, hipStream_t stream) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(stream);  // leave nothing of this call in flight
    return GDN_ERR_HIP;
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(int32_t status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: bad count, stride, alignment or size";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dims, chunk, dtype, flags or head ratio not supported";
    case GDN_ERR_SEQLENS: return "GDN_ERR_SEQLENS: cu_seqlens must start at 0, not decrease and end at n_tokens";
    case GDN_ERR_CKPT: return "GDN_ERR_CKPT: checkpoints must increase and each lie inside a prompt";
    case GDN_ERR_CAPACITY: return "GDN_ERR_CAPACITY: output list too short or slot outside the pool";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown gdn_status";
  }
}

gdn_status gdn_plan_checkpoints(const int32_t* cu_host, int32_t n_seqs, const int32_t* p0_host,
                                int32_t block, int32_t tail, int32_t* out_pos, int32_t cap,
                                int32_t* n_out) {
  if (!cu_host || !n_out) return GDN_ERR_NULL;
  if (n_seqs < 0 || block < 1 || tail < 0 || cap < 0) return GDN_ERR_SHAPE;
  if (cap > 0 && !out_pos) return GDN_ERR_NULL;
  if (cu_host[0] != 0) return GDN_ERR_SEQLENS;
  for (int32_t s = 0; s < n_seqs; ++s)
    if (cu_host[s + 1] < cu_host[s]) return GDN_ERR_SEQLENS;
  int64_t count = 0;
  std::vector<int64_t> taken;
  for (int32_t s = 0; s < n_seqs; ++s) {
    const int64_t L = cu_host[s + 1] - cu_host[s];
    const int64_t start = p0_host ? p0_host[s] : 0;
    if (start < 0) return GDN_ERR_SHAPE;
    taken.clear();
    // multiples of the block inside (start, start + L]; one in the last
    // `tail` tokens moves back a block; moved ones that hit the start or an
    // earlier one are dropped.  Candidates ascend, so "earlier one" is the
    // last taken.
    for (int64_t c = block * (start / block + 1); c <= start + L; c += block) {
      int64_t p = c;
      if (start + L - p < tail) p -= block;
      if (p <= start) continue;
      if (!taken.empty() && taken.back() >= p) continue;
      taken.push_back(p);
    }
    for (int64_t p : taken) {
      if (count < cap) out_pos[count] = (int32_t)(cu_host[s] + (p - start));
      ++count;
    }
  }
  *n_out = (int32_t)count;
  return count > cap ? GDN_ERR_CAPACITY : GDN_OK;
}

gdn_status gdn_prefill_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t n_tokens,
                              const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* init_state,
                              const int32_t* ckpt_positions, const int32_t* ckpt_positions_host,
                              int32_t n_ckpt, void* out, float* final_state, float* ckpt_buf,
                              void* stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  st = check_seqlens(cu_seqlens_host, n_seqs, n_tokens);
  if (st != GDN_OK) return st;
  if (n_seqs > 0 && !cu_seqlens) return GDN_ERR_NULL;
  if (n_tokens > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL;
  if (n_ckpt < 0) return GDN_ERR_SHAPE;
  if (n_ckpt > 0 && (!ckpt_positions || !ckpt_positions_host || !ckpt_buf)) return GDN_ERR_NULL;
  st = check_ckpts(cu_seqlens_host, n_seqs, ckpt_positions_host, n_ckpt);
  if (st != GDN_OK) return st;
  const int64_t Hqk = shape->num_qk_heads, Hv = shape->num_v_heads;
  const int64_t dk = shape->head_k_dim, dv = shape->head_v_dim;
  int64_t qs, ks, vs;
  if ((st = resolve_stride(shape, shape->q_tok_stride, Hqk * dk, &qs)) != GDN_OK) return st;
  if ((st = resolve_stride(shape, shape->k_tok_stride, Hqk * dk, &ks)) != GDN_OK) return st;
  if ((st = resolve_stride(shape, shape->v_tok_stride, Hv * dv, &vs)) != GDN_OK) return st;
  const void* ptrs[] = {q, k, v, out, init_state, final_state, ckpt_buf};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_SHAPE;
  if (n_seqs == 0) return GDN_OK;

  gdn::ScanArgs a{};
  a.cu = cu_seqlens; a.n_seqs = n_seqs; a.n_tokens = n_tokens;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.init = init_state;
  a.ckpt = ckpt_positions; a.n_ckpt = n_ckpt;
  a.out = out; a.final_state = final_state; a.ckpt_buf = ckpt_buf;
  a.q_stride = qs; a.k_stride = ks; a.v_stride = vs;
  a.Hqk = (int32_t)Hqk; a.Hv = (int32_t)Hv; a.dk = (int32_t)dk; a.dv = (int32_t)dv;
  a.chunk = shape->chunk; a.bf16 = shape->io_dtype == GDN_BF16;
  a.l2norm = (shape->flags & GDN_QK_L2NORM) != 0;
  a.scale = shape->scale; a.eps = shape->l2_eps;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return finish_launch(gdn::launch_prefill(a, s), s);
}

gdn_status gdn_prefill_conv_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t n_tokens,
                                   const void* x, int64_t x_tok_stride, const float* conv_weight,
                                   const void* conv_state_in, void* conv_state_out, const float* g,
                                   const float* beta, const float* init_state,
                                   const int32_t* ckpt_positions, const int32_t* ckpt_positions_host,
                                   int32_t n_ckpt, void* conv_ckpt, void* out, float* final_state,
                                   float* ckpt_buf, void* stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  // the kernel that fuses the conv: bf16, d_k = d_v = 128, 32-token tiles
  if (shape->io_dtype != GDN_BF16 || shape->head_k_dim != 128 || shape->head_v_dim != 128 ||
      shape->chunk < 32)
    return GDN_ERR_UNSUPPORTED;
  st = check_seqlens(cu_seqlens_host, n_seqs, n_tokens);
  if (st != GDN_OK) return st;
  if (n_seqs > 0 && (!cu_seqlens || !conv_weight)) return GDN_ERR_NULL;
  if (n_tokens > 0 && (!x || !g || !beta || !out)) return GDN_ERR_NULL;
  if (n_ckpt < 0) return GDN_ERR_SHAPE;
  if (n_ckpt > 0 && (!ckpt_positions || !ckpt_positions_host || !ckpt_buf)) return GDN_ERR_NULL;
  st = check_ckpts(cu_seqlens_host, n_seqs, ckpt_positions_host, n_ckpt);
  if (st != GDN_OK) return st;
  const int64_t Hqk = shape->num_qk_heads, Hv = shape->num_v_heads;
  const int64_t conv_dim = 2 * Hqk * 128 + Hv * 128;
  int64_t xs;
  if ((st = resolve_stride(shape, x_tok_stride, conv_dim, &xs)) != GDN_OK) return st;
  const void* ptrs[] = {x, conv_weight, conv_state_in, conv_state_out, conv_ckpt, out,
                        init_state, final_state, ckpt_buf};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_SHAPE;
  if (n_tokens > 0) {  // out must not overlap x
    const char* xb = static_cast<const char*>(x);
    const char* ob = static_cast<const char*>(out);
    const char* xe = xb + ((int64_t)(n_tokens - 1) * xs + conv_dim) * 2;
    const char* oe = ob + (int64_t)n_tokens * Hv * 128 * 2;
    if (xb < oe && ob < xe) return GDN_ERR_SHAPE;
  }
  if (n_seqs == 0) return GDN_OK;

  gdn::ScanArgs a{};
  a.cu = cu_seqlens; a.n_seqs = n_seqs; a.n_tokens = n_tokens;
  a.g = g; a.beta = beta; a.init = init_state;
  a.ckpt = ckpt_positions; a.n_ckpt = n_ckpt;
  a.out = out; a.final_state = final_state; a.ckpt_buf = ckpt_buf;
  a.Hqk = (int32_t)Hqk; a.Hv = (int32_t)Hv; a.dk = 128; a.dv = 128;
  a.chunk = shape->chunk; a.bf16 = 1;
  a.l2norm = (shape->flags & GDN_QK_L2NORM) != 0;
  a.scale = shape->scale; a.eps = shape->l2_eps;
  a.conv_x = x; a.conv_x_stride = xs; a.conv_w = conv_weight;
  a.conv_state_in = conv_state_in; a.conv_state_out = conv_state_out; a.conv_ckpt = conv_ckpt;
  a.conv_dim = (int32_t)conv_dim;
  // conv states written in place: every workgroup of a prompt reads its
  // history first, so the new windows come from a launch of their own after
  const bool in_place = conv_state_out && conv_state_out == conv_state_in;
  a.conv_state_own = conv_state_out && !in_place;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_prefill(a, s);
  if (e == hipSuccess && in_place) {
    gdn::ConvArgs c{};
    c.cu = cu_seqlens; c.n_seqs = n_seqs; c.n_tokens = n_tokens; c.conv_dim = (int32_t)conv_dim;
    c.x = x; c.x_stride = xs; c.state_in = conv_state_in; c.state_out = conv_state_out; c.bf16 = 1;
    e = gdn::launch_conv_states(c, s);
  }
  return finish_launch(e, s);
}

gdn_status gdn_decode_step(const gdn_shape* shape, int32_t batch, const void* q, const void* k,
                           const void* v, const float* g, const float* beta, float* state,
                           int64_t pool_slots, const int32_t* slot, const int32_t* slot_host,
                           void* out, const float* conv_w, void* conv_state, void* stream) {
  return gdn_decode_tokens(shape, batch, 1, q, k, v, g, beta, state, pool_slots, slot, slot_host, out,
                           nullptr, conv_w, conv_state, stream);
}

gdn_status gdn_decode_tokens(const gdn_shape* shape, int32_t batch, int32_t n_tok, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             float* state, int64_t pool_slots, const int32_t* slot,
                             const int32_t* slot_host, void* out, float* snapshots,
                             const float* conv_w, void* conv_state, void* stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  if (batch < 0 || pool_slots < 0 || n_tok < 1) return GDN_ERR_SHAPE;
  if ((int64_t)batch * n_tok > INT32_MAX) return GDN_ERR_SHAPE;
  if (!conv_w != !conv_state) return GDN_ERR_NULL;   // the conv needs both
  if (batch == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state || !out) return GDN_ERR_NULL;
  if (slot) {
    if (!slot_host) return GDN_ERR_NULL;
    if ((st = check_slots(slot_host, batch, pool_slots)) != GDN_OK) return st;
  } else if (batch > pool_slots) {
    return GDN_ERR_CAPACITY;
  }
  const int64_t Hqk = shape->num_qk_heads, Hv = shape->num_v_heads;
  const int64_t dk = shape->head_k_dim, dv = shape->head_v_dim;
  int64_t qs, ks, vs;
  if ((st = resolve_stride(shape, shape->q_tok_stride, Hqk * dk, &qs)) != GDN_OK) return st;
  if ((st = resolve_stride(shape, shape->k_tok_stride, Hqk * dk, &ks)) != GDN_OK) return st;
  if ((st = resolve_stride(shape, shape->v_tok_stride, Hv * dv, &vs)) != GDN_OK) return st;
  const void* ptrs[] = {q, k, v, out, state, snapshots, conv_w, conv_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_SHAPE;
  const int64_t conv_dim = 2 * Hqk * dk + Hv * dv;
  if (conv_w && conv_dim > INT32_MAX / 4) return GDN_ERR_SHAPE;

  gdn::DecodeArgs a{};
  a.batch = batch; a.n_tok = n_tok; a.snap = snapshots;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state = state; a.slot = slot; a.out = out;
  a.conv_w = conv_w; a.conv_state = conv_state; a.conv_dim = (int32_t)conv_dim;
  a.q_stride = qs; a.k_stride = ks; a.v_stride = vs;
  a.Hqk = (int32_t)Hqk; a.Hv = (int32_t)Hv; a.dk = (int32_t)dk; a.dv = (int32_t)dv;
  a.bf16 = shape->io_dtype == GDN_BF16;
  a.l2norm = (shape->flags & GDN_QK_L2NORM) != 0;
  a.scale = shape->scale; a.eps = shape->l2_eps;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return finish_launch(gdn::launch_decode(a, s), s);
}

gdn_status gdn_conv1d_silu_packed(const gdn_shape* shape, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_host, int32_t n_seqs,
                                  int32_t n_tokens, const void* x, int64_t x_tok_stride,
                                  const float* weight, const void* conv_state_in, void* y,
                                  int64_t y_tok_stride, void* conv_state_out,
                                  const int32_t* ckpt_positions,
                                  const int32_t* ckpt_positions_host, int32_t n_ckpt,
                                  void* conv_ckpt, void* stream) {
  gdn_status st = check_shape(shape);
  if (st != GDN_OK) return st;
  st = check_seqlens(cu_seqlens_host, n_seqs, n_tokens);
  if (st != GDN_OK) return st;
  if (n_seqs > 0 && !cu_seqlens) return GDN_ERR_NULL;
  if (!weight && n_seqs > 0) return GDN_ERR_NULL;
  if (n_tokens > 0 && (!x || !y)) return GDN_ERR_NULL;
  if (n_ckpt < 0) return GDN_ERR_SHAPE;
  if (n_ckpt > 0 && conv_ckpt && (!ckpt_positions || !ckpt_positions_host)) return GDN_ERR_NULL;
  st = check_ckpts(cu_seqlens_host, n_seqs, ckpt_positions_host, conv_ckpt ? n_ckpt : 0);
  if (st != GDN_OK) return st;
  const int64_t conv_dim = 2LL * shape->num_qk_heads * shape->head_k_dim +
                           (int64_t)shape->num_v_heads * shape->head_v_dim;
  if (conv_dim > INT32_MAX) return GDN_ERR_SHAPE;
  int64_t xs, ys;
  if ((st = resolve_stride(shape, x_tok_stride, conv_dim, &xs)) != GDN_OK) return st;
  if ((st = resolve_stride(shape, y_tok_stride, conv_dim, &ys)) != GDN_OK) return st;
  const void* ptrs[] = {x, y, conv_state_in, conv_state_out, conv_ckpt};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_SHAPE;
  if (n_tokens > 0) {  // y must not overlap x
    const char* xb = static_cast<const char*>(x);
    const char* yb = static_cast<const char*>(y);
    const int64_t eb = elem_bytes(shape);
    const char* xe = xb + ((int64_t)(n_tokens - 1) * xs + conv_dim) * eb;
    const char* ye = yb + ((int64_t)(n_tokens - 1) * ys + conv_dim) * eb;
    if (xb < ye && yb < xe) return GDN_ERR_SHAPE;
  }
  if (n_seqs == 0) return GDN_OK;

  gdn::ConvArgs a{};
  a.cu = cu_seqlens; a.n_seqs = n_seqs; a.n_tokens = n_tokens; a.conv_dim = (int32_t)conv_dim;
  a.x = x; a.x_stride = xs; a.w = weight; a.state_in = conv_state_in;
  a.y = y; a.y_stride = ys; a.state_out = conv_state_out;
  a.ckpt = conv_ckpt ? ckpt_positions : nullptr; a.n_ckpt = conv_ckpt ? n_ckpt : 0;
  a.conv_ckpt = conv_ckpt; a.bf16 = shape->io_dtype == GDN_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return finish_launch(gdn::launch_conv(a, s), s);
}

gdn_status gdn_snapshot_copy(const void* ckpt_buf, int32_t n, int64_t bytes_each, void* dst_pool,
                             int64_t pool_slots, const int64_t* dst_slot,
                             const int64_t* dst_slot_host, void* wait_event, void* copy_stream,
                             void* done_event) {
  if (n < 0 || pool_slots < 0) return GDN_ERR_SHAPE;
  if (n > 0) {
    if (!ckpt_buf || !dst_pool || !dst_slot || !dst_slot_host) return GDN_ERR_NULL;
    if (bytes_each <= 0 || bytes_each % 16 != 0) return GDN_ERR_SHAPE;
    if (!aligned16(ckpt_buf) || !aligned16(dst_pool)) return GDN_ERR_SHAPE;
    const gdn_status sc = check_slots(dst_slot_host, n, pool_slots);
    if (sc != GDN_OK) return sc;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(copy_stream);
  hipError_t e = hipSuccess;
  if (wait_event) e = hipStreamWaitEvent(s, reinterpret_cast<hipEvent_t>(wait_event), 0);
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (n > 0) {
    // A pool in host memory is bounded by the host link: the gather then runs
    // on one workgroup per item, which keeps the link saturated (faster here
    // than one DMA transfer per item) while holding few CUs.
    hipPointerAttribute_t attr{};
    const hipError_t pe = hipPointerGetAttributes(&attr, dst_pool);
    if (pe != hipSuccess) (void)hipGetLastError();   // not a HIP allocation: treat as device
    const int32_t host_dst = pe == hipSuccess && attr.type == hipMemoryTypeHost;
    gdn::CopyArgs a{ckpt_buf, n, bytes_each, dst_pool, dst_slot, host_dst};
    const gdn_status r = finish_launch(gdn::launch_snapshot_copy(a, s), s);
    if (r != GDN_OK) return r;
  }
  if (done_event) {
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(done_event), s);
    if (e != hipSuccess) return finish_launch(e, s);
  }
  return GDN_OK;
}

}  // extern "C"
