// Token-recurrent gated delta rule on fp32 VALU: the one-token decode step on
// a state pool, and a token-by-token prefill used for the fp32 io path.
//
// Work split: one workgroup owns 32 rows (value dims) of one (sequence, value
// head) state; each row is spread over LPR = DK/16 consecutive lanes, lane
// part j holding the four-element chunks at key dims 4 LPR i + 4 j (i = 0..3),
// so the LPR lanes of a row read whole 64- to 128-byte segments per load
// instruction.  Row sums (S k, S q, |k|^2, |q|^2) are lane-group reductions
// in a fixed order, so a row's arithmetic never depends on which workgroup or
// launch computes it.
#include <climits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRows = 32;  // state rows per workgroup

// q and k scaled to unit length (this lane's 16 elements; the sums of
// squares over the row's lanes).
template <int LPR>
__device__ __forceinline__ void l2norm_kq(float* kv, float* qv, float eps) {
  float sk = 0.f, sq = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) { sk = fmaf(kv[i], kv[i], sk); sq = fmaf(qv[i], qv[i], sq); }
  sk = group_sum<LPR>(sk);
  sq = group_sum<LPR>(sq);
  const float rk = __builtin_amdgcn_rsqf(sk + eps), rq = __builtin_amdgcn_rsqf(sq + eps);
#pragma unroll
  for (int i = 0; i < 16; ++i) { kv[i] *= rk; qv[i] *= rq; }
}

// One token of the recurrence for one row, this lane's 16 state entries:
//   S <- alpha S + u k^T,  u = beta (v - alpha S k)   (= alpha S (I - beta k k^T) + beta v k^T)
// Returns o = S q (already summed over the row's lanes).
template <int LPR>
__device__ __forceinline__ float row_step(float* S, const float* kv, const float* qv, float vrow, float alpha,
                                          float beta) {
  float x = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) x = fmaf(S[i], kv[i], x);
  x = group_sum<LPR>(x);
  const float u = beta * (vrow - alpha * x);
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    S[i] = fmaf(alpha, S[i], u * kv[i]);
    o = fmaf(S[i], qv[i], o);
  }
  return group_sum<LPR>(o);
}

template <int LPR>
__device__ __forceinline__ float token_step(float* S, float* kv, float* qv, float vrow, float g,
                                            float beta, int l2norm, float eps) {
  if (l2norm) l2norm_kq<LPR>(kv, qv, eps);
  return row_step<LPR>(S, kv, qv, vrow, __expf(g), beta);
}

// The lane's 16 elements of a row (chunks of four at 4 LPR i + 4 j).
template <int LPR>
__device__ __forceinline__ void load_row16f(const float* row, int j, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 x = *reinterpret_cast<const float4*>(row + 4 * LPR * i + 4 * j);
    out[4 * i] = x.x; out[4 * i + 1] = x.y; out[4 * i + 2] = x.z; out[4 * i + 3] = x.w;
  }
}
template <int LPR>
__device__ __forceinline__ void store_row16f(float* row, int j, const float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<float4*>(row + 4 * LPR * i + 4 * j) =
        make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}
template <int LPR, typename IO>
__device__ __forceinline__ void load_row16(const typename IO::T* row, int j, float* out) {
  if constexpr (IO::kBytes == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 w = *reinterpret_cast<const uint2*>(row + 4 * LPR * i + 4 * j);
      out[4 * i] = __uint_as_float(w.x << 16);
      out[4 * i + 1] = __uint_as_float(w.x & 0xFFFF0000u);
      out[4 * i + 2] = __uint_as_float(w.y << 16);
      out[4 * i + 3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  } else {
    load_row16f<LPR>(reinterpret_cast<const float*>(row), j, out);
  }
}

template <int DK, int DV, typename IO>
__global__ void __launch_bounds__(kRows * (DK / 16))
recurrent_prefill_kernel(const ScanArgs a) {
  constexpr int LPR = DK / 16;
  using T = typename IO::T;
  const int s = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int row = blockIdx.z * kRows + tid / LPR;
  const int jl = tid % LPR;
  const int j = h / (a.Hv / a.Hqk);
  const int t0 = a.cu[s], t1 = a.cu[s + 1];

  float S[16];
  const size_t head_off = ((size_t)h * DV + row) * DK;
  const size_t state_stride = (size_t)a.Hv * DV * DK;
  if (a.init) load_row16f<LPR>(a.init + (size_t)s * state_stride + head_off, jl, S);
  else {
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
  }
  int ci = lower_bound_i32(a.ckpt, a.n_ckpt, t0 + 1);
  int next = ci < a.n_ckpt ? a.ckpt[ci] : INT_MAX;

  const T* qp = static_cast<const T*>(a.q);
  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);
  T* op = static_cast<T*>(a.out);
  for (int t = t0; t < t1; ++t) {
    float kv[16], qv[16];
    load_row16<LPR, IO>(kp + (size_t)t * a.k_stride + j * DK, jl, kv);
    load_row16<LPR, IO>(qp + (size_t)t * a.q_stride + j * DK, jl, qv);
    const float vrow = load1<IO>(vp + (size_t)t * a.v_stride + (size_t)h * DV + row);
    const float g = a.g[(size_t)t * a.Hv + h], beta = a.beta[(size_t)t * a.Hv + h];
    const float o = token_step<LPR>(S, kv, qv, vrow, g, beta, a.l2norm, a.eps);
    if (jl == 0) store1<IO>(op + ((size_t)t * a.Hv + h) * DV + row, a.scale * o);
    if (t + 1 == next) {
      store_row16f<LPR>(a.ckpt_buf + (size_t)ci * state_stride + head_off, jl, S);
      ++ci;
      next = ci < a.n_ckpt ? a.ckpt[ci] : INT_MAX;
    }
  }
  if (a.final_state) store_row16f<LPR>(a.final_state + (size_t)s * state_stride + head_off, jl, S);
}

// A workgroup holds 32 RPT rows of one (sequence, value head): thread (row
// group rg, lane part jl) holds its 16 entries of rows rg, rg + 32, ...
// (RPT rows), so it keeps several state rows in flight and forms k, q and
// their norms once for them.  Each row's arithmetic is that of token_step.
template <int DK, int DV, int RPT, typename IO, bool CONV>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  constexpr int LPR = DK / 16;
  using T = typename IO::T;
  const int b = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int rg = blockIdx.z * kRows * RPT + tid / LPR;
  const int jl = tid % LPR;
  const int j = h / (a.Hv / a.Hqk);
  // a token's inputs do not depend on the slot: without the conv, token 0's
  // are requested before the slot -> state address round trip
  float kv[16], qv[16], vrow[RPT], galpha, gbeta;
  int r = 0;
  // With the conv, q, k and v are its inputs: the value of channel c at token
  // n is conv4_silu over the channel's inputs at n-3 .. n (before the
  // sequence's first token, its slot's conv state), rounded to the io dtype
  // as a stored conv output would be (channels ordered q | k | v).  The
  // workgroup computes each channel it needs once (k and q of its qk head,
  // v of its rows) into LDS, then every thread reads its values back.
  const T* cst = static_cast<const T*>(a.conv_state);
  constexpr int NCH = 2 * DK + kRows * RPT;   // k, q, v channels of this workgroup
  __shared__ float conv_out[CONV ? NCH : 1];
  auto conv_token = [&](int n) __attribute__((always_inline)) {
    const int nq = a.Hqk * DK;
    __syncthreads();   // the previous token's values have been read
    for (int e = tid; e < NCH; e += kRows * LPR) {
      const T* x;
      int64_t stride;
      int ch;
      if (e < DK) { x = static_cast<const T*>(a.k) + j * DK + e; stride = a.k_stride; ch = nq + j * DK + e; }
      else if (e < 2 * DK) { x = static_cast<const T*>(a.q) + j * DK + e - DK; stride = a.q_stride; ch = j * DK + e - DK; }
      else {
        const int col = h * DV + blockIdx.z * kRows * RPT + (e - 2 * DK);   // the workgroup's rows
        x = static_cast<const T*>(a.v) + col;
        stride = a.v_stride;
        ch = 2 * nq + col;
      }
      float xw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {   // one load each, from the token rows or the slot's window
        const int pp = n - 3 + p;
        xw[p] = load1<IO>(pp >= 0 ? x + ((size_t)b * a.n_tok + pp) * stride
                                  : cst + ((size_t)r * 3 + 3 + pp) * a.conv_dim + ch);
      }
      const float4 w = reinterpret_cast<const float4*>(a.conv_w)[ch];
      const float y = conv4_silu(conv_tap(w.x), conv_tap(w.y), conv_tap(w.z), conv_tap(w.w), xw[0], xw[1],
                                 xw[2], xw[3]);
      conv_out[e] = IO::kBytes == 2 ? round_bf16(y) : y;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[4 * i + e] = conv_out[4 * LPR * i + 4 * jl + e];
        qv[4 * i + e] = conv_out[DK + 4 * LPR * i + 4 * jl + e];
      }
#pragma unroll
    for (int i = 0; i < RPT; ++i) vrow[i] = conv_out[2 * DK + tid / LPR + kRows * i];
  };
  auto load_tok = [&](int n) __attribute__((always_inline)) {
    const size_t t = (size_t)b * a.n_tok + n;
    if constexpr (CONV) {
      conv_token(n);
    } else {
      load_row16<LPR, IO>(static_cast<const T*>(a.k) + t * a.k_stride + j * DK, jl, kv);
      load_row16<LPR, IO>(static_cast<const T*>(a.q) + t * a.q_stride + j * DK, jl, qv);
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        vrow[i] = load1<IO>(static_cast<const T*>(a.v) + t * a.v_stride + (size_t)h * DV + rg + kRows * i);
    }
    galpha = a.g[t * a.Hv + h];
    gbeta = a.beta[t * a.Hv + h];
  };
  if constexpr (CONV) {   // token 0's window reaches into the slot's conv state
    r = a.slot ? a.slot[b] : b;
    load_tok(0);
  } else {
    load_tok(0);
    r = a.slot ? a.slot[b] : b;
  }
  float* sp = a.state + ((size_t)r * a.Hv + h) * DV * DK;
  float S[RPT][16];
#pragma unroll
  for (int i = 0; i < RPT; ++i) load_row16f<LPR>(sp + (size_t)(rg + kRows * i) * DK, jl, S[i]);
  // the sequence's tokens in order, the state staying in registers; the
  // state after each token to its snapshot when asked for
  for (int n = 0; n < a.n_tok; ++n) {
    const size_t t = (size_t)b * a.n_tok + n;
    if (n > 0) load_tok(n);
    if (a.l2norm) l2norm_kq<LPR>(kv, qv, a.eps);
    const float alpha = __expf(galpha), beta = gbeta;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + kRows * i;
      const float o = row_step<LPR>(S[i], kv, qv, vrow[i], alpha, beta);
      if (jl == 0) store1<IO>(static_cast<T*>(a.out) + (t * a.Hv + h) * DV + row, a.scale * o);
      if (a.snap) store_row16f<LPR>(a.snap + ((t * a.Hv + h) * DV + row) * DK, jl, S[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) store_row16f<LPR>(sp + (size_t)(rg + kRows * i) * DK, jl, S[i]);
}

template <int DK, int DV, int RPT, typename IO>
__global__ void __launch_bounds__(kRows * (DK / 16)) decode_kernel(const DecodeArgs a) {
  decode_body<DK, DV, RPT, IO, false>(a);
}

template <int DK, int DV, int RPT, typename IO>
__global__ void __launch_bounds__(kRows * (DK / 16)) decode_conv_kernel(const DecodeArgs a) {
  decode_body<DK, DV, RPT, IO, true>(a);
}

// The conv state of each decoding sequence's slot moves on by n_tok inputs:
// entry j becomes the input at position n_tok - 3 + j (from the tokens' own
// inputs, or the old state when n_tok < 3).  A launch of its own after the
// decode, which reads the old states.  Four channels per thread; every read
// comes before every write of the same thread's channels.
template <typename IO>
__global__ void __launch_bounds__(256) conv_shift_kernel(const DecodeArgs a) {
  using T = typename IO::T;
  const int b = blockIdx.x;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c0 >= a.conv_dim) return;
  const int r = a.slot ? a.slot[b] : b;
  T* cst = static_cast<T*>(a.conv_state) + (size_t)r * 3 * a.conv_dim + c0;
  const int nq = a.Hqk * a.dk;
  const T* x;
  int64_t stride;
  if (c0 < nq) { x = static_cast<const T*>(a.q) + c0; stride = a.q_stride; }
  else if (c0 < 2 * nq) { x = static_cast<const T*>(a.k) + (c0 - nq); stride = a.k_stride; }
  else { x = static_cast<const T*>(a.v) + (c0 - 2 * nq); stride = a.v_stride; }
  float v[3][4];
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const int p = a.n_tok - 3 + jj;
    if (p >= 0) load4<IO>(x + ((size_t)b * a.n_tok + p) * stride, v[jj]);
    else load4<IO>(cst + (size_t)(3 + p) * a.conv_dim, v[jj]);
  }
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) store4<IO>(cst + (size_t)jj * a.conv_dim, v[jj]);
}

template <int DK, int DV, typename IO>
hipError_t launch_rec_prefill(const ScanArgs& a, hipStream_t st) {
  dim3 grid(a.n_seqs, a.Hv, DV / kRows);
  hipLaunchKernelGGL((recurrent_prefill_kernel<DK, DV, IO>), grid, dim3(kRows * (DK / 16)), 0, st, a);
  return hipGetLastError();
}

template <int DK, int DV, typename IO>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t st) {
  // one token: two rows per thread (32 x 32 heads: 36 us with one row, 33
  // with two, 38 with four); several tokens: up to four rows per thread, the
  // k/q loads and norms of each token shared by them (decode of 32 x 4
  // tokens 96 -> 81 us)
  constexpr int RPT = DV / kRows < 4 ? DV / kRows : 4;
  constexpr int R1 = DV / kRows < 2 ? DV / kRows : 2;
  const dim3 blk(kRows * (DK / 16));
  if (a.conv_w) {
    if (a.n_tok == 1)
      hipLaunchKernelGGL((decode_conv_kernel<DK, DV, R1, IO>), dim3(a.batch, a.Hv, DV / (kRows * R1)), blk, 0, st, a);
    else
      hipLaunchKernelGGL((decode_conv_kernel<DK, DV, RPT, IO>), dim3(a.batch, a.Hv, DV / (kRows * RPT)), blk, 0, st,
                         a);
  } else if (a.n_tok == 1) {
    hipLaunchKernelGGL((decode_kernel<DK, DV, R1, IO>), dim3(a.batch, a.Hv, DV / (kRows * R1)), blk, 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<DK, DV, RPT, IO>), dim3(a.batch, a.Hv, DV / (kRows * RPT)), blk, 0, st, a);
  }
  if (a.conv_w) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((conv_shift_kernel<IO>), dim3(a.batch, (a.conv_dim + 1023) / 1024), dim3(256), 0, st,
                       a);
  }
  return hipGetLastError();
}

#define GDN_DISPATCH(FN, ARGS, ST)                                                     \
  do {                                                                                 \
    const int dk_ = (ARGS).dk, dv_ = (ARGS).dv;                                        \
    const bool b_ = (ARGS).bf16 != 0;                                                  \
    if (b_) {                                                                          \
      if (dk_ == 32 && dv_ == 32) return FN<32, 32, IoBf16>(ARGS, ST);                  \
      if (dk_ == 32 && dv_ == 64) return FN<32, 64, IoBf16>(ARGS, ST);                  \
      if (dk_ == 32 && dv_ == 128) return FN<32, 128, IoBf16>(ARGS, ST);                \
      if (dk_ == 64 && dv_ == 32) return FN<64, 32, IoBf16>(ARGS, ST);                  \
      if (dk_ == 64 && dv_ == 64) return FN<64, 64, IoBf16>(ARGS, ST);                  \
      if (dk_ == 64 && dv_ == 128) return FN<64, 128, IoBf16>(ARGS, ST);                \
      if (dk_ == 128 && dv_ == 32) return FN<128, 32, IoBf16>(ARGS, ST);                \
      if (dk_ == 128 && dv_ == 64) return FN<128, 64, IoBf16>(ARGS, ST);                \
      if (dk_ == 128 && dv_ == 128) return FN<128, 128, IoBf16>(ARGS, ST);              \
    } else {                                                                           \
      if (dk_ == 32 && dv_ == 32) return FN<32, 32, IoF32>(ARGS, ST);                   \
      if (dk_ == 32 && dv_ == 64) return FN<32, 64, IoF32>(ARGS, ST);                   \
      if (dk_ == 32 && dv_ == 128) return FN<32, 128, IoF32>(ARGS, ST);                 \
      if (dk_ == 64 && dv_ == 32) return FN<64, 32, IoF32>(ARGS, ST);                   \
      if (dk_ == 64 && dv_ == 64) return FN<64, 64, IoF32>(ARGS, ST);                   \
      if (dk_ == 64 && dv_ == 128) return FN<64, 128, IoF32>(ARGS, ST);                 \
      if (dk_ == 128 && dv_ == 32) return FN<128, 32, IoF32>(ARGS, ST);                 \
      if (dk_ == 128 && dv_ == 64) return FN<128, 64, IoF32>(ARGS, ST);                 \
      if (dk_ == 128 && dv_ == 128) return FN<128, 128, IoF32>(ARGS, ST);               \
    }                                                                                  \
    return hipErrorInvalidValue;                                                       \
  } while (0)

}  // namespace

hipError_t launch_prefill_recurrent(const ScanArgs& a, hipStream_t st) {
  GDN_DISPATCH(launch_rec_prefill, a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) { GDN_DISPATCH(launch_dec, a, st); }

}  // namespace gdn
