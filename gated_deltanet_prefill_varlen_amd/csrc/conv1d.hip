// Width-4 causal depthwise conv + SiLU over a packed pass (the short
// convolution ahead of q, k, v in Gated Delta Networks' block design), never
// reading across a prompt boundary.  Memory-bound: every input row is read
// once per 16-token strip (plus a 3-row halo) and every output row written
// once.  A wave covers 512 consecutive channels of one token, so each row
// access is a contiguous 1 KiB (bf16) or 2 KiB (fp32) segment.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kStrip = 16;  // tokens per thread
constexpr int kVec = 8;     // channels per thread

template <typename IO>
__device__ __forceinline__ void load_hist(const ConvArgs& a, int s, int i, int c0, float* out) {
  if (a.state_in) {
    const typename IO::T* p = static_cast<const typename IO::T*>(a.state_in) +
                              ((size_t)s * 3 + i) * a.conv_dim + c0;
    load8<IO>(p, out);
  } else {
#pragma unroll
    for (int c = 0; c < kVec; ++c) out[c] = 0.f;
  }
}

// xs[pp] for a position pp of prompt s (start = cu[s]); before the prompt's
// first token it comes from the prompt's conv state.
template <typename IO>
__device__ __forceinline__ void load_ext(const ConvArgs& a, int s, int start, int pp, int c0,
                                         float* out) {
  if (pp >= start)
    load8<IO>(static_cast<const typename IO::T*>(a.x) + (size_t)pp * a.x_stride + c0, out);
  else
    load_hist<IO>(a, s, pp - start + 3, c0, out);
}

template <typename IO>
__global__ void __launch_bounds__(kThreads) conv_silu_kernel(const ConvArgs a) {
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  const int p0 = blockIdx.y * kStrip;
  if (c0 >= a.conv_dim || p0 >= a.n_tokens) return;
  const int p1 = min(p0 + kStrip, a.n_tokens);

  float w[kVec][4];
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    const float4 t = reinterpret_cast<const float4*>(a.w)[c0 + c];
    w[c][0] = t.x; w[c][1] = t.y; w[c][2] = t.z; w[c][3] = t.w;
  }
  int s = seq_of_token(a.cu, a.n_seqs, p0);
  int start = a.cu[s], end = a.cu[s + 1];
  float win[3][kVec];
#pragma unroll
  for (int j = 0; j < 3; ++j) load_ext<IO>(a, s, start, p0 - 3 + j, c0, win[j]);

  typename IO::T* yp = static_cast<typename IO::T*>(a.y);
  for (int p = p0; p < p1; ++p) {
    if (p == end) {  // first token of the next non-empty prompt: history only
      s = seq_of_token(a.cu, a.n_seqs, p);
      start = a.cu[s];
      end = a.cu[s + 1];
#pragma unroll
      for (int j = 0; j < 3; ++j) load_hist<IO>(a, s, j, c0, win[j]);
    }
    float xc[kVec], yv[kVec];
    load8<IO>(static_cast<const typename IO::T*>(a.x) + (size_t)p * a.x_stride + c0, xc);
#pragma unroll
    for (int c = 0; c < kVec; ++c) {
      float acc = w[c][0] * win[0][c];
      acc = fmaf(w[c][1], win[1][c], acc);
      acc = fmaf(w[c][2], win[2][c], acc);
      acc = fmaf(w[c][3], xc[c], acc);
      yv[c] = acc / (1.0f + expf(-acc));
      win[0][c] = win[1][c];
      win[1][c] = win[2][c];
      win[2][c] = xc[c];
    }
    store8<IO>(yp + (size_t)p * a.y_stride + c0, yv);
  }
}

// The three inputs before position e of prompt s, copied to dst[3][conv_dim].
// by_ckpt = 0: e = end of prompt blockIdx.y (conv state out);
// by_ckpt = 1: e = checkpoint blockIdx.y (its prompt found from cu).
template <typename IO>
__global__ void __launch_bounds__(kThreads) conv_window_kernel(const ConvArgs a, int by_ckpt) {
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (c0 >= a.conv_dim) return;
  const int i = blockIdx.y;
  int s, e;
  typename IO::T* dst;
  if (by_ckpt) {
    e = a.ckpt[i];
    s = seq_of_token(a.cu, a.n_seqs, e - 1);
    dst = static_cast<typename IO::T*>(a.conv_ckpt) + (size_t)i * 3 * a.conv_dim;
  } else {
    s = i;
    e = a.cu[s + 1];
    dst = static_cast<typename IO::T*>(a.state_out) + (size_t)i * 3 * a.conv_dim;
  }
  const int start = a.cu[s];
  float v[3][kVec];
#pragma unroll
  for (int j = 0; j < 3; ++j) load_ext<IO>(a, s, start, e - 3 + j, c0, v[j]);
  // all reads above happen before any write: safe when state_out == state_in
#pragma unroll
  for (int j = 0; j < 3; ++j) store8<IO>(dst + (size_t)j * a.conv_dim + c0, v[j]);
}

template <typename IO>
hipError_t launch(const ConvArgs& a, hipStream_t st) {
  const int gx = (a.conv_dim / kVec + kThreads - 1) / kThreads;
  if (a.n_tokens > 0) {
    dim3 grid(gx, (a.n_tokens + kStrip - 1) / kStrip);
    hipLaunchKernelGGL(conv_silu_kernel<IO>, grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // checkpoint windows read the conv state in, so they go before it is overwritten
  for (int i0 = 0; a.conv_ckpt && i0 < a.n_ckpt; i0 += 65535) {
    ConvArgs b = a;
    b.ckpt = a.ckpt + i0;
    b.conv_ckpt = static_cast<char*>(a.conv_ckpt) + (size_t)i0 * 3 * a.conv_dim * IO::kBytes;
    hipLaunchKernelGGL(conv_window_kernel<IO>, dim3(gx, min(65535, a.n_ckpt - i0)), dim3(kThreads),
                       0, st, b, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int s0 = 0; a.state_out && s0 < a.n_seqs; s0 += 65535) {
    ConvArgs b = a;
    b.cu = a.cu + s0;
    b.n_seqs = a.n_seqs - s0;
    if (a.state_in)
      b.state_in = static_cast<const char*>(a.state_in) + (size_t)s0 * 3 * a.conv_dim * IO::kBytes;
    b.state_out = static_cast<char*>(a.state_out) + (size_t)s0 * 3 * a.conv_dim * IO::kBytes;
    hipLaunchKernelGGL(conv_window_kernel<IO>, dim3(gx, min(65535, a.n_seqs - s0)), dim3(kThreads),
                       0, st, b, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t st) {
  return a.bf16 ? launch<IoBf16>(a, st) : launch<IoF32>(a, st);
}

}  // namespace gdn
