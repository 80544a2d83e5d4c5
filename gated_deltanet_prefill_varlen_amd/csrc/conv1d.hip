// Width-4 causal depthwise conv + SiLU over a packed pass (the short
// convolution ahead of q, k, v in Gated Delta Networks' block design), never
// reading across a prompt boundary.  Memory-bound: every input row is read
// once per strip of 16 (bf16) or 8 (fp32) tokens, plus a 3-row halo, and
// every output row written once.  A wave covers 512 consecutive channels of
// one token, so each row access is a contiguous 1 KiB (bf16) or 2 KiB (fp32)
// segment.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;     // channels per thread (tokens per thread: Raw8<IO>::kStrip)

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

// Raw 8-channel row segments: the strip's rows are all requested before the
// first is used, so a thread keeps a whole strip of loads in flight.
template <typename IO> struct Raw8;
template <> struct Raw8<IoBf16> {
  static constexpr int kStrip = 16;
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void unpack(float* out) const {
    const uint32_t r[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r[i] << 16);
      out[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  // 8 values rounded to bf16 (nearest even), two per conversion
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[0], v[1]}, b2));
    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[2], v[3]}, b2));
    o.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[4], v[5]}, b2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[6], v[7]}, b2));
    *reinterpret_cast<uint4*>(p) = o;
  }
};
template <> struct Raw8<IoF32> {
  static constexpr int kStrip = 8;
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void unpack(float* out) const {
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) { store8<IoF32>(p, v); }
};

// silu(x) = x / (1 + e^-x) with the hardware exp and reciprocal (about 1 ulp
// each, far below the bf16 output rounding); large |x| saturates to x or -0
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <typename IO>
__global__ void __launch_bounds__(kThreads) conv_silu_kernel(const ConvArgs a) {
  constexpr int kS = Raw8<IO>::kStrip;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  const int p0 = blockIdx.y * kS;
  if (c0 >= a.conv_dim || p0 >= a.n_tokens) return;
  const int np = min(kS, a.n_tokens - p0);
  const typename IO::T* xp = static_cast<const typename IO::T*>(a.x);

  Raw8<IO> raw[kS];
#pragma unroll
  for (int i = 0; i < kS; ++i)
    if (i < np) raw[i].load(xp + (size_t)(p0 + i) * a.x_stride + c0);

  float w[kVec][4];
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    const float4 t = reinterpret_cast<const float4*>(a.w)[c0 + c];
    w[c][0] = t.x; w[c][1] = t.y; w[c][2] = t.z; w[c][3] = t.w;
  }
  typedef const int32_t __attribute__((address_space(4)))* ConstI32;
  const ConstI32 cu = (ConstI32)a.cu;   // block-uniform reads: scalar loads
  int s = seq_of_token_uniform(a.cu, a.n_seqs, p0);
  int start = cu[s], end = cu[s + 1];
  float win[3][kVec];
#pragma unroll
  for (int j = 0; j < 3; ++j) load_ext<IO>(a, s, start, p0 - 3 + j, c0, win[j]);

  typename IO::T* yp = static_cast<typename IO::T*>(a.y);
#pragma unroll
  for (int i = 0; i < kS; ++i) {
    if (i < np) {
      const int p = p0 + i;
      if (p == end) {  // first token of the next non-empty prompt: history only
        s = seq_of_token_uniform(a.cu, a.n_seqs, p);
        start = cu[s];
        end = cu[s + 1];
#pragma unroll
        for (int j = 0; j < 3; ++j) load_hist<IO>(a, s, j, c0, win[j]);
      }
      float xc[kVec], yv[kVec];
      raw[i].unpack(xc);
#pragma unroll
      for (int c = 0; c < kVec; ++c) {
        float acc = w[c][0] * win[0][c];
        acc = fmaf(w[c][1], win[1][c], acc);
        acc = fmaf(w[c][2], win[2][c], acc);
        acc = fmaf(w[c][3], xc[c], acc);
        yv[c] = silu(acc);
        win[0][c] = win[1][c];
        win[1][c] = win[2][c];
        win[2][c] = xc[c];
      }
      Raw8<IO>::store(yp + (size_t)p * a.y_stride + c0, yv);
    }
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
    constexpr int kS = Raw8<IO>::kStrip;
    dim3 grid(gx, (a.n_tokens + kS - 1) / kS);
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
