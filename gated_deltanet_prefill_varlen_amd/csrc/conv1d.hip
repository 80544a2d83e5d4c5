// Width-4 causal depthwise conv + SiLU over a packed pass (the short
// convolution ahead of q, k, v in Gated Delta Networks' block design), never
// reading across a prompt boundary.  Memory-bound: every input row is read
// once per strip of 20 (bf16) or 8 (fp32) tokens, plus a 3-row halo, and
// every output row written once.  A wave covers 256 consecutive channels of
// one token, so each row access is a contiguous 512 B (bf16) or 1 KiB (fp32)
// segment.  Four channels per thread keep a bf16 strip in few enough VGPRs
// for 6 or more waves per SIMD, which hides the load latency better than 8
// channels at 3 waves.  bf16 strips stream past the caches (non-temporal
// loads and stores) except their last three rows, which the next strip
// reads again as its halo and so are loaded through the cache.
#include <climits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;     // channels per thread (tokens per thread: RawRow<IO>::kStrip)

template <typename IO>
__device__ __forceinline__ void load_hist(const ConvArgs& a, int s, int i, int c0, float* out) {
  if (a.state_in) {
    const typename IO::T* p = static_cast<const typename IO::T*>(a.state_in) +
                              ((size_t)s * 3 + i) * a.conv_dim + c0;
    load4<IO>(p, out);
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
    load4<IO>(static_cast<const typename IO::T*>(a.x) + (size_t)pp * a.x_stride + c0, out);
  else
    load_hist<IO>(a, s, pp - start + 3, c0, out);
}

// Raw 4-channel row segments: the strip's rows are all requested before the
// first is used, so a thread keeps a whole strip of loads in flight.
template <typename IO> struct RawRow;
template <> struct RawRow<IoBf16> {
  static constexpr int kStrip = 20;
  static constexpr bool kStream = true;   // non-temporal loads and stores
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  u2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u2*>(p); }
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    w = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
  }
  __device__ __forceinline__ void unpack(float* out) const {
    out[0] = __uint_as_float(w[0] << 16);
    out[1] = __uint_as_float(w[0] & 0xFFFF0000u);
    out[2] = __uint_as_float(w[1] << 16);
    out[3] = __uint_as_float(w[1] & 0xFFFF0000u);
  }
  // 4 values rounded to bf16 (nearest even), two per conversion
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const u2 o{__builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[0], v[1]}, b2)),
               __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[2], v[3]}, b2))};
    __builtin_nontemporal_store(o, reinterpret_cast<u2*>(p));
  }
};
template <> struct RawRow<IoF32> {
  static constexpr int kStrip = 8;
  static constexpr bool kStream = false;
  float4 a;
  __device__ __forceinline__ void load(const float* p) { a = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) { load(p); }
  __device__ __forceinline__ void unpack(float* out) const {
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) { store4<IoF32>(p, v); }
};

// The three inputs before position e of prompt s (history from its conv
// state where e - 3 reaches before the prompt), channels c0 .. c0 + 3, to
// dst[3][conv_dim].  All reads come before any write: safe when dst is the
// conv state being read.
template <typename IO>
__device__ __forceinline__ void copy_window(const ConvArgs& a, int s, int e, typename IO::T* dst, int c0) {
  const int start = a.cu[s];
  float v[3][kVec];
#pragma unroll
  for (int j = 0; j < 3; ++j) load_ext<IO>(a, s, start, e - 3 + j, c0, v[j]);
#pragma unroll
  for (int j = 0; j < 3; ++j) store4<IO>(dst + (size_t)j * a.conv_dim + c0, v[j]);
}

// blockIdx.x: a block of kThreads x kVec channels (the channel blocks of a
// strip are neighbours in dispatch order, so a strip's rows are read whole);
// row index b = blockIdx.y + 65535 blockIdx.z: b < n_strips a strip of
// tokens, then n_ck checkpoint windows, then the conv-state windows (the last
// three inputs of each prompt) when they are written here.
template <typename IO>
__global__ void __launch_bounds__(kThreads) conv_silu_kernel(const ConvArgs a, int n_strips, int n_ck, int n_rows) {
  constexpr int kS = RawRow<IO>::kStrip;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  const int b = blockIdx.y + 65535 * blockIdx.z;
  if (c0 >= a.conv_dim || b >= n_rows) return;
  if (b >= n_strips) {
    const int i = b - n_strips;
    if (i < n_ck) {
      const int e = a.ckpt[i];
      copy_window<IO>(a, seq_of_token(a.cu, a.n_seqs, e - 1), e,
                      static_cast<typename IO::T*>(a.conv_ckpt) + (size_t)i * 3 * a.conv_dim, c0);
    } else {
      const int sq = i - n_ck;
      copy_window<IO>(a, sq, a.cu[sq + 1], static_cast<typename IO::T*>(a.state_out) + (size_t)sq * 3 * a.conv_dim,
                      c0);
    }
    return;
  }
  const int p0 = b * kS;
  if (p0 >= a.n_tokens) return;
  const int np = min(kS, a.n_tokens - p0);
  const typename IO::T* xp = static_cast<const typename IO::T*>(a.x);

  RawRow<IO> raw[kS];
#pragma unroll
  for (int i = 0; i < kS; ++i) {
    if (i < np) {
      const typename IO::T* row = xp + (size_t)(p0 + i) * a.x_stride + c0;
      if (RawRow<IO>::kStream && i < kS - 3) raw[i].load_nt(row);
      else raw[i].load(row);   // the next strip's halo: kept in the cache
    }
  }

  float w[kVec][4];
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    const float4 t = reinterpret_cast<const float4*>(a.w)[c0 + c];
    w[c][0] = conv_tap(t.x); w[c][1] = conv_tap(t.y); w[c][2] = conv_tap(t.z); w[c][3] = conv_tap(t.w);
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
        yv[c] = conv4_silu(w[c][0], w[c][1], w[c][2], w[c][3], win[0][c], win[1][c], win[2][c], xc[c]);
        win[0][c] = win[1][c];
        win[1][c] = win[2][c];
        win[2][c] = xc[c];
      }
      RawRow<IO>::store(yp + (size_t)p * a.y_stride + c0, yv);
    }
  }
}

// Conv states out when they overwrite the conv states in: a launch of its
// own after the conv (which reads the states in), one block row per prompt.
template <typename IO>
__global__ void __launch_bounds__(kThreads) conv_state_kernel(const ConvArgs a) {
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kVec;
  if (c0 >= a.conv_dim) return;
  const int sq = blockIdx.y;
  copy_window<IO>(a, sq, a.cu[sq + 1], static_cast<typename IO::T*>(a.state_out) + (size_t)sq * 3 * a.conv_dim, c0);
}

// Each prompt's last three inputs to state_out (reading its history from
// state_in, which state_out may be), one block row per prompt.
template <typename IO>
hipError_t launch_states(const ConvArgs& a, hipStream_t st) {
  const int gc = (a.conv_dim / kVec + kThreads - 1) / kThreads;
  for (int s0 = 0; s0 < a.n_seqs; s0 += 65535) {
    ConvArgs b = a;
    b.cu = a.cu + s0;
    b.n_seqs = a.n_seqs - s0;
    if (a.state_in)
      b.state_in = static_cast<const char*>(a.state_in) + (size_t)s0 * 3 * a.conv_dim * IO::kBytes;
    b.state_out = static_cast<char*>(a.state_out) + (size_t)s0 * 3 * a.conv_dim * IO::kBytes;
    hipLaunchKernelGGL(conv_state_kernel<IO>, dim3(gc, min(65535, a.n_seqs - s0)), dim3(kThreads), 0, st, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename IO>
hipError_t launch(const ConvArgs& a, hipStream_t st) {
  constexpr int kS = RawRow<IO>::kStrip;
  const int gc = (a.conv_dim / kVec + kThreads - 1) / kThreads;
  const int64_t n_strips = (a.n_tokens + kS - 1) / kS;
  const int64_t n_ck = a.conv_ckpt ? a.n_ckpt : 0;
  // conv states out in the same launch unless they overwrite the states in
  // (the conv and the checkpoint windows read those)
  const bool in_place = a.state_out && a.state_out == a.state_in;
  const int64_t n_st = a.state_out && !in_place ? a.n_seqs : 0;
  const int64_t rows = n_strips + n_ck + n_st;
  if (rows > INT_MAX) return hipErrorInvalidValue;
  if (rows > 0) {
    const dim3 grid(gc, (uint32_t)std::min<int64_t>(rows, 65535), (uint32_t)((rows + 65534) / 65535));
    hipLaunchKernelGGL(conv_silu_kernel<IO>, grid, dim3(kThreads), 0, st, a, (int)n_strips, (int)n_ck, (int)rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return in_place ? launch_states<IO>(a, st) : hipSuccess;
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t st) {
  return a.bf16 ? launch<IoBf16>(a, st) : launch<IoF32>(a, st);
}

hipError_t launch_conv_states(const ConvArgs& a, hipStream_t st) {
  return a.bf16 ? launch_states<IoBf16>(a, st) : launch_states<IoF32>(a, st);
}

}  // namespace gdn
