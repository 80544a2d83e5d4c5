// Device helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------- bf16 --
// bf16 is handled as raw uint16 bit patterns: widening is a shift, narrowing
// rounds to nearest with ties to even (inputs are finite).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Element type tags for the io dtype.
struct IoBf16 { using T = uint16_t; static constexpr int kBytes = 2; };
struct IoF32 { using T = float; static constexpr int kBytes = 4; };

// Load 4 consecutive io elements (8-byte aligned for bf16, 16 for fp32) as fp32.
template <typename IO>
__device__ __forceinline__ void load4(const typename IO::T* p, float* out);
template <>
__device__ __forceinline__ void load4<IoBf16>(const uint16_t* p, float* out) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(w.x << 16);
  out[1] = __uint_as_float(w.x & 0xFFFF0000u);
  out[2] = __uint_as_float(w.y << 16);
  out[3] = __uint_as_float(w.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load4<IoF32>(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
}

template <typename IO>
__device__ __forceinline__ float load1(const typename IO::T* p);
template <>
__device__ __forceinline__ float load1<IoBf16>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load1<IoF32>(const float* p) { return *p; }

template <typename IO>
__device__ __forceinline__ void store1(typename IO::T* p, float x);
template <>
__device__ __forceinline__ void store1<IoBf16>(uint16_t* p, float x) { *p = (uint16_t)f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store1<IoF32>(float* p, float x) { *p = x; }

// Store 4 fp32 values as 4 consecutive io elements (bf16: nearest even).
template <typename IO>
__device__ __forceinline__ void store4(typename IO::T* p, const float* v);
template <>
__device__ __forceinline__ void store4<IoBf16>(uint16_t* p, const float* v) {
  uint2 w;
  w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<IoF32>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// 16 consecutive fp32 values, 16-byte aligned.
__device__ __forceinline__ void load16f(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = reinterpret_cast<const float4*>(p)[i];
    out[4 * i] = a.x; out[4 * i + 1] = a.y; out[4 * i + 2] = a.z; out[4 * i + 3] = a.w;
  }
}
__device__ __forceinline__ void store16f(float* p, const float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// ------------------------------------------------------------- conv --
// The width-4 causal depthwise conv + SiLU of one channel, in one operation
// order everywhere it is computed, so every kernel gives the same bits.  The
// taps arrive scaled by -log2(e) (conv_tap; w3 on the current input), x0..x3
// are the inputs oldest first.  With z' = -log2(e) z,
//   silu(z) = z / (1 + e^-z) = z' / (-log2(e) (1 + 2^z')),
// evaluated with the hardware exp2 and reciprocal (about 1 ulp each, below
// the bf16 output rounding); large |z| saturates to z or -0.
constexpr float kNegLog2e = -1.44269504088896341f;
__device__ __forceinline__ float conv_tap(float w) { return w * kNegLog2e; }
__device__ __forceinline__ float conv4_silu(float w0, float w1, float w2, float w3, float x0, float x1,
                                            float x2, float x3) {
  float zs = w0 * x0;
  zs = fmaf(w1, x1, zs);
  zs = fmaf(w2, x2, zs);
  zs = fmaf(w3, x3, zs);
  return zs * __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(zs), kNegLog2e, kNegLog2e));
}

// fp32 -> bf16 -> fp32 (nearest even), the value a bf16 store would hold.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// ------------------------------------------------------- lane reductions --
// Lane exchange inside a row of 16 lanes (DPP, no LDS round trip).
// x read from another lane of its row by DPP control CTRL.  Only in-row
// permutations are used (every source lane exists), so the bound_ctrl bit,
// set here so that the compiler folds the move into the consuming add,
// changes no value.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 16):
// pairs, then quads (quad_perm), then the two quads of a half-row
// (row_half_mirror), then the two halves of a row (row_mirror).  Each step
// adds a value equal on both partners, so every lane of the group ends with
// the same bits.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (W >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
  if constexpr (W >= 16) x += dpp_f32<0x140>(x); // row_mirror
  return x;
}

// First index i in [0, n) with a[i] >= key (n when none); a ascending.
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Index s of the sequence holding token p: cu[s] <= p < cu[s+1] (n_seqs >= 1,
// empty sequences skipped).  cu ascending, cu[0] = 0, p < cu[n_seqs].
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int n_seqs, int p) {
  int lo = 0, hi = n_seqs;  // invariant: cu[lo] <= p < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// The same search for a block-uniform p, through the constant address space:
// the compiler reads cu with scalar loads, which do not queue behind the
// block's vector loads in flight.
__device__ __forceinline__ int seq_of_token_uniform(const int32_t* cu_ptr, int n_seqs, int p) {
  typedef const int32_t __attribute__((address_space(4)))* ConstI32;
  const ConstI32 cu = (ConstI32)cu_ptr;
  int lo = 0, hi = n_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace gdn
