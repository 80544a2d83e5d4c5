// Chunked gated-delta-rule prefill on gfx950 MFMA (bf16 io).
//
// One workgroup owns one (prompt, value head) and walks the prompt's chunks
// in order; the chunk grid starts at the prompt's first token, so a prompt's
// arithmetic is the same alone or packed.  Per chunk of C tokens with entry
// state S0 (dv x dk), G = chunk-local cumsum of the log-gates, r = 1/|.|:
//   A   = strict_tril(beta_t r_t r_i e^{G_t-G_i} (k_t . k_i)),  T = (I + A)^-1
//   U   = T diag(beta) [V - diag(r e^G) K S0^T]                (WY/UT form)
//   O   = scale [diag(r_q e^G) Q S0^T + (tril(r_q r_k e^{G_t-G_i}) o Q K^T) U]
//   S_C = e^{G_C} S0 + K^T diag(r_k e^{G_C-G}) U
// (Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length", NeurIPS 2024, UT transform; gated as in Gated Delta
// Networks, ICLR 2025.)  The L2 norms enter only as fp32 row scalings, so the
// raw q/k rows are exact MFMA operands.
//
// Work split (DV/32 waves): all waves stage K and Q of the chunk in LDS and
// share the Gram / Q K^T tiles and the inversion of the 32x32 diagonal block
// of (I + A) (forward substitution, several lanes per column).  Wave w owns
// state columns v in [32w, 32w+32): its slice of S stays in MFMA accumulator
// registers for the whole prompt (fp32), laid out as S^T tiles (rows k, lane
// column v).  LDS is kept under 80 KB and registers under 256 so two
// workgroups share a CU and overlap each other's latency-bound phases.
//
// Precision: every product runs on fp16 operands with fp32 accumulation.
// The raw bf16 q/k rows convert to fp16 exactly (fp16 carries three more
// significand bits) while a row's sum of squares lies in [kQkLo, kQkHi];
// a row outside is scaled by a power of two first and its row factor
// carries the inverse.  Values the kernel computes in fp32 (S0, T, P, Y, U)
// are rounded to fp16 once per product (2^-11 relative), which holds states
// to about 4e-4 relative Frobenius against fp64 over thousands of tokens,
// with or without decay; the state itself is accumulated and carried in
// fp32, each wave's columns as 2^E S with E chosen per chunk from the
// largest |S| and |v| (kBand), so both stay well inside fp16's range.
//
// Chunks follow ChunkWalk: up to a.chunk tokens from the prompt's first
// token, cut at every checkpoint, so any checkpoint position works and a
// run resumed from a checkpoint walks the unbroken run's chunks.
#pragma once

#include <climits>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace chunked {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x16) B(16x32) on fp16 operands.  Lane l: A row l%32 and B
// column l%32, with eight k values each; D register i holds row
// 8(i/4) + 4(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mma(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// MFMA operand from an fp16 row in LDS.  The k order used by every product:
// within a 16-wide k step at offset 16*h2, lane half g (= l/32) holds
// k = 16*h2 + 4g + {0,1,2,3} and 16*h2 + 8 + 4g + {0,1,2,3}; this is exactly
// the row order of accumulator registers 8*h2 .. 8*h2+7, so an accumulator
// tile feeds the next product as its B operand without moving data.
// `p` points at element 16*h2 + 4g of the row (8-byte aligned).
__device__ __forceinline__ f16x8 lds_op(const uint16_t* p) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
  const u32x4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(f16x8, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, f16x2));
}

// Four fp16 values by an LDS transpose read (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane l names an 8-byte piece P_l (4 elements);
// lane i receives element i % 4 of P_{i/4}, P_{i/4+4}, P_{i/4+8}, P_{i/4+12}
// (lane layout checked on the GPU with an in-bounds probe).  With lane
// 4j + r naming columns 4r .. 4r+3 of row j of a row-major tile, lane i gets
// column i of rows 0..3: a 16-column x 4-row block, transposed.
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 LdsS16x4;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4*)p));
}

// Accumulator half h2 (registers 8h2..8h2+7) as a B operand.
template <int H2>
__device__ __forceinline__ f16x8 acc_half(const f32x16& x) {
  const u32x4 w = {pack_f16(x[8 * H2], x[8 * H2 + 1]), pack_f16(x[8 * H2 + 2], x[8 * H2 + 3]),
                   pack_f16(x[8 * H2 + 4], x[8 * H2 + 5]), pack_f16(x[8 * H2 + 6], x[8 * H2 + 7])};
  return __builtin_bit_cast(f16x8, w);
}

// Four bf16 values (an 8-byte row piece) as four fp16 values, exact inside
// fp16's range; ss gets their sum of squares.
__device__ __forceinline__ u32x2 bf16x4_to_f16(const u32x2& w, float& ss) {
  const float x0 = __uint_as_float(w.x << 16), x1 = __uint_as_float(w.x & 0xFFFF0000u);
  const float x2 = __uint_as_float(w.y << 16), x3 = __uint_as_float(w.y & 0xFFFF0000u);
  ss = fmaf(x3, x3, fmaf(x2, x2, fmaf(x1, x1, x0 * x0)));
  return u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
}

// 2^x on the hardware exp2 (v_exp_f32, about 1 ulp); decays are kept in
// base 2 so that none needs a multiply first.
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Total over an aligned group of W lanes (8, 16 or 32), exact in the group's
// last lane (for 32: the 16-lane sums, then the lower row's total added into
// the upper row by row_bcast:15), in a fixed order.
template <int W>
__device__ __forceinline__ float lane_group_total(float x) {
  if constexpr (W <= 16) {
    return group_sum<W>(x);
  } else {
    x = group_sum<16>(x);
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142,
                                                                      0xA, 0xF, false));
  }
}

// Inclusive prefix sum over lanes 0..31 (each 16-lane row by shifts of 1, 2,
// 4, 8, then row 0's total into row 1); a fixed order on every call.
__device__ __forceinline__ float scan32(float x) {
  auto shr = [](float v, auto ctrl) {   // lanes shifted in from outside the row read 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x += shr(x, std::integral_constant<int, 0x111>{});   // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});   // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});   // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});   // row_shr:8
  // row_bcast:15 into rows 1 and 3 (lane 15 of the row below)
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
  return x;
}

// Lane q of each aligned group of W lanes (W = 1, 2 or 4) to the whole group.
template <int W, int Q>
__device__ __forceinline__ float group_bcast(float x) {
  if constexpr (W == 1 || Q >= W) return x;   // Q >= W: never selected
  else {
    constexpr int s0 = Q, s1 = W == 4 ? Q : Q, s2 = W == 4 ? Q : 2 + Q, s3 = W == 4 ? Q : 2 + Q;
    constexpr int ctrl = s0 | (s1 << 2) | (s2 << 4) | (s3 << 6);   // quad_perm
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xF, 0xF, false));
  }
}


__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ------------------------------------------------- fp16 operand range --
// fp16 holds normal values from 2^-14 to 65504 with 11 significand bits.
// Rows of q and k whose sum of squares lies in [kQkLo, kQkHi] convert as
// they are (exactly, from bf16); a row outside is first scaled by 2^a, a
// power of two that brings its largest element into [1, 2), and its row
// factor (1/|x| with the L2 norm, else 1) carries 2^-a, so every product of
// the scan sees the same value.  The band keeps 1/|x| <= 4, which bounds the
// update operands r_k e^{G_C - G} U.
constexpr float kQkLo = 0x1p-4f, kQkHi = 0x1p20f;
// The state columns of a wave are held as 2^E S: E = 0 while the largest
// |S| entry and the chunk's largest |v| both have a binary exponent in
// [-kBand, kBand]; otherwise E brings the larger of the two into [1, 2).
// E is a function of the unscaled values, so a run resumed from a
// checkpoint takes the same E as the unbroken run, and scaling by powers of
// two is exact: results stay bit-identical.
constexpr int kBand = 6;
constexpr int kNoExp = -1024;   // exponent of an all-zero set

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running maxima of bf16 magnitudes: m holds two 16-bit maxima, w two bf16
// values (the sign bit cleared, bf16 bits order like their magnitudes).
__device__ __forceinline__ uint32_t bf16_absmax(uint32_t m, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu)));
}
__device__ __forceinline__ uint32_t fold16(uint32_t m) { return max(m & 0xFFFFu, m >> 16); }

// Maximum over aligned groups of W lanes (W a power of two <= 16), every
// lane of a group ending with it.
template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t x) {
  auto dpp = [](uint32_t v, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctrl)::value, 0xF, 0xF, true);
  };
  if constexpr (W >= 2) x = max(x, dpp(x, std::integral_constant<int, 0xB1>{}));
  if constexpr (W >= 4) x = max(x, dpp(x, std::integral_constant<int, 0x4E>{}));
  if constexpr (W >= 8) x = max(x, dpp(x, std::integral_constant<int, 0x141>{}));
  if constexpr (W >= 16) x = max(x, dpp(x, std::integral_constant<int, 0x140>{}));
  return x;
}

// Maximum over the whole wave, returned as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = group_max_u32<16>(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = max(s32[0], s32[1]);
  const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __builtin_amdgcn_readfirstlane(max(s16[0], s16[1]));
}

// Binary exponent of a bf16 magnitude (bits without the sign), kNoExp for 0.
__device__ __forceinline__ int bf16_exp(uint32_t m) { return m ? (int)(m >> 7) - 127 : kNoExp; }
// Binary exponent of a non-negative fp32 value, kNoExp for 0.
__device__ __forceinline__ int f32_exp(float x) {
  return x > 0.f ? (int)((__float_as_uint(x) >> 23) & 0xFFu) - 127 : kNoExp;
}
// The state scale exponent for a largest binary exponent M.
__device__ __forceinline__ int band_exp(int M) { return (M > kNoExp && (M > kBand || M < -kBand)) ? -M : 0; }

// Four bf16 values scaled by 2^a into four fp16 values; ss gets the squares
// of the scaled values, summed in the order bf16x4_to_f16 uses (a = 0 gives
// its bits).
__device__ __forceinline__ u32x2 bf16x4_to_f16_exp(const u32x2& w, int a, float& ss) {
  const float x0 = __builtin_amdgcn_ldexpf(__uint_as_float(w.x << 16), a);
  const float x1 = __builtin_amdgcn_ldexpf(__uint_as_float(w.x & 0xFFFF0000u), a);
  const float x2 = __builtin_amdgcn_ldexpf(__uint_as_float(w.y << 16), a);
  const float x3 = __builtin_amdgcn_ldexpf(__uint_as_float(w.y & 0xFFFF0000u), a);
  ss = fmaf(x3, x3, fmaf(x2, x2, fmaf(x1, x1, x0 * x0)));
  return u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
}

// Row factor of a q/k row scaled by 2^a whose scaled squares sum to ss.
__device__ __forceinline__ float row_factor(bool l2norm, float ss, int a, float eps) {
  return l2norm ? __builtin_amdgcn_rsqf(ss + __builtin_amdgcn_ldexpf(eps, 2 * a))
                : __builtin_amdgcn_ldexpf(1.0f, -a);
}

// ---------------------------------------------------------- chunk walk --
// A prompt [seq0, seq1) is cut into chunks of up to CT tokens from its first
// token; a chunk also ends at every checkpoint inside the prompt and the
// next one starts there.  A run resumed from a checkpoint therefore walks
// the same chunks as the unbroken run from that point on, and a prompt's
// chunks do not depend on the rest of the pack.  The walk is uniform over a
// workgroup; positions come in by scalar loads.
typedef const int32_t __attribute__((address_space(4)))* ConstI32;

struct ChunkWalk {
  int pos, end, ci, nck;   // next chunk's first token, prompt end, next checkpoint (index, position)
  __device__ void init(int seq0, int seq1, int ci0, ConstI32 ck, int n_ck) {
    pos = seq0;
    end = seq1;
    ci = ci0;
    nck = ci0 < n_ck ? ck[ci0] : INT_MAX;
  }
  // The next chunk: its first token in t0, its length returned; ck_at is the
  // index of the checkpoint it ends on, or -1.
  __device__ int next(int CT, ConstI32 ck, int n_ck, int& t0, int& ck_at) {
    t0 = pos;
    int stop = min(pos + CT, end);
    ck_at = -1;
    if (nck <= stop) {
      stop = nck;
      ck_at = ci;
      ++ci;
      nck = ci < n_ck ? ck[ci] : INT_MAX;
    }
    pos = stop;
    return stop - t0;
  }
};

// Number of chunks of the walk above, from the prompt's checkpoints.
__device__ __forceinline__ int count_chunks(int seq0, int seq1, int ci0, ConstI32 ck, int n_ck, int CT) {
  int n = 0, p = seq0;
  for (int i = ci0; i < n_ck; ++i) {
    const int c = ck[i];
    if (c >= seq1) break;
    n += (c - p + CT - 1) / CT;
    p = c;
  }
  return n + (seq1 - p + CT - 1) / CT;
}

// Two fp32 values as packed bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, b2));
}


template <int DK, int DV>
struct Cfg {
  static constexpr int CT = 32;           // tokens per chunk tile
  static constexpr int NW = DV / 32;      // waves
  static constexpr int NTH = 64 * NW;     // threads
  static constexpr int KT = DK / 32;      // 32-wide k tiles of the state
  static constexpr int LDK = DK + 12;     // row stride of sK, sQ (fp16; 8-byte aligned rows)
  static constexpr int LDT = CT + 4;      // row stride of sT, sP (fp16)
  static constexpr int LDV = DV + 24;     // row stride of the V / O tile (bf16; 16-byte rows)
  static constexpr int LDA = CT + 4;      // row stride of sA, A transposed (fp32)
  // With four waves, waves 2 and 3 run the substitution while waves 0 and 1
  // form their K S0^T and Q S0^T (waves 2 and 3 formed theirs during the
  // Gram stage); with fewer, every wave forms them after the substitution.
  static constexpr bool SPLIT = NW >= 4;
  static constexpr int SUB0 = SPLIT ? 128 : 0;       // first substitution thread
  static constexpr int SUBT = SPLIT ? 128 : NTH;     // substitution threads available
  // forward substitution: LPC lanes per column of T
  static constexpr int LPC_RAW = SUBT / CT;
  static constexpr int LPC = LPC_RAW > 4 ? 4 : (LPC_RAW < 1 ? 1 : LPC_RAW);
  static constexpr int MPL = CT / LPC;    // rows of a column held per lane
  static constexpr int oK = 0;
  static constexpr int oQ = oK + CT * LDK * 2;
  static constexpr int oV = oQ + CT * LDK * 2;        // V tile, then the O tile
  static constexpr int oT = oV + CT * LDV * 2;
  static constexpr int oP = oT + CT * LDT * 2;
  static constexpr int oA = oP + CT * LDT * 2;
  static constexpr int oS = oA + CT * LDA * 4;        // per-token scalars
  static constexpr int kScal = 12;
  static constexpr int bytes = oS + kScal * CT * 4;
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
  static_assert(NW <= 4 && LPC * CT <= SUBT, "wave roles");
  static_assert(oQ % 16 == 0 && oV % 16 == 0 && oT % 16 == 0 && oA % 16 == 0, "align");
  // the next chunk's rows wait in registers (16-byte vectors per thread)
  // while this chunk computes, when they fit in 32 registers
  // K and Q come in cells of 4 tokens x 4 key dims (four 8-byte row pieces),
  // V in 16-byte row pieces
  static constexpr int KC = DK / 4;                    // cells across a row
  static constexpr int NCK = (CT / 4 * KC + NTH - 1) / NTH;
  static constexpr int NVV = (CT * DV / 8 + NTH - 1) / NTH;
  static constexpr bool PREFETCH = NCK * 16 + NVV * 4 <= 32;
};

// per-token scalar arrays (index into the scalar block)
// (SC_VM: the chunk's largest |v| as bf16 bits, one word per staging wave)
enum { SC_G = 0, SC_BETA, SC_RK, SC_RQ, SC_CK, SC_CQ, SC_CU, SC_LA, SC_LK0, SC_LQ, SC_LK1, SC_VM };

template <int DK, int DV>
__global__ void __launch_bounds__(64 * (DV / 32), 2)
chunked_prefill_kernel(const ScanArgs a) {
  using C = Cfg<DK, DV>;
  constexpr int CT = C::CT, NTH = C::NTH, KT = C::KT, LDK = C::LDK, LDT = C::LDT;
  constexpr int LDA = C::LDA, LPC = C::LPC, MPL = C::MPL, LDV = C::LDV;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + C::oK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + C::oQ);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + C::oV);
  uint16_t* sT = reinterpret_cast<uint16_t*>(smem + C::oT);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + C::oP);
  float* sA = reinterpret_cast<float*>(smem + C::oA);
  float* sc = reinterpret_cast<float*>(smem + C::oS);
  float* sG = sc + SC_G * CT;       // cumsum of the log-gates, times log2(e)
  float* sBeta = sc + SC_BETA * CT;
  float* sRk = sc + SC_RK * CT;
  float* sRq = sc + SC_RQ * CT;
  float* sCk = sc + SC_CK * CT;     // r_k e^G
  float* sCq = sc + SC_CQ * CT;     // scale r_q e^G
  float* sCu = sc + SC_CU * CT;     // r_k e^{G_C - G}
  // base-2 exponents of the Gram and K Q^T factors: beta_t r_t r_i e^{G_t-G_i}
  // = 2^(LA_t - LK_i) and r_q,t r_k,i e^{G_t-G_i} = 2^(LQ_t - LK_i), with
  // LA = G + log2(beta r_k), LQ = G + log2(r_q), LK = G - log2(r_k) (G in
  // base 2); one copy of LK per role wave
  float* sLA = sc + SC_LA * CT;
  float* sLK0 = sc + SC_LK0 * CT;
  float* sLQ = sc + SC_LQ * CT;
  float* sLK1 = sc + SC_LK1 * CT;

  const int s = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int j = h / (a.Hv / a.Hqk);
  const int seq0 = a.cu[s], seq1 = a.cu[s + 1];
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)h * DV;
  uint16_t* og = static_cast<uint16_t*>(a.out) + (size_t)h * DV;
  const size_t sstride = (size_t)a.Hv * DV * DK;
  const int v = 32 * wave + c;       // this lane's state column (value dim)
  // K^T operands of the state update come from the row-major K tile by
  // transpose reads: the lanes of 16-lane group grp cover key columns
  // 16 (grp % 2) .. +15 of a 32-column tile and tokens 4 (grp / 2) + j; lane
  // 4j + r names the 4-column piece r of token row j
  const int grp = lane >> 4, li = lane & 15;
  const uint16_t* ktr = sK + (4 * (grp >> 1) + (li >> 2)) * LDK + 16 * (grp & 1) + 4 * (li & 3);

  // ---- state slice S^T[k][v] for v in this wave's 32 columns
  f32x16 S[KT];
  {
    const float* src = a.init ? a.init + (size_t)s * sstride + ((size_t)h * DV + v) * DK : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (src) x = *reinterpret_cast<const float4*>(src + 32 * kt + 8 * q4 + 4 * g);
        S[kt][4 * q4 + 0] = x.x; S[kt][4 * q4 + 1] = x.y;
        S[kt][4 * q4 + 2] = x.z; S[kt][4 * q4 + 3] = x.w;
      }
    }
  }
  // each wave holds 2^E S (E wave-uniform, 0 unless the state or the values
  // left the band: kBand); stores give S itself, exactly
  int E = 0;
  auto store_state = [&](float* dst) {
    auto un = [&](float x) { return E == 0 ? x : __builtin_amdgcn_ldexpf(x, -E); };
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(dst + 32 * kt + 8 * q4 + 4 * g) =
            make_float4(un(S[kt][4 * q4]), un(S[kt][4 * q4 + 1]), un(S[kt][4 * q4 + 2]), un(S[kt][4 * q4 + 3]));
  };

  // the prompt's chunks (ChunkWalk): cwalk for the chunk being computed,
  // pwalk one chunk ahead for the prefetch; checkpoint positions come in by
  // scalar loads, which never wait behind the vector loads in flight
  const ConstI32 ckp = (ConstI32)a.ckpt;
  const int ci0 = __builtin_amdgcn_readfirstlane(lower_bound_i32(a.ckpt, a.n_ckpt, seq0 + 1));
  ChunkWalk cwalk, pwalk;
  cwalk.init(seq0, seq1, ci0, ckp, a.n_ckpt);
  pwalk.init(seq0, seq1, ci0, ckp, a.n_ckpt);

  // One chunk's HBM rows into registers.  Every lane loads (row index clamped
  // into the chunk, so no load is conditional); rows past the chunk's end are
  // zeroed where they are consumed.
  // A row address is a workgroup-uniform base at the chunk's first token
  // plus a 32-bit byte offset per lane: token strides are below 2^23
  // elements, so the offsets of a chunk's rows come from 24-bit multiplies.
  const uint32_t ksb = (uint32_t)a.k_stride * 2, qsb = (uint32_t)a.q_stride * 2;
  const uint32_t vsb = (uint32_t)a.v_stride * 2, hv = (uint32_t)a.Hv;
  auto row = [](const void* base, uint32_t off) { return static_cast<const char*>(base) + off; };
  struct Cell { u32x2 k[4], q[4]; };   // rows 4 tg + r, key dims 4 kc .. 4 kc + 3
  auto ld_kq = [&](int u, int t0x, int nx, Cell& x) {
    const int e = min(tid + u * NTH, CT / 4 * C::KC - 1);
    const int tg = e / C::KC, kc = e % C::KC;
    const uint16_t* kb = kg + (size_t)t0x * a.k_stride + (size_t)j * DK;
    const uint16_t* qb = qg + (size_t)t0x * a.q_stride + (size_t)j * DK;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t t = min(4 * tg + r, nx - 1);
      x.k[r] = *reinterpret_cast<const u32x2*>(row(kb, __umul24(t, ksb) + 8 * kc));
      x.q[r] = *reinterpret_cast<const u32x2*>(row(qb, __umul24(t, qsb) + 8 * kc));
    }
  };
  auto ld_v = [&](int u, int t0x, int nx, u32x4& vx) {
    const int e = min(tid + u * NTH, CT * DV / 8 - 1);
    const uint32_t t = min(e / (DV / 8), nx - 1), c8 = (e % (DV / 8)) * 8;
    vx = *reinterpret_cast<const u32x4*>(row(vg + (size_t)t0x * a.v_stride, __umul24(t, vsb) + 2 * c8));
  };
  auto ld_gb = [&](int t0x, int nx, float& gx, float& bx) {
    const uint32_t tl = min(lane, nx - 1);
    gx = a.g[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
    bx = a.beta[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
  };
  // with PREFETCH the rows of the next chunk are held here between chunks;
  // otherwise each vector is loaded where it is consumed
  constexpr int NPK = C::PREFETCH ? C::NCK : 1, NPV = C::PREFETCH ? C::NVV : 1;
  Cell pkq[NPK];
  u32x4 pv[NPV];
  float pg, pb;
  auto fetch = [&](int t0x, int nx) {
#pragma unroll
    for (int u = 0; u < NPK; ++u) ld_kq(u, t0x, nx, pkq[u]);
#pragma unroll
    for (int u = 0; u < NPV; ++u) ld_v(u, t0x, nx, pv[u]);
    ld_gb(t0x, nx, pg, pb);
  };
  int pf_t0 = seq0, pf_n = 0;   // the prefetched chunk
  if constexpr (C::PREFETCH)
    if (seq1 > seq0) {
      int ck_at;
      pf_n = pwalk.next(a.chunk, ckp, a.n_ckpt, pf_t0, ck_at);
      fetch(pf_t0, pf_n);
    }
  // drain the state and first-chunk loads here, so that no wait inside the
  // chunk loop has to cover them (vmcnt(0); expcnt, lgkmcnt unchanged)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Operands of a chain over the full key dimension: with several waves
  // every row operand is read before the MFMA chain starts (registers are
  // free then); a single wave holds more live state, so it reads them as it
  // goes.
  constexpr bool PRE = C::NW > 1;
  constexpr int NKS = PRE ? DK / 16 : 1;

  // X = K S0^T (rows t, lane column v) and QS = S0 Q^T (rows v, lane column
  // t: the output tile comes out transposed, one token per lane) for this
  // wave's columns, S0 rounded to fp16 per k tile on the fly; an
  // accumulator half serves as the A operand (row v) as well as the B
  // operand (column v)
  auto xqs = [&](f32x16& X, f32x16& QS) {
    // the scale of this chunk, from the largest |S| entry of the wave's
    // columns (unscaled: 2^-E times the held value) and the chunk's largest
    // |v| (recorded at staging, one word per wave)
    {
      float ms = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ms = fmaxf(ms, fabsf(S[kt][i]));
      const int eS = f32_exp(__uint_as_float(wave_max_u32(__float_as_uint(ms))));
      uint32_t vm = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) vm = max(vm, reinterpret_cast<const uint32_t*>(sc)[SC_VM * CT + w]);
      const int eV = bf16_exp(__builtin_amdgcn_readfirstlane(vm));
      const int En = band_exp(max(eS == kNoExp ? kNoExp : eS - E, eV));
      if (En != E) {   // rare: rescale the held state (powers of two, exact)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kt][i] = __builtin_amdgcn_ldexpf(S[kt][i], En - E);
        E = En;
      }
    }
    f16x8 ka[NKS], qa[NKS];
    auto ld = [&](int ks, f16x8& kx, f16x8& qx) {
      const int off = c * LDK + 4 * g + 16 * ks;
      kx = lds_op(sK + off);
      qx = lds_op(sQ + off);
    };
    if constexpr (PRE)
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) ld(ks, ka[ks], qa[ks]);
    X = f32x16{};
    QS = f32x16{};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int ks = 2 * kt + h2;
        if constexpr (!PRE) ld(ks, ka[0], qa[0]);
        const f16x8& kx = ka[PRE ? ks : 0];
        const f16x8& qx = qa[PRE ? ks : 0];
        const f16x8 sh = h2 == 0 ? acc_half<0>(S[kt]) : acc_half<1>(S[kt]);
        X = mma(kx, sh, X);
        QS = mma(sh, qx, QS);
      }
    // S0 has served both products: the chunk's decay e^{G_C} goes on here,
    // in the slack of this wave's stage, rather than in the state path
    const float gC = exp2f_hw(sG[CT - 1]);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[kt][i] *= gC;
  };

  // Gram-type tile: sum over k of (row c of xa) (row c of xb), the A operand
  // rows giving the accumulator rows and the B operand rows its columns
  auto rows_mm = [&](const uint16_t* xa, const uint16_t* xb) {
    f16x8 ar[NKS], br[NKS];
    if constexpr (PRE)
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) {
        ar[ks] = lds_op(xa + c * LDK + 4 * g + 16 * ks);
        br[ks] = lds_op(xb + c * LDK + 4 * g + 16 * ks);
      }
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      if constexpr (!PRE) {
        ar[0] = lds_op(xa + c * LDK + 4 * g + 16 * ks);
        br[0] = lds_op(xb + c * LDK + 4 * g + 16 * ks);
      }
      acc = mma(ar[PRE ? ks : 0], br[PRE ? ks : 0], acc);
    }
    return acc;
  };

  int pt0 = 0, pn = 0;   // previous chunk: its O rows are still in the V/O tile
  for (;;) {
    int t0, ck_at;
    const int n = cwalk.next(a.chunk, ckp, a.n_ckpt, t0, ck_at);   // valid rows of this chunk
    if (n <= 0) break;

    // ---- 1. stage K and Q rows as fp16 (zero past n) with their L2 norms (squares summed in registers, then over
    //         the row's lanes), V rows, betas and the gate cumsum.  The rows
    //         were fetched into registers while the previous chunk ran.  The
    //         previous chunk's O rows leave the V/O tile first: read into
    //         registers before V lands, stored to HBM after.
    if constexpr (!C::PREFETCH) ld_gb(t0, n, pg, pb);
    {
      // a cell: four 8-byte row pieces of K and of Q, converted to fp16.
      // A token's squares are summed over its KC lanes (a fixed-order DPP sum
      // ending in the group's last lane).
      constexpr int KC = C::KC;
      static_assert(KC == 8 || KC == 16 || KC == 32, "cell lanes");
      static_assert(NTH % KC == 0, "cell rows");
#pragma unroll
      for (int u = 0; u < C::NCK; ++u) {
        const int e = tid + u * NTH;
        if (e < CT / 4 * KC) {             // whole lane groups per trip
          const int tg = e / KC, kc = e % KC;
          Cell x;
          if constexpr (C::PREFETCH) x = pkq[u]; else ld_kq(u, t0, n, x);
          const u32x2 z = {0u, 0u};
          float sk[4], sq[4];
          if (n < CT)   // a prompt's last chunk (uniform branch): rows past n are zeros
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * tg + r >= n) { x.k[r] = z; x.q[r] = z; }
          // rows converted as they are; a tile whose rows stray from unit
          // length (rare) is converted again with each such row scaled by
          // 2^a, its largest element brought into [1, 2) (kQkLo, kQkHi)
          auto convert = [&](const u32x2 (&xr)[4], uint16_t* dst, const int (&ax)[4], float (&ss)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const u32x2 f = bf16x4_to_f16_exp(xr[r], ax[r], ss[r]);
              *reinterpret_cast<u32x2*>(dst + (4 * tg + r) * LDK + 4 * kc) = f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) ss[r] = lane_group_total<KC>(ss[r]);
          };
          // whether row r strays (exact in the group's last lane)
          auto strays = [&](const float (&ss)[4]) {
            bool any = false;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              any |= kc == KC - 1 && 4 * tg + r < n && !(ss[r] >= kQkLo && ss[r] <= kQkHi);
            return any;
          };
          auto rescale = [&](const u32x2 (&xr)[4], uint16_t* dst, int (&ax)[4], float (&ss)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              uint32_t m = fold16(bf16_absmax(bf16_absmax(0u, xr[r].x), xr[r].y));
              m = group_max_u32<KC <= 16 ? KC : 16>(m);
              if constexpr (KC == 32) {   // the two 16-lane rows of a group
                const auto sw = __builtin_amdgcn_permlane16_swap(m, m, false, false);
                m = max(sw[0], sw[1]);
              }
              // the row's verdict, from its group's last lane
              const float tot = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                  4 * ((lane | (KC - 1))), __builtin_bit_cast(int, ss[r])));
              const bool ok = tot >= kQkLo && tot <= kQkHi;
              ax[r] = (ok || m == 0 || 4 * tg + r >= n) ? 0 : -bf16_exp(m);
            }
            convert(xr, dst, ax, ss);
          };
          int ak[4] = {0, 0, 0, 0}, aq[4] = {0, 0, 0, 0};
          convert(x.k, sK, ak, sk);
          convert(x.q, sQ, aq, sq);
          if (__builtin_amdgcn_ballot_w64(strays(sk))) rescale(x.k, sK, ak, sk);
          if (__builtin_amdgcn_ballot_w64(strays(sq))) rescale(x.q, sQ, aq, sq);
          if (kc == KC - 1) {   // zero-padded rows past n keep r = 1 (no 0 * inf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 4 * tg + r;
              sRk[t] = t < n ? row_factor(a.l2norm, sk[r], ak[r], a.eps) : 1.0f;
              sRq[t] = t < n ? row_factor(a.l2norm, sq[r], aq[r], a.eps) : 1.0f;
            }
          }
        }
      }
    }
    {
      // a thread owns the same 16-byte segments of the V/O tile for both
      u32x4 ov[C::NVV];
      uint32_t vm = 0;   // the chunk's largest |v| (bf16 bits)
#pragma unroll
      for (int u = 0; u < C::NVV; ++u) {
        const int e = tid + u * NTH;
        if (e < CT * DV / 8) {
          const int t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
          u32x4* seg = reinterpret_cast<u32x4*>(sV + t * LDV + c8);
          u32x4 vx;
          if constexpr (C::PREFETCH) vx = pv[u]; else ld_v(u, t0, n, vx);
          ov[u] = *seg;
          if (n < CT && t >= n) vx = u32x4{0u, 0u, 0u, 0u};
          *seg = vx;
#pragma unroll
          for (int i = 0; i < 4; ++i) vm = bf16_absmax(vm, vx[i]);
        }
      }
      vm = wave_max_u32(fold16(vm));
      if (lane == 0) reinterpret_cast<uint32_t*>(sc)[SC_VM * CT + wave] = vm;
      if (wave == 0) {  // betas and the inclusive scan of the log-gates (fixed order),
                        // kept in base 2 so every decay is one v_exp_f32
        const float x = scan32(lane < n ? pg : 0.f) * 1.44269504088896341f;
        if (lane < CT) {
          sG[lane] = x;
          sBeta[lane] = lane < n ? pb : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < C::NVV; ++u) {
        const int e = tid + u * NTH;
        const uint32_t t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
        if (e < CT * DV / 8 && (int)t < pn)
          *reinterpret_cast<u32x4*>(const_cast<char*>(row(og + (size_t)pt0 * a.Hv * DV,
                                                          __umul24(t, hv * (2 * DV)) + 2 * c8))) = ov[u];
      }
    }
    __syncthreads();
    if constexpr (C::PREFETCH) {
      int ck_at2;
      pf_n = pwalk.next(a.chunk, ckp, a.n_ckpt, pf_t0, ck_at2);
      if (pf_n > 0) fetch(pf_t0, pf_n);
    }

    f32x16 X, QS;   // K S0^T, Q S0^T for this wave's columns
    // ---- 3. Gram tile -> A (wave 0), K Q^T tile -> P (wave 1), per-token
    //         scalars (wave 0); waves 2, 3 form their X and QS meanwhile.
    //         Row operands are read before each MFMA chain.
    if (wave == 0) {
      // Gram K K^T: both operands are the K rows (lane column = key i = c,
      // accumulator rows = token t); A[t][i] = beta_t r_t r_i e^{G_t - G_i} k_t.k_i
      // for i < t, stored transposed with rows interleaved over the LPC lane
      // parts of the substitution, each part's rows in descending order:
      // (t, i) at i*LDA + (t % LPC)*MPL + MPL - 1 - t / LPC.  The rows a
      // substitution step still needs are then an aligned prefix of the part.
      // (the exponents are formed while the MFMA chain runs; beta = 0 gives
      // LA = -inf and a zero factor; masked entries may overflow and are
      // replaced by the select)
      if (lane < CT) {
        const float G = sG[lane], lr = __builtin_amdgcn_logf(sRk[lane]);
        sLA[lane] = G + (__builtin_amdgcn_logf(sBeta[lane]) + lr);
        sLK0[lane] = G - lr;
      }
      const f32x16 acc = rows_mm(sK, sK);
      const float lki = sLK0[c];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int tb = 8 * q4 + 4 * g;
        const float4 L4 = *reinterpret_cast<const float4*>(sLA + tb);
        const float La[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tb + r;
          const float f = exp2f_hw(La[r] - lki) * acc[4 * q4 + r];
          sA[c * LDA + (t % LPC) * MPL + MPL - 1 - t / LPC] = c < t ? f : 0.f;
        }
      }
      if (lane < CT) {
        const float G = sG[lane], GC = sG[CT - 1];
        sCk[lane] = sRk[lane] * exp2f_hw(G);
        sCq[lane] = a.scale * sRq[lane] * exp2f_hw(G);
        sCu[lane] = sRk[lane] * exp2f_hw(GC - G);
      }
    }
    if (wave == (C::NW > 1 ? 1 : 0)) {
      // K Q^T: A operand = K rows (accumulator row = key i), B operand = Q
      // rows (lane column = query t = c); P[t][i] = scale r_q,t r_k,i
      // e^{G_t - G_i} q_t.k_i for i <= t, written as row t of P (fp16), four
      // keys per 8-byte store
      if (lane < CT) {
        const float G = sG[lane];
        sLQ[lane] = G + __builtin_amdgcn_logf(sRq[lane]);
        sLK1[lane] = G - __builtin_amdgcn_logf(sRk[lane]);
      }
      const f32x16 acc = rows_mm(sK, sQ);
      const float lqt = sLQ[c];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ib = 8 * q4 + 4 * g;
        const float4 L4 = *reinterpret_cast<const float4*>(sLK1 + ib);
        const float Lk[4] = {L4.x, L4.y, L4.z, L4.w};
        float pv4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float f = a.scale * exp2f_hw(lqt - Lk[r]) * acc[4 * q4 + r];
          pv4[r] = ib + r <= c ? f : 0.f;
        }
        *reinterpret_cast<u32x2*>(sP + c * LDT + ib) =
            u32x2{pack_f16(pv4[0], pv4[1]), pack_f16(pv4[2], pv4[3])};
      }
    }
    if constexpr (C::SPLIT)
      if (wave >= 2) xqs(X, QS);
    __syncthreads();

    // ---- 4. T = (I + A)^-1 by right-looking forward substitution: column jj
    //         of T is spread over LPC consecutive lanes, lane part q keeping
    //         rows q, q+LPC, ... as running sums delta(r, jj) - sum_{i<r}
    //         A[r][i] T[i][jj].  At step i the owner lane's sum for row i is
    //         final; it is broadcast to the group and every lane folds it into
    //         its later rows (A's zero upper part leaves finished rows alone).
    //         A is stored transposed, so the column read at step i is
    //         contiguous per lane part.
    if (tid >= C::SUB0 && tid < C::SUB0 + CT * LPC) {
      const int st = tid - C::SUB0;
      const int jj = st / LPC, q = st % LPC;
      const float* ab = sA + q * MPL;
      float Tl[MPL];
#pragma unroll
      for (int m = 0; m < MPL; ++m) Tl[m] = (q + LPC * m == jj) ? 1.f : 0.f;
      // columns of A come in batches of SB steps, one batch ahead of use, so
      // the LDS latency is not paid step by step
      constexpr int SB = MPL <= 8 ? 4 : (MPL == 16 ? 2 : 1), NB = CT / SB;   // SB * MPL <= 32
      float col[2][SB][MPL];
      auto load_batch = [&](float (&dst)[SB][MPL], int bt) {
#pragma unroll
        for (int u = 0; u < SB; ++u)
#pragma unroll
          for (int p4 = 0; p4 < MPL; p4 += 4) {   // part rows MPL-1-p4 .. MPL-4-p4
            const float4 x = *reinterpret_cast<const float4*>(ab + (SB * bt + u) * LDA + p4);
            dst[u][MPL - 1 - p4] = x.x; dst[u][MPL - 2 - p4] = x.y;
            dst[u][MPL - 3 - p4] = x.z; dst[u][MPL - 4 - p4] = x.w;
          }
      };
      load_batch(col[0], 0);
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        if (bt + 1 < NB) load_batch(col[(bt + 1) & 1], bt + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SB; ++u) {   // unrolled: t % LPC and t / LPC are constants
          const int t = SB * bt + u;
          if (t < CT - 1) {
            const float own = Tl[t / LPC];
            const int qt = t % LPC;
            const float Tt = qt == 0 ? group_bcast<LPC, 0>(own)
                           : qt == 1 ? group_bcast<LPC, 1>(own)
                           : qt == 2 ? group_bcast<LPC, 2>(own) : group_bcast<LPC, 3>(own);
#pragma unroll
            for (int m = t / LPC; m < MPL; ++m) Tl[m] = fmaf(-col[bt & 1][u][m], Tt, Tl[m]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      uint16_t* tcol = sT + jj;
#pragma unroll
      for (int m = 0; m < MPL; ++m) tcol[(q + LPC * m) * LDT] = f16_bits(Tl[m]);
    }
    if constexpr (C::SPLIT)
      if (wave < 2) xqs(X, QS);
    __syncthreads();

    // ---- 5. state path for this wave's 32 value columns
    if constexpr (!C::SPLIT) xqs(X, QS);
    {
      // the LDS operands of the stage are requested ahead of their use, so the
      // LDS round trips overlap: V of this wave's columns first, then the T
      // and P row operands and (with several waves) the K^T operands of the
      // update.  V comes by four transpose reads of the
      // row-major V tile (as the K^T operands do): lane (c, g) gets column v
      // of rows 8 q4 + 4 g .. +3, the accumulator rows of registers 4q4..4q4+3.
      const uint16_t* tr = sT + c * LDT + 4 * g;
      const uint16_t* pr = sP + c * LDT + 4 * g;
      float vv[16];
      {
        const uint16_t* vtr = sV + (4 * (grp >> 1) + (li >> 2)) * LDV + 32 * wave + 16 * (grp & 1) + 4 * (li & 3);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 w = lds_tr4(vtr + 8 * q4 * LDV);
          vv[4 * q4] = __uint_as_float(w.x << 16);
          vv[4 * q4 + 1] = __uint_as_float(w.x & 0xFFFF0000u);
          vv[4 * q4 + 2] = __uint_as_float(w.y << 16);
          vv[4 * q4 + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
        if (E != 0)
#pragma unroll
          for (int i = 0; i < 16; ++i) vv[i] = __builtin_amdgcn_ldexpf(vv[i], E);
      }
      __builtin_amdgcn_sched_barrier(0);
      const f16x8 tA[2] = {lds_op(tr), lds_op(tr + 16)};

      // Y = beta (V - r_k e^G X), in place of X.  Rows past n come out as
      // exact zeros: beta is 0 there, their V and K rows are zero (so X is)
      // and r_k e^G is finite.
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int tb = 8 * q4 + 4 * g;
        const float4 b4 = *reinterpret_cast<const float4*>(sBeta + tb);
        const float4 k4 = *reinterpret_cast<const float4*>(sCk + tb);
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) X[4 * q4 + r] = bb[r] * (vv[4 * q4 + r] - kk[r] * X[4 * q4 + r]);
      }
      const f16x8 pA[2] = {lds_op(pr), lds_op(pr + 16)};
      f16x8 kta[NKS];
      auto ldt = [&](int kt, int h2) {   // K^T rows 32 kt + c, tokens as in lds_op
        const uint16_t* p = ktr + 16 * h2 * LDK + 32 * kt;
        const u32x2 lo = lds_tr4(p), hi = lds_tr4(p + 8 * LDK);
        return __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      if constexpr (PRE)
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) kta[ks] = ldt(ks / 2, ks % 2);
      // product of a 32x32 LDS block (operands a: columns 0..15, then
      // 16..31) with an accumulator tile
      auto tri_mm = [&](const f16x8 (&ao)[2], const f32x16& y, f32x16 acc) {
        acc = mma(ao[0], acc_half<0>(y), acc);
        acc = mma(ao[1], acc_half<1>(y), acc);
        return acc;
      };
      // U = T Y
      f32x16 U = tri_mm(tA, X, f32x16{});
      // O^T = scale r_q e^G (S0 Q^T) + U^T P^T: rows v, lane column token
      // t = c; the P row operands of token t serve as the B operand
      {
        const float cq = sCq[c];
#pragma unroll
        for (int i = 0; i < 16; ++i) QS[i] *= cq;
      }
      QS = mma(acc_half<0>(U), pA[0], QS);
      QS = mma(acc_half<1>(U), pA[1], QS);
      if (E != 0)
#pragma unroll
        for (int i = 0; i < 16; ++i) QS[i] = __builtin_amdgcn_ldexpf(QS[i], -E);
      // token t's columns 32w + 8 q4 + 4 g .. +3 as 8-byte bf16 pieces into
      // this wave's own columns of the V/O tile (their V was consumed above
      // by this wave only); the rows go to HBM in the next chunk's staging
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<u32x2*>(sV + c * LDV + 32 * wave + 8 * q4 + 4 * g) =
            u32x2{pack_bf16(QS[4 * q4], QS[4 * q4 + 1]), pack_bf16(QS[4 * q4 + 2], QS[4 * q4 + 3])};
      // S = e^{G_C} S0 + K^T (r_k e^{G_C - G} U), S already decayed after X
      // and QS; K^T rows by transpose reads
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 c4 = *reinterpret_cast<const float4*>(sCu + 8 * q4 + 4 * g);
        U[4 * q4] *= c4.x; U[4 * q4 + 1] *= c4.y;
        U[4 * q4 + 2] *= c4.z; U[4 * q4 + 3] *= c4.w;
      }
      const f16x8 uh[2] = {acc_half<0>(U), acc_half<1>(U)};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          if constexpr (!PRE) kta[0] = ldt(kt, h2);
          const f16x8& kx = kta[PRE ? 2 * kt + h2 : 0];
          S[kt] = mma(kx, uh[h2], S[kt]);
        }
    }
    if (ck_at >= 0) store_state(a.ckpt_buf + (size_t)ck_at * sstride + ((size_t)h * DV + v) * DK);
    pt0 = t0;
    pn = n;
    __syncthreads();
  }
  for (int e = tid; e < CT * DV / 8; e += NTH) {   // last chunk's O rows
    const int t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
    if (t < pn)
      *reinterpret_cast<u32x4*>(og + (size_t)(pt0 + t) * a.Hv * DV + c8) =
          *reinterpret_cast<const u32x4*>(sV + t * LDV + c8);
  }
  if (a.final_state) store_state(a.final_state + (size_t)s * sstride + ((size_t)h * DV + v) * DK);
}

}  // namespace chunked
}  // namespace gdn

// Instantiates the launchers for one key dimension.  The scan runs 32-token
// chunks for chunk = 32 or 64 (a checkpoint on the 64-grid is on the 32-grid
// too) and 16-token chunks, zero-padded in the 32-row tile, for chunk = 16.
#define GDN_CHUNKED_LAUNCHERS(DKV)                                                          \
  namespace gdn {                                                                          \
  namespace chunked {                                                                      \
  template <int DV>                                                                        \
  static hipError_t launch_one(const ScanArgs& a, hipStream_t st) {                        \
    using C = Cfg<DKV, DV>;                                                                \
    auto kern = chunked_prefill_kernel<DKV, DV>;                                           \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::bytes); \
    if (e != hipSuccess) return e;                                                         \
    ScanArgs b = a;                                                                        \
    b.chunk = a.chunk > C::CT ? C::CT : a.chunk;                                           \
    hipLaunchKernelGGL(kern, dim3(b.n_seqs, b.Hv), dim3(C::NTH), C::bytes, st, b);         \
    return hipGetLastError();                                                              \
  }                                                                                        \
  hipError_t launch_dk##DKV(const ScanArgs& a, hipStream_t st) {                           \
    if (a.dv == 32) return launch_one<32>(a, st);                                          \
    if (a.dv == 64) return launch_one<64>(a, st);                                          \
    if (a.dv == 128) return launch_one<128>(a, st);                                        \
    return hipErrorInvalidValue;                                                           \
  }                                                                                        \
  }                                                                                        \
  }
