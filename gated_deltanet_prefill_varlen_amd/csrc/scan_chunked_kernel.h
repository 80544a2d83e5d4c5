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
// raw bf16 q/k/v are exact MFMA operands.
//
// Work split inside the workgroup (DV/32 waves): all waves stage K, K^T and
// Q of the chunk in LDS and compute the Gram and Q K^T tiles; wave 0 inverts
// the 32x32 diagonal blocks of (I + A) by forward substitution (the
// off-diagonal block is applied to Y directly: U1 = T11 Y1,
// U2 = T22 (Y2 - A21 U1), so T21 is never formed); then wave w owns state columns
// v in [32w, 32w+32): its slice of S stays in MFMA accumulator registers for
// the whole prompt (fp32), laid out as S^T tiles (rows k, lane column v).
//
// Precision: products that carry fp32 quantities into the state use split
// bf16 operands (x = hi + lo, hi = bf16(x), lo = bf16(x - hi); the lo*lo pass
// is dropped): K S0^T with S0 split (2 passes), T Y with T and Y split (3
// passes, likewise A21 U1), K^T U' with U' split (2 passes).  The output
// products are split too (Q S0^T: 2 passes; P U with P and U split: 3): a
// dot of a unit q with a state row is ~1/sqrt(dk) of |q||S row| while single
// bf16 rounding errors are not, which costs ~1e-2 relative on outputs.
// Accumulation is fp32 throughout.
#pragma once

#include <climits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace chunked {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x16) B(16x32).  Lane l: A row l%32 and B column l%32, with
// eight k values each; D register i holds row 8(i/4) + 4(l/32) + i%4,
// column l%32.
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMA A operand from a bf16 row in LDS.  The k order used across every
// product: within a 16-wide k step at offset 16*h2, lane half g (= l/32) holds
// k = 16*h2 + 4g + {0,1,2,3} and 16*h2 + 8 + 4g + {0,1,2,3}; this is exactly
// the row order of accumulator registers 8*h2 .. 8*h2+7, so an accumulator
// tile feeds the next product as its B operand without moving data.
// `p` points at element 16*h2 + 4g of the row.
__device__ __forceinline__ bf16x8 lds_a(const uint16_t* p) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
  const u32x4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, v);
}

// Eight consecutive bf16 of a row (natural k order; both operands of a
// product read with it, so the order cancels).
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Accumulator half h2 (registers 8h2..8h2+7) as a B operand, split into
// hi + lo bf16 terms.
template <int H2>
__device__ __forceinline__ void split_half(const f32x16& x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float f = x[8 * H2 + j];
    const __bf16 h = (__bf16)f;
    hi[j] = h;
    lo[j] = (__bf16)(f - (float)h);
  }
}
template <int H2>
__device__ __forceinline__ bf16x8 hi_half(const f32x16& x) {
  bf16x8 hi;
#pragma unroll
  for (int j = 0; j < 8; ++j) hi[j] = (__bf16)x[8 * H2 + j];
  return hi;
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Row of accumulator register i for lane half g.
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

template <int DK, int DV, int NT>
struct Cfg {
  static constexpr int CT = 32 * NT;      // rows of the chunk tile
  static constexpr int NW = DV / 32;      // waves
  static constexpr int NTH = 64 * NW;     // threads
  static constexpr int KT = DK / 32;      // 32-wide k tiles of the state
  static constexpr int LDK = DK + 8;      // row stride of sK, sQ (bf16)
  static constexpr int LDT = CT + 8;      // row stride of sKT, sT, sP (bf16)
  static constexpr int LDA = 36;          // row stride of sA (fp32 diagonal 32x32 blocks)
  static constexpr int oK = 0;
  static constexpr int oQ = oK + CT * LDK * 2;
  static constexpr int oKT = oQ + CT * LDK * 2;
  static constexpr int oT = oKT + DK * LDT * 2;       // hi then lo: T11, -A21, T22
  static constexpr int oP = oT + 2 * CT * LDT * 2;
  static constexpr int oA = oP + 2 * CT * LDT * 2;    // P hi then lo
  static constexpr int oS = oA + CT * LDA * 4;        // per-token scalars (A: NT diagonal blocks)
  static constexpr int kScal = 8;
  static constexpr int bytes = oS + kScal * CT * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// per-token scalar arrays (index into the scalar block)
enum { SC_G = 0, SC_BETA, SC_RK, SC_RQ, SC_CUM, SC_CK, SC_CQ, SC_CU };

template <int DK, int DV, int NT>
__global__ void __launch_bounds__(64 * (DV / 32))
chunked_prefill_kernel(const ScanArgs a) {
  using C = Cfg<DK, DV, NT>;
  constexpr int CT = C::CT, NTH = C::NTH, KT = C::KT, LDK = C::LDK, LDT = C::LDT, LDA = C::LDA;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + C::oK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + C::oQ);
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + C::oKT);
  uint16_t* sT = reinterpret_cast<uint16_t*>(smem + C::oT);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + C::oP);
  float* sA = reinterpret_cast<float*>(smem + C::oA);
  float* sc = reinterpret_cast<float*>(smem + C::oS);
  float* sG = sc + SC_G * CT;       // raw log-gates, then their cumsum
  float* sBeta = sc + SC_BETA * CT;
  float* sRk = sc + SC_RK * CT;
  float* sRq = sc + SC_RQ * CT;
  float* sCk = sc + SC_CK * CT;     // r_k e^G
  float* sCq = sc + SC_CQ * CT;     // scale r_q e^G
  float* sCu = sc + SC_CU * CT;     // r_k e^{G_C - G}

  const int s = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int j = h / (a.Hv / a.Hqk);
  const int seq0 = a.cu[s], seq1 = a.cu[s + 1];
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);
  uint16_t* og = static_cast<uint16_t*>(a.out);
  const size_t sstride = (size_t)a.Hv * DV * DK;
  const int v = 32 * wave + c;       // this lane's state column (value dim)

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
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(dst + 32 * kt + 8 * q4 + 4 * g) =
            make_float4(S[kt][4 * q4], S[kt][4 * q4 + 1], S[kt][4 * q4 + 2], S[kt][4 * q4 + 3]);
  };

  int ci = lower_bound_i32(a.ckpt, a.n_ckpt, seq0 + 1);
  int next_ck = ci < a.n_ckpt ? a.ckpt[ci] : INT_MAX;

  for (int t0 = seq0; t0 < seq1; t0 += a.chunk) {
    const int n = min(a.chunk, seq1 - t0);   // valid rows of this chunk

    // ---- 1. stage K, Q rows (zero past n), log-gates and betas
    for (int e = tid; e < CT * DK / 8; e += NTH) {
      const int t = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
      u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
      if (t < n) {
        kv = *reinterpret_cast<const u32x4*>(kg + (size_t)(t0 + t) * a.k_stride + (size_t)j * DK + c8);
        qv = *reinterpret_cast<const u32x4*>(qg + (size_t)(t0 + t) * a.q_stride + (size_t)j * DK + c8);
      }
      *reinterpret_cast<u32x4*>(sK + t * LDK + c8) = kv;
      *reinterpret_cast<u32x4*>(sQ + t * LDK + c8) = qv;
    }
    if (tid < CT) {
      const bool ok = tid < n;
      sG[tid] = ok ? a.g[(size_t)(t0 + tid) * a.Hv + h] : 0.f;
      sBeta[tid] = ok ? a.beta[(size_t)(t0 + tid) * a.Hv + h] : 0.f;
    }
    __syncthreads();

    // ---- 2. K^T, row norms, gate cumsum
    for (int e = tid; e < DK * CT / 8; e += NTH) {
      const int k = e % DK, t8 = (e / DK) * 8;
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        w[p] = (uint32_t)sK[(t8 + 2 * p) * LDK + k] | ((uint32_t)sK[(t8 + 2 * p + 1) * LDK + k] << 16);
      const u32x4 wv = {w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(sKT + k * LDT + t8) = wv;
    }
    {
      // row norms: TPR consecutive lanes per row, at least 8 columns each
      constexpr int TPR_RAW = NTH / CT >= 1 ? NTH / CT : 1;
      constexpr int TPR = TPR_RAW < DK / 8 ? TPR_RAW : DK / 8;
      constexpr int PER = DK / TPR;
      constexpr int RPP = NTH / TPR;  // rows per pass
      static_assert(PER % 8 == 0 && (TPR & (TPR - 1)) == 0, "norm split");
      for (int r0 = 0; r0 < CT; r0 += RPP) {
        const int t = r0 + tid / TPR;
        const bool valid = t < CT;   // RPP may exceed CT; those lanes compute row 0 and discard
        const int tt = valid ? t : 0;
        const int part = tid % TPR;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < PER; e += 8) {
          const int col = part * PER + e;
          const u32x4 kk = *reinterpret_cast<const u32x4*>(sK + tt * LDK + col);
          const u32x4 qq = *reinterpret_cast<const u32x4*>(sQ + tt * LDK + col);
          const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float k0 = bf16_to_f32(kw[p] & 0xFFFFu), k1 = bf16_to_f32(kw[p] >> 16);
            const float q0 = bf16_to_f32(qw[p] & 0xFFFFu), q1 = bf16_to_f32(qw[p] >> 16);
            sk = fmaf(k0, k0, sk); sk = fmaf(k1, k1, sk);
            sq = fmaf(q0, q0, sq); sq = fmaf(q1, q1, sq);
          }
        }
        sk = group_sum<TPR>(sk);
        sq = group_sum<TPR>(sq);
        if (valid && part == 0) {   // zero-padded rows past n keep r = 1 (no 0 * inf)
          const bool nrm = a.l2norm && t < n;
          sRk[t] = nrm ? 1.0f / sqrtf(sk + a.eps) : 1.0f;
          sRq[t] = nrm ? 1.0f / sqrtf(sq + a.eps) : 1.0f;
        }
      }
    }
    if (wave == 0) {  // inclusive scan of the log-gates over the chunk (fixed order)
      float x = lane < CT ? sG[lane] : 0.f;
#pragma unroll
      for (int d = 1; d < CT; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane < CT) sG[lane] = x;
    }
    __syncthreads();

    // ---- 3. Gram and Q K^T tiles (MFMA) -> A (fp32) and P (bf16); per-token scalars
    {
      constexpr int NTILE = NT * (NT + 1) / 2;
      for (int job = wave; job < 2 * NTILE; job += C::NW) {
        const bool gram = job < NTILE;
        const int tix = gram ? job : job - NTILE;
        const int mt = tix == 0 ? 0 : 1, nt = tix == 2 ? 1 : 0;
        const uint16_t* ap = (gram ? sK : sQ) + (32 * mt + c) * LDK + 8 * g;
        const uint16_t* bp = sK + (32 * nt + c) * LDK + 8 * g;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) acc = mma(lds_row8(ap + 16 * ks), lds_row8(bp + 16 * ks), acc);
        const int col = 32 * nt + c;
        const float gc = sG[col], rkc = sRk[col];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 32 * mt + acc_row(i, g);
          if (gram) {
            const bool lower = col < t;
            const float dcy = __expf(lower ? sG[t] - gc : 0.f);
            const float av = lower ? sBeta[t] * sRk[t] * rkc * dcy * acc[i] : 0.f;
            if (mt == nt) {
              sA[t * LDA + (col - 32 * nt)] = av;           // diagonal block, fp32
            } else {                                        // -A21 as hi/lo bf16 operand
              const __bf16 hi = (__bf16)(-av);
              sT[t * LDT + col] = __builtin_bit_cast(uint16_t, hi);
              sT[CT * LDT + t * LDT + col] = bf16_bits(-av - (float)hi);
            }
          } else {
            const bool lower = col <= t;
            const float dcy = __expf(lower ? sG[t] - gc : 0.f);
            const float pv = lower ? a.scale * sRq[t] * rkc * dcy * acc[i] : 0.f;
            const __bf16 hi = (__bf16)pv;
            sP[t * LDT + col] = __builtin_bit_cast(uint16_t, hi);
            sP[CT * LDT + t * LDT + col] = bf16_bits(pv - (float)hi);
          }
        }
      }
      if (tid < CT) {
        const float G = sG[tid], GC = sG[CT - 1];
        sCk[tid] = sRk[tid] * __expf(G);
        sCq[tid] = a.scale * sRq[tid] * __expf(G);
        sCu[tid] = sRk[tid] * __expf(GC - G);
      }
    }
    __syncthreads();

    // ---- 4. diagonal blocks T_bb = (I + A_bb)^-1 by forward substitution:
    //         lane jj owns column jj % 32 of block jj / 32
    if (wave == 0 && lane < CT) {
      const int b = lane >> 5, cc = lane & 31;
      const float* ab = sA + 32 * b * LDA;
      float Tc[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        float acc[4] = {t == cc ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i4 = 0; i4 < t; i4 += 4) {
          const float4 av = *reinterpret_cast<const float4*>(ab + t * LDA + i4);
          const float ar[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (i4 + u < t) acc[u] = fmaf(-ar[u], Tc[i4 + u], acc[u]);
        }
        Tc[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
      uint16_t* tb = sT + 32 * b * LDT + 32 * b + cc;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const __bf16 hi = (__bf16)Tc[t];
        tb[t * LDT] = __builtin_bit_cast(uint16_t, hi);
        tb[CT * LDT + t * LDT] = bf16_bits(Tc[t] - (float)hi);
      }
    }
    __syncthreads();

    // ---- 5. state path for this wave's 32 value columns
    {
      // S -> split B operands
      bf16x8 Sh[KT][2], Sl[KT][2];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        split_half<0>(S[kt], Sh[kt][0], Sl[kt][0]);
        split_half<1>(S[kt], Sh[kt][1], Sl[kt][1]);
      }
      f32x16 X[NT], QS[NT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        X[mt] = f32x16{};
        QS[mt] = f32x16{};
        const uint16_t* kr = sK + (32 * mt + c) * LDK + 4 * g;
        const uint16_t* qr = sQ + (32 * mt + c) * LDK + 4 * g;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const bf16x8 ka = lds_a(kr + 32 * kt + 16 * h2);
            X[mt] = mma(ka, Sh[kt][h2], X[mt]);
            X[mt] = mma(ka, Sl[kt][h2], X[mt]);
            const bf16x8 qa = lds_a(qr + 32 * kt + 16 * h2);
            QS[mt] = mma(qa, Sh[kt][h2], QS[mt]);
            QS[mt] = mma(qa, Sl[kt][h2], QS[mt]);
          }
      }
      // Y = beta (V - r_k e^G X), in place of X
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 32 * mt + acc_row(i, g);
          const float vv = t < n ? bf16_to_f32(vg[(size_t)(t0 + t) * a.v_stride + (size_t)h * DV + v]) : 0.f;
          X[mt][i] = sBeta[t] * (vv - sCk[t] * X[mt][i]);
        }
      // U1 = T11 Y1;  U2 = T22 (Y2 - A21 U1)   (3-pass split products)
      f32x16 U[NT];
      auto tri_mm = [&](const uint16_t* rowp, const f32x16& y, f32x16 acc) {
        bf16x8 yh0, yl0, yh1, yl1;
        split_half<0>(y, yh0, yl0);
        split_half<1>(y, yh1, yl1);
        const uint16_t* lo = rowp + CT * LDT;
        const bf16x8 a0h = lds_a(rowp), a0l = lds_a(lo), a1h = lds_a(rowp + 16), a1l = lds_a(lo + 16);
        acc = mma(a0h, yh0, acc);
        acc = mma(a0l, yh0, acc);
        acc = mma(a0h, yl0, acc);
        acc = mma(a1h, yh1, acc);
        acc = mma(a1l, yh1, acc);
        acc = mma(a1h, yl1, acc);
        return acc;
      };
      U[0] = tri_mm(sT + c * LDT + 4 * g, X[0], f32x16{});
      if constexpr (NT == 2) {
        const f32x16 w = tri_mm(sT + (32 + c) * LDT + 4 * g, U[0], X[1]);        // Y2 - A21 U1
        U[1] = tri_mm(sT + (32 + c) * LDT + 32 + 4 * g, w, f32x16{});
      }
      // O = scale r_q e^G (Q S0^T) + P U, written for the chunk's valid rows
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) QS[mt][i] *= sCq[32 * mt + acc_row(i, g)];
#pragma unroll
        for (int m2 = 0; m2 <= mt; ++m2) QS[mt] = tri_mm(sP + (32 * mt + c) * LDT + 32 * m2 + 4 * g, U[m2], QS[mt]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 32 * mt + acc_row(i, g);
          if (t < n) og[((size_t)(t0 + t) * a.Hv + h) * DV + v] = bf16_bits(QS[mt][i]);
        }
      }
      // S = e^{G_C} S + K^T (r_k e^{G_C - G} U)
      const float gC = __expf(sG[CT - 1]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kt][i] *= gC;
#pragma unroll
      for (int m2 = 0; m2 < NT; ++m2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) U[m2][i] *= sCu[32 * m2 + acc_row(i, g)];
        bf16x8 uh0, ul0, uh1, ul1;
        split_half<0>(U[m2], uh0, ul0);
        split_half<1>(U[m2], uh1, ul1);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const uint16_t* kr = sKT + (32 * kt + c) * LDT + 32 * m2 + 4 * g;
          const bf16x8 a0 = lds_a(kr), a1 = lds_a(kr + 16);
          S[kt] = mma(a0, uh0, S[kt]);
          S[kt] = mma(a0, ul0, S[kt]);
          S[kt] = mma(a1, uh1, S[kt]);
          S[kt] = mma(a1, ul1, S[kt]);
        }
      }
    }
    if (t0 + n == next_ck) {
      store_state(a.ckpt_buf + (size_t)ci * sstride + ((size_t)h * DV + v) * DK);
      ++ci;
      next_ck = ci < a.n_ckpt ? a.ckpt[ci] : INT_MAX;
    }
    __syncthreads();
  }
  if (a.final_state) store_state(a.final_state + (size_t)s * sstride + ((size_t)h * DV + v) * DK);
}

}  // namespace chunked
}  // namespace gdn

// Instantiates the launchers for one key dimension.
#define GDN_CHUNKED_LAUNCHERS(DKV)                                                          \
  namespace gdn {                                                                          \
  namespace chunked {                                                                      \
  template <int DV, int NT>                                                                \
  static hipError_t launch_one(const ScanArgs& a, hipStream_t st) {                        \
    using C = Cfg<DKV, DV, NT>;                                                            \
    auto kern = chunked_prefill_kernel<DKV, DV, NT>;                                       \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::bytes); \
    if (e != hipSuccess) return e;                                                         \
    hipLaunchKernelGGL(kern, dim3(a.n_seqs, a.Hv), dim3(C::NTH), C::bytes, st, a);         \
    return hipGetLastError();                                                              \
  }                                                                                        \
  template <int DV>                                                                        \
  static hipError_t launch_nt(const ScanArgs& a, hipStream_t st) {                         \
    return a.chunk > 32 ? launch_one<DV, 2>(a, st) : launch_one<DV, 1>(a, st);             \
  }                                                                                        \
  hipError_t launch_dk##DKV(const ScanArgs& a, hipStream_t st) {                           \
    if (a.dv == 32) return launch_nt<32>(a, st);                                           \
    if (a.dv == 64) return launch_nt<64>(a, st);                                           \
    if (a.dv == 128) return launch_nt<128>(a, st);                                         \
    return hipErrorInvalidValue;                                                           \
  }                                                                                        \
  }                                                                                        \
  }
