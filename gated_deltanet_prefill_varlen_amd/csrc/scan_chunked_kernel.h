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
// Work split (DV/32 waves): all waves stage K and Q of the chunk in LDS and
// share the Gram / Q K^T tiles and the inversion of the 32x32 diagonal blocks
// of (I + A) (forward substitution, several lanes per column); the
// off-diagonal block is applied to Y directly, U1 = T11 Y1,
// U2 = T22 (Y2 - A21 U1), so T21 is never formed.  Wave w owns state columns
// v in [32w, 32w+32): its slice of S stays in MFMA accumulator registers for
// the whole prompt (fp32), laid out as S^T tiles (rows k, lane column v).
// LDS is kept under 80 KB and registers under 256 so two workgroups share a
// CU and overlap each other's latency-bound phases.
//
// Precision: every product that carries fp32 values uses split bf16 operands
// (x = hi + lo, hi = bf16(x), lo = bf16(x - hi); the lo*lo pass dropped):
// K S0^T and Q S0^T with S0 split (2 passes), T Y, A21 U1, P U with both
// sides split (3 passes), K^T U' with U' split (2 passes).  A dot of a unit q
// with a state row is ~1/sqrt(dk) of |q||S row| while single bf16 rounding
// errors are not, which is why the output products are split too.
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

// MFMA operand from a bf16 row in LDS.  The k order used by every product:
// within a 16-wide k step at offset 16*h2, lane half g (= l/32) holds
// k = 16*h2 + 4g + {0,1,2,3} and 16*h2 + 8 + 4g + {0,1,2,3}; this is exactly
// the row order of accumulator registers 8*h2 .. 8*h2+7, so an accumulator
// tile feeds the next product as its B operand without moving data.
// `p` points at element 16*h2 + 4g of the row (8-byte aligned).
__device__ __forceinline__ bf16x8 lds_op(const uint16_t* p) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
  const u32x4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed bf16 hi terms and packed bf16 lo terms
// (hi = bf16(x), lo = bf16(x - hi)), two values per conversion.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2));
}

// Accumulator half h2 (registers 8h2..8h2+7) as a B operand, split into
// hi + lo bf16 terms.
template <int H2>
__device__ __forceinline__ void split_half(const f32x16& x, bf16x8& hi, bf16x8& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split2(x[8 * H2 + 2 * p], x[8 * H2 + 2 * p + 1], hw[p], lw[p]);
  hi = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
}

// Sum of squares of the eight bf16 values in a 16-byte vector.
__device__ __forceinline__ float sumsq8(const u32x4& w) {
  float s = 0.f;
  const uint32_t r[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x0 = __uint_as_float(r[p] << 16), x1 = __uint_as_float(r[p] & 0xFFFF0000u);
    s = fmaf(x0, x0, s);
    s = fmaf(x1, x1, s);
  }
  return s;
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ void store_split(uint16_t* hi_plane, int plane_stride, int idx, float x) {
  const __bf16 h = (__bf16)x;
  hi_plane[idx] = __builtin_bit_cast(uint16_t, h);
  hi_plane[plane_stride + idx] = bf16_bits(x - (float)h);
}

// Row of accumulator register i for lane half g.
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

template <int DK, int DV, int NT>
struct Cfg {
  static constexpr int CT = 32 * NT;      // rows of the chunk tile
  static constexpr int NW = DV / 32;      // waves
  static constexpr int NTH = 64 * NW;     // threads
  static constexpr int KT = DK / 32;      // 32-wide k tiles of the state
  static constexpr int LDK = DK + 4;      // row stride of sK, sQ (bf16; 8-byte aligned rows)
  static constexpr int LDT = CT + 4;      // row stride of sT, sP (bf16)
  // forward substitution: LPC lanes per column of the diagonal blocks
  static constexpr int LPC_RAW = NTH / CT;
  static constexpr int LPC = LPC_RAW > 4 ? 4 : (LPC_RAW < 1 ? 1 : LPC_RAW);
  static constexpr int MPL = 32 / LPC;    // rows of a column held per lane
  static constexpr int LDA = 32 + 4;      // row stride of a diagonal block of A (fp32)
  static constexpr int oK = 0;
  static constexpr int oQ = oK + CT * LDK * 2;
  static constexpr int LDV = DV + 8;      // row stride of the V / O tile (bf16; 16-byte rows)
  static constexpr int oV = oQ + CT * LDK * 2;        // V tile, then the O tile
  static constexpr int oT = oV + CT * LDV * 2;        // hi then lo plane: T11, -A21, T22
  static constexpr int oP = oT + 2 * CT * LDT * 2;    // hi then lo plane
  static constexpr int oA = oP + 2 * CT * LDT * 2;    // NT diagonal blocks of A, lane-interleaved
  static constexpr int oS = oA + NT * 32 * LDA * 4;   // per-token scalars
  static constexpr int kScal = 8;
  static constexpr int bytes = oS + kScal * CT * 4;
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
  static_assert(LPC * CT <= NTH || LPC == 1, "substitution lanes");
  // the next chunk's rows wait in registers (16-byte vectors per thread)
  // while this chunk computes, when they fit in 32 registers
  static constexpr int NVK = (CT * DK / 8 + NTH - 1) / NTH;
  static constexpr int NVV = (CT * DV / 8 + NTH - 1) / NTH;
  static constexpr bool PREFETCH = (2 * NVK + NVV) * 4 <= 32;
};

// per-token scalar arrays (index into the scalar block)
enum { SC_G = 0, SC_BETA, SC_RK, SC_RQ, SC_CK, SC_CQ, SC_CU, SC_PAD };

template <int DK, int DV, int NT>
__global__ void __launch_bounds__(64 * (DV / 32), 2)
chunked_prefill_kernel(const ScanArgs a) {
  using C = Cfg<DK, DV, NT>;
  constexpr int CT = C::CT, NTH = C::NTH, KT = C::KT, LDK = C::LDK, LDT = C::LDT, LDA = C::LDA;
  constexpr int LPC = C::LPC, MPL = C::MPL, LDV = C::LDV;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + C::oK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + C::oQ);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + C::oV);
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
  constexpr int TPL = CT * LDT;     // bf16 elements per hi/lo plane

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

  // checkpoint cursor, uniform over the workgroup; the positions are read
  // through the constant address space so they come in by scalar loads and
  // never wait behind the vector loads in flight
  typedef const int32_t __attribute__((address_space(4)))* ConstI32;
  const ConstI32 ckp = (ConstI32)a.ckpt;
  int ci = __builtin_amdgcn_readfirstlane(lower_bound_i32(a.ckpt, a.n_ckpt, seq0 + 1));
  int next_ck = ci < a.n_ckpt ? ckp[ci] : INT_MAX;

  // One chunk's HBM rows into registers.  Every lane loads (row index clamped
  // into the chunk, so no load is conditional); rows past the chunk's end are
  // zeroed where they are consumed.
  u32x4 pk[C::NVK], pq[C::NVK], pv[C::NVV];
  float pg, pb;
  auto fetch = [&](int t0x, int nx) {
#pragma unroll
    for (int u = 0; u < C::NVK; ++u) {
      const int e = min(tid + u * NTH, CT * DK / 8 - 1);
      const int t = min(e / (DK / 8), nx - 1), c8 = (e % (DK / 8)) * 8;
      pk[u] = *reinterpret_cast<const u32x4*>(kg + (size_t)(t0x + t) * a.k_stride + (size_t)j * DK + c8);
      pq[u] = *reinterpret_cast<const u32x4*>(qg + (size_t)(t0x + t) * a.q_stride + (size_t)j * DK + c8);
    }
#pragma unroll
    for (int u = 0; u < C::NVV; ++u) {
      const int e = min(tid + u * NTH, CT * DV / 8 - 1);
      const int t = min(e / (DV / 8), nx - 1), c8 = (e % (DV / 8)) * 8;
      pv[u] = *reinterpret_cast<const u32x4*>(vg + (size_t)(t0x + t) * a.v_stride + c8);
    }
    const int tl = min(lane, nx - 1);
    pg = a.g[(size_t)(t0x + tl) * a.Hv + h];
    pb = a.beta[(size_t)(t0x + tl) * a.Hv + h];
  };
  if constexpr (C::PREFETCH)
    if (seq1 > seq0) fetch(seq0, min(a.chunk, seq1 - seq0));
  // drain the state and first-chunk loads here, so that no wait inside the
  // chunk loop has to cover them (vmcnt(0); expcnt, lgkmcnt unchanged)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  int pt0 = 0, pn = 0;   // previous chunk: its O tile is still in the V/O LDS tile
  for (int t0 = seq0; t0 < seq1; t0 += a.chunk) {
    const int n = min(a.chunk, seq1 - t0);   // valid rows of this chunk

    // ---- 1. stage K, Q rows (zero past n) with their L2 norms (squares summed
    //         in registers, then over the row's lanes), V rows, betas and the
    //         gate cumsum.  The rows were fetched into registers while the
    //         previous chunk ran.  The previous chunk's O rows leave the V/O
    //         tile first: read into registers before V lands, stored to HBM
    //         after (global stores issued after the loads are consumed).
    if constexpr (!C::PREFETCH) fetch(t0, n);
    {
      constexpr int VPR = DK / 8;          // 16-byte vectors per row = lanes per row
      static_assert((CT * DK / 8) % 64 == 0 && VPR <= 16, "row lanes");
#pragma unroll
      for (int u = 0; u < C::NVK; ++u) {
        const int e = tid + u * NTH;
        if (e < CT * DK / 8) {             // whole waves per trip
          const int t = e / VPR, c8 = (e % VPR) * 8;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 kv = t < n ? pk[u] : z, qv = t < n ? pq[u] : z;
          u32x2* kd = reinterpret_cast<u32x2*>(sK + t * LDK + c8);
          u32x2* qd = reinterpret_cast<u32x2*>(sQ + t * LDK + c8);
          kd[0] = u32x2{kv.x, kv.y}; kd[1] = u32x2{kv.z, kv.w};
          qd[0] = u32x2{qv.x, qv.y}; qd[1] = u32x2{qv.z, qv.w};
          float sk = sumsq8(kv), sq = sumsq8(qv);
          sk = group_sum<VPR>(sk);
          sq = group_sum<VPR>(sq);
          if (e % VPR == 0) {   // zero-padded rows past n keep r = 1 (no 0 * inf)
            const bool nrm = a.l2norm && t < n;
            sRk[t] = nrm ? 1.0f / sqrtf(sk + a.eps) : 1.0f;
            sRq[t] = nrm ? 1.0f / sqrtf(sq + a.eps) : 1.0f;
          }
        }
      }
    }
    {
      // a thread owns the same 16-byte segments of the V/O tile for both
      u32x4 ov[C::NVV];
#pragma unroll
      for (int u = 0; u < C::NVV; ++u) {
        const int e = tid + u * NTH;
        if (e < CT * DV / 8) {
          const int t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
          u32x4* seg = reinterpret_cast<u32x4*>(sV + t * LDV + c8);
          ov[u] = *seg;
          *seg = t < n ? pv[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (wave == 0) {  // betas and the inclusive scan of the log-gates (fixed order)
        float x = lane < n ? pg : 0.f;
#pragma unroll
        for (int d = 1; d < CT; d <<= 1) {
          const float y = __shfl_up(x, d, 64);
          if (lane >= d) x += y;
        }
        if (lane < CT) {
          sG[lane] = x;
          sBeta[lane] = lane < n ? pb : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < C::NVV; ++u) {
        const int e = tid + u * NTH;
        const int t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
        if (e < CT * DV / 8 && t < pn)
          *reinterpret_cast<u32x4*>(og + (size_t)(pt0 + t) * a.Hv * DV + c8) = ov[u];
      }
    }
    __syncthreads();
    if constexpr (C::PREFETCH)
      if (t0 + a.chunk < seq1) fetch(t0 + a.chunk, min(a.chunk, seq1 - t0 - a.chunk));

    // ---- 3. Gram and Q K^T tiles (MFMA, shared K operand) -> A, P; scalars
    {
      constexpr int NTILE = NT * (NT + 1) / 2;
      for (int job = wave; job < 2 * NTILE; job += C::NW) {
        const bool gram = job < NTILE;                 // Gram K K^T, else Q K^T
        const int tix = gram ? job : job - NTILE;
        const int mt = tix == 0 ? 0 : 1, nt = tix == 2 ? 1 : 0;
        const uint16_t* ar = (gram ? sK : sQ) + (32 * mt + c) * LDK + 4 * g;
        const uint16_t* br = sK + (32 * nt + c) * LDK + 4 * g;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) acc = mma(lds_op(ar + 16 * ks), lds_op(br + 16 * ks), acc);
        const int col = 32 * nt + c, lcol = c;   // global / block-local column
        const float gc = sG[col], rkc = sRk[col];
        const int qa = lcol % LPC, ma = lcol / LPC;
        const float* rowsc = gram ? sRk : sRq;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int tb = 32 * mt + 8 * q4 + 4 * g;
          const float4 G4 = *reinterpret_cast<const float4*>(sG + tb);
          const float4 B4 = *reinterpret_cast<const float4*>(sBeta + tb);
          const float4 R4 = *reinterpret_cast<const float4*>(rowsc + tb);
          const float Gr[4] = {G4.x, G4.y, G4.z, G4.w}, Br[4] = {B4.x, B4.y, B4.z, B4.w};
          const float Rr[4] = {R4.x, R4.y, R4.z, R4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = tb + r;
            const bool on = gram ? col < t : col <= t;
            const float dcy = __expf(on ? Gr[r] - gc : 0.f);
            const float f = (gram ? Br[r] : a.scale) * Rr[r] * rkc * dcy * acc[4 * q4 + r];
            const float val = on ? f : 0.f;
            if (!gram) store_split(sP, TPL, t * LDT + col, val);
            else if (mt == nt) sA[t * LDA + qa * MPL + ma] = val;
            else store_split(sT, TPL, t * LDT + col, -val);      // -A21, split operand
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

    // ---- 4. diagonal blocks T_bb = (I + A_bb)^-1 by forward substitution.
    //         LPC consecutive lanes share column jj: lane part q keeps rows
    //         q, q+LPC, ... of the column and sums their terms; a row's total
    //         is a fixed-order lane-group sum.
    if (tid < CT * LPC) {
      const int jj = tid / LPC, q = tid % LPC;
      const int b = jj >> 5, cc = jj & 31;
      const float* ab = sA + 32 * b * LDA + q * MPL;
      float Tl[MPL];
#pragma unroll
      for (int m = 0; m < MPL; ++m) Tl[m] = 0.f;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        float acc0 = 0.f, acc1 = 0.f;
        const float* arow = ab + t * LDA;
#pragma unroll
        for (int m = 0; m < (t + LPC - 1) / LPC; ++m) {
          if (m & 1) acc1 = fmaf(-arow[m], Tl[m], acc1);
          else acc0 = fmaf(-arow[m], Tl[m], acc0);
        }
        const float tot = group_sum<LPC>(acc0 + acc1) + (t == cc ? 1.f : 0.f);
        if (q == t % LPC) Tl[t / LPC] = tot;
      }
      uint16_t* tb = sT + 32 * b * LDT + 32 * b + cc;
#pragma unroll
      for (int m = 0; m < MPL; ++m) store_split(tb, TPL, (q + LPC * m) * LDT, Tl[m]);
    }
    __syncthreads();

    // ---- 5. state path for this wave's 32 value columns
    {
      // X = K S0^T and QS = Q S0^T, S0 split per k tile on the fly
      f32x16 X[NT], QS[NT];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) { X[mt] = f32x16{}; QS[mt] = f32x16{}; }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 sh, sl;
          if (h2 == 0) split_half<0>(S[kt], sh, sl); else split_half<1>(S[kt], sh, sl);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            const int off = (32 * mt + c) * LDK + 4 * g + 32 * kt + 16 * h2;
            const bf16x8 ka = lds_op(sK + off);
            const bf16x8 qa = lds_op(sQ + off);
            X[mt] = mma(ka, sh, X[mt]);
            X[mt] = mma(ka, sl, X[mt]);
            QS[mt] = mma(qa, sh, QS[mt]);
            QS[mt] = mma(qa, sl, QS[mt]);
          }
        }
      // Y = beta (V - r_k e^G X), in place of X (zero past n)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int tb = 32 * mt + 8 * q4 + 4 * g;
          const float4 b4 = *reinterpret_cast<const float4*>(sBeta + tb);
          const float4 k4 = *reinterpret_cast<const float4*>(sCk + tb);
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            const float vvv = bf16_to_f32(sV[(tb + r) * LDV + v]);
            const float y = bb[r] * (vvv - kk[r] * X[mt][i]);
            X[mt][4 * q4 + r] = tb + r < n ? y : 0.f;
          }
        }
      // product of a split 32x32 LDS block (rows at rowp) with a split tile
      auto tri_mm = [&](const uint16_t* rowp, const uint16_t* lo_plane_rowp, const f32x16& y,
                        f32x16 acc) {
        bf16x8 yh0, yl0, yh1, yl1;
        split_half<0>(y, yh0, yl0);
        split_half<1>(y, yh1, yl1);
        const bf16x8 a0h = lds_op(rowp), a0l = lds_op(lo_plane_rowp);
        const bf16x8 a1h = lds_op(rowp + 16), a1l = lds_op(lo_plane_rowp + 16);
        acc = mma(a0h, yh0, acc);
        acc = mma(a0l, yh0, acc);
        acc = mma(a0h, yl0, acc);
        acc = mma(a1h, yh1, acc);
        acc = mma(a1l, yh1, acc);
        acc = mma(a1h, yl1, acc);
        return acc;
      };
      // U1 = T11 Y1;  U2 = T22 (Y2 - A21 U1)
      f32x16 U[NT];
      {
        const uint16_t* r0 = sT + c * LDT + 4 * g;
        U[0] = tri_mm(r0, r0 + TPL, X[0], f32x16{});
        if constexpr (NT == 2) {
          const uint16_t* r1 = sT + (32 + c) * LDT + 4 * g;
          const f32x16 w = tri_mm(r1, r1 + TPL, U[0], X[1]);
          U[1] = tri_mm(r1 + 32, r1 + 32 + TPL, w, f32x16{});
        }
      }
      // O = scale r_q e^G (Q S0^T) + P U -> out rows < n
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 c4 = *reinterpret_cast<const float4*>(sCq + 32 * mt + 8 * q4 + 4 * g);
          QS[mt][4 * q4] *= c4.x; QS[mt][4 * q4 + 1] *= c4.y;
          QS[mt][4 * q4 + 2] *= c4.z; QS[mt][4 * q4 + 3] *= c4.w;
        }
        const uint16_t* pr = sP + (32 * mt + c) * LDT + 4 * g;
#pragma unroll
        for (int m2 = 0; m2 <= mt; ++m2) QS[mt] = tri_mm(pr + 32 * m2, pr + 32 * m2 + TPL, U[m2], QS[mt]);
        // O into this wave's own columns of the V/O tile (V of these columns
        // was consumed above by this wave only); stored out next chunk
#pragma unroll
        for (int i = 0; i < 16; ++i) sV[(32 * mt + acc_row(i, g)) * LDV + v] = bf16_bits(QS[mt][i]);
      }
      // S = e^{G_C} S + K^T (r_k e^{G_C - G} U); K^T operand gathered from K rows
      const float gC = __expf(sG[CT - 1]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kt][i] *= gC;
#pragma unroll
      for (int m2 = 0; m2 < NT; ++m2) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 c4 = *reinterpret_cast<const float4*>(sCu + 32 * m2 + 8 * q4 + 4 * g);
          U[m2][4 * q4] *= c4.x; U[m2][4 * q4 + 1] *= c4.y;
          U[m2][4 * q4 + 2] *= c4.z; U[m2][4 * q4 + 3] *= c4.w;
        }
        bf16x8 uh[2], ul[2];
        split_half<0>(U[m2], uh[0], ul[0]);
        split_half<1>(U[m2], uh[1], ul[1]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            // A operand: rows k = 32kt + c, k-order (tokens) 32*m2 + 16*h2 + 4g + {0..3, 8..11}
            const uint16_t* kc = sK + (32 * m2 + 16 * h2 + 4 * g) * LDK + 32 * kt + c;
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int r = (p < 2 ? 0 : 8) + 2 * (p & 1);
              w[p] = (uint32_t)kc[r * LDK] | ((uint32_t)kc[(r + 1) * LDK] << 16);
            }
            const bf16x8 ka = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            S[kt] = mma(ka, uh[h2], S[kt]);
            S[kt] = mma(ka, ul[h2], S[kt]);
          }
      }
    }
    if (t0 + n == next_ck) {
      store_state(a.ckpt_buf + (size_t)ci * sstride + ((size_t)h * DV + v) * DK);
      ci = __builtin_amdgcn_readfirstlane(ci + 1);
      next_ck = ci < a.n_ckpt ? ckp[ci] : INT_MAX;
    }
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
  /* The scan runs 32-token chunks for chunk = 32 or 64 (a 64-grid checkpoint  */         \
  /* is on the 32-grid too) and 16-token chunks, zero-padded, for chunk = 16:  */         \
  /* the 64-row tile needs more than the 256 registers of two workgroups/CU.   */         \
  template <int DV>                                                                        \
  static hipError_t launch_nt(const ScanArgs& a, hipStream_t st) {                         \
    ScanArgs b = a;                                                                        \
    b.chunk = a.chunk > 32 ? 32 : a.chunk;                                                 \
    return launch_one<DV, 1>(b, st);                                                       \
  }                                                                                        \
  hipError_t launch_dk##DKV(const ScanArgs& a, hipStream_t st) {                           \
    if (a.dv == 32) return launch_nt<32>(a, st);                                           \
    if (a.dv == 64) return launch_nt<64>(a, st);                                           \
    if (a.dv == 128) return launch_nt<128>(a, st);                                         \
    return hipErrorInvalidValue;                                                           \
  }                                                                                        \
  }                                                                                        \
  }
