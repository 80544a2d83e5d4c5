// Chunked gated-delta-rule prefill with the chunk's work pipelined over wave
// roles (d_k = d_v = 128, 32-token chunks, bf16 io).
//
// Per chunk the arithmetic is that of chunked_prefill_kernel
// (scan_chunked_kernel.h: the WY/UT form of Yang et al., NeurIPS 2024, gated
// as in Gated Delta Networks, ICLR 2025; fp16 MFMA operands, fp32
// accumulation and state).  The work split differs: one workgroup of twelve
// waves per (prompt, value head), one workgroup per CU, three waves per SIMD.
//   - state waves 0..3 each own 32 state columns in MFMA accumulators for the
//     whole prompt and run the state path of chunk c (X = K S0^T, Q S0^T, the
//     decay, Y, U = T Y, the output rows, the state update, checkpoints);
//   - in the same barrier interval the loader waves 4..7 stage chunk c+3 and
//     request the rows of chunk c+5, and the factor waves 8..11 form the Gram
//     and K Q^T tiles of chunk c+2 with the per-token factors (waves 8, 9)
//     and invert the (I + A) block of chunk c+1 (waves 10, 11).
// Only the state path depends on the state; the rest of a chunk's work runs
// ahead of it on the other waves of the same SIMDs, and each chunk costs one
// barrier.  A ring of four LDS slots (K, Q, V and P tiles and the per-token
// scalars) carries a chunk from its staging to its state path (the state
// waves store their output rows straight from registers); A and T are
// double-buffered.  A prompt of n chunks takes n + 3 intervals (rounded up
// to even).  Each role runs its own loop with the same barrier count: the
// state waves keep the state in their registers, the loader waves two
// chunks' rows in flight in theirs, loaded two intervals ahead of their
// staging.  Chunks follow ChunkWalk (32 tokens from the prompt's start, cut
// at every checkpoint); the loader and the state waves each walk them.
// fp16 range: the loader scales q/k rows far from unit length by a power
// of two (kQkLo, kQkHi) and records the chunk's largest |v|; each state wave
// holds its columns as 2^E S (kBand).
#pragma once

#include "scan_chunked_kernel.h"

namespace gdn {
namespace chunked {

template <int DK, int DV>
struct PipeCfg {
  static constexpr int CT = 32;                 // tokens per chunk
  static constexpr int NSW = DV / 32;           // state waves
  static constexpr int NLW = 4;                 // loader waves (rows in, staging)
  static constexpr int NFW = 4;                 // factor waves (Gram, K Q^T, substitution)
  static constexpr int P0 = 64 * NSW;           // first loader thread
  static constexpr int PTH = 64 * NLW;          // loader threads
  static constexpr int F0 = P0 + PTH;           // first factor thread
  static constexpr int NTH = F0 + 64 * NFW;
  static constexpr int KT = DK / 32;
  static constexpr int LDK = DK + 12;           // row strides as in Cfg
  static constexpr int LDT = CT + 4;
  static constexpr int LDV = DV + 24;
  static constexpr int LDA = CT + 4;
  static constexpr int LPC = 4, MPL = CT / LPC; // substitution: 4 lanes per column of T
  static constexpr int SUB0 = 2 * 64;           // first substitution thread (factor index)
  static constexpr int RING = 4;
  static constexpr int kScal = 12;
  static constexpr int rK = 0;                  // ring slot layout
  static constexpr int rQ = rK + CT * LDK * 2;
  static constexpr int rV = rQ + CT * LDK * 2;  // V tile
  static constexpr int rP = rV + CT * LDV * 2;
  static constexpr int rS = rP + CT * LDT * 2;
  static constexpr int SLOT = rS + kScal * CT * 4;
  static constexpr int oA = RING * SLOT;        // two A tiles (fp32, transposed)
  static constexpr int oT = oA + 2 * CT * LDA * 4;   // two T tiles (fp16)
  static constexpr int bytes = oT + 2 * CT * LDT * 2;
  static constexpr int NVV = CT * DV / 8 / PTH; // 16-byte V pieces per loader thread
  static_assert(NSW == 4 && DK == 128, "laid out for d_k = d_v = 128");
  static_assert(CT * DK / 16 == PTH && NVV * PTH == CT * DV / 8, "staging shares");
  static_assert(SUB0 + CT * LPC == 64 * NFW, "the last two factor waves substitute");
  static_assert(bytes <= 160 * 1024, "LDS of one CU");
  static_assert(SLOT % 16 == 0 && rQ % 16 == 0 && rV % 16 == 0 && rP % 16 == 0 && rS % 16 == 0 &&
                oA % 16 == 0 && oT % 16 == 0, "align");
};

template <int DK, int DV, bool CONV>
__global__ void __launch_bounds__(64 * (DV / 32 + 8), 1)
pipelined_prefill_kernel(const ScanArgs a) {
  using C = PipeCfg<DK, DV>;
  constexpr int CT = C::CT, KT = C::KT, LDK = C::LDK, LDT = C::LDT, LDA = C::LDA, LDV = C::LDV;
  constexpr int LPC = C::LPC, MPL = C::MPL, NSW = C::NSW, PTH = C::PTH;
  constexpr int NKS = DK / 16;
  extern __shared__ __align__(16) unsigned char smem[];

  // (prompt, value head) of this workgroup.  Workgroups go to the eight XCDs
  // round-robin by linear id, each XCD with its own L2: the G = Hv / Hqk
  // value heads that read the same q/k rows are given linear ids 8 apart
  // (same XCD, dispatched together), when the (prompt, qk head) groups come
  // in whole rounds of eight; otherwise the grid's own order.
  int s = blockIdx.x, h = blockIdx.y;
  {
    const int G = a.Hv / a.Hqk, P = a.n_seqs * a.Hqk;
    if (P % 8 == 0) {
      const int L = blockIdx.x + a.n_seqs * blockIdx.y;
      const int r = L % (8 * G), p = 8 * (L / (8 * G)) + r % 8;
      s = p % a.n_seqs;
      h = G * (p / a.n_seqs) + r / 8;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int grp = lane >> 4, li = lane & 15;
  const int ptid = tid - C::P0;   // loader thread index (negative in the state waves)
  const int j = h / (a.Hv / a.Hqk);
  const int seq0 = a.cu[s], seq1 = a.cu[s + 1];
  // checkpoints of this prompt: index of the first, by scalar loads
  const ConstI32 ckp = (ConstI32)a.ckpt;
  const int ci0 = __builtin_amdgcn_readfirstlane(lower_bound_i32(a.ckpt, a.n_ckpt, seq0 + 1));
  const int nch = count_chunks(seq0, seq1, ci0, ckp, a.n_ckpt, CT);

  auto slot = [&](int ch) { return smem + (ch & (C::RING - 1)) * C::SLOT; };
  auto ringK = [&](int ch) { return reinterpret_cast<uint16_t*>(slot(ch) + C::rK); };
  auto ringQ = [&](int ch) { return reinterpret_cast<uint16_t*>(slot(ch) + C::rQ); };
  auto ringV = [&](int ch) { return reinterpret_cast<uint16_t*>(slot(ch) + C::rV); };
  auto ringP = [&](int ch) { return reinterpret_cast<uint16_t*>(slot(ch) + C::rP); };
  auto ringSc = [&](int ch) { return reinterpret_cast<float*>(slot(ch) + C::rS); };
  auto bufA = [&](int ch) { return reinterpret_cast<float*>(smem + C::oA + (ch & 1) * (CT * LDA * 4)); };
  auto bufT = [&](int ch) { return reinterpret_cast<uint16_t*>(smem + C::oT + (ch & 1) * (CT * LDT * 2)); };

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)h * DV;
  uint16_t* og = static_cast<uint16_t*>(a.out) + (size_t)h * DV;
  const size_t sstride = (size_t)a.Hv * DV * DK;
  const int v = 32 * (wave & (NSW - 1)) + c;   // a state wave's column (value dim)
  // transpose-read bases (as in chunked_prefill_kernel): lanes of 16-lane
  // group grp cover columns 16 (grp % 2) .. +15 and rows 4 (grp / 2) + j of
  // a tile; lane 4j + r names the 4-column piece r of row j
  const int ktr = (4 * (grp >> 1) + (li >> 2)) * LDK + 16 * (grp & 1) + 4 * (li & 3);
  const int vtr = (4 * (grp >> 1) + (li >> 2)) * LDV + 32 * (wave & (NSW - 1)) + 16 * (grp & 1) + 4 * (li & 3);

  // ---- state slice S^T[k][v] (state waves)
  f32x16 S[KT];
  {
    const float* src = (wave < NSW && a.init) ? a.init + (size_t)s * sstride + ((size_t)h * DV + v) * DK
                                              : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (src) x = *reinterpret_cast<const float4*>(src + 32 * kt + 8 * q4 + 4 * g);
        S[kt][4 * q4 + 0] = x.x; S[kt][4 * q4 + 1] = x.y;
        S[kt][4 * q4 + 2] = x.z; S[kt][4 * q4 + 3] = x.w;
      }
  }
  // the state waves hold 2^E S (E wave-uniform, 0 unless the state or the
  // values left the band); stores give S itself, exactly
  int E = 0;
  auto store_state = [&](float* dst) {
    if (E == 0) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(dst + 32 * kt + 8 * q4 + 4 * g) =
              make_float4(S[kt][4 * q4], S[kt][4 * q4 + 1], S[kt][4 * q4 + 2], S[kt][4 * q4 + 3]);
    } else {
      auto un = [&](float x) { return __builtin_amdgcn_ldexpf(x, -E); };
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(dst + 32 * kt + 8 * q4 + 4 * g) =
              make_float4(un(S[kt][4 * q4]), un(S[kt][4 * q4 + 1]), un(S[kt][4 * q4 + 2]), un(S[kt][4 * q4 + 3]));
    }
  };

  // The scale of a chunk, from the chunk's largest |v| (vmax: bf16 bits,
  // recorded by the loader waves) and the largest |S| entry of the wave's
  // columns (unscaled: 2^-E times the held value); the held state is
  // rescaled when the scale changes (powers of two, exact).  Returns whether
  // it changed.
  auto chunk_vmax = [&](const float* sc) {
    const u32x4 vm4 = *reinterpret_cast<const u32x4*>(sc + SC_VM * CT);
    return __builtin_amdgcn_readfirstlane(max(max(vm4[0], vm4[1]), max(vm4[2], vm4[3])));
  };
  uint32_t vmax = 0;
  auto lane_absmax = [&]() {
    float ms = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ms = fmaxf(ms, fabsf(S[kt][i]));
    return ms;
  };
  auto rescale_if_needed = [&](uint32_t vmax, float ms) {
    const int eS = f32_exp(__uint_as_float(wave_max_u32(__float_as_uint(ms))));
    const int En = band_exp(max(eS == kNoExp ? kNoExp : eS - E, bf16_exp(vmax)));
    if (En == E) return false;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[kt][i] = __builtin_amdgcn_ldexpf(S[kt][i], En - E);
    E = En;
    return true;
  };

  // One 16-dim piece pc of row t of a q or k tile (bf16 bits, two 8-value
  // halves) to fp16 at dst (scaled by 2^ax), four values per step; returns
  // the row's sum of squares (each row's pieces sit on 8 neighbouring lanes).
  auto convert_piece = [&](const u32x4 (&x)[2], uint16_t* dst, int t, int pc, int ax) {
    float ss = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        float s1;
        const u32x2 f = bf16x4_to_f16_exp(u32x2{x[hh][2 * w2], x[hh][2 * w2 + 1]}, ax, s1);
        ss += s1;
        *reinterpret_cast<u32x2*>(dst + t * LDK + 16 * pc + 8 * hh + 4 * w2) = f;
        if (ax != 0) __builtin_amdgcn_sched_barrier(0);
      }
    return group_sum<8>(ss);
  };
  // The piece again when its row's sum of squares ss is outside the band:
  // scaled by 2^-e (e the binary exponent of the row's largest magnitude,
  // one tile at a time to bound the registers the rare path holds); ss
  // becomes the scaled row's, the scaling exponent is returned.
  auto rescale_piece = [&](const u32x4 (&x)[2], uint16_t* dst, int t, int pc, int n, float& ss) {
    uint32_t m = 0;   // the row's largest magnitude (bf16 bits)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = bf16_absmax(m, x[hh][i]);
    m = group_max_u32<8>(fold16(m));
    const bool ok = ss >= kQkLo && ss <= kQkHi;
    const int ax = (ok || m == 0 || t >= n) ? 0 : -bf16_exp(m);
    __builtin_amdgcn_sched_barrier(0);
    ss = convert_piece(x, dst, t, pc, ax);
    return ax;
  };

  // ---- a chunk's HBM rows into registers (loader waves), as in
  //      chunked_prefill_kernel: clamped row indices, 32-bit row offsets
  const uint32_t ksb = (uint32_t)a.k_stride * 2, qsb = (uint32_t)a.q_stride * 2;
  const uint32_t vsb = (uint32_t)a.v_stride * 2, hv = (uint32_t)a.Hv;
  auto row = [](const void* base, uint32_t off) { return static_cast<const char*>(base) + off; };
  // The loader waves hold two chunks' rows in flight in registers, loaded
  // two intervals ahead of their staging (an HBM round trip is longer than
  // an interval): rows of chunk c go to set c % 2.  Each role runs its own
  // loop, so the two sets are live only in the loader waves' loop and the
  // wait before a staging covers only its own set's loads.
  // K and Q come as row pieces of 16 key dims: loader thread e holds
  // dims 16 (e % 8) .. +15 of row e / 8, so a row's squares are summed over
  // 8 lanes
  struct Rows {
    u32x4 k[2], q[2];   // K and Q row pieces (2 x 8 bf16 each)
    u32x4 v[C::NVV];    // 16-byte V row pieces
    float g, b;         // log-gate and beta of token `lane`
    int n;              // the chunk's tokens
  };
  // the loader's walk over the chunks, in fetch order; once past the last
  // chunk a fetch takes the last chunk's rows again
  ChunkWalk fwalk;
  fwalk.init(seq0, seq1, ci0, ckp, a.n_ckpt);
  int last_t0 = seq0, last_n = 1;
  // the lane index as the loader uses it, formed where it is used: kept live
  // across the loader's loop it would be spilled, and its reload waits for
  // every row load in flight
  auto lane_here = [&]() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return (int)l;
  };
  auto fetch = [&](Rows& R) {
    const int lane = lane_here();
    int t0x, ck_at;
    int nx = fwalk.next(CT, ckp, a.n_ckpt, t0x, ck_at);
    if (nx <= 0) { t0x = last_t0; nx = last_n; }
    last_t0 = t0x;
    last_n = nx;
    R.n = nx;
    {
      const uint32_t t = min(ptid / 8, nx - 1), pb = 32 * (ptid % 8);
      const uint16_t* kb = kg + (size_t)t0x * a.k_stride + (size_t)j * DK;
      const uint16_t* qb = qg + (size_t)t0x * a.q_stride + (size_t)j * DK;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        R.k[hh] = *reinterpret_cast<const u32x4*>(row(kb, __umul24(t, ksb) + pb + 16 * hh));
        R.q[hh] = *reinterpret_cast<const u32x4*>(row(qb, __umul24(t, qsb) + pb + 16 * hh));
      }
    }
#pragma unroll
    for (int u = 0; u < C::NVV; ++u) {
      const int e = ptid + u * PTH;
      const uint32_t t = min(e / (DV / 8), nx - 1), c8 = (e % (DV / 8)) * 8;
      R.v[u] = *reinterpret_cast<const u32x4*>(row(vg + (size_t)t0x * a.v_stride, __umul24(t, vsb) + 2 * c8));
    }
    const uint32_t tl = min(lane, nx - 1);
    R.g = a.g[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
    R.b = a.beta[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
  };

  // Gram-type tile of two row-major fp16 tiles (row operands read first)
  auto rows_mm = [&](const uint16_t* xa, const uint16_t* xb) {
    f16x8 ar[NKS], br[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      ar[ks] = lds_op(xa + c * LDK + 4 * g + 16 * ks);
      br[ks] = lds_op(xb + c * LDK + 4 * g + 16 * ks);
    }
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mma(ar[ks], br[ks], acc);
    return acc;
  };

  // the loader waves' part of interval it; R holds the rows of chunk it and
  // takes those of chunk it + 2
  auto load_stage = [&](Rows& R, int it) {
    // ======== loader waves ========
    // -- staging of chunk it into its ring slot
    const int cs = it;
    if (cs < nch) {
      const int n = R.n;
      uint16_t* sK = ringK(cs);
      uint16_t* sQ = ringQ(cs);
      float* sc = ringSc(cs);
      const int t = ptid / 8, pc = ptid % 8;   // row, 16-dim piece
      u32x4 (&kx)[2] = R.k, (&qx)[2] = R.q;   // consumed here, refetched below
      if (t >= n) {   // a prompt's last chunk: rows past n are zeros
        kx[0] = kx[1] = qx[0] = qx[1] = u32x4{0u, 0u, 0u, 0u};
      }
      // rows converted as they are, then, when a row of the wave is far
      // from unit length (rare), that tile again with each such row scaled
      // by 2^a
      auto convert = [&](const u32x4 (&x)[2], uint16_t* dst, int ax) { return convert_piece(x, dst, t, pc, ax); };
      auto rescale = [&](const u32x4 (&x)[2], uint16_t* dst, float& ss) {
        return rescale_piece(x, dst, t, pc, n, ss);
      };
      float sk = convert(kx, sK, 0), sq = convert(qx, sQ, 0);
      auto off_band = [&](float ss) { return t < n && !(ss >= kQkLo && ss <= kQkHi); };
      int ak = 0, aq = 0;
      if (__builtin_amdgcn_ballot_w64(off_band(sk) || off_band(sq))) {   // rare
        // one copy of the rescaling for both tiles (a run-time pick)
#pragma unroll 1
        for (int w = 0; w < 2; ++w) {
          const u32x4 x[2] = {w ? qx[0] : kx[0], w ? qx[1] : kx[1]};
          float ss = w ? sq : sk;
          const int ax = rescale(x, w ? sQ : sK, ss);
          if (w) { aq = ax; sq = ss; } else { ak = ax; sk = ss; }
        }
      }
      if (pc == 7) {   // zero-padded rows keep r = 1
        sc[SC_RK * CT + t] = t < n ? row_factor(a.l2norm, sk, ak, a.eps) : 1.0f;
        sc[SC_RQ * CT + t] = t < n ? row_factor(a.l2norm, sq, aq, a.eps) : 1.0f;
      }
      if (wave == NSW) {   // betas and the base-2 cumsum of the log-gates
        const int lane = lane_here();
        const float xg = scan32(lane < n ? R.g : 0.f) * 1.44269504088896341f;
        if (lane < CT) {
          sc[SC_G * CT + lane] = xg;
          sc[SC_BETA * CT + lane] = lane < n ? R.b : 0.f;
        }
      }
    }
    if (cs < nch) {
      const int n = R.n;
      uint16_t* sV = ringV(cs);
      uint32_t vm = 0;   // the chunk's largest |v| (bf16 bits), per loader wave
#pragma unroll
      for (int u = 0; u < C::NVV; ++u) {
        const int e = ptid + u * PTH;
        const int t = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
        const u32x4 vx = t < n ? R.v[u] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sV + t * LDV + c8) = vx;
#pragma unroll
        for (int i = 0; i < 4; ++i) vm = bf16_absmax(vm, vx[i]);
      }
      vm = wave_max_u32(fold16(vm));
      if (lane_here() == 0) reinterpret_cast<uint32_t*>(ringSc(cs))[SC_VM * CT + wave - NSW] = vm;
    }
    // -- the rows of chunk it + 2 into R (past the last chunk the last
    //    chunk's rows again: the loads stay unconditional, so the wait for a
    //    set never has to assume the other set was not issued)
    fetch(R);
  };

  // ---- the short conv in the loads (CONV): the loader waves read the
  //      pre-conv rows x and apply the width-4 causal conv and SiLU.  The
  //      four loader waves split a chunk's rows: wave lw convolves rows
  //      8 lw .. 8 lw + 7 of the three tensors, two channels per lane of
  //      each (q and k of qk head j, v of head h), from those rows and the
  //      three before them, all requested one interval ahead; before the
  //      prompt's first token the three inputs come from its conv state (or
  //      are zeros).  Wave lw 3 also loads the gates.  The conv output,
  //      rounded to bf16 in conv1d_silu's operation order, is written to the
  //      ring slot as bf16; the Gram and K Q^T waves convert the k and q
  //      tiles to fp16 in place (convert_tile), with the sums and scalings of
  //      the unfused staging, so the scan sees the values, norms and scales
  //      the separate conv and scan give.
  const int lw = wave - NSW;
  constexpr int XR = CT / C::NLW;   // rows per loader wave
  constexpr int XH = XR + 3;        // with the three before them
  uint32_t xoff[3] = {0u, 0u, 0u};  // the lane's channel pair in q, k, v (element index in a row)
  float cw[3][2][4];                // its conv weights (taps as the conv kernel scales them)
  // the q/k windows are written by the first value head of each qk head
  const bool own_qk = h % (a.Hv / a.Hqk) == 0;
  if constexpr (CONV) {
    if (wave >= NSW && wave < NSW + C::NLW) {
      xoff[0] = (uint32_t)(j * DK + 2 * lane);
      xoff[1] = (uint32_t)((a.Hqk + j) * DK + 2 * lane);
      xoff[2] = (uint32_t)(2 * a.Hqk * DK + h * DV + 2 * lane);
#pragma unroll
      for (int tn = 0; tn < 3; ++tn)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const float4 w4 = reinterpret_cast<const float4*>(a.conv_w)[xoff[tn] + c2];
          cw[tn][c2][0] = conv_tap(w4.x); cw[tn][c2][1] = conv_tap(w4.y);
          cw[tn][c2][2] = conv_tap(w4.z); cw[tn][c2][3] = conv_tap(w4.w);
        }
    }
  }
  // the lane's channel pair of tensor tn at token position p of this
  // prompt or, before its first token, from its conv state (zeros without
  // one), as a bf16 pair
  auto x_input = [&](int p, int tn) -> uint32_t {
    // (the offset passed through an empty asm: these rare reads' addresses
    // are then formed here, not hoisted out of the loader's loop into
    // registers it has none to spare for)
    uint32_t xo = xoff[tn];
    asm volatile("" : "+v"(xo));
    if (p >= seq0)
      return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.conv_x) +
                                                (size_t)p * a.conv_x_stride + xo);
    if (!a.conv_state_in) return 0u;
    return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.conv_state_in) +
                                              ((size_t)s * 3 + (p - seq0 + 3)) * a.conv_dim + xo);
  };
  // the three inputs before position e as a conv window at dst3 ([3,
  // conv_dim]); all reads come before the writes (dst3 may be the state read)
  auto write_window = [&](void* dst3, int e) {
    uint32_t w[3][3];
#pragma unroll
    for (int tn = 0; tn < 3; ++tn)
#pragma unroll
      for (int i = 0; i < 3; ++i) w[tn][i] = x_input(e - 3 + i, tn);
    uint16_t* d = static_cast<uint16_t*>(dst3);
#pragma unroll
    for (int tn = 0; tn < 3; ++tn)
      if (tn == 2 || own_qk) {
        uint32_t xo = xoff[tn];
        asm volatile("" : "+v"(xo));
#pragma unroll
        for (int i = 0; i < 3; ++i) *reinterpret_cast<uint32_t*>(d + (size_t)i * a.conv_dim + xo) = w[tn][i];
      }
  };
  // One register set of raw rows: once the conv has consumed a chunk's rows
  // the next chunk's are requested into the same registers, so each row has
  // about an interval to arrive.
  struct RowsX {
    uint32_t x[XH][3];  // rows 8 lw - 3 .. 8 lw + 7 of the chunk: the lane's pair of q, k, v
    float g, b;         // log-gate and beta of token `lane` (wave lw 3)
    int n, ck, t0;      // the chunk's tokens, the checkpoint it ends at (or -1), its first token
    int zero;           // rows r < 3 to take as zeros (before the prompt, no conv state)
  };
  // the walk's next chunk (past the last one: the last again, no checkpoint)
  auto next_x = [&](int& t0x, int& nx, int& ck_at) {
    nx = fwalk.next(CT, ckp, a.n_ckpt, t0x, ck_at);
    if (nx <= 0) { t0x = last_t0; nx = last_n; ck_at = -1; }
    last_t0 = t0x;
    last_n = nx;
  };
  // The wave's rows of the chunk at t0x: row t = 8 lw - 3 + r (clamped to
  // the chunk's last row), each load from a wave-uniform base in scalar
  // registers and a 32-bit offset per lane (a row's bytes times at most 34
  // plus the lane's channels: below 2^32 for token strides under 2^23), with
  // no branch: a row before the prompt's first token (wave 0 only) reads the
  // prompt's conv state, or, without one, a row that is then taken as zeros.
  typedef const char __attribute__((address_space(1)))* GlobalBytes;
  auto uniform_base = [&](uint64_t p) {
    // (each half taken as unsigned: the builtin returns int, whose widening
    // would copy the low half's top bit into the high half)
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    return reinterpret_cast<GlobalBytes>(((uint64_t)hi << 32) | (uint64_t)lo);
  };
  auto fetch_x = [&](RowsX& R, int t0x, int nx) {
    const uint32_t rb = (uint32_t)a.conv_x_stride * 2;
    const uint64_t xb = reinterpret_cast<uint64_t>(a.conv_x) + ((uint64_t)t0x - 3) * (uint64_t)rb;
    int zero = 0;
#pragma unroll
    for (int r = 0; r < XH; ++r) {
      const int t = XR * lw - 3 + r;
      uint64_t base = xb;
      uint32_t roff = (uint32_t)(min(t, nx - 1) + 3) * rb;
      if (r < 3) {
        const bool hist = lw == 0 && t0x + t < seq0;   // before the prompt's first token
        const uint64_t hb = a.conv_state_in
            ? reinterpret_cast<uint64_t>(a.conv_state_in) + ((uint64_t)s * 3 + (t0x + t - seq0 + 3)) * a.conv_dim * 2
            : reinterpret_cast<uint64_t>(a.conv_x);
        base = hist ? hb : xb;
        roff = hist ? 0u : roff;
        zero |= (hist && !a.conv_state_in) ? 1 << r : 0;
      }
      const GlobalBytes bp = uniform_base(base);
#pragma unroll
      for (int tn = 0; tn < 3; ++tn)
        R.x[r][tn] = *reinterpret_cast<const uint32_t __attribute__((address_space(1)))*>(bp + (roff + 2 * xoff[tn]));
    }
    R.zero = zero;
    R.t0 = t0x;
  };
  auto gates_x = [&](RowsX& R, int t0x, int nx) {
    const uint32_t tl = min(lane, nx - 1);
    R.g = a.g[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
    R.b = a.beta[(size_t)t0x * a.Hv + h + __umul24(tl, hv)];
  };
  auto first_x = [&](RowsX& R) {
    int t0x, nx, ck_at;
    next_x(t0x, nx, ck_at);
    R.n = nx;
    R.ck = ck_at;
    fetch_x(R, t0x, nx);
    if (lw == 3) gates_x(R, t0x, nx);
  };
  // the loader waves' part of interval it with the conv: chunk it staged
  // from R, which takes the rows of chunk it + 1
  auto load_stage_x = [&](RowsX& R, int it) {
    int t0n, nn, ckn;
    next_x(t0n, nn, ckn);
    const int cs = it;
    if (cs < nch) {
      const int n = R.n;
      float* sc = ringSc(cs);
      uint32_t* dcol[3] = {reinterpret_cast<uint32_t*>(ringQ(cs)) + lane, reinterpret_cast<uint32_t*>(ringK(cs)) + lane,
                           reinterpret_cast<uint32_t*>(ringV(cs)) + lane};
      constexpr int ldw[3] = {LDK / 2, LDK / 2, LDV / 2};
      uint32_t vm = 0;   // the largest |v| of the wave's rows (bf16 bits)
      if (R.zero) {   // rows before the prompt with no conv state: zeros (rare)
#pragma unroll
        for (int r = 0; r < 3; ++r)
          if (R.zero & (1 << r))
#pragma unroll
            for (int tn = 0; tn < 3; ++tn) R.x[r][tn] = 0u;
      }
      // row 8 lw + r of the chunk: conv + SiLU of its three tensors from
      // the wave's rows r .. r + 3 (zeros past n)
      auto conv_row = [&](int r, bool valid) {
        const int t = XR * lw + r;
#pragma unroll
        for (int tn = 0; tn < 3; ++tn) {
          uint32_t o = 0;
          if (valid) {
            float y[2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
              auto in = [&](int q) {
                const uint32_t u = R.x[r + q][tn];
                return c2 == 0 ? __uint_as_float(u << 16) : __uint_as_float(u & 0xFFFF0000u);
              };
              y[c2] = conv4_silu(cw[tn][c2][0], cw[tn][c2][1], cw[tn][c2][2], cw[tn][c2][3], in(0), in(1), in(2),
                                 in(3));
            }
            o = pack_bf16(y[0], y[1]);
          }
          dcol[tn][t * ldw[tn]] = o;
          if (tn == 2) vm = bf16_absmax(vm, o);
        }
      };
      if (XR * lw + XR <= n) {   // all the wave's rows in the chunk: no branches
#pragma unroll
        for (int r = 0; r < XR; ++r) {
          conv_row(r, true);
          __builtin_amdgcn_sched_barrier(0);   // one row at a time: wider, the loop spills
        }
      } else {
#pragma unroll
        for (int r = 0; r < XR; ++r) conv_row(r, XR * lw + r < n);
      }
      if (lw == 0) {   // conv windows: at a checkpoint, and the prompt's conv state
        if (R.ck >= 0 && a.conv_ckpt)
          write_window(static_cast<uint16_t*>(a.conv_ckpt) + (size_t)R.ck * 3 * a.conv_dim, R.t0 + n);
        if (cs == nch - 1 && a.conv_state_own)
          write_window(static_cast<uint16_t*>(a.conv_state_out) + (size_t)s * 3 * a.conv_dim, R.t0 + n);
      }
      // the next chunk's rows, requested in one place (defined once per
      // trip, the loop-carried registers need no copies, whose waits would
      // drain these loads)
      fetch_x(R, t0n, nn);
      vm = wave_max_u32(fold16(vm));
      if (lw == 3) {   // betas and the base-2 cumsum of the log-gates
        const float xg = scan32(lane < n ? R.g : 0.f) * 1.44269504088896341f;
        if (lane < CT) {
          sc[SC_G * CT + lane] = xg;
          sc[SC_BETA * CT + lane] = lane < n ? R.b : 0.f;
        }
        if (lane == 0) reinterpret_cast<int*>(sc)[SC_VM * CT + 4] = n;   // for the factor waves
        gates_x(R, t0n, nn);
      }
      // the chunk's largest |v| (bf16 bits): one partial per loader wave
      if (lane == 0) reinterpret_cast<uint32_t*>(sc)[SC_VM * CT + lw] = vm;
    }
    R.n = nn;
    R.ck = ckn;
  };

  // A staged bf16 q or k tile of n rows to fp16 in place (CONV), eight rows
  // per pass with the unfused staging's lane layout (lane 8 r + pc: piece pc
  // of row r), pieces, sums and scalings, so the values and the row factors
  // rf[t] are the unfused kernel's.
  auto convert_tile = [&](uint16_t* sT, float* rf, int n) {
#pragma unroll 2   // two passes at a time (four: the factor loop spills)
    for (int p8 = 0; p8 < CT / 8; ++p8) {
      const int t = 8 * p8 + lane / 8, pc = lane % 8;
      u32x4 x[2];   // 8-byte reads: rows are 8-byte aligned
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(sT + t * LDK + 16 * pc + 8 * hh);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(sT + t * LDK + 16 * pc + 8 * hh + 4);
        x[hh] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      float ss = convert_piece(x, sT, t, pc, 0);
      int ax = 0;
      if (__builtin_amdgcn_ballot_w64(t < n && !(ss >= kQkLo && ss <= kQkHi)))   // rare
        ax = rescale_piece(x, sT, t, pc, n, ss);
      if (pc == 7) rf[t] = t < n ? row_factor(a.l2norm, ss, ax, a.eps) : 1.0f;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the fp16 rows written before the wave reads them
  };
  auto chunk_n = [&](const float* sc) { return reinterpret_cast<const int*>(sc)[SC_VM * CT + 4]; };

  // A[t][i] = beta_t r_t r_i e^{G_t - G_i} k_t.k_i (i < t) of chunk cg,
  // stored transposed with rows interleaved over the substitution's lane
  // parts, and the state path's per-token factors (with CONV the k tile is
  // converted to fp16 here first)
  auto gram = [&](int cg) {
    uint16_t* sK = ringK(cg);
    float* sc = ringSc(cg);
    float* sA = bufA(cg);
    f32x16 acc;
    if constexpr (CONV) {
      convert_tile(sK, sc + SC_RK * CT, chunk_n(sc));
      if (lane < CT) {
        const float G = sc[SC_G * CT + lane], lr = __builtin_amdgcn_logf(sc[SC_RK * CT + lane]);
        sc[SC_LA * CT + lane] = G + (__builtin_amdgcn_logf(sc[SC_BETA * CT + lane]) + lr);
        sc[SC_LK0 * CT + lane] = G - lr;
      }
      acc = rows_mm(sK, sK);
    } else {
      if (lane < CT) {
        const float G = sc[SC_G * CT + lane], lr = __builtin_amdgcn_logf(sc[SC_RK * CT + lane]);
        sc[SC_LA * CT + lane] = G + (__builtin_amdgcn_logf(sc[SC_BETA * CT + lane]) + lr);
        sc[SC_LK0 * CT + lane] = G - lr;
      }
      acc = rows_mm(sK, sK);
    }
    const float lki = sc[SC_LK0 * CT + c];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int tb = 8 * q4 + 4 * g;
      const float4 L4 = *reinterpret_cast<const float4*>(sc + SC_LA * CT + tb);
      const float La[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb + r;
        const float f = exp2f_hw(La[r] - lki) * acc[4 * q4 + r];
        sA[c * LDA + (t % LPC) * MPL + MPL - 1 - t / LPC] = c < t ? f : 0.f;
      }
    }
    if (lane < CT) {
      const float G = sc[SC_G * CT + lane], GC = sc[SC_G * CT + CT - 1];
      const float rk = sc[SC_RK * CT + lane];
      sc[SC_CK * CT + lane] = rk * exp2f_hw(G);
      if constexpr (!CONV) sc[SC_CQ * CT + lane] = a.scale * sc[SC_RQ * CT + lane] * exp2f_hw(G);
      sc[SC_CU * CT + lane] = rk * exp2f_hw(GC - G);
    }
  };
  // the q tile of chunk cq to fp16 (CONV) and its output factor
  auto convert_q = [&](int cq) {
    float* sc = ringSc(cq);
    convert_tile(ringQ(cq), sc + SC_RQ * CT, chunk_n(sc));
    if (lane < CT) sc[SC_CQ * CT + lane] = a.scale * sc[SC_RQ * CT + lane] * exp2f_hw(sc[SC_G * CT + lane]);
  };
  // P[t][i] = scale r_q,t r_k,i e^{G_t - G_i} q_t.k_i (i <= t) of chunk cp, row t fp16
  auto kq = [&](int cp) {
    float* sc = ringSc(cp);
    uint16_t* sP = ringP(cp);
    if (lane < CT) {
      const float G = sc[SC_G * CT + lane];
      sc[SC_LQ * CT + lane] = G + __builtin_amdgcn_logf(sc[SC_RQ * CT + lane]);
      sc[SC_LK1 * CT + lane] = G - __builtin_amdgcn_logf(sc[SC_RK * CT + lane]);
    }
    const f32x16 acc = rows_mm(ringK(cp), ringQ(cp));
    const float lqt = sc[SC_LQ * CT + c];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ib = 8 * q4 + 4 * g;
      const float4 L4 = *reinterpret_cast<const float4*>(sc + SC_LK1 * CT + ib);
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
  };

  // the factor waves' part of interval it: the Gram tile of chunk it - 1
  // (wave NSW + NLW), the K Q^T tile of chunk it - 1 (the next wave; with
  // CONV it converts the q tile of chunk it - 1 and forms the K Q^T tile of
  // chunk it - 2), the substitution of chunk it - 2 (the other two)
  auto factor = [&](int it) {
    const int fw = wave - NSW - C::NLW, ftid = tid - C::F0;
    const int cg = it - 1;
    if (fw == 0) {
      if (cg >= 0 && cg < nch) gram(cg);
    } else if (fw == 1) {
      if constexpr (CONV) {
        if (cg >= 0 && cg < nch) convert_q(cg);
        if (cg >= 1 && cg - 1 < nch) kq(cg - 1);
      } else {
        if (cg >= 0 && cg < nch) kq(cg);
      }
    }

    // -- T = (I + A)^-1 of chunk it - 2 (waves 6, 7): right-looking forward
    //    substitution as in chunked_prefill_kernel, LPC lanes per column
    const int cb = it - 2;
    if (cb >= 0 && cb < nch && ftid >= C::SUB0) {
      const int st = ftid - C::SUB0;
      const int jj = st / LPC, q = st % LPC;
      const float* ab = bufA(cb) + q * MPL;
      float Tl[MPL];
#pragma unroll
      for (int m = 0; m < MPL; ++m) Tl[m] = (q + LPC * m == jj) ? 1.f : 0.f;
      constexpr int SB = 4, NB = CT / SB;
      float col[2][SB][MPL];
      auto load_batch = [&](float (&dst)[SB][MPL], int bt) {
#pragma unroll
        for (int u = 0; u < SB; ++u)
#pragma unroll
          for (int p4 = 0; p4 < MPL; p4 += 4) {
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
        for (int u = 0; u < SB; ++u) {
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
      uint16_t* tcol = bufT(cb) + jj;
#pragma unroll
      for (int m = 0; m < MPL; ++m) tcol[(q + LPC * m) * LDT] = f16_bits(Tl[m]);
    }
  };

  // intervals: nch + 3, rounded up to even so that the loader loop
  // runs both of its halves on every trip (the extra interval is empty)
  const int nint = (nch + 4) & ~1;
  if (wave < NSW) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the state loads drained before the loop
    ChunkWalk swalk;
    swalk.init(seq0, seq1, ci0, ckp, a.n_ckpt);
    for (int it = 0; it < nint; ++it) {
      // ======== state path of chunk it - 3 ========
      const int cx = it - 3;
      if (cx >= 0 && cx < nch) {
        int t0, ck_at;
        const int n = swalk.next(CT, ckp, a.n_ckpt, t0, ck_at);
        const uint16_t* sK = ringK(cx);
        const uint16_t* sQ = ringQ(cx);
        uint16_t* sV = ringV(cx);
        const float* sc = ringSc(cx);
        const float* sBeta = sc + SC_BETA * CT;
        const float* sCk = sc + SC_CK * CT;
        const float* sCq = sc + SC_CQ * CT;
        const float* sCu = sc + SC_CU * CT;
        // X = K S0^T and QS = S0 Q^T for this wave's columns (S0 rounded to
        // fp16 per k tile); the chunk's decay e^{G_C} is applied to S at the
        // update.  The products are formed with the scale of the chunk
        // before, while the chunk's own scale is chosen beside them; when it
        // differs (rare) the held state is rescaled and the products formed
        // again, so every chunk runs at its own scale and the update's
        // results are not waited for before the barrier.
        f32x16 X, QS;
        u32x2 vw[4];
        float gC;
        {
          if (cx == 0) vmax = chunk_vmax(sc);
          auto products = [&]() {
            f16x8 ka[NKS], qa[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              ka[ks] = lds_op(sK + c * LDK + 4 * g + 16 * ks);
              qa[ks] = lds_op(sQ + c * LDK + 4 * g + 16 * ks);
            }
            X = f32x16{};
            QS = f32x16{};
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const f16x8 sh = h2 == 0 ? acc_half<0>(S[kt]) : acc_half<1>(S[kt]);
                X = mma(ka[2 * kt + h2], sh, X);
                QS = mma(sh, qa[2 * kt + h2], QS);
              }
          };
          products();
          // the lane's largest |S| for the scale choice, in the same region
          // as the products (its maxima fill the matrix pipe's shadow)
          const float ms = lane_absmax();
          // V of this wave's columns by transpose reads (raw bf16, before the
          // scale is known), their latency under the scale choice
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) vw[q4] = lds_tr4(sV + vtr + 8 * q4 * LDV);
          __builtin_amdgcn_sched_barrier(0);
          if (__builtin_expect(rescale_if_needed(vmax, ms), 0)) {   // rare: the scale changed
            __builtin_amdgcn_sched_barrier(0);
            products();
          }
          // the next chunk's largest |v|, staged two intervals ago
          if (cx + 1 < nch) vmax = chunk_vmax(ringSc(cx + 1));
          gC = exp2f_hw(sc[SC_G * CT + CT - 1]);
        }
        // V to fp32 (scaled by 2^E), then the T and P row operands and the
        // K^T operands of the update, requested ahead
        const uint16_t* tr = bufT(cx) + c * LDT + 4 * g;
        const uint16_t* pr = ringP(cx) + c * LDT + 4 * g;
        // beta and r_k e^G of the lane's 16 tokens, requested before the V
        // conversion so that Y does not wait for them
        float4 b4s[4], k4s[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          b4s[q4] = *reinterpret_cast<const float4*>(sBeta + 8 * q4 + 4 * g);
          k4s[q4] = *reinterpret_cast<const float4*>(sCk + 8 * q4 + 4 * g);
        }
        float vv[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 w = vw[q4];
          vv[4 * q4] = __uint_as_float(w.x << 16);
          vv[4 * q4 + 1] = __uint_as_float(w.x & 0xFFFF0000u);
          vv[4 * q4 + 2] = __uint_as_float(w.y << 16);
          vv[4 * q4 + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
        if (E != 0)
#pragma unroll
          for (int i = 0; i < 16; ++i) vv[i] = __builtin_amdgcn_ldexpf(vv[i], E);
        __builtin_amdgcn_sched_barrier(0);
        const f16x8 tA[2] = {lds_op(tr), lds_op(tr + 16)};
        // Y = beta (V - r_k e^G X), in place of X (rows past n: exact zeros)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 b4 = b4s[q4], k4 = k4s[q4];
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) X[4 * q4 + r] = bb[r] * (vv[4 * q4 + r] - kk[r] * X[4 * q4 + r]);
        }
        const f16x8 pA[2] = {lds_op(pr), lds_op(pr + 16)};
        const float cq = sCq[c];   // ahead of the K^T reads: its wait leaves them in flight
        f16x8 kta[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint16_t* p = sK + ktr + 16 * (ks % 2) * LDK + 32 * (ks / 2);
          const u32x2 lo = lds_tr4(p), hi = lds_tr4(p + 8 * LDK);
          kta[ks] = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
        // U = T Y
        f32x16 U = {};
        U = mma(tA[0], acc_half<0>(X), U);
        U = mma(tA[1], acc_half<1>(X), U);
        // the S0 Q^T part of the output: scale r_q e^G per token
#pragma unroll
        for (int i = 0; i < 16; ++i) QS[i] *= cq;
        // O^T = scale r_q e^G (S0 Q^T) + U^T P^T, token t = c per lane: its
        // two products go ahead of the update's eight, so the output rows
        // are stored while the update is still in the matrix pipe
        const f16x8 uo[2] = {acc_half<0>(U), acc_half<1>(U)};
        QS = mma(uo[0], pA[0], QS);
        QS = mma(uo[1], pA[1], QS);
        // S = (e^{G_C} S0) + K^T (r_k e^{G_C - G} U)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 c4 = *reinterpret_cast<const float4*>(sCu + 8 * q4 + 4 * g);
          U[4 * q4] *= c4.x; U[4 * q4 + 1] *= c4.y;
          U[4 * q4 + 2] *= c4.z; U[4 * q4 + 3] *= c4.w;
        }
        const f16x8 uh[2] = {acc_half<0>(U), acc_half<1>(U)};
        // each tile decayed just before its first product
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kt][i] *= gC;
          S[kt] = mma(kta[2 * kt], uh[0], S[kt]);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) S[kt] = mma(kta[2 * kt + 1], uh[1], S[kt]);
        // the wave's 32 columns of output row t (64 bytes) go to HBM in two
        // stores: the lane pair of row t (lane halves g = 0, 1, 8-byte pieces
        // at 16 q4 + 8 g) trade pieces so that each store writes 32
        // contiguous bytes of the row
        if (E != 0)
#pragma unroll
          for (int i = 0; i < 16; ++i) QS[i] = __builtin_amdgcn_ldexpf(QS[i], -E);
        {
          uint32_t P[4][2];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            P[q4][0] = pack_bf16(QS[4 * q4], QS[4 * q4 + 1]);
            P[q4][1] = pack_bf16(QS[4 * q4 + 2], QS[4 * q4 + 3]);
          }
          // half g = 0 takes the other half's pieces q4 = 0, 2; half 1 takes q4 = 1, 3
#pragma unroll
          for (int pr2 = 0; pr2 < 4; pr2 += 2)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const auto r = __builtin_amdgcn_permlane32_swap(P[pr2][d], P[pr2 + 1][d], false, false);
              P[pr2][d] = r[0];
              P[pr2 + 1][d] = r[1];
            }
          if (c < n) {
            uint16_t* orow = og + (size_t)(t0 + c) * a.Hv * DV + 32 * wave + 8 * g;
            *reinterpret_cast<u32x4*>(orow) = u32x4{P[0][0], P[0][1], P[1][0], P[1][1]};
            *reinterpret_cast<u32x4*>(orow + 16) = u32x4{P[2][0], P[2][1], P[3][0], P[3][1]};
          }
        }
        if (ck_at >= 0) store_state(a.ckpt_buf + (size_t)ck_at * sstride + ((size_t)h * DV + v) * DK);
      }
      __syncthreads();
    }
  } else if (wave >= NSW + C::NLW) {
    for (int it = 0; it < nint; ++it) {
      factor(it);
      __syncthreads();
    }
  } else if (nch > 0) {
    if constexpr (CONV) {
      RowsX R;
      first_x(R);
      for (int it = 0; it < nint; ++it) {
        load_stage_x(R, it);
        __syncthreads();
      }
    } else {
      Rows R0, R1;
      fetch(R0);
      __builtin_amdgcn_sched_barrier(0);   // chunk 0's loads first: the first staging waits for them alone
      fetch(R1);
      for (int it = 0; it < nint; it += 2) {   // two intervals per trip: R0 even, R1 odd
        load_stage(R0, it);
        __syncthreads();
        load_stage(R1, it + 1);
        __syncthreads();
      }
    }
  } else {
    // an empty prompt: its conv state passes through
    if constexpr (CONV)
      if (lw == 0 && a.conv_state_own)
        write_window(static_cast<uint16_t*>(a.conv_state_out) + (size_t)s * 3 * a.conv_dim, seq0);
    for (int it = 0; it < nint; ++it) __syncthreads();
  }
  if (wave < NSW && a.final_state)
    store_state(a.final_state + (size_t)s * sstride + ((size_t)h * DV + v) * DK);
}

}  // namespace chunked
}  // namespace gdn
