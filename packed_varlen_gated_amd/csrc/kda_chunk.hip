// Chunked packed KDA forward on CDNA4 matrix cores (bf16 tensors, Dk, Dv in {64, 128}).
//
// Computes what RFC-0026 "Ling3 KDA varlen support" defines in its Background
// section (KDA state leakage problem) with the reset of section 3.1.1:
//   S_t = diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,  o_t = scale * S_t^T q_t,
// S = 0 at every segment start; segments from cu_seqlens (RFC-0025 Design
// sections 1 and 2). The page's own kernels (a TPU Pallas chunk_kda with
// _align_seqs, chunk_local_cumsum_vector and kda_fwd_intra stages) are prior
// art; this kernel keeps the chunked idea but aligns chunks to segment starts
// by index arithmetic, so no chunk straddles a document and no padded copy of
// the sequence is ever built.
//
// Math per 64-token chunk (b_r = in-chunk inclusive cumsum of g, base 2):
//   o_r    = S_prev^T (q_r 2^{b_r})  +  sum_{s<=r} A[r,s] v_s
//   A[r,s] = beta_s sum_d q_r[d] k_s[d] 2^{b_r[d] - b_s[d]}
//   S_new  = diag(2^{b_C}) S_prev + sum_s (beta_s k_s 2^{b_C - b_s}) v_s^T
// Stable exponents: the chunk is cut into four 16-token sub-chunks; rho_j is
// the cumsum before sub-chunk j and T_j its total. Block (w, j) of A (rows in
// sub-chunk w, columns in sub-chunk j <= w) pairs the key factor
// KE_s = k_s 2^{rho_{j+1} - b_s} (<= 1) with the query factor
// q_r 2^{b_r - rho_{j+1}} (<= 1 off the diagonal, <= 2^{16 max|g| log2 e} on
// it). Per element only 2^{c} and 2^{T - c} are evaluated (c = in-sub-chunk
// cumsum); every other factor is per channel.
//
// Work-group: Dv/16 waves (8 at Dv = 128, two per SIMD) per (segment, head).
// Wave e owns the fp32 state columns [16e, 16e + 16) in registers.
//  1. prep: wave w takes sub-chunk w%4 and a share of the channels; lane =
//     4 tokens x CPL channels (8-byte buffer loads; rows past the chunk end
//     read 0 through the buffer range check). In-lane prefix + DPP quad scan
//     give c; sub-chunk totals go to LDS.                              barrier
//     Per-channel factors (one lane of each quad per channel, DPP broadcast),
//     then bf16 operands to LDS: Q^ = q 2^b, the query versions of the ten A
//     blocks, KE, Kbar^T = (beta k 2^{b_C - b})^T, V^T. The next chunk's
//     loads are issued here.                                            barrier
//  2. the ten A blocks (plus two zero blocks) on MFMA, masked and
//     beta-scaled, to LDS.                                              barrier
//  3. o^T = S^T Q^^T + V^T A^T for the wave's 16 columns, stored;
//     S = diag(2^{b_C}) S + Kbar^T V.                                   barrier
// MFMA v_mfma_f32_16x16x32_bf16: A operand lane l holds row l%16 and eight
// contraction slots of lane group l/16, B likewise for column l%16; the 16x16
// fp32 result has column l%16 and rows 4(l/16)+i. The contraction index may be
// permuted freely when A and B agree, so S^T is fed straight from the S
// accumulators (slots {4g..4g+3} of two adjacent 16-row tiles) and Q^ is read
// with the same permutation.

#include "common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr int kTailBlocks = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// A blocks (row sub-chunk w, column sub-chunk j), j <= w, in this order; the
// query version of block b lives in LDS slot b. Jobs 10 and 11 zero the blocks
// (0, 1) and (2, 3), which the A.V product reads through its 32-wide steps.
__device__ __forceinline__ void block_of(int b, int& w, int& j) {
  if (b < 1) { w = 0; j = 0; }
  else if (b < 3) { w = 1; j = b - 1; }
  else if (b < 6) { w = 2; j = b - 3; }
  else if (b < 10) { w = 3; j = b - 6; }
  else if (b == 10) { w = 0; j = 1; }
  else { w = 2; j = 3; }
}

template <int DK, int DV>
struct Cfg {
  static constexpr int NW = DV / 16;      // waves
  static constexpr int NT = NW * 64;      // threads (= 4 * DV, the launch bound)
  static constexpr int HALVES = NW / 4;   // channel shares per sub-chunk in the prep
  static constexpr int CPL = DK / HALVES / 16;  // prep channels per lane
  static constexpr int VPL = DV / HALVES / 16;  // staged v channels per lane
  static constexpr int DT = DK / 16;      // 16-row state tiles
  static constexpr int KS = DK / 32;      // contraction steps over Dk
  static constexpr int KP = DK + 8;       // token-major LDS rows (bf16 elements)
  static constexpr int TP = kC + 8;       // transposed / A rows (bf16 elements)
  static constexpr int off_qh = 0;
  static constexpr int off_qv = off_qh + kC * KP * 2;
  static constexpr int off_ke = off_qv + 10 * 16 * KP * 2;
  static constexpr int off_kbT = off_ke + kC * KP * 2;
  static constexpr int off_vT = off_kbT + DK * TP * 2;
  static constexpr int off_a = off_vT + DV * TP * 2;
  static constexpr int off_T = off_a + kC * TP * 2;      // float [4][DK]
  static constexpr int off_decay = off_T + 4 * DK * 4;   // float [DK]
  static constexpr int off_beta = off_decay + DK * 4;    // float [kC]
  static constexpr int bytes = off_beta + kC * 4;
  static_assert(CPL >= 2 && CPL <= 8 && VPL >= 2 && VPL <= 8, "prep layout");
};

template <int n>
struct alignas(2 * n) BfPack {
  bf16 v[n];
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Quad-permute DPP move (lane i of each quad receives lane SEL[i]).
template <int CTRL>
__device__ __forceinline__ float qperm(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int L>
__device__ __forceinline__ float qbcast(float x) {
  return qperm<L | (L << 2) | (L << 4) | (L << 6)>(x);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufFlags);
}

// n bf16 values from a raw buffer (n in {2, 4, 8}); out-of-range reads give 0.
template <int n>
__device__ __forceinline__ BfPack<n> bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  BfPack<n> p;
  if constexpr (n == 2) {
    const int x = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    __builtin_memcpy(&p, &x, 4);
  } else if constexpr (n == 4) {
    typedef int v2 __attribute__((ext_vector_type(2)));
    const v2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    __builtin_memcpy(&p, &x, 8);
  } else {
    typedef int v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    __builtin_memcpy(&p, &x, 16);
  }
  return p;
}

template <int n>
__device__ __forceinline__ void lds_put(bf16* dst, const float* x) {
  BfPack<n> p;
#pragma unroll
  for (int c = 0; c < n; ++c) p.v[c] = from_f32<bf16>(x[c]);
  *reinterpret_cast<BfPack<n>*>(dst) = p;
}

template <int DK, int DV>
__global__ __launch_bounds__(4 * DV, 1) void kda_chunk_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const int32_t* __restrict__ cu,
    int32_t max_segs, int64_t N, int32_t H, float scale, bf16* __restrict__ o,
    float* __restrict__ final_state, int32_t* __restrict__ flags) {
  using C = Cfg<DK, DV>;
  constexpr int NT = C::NT, CPL = C::CPL, VPL = C::VPL, DT = C::DT, KS = C::KS;
  constexpr int KP = C::KP, TP = C::TP;

  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* s_qh = reinterpret_cast<bf16*>(smem + C::off_qh);
  bf16* s_qv = reinterpret_cast<bf16*>(smem + C::off_qv);
  bf16* s_ke = reinterpret_cast<bf16*>(smem + C::off_ke);
  bf16* s_kbT = reinterpret_cast<bf16*>(smem + C::off_kbT);
  bf16* s_vT = reinterpret_cast<bf16*>(smem + C::off_vT);
  bf16* s_a = reinterpret_cast<bf16*>(smem + C::off_a);
  float* s_T = reinterpret_cast<float*>(smem + C::off_T);
  float* s_decay = reinterpret_cast<float*>(smem + C::off_decay);
  float* s_beta = reinterpret_cast<float*>(smem + C::off_beta);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;
  const int lr = lane & 15;
  const int64_t seg_blocks = int64_t(max_segs) * H;

  if (int64_t(blockIdx.x) >= seg_blocks) {
    // Positions not covered by any segment get o = 0.
    int64_t cu_last = cu ? int64_t(cu[max_segs]) : N;
    cu_last = cu_last < 0 ? 0 : (cu_last > N ? N : cu_last);
    const int64_t total = (N - cu_last) * H * DV;
    const int64_t base = cu_last * H * DV;
    for (int64_t i = (int64_t(blockIdx.x) - seg_blocks) * NT + tid; i < total;
         i += int64_t(kTailBlocks) * NT)
      o[base + i] = from_f32<bf16>(0.f);
    return;
  }

  const int slot = int(blockIdx.x / H);
  const int h = int(blockIdx.x % H);
  int64_t start = 0, end = N;
  if (cu != nullptr) {
    start = cu[slot];
    end = cu[slot + 1];
    const bool bad = start < 0 || end < start || end > N || (slot == 0 && start != 0);
    if (bad) {
      if (tid == 0 && flags != nullptr) atomicOr(flags, kFlagBadCuSeqlens);
      return;
    }
  }
  const int nchunks = int((end - start + kC - 1) / kC);

  // Prep coordinates: sub-chunk sc, channel share; lane = (channel group cg, token quad tq).
  const int sc = w & 3;
  const int share = w >> 2;
  const int cg = lane >> 2;
  const int tq = lane & 3;
  const int ch0 = share * (DK / C::HALVES) + cg * CPL;   // first prep channel of the lane
  const int vch0 = share * (DV / C::HALVES) + cg * VPL;  // first staged v channel
  const int tok0 = 16 * sc + 4 * tq;                     // first token (in chunk) of the lane
  const uint32_t rowK = uint32_t(H) * DK * 2;            // bytes between tokens (q, k, g)
  const uint32_t rowV = uint32_t(H) * DV * 2;
  const uint32_t rowB = uint32_t(H) * 2;
  // State / output coordinates: 16 columns per wave.
  const int e0 = 16 * w;

  f32x4 S[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) S[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  BfPack<CPL> xg[4], xq[4], xk[4];
  BfPack<VPL> xv[4];
  float xb[4];

  auto load_chunk = [&](int64_t p0, int Lc) {
    const int64_t tokbase = p0 * H + h;
    const uint32_t nK = uint32_t(Lc - 1) * rowK + DK * 2;
    const uint32_t nV = uint32_t(Lc - 1) * rowV + DV * 2;
    const uint32_t nB = uint32_t(Lc - 1) * rowB + 2;
    const auto rq = rsrc(q + tokbase * DK, nK), rk = rsrc(k + tokbase * DK, nK);
    const auto rg = rsrc(g + tokbase * DK, nK), rv = rsrc(v + tokbase * DV, nV);
    const auto rb = rsrc(beta + tokbase, nB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = uint32_t(tok0 + i);
      xg[i] = bload<CPL>(rg, t * rowK + ch0 * 2);
      xq[i] = bload<CPL>(rq, t * rowK + ch0 * 2);
      xk[i] = bload<CPL>(rk, t * rowK + ch0 * 2);
      xv[i] = bload<VPL>(rv, t * rowV + vch0 * 2);
      const unsigned short bb = __builtin_amdgcn_raw_buffer_load_b16(rb, t * rowB, 0, 0);
      xb[i] = __uint_as_float(uint32_t(bb) << 16);
    }
  };

  if (nchunks > 0) load_chunk(start, int((end - start) < kC ? (end - start) : kC));

  for (int c = 0; c < nchunks; ++c) {
    const int64_t p0 = start + int64_t(c) * kC;
    const int Lc = int((end - p0) < kC ? (end - p0) : kC);

    // ---- 1a. in-sub-chunk cumsum of the gates (base 2); sub-chunk totals.
    float cs[4][CPL], Tw[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        run = fmaf(to_f32(xg[i].v[cc]), kLog2e, run);
        cs[i][cc] = run;
      }
      // exclusive prefix over the quad's token groups, then the sub-chunk total
      const float p1 = qperm<0x90>(run);  // quad lanes [0,0,1,2]
      const float s1 = run + (tq >= 1 ? p1 : 0.f);
      const float p2 = qperm<0x40>(s1);   // quad lanes [0,0,0,1]
      const float inc = s1 + (tq >= 2 ? p2 : 0.f);
      const float excl = inc - run;
#pragma unroll
      for (int i = 0; i < 4; ++i) cs[i][cc] += excl;
      Tw[cc] = qbcast<3>(inc);
    }
    if (tq == 0) {
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) s_T[sc * DK + ch0 + cc] = Tw[cc];
    }
    if (share == 0 && cg == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_beta[tok0 + i] = xb[i];
    }
    __syncthreads();

    // ---- 1b. per-channel factors: lane tq computes channels cc = tq (mod 4).
    constexpr int FM = (CPL + 3) / 4;
    float fQh_m[FM], fKb_m[FM], fd_m[FM], fo0_m[FM], fo1_m[FM];
#pragma unroll
    for (int m = 0; m < FM; ++m) {
      const int cc = 4 * m + tq;
      const int ch = ch0 + (cc < CPL ? cc : 0);
      float rho[5];
      rho[0] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) rho[j + 1] = rho[j] + s_T[j * DK + ch];
      float rw = rho[0], rw1 = rho[1];
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (j == sc) {
          rw = rho[j];
          rw1 = rho[j + 1];
        }
      fQh_m[m] = ex2(rw);
      fKb_m[m] = ex2(rho[4] - rw1);
      fd_m[m] = ex2(rw - rw1);
      fo0_m[m] = ex2(rw - rho[1]);  // query factor of block (sc, 0) when sc >= 2
      fo1_m[m] = ex2(rw - rho[2]);  // query factor of block (3, 1)
      if (sc == 0 && cc < CPL) s_decay[ch] = ex2(rho[4]);
    }
    float fQh[CPL], fKb[CPL], fd[CPL], fo0[CPL], fo1[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const int m = cc / 4;
      switch (cc % 4) {
        case 0: fQh[cc] = qbcast<0>(fQh_m[m]); fKb[cc] = qbcast<0>(fKb_m[m]); fd[cc] = qbcast<0>(fd_m[m]);
                fo0[cc] = qbcast<0>(fo0_m[m]); fo1[cc] = qbcast<0>(fo1_m[m]); break;
        case 1: fQh[cc] = qbcast<1>(fQh_m[m]); fKb[cc] = qbcast<1>(fKb_m[m]); fd[cc] = qbcast<1>(fd_m[m]);
                fo0[cc] = qbcast<1>(fo0_m[m]); fo1[cc] = qbcast<1>(fo1_m[m]); break;
        case 2: fQh[cc] = qbcast<2>(fQh_m[m]); fKb[cc] = qbcast<2>(fKb_m[m]); fd[cc] = qbcast<2>(fd_m[m]);
                fo0[cc] = qbcast<2>(fo0_m[m]); fo1[cc] = qbcast<2>(fo1_m[m]); break;
        default: fQh[cc] = qbcast<3>(fQh_m[m]); fKb[cc] = qbcast<3>(fKb_m[m]); fd[cc] = qbcast<3>(fd_m[m]);
                 fo0[cc] = qbcast<3>(fo0_m[m]); fo1[cc] = qbcast<3>(fo1_m[m]); break;
      }
    }

    // ---- 1c. bf16 operands.
    const int vbase = (sc * (sc + 1)) / 2;  // LDS slot of block (sc, 0)
    float kb4[CPL][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + i;
      const float bt = xb[i];
      float qt[CPL], tmp[CPL], ke[CPL];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        qt[cc] = to_f32(xq[i].v[cc]) * ex2(cs[i][cc]);
        ke[cc] = to_f32(xk[i].v[cc]) * ex2(Tw[cc] - cs[i][cc]);
        kb4[cc][i] = ke[cc] * (bt * fKb[cc]);
        tmp[cc] = qt[cc] * fQh[cc];
      }
      lds_put<CPL>(s_qh + tok * KP + ch0, tmp);
      lds_put<CPL>(s_ke + tok * KP + ch0, ke);
      bf16* qv = s_qv + (4 * tq + i) * KP + ch0;
      // block (sc, sc): diagonal factor
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) tmp[cc] = qt[cc] * fd[cc];
      lds_put<CPL>(qv + (vbase + sc) * 16 * KP, tmp);
      if (sc >= 1) lds_put<CPL>(qv + (vbase + sc - 1) * 16 * KP, qt);  // block (sc, sc-1)
      if (sc >= 2) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) tmp[cc] = qt[cc] * fo0[cc];
        lds_put<CPL>(qv + (vbase + 0) * 16 * KP, tmp);                  // block (sc, 0)
      }
      if (sc == 3) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) tmp[cc] = qt[cc] * fo1[cc];
        lds_put<CPL>(qv + (vbase + 1) * 16 * KP, tmp);                  // block (3, 1)
      }
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) lds_put<4>(s_kbT + (ch0 + cc) * TP + tok0, kb4[cc]);
#pragma unroll
    for (int cc = 0; cc < VPL; ++cc) {
      BfPack<4> p;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.v[i] = xv[i].v[cc];
      *reinterpret_cast<BfPack<4>*>(s_vT + (vch0 + cc) * TP + tok0) = p;
    }
    // Raw registers consumed: fetch the next chunk while this one computes.
    if (c + 1 < nchunks) {
      const int64_t p1 = p0 + kC;
      load_chunk(p1, int((end - p1) < kC ? (end - p1) : kC));
    }
    __syncthreads();

    // ---- 2. A blocks (s in sub-chunk j, r in sub-chunk bw) -> A[r][s] in LDS.
#pragma unroll
    for (int job = w; job < 12; job += C::NW) {
      int bw, bj;
      block_of(job, bw, bj);
      bf16x4 out;
      if (job < 10) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          const int col = 32 * u + 8 * gq;
          const bf16x8 aop = *reinterpret_cast<const bf16x8*>(s_ke + (16 * bj + lr) * KP + col);
          const bf16x8 bop = *reinterpret_cast<const bf16x8*>(s_qv + (job * 16 + lr) * KP + col);
          acc = mfma(aop, bop, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sl = 4 * gq + i;
          const bool keep = (bj < bw) || (sl <= lr);
          out[i] = from_f32<bf16>(keep ? acc[i] * s_beta[16 * bj + sl] : 0.f);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = from_f32<bf16>(0.f);
      }
      *reinterpret_cast<bf16x4*>(s_a + (16 * bw + lr) * TP + 16 * bj + 4 * gq) = out;
    }
    __syncthreads();

    // ---- 3. outputs for columns [e0, e0 + 16), then the state update.
    {
      bf16x8 sop[KS];
#pragma unroll
      for (int u = 0; u < KS; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sop[u][i] = from_f32<bf16>(S[2 * u][i]);
          sop[u][4 + i] = from_f32<bf16>(S[2 * u + 1][i]);
        }
      const auto ro = rsrc(o + (p0 * H + h) * DV, uint32_t(Lc - 1) * rowV + DV * 2);
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(s_vT + (e0 + lr) * TP + 8 * gq);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(s_vT + (e0 + lr) * TP + 32 + 8 * gq);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (16 * t < Lc) {
          const int rrow = 16 * t + lr;
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(s_qh + rrow * KP + 32 * u + 4 * gq);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(s_qh + rrow * KP + 32 * u + 16 + 4 * gq);
            const bf16x8 bop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc = mfma(sop[u], bop, acc);
          }
          acc = mfma(v0, *reinterpret_cast<const bf16x8*>(s_a + rrow * TP + 8 * gq), acc);
          if (t >= 2) acc = mfma(v1, *reinterpret_cast<const bf16x8*>(s_a + rrow * TP + 32 + 8 * gq), acc);
          typedef int v2 __attribute__((ext_vector_type(2)));
          bf16x4 out;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = from_f32<bf16>(acc[i] * scale);
          v2 bits;
          __builtin_memcpy(&bits, &out, 8);
          __builtin_amdgcn_raw_buffer_store_b64(bits, ro, uint32_t(rrow) * rowV + (e0 + 4 * gq) * 2, 0, 0);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(s_decay + 16 * dt + 4 * gq);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[dt][i] *= dec[i];
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(s_kbT + (16 * dt + lr) * TP + 8 * gq);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(s_kbT + (16 * dt + lr) * TP + 32 + 8 * gq);
        S[dt] = mfma(a0, v0, S[dt]);
        S[dt] = mfma(a1, v1, S[dt]);
      }
    }
    __syncthreads();
  }

  if (final_state != nullptr) {
    float* fs = final_state + (int64_t(slot) * H + h) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) fs[int64_t(16 * dt + 4 * gq + i) * DV + e0 + lr] = S[dt][i];
  }
}

template <int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                       int32_t H, float scale, void* o, float* fs, int32_t* flags,
                       hipStream_t s) {
  using C = Cfg<DK, DV>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<DK, DV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = int64_t(max_segs) * H + kTailBlocks;
  hipLaunchKernelGGL((kda_chunk_kernel<DK, DV>), dim3(unsigned(blocks)), dim3(C::NT), C::bytes, s,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(g),
                     static_cast<const bf16*>(beta), cu, max_segs, N, H, scale,
                     static_cast<bf16*>(o), fs, flags);
  return hipGetLastError();
}

}  // namespace

bool kda_chunk_supported(int32_t Dk, int32_t Dv, int32_t dtype) {
  return dtype == 0 && (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
}

hipError_t launch_kda_chunk(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                            int32_t H, int32_t Dk, int32_t Dv, float scale, void* o,
                            float* final_state, int32_t* flags, hipStream_t stream) {
  if (Dk == 128 && Dv == 128)
    return launch_dims<128, 128>(q, k, v, g, beta, cu, max_segs, N, H, scale, o, final_state, flags, stream);
  if (Dk == 64 && Dv == 64)
    return launch_dims<64, 64>(q, k, v, g, beta, cu, max_segs, N, H, scale, o, final_state, flags, stream);
  if (Dk == 128 && Dv == 64)
    return launch_dims<128, 64>(q, k, v, g, beta, cu, max_segs, N, H, scale, o, final_state, flags, stream);
  if (Dk == 64 && Dv == 128)
    return launch_dims<64, 128>(q, k, v, g, beta, cu, max_segs, N, H, scale, o, final_state, flags, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
