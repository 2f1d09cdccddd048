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
// One work-group (4 waves) per (segment, head) walks the segment in 64-token
// chunks, keeping the fp32 state S [Dk, Dv] in registers (wave w owns columns
// [w*Dv/4, (w+1)*Dv/4)). With b_r the in-chunk inclusive cumsum of g (base 2
// here) and C = 64:
//   o_r   = S_prev^T (q_r * 2^{b_r})  +  sum_{s<=r} A[r,s] v_s
//   A[r,s] = beta_s * sum_d q_r[d] k_s[d] 2^{b_r[d] - b_s[d]}
//   S_new = diag(2^{b_C}) S_prev + sum_s (beta_s k_s * 2^{b_C - b_s}) v_s^T
// The exponent differences are split at 16-token sub-chunk boundaries rho_j
// (cumsum before sub-chunk j): block (row sub-chunk w, column sub-chunk j) of A
// uses q_r 2^{b_r - rho_{j+1}} and k_s 2^{rho_{j+1} - b_s}; the key factor is
// <= 1 for every block, the query factor is <= 1 off the diagonal and at most
// 2^{16 max|g| log2 e} on it. Per element only 2^{c} and 2^{T - c} are
// computed (c = in-sub-chunk cumsum, T = sub-chunk total); every other factor
// is per channel.
//
// Per chunk:
//   1. prep (channel-major: wave w = sub-chunk w, lane = Dk/64 channels):
//      cumsum of the gates, sub-chunk totals to LDS;          barrier
//      per-channel factors; bf16 operands to LDS: Q~ = q 2^c, Q^ = q 2^b,
//      KE = k 2^{T-c}, Kbar^T = (beta k 2^{b_C-b})^T and V^T; the next
//      chunk's loads are issued here;                           barrier
//   2. A^T blocks of row sub-chunk w on MFMA, masked and beta-scaled, to LDS;
//                                                              barrier
//   3. o^T = S^T Q^^T + V^T A^T for the wave's columns (MFMA), stored;
//      S = diag(2^{b_C}) S + Kbar^T V (MFMA);                  barrier
// MFMA is v_mfma_f32_16x16x32_bf16: A operand lane l holds row l%16 with 8
// contraction slots per lane group l/16, B likewise for column l%16, and the
// 16x16 fp32 result has column l%16, rows 4*(l/16)+i. A contraction index may
// be permuted freely as long as A and B agree; S^T is fed straight from the
// S accumulators by taking slots {4g..4g+3} of two adjacent 16-row tiles.

#include "common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr int kThreads = 256;
constexpr int kTailBlocks = 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int DK, int DV>
struct Smem {
  static constexpr int KP = DK + 8;  // token-major rows (bf16 elements)
  static constexpr int TP = kC + 8;  // transposed rows and A rows (bf16 elements)
  static constexpr int off_qt = 0;
  static constexpr int off_qh = off_qt + kC * KP * 2;
  static constexpr int off_ke = off_qh + kC * KP * 2;
  static constexpr int off_kbT = off_ke + kC * KP * 2;
  static constexpr int off_vT = off_kbT + DK * TP * 2;
  static constexpr int off_a = off_vT + DV * TP * 2;
  static constexpr int off_T = off_a + kC * TP * 2;    // float [4][DK]
  static constexpr int off_fa = off_T + 4 * DK * 4;    // float [10][DK]
  static constexpr int off_decay = off_fa + 10 * DK * 4;
  static constexpr int off_beta = off_decay + DK * 4;  // float [kC]
  static constexpr int bytes = off_beta + kC * 4;
};

template <int n>
struct alignas(2 * n) BfPack {
  bf16 v[n];
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void kda_chunk_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const int32_t* __restrict__ cu,
    int32_t max_segs, int64_t N, int32_t H, float scale, bf16* __restrict__ o,
    float* __restrict__ final_state, int32_t* __restrict__ flags) {
  using L = Smem<DK, DV>;
  constexpr int KP = L::KP, TP = L::TP;
  constexpr int CPL = DK / 64;  // prep channels per lane
  constexpr int VPL = DV / 64;  // staged v channels per lane
  constexpr int EW = DV / 4;    // state / output columns per wave
  constexpr int ET = EW / 16;   // 16-column tiles per wave
  constexpr int DT = DK / 16;   // 16-row state tiles
  constexpr int KS = DK / 32;   // contraction steps over Dk

  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* s_qt = reinterpret_cast<bf16*>(smem + L::off_qt);
  bf16* s_qh = reinterpret_cast<bf16*>(smem + L::off_qh);
  bf16* s_ke = reinterpret_cast<bf16*>(smem + L::off_ke);
  bf16* s_kbT = reinterpret_cast<bf16*>(smem + L::off_kbT);
  bf16* s_vT = reinterpret_cast<bf16*>(smem + L::off_vT);
  bf16* s_a = reinterpret_cast<bf16*>(smem + L::off_a);
  float* s_T = reinterpret_cast<float*>(smem + L::off_T);
  float* s_fa = reinterpret_cast<float*>(smem + L::off_fa);
  float* s_decay = reinterpret_cast<float*>(smem + L::off_decay);
  float* s_beta = reinterpret_cast<float*>(smem + L::off_beta);

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
    for (int64_t i = (int64_t(blockIdx.x) - seg_blocks) * kThreads + tid; i < total;
         i += int64_t(kTailBlocks) * kThreads)
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
  const int e0 = w * EW;

  f32x4 S[DT][ET];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int et = 0; et < ET; ++et) S[dt][et] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Raw inputs of the chunk being prepared (channel-major: token 16w+r, lane's channels).
  BfPack<CPL> xg[16], xq[16], xk[16];
  BfPack<VPL> xv[16];
  bf16 xb = from_f32<bf16>(0.f);

  auto load_chunk = [&](int64_t p0, int Lc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 16 * w + r;
      if (t < Lc) {
        const int64_t tok = (p0 + t) * H + h;
        const int64_t ok = tok * DK + lane * CPL;
        xg[r] = *reinterpret_cast<const BfPack<CPL>*>(g + ok);
        xq[r] = *reinterpret_cast<const BfPack<CPL>*>(q + ok);
        xk[r] = *reinterpret_cast<const BfPack<CPL>*>(k + ok);
        xv[r] = *reinterpret_cast<const BfPack<VPL>*>(v + tok * DV + lane * VPL);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          xg[r].v[c] = from_f32<bf16>(0.f);
          xq[r].v[c] = from_f32<bf16>(0.f);
          xk[r].v[c] = from_f32<bf16>(0.f);
        }
#pragma unroll
        for (int c = 0; c < VPL; ++c) xv[r].v[c] = from_f32<bf16>(0.f);
      }
    }
    if (lane < 16) {
      const int t = 16 * w + lane;
      xb = t < Lc ? beta[(p0 + t) * H + h] : from_f32<bf16>(0.f);
    }
  };

  if (nchunks > 0) load_chunk(start, int((end - start) < kC ? (end - start) : kC));

  for (int c = 0; c < nchunks; ++c) {
    const int64_t p0 = start + int64_t(c) * kC;
    const int Lc = int((end - p0) < kC ? (end - p0) : kC);

    // ---- 1a. cumulative gates (base 2) of sub-chunk w; totals to LDS.
    float cs[16][CPL];
    float run[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) run[cc] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        run[cc] = fmaf(to_f32(xg[r].v[cc]), kLog2e, run[cc]);
        cs[r][cc] = run[cc];
      }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) s_T[w * DK + lane * CPL + cc] = run[cc];
    if (lane < 16) s_beta[16 * w + lane] = to_f32(xb);
    __syncthreads();

    // ---- 1b. per-channel factors and the bf16 operands.
    float Tw[CPL], fQh[CPL], fKb[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const int ch = lane * CPL + cc;
      float Tj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) Tj[j] = s_T[j * DK + ch];
      float rho[5];  // rho[j] = cumsum before sub-chunk j; rho[4] = b_C
      rho[0] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) rho[j + 1] = rho[j] + Tj[j];
      float rho_w = rho[0], rho_w1 = rho[1], tw = Tj[0];
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (j == w) {
          rho_w = rho[j];
          rho_w1 = rho[j + 1];
          tw = Tj[j];
        }
      Tw[cc] = tw;
      fQh[cc] = ex2(rho_w);
      fKb[cc] = ex2(rho[4] - rho_w1);
      if (w == 0) s_decay[ch] = ex2(rho[4]);
      // Query-side factors of the A^T blocks (w, j), j <= w, rows w(w+1)/2 + j.
      const int base = (w * (w + 1)) / 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j <= w) {
          float f;
          if (j == w)
            f = ex2(-Tw[cc]);
          else if (j == w - 1)
            f = 1.f;
          else
            f = ex2(rho_w - rho[j + 1]);
          s_fa[(base + j) * DK + ch] = f;
        }
      }
    }

    bf16 kbt[CPL][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float bt = s_beta[16 * w + r];
      BfPack<CPL> pqt, pqh, pke;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        const float e1 = ex2(cs[r][cc]);
        const float e2 = ex2(Tw[cc] - cs[r][cc]);
        const float qt = to_f32(xq[r].v[cc]) * e1;
        const float ke = to_f32(xk[r].v[cc]) * e2;
        pqt.v[cc] = from_f32<bf16>(qt);
        pqh.v[cc] = from_f32<bf16>(qt * fQh[cc]);
        pke.v[cc] = from_f32<bf16>(ke);
        kbt[cc][r] = from_f32<bf16>(ke * (bt * fKb[cc]));
      }
      const int row = (16 * w + r) * KP + lane * CPL;
      *reinterpret_cast<BfPack<CPL>*>(s_qt + row) = pqt;
      *reinterpret_cast<BfPack<CPL>*>(s_qh + row) = pqh;
      *reinterpret_cast<BfPack<CPL>*>(s_ke + row) = pke;
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      bf16x8 lo, hi;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo[r] = kbt[cc][r];
        hi[r] = kbt[cc][8 + r];
      }
      bf16* dst = s_kbT + (lane * CPL + cc) * TP + 16 * w;
      *reinterpret_cast<bf16x8*>(dst) = lo;
      *reinterpret_cast<bf16x8*>(dst + 8) = hi;
    }
#pragma unroll
    for (int cc = 0; cc < VPL; ++cc) {
      bf16x8 lo, hi;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        lo[r] = xv[r].v[cc];
        hi[r] = xv[8 + r].v[cc];
      }
      bf16* dst = s_vT + (lane * VPL + cc) * TP + 16 * w;
      *reinterpret_cast<bf16x8*>(dst) = lo;
      *reinterpret_cast<bf16x8*>(dst + 8) = hi;
    }
    // The raw registers are consumed: fetch the next chunk while this one computes.
    if (c + 1 < nchunks) {
      const int64_t p1 = p0 + kC;
      load_chunk(p1, int((end - p1) < kC ? (end - p1) : kC));
    }
    __syncthreads();

    // ---- 2. A^T blocks (s in sub-chunk j, r in sub-chunk w), j <= w.
    {
      f32x4 acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int base = (w * (w + 1)) / 2;
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const int col = 32 * u + 8 * gq;
        const bf16x8 qraw = *reinterpret_cast<const bf16x8*>(s_qt + (16 * w + lr) * KP + col);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j <= w) {
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(s_fa + (base + j) * DK + col);
            const f32x4 f1 = *reinterpret_cast<const f32x4*>(s_fa + (base + j) * DK + col + 4);
            bf16x8 bop;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bop[i] = from_f32<bf16>(to_f32(qraw[i]) * f0[i]);
              bop[4 + i] = from_f32<bf16>(to_f32(qraw[4 + i]) * f1[i]);
            }
            const bf16x8 aop = *reinterpret_cast<const bf16x8*>(s_ke + (16 * j + lr) * KP + col);
            acc[j] = mfma(aop, bop, acc[j]);
          }
        }
      }
      bf16* arow = s_a + (16 * w + lr) * TP;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sl = 4 * gq + i;
          const bool keep = (j < w) || (j == w && sl <= lr);
          out[i] = from_f32<bf16>(keep ? acc[j][i] * s_beta[16 * j + sl] : 0.f);
        }
        *reinterpret_cast<bf16x4*>(arow + 16 * j + 4 * gq) = out;
      }
    }
    __syncthreads();

    // ---- 3. outputs of this chunk for columns [e0, e0 + EW), then the state update.
    {
      bf16x8 sop[KS][ET];
#pragma unroll
      for (int u = 0; u < KS; ++u)
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sop[u][et][i] = from_f32<bf16>(S[2 * u][et][i]);
            sop[u][et][4 + i] = from_f32<bf16>(S[2 * u + 1][et][i]);
          }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (16 * t < Lc) {
          const int rrow = (16 * t + lr);
          f32x4 acc[ET];
#pragma unroll
          for (int et = 0; et < ET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(s_qh + rrow * KP + 32 * u + 4 * gq);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(s_qh + rrow * KP + 32 * u + 16 + 4 * gq);
            const bf16x8 bop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int et = 0; et < ET; ++et) acc[et] = mfma(sop[u][et], bop, acc[et]);
          }
#pragma unroll
          for (int m2 = 0; m2 <= t / 2; ++m2) {
            const bf16x8 bop = *reinterpret_cast<const bf16x8*>(s_a + rrow * TP + 32 * m2 + 8 * gq);
#pragma unroll
            for (int et = 0; et < ET; ++et) {
              const bf16x8 aop =
                  *reinterpret_cast<const bf16x8*>(s_vT + (e0 + 16 * et + lr) * TP + 32 * m2 + 8 * gq);
              acc[et] = mfma(aop, bop, acc[et]);
            }
          }
          if (rrow < Lc) {
            bf16* orow = o + ((p0 + rrow) * H + h) * DV + e0 + 4 * gq;
#pragma unroll
            for (int et = 0; et < ET; ++et) {
              bf16x4 out;
#pragma unroll
              for (int i = 0; i < 4; ++i) out[i] = from_f32<bf16>(acc[et][i] * scale);
              *reinterpret_cast<bf16x4*>(orow + 16 * et) = out;
            }
          }
        }
      }

#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(s_decay + 16 * dt + 4 * gq);
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[dt][et][i] *= dec[i];
      }
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        bf16x8 vop[ET];
#pragma unroll
        for (int et = 0; et < ET; ++et)
          vop[et] = *reinterpret_cast<const bf16x8*>(s_vT + (e0 + 16 * et + lr) * TP + 32 * m2 + 8 * gq);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 aop = *reinterpret_cast<const bf16x8*>(s_kbT + (16 * dt + lr) * TP + 32 * m2 + 8 * gq);
#pragma unroll
          for (int et = 0; et < ET; ++et) S[dt][et] = mfma(aop, vop[et], S[dt][et]);
        }
      }
    }
    __syncthreads();
  }

  if (final_state != nullptr) {
    float* fs = final_state + (int64_t(slot) * H + h) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int et = 0; et < ET; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fs[int64_t(16 * dt + 4 * gq + i) * DV + e0 + 16 * et + lr] = S[dt][et][i];
  }
}

template <int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                       int32_t H, float scale, void* o, float* fs, int32_t* flags,
                       hipStream_t s) {
  constexpr int bytes = Smem<DK, DV>::bytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<DK, DV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = int64_t(max_segs) * H + kTailBlocks;
  hipLaunchKernelGGL((kda_chunk_kernel<DK, DV>), dim3(unsigned(blocks)), dim3(kThreads), bytes, s,
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
