// Backward of the packed KDA recurrence (token-serial; fp32 or bf16 tensors,
// Dk, Dv in {32, 64, 128}).
//
// RFC-0026 "Ling3 KDA varlen support", Background: S_t = diag(exp g_t) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t, S reset per segment (section
// 3.1.1) or started from the slot's initial state (section 3.3). Given do
// (and optionally the cotangent dF of the final states), per (segment, head):
//   forward sweep   dq_t = scale * S_t do_t                 (S_t recomputed)
//   backward sweep  dS_t = exp(g_{t+1}) * dS_{t+1} + scale * q_t do_t^T
//                   (dS after the last token = dF), then
//                   dk_t = beta_t dS_t v_t,  dv_t = beta_t dS_t^T k_t,
//                   dbeta_t = k_t . (dS_t v_t)
//   d initial state = exp(g_first) * dS_first.
// g enters only through the cumulative b_t = sum_{u<=t} g_u (in exp(b_t - b_s)
// and exp(b_end)), so dg_t = sum_{u >= t in the segment} (q_u dq_u - k_u dk_u)
// + sum_e dF * S_end: a reverse running sum, with no stored states.
//
// One work-group of 4 waves per (segment slot, head). Wave w owns state rows
// [w Dk/4, (w+1) Dk/4); lane l = 8 rl + cl holds RR = Dk/32 rows (rl) x
// CC = Dv/8 columns (cl) of S or dS in registers. Row sums (dq, dk) reduce
// over the 8 cl lanes, column sums (dv) over the 8 rl lanes, both by
// shuffles inside the wave; the per-wave partials of dv and dbeta go through
// LDS and are summed once per block of kTB tokens, so a token needs no
// barrier. Token inputs are staged in LDS per block, in the tensors' own type
// (exact), with exp(g) taken where it is used. The per-token q . dq terms wait
// between the sweeps in fp32, exactly: in dg for fp32 tensors, and split into
// high and low 16-bit halves over dg and dk (not yet written) for bf16.
//
// Extra work-groups past max_segs*H zero the gradients of positions >=
// cu[max_segs].

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;
constexpr int kTailBlocks = 64;

template <int DK, int DV>
struct BwdCfg {
  static constexpr int RW = DK / 4;   // rows per wave
  static constexpr int RR = RW / 8;   // rows per lane
  static constexpr int CC = DV / 8;   // columns per lane
  static_assert(RR >= 1 && CC >= 1, "shape");
};

__device__ __forceinline__ float lane_sum8(float x, int stride) {  // over 8 lanes stride apart
#pragma unroll
  for (int s = stride; s < 8 * stride; s <<= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// Park an fp32 value in the (T-typed) dg and dk slots at off, and get it back.
__device__ __forceinline__ void park(float* dg, float*, int64_t off, float x) { dg[off] = x; }
__device__ __forceinline__ void park(bf16* dg, bf16* dk, int64_t off, float x) {
  const uint32_t b = __float_as_uint(x);
  reinterpret_cast<uint16_t*>(dg)[off] = uint16_t(b >> 16);
  reinterpret_cast<uint16_t*>(dk)[off] = uint16_t(b & 0xffffu);
}
__device__ __forceinline__ float unpark(const float* dg, const float*, int64_t off) { return dg[off]; }
__device__ __forceinline__ float unpark(const bf16* dg, const bf16* dk, int64_t off) {
  const uint32_t hi = reinterpret_cast<const uint16_t*>(dg)[off];
  const uint32_t lo = reinterpret_cast<const uint16_t*>(dk)[off];
  return __uint_as_float((hi << 16) | lo);
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void kda_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const T* __restrict__ dout,
    const int32_t* __restrict__ cu, int32_t max_segs, int64_t N, int32_t H, float scale,
    const float* __restrict__ initial_state, const float* __restrict__ dfinal,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dg,
    T* __restrict__ dbeta, float* __restrict__ dinit, int32_t* __restrict__ flags) {
  using C = BwdCfg<DK, DV>;
  constexpr int RR = C::RR, CC = C::CC, RW = C::RW;
  __shared__ T s_q[kTB][DK], s_k[kTB][DK], s_g[kTB][DK];
  __shared__ float s_p[kTB][DK];  // parked q . dq (backward sweep)
  __shared__ T s_v[kTB][DV], s_do[kTB][DV];
  __shared__ float s_b[kTB];
  __shared__ float s_dvp[kTB][4][DV];  // per-wave partials of dS^T k
  __shared__ float s_dbp[kTB][4];      // per-wave partials of k . dS v

  const int tid = threadIdx.x;
  const int64_t seg_blocks = int64_t(max_segs) * H;
  if (int64_t(blockIdx.x) >= seg_blocks) {
    int64_t cu_last = cu ? int64_t(cu[max_segs]) : N;
    cu_last = cu_last < 0 ? 0 : (cu_last > N ? N : cu_last);
    const int64_t stride = int64_t(kTailBlocks) * kThreads;
    const int64_t first = (int64_t(blockIdx.x) - seg_blocks) * kThreads + tid;
    for (int64_t i = first; i < (N - cu_last) * H * DK; i += stride) {
      dq[cu_last * H * DK + i] = from_f32<T>(0.f);
      dk[cu_last * H * DK + i] = from_f32<T>(0.f);
      dg[cu_last * H * DK + i] = from_f32<T>(0.f);
    }
    for (int64_t i = first; i < (N - cu_last) * H * DV; i += stride) dv[cu_last * H * DV + i] = from_f32<T>(0.f);
    for (int64_t i = first; i < (N - cu_last) * H; i += stride) dbeta[cu_last * H + i] = from_f32<T>(0.f);
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
  const int lane = tid & 63, wv = tid >> 6;
  const int rl = lane >> 3, cl = lane & 7;
  const int row0 = wv * RW + rl * RR;  // this lane's rows: row0 .. row0 + RR - 1
  const int col0 = cl * CC;            // columns col0 .. col0 + CC - 1
  const int64_t sh = (int64_t(slot) * H + h) * DK * DV;

  // stage the inputs of tokens [t0, t0 + nt) of this head into LDS
  // (and, for the backward sweep, the parked q . dq)
  auto stage = [&](int64_t t0, int nt, bool parked) {
    for (int i = tid; i < nt * DK; i += kThreads) {
      const int tt = i / DK, d = i % DK;
      const int64_t off = ((t0 + tt) * H + h) * DK + d;
      s_q[tt][d] = q[off];
      s_k[tt][d] = k[off];
      s_g[tt][d] = g[off];
      if (parked) s_p[tt][d] = unpark(dg, dk, off);
    }
    for (int i = tid; i < nt * DV; i += kThreads) {
      const int tt = i / DV, e = i % DV;
      const int64_t off = ((t0 + tt) * H + h) * DV + e;
      s_v[tt][e] = v[off];
      s_do[tt][e] = dout[off];
    }
    if (tid < nt) s_b[tid] = to_f32(beta[(t0 + tid) * H + h]);
  };

  // ---------------- forward sweep: S_t and dq_t (q . dq parked for later)
  float S[RR][CC];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int c = 0; c < CC; ++c)
      S[r][c] = initial_state ? initial_state[sh + int64_t(row0 + r) * DV + col0 + c] : 0.f;
  for (int64_t t0 = start; t0 < end; t0 += kTB) {
    const int nt = end - t0 < kTB ? int(end - t0) : kTB;
    __syncthreads();
    stage(t0, nt, false);
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const float bt = s_b[tt];
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const int d = row0 + r;
        const float a = __expf(to_f32(s_g[tt][d])), kb = to_f32(s_k[tt][d]) * bt;
        float p = 0.f;
#pragma unroll
        for (int c = 0; c < CC; ++c) {
          S[r][c] = fmaf(a, S[r][c], kb * to_f32(s_v[tt][col0 + c]));
          p = fmaf(S[r][c], to_f32(s_do[tt][col0 + c]), p);
        }
        p = lane_sum8(p, 1) * scale;  // dq_t[d]
        if (cl == 0) {
          const int64_t off = ((t0 + tt) * H + h) * DK + d;
          dq[off] = from_f32<T>(p);
          park(dg, dk, off, to_f32(s_q[tt][d]) * p);
        }
      }
    }
  }
  // running sum of dL/db from the segment's end: sum_e dF * S_end per row
  float run[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    float p = 0.f;
    if (dfinal != nullptr) {
#pragma unroll
      for (int c = 0; c < CC; ++c) p = fmaf(dfinal[sh + int64_t(row0 + r) * DV + col0 + c], S[r][c], p);
    }
    run[r] = lane_sum8(p, 1);
  }

  // ---------------- backward sweep: dS, dk, dv, dbeta, dg
  float dS[RR][CC];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int c = 0; c < CC; ++c) dS[r][c] = dfinal ? dfinal[sh + int64_t(row0 + r) * DV + col0 + c] : 0.f;
  const int64_t nblocks = (end - start + kTB - 1) / kTB;
  for (int64_t bi = nblocks - 1; bi >= 0; --bi) {
    const int64_t t0 = start + bi * kTB;
    const int nt = end - t0 < kTB ? int(end - t0) : kTB;
    __syncthreads();
    stage(t0, nt, true);
    __syncthreads();
    for (int tt = nt - 1; tt >= 0; --tt) {
      const float bt = s_b[tt];
      const int64_t tok = t0 + tt;
      float kdu = 0.f;
      float dvp[CC];
#pragma unroll
      for (int c = 0; c < CC; ++c) dvp[c] = 0.f;
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const int d = row0 + r;
        const float qs = to_f32(s_q[tt][d]) * scale, kd = to_f32(s_k[tt][d]);
        float u = 0.f;
#pragma unroll
        for (int c = 0; c < CC; ++c) {
          dS[r][c] = fmaf(qs, to_f32(s_do[tt][col0 + c]), dS[r][c]);
          u = fmaf(dS[r][c], to_f32(s_v[tt][col0 + c]), u);
          dvp[c] = fmaf(dS[r][c], kd, dvp[c]);
        }
        u = lane_sum8(u, 1);  // (dS_t v_t)[d]
        const float dkd = bt * u;
        kdu = fmaf(kd, u, kdu);
        if (cl == 0) {
          const int64_t off = (tok * H + h) * DK + d;
          run[r] += s_p[tt][d] - kd * dkd;  // q . dq parked by the forward sweep
          dk[off] = from_f32<T>(dkd);
          dg[off] = from_f32<T>(run[r]);
        }
        // for the token before: dS_{t-1} = exp(g_t) dS_t
        const float a = __expf(to_f32(s_g[tt][d]));
#pragma unroll
        for (int c = 0; c < CC; ++c) dS[r][c] *= a;
      }
      // column sums over this wave's rows (the 8 rl lanes), then per wave to LDS
#pragma unroll
      for (int c = 0; c < CC; ++c) dvp[c] = lane_sum8(dvp[c], 8);
      kdu = lane_sum8(kdu, 8);  // cl lanes hold equal copies; lane 0 reports
      if (rl == 0) {
#pragma unroll
        for (int c = 0; c < CC; ++c) s_dvp[tt][wv][col0 + c] = dvp[c];
      }
      if (lane == 0) s_dbp[tt][wv] = kdu;
    }
    __syncthreads();
    for (int i = tid; i < nt * DV; i += kThreads) {
      const int tt = i / DV, e = i % DV;
      const float sum = (s_dvp[tt][0][e] + s_dvp[tt][1][e]) + (s_dvp[tt][2][e] + s_dvp[tt][3][e]);
      dv[((t0 + tt) * H + h) * DV + e] = from_f32<T>(s_b[tt] * sum);
    }
    if (tid < nt) dbeta[(t0 + tid) * H + h] = from_f32<T>((s_dbp[tid][0] + s_dbp[tid][1]) + (s_dbp[tid][2] + s_dbp[tid][3]));
  }
  if (dinit != nullptr) {
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
      for (int c = 0; c < CC; ++c) dinit[sh + int64_t(row0 + r) * DV + col0 + c] = dS[r][c];
  }
}

template <typename T, int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const void* dout, const int32_t* cu, int32_t max_segs,
                       int64_t N, int32_t H, float scale, const float* s0, const float* dF,
                       void* dq, void* dk, void* dv, void* dg, void* db, float* dinit,
                       int32_t* flags, hipStream_t s) {
  const int64_t blocks = int64_t(max_segs) * H + kTailBlocks;
  hipLaunchKernelGGL((kda_bwd_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(kThreads), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(g), static_cast<const T*>(beta),
                     static_cast<const T*>(dout), cu, max_segs, N, H, scale, s0, dF,
                     static_cast<T*>(dq), static_cast<T*>(dk), static_cast<T*>(dv),
                     static_cast<T*>(dg), static_cast<T*>(db), dinit, flags);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dv(int32_t Dv, const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const void* dout, const int32_t* cu, int32_t max_segs,
                     int64_t N, int32_t H, float scale, const float* s0, const float* dF, void* dq,
                     void* dk, void* dvv, void* dg, void* db, float* dinit, int32_t* flags,
                     hipStream_t s) {
  switch (Dv) {
    case 32: return launch_dims<T, DK, 32>(q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
    case 64: return launch_dims<T, DK, 64>(q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
    case 128: return launch_dims<T, DK, 128>(q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dk(int32_t Dk, int32_t Dv, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const void* dout, const int32_t* cu,
                     int32_t max_segs, int64_t N, int32_t H, float scale, const float* s0,
                     const float* dF, void* dq, void* dk, void* dvv, void* dg, void* db,
                     float* dinit, int32_t* flags, hipStream_t s) {
  switch (Dk) {
    case 32: return launch_dv<T, 32>(Dv, q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
    case 64: return launch_dv<T, 64>(Dv, q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
    case 128: return launch_dv<T, 128>(Dv, q, k, v, g, beta, dout, cu, max_segs, N, H, scale, s0, dF, dq, dk, dvv, dg, db, dinit, flags, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kda_backward(const void* q, const void* k, const void* v, const void* g,
                               const void* beta, const void* dout, const int32_t* cu,
                               int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                               float scale, int32_t dtype, const float* initial_state,
                               const float* dfinal_state, void* dq, void* dk, void* dv, void* dg,
                               void* dbeta, float* dinitial_state, int32_t* flags,
                               hipStream_t stream) {
  if (dtype == 0)
    return launch_dk<bf16>(Dk, Dv, q, k, v, g, beta, dout, cu, max_segs, N, H, scale, initial_state,
                           dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, flags, stream);
  return launch_dk<float>(Dk, Dv, q, k, v, g, beta, dout, cu, max_segs, N, H, scale, initial_state,
                          dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, flags, stream);
}

}  // namespace pkv
