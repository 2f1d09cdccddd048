// Token-serial packed KDA recurrence (generic path: fp32 or bf16 tensors, any
// supported Dk x Dv).
//
// RFC-0026 "Ling3 KDA varlen support", Background (KDA state leakage problem):
// S_t = diag(exp g_t) S_{t-1} + beta_t k_t v_t^T, reset to zero at every
// segment start (section 3.1.1). Readout o_t = scale * S_t^T q_t after the
// update. Segments come from cu_seqlens (RFC-0025 Design sections 1 and 2).
//
// One work-group of 256 threads per (segment slot, head). Thread (rg, e) keeps
// state column e, rows [rg*R, rg*R + R) in registers (R = Dk*Dv/256). Tokens
// are staged through LDS in blocks of kTB (q, k, exp(g) and v as fp32); each
// thread updates its rows and leaves a partial readout in LDS that is reduced
// over the 256/Dv row groups once per block. This path computes in fp32 with
// no chunking, so it serves the fp32 tolerance directly; the bf16 hot path is
// the chunked MFMA kernel.
//
// Extra work-groups past max_segs*H zero o for positions >= cu[max_segs].
//
// With seg_ids (the [B, T] contract of RFC-0026 section 3.1.1) a work-group
// takes one (row, head) instead of a slot: padding tokens (id 0, which the
// kernel ignores by section 3.4) leave the state alone and output 0; a real
// token whose id differs from the previous position's clears the state, by a
// zero decay for that token (as gate injection does), unless it is the row's
// first real token, which continues from the row's initial state; the final
// state is the state after the row's last real token.

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;
constexpr int kTailBlocks = 64;
constexpr float kL2NormEps = 1e-6f;  // added to a squared norm (the q/k L2 normalisation option)
static_assert(kThreads == 16 * kTB, "16 threads per staged token for the L2 norm");

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void kda_serial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const int32_t* __restrict__ cu,
    int32_t max_segs, int64_t N, int32_t H, float scale, const float* __restrict__ initial_state,
    T* __restrict__ o, float* __restrict__ final_state, int32_t* __restrict__ flags,
    const int32_t* __restrict__ seg_ids, int64_t row_len, bool qk_l2norm) {
  constexpr int RG = kThreads / DV;  // row groups
  constexpr int R = DK / RG;         // consecutive rows per thread
  static_assert(RG * DV == kThreads && R * RG == DK, "bad tile");
  __shared__ float s_q[kTB][DK];
  __shared__ float s_k[kTB][DK];
  __shared__ float s_a[kTB][DK];
  __shared__ float s_v[kTB][DV];
  __shared__ float s_b[kTB];
  __shared__ int s_rst[kTB];  // 1: clear the state before the token; 2: padding, skip it
  __shared__ int64_t s_first[kThreads / 64];
  __shared__ float s_part[kTB][RG][DV];

  const int tid = threadIdx.x;
  const int64_t seg_blocks = int64_t(max_segs) * H;

  if (int64_t(blockIdx.x) >= seg_blocks) {
    // Tail: positions not covered by any segment get o = 0.
    int64_t cu_last = cu ? int64_t(cu[max_segs]) : N;
    cu_last = cu_last < 0 ? 0 : (cu_last > N ? N : cu_last);
    const int64_t total = (N - cu_last) * H * DV;
    const int64_t base = cu_last * H * DV;
    for (int64_t i = (int64_t(blockIdx.x) - seg_blocks) * kThreads + tid; i < total;
         i += int64_t(kTailBlocks) * kThreads)
      o[base + i] = from_f32<T>(0.f);
    return;
  }

  const int slot = int(blockIdx.x / H);
  const int h = int(blockIdx.x % H);
  int64_t start = 0, end = N;
  if (seg_ids != nullptr) {
    start = int64_t(slot) * row_len;
    end = start + row_len;
  } else if (cu != nullptr) {
    start = cu[slot];
    end = cu[slot + 1];
    const bool bad = start < 0 || end < start || end > N || (slot == 0 && start != 0);
    if (bad) {
      if (tid == 0 && flags != nullptr) atomicOr(flags, kFlagBadCuSeqlens);
      return;
    }
  }

  // [B, T] ids: the row's first real position (end if there is none)
  int64_t first_real = end;
  if (seg_ids != nullptr) {
    int64_t m = end;
    for (int64_t t = start + tid; t < end; t += kThreads)
      if (seg_ids[t] != 0) { m = t; break; }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const int64_t y = __shfl_xor(m, d, 64);
      m = y < m ? y : m;
    }
    if ((tid & 63) == 0) s_first[tid >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) first_real = s_first[w] < first_real ? s_first[w] : first_real;
  }

  const int e = tid % DV;
  const int rg = tid / DV;
  const int d0 = rg * R;
  // the segment's recurrence starts from its initial state (zero if none)
  float S[R];
  const float* s0 = initial_state ? initial_state + (int64_t(slot) * H + h) * DK * DV : nullptr;
#pragma unroll
  for (int r = 0; r < R; ++r) S[r] = s0 ? s0[int64_t(d0 + r) * DV + e] : 0.f;

  for (int64_t t0 = start; t0 < end; t0 += kTB) {
    const int nt = (end - t0) < kTB ? int(end - t0) : kTB;
    __syncthreads();
    for (int i = tid; i < nt * DK; i += kThreads) {
      const int tt = i / DK, d = i % DK;
      const int64_t off = ((t0 + tt) * H + h) * DK + d;
      s_q[tt][d] = to_f32(q[off]);
      s_k[tt][d] = to_f32(k[off]);
      s_a[tt][d] = __expf(to_f32(g[off]));
    }
    for (int i = tid; i < nt * DV; i += kThreads) {
      const int tt = i / DV, ee = i % DV;
      s_v[tt][ee] = to_f32(v[((t0 + tt) * H + h) * DV + ee]);
    }
    if (tid < nt) {
      s_b[tid] = to_f32(beta[(t0 + tid) * H + h]);
      const int64_t t = t0 + tid;
      int r = 0;
      if (seg_ids != nullptr) {
        const int id = seg_ids[t];
        r = id == 0 ? 2 : (t > first_real && id != seg_ids[t - 1]) ? 1 : 0;
      }
      s_rst[tid] = r;
    }
    __syncthreads();
    if (qk_l2norm) {
      // q and k of each staged token L2-normalised over Dk: 16 threads per
      // token, each over the channels j, j + 16, ...; sums over the 16 lanes
      // by shuffles (one 64-wide wave holds four tokens' groups)
      const int tt = tid >> 4, j = tid & 15;
      float sq = 0.f, sk = 0.f;
      if (tt < nt) {
        for (int d = j; d < DK; d += 16) {
          sq = fmaf(s_q[tt][d], s_q[tt][d], sq);
          sk = fmaf(s_k[tt][d], s_k[tt][d], sk);
        }
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        sq += __shfl_xor(sq, m, 16);
        sk += __shfl_xor(sk, m, 16);
      }
      if (tt < nt) {
        const float rq = 1.f / sqrtf(sq + kL2NormEps), rk = 1.f / sqrtf(sk + kL2NormEps);
        for (int d = j; d < DK; d += 16) {
          s_q[tt][d] *= rq;
          s_k[tt][d] *= rk;
        }
      }
      __syncthreads();
    }
    for (int tt = 0; tt < nt; ++tt) {
      const float bv = s_b[tt] * s_v[tt][e];
      const int rst = s_rst[tt];  // 1: a new segment, nothing carries over
      float acc = 0.f;
      if (rst != 2) {  // uniform: one token for the whole work-group
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int d = d0 + r;
          S[r] = fmaf(rst ? 0.f : s_a[tt][d], S[r], s_k[tt][d] * bv);
          acc = fmaf(S[r], s_q[tt][d], acc);
        }
      }
      s_part[tt][rg][e] = acc;
    }
    __syncthreads();
    for (int i = tid; i < nt * DV; i += kThreads) {
      const int tt = i / DV, ee = i % DV;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < RG; ++j) sum += s_part[tt][j][ee];
      o[((t0 + tt) * H + h) * DV + ee] = from_f32<T>(scale * sum);
    }
  }

  if (final_state != nullptr) {
    float* fs = final_state + (int64_t(slot) * H + h) * DK * DV;
#pragma unroll
    for (int r = 0; r < R; ++r) fs[int64_t(d0 + r) * DV + e] = S[r];
  }
}

template <typename T, int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                       int32_t H, float scale, const float* s0, void* o, float* fs,
                       int32_t* flags, const int32_t* seg_ids, int64_t row_len, bool norm,
                       hipStream_t s) {
  const int64_t blocks = int64_t(max_segs) * H + kTailBlocks;
  hipLaunchKernelGGL((kda_serial_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(kThreads), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), static_cast<const T*>(g),
                     static_cast<const T*>(beta), cu, max_segs, N, H, scale, s0,
                     static_cast<T*>(o), fs, flags, seg_ids, row_len, norm);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dv(int32_t Dv, const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const int32_t* cu, int32_t max_segs, int64_t N, int32_t H,
                     float scale, const float* s0, void* o, float* fs, int32_t* flags,
                     const int32_t* seg_ids, int64_t row_len, bool norm, hipStream_t s) {
  switch (Dv) {
    case 32: return launch_dims<T, DK, 32>(q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
    case 64: return launch_dims<T, DK, 64>(q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
    case 128: return launch_dims<T, DK, 128>(q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dk(int32_t Dk, int32_t Dv, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const int32_t* cu, int32_t max_segs,
                     int64_t N, int32_t H, float scale, const float* s0, void* o, float* fs,
                     int32_t* flags, const int32_t* seg_ids, int64_t row_len, bool norm,
                     hipStream_t s) {
  switch (Dk) {
    case 32: return launch_dv<T, 32>(Dv, q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
    case 64: return launch_dv<T, 64>(Dv, q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
    case 128: return launch_dv<T, 128>(Dv, q, k, v, g, beta, cu, max_segs, N, H, scale, s0, o, fs, flags, seg_ids, row_len, norm, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kda_serial(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                             int32_t H, int32_t Dk, int32_t Dv, float scale, int32_t dtype,
                             bool qk_l2norm, const float* initial_state, void* o,
                             float* final_state, int32_t* flags, hipStream_t stream) {
  if (dtype == 0)
    return launch_dk<bf16>(Dk, Dv, q, k, v, g, beta, cu, max_segs, N, H, scale, initial_state, o,
                           final_state, flags, nullptr, 0, qk_l2norm, stream);
  return launch_dk<float>(Dk, Dv, q, k, v, g, beta, cu, max_segs, N, H, scale, initial_state, o,
                          final_state, flags, nullptr, 0, qk_l2norm, stream);
}

hipError_t launch_kda_serial_ids(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const int32_t* seg, int64_t B, int64_t T,
                                 int32_t H, int32_t Dk, int32_t Dv, float scale, int32_t dtype,
                                 bool qk_l2norm, const float* initial_state, void* o,
                                 float* final_state, hipStream_t stream) {
  // one "slot" per row; no cu_seqlens, so the tail blocks find nothing to zero
  const int32_t rows = int32_t(B);
  if (dtype == 0)
    return launch_dk<bf16>(Dk, Dv, q, k, v, g, beta, nullptr, rows, B * T, H, scale, initial_state,
                           o, final_state, nullptr, seg, T, qk_l2norm, stream);
  return launch_dk<float>(Dk, Dv, q, k, v, g, beta, nullptr, rows, B * T, H, scale, initial_state,
                          o, final_state, nullptr, seg, T, qk_l2norm, stream);
}

}  // namespace pkv
