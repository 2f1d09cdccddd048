// Segment-masked short causal depthwise convolution.
//
// RFC-0025 "Support attention varlen and align loss", Design section 3
// (ShortConvolution segment boundary mask): tap k weights x[t-k] and is zeroed
// when the source token belongs to another segment than t (left padding has
// id 0). No bias, no activation; here the sum is kept in fp32 and rounded once.
//
// The work is one read of x and one write of y, so it is HBM-bound. A block
// owns a tile of kTokens tokens x (256 * VEC) channels of one row. The segment
// mask of the tile is computed once into LDS as one bit per (token, tap); each
// thread then streams its VEC contiguous channels (16-byte vectors) down the
// tile, keeping the previous Kc-1 input vectors in registers, so every input
// element is read once plus a Kc-1 token halo per tile. A full tile is read in
// batches of kBatch tokens whose loads are issued one batch ahead of the
// arithmetic (a register double buffer), so each wave keeps kBatch vector
// loads in flight instead of one.

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 32;
constexpr int kBatch = 8;
static_assert(kTokens % kBatch == 0, "a full tile is whole batches");

template <typename T, int VEC>
struct Vec {
  T v[VEC];
};

// One output token: y = sum_k [mask bit k] w_k x[t-k] over the VEC channels,
// in fp32 with tap 0 first; then the history moves one token on.
template <typename T, int VEC, int KC>
__device__ __forceinline__ void conv_token(const Vec<T, VEC>& in, uint32_t m, const float (&wr)[VEC][KC],
                                           float (&hist)[KC > 1 ? KC - 1 : 1][VEC], T* dst) {
  float cur[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) cur[c] = to_f32(in.v[c]);
  Vec<T, VEC> out;
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    float acc = (m & 1u) ? wr[c][0] * cur[c] : 0.f;
#pragma unroll
    for (int k = 1; k < KC; ++k)
      if ((m >> k) & 1u) acc = fmaf(wr[c][k], hist[k - 1][c], acc);
    out.v[c] = from_f32<T>(acc);
  }
  *reinterpret_cast<Vec<T, VEC>*>(dst) = out;
#pragma unroll
  for (int j = KC - 2; j >= 1; --j)
#pragma unroll
    for (int c = 0; c < VEC; ++c) hist[j][c] = hist[j - 1][c];
  if (KC > 1) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) hist[0][c] = cur[c];
  }
}

template <typename T, int VEC, int KC>
__global__ __launch_bounds__(kThreads) void short_conv_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const int32_t* __restrict__ seg,
    T* __restrict__ y, int64_t T_len, int64_t F) {
  __shared__ uint32_t s_mask[kTokens];
  const int64_t b = blockIdx.z;
  const int64_t t0 = int64_t(blockIdx.y) * kTokens;
  const int64_t f0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * VEC;

  // Mask bit k of token t0+i: source t0+i-k exists and is in the same segment.
  if (threadIdx.x < kTokens) {
    const int64_t t = t0 + threadIdx.x;
    uint32_t m = 0;
    if (t < T_len) {
      const int32_t* srow = seg ? seg + b * T_len : nullptr;
      const int32_t me = srow ? srow[t] : 0;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int64_t src = t - k;
        if (src >= 0 && (srow == nullptr || srow[src] == me)) m |= 1u << k;
      }
    }
    s_mask[threadIdx.x] = m;
  }
  __syncthreads();
  if (f0 >= F) return;

  float wr[VEC][KC];
#pragma unroll
  for (int c = 0; c < VEC; ++c)
#pragma unroll
    for (int k = 0; k < KC; ++k) wr[c][k] = w[(f0 + c) * KC + k];

  const T* xrow = x + b * T_len * F + f0;
  T* yrow = y + b * T_len * F + f0;
  // hist[j] holds x[t-1-j] for the current t (zeros before the row start).
  float hist[KC > 1 ? KC - 1 : 1][VEC];
#pragma unroll
  for (int j = 0; j < KC - 1; ++j) {
    const int64_t src = t0 - 1 - j;
    if (src >= 0) {
      const Vec<T, VEC> in = *reinterpret_cast<const Vec<T, VEC>*>(xrow + src * F);
#pragma unroll
      for (int c = 0; c < VEC; ++c) hist[j][c] = to_f32(in.v[c]);
    } else {
#pragma unroll
      for (int c = 0; c < VEC; ++c) hist[j][c] = 0.f;
    }
  }

  const int nt = (T_len - t0) < kTokens ? int(T_len - t0) : kTokens;
  if (nt == kTokens) {
    Vec<T, VEC> buf[2][kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) buf[0][i] = *reinterpret_cast<const Vec<T, VEC>*>(xrow + (t0 + i) * F);
#pragma unroll
    for (int bb = 0; bb < kTokens / kBatch; ++bb) {
      if (bb + 1 < kTokens / kBatch) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          buf[(bb + 1) & 1][i] =
              *reinterpret_cast<const Vec<T, VEC>*>(xrow + (t0 + (bb + 1) * kBatch + i) * F);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int ti = bb * kBatch + i;
        conv_token<T, VEC, KC>(buf[bb & 1][i], s_mask[ti], wr, hist, yrow + (t0 + ti) * F);
      }
    }
    return;
  }
  for (int i = 0; i < nt; ++i) {
    const Vec<T, VEC> in = *reinterpret_cast<const Vec<T, VEC>*>(xrow + (t0 + i) * F);
    conv_token<T, VEC, KC>(in, s_mask[i], wr, hist, yrow + (t0 + i) * F);
  }
}

template <typename T, int VEC>
hipError_t launch_typed(const void* x, const float* w, const int32_t* seg, void* y, int64_t B,
                        int64_t T_len, int64_t F, int Kc, hipStream_t s) {
  const dim3 grid(unsigned((F / VEC + kThreads - 1) / kThreads), unsigned((T_len + kTokens - 1) / kTokens),
                  unsigned(B));
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
#define PKV_CONV_CASE(KC)                                                                     \
  case KC:                                                                                    \
    hipLaunchKernelGGL((short_conv_kernel<T, VEC, KC>), grid, dim3(kThreads), 0, s, xp, w, seg, \
                       yp, T_len, F);                                                         \
    break;
  switch (Kc) {
    PKV_CONV_CASE(1)
    PKV_CONV_CASE(2)
    PKV_CONV_CASE(3)
    PKV_CONV_CASE(4)
    PKV_CONV_CASE(5)
    PKV_CONV_CASE(6)
    PKV_CONV_CASE(7)
    PKV_CONV_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef PKV_CONV_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_short_conv(const void* x, const float* w, const int32_t* seg, void* y,
                             int64_t B, int64_t T_len, int64_t F, int32_t Kc, int32_t dtype,
                             hipStream_t stream) {
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(y) % 16 == 0);
  if (dtype == 0) {
    if (aligned && F % 8 == 0) return launch_typed<bf16, 8>(x, w, seg, y, B, T_len, F, Kc, stream);
    return launch_typed<bf16, 1>(x, w, seg, y, B, T_len, F, Kc, stream);
  }
  if (aligned && F % 4 == 0) return launch_typed<float, 4>(x, w, seg, y, B, T_len, F, Kc, stream);
  return launch_typed<float, 1>(x, w, seg, y, B, T_len, F, Kc, stream);
}

}  // namespace pkv
