// segment_ids [B, T] -> cu_seqlens [max_segs + 1], token -> segment index, n_segs, flags.
//
// RFC-0025 "Support attention varlen and align loss", Design section 1: mark
// boundaries, take their running count as a 1-based segment index and find
// each segment's start. Here the page's searchsorted is inverted: the k-th
// boundary (1-based) scatters its position into cu[k-1] directly, because the
// start of segment k-1 is the end of segment k-2. Row starts holding a real
// token are boundaries (RFC-0026 section 3.1.1: t = 0 always starts a
// segment); the last real segment ends one past the last non-zero position.
// doc(p) follows "Drill: Sequence Packing from scratch", section "The math".
//
// One work-group of 1024 threads walks the flattened buffer in tiles of 8192
// positions (8 consecutive positions per thread). Pass 1 counts boundaries and
// finds the last real token; pass 2 re-reads the (now L2-resident) ids, runs a
// block-wide exclusive scan of the per-thread boundary counts (wave shuffles +
// one LDS exchange per tile) and scatters. The ids of one 8B*T buffer are at
// most a few hundred KiB, so one CU finishes in a few microseconds and no
// cross-work-group synchronisation or scratch memory is needed.

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = 8;
constexpr int64_t kTile = int64_t(kThreads) * kPerThread;

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

__device__ __forceinline__ int64_t wave_max64(int64_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    int64_t y = __shfl_xor(x, d, 64);
    x = y > x ? y : x;
  }
  return x;
}

// Boundary bits of positions p0 .. p0+7 (bit j for p0 + j), positions >= N are 0.
__device__ __forceinline__ unsigned boundary_bits(const int32_t* __restrict__ seg, int64_t p0,
                                                  int64_t N, int64_t T, int64_t* last_nz) {
  unsigned bits = 0;
  int prev = (p0 > 0 && p0 < N) ? seg[p0 - 1] : 0;
  int64_t row_pos = p0 % T;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t p = p0 + j;
    if (p < N) {
      const int s = seg[p];
      if (s != 0) {
        *last_nz = p;
        if (row_pos == 0 || s != prev) bits |= 1u << j;
      }
      prev = s;
    }
    row_pos = (row_pos + 1 == T) ? 0 : row_pos + 1;
  }
  return bits;
}

__global__ __launch_bounds__(kThreads) void cu_seqlens_kernel(
    const int32_t* __restrict__ seg, int64_t N, int64_t T, int32_t max_segs,
    int32_t* __restrict__ cu, int32_t* __restrict__ token_seg, int32_t* __restrict__ n_segs_out,
    int32_t* __restrict__ flags_out) {
  __shared__ int s_wsum[kWaves];
  __shared__ int64_t s_wmax[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;

  // Pass 1: number of boundaries and last real token.
  int cnt = 0;
  int64_t last = -1;
  for (int64_t base = 0; base < N; base += kTile) {
    const int64_t p0 = base + int64_t(tid) * kPerThread;
    cnt += __popc(boundary_bits(seg, p0, N, T, &last));
  }
  cnt = wave_sum(cnt);
  last = wave_max64(last);
  if (lane == 0) {
    s_wsum[wid] = cnt;
    s_wmax[wid] = last;
  }
  __syncthreads();
  int n = 0;
  int64_t last_all = -1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    n += s_wsum[w];
    last_all = s_wmax[w] > last_all ? s_wmax[w] : last_all;
  }
  __syncthreads();
  const int64_t e_last = last_all + 1;
  const int lim = n < max_segs ? n : max_segs;
  const int64_t cu_last = n > max_segs ? N : e_last;

  // Pass 2: scan and scatter.
  int running = 0;
  for (int64_t base = 0; base < N; base += kTile) {
    const int64_t p0 = base + int64_t(tid) * kPerThread;
    int64_t dummy = -1;
    const unsigned bits = boundary_bits(seg, p0, N, T, &dummy);
    const int c = __popc(bits);
    const int incl = wave_incl_scan(c, lane);
    if (lane == 63) s_wsum[wid] = incl;
    __syncthreads();
    int wave_off = 0, tile_total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int s = s_wsum[w];
      wave_off += (w < wid) ? s : 0;
      tile_total += s;
    }
    int kth = running + wave_off + incl - c;  // boundaries before p0
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t p = p0 + j;
      if (p < N) {
        if ((bits >> j) & 1u) {
          ++kth;
          // The kth boundary starts segment kth-1, which is where slot kth-2 ends.
          if (kth >= 2 && kth <= lim) cu[kth - 1] = static_cast<int32_t>(p);
        }
        if (token_seg != nullptr) {
          int idx = -1;
          if (p < cu_last) {
            idx = (kth < max_segs ? kth : max_segs) - 1;
            idx = idx < 0 ? 0 : idx;  // padding in front of the first boundary joins segment 0
          }
          token_seg[p] = idx;
        }
      }
    }
    running += tile_total;
    __syncthreads();
  }

  // Slots past the scattered starts: last real end, or N for the merged slot.
  if (n > max_segs) {
    if (tid == 0) cu[max_segs] = static_cast<int32_t>(N);
  } else {
    for (int64_t j = (n > 1 ? n : 1) + tid; j <= max_segs; j += kThreads)
      cu[j] = static_cast<int32_t>(e_last);
  }
  if (tid == 0) {
    cu[0] = 0;
    if (n_segs_out != nullptr) *n_segs_out = n;
    if (flags_out != nullptr) {
      int32_t f = 0;
      if (n > max_segs) f |= kFlagOverflow;
      if (seg[0] == 0 && e_last > 0) f |= kFlagLeadingPad;
      *flags_out = f;
    }
  }
}

}  // namespace

hipError_t launch_cu_seqlens(const int32_t* seg, int64_t N, int64_t T, int32_t max_segs,
                             int32_t* cu, int32_t* token_seg, int32_t* n_segs, int32_t* flags,
                             hipStream_t stream) {
  hipLaunchKernelGGL(cu_seqlens_kernel, dim3(1), dim3(kThreads), 0, stream, seg, N, T, max_segs,
                     cu, token_seg, n_segs, flags);
  return hipGetLastError();
}

}  // namespace pkv
