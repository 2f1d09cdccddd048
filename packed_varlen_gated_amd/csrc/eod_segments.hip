// EOD-separated token rows -> segment ids, positions and loss segment ids.
//
// RFC-0025 "Support attention varlen and align loss", Design section 6 (data
// pipeline alignment):
// an EOD token keeps the id of the document it ends and a new segment starts
// right after it; positions restart at 0 after an EOD; positions holding the
// EOD carry no loss (loss id 0). Ids start at 1 in every row (each row is an
// independent packed sample), so for row b and position t:
//   seg[t]  = 1 + #{u < t : x[u] == eod}
//   pos[t]  = t - (1 + max{u < t : x[u] == eod})   (t if there is none)
//   loss[t] = x[t] == eod ? 0 : seg[t]
//
// One work-group of 1024 threads per row, over tiles of 4096 positions (4
// consecutive positions per thread, 16-byte loads and stores when the row is
// aligned). Per tile, a block-wide exclusive sum of the EOD counts and an
// exclusive max of "one past the last EOD" give every position its count and
// its document start; both carry to the next tile.

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 4 * kThreads;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Exclusive scans over the work-group: sum of x and max of y (y >= 0).
// *sum_all and *max_all get the totals; every thread takes part.
__device__ __forceinline__ void block_scan2(int x, int y, int* s_sum, int* s_max, int& x_excl,
                                            int& y_excl, int& sum_all, int& max_all) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int xi = x, yi = y;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int xs = __shfl_up(xi, d, 64), ys = __shfl_up(yi, d, 64);
    if (lane >= d) {
      xi += xs;
      yi = ys > yi ? ys : yi;
    }
  }
  if (lane == 63) {
    s_sum[wv] = xi;
    s_max[wv] = yi;
  }
  __syncthreads();
  int xb = 0, yb = 0, xa = 0, ya = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int a = s_sum[i], b = s_max[i];
    if (i < wv) {
      xb += a;
      yb = b > yb ? b : yb;
    }
    xa += a;
    ya = b > ya ? b : ya;
  }
  __syncthreads();  // the next call overwrites the wave totals
  // exclusive within the wave: the inclusive value of lane - 1
  const int xprev = __shfl_up(xi, 1, 64), yprev = __shfl_up(yi, 1, 64);
  x_excl = xb + (lane > 0 ? xprev : 0);
  const int yw = lane > 0 ? yprev : 0;
  y_excl = yb > yw ? yb : yw;
  sum_all = xa;
  max_all = ya;
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void eod_segments_kernel(
    const int32_t* __restrict__ tokens, int64_t T, int32_t eod, int32_t* __restrict__ seg,
    int32_t* __restrict__ pos, int32_t* __restrict__ loss) {
  __shared__ int s_sum[kWaves], s_max[kWaves];
  const int64_t row = int64_t(blockIdx.x) * T;
  int count = 0;        // EODs in the row before the tile
  int64_t doc0 = 0;     // one past the last EOD before the tile (row-relative)
  for (int64_t base = 0; base < T; base += kTile) {
    const int64_t p = base + 4 * int64_t(threadIdx.x);  // row-relative first position
    i32x4 x = {0, 0, 0, 0};
    bool in[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) in[i] = p + i < T;
    if (kVec && p + 4 <= T) {
      x = *reinterpret_cast<const i32x4*>(tokens + row + p);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (in[i]) x[i] = tokens[row + p + i];
    }
    int c = 0, last = 0;  // EODs in this thread's positions; one past the last one (tile-relative + 1)
    int e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = (in[i] && x[i] == eod) ? 1 : 0;
      c += e[i];
      if (e[i]) last = 4 * int(threadIdx.x) + i + 1;
    }
    int c_excl, last_excl, c_all, last_all;
    block_scan2(c, last, s_sum, s_max, c_excl, last_excl, c_all, last_all);
    int cnt = count + c_excl;
    int64_t start = last_excl > 0 ? base + last_excl : doc0;
    i32x4 so, po, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      so[i] = 1 + cnt;
      po[i] = int(p + i - start);
      lo[i] = e[i] ? 0 : 1 + cnt;
      if (e[i]) {  // the EOD closes its document
        cnt += 1;
        start = p + i + 1;
      }
    }
    if (kVec && p + 4 <= T) {
      *reinterpret_cast<i32x4*>(seg + row + p) = so;
      if (pos) *reinterpret_cast<i32x4*>(pos + row + p) = po;
      if (loss) *reinterpret_cast<i32x4*>(loss + row + p) = lo;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!in[i]) continue;
        seg[row + p + i] = so[i];
        if (pos) pos[row + p + i] = po[i];
        if (loss) loss[row + p + i] = lo[i];
      }
    }
    count += c_all;
    if (last_all > 0) doc0 = base + last_all;
  }
}

}  // namespace

hipError_t launch_eod_segments(const int32_t* tokens, int64_t B, int64_t T, int32_t eod_id,
                               int32_t* seg, int32_t* pos, int32_t* loss, hipStream_t stream) {
  auto aligned = [](const void* ptr) { return ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  const bool vec = T % 4 == 0 && aligned(tokens) && aligned(seg) && aligned(pos) && aligned(loss);
  if (vec)
    hipLaunchKernelGGL(eod_segments_kernel<true>, dim3(unsigned(B)), dim3(kThreads), 0, stream,
                       tokens, T, eod_id, seg, pos, loss);
  else
    hipLaunchKernelGGL(eod_segments_kernel<false>, dim3(unsigned(B)), dim3(kThreads), 0, stream,
                       tokens, T, eod_id, seg, pos, loss);
  return hipGetLastError();
}

}  // namespace pkv
