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
// One work-group of 1024 threads. The buffer is cut into groups of 4
// consecutive positions and tiles of 16384 groups (65536 positions):
//   0. only when token_seg is requested over more than one tile: the last
//      non-zero position, by a backward sweep (one step covers 4096
//      positions; packed batches end in at most a short pad);
//   A. each thread loads groups tid, tid + 1024, ... (16-byte coalesced
//      loads, all in flight at once), writes each group's 4 boundary bits to
//      LDS and tracks the last non-zero position;
//   B. each thread takes 16 consecutive groups from LDS, a block-wide scan
//      of their boundary counts gives every boundary its rank k, and the
//      k-th boundary scatters its position into cu[k-1];
//   C. only when token_seg is requested: every position's segment index,
//      from the per-group ranks left in LDS, with coalesced 16-byte stores.
// The ids are read from HBM once; the bitmask and ranks of a tile take 48 KiB
// of LDS. No cross-work-group synchronisation or scratch memory is needed.

#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupsPerThread = 16;
constexpr int kTileGroups = kThreads * kGroupsPerThread;  // 16384
constexpr int64_t kTilePos = 4 * int64_t(kTileGroups);    // 65536

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t wave_max64(int64_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const int64_t y = __shfl_xor(x, d, 64);
    x = y > x ? y : x;
  }
  return x;
}

// Four ids at p .. p+3; positions >= N read as 0. kVec: seg is 16-byte aligned.
template <bool kVec>
__device__ __forceinline__ i32x4 load4(const int32_t* __restrict__ seg, int64_t p, int64_t N) {
  if (kVec && p + 4 <= N) return *reinterpret_cast<const i32x4*>(seg + p);
  i32x4 x = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (p + i < N) x[i] = seg[p + i];
  return x;
}

// kIds: the [B, T] kernel contract of RFC-0026 section 3.1.1 instead of the
// conversion's: every id change and every row start is a boundary (id 0 is an
// id like any other), and the last segment ends at N; cu then holds exactly
// n + 1 entries (cu[n] = N; no phantoms, no flags, no token map).
template <bool kVec, bool kT4, bool kIds>
__global__ __launch_bounds__(kThreads) void cu_seqlens_kernel(
    const int32_t* __restrict__ seg, int64_t N, int64_t T, int32_t max_segs,
    int32_t* __restrict__ cu, int32_t* __restrict__ token_seg, int32_t* __restrict__ n_segs_out,
    int32_t* __restrict__ flags_out) {
  __shared__ __attribute__((aligned(16))) uint8_t s_bits[kTileGroups];   // boundary bits per group
  __shared__ __attribute__((aligned(16))) uint16_t s_rank[kTileGroups];  // boundaries before the group (in tile)
  __shared__ int s_wsum[kWaves];
  __shared__ int s_edge[kGroupsPerThread * kWaves];  // last id of each wave's groups
  __shared__ int64_t s_wmax[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;

  // 0. Last non-zero position (-1 if none), needed before the first tile's
  // token indices only when there are several tiles.
  int64_t last_nz = -1;
  const bool sweep = token_seg != nullptr && N > kTilePos;
  for (int64_t hi = sweep ? N : 0; hi > 0; hi -= 4 * kThreads) {
    const int64_t lo = hi - 4 * kThreads;
    const int64_t p = lo + 4 * int64_t(tid);
    int64_t m = -1;
    if (p + 3 >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p + i >= 0 && p + i < hi && seg[p + i] != 0) m = p + i;
    }
    m = wave_max64(m);
    if (lane == 0) s_wmax[wid] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) last_nz = s_wmax[w] > last_nz ? s_wmax[w] : last_nz;
    __syncthreads();
    if (last_nz >= 0) break;  // uniform: every thread read the same values
  }

  // Row position of a thread's first group in a tile, advanced by 4096 per group step.
  const uint32_t T32 = uint32_t(T);
  const uint32_t step = uint32_t(4 * kThreads) % T32;
  int running = 0;  // boundaries before the tile
  int first_id = 0;  // seg[0], kept from thread 0's first load for the leading-pad flag
  for (int64_t base = 0; base < N; base += kTilePos) {
    // A. boundary bits of each group. The id before group m is the last id
    // of group m - 1: lane - 1's (a shuffle), for lane 0 the wave before's
    // lane 63 (through LDS), for the tile's first group the previous tile's
    // last position.
    uint32_t rp = uint32_t((base + 4 * int64_t(tid)) % T);
    i32x4 xs[kGroupsPerThread];
#pragma unroll
    for (int j = 0; j < kGroupsPerThread; ++j) {
      const int64_t p = base + 4 * int64_t(tid + kThreads * j);
      xs[j] = p < N ? load4<kVec>(seg, p, N) : i32x4{0, 0, 0, 0};
    }
    if (lane == 63) {
#pragma unroll
      for (int j = 0; j < kGroupsPerThread; ++j) s_edge[j * kWaves + wid] = xs[j][3];
    }
    const int before_tile = (tid == 0 && base > 0) ? seg[base - 1] : 0;
    if (base == 0) first_id = xs[0][0];
    __syncthreads();
    int tile_nz = -1;  // last non-zero position in the tile, tile-relative
#pragma unroll
    for (int j = 0; j < kGroupsPerThread; ++j) {
      const int m = tid + kThreads * j;
      const i32x4 x = xs[j];
      int prev = __shfl_up(x[3], 1, 64);
      if (lane == 0)
        prev = wid > 0 ? s_edge[j * kWaves + wid - 1]
                       : (j > 0 ? s_edge[(j - 1) * kWaves + kWaves - 1] : before_tile);
      unsigned bits;
      if (kIds) {
        bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t r = rp + uint32_t(i);
          const bool row_start = kT4 ? (i == 0 && rp == 0)
                                     : (r == 0 || r == T32 || (T32 <= 2 && (r == 2 * T32 || r == 3 * T32)));
          const int pv = i == 0 ? prev : x[i - 1];
          const int64_t pos = base + 4 * int64_t(m) + i;
          if (pos < N && (row_start || x[i] != pv)) bits |= 1u << i;
        }
      } else if (kT4) {
        // T % 4 == 0: rows start only at a group's first position
        bits = unsigned(x[0] != 0 && (x[0] != prev || rp == 0)) |
               (unsigned(x[1] != 0 && x[1] != x[0]) << 1) |
               (unsigned(x[2] != 0 && x[2] != x[1]) << 2) |
               (unsigned(x[3] != 0 && x[3] != x[2]) << 3);
      } else {
        bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // r = row position of p + i, plus T when it wrapped; r <= T + 2, so
          // it is a multiple of T only as 0 or T, or 2T, 3T when T <= 2
          const uint32_t r = rp + uint32_t(i);
          const bool row_start = r == 0 || r == T32 || (T32 <= 2 && (r == 2 * T32 || r == 3 * T32));
          const int pv = i == 0 ? prev : x[i - 1];
          if (x[i] != 0 && (row_start || x[i] != pv)) bits |= 1u << i;
        }
      }
      const int nz = x[3] != 0 ? 3 : x[2] != 0 ? 2 : x[1] != 0 ? 1 : x[0] != 0 ? 0 : -1;
      if (nz >= 0) tile_nz = 4 * m + nz;  // positions >= N read as 0
      s_bits[m] = uint8_t(bits);
      rp += step;
      if (rp >= T32) rp -= T32;
    }
    const int64_t tile_last = wave_max64(tile_nz >= 0 ? base + tile_nz : int64_t(-1));
    if (lane == 0) s_wmax[wid] = tile_last;
    __syncthreads();
    if (!sweep) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) last_nz = s_wmax[w] > last_nz ? s_wmax[w] : last_nz;
    }

    // B. ranks and scatter: thread tid owns groups [16 tid, 16 tid + 16)
    const uint4 w4 = *reinterpret_cast<const uint4*>(s_bits + kGroupsPerThread * tid);
    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
    const int c = __popc(wd[0]) + __popc(wd[1]) + __popc(wd[2]) + __popc(wd[3]);
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
    const int excl = wave_off + incl - c;  // boundaries in the tile before this thread's groups
    if (token_seg != nullptr) {
      // ranks of groups 2i, 2i + 1 packed in one word (each < 4 * kTileGroups = 65536)
      uint32_t rk[kGroupsPerThread / 2];
      uint32_t r = uint32_t(excl);
#pragma unroll
      for (int gi = 0; gi < kGroupsPerThread; ++gi) {
        if (gi & 1) rk[gi >> 1] |= r << 16;
        else rk[gi >> 1] = r;
        r += __popc((wd[gi >> 2] >> (8 * (gi & 3))) & 0xFu);
      }
      uint4* dst = reinterpret_cast<uint4*>(s_rank + kGroupsPerThread * tid);
      dst[0] = uint4{rk[0], rk[1], rk[2], rk[3]};
      dst[1] = uint4{rk[4], rk[5], rk[6], rk[7]};
    }
    if (c != 0) {
      int kth = running + excl;
      const int64_t p0 = base + 4 * int64_t(kGroupsPerThread) * tid;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint32_t word = wd[qd];  // byte b holds the bits of group 4 qd + b
        while (word != 0) {
          const int bit = __builtin_ctz(word);
          word &= word - 1;
          ++kth;
          // The kth boundary starts segment kth-1, which is where slot kth-2 ends.
          if (kth >= 2 && kth <= max_segs)
            cu[kth - 1] = int32_t(p0 + 4 * (4 * qd + (bit >> 3)) + (bit & 7));
        }
      }
    }
    __syncthreads();

    // C. token -> segment index. Positions after the last real token belong to
    // no segment, unless the segments overflowed (then to the merged last slot);
    // a tile holding such positions has every boundary at or before them.
    if (token_seg != nullptr) {
      const int n_upto = running + tile_total;
      const int tail_idx = n_upto > max_segs ? max_segs - 1 : -1;
#pragma unroll 4
      for (int j = 0; j < kGroupsPerThread; ++j) {
        const int m = tid + kThreads * j;
        const int64_t p = base + 4 * int64_t(m);
        if (p >= N) break;
        const unsigned bits = s_bits[m];
        int kth = running + int(s_rank[m]);
        i32x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kth += (bits >> i) & 1u;
          int idx = (kth < max_segs ? kth : max_segs) - 1;
          idx = idx < 0 ? 0 : idx;  // padding in front of the first boundary joins segment 0
          out[i] = p + i <= last_nz ? idx : tail_idx;
        }
        if (kVec && p + 4 <= N) {
          *reinterpret_cast<i32x4*>(token_seg + p) = out;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (p + i < N) token_seg[p + i] = out[i];
        }
      }
    }
    running += tile_total;
    __syncthreads();  // the next tile overwrites s_bits and s_rank
  }

  const int n = running;
  if (kIds) {
    if (tid == 0) {
      cu[0] = 0;
      cu[n] = static_cast<int32_t>(N);
      if (n_segs_out != nullptr) *n_segs_out = n;
    }
    return;
  }
  const int64_t e_last = last_nz + 1;
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
      if (first_id == 0 && e_last > 0) f |= kFlagLeadingPad;
      *flags_out = f;
    }
  }
}

}  // namespace

hipError_t launch_cu_seqlens(const int32_t* seg, int64_t N, int64_t T, int32_t max_segs,
                             int32_t* cu, int32_t* token_seg, int32_t* n_segs, int32_t* flags,
                             hipStream_t stream) {
  const bool vec = (reinterpret_cast<uintptr_t>(seg) % 16 == 0) &&
                   (token_seg == nullptr || reinterpret_cast<uintptr_t>(token_seg) % 16 == 0);
  auto kernel = vec ? (T % 4 == 0 ? cu_seqlens_kernel<true, true, false> : cu_seqlens_kernel<true, false, false>)
                    : (T % 4 == 0 ? cu_seqlens_kernel<false, true, false> : cu_seqlens_kernel<false, false, false>);
  hipLaunchKernelGGL(kernel, dim3(1), dim3(kThreads), 0, stream, seg, N, T, max_segs, cu, token_seg,
                     n_segs, flags);
  return hipGetLastError();
}

hipError_t launch_segment_bounds(const int32_t* seg, int64_t N, int64_t T, int32_t* bounds,
                                 int32_t* n_segs, hipStream_t stream) {
  const bool vec = reinterpret_cast<uintptr_t>(seg) % 16 == 0;
  auto kernel = vec ? (T % 4 == 0 ? cu_seqlens_kernel<true, true, true> : cu_seqlens_kernel<true, false, true>)
                    : (T % 4 == 0 ? cu_seqlens_kernel<false, true, true> : cu_seqlens_kernel<false, false, true>);
  hipLaunchKernelGGL(kernel, dim3(1), dim3(kThreads), 0, stream, seg, N, T, int32_t(N), bounds,
                     static_cast<int32_t*>(nullptr), n_segs, static_cast<int32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace pkv
