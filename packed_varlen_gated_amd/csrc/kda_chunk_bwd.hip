// Chunked reverse pass of the packed KDA recurrence (bf16 tensors, Dk, Dv in
// {64, 128}), on MFMA.
//
// RFC-0026 "Ling3 KDA varlen support", Background: S_t = diag(exp g_t) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale * S_t^T q_t, S reset at every segment start
// (section 3.1.1) or started from the slot's initial state (section 3.3). With
// Lambda the adjoint of a state from everything after it, the gradients follow
// from the same chunked form the forward pass uses. Chunks are 64 tokens
// aligned to segment starts, split into four 16-token sub-chunks.
//
// Four launches:
//   plan     one work-group: per segment slot its chunk count and their prefix
//            sums (global chunk index of each segment's first chunk), the cut
//            of long segments into pieces (as in the forward pass), and the
//            pieces ranked longest first.
//   summary  per piece of a cut segment, head and role: the piece walked from a
//            zero state; its end state and the product of its decays (fp32):
//              S   <- 2^{B} S + sum_t kbar_t v_t^T,     kbar_t = beta_t k_t 2^{B - b_t}
//              Lam <- 2^{B} Lam + sum_t q'_t do_t^T,    q'_t = scale q_t 2^{b_t}
//            (b_t the log2 cumulative gate from the chunk start, B its last
//            value; rows scaled per key channel; Lambda walks backwards.)
//   walk     one work-group per (piece, head): S before every chunk (bf16 in
//            the workspace; not a segment's first when it is zero), starting
//            from the initial state composed with the
//            earlier pieces' summaries; when dL/dfinal_state is given, a
//            segment's last piece walks on to the final state and leaves
//            sum_e dL/dS_final * S_final per key channel.
//   chunk    persistent work-groups over (piece, head) items, longest first:
//            each walks its piece's chunks backwards, starting from
//            dL/dfinal_state composed with the later pieces' adjoint summaries,
//            and carries Lambda (the adjoint after the chunk, fp32 in
//            registers) from one chunk to the one before it; the segment's
//            first piece ends with d initial state = Lambda before its first
//            chunk. Per chunk, from S_c and Lambda it walks the sub-chunks
//            backwards. For sub-chunk i
//            with within-sub-chunk cumulative c_t (log2) and total T_i, S_i the
//            state before it and Lambda_i the adjoint after it (carried):
//              Qh_t = scale q_t 2^{c_t}, Kt_s = beta_s k_s 2^{-c_s},
//              A = (Qh Kt^T) masked t >= s, dA = (dO V^T) masked t >= s,
//              dq_t  = scale 2^{c_t} (S_i do_t + sum_s dA_ts Kt_s)
//              u_s   = 2^{-c_s} (2^{T_i} Lambda_i v_s + sum_t dA_ts Qh_t)
//              dk_s  = beta_s u_s,  dbeta_s = k_s . u_s
//              dv_s  = (Kt_s 2^{T_i})^T Lambda_i + sum_t A_ts do_t
//              Lambda_{i-1} = 2^{T_i} Lambda_i + sum_t Qh_t do_t^T.
//            S_i is never formed: S_i = 2^{T_0 + .. + T_{i-1}} S_c + sum over
//            j < i of 2^{T_j + .. + T_{i-1}} Kt_j^T V_j, so S_i do_t takes S_c
//            (bf16, as stored) and the blocks dA_ij = dO_i V_j^T, each scaled
//            per key channel. The blocks A_ii and dA_ij (j <= i) are computed
//            once per chunk and shared through LDS.
//            dg_t is the sum over u >= t in the chunk of (q_u dq_u - k_u dk_u)
//            plus G_c = sum_e Lambda_c * S_end (S_end the state after the
//            chunk: the next chunk's stored S, or the final state): the gate
//            gradient at the chunk's first following token, which stands for
//            all later tokens and the final-state cotangent.
//
// MFMA operand conventions (v_mfma_f32_16x16x16_bf16 and _16x16x32_bf16):
// operand lane l has row (A) or column (B) l%16 and contraction slots of lane
// group l/16; a 16x16 fp32 result has column l%16 and rows 4(l/16)+j. So a
// result X serves directly as the B operand of X or the A operand of X^T,
// and tiles of two adjacent result blocks feed a 16x16x32 product whose other
// operand is read with the same contraction-index permutation. Lambda is kept
// in two orientations (key channels per lane for the products contracting
// over Dv, value channels per lane for those over Dk). A 16x16x16 product never accumulates
// straight onto a 16x16x32 result: its own accumulator is added afterwards
// (taking the first as its C operand gave wrong rows).

#include "common.h"

namespace pkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kC = 64;
constexpr int kPlanThreads = 1024;
// Long segments are cut into pieces by their own chunk count only (as in the
// forward pass): more than kCutMin chunks -> pieces of about kPieceLen chunks,
// at most kMaxPieces of them.
constexpr int kCutMin = 128;
constexpr int kPieceLen = 64;
constexpr int kMaxPieces = 16;
constexpr int kRankBins = 2048;  // piece-length bins of the longest-first order
// The plan's record of the piece of each rank: its slot, its index j of the
// slot's m pieces, the slot's first global chunk and chunk count, the segment's
// token bounds (0, 0 when it has no chunk) and its first summary slot.
constexpr int kRecWords = 8;
enum { kRecSlot, kRecPiece, kRecPieces, kRecChunk0, kRecChunks, kRecStart, kRecEnd, kRecSum0 };
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(s16x8 a, s16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(short x) { return __uint_as_float(uint32_t(uint16_t(x)) << 16); }
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ s16x4 pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(s16x4, u32x2{pk2(a, b), pk2(c, d)});
}
__device__ __forceinline__ s16x4 pack4(f32x4 x) { return pack4(x[0], x[1], x[2], x[3]); }
__device__ __forceinline__ s16x8 join(s16x4 lo, s16x4 hi) {
  return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ f32x4 unpack4(s16x4 x) {
  return f32x4{bf2f(x[0]), bf2f(x[1]), bf2f(x[2]), bf2f(x[3])};
}

// Transposing LDS read (ds_read_b64_tr_b16): within a group of 16 lanes, when
// lane k points at row r0 + k/4, column c0 + 4 (k % 4) of a row-major bf16
// tile, lane j receives column c0 + j of rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
// The operand (column c0 + l%16, rows r0 + 4(l/16) .. +3) of a tile with row
// stride rs: the pointer each lane supplies.
__device__ __forceinline__ const bf16* tr_ptr(const bf16* tile, int rs, int r0, int c0, int lane) {
  const int n = lane & 15, g4 = lane >> 4;
  return tile + (r0 + 4 * g4 + (n >> 2)) * rs + c0 + 4 * (n & 3);
}
__device__ __forceinline__ s16x4 ld4(const bf16* p) { return *reinterpret_cast<const s16x4*>(p); }
__device__ __forceinline__ s16x8 ld8(const bf16* p) { return *reinterpret_cast<const s16x8*>(p); }
// The value of another lane of the same 16-lane row (DPP control kCtrl; every lane
// active: the zero-for-invalid-source setting, which never applies within a row,
// lets the compiler fold the move into the add that uses it).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}
// Sum over the 16 lanes of a row, in every lane: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror (lane j of an 8-lane half takes lane 7 - j),
// row_mirror (lane j of the row takes lane 15 - j).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Raw buffer resource over [base, base + bytes): accesses at offsets past the end
// are dropped (stores) or read 0 (loads).
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufFlags);
}
__device__ __forceinline__ void st_bf16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float x) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, bf16(x)), r, int(byte_off), 0, 0);
}

// cu_seqlens entry i; a NULL cu_seqlens is the single segment [0, N).
__device__ __forceinline__ int64_t cu_at(const int32_t* cu, int i, int64_t N) {
  return cu != nullptr ? int64_t(cu[i]) : (i == 0 ? 0 : N);
}

__device__ __forceinline__ bool bad_segment(int64_t start, int64_t end, int64_t N, int slot) {
  return start < 0 || end < start || end > N || (slot == 0 && start != 0);
}

// ---------------------------------------------------------------- plan
// Exclusive scan of x over the threads of the work-group (int64), in LDS.
__device__ __forceinline__ int64_t block_excl_scan(int64_t x, int64_t* s_scan, int64_t& total) {
  const int tid = threadIdx.x;
  s_scan[tid] = x;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int64_t y = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += y;
    __syncthreads();
  }
  const int64_t incl = s_scan[tid];
  total = s_scan[kPlanThreads - 1];
  __syncthreads();
  return incl - x;
}

// base[i]  = global index of slot i's first chunk (base[max_segs] = chunks);
// pbase[i] = index of slot i's first piece: a segment of n chunks is one piece,
//            or, when n exceeds kCutMin, m = min(kMaxPieces, ceil(n / kPieceLen))
//            pieces of nearly equal length (piece j = chunks [n j / m, n (j+1) / m)):
//            a function of n alone, so a segment's gradients never depend on the
//            other segments of the launch; empty slots also get one (empty) piece;
// sbase[i] = index of slot i's first piece summary (cut segments only).
// All are capped at their workspace bounds (reached only when cu_seqlens is
// invalid, which sets the flag).
__global__ __launch_bounds__(kPlanThreads) void kda_bwd_plan_kernel(
    const int32_t* __restrict__ cu, int32_t max_segs, int64_t N, int32_t H, int32_t max_chunks,
    int32_t max_pieces, int32_t max_sums, int32_t* __restrict__ base, int32_t* __restrict__ pbase,
    int32_t* __restrict__ sbase, int32_t* __restrict__ irec, int32_t* __restrict__ counter,
    int32_t* __restrict__ flags) {
  __shared__ int64_t s_scan[kPlanThreads];
  const int tid = threadIdx.x;
  int64_t running = 0, tot;
  for (int tile0 = 0; tile0 < max_segs; tile0 += kPlanThreads) {
    const int slot = tile0 + tid;
    int64_t n = 0;
    if (slot < max_segs) {
      const int64_t start = cu_at(cu, slot, N), end = cu_at(cu, slot + 1, N);
      if (bad_segment(start, end, N, slot)) {
        if (flags != nullptr) atomicOr(flags, kFlagBadCuSeqlens);
      } else {
        n = (end - start + kC - 1) / kC;
      }
    }
    const int64_t b = running + block_excl_scan(n, s_scan, tot);
    if (slot < max_segs) base[slot] = int32_t(b < max_chunks ? b : max_chunks);
    running += tot;
  }
  const int64_t chunks = running < max_chunks ? running : max_chunks;
  if (tid == 0) base[max_segs] = int32_t(chunks);
  __threadfence_block();
  __syncthreads();
  int64_t run_p = 0, run_s = 0, tot_p, tot_s;
  for (int tile0 = 0; tile0 < max_segs; tile0 += kPlanThreads) {
    const int slot = tile0 + tid;
    int64_t m = 0, ms = 0;
    if (slot < max_segs) {
      const int64_t n = int64_t(base[slot + 1]) - base[slot];
      const int64_t mc = (n + kPieceLen - 1) / kPieceLen;
      m = n > kCutMin ? (mc < kMaxPieces ? mc : kMaxPieces) : 1;
      ms = m > 1 ? m : 0;
    }
    const int64_t bp = run_p + block_excl_scan(m, s_scan, tot_p);
    const int64_t bs = run_s + block_excl_scan(ms, s_scan, tot_s);
    if (slot < max_segs) {
      pbase[slot] = int32_t(bp < max_pieces ? bp : max_pieces);
      sbase[slot] = int32_t(bs < max_sums ? bs : max_sums);
    }
    run_p += tot_p;
    run_s += tot_s;
  }
  if (tid == 0) {
    pbase[max_segs] = int32_t(run_p < max_pieces ? run_p : max_pieces);
    sbase[max_segs] = int32_t(run_s < max_sums ? run_s : max_sums);
    *counter = 0;
  }
  __threadfence_block();
  __syncthreads();
  // rank r = the r-th piece, longest first (a counting sort over the pieces'
  // chunk counts, capped at kRankBins - 1; ties in any order: results do not
  // depend on the order)
  __shared__ int s_bin[kRankBins];
  for (int b = tid; b < kRankBins; b += kPlanThreads) s_bin[b] = 0;
  __syncthreads();
  const int npieces = pbase[max_segs];
  auto piece_slot = [&](int pc) {
    int lo = 0, hi = max_segs - 1;  // the slot: last i with pbase[i] <= pc
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pbase[mid] <= pc) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto piece_bin = [&](int pc, int lo) {
    const int64_t nn = int64_t(base[lo + 1]) - base[lo];
    const int64_t jj = pc - pbase[lo], mm = int64_t(pbase[lo + 1]) - pbase[lo];
    const int64_t len = mm > 0 ? nn * (jj + 1) / mm - nn * jj / mm : 0;
    return int(len < kRankBins - 1 ? len : kRankBins - 1);
  };
  for (int pc = tid; pc < npieces; pc += kPlanThreads) atomicAdd(&s_bin[piece_bin(pc, piece_slot(pc))], 1);
  __syncthreads();
  // exclusive prefix over the bins from the longest down; thread t takes the
  // kRankBins / kPlanThreads bins below kRankBins - 1 - t * that many
  constexpr int kPer = kRankBins / kPlanThreads;
  int cnt[kPer], sum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    cnt[u] = s_bin[kRankBins - 1 - (tid * kPer + u)];
    sum += cnt[u];
  }
  int64_t all;
  int64_t before = block_excl_scan(sum, s_scan, all);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    s_bin[kRankBins - 1 - (tid * kPer + u)] = int(before);  // the bin's first rank
    before += cnt[u];
  }
  __syncthreads();
  // irec[r]: what a pass needs of the piece of rank r, in one record (the passes
  // read it with one load instead of chains of dependent ones)
  for (int pc = tid; pc < npieces; pc += kPlanThreads) {
    const int sl = piece_slot(pc);
    const int r = atomicAdd(&s_bin[piece_bin(pc, sl)], 1);
    int32_t* e = irec + kRecWords * int64_t(r);
    const int n = base[sl + 1] - base[sl];
    e[kRecSlot] = sl;
    e[kRecPiece] = pc - pbase[sl];
    e[kRecPieces] = pbase[sl + 1] - pbase[sl];
    e[kRecChunk0] = base[sl];
    e[kRecChunks] = n;
    e[kRecStart] = n > 0 ? int32_t(cu_at(cu, sl, N)) : 0;
    e[kRecEnd] = n > 0 ? int32_t(cu_at(cu, sl + 1, N)) : 0;
    e[kRecSum0] = sbase[sl];
  }
}

// Last index i in [0, n) with tab[i] <= x (tab non-decreasing, tab[0] <= x).
__device__ __forceinline__ int last_le(const int32_t* tab, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- state pass
// One wave per 16 key channels (as in the chunk pass); the gate scan of a
// chunk is split over four quarters of 16 tokens per channel; the raw inputs
// of the next chunk are loaded into registers while the current one is
// scanned and applied.
template <int DK, int DV>
struct StCfg {
  static constexpr int NW = DK / 16, NT = 64 * NW;
  static constexpr int RX = DK + 8, RY = DV + 8;
  static constexpr int o_x = 0;                        // bf16 [64][RX]: g, then kbar or q'
  static constexpr int o_k = o_x + kC * RX * 2;        // bf16 [64][RX]: k or q
  static constexpr int o_y = o_k + kC * RX * 2;        // bf16 [64][RY]: v or do
  static constexpr int o_beta = o_y + kC * RY * 2;     // fp32 [64]
  static constexpr int o_part = o_beta + kC * 4;       // fp32 [4][DK]: quarter sums of the gate
  static constexpr int o_dec = o_part + 4 * DK * 4;    // fp32 [DK]: 2^B
  static constexpr int bytes = o_dec + DK * 4;
  static constexpr int NX = kC * DK / 8 / NT;          // 16-byte pieces per thread, Dk-wide tile
  static constexpr int NY = kC * DV / 8 / NT;          // ... Dv-wide tile
};

// kSum = false (walk): one work-group per (piece, head), S role only (the grid
// holds no adjoint work-groups): the state at the piece's start is composed
// from the earlier pieces' summaries, then the piece's chunks are walked and
// the state before every chunk is stored.
// kSum = true (summary): one work-group per (summary slot, head, role) of a cut
// segment: the piece walked from a zero state; its end state (S role: after the
// piece; Lambda role: before it) and the product of its decays are stored.
template <int DK, int DV, bool kSum>
__global__ __launch_bounds__(DK * 4, (DK == 64 && DV == 128) ? 2 : 4) void kda_bwd_state_kernel(  // 64 (DK / 16) threads
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const bf16* __restrict__ dout,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ base,
    const int32_t* __restrict__ pbase, const int32_t* __restrict__ sbase,
    const int32_t* __restrict__ irec, int32_t max_segs,
    int32_t units, int64_t N, int32_t H, float scale, const float* __restrict__ initial_state,
    const float* __restrict__ dfinal, bf16* __restrict__ Sws, float* __restrict__ sumL,
    float* __restrict__ sumD, float* __restrict__ gfin, int32_t from_saved) {
  using C = StCfg<DK, DV>;
  constexpr int EB = DV / 16, NT = C::NT, NX = C::NX, NY = C::NY;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* s_x = reinterpret_cast<bf16*>(smem + C::o_x);
  bf16* s_k = reinterpret_cast<bf16*>(smem + C::o_k);
  bf16* s_y = reinterpret_cast<bf16*>(smem + C::o_y);
  float* s_beta = reinterpret_cast<float*>(smem + C::o_beta);
  float* s_part = reinterpret_cast<float*>(smem + C::o_part);
  float* s_dec = reinterpret_cast<float*>(smem + C::o_dec);

  const int64_t pairs = int64_t(units) * H;
  const bool adjoint = int64_t(blockIdx.x) >= pairs;
  const int64_t idx = adjoint ? int64_t(blockIdx.x) - pairs : int64_t(blockIdx.x);
  const int h = int(idx % H);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, g4 = lane >> 4;
  // the unit: a summary slot or a piece (the walk takes the pieces longest first, in
  // the plan's order), its segment slot and piece index j of m
  const int32_t* ubase = kSum ? sbase : pbase;
  if (idx / H >= ubase[max_segs]) return;
  const int32_t* rec = irec + kRecWords * (idx / H);  // (the walk's piece)
  const int u = kSum ? int(idx / H) : 0;
  const int slot = kSum ? last_le(ubase, max_segs, u) : rec[kRecSlot];
  const int j = kSum ? u - ubase[slot] : rec[kRecPiece];
  const int m = kSum ? pbase[slot + 1] - pbase[slot] : rec[kRecPieces];
  if (kSum && (adjoint ? j == 0 : j == m - 1)) return;  // summary not needed
  // With the states saved by the forward call (from_saved), the S role's
  // summaries are not needed, and the walk only takes a segment's last piece when
  // dL/dfinal_state is given: from the saved state before its last chunk, that
  // chunk's update gives the final state.
  const bool fin = !kSum && !adjoint && dfinal != nullptr && j == m - 1;
  if (from_saved && (kSum ? !adjoint : !fin)) return;
  const int cbase = kSum ? base[slot] : rec[kRecChunk0];
  const int64_t nseg = kSum ? int64_t(base[slot + 1]) - cbase : rec[kRecChunks];
  const int cp0 = int(nseg * j / m), c1 = int(nseg * (j + 1) / m);
  const int c0 = (!kSum && from_saved && c1 > cp0) ? c1 - 1 : cp0;
  const int nch = c1 - c0;  // chunks of this piece (walked)
  const int64_t start = nch > 0 ? (kSum ? cu_at(cu, slot, N) : rec[kRecStart]) : 0;
  const int64_t end = nch > 0 ? (kSum ? cu_at(cu, slot + 1, N) : rec[kRecEnd]) : 0;
  const int64_t sh = (int64_t(slot) * H + h) * DK * DV;
  const int d_own = 16 * w + n;  // key channel of this lane's X tiles

  if (!kSum && nch == 0) return;  // empty (or malformed) slot: no state to store
  // summary storage of slot s: L [s][role][h][Dk][Dv], D [s][role][h][Dk]
  auto sumL_at = [&](int s_, bool adj) {
    return sumL + ((int64_t(s_) * 2 + adj) * H + h) * DK * DV + int64_t(d_own) * DV + 4 * g4;
  };
  auto sumD_at = [&](int s_, bool adj) { return sumD + ((int64_t(s_) * 2 + adj) * H + h) * DK + d_own; };

  // X^T tiles: rows e = 16E + 4g4 + j, column d_own.
  f32x4 X[EB];
  float Dprod = 1.f;  // product of the decays applied (summary)
  if (kSum) {
#pragma unroll
    for (int E = 0; E < EB; ++E) X[E] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (from_saved && c0 > 0) {
    const bf16* Sp = Sws + (int64_t(cbase + c0) * H + h) * DK * DV + int64_t(d_own) * DV + 4 * g4;
#pragma unroll
    for (int E = 0; E < EB; ++E) X[E] = unpack4(ld4(Sp + 16 * E));
  } else {
    const float* src = adjoint ? dfinal : initial_state;
#pragma unroll
    for (int E = 0; E < EB; ++E)
      X[E] = src ? *reinterpret_cast<const f32x4*>(src + sh + int64_t(d_own) * DV + 16 * E + 4 * g4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    // compose over the other pieces: S <- D S + L over pieces 0 .. j-1 in order;
    // Lambda <- D Lambda + L' over pieces m-1 .. j+1
    if (m > 1) {
      const int nj = adjoint ? m - 1 - j : j;
      for (int t = 0; t < nj; ++t) {
        const int jj = adjoint ? m - 1 - t : t;
        const int s_ = rec[kRecSum0] + jj;  // (the walk only: summaries start from zero)
        const float dprod = *sumD_at(s_, adjoint);
        const float* Lp = sumL_at(s_, adjoint);
#pragma unroll
        for (int E = 0; E < EB; ++E) X[E] = dprod * X[E] + *reinterpret_cast<const f32x4*>(Lp + 16 * E);
      }
    }
  }
  auto store_state = [&](bf16* ws, int gc) {
    const int64_t off = (int64_t(gc) * H + h) * DK * DV + int64_t(d_own) * DV + 4 * g4;
#pragma unroll
    for (int E = 0; E < EB; ++E) *reinterpret_cast<s16x4*>(ws + off + 16 * E) = pack4(X[E]);
  };

  // raw inputs of one chunk: g, k (or q), v (or do), beta, as 16-byte pieces
  const bf16* srcK = adjoint ? q : k;
  const bf16* srcY = adjoint ? dout : v;
  s16x8 px[NX], pk[NX], py[NY];
  bf16 pb = bf16(0.f);  // converted when stored, so the load is not waited for early
  auto fetch = [&](int c) {
    const int64_t a = start + int64_t(kC) * c;
    const int L = int(end - a < kC ? end - a : kC);
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + NT * r, t = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
      const int64_t off = ((a + t) * H + h) * DK + c8;
      px[r] = t < L ? *reinterpret_cast<const s16x8*>(g + off) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      pk[r] = t < L ? *reinterpret_cast<const s16x8*>(srcK + off) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < NY; ++r) {
      const int i = tid + NT * r, t = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
      py[r] = t < L ? *reinterpret_cast<const s16x8*>(srcY + ((a + t) * H + h) * DV + c8)
                    : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    pb = (!adjoint && tid < L) ? beta[(a + tid) * H + h] : bf16(0.f);
  };
  auto put = [&]() {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int i = tid + NT * r, t = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
      *reinterpret_cast<s16x8*>(s_x + t * C::RX + c8) = px[r];
      *reinterpret_cast<s16x8*>(s_k + t * C::RX + c8) = pk[r];
    }
#pragma unroll
    for (int r = 0; r < NY; ++r) {
      const int i = tid + NT * r, t = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
      *reinterpret_cast<s16x8*>(s_y + t * C::RY + c8) = py[r];
    }
    if (tid < kC) s_beta[tid] = to_f32(pb);
  };

  // S role: chunks c0 .. c1-1 (a walk stores S before each and skips the last
  // update, except in a segment's last piece when dL/dfinal_state is given: there
  // it reaches the final state); Lambda role: chunks c1-1 .. c0, every update applied
  const int napply = (adjoint || kSum || fin) ? nch : nch - 1;
  auto chunk_of = [&](int it) { return adjoint ? c1 - 1 - it : c0 + it; };
  auto step = [&]() {  // the chunk whose inputs are in LDS: scan, then update X
    __syncthreads();
    {
      // quarter p4 of the tokens of channel d: local log2 cumulative gate
      const int p4 = tid / DK, d = tid % DK;
      float lb[16], acc = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        acc += to_f32(s_x[(16 * p4 + u) * C::RX + d]) * kLog2e;
        lb[u] = acc;
      }
      s_part[p4 * DK + d] = acc;
      __syncthreads();
      float off = 0.f, B = 0.f;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const float x = s_part[pp * DK + d];
        off += pp < p4 ? x : 0.f;
        B += x;
      }
      // eight tokens at a time, their reads before the in-place writes over g
#pragma unroll
      for (int u0 = 0; u0 < 16; u0 += 8) {
        float kq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kq[u] = to_f32(s_k[(16 * p4 + u0 + u) * C::RX + d]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int t = 16 * p4 + u0 + u;
          // forward: kbar = beta k 2^{B - b_t}; adjoint: q' = scale q 2^{b_t}
          s_x[t * C::RX + d] = adjoint ? bf16(scale * kq[u] * ex2(off + lb[u0 + u]))
                                       : bf16(s_beta[t] * kq[u] * ex2(B - (off + lb[u0 + u])));
        }
      }
      if (p4 == 0) s_dec[d] = ex2(B);
    }
    __syncthreads();
    const float dec = s_dec[d_own];
    if (kSum) Dprod *= dec;
#pragma unroll
    for (int E = 0; E < EB; ++E) X[E] *= dec;
#pragma unroll
    for (int kb = 0; kb < kC / 16; ++kb) {
      const s16x4 xb = tr4(tr_ptr(s_x, C::RX, 16 * kb, 16 * w, lane));
#pragma unroll
      for (int E = 0; E < EB; ++E) X[E] = mfma16(tr4(tr_ptr(s_y, C::RY, 16 * kb, 16 * E, lane)), xb, X[E]);
    }
    __syncthreads();
  };
  // Branch-free main loop (one vector-memory counter covers loads and stores, so a
  // conditional store or load here would make the wait for the prefetched inputs wait
  // for the stores too): the prefetch index is clamped, and the last step is peeled.
  bf16* ws_out = Sws;
  if (napply > 0) {
    fetch(chunk_of(0));
    put();
    fetch(chunk_of(napply > 1 ? 1 : 0));
  }
  // (a segment's first state is zero without an initial state: not stored, the
  // chunk pass takes zeros for it)
  if (!kSum && !from_saved && (c0 > 0 || initial_state != nullptr)) store_state(ws_out, cbase + chunk_of(0));
  for (int it = 0; it < napply - 1; ++it) {
    step();
    put();
    fetch(chunk_of(it + 2 < napply ? it + 2 : napply - 1));
    if (!kSum && !from_saved) store_state(ws_out, cbase + chunk_of(it + 1));
  }
  if (napply > 0) {
    step();
    if (!kSum && !from_saved && napply < nch) store_state(ws_out, cbase + chunk_of(napply));
  }
  if (fin) {
    // the gate gradient at the segment's end: sum_e dL/dS_final * S_final, per key channel
    float p = 0.f;
#pragma unroll
    for (int E = 0; E < EB; ++E) {
      const f32x4 df = *reinterpret_cast<const f32x4*>(dfinal + sh + int64_t(d_own) * DV + 16 * E + 4 * g4);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) p = fmaf(df[jj], X[E][jj], p);
    }
    p += __shfl_xor(p, 16, 64);
    p += __shfl_xor(p, 32, 64);
    if (g4 == 0) gfin[(int64_t(slot) * H + h) * DK + d_own] = p;
  }
  if (kSum) {
    const int s_ = u;
    float* Lp = sumL_at(s_, adjoint);
#pragma unroll
    for (int E = 0; E < EB; ++E) *reinterpret_cast<f32x4*>(Lp + 16 * E) = X[E];
    if (g4 == 0) *sumD_at(s_, adjoint) = Dprod;
    return;
  }
}

// ---------------------------------------------------------------- chunk pass
template <int DK, int DV>
struct ChCfg {
  // one wave per 16 key channels: 8 waves at Dk = 128, 4 at Dk = 64
  static constexpr int NW = DK / 16, NT = 64 * NW;
  static constexpr int RK = DK + 8, RV = DV + 8;
  static constexpr int o_q = 0;                         // bf16 [64][RK] raw q
  static constexpr int o_k = o_q + kC * RK * 2;         // raw k
  static constexpr int o_qh = o_k + kC * RK * 2;        // Qh = scale q 2^{c}
  static constexpr int o_kt = o_qh + kC * RK * 2;       // Kt = beta k 2^{-c}
  static constexpr int o_v = o_kt + kC * RK * 2;        // bf16 [64][RV]
  static constexpr int o_do = o_v + kC * RV * 2;
  // fp32 [DK][64]: 2^{c_t}, channel-major, the 4-token groups of row d at group
  // (t / 4) ^ sigma(d), sigma(d) = (d / 4 % 16) ^ (4 (d % 4)): the f32x4 of 16
  // consecutive channels, or of 16 channels 4 apart, meet no bank twice
  static constexpr int o_E = o_do + kC * RV * 2;
  // fp32 [7][DK]: 2^{T_j + .. + T_{i-1}} for j < i <= 3 at row i (i - 1) / 2 + j, and
  // 2^{T_3} at row 6; its first word also passes the next item's index at item ends
  static constexpr int o_fP = o_E + DK * kC * 4;
  // fp32 [4][DK]: the sub-chunk totals (log2) after the gate scan; in the same words
  // later, fp32 [4 sub-chunks][NW waves][16]: dbeta partials
  static constexpr int o_db = o_fP + 7 * DK * 4;
  static constexpr int o_T = o_db;
  static constexpr int o_beta = o_db + 4 * NW * 16 * 4; // fp32 [64]
  // bf16 [14][16][16] sub-chunk blocks, each stored column-major ([s][t]): the four
  // masked diagonal blocks of A, then dA (i, j) for j <= i at 4 + i (i + 1) / 2 + j
  static constexpr int o_blk = o_beta + kC * 4;
  static constexpr int bytes = o_blk + 14 * 256 * 2;
  // persistent work-groups per CU: as many as the LDS holds (two at Dk = Dv = 64)
  static constexpr int WG_PER_CU = bytes <= 80 * 1024 ? 2 : 1;
  static_assert(DK != 64 || DV != 64 || WG_PER_CU == 2, "two work-groups per CU at Dk = Dv = 64");
};

template <int DK, int DV>
__global__ __launch_bounds__(DK * 4, (DK == 64 && DV == 64) ? 2 : 1) void kda_bwd_chunk_kernel(  // 64 (DK / 16) threads
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const bf16* __restrict__ dout,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ base,
    const int32_t* __restrict__ pbase, const int32_t* __restrict__ sbase,
    const int32_t* __restrict__ irec, int32_t* __restrict__ counter,
    int32_t max_segs, int64_t N,
    int32_t H, float scale, const float* __restrict__ dfinal, const float* __restrict__ sumL,
    const float* __restrict__ sumD, const float* __restrict__ gfin, const bf16* __restrict__ Sws, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, bf16* __restrict__ dg, bf16* __restrict__ dbeta,
    float* __restrict__ dinit, int32_t* __restrict__ flags, int32_t has_init) {
  using C = ChCfg<DK, DV>;
  constexpr int NW = C::NW, NT = C::NT;
  // key block w per wave; value blocks split over the waves (at Dv < Dk only the
  // first Dv / 16 waves take one)
  constexpr int DB = DK / 16, EB = DV / 16, DBW = 1, EBW = EB >= NW ? EB / NW : 1;
  constexpr int RK = C::RK, RV = C::RV;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* s_q = reinterpret_cast<bf16*>(smem + C::o_q);
  bf16* s_k = reinterpret_cast<bf16*>(smem + C::o_k);
  bf16* s_qh = reinterpret_cast<bf16*>(smem + C::o_qh);
  bf16* s_kt = reinterpret_cast<bf16*>(smem + C::o_kt);
  bf16* s_v = reinterpret_cast<bf16*>(smem + C::o_v);
  bf16* s_do = reinterpret_cast<bf16*>(smem + C::o_do);
  float* s_E = reinterpret_cast<float*>(smem + C::o_E);
  float* s_T = reinterpret_cast<float*>(smem + C::o_T);
  float* s_db = reinterpret_cast<float*>(smem + C::o_db);
  float* s_beta = reinterpret_cast<float*>(smem + C::o_beta);
  float* s_fP = reinterpret_cast<float*>(smem + C::o_fP);
  bf16* s_blk = reinterpret_cast<bf16*>(smem + C::o_blk);
  int* s_item = reinterpret_cast<int*>(smem + C::o_fP);
  // row of 2^{T_j + .. + T_{i-1}} in s_fP (j < i <= 3, or j = 3, i = 4)
  auto pidx = [](int j, int i) { return i < 4 ? i * (i - 1) / 2 + j : 6; };
  auto ft_row = [&](int i) { return pidx(i, i + 1); };  // 2^{T_i}
  // word of 2^{c_t} at channel d, token t in s_E
  auto e_off = [](int d, int t) {
    return d * kC + ((((t >> 2) ^ ((d >> 2) & 15) ^ ((d & 3) << 2))) << 2) + (t & 3);
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, n = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const bool ev_active = EB >= NW || w < EB;  // wave-uniform
  auto eblk = [&](int ee) { return EB >= NW ? w * EBW + ee : w; };
  const int d_own = 16 * w + n;  // key channel of this lane's L1 tiles (DBW = 1)
  // Persistent work-groups over (piece, head) items, longest piece first (the
  // plan's order; item = rank * H + h). A work-group claims its next item when
  // it starts the current item's last chunk, and walks the piece's chunks from
  // the last to the first, carrying Lambda (the adjoint after the chunk) in
  // registers from one chunk to the one before it.
  const int n_items = pbase[max_segs] * H;
  if (tid == 0) *s_item = atomicAdd(counter, 1);
  __syncthreads();
  int item = __builtin_amdgcn_readfirstlane(*s_item);
  while (item < n_items) {
    const int rank = item / H, h = item % H;
    // the plan's record of the piece (one uniform load)
    const int32_t* rec = irec + kRecWords * rank;
    const int slot = rec[kRecSlot], j = rec[kRecPiece], m = rec[kRecPieces];
    const int cbase = rec[kRecChunk0], nseg = rec[kRecChunks];
    const int c0 = int(int64_t(nseg) * j / m), c1 = int(int64_t(nseg) * (j + 1) / m);
    const int64_t seg_start = rec[kRecStart], seg_end = rec[kRecEnd];
    const int sum0 = rec[kRecSum0];
    const int64_t sh = (int64_t(slot) * H + h) * DK * DV;
    int next = 0;

    // Lambda after the piece: dL/dfinal_state (or 0), composed with the later
    // pieces' adjoint summaries (Lambda <- D Lambda + L' over pieces m-1 .. j+1),
    // in both orientations: L1[E][dd] (rows e, column d = 16 (w DBW + dd) + n)
    // and L2[D][ee] (rows d = 16 D + 4 g4 + i, column e = 16 eblk(ee) + n).
    f32x4 L1[EB][DBW], L2[DB][EBW];
#pragma unroll
    for (int E = 0; E < EB; ++E)
      L1[E][0] = dfinal ? *reinterpret_cast<const f32x4*>(dfinal + sh + int64_t(d_own) * DV + 16 * E + 4 * g4)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int D = 0; D < DB; ++D)
#pragma unroll
      for (int ee = 0; ee < EBW; ++ee) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          L2[D][ee][i] = (dfinal && ev_active)
                             ? dfinal[sh + int64_t(16 * D + 4 * g4 + i) * DV + 16 * eblk(ee) + n] : 0.f;
      }
    for (int t = 0; t < m - 1 - j; ++t) {
      const int s_ = sum0 + (m - 1 - t);
      const int64_t ls = ((int64_t(s_) * 2 + 1) * H + h) * DK;  // adjoint role
      const float* Lp = sumL + ls * DV;
      const float* Dp = sumD + ls;
      const float dprod = Dp[d_own];
#pragma unroll
      for (int E = 0; E < EB; ++E)
        L1[E][0] = dprod * L1[E][0] + *reinterpret_cast<const f32x4*>(Lp + int64_t(d_own) * DV + 16 * E + 4 * g4);
#pragma unroll
      for (int D = 0; D < DB; ++D) {
        const f32x4 dr = *reinterpret_cast<const f32x4*>(Dp + 16 * D + 4 * g4);
#pragma unroll
        for (int ee = 0; ee < EBW; ++ee)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            L2[D][ee][i] = ev_active ? dr[i] * L2[D][ee][i] + Lp[int64_t(16 * D + 4 * g4 + i) * DV + 16 * eblk(ee) + n]
                                     : 0.f;
      }
    }
    // G, per key channel: the gate gradient from everything after the chunk being
    // walked, sum_e Lambda * S_end (Lambda the adjoint after the chunk, S_end the
    // state after it). S_end of the piece's last chunk is the next piece's first
    // stored state, or at the segment's end the final state (the walk leaves its
    // product with dL/dfinal_state); for every other chunk it is the S_c of the
    // chunk walked before it.
    auto sdot = [&](const s16x4 (&Sx)[EB][DBW]) {
      float p = 0.f;
#pragma unroll
      for (int E = 0; E < EB; ++E)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) p = fmaf(L1[E][0][jj], bf2f(Sx[E][0][jj]), p);
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      return p;
    };
    float r = 0.f;
    if (c1 > c0 && c1 < nseg) {
      const bf16* Sn = Sws + (int64_t(cbase + c1) * H + h) * DK * DV + int64_t(d_own) * DV + 4 * g4;
      s16x4 Sx[EB][DBW];
#pragma unroll
      for (int E = 0; E < EB; ++E) Sx[E][0] = ld4(Sn + 16 * E);
      r = sdot(Sx);
    } else if (c1 > c0 && gfin != nullptr) {
      r = gfin[(int64_t(slot) * H + h) * DK + d_own];
    }
    if (c1 == c0 && tid == 0) next = atomicAdd(counter, 1);  // empty piece

    for (int c = c1 - 1; c >= c0; --c) {
      if (c == c0 && tid == 0) next = atomicAdd(counter, 1);
      const int gc = cbase + c;
      const int64_t a = seg_start + int64_t(kC) * c;
      const int L = int(seg_end - a < kC ? seg_end - a : kC);
      const int nsub = (L + 15) >> 4;
      // gradient rows of this chunk's tokens (all heads); stores past token L are dropped
      const auto r_dq = rsrc(dq + a * H * DK, uint32_t(L) * H * DK * 2);
      const auto r_dk = rsrc(dk + a * H * DK, uint32_t(L) * H * DK * 2);
      const auto r_dg = rsrc(dg + a * H * DK, uint32_t(L) * H * DK * 2);
      const auto r_dv = rsrc(dv + a * H * DV, uint32_t(L) * H * DV * 2);
      const int64_t soff = (int64_t(gc) * H + h) * DK * DV;
      // S_c from the workspace, raw bf16 (the zero state before a segment's first
      // chunk without an initial state is not stored: an empty range reads zeros
      // without touching memory). Loaded once the chunk's tiles are in LDS: the
      // tiles' loads then have the work-group's outstanding requests to themselves,
      // and S_c's latency overlaps the gate scan and the sub-chunk blocks.
      s16x4 Sc[EB][DBW];
      const auto rs = rsrc(Sws + soff, (c > 0 || has_init) ? DK * DV * 2 : 0);

      // ---- load: rows of q, k, g (g into the Qh tile), v and do with 16-byte loads,
      // all issued before the first LDS store
      // Buffer resources over the chunk's rows of head h (32-bit offsets, rows
      // past the chunk's end read 0): a 64-bit address per lane and tensor
      // would be held across the chunk loop.
      {
        constexpr int NX = kC * DK / 8 / NT, NY = kC * DV / 8 / NT;
        const uint32_t rowK = uint32_t(H) * DK * 2, rowV = uint32_t(H) * DV * 2;
        const int64_t tb = a * H + h;  // token a, head h
        const uint32_t nK = uint32_t(L - 1) * rowK + DK * 2, nV = uint32_t(L - 1) * rowV + DV * 2;
        const auto rq = rsrc(q + tb * DK, nK), rk = rsrc(k + tb * DK, nK), rg = rsrc(g + tb * DK, nK);
        const auto rv = rsrc(v + tb * DV, nV), rd = rsrc(dout + tb * DV, nV);
        const auto rb = rsrc(beta + tb, uint32_t(L - 1) * H * 2 + 2);
        auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
          return __builtin_bit_cast(s16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        };
        s16x8 xq[NX], xk[NX], xg[NX], xv[NY], xd[NY];
#pragma unroll
        for (int r = 0; r < NX; ++r) {
          const int i = tid + NT * r, t = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
          const uint32_t off = uint32_t(t) * rowK + c8 * 2;
          xq[r] = ld16(rq, off);
          xk[r] = ld16(rk, off);
          xg[r] = ld16(rg, off);
        }
#pragma unroll
        for (int r = 0; r < NY; ++r) {
          const int i = tid + NT * r, t = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
          const uint32_t off = uint32_t(t) * rowV + c8 * 2;
          xv[r] = ld16(rv, off);
          xd[r] = ld16(rd, off);
        }
        const unsigned short xb = __builtin_amdgcn_raw_buffer_load_b16(rb, uint32_t(tid < kC ? tid : kC) * H * 2, 0, 0);
        // (every wave is past the previous chunk's LDS reads: its last barrier)
#pragma unroll
        for (int r = 0; r < NX; ++r) {
          const int i = tid + NT * r, t = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
          *reinterpret_cast<s16x8*>(s_q + t * RK + c8) = xq[r];
          *reinterpret_cast<s16x8*>(s_k + t * RK + c8) = xk[r];
          *reinterpret_cast<s16x8*>(s_qh + t * RK + c8) = xg[r];
        }
#pragma unroll
        for (int r = 0; r < NY; ++r) {
          const int i = tid + NT * r, t = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
          *reinterpret_cast<s16x8*>(s_v + t * RV + c8) = xv[r];
          *reinterpret_cast<s16x8*>(s_do + t * RV + c8) = xd[r];
        }
        if (tid < kC) s_beta[tid] = __uint_as_float(uint32_t(xb) << 16);
      }
      __syncthreads();
#pragma unroll
      for (int E = 0; E < EB; ++E)
        Sc[E][0] = __builtin_bit_cast(s16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                                 rs, uint32_t(d_own * DV + 16 * E + 4 * g4) * 2, 0, 0));
      // per (sub-chunk, channel): 2^{c_t}, Qh over g, Kt, and the sub-chunk total
      {
        // thread: sub-chunk j, channels d .. d + 3 (one 8-byte word of each bf16 row),
        // tokens 4 qt .. 4 qt + 3 of the sub-chunk; the four quarters qt of a unit sit
        // in the four 16-lane rows of one wave
        static_assert(NT == 4 * DK, "one thread per (sub-chunk, channel quad, quarter)");
        const int qt = g4, unit = 16 * w + n;
        const int j = unit / (DK / 4), d = 4 * (unit % (DK / 4)), tb = 16 * j + 4 * qt;
        // all reads first (Qh overwrites g in place)
        u32x2 gv[4], qv[4], kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = tb + u;
          gv[u] = *reinterpret_cast<const u32x2*>(s_qh + t * RK + d);
          qv[u] = *reinterpret_cast<const u32x2*>(s_q + t * RK + d);
          kv[u] = *reinterpret_cast<const u32x2*>(s_k + t * RK + d);
        }
        // channel d + ch of a row word pair
        auto chv = [](u32x2 x, int ch) {
          const uint32_t wd = x[ch >> 1];
          return __uint_as_float((ch & 1) ? (wd & 0xffff0000u) : (wd << 16));
        };
        // the quarter's gate sum per channel, then the sums of the quarters before it
        // (the rows of the lane's row pair by v_permlane16_swap, the pair sums by
        // v_permlane32_swap)
        float c[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          float p = 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) p += chv(gv[u], ch);
          const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
          const float ev = __uint_as_float(pr[0]), od = __uint_as_float(pr[1]);
          const float pair = ev + od;
          const auto pt = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
          c[ch] = (((qt & 1) ? ev : 0.f) + ((qt & 2) ? __uint_as_float(pt[0]) : 0.f)) * kLog2e;
        }
        float e[4][4];  // [channel][token]
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = tb + u;
          float ek[4];
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) {
            c[ch] += chv(gv[u], ch) * kLog2e;
            e[ch][u] = ex2(c[ch]);
            ek[ch] = ex2(-c[ch]);
          }
          *reinterpret_cast<u32x2*>(s_qh + t * RK + d) =
              u32x2{pk2(scale * chv(qv[u], 0) * e[0][u], scale * chv(qv[u], 1) * e[1][u]),
                    pk2(scale * chv(qv[u], 2) * e[2][u], scale * chv(qv[u], 3) * e[3][u])};
          const float bt = s_beta[t];
          *reinterpret_cast<u32x2*>(s_kt + t * RK + d) =
              u32x2{pk2(bt * chv(kv[u], 0) * ek[0], bt * chv(kv[u], 1) * ek[1]),
                    pk2(bt * chv(kv[u], 2) * ek[2], bt * chv(kv[u], 3) * ek[3])};
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch)
          *reinterpret_cast<f32x4*>(s_E + e_off(d + ch, tb)) = f32x4{e[ch][0], e[ch][1], e[ch][2], e[ch][3]};
        if (qt == 3) {
          *reinterpret_cast<f32x4*>(s_T + j * DK + d) = f32x4{c[0], c[1], c[2], c[3]};
          // 2^{-c} of Kt can leave the fp32 / bf16 range below this total
          const float cm = fminf(fminf(c[0], c[1]), fminf(c[2], c[3]));
          if (cm < kGateRangeMinLog2 && flags != nullptr) atomicOr(flags, kFlagGateRange);
        }
      }
      __syncthreads();
      // decay factors of whole sub-chunks, once per chunk
      if (tid < DK) {
        const int d = tid;
        float T[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) T[j] = s_T[j * DK + d];
#pragma unroll
        for (int i = 1; i <= 3; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int j = i - 1; j >= 0; --j) {
            acc += T[j];
            s_fP[pidx(j, i) * DK + d] = ex2(acc);
          }
        }
        s_fP[pidx(3, 4) * DK + d] = ex2(T[3]);
      }
      // the sub-chunk blocks, each computed by one wave (wave w takes blocks w, w +
      // NW, ..): A_ii = Qh_i Kt_i^T and dA_ij = dO_i V_j^T for j <= i, rows t and
      // columns s, the diagonal blocks masked to t >= s
      for (int b = w; b < 14; b += NW) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        bool diag = true;
        if (b < 4) {
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb)
            acc = mfma32(ld8(s_qh + (16 * b + n) * RK + 32 * kb + 8 * g4),
                         ld8(s_kt + (16 * b + n) * RK + 32 * kb + 8 * g4), acc);
        } else {
          const int x = b - 4, i = x < 1 ? 0 : x < 3 ? 1 : x < 6 ? 2 : 3, jb = x - i * (i + 1) / 2;
          diag = jb == i;
#pragma unroll
          for (int kb = 0; kb < DV / 32; ++kb)
            acc = mfma32(ld8(s_do + (16 * i + n) * RV + 32 * kb + 8 * g4),
                         ld8(s_v + (16 * jb + n) * RV + 32 * kb + 8 * g4), acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = (diag && 4 * g4 + j < n) ? 0.f : acc[j];
        // column-major: element (t, s) at s * 16 + t
        *reinterpret_cast<s16x4*>(s_blk + b * 256 + n * 16 + 4 * g4) = pack4(acc);
      }
      __syncthreads();

      for (int i = nsub - 1; i >= 0; --i) {
        const int t0 = 16 * i;
        const bf16* blkA = s_blk + i * 256;                          // A_ii
        const bf16* blkD = s_blk + (4 + i * (i + 1) / 2 + i) * 256;  // dA_ii
        const s16x4 opAT = ld4(blkA + n * 16 + 4 * g4);              // A-operand of A^T (rows s, slots t)
        const s16x4 opdAT = ld4(blkD + n * 16 + 4 * g4);             // A-operand of dA^T (rows s, slots t)
        const s16x4 opdA = tr4(tr_ptr(blkD, 16, 0, 0, lane));        // A-operand of dA (rows t, slots s)
        // dA_tt as those operands hold it (bf16) for this lane's tokens t = t0 +
        // 4 g4 + j. The products dA_tt Kt_t (in dq) and dA_tt Qh_t (in u) are the
        // token's pair with itself: in q dq - k dk they cancel exactly, but only
        // to bf16 rounding as computed, which swamps a small gate gradient
        // (strong forgetting); dg takes both sums without them.
        f32x4 dgs;
#pragma unroll
        for (int j = 0; j < 4; ++j) dgs[j] = bf2f(reinterpret_cast<const short*>(blkD)[(4 * g4 + j) * 17]);

        // 2^{T_i} Lambda_i in both orientations: used by u and dv, and the update
        // to Lambda before sub-chunk i accumulates onto it
#pragma unroll
        for (int dd = 0; dd < DBW; ++dd) {
          const float fT = s_fP[ft_row(i) * DK + 16 * (w * DBW + dd) + n];
#pragma unroll
          for (int E = 0; E < EB; ++E) L1[E][dd] *= fT;
        }
        if (ev_active) {
#pragma unroll
          for (int D = 0; D < DB; ++D) {
            const f32x4 fr = *reinterpret_cast<const f32x4*>(s_fP + ft_row(i) * DK + 16 * D + 4 * g4);
#pragma unroll
            for (int ee = 0; ee < EBW; ++ee) L2[D][ee] *= fr;
          }
        }

        float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dd = 0; dd < DBW; ++dd) {
          const int Dblk = w * DBW + dd;
          const int d = 16 * Dblk + n;
          // dq: dO S_i^T + dA Kt, then scale 2^{c_t}, with S_i (the state before
          // sub-chunk i) = 2^{T_0 + .. + T_{i-1}} S_c plus, per earlier sub-chunk j,
          // 2^{T_j + .. + T_{i-1}} Kt_j^T V_j: dO S_i^T takes the first term from S_c
          // (bf16, as stored) and the others as dA_ij Kt_j, each scaled per channel
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int P = 0; P < EB / 2; ++P) {
            const s16x8 oa = join(ld4(s_do + (t0 + n) * RV + 32 * P + 4 * g4),
                                  ld4(s_do + (t0 + n) * RV + 32 * P + 16 + 4 * g4));
            acc = mfma32(oa, join(Sc[2 * P][dd], Sc[2 * P + 1][dd]), acc);
          }
          if (i > 0) acc *= s_fP[pidx(0, i) * DK + d];
          for (int j = 0; j < i; ++j) {
            const s16x4 da = tr4(tr_ptr(s_blk + (4 + i * (i + 1) / 2 + j) * 256, 16, 0, 0, lane));
            const s16x4 kj = tr4(tr_ptr(s_kt, RK, 16 * j, 16 * Dblk, lane));
            acc += s_fP[pidx(j, i) * DK + d] * mfma16(da, kj, f32x4{0.f, 0.f, 0.f, 0.f});
          }
          const s16x4 ktv = tr4(tr_ptr(s_kt, RK, t0, 16 * Dblk, lane));  // Kt_t[d]
          acc += mfma16(opdA, ktv, f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 Et = *reinterpret_cast<const f32x4*>(s_E + e_off(d, t0 + 4 * g4));
          const f32x4 qv = unpack4(tr4(tr_ptr(s_q, RK, t0, 16 * Dblk, lane)));
          const f32x4 kv = unpack4(tr4(tr_ptr(s_k, RK, t0, 16 * Dblk, lane)));
          float x[4], dqv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dqv[j] = scale * Et[j] * acc[j];
            x[j] = qv[j] * (scale * Et[j] * (acc[j] - dgs[j] * bf2f(ktv[j])));  // exact product
          }
          // u: (2^{T_i} Lambda_i) v + dA^T Qh, then 2^{-c_s}
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int P = 0; P < EB / 2; ++P) {
            const s16x8 va = join(ld4(s_v + (t0 + n) * RV + 32 * P + 4 * g4),
                                  ld4(s_v + (t0 + n) * RV + 32 * P + 16 + 4 * g4));
            const s16x8 lb = join(pack4(L1[2 * P][dd]), pack4(L1[2 * P + 1][dd]));
            acc = mfma32(va, lb, acc);
          }
          const s16x4 qhv = tr4(tr_ptr(s_qh, RK, t0, 16 * Dblk, lane));  // Qh_t[d]
          acc += mfma16(opdAT, qhv, f32x4{0.f, 0.f, 0.f, 0.f});
          float dkv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = t0 + 4 * g4 + j;
            const float re = __builtin_amdgcn_rcpf(Et[j]);
            const float u = acc[j] * re;
            dkv[j] = s_beta[t] * u;
            x[j] -= kv[j] * (s_beta[t] * ((acc[j] - dgs[j] * bf2f(qhv[j])) * re));
            db[j] = fmaf(kv[j], u, db[j]);
          }
          // dg: suffix sum over the sub-chunk's tokens, plus everything after it
          float suf[4];
          suf[3] = x[3];
          suf[2] = x[2] + suf[3];
          suf[1] = x[1] + suf[2];
          suf[0] = x[0] + suf[1];
          // the four rows' sums at this lane's column: rows 2m, 2m + 1 of the lane's
          // row pair (v_permlane16_swap), then pair sums of rows 0-1 and 2-3
          // (v_permlane32_swap)
          const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(suf[0]), __float_as_uint(suf[0]), false, false);
          const float ev = __uint_as_float(pr[0]), od = __uint_as_float(pr[1]), pair = ev + od;
          const auto pt = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
          const float lo = __uint_as_float(pt[0]), hi = __uint_as_float(pt[1]);
          // rows after this lane's row g4
          const float after = ((g4 & 1) ? 0.f : od) + ((g4 & 2) ? 0.f : hi) + r;
          r += lo + hi;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t off = ((uint32_t(t0 + 4 * g4 + j) * H + h) * DK + d) * 2;
            st_bf16(r_dq, off, dqv[j]);
            st_bf16(r_dk, off, dkv[j]);
            st_bf16(r_dg, off, suf[j] + after);
          }
        }
        // dbeta partials: over this lane's channels, then the 16 lanes of a row group
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = row_sum16(db[j]);
          if (n == 0) s_db[(i * NW + w) * 16 + 4 * g4 + j] = p;
        }

        // dv: Kt (2^{T_i} Lambda_i) + A^T dO, columns e of this wave
#pragma unroll
        for (int ee = 0; ee < EBW; ++ee) {
          if (!ev_active) break;
          const int Eblk = eblk(ee);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int P = 0; P < DB / 2; ++P) {
            const int d0 = 32 * P + 4 * g4, d1 = 32 * P + 16 + 4 * g4;
            const s16x8 ka = join(ld4(s_kt + (t0 + n) * RK + d0), ld4(s_kt + (t0 + n) * RK + d1));
            const s16x8 lb = join(pack4(L2[2 * P][ee]), pack4(L2[2 * P + 1][ee]));
            acc = mfma32(ka, lb, acc);
          }
          acc += mfma16(opAT, tr4(tr_ptr(s_do, RV, t0, 16 * Eblk, lane)), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st_bf16(r_dv, ((uint32_t(t0 + 4 * g4 + j) * H + h) * DV + 16 * Eblk + n) * 2, acc[j]);
        }

        // Lambda before sub-chunk i: 2^{T_i} Lambda_i + Qh^T dO (every register index
        // static); after sub-chunk 0 it is Lambda before the chunk, carried to the
        // previous chunk
        {
#pragma unroll
          for (int dd = 0; dd < DBW; ++dd) {
            const s16x4 qb = tr4(tr_ptr(s_qh, RK, t0, 16 * (w * DBW + dd), lane));
#pragma unroll
            for (int E = 0; E < EB; ++E) L1[E][dd] = mfma16(tr4(tr_ptr(s_do, RV, t0, 16 * E, lane)), qb, L1[E][dd]);
          }
#pragma unroll
          for (int ee = 0; ee < EBW; ++ee) {
            if (!ev_active) break;
            const s16x4 ob = tr4(tr_ptr(s_do, RV, t0, 16 * eblk(ee), lane));
#pragma unroll
            for (int D = 0; D < DB; ++D) L2[D][ee] = mfma16(tr4(tr_ptr(s_qh, RK, t0, 16 * D, lane)), ob, L2[D][ee]);
          }
        }
      }
      // G for the chunk before: Lambda before this chunk with S_c, its state after
      r = sdot(Sc);

      __syncthreads();
      if (tid < L) {
        const int i = tid >> 4, s = tid & 15;
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) sum += s_db[(i * NW + ww) * 16 + s];
        dbeta[(a + tid) * H + h] = bf16(sum);
      }
    }  // chunk loop
    // d initial state: Lambda before the segment's first chunk (an empty
    // segment passes dL/dfinal_state through)
    if (j == 0 && dinit != nullptr) {
#pragma unroll
      for (int E = 0; E < EB; ++E)
        *reinterpret_cast<f32x4*>(dinit + sh + int64_t(d_own) * DV + 16 * E + 4 * g4) = L1[E][0];
    }
    if (tid == 0) *s_item = next;
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(*s_item);
    __syncthreads();  // every wave has read it before it is written again
  }  // item loop

  // positions not covered by any segment get zero gradients (grid-strided)
  int64_t cu_last = cu_at(cu, max_segs, N);
  cu_last = cu_last < 0 ? 0 : (cu_last > N ? N : cu_last);
  const int64_t stride = int64_t(gridDim.x) * NT;
  const int64_t first = int64_t(blockIdx.x) * NT + tid;
  const bf16 z = bf16(0.f);
  for (int64_t i = first; i < (N - cu_last) * H * DK; i += stride) {
    dq[cu_last * H * DK + i] = z;
    dk[cu_last * H * DK + i] = z;
    dg[cu_last * H * DK + i] = z;
  }
  for (int64_t i = first; i < (N - cu_last) * H * DV; i += stride) dv[cu_last * H * DV + i] = z;
  for (int64_t i = first; i < (N - cu_last) * H; i += stride) dbeta[cu_last * H + i] = z;
}

// Workspace layout of one call (host side).
struct BwdLayout {
  int64_t max_chunks, max_sums, max_pieces;
  size_t plan_bytes, state_bytes, sumL_bytes, sumD_bytes, gfin_bytes, bytes;
};
// Plan words: base, pbase, sbase ([max_segs + 1] each), the queue counter, then
// irec[max_pieces][kRecWords] (the record of each ranked piece).
// own_states: the states live in the workspace (not given by the caller).
BwdLayout bwd_layout(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t max_segs, bool own_states = true) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdLayout l;
  l.max_chunks = (N + kC - 1) / kC + max_segs;
  // pieces of cut segments: m <= ceil(n / kPieceLen) < n / 16 per cut segment (n > kCutMin)
  l.max_sums = l.max_chunks / 16 + 1;
  l.max_pieces = max_segs + l.max_sums;
  l.plan_bytes = up(((size_t(max_segs) + 1) * 3 + 1 + kRecWords * size_t(l.max_pieces)) * 4);
  l.state_bytes = own_states ? up(size_t(l.max_chunks) * H * Dk * Dv * 2) : 0;
  l.sumL_bytes = up(size_t(l.max_sums) * 2 * H * Dk * Dv * 4);
  l.sumD_bytes = up(size_t(l.max_sums) * 2 * H * Dk * 4);
  l.gfin_bytes = up(size_t(max_segs) * H * Dk * 4);
  l.bytes = l.plan_bytes + l.state_bytes + l.sumL_bytes + l.sumD_bytes + l.gfin_bytes;
  return l;
}

template <int DK, int DV>
hipError_t launch_dims(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const void* dout, const int32_t* cu, int32_t max_segs, int64_t N, int32_t H,
                       float scale, const float* s0, const float* dF, void* dq, void* dk, void* dv,
                       void* dg, void* db, float* dinit, int32_t* flags, void* ws,
                       hipStream_t stream, const void* states_in) {
  using SC = StCfg<DK, DV>;
  using CC = ChCfg<DK, DV>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_bwd_state_kernel<DK, DV, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SC::bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_bwd_state_kernel<DK, DV, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, SC::bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_bwd_chunk_kernel<DK, DV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, CC::bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const BwdLayout l = bwd_layout(N, H, DK, DV, max_segs, states_in == nullptr);
  const int32_t from_saved = states_in != nullptr;
  char* w = static_cast<char*>(ws);
  int32_t* base = reinterpret_cast<int32_t*>(w);
  int32_t* pbase = base + (max_segs + 1);
  int32_t* sbase = pbase + (max_segs + 1);
  int32_t* counter = sbase + (max_segs + 1);
  int32_t* irec = counter + 1;
  // the bf16 state before every chunk: the caller's (saved by the forward call,
  // only read here) or the walk's, in the workspace
  bf16* Sws = from_saved ? const_cast<bf16*>(static_cast<const bf16*>(states_in))
                         : reinterpret_cast<bf16*>(w + l.plan_bytes);
  float* sumL = reinterpret_cast<float*>(w + l.plan_bytes + l.state_bytes);
  float* sumD = reinterpret_cast<float*>(w + l.plan_bytes + l.state_bytes + l.sumL_bytes);
  // per (segment, head, key channel): sum_e dL/dS_final * S_final (written only
  // when dL/dfinal_state is given)
  float* gfin = reinterpret_cast<float*>(w + l.plan_bytes + l.state_bytes + l.sumL_bytes + l.sumD_bytes);
  const bf16* qb = static_cast<const bf16*>(q);
  const bf16* kb = static_cast<const bf16*>(k);
  const bf16* vb = static_cast<const bf16*>(v);
  const bf16* gb = static_cast<const bf16*>(g);
  const bf16* bb = static_cast<const bf16*>(beta);
  const bf16* ob = static_cast<const bf16*>(dout);
  hipLaunchKernelGGL(kda_bwd_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu, max_segs, N, H,
                     int32_t(l.max_chunks), int32_t(l.max_pieces), int32_t(l.max_sums), base, pbase,
                     sbase, irec, counter, flags);
  // summaries of the pieces of cut segments, both roles
  hipLaunchKernelGGL((kda_bwd_state_kernel<DK, DV, true>), dim3(unsigned(2 * l.max_sums * H)),
                     dim3(SC::NT), SC::bytes, stream, qb, kb, vb, gb, bb, ob, cu, base, pbase, sbase,
                     irec, max_segs, int32_t(l.max_sums), N, H, scale, s0, dF, Sws, sumL, sumD, gfin,
                     from_saved);
  // the walk, S role only: the state before every chunk (with saved states, only
  // the final-state term of the gate gradient, when dL/dfinal_state is given)
  if (!from_saved || dF != nullptr)
    hipLaunchKernelGGL((kda_bwd_state_kernel<DK, DV, false>), dim3(unsigned(l.max_pieces * H)),
                       dim3(SC::NT), SC::bytes, stream, qb, kb, vb, gb, bb, ob, cu, base, pbase, sbase,
                       irec, max_segs, int32_t(l.max_pieces), N, H, scale, s0, dF, Sws, sumL, sumD, gfin,
                       from_saved);
  // the chunks of each (piece, head) walked backwards, Lambda carried
  hipLaunchKernelGGL((kda_bwd_chunk_kernel<DK, DV>), dim3(unsigned(device_cus() * CC::WG_PER_CU)), dim3(CC::NT),
                     CC::bytes, stream, qb, kb, vb, gb, bb, ob, cu, base, pbase, sbase, irec, counter,
                     max_segs, N, H, scale, dF, sumL, sumD, dF ? gfin : nullptr, Sws, static_cast<bf16*>(dq),
                     static_cast<bf16*>(dk), static_cast<bf16*>(dv), static_cast<bf16*>(dg),
                     static_cast<bf16*>(db), dinit, flags, int32_t(s0 != nullptr));
  return hipGetLastError();
}

}  // namespace

bool kda_chunk_bwd_supported(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                             int32_t max_segs) {
  if (dtype != 0 || !(Dk == 64 || Dk == 128) || !(Dv == 64 || Dv == 128)) return false;
  if (N < 1 || H < 1 || max_segs < 1) return false;
  const int64_t max_chunks = (N + kC - 1) / kC + max_segs;
  const int64_t max_pieces = max_segs + max_chunks / 16 + 1;
  return max_pieces * H < (int64_t(1) << 31) && max_chunks * H < (int64_t(1) << 31);
}

size_t kda_chunk_bwd_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                                     int32_t max_segs, bool states_given) {
  if (!kda_chunk_bwd_supported(N, H, Dk, Dv, dtype, max_segs)) return 0;
  return bwd_layout(N, H, Dk, Dv, max_segs, !states_given).bytes;
}

size_t kda_chunk_states_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                              int32_t max_segs) {
  if (!kda_chunk_bwd_supported(N, H, Dk, Dv, dtype, max_segs)) return 0;
  return size_t((N + kC - 1) / kC + max_segs) * H * Dk * Dv * 2;
}

hipError_t launch_kda_chunk_backward(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta, const void* dout, const int32_t* cu,
                                     int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                     float scale, const float* initial_state,
                                     const float* dfinal_state, void* dq, void* dk, void* dv,
                                     void* dg, void* dbeta, float* dinitial_state, int32_t* flags,
                                     void* workspace, hipStream_t stream, const void* chunk_states) {
#define PKV_BWD_LAUNCH(DK_, DV_)                                                                  \
  if (Dk == DK_ && Dv == DV_)                                                                     \
    return launch_dims<DK_, DV_>(q, k, v, g, beta, dout, cu, max_segs, N, H, scale, initial_state, \
                                 dfinal_state, dq, dk, dv, dg, dbeta, dinitial_state, flags,       \
                                 workspace, stream, chunk_states);
  PKV_BWD_LAUNCH(64, 64)
  PKV_BWD_LAUNCH(64, 128)
  PKV_BWD_LAUNCH(128, 64)
  PKV_BWD_LAUNCH(128, 128)
#undef PKV_BWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace pkv
