// Chunked packed KDA forward on CDNA4 matrix cores (bf16 tensors, Dk, Dv in {64, 128}).
//
// Computes what RFC-0026 "Ling3 KDA varlen support" defines in its Background
// section (KDA state leakage problem) with the reset of section 3.1.1:
//   S_t = diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,  o_t = scale * S_t^T q_t,
// S = 0 at every segment start; segments come from cu_seqlens (RFC-0025
// Design sections 1 and 2). The page's own kernels (a TPU Pallas chunk_kda
// with _align_seqs, chunk_local_cumsum_vector and kda_fwd_intra stages) are
// prior art; this kernel keeps the chunked idea but aligns chunks to segment
// starts by index arithmetic, so no chunk straddles a document and no padded
// copy of the sequence is ever built.
//
// Math per 64-token chunk (b_r = in-chunk inclusive cumsum of g, base 2):
//   o_r    = S_prev^T (q_r 2^{b_r})  +  sum_{s<=r} A[r,s] v_s
//   A[r,s] = beta_s sum_d q_r[d] k_s[d] 2^{b_r[d] - b_s[d]}
//   S_new  = diag(2^{b_C}) S_prev + sum_s (beta_s k_s 2^{b_C - b_s}) v_s^T
// Stable exponents: the chunk is cut into four 16-token sub-chunks; rho_j is
// the cumsum before sub-chunk j and T_j its total. Block (w, j) of A (rows in
// sub-chunk w, columns in sub-chunk j <= w) splits 2^{b_r - b_s} at
// rho_{j+1}: key factor KE_s = k_s 2^{rho_{j+1} - b_s} (<= 1), query factor
// q_r 2^{b_r - rho_{j+1}} (<= 1 off the diagonal, <= 2^{16 max|g| log2 e} on
// it); off the diagonal the query factor is Q~_r = q_r 2^{b_r - rho_w} times
// 2^{rho_w - rho_{j+1}} (<= 1), which goes on either operand. Per element only
// 2^{c} and 2^{T - c} are evaluated (c = in-sub-chunk cumsum); every other
// factor is per channel.
//
// A work-group runs one (run, head) item at a time: 4 producer waves and 4
// consumer waves, software-pipelined over chunks (two barriers per chunk step):
//   first half  P: chunk c: per-channel factors from the sub-chunk totals,
//                  Q^ = q 2^b, Kbar^T = (beta k 2^{b_C - b})^T and 2^{b_C}
//                  (the last two to the LDS buffers of c's parity), the
//                  operand versions of the ten A blocks and KE.
//               C: chunk c-1: o^T += V^T A^T for its Dv/4 columns, packed;
//                  S = diag(2^{b_C}) S + Kbar^T V.
//   second half P: V of chunk c; the gate products of chunk c+1, its
//                  sub-chunk totals 2^T (to LDS) and the per-element factors
//                  q 2^{c} and k 2^{T - c} of chunk c+1 (in the registers of
//                  its q and k).
//               C: the stores of chunk c-1's outputs; three of the twelve A
//                  block jobs of chunk c (MFMA), masked, beta-scaled, to LDS;
//                  o^T = S^T Q^^T.
// Producer wave w owns 16-token sub-chunk w and all Dk channels; lane
// 16 tq + cg holds the 4 consecutive tokens 4 tq .. 4 tq + 3 x Dk/16 channels
// of group cg, so each 16-lane row of a load or an LDS store covers one whole
// token row (conflict-free LDS writes) and the in-sub-chunk products are an
// in-lane prefix / suffix plus a step across the four rows (v_permlane16_swap
// and v_permlane32_swap). The sub-chunk totals go through a small LDS table,
// and the sub-chunk index is uniform per wave (no divergent stores).
// Raw inputs of chunk c+1 are loaded at the start of step c. Every
// single-buffered LDS tile (Q^, KE, the A-block versions, V, A, the totals)
// is written in one half and read in the other; Kbar^T, 2^{b_C} and beta,
// which the consumers read in the next step's first half, are double-buffered
// by chunk parity.
// MFMA v_mfma_f32_16x16x32_bf16: A operand lane l holds row l%16 and eight
// contraction slots of lane group l/16, B likewise for column l%16; the 16x16
// fp32 result has column l%16 and rows 4(l/16)+i. The contraction index may be
// permuted freely when A and B agree, so S^T is fed straight from the S
// accumulators (slots {4g..4g+3} of two adjacent 16-row tiles) and Q^ is read
// with the same permutation.

#include "common.h"

#include <mutex>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// Work plan (built on the device by kda_plan_kernel; see there). How a
// segment is cut depends on its own chunk count and these constants only, so
// a segment's results never depend on the other segments of the launch.
constexpr int kPlanThreads = 1024;  // plan work-group for calls of more than kPlanSmall slots
constexpr int kPlanSmall = 256;     // and for calls of at most this many slots (fewer waves to synchronise)
constexpr int kHistBins = 2048;   // run-length bins of the longest-first order
constexpr int kCutMin = 128;      // chunks: segments of at most this many are never cut
constexpr int kRunLen = 64;       // chunks: target length of the runs of a cut segment
constexpr int kMaxRuns = 16;      // runs per segment
constexpr int kPlanHeader = 64;   // int32 words before the run table
constexpr int kGroupN = 4;        // chunks: segments of at most this many may share an item
constexpr int kGroupWin = 12;     // chunks: window of the global chunk order a group's segments start in
constexpr int kGroupMax = kGroupWin + kGroupN - 1;  // chunks of a group, at most
static_assert(kGroupMax <= 64, "a group's chunk table is one word per lane");
constexpr int kPlanCache = 8192;  // segment slots whose chunk counts the plan keeps in LDS

// A blocks (row sub-chunk w, column sub-chunk j), j <= w, in this order (the
// jobs of the consumer waves). Jobs 10 and 11 zero the blocks (0, 1) and
// (2, 3), which the A.V product reads through its 32-wide steps.
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
  static constexpr int NP = 4;              // producer waves: one per 16-token sub-chunk
  static constexpr int NT = 64 * (NP + 4);  // threads: producers + 4 consumers
  static constexpr int PCPL = DK / 16;      // producer k channels per lane (4 tokens each)
  static constexpr int PVPL = DV / 16;      // producer v channels per lane
  static constexpr int EW = DV / 4;         // consumer state / output columns
  static constexpr int ET = EW / 16;        // 16-column tiles per consumer
  static constexpr int DT = DK / 16;        // 16-row state tiles
  static constexpr int KS = DK / 32;        // contraction steps over Dk
  static constexpr int KP = DK + 8;         // Q^, KE, query versions: token-major rows (bf16)
  // Dk = Dv = 64: two work-groups per CU (LDS at most 80 KiB and at most 128
  // VGPRs each, four waves per SIMD); every other shape: one.
  static constexpr int WG_PER_CU = (DK == 64 && DV == 64) ? 2 : 1;
  static constexpr int RP = DK + (WG_PER_CU == 2 ? 8 : 16);  // Kbar: token-major rows, read transposed
  static constexpr int VP = DV + (WG_PER_CU == 2 ? 8 : 16);  // V: token-major rows, read transposed
  static constexpr int TP = kC + 8;         // A rows (bf16)
  // Small tables first: ds_read/ds_write immediates reach 64 KiB.
  static constexpr int off_item = 0;                         // int: next queue item
  static constexpr int off_decay = 16;                       // float [2][DK]
  static constexpr int off_beta = off_decay + 2 * DK * 4;    // float [2][kC]
  // 2^{sub-chunk totals}: float [4] per channel, one empty slot after every
  // group of DK/16 channels, so the 16 channel groups of a read fall on
  // distinct banks
  static constexpr int off_T = off_beta + 2 * kC * 4;
  static constexpr int off_a = off_T + (DK + 16) * 4 * 4;    // A, bf16 [kC][TP]
  static constexpr int off_v = off_a + kC * TP * 2;          // V, bf16 [kC][VP]
  static constexpr int off_kb = off_v + kC * VP * 2;         // Kbar, bf16 [2][kC][RP]
  static constexpr int off_qh = off_kb + 2 * kC * RP * 2;    // Q^, bf16 [kC][KP]
  static constexpr int off_ke = off_qh + kC * KP * 2;        // KE, bf16 [kC][KP]
  static constexpr int off_qv = off_ke + kC * KP * 2;        // A-block operand versions, bf16 [10][16][KP]
  // Dv = 128: outputs staged through LDS, bf16 [kC][DV], 16-byte chunk c of
  // row r at chunk c ^ (r % 16) (conflict-free both ways, no padding room)
  static constexpr bool stage_o = DV == 128;
  static constexpr int off_o = off_qv + 10 * 16 * KP * 2;
  static constexpr int bytes = off_o + (stage_o ? kC * DV * 2 : 0);
  static_assert(bytes <= 160 * 1024 / WG_PER_CU, "LDS budget");
};

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int n>
struct alignas(2 * n) BfPack {
  bf16 v[n];
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// The value of another lane of the same 16-lane row (DPP control kCtrl).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}
// A register of another lane of the same quad (DPP quad_perm kCtrl; every lane active).
template <int kCtrl>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), kCtrl, 0xF, 0xF, true));
}
// Sum over the 16 lanes of a row, the same bits in every lane (each step adds
// two equal partial sums in either order): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror (lane j of an 8-lane half takes lane 7 - j),
// row_mirror (lane j of the row takes lane 15 - j).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
// Added to a squared norm before the reciprocal square root (the q/k L2
// normalisation option), so a zero row stays finite.
constexpr float kL2NormEps = 1e-6f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufFlags);
}

// n bf16 values from a raw buffer (n in {4, 8}); out-of-range reads give 0.
template <int n>
__device__ __forceinline__ BfPack<n> bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  BfPack<n> p;
  if constexpr (n == 4) {
    typedef int v2 __attribute__((ext_vector_type(2)));
    const v2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    __builtin_memcpy(&p, &x, 8);
  } else {
    static_assert(n == 8, "load width");
    typedef int v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    __builtin_memcpy(&p, &x, 16);
  }
  return p;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(0): every vector memory operation of the wave has completed
// (gfx9 encoding: vmcnt 0, expcnt 7 and lgkmcnt 15, i.e. no wait on those).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Two floats -> one register of two bf16 (round to nearest even), a single
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Four floats -> four bf16 at an 8-byte aligned address.
__device__ __forceinline__ void st4(bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(dst) = u32x2{pk2(a, b), pk2(c, d)};
}
__device__ __forceinline__ void st4(bf16* dst, const float* x) { st4(dst, x[0], x[1], x[2], x[3]); }
// n floats (n in {4, 8}) -> n bf16 at an 8n/4-byte aligned address, one store.
template <int n>
__device__ __forceinline__ void stn(bf16* dst, const float* x) {
  if constexpr (n == 4) {
    st4(dst, x);
  } else {
    static_assert(n == 8, "store width");
    *reinterpret_cast<u32x4*>(dst) =
        u32x4{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7])};
  }
}

// n bf16 that are already packed in pairs (n in {4, 8}) -> one store.
template <int n>
__device__ __forceinline__ void stw(bf16* dst, const uint32_t (&w)[n / 2]) {
  if constexpr (n == 4) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
  } else {
    static_assert(n == 8, "store width");
    *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane k supplies the address of 4 consecutive bf16; lane j = 4a + b receives
// element b of the chunks supplied by lanes a, 4 + a, 8 + a, 12 + a, in that
// order. So if lane k points at row (token) r0 + k/4, column c0 + 4 (k % 4) of
// a token-major tile, lane j gets column c0 + j of rows r0 .. r0 + 3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Raw producer inputs of one chunk: 4 tokens x PCPL channels of q, k, g and
// PVPL channels of v as packed bf16 pairs. They stay packed until used, so a
// load is never waited for before its first use.
template <int PCPL, int PVPL>
struct Raw {
  uint32_t g[4][PCPL / 2];
  uint32_t v[4][PVPL / 2];
};
// q and k of one chunk (two sets alternate, so they are loaded a whole chunk
// step before use).
template <int PCPL>
struct RawQK {
  uint32_t q[4][PCPL / 2], k[4][PCPL / 2];
};

// bf16 element c of a packed pair array, as fp32 (exact).
template <int n>
__device__ __forceinline__ float bf(const uint32_t (&w)[n], int c) {
  const uint32_t x = w[c >> 1];
  return __uint_as_float((c & 1) ? (x & 0xFFFF0000u) : (x << 16));
}

// 2n packed bf16 values (n in {2, 4}) from a raw buffer; out-of-range reads give 0.
template <int n>
__device__ __forceinline__ void wload(uint32_t (&w)[n], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (n == 1) {
    w[0] = uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  } else if constexpr (n == 2) {
    typedef int v2 __attribute__((ext_vector_type(2)));
    const v2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = uint32_t(x[0]);
    w[1] = uint32_t(x[1]);
  } else {
    static_assert(n == 4, "load width");  // n in {1, 2, 4}
    typedef int v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(x[i]);
  }
}

// kState = false: the forward pass of one run (a whole segment, or a piece of
// a long one that starts from the state composed of the earlier pieces'
// results). kState = true: the state pass of a run that is not its segment's
// last: S from zero over the run and the product of its decays, both to the
// workspace (no outputs).
// kNorm: q and k are first L2-normalised per (token, head) over Dk.
// kSave: the forward pass also writes the state before every chunk to chunk_states.
template <int DK, int DV, bool kState, bool kNorm, bool kSave>
__global__ __launch_bounds__(512, (DK == 64 && DV == 64) ? 4 : 1) void kda_chunk_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const int32_t* __restrict__ cu,
    int32_t* __restrict__ plan, int32_t runs_max, int32_t max_segs, int64_t N,
    int32_t H, float scale, const float* __restrict__ initial_state, bf16* __restrict__ o,
    float* __restrict__ final_state, float* __restrict__ run_states,
    float* __restrict__ run_decays, int64_t row_len, const int32_t* __restrict__ seg_ids,
    const int32_t* __restrict__ n_dev, int32_t* __restrict__ flags, bf16* __restrict__ chunk_states,
    int32_t lds_zero) {
  using C = Cfg<DK, DV>;
  constexpr int NP = C::NP, NT = C::NT;
  constexpr int PCPL = C::PCPL, PVPL = C::PVPL, ET = C::ET, DT = C::DT, KS = C::KS;
  constexpr int KP = C::KP, TP = C::TP, RP = C::RP, VP = C::VP;

  // Tile bases are made opaque to the compiler (lds_zero is 0 at run time):
  // an LDS access then takes one base register per tile and lane pattern plus
  // a 16-bit immediate, instead of folding tile offsets beyond 64 KiB into
  // per-access address registers.
  extern __shared__ __attribute__((aligned(16))) char smem[];
  auto tile = [&](int off) { return smem + (off | lds_zero); };
  bf16* s_qh = reinterpret_cast<bf16*>(tile(C::off_qh));
  bf16* s_qv = reinterpret_cast<bf16*>(tile(C::off_qv));
  bf16* s_ke = reinterpret_cast<bf16*>(tile(C::off_ke));
  bf16* s_kb0 = reinterpret_cast<bf16*>(tile(C::off_kb));   // Kbar of even / odd chunks
  bf16* s_kb1 = reinterpret_cast<bf16*>(tile(C::off_kb + kC * RP * 2));
  bf16* s_v = reinterpret_cast<bf16*>(tile(C::off_v));
  bf16* s_a = reinterpret_cast<bf16*>(tile(C::off_a));
  float* s_decay = reinterpret_cast<float*>(tile(C::off_decay));
  float* s_beta = reinterpret_cast<float*>(tile(C::off_beta));
  float* s_T = reinterpret_cast<float*>(tile(C::off_T));
  char* s_o = tile(C::off_o);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = w < NP;

  // Persistent work-groups: each takes (run, head) items from the plan's
  // queue, a counter the plan kernel resets, in the plan's order (longest
  // run first, heads of a run together; item = rank * H + h). A work-group
  // claims its next item one step before the current one ends: the queue is
  // then served in the order work-groups free up, which is what makes the
  // longest-first order balance the load (a claim at the item's start pairs
  // each item with the one claimed after it), and the claim's latency still
  // hides behind the last step.
  int* s_item = reinterpret_cast<int*>(tile(C::off_item));
  int32_t* const counter = plan + (kState ? 3 : 2);
  const int n_items = (kState ? plan[1] : plan[0]) * H;
  // Producers and consumers each loop over the same item sequence (with the
  // same barriers), so neither role's loop keeps the other's registers live.
  // The current item's run, set by begin_item in both loops:
  int h = 0, slot = 0, run_idx = 0, sbase = 0, nchunks = 0;
  int gc0 = 0;  // global index of the run's first chunk (chunks of all slots in slot order)
  bool last = false;
  int64_t start = 0, end = 0;
  // A group of short segments (whole, in consecutive slots) is one item: its
  // chunks follow each other in token order. Lane c of ctab corrects chunk c's
  // place: chunk c starts 64 c - (ctab >> 8) tokens after start, is at most
  // 64 - (ctab & 127) tokens long, and starts a segment of the group when bit 7
  // is set. The table is zero for an ordinary item (and past chunk 63), so
  // the addressing has no branch.
  uint32_t ctab = 0;
  auto begin_item = [&](int item) __attribute__((always_inline)) {
    const int rank = item / H;
    h = item % H;
    int c0, c1;
    if constexpr (kState) {
      const int32_t* e = plan + kPlanHeader + 8 * runs_max + 4 * rank;
      slot = e[0];
      c0 = e[1];
      c1 = e[2];
      sbase = e[3];  // the state slot this run writes
    } else {
      const int32_t* e = plan + kPlanHeader + 8 * rank;
      slot = e[0];
      c0 = e[1];
      c1 = e[2];
      run_idx = e[3];  // runs of the segment before this one
      sbase = e[4];    // their state slots: sbase .. sbase + run_idx - 1
      last = e[5] != 0;
      gc0 = e[6] + c0;
      const int ns = e[7];  // > 0: slots slot .. slot + ns - 1 form a group
      ctab = 0;
      if (ns > 0) {
        start = cu[slot];
        end = cu[slot + ns];
        nchunks = c1;
        int64_t a0 = start;
        int c = 0;
        for (int j = 1; j <= ns; ++j) {
          const int64_t a1 = cu[slot + j];
          for (int64_t p = a0; p < a1; p += kC, ++c) {
            const uint32_t L = uint32_t(a1 - p < kC ? a1 - p : kC);
            if (lane == c)
              ctab = (uint32_t(int64_t(c) * kC - (p - start)) << 8) | (p == a0 && c > 0 ? 128u : 0u) |
                     (uint32_t(kC) - L);
          }
          a0 = a1;
        }
        return;
      }
    }
    // the run: chunks [c0, c1) of the segment, which are aligned to its start
    // (the plan holds well-formed, non-empty segments only)
    int64_t seg_start = 0, seg_end = N;
    if (cu != nullptr) {
      seg_start = cu[slot];
      seg_end = cu[slot + 1];
    }
    start = seg_start + int64_t(c0) * kC;
    const int64_t run_end = seg_start + int64_t(c1) * kC;
    end = seg_end < run_end ? seg_end : run_end;
    if (end < start) end = start;
    nchunks = int((end - start + kC - 1) / kC);
  };
  // A state pass with nothing to do ends before touching the queue (its
  // work-groups would otherwise line up on the counter's atomic).
  if constexpr (kState)
    if (n_items == 0) return;
  if (tid == 0) *s_item = atomicAdd(counter, 1);
  __syncthreads();
  const int first_item = __builtin_amdgcn_readfirstlane(*s_item);
  const uint32_t rowK = uint32_t(H) * DK * 2;  // bytes between tokens (q, k, g)
  const uint32_t rowV = uint32_t(H) * DV * 2;
  const uint32_t rowB = uint32_t(H) * 2;
  // chunk c's first token and length (segments, and so items, are below 2^31 tokens)
  struct CPos {
    int64_t p0;
    int len;
  };
  auto chunk_pos = [&](int c) __attribute__((always_inline)) {
    const uint32_t w = uint32_t(__builtin_amdgcn_readlane(int(ctab), c & 63));
    CPos r;
    r.p0 = start + int64_t(c) * kC - int64_t(w >> 8);
    const int rem = int(end - r.p0), cap = kC - int(w & 127u);
    r.len = rem < cap ? rem : cap;
    return r;
  };

  // ---------------------------------------------------------------- roles
  // Producer wave w: sub-chunk sw = w, all channels. Lane 16 tq + cg: 4
  // tokens [tok0, tok0 + 4), PCPL k channels from ch0 and PVPL v channels from
  // vch0, so each 16-lane row of a load or a store covers one token's row.
  const int sw = w & 3;
  const int tq = lane >> 4;
  const int cg = lane & 15;
  const int ch0 = PCPL * cg;
  const int vch0 = PVPL * cg;
  const int tok0 = 16 * sw + 4 * tq;
  // MFMA lane layout (consumers, and every wave for the A blocks).
  const int gq = lane >> 4;
  const int lr = lane & 15;
  const int ci = w - NP;               // consumer index 0..3
  const int e0 = ci * C::EW;
  // Row rho of 16-column tile et of a consumer's state / output holds channel
  // e0 + ecol(et, rho); the map puts each lane's 4 x ET output values of a
  // token next to each other (one vector store per token tile). The labels
  // are only a permutation of the consumer's columns: S, V^T and o use the
  // same one.
  auto ecol = [&](int et, int rho) { return 4 * ET * (rho >> 2) + 4 * et + (rho & 3); };

  // Loads are unconditional so the wait counts stay exact: a chunk index past
  // the segment gets an empty buffer (every read returns 0, no memory access).
  // Raw inputs are loaded ahead of their use: q, k of chunk c+1 at the start
  // of step c (two register sets alternate; the scan of chunk c+1 in the
  // second half of step c folds the gates into them), v of chunk c+1 right
  // after V of chunk c went to LDS, g of chunk c+2 after the scan of chunk c+1.
  // beta goes through LDS (double-buffered by chunk parity): wave 0 loads it a
  // step ahead.
  struct Src {
    int64_t tokbase;
    uint32_t nK, nV, nB;
  };
  auto src_of = [&](int c) __attribute__((always_inline)) {
    const bool live = c < nchunks;
    const CPos cp = chunk_pos(live ? c : 0);
    const int64_t p0 = cp.p0;
    const int Lc = live ? cp.len : 1;
    Src r;
    r.tokbase = p0 * H + h;
    r.nK = live ? uint32_t(Lc - 1) * rowK + DK * 2 : 0u;
    r.nV = live ? uint32_t(Lc - 1) * rowV + DV * 2 : 0u;
    r.nB = live ? uint32_t(Lc - 1) * rowB + 2 : 0u;
    return r;
  };
  auto load_g = [&](Raw<PCPL, PVPL>& R, int c) __attribute__((always_inline)) {
    const Src r = src_of(c);
    const auto rg = rsrc(g + r.tokbase * DK, r.nK);
#pragma unroll
    for (int i = 0; i < 4; ++i) wload(R.g[i], rg, uint32_t(tok0 + i) * rowK + ch0 * 2);
  };
  auto load_qk = [&](RawQK<PCPL>& R, int c) __attribute__((always_inline)) {
    const Src r = src_of(c);
    const auto rq = rsrc(q + r.tokbase * DK, r.nK), rk = rsrc(k + r.tokbase * DK, r.nK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = uint32_t(tok0 + i);
      if constexpr (!kState) wload(R.q[i], rq, t * rowK + ch0 * 2);
      wload(R.k[i], rk, t * rowK + ch0 * 2);
    }
  };
  // beta of a whole chunk, token = lane (one wave loads it for everyone)
  auto load_beta = [&](int c) __attribute__((always_inline)) {
    const Src r = src_of(c);
    return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rsrc(beta + r.tokbase, r.nB),
                                                         uint32_t(lane) * rowB, 0, 0));
  };
  auto load_v = [&](Raw<PCPL, PVPL>& R, int c) __attribute__((always_inline)) {
    const Src r = src_of(c);
    const auto rv = rsrc(v + r.tokbase * DV, r.nV);
#pragma unroll
    for (int i = 0; i < 4; ++i) wload(R.v[i], rv, uint32_t(tok0 + i) * rowV + vch0 * 2);
  };
  // ---- producer, second half: in-sub-chunk cumulative gates (base 2) of a
  // chunk, folded into its q and k at once. With c the inclusive cumsum at a
  // token from the start of its sub-chunk and T the sub-chunk total, the
  // registers of q and k are overwritten in place by Q~ = q 2^{c} and
  // KE = k 2^{T - c} (bf16, packed like the raw values), so only they, not
  // the cumsums, stay live until the first half; s_T gets 2^T of every
  // sub-chunk (the next half's factors are products of those). The state
  // pass has no q and folds k only.
  // smallest 2^T the producer's scans met (the gate-range check)
  float tmin = 1.f;
  auto scan = [&](const Raw<PCPL, PVPL>& R, RawQK<PCPL>& X) __attribute__((always_inline)) {
    // One exponential per gate element, 2^{g log2 e}; the factors are its
    // products: 2^{c} over the tokens up to and including this one, 2^{T - c}
    // over the tokens after it, 2^T over the sub-chunk. In-lane over the
    // lane's 4 tokens, then across the four token groups (the four rows of 16
    // lanes): row pairs through v_permlane16_swap, pair products through
    // v_permlane32_swap.
    float fq[4][PCPL], fk[4][PCPL], tot[PCPL];
#pragma unroll
    for (int c = 0; c < PCPL; ++c) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = ex2(bf(R.g[i], c) * kLog2e);
      const float p1 = e[0] * e[1], p2 = p1 * e[2], row = p2 * e[3];  // in-lane prefix products
      const float s1 = e[2] * e[3], s0 = e[1] * s1;                  // in-lane suffix products
      const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(row), __float_as_uint(row), false, false);
      const float even = __uint_as_float(pr[0]), odd = __uint_as_float(pr[1]);  // rows 2m, 2m + 1
      const float pair = even * odd;
      const auto pt = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
      const float lo = __uint_as_float(pt[0]), hi = __uint_as_float(pt[1]);  // rows 0-1, rows 2-3
      // products over the rows before / after this lane's row
      const float before = ((tq & 1) ? even : 1.f) * (tq >= 2 ? lo : 1.f);
      const float after = ((tq & 1) ? 1.f : odd) * (tq < 2 ? hi : 1.f);
      fq[0][c] = before * e[0];
      fq[1][c] = before * p1;
      fq[2][c] = before * p2;
      fq[3][c] = before * row;
      fk[0][c] = after * s0;
      fk[1][c] = after * s1;
      fk[2][c] = after * e[3];
      fk[3][c] = after;
      tot[c] = lo * hi;  // 2^T, the same bits in every lane
    }
    if (tq == 3) {
#pragma unroll
      for (int c = 0; c < PCPL; ++c) {
        s_T[(ch0 + c + cg) * 4 + sw] = tot[c];  // + cg: the table's padding
        tmin = fminf(tmin, tot[c]);
      }
    }
    // kNorm: 1 / sqrt(|x|^2 + eps) of each token's q and k; the 16 lanes of a
    // row hold the token's Dk channels, PCPL each (formed after the gate
    // products, whose temporaries are dead by then)
    float rq[4], rk[4];
    if constexpr (kNorm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < PCPL; ++c) {
          if constexpr (!kState) sq = fmaf(bf(X.q[i], c), bf(X.q[i], c), sq);
          sk = fmaf(bf(X.k[i], c), bf(X.k[i], c), sk);
        }
        if constexpr (!kState) rq[i] = __builtin_amdgcn_rsqf(row_sum16(sq) + kL2NormEps);
        rk[i] = __builtin_amdgcn_rsqf(row_sum16(sk) + kL2NormEps);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int c = 0; c < PCPL; c += 2) {
        if constexpr (kNorm) {
          if constexpr (!kState)
            X.q[i][c >> 1] = pk2((bf(X.q[i], c) * rq[i]) * fq[i][c], (bf(X.q[i], c + 1) * rq[i]) * fq[i][c + 1]);
          X.k[i][c >> 1] = pk2((bf(X.k[i], c) * rk[i]) * fk[i][c], (bf(X.k[i], c + 1) * rk[i]) * fk[i][c + 1]);
        } else {
          if constexpr (!kState) X.q[i][c >> 1] = pk2(bf(X.q[i], c) * fq[i][c], bf(X.q[i], c + 1) * fq[i][c + 1]);
          X.k[i][c >> 1] = pk2(bf(X.k[i], c) * fk[i][c], bf(X.k[i], c + 1) * fk[i][c + 1]);
        }
      }
    }
  };

  // ---- producer, first half: factors and MFMA operands of one chunk from
  // its Q~ and KE. With T_j the sub-chunk totals of a channel and
  // E_j = 2^{T_j} (from s_T): f0 = 2^{T_0 + .. + T_{w-1}} (Q^ = Q~ f0),
  // f1 = 2^{T_{w+1} + .. + T_3} (Kbar = beta KE f1), f2 = 2^{-T_w} (the
  // diagonal block's query version), decay = 2^{T_0 + .. + T_3}: products of
  // the E_j and one reciprocal. Block (w, j < w) of A needs the factor
  // 2^{T_{j+1} + .. + T_{w-1}} on one of its operands (none for j = w - 1);
  // it goes where the producers' work evens out: producer 0 stores KE 2^{T_1}
  // (block (2, 0)), producer 1 KE 2^{T_2} (block (3, 1)), producer 3 the
  // query version Q~ 2^{T_1 + T_2} (block (3, 0)), and every other
  // off-diagonal block pairs KE with Q~ itself. Version slots (16 rows each):
  // 0..3 the diagonal query versions of sub-chunks 0..3, 4..6 Q~ of
  // sub-chunks 1..3, 7 and 9 those two key versions, 8 that query version.
  // KE, Q~ and, for w = 0, Q^ are stored as they are. The
  // sub-chunk index is a compile-time constant inside (one instance per
  // sub-chunk), so every choice below is resolved without branches.
  auto produce_a_sw = [&](auto swc, const RawQK<PCPL>& R, bf16* s_qh, bf16* s_kb, float* s_dec,
                          const float* s_bet) __attribute__((always_inline)) {
    constexpr int sw = decltype(swc)::value;
    float f[3][PCPL], gk[2][PCPL], dec[PCPL];
#pragma unroll
    for (int c = 0; c < PCPL; ++c) {
      const f32x4 E = *reinterpret_cast<const f32x4*>(s_T + (ch0 + c + cg) * 4);
      f[0][c] = sw == 0 ? 1.f : sw == 1 ? E[0] : sw == 2 ? E[0] * E[1] : (E[0] * E[1]) * E[2];
      f[1][c] = sw == 3 ? 1.f : sw == 2 ? E[3] : sw == 1 ? E[2] * E[3] : E[1] * (E[2] * E[3]);
      f[2][c] = __builtin_amdgcn_rcpf(E[sw]);
      gk[0][c] = sw == 0 ? E[1] : E[2];
      gk[1][c] = E[1] * E[2];  // sub-chunk 3's query version of block (3, 0)
      dec[c] = (E[0] * E[1]) * (E[2] * E[3]);
    }
    if (sw == 0 && tq == 0) {
#pragma unroll
      for (int c = 0; c < PCPL; c += 4)
        *reinterpret_cast<f32x4*>(s_dec + ch0 + c) = f32x4{dec[c], dec[c + 1], dec[c + 2], dec[c + 3]};
    }
    const f32x4 bt4 = *reinterpret_cast<const f32x4*>(s_bet + tok0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + i;
      const float bt = bt4[i];
      float qt[PCPL], kt[PCPL], t0[PCPL], kb[PCPL];
#pragma unroll
      for (int c = 0; c < PCPL; ++c) {
        qt[c] = bf(R.q[i], c);
        kt[c] = bf(R.k[i], c);
        t0[c] = qt[c] * f[0][c];
        kb[c] = kt[c] * (bt * f[1][c]);
      }
      if constexpr (sw == 0)
        stw<PCPL>(s_qh + tok * KP + ch0, R.q[i]);
      else
        stn<PCPL>(s_qh + tok * KP + ch0, t0);
      stw<PCPL>(s_ke + tok * KP + ch0, R.k[i]);
      stn<PCPL>(s_kb + tok * RP + ch0, kb);
      bf16* qv = s_qv + (tok & 15) * KP + ch0;  // row of the token in each version slot
#pragma unroll
      for (int c = 0; c < PCPL; ++c) t0[c] = qt[c] * f[2][c];
      stn<PCPL>(qv + sw * 16 * KP, t0);
      if constexpr (sw >= 1) stw<PCPL>(qv + (3 + sw) * 16 * KP, R.q[i]);
      if constexpr (sw <= 1) {
#pragma unroll
        for (int c = 0; c < PCPL; ++c) t0[c] = kt[c] * gk[0][c];
        stn<PCPL>(qv + (sw == 0 ? 7 : 9) * 16 * KP, t0);
      }
      if constexpr (sw == 3) {
#pragma unroll
        for (int c = 0; c < PCPL; ++c) t0[c] = qt[c] * gk[1][c];
        stn<PCPL>(qv + 8 * 16 * KP, t0);
      }
    }
  };

  // State pass: only Kbar and the decay.
  auto produce_kb_sw = [&](auto swc, const RawQK<PCPL>& R, bf16* s_kb, float* s_dec,
                           const float* s_bet) __attribute__((always_inline)) {
    constexpr int sw = decltype(swc)::value;
    float f1[PCPL], dec[PCPL];
#pragma unroll
    for (int c = 0; c < PCPL; ++c) {
      const f32x4 E = *reinterpret_cast<const f32x4*>(s_T + (ch0 + c + cg) * 4);
      f1[c] = sw == 3 ? 1.f : sw == 2 ? E[3] : sw == 1 ? E[2] * E[3] : E[1] * (E[2] * E[3]);
      dec[c] = (E[0] * E[1]) * (E[2] * E[3]);
    }
    if (sw == 0 && tq == 0) {
#pragma unroll
      for (int c = 0; c < PCPL; c += 4)
        *reinterpret_cast<f32x4*>(s_dec + ch0 + c) = f32x4{dec[c], dec[c + 1], dec[c + 2], dec[c + 3]};
    }
    const f32x4 bt4 = *reinterpret_cast<const f32x4*>(s_bet + tok0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float kb[PCPL];
#pragma unroll
      for (int c = 0; c < PCPL; ++c) kb[c] = bf(R.k[i], c) * (bt4[i] * f1[c]);
      stn<PCPL>(s_kb + (tok0 + i) * RP + ch0, kb);
    }
  };

  auto produce_a = [&](const RawQK<PCPL>& R, bf16* s_qh, bf16* s_kb, float* s_dec,
                       const float* s_bet) __attribute__((always_inline)) {
    if constexpr (kState) {
      switch (sw) {
        case 0: produce_kb_sw(IntC<0>{}, R, s_kb, s_dec, s_bet); break;
        case 1: produce_kb_sw(IntC<1>{}, R, s_kb, s_dec, s_bet); break;
        case 2: produce_kb_sw(IntC<2>{}, R, s_kb, s_dec, s_bet); break;
        default: produce_kb_sw(IntC<3>{}, R, s_kb, s_dec, s_bet); break;
      }
      return;
    }
    switch (sw) {
      case 0: produce_a_sw(IntC<0>{}, R, s_qh, s_kb, s_dec, s_bet); break;
      case 1: produce_a_sw(IntC<1>{}, R, s_qh, s_kb, s_dec, s_bet); break;
      case 2: produce_a_sw(IntC<2>{}, R, s_qh, s_kb, s_dec, s_bet); break;
      default: produce_a_sw(IntC<3>{}, R, s_qh, s_kb, s_dec, s_bet); break;
    }
  };

  // ---- producer, second half: V of the chunk, token-major (the consumers
  // read it transposed).
  auto produce_b = [&](const uint32_t (&V)[4][PVPL / 2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16* dst = s_v + (tok0 + i) * VP + vch0;
      if constexpr (PVPL == 8)
        *reinterpret_cast<u32x4*>(dst) = u32x4{V[i][0], V[i][1], V[i][2], V[i][3]};
      else
        *reinterpret_cast<u32x2*>(dst) = u32x2{V[i][0], V[i][1]};
    }
  };

  // ---- consumer, second half of step c: o^T = S^T Q^^T for chunk c (S holds
  // the state after chunk c-1 by then); kept in registers until the first
  // half of step c+1 adds V^T A^T. Contraction over Dk in steps of 32.
  // The state before global chunk gc, bf16, row-major [Dk][Dv] at
  // chunk_states[gc][h]: the reverse pass's layout. Lane lr of a consumer holds
  // rows 16 dt + 4 gq .. + 3 of column e0 + ecol(et, lr); the four lanes of a
  // quad hold four consecutive columns, so a 4 x 4 transpose within the quad
  // gives each lane one row's four columns (one 8-byte store): swap the
  // off-diagonal 2 x 2 blocks with lane ^ 2 (quad_perm [2,3,0,1]), then the
  // halves of each block's rows with lane ^ 1 (quad_perm [1,0,3,2], v_perm_b32).
  auto zero_state = [&](f32x4 (&S)[DT][ET]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int et = 0; et < ET; ++et) S[dt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto save_state = [&](const f32x4 (&S)[DT][ET], int gc) __attribute__((always_inline)) {
    // one 32-bit base offset per lane plus an immediate per (dt, et)
    const auto rs = rsrc(chunk_states + (int64_t(gc) * H + h) * DK * DV, DK * DV * 2);
    const int q4 = lr & 3;
    const uint32_t lane_off = uint32_t((4 * gq + q4) * DV + e0 + 4 * ET * (lr >> 2)) * 2;
    const uint32_t sel = (q4 & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const f32x4 x = S[dt][et];
        uint32_t w0 = pk2(x[0], x[1]), w1 = pk2(x[2], x[3]);
        const uint32_t got = dppu<0x4E>((q4 & 2) ? w0 : w1);
        if (q4 & 2) w0 = got; else w1 = got;
        w0 = __builtin_amdgcn_perm(dppu<0xB1>(w0), w0, sel);
        w1 = __builtin_amdgcn_perm(dppu<0xB1>(w1), w1, sel);
        // row 16 dt + 4 gq + q4, columns e0 + 4 ET (lr / 4) + 4 et .. + 3
        typedef int v2i __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(v2i{int(w0), int(w1)}, rs, lane_off,
                                              (16 * dt * DV + 4 * et) * 2, 0);
      }
  };
  auto consume_inter = [&](const f32x4 (&S)[DT][ET], f32x4 (&acc)[4][ET]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[t][et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      bf16x8 bq[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16* row = s_qh + (16 * t + lr) * KP + 32 * u + 4 * gq;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16);
        bq[t] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const f32x4 x = S[2 * u][et], y = S[2 * u + 1][et];
        const bf16x8 sop = __builtin_bit_cast(
            bf16x8, u32x4{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(y[0], y[1]), pk2(y[2], y[3])});
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][et] = mfma(sop, bq[t], acc[t][et]);
      }
    }
  };

  // ---- consumer, first half of step c+1: o of chunk c = acc + V^T A^T
  // (contraction over tokens in steps of 32; causal: the second step only
  // for rows >= 32), scaled and stored; then S = diag(2^{b_C}) S + Kbar^T V.
  // Operands whose contraction runs over the tokens 32 m2 + 8 gq + 0..7 of
  // the chunk, read transposed from token-major tiles: lane lr gets column
  // c0(lr / 4 ...) as set by the supplying lanes (see tr4).
  const int trow = 8 * gq + (lr >> 2);  // token supplied by this lane, + 32 m2 (+ 4)
  auto vT_op = [&](int m2, int et) __attribute__((always_inline)) {    // V^T rows e0 + ecol(et, lr)
    const bf16* p = s_v + (32 * m2 + trow) * VP + e0 + 4 * ET * (lr & 3) + 4 * et;
    return join_tr(tr4(p), tr4(p + 4 * VP));
  };
  auto kbT_op = [&](const bf16* s_kb, int m2, int dt) __attribute__((always_inline)) {  // Kbar^T rows 16 dt + lr
    const bf16* p = s_kb + (32 * m2 + trow) * RP + 16 * dt + 4 * (lr & 3);
    return join_tr(tr4(p), tr4(p + 4 * RP));
  };
  // S = diag(2^{b_C}) S + Kbar^T V (the decay also multiplies into Dacc when
  // given: the state pass keeps the run's product of decays).
  auto state_update = [&](f32x4 (&S)[DT][ET], f32x4* Dacc, const bf16* s_kb, const float* s_dec) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(s_dec + 16 * dt + 4 * gq);
      if (Dacc != nullptr) Dacc[dt] *= dec;
#pragma unroll
      for (int et = 0; et < ET; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[dt][et][i] *= dec[i];
    }
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      bf16x8 vb[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) vb[et] = vT_op(m2, et);
#pragma unroll
      for (int d0 = 0; d0 < DT; d0 += 4) {
        bf16x8 kb[4];
#pragma unroll
        for (int dt = 0; dt < 4 && d0 + dt < DT; ++dt) kb[dt] = kbT_op(s_kb, m2, d0 + dt);
#pragma unroll
        for (int dt = 0; dt < 4 && d0 + dt < DT; ++dt)
#pragma unroll
          for (int et = 0; et < ET; ++et) S[d0 + dt][et] = mfma(kb[dt], vb[et], S[d0 + dt][et]);
      }
    }
  };

  auto consume_finish = [&](f32x4 (&S)[DT][ET], f32x4 (&acc)[4][ET], uint32_t (&opk)[4][2 * ET],
                            const bf16* s_kb, const float* s_dec) __attribute__((always_inline)) {
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      bf16x8 va[ET], aa[4];
#pragma unroll
      for (int et = 0; et < ET; ++et) va[et] = vT_op(m2, et);
#pragma unroll
      for (int t = 2 * m2; t < 4; ++t)
        aa[t] = *reinterpret_cast<const bf16x8*>(s_a + (16 * t + lr) * TP + 32 * m2 + 8 * gq);
#pragma unroll
      for (int t = 2 * m2; t < 4; ++t)
#pragma unroll
        for (int et = 0; et < ET; ++et) acc[t][et] = mfma(va[et], aa[t], acc[t][et]);
    }
    // acc[t][et][i] holds o of token 16t + lr, channel e0 + 4 ET gq + 4 et + i;
    // packed here, stored at the start of the next half (store_out)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const f32x4 x = acc[t][et];
        opk[t][2 * et] = pk2(x[0] * scale, x[1] * scale);
        opk[t][2 * et + 1] = pk2(x[2] * scale, x[3] * scale);
      }
    state_update(S, nullptr, s_kb, s_dec);
  };

  // ---- Dv = 128, consumer, end of the first half of step c+1: the packed
  // outputs of chunk c to the LDS stage (the producers store them).
  auto stage_out = [&](const uint32_t (&opk)[4][2 * ET]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 16 * t + lr, chunk = 4 * ci + gq;  // channels e0 + 8 gq .. + 7
      *reinterpret_cast<u32x4*>(s_o + row * (DV * 2) + ((chunk ^ (row & 15)) << 4)) =
          u32x4{opk[t][0], opk[t][1], opk[t][2], opk[t][3]};
    }
  };
  // ---- Dv = 128, producer, second half of step c+1: chunk c's outputs from
  // the stage, whole rows per store (producer w: the rows of sub-chunk w, 16
  // lanes per 256-byte row); rows past the chunk end are dropped by the range.
  auto store_rows = [&](int c) __attribute__((always_inline)) {
    const CPos cp = chunk_pos(c);
    const int64_t p0 = cp.p0;
    const int Lc = cp.len;
    const auto ro = rsrc(o + (p0 * H + h) * DV, uint32_t(Lc - 1) * rowV + DV * 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 16 * sw + 4 * m + (lane >> 4), chunk = lane & 15;
      const u32x4 x = *reinterpret_cast<const u32x4*>(s_o + row * (DV * 2) + ((chunk ^ (row & 15)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(v4i{int(x[0]), int(x[1]), int(x[2]), int(x[3])}, ro,
                                             uint32_t(row) * rowV + (chunk << 4), 0, 0);
    }
  };
  // ---- Dv = 64, consumer, second half of step c+1: the outputs of chunk c
  // packed in the first half. Issuing the stores here keeps them off the first
  // half, where the producers' loads fill the vector memory queue.
  auto store_out = [&](const uint32_t (&opk)[4][2 * ET], int c) __attribute__((always_inline)) {
    const CPos cp = chunk_pos(c);
    const int64_t p0 = cp.p0;
    const int Lc = cp.len;
    const auto ro = rsrc(o + (p0 * H + h) * DV, uint32_t(Lc - 1) * rowV + DV * 2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // rows past the chunk end fall outside the buffer range and are dropped
      const uint32_t off = uint32_t(16 * t + lr) * rowV + (e0 + 4 * ET * gq) * 2;
      if constexpr (ET == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(
            v4i{int(opk[t][0]), int(opk[t][1]), int(opk[t][2]), int(opk[t][3])}, ro, off, 0, 0);
      } else {
        typedef int v2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(v2{int(opk[t][0]), int(opk[t][1])}, ro, off, 0, 0);
      }
    }
  };

  // ---- consumer, second half: the A blocks of the chunk just prepared.
  // Jobs 0..9 are the blocks (w, j <= w), jobs 10 and 11 zero the blocks
  // (0, 1) and (2, 3) that the A.V product reads through its 32-wide steps.
  // Consumer ci takes jobs ci, ci + 4 and ci + 8 (the producers, whose work
  // per chunk sets the pace of the first half, take none). Zero jobs run on a
  // valid slot and their result is replaced, so no job branches.
  // a_blocks_mma does the products of all three jobs (their LDS operand reads
  // can all be in flight together); a_blocks_store masks, scales by beta and
  // writes them to the A tile. Keeping every write after every read of the
  // half lets the compiler overlap the reads: it cannot tell the A tile from
  // the operand tiles, so a write would hold back every later read.
  // Operand tiles (16 rows each) of the consumer's three jobs: the keys (KE
  // rows, or a key version slot) and the queries (a version slot).
  const bf16* a_key[3];
  const bf16* a_qry[3];
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    int ks = -1, qs = 0;  // key slot (-1: KE rows of block column j), query slot
    int bw, bj;
    block_of(ci + 4 * jj, bw, bj);
    switch (ci + 4 * jj) {
      case 0: qs = 0; break;            // (0, 0)
      case 1: qs = 4; break;            // (1, 0)
      case 2: qs = 1; break;            // (1, 1)
      case 3: ks = 7; qs = 5; break;    // (2, 0): KE 2^{T_1}
      case 4: qs = 5; break;            // (2, 1)
      case 5: qs = 2; break;            // (2, 2)
      case 6: qs = 8; break;            // (3, 0): Q~ 2^{T_1 + T_2}
      case 7: ks = 9; qs = 6; break;    // (3, 1): KE 2^{T_2}
      case 8: qs = 6; break;            // (3, 2)
      case 9: qs = 3; break;            // (3, 3)
      default: qs = 0; break;           // zero jobs: any valid tiles
    }
    a_key[jj] = ks < 0 ? s_ke + 16 * bj * KP : s_qv + ks * 16 * KP;
    a_qry[jj] = s_qv + qs * 16 * KP;
  }
  auto a_blocks_mma = [&](f32x4 (&ab)[3]) __attribute__((always_inline)) {
    // operands of K step u for the three jobs, read two steps ahead of their
    // products (the schedule is pinned: left to itself, the compiler keeps
    // one read pair in flight at a time here)
    bf16x8 op[2][3][2];
    auto read = [&](int u, bf16x8 (&o)[3][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) {
        const int col = 32 * u + 8 * gq;
        o[jj][0] = *reinterpret_cast<const bf16x8*>(a_key[jj] + lr * KP + col);
        o[jj][1] = *reinterpret_cast<const bf16x8*>(a_qry[jj] + lr * KP + col);
      }
    };
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) ab[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    read(0, op[0]);
    if constexpr (KS > 1) read(1, op[1]);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) ab[jj] = mfma(op[u & 1][jj][0], op[u & 1][jj][1], ab[jj]);
      __builtin_amdgcn_sched_barrier(0);
      if (u + 2 < KS) read(u + 2, op[u & 1]);
    }
  };
  auto a_blocks_store = [&](const f32x4 (&ab)[3], const float* s_bet) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int job = ci + 4 * jj;
      int bw, bj;
      block_of(job, bw, bj);
      const bool real = job < 10;
      const f32x4 bt = *reinterpret_cast<const f32x4*>(s_bet + 16 * bj + 4 * gq);
      float out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = 4 * gq + i;
        const bool keep = real && ((bj < bw) || (sl <= lr));
        out[i] = keep ? ab[jj][i] * bt[i] : 0.f;
      }
      st4(s_a + (16 * bw + lr) * TP + 16 * bj + 4 * gq, out);
    }
  };

  // ---------------------------------------------------------------- pipeline
  // Producers and consumers run separate loops with the same barrier sequence
  // (two per step), so neither role keeps the other's registers live.
  if (producer) {
    Raw<PCPL, PVPL> R;
    RawQK<PCPL> QA, QB;  // q, k of even / odd chunks
    const bool beta_wave = w == 0;
    uint32_t b0 = 0;  // raw beta of an item's first chunk (wave 0)
    // An item's first chunk: g, q, k and v to registers (R, QA), beta to b0.
    // For every item but the first, issued in the previous item's last step.
    auto load_first = [&]() __attribute__((always_inline)) {
      load_g(R, 0);
      load_qk(QA, 0);
      load_v(R, 0);
      if (beta_wave) b0 = load_beta(0);
    };
    int item = first_item;
    if (item < n_items) {
      begin_item(item);
      load_first();
    }
    while (item < n_items) {
      int next = 0;
      auto claim = [&](int s) __attribute__((always_inline)) {  // at step nchunks - 1
        if (s == nchunks - 1 && tid == 0) next = atomicAdd(counter, 1);
      };
      uint32_t bnext = 0, bnext2 = 0;  // raw beta of the next chunks (wave 0)
      if (beta_wave) {
        bnext = load_beta(1);
        s_beta[lane] = __uint_as_float(b0 << 16);
      }
      scan(R, QA);
      load_g(R, 1);
      __syncthreads();
      // Steps s = 0 .. nchunks - 1 (step s prepares chunk s and finishes
      // chunk s - 1): even steps use LDS buffers 0, odd steps buffers 1; two
      // steps per iteration (the q, k register sets alternate), the last even
      // step peeled, so the loop exits only at its bottom. Where a step skips
      // the use of loaded registers (the scan of a chunk past the item) it
      // waits for its loads instead: the compiler's wait bookkeeping merges
      // the paths of a step, and a load left pending on a rare path would
      // otherwise make every step's first LDS reads wait for the previous
      // step's loads.
      auto step_even = [&](int s) __attribute__((always_inline)) {
        claim(s);
        load_qk(QB, s + 1);
        produce_a(QA, s_qh, s_kb0, s_decay, s_beta);
        if (beta_wave) bnext2 = load_beta(s + 2);
        __syncthreads();
        if (!kState && C::stage_o && s >= 1) store_rows(s - 1);
        produce_b(R.v);
        load_v(R, s + 1);
        if (beta_wave) s_beta[kC + lane] = __uint_as_float(bnext << 16);
        if (s + 1 < nchunks) scan(R, QB); else wait_vm_all();
        load_g(R, s + 2);
        __syncthreads();
      };
      auto step_odd = [&](int s) __attribute__((always_inline)) {  // step s + 1
        claim(s + 1);
        load_qk(QA, s + 2);
        produce_a(QB, s_qh, s_kb1, s_decay + DK, s_beta + kC);
        if (beta_wave) bnext = load_beta(s + 3);
        __syncthreads();
        if (!kState && C::stage_o) store_rows(s);
        produce_b(R.v);
        load_v(R, s + 2);
        if (beta_wave) s_beta[lane] = __uint_as_float(bnext2 << 16);
        if (s + 2 < nchunks) scan(R, QA); else wait_vm_all();
        load_g(R, s + 3);
        __syncthreads();
      };
      int s = 0;
      for (; s + 2 <= nchunks; s += 2) {
        step_even(s);
        step_odd(s);
      }
      if (s < nchunks) step_even(s);
      // Step nchunks (the consumers finish the last chunk): the claimed item
      // number goes to LDS (every wave reads it after the barrier; the
      // consumers read it after this step), the last chunk's outputs are
      // stored, and the next item's first chunk is loaded, so its latency
      // overlaps this step and the consumers' end of the item.
      if (tid == 0) *s_item = next;
      __syncthreads();
      if (!kState && C::stage_o) store_rows(nchunks - 1);
      item = __builtin_amdgcn_readfirstlane(*s_item);
      if (item < n_items) {
        begin_item(item);
        load_first();
      }
      __syncthreads();
    }  // item loop
    if (flags != nullptr && tmin < kGateRangeMin)
      atomicOr(flags, kFlagGateRange);
  } else {
    // Run states and decays in the workspace: slot j, head h holds S as the
    // consumers keep it (consumer ci, tile (dt, et), lane: one f32x4 each)
    // and 2^{sum of the run's log2 gates} per key channel.
    auto state_at = [&](int j, int dt, int et) {
      return reinterpret_cast<f32x4*>(run_states) +
             (((int64_t(j) * H + h) * 4 + ci) * DT * ET + dt * ET + et) * 64 + lane;
    };
    auto decay_at = [&](int j, int dt) {
      return reinterpret_cast<f32x4*>(run_decays + (int64_t(j) * H + h) * DK + 16 * dt + 4 * gq);
    };
    for (int item = first_item; item < n_items;) {
      begin_item(item);
      // bit c: chunk c > 0 starts a segment of the group (none in an ordinary item)
      const uint64_t fresh_mask = __builtin_amdgcn_ballot_w64((ctab & 128u) != 0);
      f32x4 S[DT][ET];  // state rows [0, DK), columns [e0, e0 + EW)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int et = 0; et < ET; ++et) S[dt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kState) {
        f32x4 Dacc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) Dacc[dt] = f32x4{1.f, 1.f, 1.f, 1.f};
        __syncthreads();  // the producers' first scan
        for (int s = 0; s <= nchunks; s += 2) {
          if (s >= 1) state_update(S, Dacc, s_kb1, s_decay + DK);
          __syncthreads();
          __syncthreads();
          if (s + 1 > nchunks) break;
          state_update(S, Dacc, s_kb0, s_decay);
          __syncthreads();
          __syncthreads();
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int et = 0; et < ET; ++et) *state_at(sbase, dt, et) = S[dt][et];
        if (ci == 0 && lr == 0) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) *decay_at(sbase, dt) = Dacc[dt];
        }
      } else {
        // The segment starts from its initial state, when one is given; a
        // piece of a cut segment then folds in the pieces before it:
        // S = D_j S + L_j over them in order (D_j, L_j: piece j's decay
        // product and its state from zero).
        // Slot-indexed states; with row_len > 0 (segments from a [B, T] id
        // scan, padding segments have no items) they are row-indexed: a
        // row's first real segment starts from its row's state and its last
        // real one writes the row's final state. A real segment is the first
        // of its row when it starts the row or follows a padding segment that
        // does, and the last when it ends the row or precedes a padding
        // segment that does (runs of equal ids never cross a row start).
        int64_t init_idx = slot, fin_idx = slot;
        if (row_len > 0) {
          const int64_t a = cu[slot], e = cu[slot + 1];
          const int64_t b = a / row_len, r0 = b * row_len, r1 = r0 + row_len;
          const bool first = a == r0 || (cu[slot - 1] == r0 && seg_ids[r0] == 0);
          const bool lastr = e == r1 || (cu[slot + 2] == r1 && seg_ids[e] == 0);
          init_idx = first ? b : -1;
          fin_idx = lastr ? b : -1;
        }
        if (initial_state != nullptr && init_idx >= 0) {
          const float* s0 = initial_state + (init_idx * H + h) * DK * DV;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int et = 0; et < ET; ++et)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                S[dt][et][i] = s0[int64_t(16 * dt + 4 * gq + i) * DV + e0 + ecol(et, lr)];
        }
        for (int j = 0; j < run_idx; ++j) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const f32x4 d = *decay_at(sbase + j, dt);
#pragma unroll
            for (int et = 0; et < ET; ++et) S[dt][et] = S[dt][et] * d + *state_at(sbase + j, dt, et);
          }
        }
        f32x4 acc[4][ET];  // o^T of the chunk in flight, between its two halves
        uint32_t opk[4][2 * ET];  // packed outputs of the chunk finished in this step
        __syncthreads();  // the producers' first scan
        for (int s = 0; s <= nchunks; s += 2) {
          if (s >= 1) {
            consume_finish(S, acc, opk, s_kb1, s_decay + DK);
            if constexpr (C::stage_o) stage_out(opk);
          }
          __syncthreads();
          if (!C::stage_o && s >= 1) store_out(opk, s - 1);
          if (s < nchunks) {
            // a grouped segment after the first starts from zero (the zero state
            // before a segment's first chunk, without an initial state, is not stored)
            const bool fresh = s == 0 || ((fresh_mask >> (s & 63)) & 1);
            if (fresh && s > 0) zero_state(S);
            if constexpr (kSave)
              if (!fresh || run_idx > 0 || initial_state != nullptr) save_state(S, gc0 + s);
            f32x4 ab[3];
            a_blocks_mma(ab);
            consume_inter(S, acc);
            a_blocks_store(ab, s_beta);
          }
          __syncthreads();
          if (s + 1 > nchunks) break;
          consume_finish(S, acc, opk, s_kb0, s_decay);
          if constexpr (C::stage_o) stage_out(opk);
          __syncthreads();
          if constexpr (!C::stage_o) store_out(opk, s);
          if (s + 1 < nchunks) {
            const bool fresh = (fresh_mask >> ((s + 1) & 63)) & 1;
            if (fresh) zero_state(S);
            if constexpr (kSave)
              if (!fresh) save_state(S, gc0 + s + 1);
            f32x4 ab[3];
            a_blocks_mma(ab);
            consume_inter(S, acc);
            a_blocks_store(ab, s_beta + kC);
          }
          __syncthreads();
        }
        if (final_state != nullptr && last && fin_idx >= 0) {
          float* fs = final_state + (fin_idx * H + h) * DK * DV;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int et = 0; et < ET; ++et)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                fs[int64_t(16 * dt + 4 * gq + i) * DV + e0 + ecol(et, lr)] = S[dt][et][i];
        }
      }
      // written by the producers before the last step's first barrier
      item = __builtin_amdgcn_readfirstlane(*s_item);
    }  // item loop
  }

  if constexpr (!kState) {
    // After the queue: o = 0 at positions outside every segment, and the final
    // states of empty (and malformed) slots: their initial states, or zero;
    // grid-strided, 16-byte accesses.
    const int64_t G = gridDim.x;
    int64_t cu_last = (cu && row_len == 0) ? int64_t(cu[max_segs]) : N;
    cu_last = cu_last < 0 ? 0 : (cu_last > N ? N : cu_last);
    const int64_t n16 = (N - cu_last) * H * DV / 8;  // DV * 2 bytes is a multiple of 16
    u32x4* o16 = reinterpret_cast<u32x4*>(o + cu_last * H * DV);
    for (int64_t i = int64_t(blockIdx.x) * NT + tid; i < n16; i += G * NT) o16[i] = u32x4{0u, 0u, 0u, 0u};
    if (row_len > 0) {
      // [B, T] ids: padding segments output 0; a row of padding only passes
      // its initial state (or zero) through to its final state.
      const int n_seg = *n_dev;
      for (int u = blockIdx.x; u < n_seg; u += G) {
        const int64_t a = cu[u], e = cu[u + 1];
        if (seg_ids[a] != 0) continue;
        u32x4* oz = reinterpret_cast<u32x4*>(o + a * H * DV);
        for (int64_t i = tid; i < (e - a) * H * DV / 8; i += NT) oz[i] = u32x4{0u, 0u, 0u, 0u};
        if (final_state == nullptr || a % row_len != 0 || e - a != row_len) continue;
        const int64_t b = a / row_len;
        for (int hh = 0; hh < H; ++hh) {
          f32x4* f = reinterpret_cast<f32x4*>(final_state + (b * H + hh) * DK * DV);
          const f32x4* f0 = reinterpret_cast<const f32x4*>(initial_state + (b * H + hh) * DK * DV);
          for (int j = tid; j < DK * DV / 4; j += NT)
            f[j] = initial_state != nullptr ? f0[j] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (final_state != nullptr && cu != nullptr) {
      for (int64_t u = blockIdx.x; u < int64_t(max_segs) * H; u += G) {
        const int i = int(u / H);
        const int64_t a = cu[i], e = cu[i + 1];
        const bool bad = a < 0 || e < a || e > N || (i == 0 && a != 0);
        if (!bad && e > a) continue;
        f32x4* f = reinterpret_cast<f32x4*>(final_state + u * DK * DV);
        const f32x4* f0 = reinterpret_cast<const f32x4*>(initial_state + u * DK * DV);
        for (int j = tid; j < DK * DV / 4; j += NT)
          f[j] = initial_state != nullptr ? f0[j] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
}

// ---------------------------------------------------------------- work plan
// One work-group builds the launch's work list from cu_seqlens:
// 1. a segment of n chunks is one run when n <= kCutMin, else it is cut into
//    m = min(kMaxRuns, ceil(n / kRunLen)) nearly equal runs (run j = chunks
//    [n j / m, n (j + 1) / m)): a function of n alone, so where a segment is
//    cut (and with it the rounding of the composed states) never depends on
//    the other segments of the launch; empty and malformed segments have no
//    run (malformed ones set PKV_FLAG_BAD_CU_SEQLENS here);
// 2. in a call without initial and final states, short segments (at most
//    kGroupN chunks) in consecutive slots whose first chunks fall in one window
//    of kGroupWin chunks of the global chunk order form one item (a group):
//    its chunks run back to back, each segment from the zero state, so a
//    short document no longer pays a pipeline fill and drain of its own; the
//    outputs are those of the segments run as items of their own;
// 3. items are ranked longest first through a histogram of their lengths (ties
//    in any order: results do not depend on the order), and so are the runs
//    that are not last in their segment, which the state pass takes.
// The state slots of a segment's first m - 1 runs are consecutive from sbase
// (exclusive prefix of m - 1 over the segments, computed tile by tile).
// Chunk counts are below 2^26 (N <= INT32_MAX), so all per-segment arithmetic
// is 32-bit. One work-group of kPlanSmall threads for up to kPlanSmall slots,
// else of kPlanThreads: a call of up to 1024 slots is a single tile, so each
// pass over the slots takes one block scan.
__device__ __forceinline__ int plan_runs(int n) {
  if (n <= 0) return 0;
  if (n <= kCutMin) return 1;
  const int m = (n + kRunLen - 1) / kRunLen;
  return m < kMaxRuns ? m : kMaxRuns;
}
// chunks before run j of a segment of n chunks cut into m runs (n j < 2^30)
__device__ __forceinline__ int run_begin(int n, int m, int j) { return int(uint32_t(n * j) / uint32_t(m)); }
__device__ __forceinline__ int len_bin(int len) { return len < kHistBins - 1 ? len : kHistBins - 1; }

// Two exclusive prefixes over the work-group at once (the barriers of one);
// *tx and *ty get the sums.
template <int NT>
__device__ void block_exclusive_scan2(int x, int y, int2* s_tmp2, int* ex, int* ey, int* tx, int* ty) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ix = x, iy = y;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ux = __shfl_up(ix, d, 64), uy = __shfl_up(iy, d, 64);
    if (lane >= d) { ix += ux; iy += uy; }
  }
  if (lane == 63) s_tmp2[wv] = make_int2(ix, iy);
  __syncthreads();
  int bx = 0, by = 0, ax = 0, ay = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int2 t = s_tmp2[i];
    bx += i < wv ? t.x : 0;
    by += i < wv ? t.y : 0;
    ax += t.x;
    ay += t.y;
  }
  __syncthreads();
  *tx = ax;
  *ty = ay;
  *ex = bx + ix - x;
  *ey = by + iy - y;
}

// seg_ids (segments from a [B, T] id scan): a segment whose first id is 0 is
// padding and gets no run (its tokens leave the state alone and output 0).
template <int NT>
__global__ __launch_bounds__(NT) void kda_plan_kernel(const int32_t* __restrict__ cu,
                                                                const int32_t* __restrict__ n_dev,
                                                                const int32_t* __restrict__ seg_ids,
                                                                int32_t max_segs_arg, int32_t N,
                                                                int32_t states_max,
                                                                int32_t runs_max, int32_t group,
                                                                int32_t* __restrict__ plan,
                                                                int32_t* __restrict__ flags) {
  __shared__ int s_hr[kHistBins];  // main runs per length bin, then next free rank
  __shared__ int s_hs[kHistBins];  // state runs likewise
  __shared__ int2 s_tmp2[NT / 64];
  __shared__ int s_n[kPlanCache];  // chunk counts, when max_segs <= kPlanCache
  const int tid = threadIdx.x;
  // segment slots: the caller's count, or the one a boundary scan left on the device
  const int max_segs = n_dev != nullptr ? *n_dev : max_segs_arg;
  const int states_word_off = kPlanHeader + 8 * runs_max;
  const bool cached = max_segs <= kPlanCache;
  for (int i = tid; i < kHistBins; i += NT) s_hr[i] = s_hs[i] = 0;
  __syncthreads();
  // chunks of segment i; malformed and padding ones count 0, malformed ones are flagged
  auto chunks = [&](int i, bool& bad) -> int {
    bad = false;
    if (cu == nullptr) return int((uint32_t(N) + kC - 1) / kC);
    const int a = cu[i], e = cu[i + 1];
    bad = a < 0 || e < a || e > N || (i == 0 && a != 0);
    if (bad || e == a || (seg_ids != nullptr && seg_ids[a] == 0)) return 0;
    return int((uint32_t(e - a) + kC - 1) / kC);
  };
  bool any_bad = false;
  for (int i = tid; i < max_segs; i += NT) {
    bool bad;
    const int n = chunks(i, bad);
    if (cached) s_n[i] = n;
    any_bad = any_bad || bad;
  }
  if (any_bad && flags != nullptr) atomicOr(flags, kFlagBadCuSeqlens);
  __syncthreads();
  auto nchunks_of = [&](int i) -> int {
    bool bad;
    return cached ? s_n[i] : chunks(i, bad);
  };
  // Groups (only when group != 0): short segments (1..kGroupN chunks, one run
  // each) in consecutive slots, with no empty slot between them, whose first
  // chunks fall in the same window of kGroupWin chunks of the global chunk
  // order, share one item. The grouping only changes which work-group runs a
  // segment and when: each segment still starts from the zero state. Returns
  // 0 for a member that is not its group's first slot, else the number of
  // slots in the group (1: the segment alone); *tot gets the group's chunks.
  auto group_span = [&](int i, int n, int cb, int* tot) -> int {
    *tot = n;
    if (!group || n > kGroupN) return 1;
    const int win = cb / kGroupWin;
    if (i > 0) {
      const int np = nchunks_of(i - 1);
      if (np >= 1 && np <= kGroupN && (cb - np) / kGroupWin == win) return 0;
    }
    int j = i + 1, c = cb + n;
    while (j < max_segs && c / kGroupWin == win) {
      const int nj = nchunks_of(j);
      if (nj < 1 || nj > kGroupN) break;
      *tot += nj;
      c += nj;
      ++j;
    }
    return j - i;
  };

  // Runs of each segment, with the state-slot budget enforced in slot order:
  // a segment whose extra runs would not fit stays whole (only on malformed
  // input; the workspace bound covers every well-formed one).
  // cb: chunks of the slots before slot i (the global index of slot i's first chunk)
  auto pass = [&](auto&& body) {
    int carry = 0, ccarry = 0;
    for (int base = 0; base < max_segs; base += NT) {
      const int i = base + tid;
      bool bad;
      const int n = i >= max_segs ? 0 : cached ? s_n[i] : chunks(i, bad);
      int m = plan_runs(n);
      int tile_total, tile_chunks, esb, ecb;
      block_exclusive_scan2<NT>(m > 1 ? m - 1 : 0, n, s_tmp2, &esb, &ecb, &tile_total, &tile_chunks);
      const int sb = carry + esb;
      const int cb = ccarry + ecb;
      if (m > 1 && sb + m - 1 > states_max) m = 1;
      // a clamped segment's slots stay unused; later segments keep theirs
      if (m > 0) body(i, n, m, sb, cb);
      carry = carry + tile_total < (1 << 29) ? carry + tile_total : (1 << 29);
      ccarry += tile_chunks;
    }
  };
  // A segment of n chunks in m runs has n % m runs of q + 1 chunks and the
  // rest of q (q = n / m); its last run is one of the long ones iff n % m > 0.
  pass([&](int i, int n, int m, int, int cb) {
    int tot = n;
    const int gs = m == 1 ? group_span(i, n, cb, &tot) : 1;
    if (gs == 0) return;
    if (gs > 1) {
      atomicAdd(&s_hr[len_bin(tot)], 1);
      return;
    }
    const int q = n / m, nl = n - q * m, last_long = nl > 0;
    atomicAdd(&s_hr[len_bin(q + 1)], nl);
    atomicAdd(&s_hr[len_bin(q)], m - nl);
    atomicAdd(&s_hs[len_bin(q + 1)], nl - last_long);
    atomicAdd(&s_hs[len_bin(q)], m - nl - 1 + last_long);
  });
  __syncthreads();
  // bins to first ranks, longest first (suffix sums), consecutive bins per thread
  constexpr int kPer = kHistBins / NT;
  int cr[kPer], cs[kPer], sr = 0, ss = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int b = kHistBins - 1 - (tid * kPer + u);
    cr[u] = s_hr[b];
    cs[u] = s_hs[b];
    sr += cr[u];
    ss += cs[u];
  }
  int tr, ts, er, es;
  block_exclusive_scan2<NT>(sr, ss, s_tmp2, &er, &es, &tr, &ts);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int b = kHistBins - 1 - (tid * kPer + u);
    s_hr[b] = er;
    s_hs[b] = es;
    er += cr[u];
    es += cs[u];
  }
  __syncthreads();
  if (tid == 0) {
    plan[0] = tr;  // runs
    plan[1] = ts;  // state runs
    plan[2] = 0;   // queue counters of the forward and state passes
    plan[3] = 0;
  }
  pass([&](int i, int n, int m, int sb, int cb) {
    int tot = n;
    const int gs = m == 1 ? group_span(i, n, cb, &tot) : 1;
    if (gs == 0) return;
    if (gs > 1) {  // slots i .. i + gs - 1, chunks 0 .. tot - 1 of the group
      int32_t* e = plan + kPlanHeader + 8 * atomicAdd(&s_hr[len_bin(tot)], 1);
      e[0] = i;
      e[1] = 0;
      e[2] = tot;
      e[3] = 0;
      e[4] = sb;
      e[5] = 1;
      e[6] = cb;
      e[7] = gs;
      return;
    }
    // ranks for the segment's long and short runs, reserved in one go each
    const int q = n / m, nl = n - q * m, last_long = nl > 0;
    int rl = atomicAdd(&s_hr[len_bin(q + 1)], nl);
    int rs = atomicAdd(&s_hr[len_bin(q)], m - nl);
    int sl = atomicAdd(&s_hs[len_bin(q + 1)], nl - last_long);
    int ss = atomicAdd(&s_hs[len_bin(q)], m - nl - 1 + last_long);
    for (int j = 0; j < m; ++j) {
      const int c0 = run_begin(n, m, j), c1 = run_begin(n, m, j + 1);
      const bool lng = c1 - c0 > q;
      int32_t* e = plan + kPlanHeader + 8 * (lng ? rl++ : rs++);
      e[0] = i;
      e[1] = c0;
      e[2] = c1;
      e[3] = j;
      e[4] = sb;
      e[5] = j + 1 == m;
      e[6] = cb;
      e[7] = 0;
      if (j + 1 < m) {
        int32_t* f = plan + states_word_off + 4 * (lng ? sl++ : ss++);
        f[0] = i;
        f[1] = c0;
        f[2] = c1;
        f[3] = sb + j;
      }
    }
  });
}

struct PlanLayout {
  int64_t runs_max, states_max;
  size_t states_word_off;  // int32 words from the workspace start
  size_t off_L, off_D, bytes;
};

// Saved pieces: a cut segment has len > kCutMin * kC tokens and n =
// ceil(len / kC) chunks, and saves m - 1 < n / kRunLen <= (len + kC - 1) /
// (kC kRunLen) pieces; over at most N / (kCutMin kC + 1) such segments whose
// lengths sum to at most N, that is below the bound here (about N / 4096,
// 1/16 of one [N, H, Dk] bf16 tensor in bytes at Dv = 128).
PlanLayout plan_layout(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t max_segs) {
  PlanLayout p;
  constexpr int64_t kCutLen = int64_t(kCutMin) * kC + 1;  // shortest cut segment, tokens
  const int64_t n_cut = N / kCutLen;
  p.states_max = n_cut == 0 ? 0 : (N + (kC - 1) * n_cut) / (int64_t(kC) * kRunLen) + 1;
  p.runs_max = int64_t(max_segs) + p.states_max;
  p.states_word_off = size_t(kPlanHeader) + 8 * size_t(p.runs_max);
  const size_t table = (p.states_word_off + 4 * size_t(p.states_max)) * 4;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  p.off_L = up(table);
  p.off_D = p.off_L + up(size_t(p.states_max) * H * Dk * Dv * 4);
  p.bytes = p.off_D + up(size_t(p.states_max) * H * Dk * 4);
  return p;
}


// Arguments of one call of the chunk path.
struct Launch {
  const void *q, *k, *v, *g, *beta;
  const int32_t* cu;      // segment bounds
  const int32_t* n_dev;   // number of segments on the device (ids path) or NULL
  int32_t layout_segs;    // bound on the number of segments (workspace layout)
  int32_t max_segs;       // segment slots (0 on the ids path)
  int64_t N;
  int32_t H;
  float scale;
  const float* s0;
  void* o;
  float* fs;
  int32_t* flags;
  char* ws;
  int64_t row_len;        // > 0: ids path, segments map to rows of this length
  const int32_t* seg_ids; // ids path: the [B, T] ids
  hipStream_t stream;
  void* chunk_states;     // bf16 state before every chunk, or NULL
};

// The plan, the state pass and the forward pass over segments given by cu
// (max_segs slots), or, with n_dev, by the first *n_dev + 1 entries of cu that
// a boundary scan wrote (layout_segs bounds their number; row_len > 0 then
// maps segments to rows for the initial and final states).
template <int DK, int DV, bool kNorm, bool kSave>
hipError_t launch_dims(const Launch& a) {
  using C = Cfg<DK, DV>;
  constexpr int state_bytes = C::off_qh;  // the state pass uses the small tables, V and Kbar
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<DK, DV, false, kNorm, kSave>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<DK, DV, true, kNorm, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, state_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const PlanLayout L = plan_layout(a.N, a.H, DK, DV, a.layout_segs);
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws);
  float* states = reinterpret_cast<float*>(a.ws + L.off_L);
  float* decays = reinterpret_cast<float*>(a.ws + L.off_D);
  if (a.max_segs <= kPlanSmall)
    hipLaunchKernelGGL(kda_plan_kernel<kPlanSmall>, dim3(1), dim3(kPlanSmall), 0, a.stream, a.cu, a.n_dev,
                       a.seg_ids, a.max_segs, int32_t(a.N), int32_t(L.states_max), int32_t(L.runs_max),
                       int32_t(a.s0 == nullptr && a.fs == nullptr), plan, a.flags);
  else
    hipLaunchKernelGGL(kda_plan_kernel<kPlanThreads>, dim3(1), dim3(kPlanThreads), 0, a.stream, a.cu, a.n_dev,
                       a.seg_ids, a.max_segs, int32_t(a.N), int32_t(L.states_max), int32_t(L.runs_max),
                       int32_t(a.s0 == nullptr && a.fs == nullptr), plan, a.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const auto qp = static_cast<const bf16*>(a.q), kp = static_cast<const bf16*>(a.k);
  const auto vp = static_cast<const bf16*>(a.v), gp = static_cast<const bf16*>(a.g);
  const auto bp = static_cast<const bf16*>(a.beta);
  // persistent grids: as many work-groups as the LDS lets each CU hold
  const unsigned grid = unsigned(device_cus() * C::WG_PER_CU);
  if (L.states_max > 0) {
    hipLaunchKernelGGL((kda_chunk_kernel<DK, DV, true, kNorm, false>), dim3(grid), dim3(C::NT), state_bytes,
                       a.stream, qp, kp, vp, gp, bp, a.cu, plan, int32_t(L.runs_max), a.max_segs, a.N,
                       a.H, a.scale, static_cast<const float*>(nullptr), static_cast<bf16*>(nullptr),
                       static_cast<float*>(nullptr), states, decays, a.row_len, a.seg_ids, a.n_dev, a.flags,
                       static_cast<bf16*>(nullptr), 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((kda_chunk_kernel<DK, DV, false, kNorm, kSave>), dim3(grid), dim3(C::NT), C::bytes,
                     a.stream, qp, kp, vp, gp, bp, a.cu, plan, int32_t(L.runs_max), a.max_segs, a.N,
                     a.H, a.scale, a.s0, static_cast<bf16*>(a.o), a.fs, states, decays, a.row_len,
                     a.seg_ids, a.n_dev, a.flags, static_cast<bf16*>(a.chunk_states), 0);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_norm(bool qk_l2norm, const Launch& a) {
  if (a.chunk_states != nullptr)
    return qk_l2norm ? launch_dims<DK, DV, true, true>(a) : launch_dims<DK, DV, false, true>(a);
  return qk_l2norm ? launch_dims<DK, DV, true, false>(a) : launch_dims<DK, DV, false, false>(a);
}

hipError_t dispatch(int32_t Dk, int32_t Dv, bool qk_l2norm, const Launch& a) {
  if (Dk == 128 && Dv == 128) return launch_norm<128, 128>(qk_l2norm, a);
  if (Dk == 64 && Dv == 64) return launch_norm<64, 64>(qk_l2norm, a);
  if (Dk == 128 && Dv == 64) return launch_norm<128, 64>(qk_l2norm, a);
  if (Dk == 64 && Dv == 128) return launch_norm<64, 128>(qk_l2norm, a);
  return hipErrorInvalidValue;
}

}  // namespace

// Compute units of the current device (the persistent grids' size).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

bool kda_chunk_supported(int32_t Dk, int32_t Dv, int32_t dtype) {
  return dtype == 0 && (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
}

size_t kda_chunk_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                                 int32_t max_segs) {
  if (!kda_chunk_supported(Dk, Dv, dtype) || N < 1 || H < 1 || max_segs < 1) return 0;
  return plan_layout(N, H, Dk, Dv, max_segs).bytes;
}

// [B, T] ids path: the segment count word and bounds (N + 1 int32) first,
// then the plan's layout for at most N segments.
size_t ids_bounds_bytes(int64_t N) { return (size_t(N) * 4 + 4 + 256 + 255) / 256 * 256; }

size_t kda_chunk_ids_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype) {
  if (!kda_chunk_supported(Dk, Dv, dtype) || N < 1 || H < 1) return 0;
  return ids_bounds_bytes(N) + plan_layout(N, H, Dk, Dv, int32_t(N)).bytes;
}

hipError_t launch_kda_chunk_ids(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, const int32_t* seg, int64_t B, int64_t T,
                                int32_t H, int32_t Dk, int32_t Dv, float scale, bool qk_l2norm,
                                const float* initial_state, void* o, float* final_state,
                                int32_t* flags, void* workspace, hipStream_t stream) {
  const int64_t N = B * T;
  char* ws = static_cast<char*>(workspace);
  int32_t* n_dev = reinterpret_cast<int32_t*>(ws);
  int32_t* bounds = reinterpret_cast<int32_t*>(ws + 256);
  // segment starts of the [B, T] contract, found by the conversion's scan
  const hipError_t e = launch_segment_bounds(seg, N, T, bounds, n_dev, stream);
  if (e != hipSuccess) return e;
  const Launch a{q, k, v, g, beta, bounds, n_dev, int32_t(N), 0, N, H, scale, initial_state, o,
                 final_state, flags, ws + ids_bounds_bytes(N), T, seg, stream, nullptr};
  return dispatch(Dk, Dv, qk_l2norm, a);
}

hipError_t launch_kda_chunk(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                            int32_t H, int32_t Dk, int32_t Dv, float scale, bool qk_l2norm,
                            const float* initial_state, void* o, float* final_state,
                            int32_t* flags, void* workspace, hipStream_t stream, void* chunk_states) {
  const Launch a{q, k, v, g, beta, cu, nullptr, max_segs, max_segs, N, H, scale, initial_state, o,
                 final_state, flags, static_cast<char*>(workspace), 0, nullptr, stream, chunk_states};
  return dispatch(Dk, Dv, qk_l2norm, a);
}

// ---------------------------------------------------------------- no allocation
// Scratch of pkv_chunk_kda_varlen_noalloc: the workspace of the chunk path
// (work plan, queue counters, states and decay products of cut pieces) in a
// fixed array of the library's device memory. Each GPU the library runs on
// holds its own copy until the process ends; every call on that GPU uses it,
// so calls that overlap on one GPU race. Nothing in it needs clearing: the
// plan kernel writes the plan and resets the queue counters at the start of
// every call, and each piece's state is written before it is read.
namespace {
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

// The device address of this GPU's copy of the array, looked up once per
// device with the device current. In host code the array's name is only a
// host-side stand-in, so kernels get this pointer, never the name.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_kda_chunk_noalloc(const void* q, const void* k, const void* v, const void* g,
                                    const void* beta, const int32_t* cu, int32_t max_segs,
                                    int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                    bool qk_l2norm, const float* initial_state, void* o,
                                    float* final_state, int32_t* flags, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_kda_chunk(q, k, v, g, beta, cu, max_segs, N, H, Dk, Dv, scale, qk_l2norm,
                          initial_state, o, final_state, flags, ws, stream);
}

}  // namespace pkv
