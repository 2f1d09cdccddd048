// Shared device helpers and launcher declarations for libpkv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// Flags word bits (mirrors include/pkv.h).
constexpr int32_t kFlagOverflow = 1;
constexpr int32_t kFlagLeadingPad = 2;
constexpr int32_t kFlagBadCuSeqlens = 4;
constexpr int32_t kFlagGateRange = 8;
// The chunked bf16 paths split each 64-token chunk into 16-token sub-chunks
// and put 2^{-(sum of a sub-chunk's log2 gates)} on one operand of its
// diagonal block (the forward's query side, the reverse pass's key side).
// Below this total (log2 units; 2^-120 as a factor) that operand can leave
// the fp32 / bf16 range, and the call sets kFlagGateRange.
constexpr float kGateRangeMinLog2 = -120.f;
constexpr float kGateRangeMin = 0x1p-120f;  // 2^kGateRangeMinLog2

// Compute units of the current device (the persistent grids' size; cached per device).
int device_cus();

// Launchers (host side). Each returns the HIP error of its launch(es).
hipError_t launch_cu_seqlens(const int32_t* seg, int64_t N, int64_t T, int32_t max_segs,
                             int32_t* cu, int32_t* token_seg, int32_t* n_segs, int32_t* flags,
                             hipStream_t stream);

// The [B, T] contract's segment starts (every id change and row start):
// bounds[0..n] with bounds[n] = N, n to *n_segs.
hipError_t launch_segment_bounds(const int32_t* seg, int64_t N, int64_t T, int32_t* bounds,
                                 int32_t* n_segs, hipStream_t stream);

hipError_t launch_eod_segments(const int32_t* tokens, int64_t B, int64_t T, int32_t eod_id,
                               int32_t* seg, int32_t* pos, int32_t* loss, hipStream_t stream);

hipError_t launch_short_conv(const void* x, const float* w, const int32_t* seg, void* y,
                             int64_t B, int64_t T, int64_t F, int32_t Kc, int32_t dtype,
                             hipStream_t stream);

// qk_l2norm (every recurrence launcher): q and k are first L2-normalised per
// (token, head) over Dk.
hipError_t launch_kda_serial(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                             int32_t H, int32_t Dk, int32_t Dv, float scale, int32_t dtype,
                             bool qk_l2norm, const float* initial_state, void* o,
                             float* final_state, int32_t* flags, hipStream_t stream);

bool kda_chunk_supported(int32_t Dk, int32_t Dv, int32_t dtype);

// Workspace of the chunk path (0 when the path is not used): the work plan
// (runs, longest first) and the states and decay products of the pieces of
// cut segments.
size_t kda_chunk_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                                 int32_t max_segs);

// [B, T] segment_ids entry (RFC-0026 section 3.1.1) on the chunk path.
size_t kda_chunk_ids_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype);
hipError_t launch_kda_chunk_ids(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, const int32_t* seg, int64_t B, int64_t T,
                                int32_t H, int32_t Dk, int32_t Dv, float scale, bool qk_l2norm,
                                const float* initial_state, void* o, float* final_state,
                                int32_t* flags, void* workspace, hipStream_t stream);
// ... and on the token-serial path (one work-group per (row, head)).
hipError_t launch_kda_serial_ids(const void* q, const void* k, const void* v, const void* g,
                                 const void* beta, const int32_t* seg, int64_t B, int64_t T,
                                 int32_t H, int32_t Dk, int32_t Dv, float scale, int32_t dtype,
                                 bool qk_l2norm, const float* initial_state, void* o,
                                 float* final_state, hipStream_t stream);

// chunk_states: NULL, or where the bf16 state before every 64-token chunk is
// written (the reverse pass's layout; see kda_chunk_states_bytes).
hipError_t launch_kda_chunk(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const int32_t* cu, int32_t max_segs, int64_t N,
                            int32_t H, int32_t Dk, int32_t Dv, float scale, bool qk_l2norm,
                            const float* initial_state, void* o, float* final_state,
                            int32_t* flags, void* workspace, hipStream_t stream,
                            void* chunk_states = nullptr);

// The same with the workspace in the library's fixed per-GPU scratch array of
// kNoAllocScratchBytes (for callers that cannot allocate); the caller has
// checked that the chunk path's workspace size fits.
constexpr size_t kNoAllocScratchBytes = size_t(96) << 20;
hipError_t launch_kda_chunk_noalloc(const void* q, const void* k, const void* v, const void* g,
                                    const void* beta, const int32_t* cu, int32_t max_segs,
                                    int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                    bool qk_l2norm, const float* initial_state, void* o,
                                    float* final_state, int32_t* flags, hipStream_t stream);

// Reverse pass of the recurrence, chunked on MFMA (bf16, Dk and Dv in {64, 128}):
// the work plan, piece summaries and (unless the caller gives them) the bf16
// state before every chunk in the workspace.
bool kda_chunk_bwd_supported(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                             int32_t max_segs);
size_t kda_chunk_bwd_workspace_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                                     int32_t max_segs, bool states_given = false);
// Bytes of the per-chunk states ([ceil(N / 64) + max_segs, H, Dk, Dv] bf16), or 0
// when the shape has no chunked reverse pass.
size_t kda_chunk_states_bytes(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                              int32_t max_segs);
hipError_t launch_kda_chunk_backward(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta, const void* dout, const int32_t* cu,
                                     int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                     float scale, const float* initial_state,
                                     const float* dfinal_state, void* dq, void* dk, void* dv,
                                     void* dg, void* dbeta, float* dinitial_state, int32_t* flags,
                                     void* workspace, hipStream_t stream,
                                     const void* chunk_states = nullptr);

// Reverse pass of the recurrence, token-serial (every other shape; no workspace).
hipError_t launch_kda_backward(const void* q, const void* k, const void* v, const void* g,
                               const void* beta, const void* dout, const int32_t* cu,
                               int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                               float scale, int32_t dtype, const float* initial_state,
                               const float* dfinal_state, void* dq, void* dk, void* dv, void* dg,
                               void* dbeta, float* dinitial_state, int32_t* flags,
                               hipStream_t stream);

}  // namespace pkv
