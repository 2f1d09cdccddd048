// libpkv C ABI: argument validation and dispatch. Every check here runs before
// any HIP call, so invalid arguments are reported synchronously and nothing is
// enqueued. See include/pkv.h for the contract of each entry point.

#include "pkv.h"

#include <hip/hip_runtime.h>

#include "common.h"

namespace {

constexpr int64_t kInt32Max = 2147483647;
constexpr int32_t kKnownOptions = PKV_OPT_QK_L2NORM;

bool supported_head_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }
bool known_dtype(int32_t dt) { return dt == PKV_BF16 || dt == PKV_F32; }
int64_t elem_size(int32_t dt) { return dt == PKV_BF16 ? 2 : 4; }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + b_bytes && pb < pa + a_bytes;
}

pkv_status from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARGUMENT: return "PKV_ERR_INVALID_ARGUMENT";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
  }
  return "PKV_ERR_UNKNOWN";
}

pkv_status pkv_segment_ids_to_cu_seqlens(const int32_t* segment_ids, int64_t B, int64_t T,
                                         int32_t max_segs, int32_t* cu_seqlens,
                                         int32_t* token_seg, int32_t* n_segs, int32_t* flags,
                                         void* stream) {
  if (segment_ids == nullptr || cu_seqlens == nullptr) return PKV_ERR_INVALID_ARGUMENT;
  if (B < 1 || T < 1 || B > kInt32Max || T > kInt32Max || B * T > kInt32Max)
    return PKV_ERR_INVALID_ARGUMENT;
  if (max_segs < 1 || max_segs >= kInt32Max) return PKV_ERR_INVALID_ARGUMENT;
  return from_hip(pkv::launch_cu_seqlens(segment_ids, B * T, T, max_segs, cu_seqlens, token_seg,
                                         n_segs, flags, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_eod_to_segment_ids(const int32_t* tokens, int64_t B, int64_t T, int32_t eod_id,
                                  int32_t* segment_ids, int32_t* positions,
                                  int32_t* loss_segment_ids, void* stream) {
  if (tokens == nullptr || segment_ids == nullptr) return PKV_ERR_INVALID_ARGUMENT;
  if (B < 1 || T < 1 || B > kInt32Max || T > kInt32Max || B * T > kInt32Max)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t n = B * T * 4;
  const void* outs[3] = {segment_ids, positions, loss_segment_ids};
  for (int i = 0; i < 3; ++i) {
    if (outs[i] == nullptr) continue;
    if (overlaps(outs[i], n, tokens, n)) return PKV_ERR_INVALID_ARGUMENT;
    for (int j = 0; j < i; ++j)
      if (outs[j] != nullptr && overlaps(outs[i], n, outs[j], n)) return PKV_ERR_INVALID_ARGUMENT;
  }
  return from_hip(pkv::launch_eod_segments(tokens, B, T, eod_id, segment_ids, positions,
                                           loss_segment_ids, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_short_conv_segmask(const void* x, const float* w, const int32_t* segment_ids,
                                  void* y, int64_t B, int64_t T, int64_t F, int32_t Kc,
                                  int32_t dtype, void* stream) {
  if (x == nullptr || w == nullptr || y == nullptr) return PKV_ERR_INVALID_ARGUMENT;
  if (B < 1 || T < 1 || F < 1) return PKV_ERR_INVALID_ARGUMENT;
  if (B > 65535 || T > (int64_t(1) << 36) || F > (int64_t(1) << 36) || B * T > (int64_t(1) << 40) ||
      (B * T) > (int64_t(1) << 62) / F)
    return PKV_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype) || Kc < 1 || Kc > 8) return PKV_ERR_UNSUPPORTED;
  const int64_t bytes = B * T * F * elem_size(dtype);
  if (overlaps(x, bytes, y, bytes)) return PKV_ERR_INVALID_ARGUMENT;
  if ((T + 31) / 32 > 65535 || ((F + 255) / 256) > kInt32Max) return PKV_ERR_INVALID_ARGUMENT;
  return from_hip(pkv::launch_short_conv(x, w, segment_ids, y, B, T, F, Kc, dtype,
                                         static_cast<hipStream_t>(stream)));
}

size_t pkv_chunk_kda_varlen_workspace_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                           int32_t max_segs, int32_t dtype) {
  return pkv::kda_chunk_workspace_bytes(N, H, Dk, Dv, dtype, max_segs);
}

}  // extern "C"

namespace {

// Checks shared by pkv_chunk_kda_varlen and pkv_chunk_kda_varlen_noalloc
// (everything but the workspace); max_segs is set to 1 when cu_seqlens is NULL.
pkv_status check_kda_args(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const int32_t* cu_seqlens, int32_t& max_segs,
                          int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                          int32_t options, const float* initial_state, const void* o,
                          const float* final_state) {
  if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
      o == nullptr)
    return PKV_ERR_INVALID_ARGUMENT;
  if (N < 1 || N > kInt32Max || H < 1 || H > 65536) return PKV_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr) {
    max_segs = 1;
  } else if (max_segs < 1 || max_segs >= kInt32Max) {
    return PKV_ERR_INVALID_ARGUMENT;
  }
  if (!known_dtype(dtype) || !supported_head_dim(Dk) || !supported_head_dim(Dv) ||
      (options & ~kKnownOptions) != 0)
    return PKV_ERR_UNSUPPORTED;
  for (const void* p : {q, k, v, g, o})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(beta) % elem_size(dtype) != 0 ||
      reinterpret_cast<uintptr_t>(final_state) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(initial_state) % 16 != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t state_bytes = int64_t(max_segs) * H * Dk * Dv * 4;
  if (initial_state != nullptr && final_state != nullptr &&
      overlaps(initial_state, state_bytes, final_state, state_bytes))
    return PKV_ERR_INVALID_ARGUMENT;
  if (int64_t(max_segs) * H > (int64_t(1) << 22)) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t es = elem_size(dtype);
  const int64_t o_bytes = N * H * Dv * es;
  if (overlaps(o, o_bytes, q, N * H * Dk * es) || overlaps(o, o_bytes, k, N * H * Dk * es) ||
      overlaps(o, o_bytes, v, N * H * Dv * es) || overlaps(o, o_bytes, g, N * H * Dk * es) ||
      overlaps(o, o_bytes, beta, N * H * es))
    return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_chunk_kda_varlen(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, const int32_t* cu_seqlens, int32_t max_segs,
                                int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                int32_t dtype, int32_t options, const float* initial_state,
                                void* o, float* final_state, int32_t* flags, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const pkv_status st = check_kda_args(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, dtype,
                                       options, initial_state, o, final_state);
  const bool l2 = (options & PKV_OPT_QK_L2NORM) != 0;
  if (st != PKV_OK) return st;
  const size_t need = pkv_chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
    return PKV_ERR_WORKSPACE;
  if (pkv::kda_chunk_supported(Dk, Dv, dtype))
    return from_hip(pkv::launch_kda_chunk(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv,
                                          scale, l2, initial_state, o, final_state, flags,
                                          workspace, static_cast<hipStream_t>(stream)));
  return from_hip(pkv::launch_kda_serial(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv,
                                         scale, dtype, l2, initial_state, o, final_state, flags,
                                         static_cast<hipStream_t>(stream)));
}

size_t pkv_chunk_kda_states_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t max_segs,
                                 int32_t dtype) {
  return pkv::kda_chunk_states_bytes(N, H, Dk, Dv, dtype, max_segs);
}

pkv_status pkv_chunk_kda_varlen_states(const void* q, const void* k, const void* v, const void* g,
                                       const void* beta, const int32_t* cu_seqlens, int32_t max_segs,
                                       int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                       int32_t dtype, int32_t options, const float* initial_state,
                                       void* o, float* final_state, int32_t* flags, void* workspace,
                                       size_t workspace_bytes, void* chunk_states,
                                       size_t chunk_states_bytes, void* stream) {
  const pkv_status st = check_kda_args(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, dtype,
                                       options, initial_state, o, final_state);
  const bool l2 = (options & PKV_OPT_QK_L2NORM) != 0;
  if (st != PKV_OK) return st;
  const size_t states = pkv::kda_chunk_states_bytes(N, H, Dk, Dv, dtype, max_segs);
  if (!pkv::kda_chunk_supported(Dk, Dv, dtype) || states == 0) return PKV_ERR_UNSUPPORTED;
  const size_t need = pkv_chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
    return PKV_ERR_WORKSPACE;
  if (chunk_states == nullptr || chunk_states_bytes < states ||
      reinterpret_cast<uintptr_t>(chunk_states) % 16 != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t es = elem_size(dtype), sb = int64_t(states);
  const int64_t kb = N * H * Dk * es, vb = N * H * Dv * es;
  const int64_t fb = int64_t(max_segs) * H * Dk * Dv * 4;
  const void* others[9] = {q, k, v, g, beta, o, initial_state, final_state, workspace};
  const int64_t other_bytes[9] = {kb, kb, vb, kb, N * H * es, vb, fb, fb, int64_t(need)};
  for (int i = 0; i < 9; ++i)
    if (others[i] != nullptr && overlaps(chunk_states, sb, others[i], other_bytes[i]))
      return PKV_ERR_INVALID_ARGUMENT;
  return from_hip(pkv::launch_kda_chunk(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, scale,
                                        l2, initial_state, o, final_state, flags, workspace,
                                        static_cast<hipStream_t>(stream), chunk_states));
}

pkv_status pkv_chunk_kda_varlen_noalloc(const void* q, const void* k, const void* v,
                                        const void* g, const void* beta,
                                        const int32_t* cu_seqlens, int32_t max_segs, int64_t N,
                                        int32_t H, int32_t Dk, int32_t Dv, float scale,
                                        int32_t dtype, int32_t options, const float* initial_state,
                                        void* o, float* final_state, int32_t* flags,
                                        void* stream) {
  const pkv_status st = check_kda_args(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, dtype,
                                       options, initial_state, o, final_state);
  const bool l2 = (options & PKV_OPT_QK_L2NORM) != 0;
  if (st != PKV_OK) return st;
  const size_t need = pkv_chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, dtype);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  static_assert(PKV_NOALLOC_SCRATCH_BYTES == pkv::kNoAllocScratchBytes, "scratch size");
  if (pkv::kda_chunk_supported(Dk, Dv, dtype))
    return from_hip(pkv::launch_kda_chunk_noalloc(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk,
                                                  Dv, scale, l2, initial_state, o, final_state,
                                                  flags, static_cast<hipStream_t>(stream)));
  return from_hip(pkv::launch_kda_serial(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv,
                                         scale, dtype, l2, initial_state, o, final_state, flags,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// pkv_chunk_kda_varlen_backward, and with with_states its variant that reads the
// forward call's per-chunk states instead of recomputing them.
pkv_status kda_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const int32_t* cu_seqlens, int32_t max_segs, int64_t N, int32_t H,
                        int32_t Dk, int32_t Dv, float scale, int32_t dtype,
                        const float* initial_state, const void* do_, const float* dfinal_state,
                        void* dq, void* dk, void* dv, void* dg, void* dbeta, float* d_initial_state,
                        int32_t* flags, void* workspace, size_t workspace_bytes, bool with_states,
                        const void* chunk_states, size_t chunk_states_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
      do_ == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || dg == nullptr ||
      dbeta == nullptr)
    return PKV_ERR_INVALID_ARGUMENT;
  if (N < 1 || N > kInt32Max || H < 1 || H > 65536) return PKV_ERR_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr) {
    max_segs = 1;
  } else if (max_segs < 1 || max_segs >= kInt32Max) {
    return PKV_ERR_INVALID_ARGUMENT;
  }
  if (!known_dtype(dtype) || !supported_head_dim(Dk) || !supported_head_dim(Dv))
    return PKV_ERR_UNSUPPORTED;
  if (int64_t(max_segs) * H > (int64_t(1) << 22)) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t es = elem_size(dtype);
  for (const void* p : {q, k, v, g, do_, static_cast<const void*>(dq),
                        static_cast<const void*>(dk), static_cast<const void*>(dv),
                        static_cast<const void*>(dg)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(beta) % es != 0 || reinterpret_cast<uintptr_t>(dbeta) % es != 0 ||
      reinterpret_cast<uintptr_t>(initial_state) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dfinal_state) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(d_initial_state) % 16 != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  const size_t states = with_states ? pkv::kda_chunk_states_bytes(N, H, Dk, Dv, dtype, max_segs) : 0;
  if (with_states) {
    if (states == 0) return PKV_ERR_UNSUPPORTED;
    if (chunk_states == nullptr || chunk_states_bytes < states ||
        reinterpret_cast<uintptr_t>(chunk_states) % 16 != 0)
      return PKV_ERR_INVALID_ARGUMENT;
  }
  const int64_t kb = N * H * Dk * es, vb = N * H * Dv * es, bb = N * H * es;
  const int64_t sb = int64_t(max_segs) * H * Dk * Dv * 4;
  const int64_t cb = cu_seqlens ? (int64_t(max_segs) + 1) * 4 : 0;
  const void* ins[9] = {q, k, v, g, beta, do_, initial_state, dfinal_state, chunk_states};
  const int64_t in_bytes[9] = {kb, kb, vb, kb, bb, vb, sb, sb, int64_t(states)};
  const void* outs[6] = {dq, dk, dv, dg, dbeta, d_initial_state};
  const int64_t out_bytes[6] = {kb, kb, vb, kb, bb, sb};
  for (int i = 0; i < 6; ++i) {
    if (outs[i] == nullptr) continue;
    for (int j = 0; j < 9; ++j)
      if (ins[j] != nullptr && overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return PKV_ERR_INVALID_ARGUMENT;
    if (cu_seqlens != nullptr && overlaps(outs[i], out_bytes[i], cu_seqlens, cb))
      return PKV_ERR_INVALID_ARGUMENT;
    for (int j = 0; j < i; ++j)
      if (outs[j] != nullptr && overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return PKV_ERR_INVALID_ARGUMENT;
  }
  const size_t need = pkv::kda_chunk_bwd_workspace_bytes(N, H, Dk, Dv, dtype, max_segs, with_states);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return PKV_ERR_WORKSPACE;
    for (int i = 0; i < 9; ++i)
      if (ins[i] != nullptr && overlaps(workspace, int64_t(need), ins[i], in_bytes[i]))
        return PKV_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 6; ++i)
      if (outs[i] != nullptr && overlaps(workspace, int64_t(need), outs[i], out_bytes[i]))
        return PKV_ERR_INVALID_ARGUMENT;
    return from_hip(pkv::launch_kda_chunk_backward(
        q, k, v, g, beta, do_, cu_seqlens, max_segs, N, H, Dk, Dv, scale, initial_state,
        dfinal_state, dq, dk, dv, dg, dbeta, d_initial_state, flags, workspace,
        static_cast<hipStream_t>(stream), with_states ? chunk_states : nullptr));
  }
  return from_hip(pkv::launch_kda_backward(q, k, v, g, beta, do_, cu_seqlens, max_segs, N, H, Dk,
                                           Dv, scale, dtype, initial_state, dfinal_state, dq, dk,
                                           dv, dg, dbeta, d_initial_state, flags,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pkv_status pkv_chunk_kda_varlen_backward(const void* q, const void* k, const void* v,
                                         const void* g, const void* beta,
                                         const int32_t* cu_seqlens, int32_t max_segs, int64_t N,
                                         int32_t H, int32_t Dk, int32_t Dv, float scale,
                                         int32_t dtype, const float* initial_state,
                                         const void* do_, const float* dfinal_state, void* dq,
                                         void* dk, void* dv, void* dg, void* dbeta,
                                         float* d_initial_state, int32_t* flags, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return kda_backward(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, scale, dtype,
                      initial_state, do_, dfinal_state, dq, dk, dv, dg, dbeta, d_initial_state,
                      flags, workspace, workspace_bytes, false, nullptr, 0, stream);
}

pkv_status pkv_chunk_kda_varlen_backward_states(
    const void* q, const void* k, const void* v, const void* g, const void* beta,
    const int32_t* cu_seqlens, int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
    float scale, int32_t dtype, const float* initial_state, const void* do_,
    const float* dfinal_state, void* dq, void* dk, void* dv, void* dg, void* dbeta,
    float* d_initial_state, int32_t* flags, void* workspace, size_t workspace_bytes,
    const void* chunk_states, size_t chunk_states_bytes, void* stream) {
  return kda_backward(q, k, v, g, beta, cu_seqlens, max_segs, N, H, Dk, Dv, scale, dtype,
                      initial_state, do_, dfinal_state, dq, dk, dv, dg, dbeta, d_initial_state,
                      flags, workspace, workspace_bytes, true, chunk_states, chunk_states_bytes,
                      stream);
}

size_t pkv_chunk_kda_varlen_backward_states_workspace_size(int64_t N, int32_t H, int32_t Dk,
                                                           int32_t Dv, int32_t max_segs,
                                                           int32_t dtype) {
  if (pkv::kda_chunk_states_bytes(N, H, Dk, Dv, dtype, max_segs) == 0) return 0;
  return pkv::kda_chunk_bwd_workspace_bytes(N, H, Dk, Dv, dtype, max_segs, true);
}

size_t pkv_chunk_kda_varlen_backward_workspace_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                                    int32_t max_segs, int32_t dtype) {
  return pkv::kda_chunk_bwd_workspace_bytes(N, H, Dk, Dv, dtype, max_segs);
}

size_t pkv_chunk_kda_segment_ids_workspace_size(int64_t B, int64_t T, int32_t H, int32_t Dk,
                                                int32_t Dv, int32_t dtype) {
  if (B < 1 || T < 1 || B * T > kInt32Max) return 0;
  return pkv::kda_chunk_ids_workspace_bytes(B * T, H, Dk, Dv, dtype);
}

pkv_status pkv_chunk_kda_segment_ids(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta, const int32_t* segment_ids, int64_t B,
                                     int64_t T, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                     int32_t dtype, int32_t options, const float* initial_state,
                                     void* o, float* final_state, int32_t* flags, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr ||
      o == nullptr || segment_ids == nullptr)
    return PKV_ERR_INVALID_ARGUMENT;
  if (B < 1 || T < 1 || B > kInt32Max || T > kInt32Max || B * T > kInt32Max - 8192 || H < 1 ||
      H > 65536)
    return PKV_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype) || !supported_head_dim(Dk) || !supported_head_dim(Dv) ||
      (options & ~kKnownOptions) != 0)
    return PKV_ERR_UNSUPPORTED;
  const bool l2 = (options & PKV_OPT_QK_L2NORM) != 0;
  if (B * H > (int64_t(1) << 22)) return PKV_ERR_INVALID_ARGUMENT;
  for (const void* p : {q, k, v, g, static_cast<const void*>(o)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(beta) % elem_size(dtype) != 0 ||
      reinterpret_cast<uintptr_t>(final_state) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(initial_state) % 16 != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t N = B * T;
  const int64_t es = elem_size(dtype);
  const int64_t o_bytes = N * H * Dv * es;
  if (overlaps(o, o_bytes, q, N * H * Dk * es) || overlaps(o, o_bytes, k, N * H * Dk * es) ||
      overlaps(o, o_bytes, v, N * H * Dv * es) || overlaps(o, o_bytes, g, N * H * Dk * es) ||
      overlaps(o, o_bytes, beta, N * H * es) || overlaps(o, o_bytes, segment_ids, N * 4))
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t state_bytes = B * H * Dk * Dv * 4;
  if (initial_state != nullptr && final_state != nullptr &&
      overlaps(initial_state, state_bytes, final_state, state_bytes))
    return PKV_ERR_INVALID_ARGUMENT;
  const size_t need = pkv_chunk_kda_segment_ids_workspace_size(B, T, H, Dk, Dv, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
    return PKV_ERR_WORKSPACE;
  if (pkv::kda_chunk_supported(Dk, Dv, dtype))
    return from_hip(pkv::launch_kda_chunk_ids(q, k, v, g, beta, segment_ids, B, T, H, Dk, Dv,
                                              scale, l2, initial_state, o, final_state, flags,
                                              workspace, static_cast<hipStream_t>(stream)));
  return from_hip(pkv::launch_kda_serial_ids(q, k, v, g, beta, segment_ids, B, T, H, Dk, Dv,
                                             scale, dtype, l2, initial_state, o, final_state,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
