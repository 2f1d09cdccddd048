/*
 * pkv.h - C ABI of libpkv: packed (varlen) gated linear attention (KDA) forward
 * on AMD Instinct MI355X (gfx950).
 *
 * Three operations, following the problem statement of the pages:
 *
 *   pkv_segment_ids_to_cu_seqlens  segment ids [B, T] -> cu_seqlens [max_segs + 1]
 *       RFC-0025 "Support attention varlen and align loss", Design section 1
 *       (segment_ids -> cu_seqlens conversion); row-start rule from RFC-0026
 *       "Ling3 KDA varlen support", section 3.1.1 (API contract); doc(s) from
 *       "Drill: Sequence Packing from scratch", section "The math".
 *   pkv_short_conv_segmask         causal depthwise conv masked at segment changes
 *       RFC-0025, Design section 3 (ShortConvolution segment boundary mask).
 *   pkv_chunk_kda_varlen           S_t = diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
 *                                  o_t = scale * S_t^T q_t, S reset per segment
 *       RFC-0026, Background (KDA state leakage problem) and section 3.1.1;
 *       RFC-0025, Design sections 2 (batch flatten) and 4 (kernel wrappers).
 *
 * and the step before them in the data pipeline:
 *
 *   pkv_eod_to_segment_ids         EOD-separated token rows -> segment ids,
 *                                  positions and loss segment ids
 *       RFC-0025, Design section 6 (data pipeline alignment).
 *
 * and the kernel contract that takes segment ids directly:
 *
 *   pkv_chunk_kda_segment_ids      the recurrence with [B, T] segment_ids
 *       RFC-0026, section 3.1.1 (kernel contract) and Alternatives (Alt1).
 *
 * and the training step's reverse pass of the recurrence:
 *
 *   pkv_chunk_kda_varlen_backward  gradients of pkv_chunk_kda_varlen's outputs
 *       with respect to q, k, v, g, beta and the initial states
 *       RFC-0026, Background (the recurrence, differentiated) and section 3.3
 *       (the initial/final state arguments the wrapper carries).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer (HIP device memory or memory the
 *     GPU can address). Scalars are passed by value.
 *   - The caller allocates and owns every buffer, including the workspace. The
 *     library allocates nothing, keeps no state between calls and never
 *     synchronizes: work is enqueued on `stream` (a hipStream_t; NULL means the
 *     default stream) and results are valid once that stream has been
 *     synchronized by the caller.
 *   - Layouts are dense row-major with the last index contiguous.
 *   - Problems visible from the host (null pointers, bad sizes, unsupported
 *     shapes or dtypes, too small a workspace) return an error code
 *     synchronously, before anything is enqueued. Data-dependent conditions are
 *     reported through a device `flags` word (PKV_FLAG_*), the counterpart of
 *     the page's debug-callback warning: they never abort.
 *   - A failure of the HIP runtime to launch returns PKV_ERR_HIP.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_BF16 = 0, /* bfloat16 tensors, fp32 arithmetic inside */
    PKV_F32 = 1   /* float32 tensors, fp32 arithmetic inside */
} pkv_dtype;

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARGUMENT = 1, /* null pointer, size out of range, aliasing */
    PKV_ERR_UNSUPPORTED = 2,      /* head dim, conv width or dtype not built */
    PKV_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    PKV_ERR_HIP = 4               /* the HIP runtime refused a launch */
} pkv_status;

/* Bits of the device flags word. */
#define PKV_FLAG_OVERFLOW 1        /* more segments than max_segs: the last slot
                                      ends at B*T and merges the rest (leakage) */
#define PKV_FLAG_LEADING_PAD 2     /* padding before the first real token; it
                                      falls into segment 0 because cu[0] = 0 */
#define PKV_FLAG_BAD_CU_SEQLENS 4  /* chunk_kda_varlen saw cu[0] != 0, a
                                      decreasing pair or cu[i] > N; the outputs
                                      of the offending segments are undefined */
#define PKV_FLAG_GATE_RANGE 8      /* a chunked bf16 call met a 16-token
                                      sub-chunk whose gates sum below
                                      -120 ln 2 (about -83) on some key
                                      channel: its factor 2^(-sum log2 e) can
                                      leave the fp32 / bf16 range, so that
                                      (segment, head)'s results may be inf,
                                      NaN or inaccurate; the token-serial
                                      fp32 path is not limited this way */

/* Bits of the `options` argument of the recurrence's entry points. */
#define PKV_OPT_QK_L2NORM 1        /* RFC-0026 section 3.3's use_qk_l2norm_in_kernel:
                                      q and k are L2-normalised per (token, head)
                                      over Dk before the recurrence,
                                      x / sqrt(sum_d x_d^2 + 1e-6) in fp32 (the
                                      norm RFC-0025 Design section 5 places
                                      between the short conv and the kernel) */

/*
 * segment_ids -> cu_seqlens (FLA convention, fixed length max_segs + 1).
 *
 * segment_ids  int32 [B, T]: per row, 1-based increasing document ids; 0 is
 *              padding. The batch is treated as flattened to [B*T].
 * A boundary is a real (non-zero) token that starts a row or whose id differs
 * from the previous position. Segment i (0-based) starts at the (i+1)-th
 * boundary and ends where the next one starts, so padding between documents
 * joins the preceding segment; the last real segment ends one past the last
 * non-zero position. Slots beyond the number of segments are zero-length
 * (phantoms repeat the last end). If there are more segments than max_segs,
 * slot max_segs-1 ends at B*T and PKV_FLAG_OVERFLOW is set.
 *
 * Outputs (device, written in full by the call):
 *   cu_seqlens  int32 [max_segs + 1], cu_seqlens[0] = 0.
 *   token_seg   int32 [B*T] or NULL: doc(p) = i with cu[i] <= p < cu[i+1],
 *               -1 for p >= cu[max_segs].
 *   n_segs      int32 [1] or NULL: number of boundaries (may exceed max_segs).
 *   flags       int32 [1] or NULL: overwritten with PKV_FLAG_OVERFLOW |
 *               PKV_FLAG_LEADING_PAD as they apply.
 * Errors: PKV_ERR_INVALID_ARGUMENT if segment_ids or cu_seqlens is NULL,
 * B < 1, T < 1, B*T > INT32_MAX or max_segs < 1 or max_segs >= INT32_MAX.
 */
pkv_status pkv_segment_ids_to_cu_seqlens(const int32_t* segment_ids, int64_t B, int64_t T,
                                         int32_t max_segs, int32_t* cu_seqlens,
                                         int32_t* token_seg, int32_t* n_segs, int32_t* flags,
                                         void* stream);

/*
 * EOD-separated token rows -> segment ids, positions and loss segment ids
 * (RFC-0025 "Support attention varlen and align loss", Design section 6, data
 * pipeline alignment:
 * an EOD token keeps the id of the document it ends and a new segment starts
 * right after it; positions restart at 0 after an EOD; EOD positions carry no
 * loss). Every row is an independent packed sample with ids from 1:
 *   segment_ids[b,t]      = 1 + #{u < t : tokens[b,u] == eod_id}
 *   positions[b,t]        = t - (1 + last u < t with tokens[b,u] == eod_id),
 *                           or t when there is none
 *   loss_segment_ids[b,t] = 0 where tokens[b,t] == eod_id, else segment_ids[b,t]
 * There is no padding (segment_ids is never 0), so the result feeds
 * pkv_segment_ids_to_cu_seqlens directly.
 *
 * tokens            int32 [B, T] (device).
 * segment_ids       int32 [B, T] (device), written in full.
 * positions         int32 [B, T] or NULL.
 * loss_segment_ids  int32 [B, T] or NULL.
 * Errors: PKV_ERR_INVALID_ARGUMENT if tokens or segment_ids is NULL, B < 1,
 * T < 1, B*T > INT32_MAX, or an output overlaps the tokens or another output.
 */
pkv_status pkv_eod_to_segment_ids(const int32_t* tokens, int64_t B, int64_t T, int32_t eod_id,
                                  int32_t* segment_ids, int32_t* positions,
                                  int32_t* loss_segment_ids, void* stream);

/*
 * Segment-masked short causal depthwise convolution.
 *
 * y[b,t,f] = sum_{k<Kc} w[f,k] * x[b,t-k,f] * [t-k >= 0] * [seg[b,t-k] == seg[b,t]]
 *
 * x            [B, T, F] in `dtype`.
 * w            float32 [F, Kc]; w[f, 0] weights the current token (the page's
 *              kernel[k] for channel f).
 * segment_ids  int32 [B, T] or NULL (NULL: plain causal conv, no mask).
 * y            [B, T, F] in `dtype`, must not overlap x. Accumulation is fp32
 *              with one rounding to `dtype`. No bias, no activation.
 * Errors: PKV_ERR_INVALID_ARGUMENT for NULL x/w/y, x == y, B, T or F < 1 or
 * B*T*F > INT64 range of the kernel (2^62); PKV_ERR_UNSUPPORTED for Kc outside
 * [1, 8] or an unknown dtype.
 */
pkv_status pkv_short_conv_segmask(const void* x, const float* w, const int32_t* segment_ids,
                                  void* y, int64_t B, int64_t T, int64_t F, int32_t Kc,
                                  int32_t dtype, void* stream);

/*
 * Bytes of device workspace pkv_chunk_kda_varlen needs for these sizes
 * (0 means no workspace is needed and NULL may be passed). Host-only: no HIP
 * call. With bf16 and Dk, Dv in {64, 128} it holds the call's work plan: the
 * (segment, chunk range) runs in the order they are processed, longest first,
 * and, for segments long enough to be cut into several runs so that one
 * document does not set the length of the whole launch (more than 8192
 * tokens; where a segment is cut depends on its own length only), the state
 * and the per-channel decay product of every run but the last (fp32, about
 * N / 4096 runs x H heads x Dk x (Dv + 1) x 4 bytes, i.e. 1/16 of one
 * [N, H, Dk] bf16 tensor at Dv = 128).
 */
size_t pkv_chunk_kda_varlen_workspace_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                           int32_t max_segs, int32_t dtype);

/*
 * Packed gated linear-attention recurrence with per-segment reset.
 *
 * For every segment i = [cu[i], cu[i+1]) and head h, from S = initial_state[i, h]
 * (0 when initial_state is NULL):
 *   S_t = diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T      (S is [Dk, Dv], fp32)
 *   o_t = scale * S_t^T q_t                              (readout after the update)
 * final_state[i, h] = S after the segment's last token (the initial state, or 0,
 * for empty slots).
 * Positions p >= cu[max_segs] get o = 0.
 *
 * q, k, g     [1, N, H, Dk] in `dtype` (the batch flattened to one row, B*T = N).
 * v           [1, N, H, Dv] in `dtype`.
 * beta        [1, N, H] in `dtype`.
 * cu_seqlens  int32 [max_segs + 1] or NULL. NULL means one segment [0, N) and
 *             max_segs is taken as 1. Expected: cu[0] = 0, non-decreasing,
 *             cu[max_segs] <= N; a violation sets PKV_FLAG_BAD_CU_SEQLENS.
 * options     0 or PKV_OPT_QK_L2NORM (q and k normalised inside the call; the
 *             caller's tensors are not modified).
 * initial_state float32 [max_segs, H, Dk, Dv] or NULL (RFC-0026 section 3.3's
 *             wrapper argument, one state per segment slot); must not overlap
 *             final_state.
 * o           [1, N, H, Dv] in `dtype`; must not overlap the inputs.
 *             q, k, v, g, o, initial_state and final_state must be 16-byte
 *             aligned, beta aligned to its element size.
 * final_state float32 [max_segs, H, Dk, Dv] or NULL (not written).
 * flags       int32 [1] or NULL; PKV_FLAG_BAD_CU_SEQLENS and, on the chunked
 *             bf16 path, PKV_FLAG_GATE_RANGE are OR-ed in.
 * workspace   device buffer of at least pkv_chunk_kda_varlen_workspace_size()
 *             bytes, 16-byte aligned (NULL allowed when that size is 0);
 *             contents are scratch, overwritten by every call, so calls that
 *             share a workspace must be ordered on one stream. After the
 *             call its int32 words 0 and 1 hold the number of runs and of
 *             runs whose state was saved for the next piece (diagnostics).
 * Supported: Dk, Dv in {32, 64, 128}. The chunked bf16 path bounds exponents
 * per 16-token sub-chunk: gates whose sum over 16 consecutive tokens of a
 * segment falls below about -83 on some key channel are reported with
 * PKV_FLAG_GATE_RANGE; large positive g (outside the recurrence's decay
 * range) may lose accuracy unreported.
 * Errors: PKV_ERR_INVALID_ARGUMENT for NULL tensors, N < 1, N > INT32_MAX,
 * H < 1, max_segs < 1 (with cu_seqlens), max_segs * H > 2^22, a misaligned
 * tensor or o aliasing an input; PKV_ERR_UNSUPPORTED for other Dk/Dv, dtype or
 * an unknown options bit; PKV_ERR_WORKSPACE if the workspace is too small or
 * not 16-byte aligned.
 */
pkv_status pkv_chunk_kda_varlen(const void* q, const void* k, const void* v, const void* g,
                                const void* beta, const int32_t* cu_seqlens, int32_t max_segs,
                                int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                int32_t dtype, int32_t options, const float* initial_state,
                                void* o, float* final_state, int32_t* flags, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Bytes of the per-chunk state buffer of pkv_chunk_kda_varlen_states and
 * pkv_chunk_kda_varlen_backward_states: bf16 [ceil(N / 64) + max_segs, H, Dk, Dv]
 * (max_segs taken as 1 when cu_seqlens will be NULL). 0 when the shape has no
 * chunked path (dtype other than PKV_BF16, Dk or Dv not in {64, 128}); those
 * calls then return PKV_ERR_UNSUPPORTED.
 */
size_t pkv_chunk_kda_states_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv, int32_t max_segs,
                                 int32_t dtype);

/*
 * pkv_chunk_kda_varlen that also keeps, for the reverse pass, the state S before
 * every 64-token chunk (RFC-0026 Background recurrence; chunks aligned to the
 * segment starts as in the chunked forward pass). A training step can then run
 * pkv_chunk_kda_varlen_backward_states, which reads these states instead of
 * recomputing them from k, g, v and beta.
 *
 * Arguments, results and errors are those of pkv_chunk_kda_varlen, plus:
 * chunk_states  device buffer of at least pkv_chunk_kda_states_size() bytes,
 *               16-byte aligned, not overlapping any other argument. Chunk c of
 *               slot i (tokens cu[i] + 64 c ...) is entry b_i + c, where b_i is
 *               the number of chunks (ceil(length / 64), 0 for empty slots) of
 *               the slots before i; entry [b_i + c, h] holds head h's S
 *               (rows d, columns e) as bf16 row-major [Dk][Dv]. The
 *               zero state before a segment's first chunk is not written when
 *               initial_state is NULL; entries past the last chunk are left
 *               alone. Only the bf16 chunked path (Dk, Dv in {64, 128}).
 * Errors: as pkv_chunk_kda_varlen; PKV_ERR_UNSUPPORTED for a shape without the
 * chunked path; PKV_ERR_INVALID_ARGUMENT for a missing, small, misaligned or
 * overlapping chunk_states.
 */
pkv_status pkv_chunk_kda_varlen_states(const void* q, const void* k, const void* v, const void* g,
                                       const void* beta, const int32_t* cu_seqlens, int32_t max_segs,
                                       int64_t N, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                       int32_t dtype, int32_t options, const float* initial_state,
                                       void* o, float* final_state, int32_t* flags, void* workspace,
                                       size_t workspace_bytes, void* chunk_states,
                                       size_t chunk_states_bytes, void* stream);

/*
 * pkv_chunk_kda_varlen for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Arguments, results and errors are those of pkv_chunk_kda_varlen
 * without the workspace: the chunk path's scratch (work plan, queue counters,
 * states of the pieces of cut segments) lives in a fixed array of
 * PKV_NOALLOC_SCRATCH_BYTES in the library's device memory, one copy per GPU
 * the library runs on, held until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's copy of the array.
 * Every call on one GPU shares the array, so calls that overlap on one GPU
 * (other streams, other threads) race: order them. The array needs no
 * clearing between calls (every call rewrites what it reads).
 * Errors: as pkv_chunk_kda_varlen; PKV_ERR_WORKSPACE when
 * pkv_chunk_kda_varlen_workspace_size() for these sizes exceeds
 * PKV_NOALLOC_SCRATCH_BYTES (e.g. N = 131072, H = 32, Dk = Dv = 128 fits;
 * the limit is reached at about N = 190000 tokens for that shape);
 * PKV_ERR_HIP if the array's address cannot be found.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
pkv_status pkv_chunk_kda_varlen_noalloc(const void* q, const void* k, const void* v,
                                        const void* g, const void* beta,
                                        const int32_t* cu_seqlens, int32_t max_segs, int64_t N,
                                        int32_t H, int32_t Dk, int32_t Dv, float scale,
                                        int32_t dtype, int32_t options, const float* initial_state,
                                        void* o, float* final_state, int32_t* flags, void* stream);

/*
 * Packed KDA straight from [B, T] segment ids (RFC-0026 section 3.1.1's
 * kernel contract), with no cu_seqlens round trip and no phantom slots.
 *
 * For every row b and head h the recurrence of pkv_chunk_kda_varlen runs over
 * the row. Id 0 is padding, which the kernel ignores (RFC-0026 section 3.4):
 * a padding position leaves the state as it is and gets o = 0. A real
 * position whose id differs from the previous position's
 * (segment_ids[b, t] != segment_ids[b, t-1]) starts a new segment from zero,
 * except the row's first real position, which starts the row's first segment
 * from initial_state[b, h] (0 when initial_state is NULL). final_state[b, h]
 * is the state after the row's last real position (initial_state[b, h], or 0,
 * for a row of padding only; section 3.3's per-row shapes). Rows never share
 * state.
 *
 * q, k, g     [B, T, H, Dk]; v [B, T, H, Dv]; beta [B, T, H]; o [B, T, H, Dv]
 *             (one dtype); segment_ids int32 [B, T]; options as for
 *             pkv_chunk_kda_varlen.
 * initial_state, final_state  float32 [B, H, Dk, Dv] or NULL; must not overlap.
 * flags       int32 [1] or NULL; PKV_FLAG_GATE_RANGE is OR-ed in as for
 *             pkv_chunk_kda_varlen.
 * workspace   at least pkv_chunk_kda_segment_ids_workspace_size() bytes,
 *             16-byte aligned; scratch, as for pkv_chunk_kda_varlen (the
 *             segment starts found in the ids are kept there).
 * Errors: as pkv_chunk_kda_varlen, with B*T in place of N (B*T must not
 * exceed INT32_MAX - 8192) and no max_segs.
 */
size_t pkv_chunk_kda_segment_ids_workspace_size(int64_t B, int64_t T, int32_t H, int32_t Dk,
                                                int32_t Dv, int32_t dtype);
pkv_status pkv_chunk_kda_segment_ids(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta, const int32_t* segment_ids, int64_t B,
                                     int64_t T, int32_t H, int32_t Dk, int32_t Dv, float scale,
                                     int32_t dtype, int32_t options, const float* initial_state,
                                     void* o, float* final_state, int32_t* flags, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Reverse pass of pkv_chunk_kda_varlen: given do = dL/do and (optionally)
 * dfinal_state = dL/dfinal_state, the gradients of L with respect to every
 * input of the forward call on the same q, k, v, g, beta, cu_seqlens and
 * initial_state. Per segment and head, with S_t the forward states:
 *   dS (after the last token) = dfinal_state (0 when NULL)
 *   dS_t   = exp(g_{t+1}) * dS_{t+1} + scale * q_t do_t^T   (rows scaled)
 *   dq_t   = scale * S_t do_t          dk_t = beta_t * dS_t v_t
 *   dv_t   = beta_t * dS_t^T k_t       dbeta_t = k_t . (dS_t v_t)
 *   dg_t   = sum over the segment's u >= t of (q_u * dq_u - k_u * dk_u)
 *            + sum_e dfinal_state[:, e] * S_last[:, e]   (elementwise in Dk)
 *   d_initial_state = exp(g_first) * dS_first (dfinal_state for empty slots).
 * Positions p >= cu[max_segs] get zero gradients.
 *
 * q, k, g, v, beta, cu_seqlens, max_segs, N, H, Dk, Dv, scale, dtype and
 *             initial_state: exactly as passed to pkv_chunk_kda_varlen.
 * do          [1, N, H, Dv] in `dtype`.
 * dfinal_state float32 [max_segs, H, Dk, Dv] or NULL (zero cotangent).
 * dq, dk, dg  [1, N, H, Dk] in `dtype`; dv [1, N, H, Dv]; dbeta [1, N, H]:
 *             outputs, all written, none overlapping an input or each other.
 * d_initial_state float32 [max_segs, H, Dk, Dv] or NULL (not written).
 * flags       int32 [1] or NULL; PKV_FLAG_BAD_CU_SEQLENS is OR-ed in (the
 *             gradients of an invalid slot are then left unwritten), and on
 *             the chunked path PKV_FLAG_GATE_RANGE as in the forward call.
 * This call recomputes the states (pkv_chunk_kda_varlen_backward_states reads
 * them from the forward call instead). For bf16 with Dk, Dv in {64, 128} it is
 * chunked: the workspace holds
 * the work plan (chunk, piece and summary offsets per slot, the pieces in
 * longest-first order with a record of each, a work counter), the bf16 state at every 64-token
 * chunk boundary (the adjoint dL/dS is carried in registers while the
 * chunks are walked backwards), and, for segments long enough to be cut into
 * pieces, fp32 piece summaries (end state and decay product per piece and
 * role), and per (segment slot, head, key channel) an fp32 final-state term of
 * the gate gradient, all written and read within the call (scratch: calls sharing a
 * workspace must be ordered on one stream); see
 * pkv_chunk_kda_varlen_backward_workspace_size() for its size. Every other
 * shape runs token-serially and needs no workspace (size
 * 0, NULL allowed): between its two sweeps the dg and dk buffers hold fp32
 * intermediates. Alignment rules as for the forward call, and the workspace
 * must be 256-byte aligned. The arithmetic is fp32 (bf16 tensors are read
 * exactly; the chunked path rounds MFMA operands and the saved states to
 * bf16, like the forward's chunked path).
 * Supported: Dk, Dv in {32, 64, 128}. Errors: as pkv_chunk_kda_varlen, with
 * PKV_ERR_INVALID_ARGUMENT also for a NULL do or gradient output, or outputs
 * (or the workspace) that overlap an input or one another; PKV_ERR_WORKSPACE
 * when the workspace is needed and missing, too small or misaligned.
 */
size_t pkv_chunk_kda_varlen_backward_workspace_size(int64_t N, int32_t H, int32_t Dk, int32_t Dv,
                                                    int32_t max_segs, int32_t dtype);
pkv_status pkv_chunk_kda_varlen_backward(const void* q, const void* k, const void* v,
                                         const void* g, const void* beta,
                                         const int32_t* cu_seqlens, int32_t max_segs, int64_t N,
                                         int32_t H, int32_t Dk, int32_t Dv, float scale,
                                         int32_t dtype, const float* initial_state,
                                         const void* do_, const float* dfinal_state, void* dq,
                                         void* dk, void* dv, void* dg, void* dbeta,
                                         float* d_initial_state, int32_t* flags, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * pkv_chunk_kda_varlen_backward with the states the forward call saved
 * (pkv_chunk_kda_varlen_states on the same q, k, v, g, beta, cu_seqlens,
 * max_segs, scale and initial_state): the states before every chunk are read
 * from chunk_states instead of being recomputed, so the call reads k, g, v and
 * beta once instead of twice and keeps no states of its own. With dfinal_state
 * given, each segment's last chunk is stepped once more from its saved state to
 * reach the final state the gate gradient needs.
 *
 * Arguments, results and errors are those of pkv_chunk_kda_varlen_backward,
 * plus chunk_states (at least pkv_chunk_kda_states_size() bytes, 16-byte
 * aligned, read only, not overlapping an output or the workspace). The
 * workspace needs pkv_chunk_kda_varlen_backward_states_workspace_size() bytes.
 * Results equal pkv_chunk_kda_varlen_backward's up to the rounding of the
 * states (both round them to bf16; the forward and reverse passes sum their
 * updates in different orders). PKV_ERR_UNSUPPORTED for a shape without the
 * chunked path.
 */
size_t pkv_chunk_kda_varlen_backward_states_workspace_size(int64_t N, int32_t H, int32_t Dk,
                                                           int32_t Dv, int32_t max_segs,
                                                           int32_t dtype);
pkv_status pkv_chunk_kda_varlen_backward_states(
    const void* q, const void* k, const void* v, const void* g, const void* beta,
    const int32_t* cu_seqlens, int32_t max_segs, int64_t N, int32_t H, int32_t Dk, int32_t Dv,
    float scale, int32_t dtype, const float* initial_state, const void* do_,
    const float* dfinal_state, void* dq, void* dk, void* dv, void* dg, void* dbeta,
    float* d_initial_state, int32_t* flags, void* workspace, size_t workspace_bytes,
    const void* chunk_states, size_t chunk_states_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* pkv_status_string(int32_t status);

/* ABI version of this header (bumped on any signature change). */
#define PKV_ABI_VERSION 6
int32_t pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
