/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The library computes O = softmax(scale * Q K^T) V and the row log-sum-exp
 * LSE = ln sum_j exp(scale * q . k_j) with the online-softmax recurrence: a
 * running max m, a running denominator l and an unnormalised output o per query
 * row are updated key tile by key tile, the old state is rescaled by
 * exp(m_old - m_new) when the max grows, and the result is o / l
 * ('Online Softmax -- the mathematical heart of FlashAttention', sections 4-5;
 * 'Online Softmax' (research-hub concept page), "Key math").  The N x Nk score
 * matrix never reaches device memory.
 *
 * Conventions shared by every entry point
 *   Memory     All tensor pointers are DEVICE pointers, row-major, contiguous:
 *              Q, O [B, H, N, d]; K, V [B, H, Nk, d]; LSE [B, H, N] (fp32).
 *              Q, K, V and O must be 16-byte aligned, and one (b, h) slice of
 *              Q/O or K/V must stay below 2 GiB (FA_ERR_INVALID_ARG otherwise).
 *   Ownership  The caller allocates and owns every buffer; the library
 *              allocates nothing and keeps no pointer after a call returns.
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Calls
 *              are asynchronous on that stream; the status only reports
 *              argument checks and launch errors.  Calls are reentrant.
 *   Masking    key_lens (device int32[B] or NULL): keys j >= key_lens[b] are
 *              invisible to every query of batch b; values outside [0, Nk] are
 *              clamped on the device.  causal = 1 hides key j from query i when
 *              j > i + (Nk - N) (queries are the last N positions; j > i when
 *              N == Nk).  The two combine by AND.
 *   Empty rows A query row with no visible key gets O = 0 and LSE = -inf,
 *              never NaN ('Online Softmax & FlashAttention' (interview lesson),
 *              Step 1: the fully masked row keeps m = -inf, l = 0).
 *   Errors     Every argument is checked on the host before any launch; on an
 *              error nothing is launched.  The library never aborts.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* NULL / misaligned pointer, negative size, bad flag, too-small workspace */
    FA_ERR_UNSUPPORTED = 2,   /* valid request the library has no kernel for (e.g. bf16 with d = 96) */
    FA_ERR_HIP = 3,           /* the HIP runtime reported an error at launch */
    FA_ERR_SCRATCH_LIMIT = 4  /* the request needs more than the library's fixed scratch
                                 (fa_decode_splitkv_noalloc only) */
} fa_status;

typedef enum fa_dtype {
    FA_F32 = 0,               /* Q, K, V, O are fp32; fp32 arithmetic throughout */
    FA_BF16 = 1               /* Q, K, V, O are bf16; fp32 accumulation, bf16 MFMA operands */
} fa_dtype;

/*
 * Prefill attention forward.
 *   Computes, for every b < B, h < H, i < N:
 *     O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) V[b,h,j,:]
 *     LSE[b,h,i] = ln sum_j exp(scale * Q[b,h,i,:] . K[b,h,j,:])
 *   over the keys j visible to (b, i) (see Masking), one Q tile per
 *   workgroup, K/V tiles streamed through LDS ('Online Softmax &
 *   FlashAttention', Step 3: the outer loop runs over independent Q blocks,
 *   the inner one over K/V; Step 4: causal tiles above the diagonal are
 *   skipped, tiles on it are masked).
 *   Q, K, V, O: element type `dtype`; LSE: fp32.
 *   scale: finite and > 0 (usually 1/sqrt(d)); scale <= 0 gives
 *   FA_ERR_UNSUPPORTED, a non-finite scale FA_ERR_INVALID_ARG.
 *   causal: 0 or 1.  key_lens: device int32[B] or NULL.
 *   Supported: FA_BF16 with d in {64, 128}; FA_F32 with 1 <= d <= 256.
 *   B*H*N == 0: nothing to do, FA_OK.  Nk == 0: every row fully masked.
 */
fa_status fa_forward(const void *Q, const void *K, const void *V, void *O, float *LSE,
                     int B, int H, int N, int Nk, int d, float scale, int causal,
                     const int32_t *key_lens, fa_dtype dtype, void *stream);

/*
 * Bytes of device workspace fa_decode_splitkv needs:
 * B * H * num_splits * (d + 2) * 4 (a running max, a denominator and an
 * unnormalised output row in fp32 for every split).  Returns 0 for negative
 * arguments or num_splits < 1.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * One-query decode with the key range split into chunks (Flash-Decoding,
 * 'Online Softmax & FlashAttention', Step 5).
 *   Q, O: [B, H, 1, d]; K, V: [B, H, Nk, d]; LSE: [B, H, 1] fp32.
 *   The visible keys [0, kl) of batch b, kl = clamp(key_lens[b], 0, Nk) (Nk
 *   when key_lens is NULL), are cut into num_splits consecutive chunks of
 *   ceil(kl / num_splits) keys (trailing chunks may be short or empty).  One
 *   pass computes each chunk's partial state (m_c, l_c, o_c); a second pass
 *   merges the partials with the associative (m, l) merge
 *   m = max(m1, m2), l = exp(m1 - m) l1 + exp(m2 - m) l2 (o alike), where two
 *   -inf sides merge to (-inf, 0) ('Online Softmax & FlashAttention', Step 1),
 *   and writes O = o / l and LSE = m + ln l.  The result equals fa_forward
 *   with N = 1 and causal = 0 up to rounding.
 *   workspace: device memory of at least fa_decode_workspace_bytes(B, H, d,
 *   num_splits) bytes, 16-byte aligned, owned by the caller; its contents on
 *   entry do not matter and are overwritten.  Two calls that share a
 *   workspace must not overlap in time (same stream, or synchronised).
 *   Supported: FA_BF16 with d in {64, 128}, FA_F32 with 1 <= d <= 256 (the
 *   range of the fp32 forward); 1 <= num_splits <= 256.
 */
fa_status fa_decode_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE,
                            int B, int H, int Nk, int d, float scale,
                            const int32_t *key_lens, int num_splits,
                            void *workspace, size_t workspace_bytes,
                            fa_dtype dtype, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as fa_decode_splitkv, same arguments minus the workspace, with the
 * partial states kept in a fixed scratch array that the library holds on each
 * GPU it runs on until the process ends (fa_decode_scratch_bytes() bytes,
 * 32 MiB).  This call allocates nothing.
 *   Requests needing more than that (fa_decode_workspace_bytes(B, H, d,
 *   num_splits) > fa_decode_scratch_bytes()) return FA_ERR_SCRATCH_LIMIT
 *   before anything is launched; the other argument checks and supported
 *   cases are those of fa_decode_splitkv.  Every record of the scratch that a
 *   call reads is first written by that call (nothing needs to start at
 *   zero), and the array keeps the last call's partials afterwards.
 *   All calls on one GPU share that GPU's array: two calls that overlap in
 *   time on the same GPU (different streams, not synchronised) race and give
 *   undefined results.  Calls on different GPUs are independent.
 */
fa_status fa_decode_splitkv_noalloc(const void *Q, const void *K, const void *V, void *O,
                                    float *LSE, int B, int H, int Nk, int d, float scale,
                                    const int32_t *key_lens, int num_splits, fa_dtype dtype,
                                    void *stream);

/* Size in bytes of the fixed per-GPU scratch fa_decode_splitkv_noalloc uses. */
size_t fa_decode_scratch_bytes(void);

/*
 * Bytes of device workspace fa_softmax needs for a [rows, cols] matrix of
 * `dtype`: 0 when every row fits one workgroup's chunk (no workspace is
 * read), else 8 bytes per (row, chunk) for the chunk statistics.  Returns 0
 * for invalid arguments.
 */
size_t fa_softmax_workspace_bytes(int64_t rows, int64_t cols, fa_dtype dtype);

/*
 * Row softmax and log-sum-exp of a matrix, streamed for rows of any width
 * ('Online Softmax' (research-hub concept page), "Why it matters": the same
 * running (max, sum) pair lets softmax stream rows too wide for on-chip
 * memory; 'Online softmax in attention -- why and how', the textbook
 * two-pass softmax and its one-pass online form).
 *   For every row r < rows, over the entries x = X[r, 0:cols]:
 *     m = max_j x_j,  l = sum_j exp(x_j - m),
 *     Y[r, j] = exp(x_j - m) / l,  LSE[r] = m + ln l.
 *   -inf entries are masked (they get y = 0); a row with no finite entry, or
 *   cols == 0, gives Y = 0 and LSE = -inf, never NaN.  Entries must be finite
 *   or -inf (+inf or NaN give unspecified values in that row).
 *   X, Y: device, row-major [rows, cols], element type `dtype` (fp32, or bf16
 *   rounded to nearest even on output), 16-byte aligned base; rows may start
 *   anywhere.  Y == X (in place) is allowed, other overlap is not.  Y may be
 *   NULL: only LSE is computed and X is read once.
 *   LSE: device fp32 [rows], 4-byte aligned.
 *   X is read once when a row fits one workgroup (8192 elements) and, out of
 *   place, for rows of up to 2^21 fp32 / 2^22 bf16 elements: the workgroups
 *   of a row's 64 KiB chunks keep their chunk in registers, exchange their
 *   (m, l) pairs through the workspace and merge them with the associative
 *   merge of fa_decode_splitkv in a fixed order.  LSE-only calls, in-place
 *   calls and wider rows take two passes: one (m, l) per chunk to the
 *   workspace, then the merge and the normalisation.  Results are
 *   deterministic for a given call form.
 *   workspace: device, 16-byte aligned, at least
 *   fa_softmax_workspace_bytes(rows, cols, dtype) bytes (may be NULL when
 *   that is 0); contents on entry do not matter.  Calls sharing a workspace
 *   must not overlap in time.
 *   Limits: cols <= 2^30, rows * cols <= 2^46; rows == 0: FA_OK, no launch.
 */
fa_status fa_softmax(const void *X, void *Y, float *LSE, int64_t rows, int64_t cols,
                     fa_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace fa_forward_v1 needs: fp32 O, m and l of every
 * query row, B * H * N * (d + 2) * 4.  Returns 0 for negative arguments.
 */
size_t fa_forward_v1_workspace_bytes(int B, int H, int N, int d);

/*
 * The attention forward of fa_forward computed in the FlashAttention V1 loop
 * order, kept as an ablation ('Online Softmax & FlashAttention' (interview
 * lesson), Step 2): key/value blocks outside, query blocks inside, one
 * workgroup per (b, h); for every (key block, query block) pair the
 * normalised O and the row statistics (m, l) are read from the workspace,
 * merged with the block (O_new = (l_old e^(m_old - m_new) O_old + P V) / l_new)
 * and written back.  Same arguments, masking and outputs as fa_forward (O and
 * LSE agree with it up to rounding), plus the workspace: device, 16-byte
 * aligned, at least fa_forward_v1_workspace_bytes(B, H, N, d) bytes; its
 * contents on entry do not matter.
 *   Supported: FA_BF16 with d in {64, 128}.
 */
fa_status fa_forward_v1(const void *Q, const void *K, const void *V, void *O, float *LSE,
                        int B, int H, int N, int Nk, int d, float scale, int causal,
                        const int32_t *key_lens, void *workspace, size_t workspace_bytes,
                        fa_dtype dtype, void *stream);

/*
 * Bytes of device workspace fa_backward needs: two fp32 values per query row,
 * each head's rows padded to a multiple of 64 (8 * B * H * ceil(N / 64) * 64).
 * Returns 0 for negative arguments.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N);

/*
 * Attention backward: the gradients of L = sum dO . O with respect to Q, K
 * and V for O = fa_forward(Q, K, V) with the same scale, causal flag and
 * key_lens, recomputing the probabilities from the forward's saved LSE
 * instead of storing them ('Online softmax in attention -- why and how',
 * "Where this is heading": backward recomputes the scores from the cached
 * row statistics):
 *     P_ij = exp(scale q_i . k_j - LSE_i) over the visible keys (0 otherwise),
 *     D_i = dO_i . O_i,  dS_ij = P_ij (dO_i . v_j - D_i),
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *     dV_j = sum_i P_ij dO_i.
 *   Q, O, dO, dQ: [B, H, N, d]; K, V, dK, dV: [B, H, Nk, d], device, element
 *   type `dtype`, 16-byte aligned; LSE: fp32 [B, H, N] as written by fa_forward (-inf for a
 *   row with no visible key: its dQ row is 0).  Keys no query sees get
 *   dK = dV = 0.  dQ, dK, dV are written, never accumulated into.
 *   workspace: device, 16-byte aligned, at least fa_backward_workspace_bytes
 *   (B, H, N) bytes; contents on entry do not matter.  Calls sharing a
 *   workspace must not overlap in time.
 *   Supported: FA_BF16 with d in {64, 128} (bf16 MFMA operands, fp32
 *   accumulation) and FA_F32 with 1 <= d <= 256 (fp32 throughout, the range
 *   of the fp32 forward); anything else gives FA_ERR_UNSUPPORTED.  scale
 *   finite and > 0.
 */
fa_status fa_backward(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                      const float *LSE, void *dQ, void *dK, void *dV,
                      int B, int H, int N, int Nk, int d, float scale, int causal,
                      const int32_t *key_lens, void *workspace, size_t workspace_bytes,
                      fa_dtype dtype, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *fa_status_str(fa_status status);

/* Text of the last HIP error this thread's calls saw ("" if none). */
const char *fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
