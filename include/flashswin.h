/*
 * flashswin.h -- C ABI of the FlashSwin window-attention library for AMD MI355X (gfx950).
 *
 * The operation ([FS] = the paper card "FLASHSWIN: Unlocking Large Windows and Dense Tokens in
 * Swin Vision Transformers with Memory Efficient Attention"):
 *
 *   For every M x M window of a token grid, exact softmax attention softmax(q~ k~^T / sqrt(d)) v
 *   computed without materialising the (M^2 x M^2) score matrix, so per-window memory is O(M^2)
 *   ([FS] Abstract).  Swin's additive relative-position bias is not used; position enters as
 *   window-local 2D RoPE applied to Q and K ([FS] Abstract; Figure 1(B)).  The RoPE frequencies
 *   theta are learnable ([FS] Figure S4 parameterises them as theta = exp(omega); that chain rule
 *   is the caller's, this library returns d(loss)/d(theta)).
 *
 * Conventions (readings of what the pages leave open):
 *   - Tensors are in token-grid layout [B, Hg, Wg, heads, d], contiguous, element (b,y,x,h,i) at
 *     offset (((b*Hg + y)*Wg + x)*heads + h)*d + i.
 *   - Windows tile the grid after Swin's cyclic shift: shifted-frame row Y holds grid row
 *     (Y + shift) mod Hg (likewise columns).  Window (wy, wx) holds shifted-frame rows
 *     wy*M .. wy*M+M-1; the in-window position (r, c) is in that shifted frame.
 *   - With shift > 0, keys and queries attend only within the same Swin region: shifted-frame rows
 *     split into [0, Hg-M), [Hg-M, Hg-shift), [Hg-shift, Hg) (likewise columns); pairs from
 *     different regions are excluded (weight exactly zero).  shift == 0 means no roll, no mask.
 *   - RoPE: channels [0, d/2) rotate pairs (2j, 2j+1) by theta_row[h, j] * r, channels [d/2, d)
 *     rotate pairs (d/2+2j, d/2+2j+1) by theta_col[h, j] * c, j < d/4, as
 *     (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi), identically for Q and K.
 *   - lse[b, y, x, h] is the natural log of sum over live keys of exp(q~ . k~ / sqrt(d)).
 *
 * Execution: every call validates its arguments on the host first (no HIP call is made when a
 * check fails), then enqueues kernels on `hip_stream` (a hipStream_t; NULL = the default stream)
 * and returns without waiting.  A kernel fault surfaces at the caller's next synchronisation.
 * The library allocates no device memory and keeps no global state, apart from the fixed scratch
 * array behind flashswin_wattn_bwd_noalloc (and the per-device lookup of its address); calls are
 * thread-safe, except for overlapping flashswin_wattn_bwd_noalloc calls on one GPU (see there).
 * All device buffers are owned by the caller and must stay alive until the stream reaches them.
 */
#ifndef FLASHSWIN_H_
#define FLASHSWIN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  FSW_OK = 0,
  FSW_ERR_INVALID_ARG = 1, /* shape / pointer / alignment / shift / dtype rule violated */
  FSW_ERR_UNSUPPORTED = 2, /* valid but not implemented here (d, M, dtype combination) */
  FSW_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than flashswin_wattn_bwd_workspace_size() */
  FSW_ERR_HIP = 4,         /* a HIP launch reported an error */
  FSW_ERR_SCRATCH = 5      /* flashswin_wattn_bwd_noalloc: the shape needs more than FLASHSWIN_SCRATCH_BYTES */
} fsw_status;

/* Element type of q, k, v, out, dout, dq, dk, dv.  theta, lse and dtheta are always float32. */
typedef enum { FSW_F32 = 0, FSW_BF16 = 1 } fsw_dtype;

/*
 * Forward window attention ([FS] Abstract; Figure 1(B)).
 *
 *   q, k, v      device, [B, Hg, Wg, heads, d] of `dtype`, 16-byte aligned.
 *   theta_row,
 *   theta_col    device, float32 [heads, d/4], 4-byte aligned (angular frequency, rad per token).
 *   out          device, [B, Hg, Wg, heads, d] of `dtype`, 16-byte aligned; overwritten.
 *   lse          device, float32 [B, Hg, Wg, heads], 4-byte aligned, overwritten; or NULL when the
 *                caller does not need it (inference).
 *   out and lse may not share a byte with q, k, v, theta_row, theta_col or each other
 *   (FSW_ERR_INVALID_ARG); the inputs may share memory.
 *   B >= 0 (B == 0 returns FSW_OK with nothing enqueued); Hg, Wg >= 1; 1 <= M <= 128;
 *   0 <= shift < M; heads >= 1; d in {8, 16, 32, 64}; dtype FSW_F32 or FSW_BF16.
 *   A grid whose sides M does not divide is taken as padded to the next multiples of M, as Swin pads
 *   its feature map before the shift (the pages do not say): the shift, the windows and the Swin
 *   regions are those of the padded grid, and the added tokens are absent, no key of any query and
 *   no output.  (A caller that wants Swin's zero-valued padding tokens as keys pads q, k, v itself.)
 *   Padded grids run on the kernels their d and M select.
 *   bf16 with d == 32 and M <= 32, and bf16 with d == 64 and M*M <= 512 (M <= 22), run on the MFMA
 *   kernels; every other case runs on kernels with float32 arithmetic that stream the keys through
 *   LDS (correct for every supported shape, not tuned).  Needs no workspace.  On the MFMA kernels
 *   the rotated, scaled score operands are rounded to fp16 when every one of a window-head's is in
 *   fp16 range, else to bf16; P is rounded to bf16 for the P.V product; accumulation is float32.
 *   float32 inputs are computed in float32 throughout.
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED or FSW_ERR_HIP.
 */
int flashswin_wattn_fwd(const void* q, const void* k, const void* v,
                        const float* theta_row, const float* theta_col,
                        void* out, float* lse,
                        int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                        int M, int shift, int dtype, void* hip_stream);

/*
 * Bytes of device workspace flashswin_wattn_bwd needs for this shape (0 when B == 0).
 * Returns 0 for arguments flashswin_wattn_bwd would reject.
 */
size_t flashswin_wattn_bwd_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                          int M, int shift, int dtype);

/*
 * Backward of flashswin_wattn_fwd by recomputation from the saved log-sum-exp
 * ([FS] Abstract: exact attention with flat memory in M; Table S1: training memory).
 *
 *   q, k, v, out  the forward's inputs and output, as in flashswin_wattn_fwd.
 *   dout          device, [B, Hg, Wg, heads, d] of `dtype`: gradient of the loss w.r.t. out.
 *   lse           device, float32 [B, Hg, Wg, heads]: the forward's lse (required).
 *   theta_row/col as in the forward.
 *   dq, dk, dv    device, [B, Hg, Wg, heads, d] of `dtype`, overwritten.
 *   dtheta_row,
 *   dtheta_col    device, float32 [heads, d/4], overwritten with d(loss)/d(theta), summed over
 *                 the whole batch, all windows and tokens, in a fixed order (bit-reproducible).
 *   workspace     device scratch of at least flashswin_wattn_bwd_workspace_size() bytes,
 *                 256-byte aligned; contents on entry are ignored.
 *   dq, dk, dv, dtheta_row, dtheta_col and the workspace may not share a byte with any input or
 *   with each other (FSW_ERR_INVALID_ARG).
 * Same shape rules and return codes as the forward, plus FSW_ERR_WORKSPACE.
 */
int flashswin_wattn_bwd(const void* q, const void* k, const void* v,
                        const void* out, const void* dout, const float* lse,
                        const float* theta_row, const float* theta_col,
                        void* dq, void* dk, void* dv,
                        float* dtheta_row, float* dtheta_col,
                        void* workspace, size_t workspace_bytes,
                        int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                        int M, int shift, int dtype, void* hip_stream);

/*
 * Forward from a packed qkv tensor, the layout a fused qkv projection writes ([FS] Figure 1(B):
 * the qkv projection feeds RoPE and the fused attention kernel).
 *
 *   qkv          device, [B, Hg, Wg, 3, heads, d] of `dtype`, 16-byte aligned: q, k and v are the
 *                slices qkv[..., 0, :, :], qkv[..., 1, :, :], qkv[..., 2, :, :], read in place
 *                (no split, no copy).
 *   out, lse     as in flashswin_wattn_fwd ([B, Hg, Wg, heads, d] and [B, Hg, Wg, heads]); they may
 *                not share a byte with qkv, theta_row, theta_col or each other.
 * Same shape rules and return codes as flashswin_wattn_fwd.  out and lse are bit-identical to
 * flashswin_wattn_fwd on the three slices.
 */
int flashswin_wattn_fwd_packed(const void* qkv, const float* theta_row, const float* theta_col,
                               void* out, float* lse,
                               int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                               int M, int shift, int dtype, void* hip_stream);

/*
 * Backward of flashswin_wattn_fwd_packed: the gradient is written packed as well.
 *
 *   qkv           the forward's packed input, [B, Hg, Wg, 3, heads, d].
 *   out, dout,
 *   lse, theta    as in flashswin_wattn_bwd.
 *   dqkv          device, [B, Hg, Wg, 3, heads, d] of `dtype`, 16-byte aligned, overwritten with
 *                 dq, dk, dv in the places of q, k, v.
 *   dqkv, dtheta_row, dtheta_col and the workspace may not share a byte with any input or with
 *   each other.
 *   dtheta_row/col, workspace  as in flashswin_wattn_bwd; the workspace size is
 *                 flashswin_wattn_bwd_workspace_size() of the same shape.
 * Same shape rules and return codes as flashswin_wattn_bwd.  Results are bit-identical to
 * flashswin_wattn_bwd on the slices.
 */
int flashswin_wattn_bwd_packed(const void* qkv, const void* out, const void* dout, const float* lse,
                               const float* theta_row, const float* theta_col,
                               void* dqkv, float* dtheta_row, float* dtheta_col,
                               void* workspace, size_t workspace_bytes,
                               int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                               int M, int shift, int dtype, void* hip_stream);

/* Largest rank of the low-rank bias factors of flashswin_wattn_fwd_lowrank / _bwd_lowrank. */
#define FLASHSWIN_MAX_RANK 32

/*
 * flashswin_wattn_fwd with a rank-r additive bias on the scores: the learned low-rank bias
 * factorization of the FlashBias comparison model ([FS] Table S1: a trainable rank-16 bias
 * factorization whose parameters grow with the window; Table 4 caption), folded into the fused
 * attention as r extra score channels.
 *
 *   bias_u,
 *   bias_w       device, float32 [heads, M*M, rank], 4-byte aligned: per head, factors over the
 *                in-window token index n = r*M + c (shifted frame, as for RoPE).  The pair (query i,
 *                key j) adds sum_t bias_u[h, n_i, t] * bias_w[h, n_j, t] to its scaled score
 *                q~ . k~ / sqrt(d), before the region mask.  Factors shared by all heads are passed
 *                repeated per head.
 *   rank         1 <= rank <= FLASHSWIN_MAX_RANK (rank < 1: FSW_ERR_INVALID_ARG; larger:
 *                FSW_ERR_UNSUPPORTED).
 *   Every other argument as in flashswin_wattn_fwd; out and lse may not share a byte with the
 *   factors.  LSE includes the bias.  bf16 with d = 32, windows of at most 512 tokens and grids that
 *   M divides runs on the MFMA forward with the bias as extra score channels; every other supported
 *   d, M, dtype and padded grid runs on the float32-arithmetic kernels.
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED or FSW_ERR_HIP.
 */
int flashswin_wattn_fwd_lowrank(const void* q, const void* k, const void* v,
                                const float* theta_row, const float* theta_col,
                                const float* bias_u, const float* bias_w, int rank,
                                void* out, float* lse,
                                int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                int M, int shift, int dtype, void* hip_stream);

/*
 * Bytes of workspace flashswin_wattn_bwd_lowrank needs: the workspace of the kernels that serve the
 * shape plus room for partial sums of both factor gradients (2 * windows * heads * M*M * rank * 4
 * bytes, and 8 bytes per head on the MFMA kernels).  0 when B == 0 and for arguments that call would
 * reject.
 */
size_t flashswin_wattn_bwd_lowrank_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                                  int M, int shift, int dtype, int rank);

/*
 * Backward of flashswin_wattn_fwd_lowrank ([FS] Table S1: the trainable factorization).  Besides
 * the outputs of flashswin_wattn_bwd it writes the factor gradients
 *   dbias_u      device, float32 [heads, M*M, rank], 4-byte aligned, overwritten:
 *                sum over all windows of dS W (dS = dL/d(score) = P (dP - Delta));
 *   dbias_w      likewise, sum over all windows of dS^T U.
 * Both are summed over the windows in a fixed order (bit-reproducible).  The outputs may not share
 * a byte with any input, the workspace or each other.  lse must come from
 * flashswin_wattn_fwd_lowrank with the same factors.  bf16 with d = 32, windows of at most 256
 * tokens (M <= 16) and grids that M divides runs on the whole-window MFMA kernels (the factors as
 * extra channels of the score products, their gradients from the extra output rows, summed per
 * group of windows); every other supported shape runs on the float32-arithmetic kernels.
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED, FSW_ERR_WORKSPACE or FSW_ERR_HIP.
 */
int flashswin_wattn_bwd_lowrank(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse,
                                const float* theta_row, const float* theta_col,
                                const float* bias_u, const float* bias_w, int rank,
                                void* dq, void* dk, void* dv, float* dtheta_row, float* dtheta_col,
                                float* dbias_u, float* dbias_w,
                                void* workspace, size_t workspace_bytes,
                                int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                int M, int shift, int dtype, void* hip_stream);

/*
 * Bytes of workspace flashswin_wattn_fwd_materialized needs: the float32 score rows of every
 * window-head, heads * windows * N * NP * 4 with N = M*M and NP = N rounded up to a multiple of 32.
 * 0 when B == 0 and for arguments that call would reject (including dtype other than bf16 or d != 32).
 */
size_t flashswin_wattn_fwd_materialized_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                                       int M, int shift, int dtype);

/*
 * Forward window attention computed the standard Swin way, with the score matrix of every window
 * materialized in HBM: a comparison path for memory and time, not the method's path ([FS] Abstract:
 * standard window attention materializes the M^2 x M^2 score matrix, O(M^4) memory per window, and
 * adds the learned relative-position bias elementwise to the scores; Figure 1(C) and Table S1: memory
 * against M; Figure S1: throughput against M).
 *
 *   Same attention as flashswin_wattn_fwd (RoPE, shift, region mask, scale 1/sqrt(d)), plus an
 *   optional bias:
 *   bias         device, float32 [heads, 2M-1, 2M-1], 4-byte aligned, or NULL for none: the pair of
 *                query i and key j at in-window positions (r_i, c_i), (r_j, c_j) adds
 *                bias[h, r_i - r_j + M - 1, c_i - c_j + M - 1] to its score.
 *   workspace    device, at least flashswin_wattn_fwd_materialized_workspace_size() bytes, 256-byte
 *                aligned: the float32 scores, then the bf16 probabilities in place.
 *   q, k, v, theta_row, theta_col, out, lse: as in flashswin_wattn_fwd (lse may be NULL).  out, lse and
 *   the workspace may not share a byte with any input or with each other.
 *   Three kernels: scores (MFMA, fp16 operands when in range, else bf16; float32 scores), row softmax
 *   (bf16 probabilities), P.V (MFMA).  Implemented for dtype FSW_BF16, d == 32, M <= 32 and grids
 *   that M divides only (FSW_ERR_UNSUPPORTED otherwise).
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED, FSW_ERR_WORKSPACE or FSW_ERR_HIP.
 */
int flashswin_wattn_fwd_materialized(const void* q, const void* k, const void* v,
                                     const float* theta_row, const float* theta_col, const float* bias,
                                     void* out, float* lse, void* workspace, size_t workspace_bytes,
                                     int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                     int M, int shift, int dtype, void* hip_stream);

/*
 * Bytes of the operand summary of flashswin_wattn_fwd_stats / _bwd_stats: 16 per window-head,
 * B * ceil(Hg/M) * ceil(Wg/M) * heads * 16.  0 for arguments those calls would reject.
 */
size_t flashswin_wattn_stats_bytes(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                                   int shift, int dtype);

/*
 * The forward of flashswin_wattn_fwd (rank == 0) or of flashswin_wattn_fwd_lowrank (rank >= 1, same
 * factor rules), which also writes a per-window-head summary of its inputs for
 * flashswin_wattn_bwd_stats: the same attention ([FS] Abstract: fused window attention, recomputed in
 * the backward from the saved log-sum-exp), with no change to out or lse.
 *
 *   bias_u, bias_w, rank  as in flashswin_wattn_fwd_lowrank; rank == 0: no bias (bias_u and bias_w are
 *                not read and may be NULL).
 *   stats        device, float32, flashswin_wattn_stats_bytes() bytes, 4-byte aligned, overwritten:
 *                per window-head (window-major, heads fastest) four values that summarize the largest
 *                |component| of that window's q, k and v rows of the head.  The content is private to
 *                this library version; pass it unchanged to flashswin_wattn_bwd_stats with the same
 *                q, k and v.  Written for dtype FSW_BF16 with d 32 or 64 (the shapes whose backward
 *                reads it); left unwritten otherwise.
 *   Every other argument as in flashswin_wattn_fwd; stats may not share a byte with an input, out
 *   or lse.  The MFMA forward computes the summary from the rows it already holds (no extra reads);
 *   the other forward kernels are followed by one pass over q, k and v.
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED or FSW_ERR_HIP.
 */
int flashswin_wattn_fwd_stats(const void* q, const void* k, const void* v,
                              const float* theta_row, const float* theta_col,
                              const float* bias_u, const float* bias_w, int rank,
                              void* out, float* lse, float* stats,
                              int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                              int M, int shift, int dtype, void* hip_stream);

/*
 * The backward of flashswin_wattn_bwd (rank == 0) or of flashswin_wattn_bwd_lowrank (rank >= 1) with
 * the summary of flashswin_wattn_fwd_stats: the prologue that computes Delta = rowsum(dO * O) reads
 * only O and dO instead of O, dO, q, k and v (the MFMA kernels size their fp16 operand scaling from
 * the summary).  Outputs are bit-identical to those calls on grids that M divides; on a padded grid
 * the summary, which covers only grid tokens, may choose another power-of-two operand scale, with
 * the same error bound.
 *
 *   stats        device, float32, flashswin_wattn_stats_bytes() bytes, 4-byte aligned: written by
 *                flashswin_wattn_fwd_stats for the same q, k, v and shape; read only.
 *   dbias_u, dbias_w  as in flashswin_wattn_bwd_lowrank when rank >= 1; not written (may be NULL)
 *                when rank == 0.
 *   workspace    flashswin_wattn_bwd_workspace_size() bytes (rank == 0) or
 *                flashswin_wattn_bwd_lowrank_workspace_size() bytes (rank >= 1).
 *   Every other argument as in flashswin_wattn_bwd; the outputs may not share a byte with stats.
 * Returns FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED, FSW_ERR_WORKSPACE or FSW_ERR_HIP.
 */
int flashswin_wattn_bwd_stats(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse,
                              const float* theta_row, const float* theta_col,
                              const float* bias_u, const float* bias_w, int rank, const float* stats,
                              void* dq, void* dk, void* dv, float* dtheta_row, float* dtheta_col,
                              float* dbias_u, float* dbias_w,
                              void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                              int M, int shift, int dtype, void* hip_stream);

/*
 * flashswin_wattn_fwd_packed that also writes the operand summary of flashswin_wattn_fwd_stats
 * (stats: flashswin_wattn_stats_bytes() bytes, 4-byte aligned, not sharing a byte with qkv, theta,
 * out or lse), for flashswin_wattn_bwd_packed_stats.  out and lse are bit-identical to
 * flashswin_wattn_fwd_packed.  Returns as flashswin_wattn_fwd_packed.
 */
int flashswin_wattn_fwd_packed_stats(const void* qkv, const float* theta_row, const float* theta_col,
                                     void* out, float* lse, float* stats,
                                     int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                     int M, int shift, int dtype, void* hip_stream);

/*
 * flashswin_wattn_bwd_packed with the summary of flashswin_wattn_fwd_packed_stats (read only; the
 * outputs may not share a byte with it): the prologue reads O and dO only.  Results as
 * flashswin_wattn_bwd_stats describes against flashswin_wattn_bwd (bit-identical on grids that M
 * divides).  Returns as flashswin_wattn_bwd_packed.
 */
int flashswin_wattn_bwd_packed_stats(const void* qkv, const void* out, const void* dout, const float* lse,
                                     const float* theta_row, const float* theta_col, const float* stats,
                                     void* dqkv, float* dtheta_row, float* dtheta_col,
                                     void* workspace, size_t workspace_bytes,
                                     int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                     int M, int shift, int dtype, void* hip_stream);

/* Size of the fixed per-GPU scratch array behind flashswin_wattn_bwd_noalloc: 32 MiB. */
#define FLASHSWIN_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * flashswin_wattn_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a fixed array of FLASHSWIN_SCRATCH_BYTES that the library places on every GPU it
 * runs on and holds until the process ends; its device address is looked up once per device, on
 * the first call with that device current.  This call makes no allocation of its own (no hipMalloc,
 * no hipFree, no allocating library routine).
 *
 *   Arguments, layouts, ownership of the caller's buffers and results: as flashswin_wattn_bwd, whose
 *   kernels it runs; the gradients are bit-identical to flashswin_wattn_bwd's.
 *   Returns FSW_ERR_SCRATCH, before any HIP call, when flashswin_wattn_bwd_workspace_size() of the
 *   shape exceeds FLASHSWIN_SCRATCH_BYTES (e.g. the bf16 M = 32 backward of 128 images of
 *   128 x 128 tokens and 3 heads needs 26.8 MB and fits; 200 such images need 41.9 MB and do not).  FSW_ERR_HIP when
 *   the scratch address cannot be looked up.  Otherwise the codes of flashswin_wattn_bwd.
 *   Every call on one GPU shares that GPU's array, and each call overwrites it: calls that overlap
 *   on one GPU (two host threads, or two streams whose work can run concurrently) race and give
 *   wrong results.  Calls queued on one stream are ordered and safe.  No part of the array needs
 *   to start cleared: every workspace section is written before it is read.
 */
int flashswin_wattn_bwd_noalloc(const void* q, const void* k, const void* v,
                                const void* out, const void* dout, const float* lse,
                                const float* theta_row, const float* theta_col,
                                void* dq, void* dk, void* dv,
                                float* dtheta_row, float* dtheta_col,
                                int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                int M, int shift, int dtype, void* hip_stream);

/* Static, human-readable name of a status code. */
const char* flashswin_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int flashswin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSWIN_H_ */
