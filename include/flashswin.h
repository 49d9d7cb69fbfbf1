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
 * The library allocates no device memory and keeps no global state; calls are thread-safe.
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
  FSW_ERR_HIP = 4          /* a HIP launch reported an error */
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
 *   B >= 0 (B == 0 returns FSW_OK with nothing enqueued); Hg, Wg positive multiples of M;
 *   1 <= M <= 32; 0 <= shift < M; heads >= 1; d in {8, 16, 32, 64}; dtype FSW_F32 or FSW_BF16.
 *   Needs no workspace.  bf16 inputs are rounded once more to bf16 after the rotation and the
 *   scaling, P is rounded to bf16 for the P.V product, accumulation is float32; float32 inputs
 *   are computed in float32 throughout.
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

/* Static, human-readable name of a status code. */
const char* flashswin_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int flashswin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSWIN_H_ */
