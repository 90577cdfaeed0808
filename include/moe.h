/*
 * moe.h: C ABI of the MI355X (gfx950) routed SwiGLU mixture-of-experts forward.
 *
 * What it computes (one GPU, every expert local):
 *   for each live token t, with its top-k expert ids e_j and probabilities p_j,
 *     out[t] = sum over j in ascending e_j order, as an fp32 fused
 *              multiply-add chain from +0:  p_j * FC2_e( swiglu( FC1_e(x[t]) ) )
 *   where FC1_e yields gate g and up u, swiglu = silu(g) * u = g/(1+exp(-g)) * u,
 *   and the FC2 input is rounded to bf16 (bf16 precision) or re-quantized to
 *   MXFP8 per 32-element block (mxfp8 precision).
 *
 * Sources (web pages):
 *   Megatron-LM PR #7830 ("flashinfer_mega" backend), section "1. Mega backend
 *     for generation": canonical (ascending) expert-id order before the combine;
 *     kernel weight layout with gate/up interleaved in blocks of 32, K-major;
 *     a caller-owned kernel-weight buffer that a refit rewrites in place;
 *     construction-time rejection of configurations the kernels cannot run.
 *   Megatron-LM PR #7798 (moe_training_matches_inference), "Background" and
 *     "What is changed": activation and FC2-input quantization fused into the
 *     FC1 epilogue; probabilities applied after FC2; finalize = fp32 fused
 *     multiply-adds of probability and row, from zero, in the listed order.
 *   Megatron-LM PR #8367 (bound the MoE expert kernels by token count),
 *     "Problem": the live token count is a device-side value; the result is
 *     returned in fp32 without a bf16 downcast.
 *   Megatron-Core API docs, core.transformer.moe.training_matches_inference,
 *     `_route`: [tokens, topk] probabilities and expert ids.
 *   cudnn-frontend PR #448 (MoeEp), constructor/forward contract and the MoeEp
 *     class docstring: rows grouped by expert ascending, token-major inside an
 *     expert; MXFP8 = E4M3 data with one E8M0 scale per 32 elements.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers of the caller, 16-byte aligned,
 *     row-major, dense.  bf16 data is passed as its 16-bit patterns.
 *   - The library never allocates device memory and never synchronizes the
 *     stream, except moe_check (which reads the error word) and
 *     moe_get_indices (which copies to host).  moe_route and moe_forward only
 *     enqueue work on `stream`, so they can be captured in a HIP graph; a bf16
 *     forward above 1024 tokens may run its 64-row GEMM launches on a side
 *     stream of the library (one per GPU, default priority, created by the
 *     first bf16 moe_load_weights there and kept until the process ends),
 *     forked from `stream` and joined back to it with events, so the work
 *     still completes in `stream` order and is captured with it.
 *   - The live token count is read from device memory (live_rows_dev, int32,
 *     in TOKENS).  It is clamped to [0, T_cap]; a value outside sets an error
 *     bit (see moe_check).  Token rows >= live are never read and rows >= live
 *     of every output are never written.
 *   - Host-detectable errors return a negative moe_status and set a
 *     thread-local message (moe_last_error); nothing is enqueued then.
 *   - Calls that share a workspace must be ordered (same stream or events).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx* moe_handle;

typedef enum { MOE_BF16 = 0, MOE_MXFP8 = 1, MOE_MXFP4 = 2 } moe_precision;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,      /* bad size, null or misaligned pointer     */
    MOE_ERR_UNSUPPORTED = -2,      /* configuration the kernels cannot run     */
    MOE_ERR_NOT_LOADED = -3,       /* forward before any moe_load_weights      */
    MOE_ERR_HIP = -4,              /* a HIP runtime call failed                */
    MOE_ERR_DEVICE_CONTRACT = -5,  /* moe_check found contract-violation bits  */
} moe_status;

/* Device-side contract-violation bits reported by moe_check. */
#define MOE_DEVERR_BAD_EXPERT_ID 1u   /* id outside [0, E) in a live token: route dropped */
#define MOE_DEVERR_DUP_EXPERT_ID 2u   /* same id twice in a live token: repeat dropped    */
#define MOE_DEVERR_LIVE_ABOVE_CAP 4u  /* live > T_cap: clamped to T_cap                  */
#define MOE_DEVERR_LIVE_NEGATIVE 8u   /* live < 0: treated as 0                          */
#define MOE_DEVERR_FUSED_WAIT 16u     /* MOE_FUSED_FFN: an FC2 tile's wait for its FC1
                                         rows ran past 0.2 s (workgroups not all
                                         resident, e.g. other work on the GPU): the
                                         outputs of that call are invalid            */

/* Create a handle for E experts, hidden size H, expert FFN size F, top-k.
 * Checks (Megatron-LM PR #7830, construction-time validation; cudnn-frontend
 * PR #448, MXFP8 block of 32): 1 <= E <= 1024; 1 <= topk <= min(E, 16);
 * H and F positive multiples of 32 (the interleave block and the MX
 * block); precision MOE_BF16, MOE_MXFP8 or MOE_MXFP4, else
 * MOE_ERR_UNSUPPORTED.  MOE_MXFP4: weights in E2M1 (the OCP MX 4-bit float)
 * with one E8M0 scale per 32 elements of K, activations and the SwiGLU rows
 * in MXFP8 as with MOE_MXFP8 (the CDNA4-native counterpart of a 4-bit-weight,
 * 8-bit-activation expert GEMM).  Host only: no device work; the device is
 * the one current at the first launch. */
moe_status moe_create(int E, int H, int F, int topk, int precision, moe_handle* out);

/* Free the handle (host state only).  NULL is ignored. */
void moe_destroy(moe_handle h);

/* Size in bytes of the caller-owned kernel-weight buffer (kbuf). */
size_t moe_weight_bytes(moe_handle h);

/* Pack the weights into the caller-owned buffer kbuf, in place (Megatron-LM
 * PR #7830: caller-owned kernel-weight buffer, refit rewrites it in place).
 *   w1: bf16 [E][2F][H]; rows 0..F-1 of each expert are gate, F..2F-1 up.
 *   w2: bf16 [E][H][F].
 *   Row order: FC1 packed row 64b+i = gate row 32b+i (i < 32) or up row
 *     F+32b+i-32 (i >= 32); FC2 rows [H] unchanged.  Rows are K-major and
 *     tiled into MFMA operand blocks so that one wave's load is 1 KB contiguous.
 *     For a section with N rows of K elements per expert:
 *   kbuf layout (bf16): FC1 section (N = 2F, K = H) then FC2 section (N = H,
 *     K = F) of 1 KB blocks (16 rows x 32 K).  With c = n/16, s = k/32,
 *     KS = K/32, g = c/32 and w = min(32, N/16 - 32g) (the width of c's
 *     512-row group), element (e, n, k) is at element index
 *       (e*(N/16)*KS + g*32*KS + s*w + c%32)*512 + ((k%32)/8)*128 + (n%16)*8 + k%8,
 *     so that one K step of a 512-row group is one contiguous run of blocks.
 *   kbuf layout (mxfp8): sections FC1 codes, FC2 codes, FC1 scales, FC2
 *     scales, each starting at a multiple of 256 bytes.  With KS = ceil(K/128)
 *     and KQ = ceil(KS/4), code (e, n, k) at byte
 *       (((e*(N/16) + n/16)*KS + k/128)*2 + (k%128)/64)*1024
 *         + ((k%64)/16*16 + n%16)*16 + k%16,
 *     and the E8M0 scale of 32-block b = k/32 of row n at byte
 *       ((e*(N/16) + n/16)*KQ + (b/4)/4)*256 + ((b%4)*16 + n%16)*4 + (b/4)%4;
 *     positions past K hold code 0 and scale 127.  Scale = power-of-two
 *     ceiling of the block's max magnitude / 448 (so no code saturates).
 *   kbuf layout (mxfp4): sections as mxfp8, with one 1 KB code block per 16
 *     rows x 128 K and the blocks of an expert in 512-row groups (one K step
 *     of a group is one contiguous run): with c = n/16, t = k/128,
 *     g = c/32 and w = min(32, N/16 - 32g), code (e, n, k) in byte
 *       (e*(N/16)*KS + g*32*KS + t*w + c%32)*1024 + ((k%128)/32*16 + n%16)*16
 *         + (k%32)/2,
 *     the low nibble for even k; the scale of 32-block b = k/32 at byte
 *       (e*(N/16)*KQ + g*32*KQ + (b/16)*w + c%32)*256 + ((b%4)*16 + n%16)*4
 *         + (b/4)%4,
 *     the scale = power-of-two ceiling of the block's max magnitude / 6,
 *     codes rounded to the nearest E2M1 value with ties to the even code.
 * The handle remembers kbuf: every later forward reads it.  Calling again
 * (same or another buffer) is the refit; forwards enqueued before it on the
 * same stream read the old contents.  w1/w2 may be freed once the work on
 * `stream` is complete.  kbuf_bytes must be >= moe_weight_bytes(h). */
moe_status moe_load_weights(moe_handle h, const void* w1, const void* w2, void* kbuf,
                            size_t kbuf_bytes, hipStream_t stream);

/* Workspace bytes for a token capacity T_cap (0 for a NULL handle or a
 * negative T_cap).  The workspace is caller-owned device memory with no
 * required initial contents: every launch writes what a later launch of the
 * same call reads, so a fresh allocation (or one left by another handle) can
 * be passed as is.  Its bytes are the library's until the work enqueued on it
 * has finished; moe_get_indices, moe_get_rows and moe_check read the state of
 * the last moe_route / moe_forward that used it. */
size_t moe_workspace_bytes(moe_handle h, int64_t T_cap);

/* Router (Megatron-Core `_route`): for each live token, softmax over the E
 * logits, the top-k experts by logit (ties to the lower id), probabilities
 * renormalized over the selected experts, written with ids ascending.
 *   logits: fp32 [T_cap][E]; ids: int32 [T_cap][topk]; probs: fp32 [T_cap][topk].
 * ws: a workspace of this handle (its header receives the live-count bits). */
moe_status moe_route(moe_handle h, const float* logits, int64_t T_cap,
                     const int32_t* live_rows_dev, int32_t* ids, float* probs, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* The routed SwiGLU MoE forward (Megatron-LM PR #8367, "Problem": a device-
 * side active-token count bounds the expert work and the finalize returns
 * fp32; cudnn-frontend PR #448, MoeEp forward(activation, fc1_weight,
 * fc2_weight, topk_idx, topk_weights), with the weights bound by
 * moe_load_weights instead of passed per call).
 *   x: bf16 [T_cap][H]; expert_ids: int32 [T_cap][topk], any order per token
 *   (sorted ascending here); probs: fp32 [T_cap][topk]; out: fp32 [T_cap][H].
 *   ws: ws_bytes >= moe_workspace_bytes(h, T_cap).
 *   out[t] for live t is the fp32 chain of the file header; rows >= live are
 *   not written.
 * Every token's output bits are independent of the other tokens, of T_cap
 * and of the live count.  Errors: MOE_ERR_INVALID_ARG (NULL or misaligned
 * pointer, T_cap outside [0, 2^26], ws_bytes too small), MOE_ERR_NOT_LOADED
 * (no moe_load_weights yet), MOE_ERR_HIP (a launch failed); nothing is
 * enqueued on an error.  Contract violations inside the data (ids, live
 * count) are reported by moe_check. */
moe_status moe_forward(moe_handle h, const void* x, const int32_t* expert_ids,
                       const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* How moe_forward_ex combines a token's routes. */
typedef enum {
    MOE_COMBINE_FP32 = 0,  /* moe_forward's combine: out fp32 [T_cap][H]                  */
    MOE_COMBINE_BF16 = 1,  /* the same fp32 chain rounded to bf16: out bf16 [T_cap][H]     */
    MOE_COMBINE_ROWS = 2,  /* each route unscaled: out fp32 [T_cap][topk][H]              */
} moe_combine;

/* Added to MOE_COMBINE_FP32 or MOE_COMBINE_BF16: apply each route's
 * probability inside FC1 instead of in the combine (cudnn-frontend PR #448,
 * the MoeEp constructor's apply_topk_in_fc1 option).  The pages give no
 * arithmetic for it; here the fp32 SwiGLU row is multiplied by the route's
 * probability before the FC2-input rounding (bf16 nearest even, or the MXFP8
 * requantization per 32-block), FC2 returns the weighted row, and the combine
 * adds a token's weighted rows as an fp32 chain from +0 in canonical order
 * (the fused multiply-add of the default combine with p = 1); MOE_COMBINE_BF16
 * rounds that sum to bf16.  Not valid with MOE_COMBINE_ROWS. */
#define MOE_APPLY_TOPK_IN_FC1 0x100

/* Added to any combine (bf16 weights only): run FC1 and FC2 as one persistent
 * launch instead of two (Megatron-LM PR #7830, "What does this PR do?": one
 * fused kernel for the expert MLP; cudnn-frontend PR #448's MegaMoE files
 * fc1_fc2_fuse_sched, grid_sync).  Every 64-row M tile has a readiness
 * counter; an FC1 tile releases its SwiGLU rows at device scope and counts
 * itself; an FC2 tile first issues its weight loads, then waits until all
 * FC1 column tiles of its M tile are counted, then reads the rows.  The
 * 64-row tile design takes every tile in this mode (also above 1024 tokens),
 * with the same arithmetic as always, so the outputs are bit-identical to the
 * two-launch path.  The waits are bounded: if one runs past 0.2 s (possible
 * only when not every workgroup is resident, e.g. with other work on the
 * GPU), it flags MOE_DEVERR_FUSED_WAIT for moe_check and the call's outputs
 * are invalid.  With another precision: MOE_ERR_INVALID_ARG. */
#define MOE_FUSED_FFN 0x200

/* Added to any combine (bf16 weights only; implies MOE_FUSED_FFN): the
 * finalize runs in the same persistent launch as FC1 and FC2, so the whole
 * forward after the permutation is one launch (Megatron-LM PR #7830, "What
 * does this PR do?": dispatch, expert MLP and combine in one fused kernel;
 * cudnn-frontend PR #448's MegaMoE file list, fc1_fc2_fuse_sched).  The
 * permutation stage sets, for every live token and 512-column block of the
 * output, the number of the token's kept routes; an FC2 tile, once its fp32
 * rows are released at device scope, counts each of its rows' tokens down,
 * and the workgroup that takes a count to zero combines that token's
 * 512-column block at once (no workgroup ever waits for another here).  The
 * combine is the finalize's own arithmetic (the fp32 chain from +0 in
 * canonical order, its bf16 rounding, or row mode), so outputs are
 * bit-identical to the separate finalize.  A live token whose routes were all
 * dropped is written by the permutation stage (+0 in every mode).  Errors as
 * MOE_FUSED_FFN. */
#define MOE_FUSED_FINALIZE 0x400

/* moe_forward with a choice of combine; every stage before the combine is
 * moe_forward's, so the FC2 rows are bit-identical across the three (without
 * MOE_APPLY_TOPK_IN_FC1, which changes the FC2 rows).
 *   MOE_COMBINE_FP32: exactly moe_forward.
 *   MOE_COMBINE_BF16 (Megatron-LM PR #7798, "What is changed": the
 *     BF16_RANK_PARTIALS unpermute, which on one rank adds a token's routes as
 *     fp32 fused multiply-adds of probability and row from zero, in the listed
 *     order, and quantizes the sum to BF16 as FlashInfer's finalize does):
 *     out[t][m] = bf16_rne(the fp32 chain of moe_forward); out is bf16 (uint16
 *     bits) [T_cap][H].
 *   MOE_COMBINE_ROWS (Megatron-LM PR #7798, "What is changed", expert compute;
 *     Megatron-Core API docs, expert_value_pass): every route runs as a top-1
 *     token with probability 1.0, so the finalize returns its expert output
 *     unscaled: out[t][j][m] = fma(1, O_j[m], +0.0f) for the j-th route of
 *     token t in canonical (ascending expert id) order, where O_j is that
 *     route's fp32 FC2 row; -0 comes back as +0 and a dropped route (invalid
 *     or repeated id) as a row of +0.  out is fp32 [T_cap][topk][H].  probs
 *     is not read and may be NULL.
 * combine may carry MOE_APPLY_TOPK_IN_FC1 (fp32 and bf16 combines),
 * MOE_FUSED_FFN and MOE_FUSED_FINALIZE (bf16 weights).
 * Rows of tokens >= live are never written in any mode.  Errors: an unknown
 * combine, or MOE_APPLY_TOPK_IN_FC1 with row mode, is MOE_ERR_INVALID_ARG;
 * otherwise as moe_forward. */
moe_status moe_forward_ex(moe_handle h, const void* x, const int32_t* expert_ids,
                          const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                          int combine, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward_ex without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The workspace is a 64 MiB device array that the
 * library holds on each GPU it runs on until the process ends; its address is
 * looked up once per GPU (hipGetSymbolAddress) at the first call there.  The
 * call allocates nothing and enqueues the same kernels as moe_forward_ex.
 *   Arguments as moe_forward_ex, minus ws / ws_bytes.
 *   Limit: T_cap with moe_workspace_bytes(h, T_cap) <= 64 MiB (about 600
 *   tokens at hidden 2048, FFN 1024, top-6); a larger T_cap returns
 *   MOE_ERR_INVALID_ARG with nothing enqueued.
 *   Every call on one GPU shares that GPU's array, from any handle or stream:
 *   calls that overlap in time on one GPU race and must be ordered by the
 *   caller.  Nothing needs to start at zero (see moe_workspace_bytes); the
 *   array keeps the last call's contents, and contract-violation bits are
 *   not reported (moe_check needs a caller workspace).
 * Errors: as moe_forward_ex; MOE_ERR_HIP if the array's address cannot be
 * looked up. */
moe_status moe_forward_noalloc(moe_handle h, const void* x, const int32_t* expert_ids,
                               const float* probs, int64_t T_cap, const int32_t* live_rows_dev,
                               int combine, void* out, hipStream_t stream);

/* Copy the permutation of the last forward to host arrays (synchronizes the
 * stream).  The grouping is cudnn-frontend PR #448's route index (MoeEp class
 * docstring): rows grouped by local expert in ascending order, token-major
 * inside an expert; on one GPU the source rank is always 0 and is dropped.
 * counts: int32 [E]; offsets: int32 [E+1]; perm_src: int32 [n_rows]
 * (= t*topk + j of the route at each grouped row, experts ascending, tokens
 * ascending within an expert); dst: int32 [T*topk] (grouped row of each
 * route, -1 if dropped); n_rows_out / T_out: the row and live-token counts.
 * perm_src and dst must hold T_cap*topk entries.  Any output may be NULL. */
moe_status moe_get_indices(moe_handle h, const void* ws, int64_t T_cap, int32_t* counts,
                           int32_t* offsets, int32_t* perm_src, int32_t* dst,
                           int32_t* n_rows_out, int32_t* T_out, hipStream_t stream);

/* Copy intermediate rows of the last forward to host arrays (synchronizes
 * the stream), in grouped-row order.  fc2_rows: fp32 [n_rows][H], the
 * unweighted FC2 output rows.  fc1_out_rows: the FC2 operand rows, bf16
 * [n_rows][F] (bf16 precision) or E4M3 codes [n_rows][F] followed by E8M0
 * scales [n_rows][F/32] (mxfp8, mxfp4).  sorted_ids / sorted_probs: int32 /
 * fp32 [T][topk], each token's routes in canonical order.  x_codes /
 * x_scales (mxfp8, mxfp4; must be NULL for bf16): the quantized activations,
 * E4M3 codes uint8 [T][H] and E8M0 scale bytes uint8 [T][H/32] (T = the live
 * tokens of the last forward).  Any output may be NULL.  For tests and
 * debugging.  Errors: MOE_ERR_INVALID_ARG for a NULL handle or workspace, or
 * x_codes / x_scales with bf16; MOE_ERR_HIP if a copy fails. */
moe_status moe_get_rows(moe_handle h, const void* ws, int64_t T_cap, float* fc2_rows,
                        void* fc1_out_rows, int32_t* sorted_ids, float* sorted_probs,
                        void* x_codes, void* x_scales, hipStream_t stream);

/* Synchronize the stream, return the contract-violation bits (MOE_DEVERR_*)
 * of the last moe_route or moe_forward that ran on this workspace in
 * *err_bits, and clear them.  Each of those calls overwrites the bits, so
 * after a route and a forward they are the forward's (which checks the same
 * live count as well as the ids); a workspace no call has run on yet holds no
 * meaningful bits.  Returns MOE_OK when no bit is set and
 * MOE_ERR_DEVICE_CONTRACT (with *err_bits filled in and moe_last_error naming
 * the bits) when any is: the device-side half of the error contract, whose
 * violations cannot be returned by the enqueueing call itself
 * (Megatron-LM PR #7798, review discussion of the MXFP8 tile floor: a
 * broken assumption should fail loudly rather than change numbers).  MOE_ERR_INVALID_ARG for NULL
 * arguments, MOE_ERR_HIP if the copy fails. */
moe_status moe_check(moe_handle h, void* ws, hipStream_t stream, uint32_t* err_bits);

/* Stage timing hook (for profiling).  With events != NULL, every later
 * moe_forward on this handle records, on its stream, events[0] before its
 * first kernel and events[i] after stage i: 1 permutation (sort, histogram,
 * scan, scatter), 2 MXFP8 activation quantization (nothing in bf16), 3 FC1 +
 * SwiGLU, 4 FC2, 5 finalize.  events[2] and events[3] are the start and end
 * of the FC1 + SwiGLU launch itself, recorded by its dispatch (no marker
 * packets around it), so events[3] - events[2] is that launch's duration
 * (MXFP4 above a 1024-token capacity, where the stage is two launches: the
 * first one's start and the second one's end).
 * n_events must be 6; NULL entries are not recorded.  The events are the
 * caller's; pass events = NULL to stop. */
moe_status moe_set_stage_events(moe_handle h, hipEvent_t* events, int n_events);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
