/*
 * moe.h - C ABI of one GPU's trainable mixture-of-experts layer on MI355X (gfx950).
 *
 * The layer is the one described on the Prime Mega MoE pages (news item,
 * section "How does the fused kernel work?"): tokens are dispatched to their
 * top-k experts, each expert applies two linear layers with SwiGLU in between,
 * and the expert outputs are combined with the routing weights; the same
 * section adds the training (backward) pass.  Section "How do developers use
 * it?" lists the precisions bf16, mxfp8, fp8 and fp8_bwd.
 *
 * Shapes (all row-major):
 *   x, y, dy, dx   [T, D]         tokens x model dim
 *   topk_idx       [T, K] int32   expert id of each (token, slot); p = t*K + k
 *   topk_w         [T, K] fp32    routing weight of each (token, slot)
 *   w1, dw1        [E, 2F, D]     expert linear 1; rows 0..F-1 gate, F..2F-1 up
 *   w2, dw2        [E, D, F]      expert linear 2 (down)
 *   dtopk_w        [T, K] fp32    gradient of the loss wrt topk_w
 * Forward:  h = W1[e] x_t, a = silu(h[:F]) * h[F:], o = W2[e] a, y_t = sum_k w o.
 * Backward of a loss L with dL/dy = dy: dx, dW1, dW2 and dtopk_w = <dy_t, o>.
 *
 * Element types by mode:
 *   MOE_FP32            x y dy dx w1 w2 dw1 dw2 fp32; fp32 GEMMs (vector ALU)
 *   MOE_FP32_BF16GEMM   fp32 storage, GEMM operands rounded to bf16, fp32 accumulate
 *   MOE_BF16            bf16 storage (raw 16-bit bfloat16), bf16 GEMMs, fp32 accumulate
 *   MOE_FP8_BWD         bf16 storage, bf16 forward, blockwise-FP8 backward GEMMs
 *   MOE_MXFP8           bf16 storage, MXFP8 GEMMs forward and backward
 *   MOE_FP8             bf16 storage, blockwise-FP8 GEMMs forward and backward
 * FP8 operands are OCP e4m3 (round to nearest even, saturating at 448).  Blockwise
 * FP8: one fp32 scale amax/448 per 1x128 activation tile along the GEMM's
 * contraction axis (for the weight gradients: 128 consecutive tokens of one
 * expert, from the expert's first token) and per 128x128 weight block.  MXFP8:
 * one e8m0 scale 2^X per 32 contraction elements of every operand, X the
 * smallest integer with amax <= 448 * 2^X.  The FP8 modes need D % 256 == 0 and
 * F % 256 == 0, and `wprep` (filled by moe_prepare_weights) in moe_fwd/moe_bwd.
 * Intermediates are kept in bf16 (fp32 accumulators, rounded once when stored),
 * in fp32 in MOE_FP32; SwiGLU, its backward, the routing-weight products and
 * all row sums are fp32.
 *
 * Ownership and threading:
 *   - Every pointer is a device pointer unless noted.  The caller allocates and
 *     owns every buffer, including `scratch` and `wprep`; the library never
 *     allocates or frees device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     asynchronously and return without synchronizing, except moe_check and
 *     moe_profile_collect.
 *   - Inputs are never modified.  Calls on distinct scratch buffers are
 *     independent; the library keeps no state except the opt-in profiler.
 *   - Buffers must be 16-byte aligned and must not overlap.
 *
 * Errors: every call returns MOE_OK (0) or a negative MOE_E* code found on the
 * host before anything is enqueued.  Errors found by the GPU (an expert id out
 * of range) are latched in a word inside `scratch`, which moe_route and moe_fwd
 * clear when they start; moe_check returns and clears it.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

enum moe_mode {
  MOE_FP32 = 0,
  MOE_FP32_BF16GEMM = 1,
  MOE_BF16 = 2,
  MOE_FP8_BWD = 3,
  MOE_MXFP8 = 4,
  MOE_FP8 = 5
};

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null pointer, non-positive or inconsistent sizes, bad mode */
  MOE_ESCRATCH = -2,     /* scratch_bytes / wprep_bytes smaller than required */
  MOE_EALIGN = -3,       /* a buffer is not 16-byte aligned */
  MOE_EUNSUPPORTED = -4, /* valid request this library cannot run (mode or shape) */
  MOE_EHIP = -5,         /* a HIP launch or runtime call failed */
  MOE_EINDEX = -6,       /* (device) a topk_idx entry was outside [0, E) */
  MOE_ETIMEOUT = -7      /* (device) a bounded wait in a persistent kernel expired */
};

/* Flags (moe_desc.flags). */
/* Forward as one overlapped launch: dispatch, W1 + SwiGLU and W2 ordered by
 * per-XCD ticket queues, the single-GPU form of the pages' overlap of token
 * arrival with expert compute (Prime Mega MoE news item, "How does the fused
 * kernel work?"): a W1 tile starts as soon as the dispatch items holding its
 * rows are written, a W2 tile as soon as the W1 tiles of its rows are done.
 * Applies to the bf16-GEMM modes (MOE_FP32_BF16GEMM, MOE_BF16, MOE_FP8_BWD)
 * with D % 256 == 0 and F % 128 == 0; elsewhere it has no effect.  Results are
 * bit-identical to the default one-kernel-per-step forward, which is faster on
 * MI355X at the Qwen3 shapes and therefore the default. */
#define MOE_FLAG_OVERLAP 0x1u
/* Diagnostics only, with MOE_FLAG_OVERLAP: every bounded wait of the
 * overlapped forward targets a value that is never reached and gives up after
 * 1 us, so moe_check reports MOE_ETIMEOUT; the outputs of that call are
 * undefined.  Exists to test the timeout path without a real stall. */
#define MOE_FLAG_QUEUE_TIMEOUT_TEST 0x2u
/* Activation recompute, the layer-level form of the full activation
 * checkpointing the pages' training runs use (Prime Mega MoE news item, "How
 * fast is Prime Mega MoE?"): the forward keeps the linear-1 output H [T*K, 2F]
 * out of the saved state (the W1 epilogue stores only the SwiGLU output A), and
 * moe_bwd first recomputes H with the same W1 GEMM, bit-identical to the
 * forward's, into the buffer the SwiGLU backward then overwrites in place with
 * dH.  moe_scratch_bytes is smaller by the H region (T*K*2F elements); every
 * output is bit-identical to the default; the backward does 4*T*K*D*F more
 * flops.  MOE_VIEW_H is not available (MOE_EINVAL).  All modes. */
#define MOE_FLAG_RECOMPUTE 0x4u
/* Backward with each dgrad and its weight gradient in one launch: W2 dgrad +
 * SwiGLU-backward beside the W2 weight gradient, then the W1 dgrad beside the
 * W1 weight gradient, their tiles taken from shared per-XCD queues, so that
 * one GEMM's tiles fill the other's tail and their epilogues fall between the
 * other's main loops (the single-GPU form of the overlapping backward the
 * pages add to the fused kernel: Prime Mega MoE news item, "How does the fused
 * kernel work?").  Needs D % 256 == 0, F % 256 == 0 and E <= 256, in MOE_BF16
 * and the FP8 modes.  It is the default for MOE_BF16 when T*K <= 4096*E (at
 * most 4096 routed pairs per expert on average), where it measured 0.7-0.9%
 * faster on MI355X at the Qwen3 shapes (with 8192 per expert it measured up to
 * 8% slower); MOE_FLAG_OVERLAP_BWD selects it in every mode (in the FP8 modes
 * it measured 4-10% slower), MOE_FLAG_SERIAL_BWD selects one kernel per GEMM
 * in every mode, and setting both is MOE_EINVAL.  Results
 * are bit-identical either way (the same tile code in the same accumulation
 * order). */
#define MOE_FLAG_OVERLAP_BWD 0x8u
#define MOE_FLAG_SERIAL_BWD 0x10u

/* Layer descriptor, passed by host pointer.  Requirements: T >= 0; E, K >= 1;
 * K <= E; E <= 1024; D % 64 == 0 and F % 64 == 0; T * K < 2^31 (else
 * MOE_EINVAL).  The kernels address one expert's rows and one expert's weight
 * matrix through 32-bit buffer ranges, and an expert may receive every routed
 * pair, so shapes with T * K * max(D, 2F) * s >= 2^31 or 2F * D * s >= 2^31
 * (s = 4 bytes in MOE_FP32, else 2), or, in the FP8 modes, with
 * 256 * Npad >= 2^31 (Npad = 128 * floor((T*K + 127*E) / 128)), give
 * MOE_EUNSUPPORTED instead of wrapping; moe_scratch_bytes then returns 0.  T = 0 is a
 * layer with no tokens: moe_route and moe_fwd leave zero counts and offsets,
 * moe_bwd writes zero dw1 and dw2 (every expert has no tokens), and the [T, ...]
 * buffers (x, y, dy, dx, topk_idx, topk_w, dtopk_w) may be null. */
typedef struct moe_desc {
  int32_t T, D, F, E, K;
  int32_t mode;  /* enum moe_mode */
  int32_t flags; /* MOE_FLAG_* */
} moe_desc;

/* Size in bytes of the scratch buffer for `d` (host call; 0 if `d` is invalid).
 * The scratch holds the routing metadata (the stable by-expert sort of the
 * routed pairs: the pages' sorting of tokens by expert, "Why is MoE training
 * communication-bound?") and the intermediates kept between forward and
 * backward (the pages keep intermediates in scratch memory that only the GPU
 * uses rather than in framework tensors, "How does the fused kernel work?").  Its layout is private. */
size_t moe_scratch_bytes(const moe_desc* d);

/* Size in bytes of the prepared-weight buffer: quantised weight copies for the
 * FP8 modes (each weight in the orientation of each GEMM that reads it), bf16
 * copies for MOE_FP32_BF16GEMM, 0 for MOE_BF16 (where `wprep` may be NULL).
 * The FP8 formats are the pages' blockwise FP8 and MXFP8 ("How does the fused
 * kernel work?"), selected by the precision names of "How do developers use
 * it?".  Host call; 0 if `d` is invalid. */
size_t moe_wprep_bytes(const moe_desc* d);

/* Fill `wprep` from w1/w2 (bf16 in the FP8 modes, fp32 in MOE_FP32_BF16GEMM; a
 * no-op returning MOE_OK in MOE_BF16).  Must be called again whenever the
 * weights change.  FP8 modes: every weight is quantised to e4m3 in 128 x 128
 * blocks (blockwise) or groups of 32 along the contraction (MXFP8), once per
 * orientation a GEMM reads it in (the weight side of the pages' FP8 kernels,
 * "How does the fused kernel work?").  w1, w2: [E, 2F, D] and [E, D, F] device
 * buffers; wprep: device, wprep_bytes >= moe_wprep_bytes(d) (MOE_ESCRATCH).
 * 16-byte alignment (MOE_EALIGN).  Asynchronous on `stream`. */
int moe_prepare_weights(const moe_desc* d, const void* w1, const void* w2,
                        void* wprep, size_t wprep_bytes, void* stream);

/* Routing metadata only (moe_fwd runs it itself): the pages' sort of the
 * tokens by destination expert ("Why is MoE training communication-bound?",
 * the tokens are sorted on the GPU before the exchange), here a stable
 * counting sort of the routed pairs.  topk_idx: device int32 [T, K], 4-byte aligned; scratch as
 * in moe_fwd.  For the flat pair index
 * p = t*K + k with expert e = topk_idx[p]:
 *   counts[e] = #{p : idx_p = e}; offsets = exclusive prefix sum, offsets[E]
 *   = number of valid pairs; pos[p] = offsets[e] + #{p' < p : idx_p' = e}
 *   (stable by p; -1 for an id outside [0, E), which also latches MOE_EINDEX);
 *   src[pos[p]] = p.  All int32, in scratch; see moe_routing_view. */
int moe_route(const moe_desc* d, const int32_t* topk_idx, void* scratch,
              size_t scratch_bytes, void* stream);

/* Device pointers into `scratch` for counts [E], offsets [E+1], pos [T*K] and
 * src [T*K] (src entries past offsets[E] are unspecified): the routing
 * metadata of moe_route ("Why is MoE training communication-bound?").  Host
 * arithmetic only, nothing is read or launched; any output pointer may be
 * NULL.  Takes the descriptor and scratch size to locate the regions and to
 * check that the buffer holds them (MOE_ESCRATCH). */
int moe_routing_view(const moe_desc* d, const void* scratch, size_t scratch_bytes,
                     int32_t** counts, int32_t** offsets, int32_t** pos, int32_t** src);

/* Intermediates in scratch, for tests and tools (row r is the r-th routed pair
 * in expert order, i.e. pair src[r]):
 *   MOE_VIEW_XPERM  [T*K, D]   dispatched tokens (bf16; fp32 in MOE_FP32).  Not
 *                              stored in MOE_MXFP8 and MOE_FP8 without
 *                              MOE_FLAG_RECOMPUTE (only their FP8 codes are).  In
 *                              MOE_BF16 at D % 64 == 0 and 2F % 256 == 0 no
 *                              dispatch kernel runs: the linear-1 GEMM gathers
 *                              the token rows and writes these (and WPERM)
 *   MOE_VIEW_H      [T*K, 2F]  linear-1 output: gate | up
 *   MOE_VIEW_A      [T*K, F]   SwiGLU output
 *   MOE_VIEW_O      [T*K, D]   linear-2 output (unweighted)
 *   MOE_VIEW_DYPERM [T*K, D]   dispatched upstream gradient times the routing
 *                              weight, w * dy (fp32 product, stored once).  Not
 *                              stored in the FP8 modes (only its FP8 codes are)
 *   In MOE_BF16 at D % 64 == 0 and 2F % 256 == 0 the GEMMs carry the routing
 *   weights instead: A holds w * A (rounded once), O holds w * O, DYPERM holds
 *   dy itself, and dtopk_w comes from the W2 dgrad (sum over f of its fp32
 *   dy W2^T against the SwiGLU output recomputed from H).
 *   MOE_VIEW_DH     [T*K, 2F]  gradient wrt linear-1 output
 *   MOE_VIEW_DXPERM [T*K, D]   gradient wrt dispatched tokens
 *   MOE_VIEW_WPERM  [T*K] fp32 routing weight of each routed pair
 * FP8 modes only (contents of the last GEMM that used them; C = max(D, 2F),
 * Npad = 128 * floor((T*K + 127*E) / 128)):
 *   MOE_VIEW_Q_ROWS        [T*K, C] e4m3 codes of an activation quantised along its rows
 *   MOE_VIEW_Q_ROWS_SCALE  [C/128, T*K] 4-byte scale entries
 *   MOE_VIEW_Q_TOK_A/B     [C, Npad] e4m3 codes quantised along tokens (expert e's
 *                          tokens in columns 128*p[e] .. , p = prefix of ceil(count/128));
 *                          after moe_bwd, A holds dH's and B x_perm's
 *   MOE_VIEW_Q_TOK_A/B_SCALE [Npad/128, C] 4-byte scale entries
 * A 4-byte entry is an fp32 scale (blockwise) or four e8m0 bytes, one per 32
 * consecutive contraction elements of the 128-element step (MXFP8).
 *   MOE_VIEW_QUEUE  the overlapped forward's schedule (MOE_FLAG_OVERLAP), as
 *                   its last launch wrote it: int32 control words, dispatch
 *                   flags, W1-done counters and per-XCD ticket tables. */
enum moe_view {
  MOE_VIEW_XPERM = 0, MOE_VIEW_H = 1, MOE_VIEW_A = 2, MOE_VIEW_O = 3,
  MOE_VIEW_DYPERM = 4, MOE_VIEW_DH = 5, MOE_VIEW_DXPERM = 6, MOE_VIEW_WPERM = 7,
  MOE_VIEW_Q_ROWS = 8, MOE_VIEW_Q_ROWS_SCALE = 9, MOE_VIEW_Q_TOK_A = 10,
  MOE_VIEW_Q_TOK_A_SCALE = 11, MOE_VIEW_Q_TOK_B = 12, MOE_VIEW_Q_TOK_B_SCALE = 13,
  MOE_VIEW_QUEUE = 14
};
int moe_scratch_view(const moe_desc* d, const void* scratch, size_t scratch_bytes,
                     int which, void** ptr, size_t* bytes);

/* Forward pass of the fused layer of the pages ("How does the fused kernel
 * work?": dispatch, the two expert linear layers with SwiGLU, combine, with
 * intermediates in scratch memory).  Runs the routing step, the dispatch
 * (x -> expert-contiguous rows), expert linear 1 with SwiGLU fused into its
 * epilogue, expert linear 2,
 * and the weighted combine y_t = sum_k w[t,k] o_{t,k} (an fp32 gather-reduce in
 * ascending k, rounded once).  In MOE_BF16 and MOE_FP8_BWD at D % 64 == 0 and
 * 2F % 256 == 0 the dispatch is part of expert linear 1 (its loader gathers x's
 * rows); in MOE_BF16 there the weights also enter in that GEMM's epilogue
 * (w * silu(g) * u), so the combine sums w * o rows.  Writes `y`; leaves the
 * routing metadata and the intermediates needed by moe_bwd in `scratch`.
 * `wprep` is ignored in the bf16/fp32 modes. */
int moe_fwd(const moe_desc* d, const void* x, const int32_t* topk_idx, const float* topk_w,
            const void* w1, const void* w2, const void* wprep, void* y,
            void* scratch, size_t scratch_bytes, void* stream);

/* Backward pass of the fused layer (the training pass the pages add to the
 * kernel: "How does the fused kernel work?", and the Russian page's
 * "Объединённое ядро, дополненное для обучения"), for the forward that last
 * used `scratch` (which must be passed back unmodified, with the same
 * descriptor, topk_w and weights).  It reads that forward's routing, x_perm
 * and saved intermediates from `scratch`, so it takes neither x nor topk_idx.
 * Steps:
 * combine-backward (dispatch of w * dy to the expert rows, and the
 * routing-weight gradient dtopk_w[t,k] = <dy_t, o_{t,k}> from the saved expert
 * output, an fp32 dot product), the W2 dgrad with SwiGLU-backward fused into
 * its epilogue, the W2 and W1 wgrads (per-expert reductions over that expert's
 * tokens, no atomics), the W1 dgrad and the un-permute reduction of dx (fp32
 * sum over k).  In MOE_BF16 at D % 64 == 0 and 2F % 256 == 0, dy is
 * dispatched unscaled and the W2 dgrad's epilogue applies w and forms
 * dtopk_w[t,k] as sum_f (dy_t W2^T)[f] a_{t,k}[f] (the same value in exact
 * arithmetic, a_{t,k} recomputed from the saved H), summed over 64-column
 * partials in column order.  Overwrites dx, dw1, dw2 (experts with no tokens get zeros) and
 * dtopk_w (0 for a slot whose expert id is out of range). */
int moe_bwd(const moe_desc* d, const void* dy, const float* topk_w,
            const void* w1, const void* w2, const void* wprep,
            void* dx, void* dw1, void* dw2, float* dtopk_w,
            void* scratch, size_t scratch_bytes, void* stream);

/* moe_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward with the same kernels and results as moe_fwd, run in a scratch
 * buffer the library owns instead of the caller's.  That buffer is a device
 * array of MOE_NOALLOC_SCRATCH_BYTES; each GPU the library runs on holds its
 * own copy from the first call on that device until the process ends.  The
 * call allocates nothing (make the first call on a device outside graph
 * capture: it resolves the array's address).  Descriptors whose
 * moe_scratch_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES return MOE_ESCRATCH (at
 * the Qwen3-30B shape, about 1,300 tokens at top-8); invalid ones return what
 * moe_fwd returns.  Arguments, layouts and the other errors are moe_fwd's.
 * The saved state stays in the library's buffer, so moe_bwd cannot follow this
 * call (it is a forward for inference), and an expert id out of range is
 * skipped as in moe_fwd but not reported (moe_check needs the scratch).  Every
 * call on a GPU shares that GPU's buffer and keeps the last call's contents:
 * calls that overlap on one GPU (different streams or threads) race. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int moe_fwd_noalloc(const moe_desc* d, const void* x, const int32_t* topk_idx,
                    const float* topk_w, const void* w1, const void* w2, const void* wprep,
                    void* y, void* stream);

/* Router ahead of the layer (the step that makes the top-k routing decision the
 * layer consumes: Prime Mega MoE news item, "TL;DR", 128 experts with top-8
 * routing, and "Why is MoE training communication-bound?", each token goes to a
 * small subset of experts).  Per token t, with logits z = logits[t, 0..E-1]:
 *   p = softmax(z); the K experts of largest p in descending order, ties to the
 *   lower expert index (the selection is exactly that of the logits);
 *   topk_w[t,k] = p[topk_idx[t,k]] / sum_k' p[topk_idx[t,k']] (fp32).
 * Reads only T, E, K of `d`: requires T >= 0, 1 <= K <= E (else MOE_EINVAL),
 * E <= 512 and K <= 64 (else MOE_EUNSUPPORTED).  logits: device float32
 * [T, E] row-major, not NaN; topk_idx: device int32 [T, K] and topk_w: device
 * float32 [T, K], written (the layout moe_fwd reads).  A token whose logits are
 * all -inf gets NaN weights, as the definition does.  All pointers 4-byte
 * aligned (MOE_EALIGN).  With T = 0 it returns MOE_OK and touches nothing
 * (pointers may be null).  Asynchronous on `stream`; allocates nothing. */
int moe_router_fwd(const moe_desc* d, const float* logits, int32_t* topk_idx, float* topk_w,
                   void* stream);

/* Router backward: dlogits = dL/dlogits for the upstream gradient
 * dtopk_w = dL/dtopk_w [T, K] (for instance moe_bwd's), by the chain rule
 * through the renormalisation and the softmax, which reduces to
 * dlogits[t, j] = w_j (dw_j - sum_k w_k dw_k) for a selected expert j and 0 for
 * every other expert.  topk_idx and topk_w are moe_router_fwd's outputs
 * (distinct ids per token; ids outside [0, E) are skipped).  dlogits: device
 * float32 [T, E], every entry written.  Same requirements as moe_router_fwd. */
int moe_router_bwd(const moe_desc* d, const int32_t* topk_idx, const float* topk_w,
                   const float* dtopk_w, float* dlogits, void* stream);

/* Synchronizes `stream`, returns the latched device error (MOE_OK, MOE_EINDEX
 * or MOE_ETIMEOUT) of `scratch` and clears it.  Error reporting of this
 * library (the pages define no error interface): the descriptor and scratch
 * size locate the error word and check the buffer (MOE_ESCRATCH). */
int moe_check(const moe_desc* d, void* scratch, size_t scratch_bytes, void* stream);

/* Text of a status code (static string, host). */
const char* moe_strerror(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Opt-in kernel profiler (process-wide, for benchmarks).  While enabled, every
 * kernel the library launches is bracketed by HIP events recorded on the
 * stream it is launched on.  moe_profile_collect synchronizes those events,
 * adds their durations to per-kernel totals and returns the number of distinct
 * kernels; moe_profile_get reads entry i (name valid until the next reset);
 * moe_profile_reset clears the totals. */
int moe_profile_enable(int on);
int moe_profile_collect(void);
int moe_profile_get(int i, const char** name, double* total_ms, int64_t* launches);
int moe_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
