/*
 * ttt.h — C ABI of the MI355X (gfx950) chunk-wise fast-weight library.
 *
 * The library runs the hot path of In-Place Test-Time Training for one gated
 * MLP layer whose final projection W_down is the fast weight (paperlayer.ai
 * summary, sec. 3 "In-Place Adaptation"; iplexlaw.co.kr walkthrough, sec. 2):
 *
 *   Z        = SiLU(x W_gate^T) * (x W_up^T)          (W_up, W_gate frozen)
 *   V[t]     = E_tgt[ids[t+1]]                         (next-token target row)
 *   chunk i  : y[chunk i] = Z[chunk i] W_{i-1}^T       (apply, pre-update state)
 *              W_i = W_{i-1} + eta V[chunk i]^T Z[chunk i]   (update)
 *
 * The update rule is the pages' simplified form dW_down = eta V^T Z
 * (iplexlaw sec. 2 and sec. 4); apply-then-update over non-overlapping chunks
 * follows iplexlaw sec. 3 and paperlayer sec. 3 "Chunk-Wise Updates"; the
 * target is V^ = Conv1D(X0) W_target with the kernel reduced to the next-token
 * tap and W_target folded into E_tgt (paperlayer sec. 3 "LM-Aligned
 * Objective"); state reset at document ends follows paperlayer App. B.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     row-major, densely packed, owned by the caller. They must stay valid
 *     until the work queued on `hip_stream` has completed.
 *   - `hip_stream` is a hipStream_t (NULL = the default stream). Work is
 *     queued asynchronously; no call synchronises the host except where noted.
 *   - Argument errors are detected before any device work is queued.
 *   - Return value 0 = success; a negative TTT_E_* code otherwise, with a
 *     message available from ttt_last_error() (thread-local).
 *   - No C++ exception crosses the ABI. A handle is not thread-safe: calls on
 *     one handle must come from one thread at a time and, when they are on
 *     different streams, be ordered by the caller.
 *   - Only gfx950 devices are accepted (TTT_E_NODEV otherwise).
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ttt_handle ttt_handle; /* opaque, owned by the library */

/* Activation/weight element type. The fast-weight state is always fp32.
 * The handle keeps each sequence's fast weight as D = W - W_down0, the change
 * since its last reset, in fp32 (W_down0 is kept beside it): the updates are
 * small next to W, and held this way they accumulate with fp32 relative
 * precision even when each one is far below the fp32 resolution of W itself
 * (as with clipped updates), also across calls.
 * TTT_F32:  x, W_up, W_gate, W_down0, E_tgt and y are float.
 * TTT_BF16: they are bfloat16 (uint16 bit patterns); matrix products run on
 *           bf16 MFMA with fp32 accumulation. */
typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

enum {
  TTT_OK = 0,
  TTT_E_NULL = -1,  /* a required pointer is NULL                           */
  TTT_E_SHAPE = -2, /* a size is out of range or violates an alignment rule */
  TTT_E_DTYPE = -3, /* unknown dtype                                         */
  TTT_E_NOMEM = -4, /* device allocation failed                              */
  TTT_E_HIP = -5,   /* a HIP runtime call or kernel launch failed            */
  TTT_E_NODEV = -6, /* no device, or the current device is not gfx950        */
  TTT_E_ARG = -7    /* other invalid argument (e.g. batch index, non-finite eta) */
};

/*
 * ttt_init — create a handle for one layer.
 *
 *   W_up, W_gate : [f][d] frozen up and gate projections (dtype `dt`).
 *   W_down0      : [d][f] initial fast weight (dtype `dt`). The three
 *                  weight pointers must be 16-byte aligned.
 *   d, f         : model width and hidden width, at most 65536; multiples of
 *                  64 on the fp32 path and of 256 on the bf16 path (the MFMA
 *                  kernels work on whole 256 x 256 tiles of the state).
 *   C            : chunk length in tokens, C >= 1. Chunks are counted from the
 *                  first token of each ttt_forward_chunked call.
 *   eta          : learning rate of the update (finite).
 *   max_batch    : number of independent sequences (fast-weight states) the
 *                  handle holds, 1 .. 4096.
 *
 * The library copies the weights into buffers it owns (re-laid out for its
 * kernels) and keeps an fp32 image of W_down0. Every state starts equal to
 * W_down0. The caller may free its weight buffers once the queued copies have
 * completed on `hip_stream`. On success *out receives the handle; on failure
 * *out is set to NULL and nothing is leaked.
 */
int ttt_init(ttt_handle **out, const void *W_up, const void *W_gate, const void *W_down0, int d, int f,
             int C, float eta, ttt_dtype dt, int max_batch, void *hip_stream);

/*
 * ttt_forward_chunked — run the chunk-wise apply-then-update scan over one
 * block of tokens for sequences 0 .. B-1.
 *
 *   x       : [B][T][d] layer input (dtype of the handle).
 *   ids     : [B][T+1] int32 token ids; ids[b][t] is the token at position t
 *             and ids[b][T] the look-ahead token after the block. The target
 *             of position t is row ids[b][t+1] of E_tgt; an id outside
 *             [0, vocab) (e.g. -1 at a document end) gives a zero target row.
 *   E_tgt   : [vocab][d] target-embedding table (dtype of the handle).
 *   B       : 0 .. max_batch. T: tokens per sequence, 0 .. 2^23.
 *   y       : [B][T][d] output (dtype of the handle), written in full.
 *   W_final : optional [B][d][f] fp32 output; receives each sequence's fast
 *             weight after the block, W_down0 + D rounded to fp32 (NULL = not
 *             wanted). ttt_state_delta gives D itself.
 *
 * x, E_tgt and y must be 16-byte aligned (TTT_E_ARG otherwise).
 *
 * Each sequence starts from its current state (W_down0 after init or reset,
 * else what the previous call left) and keeps the final state in the handle,
 * so consecutive calls continue one stream (the last chunk of a call may be
 * short; to continue chunking seamlessly, make T a multiple of C). Scratch
 * memory is allocated by the library on first use and grown when B*T grows;
 * that allocation is the only point where this call may block the host.
 */
int ttt_forward_chunked(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab, int B,
                        int T, void *y, float *W_final, void *hip_stream);

/*
 * ttt_forward_chunked_noalloc — ttt_forward_chunked for callers that cannot
 * allocate device memory during the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * layouts, semantics and results (bit for bit) as ttt_forward_chunked, but the
 * scratch of the call (target rows, Z, snapshots, group scores,
 * clipping partials) lives in a fixed workspace of
 * TTT_NOALLOC_WORKSPACE_BYTES inside the library: a file-scope device array
 * that each GPU the library runs on holds until the process ends, its address
 * taken in ttt_init. The call performs no hipMalloc, hipFree or other
 * allocation. A call whose scratch would exceed the workspace returns
 * TTT_E_SHAPE before any device work, naming the bytes it needs (roughly
 * B*T*(4f + 2d) bytes plus 2*d*f per group of the plan on the bf16 path, so
 * small layers and short blocks; larger calls use ttt_forward_chunked).
 * Every call on one GPU shares that GPU's workspace, whichever handle it
 * comes from, and leaves its contents behind (each call writes every part it
 * reads): calls that overlap in time on one GPU, e.g. on two streams, race
 * and must be ordered by the caller.
 */
#define TTT_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int ttt_forward_chunked_noalloc(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab,
                                int B, int T, void *y, float *W_final, void *hip_stream);

/*
 * ttt_forward_docs — ttt_forward_chunked over streams that pack several
 * documents (paperlayer App. B; iplexlaw sec. 6: the fast weight returns to its
 * initial value at document boundaries, so no state crosses between
 * independent documents).
 *   doc_counts : host array [B]; doc_counts[b] documents start inside
 *                sequence b's block besides the one it opens with (0 .. T-1).
 *   doc_starts : host array, the concatenated start positions: sequence b's
 *                are the next doc_counts[b] entries, strictly increasing inside
 *                (0, T). NULL allowed when every count is 0.
 * The first document continues the sequence's current state (like
 * ttt_forward_chunked); at every listed start the state returns to W_down0 and
 * chunking restarts from that token. A document's last target row lies in its
 * last chunk, whose update the reset discards, so no target crosses a
 * document end. The final state is the last document's, kept in the handle as
 * usual. On a bf16 handle with eta != 0 (also with clipping and the general
 * target) the call is one launch sequence in which every document is a
 * sequence of its own, with its own scratch slots and snapshot groups, and
 * the state a sequence's last document leaves is copied back once at the end.
 * On an fp32 handle, or with eta = 0, documents run one after the other on
 * the stream (B = 1 launches per document). With profiling on,
 * ttt_phase_times sums a call's launch sequences.
 * Other arguments, ownership and errors as ttt_forward_chunked.
 */
int ttt_forward_docs(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab, int B, int T,
                     const int32_t *doc_starts, const int32_t *doc_counts, void *y, float *W_final,
                     void *hip_stream);

/*
 * ttt_reset — restore the fast weight of sequence b (or of every sequence if
 * b == -1) to W_down0 (D = 0): the document-boundary reset (paperlayer App. B;
 * iplexlaw sec. 6). Queued on `hip_stream`.
 */
int ttt_reset(ttt_handle *h, int b, void *hip_stream);

/* ttt_destroy — free the handle and everything it owns (synchronises the device). NULL is a no-op. */
void ttt_destroy(ttt_handle *h);

/* ttt_last_error — message for the last nonzero return on this thread ("" if none). */
const char *ttt_last_error(void);

/*
 * ttt_set_group_chunks — tuning knob of the two-level scan (no effect on the
 * result beyond rounding). The library keeps each state resident across the
 * whole block of tokens and takes a snapshot of it (bf16 on the bf16 path,
 * fp32 on the fp32 path) at the start of every group of G chunks; the outputs
 * of a group are formed from its snapshot plus the block-causal term of the
 * earlier chunks inside the group. This is the pages' exclusive prefix over
 * chunk updates (iplexlaw sec. 6; paperlayer App. B) taken at two levels.
 * G = 0 restores the default (about 1024 tokens per group, rounded so that
 * G*C is a multiple of 64). G*C must be a multiple of 64; TTT_E_SHAPE
 * otherwise.
 */
int ttt_set_group_chunks(ttt_handle *h, int G);

/*
 * ttt_plan — host-only query of the layout a call with T tokens and chunk C
 * would use (no device work; usable without a GPU):
 *   *G       : chunks per snapshot group;  *L = G*C tokens per group;
 *   *ngroups : groups in the call (ceil(T / L));
 *   *T_pad   : token slots per sequence in the scratch buffers (T rounded up to 256).
 * When C >= T the call is a single chunk and C is taken as T.
 * Any output pointer may be NULL. `G_override` as in ttt_set_group_chunks.
 */
int ttt_plan(int T, int C, int G_override, int *G, int *L, int *ngroups, int *T_pad);

/*
 * ttt_set_target_conv — the general LM-aligned target V^ = Conv1D(X0) W_target
 * (paperlayer sec. 3 "LM-Aligned Objective"; iplexlaw sec. 4 and sec. 6, a
 * depthwise kernel of size 5 over the token embeddings and a learnable
 * projection) in place of the next-token rows of E_tgt.
 *   conv_w   : [K][d] depthwise tap weights (dtype of the handle); tap k of
 *              target row t reads the embedding of the token at position
 *              t+1+k (ids[b][t+1+k]).
 *   K        : 1 .. 64 taps; K = 0 restores the next-token target (the other
 *              arguments are then ignored).
 *   W_target : [d][d] projection (dtype of the handle): V^[t] = U[t] W_target.
 * After this call the E_tgt argument of ttt_forward_chunked is the token
 * embedding table X0 [vocab][d]. The chunk boundary pads the convolution: row t
 * of chunk i uses tap positions only up to min((i+1)C, T), the first token of
 * the next chunk (already that chunk's input); later taps are zero, so no output
 * depends on a later token. With K = 1, conv_w = 1 and W_target = I the result
 * equals the next-token target. Both arrays are copied (the caller may free
 * them once the stream has run the copy); they must be 16-byte aligned.
 * Synchronises `hip_stream`. Adds [B][T][d] of scratch per forward.
 */
int ttt_set_target_conv(ttt_handle *h, const void *conv_w, int K, const void *W_target, void *hip_stream);

/*
 * ttt_set_clip — Frobenius-norm clipping of each chunk update (paperlayer
 * App. C.2 "Inference Stability", threshold 1e-5 in the reported long-context
 * evaluations; iplexlaw sec. 6): with tau > 0, chunk i's update
 * dW_i = eta V_i^T Z_i is applied as dW_i * min(1, tau / ||dW_i||_F), in the
 * state and in the outputs of later chunks alike. tau = 0 or +inf turns it
 * off (the default); tau < 0 or NaN returns TTT_E_ARG. The norm is taken from
 * the chunk Grams, ||V_i^T Z_i||_F^2 = sum_{s,t in chunk i} <v_s,v_t><z_s,z_t>,
 * in fp32. Applies to later ttt_forward_chunked calls; needs extra scratch:
 * small fp32 buffers; on a bf16 handle 1 KB per token slot and per 256-token
 * span of a chunk (the Gram kernel's fp32 partial products: 128 MB at
 * T = 131072, C = 256); plus [B][T][d] target rows in the handle's dtype on
 * an fp32 handle or with the general target (a bf16 handle with the plain
 * target reads the rows from E_tgt through the ids when vocab*d*2 < 2^31).
 */
int ttt_set_clip(ttt_handle *h, float tau);

/*
 * ttt_state_delta — copy D = W - W_down0 of sequences 0 .. B-1, the change of
 * each fast weight since its last reset (or init), to dW ([B][d][f] fp32,
 * device, 16-byte aligned), queued on `hip_stream` after the work already
 * there. Where the updates are much smaller than W (clipped updates at the
 * pages' tau = 1e-5 move each element by about 1e-9 against |W| ~ 1e-2), the
 * fp32 W_final cannot resolve them (its rounding alone is about 3% of D
 * there), while D carries them at fp32 relative precision. B in [0,
 * max_batch] (TTT_E_SHAPE otherwise); dW NULL with B > 0 is TTT_E_NULL.
 */
int ttt_state_delta(ttt_handle *h, float *dW, int B, void *hip_stream);

/*
 * ttt_set_output_f32 — on a bf16 handle, later forward calls write y as fp32
 * ([B][T][d] float, 4 bytes per element) instead of bf16: the output GEMM's
 * fp32 accumulators are stored without the final rounding to bf16. The
 * fast-weight contribution to y is often a small fraction of y (a few percent
 * on short streams), and bf16 rounding of y alone then blurs it by up to
 * 2^-9 |y|; callers that keep a residual stream in fp32 avoid that rounding.
 * on = 0 restores bf16 y. No effect on an fp32 handle (y is always fp32).
 * Returns TTT_E_NULL for a NULL handle.
 */
int ttt_set_output_f32(ttt_handle *h, int on);

/*
 * ttt_set_profiling / ttt_phase_times — per-phase device timing of the
 * forward calls, from HIP events recorded on their streams.
 * Phases: 0 target gather, 1 up/gate GEMM + SwiGLU, 2 clipping factors
 * (0 when clipping is off), 3 state update with snapshots, 4 within-group
 * scores, 5 output GEMM, 6 final-state copy. With clipping on a bf16 handle
 * and the plain target, the gather runs after the factors (it applies them)
 * and counts in phase 2.
 * Each launch sequence (a ttt_forward_chunked call, or one document of a
 * ttt_forward_docs call) records one set of events in a ring of 16 sets, so
 * calls need not wait for each other. ttt_phase_times waits for the sets
 * recorded since the previous read and writes `n` (<= 7) milliseconds per
 * phase to ms[]: the sum over those sets divided by the number of forward
 * calls among them (the mean per call; a call with documents sums them).
 * With no call since the previous read it writes the previous figures again.
 * A phase that did not run reads only the spacing of its two events (a few
 * microseconds). When a launch sequence finds all 16 sets unread, the oldest
 * is folded into running sums first (the host waits for that set, recorded
 * 16 sequences earlier, to complete), so any number of calls or documents
 * may come between two reads. ttt_set_profiling resets the window.
 */
int ttt_set_profiling(ttt_handle *h, int on);
int ttt_phase_times(ttt_handle *h, float *ms, int n);

/* ttt_workspace_bytes — device bytes the handle currently owns (weights, states, scratch). */
int ttt_workspace_bytes(ttt_handle *h, size_t *bytes);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H */
