/*
 * wkv7.h -- C ABI of libwkv7: the RWKV-7 WKV7 time-mix recurrence, forward
 * and backward, on AMD Instinct MI355X (gfx950).
 *
 * The operation (rwkv-mlx page, section "Metal kernel architecture",
 * forward block, in its per-element reading): every head (b, h) carries a
 * D x D fp32 state S, rows i paired with v and y, columns j paired with r, w,
 * k, a and b.  Per token t:
 *
 *     sa[i]   = sum_j S[i][j] a_t[j]                 (state before the update)
 *     S[i][j] = w_t[j] S[i][j] + v_t[i] k_t[j] + sa[i] b_t[j]
 *     y_t[i]  = sum_j S[i][j] r_t[j]                 (state after the update)
 *
 * The backward walks the sequence in reverse from per-chunk state
 * checkpoints (same section, backward block, and the paragraph after it on
 * why checkpoints are kept every 32 tokens).  Unlike the page's design, this
 * library never reconstructs an earlier state by dividing by w: it re-runs
 * each chunk forward from its checkpoint.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - D must be 64.  B, T, H must be >= 1.  CHUNK = 32; NC = ceil(T / 32).
 * - Token tensors (r, w, k, v, a, b, y, dy and the six input gradients) are
 *   dense row-major (B, T, H, D): element (b,t,h,d) at ((b*T + t)*H + h)*D + d.
 * - State tensors (h0, hT, dhT, dh0) are dense row-major (B, H, D, D) with
 *   S[i][j] at i*D + j.  Checkpoints are (B, H, NC, D, D); checkpoint c is the
 *   state ENTERING chunk c, i.e. after 32*c tokens (checkpoint 0 is h0).
 * - r, w, k, v, a, b share one storage type, `in_dtype` (fp32 or bf16).
 *   Everything else is fp32.  All arithmetic is fp32 (fp32 accumulation;
 *   with bf16 inputs the matrix-core products use a two-term bf16 split of
 *   every fp32 operand, good to about 2^-17 relative per product).
 * - Decay w must lie in [1/8, 1].  (RWKV-7's decay exp(-e^-0.5 * sigmoid(x))
 *   lies in (0.545, 1).)  Within a chunk, running products of up to 32 decays
 *   and their reciprocals are used as scale factors; at w >= 1/8 they stay
 *   within 2^-96 .. 2^96.  Values outside the range are not detected and give
 *   unspecified (possibly non-finite) results.  NaN/Inf inputs propagate.
 * - Every pointer must be a device pointer (hipMalloc'd or equivalent) aligned
 *   to 16 bytes.  Optional pointers may be NULL where stated.
 * - The library allocates nothing, frees nothing and keeps no pointer after a
 *   call returns.  Its only mutable global state is a per-device, per-kernel
 *   flag recording that the kernel's dynamic LDS limit has been raised, set
 *   once under a lock by the first launch on that device.  Every entry point
 *   may therefore be called from several host threads at once; calls on
 *   different streams may run concurrently if their outputs do not overlap.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every entry point is
 *   asynchronous: it only enqueues kernels and never synchronises.
 * - Argument, shape, alignment, workspace and aliasing errors are detected on
 *   the host BEFORE anything is enqueued; no output is touched then.  A
 *   failed launch returns WKV7_ERR_HIP.  Faults during execution surface at
 *   the caller's next synchronisation.
 * - Outputs must not overlap each other or any input, except where an entry
 *   point allows it explicitly (hT may equal h0).
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WKV7_OK = 0,
    WKV7_ERR_ARG = 1,       /* NULL where a pointer is required, bad enum   */
    WKV7_ERR_SHAPE = 2,     /* D != 64, B/T/H < 1, sizes overflowing int64,
                               or B*T*H*D*4 > 0xFFFFFF00: token tensors are
                               addressed with 32-bit byte offsets (at D = 64,
                               B*T*H below 2^24); split larger batches.
                               Checkpoints and state gradients are addressed
                               per chunk with 64-bit bases, so they set no
                               further limit (B = H = 1 allows T up to
                               16,777,215, 8 GiB of checkpoints)            */
    WKV7_ERR_DTYPE = 3,     /* in_dtype not a wkv7_dtype                    */
    WKV7_ERR_ALIGN = 4,     /* a pointer not 16-byte aligned                */
    WKV7_ERR_ALIAS = 5,     /* an output overlaps an input or another output */
    WKV7_ERR_HIP = 6,       /* kernel launch failed                         */
    WKV7_ERR_WORKSPACE = 7  /* workspace NULL or smaller than required      */
} wkv7_status;

typedef enum {
    WKV7_F32 = 0,
    WKV7_BF16 = 1
} wkv7_dtype;

/* Library version, major*10000 + minor*100 + patch. */
int wkv7_version(void);

/* Chunk length used for checkpoints (32). */
int wkv7_chunk_len(void);

/* NC = ceil(T / 32) for T >= 1; 0 for T < 1. */
int64_t wkv7_num_chunks(int64_t T);

/* Static string naming a status code (never NULL). */
const char *wkv7_status_str(int status);

/* Bytes of the chunk operands (see wkv7_chunk_prepare): B*H*NC*(4096 + 36864).
 * 0 for invalid shapes. */
size_t wkv7_chunk_ops_bytes(int B, int T, int H, int D);

/* Bytes of device workspace wkv7_fwd needs: wkv7_chunk_ops_bytes(...) when
 * T > 1, else 0.  0 for invalid shapes. */
size_t wkv7_fwd_workspace_bytes(int B, int T, int H, int D);

/* Bytes of device workspace wkv7_bwd needs: one fp32 D x D state gradient per
 * chunk (B*H*NC*D*D*4) plus wkv7_chunk_ops_bytes(...).  0 for invalid shapes. */
size_t wkv7_bwd_workspace_bytes(int B, int T, int H, int D);

/*
 * Per-chunk operands of the chunked evaluation: everything about a chunk
 * that depends on its r, w, k, a, b but not on the state.  Within chunk c
 * (tokens 32c .. 32c+31; a shorter last chunk is padded with w = 1 and
 * r = k = a = b = 0) let g_t be the running product of w over the chunk's
 * tokens up to t.  Unrolling the forward block of the rwkv-mlx page ("Metal
 * kernel architecture") over the chunk gives, for the state S0 entering the
 * chunk and the chunk's v rows V,
 *     S_end = S0 P + V^T M,      Y = E S0^T + F V,
 * and for the backward block, with G the gradient at the chunk's end,
 *     G_start = G P^T + DY^T E,  dv = M G^T + F^T DY,
 * where P (D x D), M, E (32 x D) and F (32 x 32) depend on r, w, k, a, b only
 * (through the decays g and the 32 x 32 coupling
 *     L[t][s] = sum_j a_t[j] g_{t-1}[j] b_s[j] / g_s[j]  for s < t
 * of token s's b into token t's sa; P, M, E, F involve (I - L)^-1).
 *
 * chunk_ops receives, in this order:
 *   (B, H, NC, 32, 32) fp32: (I - L)^-1 of every chunk, row-major;
 *   (B, H, NC) blocks of 36864 bytes: P, M, E, F of every chunk, in a
 *   library-internal format (bf16 hi/lo planes for bf16 inputs, fp32 for
 *   fp32 inputs).  Only this library's kernels read them.
 * The forward and the backward of one step may share one chunk_ops.
 *
 *   r, w, k, a, b : (B,T,H,D), in_dtype, required.
 *   chunk_ops     : output, required, wkv7_chunk_ops_bytes(...) bytes.
 */
wkv7_status wkv7_chunk_prepare(int B, int T, int H, int D, wkv7_dtype in_dtype,
                               const void *r, const void *w, const void *k,
                               const void *a, const void *b,
                               void *chunk_ops, void *stream);

/*
 * Forward (rwkv-mlx page, "Metal kernel architecture", forward block).
 *
 *   r, w, k, v, a, b : (B,T,H,D), in_dtype, required.
 *   h0               : (B,H,D,D) fp32 initial state, or NULL for zero.
 *   y                : (B,T,H,D) fp32 output, or NULL if not wanted.
 *   h_ckpt           : (B,H,NC,D,D) fp32 checkpoints, or NULL (inference:
 *                      nothing kept for a backward).
 *   hT               : (B,H,D,D) fp32 final state, or NULL.  hT may be the
 *                      same pointer as h0 (state updated in place), but must
 *                      not otherwise overlap h0.
 *   workspace        : device scratch of wkv7_fwd_workspace_bytes(...) bytes;
 *                      may be NULL when that is 0 (T == 1).  Clobbered; on
 *                      return it holds the chunk operands (wkv7_chunk_prepare).
 * At least one of y, h_ckpt, hT must be non-NULL.
 * Equivalent to wkv7_chunk_prepare into the workspace, then wkv7_fwd_scan.
 */
wkv7_status wkv7_fwd(int B, int T, int H, int D, wkv7_dtype in_dtype,
                     const void *r, const void *w, const void *k,
                     const void *v, const void *a, const void *b,
                     const float *h0, float *y, float *h_ckpt, float *hT,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): wkv7_fwd without a
 * workspace argument.  The chunk operands go to a static device array of
 * wkv7_fwd_noalloc_max_bytes() bytes (128 MiB) inside the library, one copy
 * per GPU, held until the process ends; its device address is looked up once
 * per device on the first call there.  Nothing is allocated or freed by the
 * call itself.
 *
 *   Arguments, results and errors as wkv7_fwd (T == 1 uses no scratch).
 *   WKV7_ERR_WORKSPACE: the call would need more than
 *     wkv7_fwd_noalloc_max_bytes() of chunk operands, i.e.
 *     wkv7_fwd_workspace_bytes(B,T,H,D) > 128 MiB (B*H*NC > 3276 chunks);
 *     detected on the host, nothing is enqueued.
 *   WKV7_ERR_HIP: the scratch's address could not be looked up.
 * All calls on one GPU share that GPU's array and leave their chunk operands
 * in it: two calls that overlap in time on one GPU (different streams, or
 * host threads without ordering) race and give wrong results.  Calls in
 * order on one stream are safe.
 */
size_t wkv7_fwd_noalloc_max_bytes(void);
wkv7_status wkv7_fwd_noalloc(int B, int T, int H, int D, wkv7_dtype in_dtype,
                             const void *r, const void *w, const void *k,
                             const void *v, const void *a, const void *b,
                             const float *h0, float *y, float *h_ckpt, float *hT,
                             void *stream);

/*
 * Forward given the chunk operands (from wkv7_chunk_prepare for the same r, w,
 * k, a, b): the state is carried from chunk to chunk, S_end = S0 P + V^T M,
 * and every chunk's y = E S0^T + F V.  Arguments as wkv7_fwd; chunk_ops is
 * required.
 */
wkv7_status wkv7_fwd_scan(int B, int T, int H, int D, wkv7_dtype in_dtype,
                          const void *v, const void *chunk_ops, const float *h0,
                          float *y, float *h_ckpt, float *hT, void *stream);

/*
 * Backward (rwkv-mlx page, "Metal kernel architecture", backward block:
 * chunks in reverse from the checkpoints, producing dr, dw, dk, dv, da, db).
 *
 *   dy               : (B,T,H,D) fp32 gradient of the loss w.r.t. y, required.
 *   dhT              : (B,H,D,D) fp32 gradient w.r.t. the final state, or NULL
 *                      for zero.
 *   r..b             : the forward's inputs, in_dtype, required.
 *   h_ckpt           : (B,H,NC,D,D) checkpoints written by wkv7_fwd for the
 *                      same inputs and h0, required.
 *   dr,dw,dk,dv,da,db: (B,T,H,D) fp32 outputs, required.
 *   dh0              : (B,H,D,D) fp32 gradient w.r.t. h0, or NULL.
 *   workspace        : device scratch of at least
 *                      wkv7_bwd_workspace_bytes(B,T,H,D) bytes, required; its
 *                      contents on entry do not matter and are clobbered.
 * Equivalent to wkv7_chunk_prepare (into the workspace after its first
 * part), wkv7_bwd_scan (the workspace's first part as dh_ckpt), then
 * wkv7_bwd_inputs.
 */
wkv7_status wkv7_bwd(int B, int T, int H, int D, wkv7_dtype in_dtype,
                     const float *dy, const float *dhT,
                     const void *r, const void *w, const void *k,
                     const void *v, const void *a, const void *b,
                     const float *h_ckpt,
                     float *dr, float *dw, float *dk, float *dv,
                     float *da, float *db, float *dh0,
                     void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Backward, first stage: the gradient w.r.t. the state at every chunk
 * boundary, walking the chunks in reverse (rwkv-mlx page, "Metal kernel
 * architecture", backward block), and dv.  The state gradient obeys its own
 * recurrence, driven by dy and the chunk operands: G_start = G P^T + DY^T E,
 * dv = M G^T + F^T DY.  Needs neither the inputs nor the checkpoints.
 *
 *   dy, dhT  : as for wkv7_bwd.
 *   chunk_ops: from wkv7_chunk_prepare for the forward's r, w, k, a, b.
 *   dh_ckpt  : (B,H,NC,D,D) fp32 output, required: dh_ckpt[c] is the gradient
 *              w.r.t. checkpoint c (the state entering chunk c).
 *   dv       : (B,T,H,D) fp32 output (the gradient w.r.t. v), or NULL.
 *   dh0      : (B,H,D,D) fp32 output (equals dh_ckpt[0]), or NULL.
 */
wkv7_status wkv7_bwd_scan(int B, int T, int H, int D, wkv7_dtype in_dtype,
                          const float *dy, const float *dhT, const void *chunk_ops,
                          float *dh_ckpt, float *dv, float *dh0, void *stream);

/*
 * Backward, second stage: dr, dw, dk, da, db for every token, all chunks in
 * parallel, each chunk recomputed forward from its checkpoint (never by
 * dividing by w).
 *
 *   dy, dhT, r..b, h_ckpt : as for wkv7_bwd.
 *   chunk_ops: from wkv7_chunk_prepare for the same inputs, required (only
 *              its (I - L)^-1 part is read).
 *   dh_ckpt  : (B,H,NC,D,D) written by wkv7_bwd_scan for the same inputs.
 *   dr, dw, dk, da, db : (B,T,H,D) fp32 outputs, required.
 */
wkv7_status wkv7_bwd_inputs(int B, int T, int H, int D, wkv7_dtype in_dtype,
                            const float *dy, const float *dhT,
                            const void *r, const void *w, const void *k,
                            const void *v, const void *a, const void *b,
                            const void *chunk_ops, const float *h_ckpt,
                            const float *dh_ckpt,
                            float *dr, float *dw, float *dk, float *da, float *db,
                            void *stream);

/*
 * Token-by-token forward (same definition as wkv7_fwd, same rules, no
 * workspace), evaluated one token after another on the vector units instead
 * of in chunks on the matrix cores.  This is the path wkv7_fwd itself takes
 * for one-token calls (the recurrent step of RNN-mode inference, RWKV-LM
 * README page, the pip-package usage that hands the state from call to
 * call).  Exposed so that callers can pick it explicitly.
 */
wkv7_status wkv7_fwd_sequential(int B, int T, int H, int D, wkv7_dtype in_dtype,
                                const void *r, const void *w, const void *k,
                                const void *v, const void *a, const void *b,
                                const float *h0, float *y, float *h_ckpt, float *hT,
                                void *stream);

/*
 * The layer with its time-mix prologue: w, a and b are not passed but formed
 * inside the kernels' loads from the layer's raw projections, per token and
 * head (the pages print no formula for this step; these are the definitions
 * of RWKV-7's decay, removal key and replacement key that the workloads use,
 * read as the layer's own arithmetic):
 *
 *     w[j] = exp(-e^-1/2 * sigmoid(w_raw[j]))
 *     kh   = kappa / |kappa|        (L2 norm over the head's D channels;
 *                                    a zero kappa gives kh = 0)
 *     a    = -kh,   b[j] = kh[j] * sigmoid(alpha[j])
 *
 * w_raw, kappa and alpha are (B,T,H,D) in_dtype, like r, k, v; w never exists
 * in memory, so the decay-range rule above is met by construction.
 *
 * wkv7_fwd_proj: as wkv7_fwd with (w_raw, kappa, alpha) in place of (w, a, b),
 * the same workspace rule included (wkv7_fwd_workspace_bytes; none for T == 1,
 * where the one-token step applies the prologue to its loads as well).
 */
wkv7_status wkv7_fwd_proj(int B, int T, int H, int D, wkv7_dtype in_dtype,
                          const void *r, const void *w_raw, const void *k,
                          const void *v, const void *kappa, const void *alpha,
                          const float *h0, float *y, float *h_ckpt, float *hT,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * wkv7_bwd_proj: as wkv7_bwd with (w_raw, kappa, alpha) in place of (w, a, b)
 * and the chain rule through the prologue applied before the stores:
 *
 *     dw_raw[j] = dw[j] * w[j] * (-e^-1/2) * s(1 - s),  s = sigmoid(w_raw[j])
 *     g         = -da + db * sigmoid(alpha)              (gradient w.r.t. kh)
 *     dkappa    = (g - kh (kh . g)) / |kappa|            (0 for kappa = 0)
 *     dalpha[j] = db[j] * kh[j] * s(1 - s),  s = sigmoid(alpha[j])
 *
 * dw_raw, dkappa, dalpha take the places of dw, da, db (fp32, required); the
 * other arguments and the workspace are as for wkv7_bwd, h_ckpt from
 * wkv7_fwd_proj.
 */
wkv7_status wkv7_bwd_proj(int B, int T, int H, int D, wkv7_dtype in_dtype,
                          const float *dy, const float *dhT,
                          const void *r, const void *w_raw, const void *k,
                          const void *v, const void *kappa, const void *alpha,
                          const float *h_ckpt,
                          float *dr, float *dw_raw, float *dk, float *dv,
                          float *dkappa, float *dalpha, float *dh0,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Diagnostic, not for training: the backward of the rwkv-mlx page's Metal
 * design ("Metal kernel architecture", backward block, and the paragraph
 * after it on error growth), which walks each chunk in reverse from an exact
 * state and rebuilds every earlier state by undoing the update, i.e. by
 * dividing by w, instead of recomputing it from a checkpoint as wkv7_bwd
 * does.  Rounding errors grow by about (1/w) per token walked, which is why
 * wkv7_bwd recomputes.  sa, which the division needs before the earlier state
 * is known, is solved from the update itself: with z = S_t[i] - v[i] k,
 * sa[i] = (z . (a / w)) / (1 + b . (a / w)) and S_{t-1}[i] = (z - sa[i] b) / w.
 * One wave per head, one state row per lane; slow by design.
 *
 *   dy, dhT, r..b : as for wkv7_bwd.
 *   h_ckpt        : checkpoints from wkv7_fwd; required when restart = 1.
 *   hT            : (B,H,D,D) final state from wkv7_fwd, required.
 *   restart       : 1 = each chunk's walk starts from the exact state at the
 *                   chunk's end (checkpoint c + 1, hT for the last chunk): at
 *                   most 32 divisions in a row, the page's design; 0 = one
 *                   walk over the whole sequence from hT (T divisions in a row).
 *                   Other values: WKV7_ERR_ARG.
 *   dr..db, dh0   : as for wkv7_bwd (dh0 may be NULL).  No workspace.
 * w must be nonzero; results are not finite when 1 + b . (a / w) is zero.
 */
wkv7_status wkv7_bwd_division(int B, int T, int H, int D, wkv7_dtype in_dtype,
                              const float *dy, const float *dhT,
                              const void *r, const void *w, const void *k,
                              const void *v, const void *a, const void *b,
                              const float *h_ckpt, const float *hT, int restart,
                              float *dr, float *dw, float *dk, float *dv,
                              float *da, float *db, float *dh0, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
