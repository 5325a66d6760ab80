/*
 * essh.h -- C ABI of the MI355X (gfx950) selective spectral mixer core.
 *
 * The method is the selective spectral mixer of "Elastic Selective Spectral
 * Hybrids for Train-Once, Export-Many Budgeted Inference" (ESSH).  Each
 * retained spectral channel k < K_T is a bank of m damped-rotation modes:
 * a complex diagonal recurrence whose per-step decay is set by a
 * token-dependent clock, with a write gate on the injected channel value and
 * a read gate on the readout (Sec. 4.1, Eq. 5; App. B, Eq. 9).  In complex
 * form (App. B.1: a damped rotation rho R(theta) acting on a 2-vector is
 * multiplication by rho e^{i theta}, injection along e_1 adds to the real
 * part, reading with (kc, -ks) is Re(c h) with c = kc + i ks):
 *
 *   lambda_kj(t) = rho_kj * exp(-delta(t)) * e^{i theta_kj}
 *   h_kj(t)      = lambda_kj(t) * h_kj(t-1) + g_w(t) * v_k(t)       (per value p)
 *   y_k(t)       = sum_j g_r(t) * Re(c_kj * h_kj(t))                 (the core output z^core)
 *
 * Optionally with the zero-lag correction of App. C.3 (Eq. 24), coefficients
 * a_kj:  z_k(t) = y_k(t) - sum_j a_kj * g_r(t) * g_w(t) * kc_kj * v_k(t)
 * (per-mode gates in that sum when the controls are per mode).  It changes
 * only the lag-zero coefficient and adds no state.
 *
 * Channels k >= K_T are never read, computed or written (tier truncation,
 * App. C.4 and D.2; Sec. 4.3).
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer owned by the caller; the
 *     library keeps no reference after the call returns and holds no global
 *     state, so calls are re-entrant.  Work is enqueued on `stream`
 *     (a hipStream_t; 0 is the null stream) and the call returns without
 *     waiting.  Errors detected on the host are returned synchronously and no
 *     work is enqueued; errors of device execution surface at the caller's
 *     next synchronisation of the stream, as for any HIP launch.
 *   - Arrays are dense and row-major.  Shapes use the fields of essh_dims:
 *       v, y            [B, L, K, P]          io dtype
 *       delta           [B, L, K]   (or [B, L, K, m] if ctrl_per_mode) fp32, >= 0
 *       g_w, g_r        [B, L, K]   (or [B, L, K, m] if ctrl_per_mode) io dtype
 *       rho, theta      [K, m]                fp32, 0 < rho < 1
 *       c               [K, m, 2]             fp32, (re, im) = (kc, ks)
 *       zl              [K, m]                fp32 zero-lag coefficients a, or NULL
 *       state           [B, K, m, 2, P]       fp32, real plane then imaginary plane
 *     The channel stride of every array is the full K even when K_T < K.
 *   - Clock and gate values are post-activation: the kernels apply neither
 *     softplus nor sigmoid (App. C.2 defines those projections upstream).
 *   - v, y, g_w, g_r, delta and state must be 16-byte aligned; rho, theta, c,
 *     zl 4-byte aligned.  P * sizeof(io dtype) must be a multiple of 16 bytes.
 */
#ifndef ESSH_H
#define ESSH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ESSH_OK = 0,
    ESSH_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size, K_T outside [1, K] */
    ESSH_ERR_UNSUPPORTED = -2,   /* m, P, Lc or dtype outside the compiled set */
    ESSH_ERR_WORKSPACE = -3,     /* workspace missing or smaller than essh_prefill_workspace_bytes() */
    ESSH_ERR_HIP = -4,           /* a HIP launch or query failed on the host side */
    ESSH_ERR_SCRATCH = -5        /* essh_mixer_prefill_noalloc: dims need more than its static scratch */
} essh_status;

/* Size of the static device scratch of essh_mixer_prefill_noalloc, per GPU. */
#define ESSH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum { ESSH_F32 = 0, ESSH_BF16 = 1 } essh_dtype;

typedef struct {
    int32_t B;             /* batch rows, >= 0 (0: nothing to do)                          */
    int32_t L;             /* positions per call, >= 0 (decode ignores it)                 */
    int32_t K;             /* full channel count; channel stride of every [.., K, ..] array */
    int32_t m;             /* modes per channel: 1, 2, 4 or 8                              */
    int32_t P;             /* values per channel: 16, 32, 64 or 128                         */
    int32_t K_T;           /* retained tier, 1 <= K_T <= K                                 */
    int32_t Lc;            /* prefill chunk length: 32, 64 or 128; 0 selects 64 (Sec. 4.3 Q=64) */
    int32_t ctrl_per_mode; /* 0: delta/g_w/g_r per channel [B,L,K]; 1: per mode [B,L,K,m] (Eq. 5) */
    int32_t io_dtype;      /* essh_dtype of v, g_w, g_r and y; delta, tables and state are fp32 */
} essh_dims;

/* ABI version of this header (major * 100 + minor). */
#define ESSH_ABI_VERSION 101
int32_t essh_abi_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char* essh_status_string(essh_status status);

/*
 * essh_state_init -- zero the recurrent mode state, H(0) = 0 (Eq. 5).
 *   state     [n_layers, B, K, m, 2, P] fp32, written (all K channels).
 *   n_layers  >= 1; use 1 for a single mixer.
 * Uses a fill kernel (no hipMemset), so it may be captured in a HIP graph.
 * Errors: ESSH_ERR_INVALID_ARG for a null/misaligned state or bad sizes.
 */
essh_status essh_state_init(float* state, int32_t n_layers, const essh_dims* d, hipStream_t stream);

/*
 * essh_prefill_workspace_bytes -- device workspace that essh_mixer_prefill
 * needs for these dims (0 if none).  Returns 0 for invalid dims as well;
 * essh_mixer_prefill reports those.
 */
size_t essh_prefill_workspace_bytes(const essh_dims* d);

/*
 * essh_mixer_prefill -- the chunked parallel scan (Sec. 4.3, Fig. 2A).
 *
 * Runs the recurrence above over positions 0..L-1 of every batch row for the
 * retained channels k < K_T and writes y for those channels.  Within a chunk
 * of Lc positions the source-to-target contributions are evaluated as a
 * matrix product (Sec. 4.3, the within-chunk matrix G_k); only the 2 m P
 * mode-state entries of a channel are carried from chunk to chunk (Eq. 6
 * gives the closed-form transition product that makes this exact).
 *
 *   v, delta, g_w, g_r   inputs, layouts above (read only for k < K_T)
 *   rho, theta, c        mode tables [K, m] / [K, m, 2]
 *   zl                   zero-lag coefficients [K, m] (Eq. 24), or NULL: output z^core
 *   state_in             [B, K, m, 2, P] state entering position 0, or NULL for H = 0
 *   state_out            [B, K, m, 2, P] state after position L-1, or NULL;
 *                        may alias state_in.  Channels k >= K_T untouched.
 *   y                    [B, L, K, P] output; channels k >= K_T untouched.
 *   workspace            device scratch of at least essh_prefill_workspace_bytes(d)
 *                        bytes (may be NULL if that is 0); 256-byte aligned;
 *                        owned by the caller.  It holds the look-back records
 *                        of a segmented scan (used when B * K_T is too small to
 *                        fill the GPU).  Zero-fill it once before its first
 *                        use and again whenever it is bound to other dims;
 *                        every call leaves it ready for the next call with
 *                        the same dims, so it is not cleared per call (a
 *                        captured graph replays without a memset).  Calls
 *                        that share one workspace must be ordered (one
 *                        stream, or events): concurrent calls on one
 *                        workspace race.  Every wait inside the scan is
 *                        bounded; if one ever runs out, the kernel ORs a
 *                        nonzero code into 32-bit word 1 (byte offset 4) of
 *                        the workspace and that call's y and state_out are
 *                        invalid (1: a look-back wait ran out; 2: more
 *                        tickets than workgroups, i.e. a workspace that was
 *                        not zero-filled).  The word is sticky: the library
 *                        never clears it, so a caller reads it after
 *                        synchronising (one read covers every call since it
 *                        was last cleared) and zeroes it itself.
 *   stream               HIP stream to enqueue on.
 * y must not overlap any input.  Results do not depend on Lc beyond rounding.
 */
essh_status essh_mixer_prefill(const essh_dims* d,
                               const void* v, const float* delta, const void* g_w, const void* g_r,
                               const float* rho, const float* theta, const float* c, const float* zl,
                               const float* state_in, float* state_out, void* y,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * essh_mixer_prefill_noalloc -- essh_mixer_prefill without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * look-back records live in a static device array of
 * ESSH_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on
 * that GPU until the process ends; the call allocates nothing.
 *
 * Arguments, layouts and results are those of essh_mixer_prefill, except:
 *   scan_error           NULL, or a 4-byte-aligned device word into which the
 *                        call ORs its scan error code (the codes of the
 *                        workspace error word of essh_mixer_prefill), in
 *                        stream order; the caller zeroes it.
 * Each call clears the part of the array that must start at zero, so no
 * earlier call's contents matter.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (several streams, or several
 * host threads) race and give invalid results; order them.
 * Returns ESSH_ERR_SCRATCH, before launching anything, when
 * essh_prefill_workspace_bytes(d) exceeds ESSH_NOALLOC_SCRATCH_BYTES (for
 * example 1 x 131072 positions at K_T = 24, m = 4, P = 64 needs about 51 MB;
 * at K_T = 12, about 20 MB).
 */
essh_status essh_mixer_prefill_noalloc(const essh_dims* d,
                                       const void* v, const float* delta, const void* g_w, const void* g_r,
                                       const float* rho, const float* theta, const float* c, const float* zl,
                                       const float* state_in, float* state_out, void* y,
                                       uint32_t* scan_error, hipStream_t stream);

/*
 * essh_mixer_decode_step -- one token through n_layers independent mixers
 * (the fused recurrent decode of Sec. 4.3 / Sec. 5.3: state update and
 * readout in one kernel, the state read once and written once, discarded
 * channels skipped).
 *
 *   n_layers             >= 1 independent mixers updated by one launch
 *   d                    dims of one mixer (L is ignored; Lc ignored)
 *   v                    [n_layers, B, K, P] io dtype
 *   delta                [n_layers, B, K] (or [n_layers, B, K, m]) fp32
 *   g_w, g_r             [n_layers, B, K] (or [n_layers, B, K, m]) io dtype
 *   rho, theta           [n_layers, K, m] fp32;  c [n_layers, K, m, 2] fp32
 *   zl                   [n_layers, K, m] fp32 zero-lag coefficients, or NULL
 *   state                [n_layers, B, K, m, 2, P] fp32, updated in place (k < K_T only)
 *   y                    [n_layers, B, K, P] io dtype; channels k >= K_T untouched
 *
 * Returns ESSH_ERR_UNSUPPORTED when B or n_layers exceeds 65535 (one launch
 * covers layers x batch rows as grid extents) or n_layers * B * K * P exceeds 2^30.
 */
essh_status essh_mixer_decode_step(int32_t n_layers, const essh_dims* d,
                                   const void* v, const float* delta, const void* g_w, const void* g_r,
                                   const float* rho, const float* theta, const float* c, const float* zl,
                                   float* state, void* y, hipStream_t stream);

/*
 * essh_decode_fused_step -- one token through n_layers independent mixer layers, the
 * projections included (the fused recurrent decode of Sec. 4.3 / Sec. 5.3 with App. C.2,
 * C.3 and C.4):
 *   v0_k = W_in_k u, then the channel-local blend of Eq. 23,
 *          v_k = (1 - beta_k) v0_k + beta_k v0_k / sqrt(P^-1 |v0_k|^2 + eps_norm);
 *   per (channel, mode): write gate 2 sigmoid(w.u + b), read gate 2 sigmoid(w.u + b),
 *          clock increment softplus(w.u + b)  (App. C.2);
 *   the mode update and readout with those per-mode controls and, when zl is given, the
 *          zero-lag term (Eq. 5, Eq. 24): z_k;
 *   y = K_T^-1/2 sum_{k < K_T} W_out_k z_k  (App. C.4).
 * Channels k >= K_T are never read, computed or written.  Each weight byte is read once.
 *
 *   n_layers   >= 1 independent layers in one call (arrays stacked on a leading axis)
 *   d          dims of one mixer: B, K, m, P, K_T and io_dtype (the dtype of u); L, Lc and
 *              ctrl_per_mode are ignored (the controls are per mode, computed here)
 *   d_model    model width: a multiple of 8, at most 8192; K_T * P at most 8192
 *   u          [n_layers, B, d_model] io dtype: the normalized mixer input
 *   w_in       [n_layers, K, P, d_model] bf16, 16-byte aligned: row (k, p) of W_in
 *   beta       [n_layers, K] fp32 blend coefficients;  eps_norm > 0
 *   w_ctl      [n_layers, K, m, 3, d_model] bf16, 16-byte aligned: rows (write gate,
 *              read gate, clock) of each (channel, mode)
 *   b_ctl      [n_layers, K, m, 3] fp32: their biases
 *   rho, theta [n_layers, K, m] fp32; c [n_layers, K, m, 2] fp32; zl [n_layers, K, m] or NULL
 *   w_out      [n_layers, d_model, K, P] bf16, 16-byte aligned: row o of W_out, its columns
 *              grouped by channel (the first K_T P columns are read)
 *   state      [n_layers, B, K, m, 2, P] fp32, updated in place (channels < K_T)
 *   z          [n_layers, B, K, P] fp32 out: corrected channel outputs (channels < K_T)
 *   y          [n_layers, B, d_model] fp32 out
 *   stream     HIP stream to enqueue on (two launches).
 * Accumulation is fp32.  Returns ESSH_ERR_UNSUPPORTED for d_model or K_T * P outside the
 * bounds above, or B, n_layers or K_T above 65535.  Buffers must not overlap.
 */
essh_status essh_decode_fused_step(int32_t n_layers, const essh_dims* d, int32_t d_model, const void* u,
                                   const void* w_in, const float* beta, float eps_norm, const void* w_ctl,
                                   const float* b_ctl, const float* rho, const float* theta, const float* c,
                                   const float* zl, const void* w_out, float* state, float* z, float* y,
                                   hipStream_t stream);

/*
 * essh_prefill_backward_workspace_bytes -- device workspace, in bytes, that
 * essh_mixer_prefill_backward needs for dims d (0 if d is invalid).
 */
size_t essh_prefill_backward_workspace_bytes(const essh_dims* d);

/*
 * essh_mixer_prefill_backward -- gradients of the prefill (training's backward pass).
 *
 * Differentiates the computation of essh_mixer_prefill (Sec. 4.1 Eq. 5, Eq. 9, and App. C.3
 * Eq. 24 when zl is given) for a loss L with dL/dy = dy and dL/dstate_out = dstate_out, by
 * the chunked scan of Sec. 4.3 run backwards: the adjoint of each mode state runs from the
 * last position to the first with the conjugate poles, and only the 2 m P mode-state entries
 * of a channel (and their adjoints) cross sub-block and segment boundaries.
 *
 *   d          dims as for the prefill; ctrl_per_mode must be 0 (per-channel controls);
 *              Lc is ignored (sub-blocks of 16 positions).  B * K_T at most 65535.
 *   v .. zl, state_in   the forward inputs, exactly as passed to essh_mixer_prefill
 *   dy         [B, L, K, P] io dtype, 16-byte aligned: dL/dy
 *   dstate_out [B, K, m, 2, P] fp32 or NULL (the final state carries no gradient)
 *   dv         [B, L, K, P] io dtype, 16-byte aligned, out: dL/dv
 *   ddelta     [B, L, K] fp32 out: dL/ddelta
 *   dg_w, dg_r [B, L, K] fp32 out (also for bf16 io): dL/dg_w, dL/dg_r
 *   drho, dtheta [K, m] fp32 out;  dc [K, m, 2] fp32 out (d/dRe c, d/dIm c)
 *   dzl        [K, m] fp32 out or NULL: dL/dzl (evaluated at zl, or at zero when zl is NULL)
 *   dstate_in  [B, K, m, 2, P] fp32 out or NULL: dL/dstate_in
 *   workspace  device memory of at least essh_prefill_backward_workspace_bytes(d) bytes,
 *              256-byte aligned, owned by the caller; no contents need to be preserved
 *   stream     HIP stream to enqueue on (four or five launches).
 * Every output of channels k < K_T is overwritten (the mode-table gradients are sums over
 * the batch and all positions, not accumulated into the caller's values); entries of channels
 * k >= K_T are never read or written.  Arithmetic is fp32 throughout (fp32 matrix cores).
 * Returns ESSH_ERR_UNSUPPORTED for ctrl_per_mode = 1 or B * K_T above 65535,
 * ESSH_ERR_WORKSPACE when the workspace is missing, misaligned or too small.  Output buffers
 * must not overlap inputs or each other.
 */
essh_status essh_mixer_prefill_backward(const essh_dims* d,
                                        const void* v, const float* delta, const void* g_w, const void* g_r,
                                        const float* rho, const float* theta, const float* c, const float* zl,
                                        const float* state_in, const void* dy, const float* dstate_out,
                                        void* dv, float* ddelta, float* dg_w, float* dg_r,
                                        float* drho, float* dtheta, float* dc, float* dzl, float* dstate_in,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ESSH_H */
