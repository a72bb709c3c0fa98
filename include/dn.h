/*
 * dn.h -- C ABI of the chunkwise gated delta-rule operator for AMD MI355X (gfx950).
 *
 * The operator (per batch element and head; the state S is d_v x d_k):
 *
 *     S_t = S_{t-1} Diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,     o_t = S_t q_t
 *
 * with S_0 = h0 and hT = S_T.  g_t is the natural-log decay: absent (DeltaNet),
 * one scalar per step (Gated DeltaNet) or one value per key channel (Kimi Delta
 * Attention).  Sources:
 *   - ReWY abstract (paperdot listing): delta-rule linear attention for DeltaNet,
 *     GDN and KDA; chunkwise evaluation; a backward in which the chunk correction
 *     is differentiated as one triangular residual system (no inverse adjoint),
 *     centred contractions for vector gates and key-gradient reuse for scalar
 *     gates; exact in exact arithmetic; fp32 working matrices.
 *   - SFDA technical summary (gist.science), "Kernarchitektur": the update
 *     S_t = (I - beta k k*) Lambda_t S_{t-1} + beta k v*, which with zero phase is
 *     KDA; this header uses its transpose (S is d_v x d_k, o = S q).
 *     "Der konstruktive Chunk-WY-Theorem" / "Zentrale Beitraege": chunk products
 *     in WY form and the exact affine chunk transfer used by the forward and by
 *     the chunk-parallel scan (DN_FLAG_NO_SCAN); the phase-controlled gate and
 *     its real 2 x 2 rotation-decay form (dn_recurrent_phase_fwd).
 *   - KLA abstract (thelatestinai): GDN as gated decay plus delta-rule residual
 *     write; the Kaczmarz step beta_t = eta_t / (||k_t||^2 + eps) changes only
 *     the step size.  Callers either pass beta themselves or set
 *     DN_FLAG_KACZMARZ and pass eta in its place (see dn_shape).
 *   - Fast Weight Attention abstract (papers.fzhiy.net): read-after-write output,
 *     o_t reads the state after step t's write.
 * There is no query scale.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer, 16-byte aligned, dense and
 *     row-major in the layout given below.  The caller owns all memory.  The
 *     library never allocates, frees or synchronises: it validates the
 *     arguments on the host, then enqueues kernels on `stream` (a hipStream_t;
 *     NULL = the default stream) and returns.
 *   - Outputs must not overlap inputs, each other or the workspace.
 *   - On any error nothing is enqueued, a negative dn_status is returned and
 *     dn_last_error() describes it.  No C++ exception crosses this boundary.
 *   - NaN / Inf in the inputs propagate to the outputs; they are not errors.
 *   - The library keeps no state between calls except the per-thread error text,
 *     while dn_profile_enable(1) is in effect the recorded timing events, and
 *     the per-device scratch array of dn_chunk_fwd_noalloc; calls from several
 *     host threads are safe.  Two calls that share a workspace (or, for
 *     dn_chunk_fwd_noalloc, a GPU) must be ordered on one stream.
 *
 * Layouts (BH = B * H, NT = ceil(T / C)); "io" is the element type chosen by
 * dn_shape.dtype (fp32 or bf16), everything marked fp32 is always fp32:
 *     q, k, dq, dk       io   [B][H][T][dk]
 *     v, o, dout, dv     io   [B][H][T][dv]
 *     beta, dbeta        fp32 [B][H][T]
 *     g, dg              fp32 [B][H][T] (DN_GATE_SCALAR) or [B][H][T][dk] (DN_GATE_VECTOR)
 *     h0, hT, dh0, dhT   fp32 [B][H][dv][dk]
 *     states             the forward's saved buffer, regions at the byte offsets
 *                        dn_states_layout() gives (each 256-byte aligned):
 *                          io   [B][H][NT][dv][dk]  state entering each chunk
 *                          io   [B][H][NT][C][C]    (I + A)^{-1} of each chunk
 *                          io   [B][H][NT][C][C]    causal intra-chunk scores
 *                          io   [B][H][NT][C][dv]   U = (I + A)^{-1} R of each chunk
 *                                                   (R = diag(beta)(V - X), the
 *                                                   chunk's residual; rows past T
 *                                                   zero)
 *                          fp32 like g              in-chunk cumulative log-decay
 *                                                   (absent without a gate)
 *                          fp32 [2][B][H][T]        DN_FLAG_KACZMARZ only: beta_t,
 *                                                   then 1 / (||k_t||^2 + eps)
 * The saved quantities are kept in the types the kernels use them in (the state
 * and the per-chunk matrices are matrix-core operands in the io type), so the
 * backward reads exactly the operand values the forward used; the running
 * state itself and hT are fp32.
 */
#ifndef DN_H
#define DN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DN_OK = 0,
    DN_ERR_INVALID = -1,      /* NULL / misaligned / overlapping pointer, bad enum */
    DN_ERR_SHAPE = -2,        /* negative or inconsistent sizes */
    DN_ERR_DTYPE = -3,        /* unknown dtype */
    DN_ERR_WORKSPACE = -4,    /* workspace missing or smaller than dn_workspace_bytes() */
    DN_ERR_UNSUPPORTED = -5,  /* valid but not implemented (see dn_shape) */
    DN_ERR_HIP = -6           /* the HIP runtime refused a launch */
} dn_status;

typedef enum { DN_F32 = 0, DN_BF16 = 1 } dn_dtype;

typedef enum { DN_GATE_NONE = 0, DN_GATE_SCALAR = 1, DN_GATE_VECTOR = 2 } dn_gate;

/* Which call a workspace is sized for. */
typedef enum {
    DN_PASS_FWD = 0,           /* dn_chunk_fwd (states saved or not) */
    DN_PASS_BWD = 1,           /* dn_chunk_bwd with the forward's saved buffer */
    DN_PASS_BWD_RECOMPUTE = 2  /* dn_chunk_bwd with states == NULL (states recomputed) */
} dn_pass;

/*
 * Kaczmarz step size (KLA abstract): with this flag the `beta` argument of every
 * entry point carries eta [B][H][T] fp32 and the operator uses
 *     beta_t = eta_t / (||k_t||^2 + eps)
 * with ||k_t||^2 summed in fp32 over the keys as given (io type).  The backward
 * then writes d eta (= d beta / (||k_t||^2 + eps)) to `dbeta`, and dk includes
 * the path through the step size, -2 (d beta_t) beta_t k_t / (||k_t||^2 + eps).
 * A zero key with eps == 0 gives Inf / NaN like any other division by zero.
 */
#define DN_FLAG_KACZMARZ 1u

/*
 * Chunk-parallel state scan (exact affine chunk transfer, SFDA summary, "Exakter
 * Affiner Chunk-Transfer"; chunk-WY theorem): when the sequential state passes
 * would occupy few compute units (few heads: (dv / 16) * B * H < 128) and the
 * sequence has at least 32 chunks, the forward and backward split the chunks
 * into segments, run every segment from a zero state together with its d_k x
 * d_k transition matrix, compose the segments' boundary states in fp32, and
 * rerun each segment from its true boundary state.  Results equal the
 * sequential pass up to rounding (the transition is formed with the same
 * matrix-core operands).  This flag forces the sequential pass.
 */
#define DN_FLAG_NO_SCAN 2u

/*
 * Per-channel gate (DN_GATE_VECTOR): the C x C products split each pair's decay
 * at the gate of a 16-step block boundary (the centred contraction, ReWY
 * abstract), so every factor is finite while a channel's log-decay summed over
 * any 16 consecutive steps stays above -87 (e.g. g >= -5.4 per step); beyond
 * that the factors overflow and the results are Inf / NaN, with DN_OK.
 *
 * Problem shape.  Supported: B, H, T >= 0 with B*H <= 65535; dk == dv in
 * {16, 32, 64, 128}; C in {16, 32, 64}; any T (a last, shorter chunk is
 * handled exactly); fp32 with a vector gate needs dk <= 64, and C <= 32 at
 * dk = 64.  fp32 I/O keeps every working matrix in fp32 (the matrix-core
 * operands too); bf16 I/O uses bf16 operands with fp32 accumulation -- a caller
 * who wants fp32 working matrices for bf16 data passes its exact fp32 copy.  flags: DN_FLAG_KACZMARZ and / or DN_FLAG_NO_SCAN (other bits:
 * DN_ERR_INVALID; the recurrent entry points ignore DN_FLAG_NO_SCAN); eps:
 * read only with DN_FLAG_KACZMARZ, finite and >= 0.  Anything else returns
 * DN_ERR_UNSUPPORTED.
 */
typedef struct {
    int32_t B, H, T, dk, dv, C;
    int32_t dtype;   /* dn_dtype */
    int32_t gate;    /* dn_gate  */
    uint32_t flags;  /* DN_FLAG_* */
    float eps;       /* Kaczmarz denominator offset */
} dn_shape;

/* Bytes of the saved buffer `states` for this shape (the regions listed under
 * Layouts, each rounded up to 256 bytes).  0 on bad shape. */
size_t dn_states_bytes(const dn_shape* shape);

/* Byte offsets of the regions of `states`: {chunk-entry states, (I + A)^{-1},
 * intra-chunk scores, U, cumulative log-decay, Kaczmarz step data, total}; an
 * absent region has zero size.  DN_OK or a shape error. */
dn_status dn_states_layout(const dn_shape* shape, size_t offsets[7]);

/* Workspace bytes the given pass needs (0 on bad shape).  Workspace contents
 * are scratch: nothing is carried from one call to the next. */
size_t dn_workspace_bytes(const dn_shape* shape, int pass);

/*
 * Forward pass (chunkwise: per-chunk WY/UT construction with a unit-lower-
 * triangular solve, the inter-chunk state recurrence, the causal intra-chunk
 * output -- ReWY abstract; SFDA summary, chunk-WY theorem and affine transfer).
 *   inputs : q, k, v, beta (eta with DN_FLAG_KACZMARZ); g (must be NULL iff
 *            gate == DN_GATE_NONE); h0 (NULL = zero initial state)
 *   outputs: o; hT (NULL = not wanted); states (dn_states_bytes(shape) bytes:
 *            what the backward reuses; NULL = not saved, i.e. the
 *            recomputation policy: dn_chunk_bwd is then called with
 *            states == NULL)
 *   ws     : device workspace of ws_bytes >= dn_workspace_bytes(shape, DN_PASS_FWD)
 */
dn_status dn_chunk_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, void* o, float* hT,
                       void* states, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass in the reduced ReWY form: vector-Jacobian products of
 * L = <O, dout> + <hT, dhT> with respect to every input.
 *   inputs : q, k, v, beta, g, h0 as given to dn_chunk_fwd; dout; dhT (NULL =
 *            zero); states as written by dn_chunk_fwd (the backward then skips
 *            the per-chunk preparation), or NULL to recompute everything here
 *   outputs: dq, dk, dv, dbeta (d eta with DN_FLAG_KACZMARZ); dg (must be
 *            NULL iff gate == DN_GATE_NONE; same layout as g); dh0 (NULL = not
 *            wanted)
 *   ws     : >= dn_workspace_bytes(shape, states ? DN_PASS_BWD : DN_PASS_BWD_RECOMPUTE)
 */
dn_status dn_chunk_bwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, const void* dout,
                       const float* dhT, const void* states, void* dq, void* dk, void* dv,
                       float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * The forward without saved states (as dn_chunk_fwd with states == NULL), for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace: its scratch
 * (the per-chunk log-decay, (I + A)^{-1} and scores, the Kaczmarz step data and
 * the scan's segment buffers -- what dn_workspace_bytes(shape, DN_PASS_FWD)
 * counts) lives in a device array of the library, DN_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU, set up on the first call on each device (the current
 * device must be the one the pointers and the stream belong to) and held until
 * the process ends.  The call allocates nothing and frees nothing.
 *   arguments, layouts, validation and errors: as for dn_chunk_fwd
 *   DN_ERR_WORKSPACE when dn_workspace_bytes(shape, DN_PASS_FWD) exceeds
 *   DN_NOALLOC_SCRATCH_BYTES (nothing is enqueued); DN_ERR_HIP when the
 *   device's array cannot be located
 * Every call on one GPU uses the same array, and nothing in it is carried from
 * one call to the next: calls that overlap on one GPU (on different streams,
 * or from several host threads without ordering) race.
 */
#define DN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dn_status dn_chunk_fwd_noalloc(const dn_shape* shape, const void* q, const void* k, const void* v,
                               const float* beta, const float* g, const float* h0, void* o, float* hT,
                               void* stream);

/*
 * Recurrent evaluation (decode): the T steps of the recurrence for every batch
 * element and head, one token at a time (the recurrent form of the Fast Weight
 * Attention abstract; the decode setting of the KLA abstract), with the state
 * updated in place.  Same per-step arithmetic as the chunkwise forward.
 *   shape  : B, H, T (steps; 0 is a no-op), dk in {16, 32, 64, 128}, dv a
 *            positive multiple of 16 (may differ from dk), dtype, gate; C unused
 *   inputs : q, k [B][H][T][dk], v [B][H][T][dv] (io); beta [B][H][T] fp32 (eta
 *            with DN_FLAG_KACZMARZ); g as for dn_chunk_fwd (NULL iff gate ==
 *            DN_GATE_NONE)
 *   state  : fp32 [B][H][dv][dk]: the state before step 1 on entry, after step T
 *            on return (in place; it may not overlap any other argument)
 *   outputs: o [B][H][T][dv] (io)
 * Validation and errors as for dn_chunk_fwd; no workspace.
 */
dn_status dn_recurrent_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, float* state, void* o, void* stream);

/*
 * Recurrent evaluation with the phase-controlled gate (SFDA summary,
 * "Kernarchitektur" and its real implementation with 2 x 2 rotation-decay
 * blocks; read with real inputs): the state is complex, S = S_re + i S_im, and
 * every step applies per key channel c the gate exp(g_t[c]) exp(i theta_t[c]),
 * then the erase with the real key and the write of the real value:
 *     S_t = S_{t-1} diag(exp(g_t + i theta_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = Re(S_t q_t).
 * With theta = 0 and S_im = 0 this is dn_recurrent_fwd (KDA for a vector g).
 * The chunkwise form with its backward is dn_chunk_phase_fwd / dn_chunk_phase_bwd.
 *   shape  : as for dn_recurrent_fwd; the gate type says how g is laid out (none:
 *            no decay; scalar: one log-decay per step; vector: one per channel)
 *   inputs : q, k, v, beta (eta with DN_FLAG_KACZMARZ), g as for dn_recurrent_fwd;
 *            theta fp32 [B][H][T][dk] (radians)
 *   state  : state_re, state_im fp32 [B][H][dv][dk], in place (neither may
 *            overlap any other argument)
 *   outputs: o [B][H][T][dv] (io)
 * Validation and errors as for dn_recurrent_fwd; no workspace.
 */
dn_status dn_recurrent_phase_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                                 const float* beta, const float* g, const float* theta, float* state_re,
                                 float* state_im, void* o, void* stream);

/*
 * Chunkwise form of the phase-controlled gate, forward and backward (SFDA
 * summary, "Der konstruktive Chunk-WY-Theorem" with the gate of "Kernarchitektur",
 * read as for dn_recurrent_phase_fwd: real q, k, v, beta, a complex state and
 * per key channel the gate exp(g_t + i theta_t)):
 *     S_t = S_{t-1} diag(exp(g_t + i theta_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = Re(S_t q_t),  S_0 = h0_re + i h0_im,  S_T = hT_re + i hT_im.
 * In chunks of 16 steps: per chunk the complex UT / WY construction (pairwise
 * complex decays in the C x C products, so any g <= 0 is safe), the exact
 * chunk transfer of the state and the intra-chunk output; the backward takes
 * the chunks back in reverse with one transposed (conjugated) triangular solve
 * per chunk.  The per-chunk products run for all chunks at once, the state
 * recurrences over (head, block of 16 state rows); fp32 arithmetic throughout.
 *   shape  : dk == dv in {16, 32, 64, 128}; C == 16; dtype fp32 or bf16 (q, k, v, o,
 *            dout, dq, dk, dv); gate as for dn_chunk_fwd; DN_FLAG_KACZMARZ is not
 *            supported here (DN_ERR_UNSUPPORTED); DN_FLAG_NO_SCAN is ignored
 *   inputs : q, k, v, beta, g as for dn_chunk_fwd; theta fp32 [B][H][T][dk]
 *            (radians); h0_re, h0_im fp32 [B][H][dv][dk] (NULL = zero)
 *   outputs: o; hT_re, hT_im (NULL = not wanted); states (dn_phase_states_bytes
 *            bytes, fp32; NULL = not saved): the complex state entering each
 *            chunk [B][H][NT][2][dv][dk] (real part, then imaginary; NT =
 *            ceil(T / 16)), then, from the next 256-byte boundary, per chunk
 *            [B][H][NT][6][16][16] the matrices (I + A)^{-1}, P and G (real,
 *            imaginary, each); written by the forward for the backward, which
 *            recomputes them (from h0_re, h0_im) when it gets NULL
 *   backward: the vector-Jacobian products of
 *            L = <o, dout> + <hT_re, dhT_re> + <hT_im, dhT_im>  (dhT_* NULL = zero):
 *            dq, dk, dv (io), dbeta, dg (NULL iff no gate; layout of g), dtheta
 *            (like theta) fp32; dh0_re, dh0_im (NULL = not wanted)
 *   ws     : device scratch of ws_bytes >= dn_phase_workspace_bytes(shape, pass):
 *            the forward needs it only when states is NULL (DN_PASS_FWD: the
 *            per-chunk matrices), the backward always (DN_PASS_BWD: lambda and
 *            the state cotangent of each chunk; DN_PASS_BWD_RECOMPUTE, when
 *            states is NULL: those, then the recomputed states and matrices in
 *            the layout of the saved buffer)
 * Validation and errors as for dn_chunk_fwd.
 */
size_t dn_phase_states_bytes(const dn_shape* shape);
size_t dn_phase_workspace_bytes(const dn_shape* shape, int pass);
dn_status dn_chunk_phase_fwd(const dn_shape* shape, const void* q, const void* k, const void* v, const float* beta,
                             const float* g, const float* theta, const float* h0_re, const float* h0_im, void* o,
                             float* hT_re, float* hT_im, float* states, void* ws, size_t ws_bytes, void* stream);
dn_status dn_chunk_phase_bwd(const dn_shape* shape, const void* q, const void* k, const void* v, const float* beta,
                             const float* g, const float* theta, const float* h0_re, const float* h0_im,
                             const void* dout, const float* dhT_re, const float* dhT_im, const float* states, void* dq,
                             void* dk, void* dv, float* dbeta, float* dg, float* dtheta, float* dh0_re, float* dh0_im,
                             void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* dn_status_string(dn_status status);

/* Detail text of the last error on the calling thread ("" if none). */
const char* dn_last_error(void);

/*
 * Diagnostics: byte offsets of the workspace regions a pass uses, in the order
 * {cumulative log-decay, (I+A)^{-1} per chunk, intra-chunk scores per chunk,
 * triangular-residual adjoint, state cotangent per chunk, recomputed states,
 * Kaczmarz step data (as in the saved buffer), scan segment summaries
 * [B][H][nseg][dv + dk][dk] fp32, scan boundary states [B][H][nseg][dv][dk] fp32
 * (both only when the scan is used), total}; a region the pass does
 * not use has zero size (the next offset is equal).  DN_PASS_FWD places the
 * per-chunk data there only when the forward saves nothing; DN_PASS_BWD takes
 * it from the saved buffer.  Returns DN_OK or an error for a bad shape / pass.
 */
dn_status dn_workspace_layout(const dn_shape* shape, int pass, size_t offsets[10]);

/*
 * Diagnostics: per-kernel timing.  dn_profile_enable(1) makes every later
 * launch record a pair of hipEvents on its stream (creating two event objects
 * per launch); dn_profile_enable(0) stops it.  dn_profile_collect waits for
 * the recorded events, writes up to max_kernels entries -- the kernel name
 * (NUL-terminated, at most 31 characters, in names[32*i ...]), its summed
 * milliseconds and its launch count -- releases the events and returns the
 * number of entries.  Any output pointer may be NULL.
 */
dn_status dn_profile_enable(int on);
int dn_profile_collect(char* names, double* total_ms, int* launches, int max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* DN_H */
