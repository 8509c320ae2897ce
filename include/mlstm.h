/*
 * mlstm.h -- C ABI of the MI355X (gfx950) mLSTM cell library (forward and
 * backward).
 *
 * The operation is the mLSTM cell of xLSTM: exponential input and forget
 * gates in log space with the stabilizer m_t = max(f~_t + m_{t-1}, i~_t)
 * (xLSTM note, section "sLSTM"), the matrix memory C_t = f_t C_{t-1} +
 * i_t v_t k_t^T, the normalizer n_t = f_t n_{t-1} + i_t k_t and the read-out
 * h_t = o_t * C_t q_t / max(|n_t^T q_t|, 1) with o_t = sigmoid(o~_t) (same
 * note, section "mLSTM (matrix LSTM)" and its example recurrent step).  The
 * library keeps the state in stabilized variables:
 *
 *   C'_t = C_t e^{-m_t}  [d_qk x d_v, key index first],
 *   n'_t = n_t e^{-m_t}  [d_qk],   m_t,
 *
 * and evaluates the read-out as sigmoid(o~_t) * C'^T q / max(|n'^T q|, e^{-m_t}),
 * which equals the unstabilized formula exactly.  f~ is the log of the forget
 * gate: the library applies exp to it and nothing else (no sigmoid).
 *
 * Three entry points compute it or its gradients:
 *   mlstm_fwd_chunkwise -- a whole sequence, chunkwise-parallel (prefill);
 *   mlstm_step          -- one token of the recurrence (decode);
 *   mlstm_bwd_chunkwise -- gradients of a whole sequence (training);
 * mlstm_layer_fwd runs the layer's input projections in front of the first
 * of them, and mlstm_slstm_fwd is the forward of xLSTM's other cell, the
 * sLSTM.
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers (HIP memory on the current
 *    device), dense, C-contiguous, in the layouts given per argument.  The
 *    caller owns every buffer; the library allocates nothing, keeps no state
 *    between calls and never synchronizes: work is enqueued on `stream`
 *    (a hipStream_t; NULL = the null stream) and the call returns at once.
 *    (Exceptions: mlstm_layer_fwd keeps a hipBLASLt handle per device, and
 *    mlstm_step_noalloc works in a fixed scratch array that each device
 *    holds for the life of the process.)
 *  - q, k, v, o_pre and h have the I/O dtype `io` (float32 or bfloat16);
 *    i_pre, f_pre and the state (C, n, m) are always float32.
 *  - Every pointer, workspace included, must be 16-byte aligned (the kernels
 *    move 16 bytes per lane; hipMalloc and torch allocations are 256-byte
 *    aligned, a view at an offset may not be): MLSTM_ERR_ALIGN otherwise.
 *  - Arguments are validated on the host before any device work.  An invalid
 *    call returns an error status and enqueues nothing.  A HIP launch error
 *    returns MLSTM_ERR_HIP.  No exception crosses the ABI.
 *  - Supported shapes: 1 <= d_qk <= 256 and 1 <= d_v <= 512, both multiples
 *    of 16; chunk in {16, 32, 64, 128}; any T >= 1; B, H >= 1.
 *  - Gate values: i~ may be any float including -inf (an input gate of 0).
 *    f~ must be finite for the chunkwise calls (forward and backward): they
 *    work with in-chunk cumulative sums of f~, so f~ = -inf (a forget gate
 *    of exactly 0) yields NaN, and very negative values lose float32
 *    precision there (about ulp(sum of a chunk's f~) in every decay, ~1e-3
 *    relative at f~ = -1e4).  A log-sigmoid of any finite float is finite.
 *    mlstm_step takes each gate alone and accepts f~ = -inf.
 *  - chunk is the longest token block the caller allows between two state
 *    passes.  The chunkwise form computes the same recurrence for every
 *    block length, so where the tiles of the requested chunk do not fit in a
 *    compute unit's 160 KB of LDS for this d_qk, d_v and dtype, the kernels
 *    use the longest of chunk/2, chunk/4, ... (>= 16) that does (for example
 *    64 for bfloat16 with d_qk = 256, d_v = 512 and chunk = 128);
 *    mlstm_fwd_chunkwise_schedule reports the length used.
 */
#ifndef MLSTM_H
#define MLSTM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLSTM_F32 = 0,   /* float32 */
    MLSTM_BF16 = 1   /* bfloat16 (outputs rounded to nearest even) */
} mlstm_dtype_t;

typedef enum {
    MLSTM_OK = 0,
    MLSTM_ERR_NULL = 1,        /* a required pointer is NULL */
    MLSTM_ERR_SHAPE = 2,       /* a size is <= 0 or the byte sizes overflow */
    MLSTM_ERR_UNSUPPORTED = 3, /* valid but not implemented: d_qk, d_v, chunk, dtype */
    MLSTM_ERR_STATE_ARGS = 4,  /* initial or final state given only in part */
    MLSTM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the query says */
    MLSTM_ERR_ALIAS = 6,       /* buffers overlap in a way the call does not allow */
    MLSTM_ERR_HIP = 7,         /* the HIP runtime reported an error */
    MLSTM_ERR_ALIGN = 8,       /* a pointer is not 16-byte aligned */
    MLSTM_ERR_BLAS = 9,        /* a hipBLASLt call failed (layer projections) */
    MLSTM_ERR_SCRATCH = 10     /* the shape needs more than mlstm_step_noalloc's fixed scratch */
} mlstm_status_t;

/* Bytes of the fixed per-device scratch array of mlstm_step_noalloc. */
#define MLSTM_STEP_NOALLOC_MAX_BYTES ((size_t)32 << 20)

/* Kernel strategy of the chunkwise forward (the result is the same up to
 * rounding; only the schedule differs). */
typedef enum {
    MLSTM_VARIANT_AUTO = 0,    /* chosen from the shape (what mlstm_fwd_chunkwise does) */
    MLSTM_VARIANT_FUSED = 1,   /* one pass; each workgroup walks all chunks of its sequence */
    MLSTM_VARIANT_SEGSCAN = 2  /* sequence split into segments: local states, a scan over
                                  segments, then the fused pass seeded per segment */
} mlstm_variant_t;

/* Human-readable name of a status (static string, never NULL). */
const char *mlstm_status_string(mlstm_status_t s);

/* Library version string (static). */
const char *mlstm_version(void);

/*
 * Schedule of a chunkwise call, host-only (touches no device): the chunk
 * length the kernels use (*kernel_chunk, <= chunk) and the number of
 * segments each sequence is split into (*segments; 1 unless the variant is
 * the segment scan).  Same validation and errors as mlstm_fwd_chunkwise's
 * shape checks; NULL outputs -> MLSTM_ERR_NULL.
 */
mlstm_status_t mlstm_fwd_chunkwise_schedule(int B, int H, int T, int d_qk, int d_v, int chunk,
                                            mlstm_dtype_t io, mlstm_variant_t variant,
                                            int *kernel_chunk, int *segments);

/*
 * Bytes of device workspace mlstm_fwd_chunkwise needs for this shape with
 * MLSTM_VARIANT_AUTO (written to *bytes; 0 means none).  Host-only: touches
 * no device.  The segment-scan variant keeps one float32 state per segment
 * boundary in it.
 */
mlstm_status_t mlstm_fwd_chunkwise_workspace_size(int B, int H, int T, int d_qk, int d_v,
                                                  int chunk, mlstm_dtype_t io, size_t *bytes);

/* As above for an explicit variant. */
mlstm_status_t mlstm_fwd_chunkwise_workspace_size_variant(int B, int H, int T, int d_qk,
                                                          int d_v, int chunk, mlstm_dtype_t io,
                                                          mlstm_variant_t variant,
                                                          size_t *bytes);

/*
 * Chunkwise-parallel forward over a whole sequence (prefill).
 *
 *  q, k      [B, H, T, d_qk]  io dtype   queries, keys (no scaling applied)
 *  v         [B, H, T, d_v]   io dtype   values
 *  i_pre     [B, H, T]        float32    input-gate pre-activation i~ (i = e^{i~})
 *  f_pre     [B, H, T]        float32    log forget gate f~ (f = e^{f~})
 *  o_pre     [B, H, T, d_v]   io dtype   output-gate pre-activation o~
 *  C0, n0, m0  [B, H, d_qk, d_v], [B, H, d_qk], [B, H]  float32: initial
 *            stabilized state, or all three NULL for the zero state
 *            (C = 0, n = 0, m = 0).
 *  h         [B, H, T, d_v]   io dtype   output (written)
 *  C_T, n_T, m_T  same shapes as C0, n0, m0: final stabilized state, or all
 *            three NULL when not wanted.  C_T may be exactly C0 (same pointer;
 *            likewise n_T/n0, m_T/m0): the state is then updated in place.
 *  chunk     longest chunk L of the chunkwise form (16, 32, 64 or 128; see
 *            the conventions above for the length the kernels use).
 *  workspace device buffer of at least the queried size (may be NULL when
 *            the query gives 0); its contents on entry are irrelevant.
 *
 * Errors: NULL input/output pointer -> MLSTM_ERR_NULL; state triples given
 * in part -> MLSTM_ERR_STATE_ARGS; h overlapping any input, or a partial
 * overlap between state buffers -> MLSTM_ERR_ALIAS; workspace too small ->
 * MLSTM_ERR_WORKSPACE.
 */
mlstm_status_t mlstm_fwd_chunkwise(const void *q, const void *k, const void *v,
                                   const float *i_pre, const float *f_pre, const void *o_pre,
                                   const float *C0, const float *n0, const float *m0,
                                   void *h, float *C_T, float *n_T, float *m_T,
                                   int B, int H, int T, int d_qk, int d_v, int chunk,
                                   mlstm_dtype_t io, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* mlstm_fwd_chunkwise with an explicit kernel strategy (for tests and
 * measurement; AUTO is what mlstm_fwd_chunkwise uses). */
mlstm_status_t mlstm_fwd_chunkwise_variant(const void *q, const void *k, const void *v,
                                           const float *i_pre, const float *f_pre,
                                           const void *o_pre, const float *C0, const float *n0,
                                           const float *m0, void *h, float *C_T, float *n_T,
                                           float *m_T, int B, int H, int T, int d_qk, int d_v,
                                           int chunk, mlstm_dtype_t io, mlstm_variant_t variant,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/*
 * Bytes of device workspace mlstm_step can use for this shape (0 when the
 * shape gains nothing from it; then the workspace argument is ignored).
 * bytes NULL -> MLSTM_ERR_NULL; unsupported shape -> as mlstm_step.
 */
mlstm_status_t mlstm_step_workspace_size(int B, int H, int d_qk, int d_v, mlstm_dtype_t io,
                                         size_t *bytes);

/*
 * One step of the recurrence for B*H independent cells (decode): the
 * per-token update of the memory, normalizer and stabilizer and the gated
 * read-out (xLSTM note, section "mLSTM (matrix LSTM)" and its example
 * recurrent step; one token of the forward above).
 *
 *  q, k      [B, H, d_qk]  io dtype;   v, o_pre [B, H, d_v]  io dtype
 *  i_pre, f_pre [B, H]     float32
 *  C_in, n_in, m_in  [B, H, d_qk, d_v], [B, H, d_qk], [B, H] float32: state
 *            before the token, or all three NULL for the zero state
 *  h         [B, H, d_v]   io dtype (written)
 *  C_out, n_out, m_out  state after the token (required).  Each may be
 *            exactly the matching *_in pointer (in-place update, the usual
 *            decode loop); any other overlap is MLSTM_ERR_ALIAS.
 *  workspace optional device buffer of workspace_bytes.  NULL: one workgroup
 *            streams each cell's memory.  Given (at least the size
 *            mlstm_step_workspace_size reports, when that is not 0), each
 *            cell's memory is split into row blocks streamed by separate
 *            workgroups, whose partial read-outs a second launch sums there
 *            (faster for large memories).  Scratch only: no initial contents
 *            are needed and none are kept, but two calls that may run at the
 *            same time need separate buffers.  Too small ->
 *            MLSTM_ERR_WORKSPACE; overlapping any tensor argument ->
 *            MLSTM_ERR_ALIAS.
 */
mlstm_status_t mlstm_step(const void *q, const void *k, const void *v,
                          const float *i_pre, const float *f_pre, const void *o_pre,
                          const float *C_in, const float *n_in, const float *m_in,
                          void *h, float *C_out, float *n_out, float *m_out,
                          int B, int H, int d_qk, int d_v, mlstm_dtype_t io,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * mlstm_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, checks, results and errors as mlstm_step given a
 * workspace, except that the row split's workspace is a fixed scratch array
 * inside the library, MLSTM_STEP_NOALLOC_MAX_BYTES per device, so the call
 * allocates nothing (not even through another library).  The caller still
 * passes every input and output.
 *
 *  - A shape whose workspace (mlstm_step_workspace_size) exceeds
 *    MLSTM_STEP_NOALLOC_MAX_BYTES -> MLSTM_ERR_SCRATCH, nothing enqueued:
 *    32 MiB holds the partial read-outs of 4064 cells at d_qk = 256,
 *    d_v = 512 (B*H cells need B*H*4*(d_v+4)*4 bytes there).  A shape that
 *    gains nothing from the split runs the one-workgroup kernel and uses
 *    no scratch.
 *  - The scratch belongs to the device of `stream` (the current device for
 *    the null stream); its address there is looked up on the first call on
 *    that device, with that device current (a failure -> MLSTM_ERR_HIP).
 *  - Every call on one device shares that device's array and leaves its own
 *    partial results in it; each call writes what it reads before reading
 *    it, so no contents need clearing.  Calls that may run at the same time
 *    on one device (different streams, or overlapping graphs) race: the
 *    caller orders them.
 */
mlstm_status_t mlstm_step_noalloc(const void *q, const void *k, const void *v,
                                  const float *i_pre, const float *f_pre, const void *o_pre,
                                  const float *C_in, const float *n_in, const float *m_in,
                                  void *h, float *C_out, float *n_out, float *m_out,
                                  int B, int H, int d_qk, int d_v, mlstm_dtype_t io,
                                  void *stream);

/*
 * Gradients of a loss L with respect to every input of mlstm_fwd_chunkwise,
 * given dL/dh (training).  Reverse mode of the same recurrence: the
 * read-out C q / max(|n^T q|, 1) does not depend on the stabilizer, so m is
 * not differentiated, and where |n'^T q| is at the floor e^{-m} the
 * normalizer gets no gradient (the floor's branch).  The call recomputes the
 * forward's states (one pass storing the state at every 32-token chunk
 * start in the workspace) and then runs backwards over the chunks.
 *
 *  q, k, v, i_pre, f_pre, o_pre, C0, n0, m0   as for mlstm_fwd_chunkwise
 *            (the forward's inputs; C0, n0, m0 all NULL for the zero state)
 *  dh        [B, H, T, d_v]   io dtype   dL/dh
 *  dq, dk    [B, H, T, d_qk]  float32    dL/dq, dL/dk (written)
 *  dv, d_o   [B, H, T, d_v]   float32    dL/dv, dL/do~ (written)
 *  d_i, d_f  [B, H, T]        float32    dL/di~, dL/df~ (written)
 *  dC0, dn0, dm0  [B, H, d_qk, d_v], [B, H, d_qk], [B, H] float32: dL with
 *            respect to the initial state (of the zero state when C0, n0,
 *            m0 are NULL), or all three NULL when not wanted.
 *  chunk     as for mlstm_fwd_chunkwise (accepted for symmetry: this
 *            version always works in chunks of 32 tokens, which the
 *            chunkwise form allows without changing the result).
 *  workspace device buffer of at least mlstm_bwd_chunkwise_workspace_size
 *            bytes; contents on entry are irrelevant.
 *
 * Gradients are float32 for either io dtype.  Supported heads: d_qk <= 256
 * and d_v <= 512, multiples of 16: the chunks' local terms are computed in
 * parallel and the carried gradient is scanned by blocks of value columns,
 * with the per-chunk states, rows and carried gradients kept in the
 * workspace, about T/32 * (2 d_qk d_v + 32 d_v) floats per sequence.
 * Larger heads, and sequences with (T + 32) * max(d_qk, d_v) >= 2^29
 * (one sequence's q, k or v, or their gradients, at 2 GiB or more in float32),
 * return MLSTM_ERR_UNSUPPORTED.
 * Errors as for mlstm_fwd_chunkwise; every output must overlap no input, no
 * other output and no workspace (MLSTM_ERR_ALIAS).
 */
mlstm_status_t mlstm_bwd_chunkwise_workspace_size(int B, int H, int T, int d_qk, int d_v,
                                                  int chunk, mlstm_dtype_t io, size_t *bytes);
mlstm_status_t mlstm_bwd_chunkwise(const void *q, const void *k, const void *v,
                                   const float *i_pre, const float *f_pre, const void *o_pre,
                                   const float *C0, const float *n0, const float *m0,
                                   const void *dh, float *dq, float *dk, float *dv,
                                   float *d_i, float *d_f, float *d_o,
                                   float *dC0, float *dn0, float *dm0,
                                   int B, int H, int T, int d_qk, int d_v, int chunk,
                                   mlstm_dtype_t io, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * Bytes of device workspace mlstm_layer_fwd needs for this shape (the
 * projected q, k, v, o~, the gate pre-activations, the cell's workspace and
 * 32 MiB for the GEMMs).  Unsupported shape -> as mlstm_layer_fwd.
 */
mlstm_status_t mlstm_layer_fwd_workspace_size(int B, int T, int d_model, int H, int d_qk, int d_v,
                                              int chunk, mlstm_dtype_t io, size_t *bytes);

/*
 * The mLSTM layer forward: the input projections of the xLSTM notes' example
 * mLSTM module (section "mLSTM", its listing of the recurrent forward: linear
 * maps with bias from each token to the query, key, value, output-gate
 * pre-activation and scalar input- and forget-gate pre-activations), then the
 * chunkwise cell of mlstm_fwd_chunkwise over every (head, batch) cell.  The
 * forget pre-activation is the log of the forget gate, as in the cell.
 *
 *  x         [B, T, d_model]        io dtype; d_model a multiple of 8
 *  W_q, W_k  [H, d_qk, d_model]     io dtype (row-major: out x in, per head)
 *  W_v, W_o  [H, d_v, d_model]      io dtype
 *  W_i, W_f  [H, d_model]           io dtype
 *  b_q, b_k  [H, d_qk]; b_v, b_o [H, d_v]; b_i, b_f [H]   float32
 *  C0, n0, m0  [H, B, d_qk, d_v], [H, B, d_qk], [H, B] float32, or all NULL
 *  h         [H, B, T, d_v]         io dtype (written)
 *  C_T, n_T, m_T  [H, B, ...] float32, or all NULL
 *  chunk, io as for mlstm_fwd_chunkwise (d_qk, d_v, chunk: its rules)
 *  workspace at least mlstm_layer_fwd_workspace_size bytes
 *
 * Cells are ordered head-major (h, then b) in every per-cell tensor: one
 * head's projection of all tokens is then one GEMM writing the cell's layout.
 * The projections run on hipBLASLt (fp32 accumulation, q, k, v, o~ rounded to
 * the io dtype, gate pre-activations kept in float32); the library creates
 * one hipBLASLt handle per device on first use and keeps it, with the
 * algorithm chosen per GEMM shape, until the process ends.  Errors: as
 * mlstm_fwd_chunkwise, plus MLSTM_ERR_BLAS when a hipBLASLt call fails (the
 * projections enqueued before it may have run).  Every check runs on the host
 * before the first projection is enqueued: a state triple given in part ->
 * MLSTM_ERR_STATE_ARGS; any pointer misaligned -> MLSTM_ERR_ALIGN; h, C_T,
 * n_T, m_T and the workspace overlapping a layer input, each other, or an
 * initial-state buffer -> MLSTM_ERR_ALIAS, except that C_T, n_T, m_T may
 * coincide exactly with C0, n0, m0 (the state updated in place).
 */
mlstm_status_t mlstm_layer_fwd(const void *x, const void *W_q, const void *W_k, const void *W_v,
                               const void *W_o, const void *W_i, const void *W_f,
                               const float *b_q, const float *b_k, const float *b_v,
                               const float *b_o, const float *b_i, const float *b_f,
                               const float *C0, const float *n0, const float *m0,
                               void *h, float *C_T, float *n_T, float *m_T,
                               int B, int T, int d_model, int H, int d_qk, int d_v, int chunk,
                               mlstm_dtype_t io, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * The sLSTM cell forward, the scalar-memory cell of xLSTM (xLSTM note,
 * section "sLSTM": exponential input and forget gates with the log-space
 * stabilizer m_t = max(f~_t + m_{t-1}, i~_t) and a normalization; a scalar
 * memory with memory mixing).  Per (batch, head) group of d cells and token t:
 *   pre_g = gx[b,h,t,g] + R[h,g] h_{t-1}      g = 0..3: z, i, f, o (row j of
 *                                            R[h,g] feeds cell j)
 *   m_t = max(f~ + m_{t-1}, i~),  f' = e^{f~ + m_{t-1} - m_t},  i' = e^{i~ - m_t}
 *   c_t = f' c_{t-1} + i' tanh(z~),  n_t = f' n_{t-1} + i',
 *   h_t = sigmoid(o~) c_t / n_t               (elementwise over the d cells)
 * c and n are kept stabilized (times e^{-m_t}); h does not depend on it.
 *
 *  gx        [B, H, T, 4, d]  io dtype: the input part (W_g x_t + b_g) of
 *            every pre-activation, gate order z, i, f, o
 *  R         [H, 4, d, d]     io dtype: recurrent (memory-mixing) weights
 *  c0, n0, m0, h0  [B, H, d] float32, all four or all NULL (zero state)
 *  h         [B, H, T, d]     io dtype (written)
 *  c_T, n_T, m_T, h_T  [B, H, d] float32, all four or all NULL; each may be
 *            exactly its initial-state pointer (in place)
 *  d         multiple of 16, at most 128 (the four d x d matrices of a head
 *            live in one compute unit's registers)
 *
 * Errors as for the other calls (MLSTM_ERR_STATE_ARGS for an incomplete
 * state set).
 */
mlstm_status_t mlstm_slstm_fwd(const void *gx, const void *R, const float *c0, const float *n0,
                               const float *m0, const float *h0, void *h, float *c_T,
                               float *n_T, float *m_T, float *h_T, int B, int H, int T, int d,
                               mlstm_dtype_t io, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MLSTM_H */
