/*
 * deltarule.h -- C ABI of the chunkwise gated-delta-rule forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (paper orientation, S in R^{dv x dk}):
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,                      a_t = exp(g_t)
 * as defined by the page "TileLang 实战：KDA 从零到一–Kimi Delta Attention"
 * (opening equation and section 3.1).  Its special cases:
 *   - gdn_fwd: one scalar gate per token and head (Gated DeltaNet; page
 *     "Gated DeltaNet", section "DeltaNet 与 Gated Delta Rule");
 *   - decay_la_fwd: no delta term, S_t = a_t S_{t-1} + v_t k_t^T (page
 *     "TileLang 实战：KDA 从零到一--标量衰减", section 1.1; RetNet /
 *     Lightning-style decay on the page "07 · linear 路线（二）：衰减机制的演进",
 *     sections 1-2).
 * The plain entry points apply no output scale and take q, k, beta and g as
 * given; the kind-generic entry points dr_forward / dr_forward_varlen /
 * dr_decode can apply an input prologue first (see dr_prologue).
 *
 * Conventions shared by every entry point
 *   Pointers: all tensor pointers are DEVICE pointers owned by the caller.
 *     The library allocates nothing and keeps no pointer after returning.
 *   Layout: dense, row-major, time-major [B, T, H, D] for q, k, v, o and the
 *     per-channel gate; [B, T, H] for scalar gates and beta.  The recurrent
 *     state h0 / hT is fp32 [B, H, Dk, Dv], i.e. the TRANSPOSE of the pages'
 *     S (key index first), as the pages' own kernels store it ("TileLang
 *     实战：KDA 从零到一--标量衰减", section 4.0).
 *   Alignment: every device pointer must be 16-byte aligned.
 *   Dtypes: q, k, v, o are DR_F32 (float) or DR_BF16 (bfloat16 bit pattern,
 *     uint16 storage); g, beta, h0, hT are always float.
 *   Gates: g = ln a, natural log, expected <= 0 (a in (0, 1]).  The library
 *     does not clamp.  Per-channel gates should be lower-bounded (the KDA
 *     page, section 2: a >= 0.9 keeps 2^(-gamma) small); the range is
 *     reported through `flags`, see DR_FLAG_*.
 *   Shapes: B, H >= 1, T >= 0 (T = 0 copies h0 to hT, or zeros it),
 *     Dk == Dv in {64, 128}, C == 64.  The dense forward (kda_fwd, gdn_fwd,
 *     decay_la_fwd, dr_forward, dr_forward_noalloc, dr_intra / dr_inter)
 *     also takes C == 128 (bf16 I/O, and fp32 I/O at Dk = 64): 128-token
 *     chunks built from two 64-token sub-chunks whose gate cumsum restarts
 *     at the sub-chunk ("TileLang 实战：KDA 从零到一–Kimi Delta Attention",
 *     section 2.3, the sub-chunk safeguard), so 2^(-gamma) never spans more
 *     than 64 positions; the rows of the 128 x 128 UT system are then
 *     joined by block elimination.  Other entry points return
 *     DR_ERR_UNSUPPORTED for C == 128.  T need not be a multiple of C: the
 *     last chunk is masked.
 *   Streams: `stream` is a hipStream_t (0 = the null stream).  All work is
 *     enqueued on it; nothing synchronises with the host.
 *   Debugging: with the environment variable DR_POISON_WORKSPACE=1 every
 *     entry point that takes a workspace first fills it with NaN (all-ones
 *     32-bit words, on `stream`), so that a kernel reading workspace the
 *     call has not written shows as NaN in the results.  (Stages 1 and 2 of
 *     dr_forward_stage and dr_inter read what an earlier call wrote and do
 *     not poison.)
 *   Errors: argument problems are detected on the host and return a negative
 *     status with nothing enqueued.  A failed launch returns DR_ERR_HIP.
 *     No exception crosses the ABI.  All entry points are reentrant; calls
 *     that share a workspace must not overlap.
 */
#ifndef DELTARULE_H
#define DELTARULE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DR_OK = 0,
    DR_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or dtype   */
    DR_ERR_UNSUPPORTED = -2,   /* valid but not built: Dk/Dv/C combination     */
    DR_ERR_HIP = -3,           /* a HIP launch failed                          */
    DR_ERR_WORKSPACE = -4,     /* workspace pointer null or too small          */
    DR_ERR_SCRATCH_LIMIT = -5  /* dr_forward_noalloc: problem exceeds the
                                  library's static scratch array            */
} dr_status;

typedef enum { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;
typedef enum { DR_KIND_KDA = 0, DR_KIND_GDN = 1, DR_KIND_DECAY_LA = 2 } dr_kind;

/* Gate-range flags, OR-ed into *flags (a device uint32) when flags != NULL.
 * The caller clears the word before the call and reads it after syncing.
 * Only the per-channel (KDA) path materialises 2^(-gamma):
 * (At C == 128 "chunk" means each 64-token sub-chunk, the span over which
 * the kernels form 2^(-gamma).)
 *   DR_FLAG_KM_FP16_RANGE: some chunk has -gamma_log2 >= 16 somewhere, so
 *     |k| * 2^(-gamma) could exceed the fp16 maximum 65504 (values are kept in
 *     bf16/fp32 here, so results stay valid);
 *   DR_FLAG_KM_OVERFLOW:   some chunk has -gamma_log2 >= 126: 2^(-gamma) is
 *     near the fp32/bf16 limit and results are not trustworthy. */
#define DR_FLAG_KM_FP16_RANGE 0x1u
#define DR_FLAG_KM_OVERFLOW   0x2u
/* Packed-sequence forwards only: cu_seqlens was not 0 = cu[0] <= cu[1] <=
 * ... <= cu[N] = T.  The kernels clamp the offsets into [0, T] (they stay in
 * bounds) but the results are not meaningful. */
#define DR_FLAG_BAD_SEQLENS   0x4u

/* Bytes of device workspace kda_fwd / gdn_fwd / decay_la_fwd / dr_forward
 * need for these sizes (0 for invalid sizes): the workspace of the path the
 * forward takes (see kda_fwd), which depends on the sizes and on the
 * DR_FWD_PATH environment variable only. */
size_t dr_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype);
/* Bytes of the segment-parallel path's workspace (dr_forward_stage): the
 * effective queries of every chunk in the I/O dtype ([B*H*NT][C][Dk]),
 * each segment's exit map [M | N] in fp32 ([Dk][Dk+Dv]) and its entry state
 * in the I/O dtype ([Dv][Dk]); 0 where that path is not built (fp32 I/O at
 * Dk = 128) or for invalid sizes. */
size_t dr_segment_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype);
/* Bytes of the record workspace of dr_intra / dr_inter: B*H*ceil(T/C)
 * records of dr_record_bytes(). */
size_t dr_record_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype);

/*
 * Full forward, KDA (per-channel gate).
 *   q, k:  [B,T,H,Dk] (dtype);  v: [B,T,H,Dv] (dtype)
 *   g:     [B,T,H,Dk] float, ln a
 *   beta:  [B,T,H] float
 *   h0:    [B,H,Dk,Dv] float, or NULL for a zero initial state
 *   o:     [B,T,H,Dv] (dtype), written
 *   hT:    [B,H,Dk,Dv] float, written, or NULL
 *   workspace: device buffer of at least dr_workspace_bytes(DR_KIND_KDA, ...)
 *   flags: device uint32 or NULL (see DR_FLAG_*)
 * Steps (all on `stream`): chunk-local log2 cumsum of g, the separable
 * exponent prep, the UT transform, the state pass and the chunk output.
 * Page sections: "TileLang 实战：KDA 从零到一–Kimi Delta Attention" sections
 * 1.2, 3.2, 3.3; "RNN的复兴04" (DPLR) section 5.3.5.
 * Two execution paths compute the same result (to rounding).  The
 * segment-parallel one runs where it is built (C == 64 with bf16 I/O, or
 * fp32 I/O at Dk = 64) unless the environment variable DR_FWD_PATH=records
 * selects the record path; the record path runs everywhere else:
 *   segment-parallel (bf16 I/O, and fp32 I/O at Dk = 64): the chunks of each
 *     (b, h) are grouped into segments (sizes chosen from B*H and T only).
 *     One kernel runs every segment from the entry state [I | 0], carrying
 *     the segment's transition and its zero-entry state through the chunks'
 *     cumsum, prep, UT transform and state update, and writes each chunk's
 *     output from a zero entry state plus its effective queries; a second
 *     kernel composes the segment entry states (and hT); a third adds
 *     q_eff S_in to the outputs of all segments but the first.  This is the
 *     entry-state hand-off of sequence-split evaluation ("Gated DeltaNet",
 *     section "前向计算的矩阵分解") inside one GPU.
 *   record path: dr_intra then dr_inter (always at C == 128).
 */
dr_status kda_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, void* o, float* hT,
                  int B, int T, int H, int Dk, int Dv, int C, int dtype,
                  void* workspace, size_t workspace_bytes, unsigned* flags,
                  void* stream);

/* Full forward, Gated DeltaNet: as kda_fwd but g is [B,T,H] (one scalar gate
 * per token and head).  The decay inside a chunk uses the ratio form
 * 2^(gamma_i - gamma_j), evaluated only where j <= i ("TileLang 实战：KDA
 * 从零到一--标量衰减" section 2.2), so no flag is ever raised. */
dr_status gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, void* o, float* hT,
                  int B, int T, int H, int Dk, int Dv, int C, int dtype,
                  void* workspace, size_t workspace_bytes, unsigned* flags,
                  void* stream);

/* Full forward, scalar-decay linear attention without the delta term:
 * S_t = a_t S_{t-1} + v_t k_t^T, o_t = S_t q_t; g is [B,T,H]; no beta. */
dr_status decay_la_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* h0, void* o, float* hT,
                       int B, int T, int H, int Dk, int Dv, int C, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---- packed sequences (varlen) ------------------------------------------- */

/*
 * Forward over N sequences packed along the token axis: token range
 * [cu_seqlens[i], cu_seqlens[i+1]) is sequence i.  Chunks never cross a
 * sequence boundary (each sequence is chunked from its own first token, its
 * last chunk masked), and each sequence has its own initial and final state:
 * the results equal N separate forwards.
 *   q, k, o: [T,H,Dk|Dv] (dtype; a batch of one), v: [T,H,Dv]
 *   g:       [T,H,Dk] float (kda) or [T,H] float; beta: [T,H] float
 *   cu_seqlens: DEVICE int32 [N+1], 4-byte aligned, with 0 = cu[0] <= cu[1]
 *            <= ... <= cu[N] = T.  Its contents are not read on the host:
 *            violations raise DR_FLAG_BAD_SEQLENS and are clamped.
 *   h0, hT:  [N,H,Dk,Dv] float or NULL
 *   workspace: at least dr_workspace_bytes_varlen(...): chunk records of all
 *            sequences plus the chunk table built on the device
 * Other arguments, conventions and errors as for kda_fwd / gdn_fwd /
 * decay_la_fwd.  N >= 1.
 */
size_t dr_workspace_bytes_varlen(int kind, int N, int T, int H, int Dk, int Dv, int C, int dtype);
dr_status kda_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int* cu_seqlens, int N,
                         const float* h0, void* o, float* hT,
                         int T, int H, int Dk, int Dv, int C, int dtype,
                         void* workspace, size_t workspace_bytes, unsigned* flags,
                         void* stream);
dr_status gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int* cu_seqlens, int N,
                         const float* h0, void* o, float* hT,
                         int T, int H, int Dk, int Dv, int C, int dtype,
                         void* workspace, size_t workspace_bytes, unsigned* flags,
                         void* stream);
dr_status decay_la_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                              const int* cu_seqlens, int N,
                              const float* h0, void* o, float* hT,
                              int T, int H, int Dk, int Dv, int C, int dtype,
                              void* workspace, size_t workspace_bytes, unsigned* flags,
                              void* stream);

/* ---- recurrent decode step ----------------------------------------------- */

/*
 * Decode: apply T new tokens per (b, h), one after the other, to a state kept
 * between calls, and return their outputs.  Same recurrence as kda_fwd, token
 * by token ("TileLang 实战：KDA 从零到一–Kimi Delta Attention" opening equation
 * and section 3.1; "Gated DeltaNet" section "Recurrent 算法代码解析"):
 *   S <- Diag(a_t) S;  r = beta_t (v_t - S^T k_t);  S <- S + k_t r^T;  o_t = S^T q_t
 * (decay_la_decode: S <- a_t S + k_t v_t^T).
 *   q, k:  [B,T,H,Dk] (dtype);  v: [B,T,H,Dv] (dtype)
 *   g:     [B,T,H,Dk] float for kda_decode, [B,T,H] float otherwise (ln a)
 *   beta:  [B,T,H] float (not for decay_la_decode)
 *   state: [B,H,Dk,Dv] float, the layout of h0/hT: read, then overwritten
 *          with the state after the T tokens (pass a forward's hT to
 *          continue a prefilled sequence)
 *   o:     [B,T,H,Dv] (dtype), written
 * Sizes as for the forward (Dk == Dv in {64, 128}); T = 0 leaves the state
 * unchanged and launches nothing.  All arithmetic is fp32; the state is read
 * and written once per call.  Nothing is allocated.  o may not alias the
 * inputs or the state.
 */
dr_status kda_decode(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, float* state, void* o,
                     int B, int T, int H, int Dk, int Dv, int dtype, void* stream);
dr_status gdn_decode(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, float* state, void* o,
                     int B, int T, int H, int Dk, int Dv, int dtype, void* stream);
dr_status decay_la_decode(const void* q, const void* k, const void* v, const float* g,
                          float* state, void* o,
                          int B, int T, int H, int Dk, int Dv, int dtype, void* stream);

/* ---- input prologue ------------------------------------------------------ */

/*
 * Optional elementwise pre-pass, fused into the kernels' input loads, that
 * turns a layer's raw projections into the recurrence's inputs (page "Gated
 * DeltaNet": the layer forward, section "门控与 Head 映射", and the token loads
 * of the recurrent kernel, section "加载 Token 与写入系数").  In this order:
 *   DR_PRO_QK_L2NORM    q <- q / sqrt(sum_d q_d^2 + 1e-6), the same for k,
 *                       per token and head over the Dk key channels
 *   (always)            q <- q * scale
 *   DR_PRO_BETA_SIGMOID beta <- 1 / (1 + exp(-beta))      (not for decay_la)
 *   DR_PRO_BETA_X2      with DR_PRO_BETA_SIGMOID: beta <- 2 / (1 + exp(-beta)),
 *                       a write strength in (0, 2)
 *   DR_PRO_GATE         scalar gates (gdn, decay_la) only:
 *                       g <- -exp(A_log[h]) * log(1 + exp(g + dt_bias[h])),
 *                       so the gate input g is the raw projection `a`
 * The transformed values are what the forward computes with; the input
 * tensors are not modified.  A NULL prologue, or ops = 0 with scale = 1,
 * runs the plain path.  The struct is read on the host during the call; the
 * A_log / dt_bias arrays are read by the kernels (device memory, 4-byte
 * aligned).
 * Errors: unknown bits, a non-finite scale, DR_PRO_BETA_X2 without
 * DR_PRO_BETA_SIGMOID, beta ops for decay_la, or DR_PRO_GATE without A_log
 * return DR_ERR_INVALID_ARG; DR_PRO_GATE for the per-channel (kda) gate
 * returns DR_ERR_UNSUPPORTED (the pages define gate generation for the scalar
 * gate only).
 */
#define DR_PRO_QK_L2NORM    0x1u
#define DR_PRO_BETA_SIGMOID 0x2u
#define DR_PRO_BETA_X2      0x4u
#define DR_PRO_GATE         0x8u
typedef struct {
    unsigned ops;            /* OR of DR_PRO_*                                */
    float scale;             /* query scale after normalisation (1 = none)    */
    const float* A_log;      /* DEVICE float [H], DR_PRO_GATE                 */
    const float* dt_bias;    /* DEVICE float [H] or NULL (no bias)            */
} dr_prologue;

/* kda_fwd / gdn_fwd / decay_la_fwd selected by `kind` (DR_KIND_*), with a
 * prologue (may be NULL).  beta is ignored for decay_la. */
dr_status dr_forward(int kind, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* h0, void* o, float* hT,
                     int B, int T, int H, int Dk, int Dv, int C, int dtype,
                     const dr_prologue* prologue, void* workspace, size_t workspace_bytes,
                     unsigned* flags, void* stream);
/*
 * dr_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, layouts, results and errors are those
 * of dr_forward; the same kernels run.  The workspace is a fixed device array
 * inside the library of DR_NOALLOC_SCRATCH_BYTES bytes (also returned by
 * dr_noalloc_scratch_bytes()).  Every GPU the library's code is loaded on
 * holds its own copy until the process ends.  The call itself allocates
 * nothing: its only set-up is a lookup of the array's device address, once
 * per device, on the first call on that device.
 *   Limit: problems whose dr_workspace_bytes(...) exceeds the array return
 *     DR_ERR_SCRATCH_LIMIT with nothing enqueued.
 *   Sharing: all calls on one GPU use that GPU's single array.  Calls that
 *     can overlap on one GPU (different streams, or several host threads
 *     without ordering) race on it and give wrong results; serialise them.
 *     Nothing in the array needs to be cleared between calls: each call
 *     writes every workspace byte it reads.
 */
#define DR_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t dr_noalloc_scratch_bytes(void);
dr_status dr_forward_noalloc(int kind, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* h0, void* o, float* hT,
                             int B, int T, int H, int Dk, int Dv, int C, int dtype,
                             const dr_prologue* prologue, unsigned* flags, void* stream);
/* The packed-sequence forwards selected by `kind`, with a prologue. */
dr_status dr_forward_varlen(int kind, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int* cu_seqlens, int N,
                            const float* h0, void* o, float* hT,
                            int T, int H, int Dk, int Dv, int C, int dtype,
                            const dr_prologue* prologue, void* workspace, size_t workspace_bytes,
                            unsigned* flags, void* stream);
/* The decode steps selected by `kind`, with a prologue applied to each new
 * token. */
dr_status dr_decode(int kind, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, float* state, void* o,
                    int B, int T, int H, int Dk, int Dv, int dtype,
                    const dr_prologue* prologue, void* stream);

/* ---- backward -------------------------------------------------------------- */

/*
 * Gradients of the forward selected by `kind` (the plain path: inputs as the
 * recurrence takes them, no prologue) with respect to q, k, v, g, beta and
 * h0, given the adjoints of o and hT (page "Gated DeltaNet", section
 * "反向传播：状态伴随与三角变换梯度"): the chunk operands are recomputed, the
 * chunk entry states rebuilt by a forward state pass, the state adjoint run
 * backwards over the chunks, and the per-chunk gradients taken through the
 * triangular inverse; the gate gradient is the reverse cumulative sum of the
 * log-gate adjoint inside each chunk.
 *   q, k, v, g, beta, h0: as for the forward (same sizes and layouts)
 *   dout:  [B,T,H,Dv] (dtype), the adjoint of o
 *   dhT:   [B,H,Dk,Dv] float, the adjoint of hT, or NULL (zero)
 *   dq, dk: [B,T,H,Dk] (dtype); dv: [B,T,H,Dv] (dtype), written
 *   dg:    float, shape of g, written
 *   dbeta: [B,T,H] float, written (delta kinds; ignored for decay_la)
 *   dh0:   [B,H,Dk,Dv] float, written, or NULL
 *   workspace: at least dr_backward_workspace_bytes(...): the recomputed
 *          chunk operands (fp32; for bf16 I/O also their bf16 copies for the
 *          reverse pass), the chunk entry states S_c, exit adjoints dS'_c
 *          ([Dk,Dv] per chunk), Vnew_c and dVnew_c (all four in the I/O
 *          dtype), and for bf16 I/O the reverse pass's segment maps and exit
 *          adjoints
 * Reverse pass (the state adjoint): with bf16 I/O the segment-parallel one:
 * the chunks of each (b, h) are grouped into segments, each segment's
 * affine adjoint map is formed from an identity start, the maps are
 * composed, and every segment is rerun from its true exit adjoint; the
 * environment variable DR_BWD_REV=slices selects the value-slice kernel
 * instead (the only one for fp32 I/O).
 * Gradient kernel (dq, dk, dv, dg, dbeta per chunk): with bf16 I/O one whose
 * operands are bf16 in LDS (two workgroups per compute unit), which forms
 * the chunk's P = N - M S as (I + diag(beta) L) Vnew (the same matrix, since
 * Vnew = (I + diag(beta) L)^-1 (N - M S)); DR_BWD_GRAD=f32lds selects the
 * kernel with fp32 LDS operands instead (the only one for fp32 I/O).
 * Chunk operands: on the path that takes both bf16 kernels above (the
 * default for bf16 I/O) one kernel recomputes them and also writes the chunk
 * records the forward state pass reads, so the forward's record kernel does
 * not run; on the other paths it runs first and a separate kernel
 * recomputes the operands in fp32.
 * Precision: accumulation is fp32 throughout. With fp32 I/O every product
 * runs on fp32 MFMA with fp32 operands.  With bf16 I/O the chunk-form L (and
 * Aqk except under per-channel gates), the segment-parallel reverse pass, and
 * the gradient kernel's products take bf16 operands (bf16 MFMA): in the
 * product T^T dVnew, which gives dv and dbeta's value term, T is split into
 * bf16 high and low parts; S_c, dS'_c, Vnew_c and dVnew_c are stored in
 * bf16; the entry states come from the forward's state pass on the bf16
 * records.
 * Reproducibility: every reduction (the dbeta and dg partials of the waves
 * of a chunk, the per-head sums of dr_backward_prologue) adds its terms in a
 * fixed order, so repeated calls with the same arguments give bit-identical
 * results.  Gate range: the backward raises no DR_FLAG_KM_* flags; they are
 * those of the forward call on the same inputs, which is the caller's check
 * (dr_backward_varlen's flags carries DR_FLAG_BAD_SEQLENS only).  Other
 * conventions and errors as for kda_fwd.  T = 0 writes dh0 = dhT (or zero)
 * and nothing else.  C must be 64.
 */
size_t dr_backward_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype);
dr_status dr_backward(int kind, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* h0, const void* dout, const float* dhT,
                      void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                      int B, int T, int H, int Dk, int Dv, int C, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward through the input prologue: the gradients with respect to the RAW
 * inputs a forward with the same dr_prologue took (dr_forward), i.e. the
 * recurrence's backward followed by the chain rule through the prologue
 * ("Gated DeltaNet", sections "门控与 Head 映射", "加载 Token 与写入系数" and
 * "反向传播：状态伴随与三角变换梯度"):
 *   dq = scale (dq^ - y_q (y_q . dq^)) / n_q,  dk = (dk^ - y_k (y_k . dk^)) / n_k
 *        (y = x / n, n = sqrt(|x|^2 + 1e-6); without DR_PRO_QK_L2NORM dq =
 *        scale dq^, dk = dk^)
 *   dbeta (raw logits) = s sigmoid(b) (1 - sigmoid(b)) dbeta^   (DR_PRO_BETA_SIGMOID)
 *   dg (raw gate input a) = -exp(A_log) sigmoid(a + dt_bias) dg^ (DR_PRO_GATE)
 *   dA_log[h] = sum over tokens of g^ dg^,  ddt_bias[h] = sum of dg
 * where ^ marks the recurrence's inputs and their gradients.  Arguments as
 * for dr_backward plus:
 *   dA_log:   DEVICE float [H], written (required with DR_PRO_GATE, else
 *             ignored); ddt_bias: DEVICE float [H], written (required when
 *             the prologue has a dt_bias, else ignored).  Both are sums of
 *             per-workgroup partials (kept in the workspace) added in a
 *             fixed order by one more kernel.
 *   prologue: as for dr_forward; NULL gives dr_backward.
 *   workspace: at least dr_backward_prologue_workspace_bytes(...): the
 *             recurrence's inputs (q^, k^, g^, beta^) plus dr_backward's.
 * dq, dk, dg and dbeta are first written with the recurrence's gradients and
 * then transformed in place.
 */
size_t dr_backward_prologue_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype);
dr_status dr_backward_prologue(int kind, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* h0, const void* dout, const float* dhT,
                               void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                               float* dA_log, float* ddt_bias,
                               int B, int T, int H, int Dk, int Dv, int C, int dtype,
                               const dr_prologue* prologue, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Backward of the packed-sequence forward (dr_forward_varlen): N sequences
 * concatenated along the token axis, each with its own state chain; chunks
 * never straddle two sequences ("Gated DeltaNet", section "反向传播：状态伴随
 * 与三角变换梯度", run per sequence as the packed forward runs).  The
 * gradients of each sequence are those dr_backward(_prologue) gives for that
 * sequence alone.
 *   q, k, v, g, beta, dout, dq, dk, dv, dg, dbeta: as for dr_backward with
 *          B = 1 and T the packed token count
 *   cu_seqlens: DEVICE int [N+1] token offsets, 0 = cu[0] <= ... <= cu[N] = T
 *          (4-byte aligned).  Offsets are clamped into [0, T] and made
 *          non-decreasing on the device; malformed ones raise
 *          DR_FLAG_BAD_SEQLENS in *flags (flags may be NULL).
 *   h0, dhT, dh0: [N,H,Dk,Dv] float, one state per sequence (may be NULL)
 *   dA_log, ddt_bias, prologue: as for dr_backward_prologue (prologue NULL:
 *          the plain path; dA_log / ddt_bias then ignored)
 *   workspace: at least dr_backward_varlen_workspace_bytes(kind, N, T, H,
 *          Dk, Dv, C, dtype, with_prologue), with_prologue nonzero when a
 *          prologue that does something is passed: the chunk table and
 *          sequence descriptors, then dr_backward's per-chunk buffers for
 *          ceil(T/C) + N chunk slots per head (plus the prologue's part).
 * The segment-parallel reverse pass (bf16 I/O) takes one segment per
 * sequence and head.  A sequence of length 0 gets dh0 = dhT (or zero).
 * Other conventions and errors as for dr_backward.
 */
size_t dr_backward_varlen_workspace_bytes(int kind, int N, int T, int H, int Dk, int Dv, int C, int dtype,
                                          int with_prologue);
dr_status dr_backward_varlen(int kind, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int* cu_seqlens, int N, const float* h0,
                             const void* dout, const float* dhT, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dh0, float* dA_log, float* ddt_bias,
                             int T, int H, int Dk, int Dv, int C, int dtype,
                             const dr_prologue* prologue, void* workspace, size_t workspace_bytes,
                             unsigned* flags, void* stream);

/* ---- the individual steps ---------------------------------------------- */

/*
 * Step a1: chunk-local inclusive cumsum of log gates, converted to log2 units:
 *   gamma[b, cC + r, h, d] = log2(e) * sum_{s <= r} g[b, cC + s, h, d]
 * restarting in every chunk of C tokens ("TileLang 实战：KDA 从零到一–Kimi Delta
 * Attention" section 0; "07 · linear 路线（二）" section 3.5: the cumsum is local).
 *   g, gamma: [B,T,H,D] float (D = Dk for per-channel gates, D = 1 for scalar
 *   gates).  D in [1, 256].  gamma may not alias g.
 */
dr_status dr_chunk_cumsum(const float* g, float* gamma, int B, int T, int H, int D, int C,
                          void* stream);

/*
 * Step a2: separable-exponent prep for per-channel gates ("TileLang 实战：KDA
 * 从零到一–Kimi Delta Attention" section 1.2; "RNN的复兴04" section 5.3.4):
 *   kp   = k * 2^gamma,        km = k * 2^(-gamma),     qp = q * 2^gamma,
 *   kbar = k * 2^(gamma_last - gamma)  (gamma_last: last valid row of the chunk),
 *   phi[b, c, h, d] = 2^(gamma_last)
 *   q, k, kp, km, qp, kbar: [B,T,H,Dk] (dtype); gamma: [B,T,H,Dk] float (from
 *   step a1); phi: [B,ceil(T/C),H,Dk] float.  Any output pointer may be NULL
 *   to skip it.  flags: as for kda_fwd.
 */
dr_status dr_kda_prep(const void* q, const void* k, const float* gamma,
                      void* qp, void* kp, void* km, void* kbar, float* phi,
                      int B, int T, int H, int Dk, int C, int dtype, unsigned* flags,
                      void* stream);

/*
 * K1 alone: steps a1 + a2 + a3 fused, chunk-parallel.  Fills `workspace`
 * with one record per (b, h, chunk), record index (b*H + h)*NT + c,
 * NT = ceil(T/C).  A record holds, in elements of the I/O dtype (r, i =
 * positions in the chunk, d = key channel, e = value channel):
 *   W    C*Dk     W = T diag(beta) K+   (delta kinds; unused for decay_la)
 *   Qt   C*Dk     q * 2^gamma
 *   KbT  Dk*C     k * 2^(gamma_last - gamma), key-major
 *   Aqk  C*C      Tril_incl(Q~ K-^T)  (zero above the diagonal)
 *   UT   Dv*C     U = T diag(beta) V  (decay_la: V)
 *   phi  Dk float 2^(gamma_last)
 * with T = (I + A)^-1, A = diag(beta) StrictLower(K+ K-^T) ("TileLang 实战：
 * KDA 从零到一–Kimi Delta Attention" sections 3.2-3.3, row-beta pairing).
 * Each block is stored in the MFMA fragment order the state pass reads
 * (lane l, element j, 32-row blocks split by prow(h, r) = 8(r/4) + 4h + r%4,
 * pw(w, r) = 32(w/2) + prow(w%2, r)):
 *   W, Qt [w<C/16][kb<Dk/32][l<64][j<8] = X[pw(w, l%16)][32kb + 8(l/16) + j]
 *   KbT   [w<Dk/32][h<2][kb<C/32][l][j<8] = Kbar[32kb + 8(l/16) + j][32w + prow(h, l%16)]
 *   Aqk   [w<C/16][kb<C/32][l][j<8] = Aqk[pw(w, l%16)][32kb + 8(l/16) + j]
 *   UT    [t<Dv/16][w<C/16][l][i<4] = U[32(w/2) + 8(l/16) + 4(w%2) + i][16t + l%16]
 * Rows of a ragged last chunk beyond T are zero.  At C == 128 the record is
 * that of the whole 128-token chunk (gamma based at its start, Kbar and phi
 * at its end, Aqk 128 x 128) although the kernel builds it from the two
 * sub-chunks.  Record size:
 * dr_record_bytes(); workspace: dr_record_workspace_bytes().  For GDN / decay_la, g is [B,T,H] and beta may be NULL
 * for decay_la.
 */
dr_status dr_intra(int kind, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                   void* workspace, size_t workspace_bytes, unsigned* flags, void* stream);

/*
 * K2 alone: steps a4 + a5 fused.  For each (b, h), in chunk order:
 *   Vnew = U - W S  (decay_la: Vnew = V),
 *   O    = Qt S + Aqk Vnew,
 *   S   <- Diag(phi) S + KbT Vnew
 * starting from S = h0 (or 0) and writing o and hT ("RNN的复兴04" section
 * 5.3.5; "TileLang 实战：KDA 从零到一–Kimi Delta Attention" section 3.2).
 * Reads the records written by dr_intra with the same arguments.
 */
dr_status dr_inter(int kind, const float* h0, void* o, float* hT,
                   int B, int T, int H, int Dk, int Dv, int C, int dtype,
                   const void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of one workspace record (0 for unsupported sizes; C is 64, or 128
 * where built). */
size_t dr_record_bytes(int Dk, int Dv, int C, int dtype);

/*
 * One stage of the segment-parallel forward that kda_fwd / gdn_fwd /
 * decay_la_fwd / dr_forward run, for callers that time or split them; the
 * three stages in order on one stream, with the same arguments and
 * workspace, equal dr_forward:
 *   stage 0  local segment pass: reads q, k, v, g, beta, h0 (segment 0 starts
 *            from it), writes o (final for the first segment) and the
 *            workspace;
 *   stage 1  entry-state composition: reads the workspace, writes hT (may be
 *            NULL) and the segment entry states into the workspace;
 *   stage 2  output correction: reads the workspace, updates o.
 * Arguments a stage does not use may be NULL.  The workspace is sized by
 * dr_segment_workspace_bytes.  Returns DR_ERR_UNSUPPORTED for sizes the
 * segment path is not built for (fp32 I/O at Dk = 128).
 */
dr_status dr_forward_stage(int stage, int kind, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* h0, void* o, float* hT,
                           int B, int T, int H, int Dk, int Dv, int C, int dtype,
                           const dr_prologue* prologue, void* workspace, size_t workspace_bytes,
                           unsigned* flags, void* stream);

/* Human-readable text for a status code (static storage). */
const char* dr_status_string(int status);

/* ABI version of this library: 7 (1, plus the prologue entry points in 2, the
 * backward in 3, the backward through the prologue in 4, the packed-sequence
 * backward in 5, the allocation-free forward, the segment-parallel forward's
 * stages and the record workspace query in 6, 128-token sub-chunked chunks
 * for the dense forward in 7). */
int dr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTARULE_H */
