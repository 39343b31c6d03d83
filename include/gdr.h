/*
 * gdr.h -- C ABI of the MI355X (gfx950) gated delta-rule mixer library, libgdr.
 *
 * The mixer keeps a fixed-size state S in R^{d_k x d_v} per (sequence, value
 * head) and, per token t, with alpha_t = exp(g_t):
 *
 *   e_t  = beta_t k_t            (tied gates: Gated DeltaNet, KDA)
 *        = b_t (.) k_t           (decoupled erase gate on the key axis: Gated DeltaNet-2)
 *   z_t  = beta_t v_t  |  w_t (.) v_t   (write gate on the value axis)
 *   S_t  = (I - k_t e_t^T) Diag(alpha_t) S_{t-1} + k_t z_t^T
 *   o_t  = scale * S_t^T q_t     (read after the write)
 *
 * Sources, by page title and section:
 *   "Resumo Técnico: Gated DeltaNet-2", section "Regra Delta Portão-2": the
 *     update equation above, the erase gate b_t in [0,1]^{d_k} and write gate
 *     w_t in [0,1]^{d_v}; tying b = w = beta recovers KDA, and a scalar alpha
 *     recovers Gated DeltaNet.
 *   "Uma análise das variantes de atenção linear da família DeltaNet",
 *     sections "Gated DeltaNet: esquecer primeiro o estado inteiro" (forget,
 *     predict, correct, write, in that order), "Kimi Delta Attention:
 *     atenuação por canal" (per-key-channel decay, read after write, read
 *     scale), "Transição diagonal-mais-baixo-posto" (g = log alpha <= 0 is
 *     what is stored; the d_k x d_v state layout), "Kernel Triton recorrente
 *     fundido para decode" (the recurrent form for decode) and "Chunkwise
 *     KDA" (the chunked form gives exactly the same state and outputs).
 *   "Gated DeltaNet: o mixer em 48 das 64 camadas", section "Conceito": 16 QK
 *     heads serve 48 V heads; the fp32 state of 48 heads of 128 x 128 is
 *     about 3 MiB per layer.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers are device pointers to contiguous row-major arrays, owned by the
 *   caller. The library never frees caller memory and keeps no pointer after
 *   a call returns.
 * - Layouts (io = the desc's io dtype, float32 or bfloat16):
 *     q, k : [B, T, H_qk, d_k] io      v, o : [B, T, H_v, d_v] io
 *     beta : [B, T, H_v] float32
 *     g    : [B, T, H_v] float32 (GDR_DECAY_SCALAR) or [B, T, H_v, d_k] float32
 *            (GDR_DECAY_CHANNEL); g = log(alpha) must be finite and <= 0
 *     b    : [B, T, H_v, d_k] io       w : [B, T, H_v, d_v] io
 *     S    : [B, H_v, d_k, d_v] float32; row i is key channel i, column j
 *            value channel j.
 *   For decode the T axis is absent (one token per sequence).
 * - Alignment: every array pointer must be 16-byte aligned (the kernels use
 *   16-byte vector accesses), except beta and a scalar-decay g, which need
 *   4 bytes. A misaligned pointer is rejected with GDR_E_INVAL.
 * - V head h reads QK head h / (H_v / H_qk): each QK head serves a contiguous
 *   group of H_v / H_qk V heads.
 * - Gate modes: beta != NULL and b == w == NULL (tied), or beta == NULL and
 *   both b and w != NULL (decoupled). g == NULL exactly when decay is
 *   GDR_DECAY_NONE (alpha = 1, plain DeltaNet). Anything else: GDR_E_INVAL.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream): they validate, enqueue kernels and return without synchronising.
 *   Arguments are validated before any HIP call; a rejected call enqueues
 *   nothing. Inputs are not checked for NaN/Inf (that would cost a pass over
 *   memory): non-finite inputs give non-finite outputs.
 * - Every call returns a gdr_status. On a non-OK status, gdr_last_error()
 *   returns a message for the calling thread.
 * - Supported: d_k, d_v in {32, 64, 128}; chunk == 64; io float32 or
 *   bfloat16. Arithmetic: state and accumulation in float32; bfloat16 io runs
 *   the chunk products on bf16 matrix cores, float32 io on float32 ones.
 *   Any finite g <= 0 is accepted by every call: the chunked forward and
 *   backward reference the decay inside a chunk to its 16-token blocks
 *   ("Pipeline Triton da versão por chunks": the diagonal 16-token blocks
 *   first), so no factor they form exceeds exp(40), and a block that decays
 *   further is formed entry by entry.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_E_INVAL = -1,        /* bad pointer, size or gate combination */
    GDR_E_UNSUPPORTED = -2,  /* valid request this build does not implement */
    GDR_E_HIP = -3,          /* a HIP runtime call or kernel launch failed */
    GDR_E_NOMEM = -4         /* device allocation failed (gdr_state_alloc) */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef enum { GDR_DECAY_NONE = 0, GDR_DECAY_SCALAR = 1, GDR_DECAY_CHANNEL = 2 } gdr_decay;

typedef struct {
    int B;         /* sequences */
    int T;         /* tokens per sequence (prefill); ignored by decode */
    int H_qk;      /* query/key heads */
    int H_v;       /* value heads; a multiple of H_qk */
    int d_k;       /* key head dim */
    int d_v;       /* value head dim */
    int io_dtype;  /* gdr_dtype of q, k, v, b, w, o */
    int decay;     /* gdr_decay */
    int chunk;     /* chunk length of the prefill schedule (64) */
    float scale;   /* read scale s in o = s S^T q (1 for plain Gated DeltaNet) */
} gdr_desc;

/* Bytes of one fp32 state block [B, H_v, d_k, d_v]; 0 if a size is not
 * positive. Needs no GPU. Example: (1, 48, 128, 128) -> 3,145,728 (3 MiB). */
size_t gdr_state_bytes(int B, int H_v, int d_k, int d_v);

/* Allocate a zero-filled fp32 state [B, H_v, d_k, d_v] on the current device
 * (hipMalloc, then a zero fill enqueued on `stream`). *state receives the
 * pointer and *bytes (if not NULL) its size. Free with gdr_state_free. */
int gdr_state_alloc(int B, int H_v, int d_k, int d_v, float **state, size_t *bytes, void *stream);

/* Free a state from gdr_state_alloc (NULL is a no-op). Synchronises the
 * device like hipFree. */
int gdr_state_free(float *state);

/* Device workspace bytes gdr_chunk_fwd needs for `desc`; needs no GPU.
 * The workspace holds, per (sequence, V head, chunk), the chunk's factors
 * that do not depend on the state: the erase-side WY factor Y (C x d_k), the
 * write-side factor U_z (d_v x C) and the in-chunk read matrix A (C x C), in
 * the io dtype; with per-channel decay also the decayed queries (C x d_k) and
 * the keys decayed to the chunk end (d_k x C), and the end-of-chunk decay
 * (d_k float32); with a scalar decay (or none) instead two per-token decay
 * tables (2 C float32), and one k^T (d_k x C) and one q (C x d_k), io dtype,
 * per (sequence, QK head, chunk). For long sequences with few heads it also
 * holds, per (sequence, V head, sweep segment but the last), three
 * d_k x d_v float32 matrices of the segmented sweep (the segment's
 * transition, its end state from a zero entry, and the entry state of the
 * next segment). Returns 0 bytes when B or T is 0. */
int gdr_chunk_workspace_bytes(const gdr_desc *desc, size_t *bytes);

/* Chunkwise-parallel prefill over T tokens: "Chunkwise KDA" and "Pipeline
 * Triton da versão por chunks" (family analysis page); "Treinamento Paralelo
 * Eficiente por Blocos" (Gated DeltaNet-2 summary page). Per 64-token chunk:
 * cumulative log decay, decay absorbed into the erase/write factors, the
 * unit-lower-triangular (I + T) system solved on chip, then one sweep over
 * chunks that carries the fp32 state.
 *   S0: initial state, or NULL for zeros. ST: final state; may equal S0
 *   (in-place update). o: outputs. T may be any positive length (the last
 *   chunk may be partial). workspace: at least gdr_chunk_workspace_bytes;
 *   its contents on entry are ignored. Float32 io at d = 128 takes tied
 *   gates (beta) with a scalar decay or none; other gate and decay modes
 *   at that size return GDR_E_UNSUPPORTED (gdr_recurrent_fwd serves them). */
int gdr_chunk_fwd(const gdr_desc *desc, const void *q, const void *k, const void *v,
                  const float *g, const float *beta, const void *b, const void *w,
                  const float *S0, void *o, float *ST, void *workspace, size_t workspace_bytes,
                  void *stream);

/* gdr_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Same arguments, layouts, rules and results as gdr_chunk_fwd,
 * without the workspace arguments: the workspace is the library's own
 * device array of GDR_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU, reserved
 * when the library's code is loaded on that GPU and held until the process
 * ends. The call allocates nothing; its first call on a device looks the
 * array's address up (hipGetSymbolAddress), with that device current.
 *   Limit: gdr_chunk_workspace_bytes(desc) <= GDR_NOALLOC_SCRATCH_BYTES,
 *   else GDR_E_UNSUPPORTED before anything is enqueued (a 64 MiB array
 *   holds, for example, the workspace of a 1024-token call with 48 V heads
 *   of d = 128 in bfloat16).
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents (the call needs none of them: every workspace element
 *   it reads it first writes). Calls that overlap in time on one GPU (on
 *   different streams, or from different host threads without ordering)
 *   race on the array and give wrong results; order them on one stream.
 *   The stream must belong to the current device. */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdr_chunk_fwd_noalloc(const gdr_desc *desc, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const void *b, const void *w,
                          const float *S0, void *o, float *ST, void *stream);

/* One recurrent decode step for B sequences, one token each ("Kernel Triton
 * recorrente fundido para decode", family analysis page): reads and writes
 * every state S[b, h] in place exactly once. q, k: [B, H_qk, d_k];
 * v, o: [B, H_v, d_v]; beta: [B, H_v]; g: [B, H_v] or [B, H_v, d_k];
 * b: [B, H_v, d_k]; w: [B, H_v, d_v]. desc->T and desc->chunk are ignored. */
int gdr_decode_step(const gdr_desc *desc, const void *q, const void *k, const void *v,
                    const float *g, const float *beta, const void *b, const void *w,
                    float *S, void *o, void *stream);

/* Fused recurrent forward over T tokens from a persistent state ("Kernel
 * Triton recorrente fundido para decode", family analysis page): the
 * token-by-token recurrence with each state block held in registers, so every
 * state is read once and written once per call whatever T is. Meant for short
 * runs from a live state (a few new tokens per sequence in serving, or
 * checking k drafted tokens), where the chunked form's per-chunk factors cost
 * more than they save. Arithmetic is about 4 d_k d_v flops per token and head
 * on the vector units, so long prefills belong to gdr_chunk_fwd.
 *   Layouts, gate modes and results (up to rounding order) as gdr_chunk_fwd;
 *   desc->chunk is ignored and no workspace is needed. S0: initial state, or
 *   NULL for zeros. ST: final state; may equal S0 (in-place update) and must
 *   not otherwise overlap it (GDR_E_INVAL). T == 0 writes S0 (or zeros) to ST
 *   and touches no per-token array. Supported: d_k == d_v in {32, 64, 128},
 *   io float32 or bfloat16. */
int gdr_recurrent_fwd(const gdr_desc *desc, const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const void *b, const void *w,
                      const float *S0, void *o, float *ST, void *stream);

/* The input stage: the step just before the recurrence, turning raw
 * projections into q, k, v and gates ("Gated DeltaNet: o mixer em 48 das 64
 * camadas", section "Conceito": a short causal depthwise convolution of
 * kernel 4 over the projected sequences; family analysis page, "Notação e
 * ordem da derivação": normalised keys; Gated DeltaNet-2 post, its code
 * listing: sigmoid erase and write gates). With it, per token t:
 *   x'_t = sum_{j=0..3} conv_w[c][j] x_{t-3+j}   per channel c, tokens before
 *          t = 0 taken from conv_in (zeros if NULL); no activation follows
 *   q = x'_q / sqrt(|x'_q|^2 + 1e-12), k likewise (per token and head over
 *          d_k); v = x'_v
 *   beta = sigmoid(beta_in); b = sigmoid(b_in); w = sigmoid(w_in)
 *   g = -c_h softplus(g_in), c_h = decay_scale[h] (1 if NULL)
 * Convolution channels are ordered: the H_qk*d_k channels of q, then those
 * of k, then the H_v*d_v channels of v (head-major in each).
 * Alignment: conv_w, conv_in and conv_out 16 bytes; decay_scale 4 bytes. */
typedef struct {
    const float *conv_w;       /* [2*H_qk*d_k + H_v*d_v, 4] float32 taps; tap 3
                                  multiplies the current token. Required. */
    const void *conv_in;       /* [B, 3, channels] io: the 3 raw tokens before
                                  this call (row 2 = the latest); NULL = zeros */
    void *conv_out;            /* [B, 3, channels] io: written with the last 3
                                  raw tokens (rows before the call's first
                                  token come from conv_in), the next call's
                                  conv_in; NULL = not written. Must not
                                  overlap conv_in (ping-pong two buffers). */
    const float *decay_scale;  /* [H_v] float32 c_h > 0, or NULL for 1 */
} gdr_input_stage;

/* gdr_chunk_fwd with the input stage in front of it. With a scalar decay
 * (or none) the stage is fused into the prefill's load stage: the per-chunk
 * kernel reads the raw projections (plus the 3 tokens before each chunk) and
 * applies the convolution, the normalisation and the activations before
 * building the chunk's factors, so the processed q, k, v never travel
 * through memory. With a per-channel decay the convolution and the
 * normalisation run as a pass of their own that writes the processed q, k,
 * v (io dtype) into the workspace; the prefill reads them there and applies
 * the gate and decay activations to the raw g, beta, b and w as it loads
 * them. Arguments as gdr_recurrent_fwd_in, plus a workspace of at least
 * gdr_chunk_fwd_in_workspace_bytes (gdr_chunk_workspace_bytes plus, for a
 * per-channel decay, the processed q, k, v). The chunk products run on
 * bf16 matrix cores for bf16 io, so the processed q, k and v are rounded to
 * bf16 there, as the io values of gdr_chunk_fwd are. */
int gdr_chunk_fwd_in_workspace_bytes(const gdr_desc *desc, size_t *bytes);

int gdr_chunk_fwd_in(const gdr_desc *desc, const gdr_input_stage *stage, const void *q, const void *k,
                     const void *v, const float *g, const float *beta, const void *b, const void *w,
                     const float *S0, void *o, float *ST, void *workspace, size_t workspace_bytes,
                     void *stream);

/* gdr_recurrent_fwd with the input stage fused into its token loop: q, k, v
 * are the raw projections (before the convolution), beta, b, w the gate
 * inputs before the sigmoid and g the decay input before -c softplus, in
 * gdr_recurrent_fwd's layouts. A decode step is the T = 1 call, with conv_in
 * and conv_out alternating between two buffers. stage must be non-NULL with
 * conv_w set; GDR_E_INVAL otherwise (or if conv_out overlaps conv_in). */
int gdr_recurrent_fwd_in(const gdr_desc *desc, const gdr_input_stage *stage, const void *q, const void *k,
                         const void *v, const float *g, const float *beta, const void *b, const void *w,
                         const float *S0, void *o, float *ST, void *stream);

/* Gradients of the recurrence ("Resumo Técnico: Gated DeltaNet-2", section
 * "Treinamento Paralelo Eficiente por Blocos", names a gate-aware backward
 * pass; what is computed is the exact gradient of the forward recurrence of
 * gdr_recurrent_fwd / gdr_chunk_fwd, walking the tokens in reverse):
 *   dS    += s q_t dO_t^T,  dq_t = s S_t dO_t,  du_t = dS^T k_t
 *   dk_t   = dS u_t + (beta_t or b_t) . de_t,   de_t = -Sbar_t du_t
 *   dSbar  = dS - e_t du_t^T,  dg_t = alpha_t . rowsum(dSbar . S_{t-1})
 *            (summed over d_k for a scalar decay),  dS = Diag(alpha_t) dSbar
 *   tied gates: dbeta_t = k_t . de_t + v_t . du_t, dv_t = beta_t du_t
 *   decoupled:  db_t = k_t . de_t, dw_t = v_t . du_t, dv_t = w_t . du_t
 * with Sbar_t = Diag(alpha_t) S_{t-1}, u_t = z_t - Sbar_t^T e_t. Keys and
 * queries shared by grouped V heads receive the sum over those heads.
 *   Inputs: q, k, v, g, beta, b, w, S0 exactly as given to the forward call
 *   (same desc; desc->chunk is ignored); dO [B,T,H_v,d_v] in the io dtype
 *   (dL/do); dST [B,H_v,d_k,d_v] float32 (dL/dS_T) or NULL for zeros.
 *   Outputs, all float32, in the layouts of the matching inputs: dq, dk
 *   [B,T,H_qk,d_k] and dv [B,T,H_v,d_v] (required); dg (exactly when g is
 *   given), dbeta (exactly when beta is), db and dw (exactly when b and w
 *   are); dS0 [B,H_v,d_k,d_v] (dL/dS0) or NULL (not written).
 *   Outputs must not overlap one another, the inputs or the workspace
 *   (GDR_E_INVAL). Alignment as the forward calls; dg 16 bytes for a
 *   per-channel decay, else 4; dbeta 4.
 *   workspace: gdr_recurrent_bwd_workspace_bytes bytes, owned by the caller,
 *   holding the state entering every block of 4 tokens
 *   (ceil(T/4) * B * H_v * d_k * d_v floats) and per-column-tile partial
 *   sums (about 16 * B * T * H_v * d_k bytes per 32 value columns).
 *   Work: a forward pass that stores the checkpoints, a reverse pass that
 *   replays each block of 4 tokens from its checkpoint before walking it
 *   backwards, and a reduction over column tiles and grouped heads; vector
 *   units only. T == 0 writes dST (or zeros) to dS0 and touches nothing
 *   else. Supported: d_k == d_v in {32, 64, 128}, io float32 or bfloat16. */
int gdr_recurrent_bwd_workspace_bytes(const gdr_desc *desc, size_t *bytes);
int gdr_recurrent_bwd(const gdr_desc *desc, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const void *b, const void *w, const float *S0, const void *dO,
                      const float *dST, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *db,
                      float *dw, float *dS0, void *workspace, size_t workspace_bytes, void *stream);

/* The same gradients in chunked form, parallel over chunks of 64 tokens
 * ("Resumo Técnico: Gated DeltaNet-2", section "Treinamento Paralelo
 * Eficiente por Blocos"; the chunked forward of "Uma análise das variantes
 * de atenção linear da família DeltaNet", section "Chunkwise KDA" and its
 * subsections, differentiated line by line). Per chunk, with S the state entering it,
 * G the in-chunk sums of g, E~ = e . exp(G), Q~ = q . exp(G),
 * Kend = k . exp(G_end - G), Gamma = exp(G_end), T and A the decayed
 * products of e, q with k below the diagonal, L = (I + T)^-1, Y = L E~ and
 * U = L Z - Y S:
 *   dU = s A^T dO + Kend dS_next,  dS = Gamma . dS_next + s Q~^T dO - Y^T dU
 *   dR = L^T dU (= dZ),  dT = -dR U^T,  dA = s dO U^T,
 *   dE~ = -dR S^T + dT K~,  dQ~ = s dO S^T + dA K~,  dKend = U dS_next^T,
 * then the gates and the exponentials as in the recurrence's gradient.
 *   Arguments, outputs, overlap and alignment rules: as gdr_recurrent_bwd,
 *   with desc->chunk == 64 (GDR_E_UNSUPPORTED otherwise).
 *   workspace: gdr_chunk_bwd_workspace_bytes bytes, owned by the caller:
 *   float32 per chunk unit (sequence, V head, chunk), about
 *   4 * (10 * 64 * d + 4 * 64 * 64 + 2 * d * d) bytes, plus two
 *   B * T * H_v * d_k float32 arrays when H_v > H_qk.
 *   Work: five launches (a per-chunk pass forming the factors and solving
 *   the unit lower triangular system, a forward pass over chunks storing the
 *   states, a backward pass over chunks storing dS and dU, and two per-chunk
 *   gradient passes), plus a sum over grouped V heads; fp32 vector
 *   arithmetic. T == 0 writes dST (or zeros) to dS0 and touches nothing
 *   else. Supported: d_k == d_v in {32, 64, 128}, io float32 or bfloat16,
 *   every decay and gate mode. */
int gdr_chunk_bwd_workspace_bytes(const gdr_desc *desc, size_t *bytes);
int gdr_chunk_bwd(const gdr_desc *desc, const void *q, const void *k, const void *v, const float *g,
                  const float *beta, const void *b, const void *w, const float *S0, const void *dO,
                  const float *dST, float *dq, float *dk, float *dv, float *dg, float *dbeta, float *db, float *dw,
                  float *dS0, void *workspace, size_t workspace_bytes, void *stream);

/* ---- Normalised linear attention ----
 * The read with a normaliser of page "Linear attention e fast weights",
 * section "Conceito": the output for token t is the average of the values
 * v_i, i <= t, weighted by phi(q_t) . phi(k_i), kept incrementally as a
 * matrix state and a normaliser per (sequence, V head):
 *   S_t = S_{t-1} + phi(k_t) v_t^T,   z_t = z_{t-1} + phi(k_t),
 *   o_t = S_t^T phi(q_t) / (z_t^T phi(q_t)).
 * The feature map phi is the caller's: phq and phk are phi(q) and phi(k)
 * (for a weighted average phi must be non-negative and z_t^T phi(q_t) > 0;
 * a zero normaliser gives the IEEE quotient, not an error).
 *   desc: decay must be GDR_DECAY_NONE; scale, and the gates of the other
 *   calls, do not apply (the normaliser cancels any read scale). d_k == d_v
 *   in {32, 64, 128}, io float32 or bfloat16; chunk == 64 for the prefill.
 *   phq, phk: [B, T, H_qk, d] io; v, o: [B, T, H_v, d] io; V head h reads QK
 *   head h / (H_v / H_qk). S: [B, H_v, d, d] float32 (row = key channel);
 *   z: [B, H_v, d] float32. Alignment 16 bytes for every array.
 *   Arithmetic: float32 state and normaliser; with bfloat16 io the chunk
 *   products run on bf16 matrix cores (the state enters Q S rounded to
 *   bf16), with float32 io on float32 matrix cores. */

/* Device workspace bytes gdr_norm_la_fwd needs (0 when the sequence is not
 * split into segments); needs no GPU. It holds, per (sequence, V head,
 * segment of the sequence run side by side), a d x d + d float32 slab: the
 * segment's sums, then the state entering it. */
int gdr_norm_la_workspace_bytes(const gdr_desc *desc, size_t *bytes);

/* Prefill over T tokens from (S0, z0) (NULL: zeros) to (ST, zT), in the
 * chunked form (64-token chunks: A = tril(phq phk^T), O = (Q S + A V) /
 * (Q z + rowsum A)). ST may be S0 and zT may be z0 (in-place update);
 * outputs must not otherwise overlap inputs or one another (GDR_E_INVAL).
 * T == 0 writes S0 and z0 (or zeros) to ST and zT. */
int gdr_norm_la_fwd(const gdr_desc *desc, const void *phq, const void *phk, const void *v,
                    const float *S0, const float *z0, void *o, float *ST, float *zT,
                    void *workspace, size_t workspace_bytes, void *stream);

/* One decode step for B sequences, one token each: phq, phk [B, H_qk, d],
 * v, o [B, H_v, d]; S and z updated in place. desc->T and desc->chunk are
 * ignored. */
int gdr_norm_la_decode_step(const gdr_desc *desc, const void *phq, const void *phk, const void *v,
                            float *S, float *z, void *o, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *gdr_last_error(void);

/* Library ABI version: 1. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
