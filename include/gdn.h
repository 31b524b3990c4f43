/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated-delta-rule forward library.
 *
 * One recurrence covers every model served here. With S in R^{dk x dv} (rows are
 * key channels) and per token (or per Householder sub-step) vectors a, b in R^dk,
 * w in R^dv and a forget vector alpha in (0,1]^dk:
 *
 *     S_t = (I - a_t b_t^T) Diag(alpha_t) S_{t-1} + a_t w_t^T,     o_t = S_t^T q_t
 *
 *   FG2-GDN   a = b = sqrt(beta) . k,  w = sqrt(beta) . v,  alpha per channel
 *             (FG2-GDN, "Enhancing Long-Context Gated Delta Networks with Doubly
 *             Fine-Grained Control": summary section 2, reading notes section 2.2,
 *             eq. (11)). With beta_v given: w = sqrt(beta_v) . v (FG2-GDN+, eq. (13)).
 *   KDA       a = b = sqrt(beta) k, w = sqrt(beta) v, beta scalar, alpha per channel
 *   GDN       as KDA with a scalar alpha (GDN2-stability page, "Problem Description")
 *   DELTAPRODUCT  n_h steps per token; step i: a = k_i, b = beta_i k_i, w = beta_i v_i;
 *             the scalar gate alpha acts once per token before step 1; q is read after
 *             step n_h (DeltaProduct summary, "Approach")
 *   ASYM      GDN2 / RWKV-7-style  S' = S' D (I - eta j k^T) + eta v k^T, o = S' q
 *             (GDN2-stability page, eq. (1)); the library state is S = S'^T, so
 *             a = k, b = eta j, w = eta v, alpha = D.
 *
 * Layouts: every array is row-major and contiguous; every pointer is a device
 * pointer aligned to 16 bytes.
 *   q, o                      [B, T, H, dk] / [B, T, H, dv]
 *   k, v (all but DP)         [B, T, H, dk] / [B, T, H, dv]
 *   k, v (DELTAPRODUCT)       [B, T, H, n_h, dk] / [B, T, H, n_h, dv]
 *   FG2   alpha, beta         [B, T, H, dk];  beta_v [B, T, H, dv] (optional)
 *   KDA   alpha [B, T, H, dk];  beta [B, T, H]
 *   GDN   alpha, beta         [B, T, H]
 *   DELTAPRODUCT  alpha (gate) [B, T, H];  beta [B, T, H, n_h]
 *   ASYM  alpha (= D) [B, T, H, dk];  j [B, T, H, dk];  eta [B, T, H]
 *   s0, s_final, state        [B, H, dk, dv] float32
 * dtype covers q, k, v, alpha, beta, beta_v, j, eta and o. The state is float32.
 *
 * Ownership: the caller owns every buffer, the workspace included. The library
 * allocates nothing on the device, keeps no state between calls and may be called
 * from several host threads at once.
 *
 * Semantics: calls are asynchronous and stream-ordered (stream is a hipStream_t;
 * NULL means the default stream); they return after enqueueing and never
 * synchronise the host. Results are bitwise deterministic for equal inputs and
 * launch parameters.
 *
 * Errors: 0 is success; negative codes below. Arguments are validated before
 * anything is enqueued: on an error nothing is launched and no output is touched.
 * Out-of-domain values (beta < 0, alpha outside (0, 1]) are not checked on the
 * device; they give NaN or Inf. Decay range of the chunked path: GDN and
 * DELTAPRODUCT (one decay per step) take any alpha in (0, 1]. The per-channel
 * decays (FG2, KDA, ASYM) are factored through reference points inside each
 * 16-step tile of a chunk, so the result stays in float32 range as long as no
 * channel decays by more than e^-87 over 8 consecutive steps (for instance,
 * alpha >= 1.9e-5 at every step); stronger decay over such a window can give NaN.
 * The recurrent entry point has no such limit.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3

enum gdn_variant {
  GDN_VARIANT_FG2 = 0,
  GDN_VARIANT_KDA = 1,
  GDN_VARIANT_GDN = 2,
  GDN_VARIANT_DELTAPRODUCT = 3,
  GDN_VARIANT_ASYM = 4
};

enum gdn_dtype { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };

enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_ARG = -1,         /* null pointer, bad shape, misaligned pointer     */
  GDN_ERR_UNSUPPORTED = -2, /* valid but not implemented (size, chunk, n_h)   */
  GDN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  GDN_ERR_HIP = -4          /* a HIP launch reported an error                 */
};

/* GDN2 stabilisers: gdn_asym_stabilize's mode, and gdn_args.stabilize. */
enum gdn_stabilize_mode { GDN_STABILIZE_CLIP_DECAY = 1, GDN_STABILIZE_PROJECT_J = 2 };

typedef struct gdn_args {
  int32_t variant;  /* enum gdn_variant */
  int32_t dtype;    /* enum gdn_dtype   */
  int64_t B, T, H;  /* batch, tokens (T >= 0), heads                          */
  int64_t dk, dv;   /* key and value head dims, each in {16, 32, 64, 128}     */
  int32_t chunk;    /* chunk length C in {16, 32, 64} (chunked entry points);
                       fp32 with dk = 128 runs 64 as 32 (same result up to
                       rounding, workspace sized for 32)                      */
  int32_t n_h;      /* Householder steps per token (DELTAPRODUCT, 1..8), else 1;
                       chunked entry points lay a token out as n_h steps, 4 for
                       n_h = 3 and 8 for n_h = 5..7 (the extra ones identity
                       steps) and need chunk / steps >= 8 output rows a chunk:
                       n_h 1..8 with chunk 64 (fp32 with dk = 128 runs 32-step
                       chunks: n_h 1..4), n_h 1..4 with chunk 32, n_h 1..2 with
                       chunk 16; GDN_ERR_UNSUPPORTED otherwise;
                       gdn_recurrent_step takes every n_h                     */
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;   /* unused by ASYM */
  const void* beta_v; /* FG2 only, optional (NULL: the value uses beta)       */
  const void* j;      /* ASYM only */
  const void* eta;    /* ASYM only */
  const float* s0;    /* initial state, NULL means zero                        */
  float* s_final;     /* final state, NULL means not written; may alias s0     */
  void* o;            /* outputs; ignored by gdn_final_state                   */
  int32_t stabilize;  /* ASYM only: 0, or a gdn_stabilize_mode applied to every
                         token's D or j inside the pass (as gdn_asym_stabilize
                         would, without its extra pass over the inputs or the
                         rounding of D' / j' to the input dtype)                */
} gdn_args;

/* Bytes of device workspace gdn_chunk_fwd / gdn_final_state need for *args
 * (0 for an invalid argument set). */
size_t gdn_workspace_bytes(const gdn_args* args);

/* Chunkwise-parallel forward pass: writes o for all T tokens and, when
 * s_final != NULL, the state after token T. The sequence is cut into chunks of
 * `chunk` steps (tokens, or Householder sub-steps for DELTAPRODUCT, whose chunk
 * must then be a multiple of n_h); inside a chunk the work is parallel (the
 * WY/UT form of the FG2-GDN reading notes, section 2.4), between chunks the state
 * is carried. T = 0 copies s0 (or zeros) to s_final. ws must hold
 * gdn_workspace_bytes(args) bytes and be 256-byte aligned. */
int gdn_chunk_fwd(const gdn_args* args, void* ws, size_t ws_bytes, void* stream);

/* Same pass computing the final state only (o is not read or written;
 * s_final must be non-NULL): the state S_T the recurrence above reaches after T
 * tokens (FG2-GDN reading notes, section 2.2 eq. (11), the state a chunked
 * prefill hands to decoding). */
int gdn_final_state(const gdn_args* args, void* ws, size_t ws_bytes, void* stream);

/* The two stages of gdn_chunk_fwd, for callers that schedule them separately
 * (gdn_chunk_fwd is exactly prepare followed by scan on one stream).
 * gdn_chunk_prepare runs the chunk-local work (decay cumsum, masked Grams, the
 * UT inverse T = (I + M)^{-1}, W = T B+, U~ = T Wv; FG2-GDN reading notes,
 * section 2.4) into ws; gdn_chunk_scan carries the state across chunks and writes
 * o and s_final. Both take the same args, ws and ws_bytes; with args->o == NULL
 * the pair computes the final state only (as gdn_final_state). ws must not be
 * modified between the two calls. */
int gdn_chunk_prepare(const gdn_args* args, void* ws, size_t ws_bytes, void* stream);
int gdn_chunk_scan(const gdn_args* args, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device buffer gdn_chunk_fwd_static keeps on each device. */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_fwd without a workspace, for callers that cannot allocate device
 * memory: code under stream capture, serving loops that must not allocate, and
 * harnesses that forbid hipMalloc. The call itself allocates nothing. The chunk
 * records live in a buffer of GDN_STATIC_SCRATCH_BYTES inside the library, one per
 * device, created when the library's code is loaded on that device and held until
 * the process ends; its device address is looked up once per device, on the first
 * call made with that device current. The sequence runs in blocks of as many
 * chunks as the buffer holds for all B*H sequences (one prepare and one scan
 * launch per block, each block starting from the state the previous one left), so
 * o and s_final are bitwise equal to gdn_chunk_fwd's for the same args.
 * Arguments, layouts and errors are those of gdn_chunk_fwd, plus
 * GDN_ERR_UNSUPPORTED when one chunk's records for all B*H sequences, plus
 * B*H*dk*dv*4 bytes for the carried state when s_final is NULL, exceed the buffer
 * (bf16, dk = dv = 128, chunk 64: 72 KiB of records per sequence, so B*H <= 910
 * with s_final given, B*H <= 481 without).
 * All calls on one device share its buffer, and the buffer keeps the last call's
 * contents: calls that may overlap on one device (several streams or host threads)
 * race and must be serialised by the caller. */
int gdn_chunk_fwd_static(const gdn_args* args, void* stream);

/* Token-sequential recurrence: advances state_inout ([B, H, dk, dv] float32,
 * updated in place) by args->T tokens, writing o for each (T = 1 is one decode
 * step): the step above applied token by token, exactly as the FG2-GDN reading
 * notes write it (section 2.2 eq. (11); section 2.1 eq. (6) for the delta rule it
 * extends; GDN2-stability page eq. (1) for ASYM; DeltaProduct summary, "Approach",
 * for the n_h sub-steps). args->s0, args->s_final and args->chunk are ignored. No
 * workspace. */
int gdn_recurrent_step(const gdn_args* args, float* state_inout, void* stream);

/* GDN2 stabilisers: token-wise transforms of the ASYM inputs that bound the spectral norm of each step's transition D (I - eta j k^T)
 * (GDN2-stability page: "The Spectral Norm" gives rho = ||I - eta j k^T||_2 in closed
 * form; "Simple Strategy" clips D; "Modifying Itself" moves j). args is an ASYM
 * argument set (variant GDN_VARIANT_ASYM, shapes as for the forward pass); only k,
 * j, alpha (= D) and eta are read, in args->dtype, and out has the same dtype.
 * The page's unit-norm j and k are not required: their norms are folded into eta.
 *   GDN_STABILIZE_CLIP_DECAY  out [B, T, H, dk] = min(D, 1/rho) per channel; then
 *                             ||D' (I - eta j k^T)||_2 <= 1.
 *   GDN_STABILIZE_PROJECT_J   out [B, T, H, dk] = j' = s k + lam (j - s k) with
 *                             s = j^T k / ||k||^2: eta j'^T k = eta j^T k (the erase
 *                             rate c is kept) and, with g = max_i D_i and
 *                             tau = (c - 1) g + 1/g, ||I - eta j' k^T||_2 <= 1/g
 *                             whenever tau >= |c|. lam = min(1, sqrt((tau^2 - c^2) /
 *                             (eta^2 ||k||^2 ||j - s k||^2))); lam = 1 when that
 *                             denominator is 0; lam = 0 when tau^2 <= c^2 (no j'
 *                             reaches the bound; only c < 0 gets there).
 * args->stabilize is ignored here; setting it on the forward entry points applies
 * the same transform inside the pass instead. out must be 16-byte aligned; it may be
 * args->alpha (mode 1) or args->j (mode 2) for an in-place update, and must not
 * overlap any other input. k = 0 rows give
 * NaN in mode 2. T = 0 does nothing. Errors: GDN_ERR_ARG for a variant other than
 * ASYM, a mode outside the enum, or a null or misaligned k, j, alpha, eta or out. */
int gdn_asym_stabilize(const gdn_args* args, int mode, void* out, void* stream);

/* Gradient outputs of gdn_recurrent_bwd, all float32, laid out like the matching
 * input (dalpha like alpha, dbeta like beta, ...; ds0 like s0). Pointers for inputs
 * the variant does not take must be NULL; the others must be non-NULL and 16-byte
 * aligned, except ds0, which may be NULL (not written). */
typedef struct gdn_grads {
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* dbeta;    /* FG2, KDA, GDN */
  float* dbeta_v;  /* FG2 with beta_v */
  float* dj;       /* ASYM */
  float* deta;     /* ASYM */
  float* ds0;
} gdn_grads;

/* Bytes of device workspace gdn_recurrent_bwd needs (0 for an invalid set). Per
 * token (or sub-step) and head: the float32 step operands (4 dk + 2 dv floats), the
 * records of the 16-step chunks ((80 dk + 32 dv + dk + 512) / 16 floats), the state
 * before every even chunk and the state gradient after every odd one (dk dv / 16
 * floats) and the row gradients (4 dk + dv floats); chunks are counted in pairs. 13.2
 * KiB per token and head at dk = dv = 128: 0.88 GB for 4,096 tokens x 16 heads. */
size_t gdn_bwd_workspace_bytes(const gdn_args* args);

/* Backward pass (reverse-mode gradients) of the token recurrence for every variant
 * (FG2, FG2+, KDA, GDN, ASYM, and DELTAPRODUCT through its Householder sub-steps,
 * DeltaProduct summary, "Approach"; dalpha is then the gate's gradient [B, T, H]).
 * The pages give the forward pass only; this is the derivative of the same recurrence
 * (FG2-GDN reading notes, section 2.2 eq. (11), section 2.3 eq. (13); GDN2-stability
 * page, eq. (1)), taken through the chunkwise WY / UT form of section 2.4 on 16-step
 * chunks. gdn_args.stabilize must be 0 (GDN_ERR_UNSUPPORTED otherwise), and
 * B * H * T * n_h may not exceed 2^33 (GDN_ERR_UNSUPPORTED). args as for the forward
 * pass (o, s_final and chunk are ignored; s0 NULL means zero); d_o [B, T, H, dv] in
 * args->dtype is dL/do; d_s_final [B, H, dk, dv] float32 is dL/dS_T (NULL: zero).
 * Gradients with respect to beta and beta_v are singular at 0 (their square roots
 * enter the step). ws must hold gdn_bwd_workspace_bytes(args) bytes, 256-byte
 * aligned. Decay factors span at most 8 steps of a chunk, so, as in the chunked
 * forward pass, results stay in float32 range while no channel decays by more than
 * e^-87 over 8 consecutive steps (alpha >= 1.9e-5 at every step suffices); beyond
 * that they can overflow. Every sum has a fixed order: results are deterministic. */
int gdn_recurrent_bwd(const gdn_args* args, const void* d_o, const float* d_s_final,
                      const gdn_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* gdn_status_str(int status);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
