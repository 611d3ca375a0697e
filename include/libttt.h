/*
 * libttt -- large-chunk test-time-training (TTT) layer forward for AMD MI355X (gfx950).
 *
 * The layer keeps fast weights W per (batch, head) and walks the sequence chunk by chunk.
 * For every chunk of `chunk` tokens it
 *   - applies the fast-weight net to the chunk's queries (the "apply" phase: LaCT explainer
 *     page, peacm.com, §2.1, eq. 2),
 *   - sums the gradient of the chunk's per-token eta-weighted inner loss over all of the
 *     chunk's keys and values (the "update" phase, same section, eqs. 4-5),
 *   - optionally orthogonalises that gradient with Muon's 5-step Newton-Schulz iteration
 *     (same page §2.2.1, eqs. 9-10), subtracts it from W,
 *   - and optionally rescales every row of W back to its pre-update L2 norm (§2.2.1, eq. 8).
 * Under the shifted block-causal order (same page §3.2, Fig. 3c) a chunk's queries see
 * the state left by the previous chunks; the image-set order (§3.1) updates first.
 *
 * Fast-weight nets (f maps a d-vector to a d-vector):
 *   SwiGLU   f(x) = W2 (silu(W1 x) * (W3 x)),  W1, W3: [hidden x dim], W2: [dim x hidden]
 *   GELU-MLP f(x) = W2 gelu(W1 x)             (exact erf GELU; the TTT-layer explainer
 *                                              page, aivaro.ru, §4: a 2-layer MLP)
 *   LINEAR   f(x) = W x,  W: [dim x dim]
 * Losses over a chunk S:  DOT  -sum_t eta_t <f(k_t), v_t>;   MSE  sum_t eta_t |f(k_t)-v_t|^2
 * (the Modular TTT abstract names both as interchangeable choices).
 *
 * Conventions for every entry point:
 *   - Pointers named q, k, v, out, eta, w0, src, dst are DEVICE pointers owned by the
 *     caller, 16-byte aligned, contiguous.  q, k, v, out: [batch][heads][tokens][dim] in the
 *     activation dtype (fp32 or bf16); eta: [batch][heads][tokens] fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on it and
 *     the call returns without waiting, except ttt_state_health and ttt_destroy_state.
 *   - All argument checks run on the host before anything is enqueued.  A failing call
 *     returns a status and enqueues nothing; ttt_last_error() then holds a message.
 *   - The library owns the state and all of its workspace, allocated in ttt_init_state;
 *     forward calls allocate nothing.  One state must not be used from two streams at once.
 *   - Nothing aborts, throws across the ABI or prints.
 */
#ifndef LIBTTT_H
#define LIBTTT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ttt_state ttt_state;

typedef enum {
  TTT_OK = 0,
  TTT_E_NULL = 1,        /* a required pointer is NULL                                  */
  TTT_E_SHAPE = 2,       /* a size is out of range or not a multiple it must be           */
  TTT_E_DTYPE = 3,       /* unknown activation dtype                                     */
  TTT_E_CONFIG = 4,      /* inconsistent or unknown enum / option value                  */
  TTT_E_UNSUPPORTED = 5, /* valid combination that this library does not implement       */
  TTT_E_ALLOC = 6,       /* device allocation failed                                     */
  TTT_E_HIP = 7,         /* a HIP runtime call failed (detail in ttt_last_error)         */
  TTT_E_NONFINITE = 8,   /* a NaN or Inf reached the fast-weight state                   */
  TTT_E_ALIGN = 9        /* a pointer is not 16-byte aligned                             */
} ttt_status;

typedef enum { TTT_FW_SWIGLU = 0, TTT_FW_MLP_GELU = 1, TTT_FW_LINEAR = 2 } ttt_fw;
typedef enum { TTT_LOSS_DOT = 0, TTT_LOSS_MSE = 1 } ttt_loss;
typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;
typedef enum { TTT_APPLY_THEN_UPDATE = 0, TTT_UPDATE_THEN_APPLY = 1 } ttt_order;
typedef enum { TTT_PATH_AUTO = 0, TTT_PATH_STAGED = 1, TTT_PATH_RESIDENT = 2 } ttt_path;

/*
 * Layer configuration.  Limits: batch, heads >= 1; batch*heads <= 65535; dim and hidden
 * multiples of 16 with 16 <= dim <= 1024 and 16 <= hidden <= 4096 (hidden is ignored for
 * LINEAR); 1 <= chunk <= 2^30; ns_steps in {0, 1..8}; with ns_steps > 0 and a two-matrix
 * or three-matrix net, dim <= hidden.
 *
 * Precision of the arithmetic.  All GEMMs run on bf16 MFMA with fp32 accumulation; all
 * elementwise math is fp32; the state is fp32.  An fp32 operand is fed to the MFMA as a
 * sum of `planes` bf16 numbers (1: plain bf16; 2: hi+lo, ~16 significant bits; 3: ~24
 * bits), and products of planes i, j are kept when i + j < max(planes of the two sides).
 * bf16 activations are exact in one plane.  Each field below is 1, 2 or 3:
 *   apply_planes   fast weights and hidden activations on the query (apply) path
 *   grad_planes    fast weights, back-propagated errors and fp32 activations on the
 *                  gradient path (the one that carries the state from chunk to chunk)
 *   ns_planes      every Newton-Schulz iteration after the first
 *   ns_lead_planes the first Newton-Schulz iteration
 * A value of 0 selects the default: 3 for fp32 activations, else 1 (apply), 2 (grad),
 * 2 (ns, ns_lead).
 *
 * Execution path.  STAGED runs each chunk as a sequence of stage kernels (any supported
 * configuration).  RESIDENT runs all chunks of a call in one kernel that keeps each
 * problem's fast weights on chip; it serves the small-chunk GELU-MLP layer only: fw
 * MLP_GELU, dim 64, hidden 256, chunk <= 64, ns_steps 0, no renorm, bf16 activations,
 * APPLY_THEN_UPDATE, apply_planes and grad_planes 1 (explicitly or by default they must
 * resolve to 1).  AUTO picks RESIDENT where it applies, else STAGED; asking for RESIDENT
 * elsewhere is TTT_E_UNSUPPORTED.  The two paths order their roundings differently;
 * both keep the bf16 accuracy bound of the single-plane setting.
 */
typedef struct {
  int32_t batch, heads, dim, hidden, chunk;
  int32_t fw;         /* ttt_fw    */
  int32_t loss;       /* ttt_loss  */
  int32_t act;        /* ttt_dtype of q, k, v and out */
  int32_t order;      /* ttt_order */
  int32_t ns_steps;   /* 0: W <- W - grad;  n > 0: W <- W - NS_n(grad)  (Muon uses 5) */
  int32_t row_renorm; /* 0 or 1 */
  int32_t apply_planes, grad_planes, ns_planes, ns_lead_planes;
  int32_t path;       /* ttt_path */
  /* Step.  Per chunk every matrix i of the state becomes (1 - weight_decay) W_i - lr[i] U_i
   * (U_i the summed gradient, or its Newton-Schulz orthogonalisation), then the optional
   * row renorm rescales each row to its norm before the step.  lr[i] is indexed in the
   * state's matrix order (SwiGLU W1, W3, W2; GELU W1, W2; linear W); 0 selects 1, and
   * entries past the net's matrices are ignored.  Each lr[i] must be finite and >= 0;
   * weight_decay finite and in [0, 1).  Zero-initialised fields give the plain step
   * W <- W - U.  (The Modular TTT abstract names the learning rate and the weight decay as
   * design dimensions of the inner learner; the LaCT explainer page, §4.2, suggests a
   * smaller Muon step when the loss oscillates.)                                         */
  float lr[3];
  float weight_decay;
} ttt_config;

/* Host-only check of a configuration (no HIP call).  TTT_OK or the first problem found. */
ttt_status ttt_validate_config(const ttt_config* cfg);

/* Number of fp32 values in the whole state (all matrices, all batch*heads problems), the
 * size of the buffers ttt_get_state / ttt_set_state take.  Host only.                  */
ttt_status ttt_state_numel(const ttt_config* cfg, int64_t* numel);

/*
 * Create a state: allocate the fast weights and every workspace buffer on the current
 * HIP device, and copy the initial weights.  w0 (device, fp32) holds the per-head initial
 * matrices, matrix by matrix, each [heads][rows][cols] row-major:
 *   SWIGLU: W1 [H][hidden][dim], W3 [H][hidden][dim], W2 [H][dim][hidden]
 *   GELU:   W1 [H][hidden][dim], W2 [H][dim][hidden];   LINEAR: W [H][dim][dim]
 * and every batch element starts from its head's matrices.  On success *out owns the
 * state; on failure *out is NULL and nothing stays allocated.
 */
ttt_status ttt_init_state(const ttt_config* cfg, const float* w0, void* stream,
                          ttt_state** out);

/* One chunk: q, k, v, out [batch][heads][chunk][dim]; eta [batch][heads][chunk].  out
 * receives the chunk's outputs, the state advances by one update.                   */
ttt_status ttt_chunk_forward(ttt_state* s, const void* q, const void* k, const void* v,
                             const float* eta, void* out, void* stream);

/* A whole sequence: tensors [batch][heads][seq_len][dim], eta [batch][heads][seq_len];
 * seq_len must be a multiple of the chunk size (0 is allowed and does nothing).  Equal,
 * bit for bit, to seq_len/chunk calls of ttt_chunk_forward on the consecutive chunks.  */
ttt_status ttt_sequence_forward(ttt_state* s, const void* q, const void* k, const void* v,
                                const float* eta, void* out, int64_t seq_len, void* stream);

/*
 * Backward of one chunk's apply step (the LaCT explainer page, §2.1, eq. 2; the query-view
 * rule of the train-view forward / backward / query-view split the Modular TTT abstract
 * describes).  With the state as it stands -- the state that chunk's queries were answered
 * with: before that chunk's ttt_chunk_forward under the shifted order, after it under the
 * update-then-apply order, or any state restored with ttt_set_state -- computes for every
 * (batch, head) problem
 *   dq = d/dQ  sum_t <dout_t, f_W(q_t)>      [B][H][chunk][dim], activation dtype
 *   dw = d/dW  sum_t <dout_t, f_W(q_t)>      fp32, the ttt_get_state layout (every matrix)
 * q, dout: [B][H][chunk][dim] device tensors in the activation dtype.  All four pointers
 * are device pointers, caller-owned, 16-byte aligned.  The state is not changed.  Only the
 * backward through the apply is computed, not through the fast-weight updates (those
 * gradients with respect to k, v, eta and W0 are not provided).  States served by the
 * resident path return TTT_E_UNSUPPORTED (create them with path STAGED).  Enqueued on
 * stream with no host synchronisation; status codes as for the forward calls.
 */
ttt_status ttt_apply_backward(ttt_state* s, const void* q, const void* dout, void* dq,
                              float* dw, void* stream);

/* Copy the fp32 state out / in.  Layout: matrix by matrix, each [batch][heads][rows][cols]
 * with the shapes listed under ttt_init_state.  dst/src: device, ttt_state_numel values. */
ttt_status ttt_get_state(const ttt_state* s, float* dst, void* stream);
ttt_status ttt_set_state(ttt_state* s, const float* src, void* stream);

/* Wait for the state's work and report TTT_E_NONFINITE if any update so far produced a
 * NaN or Inf row norm in the fast weights (the flag is sticky until ttt_set_state).    */
ttt_status ttt_state_health(ttt_state* s);

/* Wait for the state's work and free it.  NULL is accepted.                            */
ttt_status ttt_destroy_state(ttt_state* s);

/*
 * Measurement hooks.  Between ttt_profile_begin and ttt_profile_end, every launch of the
 * chosen stage kernel on the state's stream is bracketed by a pair of HIP events (at most
 * max_launches launches are timed; later ones run untimed).  ttt_profile_end waits for the
 * stream and returns the number of timed launches and the sum of their durations in ms.
 * Stages: 0 front (query rows), 1 front (key rows), 2 output GEMM, 3 token contraction,
 * 4 Newton-Schulz Gram, 5 Newton-Schulz polynomial, 6 Newton-Schulz update,
 * 7 update + renorm, 8 fp32 plane split, 9 MSE error / dH GEMMs,
 * 10 device-resident chunk loop (one launch per call).
 * The hooks create and destroy HIP events but allocate no device memory.
 */
typedef enum {
  TTT_STAGE_FRONT_Q = 0, TTT_STAGE_FRONT_K = 1, TTT_STAGE_OUT = 2, TTT_STAGE_CONTRACT = 3,
  TTT_STAGE_NS_GRAM = 4, TTT_STAGE_NS_POLY = 5, TTT_STAGE_NS_UPDATE = 6, TTT_STAGE_RENORM = 7,
  TTT_STAGE_SPLIT = 8, TTT_STAGE_MSE = 9, TTT_STAGE_RESIDENT = 10, TTT_STAGE_DQ = 11,
  TTT_STAGE_COUNT = 12
} ttt_stage;
ttt_status ttt_profile_begin(ttt_state* s, int32_t stage, int32_t max_launches);
ttt_status ttt_profile_end(ttt_state* s, int64_t* launches, double* total_ms);

/* Static description of a status, and the calling thread's last error message.         */
const char* ttt_status_str(ttt_status st);
const char* ttt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBTTT_H */
