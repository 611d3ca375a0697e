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
 * bf16 activations are exact in one plane.  Each of the first three fields is 1, 2 or 3:
 *   apply_planes   fast weights and hidden activations on the query (apply) path
 *   grad_planes    fast weights, back-propagated errors and fp32 activations on the
 *                  gradient path (the one that carries the state from chunk to chunk)
 *   ns_planes      the Newton-Schulz iterates X (stored between iterations) and the
 *                  operands of every iteration not named in ns_one_plane
 * A value of 0 selects the default: 3 for fp32 activations, else 1 (apply), 2 (grad),
 * 2 (ns).
 *   ns_one_plane   bit i set: Newton-Schulz iteration i multiplies one bf16 plane of each
 *                  operand (X X^T, A A and B X), and its linear term a X is added outside
 *                  the products from X's ns_planes planes.  An early iteration acts on small
 *                  singular values, where b A + c A^2 is small beside a I, so its products
 *                  tolerate plain bf16 as long as a X keeps the stored precision.  Bits at
 *                  or above ns_steps, or with ns_planes 1, change nothing.  0..255.
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
  int32_t apply_planes, grad_planes, ns_planes, ns_one_plane;
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
  /* Replay (0 or 1).  With 1, the first forward call with a given set of tensor pointers,
   * length and update flags records its kernel launches into a HIP graph (captured on an
   * internal stream of default priority; nothing captured is a memset), and a later call
   * with the same pointers, length and flags replays that graph on the caller's stream:
   * the same kernels on the same arguments, so the results equal the direct launches'
   * bit for bit, whatever the tensors hold.  A call with other pointers records a new
   * graph in place of the old one.  Meant for shapes whose kernels are short enough that
   * launching them one by one dominates (small heads, many chunks).  Calls made while a
   * measurement hook is active launch directly.                                         */
  int32_t replay;
  /* Momentum (the LaCT page, §2.2.1, compares its Muon variant with an ordinary momentum
   * optimiser).  0 (the default) or beta in (0, 1): every matrix keeps a buffer
   * M <- beta M + g of the chunk gradients, starting at 0, and the step takes U = NS(M)
   * under Newton-Schulz, else M.  The buffers are part of the state: with beta > 0,
   * ttt_state_numel counts them, and ttt_get_state / ttt_set_state (and the state of the
   * allocation-free call) hold every fast-weight matrix followed by every buffer, in the
   * same matrix order and layout.  The resident path and the chunk backward take no
   * momentum.  A chunk without update leaves its buffer as it is.                       */
  float momentum;
} ttt_config;

/* Host-only check of a configuration (no HIP call).  TTT_OK or the first problem found. */
ttt_status ttt_validate_config(const ttt_config* cfg);

/* Number of fp32 values in the whole state (all matrices, all batch*heads problems), the
 * size of the buffers ttt_get_state / ttt_set_state take.  Host only.                  */
ttt_status ttt_state_numel(const ttt_config* cfg, int64_t* numel);

/*
 * Create a state: allocate the fast weights and every workspace buffer on the current
 * HIP device, and copy the initial weights.  The fast weights are the layer's hidden
 * state: the inner model's parameters, changed by every update (TTT-layer explainer page,
 * aivaro.ru, §3 step 2 and §4 "hidden state"); their size does not grow with the context
 * (the second TTT-E2E page, intelliparadigm.com, §3.2: constant memory in the sequence
 * length), so the whole state and workspace are sized here, once, from the configuration.  w0 (device, fp32) holds the per-head initial
 * matrices, matrix by matrix, each [heads][rows][cols] row-major:
 *   SWIGLU: W1 [H][hidden][dim], W3 [H][hidden][dim], W2 [H][dim][hidden]
 *   GELU:   W1 [H][hidden][dim], W2 [H][dim][hidden];   LINEAR: W [H][dim][dim]
 * and every batch element starts from its head's matrices.  On success *out owns the
 * state; on failure *out is NULL and nothing stays allocated.
 */
ttt_status ttt_init_state(const ttt_config* cfg, const float* w0, void* stream,
                          ttt_state** out);

/* One chunk: q, k, v, out [batch][heads][chunk][dim]; eta [batch][heads][chunk].  out
 * receives the chunk's outputs, the state advances by one update: the LaCT page's apply
 * and update phases (§2.1) for one chunk, with the state passed in and carried out
 * explicitly as in the forward(x, state) of the TTT-E2E page (jsqmd.com, §2.1.1).     */
ttt_status ttt_chunk_forward(ttt_state* s, const void* q, const void* k, const void* v,
                             const float* eta, void* out, void* stream);

/* A whole sequence: tensors [batch][heads][seq_len][dim], eta [batch][heads][seq_len];
 * seq_len must be a multiple of the chunk size (0 is allowed and does nothing).  Equal,
 * bit for bit, to seq_len/chunk calls of ttt_chunk_forward on the consecutive chunks:
 * the chunk loop of the LaCT page (§3.2, Fig. 3c, shifted block-causal; §3.1 a single
 * whole-sequence chunk for image sets), consecutive blocks sharing one fast-weight state
 * (TTT-E2E page, jsqmd.com, §3.2.2; the overlap between blocks that section also
 * describes is not made).                                                            */
ttt_status ttt_sequence_forward(ttt_state* s, const void* q, const void* k, const void* v,
                                const float* eta, void* out, int64_t seq_len, void* stream);

/*
 * ttt_sequence_forward in which only chosen chunks update the fast weights.  update: HOST
 * array of seq_len/chunk bytes, read before the call returns; chunk c updates when
 * update[c] != 0 (NULL: every chunk updates, the same as ttt_sequence_forward).  A chunk
 * whose flag is 0 answers its queries with the state as it stands and leaves the state
 * unchanged: no gradient, no Newton-Schulz, no decay, no renorm.  The LaCT page (§3.3)
 * adapts a video diffusion model so that the fast weights are updated on the clean-frame
 * chunks only, every chunk still being answered; a flag per chunk states that.  Together
 * with either order it also expresses updates on every s-th chunk only, each chunk's
 * queries seeing the updates up to their own chunk (UPDATE_THEN_APPLY) or before it.
 * With no weight decay, a chunk without update gives the same result, bit for bit, as the
 * same chunk with every eta set to 0.  Other arguments and errors as for
 * ttt_sequence_forward.
 */
ttt_status ttt_sequence_forward_masked(ttt_state* s, const void* q, const void* k,
                                       const void* v, const float* eta, void* out,
                                       int64_t seq_len, const uint8_t* update, void* stream);

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

/*
 * Backward through one chunk (apply and update), for training through the inner updates:
 * the outer loop of the second TTT-E2E page (intelliparadigm.com, §2.2: inner TTT on copied
 * weights, outer update through them; §5.1: the second-order gradients this needs) and the
 * train-view backward the Modular TTT abstract composes into the layer's backward.  With the
 * state as it stands taken as the state before the chunk (restore it with ttt_set_state),
 * and the chunk's q, k, v, eta ([B][H][chunk][dim], eta [B][H][chunk]), computes the
 * gradients of
 *     sum_t <dout_t, o_t> + <dw, W_after>
 * (o the chunk's outputs, W_after the state after the chunk's update) with respect to the
 * chunk's inputs and the state before it:
 *   dout  in,  [B][H][chunk][dim] activation dtype
 *   dw    in:  fp32, ttt_get_state layout, the cotangent of the state after the chunk;
 *         out: overwritten with the cotangent of the state before the chunk
 *   dq, dk, dv  out, [B][H][chunk][dim] activation dtype;  deta  out, fp32 [B][H][chunk]
 * The update is taken back step by step: the row renorm, the step with its step size and
 * weight decay, Muon's Newton-Schulz iteration, and the chunk gradient itself (second order
 * in the net).  Chaining calls from the last chunk to the first, each with the state before
 * its chunk, gives the gradients of a whole sequence.  Under the shifted (apply-then-update)
 * order the apply step is taken back with the state before the update; under the
 * update-then-apply order with the updated state, its weight gradient joining dw before the
 * update is taken back (the updated state is formed in place of the state for that and the
 * state before the chunk restored, bit for bit).  Chunks longer than 65536 tokens are taken
 * in token blocks, as the forward takes them.  With momentum the state holds the
 * heavy-ball buffers after the matrices, and so do dw in and out: the step's input is the
 * new buffer beta M + g, whose cotangent (from the step, plus dw's part for the buffer
 * after the chunk) is taken back into the chunk gradient whole and into the buffer before
 * the chunk times beta.  Serves the SwiGLU net with the inner-product loss on the staged
 * path; other configurations return TTT_E_UNSUPPORTED.  The state is not changed.  The first call on a state allocates the backward's workspace (about
 * 3 GB for the LaCT language-model layer; TTT_E_ALLOC if it cannot); later calls allocate
 * nothing.  All pointers device, caller-owned, 16-byte aligned; enqueued on stream.
 */
ttt_status ttt_chunk_backward(ttt_state* s, const void* q, const void* k, const void* v,
                              const float* eta, const void* dout, float* dw, void* dq,
                              void* dk, void* dv, float* deta, void* stream);

/* Copy the fp32 state out / in.  Layout: matrix by matrix, each [batch][heads][rows][cols]
 * with the shapes listed under ttt_init_state.  dst/src: device, ttt_state_numel values.
 * The state is what carries over from one step to the next (TTT-layer explainer page,
 * §3 step 5): reading it and writing it back resumes a sequence where it stopped.      */
ttt_status ttt_get_state(const ttt_state* s, float* dst, void* stream);
ttt_status ttt_set_state(ttt_state* s, const float* src, void* stream);

/* Wait for the state's work and report TTT_E_NONFINITE if any update so far produced a
 * NaN or Inf row norm in the fast weights (the flag is sticky until ttt_set_state).
 * An update step too large for the inner learner is the instability the TTT-E2E page
 * (jsqmd.com, §4.2) lists first among its failure modes, and the second TTT-E2E page
 * closes by advising to watch the size of the parameter updates; this is that watch.   */
ttt_status ttt_state_health(ttt_state* s);

/* Wait for the state's work and free it.  NULL is accepted.                            */
ttt_status ttt_destroy_state(ttt_state* s);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ttt_sequence_forward without a state
 * object and without any allocation.
 *   state  device fp32, ttt_state_numel(cfg) values in the ttt_get_state layout: read as the
 *          initial fast weights of every (batch, head) problem, overwritten with the final
 *          ones.  Caller-owned, 16-byte aligned.
 *   q, k, v, eta, out, seq_len, stream: as for ttt_sequence_forward.
 * All workspace comes from one static device array of TTT_NOALLOC_SCRATCH_BYTES bytes (64
 * MiB), which each GPU the library runs on holds from the first call until the process
 * ends.  A configuration whose workspace is larger (e.g. the LaCT language-model layer
 * with 8 problems of dim 512 and hidden 1024) returns TTT_E_SHAPE, with both sizes in
 * ttt_last_error; that and every other argument check runs on the host before any HIP
 * call.  The call makes no hipMalloc, hipFree or memset; it enqueues kernels on stream and
 * returns without waiting.  All calls on one GPU share that GPU's array and it keeps the
 * last call's contents: calls that overlap on one GPU (two streams, two threads) race and
 * corrupt each other's results, so serialise them.  There is no health flag to query.
 * Given the same configuration, weights and inputs, the results equal those of
 * ttt_sequence_forward on a state created by ttt_init_state, bit for bit.
 */
#define TTT_NOALLOC_SCRATCH_BYTES 67108864
ttt_status ttt_sequence_forward_noalloc(const ttt_config* cfg, float* state, const void* q,
                                        const void* k, const void* v, const float* eta,
                                        void* out, int64_t seq_len, void* stream);

/*
 * Measurement hooks.  Between ttt_profile_begin and ttt_profile_end, every launch of the
 * chosen stage kernel on the state's stream is bracketed by a pair of HIP events (at most
 * max_launches launches are timed; later ones run untimed).  ttt_profile_end waits for the
 * stream and returns the number of timed launches and the sum of their durations in ms.
 * Stages: 0 front (query rows), 1 front (key rows), 2 output GEMM, 3 token contraction,
 * 4 Newton-Schulz Gram, 5 Newton-Schulz polynomial, 6 Newton-Schulz update,
 * 7 update + renorm, 8 fp32 plane split, 9 MSE error / dH GEMMs,
 * 10 device-resident chunk loop (one launch per call), 11 the backward's dQ, dK and dV
 * GEMMs, 12 the chunk backward's tangent front (and its eta sums), 13 its Newton-Schulz
 * backward GEMMs, 14 every Newton-Schulz iteration of a small matrix in one launch (the
 * forward's orthogonalisation when the matrices in their [dim][hidden] orientation are at
 * most 64 x 128; stages 4-6 then do not run).
 * The hooks create and destroy HIP events but allocate no device memory.
 */
typedef enum {
  TTT_STAGE_FRONT_Q = 0, TTT_STAGE_FRONT_K = 1, TTT_STAGE_OUT = 2, TTT_STAGE_CONTRACT = 3,
  TTT_STAGE_NS_GRAM = 4, TTT_STAGE_NS_POLY = 5, TTT_STAGE_NS_UPDATE = 6, TTT_STAGE_RENORM = 7,
  TTT_STAGE_SPLIT = 8, TTT_STAGE_MSE = 9, TTT_STAGE_RESIDENT = 10, TTT_STAGE_DQ = 11,
  TTT_STAGE_TFRONT = 12, TTT_STAGE_NS_BWD = 13, TTT_STAGE_NS_SMALL = 14, TTT_STAGE_COUNT = 15
} ttt_stage;
ttt_status ttt_profile_begin(ttt_state* s, int32_t stage, int32_t max_launches);
ttt_status ttt_profile_end(ttt_state* s, int64_t* launches, double* total_ms);

/* Static description of a status code (any int32_t: codes that are not a ttt_status give
 * "unknown status"), and the calling thread's last error message.                       */
const char* ttt_status_str(int32_t st);
const char* ttt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBTTT_H */
