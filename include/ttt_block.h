/*
 * libttt block API: the LaCT block around the large-chunk TTT layer, on gfx950.
 *
 * [LaCT] "LaCT技术解析：大块测试时训练提升长序列建模效率" (peacm.com), §2.1 and Fig. 2: a
 * block stacks window attention (the dependencies inside a chunk), the large-chunk TTT
 * layer (the long-range ones) and a feed-forward layer (channel mixing).  §3.1: for an
 * image set the attention window covers one whole image; §3.2: for text a sliding window
 * is used beside the TTT layer.
 *
 * Where the page leaves the block's details open this library takes the plainest reading:
 *   h = x + Attn(n(x));  h = h + TTT(n(h));  y = h + FFN(n(h))
 * n the RMS normalisation over the model width without a learned scale (eps 1e-6);
 * Attn: heads of dimension 128 over the model width, one projection to q, k, v and one
 * back, scores scaled by 1/sqrt(128) and softmax over the window; TTT: one projection to
 * the TTT heads' q, k, v (q and k normalised to unit length per head and token), a
 * per-head step size eta = 0.01 sigmoid(n(h) . w_eta[head]), the TTT layer of libttt.h
 * per head, one projection back; FFN: W_down gelu(W_up x) with the exact erf GELU.  No
 * biases.  Activations are bf16 between the sub-layers, accumulation is fp32.
 *
 * All tensors are device memory, caller-owned, 16-byte aligned.  Every call is enqueued
 * on `stream` (a hipStream_t; NULL is the null stream) without host synchronisation.
 * Status codes and ttt_last_error as in libttt.h.
 */
#ifndef TTT_BLOCK_H
#define TTT_BLOCK_H

#include "libttt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Attention window kinds ([LaCT] §2.1): SLIDING lets token t attend to tokens
 * t - window + 1 .. t (text); BLOCK splits the sequence into blocks of `window` tokens
 * (one image each) and lets every token attend to every token of its own block.         */
typedef enum { TTT_WINDOW_SLIDING = 0, TTT_WINDOW_BLOCK = 1 } ttt_window_mode;

#define TTT_ATTN_HEAD_DIM 128

/*
 * Window attention of one layer ([LaCT] §2.1 window attention).  For batch element b,
 * head h (of heads, each TTT_ATTN_HEAD_DIM wide) and token t:
 *   out[b, t, h] = sum_j softmax_j(q[b,t,h] . k[b,j,h] / sqrt(128)) v[b,j,h]
 * over the tokens j the window lets t see.  Element e of head h of token t of batch b is
 * at  base + ((b * seq_len + t) * ld + h * 128 + e)  for q, k and v (bf16), and at
 * out + (b * seq_len + t) * ld_out + h * 128 + e  for the output (bf16), so q, k and v
 * may be thirds of one projection's output rows; out may not overlap them (TTT_E_CONFIG).
 * Limits: batch, heads >= 1; window >= 1;
 * 0 <= seq_len < 2^31; ld, ld_out >= heads * 128 and multiples of 8; ld < 2^24.  The
 * scores and their softmax are fp32; the probabilities are rounded to bf16 for the
 * product with v, and the normaliser sums the rounded values, so each output is a convex
 * combination of the values in its window.
 */
ttt_status ttt_window_attention(const void* q, const void* k, const void* v, int64_t ld,
                                void* out, int64_t ld_out, int32_t batch, int32_t heads,
                                int64_t seq_len, int32_t window, int32_t window_mode,
                                void* stream);

/* Epilogues of ttt_linear. */
typedef enum { TTT_LINEAR_PLAIN = 0, TTT_LINEAR_RESIDUAL = 1, TTT_LINEAR_GELU = 2 } ttt_linear_epi;

/*
 * One projection of the block (bf16, fp32 accumulation): for every row r < rows and
 * output column n < out_features,
 *   acc = sum_i x[r][i] w[n][i]
 *   y[r][n] = bf16(acc)              PLAIN
 *           = bf16(resid[r][n] + acc) RESIDUAL (resid bf16 with y's layout; may equal y)
 *           = bf16(gelu(acc))        GELU (exact erf form)
 * x [rows][in_features], w [out_features][in_features], y [rows][out_features], all
 * row-major bf16.  Limits: rows >= 0; in_features and out_features multiples of 8 in
 * [8, 65536].  x and w must not overlap y.
 */
ttt_status ttt_linear(const void* x, const void* w, const void* resid, void* y, int64_t rows,
                      int32_t in_features, int32_t out_features, int32_t epilogue,
                      void* stream);

typedef struct {
  int32_t batch;        /* sequences per call, >= 1; equal to ttt.batch                  */
  int32_t dim;          /* model width D: a multiple of 128, at most 8192; ttt.heads *
                           ttt.dim must equal it                                          */
  int32_t window;       /* attention window in tokens, >= 1                               */
  int32_t window_mode;  /* ttt_window_mode                                                */
  int32_t ffn_hidden;   /* MLP hidden width: a multiple of 8, <= 65536 (0 selects 4 D)     */
  int32_t reserved;     /* 0                                                              */
  int64_t max_seq_len;  /* longest seq_len a forward call may pass (sizes the workspace)  */
  ttt_config ttt;       /* the TTT sub-layer; bf16 activations, any other option of
                           libttt.h (heads at most 16)                                    */
} ttt_block_config;

/* The block's projection weights, bf16, row-major [out features][in features], device
 * memory that the caller keeps alive and unchanged while the block is used. */
typedef struct {
  const void* attn_qkv;  /* [3 D][D]: rows 0..D-1 give q, D..2D-1 k, 2D..3D-1 v          */
  const void* attn_out;  /* [D][D]                                                       */
  const void* ttt_qkv;   /* [3 D][D]: the TTT heads' q, k, v (head h: rows h dim .. )      */
  const void* ttt_eta;   /* [ttt.heads][D]                                               */
  const void* ttt_out;   /* [D][D]                                                       */
  const void* ffn_up;    /* [F][D]                                                       */
  const void* ffn_down;  /* [D][F]                                                       */
} ttt_block_weights;

typedef struct ttt_block ttt_block;

/*
 * Create a block on the current HIP device: check the configuration, create the TTT
 * sub-layer's state from w0 (the layout ttt_init_state takes), keep a copy of that initial
 * state, and allocate the workspace for max_seq_len tokens per sequence (about
 * 2 (10 D + F) bytes per token, plus the TTT state's own).  The weights are referenced,
 * not copied.  On failure *out is NULL and nothing stays allocated.
 */
ttt_status ttt_block_init(const ttt_block_config* cfg, const ttt_block_weights* w,
                          const float* w0, void* stream, ttt_block** out);

/*
 * One block over `batch` whole sequences: x, y [batch][seq_len][D] bf16 (y may equal x).
 * seq_len: 0 <= seq_len <= max_seq_len, a multiple of ttt.chunk.  Every call starts the
 * TTT sub-layer from the initial state given to ttt_block_init (each call is a sequence
 * of its own); afterwards the sub-layer's state (ttt_block_ttt_state) holds the fast
 * weights at the sequence's end.
 */
ttt_status ttt_block_forward(ttt_block* b, const void* x, void* y, int64_t seq_len,
                             void* stream);

/* The TTT sub-layer's state (owned by the block), for ttt_get_state and the other calls
 * of libttt.h that read it.  NULL for NULL.                                              */
ttt_state* ttt_block_ttt_state(ttt_block* b);

/* Wait for the block's work and free it.  NULL is accepted.                             */
ttt_status ttt_block_destroy(ttt_block* b);

#ifdef __cplusplus
}
#endif

#endif /* TTT_BLOCK_H */
