// Host side of the block API (include/ttt_block.h): argument checks, the block's workspace,
// and the order of its launches.  The TTT sub-layer runs through the public calls of
// libttt.h on a state the block owns.
#include "ttt_block.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>

#include "ttt_block_internal.h"

using namespace ttt;

namespace {

ttt_status failf(ttt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return report(st, buf);
}

#define BLK_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return failf(TTT_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),    \
                   __FILE__, __LINE__);                                                 \
  } while (0)

#define BLK_TRY(expr)                  \
  do {                                 \
    ttt_status s_ = (expr);            \
    if (s_ != TTT_OK) return s_;       \
  } while (0)

ttt_status need(const void* p, const char* name) {
  if (!p) return failf(TTT_E_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16)
    return failf(TTT_E_ALIGN, "%s is not 16-byte aligned", name);
  return TTT_OK;
}

constexpr int64_t INT31 = (int64_t)1 << 31;

ttt_status check_attention(int64_t ld, int64_t ld_out, int32_t batch, int32_t heads,
                           int64_t T, int32_t window, int32_t mode) {
  if (batch < 1 || heads < 1) return failf(TTT_E_SHAPE, "batch %d, heads %d", batch, heads);
  if (window < 1) return failf(TTT_E_SHAPE, "window %d < 1", window);
  if (mode != TTT_WINDOW_SLIDING && mode != TTT_WINDOW_BLOCK)
    return failf(TTT_E_CONFIG, "unknown window mode %d", mode);
  if (T < 0 || T >= INT31) return failf(TTT_E_SHAPE, "seq_len %lld out of range", (long long)T);
  if (ld < (int64_t)heads * ATT_D || ld % 8 || ld >= ((int64_t)1 << 24))
    return failf(TTT_E_SHAPE, "ld %lld: at least heads * 128, a multiple of 8, below 2^24",
                 (long long)ld);
  if (ld_out < (int64_t)heads * ATT_D || ld_out % 8)
    return failf(TTT_E_SHAPE, "ld_out %lld: at least heads * 128 and a multiple of 8",
                 (long long)ld_out);
  const int64_t total = (T + ATT_Q - 1) / ATT_Q * heads * batch;
  if (total >= INT31) return failf(TTT_E_SHAPE, "batch * heads * seq_len too large");
  return TTT_OK;
}

AttnArgs attention_args(const void* q, const void* k, const void* v, int64_t ld, void* out,
                        int64_t ld_out, int32_t batch, int32_t heads, int64_t T,
                        int32_t window, int32_t mode) {
  AttnArgs a;
  a.q = static_cast<const u16*>(q);
  a.k = static_cast<const u16*>(k);
  a.v = static_cast<const u16*>(v);
  a.out = static_cast<u16*>(out);
  a.ld = ld;
  a.ldo = ld_out;
  a.T = (int32_t)T;
  a.heads = heads;
  a.window = window;
  a.mode = mode;
  a.qblocks = (int32_t)((T + ATT_Q - 1) / ATT_Q);
  a.total = a.qblocks * heads * batch;
  a.scale2 = (float)(1.4426950408889634 / std::sqrt((double)ATT_D));
  return a;
}

ttt_status check_linear(int64_t rows, int32_t K, int32_t N, int32_t epi) {
  if (rows < 0) return failf(TTT_E_SHAPE, "rows %lld < 0", (long long)rows);
  if (K < 8 || K > 65536 || K % 8)
    return failf(TTT_E_SHAPE, "in_features %d: a multiple of 8 in [8, 65536]", K);
  if (N < 8 || N > 65536 || N % 8)
    return failf(TTT_E_SHAPE, "out_features %d: a multiple of 8 in [8, 65536]", N);
  if (epi < TTT_LINEAR_PLAIN || epi > TTT_LINEAR_GELU)
    return failf(TTT_E_CONFIG, "unknown epilogue %d", epi);
  if ((rows + 127) / 128 * ((N + 127) / 128) >= INT31)
    return failf(TTT_E_SHAPE, "rows * out_features too large");
  return TTT_OK;
}

LinearArgs linear_args(const void* x, const void* w, const void* resid, void* y, int64_t rows,
                       int32_t K, int32_t N) {
  LinearArgs a;
  a.x = static_cast<const u16*>(x);
  a.w = static_cast<const u16*>(w);
  a.resid = static_cast<const u16*>(resid);
  a.y = static_cast<u16*>(y);
  a.rows = rows;
  a.K = K;
  a.N = N;
  // 256 x 256 tiles where they give at least two workgroups per CU (one fits a CU) and the
  // K loop is long; shorter ones gain nothing from them (measured at K = 1024)
  const int64_t wide = ((rows + 255) / 256) * ((N + 255) / 256);
  a.tile = wide >= LINEAR_WIDE_MIN && K >= LINEAR_WIDE_K ? 256 : 128;
  a.tiles_n = (N + a.tile - 1) / a.tile;
  a.tiles_m = (int32_t)((rows + a.tile - 1) / a.tile);
  a.tiles = (int64_t)a.tiles_m * a.tiles_n;
  // row tiles per group: 8 measured best or within a few percent of it for every projection
  // of the block at width 1024 (in 1024 or 4096 features, out 1024 to 4096)
  a.group_m = std::min<int32_t>(a.tiles_m, 8);
  return a;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

struct ttt_block {
  ttt_block_config cfg;
  ttt_block_weights w;
  int F = 0;
  ttt_state* ttt = nullptr;
  float* s0 = nullptr;    // the TTT sub-layer's initial state
  char* arena = nullptr;  // the workspace
  u16 *nrm = nullptr, *qkv = nullptr, *att = nullptr, *hid = nullptr, *ffn = nullptr;
  u16 *tq = nullptr, *tk = nullptr, *tv = nullptr, *to = nullptr;
  float* eta = nullptr;
};

namespace {

ttt_status check_block_config(const ttt_block_config* c, int* F) {
  if (!c) return failf(TTT_E_NULL, "config is NULL");
  if (c->batch < 1) return failf(TTT_E_SHAPE, "batch %d < 1", c->batch);
  if (c->dim < ATT_D || c->dim > 8192 || c->dim % ATT_D)
    return failf(TTT_E_SHAPE, "dim %d: a multiple of 128 in [128, 8192]", c->dim);
  if (c->window < 1) return failf(TTT_E_SHAPE, "window %d < 1", c->window);
  if (c->window_mode != TTT_WINDOW_SLIDING && c->window_mode != TTT_WINDOW_BLOCK)
    return failf(TTT_E_CONFIG, "unknown window mode %d", c->window_mode);
  const int f = c->ffn_hidden ? c->ffn_hidden : 4 * c->dim;
  if (f < 8 || f > 65536 || f % 8)
    return failf(TTT_E_SHAPE, "ffn_hidden %d: a multiple of 8 in [8, 65536]", f);
  if (c->reserved) return failf(TTT_E_CONFIG, "reserved field must be 0");
  if (c->max_seq_len < 0 || c->max_seq_len >= INT31)
    return failf(TTT_E_SHAPE, "max_seq_len %lld out of range", (long long)c->max_seq_len);
  const ttt_config& t = c->ttt;
  BLK_TRY(ttt_validate_config(&t));
  if (t.batch != c->batch)
    return failf(TTT_E_SHAPE, "ttt.batch %d differs from batch %d", t.batch, c->batch);
  if ((int64_t)t.heads * t.dim != c->dim)
    return failf(TTT_E_SHAPE, "ttt.heads * ttt.dim = %lld differs from dim %d",
                 (long long)t.heads * t.dim, c->dim);
  if (t.heads > BLK_MAX_TTT_HEADS)
    return failf(TTT_E_UNSUPPORTED, "ttt.heads %d above %d", t.heads, BLK_MAX_TTT_HEADS);
  if (t.act != TTT_BF16) return failf(TTT_E_DTYPE, "the block's TTT layer takes bf16");
  const int64_t rows = (int64_t)c->batch * c->max_seq_len;
  BLK_TRY(check_linear(rows, c->dim, 3 * c->dim, TTT_LINEAR_PLAIN));
  BLK_TRY(check_linear(rows, c->dim, f, TTT_LINEAR_GELU));
  BLK_TRY(check_linear(rows, f, c->dim, TTT_LINEAR_RESIDUAL));
  BLK_TRY(check_attention(3 * c->dim, c->dim, c->batch, c->dim / ATT_D, c->max_seq_len,
                          c->window, c->window_mode));
  *F = f;
  return TTT_OK;
}

void release(ttt_block* b) {
  if (!b) return;
  if (b->ttt) ttt_destroy_state(b->ttt);
  if (b->s0) (void)hipFree(b->s0);
  if (b->arena) (void)hipFree(b->arena);
  delete b;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

ttt_status ttt_window_attention(const void* q, const void* k, const void* v, int64_t ld,
                                void* out, int64_t ld_out, int32_t batch, int32_t heads,
                                int64_t seq_len, int32_t window, int32_t window_mode,
                                void* stream) {
  BLK_TRY(check_attention(ld, ld_out, batch, heads, seq_len, window, window_mode));
  if (seq_len == 0) return TTT_OK;
  BLK_TRY(need(q, "q"));
  BLK_TRY(need(k, "k"));
  BLK_TRY(need(v, "v"));
  BLK_TRY(need(out, "out"));
  // every workgroup reads keys and values of other workgroups' queries: the output may not
  // share memory with the inputs
  const size_t rows = (size_t)batch * (size_t)seq_len;
  const size_t in_bytes = ((rows - 1) * (size_t)ld + (size_t)heads * ATT_D) * 2;
  const size_t out_bytes = ((rows - 1) * (size_t)ld_out + (size_t)heads * ATT_D) * 2;
  if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
      overlaps(out, out_bytes, v, in_bytes))
    return failf(TTT_E_CONFIG, "out overlaps q, k or v");
  const AttnArgs a = attention_args(q, k, v, ld, out, ld_out, batch, heads, seq_len, window,
                                    window_mode);
  BLK_HIP(launch_window_attention(a, static_cast<hipStream_t>(stream)));
  return TTT_OK;
}

ttt_status ttt_linear(const void* x, const void* w, const void* resid, void* y, int64_t rows,
                      int32_t in_features, int32_t out_features, int32_t epilogue,
                      void* stream) {
  BLK_TRY(check_linear(rows, in_features, out_features, epilogue));
  if (rows == 0) return TTT_OK;
  BLK_TRY(need(x, "x"));
  BLK_TRY(need(w, "w"));
  BLK_TRY(need(y, "y"));
  if (epilogue == TTT_LINEAR_RESIDUAL) BLK_TRY(need(resid, "resid"));
  const size_t ny = (size_t)rows * out_features * 2;
  if (overlaps(x, (size_t)rows * in_features * 2, y, ny) ||
      overlaps(w, (size_t)out_features * in_features * 2, y, ny))
    return failf(TTT_E_CONFIG, "x or w overlaps y");
  const LinearArgs a = linear_args(x, w, resid, y, rows, in_features, out_features);
  BLK_HIP(launch_linear(a, epilogue, static_cast<hipStream_t>(stream)));
  return TTT_OK;
}

ttt_status ttt_block_init(const ttt_block_config* cfg, const ttt_block_weights* w,
                          const float* w0, void* stream, ttt_block** out) {
  if (!out) return failf(TTT_E_NULL, "out is NULL");
  *out = nullptr;
  int F = 0;
  BLK_TRY(check_block_config(cfg, &F));
  if (!w) return failf(TTT_E_NULL, "weights are NULL");
  BLK_TRY(need(w->attn_qkv, "attn_qkv"));
  BLK_TRY(need(w->attn_out, "attn_out"));
  BLK_TRY(need(w->ttt_qkv, "ttt_qkv"));
  BLK_TRY(need(w->ttt_eta, "ttt_eta"));
  BLK_TRY(need(w->ttt_out, "ttt_out"));
  BLK_TRY(need(w->ffn_up, "ffn_up"));
  BLK_TRY(need(w->ffn_down, "ffn_down"));
  ttt_block* b = new (std::nothrow) ttt_block();
  if (!b) return failf(TTT_E_ALLOC, "out of host memory");
  b->cfg = *cfg;
  b->w = *w;
  b->F = F;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ttt_status r = ttt_init_state(&cfg->ttt, w0, stream, &b->ttt);
  if (r != TTT_OK) {
    release(b);
    return r;
  }
  int64_t numel = 0;
  ttt_state_numel(&cfg->ttt, &numel);
  if (hipMalloc(&b->s0, (size_t)numel * sizeof(float)) != hipSuccess) {
    release(b);
    return failf(TTT_E_ALLOC, "initial state copy of %lld floats", (long long)numel);
  }
  if ((r = ttt_get_state(b->ttt, b->s0, stream)) != TTT_OK) {
    release(b);
    return r;
  }
  const int64_t rows = (int64_t)cfg->batch * cfg->max_seq_len, D = cfg->dim;
  const size_t el = (size_t)std::max<int64_t>(rows, 1) * 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t onrm = take(el * D), oqkv = take(el * 3 * D), oatt = take(el * D),
               ohid = take(el * D), offn = take(el * F), otq = take(el * D), otk = take(el * D),
               otv = take(el * D), oto = take(el * D),
               oeta = take((size_t)std::max<int64_t>(rows, 1) * cfg->ttt.heads * sizeof(float));
  if (hipMalloc(&b->arena, off) != hipSuccess) {
    release(b);
    return failf(TTT_E_ALLOC, "block workspace of %zu bytes", off);
  }
  b->nrm = reinterpret_cast<u16*>(b->arena + onrm);
  b->qkv = reinterpret_cast<u16*>(b->arena + oqkv);
  b->att = reinterpret_cast<u16*>(b->arena + oatt);
  b->hid = reinterpret_cast<u16*>(b->arena + ohid);
  b->ffn = reinterpret_cast<u16*>(b->arena + offn);
  b->tq = reinterpret_cast<u16*>(b->arena + otq);
  b->tk = reinterpret_cast<u16*>(b->arena + otk);
  b->tv = reinterpret_cast<u16*>(b->arena + otv);
  b->to = reinterpret_cast<u16*>(b->arena + oto);
  b->eta = reinterpret_cast<float*>(b->arena + oeta);
  if (hipStreamSynchronize(st) != hipSuccess) {
    release(b);
    return failf(TTT_E_HIP, "block initialisation failed on the stream");
  }
  *out = b;
  return TTT_OK;
}

ttt_status ttt_block_forward(ttt_block* b, const void* x, void* y, int64_t T, void* stream) {
  if (!b) return failf(TTT_E_NULL, "block is NULL");
  const ttt_block_config& c = b->cfg;
  if (T < 0 || T > c.max_seq_len)
    return failf(TTT_E_SHAPE, "seq_len %lld outside [0, max_seq_len %lld]", (long long)T,
                 (long long)c.max_seq_len);
  if (T % c.ttt.chunk)
    return failf(TTT_E_SHAPE, "seq_len %lld is not a multiple of the chunk %d", (long long)T,
                 c.ttt.chunk);
  BLK_TRY(need(x, "x"));
  BLK_TRY(need(y, "y"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  BLK_TRY(ttt_set_state(b->ttt, b->s0, stream));
  if (T == 0) return TTT_OK;
  const int D = c.dim, F = b->F, B = c.batch, H = c.ttt.heads, d = c.ttt.dim;
  const int64_t rows = (int64_t)B * T;
  const u16* X = static_cast<const u16*>(x);
  auto rms = [&](const u16* in, const void* w_eta) {
    RmsArgs a;
    a.x = in;
    a.y = b->nrm;
    a.rows = rows;
    a.D = D;
    a.w_eta = static_cast<const u16*>(w_eta);
    a.eta = b->eta;
    a.heads = H;
    a.T = (int32_t)T;
    return launch_rmsnorm(a, st);
  };
  auto lin = [&](const void* in, const void* w, const void* resid, void* out, int K, int N,
                 int epi) { return launch_linear(linear_args(in, w, resid, out, rows, K, N), epi, st); };
  // h = x + Attn(n(x))
  BLK_HIP(rms(X, nullptr));
  BLK_HIP(lin(b->nrm, b->w.attn_qkv, nullptr, b->qkv, D, 3 * D, TTT_LINEAR_PLAIN));
  BLK_HIP(launch_window_attention(attention_args(b->qkv, b->qkv + D, b->qkv + 2 * D, 3 * D,
                                                 b->att, D, B, D / ATT_D, T, c.window,
                                                 c.window_mode), st));
  BLK_HIP(lin(b->att, b->w.attn_out, X, b->hid, D, D, TTT_LINEAR_RESIDUAL));
  // h = h + TTT(n(h))
  BLK_HIP(rms(b->hid, b->w.ttt_eta));
  BLK_HIP(lin(b->nrm, b->w.ttt_qkv, nullptr, b->qkv, D, 3 * D, TTT_LINEAR_PLAIN));
  {
    HeadSplitArgs a;
    a.qkv = b->qkv;
    a.q = b->tq;
    a.k = b->tk;
    a.v = b->tv;
    a.T = (int32_t)T;
    a.B = B;
    a.H = H;
    a.d = d;
    BLK_HIP(launch_split(a, st));
  }
  BLK_TRY(ttt_sequence_forward(b->ttt, b->tq, b->tk, b->tv, b->eta, b->to, T, stream));
  {
    HeadMergeArgs a;
    a.o = b->to;
    a.y = b->att;
    a.T = (int32_t)T;
    a.B = B;
    a.H = H;
    a.d = d;
    BLK_HIP(launch_merge(a, st));
  }
  BLK_HIP(lin(b->att, b->w.ttt_out, b->hid, b->hid, D, D, TTT_LINEAR_RESIDUAL));
  // y = h + FFN(n(h))
  BLK_HIP(rms(b->hid, nullptr));
  BLK_HIP(lin(b->nrm, b->w.ffn_up, nullptr, b->ffn, D, F, TTT_LINEAR_GELU));
  BLK_HIP(lin(b->ffn, b->w.ffn_down, b->hid, y, F, D, TTT_LINEAR_RESIDUAL));
  return TTT_OK;
}

ttt_state* ttt_block_ttt_state(ttt_block* b) { return b ? b->ttt : nullptr; }

ttt_status ttt_block_destroy(ttt_block* b) {
  if (!b) return TTT_OK;
  const hipError_t e = hipDeviceSynchronize();
  release(b);
  if (e != hipSuccess)
    return failf(TTT_E_HIP, "hipDeviceSynchronize failed: %s", hipGetErrorString(e));
  return TTT_OK;
}

}  // extern "C"
