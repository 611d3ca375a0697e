// Host side of libttt: argument checks, state and workspace ownership, and the chunk loop
// that enqueues the stage kernels of ttt_kernels.hip.  See include/libttt.h for the ABI.
#include "libttt.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "ttt_internal.h"

using namespace ttt;

namespace {

thread_local std::string g_err;

ttt_status fail(ttt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(TTT_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),     \
                  __FILE__, __LINE__);                                                  \
  } while (0)

constexpr int64_t SUBBLOCK_MAX = 65536;  // tokens per gradient / apply launch

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Dims {
  int P, nm, d, dh, n;      // problems, matrices, dim, hidden, columns of X orientation
  int rows[3], cols[3], tr[3];
  int ap, gp, np, wp, in_q, in_kv;
  int ns_one;               // bit i: Newton-Schulz iteration i on one bf16 plane
  int64_t sb;               // tokens per gradient / apply block
  bool mom;                 // momentum buffers follow the weights in the state
};

ttt_status resolve(const ttt_config* c, ttt_config* out) {
  if (!c) return fail(TTT_E_NULL, "config is NULL");
  ttt_config r = *c;
  if (r.fw < 0 || r.fw > 2) return fail(TTT_E_CONFIG, "unknown fw %d", r.fw);
  if (r.loss < 0 || r.loss > 1) return fail(TTT_E_CONFIG, "unknown loss %d", r.loss);
  if (r.act < 0 || r.act > 1) return fail(TTT_E_DTYPE, "unknown activation dtype %d", r.act);
  if (r.order < 0 || r.order > 1) return fail(TTT_E_CONFIG, "unknown order %d", r.order);
  if (r.row_renorm != 0 && r.row_renorm != 1)
    return fail(TTT_E_CONFIG, "row_renorm must be 0 or 1 (got %d)", r.row_renorm);
  if (r.ns_steps < 0 || r.ns_steps > 8)
    return fail(TTT_E_CONFIG, "ns_steps must be in [0, 8] (got %d)", r.ns_steps);
  if (r.batch < 1 || r.heads < 1) return fail(TTT_E_SHAPE, "batch and heads must be >= 1");
  if ((int64_t)r.batch * r.heads > 65535)
    return fail(TTT_E_SHAPE, "batch*heads = %lld exceeds 65535", (long long)r.batch * r.heads);
  if (r.dim < 16 || r.dim > 1024 || r.dim % 16)
    return fail(TTT_E_SHAPE, "dim must be a multiple of 16 in [16, 1024] (got %d)", r.dim);
  if (r.fw == TTT_FW_LINEAR) {
    r.hidden = r.dim;
  } else if (r.hidden < 16 || r.hidden > 4096 || r.hidden % 16) {
    return fail(TTT_E_SHAPE, "hidden must be a multiple of 16 in [16, 4096] (got %d)", r.hidden);
  }
  if (r.chunk < 1 || r.chunk > (1 << 30))
    return fail(TTT_E_SHAPE, "chunk must be in [1, 2^30] (got %d)", r.chunk);
  if (r.ns_steps > 0 && r.fw != TTT_FW_LINEAR && r.dim > r.hidden)
    return fail(TTT_E_UNSUPPORTED, "Newton-Schulz needs dim <= hidden (dim %d, hidden %d)",
                r.dim, r.hidden);
  const bool f32 = r.act == TTT_F32;
  int* pl[3] = {&r.apply_planes, &r.grad_planes, &r.ns_planes};
  const int dflt[3] = {f32 ? 3 : 1, f32 ? 3 : 2, f32 ? 3 : 2};
  const char* nm[3] = {"apply_planes", "grad_planes", "ns_planes"};
  for (int i = 0; i < 3; ++i) {
    if (*pl[i] == 0) *pl[i] = dflt[i];
    if (*pl[i] < 1 || *pl[i] > 3)
      return fail(TTT_E_CONFIG, "%s must be 0 (default) or 1..3 (got %d)", nm[i], *pl[i]);
  }
  if (r.ns_one_plane < 0 || r.ns_one_plane > 255)
    return fail(TTT_E_CONFIG, "ns_one_plane must be a bit mask in [0, 255] (got %d)",
                r.ns_one_plane);
  if (r.path < TTT_PATH_AUTO || r.path > TTT_PATH_RESIDENT)
    return fail(TTT_E_CONFIG, "unknown path %d", r.path);
  for (int i = 0; i < 3; ++i) {
    if (!std::isfinite(r.lr[i]) || r.lr[i] < 0.f)
      return fail(TTT_E_CONFIG, "lr[%d] must be finite and >= 0 (got %g)", i, (double)r.lr[i]);
    if (r.lr[i] == 0.f) r.lr[i] = 1.f;
  }
  if (!std::isfinite(r.weight_decay) || r.weight_decay < 0.f || r.weight_decay >= 1.f)
    return fail(TTT_E_CONFIG, "weight_decay must be in [0, 1) (got %g)", (double)r.weight_decay);
  const bool resident_ok = r.momentum == 0.f &&
      small_supported(r.fw == TTT_FW_MLP_GELU ? FW_GELU : -1, r.ns_steps, r.row_renorm,
                      r.act == TTT_BF16, r.order == TTT_APPLY_THEN_UPDATE, r.dim, r.hidden,
                      r.chunk, r.apply_planes, r.grad_planes);
  if (r.path == TTT_PATH_RESIDENT && !resident_ok)
    return fail(TTT_E_UNSUPPORTED,
                "the resident path needs the GELU MLP with dim 64, hidden 256, chunk <= 64, "
                "no Newton-Schulz, no renorm, bf16 activations, apply-then-update and one "
                "bf16 plane");
  if (r.path == TTT_PATH_AUTO) r.path = resident_ok ? TTT_PATH_RESIDENT : TTT_PATH_STAGED;
  if (r.replay != 0 && r.replay != 1)
    return fail(TTT_E_CONFIG, "replay must be 0 or 1 (got %d)", r.replay);
  if (!std::isfinite(r.momentum) || r.momentum < 0.f || r.momentum >= 1.f)
    return fail(TTT_E_CONFIG, "momentum must be in [0, 1) (got %g)", (double)r.momentum);
  if (r.momentum > 0.f && r.path == TTT_PATH_RESIDENT)
    return fail(TTT_E_UNSUPPORTED, "the resident path takes no momentum");
  if (out) *out = r;
  return TTT_OK;
}

Dims dims_of(const ttt_config& c) {
  Dims D{};
  D.P = c.batch * c.heads;
  D.d = c.dim;
  D.dh = c.hidden;
  if (c.fw == TTT_FW_SWIGLU) {
    D.nm = 3;
    D.n = c.hidden;
    int r[3] = {c.hidden, c.hidden, c.dim}, k[3] = {c.dim, c.dim, c.hidden}, t[3] = {1, 1, 0};
    for (int i = 0; i < 3; ++i) { D.rows[i] = r[i]; D.cols[i] = k[i]; D.tr[i] = t[i]; }
  } else if (c.fw == TTT_FW_MLP_GELU) {
    D.nm = 2;
    D.n = c.hidden;
    D.rows[0] = c.hidden; D.cols[0] = c.dim; D.tr[0] = 1;
    D.rows[1] = c.dim; D.cols[1] = c.hidden; D.tr[1] = 0;
  } else {
    D.nm = 1;
    D.n = c.dim;
    D.rows[0] = c.dim; D.cols[0] = c.dim; D.tr[0] = 0;
  }
  D.ap = c.apply_planes;
  D.gp = c.grad_planes;
  D.np = c.ns_planes;
  D.ns_one = c.ns_planes > 1 ? c.ns_one_plane & ((1 << c.ns_steps) - 1) : 0;
  D.wp = std::max(D.ap, D.gp);
  D.in_q = c.act == TTT_F32 ? D.ap : 1;
  D.in_kv = c.act == TTT_F32 ? D.gp : 1;
  D.sb = std::min<int64_t>(c.chunk, SUBBLOCK_MAX);
  D.mom = c.momentum > 0.f;
  return D;
}

// values of the fast-weight matrices alone, and of the whole state (with the buffers)
int64_t weights_numel(const Dims& D) {
  int64_t n = 0;
  for (int m = 0; m < D.nm; ++m) n += (int64_t)D.P * D.rows[m] * D.cols[m];
  return n;
}
int64_t state_numel(const Dims& D) { return weights_numel(D) * (D.mom ? 2 : 1); }

}  // namespace

// ============================================================================ state
struct ttt_state {
  ttt_config cfg;
  Dims D;
  char* arena = nullptr;
  size_t arena_bytes = 0;
  hipStream_t last = nullptr;
  int device = 0;

  float* W = nullptr;   // [state_numel] matrix by matrix, each [P][rows][cols]
  float* U = nullptr;   // same layout
  float* Wm[3] = {};    // per-matrix views
  float* Mm[3] = {};    // momentum buffers (after the weights in W), or null
  float* Um[3] = {};
  u16* Wpl[3] = {};     // planes [wp][P][rows][cols]
  // token-major workspaces, [planes][P][sb][cols]
  u16 *qpl = nullptr, *kpl = nullptr, *vpl = nullptr;  // fp32 activations as planes
  u16* nk = nullptr;                                   // -eta * K (linear net, dot loss)
  u16* hq = nullptr;                                   // query hidden [ap][P][sb][dh]
  u16 *dz1 = nullptr, *dz3 = nullptr, *pk = nullptr;   // [gp][P][sb][dh]
  u16 *hk = nullptr, *e = nullptr;                     // MSE: hidden, output error
  float *fa = nullptr, *fb = nullptr;                  // MSE: derivative factors
  float* G = nullptr;     // [nm][P][d][n]
  float* part = nullptr;  // [nm*P][contract tiles]
  float* gpart = nullptr; // token-split partial sums [ksplit][nm][P][d][n]
  int ksplit = 1;
  u16 *xpl[2] = {}, *apl = nullptr, *bpl = nullptr;
  int* health = nullptr;
  float* neg1 = nullptr;  // [sb] of -1: the apply backward's eta
  int contract_tiles = 0;
  int part_sub = 1;       // sum-of-squares parts per contraction tile (CONTRACT_SUM_SUB if split)
  int part_n = 0;         // sum-of-squares parts per matrix: contract_tiles x part_sub
  bool resident = false;  // the device-resident chunk loop serves this state (Wpl unused)
  // backward through an update: workspace allocated by the first ttt_chunk_backward call
  struct Bwd {
    char* arena = nullptr;
    float *g32 = nullptr, *du = nullptr, *dx32[2] = {}, *t32 = nullptr, *dg32 = nullptr;
    float *dws = nullptr, *dwg = nullptr, *dwa = nullptr;
    float* wbak = nullptr;          // update-then-apply: the weights before the chunk
    float *dotpart = nullptr, *eta_part = nullptr;
    u16* xit[8] = {};               // Newton-Schulz iterates 1..steps-1 (0 is xpl[0])
    u16 *dxp[2] = {}, *tp = nullptr, *sp = nullptr, *dgp = nullptr;
    u16 *pd = nullptr, *a1 = nullptr, *a3 = nullptr;
  } bw;
  // measurement hooks
  int prof_stage = -1, prof_cap = 0, prof_n = 0;
  hipEvent_t* prof_ev = nullptr;
  // replay: the last recorded forward call's graph and what it was recorded for
  hipStream_t cap = nullptr;
  hipGraphExec_t gexec = nullptr;
  struct GraphKey {
    const void *q, *k, *v, *eta, *out;
    int64_t T;
    uint64_t flags;   // hash of the update flags (0: none)
    bool operator==(const GraphKey& o) const {
      return q == o.q && k == o.k && v == o.v && eta == o.eta && out == o.out && T == o.T &&
             flags == o.flags;
    }
  } gkey{};
};

namespace {

struct Carver {
  size_t off = 0;
  template <class T>
  size_t take(int64_t count) {
    size_t o = off;
    off += round_up(std::max<int64_t>(count, 1) * (int64_t)sizeof(T), 256);
    return o;
  }
};

// Plan the arena layout; with base == nullptr only the size is computed.  With ext_w the
// fp32 state lives in that caller buffer instead of the arena (and no apply-backward
// buffer is carved: only the allocation-free sequence call lays a state out so).
size_t layout(ttt_state* s, char* base, float* ext_w = nullptr) {
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  const int64_t P = D.P, d = D.d, dh = D.dh, n = D.n, sb = D.sb;
  const bool mse = c.loss == TTT_LOSS_MSE;
  const bool lin = c.fw == TTT_FW_LINEAR;
  const bool f32 = c.act == TTT_F32;
  Carver C;
  size_t oW = ext_w ? 0 : C.take<float>(state_numel(D));
  size_t oU = C.take<float>(weights_numel(D));
  size_t oWpl[3];
  for (int m = 0; m < D.nm; ++m) oWpl[m] = C.take<u16>(D.wp * P * D.rows[m] * D.cols[m]);
  size_t oq = 0, ok = 0, ov = 0;
  if (f32) {
    oq = C.take<u16>(D.in_q * P * sb * d);
    ok = C.take<u16>(D.in_kv * P * sb * d);
    ov = C.take<u16>(D.in_kv * P * sb * d);
  }
  size_t onk = (lin && !mse) ? C.take<u16>(D.gp * P * sb * d) : 0;
  size_t ohq = lin ? 0 : C.take<u16>(D.ap * P * sb * dh);
  size_t odz1 = 0, odz3 = 0, opk = 0, ohk = 0, ofa = 0, ofb = 0, oe = 0;
  if (!lin) {
    odz1 = C.take<u16>(D.gp * P * sb * dh);
    if (c.fw == TTT_FW_SWIGLU) odz3 = C.take<u16>(D.gp * P * sb * dh);
    if (!mse) opk = C.take<u16>(D.gp * P * sb * dh);
  }
  if (mse) {
    if (!lin) {
      ohk = C.take<u16>(D.gp * P * sb * dh);
      ofa = C.take<float>(P * sb * dh);
      if (c.fw == TTT_FW_SWIGLU) ofb = C.take<float>(P * sb * dh);
    }
    oe = C.take<u16>(D.gp * P * sb * d);
  }
  size_t oG = C.take<float>(D.nm * P * d * n);
  const int ctiles = (int)(((d + CONTRACT_BM - 1) / CONTRACT_BM) * ((n + CONTRACT_BN - 1) / CONTRACT_BN));
  const int ksp = contract_split_max(ctiles, (int)(D.nm * P));
  const int psub = ksp > 1 ? CONTRACT_SUM_SUB : 1;
  size_t opart = C.take<float>((int64_t)D.nm * P * ctiles * psub);
  size_t ogp = ksp > 1 ? C.take<float>(ksp * D.nm * P * d * n) : 0;
  size_t ox[2] = {0, 0}, oa = 0, ob = 0;
  if (c.ns_steps > 0) {
    for (int i = 0; i < 2; ++i) ox[i] = C.take<u16>(D.np * D.nm * P * d * n);
    oa = C.take<u16>(D.np * D.nm * P * d * d);
    ob = C.take<u16>(D.np * D.nm * P * d * d);
  }
  size_t oh = C.take<int>(1);
  const size_t on1 = (s->resident || ext_w) ? 0 : C.take<float>(D.sb);
  if (base) {
    auto F = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
    auto H = [&](size_t o) { return reinterpret_cast<u16*>(base + o); };
    s->W = ext_w ? ext_w : F(oW);
    s->U = F(oU);
    int64_t acc = 0;
    for (int m = 0; m < D.nm; ++m) {
      s->Wm[m] = s->W + acc;
      s->Mm[m] = D.mom ? s->W + weights_numel(D) + acc : nullptr;
      s->Um[m] = s->U + acc;
      acc += P * D.rows[m] * D.cols[m];
      s->Wpl[m] = H(oWpl[m]);
    }
    if (f32) { s->qpl = H(oq); s->kpl = H(ok); s->vpl = H(ov); }
    s->nk = (lin && !mse) ? H(onk) : nullptr;
    s->hq = lin ? nullptr : H(ohq);
    if (!lin) {
      s->dz1 = H(odz1);
      s->dz3 = c.fw == TTT_FW_SWIGLU ? H(odz3) : nullptr;
      s->pk = mse ? nullptr : H(opk);
    }
    if (mse) {
      if (!lin) {
        s->hk = H(ohk); s->fa = F(ofa);
        s->fb = c.fw == TTT_FW_SWIGLU ? F(ofb) : nullptr;
      }
      s->e = H(oe);
    }
    s->G = F(oG);
    s->part = F(opart);
    s->contract_tiles = ctiles;
    s->part_sub = psub;
    s->part_n = ctiles * psub;
    s->ksplit = ksp;
    s->gpart = ksp > 1 ? F(ogp) : nullptr;
    if (c.ns_steps > 0) {
      for (int i = 0; i < 2; ++i) s->xpl[i] = H(ox[i]);
      s->apl = H(oa); s->bpl = H(ob);
    }
    s->health = reinterpret_cast<int*>(base + oh);
    if (!s->resident && !ext_w) s->neg1 = F(on1);
  }
  return C.off;
}

PlaneBuf pbuf(u16* base, int np, int64_t plane_stride, int64_t zstride, int64_t ld) {
  PlaneBuf b;
  b.base = base; b.plane_stride = plane_stride; b.zstride = zstride; b.ld = ld; b.np = np;
  return b;
}

// Launch `call` as stage `id`, bracketed by profiling events when that stage is traced.
template <class F>
hipError_t staged(ttt_state* s, int id, hipStream_t st, F call) {
  const bool rec = s->prof_stage == id && s->prof_n < s->prof_cap;
  if (rec) {
    hipError_t e = hipEventRecord(s->prof_ev[2 * s->prof_n], st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = call();
  if (rec && e == hipSuccess) {
    e = hipEventRecord(s->prof_ev[2 * s->prof_n + 1], st);
    ++s->prof_n;
  }
  return e;
}
#define STAGED(id, expr) HIP_TRY(staged(s, id, st, [&]() { return (expr); }))

// Operand over a caller tensor: element (r, k) of problem z at p + z*zstride + r*ld + k.
Operand act_operand(const void* p, int64_t zstride, int64_t ld, int rows) {
  return make_operand(static_cast<const u16*>(p), 0, ld, zstride, 1, rows);
}

ttt_status refresh_planes(ttt_state* s, bool with_update, hipStream_t st) {
  const Dims& D = s->D;
  RenormArgs r{};
  r.P = D.P; r.np = D.wp; r.renorm = with_update && s->cfg.row_renorm; r.nm = D.nm;
  r.keep = 1.f - s->cfg.weight_decay;
  r.health = s->health;
  r.max_rows = 0;
  for (int m = 0; m < D.nm; ++m) {
    RenormMat& M = r.m[m];
    M.W = s->Wm[m];
    M.U = with_update ? s->Um[m] : nullptr;
    M.lr = s->cfg.lr[m];
    M.rows = D.rows[m]; M.cols = D.cols[m];
    M.pl = s->Wpl[m];
    M.pl_stride = (int64_t)D.P * D.rows[m] * D.cols[m];
    r.max_rows = std::max(r.max_rows, D.rows[m]);
  }
  STAGED(TTT_STAGE_RENORM, launch_renorm(r, st));
  return TTT_OK;
}

// Tensor views of one token range [t0, t0+nr) of the caller's [B][H][T][d] tensors.
struct Rows {
  const char *q, *k, *v;
  const float* eta;
  char* out;
  int64_t T;    // tokens per problem in the caller's tensors
  int64_t t0;   // first token of the range
  int nr;       // number of tokens
  bool split;   // fp32 activations: q, k and v of the range already split into their planes
};

ttt_status apply_rows(ttt_state* s, const Rows& R, hipStream_t st) {
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  const size_t es = c.act == TTT_BF16 ? 2 : 4;
  const int P = D.P, d = D.d, dh = D.dh;
  const char* q = R.q + R.t0 * d * es;
  Operand xq;
  if (c.act == TTT_F32) {
    SplitArgs sa{};
    sa.x = q; sa.x_zstride = R.T * d; sa.n = R.nr; sa.d = d;
    sa.out = pbuf(s->qpl, D.in_q, (int64_t)P * D.sb * d, D.sb * d, d);
    if (!R.split) STAGED(TTT_STAGE_SPLIT, launch_split(sa, P, st));
    xq = operand_of(sa.out, D.in_q, R.nr);
  } else {
    xq = act_operand(q, R.T * d, d, R.nr);
  }
  OutArgs o{};
  o.nrows = R.nr; o.N = d;
  o.out = R.out + R.t0 * d * es; o.out_zstride = R.T * d; o.out_bf16 = c.act == TTT_BF16;
  if (c.fw == TTT_FW_LINEAR) {
    o.a = xq;
    o.b = operand_of(pbuf(s->Wpl[0], D.ap, (int64_t)P * d * d, (int64_t)d * d, d), D.ap, d);
    o.K = d;
    STAGED(TTT_STAGE_OUT, launch_out(OUT_Q, o, P, st));
    return TTT_OK;
  }
  FrontArgs f{};
  f.A[0] = xq;
  f.B[0] = operand_of(pbuf(s->Wpl[0], D.ap, (int64_t)P * dh * d, (int64_t)dh * d, d), D.ap, dh);
  if (c.fw == TTT_FW_SWIGLU)
    f.B[1] = operand_of(pbuf(s->Wpl[1], D.ap, (int64_t)P * dh * d, (int64_t)dh * d, d), D.ap, dh);
  f.nrows = R.nr; f.K = d; f.N = dh;
  f.o1 = pbuf(s->hq, D.ap, (int64_t)P * D.sb * dh, D.sb * dh, dh);
  STAGED(TTT_STAGE_FRONT_Q, launch_front(c.fw == TTT_FW_SWIGLU ? FW_SWIGLU : FW_GELU, FRONT_Q, f, P, st));
  const int w2 = D.nm - 1;
  o.a = operand_of(f.o1, D.ap, R.nr);
  o.b = operand_of(pbuf(s->Wpl[w2], D.ap, (int64_t)P * d * dh, (int64_t)d * dh, dh), D.ap, d);
  o.K = dh;
  STAGED(TTT_STAGE_OUT, launch_out(OUT_Q, o, P, st));
  return TTT_OK;
}

// Gradient of one token block; the contraction adds into G (first block writes it).
// The chunk-summed contractions of one token block into G, and after the chunk's last
// block into U (plain step; weight orientation) or the first Newton-Schulz input (muon).
// ca holds the per-matrix operands and sizes (and ca.g32, a copy of the final sum).
ttt_status contract_all(ttt_state* s, ContractArgs ca, float* U, bool muon, bool first,
                        bool last, hipStream_t st) {
  const Dims& D = s->D;
  const int P = D.P, d = D.d;
  float* const G = s->G;
  ca.G = G;
  ca.accum_in = first ? 0 : 1;
  ca.last = last ? 1 : 0;
  ca.muon = muon;
  const int64_t Z = (int64_t)D.nm * P;
  if (ca.muon) ca.x = pbuf(s->xpl[0], D.np, Z * d * D.n, (int64_t)d * D.n, D.n);
  ca.part = s->part;
  ca.psub = s->part_sub;
  ca.U = U;
  ca.gpart = s->gpart;
  ca.gpart_stride = (int64_t)D.nm * P * d * D.n;
  ca.ksplit = s->ksplit;
  ca.tr_mask = D.tr[0] | (D.tr[1] << 1) | (D.tr[2] << 2);
  // operands of one launch share a plane count per side: group the matrices accordingly
  int m0 = 0;
  while (m0 < D.nm) {
    int m1 = m0 + 1;
    while (m1 < D.nm && ca.a[m1].planes == ca.a[m0].planes && ca.b[m1].planes == ca.b[m0].planes) ++m1;
    ContractArgs cg = ca;
    for (int m = m0; m < m1; ++m) { cg.a[m - m0] = ca.a[m]; cg.b[m - m0] = ca.b[m]; }
    cg.G = G + (int64_t)m0 * P * d * D.n;
    if (s->gpart) cg.gpart = s->gpart + (int64_t)m0 * P * d * D.n;
    cg.U = U + (int64_t)m0 * P * d * D.n;
    if (ca.mom) cg.mom = ca.mom + (int64_t)m0 * P * d * D.n;
    if (ca.g32) cg.g32 = ca.g32 + (int64_t)m0 * P * d * D.n;
    if (ca.muon) cg.x.base = ca.x.base + (int64_t)m0 * P * ca.x.zstride;
    cg.part = s->part + (int64_t)m0 * P * s->part_n;
    cg.tr_mask = ca.tr_mask >> m0;
    STAGED(TTT_STAGE_CONTRACT, launch_contract(cg, m1 - m0, st));
    m0 = m1;
  }
  return TTT_OK;
}

// g32: the last block's epilogue also stores the step's input (the gradient, with momentum
// beta M + the gradient) in fp32 in the X orientation here (the backward's Newton-Schulz
// scaling needs it).
// read_mom: the momentum buffers are read, not replaced (the backward's recompute).
ttt_status grad_rows(ttt_state* s, const Rows& R, bool first, bool last, hipStream_t st,
                     float* g32 = nullptr, bool read_mom = false) {
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  const size_t es = c.act == TTT_BF16 ? 2 : 4;
  const int P = D.P, d = D.d, dh = D.dh;
  const int64_t SB = D.sb;
  const bool mse = c.loss == TTT_LOSS_MSE, lin = c.fw == TTT_FW_LINEAR;
  const bool sw = c.fw == TTT_FW_SWIGLU;
  const char* k = R.k + R.t0 * d * es;
  const char* v = R.v + R.t0 * d * es;
  const float* eta = R.eta + R.t0;
  const int gi = D.in_kv, gp = D.gp;

  // token-major planes of this block: [planes][P][SB][cols]
  auto tok = [&](u16* b, int np, int cols) {
    return pbuf(b, np, (int64_t)P * SB * cols, SB * cols, cols);
  };
  SplitArgs sa{};
  sa.x_zstride = R.T * d; sa.x_bf16 = c.act == TTT_BF16; sa.eta = eta; sa.eta_zstride = R.T;
  sa.n = R.nr; sa.d = d;
  Operand xk, xv;
  if (c.act == TTT_F32) {
    SplitArgs sv = sa;
    sa.x = k; sa.out = tok(s->kpl, gi, d);
    sv.x = v; sv.out = tok(s->vpl, gi, d);
    if (!R.split) STAGED(TTT_STAGE_SPLIT, launch_split2(sa, sv, P, st));
    xk = operand_of(sa.out, gi, R.nr);
    xv = operand_of(sv.out, gi, R.nr);
  } else {
    xk = act_operand(k, R.T * d, d, R.nr);
    xv = act_operand(v, R.T * d, d, R.nr);
  }
  // the same tensors read column-wise by the contractions: rows of the operand = features
  auto as_cols = [&](Operand o, int cols) { o.rows = cols; return o; };

  auto wop = [&](int m, int np) {
    return operand_of(pbuf(s->Wpl[m], np, (int64_t)P * D.rows[m] * D.cols[m],
                           (int64_t)D.rows[m] * D.cols[m], D.cols[m]), np, D.rows[m]);
  };
  const int w2 = D.nm - 1;
  // W2 [d][dh] read column-wise: the operand's rows are W2's columns (the hidden index)
  Operand w2c{};
  if (!lin) w2c = operand_of(pbuf(s->Wpl[w2], gp, (int64_t)P * d * dh, (int64_t)d * dh, dh), gp, dh);

  PlaneBuf dz1{}, dz3{}, pk{}, hk{}, e{}, nk{};
  if (!lin) {
    dz1 = tok(s->dz1, gp, dh);
    if (sw) dz3 = tok(s->dz3, gp, dh);
  }
  if (!lin && !mse) {
    pk = tok(s->pk, gp, dh);
    FrontArgs f{};
    f.A[0] = xk; f.A[1] = xv; f.B[0] = wop(0, gp);
    if (sw) f.B[1] = wop(1, gp);
    f.B[sw ? 2 : 1] = w2c;
    f.eta = eta; f.eta_zstride = R.T;
    f.nrows = R.nr; f.K = d; f.N = dh;
    f.o1 = dz1; f.o2 = dz3; f.o3 = pk;
    STAGED(TTT_STAGE_FRONT_K, launch_front(sw ? FW_SWIGLU : FW_GELU, FRONT_K_DOT, f, P, st));
  } else if (mse) {
    Operand ok_a;
    if (!lin) {
      hk = tok(s->hk, gp, dh);
      FrontArgs f{};
      f.A[0] = xk; f.B[0] = wop(0, gp);
      if (sw) f.B[1] = wop(1, gp);
      f.nrows = R.nr; f.K = d; f.N = dh;
      f.o1 = hk;
      f.fa = s->fa; f.fb = s->fb; f.f_zstride = SB * dh;
      STAGED(TTT_STAGE_FRONT_K, launch_front(sw ? FW_SWIGLU : FW_GELU, FRONT_K_MSE, f, P, st));
      ok_a = operand_of(hk, gp, R.nr);
    } else {
      ok_a = xk;
    }
    e = tok(s->e, gp, d);
    OutArgs o{};
    o.a = ok_a;
    o.b = wop(w2, gp);   // W2 [d][dh] (or W [d][d]) as the [N][K] operand
    o.nrows = R.nr; o.K = lin ? d : dh; o.N = d;
    o.vin = v; o.v_zstride = R.T * d; o.v_bf16 = c.act == TTT_BF16;
    o.eta = eta; o.eta_zstride = R.T;
    o.e = e;
    STAGED(TTT_STAGE_MSE, launch_out(OUT_K_MSE, o, P, st));
    if (!lin) {
      OutArgs h{};
      h.a = operand_of(e, gp, R.nr);
      h.b = w2c;
      h.nrows = R.nr; h.K = d; h.N = dh;
      h.fa = s->fa; h.fb = s->fb; h.f_zstride = SB * dh;
      h.dz1 = dz1; h.dz3 = dz3; h.swiglu = sw;
      STAGED(TTT_STAGE_MSE, launch_out(DH_MSE, h, P, st));
    }
  } else {  // linear net, inner-product loss: the gradient is V^T (-eta K)
    nk = tok(s->nk, gp, d);
    sa.x = k; sa.neg_eta = 1; sa.out = nk;
    STAGED(TTT_STAGE_SPLIT, launch_split(sa, P, st));
  }

  // contraction: X_m [d x n] = sum over tokens of A_m[t][:]^T B_m[t][:]
  ContractArgs ca{};
  ca.P = P; ca.M = d; ca.N = D.n; ca.K = R.nr;
  auto colop = [&](const PlaneBuf& b, int cols) {
    return operand_of(b, b.np, cols);
  };
  if (lin) {
    if (mse) { ca.a[0] = colop(e, d); ca.b[0] = as_cols(xk, d); }
    else { ca.a[0] = as_cols(xv, d); ca.b[0] = colop(nk, d); }
  } else {
    ca.a[0] = as_cols(xk, d); ca.b[0] = colop(dz1, dh);
    int m = 1;
    if (sw) { ca.a[1] = as_cols(xk, d); ca.b[1] = colop(dz3, dh); m = 2; }
    if (mse) { ca.a[m] = colop(e, d); ca.b[m] = colop(hk, dh); }
    else { ca.a[m] = as_cols(xv, d); ca.b[m] = colop(pk, dh); }
  }
  if (D.mom) {   // the chunk's gradient enters the momentum buffers in the last epilogue
    ca.mom = s->Mm[0];
    ca.beta = c.momentum;
    ca.mom_write = read_mom ? 0 : 1;
  }
  ca.g32 = g32;
  return contract_all(s, ca, s->U, c.ns_steps > 0, first, last, st);
}

// keep: write iterate it + 1 to keep[it + 1] (kept for the backward) instead of the
// ping-pong buffers; iterate 0 stays in xpl[0].
ttt_status newton_schulz(ttt_state* s, hipStream_t st, u16* const* keep = nullptr) {
  const Dims& D = s->D;
  const int steps = s->cfg.ns_steps;
  const int Z = D.nm * D.P, M = D.d, N = D.n;
  auto iterate = [&](int i) { return (keep && i > 0) ? keep[i] : s->xpl[i & 1]; };
  if (!keep && M <= NS_SMALL_M && N <= NS_SMALL_N) {
    // every iteration of each matrix in one workgroup (the iterates stay in LDS)
    NsArgs a{};
    a.Z = Z; a.M = M; a.N = N; a.P = D.P;
    a.coef_a = 3.4445f; a.coef_b = -4.7750f; a.coef_c = 2.0315f;
    a.part = s->part; a.nparts = s->part_n;
    a.eps = 1e-7f;
    a.steps = steps;
    a.one = D.ns_one;
    a.xin = pbuf(s->xpl[0], D.np, (int64_t)Z * M * N, (int64_t)M * N, N);
    a.U = s->U;
    a.tr_mask = D.tr[0] | (D.tr[1] << 1) | (D.tr[2] << 2);
    STAGED(TTT_STAGE_NS_SMALL, launch_ns_small(a, st));
    return TTT_OK;
  }
  for (int it = 0; it < steps; ++it) {
    // products on pk planes; the iterates X keep D.np planes between iterations
    const int pk = ((D.ns_one >> it) & 1) ? 1 : D.np;
    NsArgs a{};
    a.Z = Z; a.M = M; a.N = N; a.P = D.P;
    a.pl = pk;
    a.fold = pk == D.np;   // a I folded into B' where B' holds X's precision
    a.coef_a = 3.4445f; a.coef_b = -4.7750f; a.coef_c = 2.0315f;
    a.part = s->part; a.nparts = s->part_n; a.first = it == 0; a.last = it == steps - 1;
    a.eps = 1e-7f;
    a.xin = pbuf(iterate(it), D.np, (int64_t)Z * M * N, (int64_t)M * N, N);
    a.aout = pbuf(s->apl, pk, (int64_t)Z * M * M, (int64_t)M * M, M);
    STAGED(TTT_STAGE_NS_GRAM, launch_ns_gram(a, st));
    a.ain = a.aout;
    a.aout = pbuf(s->bpl, pk, (int64_t)Z * M * M, (int64_t)M * M, M);
    STAGED(TTT_STAGE_NS_POLY, launch_ns_poly(a, st));
    a.ain = a.aout;
    a.xout = pbuf(it + 1 < steps ? iterate(it + 1) : s->xpl[(it + 1) & 1], D.np,
                  (int64_t)Z * M * N, (int64_t)M * N, N);
    a.U = s->U;
    a.tr_mask = D.tr[0] | (D.tr[1] << 1) | (D.tr[2] << 2);
    STAGED(TTT_STAGE_NS_UPDATE, launch_ns_update(a, st));
  }
  return TTT_OK;
}

// Backward of the apply step over one block of query rows: dQ rows, and the weight
// gradients of sum <dO, f_W(Q)> summed into dw over the chunk's blocks.  It reuses the
// gradient path: the key-row front takes the queries as keys, dO as values and eta = -1
// (the inner-product loss is then +sum <f(q), dO>), the contractions sum the weight
// gradients (their plain-step output is the gradient itself), and k_dq forms
// dQ = sum_m dZ_m W_m.
ttt_status apply_bwd_rows(ttt_state* s, const Rows& R, bool first, bool last, float* dw,
                          hipStream_t st) {
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  const size_t es = c.act == TTT_BF16 ? 2 : 4;
  const int P = D.P, d = D.d, dh = D.dh;
  const int64_t SB = D.sb;
  const bool lin = c.fw == TTT_FW_LINEAR, sw = c.fw == TTT_FW_SWIGLU;
  const char* q = R.q + R.t0 * d * es;
  const char* o = R.v + R.t0 * d * es;   // dO rows
  const int gi = D.in_kv, gp = D.gp;
  auto tok = [&](u16* b, int np, int cols) {
    return pbuf(b, np, (int64_t)P * SB * cols, SB * cols, cols);
  };
  Operand xq, xo;
  if (c.act == TTT_F32) {
    SplitArgs sa{};
    sa.x_zstride = R.T * d; sa.x_bf16 = 0; sa.n = R.nr; sa.d = d;
    SplitArgs so = sa;
    sa.x = q; sa.out = tok(s->kpl, gi, d);
    so.x = o; so.out = tok(s->vpl, gi, d);
    STAGED(TTT_STAGE_SPLIT, launch_split2(sa, so, P, st));
    xq = operand_of(sa.out, gi, R.nr);
    xo = operand_of(so.out, gi, R.nr);
  } else {
    xq = act_operand(q, R.T * d, d, R.nr);
    xo = act_operand(o, R.T * d, d, R.nr);
  }
  auto as_cols = [&](Operand op, int cols) { op.rows = cols; return op; };
  auto wop = [&](int m, int np) {
    return operand_of(pbuf(s->Wpl[m], np, (int64_t)P * D.rows[m] * D.cols[m],
                           (int64_t)D.rows[m] * D.cols[m], D.cols[m]), np, D.rows[m]);
  };
  auto colop = [&](const PlaneBuf& b, int cols) { return operand_of(b, b.np, cols); };
  ContractArgs ca{};
  ca.P = P; ca.M = d; ca.N = D.n; ca.K = R.nr;
  DqArgs da{};
  da.nrows = R.nr; da.N = d;
  da.out = R.out + R.t0 * d * es; da.out_zstride = R.T * d; da.out_bf16 = c.act == TTT_BF16;
  int np = 1;
  if (lin) {
    ca.a[0] = as_cols(xo, d); ca.b[0] = as_cols(xq, d);
    da.a[0] = xo; da.b[0] = as_cols(wop(0, gp), d); da.K = d;
  } else {
    // P = H_q lands in the inner-product loss's P buffer, or for an MSE state in its
    // hidden-activation buffer (the same shape; the MSE forward path has no P buffer)
    u16* const pbuf_q = s->pk ? s->pk : s->hk;
    if (!s->dz1 || !pbuf_q || (sw && !s->dz3))
      return fail(TTT_E_HIP, "apply backward: gradient workspace missing");
    const PlaneBuf dz1 = tok(s->dz1, gp, dh), pk = tok(pbuf_q, gp, dh);
    PlaneBuf dz3{};
    if (sw) dz3 = tok(s->dz3, gp, dh);
    const int w2 = D.nm - 1;
    FrontArgs f{};
    f.A[0] = xq; f.A[1] = xo; f.B[0] = wop(0, gp);
    if (sw) f.B[1] = wop(1, gp);
    f.B[sw ? 2 : 1] =
        operand_of(pbuf(s->Wpl[w2], gp, (int64_t)P * d * dh, (int64_t)d * dh, dh), gp, dh);
    f.eta = s->neg1; f.eta_zstride = 0;
    f.nrows = R.nr; f.K = d; f.N = dh;
    f.o1 = dz1; f.o2 = dz3; f.o3 = pk;
    STAGED(TTT_STAGE_FRONT_K, launch_front(sw ? FW_SWIGLU : FW_GELU, FRONT_K_DOT, f, P, st));
    ca.a[0] = as_cols(xq, d); ca.b[0] = colop(dz1, dh);
    int m = 1;
    if (sw) { ca.a[1] = as_cols(xq, d); ca.b[1] = colop(dz3, dh); m = 2; }
    ca.a[m] = as_cols(xo, d); ca.b[m] = colop(pk, dh);
    da.a[0] = operand_of(dz1, gp, R.nr); da.b[0] = as_cols(wop(0, gp), d); da.K = dh;
    if (sw) {
      da.a[1] = operand_of(dz3, gp, R.nr); da.b[1] = as_cols(wop(1, gp), d);
      np = 2;
    }
  }
  ttt_status r = contract_all(s, ca, dw, false, first, last, st);
  if (r != TTT_OK) return r;
  STAGED(TTT_STAGE_DQ, launch_dq(da, np, P, st));
  return TTT_OK;
}

// One chunk: apply and update in the configured order, or (update == false) apply only
// with the state as it stands.
ttt_status run_chunk(ttt_state* s, const Rows& R00, hipStream_t st, bool update = true) {
  const ttt_config& c = s->cfg;
  const Dims& D = s->D;
  const int64_t b = c.chunk;
  ttt_status r;
  Rows R0 = R00;
  if (update && c.act == TTT_F32 && b <= D.sb) {
    // fp32 activations of a chunk in one token block: q, k and v into their bf16 planes in
    // one launch (the apply and gradient launches then read the planes)
    const int P = D.P, d = D.d;
    SplitArgs sq{};
    sq.x = R0.q + R0.t0 * d * 4; sq.x_zstride = R0.T * d; sq.n = (int)b; sq.d = d;
    sq.out = pbuf(s->qpl, D.in_q, (int64_t)P * D.sb * d, D.sb * d, d);
    SplitArgs sk = sq, sv = sq;
    sk.x = R0.k + R0.t0 * d * 4;
    sk.out = pbuf(s->kpl, D.in_kv, (int64_t)P * D.sb * d, D.sb * d, d);
    sv.x = R0.v + R0.t0 * d * 4;
    sv.out = pbuf(s->vpl, D.in_kv, (int64_t)P * D.sb * d, D.sb * d, d);
    STAGED(TTT_STAGE_SPLIT, launch_split3(sq, sk, sv, P, st));
    R0.split = true;
  }
  auto apply_all = [&]() -> ttt_status {
    for (int64_t o = 0; o < b; o += D.sb) {
      Rows R = R0;
      R.t0 = R0.t0 + o;
      R.nr = (int)std::min<int64_t>(D.sb, b - o);
      ttt_status x = apply_rows(s, R, st);
      if (x != TTT_OK) return x;
    }
    return TTT_OK;
  };
  if (!update) return apply_all();
  if (c.order == TTT_APPLY_THEN_UPDATE && (r = apply_all()) != TTT_OK) return r;
  for (int64_t o = 0; o < b; o += D.sb) {
    Rows R = R0;
    R.t0 = R0.t0 + o;
    R.nr = (int)std::min<int64_t>(D.sb, b - o);
    if ((r = grad_rows(s, R, o == 0, o + D.sb >= b, st)) != TTT_OK) return r;
  }
  if (c.ns_steps > 0 && (r = newton_schulz(s, st)) != TTT_OK) return r;
  if ((r = refresh_planes(s, true, st)) != TTT_OK) return r;
  if (c.order == TTT_UPDATE_THEN_APPLY && (r = apply_all()) != TTT_OK) return r;
  return TTT_OK;
}

ttt_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(TTT_E_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16)
    return fail(TTT_E_ALIGN, "%s is not 16-byte aligned", name);
  return TTT_OK;
}

// ---------------------------------------------------------------- backward through an update
// Workspace of the chunk backward, carved from one allocation made by the first call.
ttt_status ensure_bwd(ttt_state* s) {
  if (s->bw.arena) return TTT_OK;
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  const int64_t P = D.P, d = D.d, dh = D.dh, n = D.n, sb = D.sb, Z = (int64_t)D.nm * P;
  const int64_t xs = Z * d * n;   // one X-orientation tensor
  const bool muon = c.ns_steps > 0;
  Carver C;
  size_t og = muon ? C.take<float>(xs) : 0, odu = C.take<float>(xs);
  size_t odx[2] = {0, 0}, ot = 0, odxp[2] = {0, 0}, otp = 0, osp = 0, odot = 0;
  size_t oit[8] = {};
  if (muon) {
    for (int i = 0; i < 2; ++i) odx[i] = C.take<float>(xs);
    ot = C.take<float>(Z * d * d);
    for (int i = 0; i < 2; ++i) odxp[i] = C.take<u16>(D.np * xs);
    otp = C.take<u16>(D.np * Z * d * d);
    osp = C.take<u16>(D.np * Z * d * d);
    odot = C.take<float>(Z * gemm2_tiles(d, n));
    for (int i = 1; i < c.ns_steps; ++i) oit[i] = C.take<u16>(D.np * xs);
  }
  size_t odg = C.take<float>(xs), odgp = C.take<u16>(D.gp * xs);
  const int64_t sn = weights_numel(D);
  size_t ows = C.take<float>(sn), owg = C.take<float>(sn), owa = C.take<float>(sn);
  const bool uta = c.order == TTT_UPDATE_THEN_APPLY;
  size_t owb = uta ? C.take<float>(sn) : 0;
  size_t oep = C.take<float>(P * sb * ((dh + 63) / 64));
  size_t opd = C.take<u16>(D.gp * P * sb * dh), oa1 = C.take<u16>(D.gp * P * sb * dh),
         oa3 = C.take<u16>(D.gp * P * sb * dh);
  char* base = nullptr;
  hipError_t e = hipMalloc(&base, C.off);
  if (e != hipSuccess)
    return fail(e == hipErrorOutOfMemory ? TTT_E_ALLOC : TTT_E_HIP,
                "backward workspace of %zu bytes: %s", C.off, hipGetErrorString(e));
  auto F = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  auto H = [&](size_t o) { return reinterpret_cast<u16*>(base + o); };
  ttt_state::Bwd& b = s->bw;
  b.arena = base;
  b.g32 = muon ? F(og) : nullptr;
  b.du = F(odu);
  if (muon) {
    for (int i = 0; i < 2; ++i) { b.dx32[i] = F(odx[i]); b.dxp[i] = H(odxp[i]); }
    b.t32 = F(ot); b.tp = H(otp); b.sp = H(osp); b.dotpart = F(odot);
    b.xit[0] = s->xpl[0];
    for (int i = 1; i < c.ns_steps; ++i) b.xit[i] = H(oit[i]);
  }
  b.dg32 = F(odg); b.dgp = H(odgp);
  b.dws = F(ows); b.dwg = F(owg); b.dwa = F(owa);
  b.wbak = uta ? F(owb) : nullptr;
  b.eta_part = F(oep);
  b.pd = H(opd); b.a1 = H(oa1); b.a3 = H(oa3);
  return TTT_OK;
}

// Backward of the Newton-Schulz iteration: from dU (X orientation, in bw.du) to dG (bw.dg32
// and its planes), with the iterates kept by the forward recompute.
ttt_status ns_backward(ttt_state* s, hipStream_t st) {
  const Dims& D = s->D;
  ttt_state::Bwd& b = s->bw;
  const int steps = s->cfg.ns_steps;
  const int Z = D.nm * D.P, M = D.d, N = D.n, np = D.np;
  const int64_t xs = (int64_t)Z * M * N, as = (int64_t)Z * M * M;
  const float ca = 3.4445f, cb = -4.7750f, cc = 2.0315f, eps = 1e-7f;
  auto xpb = [&](u16* p) { return pbuf(p, np, xs, (int64_t)M * N, N); };
  auto apb = [&](u16* p) { return pbuf(p, np, as, (int64_t)M * M, M); };
  // dX_5 = dU, as planes for the products
  SplitArgs sa{};
  sa.x = b.du; sa.x_zstride = (int64_t)M * N; sa.n = M; sa.d = N;
  sa.out = xpb(b.dxp[0]);
  STAGED(TTT_STAGE_SPLIT, launch_split(sa, Z, st));
  const float* dx32 = b.du;
  int cur = 0;
  for (int it = steps - 1; it >= 0; --it) {
    const bool first = it == 0;
    // A and B' = a I + b A + c A^2 of this iteration, from its iterate (iteration 0's
    // iterate holds G, the Gram's scale s^2 applied in its epilogue)
    NsArgs a{};
    a.Z = Z; a.M = M; a.N = N; a.P = D.P; a.pl = np; a.fold = 1;
    a.coef_a = ca; a.coef_b = cb; a.coef_c = cc;
    a.part = s->part; a.nparts = s->part_n; a.first = first; a.last = 0; a.eps = eps;
    a.xin = xpb(b.xit[it]);
    a.aout = apb(s->apl);
    STAGED(TTT_STAGE_NS_GRAM, launch_ns_gram(a, st));
    a.ain = a.aout;
    a.aout = apb(s->bpl);
    STAGED(TTT_STAGE_NS_POLY, launch_ns_poly(a, st));
    const Operand X = operand_of(xpb(b.xit[it]), np, M);        // rows of X, K = N
    const Operand dX = operand_of(xpb(b.dxp[cur]), np, M);
    // T = dX X^T + X dX^T   (iteration 0: X = s G, s from the forward's tile sums)
    Gemm2Args g{};
    g.M = M; g.N = M; g.K = N; g.Z = Z;
    g.a[0] = dX; g.b[0] = X; g.a[1] = X; g.b[1] = dX;
    g.alpha = 1.f; g.beta = 0.f;
    g.cout = b.t32; g.pout = apb(b.tp);
    g.spart = first ? s->part : nullptr; g.nspart = s->part_n; g.eps = eps;
    STAGED(TTT_STAGE_NS_BWD, launch_gemm2(g, false, st, true));   // T is symmetric
    // S = b T + c (T A + A T) (A, T symmetric: rows serve as columns); iteration 0 takes
    // the factor s of X0 = s G here, so that the next product can use G's planes
    Gemm2Args h{};
    h.M = M; h.N = M; h.K = M; h.Z = Z;
    h.a[0] = operand_of(apb(b.tp), np, M); h.b[0] = operand_of(apb(s->apl), np, M);
    h.a[1] = h.b[0]; h.b[1] = h.a[0];
    h.alpha = cc; h.beta = cb; h.cin = b.t32;
    h.pout = apb(b.sp);
    h.spart = first ? s->part : nullptr; h.nspart = s->part_n; h.eps = eps;
    STAGED(TTT_STAGE_NS_BWD, launch_gemm2(h, false, st, true));   // so is S
    // dX_prev = B' dX + S X, the X-side operands read by columns (K = M)
    Gemm2Args u{};
    u.M = M; u.N = N; u.K = M; u.Z = Z;
    u.a[0] = operand_of(apb(s->bpl), np, M); u.b[0] = operand_of(xpb(b.dxp[cur]), np, N);
    u.a[1] = operand_of(apb(b.sp), np, M); u.b[1] = operand_of(xpb(b.xit[it]), np, N);
    u.alpha = 1.f; u.beta = 0.f;
    u.cout = b.dx32[1 - cur];
    if (!first) u.pout = xpb(b.dxp[1 - cur]);
    if (first) { u.gref = b.g32; u.gpart = b.dotpart; }
    STAGED(TTT_STAGE_NS_BWD, launch_gemm2(u, true, st));
    dx32 = b.dx32[1 - cur];
    cur = 1 - cur;
  }
  NsFinArgs f{};
  f.G = b.g32; f.dX = dx32;
  f.ss_part = s->part; f.nss = s->part_n;
  f.dot_part = b.dotpart; f.ndot = gemm2_tiles(M, N);
  f.per = (int64_t)M * N; f.eps = eps;
  f.dG = b.dg32;
  f.pout = pbuf(b.dgp, D.gp, xs, (int64_t)M * N, N);
  STAGED(TTT_STAGE_NS_BWD, launch_ns_fin(f, Z, st));
  return TTT_OK;
}

// The gradient's backward over one block of key rows: the tangent front, then dK, dV, d eta
// and the weight gradients (summed into bw.dwg over the chunk's blocks).
ttt_status grad_bwd_rows(ttt_state* s, const Rows& R, bool first, bool last, void* dk,
                         void* dv, float* deta, hipStream_t st) {
  const Dims& D = s->D;
  const ttt_config& c = s->cfg;
  ttt_state::Bwd& b = s->bw;
  const size_t es = c.act == TTT_BF16 ? 2 : 4;
  const int P = D.P, d = D.d, dh = D.dh, gp = D.gp;
  const int64_t SB = D.sb, Z = (int64_t)D.nm * P, xs = Z * d * D.n;
  const char* k = R.k + R.t0 * d * es;
  const char* v = R.v + R.t0 * d * es;
  const float* eta = R.eta + R.t0;
  auto tok = [&](u16* p, int cols) { return pbuf(p, gp, (int64_t)P * SB * cols, SB * cols, cols); };
  Operand xk, xv;
  if (c.act == TTT_F32) {
    SplitArgs sa{};
    sa.x_zstride = R.T * d; sa.n = R.nr; sa.d = d;
    SplitArgs sv = sa;
    sa.x = k; sa.out = pbuf(s->kpl, D.in_kv, (int64_t)P * SB * d, SB * d, d);
    sv.x = v; sv.out = pbuf(s->vpl, D.in_kv, (int64_t)P * SB * d, SB * d, d);
    STAGED(TTT_STAGE_SPLIT, launch_split2(sa, sv, P, st));
    xk = operand_of(sa.out, D.in_kv, R.nr);
    xv = operand_of(sv.out, D.in_kv, R.nr);
  } else {
    xk = act_operand(k, R.T * d, d, R.nr);
    xv = act_operand(v, R.T * d, d, R.nr);
  }
  auto as_cols = [&](Operand o, int cols) { o.rows = cols; return o; };
  auto wop = [&](int m) {
    return operand_of(pbuf(s->Wpl[m], gp, (int64_t)P * D.rows[m] * D.cols[m],
                           (int64_t)D.rows[m] * D.cols[m], D.cols[m]), gp, D.rows[m]);
  };
  // D_m, the gradient's cotangent, X orientation [d][dh] per (matrix, problem)
  auto dop = [&](int m, int rows) {
    PlaneBuf pb = pbuf(b.dgp + (int64_t)m * P * d * D.n, gp, xs, (int64_t)d * D.n, D.n);
    return operand_of(pb, gp, rows);
  };
  const PlaneBuf pp = tok(s->pk, dh), ppd = tok(b.pd, dh), pa1 = tok(b.a1, dh),
                 pa3 = tok(b.a3, dh), pz1 = tok(s->dz1, dh), pz3 = tok(s->dz3, dh);
  TFrontArgs t{};
  t.A[0] = xk; t.A[1] = xv;
  t.B[0] = wop(0); t.B[1] = wop(1);
  t.B[2] = dop(0, dh); t.B[3] = dop(1, dh);            // read by columns: rows = hidden
  t.B[4] = operand_of(pbuf(s->Wpl[2], gp, (int64_t)P * d * dh, (int64_t)d * dh, dh), gp, dh);
  t.B[5] = dop(2, dh);
  t.eta = eta; t.eta_zstride = R.T;
  t.nrows = R.nr; t.K = d; t.N = dh;
  t.p = pp; t.pd = ppd; t.a1 = pa1; t.a3 = pa3; t.dz1 = pz1; t.dz3 = pz3;
  const int ntn = (dh + 63) / 64;
  t.eta_part = b.eta_part; t.part_zstride = SB * ntn;
  STAGED(TTT_STAGE_TFRONT, launch_tfront(t, P, st));
  EtaSumArgs es_{};
  es_.part = b.eta_part; es_.part_zstride = SB * ntn; es_.nparts = ntn; es_.nrows = R.nr;
  es_.deta = deta + R.t0; es_.deta_zstride = R.T;
  STAGED(TTT_STAGE_TFRONT, launch_eta_sum(es_, P, st));
  // dK = A1 W1 + A3 W3 + dZ1 D1 + dZ3 D3: W by columns, D (X orientation) by rows
  DqArgs kq{};
  kq.a[0] = operand_of(pa1, gp, R.nr); kq.b[0] = as_cols(wop(0), d);
  kq.a[1] = operand_of(pa3, gp, R.nr); kq.b[1] = as_cols(wop(1), d);
  kq.a[2] = operand_of(pz1, gp, R.nr); kq.b[2] = dop(0, d);
  kq.a[3] = operand_of(pz3, gp, R.nr); kq.b[3] = dop(1, d);
  kq.nrows = R.nr; kq.K = dh; kq.N = d;
  kq.out = static_cast<char*>(dk) + R.t0 * d * es; kq.out_zstride = R.T * d;
  kq.out_bf16 = c.act == TTT_BF16;
  STAGED(TTT_STAGE_DQ, launch_rowgemm(kq, 4, P, st));
  // dV = P D2^T + Pd W2^T (-eta J), both by rows
  DqArgs vq{};
  vq.a[0] = operand_of(pp, gp, R.nr); vq.b[0] = dop(2, d);
  vq.a[1] = operand_of(ppd, gp, R.nr); vq.b[1] = wop(2);
  vq.nrows = R.nr; vq.K = dh; vq.N = d;
  vq.out = static_cast<char*>(dv) + R.t0 * d * es; vq.out_zstride = R.T * d;
  vq.out_bf16 = c.act == TTT_BF16;
  STAGED(TTT_STAGE_DQ, launch_rowgemm(vq, 2, P, st));
  // weight gradients: A1^T K, A3^T K, V^T Pd, as the forward's contractions
  ContractArgs ca{};
  ca.P = P; ca.M = d; ca.N = D.n; ca.K = R.nr;
  ca.a[0] = as_cols(xk, d); ca.b[0] = operand_of(pa1, gp, dh);
  ca.a[1] = as_cols(xk, d); ca.b[1] = operand_of(pa3, gp, dh);
  ca.a[2] = as_cols(xv, d); ca.b[2] = operand_of(ppd, gp, dh);
  return contract_all(s, ca, b.dwg, false, first, last, st);
}

ttt_status chunk_backward(ttt_state* s, const void* q, const void* k, const void* v,
                          const float* eta, const void* dout, float* dw, void* dq, void* dk,
                          void* dv, float* deta, hipStream_t st) {
  const ttt_config& c = s->cfg;
  const Dims& D = s->D;
  ttt_status r;
  if ((r = ensure_bwd(s)) != TTT_OK) return r;
  ttt_state::Bwd& b = s->bw;
  const int64_t ch = c.chunk;
  const bool muon = c.ns_steps > 0;
  Rows R0{};
  R0.q = static_cast<const char*>(q);
  R0.k = static_cast<const char*>(k);
  R0.v = static_cast<const char*>(v);
  R0.eta = eta;
  R0.T = ch;
  auto block = [&](int64_t o) {
    Rows R = R0;
    R.t0 = o;
    R.nr = (int)std::min<int64_t>(D.sb, ch - o);
    return R;
  };
  // 1. the chunk's update again: gradient (and G in the X orientation), Newton-Schulz with
  //    its iterates kept, U in the weight orientation
  for (int64_t o = 0; o < ch; o += D.sb)
    if ((r = grad_rows(s, block(o), o == 0, o + D.sb >= ch, st, muon ? b.g32 : nullptr,
                       true)) != TTT_OK)
      return r;
  if (muon && (r = newton_schulz(s, st, b.xit)) != TTT_OK) return r;
  const int64_t sn = weights_numel(D);
  // dout of the step: the cotangent of the state after the chunk, and under the
  // update-then-apply order also the apply step's (its queries saw the updated state)
  const float* dw_after = dw;
  if (c.order == TTT_UPDATE_THEN_APPLY) {
    // 1b. the updated state in place of the state (the apply kernels read the state's
    //     planes), the apply backward with it, then the state before the chunk back
    HIP_TRY(hipMemcpyAsync(b.wbak, s->W, sn * sizeof(float), hipMemcpyDeviceToDevice, st));
    if ((r = refresh_planes(s, true, st)) != TTT_OK) return r;
    for (int64_t o = 0; o < ch; o += D.sb) {
      Rows R = block(o);
      R.v = static_cast<const char*>(dout);
      R.out = static_cast<char*>(dq);
      if ((r = apply_bwd_rows(s, R, o == 0, o + D.sb >= ch, b.dwa, st)) != TTT_OK) return r;
    }
    HIP_TRY(hipMemcpyAsync(s->W, b.wbak, sn * sizeof(float), hipMemcpyDeviceToDevice, st));
    if ((r = refresh_planes(s, false, st)) != TTT_OK) return r;
    Add3Args ad{};
    ad.x = b.dwa; ad.y = dw; ad.out = b.dwa; ad.n = sn;
    STAGED(TTT_STAGE_RENORM, launch_add3(ad, st));
    dw_after = b.dwa;
  }
  // 2. step and renorm: dW_step, and dU in the X orientation
  StepBwdArgs sb{};
  sb.P = D.P; sb.nm = D.nm; sb.renorm = c.row_renorm; sb.keep = 1.f - c.weight_decay;
  int64_t off = 0, xoff = 0;
  for (int m = 0; m < D.nm; ++m) {
    StepBwdMat& M = sb.m[m];
    M.W = s->Wm[m]; M.U = s->Um[m]; M.dout = dw_after + off; M.dw = b.dws + off;
    M.du = b.du + xoff;
    M.rows = D.rows[m]; M.cols = D.cols[m]; M.tr = D.tr[m]; M.lr = c.lr[m];
    sb.max_rows = std::max(sb.max_rows, D.rows[m]);
    off += (int64_t)D.P * D.rows[m] * D.cols[m];
    xoff += (int64_t)D.P * D.d * D.n;
  }
  STAGED(TTT_STAGE_RENORM, launch_step_bwd(sb, st));
  // 3. Newton-Schulz backward (or the plain step's dG = dU), planes for the products.
  //    With momentum the step's input is M' = beta M + g: the cotangent given for the
  //    buffer after the chunk joins dG, which reaches the gradient whole and the buffer
  //    before the chunk (dw's second half, in place) times beta.
  if (muon && (r = ns_backward(s, st)) != TTT_OK) return r;
  float* const dg = muon ? b.dg32 : b.du;
  if (D.mom) {
    MomBwdArgs mb{};
    mb.P = D.P; mb.nm = D.nm; mb.beta = c.momentum;
    int64_t moff = sn, xo = 0;
    for (int m = 0; m < D.nm; ++m) {
      MomBwdMat& M = mb.m[m];
      M.dg = dg + xo; M.dm = dw + moff;
      M.rows = D.rows[m]; M.cols = D.cols[m]; M.tr = D.tr[m];
      moff += (int64_t)D.P * D.rows[m] * D.cols[m];
      xo += (int64_t)D.P * D.d * D.n;
    }
    STAGED(TTT_STAGE_RENORM, launch_mom_bwd(mb, st));
  }
  if (!muon || D.mom) {
    SplitArgs sa{};
    sa.x = dg; sa.x_zstride = (int64_t)D.d * D.n; sa.n = D.d; sa.d = D.n;
    sa.out = pbuf(b.dgp, D.gp, (int64_t)D.nm * D.P * D.d * D.n, (int64_t)D.d * D.n, D.n);
    STAGED(TTT_STAGE_SPLIT, launch_split(sa, D.nm * D.P, st));
  }
  // 4. the gradient's backward per block of key rows
  for (int64_t o = 0; o < ch; o += D.sb)
    if ((r = grad_bwd_rows(s, block(o), o == 0, o + D.sb >= ch, dk, dv, deta, st)) != TTT_OK)
      return r;
  // 5. the apply step (the shifted order answers with the state before the update)
  const bool shifted = c.order == TTT_APPLY_THEN_UPDATE;
  for (int64_t o = 0; shifted && o < ch; o += D.sb) {
    Rows R = block(o);
    R.v = static_cast<const char*>(dout);
    R.out = static_cast<char*>(dq);
    if ((r = apply_bwd_rows(s, R, o == 0, o + D.sb >= ch, b.dwa, st)) != TTT_OK) return r;
  }
  // 6. dW before the chunk (the update-then-apply order's apply part went into the step's
  //    cotangent above)
  Add3Args ad{};
  ad.x = shifted ? b.dwa : b.dws; ad.y = shifted ? b.dws : b.dwg; ad.w = shifted ? b.dwg : nullptr;
  ad.out = dw; ad.n = sn;
  STAGED(TTT_STAGE_RENORM, launch_add3(ad, st));
  return TTT_OK;
}

// Chunks [c0, c1) on the resident path (one launch; every chunk updates).
ttt_status resident_run(ttt_state* s, const void* q, const void* k, const void* v,
                        const float* eta, void* out, int64_t T, int64_t c0, int64_t c1,
                        hipStream_t st) {
  const Dims& D = s->D;
  const int64_t t0 = c0 * s->cfg.chunk;
  SmallArgs a{};
  a.q = static_cast<const u16*>(q) + t0 * D.d;
  a.k = static_cast<const u16*>(k) + t0 * D.d;
  a.v = static_cast<const u16*>(v) + t0 * D.d;
  a.eta = eta + t0;
  a.out = static_cast<u16*>(out) + t0 * D.d;
  a.W1 = s->Wm[0];
  a.W2 = s->Wm[1];
  a.health = s->health;
  a.T = T;
  a.chunk = s->cfg.chunk;
  a.nchunks = (int)(c1 - c0);
  a.P = D.P;
  a.e_scale = s->cfg.lr[1];
  a.dz_scale = s->cfg.lr[0] / s->cfg.lr[1];
  a.keep = 1.f - s->cfg.weight_decay;
  STAGED(TTT_STAGE_RESIDENT, launch_small(a, s->cfg.loss == TTT_LOSS_MSE, st));
  return TTT_OK;
}

// The chunk loop's launches on st.  update: NULL (every chunk updates) or one flag per
// chunk of the call (host memory).
ttt_status forward_body(ttt_state* s, const void* q, const void* k, const void* v,
                        const float* eta, void* out, int64_t T, int64_t nchunks,
                        hipStream_t st, const uint8_t* update) {
  ttt_status r;
  Rows R{};
  R.q = static_cast<const char*>(q);
  R.k = static_cast<const char*>(k);
  R.v = static_cast<const char*>(v);
  R.eta = eta;
  R.out = static_cast<char*>(out);
  R.T = T;
  if (s->resident) {
    // every run of updating chunks in one launch (W updated in place, on chip); a chunk
    // that does not update is answered by the staged apply kernels from planes of W
    for (int64_t c0 = 0; c0 < nchunks;) {
      const bool up = !update || update[c0];
      int64_t c1 = c0 + 1;
      while (c1 < nchunks && (!update || update[c1]) == up) ++c1;
      if (up) {
        if ((r = resident_run(s, q, k, v, eta, out, T, c0, c1, st)) != TTT_OK) return r;
      } else {
        if ((r = refresh_planes(s, false, st)) != TTT_OK) return r;
        for (int64_t ci = c0; ci < c1; ++ci) {
          R.t0 = ci * s->cfg.chunk;
          if ((r = run_chunk(s, R, st, false)) != TTT_OK) return r;
        }
      }
      c0 = c1;
    }
    return TTT_OK;
  }
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    R.t0 = ci * s->cfg.chunk;
    if ((r = run_chunk(s, R, st, !update || update[ci])) != TTT_OK) return r;
  }
  return TTT_OK;
}

ttt_status forward(ttt_state* s, const void* q, const void* k, const void* v, const float* eta,
                   void* out, int64_t T, int64_t nchunks, void* stream,
                   const uint8_t* update = nullptr) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  if (T == 0) return TTT_OK;
  ttt_status r;
  if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v")) ||
      (r = check_ptr(eta, "eta")) || (r = check_ptr(out, "out")))
    return r;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s->last = st;
  if (!s->cfg.replay || s->prof_ev)
    return forward_body(s, q, k, v, eta, out, T, nchunks, st, update);
  ttt_state::GraphKey key{q, k, v, eta, out, T, 0};
  if (update) {
    uint64_t h = 1469598103934665603ull;   // FNV-1a over the flags
    for (int64_t i = 0; i < nchunks; ++i) h = (h ^ (update[i] ? 1u : 0u)) * 1099511628211ull;
    key.flags = h | 1;
  }
  if (s->gexec && key == s->gkey) {
    HIP_TRY(hipGraphLaunch(s->gexec, st));
    return TTT_OK;
  }
  if (!s->cap) HIP_TRY(hipStreamCreateWithFlags(&s->cap, hipStreamNonBlocking));
  HIP_TRY(hipStreamBeginCapture(s->cap, hipStreamCaptureModeThreadLocal));
  r = forward_body(s, q, k, v, eta, out, T, nchunks, s->cap, update);
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(s->cap, &g);
  if (r != TTT_OK) {
    if (g) (void)hipGraphDestroy(g);
    return r;
  }
  if (e != hipSuccess) return fail(TTT_E_HIP, "graph capture failed: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (e != hipSuccess) return fail(TTT_E_HIP, "graph instantiation failed: %s", hipGetErrorString(e));
  if (s->gexec) hipGraphExecDestroy(s->gexec);
  s->gexec = ex;
  s->gkey = key;
  HIP_TRY(hipGraphLaunch(ex, st));
  return TTT_OK;
}

}  // namespace

// ============================================================================ workspace-only runs
namespace ttt {

// A whole sequence with the fp32 state in the caller's buffer w (read, then overwritten
// with the final state) and every workspace buffer carved from ws (ws_bytes long); no
// allocation.  With ws == nullptr only the checks run and *need receives the workspace
// size.  The host checks (configuration, pointers, seq_len, workspace size) all run
// before any HIP call.
ttt_status sequence_in_workspace(const ttt_config* cfg, float* w, const void* q, const void* k,
                                 const void* v, const float* eta, void* out, int64_t seq_len,
                                 char* ws, size_t ws_bytes, size_t* need, void* stream) {
  ttt_config r;
  ttt_status st = resolve(cfg, &r);
  if (st != TTT_OK) return st;
  if ((st = check_ptr(w, "state")) != TTT_OK) return st;
  if (seq_len < 0) return fail(TTT_E_SHAPE, "seq_len is negative");
  if (seq_len % r.chunk)
    return fail(TTT_E_SHAPE, "seq_len %lld is not a multiple of the chunk %d",
                (long long)seq_len, r.chunk);
  if (seq_len > 0 && ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
                      (st = check_ptr(v, "v")) || (st = check_ptr(eta, "eta")) ||
                      (st = check_ptr(out, "out"))))
    return st;
  ttt_state s;
  r.replay = 0;   // a graph would outlive this call's stack state
  s.cfg = r;
  s.D = dims_of(r);
  s.resident = r.path == TTT_PATH_RESIDENT;
  const size_t bytes = layout(&s, nullptr, w);
  if (need) *need = bytes;
  if (bytes > ws_bytes)
    return fail(TTT_E_SHAPE,
                "this configuration needs %zu bytes of workspace; the allocation-free call "
                "holds %zu", bytes, ws_bytes);
  if (!ws) return TTT_OK;
  layout(&s, ws, w);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  s.last = hs;
  // the array keeps the previous call's contents: the health flag is the one buffer read
  // before it is written
  HIP_TRY(launch_fill_zero(s.health, 1, hs));
  if (!s.resident && (st = refresh_planes(&s, false, hs)) != TTT_OK) return st;
  if (seq_len == 0) return TTT_OK;
  return forward(&s, q, k, v, eta, out, seq_len, seq_len / r.chunk, stream);
}

ttt_status report(ttt_status st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace ttt

// ============================================================================ C ABI
extern "C" {

ttt_status ttt_validate_config(const ttt_config* cfg) { return resolve(cfg, nullptr); }

ttt_status ttt_state_numel(const ttt_config* cfg, int64_t* numel) {
  ttt_config r;
  ttt_status st = resolve(cfg, &r);
  if (st != TTT_OK) return st;
  if (!numel) return fail(TTT_E_NULL, "numel is NULL");
  *numel = state_numel(dims_of(r));
  return TTT_OK;
}

ttt_status ttt_init_state(const ttt_config* cfg, const float* w0, void* stream,
                          ttt_state** out) {
  if (!out) return fail(TTT_E_NULL, "out is NULL");
  *out = nullptr;
  ttt_config r;
  ttt_status st = resolve(cfg, &r);
  if (st != TTT_OK) return st;
  if ((st = check_ptr(w0, "w0")) != TTT_OK) return st;
  ttt_state* s = new (std::nothrow) ttt_state();
  if (!s) return fail(TTT_E_ALLOC, "host allocation failed");
  s->cfg = r;
  s->D = dims_of(r);
  s->resident = r.path == TTT_PATH_RESIDENT;
  s->arena_bytes = layout(s, nullptr);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  s->last = hs;
  hipError_t e = hipGetDevice(&s->device);
  if (e == hipSuccess) e = hipMalloc(&s->arena, s->arena_bytes);
  if (e != hipSuccess) {
    ttt_status code = (e == hipErrorOutOfMemory) ? TTT_E_ALLOC : TTT_E_HIP;
    fail(code, "device allocation of %zu bytes failed: %s", s->arena_bytes, hipGetErrorString(e));
    delete s;
    return code;
  }
  layout(s, s->arena);
  auto cleanup = [&](ttt_status code) {
    hipFree(s->arena);
    delete s;
    return code;
  };
  e = hipMemsetAsync(s->arena, 0, s->arena_bytes, hs);
  // broadcast the per-head initial matrices over the batch
  const Dims& D = s->D;
  const float* src = w0;
  for (int m = 0; m < D.nm && e == hipSuccess; ++m) {
    const size_t per_head = (size_t)D.rows[m] * D.cols[m];
    for (int b = 0; b < r.batch && e == hipSuccess; ++b)
      e = hipMemcpyAsync(s->Wm[m] + (size_t)b * r.heads * per_head, src,
                         per_head * r.heads * sizeof(float), hipMemcpyDeviceToDevice, hs);
    src += per_head * r.heads;
  }
  if (e == hipSuccess && s->neg1) {
    std::vector<float> m1((size_t)D.sb, -1.f);
    e = hipMemcpyAsync(s->neg1, m1.data(), m1.size() * sizeof(float), hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);   // m1 is released on return
  }
  if (e != hipSuccess) return cleanup(fail(TTT_E_HIP, "init copy failed: %s", hipGetErrorString(e)));
  st = refresh_planes(s, false, hs);
  if (st != TTT_OK) return cleanup(st);
  *out = s;
  return TTT_OK;
}

ttt_status ttt_chunk_forward(ttt_state* s, const void* q, const void* k, const void* v,
                             const float* eta, void* out, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  return forward(s, q, k, v, eta, out, s->cfg.chunk, 1, stream);
}

ttt_status ttt_apply_backward(ttt_state* s, const void* q, const void* dout, void* dq,
                              float* dw, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  ttt_status r;
  if ((r = check_ptr(q, "q")) || (r = check_ptr(dout, "dout")) || (r = check_ptr(dq, "dq")) ||
      (r = check_ptr(dw, "dw")))
    return r;
  if (s->resident)
    return fail(TTT_E_UNSUPPORTED, "the apply backward needs a state on the staged path");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s->last = st;
  const Dims& D = s->D;
  const int64_t b = s->cfg.chunk;
  for (int64_t o = 0; o < b; o += D.sb) {
    Rows R{};
    R.q = static_cast<const char*>(q);
    R.v = static_cast<const char*>(dout);
    R.out = static_cast<char*>(dq);
    R.T = b;
    R.t0 = o;
    R.nr = (int)std::min<int64_t>(D.sb, b - o);
    if ((r = apply_bwd_rows(s, R, o == 0, o + D.sb >= b, dw, st)) != TTT_OK) return r;
  }
  return TTT_OK;
}

ttt_status ttt_chunk_backward(ttt_state* s, const void* q, const void* k, const void* v,
                              const float* eta, const void* dout, float* dw, void* dq,
                              void* dk, void* dv, float* deta, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  ttt_status r;
  if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v")) ||
      (r = check_ptr(eta, "eta")) || (r = check_ptr(dout, "dout")) || (r = check_ptr(dw, "dw")) ||
      (r = check_ptr(dq, "dq")) || (r = check_ptr(dk, "dk")) || (r = check_ptr(dv, "dv")) ||
      (r = check_ptr(deta, "deta")))
    return r;
  const ttt_config& c = s->cfg;
  if (s->resident || c.fw != TTT_FW_SWIGLU || c.loss != TTT_LOSS_DOT)
    return fail(TTT_E_UNSUPPORTED,
                "the chunk backward serves the SwiGLU net with the inner-product loss, on the "
                "staged path");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s->last = st;
  return chunk_backward(s, q, k, v, eta, dout, dw, dq, dk, dv, deta, st);
}

ttt_status ttt_sequence_forward(ttt_state* s, const void* q, const void* k, const void* v,
                                const float* eta, void* out, int64_t seq_len, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  if (seq_len < 0) return fail(TTT_E_SHAPE, "seq_len is negative");
  if (seq_len % s->cfg.chunk)
    return fail(TTT_E_SHAPE, "seq_len %lld is not a multiple of the chunk %d",
                (long long)seq_len, s->cfg.chunk);
  return forward(s, q, k, v, eta, out, seq_len, seq_len / s->cfg.chunk, stream);
}

ttt_status ttt_sequence_forward_masked(ttt_state* s, const void* q, const void* k,
                                       const void* v, const float* eta, void* out,
                                       int64_t seq_len, const uint8_t* update, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  if (seq_len < 0) return fail(TTT_E_SHAPE, "seq_len is negative");
  if (seq_len % s->cfg.chunk)
    return fail(TTT_E_SHAPE, "seq_len %lld is not a multiple of the chunk %d",
                (long long)seq_len, s->cfg.chunk);
  return forward(s, q, k, v, eta, out, seq_len, seq_len / s->cfg.chunk, stream, update);
}

ttt_status ttt_get_state(const ttt_state* s, float* dst, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  ttt_status st = check_ptr(dst, "dst");
  if (st != TTT_OK) return st;
  HIP_TRY(hipMemcpyAsync(dst, s->W, state_numel(s->D) * sizeof(float), hipMemcpyDeviceToDevice,
                         static_cast<hipStream_t>(stream)));
  return TTT_OK;
}

ttt_status ttt_set_state(ttt_state* s, const float* src, void* stream) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  ttt_status st = check_ptr(src, "src");
  if (st != TTT_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  s->last = hs;
  HIP_TRY(hipMemcpyAsync(s->W, src, state_numel(s->D) * sizeof(float), hipMemcpyDeviceToDevice, hs));
  HIP_TRY(hipMemsetAsync(s->health, 0, sizeof(int), hs));
  return refresh_planes(s, false, hs);
}

ttt_status ttt_state_health(ttt_state* s) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  HIP_TRY(hipStreamSynchronize(s->last));
  int h = 0;
  HIP_TRY(hipMemcpy(&h, s->health, sizeof(int), hipMemcpyDeviceToHost));
  if (h) return fail(TTT_E_NONFINITE, "a NaN or Inf reached the fast-weight state");
  return TTT_OK;
}

ttt_status ttt_destroy_state(ttt_state* s) {
  if (!s) return TTT_OK;
  hipError_t e1 = hipStreamSynchronize(s->last);
  if (s->prof_ev) {
    for (int i = 0; i < 2 * s->prof_cap; ++i) hipEventDestroy(s->prof_ev[i]);
    delete[] s->prof_ev;
  }
  if (s->gexec) hipGraphExecDestroy(s->gexec);
  if (s->cap) hipStreamDestroy(s->cap);
  hipError_t e2 = hipFree(s->arena);
  if (e2 == hipSuccess && s->bw.arena) e2 = hipFree(s->bw.arena);
  delete s;
  if (e1 != hipSuccess) return fail(TTT_E_HIP, "sync before free failed: %s", hipGetErrorString(e1));
  if (e2 != hipSuccess) return fail(TTT_E_HIP, "hipFree failed: %s", hipGetErrorString(e2));
  return TTT_OK;
}

ttt_status ttt_profile_begin(ttt_state* s, int32_t stage, int32_t max_launches) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  if (stage < 0 || stage >= TTT_STAGE_COUNT) return fail(TTT_E_CONFIG, "unknown stage %d", stage);
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(TTT_E_CONFIG, "max_launches must be in [1, 2^20]");
  if (s->prof_ev) return fail(TTT_E_CONFIG, "profiling already active");
  hipEvent_t* ev = new (std::nothrow) hipEvent_t[2 * (size_t)max_launches];
  if (!ev) return fail(TTT_E_ALLOC, "host allocation failed");
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) hipEventDestroy(ev[j]);
      delete[] ev;
      return fail(TTT_E_HIP, "hipEventCreate failed: %s", hipGetErrorString(e));
    }
  }
  s->prof_ev = ev;
  s->prof_cap = max_launches;
  s->prof_n = 0;
  s->prof_stage = stage;
  return TTT_OK;
}

ttt_status ttt_profile_end(ttt_state* s, int64_t* launches, double* total_ms) {
  if (!s) return fail(TTT_E_NULL, "state is NULL");
  if (!s->prof_ev) return fail(TTT_E_CONFIG, "profiling is not active");
  hipError_t e = hipStreamSynchronize(s->last);
  double tot = 0;
  for (int i = 0; i < s->prof_n && e == hipSuccess; ++i) {
    float ms = 0;
    e = hipEventElapsedTime(&ms, s->prof_ev[2 * i], s->prof_ev[2 * i + 1]);
    tot += ms;
  }
  const int n = s->prof_n;
  for (int i = 0; i < 2 * s->prof_cap; ++i) hipEventDestroy(s->prof_ev[i]);
  delete[] s->prof_ev;
  s->prof_ev = nullptr;
  s->prof_stage = -1;
  s->prof_n = s->prof_cap = 0;
  if (e != hipSuccess) return fail(TTT_E_HIP, "event timing failed: %s", hipGetErrorString(e));
  if (launches) *launches = n;
  if (total_ms) *total_ms = tot;
  return TTT_OK;
}

const char* ttt_status_str(int32_t st) {
  switch (st) {
    case TTT_OK: return "ok";
    case TTT_E_NULL: return "null pointer";
    case TTT_E_SHAPE: return "bad shape";
    case TTT_E_DTYPE: return "bad dtype";
    case TTT_E_CONFIG: return "bad configuration";
    case TTT_E_UNSUPPORTED: return "unsupported configuration";
    case TTT_E_ALLOC: return "allocation failed";
    case TTT_E_HIP: return "HIP runtime error";
    case TTT_E_NONFINITE: return "non-finite value in the state";
    case TTT_E_ALIGN: return "misaligned pointer";
  }
  return "unknown status";
}

const char* ttt_last_error(void) { return g_err.c_str(); }

}  // extern "C"
