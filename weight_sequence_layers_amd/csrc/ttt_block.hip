// Kernels of the LaCT block around the TTT layer ([LaCT] §2.1, Fig. 2): window attention,
// the block's projections (an MFMA GEMM with plain, residual and GELU epilogues), RMS
// normalisation with the TTT step-size projection, and the moves between token-major rows
// and the TTT layer's per-head layout.
#include "ttt_block_internal.h"

namespace ttt {
namespace {

// ------------------------------------------------------------------------ window attention
// One workgroup: 4 waves, 128 consecutive queries of one (batch, head), 32 per wave.  The
// keys the window allows for any of them are visited in steps of 64; each step's K and V
// tiles are loaded straight into LDS one step ahead (two stages).  Per step a wave
//   S^T = K Q^T  on the MFMA with K as the A operand, so each lane holds one query
//               (lane % 32) and 16 keys of each 32-key tile: the softmax of a query needs
//               its own 32 values and one exchange with lane ^ 32;
//   O^T += V^T P^T  with the P fragment taken straight from the lane's S values: the
//               contraction runs over keys in an order that pairs each lane's keys with
//               the V rows the transposing LDS read hands the same lane.
// The softmax is online in base 2 (scores scaled by log2(e) / sqrt(128)), fp32, with the
// probabilities rounded to bf16 for the MFMA and summed after rounding.
constexpr int KT_BYTES = ATT_KV * 64 * 2;      // one 64-dim half of a K tile
constexpr int VT_BYTES = ATT_KV * ATT_D * 2;   // a V tile, key rows of 128 dims
constexpr int ATT_STAGE = 2 * KT_BYTES + VT_BYTES;

// A-operand fragment of V^T (32 dims x 16 keys) for the keys key_base + 4 (lane / 32) +
// (0..3) and + 8: element i of lane (dim dim_base + lane % 32) is V[key_base + 4 (lane / 32)
// + (i & 3) + 8 (i >> 2)][dim].  The V tile holds key rows of 128 dims, swizzled as the
// column-layout tile loads store them.
__device__ __forceinline__ bf16x8 read_vt_frag(const char* tile, int dim_base, int key_base) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int m = dim_base + 16 * (g & 1) + 4 * (j & 3);
  const int k0 = key_base + 4 * (g >> 1) + (j >> 2);
  s16x4 lo, hi;
  {
    const char* p = tile + k0 * ATT_D * 2 + (((m >> 3) ^ swz_col<ATT_D>(k0)) << 4) + (m & 7) * 2;
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  }
  {
    const int k = k0 + 8;
    const char* p = tile + k * ATT_D * 2 + (((m >> 3) ^ swz_col<ATT_D>(k)) << 4) + (m & 7) * 2;
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  }
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_window_attention(AttnArgs a) {
  constexpr int NT = 256, QB = ATT_Q;
  __shared__ __attribute__((aligned(1024))) char st0[ATT_STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[ATT_STAGE];
  const int id = xcd_block(blockIdx.x, a.total);
  const int qb = id % a.qblocks, bh = id / a.qblocks;
  const int h = bh % a.heads, b = bh / a.heads;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = a.T, W = a.window;
  const int q0 = qb * QB;
  const int t = q0 + 32 * w + (lane & 31);

  // keys the workgroup visits, and each lane's own window [lo_t, hi_t)
  const int qlast = min(q0 + QB, T) - 1;
  int lo, hi, lo_t, hi_t;
  if (a.mode == TTT_WINDOW_SLIDING) {
    lo = max(0, q0 - W + 1);
    hi = qlast + 1;
    lo_t = t - W + 1;
    hi_t = t + 1;
  } else {
    lo = (q0 / W) * W;
    hi = (int)min<int64_t>(T, ((int64_t)(qlast / W) + 1) * W);
    lo_t = (t / W) * W;
    hi_t = (int)min<int64_t>(T, (int64_t)lo_t + W);
  }
  if (t >= T) lo_t = hi_t = 0;   // padding rows: every key masked, nothing stored
  const int len_t = hi_t - lo_t;
  const int nsteps = (hi - lo + ATT_KV - 1) / ATT_KV;
  // keys [in_lo, in_hi) lie inside the window of every query of this wave: a step wholly in
  // that range needs no mask (empty range for a wave of padding rows)
  int in_lo, in_hi;
  {
    const int w0 = q0 + 32 * w, wl = min(w0 + 31, T - 1);
    if (w0 >= T) {
      in_lo = 1;
      in_hi = 0;
    } else if (a.mode == TTT_WINDOW_SLIDING) {
      in_lo = wl - W + 1;
      in_hi = w0 + 1;
    } else {
      in_lo = (wl / W) * W;
      in_hi = (int)min<int64_t>(T, ((int64_t)(w0 / W) + 1) * W);
    }
  }

  const int64_t row0 = (int64_t)b * T;
  const u16* kb = a.k + row0 * a.ld + (int64_t)h * ATT_D;
  const u16* vb = a.v + row0 * a.ld + (int64_t)h * ATT_D;

  // this lane's query fragments: dims 16 s + 8 (lane / 32) .. + 7 of query t
  bf16x8 qf[8];
  {
    const u16* qr = a.q + (row0 + t) * a.ld + (int64_t)h * ATT_D + 8 * hl;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (t < T) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
      else qf[s] = bf16x8{};
    }
  }

  TileLoad<ATT_KV, NT, 64> lk;
  TileLoad<ATT_D, NT, 64> lv;
  lk.init(make_operand(nullptr, 0, a.ld, 0, 1, ATT_KV), 0, false, 0);
  lv.init(make_operand(nullptr, 0, a.ld, 0, 1, ATT_D), 0, true, 0);
  // keys at or past the end of the sequence lie past the resource's end and load as 0
  auto issue = [&](char* st, int kv0) __attribute__((always_inline)) {
    const uint32_t nrec = (uint32_t)min(T - kv0, ATT_KV) * (uint32_t)(a.ld * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kb + (int64_t)kv0 * a.ld), (short)0, (int)nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vb + (int64_t)kv0 * a.ld), (short)0, (int)nrec, 0x00020000);
#pragma unroll
    for (int c = 0; c < lk.C; ++c) {
      dma16(rk, (lds_void_t*)(st + c * NT * 16 + lk.slice), lk.off[c]);
      dma16(rk, (lds_void_t*)(st + KT_BYTES + c * NT * 16 + lk.slice), lk.off[c] + 128);
    }
#pragma unroll
    for (int c = 0; c < lv.C; ++c)
      dma16(rv, (lds_void_t*)(st + 2 * KT_BYTES + c * NT * 16 + lv.slice), lv.off[c]);
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (nsteps > 0) issue(st0, lo);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < nsteps; ++i) {
    char* cur = (i & 1) ? st1 : st0;
    char* nxt = (i & 1) ? st0 : st1;
    const int kv0 = lo + i * ATT_KV;
    if (i + 1 < nsteps) issue(nxt, kv0 + ATT_KV);

    f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const char* kh = cur + (s >> 2) * KT_BYTES;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            read_frag<false, ATT_KV, 64>(kh, 32 * kt, s & 3), qf[s], sc[kt], 0, 0, 0);
    }
    // element v of tile kt: key kv0 + 32 kt + 8 (v / 4) + 4 (lane / 32) + v % 4.  Scores
    // stay unscaled until the exponent: the scale is positive, so the maximum is taken on
    // raw scores and p = exp2(s scale2 - m) is one fused multiply-add and one exp2.
    if (kv0 < in_lo || kv0 + ATT_KV > in_hi) {   // wave-uniform: a window edge in this step
      const int base = kv0 + 4 * hl - lo_t;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int dk = base + 32 * kt + 8 * (v >> 2) + (v & 3);
          if ((unsigned)dk >= (unsigned)len_t) sc[kt][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale2;
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    if (__any(mnew != m)) {   // wave-uniform: some running maximum moved
      const float alpha = __builtin_amdgcn_exp2f(m - mref);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[d][v] *= alpha;
    }
    m = mnew;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 p = static_cast<__bf16>(
              __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * sp + e], a.scale2, -mref)));
          pf[e] = p;
          l += static_cast<float>(p);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_vt_frag(cur + 2 * KT_BYTES, 32 * d, 32 * kt + 16 * sp), pf, o[d], 0, 0, 0);
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // element v of o[d]: dim 32 d + 8 (v / 4) + 4 (lane / 32) + v % 4 of query t
  const float lt = l + __shfl_xor(l, 32);
  if (t < T) {
    const float inv = 1.f / lt;
    u16* orow = a.out + (row0 + t) * a.ldo + (int64_t)h * ATT_D + 4 * hl;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 wv;
        wv.x = f2bf(o[d][4 * g] * inv) | ((uint32_t)f2bf(o[d][4 * g + 1] * inv) << 16);
        wv.y = f2bf(o[d][4 * g + 2] * inv) | ((uint32_t)f2bf(o[d][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * d + 8 * g) = wv;
      }
  }
}

// ------------------------------------------------------------------------ projections
// y = epilogue(x w^T): 128 x 128 tiles of rows x output features, 4 waves of 64 x 64,
// K (input features) in steps of 64 through two LDS stages.  The tile's rows and weight
// rows are addressed from the tile's origin, so offsets stay within 32 bits for any
// number of rows.
//
// Tile order: each XCD runs a contiguous range of tiles (xcd_block), and within it the
// tiles go in groups of group_m row tiles that walk the output features together, row
// tile fastest: the workgroups resident on an XCD at one time then read a few row panels
// and a few weight panels, each from its L2 several times, instead of one row panel and
// a stream through the whole weight matrix (larger than an XCD's L2 for the block's
// widths).  Groups of 8 row tiles, against one row tile at a time, at the LM block's
// shapes (warm, interleaved, normally distributed data): q/k/v 809 -> 913, MLP up 690 ->
// 790, MLP down 866 -> 925 TFLOP/s; the 1024-wide output projection unchanged.
using GL = Gemm<128, 128, 2, 2, 1, 1, L_ROW, L_ROW, 0, 64, true>;

// GELU(x) = x Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2, erfc from the Chebyshev fit of
// Numerical Recipes (erfcc, fractional error below 1.2e-7 for every argument), so the
// function has no branches: t = 1 / (1 + z / 2), erfc(z) = t exp(-z^2 + P(t)), z = |x| /
// sqrt 2, and erfc(-z) = 2 - erfc(z).
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.f + 0.5f * z);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float ec = t * __builtin_amdgcn_exp2f((p - z * z) * 1.44269504088896341f);
  const float phi = x >= 0.f ? 1.f - 0.5f * ec : 0.5f * ec;
  return x * phi;
}

// Two workgroups fit a CU's LDS; the register budget is held to the same two waves per SIMD
// (the GELU epilogue alone would take more).
template <int EPI>
__global__ __launch_bounds__(GL::NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_blk_linear(LinearArgs a) {
  GEMM_LDS(GL);
  const int id = xcd_block(blockIdx.x, (int)a.tiles);
  // group of group_m row tiles (the last group may be shorter), row tile fastest
  const int gsz = a.group_m * a.tiles_n;
  const int grp = id / gsz, in = id - grp * gsz;
  const int gm = min(a.group_m, a.tiles_m - grp * a.group_m);
  const int tm = grp * a.group_m + in % gm, tn = in / gm;
  const int64_t m0 = (int64_t)tm * GL::TBM;
  const int n0 = tn * GL::TBN;
  const int rl = (int)min<int64_t>(GL::TBM, a.rows - m0), cl = min(GL::TBN, a.N - n0);
  const Operand A = make_operand(a.x + m0 * a.K, 0, a.K, 0, 1, rl);
  const Operand B = make_operand(a.w + (int64_t)n0 * a.K, 0, a.K, 0, 1, cl);
  GL g;
  g.zero();
  g.run(&A, &B, 0, 0, 0, a.K, GEMM_STAGES);
  if constexpr (EPI == TTT_LINEAR_GELU) {
    g.for_each([&](int i, int j, int v, int, int) __attribute__((always_inline)) {
      g.acc[0][i][j][v] = gelu_erf(g.acc[0][i][j][v]);
    });
  }
  if constexpr (EPI == TTT_LINEAR_RESIDUAL) {
    // four consecutive output features of one row per run; the output width is a multiple
    // of 8, so a run is inside the matrix whenever its first column is
    g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
      if (r < rl && c < cl) {
        const uint2 rv = *reinterpret_cast<const uint2*>(a.resid + (m0 + r) * a.N + n0 + c);
        g.acc[0][i][j][4 * q] += bf2f(rv.x & 0xffffu);
        g.acc[0][i][j][4 * q + 1] += bf2f(rv.x >> 16);
        g.acc[0][i][j][4 * q + 2] += bf2f(rv.y & 0xffffu);
        g.acc[0][i][j][4 * q + 3] += bf2f(rv.y >> 16);
      }
    });
  }
  PlaneBuf o;
  o.base = a.y + m0 * a.N;
  o.plane_stride = 0;
  o.zstride = 0;
  o.ld = a.N;
  o.np = 1;
  store_tile_planes<GL, TILE_NORMAL>(g.acc[0], smem, o, 0, 0, n0, rl, cl);
}

// The same on 256 x 256 tiles, sixteen waves of 64 x 64, for launches with many such tiles
// and a long K loop: four times the MFMA work per K step for the same per-step cost.  The
// two stages take 128 KB of LDS, so the tile is not staged for the store: each lane writes
// its runs of four output features as 8-byte stores (the same rounding as the staged
// store).  In the block (interleaved runs against the 128 x 128 kernel) the MLP down
// projection (4096 or 3072 input features) goes 1.19 -> 1.03 ms at the LM shape and
// 5.85 -> 5.15 ms at the image set's; the 1024-feature projections gain nothing (the
// unstaged store costs what the longer steps save), so they keep the 128 x 128 tiles.
using GLW = Gemm<256, 256, 4, 4, 1, 1, L_ROW, L_ROW, 0, 64, true>;

template <int EPI>
__global__ __launch_bounds__(GLW::NT) void k_blk_linear_wide(LinearArgs a) {
  GEMM_LDS_EPI(GLW, 0);
  const int id = xcd_block(blockIdx.x, (int)a.tiles);
  const int gsz = a.group_m * a.tiles_n;
  const int grp = id / gsz, in = id - grp * gsz;
  const int gm = min(a.group_m, a.tiles_m - grp * a.group_m);
  const int tm = grp * a.group_m + in % gm, tn = in / gm;
  const int64_t m0 = (int64_t)tm * GLW::TBM;
  const int n0 = tn * GLW::TBN;
  const int rl = (int)min<int64_t>(GLW::TBM, a.rows - m0), cl = min(GLW::TBN, a.N - n0);
  const Operand A = make_operand(a.x + m0 * a.K, 0, a.K, 0, 1, rl);
  const Operand B = make_operand(a.w + (int64_t)n0 * a.K, 0, a.K, 0, 1, cl);
  GLW g;
  g.zero();
  g.run(&A, &B, 0, 0, 0, a.K, GEMM_STAGES);
  // runs of four consecutive output features of one row; the output width is a multiple
  // of 8, so a run is inside the matrix whenever its first column is
  g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
    if (r < rl && c < cl) {
      const int64_t off = (m0 + r) * a.N + n0 + c;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = g.acc[0][i][j][4 * q + e];
        if constexpr (EPI == TTT_LINEAR_GELU) x[e] = gelu_erf(x[e]);
      }
      if constexpr (EPI == TTT_LINEAR_RESIDUAL) {
        const uint2 rv = *reinterpret_cast<const uint2*>(a.resid + off);
        x[0] += bf2f(rv.x & 0xffffu);
        x[1] += bf2f(rv.x >> 16);
        x[2] += bf2f(rv.y & 0xffffu);
        x[3] += bf2f(rv.y >> 16);
      }
      u16 h[4][3];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_planes(x[e], 1, h[e]);
      *reinterpret_cast<uint2*>(a.y + off) =
          make_uint2(h[0][0] | ((uint32_t)h[1][0] << 16), h[2][0] | ((uint32_t)h[3][0] << 16));
    }
  });
}

// ------------------------------------------------------------------------ RMS norm
// One wave per row: the sum of squares, then the normalised row rounded to bf16 and, for
// the TTT sub-layer, its dot product with each head's step-size weights.
__global__ __launch_bounds__(256) void k_blk_rmsnorm(RmsArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const u16* x = a.x + row * a.D;
  u16* y = a.y + row * a.D;
  float ss = 0.f;
  for (int c = 4 * lane; c < a.D; c += 256) {
    const uint2 w = *reinterpret_cast<const uint2*>(x + c);
    const float f0 = bf2f(w.x & 0xffffu), f1 = bf2f(w.x >> 16);
    const float f2 = bf2f(w.y & 0xffffu), f3 = bf2f(w.y >> 16);
    ss += f0 * f0 + f1 * f1 + f2 * f2 + f3 * f3;
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)a.D + 1e-6f);
  float dots[BLK_MAX_TTT_HEADS];
#pragma unroll
  for (int h = 0; h < BLK_MAX_TTT_HEADS; ++h) dots[h] = 0.f;
  for (int c = 4 * lane; c < a.D; c += 256) {
    const uint2 w = *reinterpret_cast<const uint2*>(x + c);
    const u16 y0 = f2bf(bf2f(w.x & 0xffffu) * r), y1 = f2bf(bf2f(w.x >> 16) * r);
    const u16 y2 = f2bf(bf2f(w.y & 0xffffu) * r), y3 = f2bf(bf2f(w.y >> 16) * r);
    uint2 o;
    o.x = y0 | ((uint32_t)y1 << 16);
    o.y = y2 | ((uint32_t)y3 << 16);
    *reinterpret_cast<uint2*>(y + c) = o;
    if (a.w_eta) {
#pragma unroll
      for (int h = 0; h < BLK_MAX_TTT_HEADS; ++h)
        if (h < a.heads) {
          const uint2 e = *reinterpret_cast<const uint2*>(a.w_eta + (int64_t)h * a.D + c);
          dots[h] += bf2f(y0) * bf2f(e.x & 0xffffu) + bf2f(y1) * bf2f(e.x >> 16) +
                     bf2f(y2) * bf2f(e.y & 0xffffu) + bf2f(y3) * bf2f(e.y >> 16);
        }
    }
  }
  if (a.w_eta) {
    const int64_t bb = row / a.T, tt = row % a.T;
#pragma unroll
    for (int h = 0; h < BLK_MAX_TTT_HEADS; ++h)
      if (h < a.heads) {
        const float z = wave_sum(dots[h]);
        if (lane == 0) a.eta[(bb * a.heads + h) * a.T + tt] = 0.01f / (1.f + expf(-z));
      }
  }
}

// ------------------------------------------------------------------------ head moves
// One wave per (row, TTT head): q and k scaled to unit length (fp32 norms), v copied.
__global__ __launch_bounds__(256) void k_blk_split(HeadSplitArgs a) {
  const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.T;
  if (id >= rows * a.H) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = id / a.H;
  const int h = (int)(id % a.H);
  const int64_t bb = row / a.T, tt = row % a.T;
  const int D = a.H * a.d;
  const u16* src = a.qkv + row * 3 * D + (int64_t)h * a.d;
  const int64_t dst = ((bb * a.H + h) * a.T + tt) * a.d;
  uint2 qv[4], kv[4];
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < a.d) {
      qv[i] = *reinterpret_cast<const uint2*>(src + c);
      kv[i] = *reinterpret_cast<const uint2*>(src + D + c);
      const float q0 = bf2f(qv[i].x & 0xffffu), q1 = bf2f(qv[i].x >> 16);
      const float q2 = bf2f(qv[i].y & 0xffffu), q3 = bf2f(qv[i].y >> 16);
      const float k0 = bf2f(kv[i].x & 0xffffu), k1 = bf2f(kv[i].x >> 16);
      const float k2 = bf2f(kv[i].y & 0xffffu), k3 = bf2f(kv[i].y >> 16);
      sq += q0 * q0 + q1 * q1 + q2 * q2 + q3 * q3;
      sk += k0 * k0 + k1 * k1 + k2 * k2 + k3 * k3;
    }
  }
  const float iq = 1.f / sqrtf(wave_sum(sq)), ik = 1.f / sqrtf(wave_sum(sk));
  auto scale = [](uint2 x, float s) __attribute__((always_inline)) {
    uint2 o;
    o.x = f2bf(bf2f(x.x & 0xffffu) * s) | ((uint32_t)f2bf(bf2f(x.x >> 16) * s) << 16);
    o.y = f2bf(bf2f(x.y & 0xffffu) * s) | ((uint32_t)f2bf(bf2f(x.y >> 16) * s) << 16);
    return o;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * (lane + 64 * i);
    if (c < a.d) {
      *reinterpret_cast<uint2*>(a.q + dst + c) = scale(qv[i], iq);
      *reinterpret_cast<uint2*>(a.k + dst + c) = scale(kv[i], ik);
      *reinterpret_cast<uint2*>(a.v + dst + c) =
          *reinterpret_cast<const uint2*>(src + 2 * D + c);
    }
  }
}

// One thread per 8 outputs: [B][H][T][d] -> [B T][H d].
__global__ __launch_bounds__(256) void k_blk_merge(HeadMergeArgs a) {
  const int D = a.H * a.d;
  const int64_t total = (int64_t)a.B * a.T * D / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t e = i * 8, row = e / D;
  const int col = (int)(e % D), h = col / a.d, dd = col % a.d;
  const int64_t bb = row / a.T, tt = row % a.T;
  *reinterpret_cast<uint4*>(a.y + e) =
      *reinterpret_cast<const uint4*>(a.o + ((bb * a.H + h) * a.T + tt) * a.d + dd);
}

}  // namespace

hipError_t launch_window_attention(const AttnArgs& a, hipStream_t st) {
  if (a.total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_window_attention, dim3(a.total), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_linear(const LinearArgs& a, int epilogue, hipStream_t st) {
  if (a.tiles == 0) return hipSuccess;
  if (a.tile == GLW::TBM) {
    const dim3 grid((unsigned)a.tiles), block(GLW::NT);
    if (epilogue == TTT_LINEAR_RESIDUAL)
      hipLaunchKernelGGL(k_blk_linear_wide<TTT_LINEAR_RESIDUAL>, grid, block, 0, st, a);
    else if (epilogue == TTT_LINEAR_GELU)
      hipLaunchKernelGGL(k_blk_linear_wide<TTT_LINEAR_GELU>, grid, block, 0, st, a);
    else
      hipLaunchKernelGGL(k_blk_linear_wide<TTT_LINEAR_PLAIN>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.tile != GL::TBM) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.tiles), block(GL::NT);
  if (epilogue == TTT_LINEAR_RESIDUAL)
    hipLaunchKernelGGL(k_blk_linear<TTT_LINEAR_RESIDUAL>, grid, block, 0, st, a);
  else if (epilogue == TTT_LINEAR_GELU)
    hipLaunchKernelGGL(k_blk_linear<TTT_LINEAR_GELU>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(k_blk_linear<TTT_LINEAR_PLAIN>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const RmsArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_blk_rmsnorm, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_split(const HeadSplitArgs& a, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.T * a.H;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(k_blk_split, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge(const HeadMergeArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.T * a.H * a.d / 8;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_blk_merge, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ttt
