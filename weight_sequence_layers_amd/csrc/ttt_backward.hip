// HIP kernels of the backward through one chunk's fast-weight update (gfx950).
//
// The outer loop of the second TTT-E2E page (intelliparadigm.com, §2.2) trains through the
// inner updates; §5.1 of the same page names the second-order gradients this takes.  For a
// cotangent on the state after a chunk, the chain runs back through the row renorm and the
// step (k_step_bwd), through Muon's Newton-Schulz iteration (k_gemm2 per iteration, then
// k_ns_fin for the Frobenius scaling), and through the chunk gradient itself: k_tfront
// forms the forward-mode tangents of the net along the gradient's cotangent together with
// the per-token second-order terms, k_rowgemm the key and value gradients, and the token
// contractions of ttt_kernels.hip the weight gradients.
#include <math.h>

#include <algorithm>

#include "ttt_internal.h"

namespace ttt {

namespace {

// logistic function with the hardware reciprocal (as the forward kernels)
__device__ __forceinline__ float sigm_b(float z) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

}  // namespace

// ------------------------------------------------------------------------ tangent front
// Products (tile rows = tokens, columns = hidden units): 0 Z1 = K W1^T, 1 Z3 = K W3^T,
// 2 Zd1 = K D1^T, 3 Zd3 = K D3^T (K for all four), 4 V W2, 5 V D2 (V).  Per element, with
// s = sigmoid(Z1), silu = Z1 s, silu' = s (1 + Z1 (1 - s)), silu'' = s (1 - s)(2 + Z1 (1 - 2 s)):
//   H = silu Z3,  Hd = silu' Zd1 Z3 + silu Zd3            (the net's hidden and its tangent)
//   Dl = -eta (V W2),  G2 = -eta (V D2)                    (W2^T e and D2^T e, e = -eta v)
//   A1 = G2 silu' Z3 + Dl (silu'' Zd1 Z3 + silu' Zd3),  A3 = G2 silu + Dl silu' Zd1
//   dZ1 = Dl silu' Z3,  dZ3 = Dl silu
// stored as planes of -eta H, -eta Hd, A1, A3, dZ1 and dZ3; and each row's share of
// d eta = -sum_h ((V D2) H + (V W2) Hd) over the tile's columns.
template <int BM, int BN, int WGM, int WGN, int BK>
__global__ __launch_bounds__(WGM * WGN * 64) void k_tfront(TFrontArgs a) {
  using G = Gemm<BM, BN, WGM, WGN, 2, 6, 0, 0b111100, 0, BK, true, 1, 4>;
  GEMM_LDS(G);
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int z = lid / a.tiles, tile = lid % a.tiles;
  const int tn_ = tile % a.tiles_n;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = tn_ * BN;

  G g;
  g.zero();
  g.run(a.A, a.B, m0, n0, z, a.K, GEMM_STAGES);

  const float* eta = a.eta + (int64_t)z * a.eta_zstride;
  float rs[G::TM];
#pragma unroll
  for (int i = 0; i < G::TM; ++i) rs[i] = 0.f;
  g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
    const int row = m0 + r;
    const float e = row < a.nrows ? eta[row] : 0.f;
    const float z1 = g.acc[0][i][j][v], z3 = g.acc[1][i][j][v];
    const float zd1 = g.acc[2][i][j][v], zd3 = g.acc[3][i][j][v];
    const float vw2 = g.acc[4][i][j][v], vd2 = g.acc[5][i][j][v];
    const float s = sigm_b(z1);
    const float sl = z1 * s;
    const float s1 = s * (1.f + z1 * (1.f - s));
    const float s2 = s * (1.f - s) * (2.f + z1 * (1.f - 2.f * s));
    const float h = sl * z3;
    const float hd = s1 * zd1 * z3 + sl * zd3;
    const float dl = -e * vw2, g2 = -e * vd2;
    g.acc[0][i][j][v] = -e * h;
    g.acc[1][i][j][v] = -e * hd;
    g.acc[2][i][j][v] = g2 * s1 * z3 + dl * (s2 * zd1 * z3 + s1 * zd3);
    g.acc[3][i][j][v] = g2 * sl + dl * s1 * zd1;
    g.acc[4][i][j][v] = dl * s1 * z3;
    g.acc[5][i][j][v] = dl * sl;
    rs[i] -= vd2 * h + vw2 * hd;
  });
  const int cl = min(BN, a.N - n0);
  const int rn = min(BM, a.nrows - m0);
  store_planes<G, TILE_NORMAL, 1>(g.acc[0], smem, a.p, z, m0, n0, rn, cl);
  store_planes<G, TILE_NORMAL, 1>(g.acc[1], smem, a.pd, z, m0, n0, rn, cl);
  store_planes<G, TILE_NORMAL, 1>(g.acc[2], smem, a.a1, z, m0, n0, rn, cl);
  store_planes<G, TILE_NORMAL, 1>(g.acc[3], smem, a.a3, z, m0, n0, rn, cl);
  store_planes<G, TILE_NORMAL, 1>(g.acc[4], smem, a.dz1, z, m0, n0, rn, cl);
  store_planes<G, TILE_NORMAL, 1>(g.acc[5], smem, a.dz3, z, m0, n0, rn, cl);
  // the eta shares: a row's elements sit in lanes l and l + 32 of the waves of one wave
  // row (swapped layout), summed here in a fixed order
  float* red = reinterpret_cast<float*>(smem);   // [WGN][BM]
  const int lane = threadIdx.x & 63;
  const int wmn = (int)(threadIdx.x >> 6);
  const int wn = wmn % WGN, wm0 = (wmn / WGN) * (BM / WGM);
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
    const float t = rs[i] + __shfl_xor(rs[i], 32, 64);
    if (lane < 32) red[wn * BM + wm0 + i * 32 + lane] = t;
  }
  lds_barrier();
  for (int r = threadIdx.x; r < BM; r += G::NT) {
    float t = 0.f;
    for (int w = 0; w < WGN; ++w) t += red[w * BM + r];
    if (m0 + r < a.nrows)
      a.eta_part[(int64_t)z * a.part_zstride + (int64_t)(m0 + r) * a.tiles_n + tn_] = t;
  }
}

__global__ __launch_bounds__(256) void k_eta_sum(EtaSumArgs a) {
  const int z = blockIdx.y;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < a.nrows; t += gridDim.x * 256) {
    const float* p = a.part + (int64_t)z * a.part_zstride + (int64_t)t * a.nparts;
    float s = 0.f;
    for (int j = 0; j < a.nparts; ++j) s += p[j];
    a.deta[(int64_t)z * a.deta_zstride + t] = s;
  }
}

// ------------------------------------------------------------------------ dK and dV
// out = sum over NP pairs of A_m B_m^T, all products in one accumulator; B_m read by
// columns where bit m of LBM is set.  Stored in the activation dtype.
template <int BM, int BN, int WGM, int WGN, int NP, int LBM>
__global__ __launch_bounds__(WGM * WGN * 64) void k_rowgemm(DqArgs a) {
  using G = Gemm<BM, BN, WGM, WGN, NP, NP, 0, LBM, 0, 32, true, 1, -1, true>;
  GEMM_LDS(G);
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int z = lid / a.tiles, tile = lid % a.tiles;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;
  G g;
  g.zero();
  g.run(a.a, a.b, m0, n0, z, a.K, GEMM_STAGES);
  const int cl = min(BN, a.N - n0);
  const int rn = min(BM, a.nrows - m0);
  if (a.out_bf16) {
    PlaneBuf o;
    o.base = static_cast<u16*>(a.out); o.plane_stride = 0; o.zstride = a.out_zstride;
    o.ld = a.N; o.np = 1;
    store_tile_planes<G, TILE_NORMAL>(g.acc[0], smem, o, z, m0, n0, rn, cl);
  } else {
    g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
      const int row = m0 + r, col = n0 + c;
      if (row < a.nrows && col < a.N)
        static_cast<float*>(a.out)[(int64_t)z * a.out_zstride + (int64_t)row * a.N + col] =
            g.acc[0][i][j][v];
    });
  }
}

// ------------------------------------------------------------------------ step and renorm
// One wave per row (rows of all problems flattened), the row's W, U and cotangent held in
// registers (CPL 16-byte chunks per lane).
template <int CPL>
__global__ __launch_bounds__(256) void k_step_bwd(StepBwdArgs a) {
  const StepBwdMat& M = a.m[blockIdx.y];
  const int lane = threadIdx.x & 63;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gr >= M.rows * a.P) return;
  const int n4 = M.cols / 4;
  const int64_t ro = (int64_t)gr * M.cols;
  const float4* w4 = reinterpret_cast<const float4*>(M.W + ro);
  const float4* u4 = reinterpret_cast<const float4*>(M.U + ro);
  const float4* d4 = reinterpret_cast<const float4*>(M.dout + ro);
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 w[CPL], y[CPL], d[CPL];
  float so = 0.f, sn = 0.f, sp = 0.f;
  const float keep = a.keep, lr = M.lr;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int i = lane + 64 * k;
    w[k] = i < n4 ? w4[i] : zero;
    const float4 u = i < n4 ? u4[i] : zero;
    d[k] = i < n4 ? d4[i] : zero;
    y[k] = make_float4(fmaf(-lr, u.x, keep * w[k].x), fmaf(-lr, u.y, keep * w[k].y),
                       fmaf(-lr, u.z, keep * w[k].z), fmaf(-lr, u.w, keep * w[k].w));
    so += w[k].x * w[k].x + w[k].y * w[k].y + w[k].z * w[k].z + w[k].w * w[k].w;
    sn += y[k].x * y[k].x + y[k].y * y[k].y + y[k].z * y[k].z + y[k].w * y[k].w;
    sp += y[k].x * d[k].x + y[k].y * d[k].y + y[k].z * d[k].z + y[k].w * d[k].w;
  }
  so = wave_sum(so);
  sn = wave_sum(sn);
  sp = wave_sum(sp);
  // renorm: out = y |w| / |y|;  dY = |w|/|y| (dout - yh <yh, dout>),  dW_ref = <yh, dout> w / |w|
  float cy = 1.f, cproj = 0.f, cw = 0.f;
  if (a.renorm && sn > 0.f) {
    const float nw = sqrtf(so), ny = sqrtf(sn);
    cy = nw / ny;
    cproj = cy * sp / sn;                 // coefficient of y in dY
    cw = nw > 0.f ? sp / (ny * nw) : 0.f; // coefficient of w in dW_ref
  }
  float4* dw4 = reinterpret_cast<float4*>(M.dw + ro);
  const int p = gr / M.rows, r = gr % M.rows;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int i = lane + 64 * k;
    if (i >= n4) continue;
    const float4 dy = make_float4(cy * d[k].x - cproj * y[k].x, cy * d[k].y - cproj * y[k].y,
                                  cy * d[k].z - cproj * y[k].z, cy * d[k].w - cproj * y[k].w);
    dw4[i] = make_float4(fmaf(keep, dy.x, cw * w[k].x), fmaf(keep, dy.y, cw * w[k].y),
                         fmaf(keep, dy.z, cw * w[k].z), fmaf(keep, dy.w, cw * w[k].w));
    const float du[4] = {-lr * dy.x, -lr * dy.y, -lr * dy.z, -lr * dy.w};
    if (M.tr) {
      // X orientation [cols][rows] per problem
      float* base = M.du + (int64_t)p * M.rows * M.cols;
#pragma unroll
      for (int e = 0; e < 4; ++e) base[(int64_t)(4 * i + e) * M.rows + r] = du[e];
    } else {
      reinterpret_cast<float4*>(M.du + ro)[i] = make_float4(du[0], du[1], du[2], du[3]);
    }
  }
}

// ------------------------------------------------------------------------ Newton-Schulz
// out = sc (alpha (A0 B0^T + A1 B1^T) + beta cin), sc the optional per-matrix scale; B
// operands read by rows (LBM 0) or columns.
// SYM: the output is symmetric (M = N): only the upper tiles run, and each off-diagonal
// tile's planes are stored with their mirror (the fp32 output, read back only where the
// upper tiles lie, is stored as computed).
template <int BM, int BN, int WGM, int WGN, int LBM, bool SYM = false>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm2(Gemm2Args a) {
  using G = Gemm<BM, BN, WGM, WGN, 2, 2, 0, LBM, 0, 32, true, 1, -1, true>;
  static_assert(!SYM || BM == BN, "symmetric outputs take square tiles");
  GEMM_LDS_EPI(G, (SYM ? store_lds_bytes<G, TILE_BOTH, 1>() : G::STORE_LDS));
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int zz = lid / a.tiles, tile = lid % a.tiles;
  const int M = a.M, N = a.N;
  int ti, tj;
  if (SYM) tri_tile(tile, (M + BM - 1) / BM, ti, tj);
  else {
    ti = tile / a.tiles_n;
    tj = tile % a.tiles_n;
  }
  const int m0 = ti * BM;
  const int n0 = tj * BN;
  G g;
  g.zero();
  g.run(a.a, a.b, m0, n0, zz, a.K, GEMM_STAGES);
  const int64_t base = (int64_t)zz * M * N;
  float sc = 1.f;
  if (a.spart) {
    sc = 1.f / (sqrtf(sum_parts(a.spart + (int64_t)zz * a.nspart, a.nspart)) + a.eps);
  }
  const float alpha = a.alpha * sc, beta = a.beta * sc;
  float gs = 0.f;
  g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
    const int R = m0 + r, C = n0 + c;
    const bool in = R < M && C < N;   // N is a multiple of 16: a run is wholly in or out
    float4 ci = make_float4(0.f, 0.f, 0.f, 0.f);
    if (in && a.cin) ci = *reinterpret_cast<const float4*>(a.cin + base + (int64_t)R * N + C);
    const float cv[4] = {ci.x, ci.y, ci.z, ci.w};
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = in ? fmaf(alpha, g.acc[0][i][j][4 * q + e], beta * cv[e]) : 0.f;
      g.acc[0][i][j][4 * q + e] = x[e];
    }
    if (in && a.cout)
      *reinterpret_cast<float4*>(a.cout + base + (int64_t)R * N + C) =
          make_float4(x[0], x[1], x[2], x[3]);
    if (in && a.gref) {
      const float4 gr = *reinterpret_cast<const float4*>(a.gref + base + (int64_t)R * N + C);
      gs += x[0] * gr.x + x[1] * gr.y + x[2] * gr.z + x[3] * gr.w;
    }
  });
  if (a.pout.np > 0) {
    const int rl = min(BM, M - m0), cl = min(BN, N - n0);
    if (SYM && ti != tj)
      store_planes<G, TILE_BOTH, 1>(g.acc[0], smem, a.pout, zz, m0, n0, rl, cl);
    else
      store_tile_planes<G, TILE_NORMAL>(g.acc[0], smem, a.pout, zz, m0, n0, rl, cl);
  }
  if (a.gpart) {
    const float t = block_sum(gs, reinterpret_cast<float*>(smem));
    if (threadIdx.x == 0) a.gpart[(int64_t)zz * a.tiles + tile] = t;
  }
}

// dG = dX0 s - G <G, dX0> s^2 / |G|_F with s = 1 / (|G|_F + eps); runs of 8 values a thread.
__global__ __launch_bounds__(256) void k_ns_fin(NsFinArgs a) {
  const int zz = blockIdx.y;
  float ss = 0.f, dot = 0.f;
  ss = sum_parts(a.ss_part + (int64_t)zz * a.nss, a.nss);
  for (int i = 0; i < a.ndot; ++i) dot += a.dot_part[(int64_t)zz * a.ndot + i];
  const float nrm = sqrtf(ss);
  const float s = 1.f / (nrm + a.eps);
  const float cg = nrm > 0.f ? dot * s * s / nrm : 0.f;
  const int64_t base = (int64_t)zz * a.per;
  for (int64_t e8 = (int64_t)blockIdx.x * 256 + threadIdx.x; e8 * 8 < a.per;
       e8 += (int64_t)gridDim.x * 256) {
    const int64_t o = base + e8 * 8;
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 d = *reinterpret_cast<const float4*>(a.dX + o + 4 * h);
      const float4 gg = *reinterpret_cast<const float4*>(a.G + o + 4 * h);
      x[4 * h + 0] = d.x * s - gg.x * cg;
      x[4 * h + 1] = d.y * s - gg.y * cg;
      x[4 * h + 2] = d.z * s - gg.z * cg;
      x[4 * h + 3] = d.w * s - gg.w * cg;
      *reinterpret_cast<float4*>(a.dG + o + 4 * h) =
          make_float4(x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]);
    }
    u16 hq[8][3];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_planes(x[e], a.pout.np, hq[e]);
    for (int q = 0; q < a.pout.np; ++q) {
      uint4 w;
      w.x = hq[0][q] | ((uint32_t)hq[1][q] << 16);
      w.y = hq[2][q] | ((uint32_t)hq[3][q] << 16);
      w.z = hq[4][q] | ((uint32_t)hq[5][q] << 16);
      w.w = hq[6][q] | ((uint32_t)hq[7][q] << 16);
      *reinterpret_cast<uint4*>(a.pout.base + q * a.pout.plane_stride + zz * a.pout.zstride +
                                e8 * 8) = w;
    }
  }
}

// ------------------------------------------------------------------------ momentum
// One workgroup per 32 x 32 tile of a matrix's weight orientation.  Where the X orientation
// is the transpose, the tile of dm passes through LDS so that both sides read and write
// along their own rows.  Every element is read and written by one thread per phase.
constexpr int MOM_TILE = 32;

__global__ __launch_bounds__(256) void k_mom_bwd(MomBwdArgs a) {
  const MomBwdMat& M = a.m[blockIdx.z];
  const int tiles_c = (M.cols + MOM_TILE - 1) / MOM_TILE;
  if ((int)blockIdx.x >= ((M.rows + MOM_TILE - 1) / MOM_TILE) * tiles_c) return;
  const int r0 = ((int)blockIdx.x / tiles_c) * MOM_TILE;
  const int c0 = ((int)blockIdx.x % tiles_c) * MOM_TILE;
  const int64_t base = (int64_t)blockIdx.y * M.rows * M.cols;
  const int tx = threadIdx.x % MOM_TILE, ty = threadIdx.x / MOM_TILE;
  constexpr int STEP = 256 / MOM_TILE;
  if (!M.tr) {
    for (int i = ty; i < MOM_TILE; i += STEP) {
      const int r = r0 + i, c = c0 + tx;
      if (r < M.rows && c < M.cols) {
        const int64_t o = base + (int64_t)r * M.cols + c;
        const float t = M.dg[o] + M.dm[o];
        M.dg[o] = t;
        M.dm[o] = a.beta * t;
      }
    }
    return;
  }
  __shared__ float sh[MOM_TILE][MOM_TILE + 1];
  for (int i = ty; i < MOM_TILE; i += STEP) {      // sh[i][j] = dm[r0 + i][c0 + j]
    const int r = r0 + i, c = c0 + tx;
    sh[i][tx] = (r < M.rows && c < M.cols) ? M.dm[base + (int64_t)r * M.cols + c] : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < MOM_TILE; i += STEP) {      // X row c0 + i, column r0 + tx
    const int c = c0 + i, r = r0 + tx;
    if (r < M.rows && c < M.cols) {
      const int64_t o = base + (int64_t)c * M.rows + r;
      const float t = M.dg[o] + sh[tx][i];
      M.dg[o] = t;
      sh[tx][i] = t;
    }
  }
  __syncthreads();
  for (int i = ty; i < MOM_TILE; i += STEP) {
    const int r = r0 + i, c = c0 + tx;
    if (r < M.rows && c < M.cols) M.dm[base + (int64_t)r * M.cols + c] = a.beta * sh[i][tx];
  }
}

__global__ __launch_bounds__(256) void k_add3(Add3Args a) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i * 4 < a.n;
       i += (int64_t)gridDim.x * 256) {
    float4 x = reinterpret_cast<const float4*>(a.x)[i];
    if (a.y) {
      const float4 y = reinterpret_cast<const float4*>(a.y)[i];
      x = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
    if (a.w) {
      const float4 w = reinterpret_cast<const float4*>(a.w)[i];
      x = make_float4(x.x + w.x, x.y + w.y, x.z + w.z, x.w + w.w);
    }
    reinterpret_cast<float4*>(a.out)[i] = x;
  }
}

// ============================================================================ launchers
hipError_t launch_tfront(const TFrontArgs& a0, int Z, hipStream_t s) {
  constexpr int BM = 128, BN = 64, WGM = 4, WGN = 2, BK = 32;
  TFrontArgs a = a0;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.nrows + BM - 1) / BM) * a.tiles_n;
  if (a.tiles == 0 || Z == 0) return hipSuccess;
  hipLaunchKernelGGL((k_tfront<BM, BN, WGM, WGN, BK>), dim3(a.tiles * Z), dim3(WGM * WGN * 64),
                     0, s, a);
  return hipGetLastError();
}

int tfront_col_tiles(int N) { return (N + 63) / 64; }

hipError_t launch_eta_sum(const EtaSumArgs& a, int Z, hipStream_t s) {
  if (Z == 0 || a.nrows == 0) return hipSuccess;
  const int blocks = std::min(1024, (a.nrows + 255) / 256);
  hipLaunchKernelGGL(k_eta_sum, dim3(blocks, Z), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowgemm(const DqArgs& a0, int np, int Z, hipStream_t s) {
  constexpr int BM = 128, BN = 128, WGM = 2, WGN = 4;
  DqArgs a = a0;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.nrows + BM - 1) / BM) * a.tiles_n;
  if (a.tiles == 0 || Z == 0) return hipSuccess;
  const dim3 grid(a.tiles * Z), block(WGM * WGN * 64);
  if (np == 4) hipLaunchKernelGGL((k_rowgemm<BM, BN, WGM, WGN, 4, 0b0011>), grid, block, 0, s, a);
  else if (np == 2) hipLaunchKernelGGL((k_rowgemm<BM, BN, WGM, WGN, 2, 0>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_step_bwd(const StepBwdArgs& a, hipStream_t s) {
  if (a.P == 0 || a.nm == 0) return hipSuccess;
  int cols = 0;
  for (int m = 0; m < a.nm; ++m) cols = std::max(cols, a.m[m].cols);
  const dim3 grid((a.max_rows * a.P + 3) / 4, a.nm);
  if (cols <= 256) hipLaunchKernelGGL(k_step_bwd<1>, grid, dim3(256), 0, s, a);
  else if (cols <= 512) hipLaunchKernelGGL(k_step_bwd<2>, grid, dim3(256), 0, s, a);
  else if (cols <= 1024) hipLaunchKernelGGL(k_step_bwd<4>, grid, dim3(256), 0, s, a);
  else if (cols <= 2048) hipLaunchKernelGGL(k_step_bwd<8>, grid, dim3(256), 0, s, a);
  else if (cols <= 4096) hipLaunchKernelGGL(k_step_bwd<16>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

int gemm2_tiles(int M, int N) { return ((M + 127) / 128) * ((N + 127) / 128); }

hipError_t launch_gemm2(const Gemm2Args& a0, bool bcols, hipStream_t s, bool sym) {
  constexpr int BM = 128, BN = 128, WGM = 2, WGN = 4;
  Gemm2Args a = a0;
  if (sym && (a.M != a.N || bcols || a.gref || a.gpart)) return hipErrorInvalidValue;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = sym ? ns_tri_tiles(a.M, BM) : ((a.M + BM - 1) / BM) * a.tiles_n;
  if (a.tiles == 0 || a.Z == 0) return hipSuccess;
  const dim3 grid(a.tiles * a.Z), block(WGM * WGN * 64);
  if (sym) hipLaunchKernelGGL((k_gemm2<BM, BN, WGM, WGN, 0, true>), grid, block, 0, s, a);
  else if (bcols) hipLaunchKernelGGL((k_gemm2<BM, BN, WGM, WGN, 0b11>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_gemm2<BM, BN, WGM, WGN, 0>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ns_fin(const NsFinArgs& a, int Z, hipStream_t s) {
  if (Z == 0 || a.per == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(256, (a.per / 8 + 255) / 256);
  hipLaunchKernelGGL(k_ns_fin, dim3(blocks, Z), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mom_bwd(const MomBwdArgs& a, hipStream_t s) {
  if (a.P == 0 || a.nm == 0) return hipSuccess;
  int tiles = 0;
  for (int m = 0; m < a.nm; ++m)
    tiles = std::max(tiles, ((a.m[m].rows + MOM_TILE - 1) / MOM_TILE) *
                                ((a.m[m].cols + MOM_TILE - 1) / MOM_TILE));
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mom_bwd, dim3(tiles, a.P, a.nm), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_add3(const Add3Args& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(4096, (a.n / 4 + 255) / 256);
  hipLaunchKernelGGL(k_add3, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
