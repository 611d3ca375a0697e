// HIP kernels of the large-chunk TTT layer forward for gfx950.
//
// The chunk step is a short pipeline of stage kernels, each batched over all (batch, head)
// problems in one launch:
//   front   Z-GEMMs of the fast-weight net on the chunk's query or key rows, with the
//           activation, its derivative and the back-propagated error fused in the epilogue
//           (LaCT explainer page, peacm.com, §2.1: apply and update phases);
//   out     the net's output GEMM (queries: the layer output; keys under MSE: the error)
//   contract  the chunk-summed weight gradients, token index contracted on MFMA
//           (same page, eqs. 4-5: one gradient summed over the whole chunk);
//   ns_*    Muon's Newton-Schulz iteration (same page §2.2.1, eqs. 9-10) as Gram,
//           polynomial and update GEMMs on 1..3 bf16 planes;
//   renorm  W <- W - U and the per-row L2 restore (same page §2.2.1, eq. 8), which also
//           writes the bf16 planes every GEMM of the next chunk reads.
#include <math.h>

#include "ttt_internal.h"

namespace ttt {

// ------------------------------------------------------------------------ elementwise math
__device__ __forceinline__ float sigm(float z) { return 1.f / (1.f + __expf(-z)); }
__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_d(float z) {
  return 0.5f * (1.f + erff(z * 0.70710678118654752f)) +
         z * __expf(-0.5f * z * z) * 0.39894228040143268f;
}

__device__ __forceinline__ void put_planes(const PlaneBuf& b, int z, int64_t off, float x) {
  u16 h[3];
  split_planes(x, b.np, h);
  u16* p = b.base + (int64_t)z * b.zstride + off;
#pragma unroll
  for (int q = 0; q < 3; ++q)
    if (q < b.np) p[q * b.plane_stride] = h[q];
}

__device__ __forceinline__ float load_act(const void* p, int64_t off, int is_bf16) {
  return is_bf16 ? bf2f(static_cast<const u16*>(p)[off]) : static_cast<const float*>(p)[off];
}

// ------------------------------------------------------------------------ front
template <int FW, int MODE>
struct FrontShape {
  static constexpr bool DOT = MODE == FRONT_K_DOT;
  static constexpr int NA = DOT ? 2 : 1;
  static constexpr int NB = (FW == FW_SWIGLU ? 2 : 1) + (DOT ? 1 : 0);
  static constexpr int NP = NB;
};

template <int BM, int BN, int FW, int MODE>
__global__ __launch_bounds__(256) void k_front(FrontArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using FS = FrontShape<FW, MODE>;
  constexpr int NA = FS::NA, NB = FS::NB, NP = FS::NP;
  const int z = blockIdx.y;
  const int m0 = (blockIdx.x / a.tiles_n) * BM;
  const int n0 = (blockIdx.x % a.tiles_n) * BN;

  Operand A[NA];
  Operand B[NB];
  int IA[NP], IB[NP];
  A[0] = a.x;
  if constexpr (FS::DOT) A[NA - 1] = a.v;
  B[0] = a.w1;
  if constexpr (FW == FW_SWIGLU) B[1] = a.w3;
  if constexpr (FS::DOT) B[NB - 1] = a.w2t;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    IB[p] = p;
    IA[p] = (FS::DOT && p == NP - 1) ? 1 : 0;
  }

  MultiGemm<BM, BN, NA, NB, NP> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, z, a.K, smem);

  g.for_each([&](int i, int j, int v, int r, int c) {
    const int row = m0 + r, col = n0 + c;
    if (row >= a.mrows || col >= a.N) return;
    const float z1 = g.acc[0][i][j][v];
    if constexpr (MODE == FRONT_Q) {
      float h;
      if constexpr (FW == FW_SWIGLU) h = z1 * sigm(z1) * g.acc[1][i][j][v];
      else h = gelu_f(z1);
      put_planes(a.o1, z, (int64_t)row * a.o1.ld + col, h);
    } else if constexpr (MODE == FRONT_K_DOT) {
      const float e = row < a.nrows ? a.eta[(int64_t)z * a.eta_zstride + row] : 0.f;
      const float y = g.acc[NP - 1][i][j][v];
      const float dh = -e * y;
      if constexpr (FW == FW_SWIGLU) {
        const float z3 = g.acc[1][i][j][v];
        const float s = sigm(z1);
        const float act = z1 * s;
        put_planes(a.o1, z, (int64_t)col * a.o1.ld + row, dh * z3 * s * (1.f + z1 * (1.f - s)));
        put_planes(a.o2, z, (int64_t)col * a.o2.ld + row, dh * act);
        put_planes(a.o3, z, (int64_t)col * a.o3.ld + row, -e * act * z3);
      } else {
        put_planes(a.o1, z, (int64_t)col * a.o1.ld + row, dh * gelu_d(z1));
        put_planes(a.o3, z, (int64_t)col * a.o3.ld + row, -e * gelu_f(z1));
      }
    } else {  // FRONT_K_MSE
      float h, f1, f3 = 0.f;
      if constexpr (FW == FW_SWIGLU) {
        const float z3 = g.acc[1][i][j][v];
        const float s = sigm(z1);
        const float act = z1 * s;
        h = act * z3;
        f1 = z3 * s * (1.f + z1 * (1.f - s));
        f3 = act;
      } else {
        h = gelu_f(z1);
        f1 = gelu_d(z1);
      }
      put_planes(a.o2, z, (int64_t)col * a.o2.ld + row, h);
      if (row < a.nrows) {
        put_planes(a.o1, z, (int64_t)row * a.o1.ld + col, h);
        const int64_t fo = (int64_t)z * a.f_zstride + (int64_t)row * a.N + col;
        a.fa[fo] = f1;
        if constexpr (FW == FW_SWIGLU) a.fb[fo] = f3;
      }
    }
  });
}

// ------------------------------------------------------------------------ out / dH
template <int BM, int BN, int MODE>
__global__ __launch_bounds__(256) void k_out(OutArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int z = blockIdx.y;
  const int m0 = (blockIdx.x / a.tiles_n) * BM;
  const int n0 = (blockIdx.x % a.tiles_n) * BN;
  Operand A[1] = {a.a};
  Operand B[1] = {a.b};
  const int IA[1] = {0}, IB[1] = {0};
  MultiGemm<BM, BN, 1, 1, 1> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, z, a.K, smem);

  g.for_each([&](int i, int j, int v, int r, int c) {
    const int row = m0 + r, col = n0 + c;
    if (row >= a.mrows || col >= a.N) return;
    const float x = g.acc[0][i][j][v];
    if constexpr (MODE == OUT_Q) {
      if (row >= a.nrows) return;
      const int64_t o = (int64_t)z * a.out_zstride + (int64_t)row * a.N + col;
      if (a.out_bf16) static_cast<u16*>(a.out)[o] = f2bf(x);
      else static_cast<float*>(a.out)[o] = x;
    } else if constexpr (MODE == OUT_K_MSE) {
      float e = 0.f;
      if (row < a.nrows) {
        const float vv = load_act(a.vin, (int64_t)z * a.v_zstride + (int64_t)row * a.N + col,
                                  a.v_bf16);
        e = 2.f * a.eta[(int64_t)z * a.eta_zstride + row] * (x - vv);
        put_planes(a.e, z, (int64_t)row * a.e.ld + col, e);
      }
      put_planes(a.et, z, (int64_t)col * a.et.ld + row, e);
    } else {  // DH_MSE
      float d1 = 0.f, d3 = 0.f;
      if (row < a.nrows) {
        const int64_t fo = (int64_t)z * a.f_zstride + (int64_t)row * a.N + col;
        d1 = x * a.fa[fo];
        if (a.swiglu) d3 = x * a.fb[fo];
      }
      put_planes(a.dz1t, z, (int64_t)col * a.dz1t.ld + row, d1);
      if (a.swiglu) put_planes(a.dz3t, z, (int64_t)col * a.dz3t.ld + row, d3);
    }
  });
}

// ------------------------------------------------------------------------ block reduction
__device__ __forceinline__ float block_sum_256(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  const float t = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return t;
}

// ------------------------------------------------------------------------ contraction
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_contract(ContractArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int zz = blockIdx.y;
  const int m = zz / a.P, p = zz % a.P;
  const int m0 = (blockIdx.x / a.tiles_n) * BM;
  const int n0 = (blockIdx.x % a.tiles_n) * BN;
  Operand A[1] = {a.a[m]};
  Operand B[1] = {a.b[m]};
  const int IA[1] = {0}, IB[1] = {0};
  MultiGemm<BM, BN, 1, 1, 1> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, p, a.K, smem);

  const int M = a.M, N = a.N;
  const int64_t base = (int64_t)zz * M * N;
  const int tr = (a.tr_mask >> m) & 1;
  float ss = 0.f;
  g.for_each([&](int i, int j, int v, int r, int c) {
    const int row = m0 + r, col = n0 + c;
    if (row >= M || col >= N) return;
    float x = g.acc[0][i][j][v];
    const int64_t off = base + (int64_t)row * N + col;
    if (a.accum_in) x += a.G[off];
    if (!a.last) {
      a.G[off] = x;
    } else if (a.muon) {
      a.G[off] = x;
      put_planes(a.x, zz, (int64_t)row * N + col, x);
      put_planes(a.xt, zz, (int64_t)col * M + row, x);
      ss += x * x;
    } else {
      a.U[tr ? base + (int64_t)col * M + row : off] = x;
    }
  });
  if (a.last && a.muon) {
    const float t = block_sum_256(ss, reinterpret_cast<float*>(smem));
    if (threadIdx.x == 0) a.part[(int64_t)zz * a.tiles + blockIdx.x] = t;
  }
}

// ------------------------------------------------------------------------ Newton-Schulz
__device__ __forceinline__ float ns_scale(const NsArgs& a, int zz) {
  float t = 0.f;
  for (int i = 0; i < a.nparts; ++i) t += a.part[(int64_t)zz * a.nparts + i];
  return 1.f / (sqrtf(t) + a.eps);
}

__device__ __forceinline__ void tri_tile(int t, int nt, int& ti, int& tj) {
  ti = 0;
  while (t >= nt - ti) {
    t -= nt - ti;
    ++ti;
  }
  tj = ti + t;
}

// A = s^2 X X^T, upper tiles computed, both triangles written.
template <int T>
__global__ __launch_bounds__(256) void k_ns_gram(NsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int zz = blockIdx.y;
  const int M = a.M;
  int ti, tj;
  tri_tile(blockIdx.x, (M + T - 1) / T, ti, tj);
  const int m0 = ti * T, n0 = tj * T;
  Operand X = operand_of(a.xin, a.xin.np, M);
  Operand A[1] = {X};
  Operand B[1] = {X};
  const int IA[1] = {0}, IB[1] = {0};
  MultiGemm<T, T, 1, 1, 1> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, zz, a.N, smem);
  float s2 = 1.f;
  if (a.first) {
    const float s = ns_scale(a, zz);
    s2 = s * s;
  }
  const int64_t base = (int64_t)zz * M * M;
  g.for_each([&](int i, int j, int v, int r, int c) {
    const int R = m0 + r, C = n0 + c;
    if (R >= M || C >= M || R > C) return;
    const float x = s2 * g.acc[0][i][j][v];
    a.afp[base + (int64_t)R * M + C] = x;
    a.afp[base + (int64_t)C * M + R] = x;
    put_planes(a.aout, zz, (int64_t)R * M + C, x);
    put_planes(a.aout, zz, (int64_t)C * M + R, x);
  });
}

// B = b A + c A A  (A symmetric, so A serves as its own transposed operand).
template <int T>
__global__ __launch_bounds__(256) void k_ns_poly(NsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int zz = blockIdx.y;
  const int M = a.M;
  int ti, tj;
  tri_tile(blockIdx.x, (M + T - 1) / T, ti, tj);
  const int m0 = ti * T, n0 = tj * T;
  Operand Ao = operand_of(a.ain, a.ain.np, M);
  Operand A[1] = {Ao};
  Operand B[1] = {Ao};
  const int IA[1] = {0}, IB[1] = {0};
  MultiGemm<T, T, 1, 1, 1> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, zz, M, smem);
  const int64_t base = (int64_t)zz * M * M;
  g.for_each([&](int i, int j, int v, int r, int c) {
    const int R = m0 + r, C = n0 + c;
    if (R >= M || C >= M || R > C) return;
    const float x = a.coef_b * a.afp[base + (int64_t)R * M + C] + a.coef_c * g.acc[0][i][j][v];
    put_planes(a.aout, zz, (int64_t)R * M + C, x);
    put_planes(a.aout, zz, (int64_t)C * M + R, x);
  });
}

// X' = a X + B X  (iteration 0: X = s G with the scale folded into the epilogue).
template <int T>
__global__ __launch_bounds__(256) void k_ns_update(NsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int zz = blockIdx.y;
  const int M = a.M, N = a.N;
  const int m0 = (blockIdx.x / a.tiles_n) * T;
  const int n0 = (blockIdx.x % a.tiles_n) * T;
  Operand A[1] = {operand_of(a.ain, a.ain.np, M)};
  Operand B[1] = {operand_of(a.xtin, a.xtin.np, N)};
  const int IA[1] = {0}, IB[1] = {0};
  MultiGemm<T, T, 1, 1, 1> g;
  g.zero();
  g.run(A, B, IA, IB, m0, n0, zz, M, smem);
  const float sc = a.first ? ns_scale(a, zz) : 1.f;
  const int64_t base = (int64_t)zz * M * N;
  const int m = zz / a.P;
  const int tr = (a.tr_mask >> m) & 1;
  g.for_each([&](int i, int j, int v, int r, int c) {
    const int R = m0 + r, C = n0 + c;
    if (R >= M || C >= N) return;
    const int64_t off = base + (int64_t)R * N + C;
    const float x = sc * (a.coef_a * a.G[off] + g.acc[0][i][j][v]);
    if (!a.last) {
      a.G[off] = x;
      put_planes(a.xout, zz, (int64_t)R * N + C, x);
      put_planes(a.xtout, zz, (int64_t)C * M + R, x);
    } else {
      a.U[tr ? base + (int64_t)C * M + R : off] = x;
    }
  });
}

// ------------------------------------------------------------------------ renorm / update
// One wavefront per weight row (rows of all problems flattened).  Both norms are summed
// by the same code over the same element order, so a zero update leaves the row bit-exact.
__global__ __launch_bounds__(256) void k_renorm(RenormArgs a) {
  const int m = blockIdx.y;
  const RenormMat& M = a.m[m];
  const int lane = threadIdx.x & 63;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gr >= M.rows * a.P) return;
  const int p = gr / M.rows, r = gr % M.rows;
  const int cols = M.cols;
  float* w = M.W + (int64_t)gr * cols;
  const float* u = M.U ? M.U + (int64_t)gr * cols : nullptr;
  float so = 0.f, sn = 0.f;
  if (u) {
    for (int c = lane; c < cols; c += 64) {
      const float x = w[c];
      const float y = x - u[c];
      so += x * x;
      sn += y * y;
    }
  }
  so = wave_sum(so);
  sn = wave_sum(sn);
  float scale = 1.f;
  if (u && a.renorm && sn > 0.f) scale = sqrtf(so) / sqrtf(sn);
  if (u && lane == 0 && (!isfinite(so) || !isfinite(sn))) *a.health = 1;
  for (int c = lane; c < cols; c += 64) {
    float x = w[c];
    if (u) {
      x = (x - u[c]) * scale;
      w[c] = x;
    }
    u16 h[3];
    split_planes(x, a.np, h);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (q < a.np) {
        M.pl[q * M.pl_stride + (int64_t)gr * cols + c] = h[q];
        if (M.plt)
          M.plt[q * M.plt_stride + (int64_t)p * cols * M.rows + (int64_t)c * M.rows + r] = h[q];
      }
    }
  }
}

// ------------------------------------------------------------------------ token transpose
// Rows [n][d] of a chunk (activation dtype) -> planes [d][bpad], optionally scaled by
// -eta_t; columns t in [n, bpad) are written as zeros.
__global__ __launch_bounds__(256) void k_transpose(TransposeArgs a) {
  __shared__ float tile[64][65];
  const int z = blockIdx.z;
  const int t0 = blockIdx.x * 64, i0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int rr = 0; rr < 16; ++rr) {
    const int t = t0 + ty + 4 * rr, i = i0 + tx;
    float val = 0.f;
    if (t < a.n && i < a.d) {
      val = load_act(a.x, (int64_t)z * a.x_zstride + (int64_t)t * a.d + i, a.x_bf16);
      if (a.neg_eta) val *= -a.eta[(int64_t)z * a.eta_zstride + t];
    }
    tile[ty + 4 * rr][tx] = val;
  }
  __syncthreads();
  for (int rr = 0; rr < 16; ++rr) {
    const int i = i0 + ty + 4 * rr, t = t0 + tx;
    if (i < a.d && t < a.bpad) put_planes(a.out, z, (int64_t)i * a.out.ld + t, tile[tx][ty + 4 * rr]);
  }
}

// fp32 rows -> bf16 planes, same layout.
__global__ __launch_bounds__(256) void k_split(SplitArgs a) {
  const int z = blockIdx.y;
  const int64_t total = (int64_t)a.n * a.d;
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
    put_planes(a.out, z, e, a.x[(int64_t)z * a.x_zstride + e]);
}

// ============================================================================ launchers
static constexpr int LDS_MAX = 160 * 1024;

template <class K>
static hipError_t set_lds(K kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int BM, int BN, int FW, int MODE>
static hipError_t front_bm(const FrontArgs& a0, int Z, hipStream_t s) {
  using FS = FrontShape<FW, MODE>;
  using TS = TileShape<BM, BN, FS::NA, FS::NB>;
  FrontArgs a = a0;
  int pa[2] = {a.x.planes, a.v.planes};
  int pb[3];
  pb[0] = a.w1.planes;
  int nb = 1;
  if (FW == FW_SWIGLU) pb[nb++] = a.w3.planes;
  if (FS::DOT) pb[nb++] = a.w2t.planes;
  const int lds = 2 * TS::stage_bytes(pa, pb);
  if (lds > LDS_MAX) return hipErrorInvalidValue;
  auto kern = k_front<BM, BN, FW, MODE>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int tiles_m = (a.mrows + BM - 1) / BM;
  if (tiles_m == 0 || Z == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(tiles_m * a.tiles_n, Z), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FW, int MODE>
static hipError_t front_fm(const FrontArgs& a, int Z, hipStream_t s) {
  using FS = FrontShape<FW, MODE>;
  using TS = TileShape<128, 64, FS::NA, FS::NB>;
  int pa[2] = {a.x.planes, a.v.planes};
  int pb[3];
  pb[0] = a.w1.planes;
  int nb = 1;
  if (FW == FW_SWIGLU) pb[nb++] = a.w3.planes;
  if (FS::DOT) pb[nb++] = a.w2t.planes;
  if (2 * TS::stage_bytes(pa, pb) <= LDS_MAX) return front_bm<128, 64, FW, MODE>(a, Z, s);
  return front_bm<64, 64, FW, MODE>(a, Z, s);
}

hipError_t launch_front(int fw, int mode, const FrontArgs& a, int Z, hipStream_t s) {
  if (fw == FW_SWIGLU) {
    if (mode == FRONT_Q) return front_fm<FW_SWIGLU, FRONT_Q>(a, Z, s);
    if (mode == FRONT_K_DOT) return front_fm<FW_SWIGLU, FRONT_K_DOT>(a, Z, s);
    return front_fm<FW_SWIGLU, FRONT_K_MSE>(a, Z, s);
  }
  if (mode == FRONT_Q) return front_fm<FW_GELU, FRONT_Q>(a, Z, s);
  if (mode == FRONT_K_DOT) return front_fm<FW_GELU, FRONT_K_DOT>(a, Z, s);
  return front_fm<FW_GELU, FRONT_K_MSE>(a, Z, s);
}

template <int MODE>
static hipError_t out_m(const OutArgs& a0, int Z, hipStream_t s) {
  constexpr int BM = 128, BN = 64;
  using TS = TileShape<BM, BN, 1, 1>;
  OutArgs a = a0;
  int pa[1] = {a.a.planes}, pb[1] = {a.b.planes};
  const int lds = 2 * TS::stage_bytes(pa, pb);
  auto kern = k_out<BM, BN, MODE>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int tiles_m = (a.mrows + BM - 1) / BM;
  if (tiles_m == 0 || Z == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(tiles_m * a.tiles_n, Z), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_out(int mode, const OutArgs& a, int Z, hipStream_t s) {
  if (mode == OUT_Q) return out_m<OUT_Q>(a, Z, s);
  if (mode == OUT_K_MSE) return out_m<OUT_K_MSE>(a, Z, s);
  return out_m<DH_MSE>(a, Z, s);
}

hipError_t launch_contract(const ContractArgs& a0, int nm, hipStream_t s) {
  constexpr int BM = CONTRACT_BM, BN = CONTRACT_BN;
  using TS = TileShape<BM, BN, 1, 1>;
  ContractArgs a = a0;
  int lds = 0;
  for (int m = 0; m < nm; ++m) {
    int pa[1] = {a.a[m].planes}, pb[1] = {a.b[m].planes};
    const int l = 2 * TS::stage_bytes(pa, pb);
    lds = l > lds ? l : lds;
  }
  auto kern = k_contract<BM, BN>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.M + BM - 1) / BM) * a.tiles_n;
  if (a.tiles == 0 || a.P == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(a.tiles, nm * a.P), dim3(256), lds, s, a);
  return hipGetLastError();
}

int ns_tile(int Z, int M) {
  const int t128 = (M + 127) / 128;
  return (Z * t128 * (t128 + 1) / 2 >= 256) ? 128 : 64;
}
int ns_tri_tiles(int M, int tile) {
  const int t = (M + tile - 1) / tile;
  return t * (t + 1) / 2;
}

template <int T, int STAGE>
static hipError_t ns_t(const NsArgs& a0, hipStream_t s) {
  using TS = TileShape<T, T, 1, 1>;
  NsArgs a = a0;
  int pa[1], pb[1];
  if (STAGE == 0) { pa[0] = pb[0] = a.xin.np; }
  else if (STAGE == 1) { pa[0] = pb[0] = a.ain.np; }
  else { pa[0] = a.ain.np; pb[0] = a.xtin.np; }
  const int lds = 2 * TS::stage_bytes(pa, pb);
  if (a.Z == 0) return hipSuccess;
  if (STAGE == 2) {
    a.tiles_n = (a.N + T - 1) / T;
    a.tiles = ((a.M + T - 1) / T) * a.tiles_n;
    auto kern = k_ns_update<T>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.tiles, a.Z), dim3(256), lds, s, a);
  } else {
    a.tiles = ns_tri_tiles(a.M, T);
    if (STAGE == 0) {
      auto kern = k_ns_gram<T>;
      hipError_t e = set_lds(kern, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(a.tiles, a.Z), dim3(256), lds, s, a);
    } else {
      auto kern = k_ns_poly<T>;
      hipError_t e = set_lds(kern, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(a.tiles, a.Z), dim3(256), lds, s, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_ns_gram(const NsArgs& a, hipStream_t s) {
  return ns_tile(a.Z, a.M) == 128 ? ns_t<128, 0>(a, s) : ns_t<64, 0>(a, s);
}
hipError_t launch_ns_poly(const NsArgs& a, hipStream_t s) {
  return ns_tile(a.Z, a.M) == 128 ? ns_t<128, 1>(a, s) : ns_t<64, 1>(a, s);
}
hipError_t launch_ns_update(const NsArgs& a, hipStream_t s) {
  return ns_tile(a.Z, a.M) == 128 ? ns_t<128, 2>(a, s) : ns_t<64, 2>(a, s);
}

hipError_t launch_renorm(const RenormArgs& a, hipStream_t s) {
  if (a.P == 0 || a.nm == 0) return hipSuccess;
  const int blocks = (a.max_rows * a.P + 3) / 4;
  hipLaunchKernelGGL(k_renorm, dim3(blocks, a.nm), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, int Z, hipStream_t s) {
  if (Z == 0 || a.bpad == 0) return hipSuccess;
  hipLaunchKernelGGL(k_transpose, dim3(a.bpad / 64, (a.d + 63) / 64, Z), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split(const SplitArgs& a, int Z, hipStream_t s) {
  if (Z == 0 || a.n == 0) return hipSuccess;
  int64_t total = (int64_t)a.n * a.d;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_split, dim3(blocks, Z), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t prepare_kernels() { return hipSuccess; }

}  // namespace ttt
