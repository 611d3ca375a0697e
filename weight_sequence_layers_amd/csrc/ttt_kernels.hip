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

#include <type_traits>

#include "ttt_internal.h"

namespace ttt {

// ------------------------------------------------------------------------ elementwise math
// logistic function; the hardware reciprocal (about 1 ulp) in place of an IEEE division,
// whose fix-up sequence dominated the gradient front's epilogue
__device__ __forceinline__ float sigm(float z) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}
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

// The Gemm of a front: one operand per tensor (plane pairs as K segments), or with PR > 0
// (every operand in PR bf16 planes) the plane-resident grouped product, all plane tiles of a
// K step loaded once, for launches too small to fill the GPU.
template <int BM, int BN, int WGM, int WGN, int FW, int MODE, int BK, int PR>
struct FrontGemm {
  using FS = FrontShape<FW, MODE>;
  static constexpr int NA = FS::NA, NB = FS::NB;
  // the inner-product loss reads W2 [dim][hidden] column-wise for V W2; the epilogue
  // stores planes only, which the swapped accumulator layout packs
  using type = std::conditional_t<
      PR == 0, Gemm<BM, BN, WGM, WGN, NA, NB, 0, FS::DOT ? (1 << (NB - 1)) : 0, 0, BK, true>,
      Gemm<BM, BN, WGM, WGN, NA * (PR ? PR : 1), NB * (PR ? PR : 1), 0,
           FS::DOT ? ((1 << PR) - 1) << ((NB - 1) * PR) : 0, PR, BK, true, 1, -1, false, NB>>;
};

template <int BM, int BN, int WGM, int WGN, int FW, int MODE, int BK, int PR = 0>
__global__ __launch_bounds__(WGM * WGN * 64) void k_front(FrontArgs a) {
  using FS = FrontShape<FW, MODE>;
  constexpr int NA = FS::NA, NB = FS::NB;
  using G = typename FrontGemm<BM, BN, WGM, WGN, FW, MODE, BK, PR>::type;
  GEMM_LDS(G);
  // two planes per store pass where the stage buffer already has room for them
  constexpr int SP = G::STAGE >= store_lds_bytes<G, TILE_NORMAL, 2>() ? 2 : 1;
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int z = lid / a.tiles, tile = lid % a.tiles;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;

  G g;
  g.zero();
  if constexpr (PR == 0) {
    g.run(a.A, a.B, m0, n0, z, a.K, GEMM_STAGES);
  } else {
    Operand Aq[NA * PR], Bq[NB * PR];   // one operand per plane
#pragma unroll
    for (int i = 0; i < NA * PR; ++i) {
      Aq[i] = a.A[i / PR];
      Aq[i].p += (i % PR) * a.A[i / PR].pstride;
      Aq[i].planes = 1;
    }
#pragma unroll
    for (int i = 0; i < NB * PR; ++i) {
      Bq[i] = a.B[i / PR];
      Bq[i].p += (i % PR) * a.B[i / PR].pstride;
      Bq[i].planes = 1;
    }
    g.run(Aq, Bq, m0, n0, z, a.K, GEMM_STAGES);
  }

  const float* eta = a.eta + (int64_t)z * a.eta_zstride;
  g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
    const int row = m0 + r, col = n0 + c;
    const float z1 = g.acc[0][i][j][v];
    if constexpr (MODE == FRONT_Q) {
      if constexpr (FW == FW_SWIGLU) g.acc[0][i][j][v] = z1 * sigm(z1) * g.acc[1][i][j][v];
      else g.acc[0][i][j][v] = gelu_f(z1);
    } else if constexpr (MODE == FRONT_K_DOT) {
      const float e = row < a.nrows ? eta[row] : 0.f;
      const float dh = -e * g.acc[NB - 1][i][j][v];
      if constexpr (FW == FW_SWIGLU) {
        const float z3 = g.acc[1][i][j][v];
        const float s = sigm(z1);
        const float act = z1 * s;
        g.acc[0][i][j][v] = dh * z3 * s * (1.f + z1 * (1.f - s));
        g.acc[1][i][j][v] = dh * act;
        g.acc[2][i][j][v] = -e * act * z3;
      } else {
        g.acc[0][i][j][v] = dh * gelu_d(z1);
        g.acc[1][i][j][v] = -e * gelu_f(z1);
      }
    } else {  // FRONT_K_MSE: hidden activation and its derivative factors
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
      g.acc[0][i][j][v] = h;
      if (row < a.nrows && col < a.N) {
        const int64_t fo = (int64_t)z * a.f_zstride + (int64_t)row * a.N + col;
        a.fa[fo] = f1;
        if constexpr (FW == FW_SWIGLU) a.fb[fo] = f3;
      }
    }
  });
  const int cl = min(BN, a.N - n0);
  const int rn = min(BM, a.nrows - m0);   // rows holding tokens
  if constexpr (MODE == FRONT_K_DOT) {
    store_planes<G, TILE_NORMAL, SP>(g.acc[0], smem, a.o1, z, m0, n0, rn, cl);
    if constexpr (FW == FW_SWIGLU) {
      store_planes<G, TILE_NORMAL, SP>(g.acc[1], smem, a.o2, z, m0, n0, rn, cl);
      store_planes<G, TILE_NORMAL, SP>(g.acc[2], smem, a.o3, z, m0, n0, rn, cl);
    } else {
      store_planes<G, TILE_NORMAL, SP>(g.acc[1], smem, a.o3, z, m0, n0, rn, cl);
    }
  } else {
    store_planes<G, TILE_NORMAL, SP>(g.acc[0], smem, a.o1, z, m0, n0, rn, cl);
  }
}

// ------------------------------------------------------------------------ out / dH
// PR > 0 (the query output with PR bf16 planes on both operands): the plane-resident
// product, every plane tile loaded once per K step, for launches too small to fill the GPU.
template <int BM, int BN, int WGM, int WGN, int MODE, int PR = 0>
__global__ __launch_bounds__(WGM * WGN * 64) void k_out(OutArgs a) {
  // dH = E W2 reads W2 [dim][hidden] column-wise; the query output (a plane store) takes
  // the swapped accumulator layout
  static_assert(PR == 0 || MODE == OUT_Q, "plane-resident form for the query output");
  constexpr int NP = PR ? PR : 1;
  using G = Gemm<BM, BN, WGM, WGN, NP, NP, 0, MODE == DH_MSE ? 1 : 0, PR, 64, MODE == OUT_Q>;
  GEMM_LDS(G);
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int z = lid / a.tiles, tile = lid % a.tiles;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;
  G g;
  g.zero();
  if constexpr (PR == 0) {
    g.run(&a.a, &a.b, m0, n0, z, a.K, GEMM_STAGES);
  } else {
    Operand Aq[PR], Bq[PR];   // one operand per plane
#pragma unroll
    for (int q = 0; q < PR; ++q) {
      Aq[q] = a.a;
      Aq[q].p += q * a.a.pstride;
      Aq[q].planes = 1;
      Bq[q] = a.b;
      Bq[q].p += q * a.b.pstride;
      Bq[q].planes = 1;
    }
    g.run(Aq, Bq, m0, n0, z, a.K, GEMM_STAGES);
  }

  const int cl = min(BN, a.N - n0);
  const int rn = min(BM, a.nrows - m0);
  if constexpr (MODE == OUT_Q) {
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
  } else if constexpr (MODE == OUT_K_MSE) {
    const float* eta = a.eta + (int64_t)z * a.eta_zstride;
    g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
      const int row = m0 + r, col = n0 + c;
      float e = 0.f;
      if (row < a.nrows && col < a.N) {
        const float vv = load_act(a.vin, (int64_t)z * a.v_zstride + (int64_t)row * a.N + col,
                                  a.v_bf16);
        e = 2.f * eta[row] * (g.acc[0][i][j][v] - vv);
      }
      g.acc[0][i][j][v] = e;
    });
    store_tile_planes<G, TILE_NORMAL>(g.acc[0], smem, a.e, z, m0, n0, rn, cl);
  } else {  // DH_MSE
    f32x16 d3[G::TM][G::TN];
    g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
      const int row = m0 + r, col = n0 + c;
      float x1 = 0.f, x3 = 0.f;
      if (row < a.nrows && col < a.N) {
        const int64_t fo = (int64_t)z * a.f_zstride + (int64_t)row * a.N + col;
        x1 = g.acc[0][i][j][v] * a.fa[fo];
        if (a.swiglu) x3 = g.acc[0][i][j][v] * a.fb[fo];
      }
      g.acc[0][i][j][v] = x1;
      d3[i][j][v] = x3;
    });
    store_tile_planes<G, TILE_NORMAL>(g.acc[0], smem, a.dz1, z, m0, n0, rn, cl);
    if (a.swiglu) store_tile_planes<G, TILE_NORMAL>(d3, smem, a.dz3, z, m0, n0, rn, cl);
  }
}

// ------------------------------------------------------------------------ apply backward
// dQ = sum_m dZ_m W_m for the NP (dZ_m, W_m) pairs: accumulator m takes pair m, and the
// epilogue adds them and stores dQ like the apply output.
template <int BM, int BN, int WGM, int WGN, int NP>
__global__ __launch_bounds__(WGM * WGN * 64) void k_dq(DqArgs a) {
  // W_m [hidden][dim] read column-wise; swapped accumulator layout for the packed store
  using G = Gemm<BM, BN, WGM, WGN, NP, NP, 0, (1 << NP) - 1, 0, 64, true>;
  GEMM_LDS(G);
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int z = lid / a.tiles, tile = lid % a.tiles;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;
  G g;
  g.zero();
  g.run(a.a, a.b, m0, n0, z, a.K, GEMM_STAGES);
  if constexpr (NP == 2) {
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j) g.acc[0][i][j] += g.acc[1][i][j];
  }
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

// ------------------------------------------------------------------------ contraction
// PA = PB = 0: the operands' plane pairs run as K segments (any plane counts, K step 64).
// Else A has PA planes and B has PB, all loaded once per K step of 32 (plane-resident).
template <int PA, int PB>
struct ContractGemm {
  static constexpr int NA = PA ? PA : 1, NB = PB ? PB : 1;
  static constexpr int PL = PA ? (PA > PB ? PA : PB) : 0;
};
template <int BM, int BN, int WGM, int WGN, int PA, int PB>
__global__ __launch_bounds__(WGM * WGN * 64) void k_contract(ContractArgs a) {
  using CG = ContractGemm<PA, PB>;
  // both operands token-major (read column-wise); the plane-resident form steps K by 32
  // where two of its workgroups share a CU, and by 64 on 64-row tiles (few workgroups, so
  // half the steps is worth the LDS of one workgroup per CU)
  using G = Gemm<BM, BN, WGM, WGN, CG::NA, CG::NB, (1 << CG::NA) - 1, (1 << CG::NB) - 1, CG::PL,
                 (PA && BM > 64) ? 32 : 64>;
  GEMM_LDS(G);
  // logical block order (token range, matrix and problem, tile)
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int tile = lid % a.tiles, zk = lid / a.tiles;
  const int zz = zk % a.nz, ks = zk / a.nz;
  const int m = zz / a.P, p = zz % a.P;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;
  // this workgroup's token range: the operands' token-major rows k0 ..
  Operand A = a.a[m], B = a.b[m];
  const int k0 = ks * a.kchunk;
  A.p += (int64_t)k0 * A.ld;
  B.p += (int64_t)k0 * B.ld;
  G g;
  g.zero();
  if constexpr (PA == 0) {
    g.run(&A, &B, m0, n0, p, min(a.kchunk, a.K - k0), GEMM_STAGES);
  } else {
    Operand Aq[PA], Bq[PB];   // one operand per plane
#pragma unroll
    for (int q = 0; q < PA; ++q) {
      Aq[q] = A;
      Aq[q].p += q * A.pstride;
      Aq[q].planes = 1;
    }
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      Bq[q] = B;
      Bq[q].p += q * B.pstride;
      Bq[q].planes = 1;
    }
    g.run(Aq, Bq, m0, n0, p, min(a.kchunk, a.K - k0), GEMM_STAGES);
  }

  const int M = a.M, N = a.N;
  const int64_t base = (int64_t)zz * M * N;
  // a token range's partial tile goes to its slice of gpart, with no epilogue
  const bool split = a.ksplit > 1;
  float* const gout = split ? a.gpart + ks * a.gpart_stride : a.G;
  const bool accum = !split && a.accum_in, last = !split && a.last;
  const int tr = (a.tr_mask >> m) & 1;
  float ss = 0.f;
  g.for_each([&](int i, int j, int v, int r, int c) __attribute__((always_inline)) {
    const int row = m0 + r, col = n0 + c;
    float x = g.acc[0][i][j][v];
    if (row < M && col < N) {
      const int64_t off = base + (int64_t)row * N + col;
      const int64_t widx = tr ? base + (int64_t)col * M + row : off;   // weight orientation
      if (accum) x += a.G[off];
      if (last && a.mom) {
        x = fmaf(a.beta, a.mom[widx], x);
        if (a.mom_write) a.mom[widx] = x;
      }
      if (last && a.g32) a.g32[off] = x;
      if (!last) {
        gout[off] = x;
      } else if (a.muon) {
        ss += x * x;
      } else {
        a.U[widx] = x;
      }
    }
    g.acc[0][i][j][v] = x;
  });
  if (last && a.muon) {
    const int rl = min(BM, M - m0), cl = min(BN, N - n0);
    store_tile_planes<G, TILE_NORMAL>(g.acc[0], smem, a.x, zz, m0, n0, rl, cl);
    const float t = block_sum(ss, reinterpret_cast<float*>(smem));
    if ((int)threadIdx.x < a.psub)
      a.part[((int64_t)zz * a.tiles + tile) * a.psub + threadIdx.x] = threadIdx.x == 0 ? t : 0.f;
  }
}

// Second pass of a token-split contraction: the ksplit partial tiles added in split order,
// then the same epilogue as k_contract (the running sum in G, or the X0 planes with the
// sum of squares, or U).  A tile is spread over CONTRACT_SUM_SUB workgroups of 256
// threads, one per band of 16 rows; each thread takes one run of 8 columns (N is a
// multiple of 16) and each band stores its own part of the sum of squares.
constexpr int CONTRACT_SUM_THREADS = 256;

template <int BM, int BN>
__global__ __launch_bounds__(CONTRACT_SUM_THREADS) void k_contract_sum(ContractArgs a) {
  constexpr int RUNS = BN / 8, ROWS = CONTRACT_SUM_THREADS / RUNS;
  static_assert(BM == ROWS * CONTRACT_SUM_SUB, "one band of ROWS rows per part");
  __shared__ float red[CONTRACT_SUM_THREADS / 64];
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int band = lid % CONTRACT_SUM_SUB, tz = lid / CONTRACT_SUM_SUB;
  const int zz = tz / a.tiles, tile = tz % a.tiles;
  const int m = zz / a.P;
  const int M = a.M, N = a.N;
  const int row = (tile / a.tiles_n) * BM + band * ROWS + (int)threadIdx.x / RUNS;
  const int col = (tile % a.tiles_n) * BN + ((int)threadIdx.x % RUNS) * 8;
  const int64_t base = (int64_t)zz * M * N;
  const int tr = (a.tr_mask >> m) & 1;
  float ss = 0.f;
  if (row < M && col < N) {
    const int64_t off = base + (int64_t)row * N + col;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    // the partials in split order, eight at a time, each batch's loads issued before its
    // first add
    for (int k0 = 0; k0 < a.ksplit; k0 += 8) {
      float4 pu[8], pw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k0 + k < a.ksplit) {
          const float4* src =
              reinterpret_cast<const float4*>(a.gpart + (k0 + k) * a.gpart_stride + off);
          pu[k] = src[0];
          pw[k] = src[1];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k0 + k < a.ksplit) {
          const float4 u = pu[k], w = pw[k];
          x[0] += u.x; x[1] += u.y; x[2] += u.z; x[3] += u.w;
          x[4] += w.x; x[5] += w.y; x[6] += w.z; x[7] += w.w;
        }
      }
    }
    if (a.accum_in) {
      const float4* src = reinterpret_cast<const float4*>(a.G + off);
      const float4 u = src[0], w = src[1];
      x[0] += u.x; x[1] += u.y; x[2] += u.z; x[3] += u.w;
      x[4] += w.x; x[5] += w.y; x[6] += w.z; x[7] += w.w;
    }
    if (a.last && a.mom) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t widx = tr ? base + (int64_t)(col + e) * M + row : off + e;
        x[e] = fmaf(a.beta, a.mom[widx], x[e]);
        if (a.mom_write) a.mom[widx] = x[e];
      }
    }
    if (a.last && a.g32) {
      float4* dst = reinterpret_cast<float4*>(a.g32 + off);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    if (!a.last) {
      float4* dst = reinterpret_cast<float4*>(a.G + off);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else if (a.muon) {
      u16 h[8][3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += x[e] * x[e];
        split_planes(x[e], a.x.np, h[e]);
      }
      for (int q = 0; q < a.x.np; ++q) {
        uint4 w;
        w.x = h[0][q] | ((uint32_t)h[1][q] << 16);
        w.y = h[2][q] | ((uint32_t)h[3][q] << 16);
        w.z = h[4][q] | ((uint32_t)h[5][q] << 16);
        w.w = h[6][q] | ((uint32_t)h[7][q] << 16);
        *reinterpret_cast<uint4*>(a.x.base + q * a.x.plane_stride + (int64_t)zz * a.x.zstride +
                                  (int64_t)row * a.x.ld + col) = w;
      }
    } else if (tr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a.U[base + (int64_t)(col + e) * M + row] = x[e];
    } else {
      float4* dst = reinterpret_cast<float4*>(a.U + off);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
  if (a.last && a.muon) {
    const float t = block_sum(ss, red);
    if (threadIdx.x == 0) a.part[(int64_t)tz * CONTRACT_SUM_SUB + band] = t;
  }
}

// ------------------------------------------------------------------------ Newton-Schulz
__device__ __forceinline__ float ns_scale(const NsArgs& a, int zz) {
  return 1.f / (sqrtf(sum_parts(a.part + (int64_t)zz * a.nparts, a.nparts)) + a.eps);
}


// Store a tile of a symmetric M x M matrix computed at tile (ti, tj), ti <= tj, as planes
// of the full matrix (the symmetrised diagonal tile, or an upper tile and its mirror), NP
// planes per pass.
template <class G, int NP>
__device__ __forceinline__ void store_sym(const f32x16 (&v)[G::TM][G::TN], char* smem,
                                          const PlaneBuf& dst, int zz, int m0, int n0, int M,
                                          bool diag) {
  const int rl = min(G::TBM, M - m0), cl = min(G::TBN, M - n0);
  if (diag) store_planes<G, TILE_SYM, NP>(v, smem, dst, zz, m0, n0, rl, cl);
  else store_planes<G, TILE_BOTH, NP>(v, smem, dst, zz, m0, n0, rl, cl);
}

// A = s^2 X X^T: upper tiles computed; A planes written for the full symmetric matrix.
template <int T, int WGM, int WGN, int PL, int SP, int WGK>
__global__ __launch_bounds__(WGM * WGN * WGK * 64) void k_ns_gram(NsArgs a) {
  // swapped accumulator layout: runs of four columns, stored as 16-byte vectors
  using G = Gemm<T, T, WGM, WGN, PL, PL, 0, 0, PL, 64, true, WGK>;
  GEMM_LDS_EPI(G, (store_lds_bytes<G, TILE_BOTH, SP>()));
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int zz = lid / a.tiles;
  const int M = a.M;
  int ti, tj;
  tri_tile(lid % a.tiles, (M + T - 1) / T, ti, tj);
  const int m0 = ti * T, n0 = tj * T;
  Operand X[PL];
#pragma unroll
  for (int q = 0; q < PL; ++q) X[q] = plane_operand(a.xin, q, M);
  G g;
  g.zero();
  g.run(X, X, m0, n0, zz, a.N, GEMM_STAGES);
  g.reduce(smem);
  float s2 = 1.f;
  if (a.first) {
    const float s = ns_scale(a, zz);
    s2 = s * s;
  }
  if (a.first) {
    g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) g.acc[0][i][j][4 * q + e] *= s2;
    });
  }
  store_sym<G, SP>(g.acc[0], smem, a.aout, zz, m0, n0, M, ti == tj);
}

// B' = a I + b A + c A A  (A symmetric, so A serves as its own transposed operand); the
// a I term folds the iteration's a X into the update GEMM: X' = a X + B X = B' X.  Without
// fold the stage writes B = b A + c A A and the update adds a X itself (a one-plane B' would
// round a, and with it every row of X', to bf16).
template <int T, int WGM, int WGN, int PL, int SP, int WGK>
__global__ __launch_bounds__(WGM * WGN * WGK * 64) void k_ns_poly(NsArgs a) {
  // swapped accumulator layout: runs of four columns, read as 16-byte vectors
  using G = Gemm<T, T, WGM, WGN, PL, PL, 0, 0, PL, 64, true, WGK>;
  GEMM_LDS_EPI(G, (store_lds_bytes<G, TILE_BOTH, SP>()));
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int zz = lid / a.tiles;
  const int M = a.M;
  int ti, tj;
  tri_tile(lid % a.tiles, (M + T - 1) / T, ti, tj);
  const int m0 = ti * T, n0 = tj * T;
  Operand Ao[PL];
#pragma unroll
  for (int q = 0; q < PL; ++q) Ao[q] = plane_operand(a.ain, q, M);
  // The linear term b A reads A from its planes (the sum of the planes holds A to about
  // 16 significant bits with two planes, as the products do).  A(ti, tj) is the A-operand
  // tile of the K steps k0 in [n0, n0 + T): with K a multiple of the step, the K order is
  // rotated so that those are the last one or two steps, whose tiles the two stage buffers
  // still hold when the loop ends, and the epilogue reads A there instead of from memory.
  constexpr bool LDS_A = T == 128 && WGK == 1 && G::BK == 64;
  const int ncs = (min(n0 + T, M) - n0 + 63) / 64;   // steps that cover the tile's columns
  const bool from_lds = LDS_A && M % 64 == 0;
  const int krot = from_lds ? (n0 + 64 * ncs) % M : 0;
  G g;
  g.zero();
  g.run(Ao, Ao, m0, n0, zz, M, GEMM_STAGES, krot);
  g.reduce(smem);
  const int nk = M / 64;   // (from_lds only) steps of the loop; step t used stage t & 1
  const u16* ap = a.ain.base + (int64_t)zz * a.ain.zstride;
  g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
    const int R = m0 + r, C = n0 + c;
    float av[4] = {0.f, 0.f, 0.f, 0.f};
    if (R < M && C < M) {
      if (LDS_A && from_lds) {
        // column c lies in step nk - ncs + c / 64; row r, k-column c % 64 of its A tile
        const int t = nk - ncs + c / 64;
        const char* st = (t & 1) ? gemm_st1_ : gemm_st0_;
        const int kc = c % 64;
#pragma unroll
        for (int pq = 0; pq < PL; ++pq) {
          const uint2 h = *reinterpret_cast<const uint2*>(
              st + pq * G::A_TILE + r * 128 + (((kc >> 3) ^ swz_row<64>(r)) << 4) + (kc & 7) * 2);
          av[0] += bf2f((u16)(h.x & 0xFFFFu));
          av[1] += bf2f((u16)(h.x >> 16));
          av[2] += bf2f((u16)(h.y & 0xFFFFu));
          av[3] += bf2f((u16)(h.y >> 16));
        }
      } else {
#pragma unroll
        for (int pq = 0; pq < PL; ++pq) {
          const uint2 h = *reinterpret_cast<const uint2*>(ap + pq * a.ain.plane_stride +
                                                          (int64_t)R * a.ain.ld + C);
          av[0] += bf2f((u16)(h.x & 0xFFFFu));
          av[1] += bf2f((u16)(h.x >> 16));
          av[2] += bf2f((u16)(h.y & 0xFFFFu));
          av[3] += bf2f((u16)(h.y >> 16));
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = 0.f;
      if (R < M && C + e < M && (ti != tj || R <= C + e))
        x = a.coef_b * av[e] + a.coef_c * g.acc[0][i][j][4 * q + e] +
            (a.fold && R == C + e ? a.coef_a : 0.f);
      g.acc[0][i][j][4 * q + e] = x;
    }
  });
  store_sym<G, SP>(g.acc[0], smem, a.aout, zz, m0, n0, M, ti == tj);
}

// Store the tile v (swapped layout, already scaled) plus ca X as planes of dst, X being
// the sum of xin's XNP planes at the same place: the fp32 tile goes through LDS in passes
// of PR rows, and each thread then takes runs of 8 columns of one row, so that X is read,
// and the planes written, with 16-byte row-contiguous accesses.  Each pass issues its X
// loads before staging the tile, so their latency overlaps the LDS work.  smem needs
// PR (TBN + 4) 4 bytes.  Contains barriers: call from every thread.
template <class G, int PR, int XNP>
__device__ __forceinline__ void store_planes_lin(const f32x16 (&v)[G::TM][G::TN], char* smem,
                                                 const PlaneBuf& dst, const PlaneBuf& xin,
                                                 int z, int row0, int col0, int rlim, int clim,
                                                 float ca) {
  static_assert(G::SW, "runs of columns need the swapped layout");
  constexpr int TBN = G::TBN, LD = TBN + 4, CPR = TBN / 8;
  constexpr int ITER = (PR * CPR + G::NT - 1) / G::NT;   // row runs per thread and pass
  float* t = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int wm0 = G::wm0(), wn0 = G::wn0();
  const u16* const xz = xin.base + (int64_t)z * xin.zstride;
  u16* const dz = dst.base + (int64_t)z * dst.zstride;
#pragma unroll
  for (int p0 = 0; p0 < G::TBM; p0 += PR) {
    uint4 xv[ITER][XNP];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int ch = threadIdx.x + it * G::NT;
      const int rr = ch / CPR, cc = (ch % CPR) * 8;
      const bool ok = ch < PR * CPR && p0 + rr < rlim && cc < clim;
      const int64_t off = (int64_t)(row0 + p0 + rr) * xin.ld + col0 + cc;
#pragma unroll
      for (int q = 0; q < XNP; ++q)
        xv[it][q] = ok ? *reinterpret_cast<const uint4*>(xz + q * xin.plane_stride + off)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
    lds_barrier();
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (!G::owns(tm, tn, g)) continue;
          const int r = wm0 + tm * 32 + G::elem_row(4 * g, lane) - p0;
          const int c = wn0 + tn * 32 + G::elem_col(4 * g, lane);
          if (r >= 0 && r < PR)
            *reinterpret_cast<f32x4*>(t + r * LD + c) =
                f32x4{v[tm][tn][4 * g], v[tm][tn][4 * g + 1], v[tm][tn][4 * g + 2],
                      v[tm][tn][4 * g + 3]};
        }
    lds_barrier();
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int ch = threadIdx.x + it * G::NT;
      const int rr = ch / CPR, cc = (ch % CPR) * 8;
      const int gr = p0 + rr;
      if (ch >= PR * CPR || gr >= rlim || cc >= clim) continue;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(t + rr * LD + cc);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(t + rr * LD + cc + 4);
      const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      float lin[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < XNP; ++q) {
        const uint32_t w[4] = {xv[it][q].x, xv[it][q].y, xv[it][q].z, xv[it][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lin[2 * e] += bf2f((u16)(w[e] & 0xFFFFu));
          lin[2 * e + 1] += bf2f((u16)(w[e] >> 16));
        }
      }
      u16 hq[8][XNP];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = fmaf(ca, lin[e], x[e]);
#pragma unroll
        for (int q = 0; q < XNP; ++q) {
          hq[e][q] = f2bf(r);
          r -= bf2f(hq[e][q]);
        }
      }
      const int64_t off = (int64_t)(row0 + gr) * dst.ld + col0 + cc;
#pragma unroll
      for (int q = 0; q < XNP; ++q) {
        uint4 o;
        o.x = hq[0][q] | ((uint32_t)hq[1][q] << 16);
        o.y = hq[2][q] | ((uint32_t)hq[3][q] << 16);
        o.z = hq[4][q] | ((uint32_t)hq[5][q] << 16);
        o.w = hq[6][q] | ((uint32_t)hq[7][q] << 16);
        *reinterpret_cast<uint4*>(dz + q * dst.plane_stride + off) = o;
      }
    }
  }
  lds_barrier();
}

// X' = B' X, or X' = B X + a X without fold, a X taken from all of xin's planes
// (iteration 0: X = s G, with the scale s applied in the epilogue).
template <int BM, int BN, int WGM, int WGN, int PL, int BK, int SP, int WGK>
__global__ __launch_bounds__(WGM * WGN * WGK * 64) void k_ns_update(NsArgs a) {
  // X [M][N] read column-wise; swapped accumulator layout for packed plane stores
  using G = Gemm<BM, BN, WGM, WGN, PL, PL, 0, (1 << PL) - 1, PL, BK, true, WGK>;
  constexpr int LIN_ROWS = BM / 2;   // rows per LDS pass of the a X epilogue
  constexpr int EPI = store_lds_bytes<G, TILE_NORMAL, SP>() > LIN_ROWS * (BN + 4) * 4
                          ? store_lds_bytes<G, TILE_NORMAL, SP>()
                          : LIN_ROWS * (BN + 4) * 4;
  GEMM_LDS_EPI(G, EPI);
  const int lid = xcd_block(blockIdx.x, gridDim.x);
  const int zz = lid / a.tiles, tile = lid % a.tiles;
  const int M = a.M, N = a.N;
  const int m0 = (tile / a.tiles_n) * BM;
  const int n0 = (tile % a.tiles_n) * BN;
  Operand Ao[PL], Bo[PL];   // B' planes; X [M][N] planes read as their columns
#pragma unroll
  for (int q = 0; q < PL; ++q) {
    Ao[q] = plane_operand(a.ain, q, M);
    Bo[q] = plane_operand(a.xin, q, N);
  }
  G g;
  g.zero();
  g.run(Ao, Bo, m0, n0, zz, M, GEMM_STAGES);
  g.reduce(smem);
  const float sc = a.first ? ns_scale(a, zz) : 1.f;
  const int64_t base = (int64_t)zz * M * N;
  const int m = zz / a.P;
  const int tr = (a.tr_mask >> m) & 1;
  // runs of four columns (N is a multiple of 16, so a run lies wholly inside or outside):
  // U in the weight orientation is written as one 16-byte store per run, or transposed as
  // four 4-byte stores that consecutive lanes (consecutive rows) make contiguous
  const u16* const xp = a.xin.base + (int64_t)zz * a.xin.zstride;
  g.for_each4([&](int i, int j, int q, int r, int c) __attribute__((always_inline)) {
    const int R = m0 + r, C = n0 + c;
    const bool in = R < M && C < N;
    float lin[4] = {0.f, 0.f, 0.f, 0.f};
    if (!a.fold && a.last && in) {   // (otherwise a X is added by store_planes_lin)
      for (int pq = 0; pq < a.xin.np; ++pq) {
        const uint2 h = *reinterpret_cast<const uint2*>(xp + pq * a.xin.plane_stride +
                                                        (int64_t)R * a.xin.ld + C);
        lin[0] += bf2f((u16)(h.x & 0xFFFFu));
        lin[1] += bf2f((u16)(h.x >> 16));
        lin[2] += bf2f((u16)(h.y & 0xFFFFu));
        lin[3] += bf2f((u16)(h.y >> 16));
      }
    }
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = in ? sc * fmaf(a.coef_a, lin[e], g.acc[0][i][j][4 * q + e]) : 0.f;
      g.acc[0][i][j][4 * q + e] = x[e];
    }
    if (a.last && in) {
      if (tr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a.U[base + (int64_t)(C + e) * M + R] = x[e];
      } else {
        *reinterpret_cast<float4*>(a.U + base + (int64_t)R * N + C) =
            make_float4(x[0], x[1], x[2], x[3]);
      }
    }
  });
  if (!a.last) {
    const int rl = min(BM, M - m0), cl = min(BN, N - n0);
    if (a.fold)
      store_planes<G, TILE_NORMAL, SP>(g.acc[0], smem, a.xout, zz, m0, n0, rl, cl);
    else if (a.xin.np == 2)   // (one-plane iterates are always folded)
      store_planes_lin<G, LIN_ROWS, 2>(g.acc[0], smem, a.xout, a.xin, zz, m0, n0, rl, cl,
                                       a.coef_a * sc);
    else
      store_planes_lin<G, LIN_ROWS, 3>(g.acc[0], smem, a.xout, a.xin, zz, m0, n0, rl, cl,
                                       a.coef_a * sc);
  }
}

// ------------------------------------------------------------------------ renorm / update
// W <- keep W - lr U for every row of every matrix, then (renorm) each row back to its
// norm before the step; the bf16 planes of the new W for the next chunk's GEMMs.  One wave
// per row (rows of all problems flattened): the row's W and U are held in registers (CPL
// 16-byte chunks per lane, rows of up to 256 CPL values), so each is read once and
// written once with 16-byte accesses.  Both norms are summed by the same code over the
// same element order, so a zero update with no decay leaves the row bit-exact.  With U
// null only the planes are refreshed.
template <int CPL>
__global__ __launch_bounds__(256) void k_renorm(RenormArgs a) {
  const int m = blockIdx.y;
  const RenormMat& M = a.m[m];
  const int lane = threadIdx.x & 63;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gr >= M.rows * a.P) return;
  const int n4 = M.cols / 4;   // 16-byte chunks in the row (cols is a multiple of 16)
  float4* w = reinterpret_cast<float4*>(M.W + (int64_t)gr * M.cols);
  float4 x[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int i = lane + 64 * k;
    x[k] = i < n4 ? w[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (M.U) {
    const float4* u = reinterpret_cast<const float4*>(M.U + (int64_t)gr * M.cols);
    const float keep = a.keep, step = M.lr;
    float so = 0.f, sn = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int i = lane + 64 * k;
      const float4 d = i < n4 ? u[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 y = make_float4(fmaf(-step, d.x, keep * x[k].x), fmaf(-step, d.y, keep * x[k].y),
                                   fmaf(-step, d.z, keep * x[k].z), fmaf(-step, d.w, keep * x[k].w));
      // explicit fused steps in one order for both sums, so that y == x gives so == sn
      so = fmaf(x[k].w, x[k].w, fmaf(x[k].z, x[k].z, fmaf(x[k].y, x[k].y, fmaf(x[k].x, x[k].x, so))));
      sn = fmaf(y.w, y.w, fmaf(y.z, y.z, fmaf(y.y, y.y, fmaf(y.x, y.x, sn))));
      x[k] = y;
    }
    so = wave_sum(so);
    sn = wave_sum(sn);
    float scale = 1.f;
    if (a.renorm && sn > 0.f) scale = sqrtf(so) / sqrtf(sn);
    if (lane == 0 && (!isfinite(so) || !isfinite(sn))) *a.health = 1;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int i = lane + 64 * k;
      x[k] = make_float4(x[k].x * scale, x[k].y * scale, x[k].z * scale, x[k].w * scale);
      if (i < n4) w[i] = x[k];
    }
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int i = lane + 64 * k;
    if (i >= n4) continue;
    u16 h[4][3];
    split_planes(x[k].x, a.np, h[0]);
    split_planes(x[k].y, a.np, h[1]);
    split_planes(x[k].z, a.np, h[2]);
    split_planes(x[k].w, a.np, h[3]);
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q < a.np) {
        uint2 v;
        v.x = h[0][q] | ((uint32_t)h[1][q] << 16);
        v.y = h[2][q] | ((uint32_t)h[3][q] << 16);
        *reinterpret_cast<uint2*>(M.pl + q * M.pl_stride + (int64_t)gr * M.cols + 4 * i) = v;
      }
  }
}

// Token rows [n][d] (activation dtype) -> bf16 planes in the same layout, optionally with
// row t scaled by -eta_t.
__device__ __forceinline__ void split_rows(const SplitArgs& a) {
  const int z = blockIdx.y;
  const int64_t total = (int64_t)a.n * a.d;
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    float x = load_act(a.x, (int64_t)z * a.x_zstride + e, a.x_bf16);
    if (a.neg_eta) x *= -a.eta[(int64_t)z * a.eta_zstride + e / a.d];
    put_planes(a.out, z, e, x);
  }
}

__global__ __launch_bounds__(256) void k_split(SplitArgs a) { split_rows(a); }

// two tensors of the same shape in one launch (blockIdx.z picks the tensor)
__global__ __launch_bounds__(256) void k_split2(SplitArgs a, SplitArgs b) {
  if (blockIdx.z == 0) split_rows(a);
  else split_rows(b);
}

// three tensors of the same shape in one launch
__global__ __launch_bounds__(256) void k_split3(SplitArgs a, SplitArgs b, SplitArgs c) {
  if (blockIdx.z == 0) split_rows(a);
  else if (blockIdx.z == 1) split_rows(b);
  else split_rows(c);
}

// ============================================================================ launchers
// Every GEMM kernel holds its LDS in static __shared__ arrays (GEMM_LDS): launches pass no
// dynamic LDS.

template <int BM, int BN, int WGM, int WGN, int FW, int MODE, int BK = 64, int PR = 0>
static hipError_t front_t(const FrontArgs& a0, int Z, hipStream_t s) {
  using G = typename FrontGemm<BM, BN, WGM, WGN, FW, MODE, BK, PR>::type;
  FrontArgs a = a0;
  auto kern = k_front<BM, BN, WGM, WGN, FW, MODE, BK, PR>;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int tiles_m = (a.nrows + BM - 1) / BM;
  a.tiles = tiles_m * a.tiles_n;
  if (a.tiles == 0 || Z == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(a.tiles * Z), dim3(G::NT), 0, s, a);
  return hipGetLastError();
}

// Fronts step K by 32, which keeps their LDS low enough for two workgroups per CU (61 KB
// for the SwiGLU apply front), except the SwiGLU inner-product gradient front: its three
// accumulators limit it to one workgroup per CU, and it keeps steps of 64.
template <int FW, int MODE>
static hipError_t front_fm(const FrontArgs& a, int Z, hipStream_t s) {
  return front_t<128, 128, 2, 4, FW, MODE, 32>(a, Z, s);
}

// A launch with fewer 128 x 128 tiles than CUs (few tokens, or a narrow hidden layer) takes
// 64 x 64 tiles on four waves: four times the workgroups, each with a quarter of the tile's
// loads per K step and of its epilogue's stores.
constexpr int SMALL_TILE_BELOW = 256;
static bool small_tiles(int rows, int cols, int Z) {
  return (int64_t)((rows + 127) / 128) * ((cols + 127) / 128) * Z < SMALL_TILE_BELOW;
}

hipError_t launch_front(int fw, int mode, const FrontArgs& a, int Z, hipStream_t s) {
  if (fw == FW_SWIGLU) {
    const bool small = small_tiles(a.nrows, a.N, Z);
    // small launches whose operands all hold the same number (2 or 3) of planes: the
    // plane-resident grouped product (the key-row front steps K by 32 for LDS)
    const int na = mode == FRONT_K_DOT ? 2 : 1, nb = mode == FRONT_K_DOT ? 3 : 2;
    int pr = a.A[0].planes;
    for (int i = 0; i < na; ++i) pr = a.A[i].planes == pr ? pr : 0;
    for (int i = 0; i < nb; ++i) pr = a.B[i].planes == pr ? pr : 0;
    if (!small || pr < 2) pr = 0;
    if (mode == FRONT_Q) {
      if (pr == 2) return front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_Q, 64, 2>(a, Z, s);
      if (pr == 3) return front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_Q, 64, 3>(a, Z, s);
      return small ? front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_Q, 64>(a, Z, s)
                   : front_fm<FW_SWIGLU, FRONT_Q>(a, Z, s);
    }
    if (mode == FRONT_K_DOT) {
      if (pr == 2) return front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_K_DOT, 32, 2>(a, Z, s);
      if (pr == 3) return front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_K_DOT, 32, 3>(a, Z, s);
      return small ? front_t<64, 64, 2, 2, FW_SWIGLU, FRONT_K_DOT>(a, Z, s)
                   : front_t<128, 128, 2, 4, FW_SWIGLU, FRONT_K_DOT>(a, Z, s);
    }
    return front_fm<FW_SWIGLU, FRONT_K_MSE>(a, Z, s);
  }
  if (mode == FRONT_Q) return front_fm<FW_GELU, FRONT_Q>(a, Z, s);
  if (mode == FRONT_K_DOT) return front_fm<FW_GELU, FRONT_K_DOT>(a, Z, s);
  return front_fm<FW_GELU, FRONT_K_MSE>(a, Z, s);
}

template <int MODE, int BM = 128, int BN = 128, int WGM = 2, int WGN = 4>
static hipError_t out_m(const OutArgs& a0, int Z, hipStream_t s, int pr = 0) {
  using G = Gemm<BM, BN, WGM, WGN, 1, 1, 0, MODE == DH_MSE ? 1 : 0>;
  OutArgs a = a0;
  auto kern = k_out<BM, BN, WGM, WGN, MODE>;
  if constexpr (MODE == OUT_Q && BM == 64) {   // (small tiles only: LDS of all planes)
    if (pr == 2) kern = k_out<BM, BN, WGM, WGN, MODE, 2>;
    if (pr == 3) kern = k_out<BM, BN, WGM, WGN, MODE, 3>;
  }
  a.tiles_n = (a.N + BN - 1) / BN;
  const int tiles_m = (a.nrows + BM - 1) / BM;
  a.tiles = tiles_m * a.tiles_n;
  if (a.tiles == 0 || Z == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(a.tiles * Z), dim3(G::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dq(const DqArgs& a0, int np, int Z, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  using G = Gemm<BM, BN, 2, 4, 1, 1>;   // block size
  DqArgs a = a0;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.nrows + BM - 1) / BM) * a.tiles_n;
  if (a.tiles == 0 || Z == 0) return hipSuccess;
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  auto kern = np == 2 ? k_dq<BM, BN, 2, 4, 2> : k_dq<BM, BN, 2, 4, 1>;
  hipLaunchKernelGGL(kern, dim3(a.tiles * Z), dim3(G::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_out(int mode, const OutArgs& a, int Z, hipStream_t s) {
  if (mode == OUT_Q)
    // small launches with several planes on both sides take the plane-resident product
    return small_tiles(a.nrows, a.N, Z)
               ? out_m<OUT_Q, 64, 64, 2, 2>(a, Z, s, a.a.planes == a.b.planes ? a.a.planes : 0)
               : out_m<OUT_Q>(a, Z, s);
  if (mode == OUT_K_MSE) return out_m<OUT_K_MSE>(a, Z, s);
  return out_m<DH_MSE>(a, Z, s);
}

// Token ranges: enough for about two workgroups per CU (256 CUs) when the output tiles
// alone are fewer, at most CONTRACT_SPLIT_MAX, each range at least 128 tokens.
constexpr int CONTRACT_SLOTS = 512, CONTRACT_RANGE_MIN = 128;

int contract_split_max(int tiles, int nz) {
  const int64_t wgs = (int64_t)tiles * nz;
  if (wgs <= 0) return 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>(CONTRACT_SPLIT_MAX, CONTRACT_SLOTS / wgs));
}

// plane counts 1 x 2, 1 x 3, 2 x 1, 3 x 1, 2 x 2 and 3 x 3: plane-resident (NA + NB tiles a
// K step instead of two per plane product, one pass over the K range instead of one per
// pair); one plane on both sides is a single product; other mixes run plane pairs as K
// segments
template <int BM>
static void (*contract_kernel(int pa, int pb))(ContractArgs) {
  constexpr int BN = CONTRACT_BN;
  if (pa == 1 && pb == 2) return k_contract<BM, BN, 2, 4, 1, 2>;
  if (pa == 1 && pb == 3) return k_contract<BM, BN, 2, 4, 1, 3>;
  if (pa == 2 && pb == 1) return k_contract<BM, BN, 2, 4, 2, 1>;
  if (pa == 3 && pb == 1) return k_contract<BM, BN, 2, 4, 3, 1>;
  if (pa == 2 && pb == 2) return k_contract<BM, BN, 2, 4, 2, 2>;
  if (pa == 3 && pb == 3) return k_contract<BM, BN, 2, 4, 3, 3>;
  return k_contract<BM, BN, 2, 4, 0, 0>;
}

hipError_t launch_contract(const ContractArgs& a0, int nm, hipStream_t s) {
  constexpr int BN = CONTRACT_BN;
  using G = Gemm<CONTRACT_BM, BN, 2, 4, 1, 1, 1, 1>;   // block size (the same for every instance)
  ContractArgs a = a0;
  const int pa = a.a[0].planes, pb = a.b[0].planes;
  // matrices of at most 64 rows (dim 64) take 64-row tiles: the same tiles (one row of
  // them) without the 64 rows of padding a 128-row tile would carry through the MFMAs
  const bool rows64 = a.M <= 64;
  const int BM = rows64 ? 64 : CONTRACT_BM;
  auto kern = rows64 ? contract_kernel<64>(pa, pb) : contract_kernel<CONTRACT_BM>(pa, pb);
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles = ((a.M + BM - 1) / BM) * a.tiles_n;
  a.nz = nm * a.P;
  if (a.tiles == 0 || a.nz == 0 || a.K <= 0) return hipSuccess;
  // a split's second pass stores CONTRACT_SUM_SUB parts per tile
  int ks = std::min(a.gpart && a.psub == CONTRACT_SUM_SUB ? a.ksplit : 1,
                    contract_split_max(a.tiles, a.nz));
  ks = std::max(1, std::min(ks, a.K / CONTRACT_RANGE_MIN));
  a.kchunk = ks > 1 ? (((a.K + ks - 1) / ks + 63) / 64) * 64 : a.K;
  a.ksplit = (a.K + a.kchunk - 1) / a.kchunk;
  hipLaunchKernelGGL(kern, dim3(a.tiles * a.nz * a.ksplit), dim3(G::NT), 0, s, a);
  if (a.ksplit > 1) {
    // the tiles are those of 128 rows either way (one row of them when rows64)
    auto sum = k_contract_sum<CONTRACT_BM, BN>;
    hipLaunchKernelGGL(sum, dim3(a.tiles * a.nz * CONTRACT_SUM_SUB), dim3(CONTRACT_SUM_THREADS),
                       0, s, a);
  }
  return hipGetLastError();
}

int ns_tri_tiles(int M, int tile) {
  const int t = (M + tile - 1) / tile;
  return t * (t + 1) / 2;
}

// One Newton-Schulz stage (0 Gram, 1 polynomial, 2 update) on T x T tiles of WGM x WGN
// waves, storing SP planes per pass; the update steps K by BK.
template <int T, int STAGE, int PL, int WGM = 2, int WGN = (T >= 128 ? 4 : 2), int BK = 64,
          int SP = PL, int WGK = 1>
static hipError_t ns_t(const NsArgs& a0, hipStream_t s) {
  NsArgs a = a0;
  if (a.Z == 0) return hipSuccess;
  if constexpr (STAGE == 2) {
    using G = Gemm<T, T, WGM, WGN, PL, PL, 0, (1 << PL) - 1, PL, BK, true, WGK>;
    a.tiles_n = (a.N + T - 1) / T;
    a.tiles = ((a.M + T - 1) / T) * a.tiles_n;
    auto kern = k_ns_update<T, T, WGM, WGN, PL, BK, SP, WGK>;
    hipLaunchKernelGGL(kern, dim3(a.tiles * a.Z), dim3(G::NT), 0, s, a);
  } else {
    using G = Gemm<T, T, WGM, WGN, PL, PL, 0, 0, PL, 64, true, WGK>;
    a.tiles = ns_tri_tiles(a.M, T);
    const dim3 grid(a.tiles * a.Z);
    if constexpr (STAGE == 0) {
      auto kern = k_ns_gram<T, WGM, WGN, PL, SP, WGK>;
      hipLaunchKernelGGL(kern, grid, dim3(G::NT), 0, s, a);
    } else {
      auto kern = k_ns_poly<T, WGM, WGN, PL, SP, WGK>;
      hipLaunchKernelGGL(kern, grid, dim3(G::NT), 0, s, a);
    }
  }
  return hipGetLastError();
}

// the plane count of the iteration's operands picks the plane-resident instantiation
template <int T, int STAGE>
static hipError_t ns_planes(const NsArgs& a, int np, hipStream_t s) {
  if (np == 1) return ns_t<T, STAGE, 1>(a, s);
  if (np == 2) return ns_t<T, STAGE, 2>(a, s);
  if (np == 3) return ns_t<T, STAGE, 3>(a, s);
  return hipErrorInvalidValue;
}

// The Gram and polynomial stages take 128x128 upper tiles (sixteen waves of 32x32 tiles,
// four a SIMD, one plane per store pass) when the operands have at most two planes and
// the launch has enough such tiles to cover most CUs.  Else they take 64x64 upper tiles
// on eight waves: two groups of 2 x 2 waves, each group taking half of every K step,
// whose partial tiles are summed through LDS before the epilogue (such launches have
// fewer workgroups than CUs, so each workgroup's time is the stage's time).
static bool ns_sym_wide(const NsArgs& a, int np) {
  return np <= 2 && (int64_t)ns_tri_tiles(a.M, 128) * a.Z >= 192;
}
template <int STAGE>
static hipError_t ns_sym(const NsArgs& a, int np, hipStream_t s) {
  if (ns_sym_wide(a, np))
    return np == 1 ? ns_t<128, STAGE, 1, 4, 4, 64, 1>(a, s)
                   : ns_t<128, STAGE, 2, 4, 4, 64, 1>(a, s);
  if (np == 1) return ns_t<64, STAGE, 1, 2, 2, 64, 1, 2>(a, s);
  if (np == 2) return ns_t<64, STAGE, 2, 2, 2, 64, 2, 2>(a, s);
  if (np == 3) return ns_t<64, STAGE, 3, 2, 2, 64, 3, 2>(a, s);
  return hipErrorInvalidValue;
}
hipError_t launch_ns_gram(const NsArgs& a, hipStream_t s) {
  if (a.pl > a.xin.np || a.aout.np != a.pl) return hipErrorInvalidValue;
  return ns_sym<0>(a, a.pl, s);
}
hipError_t launch_ns_poly(const NsArgs& a, hipStream_t s) {
  if (a.ain.np != a.pl || a.aout.np != a.pl) return hipErrorInvalidValue;
  return ns_sym<1>(a, a.pl, s);
}
// The update takes 128x128 tiles when they give at least two workgroups per CU (256 CUs)
// and the operands have at most two planes (three would not fit LDS); else 64x64 tiles.
// With two planes the 128x128 kernel steps K by 32 and stores one plane per pass, which
// keeps its LDS at 66 KB: two workgroups share a CU, one's epilogue overlapping the
// other's main loop.
hipError_t launch_ns_update(const NsArgs& a, hipStream_t s) {
  const int64_t big = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.Z;
  if (a.ain.np != a.pl || a.pl > a.xin.np || (!a.last && a.xout.np != a.xin.np))
    return hipErrorInvalidValue;
  // three planes: 64x64 tiles stepping K by 32 (52 KB of LDS, three workgroups per CU)
  if (a.pl == 3) return ns_t<64, 2, 3, 2, 2, 32, 3>(a, s);
  if (big < 512) return ns_planes<64, 2>(a, a.pl, s);
  return a.pl == 1 ? ns_t<128, 2, 1>(a, s) : ns_t<128, 2, 2, 2, 4, 32, 1>(a, s);
}

hipError_t launch_renorm(const RenormArgs& a, hipStream_t s) {
  if (a.P == 0 || a.nm == 0) return hipSuccess;
  int cols = 0;
  for (int m = 0; m < a.nm; ++m) cols = std::max(cols, a.m[m].cols);
  const dim3 grid((a.max_rows * a.P + 3) / 4, a.nm);
  if (cols <= 256) hipLaunchKernelGGL(k_renorm<1>, grid, dim3(256), 0, s, a);
  else if (cols <= 512) hipLaunchKernelGGL(k_renorm<2>, grid, dim3(256), 0, s, a);
  else if (cols <= 1024) hipLaunchKernelGGL(k_renorm<4>, grid, dim3(256), 0, s, a);
  else if (cols <= 2048) hipLaunchKernelGGL(k_renorm<8>, grid, dim3(256), 0, s, a);
  else if (cols <= 4096) hipLaunchKernelGGL(k_renorm<16>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
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

hipError_t launch_split2(const SplitArgs& a, const SplitArgs& b, int Z, hipStream_t s) {
  if (a.n != b.n || a.d != b.d) return hipErrorInvalidValue;
  if (Z == 0 || a.n == 0) return hipSuccess;
  int64_t total = (int64_t)a.n * a.d;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_split2, dim3(blocks, Z, 2), dim3(256), 0, s, a, b);
  return hipGetLastError();
}

hipError_t launch_split3(const SplitArgs& a, const SplitArgs& b, const SplitArgs& c, int Z,
                         hipStream_t s) {
  if (a.n != b.n || a.d != b.d || a.n != c.n || a.d != c.d) return hipErrorInvalidValue;
  if (Z == 0 || a.n == 0) return hipSuccess;
  int64_t total = (int64_t)a.n * a.d;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_split3, dim3(blocks, Z, 3), dim3(256), 0, s, a, b, c);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_zero(int* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

hipError_t launch_fill_zero(int* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3(std::min(1024, (n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t prepare_kernels() { return hipSuccess; }

}  // namespace ttt
