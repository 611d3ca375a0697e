// Device-side building blocks for gfx950 (CDNA4): bf16 planes, MFMA tile GEMM main loop,
// wavefront reductions.  Everything here is written for 64-lane wavefronts and the
// v_mfma_f32_32x32x16_bf16 matrix instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------------ bf16 helpers
__device__ __forceinline__ u16 f2bf(float x) {
  __bf16 b = static_cast<__bf16>(x);   // round to nearest even
  return __builtin_bit_cast(u16, b);
}
__device__ __forceinline__ float bf2f(u16 h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// Split x into `np` bf16 planes whose sum approximates x: plane 0 = bf16(x), plane i the
// bf16 rounding of what the earlier planes left (each difference is exact in fp32).
__device__ __forceinline__ void split_planes(float x, int np, u16 out[3]) {
  float r = x;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i < np) {
      u16 h = f2bf(r);
      out[i] = h;
      r = r - bf2f(h);
    }
  }
}

// ------------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------------------ GEMM operands
// A K-contiguous operand made of 1..3 bf16 planes: element (r, k) of problem z lives at
// p[plane][z * zstride + r * ld + k].  Rows >= rows and k >= K read as zero.
struct Operand {
  const u16* p[3];
  int64_t ld;
  int64_t zstride;
  int32_t planes;
  int32_t rows;
};

__host__ __device__ inline Operand make_operand(const u16* p0, const u16* p1, const u16* p2,
                                                int64_t ld, int64_t zstride, int planes,
                                                int rows) {
  Operand o;
  o.p[0] = p0; o.p[1] = p1; o.p[2] = p2;
  o.ld = ld; o.zstride = zstride; o.planes = planes; o.rows = rows;
  return o;
}

// Multi-product tile GEMM main loop.
//   NA A-operands (tile rows = M), NB B-operands (tile rows = N), NP products; product p
//   accumulates  C_p[m][n] += sum_k A_{IA[p]}[m][k] * B_{IB[p]}[n][k]  over all plane pairs
//   (i, j) with i + j < max(planes of A_{IA[p]}, planes of B_{IB[p]}).
// Block: 256 threads = 4 waves in a 2 x 2 layout; wave tile (BM/2) x (BN/2) made of 32x32
// MFMA tiles.  K is walked in steps of 32 through two LDS buffers (double buffering with
// a register prefetch of the next step's global loads).  LDS rows are padded to 80 bytes
// so that the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
template <int BM, int BN, int NA, int NB>
struct TileShape {
  static constexpr int BK = 32;
  static constexpr int BKP = 40;                 // padded row length in elements
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int CA = BM * 4 / 256;        // 16-byte chunks per thread per A plane
  static constexpr int CB = BN * 4 / 256;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes are multiples of 64");
  // LDS bytes for one buffer with the given plane counts
  __host__ __device__ static int stage_bytes(const int* pa, const int* pb) {
    int n = 0;
    for (int i = 0; i < NA; ++i) n += pa[i] * BM * BKP * 2;
    for (int i = 0; i < NB; ++i) n += pb[i] * BN * BKP * 2;
    return n;
  }
};

template <int BM, int BN, int NA, int NB, int NP>
struct MultiGemm {
  using S = TileShape<BM, BN, NA, NB>;
  static constexpr int BK = S::BK, BKP = S::BKP, TM = S::TM, TN = S::TN;
  static constexpr int CA = S::CA, CB = S::CB;

  f32x16 acc[NP][TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[p][i][j][v] = 0.f;
  }

  // Run the K loop.  A[] / B[] describe the operands, m0 / n0 the tile origin, z the
  // problem index, K the contraction length (a multiple of 8), smem the dynamic LDS.
  __device__ __forceinline__ void run(const Operand (&A)[NA], const Operand (&B)[NB],
                                      const int (&IA)[NP], const int (&IB)[NP], int m0,
                                      int n0, int z, int K, char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave >> 1) * S::WM;
    const int wn0 = (wave & 1) * S::WN;

    int pa[NA], pb[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = A[i].planes;
#pragma unroll
    for (int i = 0; i < NB; ++i) pb[i] = B[i].planes;
    const int stage = S::stage_bytes(pa, pb);

    // byte offsets of each operand-plane tile inside one LDS stage
    int offA[NA][3], offB[NB][3];
    {
      int o = 0;
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          offA[i][q] = o;
          if (q < pa[i]) o += BM * BKP * 2;
        }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          offB[i][q] = o;
          if (q < pb[i]) o += BN * BKP * 2;
        }
    }

    uint4 ra[NA][3][CA];
    uint4 rb[NB][3][CB];

    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int c = 0; c < CA; ++c) {
            if (q < pa[i]) {
              const int ch = tid + c * 256;
              const int r = ch >> 2, kc = (ch & 3) * 8;
              const int gr = m0 + r, gk = k0 + kc;
              uint4 v = make_uint4(0, 0, 0, 0);
              if (gr < A[i].rows && gk < K)
                v = *reinterpret_cast<const uint4*>(A[i].p[q] + (int64_t)z * A[i].zstride +
                                                    (int64_t)gr * A[i].ld + gk);
              ra[i][q][c] = v;
            }
          }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int c = 0; c < CB; ++c) {
            if (q < pb[i]) {
              const int ch = tid + c * 256;
              const int r = ch >> 2, kc = (ch & 3) * 8;
              const int gr = n0 + r, gk = k0 + kc;
              uint4 v = make_uint4(0, 0, 0, 0);
              if (gr < B[i].rows && gk < K)
                v = *reinterpret_cast<const uint4*>(B[i].p[q] + (int64_t)z * B[i].zstride +
                                                    (int64_t)gr * B[i].ld + gk);
              rb[i][q][c] = v;
            }
          }
    };
    auto sstore = [&](char* buf) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int c = 0; c < CA; ++c) {
            if (q < pa[i]) {
              const int ch = tid + c * 256;
              const int r = ch >> 2, kc = (ch & 3) * 8;
              *reinterpret_cast<uint4*>(buf + offA[i][q] + (r * BKP + kc) * 2) = ra[i][q][c];
            }
          }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int c = 0; c < CB; ++c) {
            if (q < pb[i]) {
              const int ch = tid + c * 256;
              const int r = ch >> 2, kc = (ch & 3) * 8;
              *reinterpret_cast<uint4*>(buf + offB[i][q] + (r * BKP + kc) * 2) = rb[i][q][c];
            }
          }
    };
    auto compute = [&](const char* buf) {
      const int fr = lane & 31;
      const int fk = (lane >> 5) * 8;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8 fa[NA][3][TM];
        bf16x8 fb[NB][3][TN];
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
          for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int t = 0; t < TM; ++t)
              if (q < pa[i])
                fa[i][q][t] = *reinterpret_cast<const bf16x8*>(
                    buf + offA[i][q] + ((wm0 + t * 32 + fr) * BKP + s * 16 + fk) * 2);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int t = 0; t < TN; ++t)
              if (q < pb[i])
                fb[i][q][t] = *reinterpret_cast<const bf16x8*>(
                    buf + offB[i][q] + ((wn0 + t * 32 + fr) * BKP + s * 16 + fk) * 2);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int ia = IA[p], ib = IB[p];
          const int P = pa[ia] > pb[ib] ? pa[ia] : pb[ib];
#pragma unroll
          for (int qi = 0; qi < 3; ++qi)
#pragma unroll
            for (int qj = 0; qj < 3; ++qj) {
              if (qi < pa[ia] && qj < pb[ib] && qi + qj < P) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                  for (int tn = 0; tn < TN; ++tn)
                    acc[p][tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fa[ia][qi][tm], fb[ib][qj][tn], acc[p][tm][tn], 0, 0, 0);
              }
            }
        }
      }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk == 0) return;
    gload(0);
    sstore(smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = smem + (kt & 1) * stage;
      char* nxt = smem + ((kt + 1) & 1) * stage;
      if (kt + 1 < nk) gload((kt + 1) * BK);
      compute(cur);
      if (kt + 1 < nk) sstore(nxt);
      __syncthreads();
    }
  }

  // Visit every accumulator element owned by this thread:
  //   f(tm, tn, v, row, col)  with row/col relative to the block tile origin.
  // Element v of a 32x32 MFMA tile sits at row 8*(v/4) + 4*(lane/32) + v%4, col lane%32.
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave >> 1) * S::WM;
    const int wn0 = (wave & 1) * S::WN;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm0 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn0 + tn * 32 + (lane & 31);
          f(tm, tn, v, row, col);
        }
  }
};

}  // namespace ttt
