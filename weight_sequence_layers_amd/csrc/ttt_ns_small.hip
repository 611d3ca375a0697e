// Newton-Schulz orthogonalisation of small matrices in one launch: every iteration of one
// matrix in one workgroup, its iterates kept in LDS.
//
// The iteration is the quintic of the Muon step ([LaCT] §2.2, the update's orthogonalised
// gradient): X0 = G / (|G|_F + eps), then per iteration A = X X^T, B = b A + c A A and
// X' = a X + B X.  The staged path runs it as three GEMM launches per iteration, which for
// matrices of a few tens of thousands of elements are bound by each launch's latency; here
// one workgroup of eight waves holds the whole matrix (X up to 64 x 128) and its A and B as
// bf16 planes in LDS and runs every product on the MFMA from there.  The roundings are the
// staged path's: A and B are stored on the iteration's product planes, X' on the iterate
// planes, the linear term a X is folded into B as a I when the products keep the iterate's
// precision and otherwise added from all of the iterate's planes, and the 1 / (|G|_F + eps)
// scale enters the first Gram product squared and the first update once.
#include "ttt_internal.h"

namespace ttt {
namespace {

constexpr int SM = NS_SMALL_M, SN = NS_SMALL_N;
constexpr int XS = SN + 8;   // row stride of X planes in LDS (elements): 272 bytes
constexpr int AS = SM + 8;   // row stride of A and B planes: 144 bytes

// A-operand (or row-read B-operand) fragment: rows row0 + lane % 32, k = k0 + 8 (lane / 32)
// .. + 7 of a row-major LDS array with row stride `stride` elements.
__device__ __forceinline__ bf16x8 frag_rows(const u16* base, int stride, int row0, int k0) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 31)) * stride + k0 +
                                          8 * (lane >> 5));
}

// B-operand fragment of a row-major [k][n] LDS array: column n0 + lane % 32, k = k0 + 8
// (lane / 32) .. + 7, by two transposing reads (within each 16-lane group, lane j receives
// element j % 4 of the 4-element rows addressed by lanes 4 e + j / 4; lane 4 e + q addresses
// row kb + e at column base + 4 q, so lane j gets rows kb .. kb + 3 of column base + j).
__device__ __forceinline__ bf16x8 frag_cols(const u16* base, int stride, int n0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int m = n0 + 16 * (g & 1) + 4 * (j & 3);
  const int kb = k0 + 8 * (g >> 1) + (j >> 2);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + kb * stride + m));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + (kb + 4) * stride + m));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 1 / (|G|_F + eps) from the per-tile sums of squares the contraction left for matrix z
__device__ __forceinline__ float ns_scale_of(const float* part, int nparts, float eps, int z) {
  float t = 0.f;
  for (int i = 0; i < nparts; ++i) t += part[(int64_t)z * nparts + i];
  return 1.f / (sqrtf(t) + eps);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Store the fp32 tile value x at (r, c) as `np` planes into planes[q][r * stride + c].
__device__ __forceinline__ void put_planes(u16* planes, int pstride, int np, int stride, int r,
                                           int c, float x) {
  u16 h[3];
  split_planes(x, np, h);
#pragma unroll
  for (int q = 0; q < 3; ++q)
    if (q < np) planes[q * pstride + r * stride + c] = h[q];
}

// Partial 32 x 32 tile (ti, tj) of an A B^T-shaped product, both operands read as rows,
// over k in [k0, k0 + KL) and the plane pairs (qa, qb), qa + qb < PK.
template <int PK, int KL>
__device__ __forceinline__ f32x16 prod_rows(const u16* A, int apst, int astr, const u16* B,
                                            int bpst, int bstr, int ti, int tj, int k0) {
  f32x16 acc = f32x16{};
#pragma unroll
  for (int qa = 0; qa < PK; ++qa)
#pragma unroll
    for (int qb = 0; qb + qa < PK; ++qb)
#pragma unroll
      for (int k = 0; k < KL; k += 16)
        acc = mfma(frag_rows(A + qa * apst, astr, 32 * ti, k0 + k),
                   frag_rows(B + qb * bpst, bstr, 32 * tj, k0 + k), acc);
  return acc;
}

// Waves 4..7 hand their partial tiles (NT of them) to waves 0..3 through red (run j of four
// values of wave tile t at red + ((t 4 NT + j) 64 + lane) 4: consecutive lanes, consecutive
// 16 bytes); returns with the sums in the accumulators of waves 0..3.  w is wave-uniform.
// Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ void reduce_halves(f32x16 (&acc)[NT], float* red, int w, int lane) {
  float* slot = red + ((w & 3) * 4 * NT * 64 + lane) * 4;
  if (w >= 4) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int v = 0; v < 16; v += 4)
        *reinterpret_cast<f32x4*>(slot + (4 * u + v / 4) * 256) =
            f32x4{acc[u][v], acc[u][v + 1], acc[u][v + 2], acc[u][v + 3]};
  }
  __syncthreads();
  if (w < 4) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(slot + (4 * u + v / 4) * 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[u][v + e] += x[e];
      }
  }
}

// One iteration with PK product planes (PK = NP folds a I into B).  Eight waves: wave w
// computes tile w & 3 of each product over half of its K range (w >> 2 picks the half),
// and waves 0..3 finish the tiles.  No element needs a bounds check in LDS: X is zero
// outside [M][N], so A is zero outside [M][M], B outside [M][M] but for a on the padded
// diagonal (which multiplies zero rows of X), and X' is zero outside [M][N] again; only
// the store of U to memory checks.
template <int NP, int PK>
__device__ __forceinline__ void ns_iteration(const NsArgs& a, u16* xs, u16* as_, u16* bs,
                                             float* red, int z, float s, bool first,
                                             bool last) {
  constexpr bool fold = PK == NP;
  const int M = a.M, N = a.N;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wt = w & 3, kh = w >> 2;
  const int ti = wt >> 1, tj = wt & 1;

  // A = X X^T (s^2 G G^T in the first iteration)
  {
    f32x16 acc[1] = {prod_rows<PK, SN / 2>(xs, SM * XS, XS, xs, SM * XS, XS, ti, tj,
                                           kh * (SN / 2))};
    reduce_halves<1>(acc, red, w, lane);
    if (w < 4) {
      const float s2 = first ? s * s : 1.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * ti + 8 * (v >> 2) + 4 * hl + (v & 3), c = 32 * tj + (lane & 31);
        put_planes(as_, SM * AS, PK, AS, r, c, acc[0][v] * s2);
      }
    }
  }
  __syncthreads();

  // B = b A + c A A (+ a I folded), the linear term from A's stored planes
  {
    f32x16 acc[1] = {prod_rows<PK, SM / 2>(as_, SM * AS, AS, as_, SM * AS, AS, ti, tj,
                                           kh * (SM / 2))};
    reduce_halves<1>(acc, red, w, lane);
    if (w < 4) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * ti + 8 * (v >> 2) + 4 * hl + (v & 3), c = 32 * tj + (lane & 31);
        float av = 0.f;
#pragma unroll
        for (int q = 0; q < PK; ++q) av += bf2f(as_[q * SM * AS + r * AS + c]);
        const float x =
            a.coef_b * av + a.coef_c * acc[0][v] + (fold && r == c ? a.coef_a : 0.f);
        put_planes(bs, SM * AS, PK, AS, r, c, x);
      }
    }
  }
  __syncthreads();

  // X' = B X (+ a X from all of X's planes), times s in the first iteration
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const int ri = wt & 1, cj = 2 * (wt >> 1);
#pragma unroll
  for (int qa = 0; qa < PK; ++qa)
#pragma unroll
    for (int qb = 0; qb + qa < PK; ++qb)
#pragma unroll
      for (int k = 0; k < SM / 2; k += 16) {
        const int k0 = kh * (SM / 2) + k;
        const bf16x8 fa = frag_rows(bs + qa * SM * AS, AS, 32 * ri, k0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[u] = mfma(fa, frag_cols(xs + qb * SM * XS, XS, 32 * (cj + u), k0), acc[u]);
      }
  reduce_halves<2>(acc, red, w, lane);   // every wave has read X once this returns
  if (w < 4) {
    const float sc = first ? s : 1.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * ri + 8 * (v >> 2) + 4 * hl + (v & 3);
        const int c = 32 * (cj + u) + (lane & 31);
        float lin = 0.f;
        if (!fold) {
#pragma unroll
          for (int q = 0; q < NP; ++q) lin += bf2f(xs[q * SM * XS + r * XS + c]);
        }
        acc[u][v] = sc * fmaf(a.coef_a, lin, acc[u][v]);
      }
    if (last) {
      const int tr = (a.tr_mask >> (z / a.P)) & 1;
      float* U = a.U + (int64_t)z * M * N;
      const bool whole = 32 * (ri + 1) <= M && 32 * (cj + 2) <= N;   // wave-uniform
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * ri + 8 * (v >> 2) + 4 * hl + (v & 3);
          const int c = 32 * (cj + u) + (lane & 31);
          if (whole || (r < M && c < N)) {
            if (tr) U[(int64_t)c * M + r] = acc[u][v];
            else U[(int64_t)r * N + c] = acc[u][v];
          }
        }
    }
  }
  // every wave's products have read X before the barrier in reduce_halves, and the a X
  // term above reads X only where the same wave writes X' below
  if (!last) {
    if (w < 4) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * ri + 8 * (v >> 2) + 4 * hl + (v & 3);
          const int c = 32 * (cj + u) + (lane & 31);
          put_planes(xs, SM * XS, NP, XS, r, c, acc[u][v]);
        }
    }
    __syncthreads();
  }
}

template <int NP>
__global__ __launch_bounds__(512) void k_ns_small(NsArgs a) {
  __shared__ __attribute__((aligned(16))) u16 xs[NP * SM * XS];
  __shared__ __attribute__((aligned(16))) u16 as_[NP * SM * AS];
  __shared__ __attribute__((aligned(16))) u16 bs[NP * SM * AS];
  __shared__ __attribute__((aligned(16))) float red[4 * 64 * 32];
  const int z = blockIdx.x;
  const int M = a.M, N = a.N;

  // the gradient's planes, zero outside [M][N]
  for (int i = threadIdx.x; i < NP * SM * (SN / 8); i += 512) {
    const int q = i / (SM * (SN / 8)), rem = i % (SM * (SN / 8));
    const int r = rem / (SN / 8), c = (rem % (SN / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < M && c < N)
      v = *reinterpret_cast<const uint4*>(a.xin.base + q * a.xin.plane_stride +
                                          (int64_t)z * a.xin.zstride + (int64_t)r * a.xin.ld + c);
    *reinterpret_cast<uint4*>(xs + q * SM * XS + r * XS + c) = v;
  }
  const float s = ns_scale_of(a.part, a.nparts, a.eps, z);
  __syncthreads();
  for (int it = 0; it < a.steps; ++it) {
    const bool first = it == 0, last = it == a.steps - 1;
    if (NP > 1 && ((a.one >> it) & 1))
      ns_iteration<NP, 1>(a, xs, as_, bs, red, z, s, first, last);
    else
      ns_iteration<NP, NP>(a, xs, as_, bs, red, z, s, first, last);
  }
}

}  // namespace

hipError_t launch_ns_small(const NsArgs& a, hipStream_t st) {
  if (a.Z == 0 || a.steps == 0) return hipSuccess;
  if (a.xin.np == 1) hipLaunchKernelGGL(k_ns_small<1>, dim3(a.Z), dim3(512), 0, st, a);
  else if (a.xin.np == 2) hipLaunchKernelGGL(k_ns_small<2>, dim3(a.Z), dim3(512), 0, st, a);
  else hipLaunchKernelGGL(k_ns_small<3>, dim3(a.Z), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace ttt
