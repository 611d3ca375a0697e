// Newton-Schulz orthogonalisation of small matrices in one launch: every iteration of one
// matrix in one workgroup, its iterates kept in LDS.
//
// The iteration is the quintic of the Muon step ([LaCT] §2.2, the update's orthogonalised
// gradient): X0 = G / (|G|_F + eps), then per iteration A = X X^T, B = b A + c A A and
// X' = a X + B X.  The staged path runs it as three GEMM launches per iteration, which for
// matrices of a few tens of thousands of elements are bound by each launch's latency; here
// one workgroup of sixteen waves holds the whole matrix (X up to 64 x 128) and its A and B as
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
  return 1.f / (sqrtf(sum_parts(part + (int64_t)z * nparts, nparts)) + eps);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four consecutive values of one row as `np` planes: planes[q][off .. off + 3], one 8-byte
// LDS store per plane (off is a multiple of 4).
__device__ __forceinline__ void put_run(u16* planes, int pstride, int np, int off,
                                        const float (&x)[4]) {
  u16 h[4][3];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_planes(x[e], np, h[e]);
#pragma unroll
  for (int q = 0; q < 3; ++q)
    if (q < np)
      *reinterpret_cast<uint2*>(planes + q * pstride + off) =
          make_uint2(h[0][q] | ((uint32_t)h[1][q] << 16), h[2][q] | ((uint32_t)h[3][q] << 16));
}

// The sum of the first np planes of four consecutive values planes[q][off .. off + 3].
__device__ __forceinline__ void sum_run(const u16* planes, int pstride, int np, int off,
                                        float (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = 0.f;
#pragma unroll
  for (int q = 0; q < 3; ++q)
    if (q < np) {
      const uint2 w = *reinterpret_cast<const uint2*>(planes + q * pstride + off);
      x[0] += bf2f((u16)(w.x & 0xffff));
      x[1] += bf2f((u16)(w.x >> 16));
      x[2] += bf2f((u16)(w.y & 0xffff));
      x[3] += bf2f((u16)(w.y >> 16));
    }
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

// Waves w and w ^ 8 hold the two K halves of the same tile.  Each keeps half of the tile's
// accumulator (wave w >> 3 = h keeps elements 8 h .. 8 h + 7, the tile's rows 16 h .. 16 h
// + 15 in the accumulator layout) and hands the other half to its partner through red (run
// j of wave w at red + ((2 w + j) 64 + lane) 4: consecutive lanes, consecutive 16 bytes).
// On return own holds the full sums of the kept half, the K half 0 partial plus the K half
// 1 partial.  w is wave-uniform.  Contains a barrier: call from every thread.
__device__ __forceinline__ void exchange_halves(const f32x16& acc, float (&own)[8], float* red,
                                                int w, int lane) {
  const int kh = w >> 3;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = acc[4 * j + e], hi = acc[8 + 4 * j + e];
      own[4 * j + e] = kh ? hi : lo;
      out[e] = kh ? lo : hi;
    }
    *reinterpret_cast<f32x4*>(red + ((2 * w + j) * 64 + lane) * 4) = out;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(red + ((2 * (w ^ 8) + j) * 64 + lane) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) own[4 * j + e] += x[e];
  }
}

// Waves w & 3 + 4 q, q = 0 .. 3, hold the four K quarters of the same tile.  Wave q = w >> 2
// keeps run q of the accumulator (elements 4 q .. 4 q + 3, the tile's rows 8 q .. 8 q + 7)
// and hands each of its three other runs to the wave that keeps it through red (run g of
// wave w in slot 3 w + (g < q ? g : g - 1), 64 lanes x 16 bytes).  On return own holds the
// kept run summed over the quarters in K order.  w is wave-uniform.  Contains a barrier:
// call from every thread.
__device__ __forceinline__ void exchange_quarters(const f32x16& acc, float (&own)[4],
                                                  float* red, int w, int lane) {
  const int kq = w >> 2, wt = w & 3;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    if (g != kq)
      *reinterpret_cast<f32x4*>(red + ((3 * w + (g < kq ? g : g - 1)) * 64 + lane) * 4) =
          f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) own[e] = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 x;
    if (q == kq) {
      x = f32x4{acc[4 * kq], acc[4 * kq + 1], acc[4 * kq + 2], acc[4 * kq + 3]};
    } else {
      const int slot = 3 * (4 * q + wt) + (kq < q ? kq : kq - 1);
      x = *reinterpret_cast<const f32x4*>(red + (slot * 64 + lane) * 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) own[e] += x[e];
  }
}

// One iteration with PK product planes (PK = NP folds a I into B).  Sixteen waves: for the
// Gram and polynomial products waves w & 3 + 4 q compute tile w & 3 over the four quarters
// of its K range and then finish a quarter of the tile each; for the update waves w and
// w + 8 compute tile w & 7 over the two halves of its K range and finish half of it each.
// In the accumulator layout a lane holds runs of four consecutive rows of one column.  A
// and B are symmetric, so such a run is stored at the mirror position as four consecutive
// columns of one row, one 8-byte LDS store a plane (A's planes are read back for b A the
// same way); the update computes the transposed tile X'^T = X^T B, so that its runs are
// four consecutive columns of X'.  No element needs a bounds check in LDS: X is zero outside
// [M][N], so A is zero outside [M][M], B outside [M][M] but for a on the padded diagonal
// (which multiplies zero rows of X), and X' is zero outside [M][N] again; only the store of
// U to memory checks.
template <int NP, int PK>
__device__ __forceinline__ void ns_iteration(const NsArgs& a, u16* xs, u16* as_, u16* bs,
                                             float* red, int z, float s, bool first,
                                             bool last) {
  constexpr bool fold = PK == NP;
  const int M = a.M, N = a.N;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wt = w & 3, kq = w >> 2;
  const int ti = wt >> 1, tj = wt & 1;
  const int ln = lane & 31;
  // first row of this wave's kept run of the Gram and polynomial tiles, the column of this
  // lane
  const int rq = 32 * ti + 8 * kq + 4 * hl;
  const int c = 32 * tj + ln;

  // A = X X^T (s^2 G G^T in the first iteration)
  {
    const f32x16 acc = prod_rows<PK, SN / 4>(xs, SM * XS, XS, xs, SM * XS, XS, ti, tj,
                                             kq * (SN / 4));
    float own[4];
    exchange_quarters(acc, own, red, w, lane);
    const float s2 = first ? s * s : 1.f;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = own[e] * s2;
    put_run(as_, SM * AS, PK, c * AS + rq, x);   // A[c][r .. r + 3]
  }
  __syncthreads();

  // B = b A + c A A (+ a I folded), the linear term from A's stored planes
  {
    const f32x16 acc = prod_rows<PK, SM / 4>(as_, SM * AS, AS, as_, SM * AS, AS, ti, tj,
                                             kq * (SM / 4));
    float own[4];
    exchange_quarters(acc, own, red, w, lane);
    float av[4], x[4];
    sum_run(as_, SM * AS, PK, c * AS + rq, av);   // A[r .. r + 3][c] by symmetry
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = a.coef_b * av[e] + a.coef_c * own[e] + (fold && rq + e == c ? a.coef_a : 0.f);
    put_run(bs, SM * AS, PK, c * AS + rq, x);
  }
  __syncthreads();

  // X'^T = X^T B (+ a X from all of X's planes), times s in the first iteration: tile rows
  // are columns of X', tile columns rows of X'
  const int t8 = w & 7, kh = w >> 3;
  const int ri = t8 & 1, cj = t8 >> 1;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int qa = 0; qa < PK; ++qa)
#pragma unroll
    for (int qb = 0; qb + qa < PK; ++qb)
#pragma unroll
      for (int k = 0; k < SM / 2; k += 16) {
        const int k0 = kh * (SM / 2) + k;
        acc = mfma(frag_cols(xs + qb * SM * XS, XS, 32 * cj, k0),
                   frag_rows(bs + qa * SM * AS, AS, 32 * ri, k0), acc);
      }
  float own[8];
  exchange_halves(acc, own, red, w, lane);   // every wave has read X once this returns
  const float sc = first ? s : 1.f;
  const int r = 32 * ri + ln;
  const int tr = (a.tr_mask >> (z / a.P)) & 1;
  float* U = a.U + (int64_t)z * M * N;
  // the a X term reads X only where the same lane writes X' below
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int c0 = 32 * cj + 16 * kh + 8 * g + 4 * hl;
    float lin[4] = {0.f, 0.f, 0.f, 0.f}, x[4];
    if (!fold) sum_run(xs, SM * XS, NP, r * XS + c0, lin);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = sc * fmaf(a.coef_a, lin[e], own[4 * g + e]);
    if (last) {
      // N is a multiple of 16, so a run starting inside the matrix lies inside it
      if (r < M && c0 < N) {
        if (tr) {
#pragma unroll
          for (int e = 0; e < 4; ++e) U[(int64_t)(c0 + e) * M + r] = x[e];
        } else {
          *reinterpret_cast<float4*>(U + (int64_t)r * N + c0) = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
    } else {
      put_run(xs, SM * XS, NP, r * XS + c0, x);
    }
  }
  if (!last) __syncthreads();
}

constexpr int NS_SMALL_THREADS = 1024;   // sixteen waves

template <int NP>
__global__ __launch_bounds__(NS_SMALL_THREADS) void k_ns_small(NsArgs a) {
  __shared__ __attribute__((aligned(16))) u16 xs[NP * SM * XS];
  __shared__ __attribute__((aligned(16))) u16 as_[NP * SM * AS];
  __shared__ __attribute__((aligned(16))) u16 bs[NP * SM * AS];
  // exchange slots: three runs of 64 lanes x 4 floats for each of the sixteen waves
  __shared__ __attribute__((aligned(16))) float red[3 * 16 * 64 * 4];
  const int z = blockIdx.x;
  const int M = a.M, N = a.N;

  // the gradient's planes, zero outside [M][N]
  for (int i = threadIdx.x; i < NP * SM * (SN / 8); i += NS_SMALL_THREADS) {
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
  if (a.xin.np == 1) hipLaunchKernelGGL(k_ns_small<1>, dim3(a.Z), dim3(NS_SMALL_THREADS), 0, st, a);
  else if (a.xin.np == 2) hipLaunchKernelGGL(k_ns_small<2>, dim3(a.Z), dim3(NS_SMALL_THREADS), 0, st, a);
  else hipLaunchKernelGGL(k_ns_small<3>, dim3(a.Z), dim3(NS_SMALL_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace ttt
