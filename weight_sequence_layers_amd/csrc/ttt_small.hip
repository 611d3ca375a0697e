// Device-resident chunk loop for small fast weights: the classic small-chunk TTT layer
// (2-layer GELU MLP, dim 64, hidden 256, chunks of at most 64 tokens, plain gradient step),
// which the TTT-layer explainer page (aivaro.ru, §3-4) describes and the LaCT explainer
// page (peacm.com, §1.1) names as the inefficient regime of small per-chunk updates.
//
// One workgroup owns one (batch, head) problem for the whole sequence.  Its fast weights
// stay on chip from the first chunk to the last: fp32 in registers, laid out as the MFMA
// accumulators of the weight-gradient GEMMs, and as bf16 copies in LDS for the GEMM
// operands.  The gradient GEMMs take the negated output error as their left operand and
// accumulate straight into the fp32 state, which is the step W <- W - g.  Every chunk
// runs seven small MFMA GEMMs on LDS-staged operands; only q, k, v, eta and the outputs
// touch HBM, and the next chunk's inputs are loaded into registers while the current
// chunk computes.
#include <math.h>

#include "ttt_internal.h"

namespace ttt {

namespace small {

constexpr int D = 64, DH = 256, BT = 64;     // dim, hidden, tokens per chunk (max)
constexpr int S64 = D + 8;                     // padded LDS row strides (elements)
constexpr int S256 = DH + 16;
constexpr int NT = 256;

// LDS layout (bytes)
constexpr int OFF_QE = 0;                            // Q, then O staging, then -E  [64][S64]
constexpr int OFF_K = OFF_QE + BT * S64 * 2;         // K                           [64][S64]
constexpr int OFF_V = OFF_K + BT * S64 * 2;          // V                           [64][S64]
// The hidden-by-token and weight buffers are stored transposed (H^T, W1^T, W2^T) so that
// the four accumulator rows a lane holds side by side land in one 8-byte LDS store.
constexpr int OFF_HT = OFF_V + BT * S64 * 2;         // H^T (queries, keys), -dZ^T  [256][S64]
constexpr int OFF_W1T = OFF_HT + DH * S64 * 2;       // W1^T bf16                   [64][S256]
constexpr int OFF_W2T = OFF_W1T + D * S256 * 2;      // W2^T bf16                   [256][S64]
constexpr int OFF_ETA = OFF_W2T + DH * S64 * 2;      // eta                         [64] fp32
constexpr int LDS = OFF_ETA + BT * 4;

typedef __attribute__((address_space(3))) char lds_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every LDS access is lds + (a per-thread byte offset) + (a compile-time constant), so the
// constant lands in the instruction's offset field.
template <class T>
__device__ __forceinline__ __attribute__((address_space(3))) T& at(lds_t* lds, uint32_t off) {
  return *reinterpret_cast<__attribute__((address_space(3))) T*>(lds + off);
}

// GELU z Phi(z) with the normal CDF Phi, and its derivative Phi(z) + z phi(z).  Phi comes
// from Abramowitz & Stegun's rational approximation 7.1.26 of erf (absolute error at most
// 1.5e-7, far below the bf16 rounding these values then take): with x = |z| / sqrt(2),
// t = 1 / (1 + 0.3275911 x) and e = exp(-x^2) = exp(-z^2 / 2),
//   Phi(-|z|) = erfc(x) / 2 = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e / 2,
// one reciprocal and one exponential, no branches; e also gives phi(z) = e / sqrt(2 pi).
// The constants below fold 1/sqrt(2) into 0.3275911, the 1/2 into a1..a5, and log2(e)
// into the exponent (exp2 is the native instruction).
__device__ __forceinline__ float std_normal_tail(float z, float& e) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2316418883f, fabsf(z), 1.f));   // 0.3275911 / sqrt 2
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.5307027145f, -0.7265760135f), 0.7107068705f),
                       -0.142248368f),
               0.127414796f);                                                  // a_i / 2
  e = __builtin_amdgcn_exp2f(z * z * -0.72134752044f);                        // -log2(e) / 2
  return poly * e;
}
__device__ __forceinline__ float gelu(float z) {
  float e;
  const float h = std_normal_tail(z, e);
  return z * (z >= 0.f ? 1.f - h : h);
}
__device__ __forceinline__ void gelu_and_d(float z, float& g, float& gd) {
  float e;
  const float h = std_normal_tail(z, e);
  const float cdf = z >= 0.f ? 1.f - h : h;
  g = z * cdf;
  gd = fmaf(z * e, 0.39894228040143268f, cdf);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-thread parts of the fragment offsets (bytes).  The MFMA operand fragment of lane l
// holds element (row l % 32, k 8 (l / 32) .. +7).
//  row layout ((r, k) at r S + k): one 16-byte read at (l % 32) S + 8 (l / 32).
//  column layout ((r, k) at k S + r): two transposing 8-byte reads.  Within a 16-lane
//    group, lane j receives element j % 4 of the 4-element rows addressed by lanes
//    4e + j / 4 (e = 0..3); lane 4e + q addresses k-row e at column 4q, so lane j of
//    group g gets rows 16 (g & 1) + j over k = 8 (g >> 1) + e, and the second read covers
//    k + 4 .. k + 7.
__device__ __forceinline__ uint32_t frag_row_off(int S) {
  const int l = threadIdx.x & 63;
  return ((l & 31) * S + 8 * (l >> 5)) * 2;
}
__device__ __forceinline__ uint32_t frag_col_off(int S) {
  const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  return ((8 * (g >> 1) + (j >> 2)) * S + 16 * (g & 1) + 4 * (j & 3)) * 2;
}
// Accumulator element v of a 32 x 32 tile sits at row 8 (v / 4) + 4 (l / 32) + v % 4,
// column l % 32: per-thread part of its offset, and the constant part.
__device__ __forceinline__ uint32_t acc_off(int S) {
  const int l = threadIdx.x & 63;
  return (4 * (l >> 5) * S + (l & 31)) * 2;
}
constexpr uint32_t acc_const(int S, int v) { return (8 * (v >> 2) + (v & 3)) * S * 2; }
// The same tile written transposed ((r, c) at c S + r): elements v = 4q .. 4q + 3 are
// consecutive and go out as one 8-byte store at per-thread part + 8 q * 2.
__device__ __forceinline__ uint32_t acc_t_off(int S) {
  const int l = threadIdx.x & 63;
  return ((l & 31) * S + 4 * (l >> 5)) * 2;
}
__device__ __forceinline__ bf16x4 pack4(const f32x16& x, int q) {
  return __builtin_convertvector(
      (f32x4){x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]}, bf16x4);
}

template <int S>
__device__ __forceinline__ bf16x8 frag_row(lds_t* lds, uint32_t off, int r0, int k0) {
  return at<bf16x8>(lds, off + (r0 * S + k0) * 2);
}
template <int S>
__device__ __forceinline__ bf16x8 frag_col(lds_t* lds, uint32_t off, int r0, int k0) {
  const uint32_t o = off + (k0 * S + r0) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(lds + o));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(lds + o + 4 * S * 2));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void zero(f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
}

// scale a register-resident 64 x 64 block (weight decay of the state, step-size ratio)
__device__ __forceinline__ void scale_state(f32x16 (&w)[2][2], float keep) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) w[i][j] *= keep;
}

// acc[i][j] += A(32 i + [0, 32), :) B(32 j + [0, 32), :)^T over k in [0, KLEN): a 64 x 64
// block of a product per wave.  a_off / b_off: byte offsets of the operands' (0, 0)
// elements including this thread's fragment part.
template <bool ACOL, int SA, bool BCOL, int SB, int KLEN>
__device__ __forceinline__ void mma_2x2(f32x16 (&acc)[2][2], lds_t* lds, uint32_t a_off,
                                        uint32_t b_off) {
#pragma unroll
  for (int k0 = 0; k0 < KLEN; k0 += 16) {
    bf16x8 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[i] = ACOL ? frag_col<SA>(lds, a_off, 32 * i, k0) : frag_row<SA>(lds, a_off, 32 * i, k0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = BCOL ? frag_col<SB>(lds, b_off, 32 * j, k0) : frag_row<SB>(lds, b_off, 32 * j, k0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
  }
}

// One 32 x 32 tile of H W2^T over K = 256, both operands read from transposed buffers
// (H^T, W2^T: column layout, stride S64).
__device__ __forceinline__ f32x16 mma_k256(lds_t* lds, uint32_t h_off, uint32_t w_off) {
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int k0 = 0; k0 < 256; k0 += 16)
    acc = mfma(frag_col<S64>(lds, h_off, 0, k0), frag_col<S64>(lds, w_off, 0, k0), acc);
  return acc;
}

// An opaque copy of x: a value the compiler cannot see through, so that addresses built
// from it are formed inside the chunk loop instead of being hoisted into registers.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

}  // namespace small

// One chunk's q, k, v rows (64 x 64 bf16 each) move through registers: 2 x 16 bytes per
// thread and tensor, loaded one chunk ahead.
struct ChunkRegs {
  small::u32x4 q[2], k[2], v[2];
  float eta;
};

// SCALED: step sizes other than 1 or a weight decay (a separate instance, so that the
// plain step compiles without any of it)
template <int LOSS, bool SCALED>
__global__ __launch_bounds__(256) void k_small_gelu(SmallArgs a) {
  using namespace small;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  lds_t* const lds = (lds_t*)smem;

  const int p = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6;
  const int b = a.chunk;

  // wave parts of the offsets (bytes)
  const uint32_t w_rows64 = 64 * w * S64 * 2;   // rows [64w, ..) of an S64 tile
  const uint32_t w_cols = 64 * w * 2;           // columns [64w, ..) of an S256 tile
  const int wr = 32 * (w >> 1), wc = 32 * (w & 1);   // this wave's 32 x 32 tile of a 64 x 64
  // chunk rows moved by this thread: tid / 8 and 32 + tid / 8, 16-byte column block tid % 8
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const float es = a.e_scale;   // step size of W2, folded into the staged eta (so into -E)

  // fp32 state, as gradient-GEMM accumulators:
  //   w1: W1 rows (hidden) [64w, +64) x all 64 columns;  w2: all 64 rows x W2 columns
  //   [64w, +64).  They move through buffer loads / stores whose per-element part is a
  //   scalar offset.
  const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
      a.W1 + (int64_t)p * DH * D, (short)0, DH * D * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
      a.W2 + (int64_t)p * D * DH, (short)0, D * DH * 4, 0x00020000);
  const int hl = (tid & 63) >> 5, cl = tid & 31;
  const uint32_t vo1 = ((64 * w + 4 * hl) * D + cl) * 4;
  const uint32_t vo2 = ((4 * hl) * DH + 64 * w + cl) * 4;
  auto so1 = [](int i, int j, int v) { return ((32 * i + 8 * (v >> 2) + (v & 3)) * D + 32 * j) * 4; };
  auto so2 = [](int i, int j, int v) { return ((32 * i + 8 * (v >> 2) + (v & 3)) * DH + 32 * j) * 4; };
  f32x16 w1[2][2], w2[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        w1[i][j][v] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs1, vo1, so1(i, j, v), 0));
        w2[i][j][v] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs2, vo2, so2(i, j, v), 0));
      }

  // per-thread offset parts; re-laundered at the top of every chunk
  uint32_t fr64, fc64, fc256, ac64, at64, at256, ld64;
  auto bind = [&]() __attribute__((always_inline)) {
    fr64 = opaque(frag_row_off(S64));
    fc64 = opaque(frag_col_off(S64));
    fc256 = opaque(frag_col_off(S256));
    ac64 = opaque(acc_off(S64));
    at64 = opaque(acc_t_off(S64));
    at256 = opaque(acc_t_off(S256));
    ld64 = opaque((lr * S64 + lc) * 2);
  };

  // bf16 copies of the state for the GEMM operands: w1 rows (hidden) become W1^T columns,
  // w2 rows (dim) become W2^T columns
  auto publish_w = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          at<bf16x4>(lds, OFF_W1T + at256 + w_cols + (32 * j * S256 + 32 * i + 8 * q) * 2) =
              pack4(w1[i][j], q);
          at<bf16x4>(lds, OFF_W2T + at64 + w_rows64 + (32 * j * S64 + 32 * i + 8 * q) * 2) =
              pack4(w2[i][j], q);
        }
  };
  // a 64 x 256 block (rows: tokens; this wave's columns [64w, +64) of hidden) into H^T
  auto put_h = [&](const f32x16 (&x)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          at<bf16x4>(lds, OFF_HT + at64 + w_rows64 + (32 * j * S64 + 32 * i + 8 * q) * 2) =
              pack4(x[i][j], q);
  };
  auto load_chunk = [&](int c, ChunkRegs& R) __attribute__((always_inline)) {
    const int64_t base = (int64_t)p * a.T + (int64_t)c * b;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lr + 32 * h;
      const bool ok = t < b;
      const int64_t o = (base + t) * D + lc;
      const u32x4 zero4 = {0u, 0u, 0u, 0u};
      R.q[h] = ok ? *reinterpret_cast<const u32x4*>(a.q + o) : zero4;
      R.k[h] = ok ? *reinterpret_cast<const u32x4*>(a.k + o) : zero4;
      R.v[h] = ok ? *reinterpret_cast<const u32x4*>(a.v + o) : zero4;
    }
    R.eta = (tid < b) ? a.eta[base + tid] : 0.f;
  };
  auto stage_chunk = [&](const ChunkRegs& R) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      at<u32x4>(lds, OFF_QE + ld64 + h * 32 * S64 * 2) = R.q[h];
      at<u32x4>(lds, OFF_K + ld64 + h * 32 * S64 * 2) = R.k[h];
      at<u32x4>(lds, OFF_V + ld64 + h * 32 * S64 * 2) = R.v[h];
    }
    if (tid < BT) at<float>(lds, OFF_ETA + tid * 4) = SCALED ? es * R.eta : R.eta;
  };

  bind();
  publish_w();
  ChunkRegs nxt;
  load_chunk(0, nxt);
  stage_chunk(nxt);
  __syncthreads();

  f32x16 acc[2][2], gd[2][2];
  for (int c = 0; c < a.nchunks; ++c) {
    bind();
    if (c + 1 < a.nchunks) load_chunk(c + 1, nxt);   // in flight during this chunk

    // 1. apply: gelu(Q W1^T) -> H^T
    zero(acc);
    mma_2x2<false, S64, true, S256, 64>(acc, lds, OFF_QE + fr64, OFF_W1T + fc256 + w_cols);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = gelu(acc[i][j][v]);
    __syncthreads();                                   // Q read by every wave
    put_h(acc);
    __syncthreads();
    // 2. O = H W2^T, staged through the Q buffer, then 16-byte stores
    {
      const f32x16 o = mma_k256(lds, OFF_HT + fc64 + wr * 2, OFF_W2T + fc64 + wc * 2);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        at<u16>(lds, OFF_QE + ac64 + (wr * S64 + wc) * 2 + acc_const(S64, v)) = f2bf(o[v]);
    }
    __syncthreads();
    {
      const int64_t base = (int64_t)p * a.T + (int64_t)c * b;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = lr + 32 * h;
        if (t < b)
          *reinterpret_cast<u32x4*>(a.out + (base + t) * D + lc) =
              at<u32x4>(lds, OFF_QE + ld64 + h * 32 * S64 * 2);
      }
    }
    // 3. keys: Z = K W1^T; gelu(Z) -> H^T, gelu'(Z) stays in registers
    zero(acc);
    mma_2x2<false, S64, true, S256, 64>(acc, lds, OFF_K + fr64, OFF_W1T + fc256 + w_cols);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float g, d1;
          gelu_and_d(acc[i][j][v], g, d1);
          acc[i][j][v] = g;
          gd[i][j][v] = d1;
        }
    __syncthreads();                                   // O copied out, query H read
    put_h(acc);
    __syncthreads();
    // 4. negated output error -> Q buffer.  MSE: -2 eta (gelu(Z) W2^T - V).  Inner
    //    product: the error of -eta <f, v> is -eta v, negated +eta v.
    if constexpr (LOSS == 1) {
      const f32x16 o = mma_k256(lds, OFF_HT + fc64 + wr * 2, OFF_W2T + fc64 + wc * 2);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t e_off = OFF_QE + ac64 + (wr * S64 + wc) * 2 + acc_const(S64, v);
        const uint32_t v_off = e_off - OFF_QE + OFF_V;
        const float eta = at<float>(lds, OFF_ETA + (wr + 4 * hl + 8 * (v >> 2) + (v & 3)) * 4);
        at<u16>(lds, e_off) = f2bf(2.f * eta * (bf2f(at<u16>(lds, v_off)) - o[v]));
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float eta = at<float>(lds, OFF_ETA + (lr + 32 * h) * 4);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8)
          at<u16>(lds, OFF_QE + ld64 + (h * 32 * S64 + e8) * 2) =
              f2bf(eta * bf2f(at<u16>(lds, OFF_V + ld64 + (h * 32 * S64 + e8) * 2)));
      }
    }
    __syncthreads();
    // 5. W2 <- keep W2 - lr2 E^T gelu(Z)  (the step size is in the staged eta, so in -E)
    if constexpr (SCALED) scale_state(w2, a.keep);
    mma_2x2<true, S64, false, S64, 64>(w2, lds, OFF_QE + fc64, OFF_HT + fr64 + w_rows64);
    // 6. -dH = (-E) W2 with the pre-update bf16 W2; -dZ = -dH gelu'(Z) -> H^T
    zero(acc);
    mma_2x2<false, S64, false, S64, 64>(acc, lds, OFF_QE + fr64, OFF_W2T + fr64 + w_rows64);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] *= gd[i][j];
    if constexpr (SCALED) scale_state(acc, a.dz_scale);   // W1's step size over W2's
    __syncthreads();                                   // gelu(Z) read by every wave
    put_h(acc);
    __syncthreads();
    // 7. W1 <- keep W1 - lr1 dZ^T K
    if constexpr (SCALED) scale_state(w1, a.keep);
    mma_2x2<false, S64, true, S64, 64>(w1, lds, OFF_HT + fr64 + w_rows64, OFF_K + fc64);
    __syncthreads();                                   // every read of W, K, V, E done
    publish_w();
    if (c + 1 < a.nchunks) stage_chunk(nxt);
    __syncthreads();
  }

  // write the state back and flag non-finite values
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // (copied out first: a bit cast straight from a vector element reads element 0)
        const float x1 = w1[i][j][v], x2 = w2[i][j][v];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x1), rs1, vo1,
                                              so1(i, j, v), 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x2), rs2, vo2,
                                              so2(i, j, v), 0);
        bad |= !isfinite(x1) || !isfinite(x2);
      }
  if (bad) *a.health = 1;
}

bool small_supported(int fw, int ns_steps, int renorm, int act_bf16, int apply_first, int dim,
                     int hidden, int chunk, int ap, int gp) {
  return fw == FW_GELU && ns_steps == 0 && !renorm && act_bf16 && apply_first &&
         dim == small::D && hidden == small::DH && chunk >= 1 && chunk <= small::BT &&
         ap == 1 && gp == 1;
}

template <int LOSS, bool SCALED>
static hipError_t launch_small_t(const SmallArgs& a, hipStream_t s) {
  auto kern = k_small_gelu<LOSS, SCALED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, small::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.P), dim3(small::NT), small::LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_small(const SmallArgs& a, int loss, hipStream_t s) {
  if (a.P == 0 || a.nchunks == 0) return hipSuccess;
  if (a.chunk < 1 || a.chunk > small::BT) return hipErrorInvalidValue;
  const bool scaled = a.e_scale != 1.f || a.dz_scale != 1.f || a.keep != 1.f;
  if (loss == 1) return scaled ? launch_small_t<1, true>(a, s) : launch_small_t<1, false>(a, s);
  return scaled ? launch_small_t<0, true>(a, s) : launch_small_t<0, false>(a, s);
}

}  // namespace ttt
