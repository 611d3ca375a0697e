// Internal interface between the host library (libttt.cpp) and the HIP kernels
// (ttt_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttt_device.hpp"

namespace ttt {

__host__ __device__ inline Operand operand_of(const PlaneBuf& b, int np, int rows) {
  return make_operand(b.base, b.plane_stride, b.ld, b.zstride, np, rows);
}
// plane q of b alone, as a one-plane operand
__host__ __device__ inline Operand plane_operand(const PlaneBuf& b, int q, int rows) {
  return make_operand(b.base + q * b.plane_stride, 0, b.ld, b.zstride, 1, rows);
}

enum FwKind { FW_SWIGLU = 0, FW_GELU = 1, FW_LINEAR = 2 };
enum FrontMode { FRONT_Q = 0, FRONT_K_DOT = 1, FRONT_K_MSE = 2 };
enum OutMode { OUT_Q = 0, OUT_K_MSE = 1, DH_MSE = 2 };

// Z-GEMMs over rows of Q or K: X W1^T (and X W3^T), plus V W2 for the inner-product loss.
struct FrontArgs {
  // A operands: [0] the rows (Q or K), [1] V (inner-product loss only).
  // B operands in product order: W1, then W3 (SwiGLU), then W2 read column-wise
  // (inner-product loss).
  Operand A[2];
  Operand B[3];
  const float* eta;
  int64_t eta_zstride;
  int nrows;   // token rows
  int K;       // dim
  int N;       // hidden
  int tiles_n, tiles;
  PlaneBuf o1, o2, o3;  // Q: hidden | K_DOT: dZ1, dZ3 (or dZ), P | K_MSE: H; all [rows][hidden]
  float* fa;            // K_MSE: derivative factors [rows][hidden]
  float* fb;
  int64_t f_zstride;
};

// GEMMs that end in the model dimension (O = H W2^T, Ok = H W2^T) and the hidden-error GEMM
// dH = E W2 for the MSE loss.
struct OutArgs {
  Operand a, b;
  int nrows, K, N, tiles_n, tiles;
  // OUT_Q
  void* out;
  int64_t out_zstride;
  int out_bf16;
  // OUT_K_MSE
  const void* vin;
  int64_t v_zstride;
  int v_bf16;
  const float* eta;
  int64_t eta_zstride;
  PlaneBuf e;      // E [rows][dim]
  // DH_MSE
  const float* fa;
  const float* fb;
  int64_t f_zstride;
  PlaneBuf dz1, dz3;  // [rows][hidden]
  int swiglu;
};

// Backward of the apply step with respect to the queries: dQ [rows][dim] = sum over the
// NP pairs of A_m [rows][hidden] (row-wise) times B_m = W_m [hidden][dim] (column-wise).
struct DqArgs {
  Operand a[2], b[2];
  int nrows, K, N, tiles_n, tiles;
  void* out;            // [problems][rows][dim] in the activation dtype
  int64_t out_zstride;
  int out_bf16;
};

// Token contractions: X_m[i][j] = sum_t A_m[t][i] B_m[t][j] for every matrix m and problem
// (both operands token-major, read as columns).
struct ContractArgs {
  Operand a[3], b[3];
  int P, M, N, K, tiles_n, tiles;
  float* G;        // [nm][P][M][N]
  int accum_in;    // add the running sum held in G
  int last;        // last token block of the chunk
  int muon;        // write X0 planes and per-tile sums of squares
  PlaneBuf x;
  float* part;     // [nm*P][tiles]
  float* U;        // plain step: U in weight orientation [nm][P][rows][cols]
  int tr_mask;     // bit m: matrix m's weight is the transpose of its X orientation
  // Token split: with ksplit > 1 the launch sums ksplit token ranges of kchunk tokens in
  // separate workgroups, which write partial tiles to gpart [ksplit][nm][P][M][N] (splits
  // gpart_stride elements apart); a second kernel adds them and applies the epilogue.
  // The caller sets ksplit to the capacity of gpart; launch_contract picks the split.
  float* gpart;
  int64_t gpart_stride;
  int ksplit, kchunk;
  int nz;          // nm * P of the launch (set by launch_contract)
};

// Newton-Schulz stages on Z = nm*P matrices X [M x N] (M <= N).
struct NsArgs {
  int Z, M, N, tiles_n, tiles;
  float coef_a, coef_b, coef_c;
  const float* part;  // iteration 0: per-tile sums of squares of the unscaled gradient
  int nparts;
  int first;          // iteration 0 (fold the 1/(|G|_F + eps) scale)
  int last;           // final iteration: write U instead of planes
  float eps;
  PlaneBuf xin;       // gram, update: X planes [M][N] (iteration 0: planes of G)
  PlaneBuf ain;       // poly: A planes [M][M] ; update: B planes [M][M]
  PlaneBuf aout;      // gram: A planes ; poly: B planes
  PlaneBuf xout;
  float* U;           // last: U in weight orientation
  int tr_mask;
  int P;
};

struct RenormMat {
  float* W;        // [P][rows][cols]
  const float* U;  // same layout, or null (planes refresh only)
  int rows, cols;
  u16* pl;         // planes [np][P][rows][cols]
  int64_t pl_stride;
  float lr;        // step size: W' = keep W - lr U
};
struct RenormArgs {
  RenormMat m[3];
  int P, np, renorm, nm, max_rows;
  float keep;      // 1 - weight decay
  int* health;
};

struct SplitArgs {
  const void* x;   // rows [n][d] of problem z at x + z * x_zstride (elements)
  int64_t x_zstride;
  int x_bf16;
  const float* eta;
  int64_t eta_zstride;
  int neg_eta;     // multiply row t by -eta_t
  int n, d;
  PlaneBuf out;    // [np][Z][rows][d]
};

// Device-resident chunk loop (GELU MLP, dim 64, hidden 256, chunk <= 64, plain gradient
// step, bf16 activations): one workgroup per problem runs every chunk of the call.
struct SmallArgs {
  const u16 *q, *k, *v;  // [P][T][64] bf16
  const float* eta;      // [P][T]
  u16* out;              // [P][T][64] bf16
  float *W1, *W2;        // state: W1 [P][256][64], W2 [P][64][256], fp32, updated in place
  int* health;           // set to 1 if the final state holds a non-finite value
  int64_t T;             // tokens per problem in the caller's tensors
  int chunk, nchunks, P;
  float e_scale;         // step size of W2: scales the negated output error
  float dz_scale;        // step size of W1 over that of W2: scales the negated dZ
  float keep;            // 1 - weight decay, applied to the state before each step
};

// ---------------------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  `lds_limit` handling and tile choice are
// internal.  `Z` is the number of (batch, head) problems.
hipError_t launch_front(int fw, int mode, const FrontArgs& a, int Z, hipStream_t s);
hipError_t launch_out(int mode, const OutArgs& a, int Z, hipStream_t s);
hipError_t launch_contract(const ContractArgs& a, int nm, hipStream_t s);
hipError_t launch_dq(const DqArgs& a, int np, int Z, hipStream_t s);
// token ranges a contraction of `tiles` output tiles per matrix over nz matrices may split
// into (the host sizes the partial-sum buffer with it)
int contract_split_max(int tiles, int nz);
hipError_t launch_ns_gram(const NsArgs& a, hipStream_t s);
hipError_t launch_ns_poly(const NsArgs& a, hipStream_t s);
hipError_t launch_ns_update(const NsArgs& a, hipStream_t s);
hipError_t launch_renorm(const RenormArgs& a, hipStream_t s);
hipError_t launch_split(const SplitArgs& a, int Z, hipStream_t s);
hipError_t launch_small(const SmallArgs& a, int loss, hipStream_t s);
bool small_supported(int fw, int ns_steps, int renorm, int act_bf16, int apply_first, int dim,
                     int hidden, int chunk, int ap, int gp);
hipError_t prepare_kernels();  // raise dynamic-LDS limits once per process

// tile sizes used by the contraction and Newton-Schulz stages (the host sizes buffers)
constexpr int CONTRACT_BM = 128, CONTRACT_BN = 128;
int ns_tri_tiles(int M, int tile);

}  // namespace ttt
