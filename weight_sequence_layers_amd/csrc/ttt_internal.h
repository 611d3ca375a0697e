// Internal interface between the host library (libttt.cpp) and the HIP kernels
// (ttt_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libttt.h"
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
// Also the chunk backward's dK (four pairs) and dV (two pairs) GEMMs: out = sum_m A_m B_m^T
// with each B_m read by rows or by columns (the launcher's layout mask).
struct DqArgs {
  Operand a[4], b[4];
  int nrows, K, N, tiles_n, tiles;
  void* out;            // [problems][rows][dim] in the activation dtype
  int64_t out_zstride;
  int out_bf16;
};

// ---------------------------------------------------------------- backward through an update
// Tangent front of the chunk backward (SwiGLU net, inner-product loss): on the chunk's key
// rows, the six products Z1 = K W1^T, Z3 = K W3^T, Zd1 = K D1^T, Zd3 = K D3^T (D the
// cotangent of the chunk gradient), V W2 and V D2, and in the epilogue the per-token terms
// of the gradient's backward.
struct TFrontArgs {
  Operand A[2];         // K rows, V rows
  Operand B[6];         // W1, W3 (rows); D1, D3, W2, D2 (read by columns)
  const float* eta;
  int64_t eta_zstride;
  int nrows, K, N, tiles_n, tiles;
  PlaneBuf p, pd, a1, a3, dz1, dz3;   // [rows][hidden]: -eta H, -eta Hd, A1, A3, dZ1, dZ3
  float* eta_part;      // [Z][rows][tiles_n]: the tile's share of -sum_h (V D2 . H + V W2 . Hd)
  int64_t part_zstride;
};

// Sum of the eta partials: deta[z][t] = sum_j part[z][t][j] (j < nparts), fixed order.
struct EtaSumArgs {
  const float* part;
  int64_t part_zstride;
  int nparts, nrows;
  float* deta;          // [Z][T] caller tensor (stride deta_zstride)
  int64_t deta_zstride;
};

// Backward of the step and row renorm for one matrix kind (one wave per row, like k_renorm):
// Y = keep W - lr U, out = renorm(Y) (or Y).  Writes dW_step = (renorm: <yh, dOut> / |w| w)
// + keep dY and dU = -lr dY (the latter in the X orientation: transposed when tr).
struct StepBwdMat {
  const float* W;       // [P][rows][cols]
  const float* U;
  const float* dout;    // cotangent of the new matrix
  float* dw;            // dW_step
  float* du;            // dU, X orientation
  int rows, cols, tr;
  float lr;
};
struct StepBwdArgs {
  StepBwdMat m[3];
  int P, nm, renorm, max_rows;
  float keep;
};

// Generic two-pair GEMM of the Newton-Schulz backward: out = alpha (A0 B0^T + A1 B1^T) + beta cin
// over Z matrices of M x N, B operands read by rows or columns (the launcher's mask); fp32
// and/or plane outputs; optionally per-tile sums of out * gref (the Frobenius inner product).
struct Gemm2Args {
  Operand a[2], b[2];
  int M, N, K, Z, tiles_n, tiles;
  float alpha, beta;
  const float* cin;     // [Z][M][N] or null
  float* cout;          // [Z][M][N] or null
  PlaneBuf pout;        // planes, or np = 0
  const float* gref;    // [Z][M][N] or null
  float* gpart;         // [Z][tiles] per-tile sums of out * gref
  // optional per-matrix factor 1 / (sqrt(sum of spart[z][0 .. nspart)) + eps) on the whole
  // output (the Newton-Schulz scale of iteration 0, from the forward's tile sums)
  const float* spart;
  int nspart;
  float eps;
};

// Backward of X0 = G / (|G|_F + eps): dG = dX0 s - G <G, dX0> s^2 / |G|_F, s = 1 / (|G|_F + eps).
struct NsFinArgs {
  const float* G;       // [Z][M][N] X orientation
  const float* dX;      // [Z][M][N]
  const float* ss_part; // [Z][nss] sums of squares of G (forward contraction tiles)
  int nss;
  const float* dot_part;  // [Z][ndot] sums of G . dX0
  int ndot;
  int64_t per;          // M * N
  float eps;
  float* dG;            // [Z][M][N] fp32
  PlaneBuf pout;        // planes of dG
};

// Momentum's backward, per matrix and problem: t = dg + dm, dg <- t, dm <- beta t, with dg
// in the X orientation and dm in the weight orientation [rows][cols] (the X orientation
// is [cols][rows] where tr).
struct MomBwdMat {
  float* dg;
  float* dm;
  int rows, cols, tr;
};
struct MomBwdArgs {
  MomBwdMat m[3];
  int P, nm;
  float beta;
};

// out[i] = x[i] + y[i] + w[i] over n values (any of y, w may be null).
struct Add3Args {
  const float *x, *y, *w;
  float* out;
  int64_t n;
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
  float* part;     // [nm*P][tiles][psub]
  int psub;        // parts per tile: 1, or CONTRACT_SUM_SUB when the launch may split
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
  // momentum: with mom, the last epilogue replaces the sum x by beta M + x and, with
  // mom_write, stores it in M (weight orientation, like U) before using it (the backward's
  // recompute reads M only)
  float* mom;
  float beta;
  int mom_write;
  // with g32, the last epilogue also stores the final sum (after momentum) in fp32 in the X
  // orientation [nm][P][M][N] (the backward's Newton-Schulz scaling reads it)
  float* g32;
};

// Newton-Schulz stages on Z = nm*P matrices X [M x N] (M <= N).
struct NsArgs {
  int Z, M, N, tiles_n, tiles;
  int pl;             // bf16 planes of every product operand in this iteration
  int fold;           // B' = a I + b A + c A^2 (else B = b A + c A^2 and the update adds
                      // a X from all of xin's planes in its epilogue)
  float coef_a, coef_b, coef_c;
  const float* part;  // iteration 0: per-tile sums of squares of the unscaled gradient
  int nparts;
  int first;          // iteration 0 (fold the 1/(|G|_F + eps) scale)
  int last;           // final iteration: write U instead of planes
  float eps;
  PlaneBuf xin;       // gram, update: X planes [M][N] (iteration 0: planes of G); the
                      // products read its first pl planes
  PlaneBuf ain;       // poly: A planes [M][M] ; update: B planes [M][M]
  PlaneBuf aout;      // gram: A planes ; poly: B planes
  PlaneBuf xout;
  float* U;           // last: U in weight orientation
  int tr_mask;
  int P;
  int steps;          // fused small-matrix launch: all iterations, and
  int one;            // the one-plane iteration mask
};

// matrices the fused Newton-Schulz launch takes: X orientation up to 64 x 128
constexpr int NS_SMALL_M = 64, NS_SMALL_N = 128;

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
// backward through an update (ttt_backward.hip)
hipError_t launch_tfront(const TFrontArgs& a, int Z, hipStream_t s);
hipError_t launch_eta_sum(const EtaSumArgs& a, int Z, hipStream_t s);
// dK (np 4: B0, B1 by columns, B2, B3 by rows) and dV (np 2, both by rows)
hipError_t launch_rowgemm(const DqArgs& a, int np, int Z, hipStream_t s);
hipError_t launch_step_bwd(const StepBwdArgs& a, hipStream_t s);
// bcols: B operands read by columns (the dX update) or by rows (T and S)
// sym: a symmetric output (M = N, no gref / gpart, bcols false): upper tiles only, each
// off-diagonal one's planes stored with their mirror
hipError_t launch_gemm2(const Gemm2Args& a, bool bcols, hipStream_t s, bool sym = false);
hipError_t launch_ns_fin(const NsFinArgs& a, int Z, hipStream_t s);
hipError_t launch_add3(const Add3Args& a, hipStream_t s);
hipError_t launch_mom_bwd(const MomBwdArgs& a, hipStream_t s);
int gemm2_tiles(int M, int N);
// token ranges a contraction of `tiles` output tiles per matrix over nz matrices may split
// into (the host sizes the partial-sum buffer with it)
int contract_split_max(int tiles, int nz);
hipError_t launch_ns_gram(const NsArgs& a, hipStream_t s);
hipError_t launch_ns_poly(const NsArgs& a, hipStream_t s);
hipError_t launch_ns_small(const NsArgs& a, hipStream_t s);
hipError_t launch_ns_update(const NsArgs& a, hipStream_t s);
hipError_t launch_renorm(const RenormArgs& a, hipStream_t s);
hipError_t launch_split(const SplitArgs& a, int Z, hipStream_t s);
// two tensors of the same rows and width (a.n == b.n, a.d == b.d) in one launch
hipError_t launch_split2(const SplitArgs& a, const SplitArgs& b, int Z, hipStream_t s);
// three such tensors in one launch
hipError_t launch_split3(const SplitArgs& a, const SplitArgs& b, const SplitArgs& c, int Z,
                         hipStream_t s);
hipError_t launch_small(const SmallArgs& a, int loss, hipStream_t s);
bool small_supported(int fw, int ns_steps, int renorm, int act_bf16, int apply_first, int dim,
                     int hidden, int chunk, int ap, int gp);
hipError_t prepare_kernels();  // raise dynamic-LDS limits once per process
// n int32 zeros at p (a kernel, not a memset: also safe inside a captured graph)
hipError_t launch_fill_zero(int* p, int n, hipStream_t s);

// A whole sequence with the fp32 state in the caller's buffer w and all workspace carved
// from ws (ws_bytes), allocating nothing; with ws == nullptr only the host checks run and
// *need gets the workspace size (libttt.cpp).
// Set the calling thread's last-error message (ttt_last_error) and return st.
ttt_status report(ttt_status st, const char* msg);
ttt_status sequence_in_workspace(const ttt_config* cfg, float* w, const void* q, const void* k,
                                 const void* v, const float* eta, void* out, int64_t seq_len,
                                 char* ws, size_t ws_bytes, size_t* need, void* stream);

// tile sizes used by the contraction and Newton-Schulz stages (the host sizes buffers)
constexpr int CONTRACT_BM = 128, CONTRACT_BN = 128;
constexpr int CONTRACT_SPLIT_MAX = 16;   // token ranges of one contraction at most
// Parts of a contraction tile's sum of squares (the Newton-Schulz input's Frobenius norm)
// where the contraction may split its tokens: one per band of 16 rows, so that the split's
// second pass spreads a tile over that many workgroups.  An unsplit launch of such a
// contraction stores its tile's sum in the first part and zeros in the others.  Where the
// contraction never splits, a tile has one part.
constexpr int CONTRACT_SUM_SUB = 8;
int ns_tri_tiles(int M, int tile);

}  // namespace ttt
