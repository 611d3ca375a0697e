// Internal interface between the block's host code (ttt_block.cpp) and its kernels
// (ttt_block.hip).  Not part of the public ABI.
#pragma once

#include "ttt_block.h"
#include "ttt_internal.h"

namespace ttt {

constexpr int ATT_D = TTT_ATTN_HEAD_DIM;   // attention head dimension
constexpr int ATT_Q = 128;                 // queries per workgroup (4 waves x 32)
constexpr int ATT_KV = 64;                 // keys per step
constexpr int BLK_MAX_TTT_HEADS = 16;      // step-size projections per row
// 256 x 256 projection tiles for launches with at least LINEAR_WIDE_MIN of them and at least
// LINEAR_WIDE_K input features
constexpr int64_t LINEAR_WIDE_MIN = 512;
constexpr int32_t LINEAR_WIDE_K = 2048;

struct AttnArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* out;
  int64_t ld, ldo;
  int32_t T, heads, window, mode, qblocks, total;
  float scale2;   // log2(e) / sqrt(ATT_D)
};

struct LinearArgs {
  const u16* x;
  const u16* w;
  const u16* resid;
  u16* y;
  int64_t rows;
  int32_t K, N, tiles_n, tiles_m, group_m;
  int64_t tiles;
  int32_t tile;   // block tile edge: 128, or 256 for launches with many such tiles
};

// RMS normalisation of rows of x [rows][D] into y; with w_eta, also the TTT step sizes
// eta [b][h][t] = 0.01 sigmoid(y_row . w_eta[h]) for row = b T + t.
struct RmsArgs {
  const u16* x;
  u16* y;
  int64_t rows;
  int32_t D;
  const u16* w_eta;
  float* eta;
  int32_t heads;
  int32_t T;
};

// qkv rows [B T][3 D] -> q, k (unit length per head), v as [B][H][T][d]
struct HeadSplitArgs {
  const u16* qkv;
  u16 *q, *k, *v;
  int32_t T, B, H, d;
};

// o [B][H][T][d] -> y [B T][H d]
struct HeadMergeArgs {
  const u16* o;
  u16* y;
  int32_t T, B, H, d;
};

hipError_t launch_window_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_linear(const LinearArgs& a, int epilogue, hipStream_t st);
hipError_t launch_rmsnorm(const RmsArgs& a, hipStream_t st);
hipError_t launch_split(const HeadSplitArgs& a, hipStream_t st);
hipError_t launch_merge(const HeadMergeArgs& a, hipStream_t st);

}  // namespace ttt
