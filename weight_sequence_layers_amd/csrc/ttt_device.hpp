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
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Sum of v over the workgroup (every thread gets it); scratch: one float per wave of LDS.
// Contains barriers: call from every thread.
__device__ __forceinline__ void lds_barrier();
__device__ __forceinline__ float block_sum(float v, float* scratch);

// ------------------------------------------------------------------------ GEMM operands
// A K-contiguous operand made of 1..3 bf16 planes: element (r, k) of plane q, problem z
// lives at p[q * pstride + z * zstride + r * ld + k].  Rows >= rows and k >= K read as zero.
struct Operand {
  const u16* p;
  int64_t pstride;
  int64_t ld;
  int64_t zstride;
  int32_t planes;
  int32_t rows;
};

__host__ __device__ inline Operand make_operand(const u16* p, int64_t pstride, int64_t ld,
                                                int64_t zstride, int planes, int rows) {
  Operand o;
  o.p = p; o.pstride = pstride; o.ld = ld; o.zstride = zstride; o.planes = planes; o.rows = rows;
  return o;
}

// A buffer of 1..3 bf16 planes: plane q of problem z, row r, column c lives at
// base[q * plane_stride + z * zstride + r * ld + c].
struct PlaneBuf {
  u16* base;
  int64_t plane_stride;
  int64_t zstride;
  int64_t ld;
  int32_t np;
};

// ------------------------------------------------------------------------ GEMM core
// Multi-product tile GEMM main loop for gfx950.
//
//   NA A-operands (tile rows = M) and NB B-operands (tile rows = N); product p < NB
//   accumulates  C_p[m][n] += sum_k A_{ia(p)}[m][k] * B_p[n][k]  with ia(p) = 1 for the
//   last product when NA == 2, else 0.
//
// Operand layouts in memory (bit i of the template masks LAM / LBM is operand i's layout):
//   L_ROW  element (r, k) at r * ld + k   (rows contiguous along K)
//   L_COL  element (r, k) at k * ld + r   (K-rows contiguous along the M / N index)
// Both are staged into LDS without rearrangement and read into MFMA fragments with
// ds_read_b128 (L_ROW) or the gfx950 transposing ds_read_b64_tr_b16 (L_COL), so no
// operand is ever transposed in memory.
//
// Planes: the A operands share one plane count PA, the B operands one count PB.  The pair
// (qa, qb) of planes is taken when qa + qb < max(PA, PB); each taken pair is one "segment"
// of the K loop, so a multi-plane product is a longer K loop over the same LDS tiles and
// the inner loop has no plane-dependent control flow.
//
// Block: WGM x WGN waves, wave tile (BM/WGM) x (BN/WGN) of 32x32x16 MFMA tiles.  K steps of
// BK (64, or 32 to halve the LDS of a stage) through two LDS stages, filled by direct
// global-to-LDS buffer loads one step ahead.
// Elements outside an operand read as zero (out-of-range buffer loads return 0).  16-byte
// LDS chunks are XOR-swizzled by row so that fragment reads spread over the banks.
enum Layout { L_ROW = 0, L_COL = 1 };

// row tiles (BK / 8 chunks of 16 bytes per row): the rows one 16-lane read phase touches
// land on distinct banks
template <int BK>
__device__ __forceinline__ int swz_row(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }
// column tiles: rows k..k+3 read together by one transposing read land on distinct banks
template <int R>
__device__ __forceinline__ int swz_col(int k) { return R >= 128 ? (k & 3) << 2 : (k & 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte-per-lane direct load from a buffer into LDS (lane l writes dst + 16 l).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_void_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
}

// Per-thread load plan of one operand tile (R rows x BK k) in either layout.
template <int R, int NT, int BK = 64>
struct TileLoad {
  static_assert(BK == 64 || BK == 32, "K step of 64 or 32");
  static constexpr int CHUNKS = R * BK / 8;        // 16-byte chunks per tile
  static constexpr int NW = NT / 64;               // waves of the block
  // PART: fewer chunks than threads; CHUNKS / 64 of the waves load the tile, one chunk a
  // lane, starting at wave rot (so that the tiles of one step spread over all waves)
  static constexpr bool PART = CHUNKS < NT;
  static constexpr int C = PART ? 1 : CHUNKS / NT;  // per thread
  static constexpr int BYTES = R * BK * 2;
  static_assert(PART ? NT % CHUNKS == 0 && CHUNKS % 64 == 0 : CHUNKS % NT == 0,
                "uneven tile load");
  static_assert(R % 64 == 0, "tile rows must be a multiple of 64");
  uint32_t off[C];   // byte offset of the chunk at k0 = 0, or an out-of-range value
  int kk[C];         // k of the chunk's first element relative to k0
  uint32_t kstride;  // bytes per unit of k0
  int slice;         // LDS byte offset of this wave's 1 KB slice in round 0 (wave-uniform)
  bool act;          // whether this wave loads the tile (wave-uniform)

  // Chunks go to LDS by direct (DMA) loads, which write lane l of a wave's load to 16 l
  // bytes past the wave's base: the wave at loader position w fills LDS chunk
  // p = c NT + 64 w + lane in round c, so it loads the global chunk that the swizzled
  // layout keeps at p (XOR is its own inverse).
  __device__ __forceinline__ void init(const Operand& o, int row0, bool col, int rot = 0) {
    const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
    const int w = PART ? (wave - rot % NW + NW) % NW : wave;
    act = !PART || w < CHUNKS / 64;
    slice = __builtin_amdgcn_readfirstlane(w) * 64 * 16;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = w * 64 + lane + c * NT;
      if (!act) {
        kk[c] = 0;
        off[c] = 0xC0000000u;
      } else if (!col) {
        const int r = ch / (BK / 8), kc = (ch % (BK / 8)) ^ swz_row<BK>(r);
        kk[c] = kc * 8;
        off[c] = (row0 + r < o.rows) ? (uint32_t)(((int64_t)(row0 + r) * o.ld + kc * 8) * 2)
                                     : 0xC0000000u;
      } else {
        const int k = ch / (R / 8), mc = (ch % (R / 8)) ^ swz_col<R>(k);
        kk[c] = k;
        off[c] = (row0 + mc * 8 < o.rows) ? (uint32_t)(((int64_t)k * o.ld + row0 + mc * 8) * 2)
                                          : 0xC0000000u;
      }
    }
    kstride = col ? (uint32_t)(o.ld * 2) : 2u;
  }
};

// MFMA fragment (32 rows x 16 k) of a staged tile for k-substep s.
template <bool COL, int R, int BK = 64>
__device__ __forceinline__ bf16x8 read_frag(const char* tile, int row_base, int s) {
  const int lane = threadIdx.x & 63;
  if (!COL) {
    const int r = row_base + (lane & 31);
    const int ch = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(tile + r * (BK * 2) +
                                            ((ch ^ swz_row<BK>(r)) << 4));
  } else {
    // ds_read_b64_tr_b16: within each 16-lane group, lane j receives element (j % 4) of
    // the 4-element rows addressed by lanes 4e + j/4, e = 0..3.  Lane 4e + q addresses
    // k-row kb + e at m + 4q, so lane j gets A[m + j][kb + e] for e = 0..3.
    const int g = lane >> 4, j = lane & 15;
    const int m = row_base + 16 * (g & 1) + 4 * (j & 3);
    const int kb = 16 * s + 8 * (g >> 1) + (j >> 2);
    s16x4 lo, hi;
    {
      const int k = kb;
      const char* a = tile + k * R * 2 + (((m >> 3) ^ swz_col<R>(k)) << 4) + (m & 7) * 2;
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(a));
    }
    {
      const int k = kb + 4;
      const char* a = tile + k * R * 2 + (((m >> 3) ^ swz_col<R>(k)) << 4) + (m & 7) * 2;
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(a));
    }
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

// ------------------------------------------------------------------------ LDS barrier
// Workgroup barrier for LDS reuse: each thread first waits for its own LDS operations only,
// not for its outstanding global stores (which __syncthreads' release fence would wait
// for).  The empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maximum
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The sum of n partial sums p[0 .. n) in one fixed order: eight interleaved running sums
// (eight loads in flight at a time), the remainder into the first of them, then the eight
// in order.
__device__ __forceinline__ float sum_parts(const float* p, int n) {
  float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int i = 0;
  for (; i + 8 <= n; i += 8)
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] += p[i + j];
  for (int j = 0; i + j < n; ++j) t[j] += p[i + j];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += t[j];
  return s;
}

__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lds_barrier();
  if (lane == 0) scratch[wave] = v;
  lds_barrier();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += scratch[w];
  lds_barrier();
  return t;
}

// PL > 0 selects the plane-resident product: A[0..NA) and B[0..NB) are the bf16 planes of
// one A and one B (each operand with planes = 1), PL = max(NA, NB); every K step loads all
// NA + NB plane tiles once and accumulates the plane products (i, j) with i + j < PL into
// one accumulator.  With PG > 1 groups: B holds the PL planes of each of PG operands
// (B[g PL + j]) and A those of NA / PL operands, and accumulator g takes the plane products
// of B operand g with its A operand (paired as products are below).
// PL = 0 keeps one accumulator per B operand and runs plane pairs as K segments.
//
// SW selects the accumulator layout.  The MFMA computes D = A B with A's fragment giving
// D's rows and B's its columns.  SW = false feeds the A tile as A: element v of a lane's
// 32 x 32 tile sits at row 8 (v / 4) + 4 (lane / 32) + v % 4, column lane % 32.  SW = true
// feeds the B tile as A, computing the transposed tile: element v then sits at row
// lane % 32, column 8 (v / 4) + 4 (lane / 32) + v % 4, so each lane holds runs of four
// consecutive columns, which the tile stores write to LDS four at a time.
//
// WGK > 1 splits every K step among WGK groups of WGM x WGN waves (group k takes
// k-substeps [k, k + 1) BK / 16 / WGK of each step for its whole wave tile), for blocks
// that would otherwise run too few waves per CU.  reduce() then sums the groups' partial
// tiles through LDS into one owner per run of four accumulator elements (run g of tile t
// to group (4 t + g) mod WGK); for_each, for_each4 and the tile stores visit the owned
// runs only.
//
// SUM = true (PL = 0) accumulates every product into one accumulator (the kernel wants only
// their sum).
//
// Pairing of A operands with products (PL = 0): NB0 >= 0 gives products p < NB0 A[0] and
// the others A[1]; else with NA == NB product p takes A[p], and otherwise every product
// takes A[0] except, with NA == 2, the last, which takes A[1].
template <int BM, int BN, int WGM, int WGN, int NA, int NB, int LAM = 0, int LBM = 0, int PL = 0,
          int BK_ = 64, bool SW_ = false, int WGK_ = 1, int NB0 = -1, bool SUM = false,
          int PG = 1>
struct Gemm {
  static constexpr bool SW = SW_;
  static constexpr int WGK = WGK_;
  static constexpr int NT = WGM * WGN * WGK * 64;
  static constexpr int TBM = BM, TBN = BN;
  static constexpr int STORE_LDS = (BM + 8) * (BN + 8) * 2;
  static constexpr int BK = BK_;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int SPW = BK / 16 / WGK;   // k-substeps of a step per wave
  static_assert(SPW >= 1 && SPW * 16 * WGK == BK, "K step must split evenly among groups");
  using TA = TileLoad<BM, NT, BK>;
  using TB = TileLoad<BN, NT, BK>;
  static constexpr bool acol(int i) { return (LAM >> i) & 1; }
  static constexpr bool bcol(int i) { return (LBM >> i) & 1; }
  static constexpr int A_TILE = TA::BYTES, B_TILE = TB::BYTES;
  static constexpr int STAGE = NA * A_TILE + NB * B_TILE;
  // The reduction of the groups' partial tiles (WGK > 1) runs one accumulator at a time,
  // in RED_R rounds over each wave's 32 x 32 tiles, so that a round's slots fit in
  // max(STAGE, 32 KB) where whole accumulators would not.
  static constexpr int RED_FULL = WGK > 1 ? BM * BN * 4 * (WGK - 1) : 0;
  static constexpr int red_rounds() {
    const int cap = STAGE > 32768 ? STAGE : 32768;
    int r = 1;
    while (r < TM * TN && ((TM * TN) % r != 0 || RED_FULL / r > cap)) ++r;
    return r;
  }
  static constexpr int RED_R = red_rounds();
  static constexpr int RED_LDS = RED_FULL / RED_R;   // LDS the reduction takes
  // LDS: stage buffer 0 (also the epilogue's staging area) and stage buffer 1, declared as
  // two separate __shared__ arrays by the kernel (GEMM_LDS)
  static_assert(TM >= 1 && TN >= 1, "tile too small for the block");
  static_assert(PL == 0 || (PG == 1 ? PL == (NA > NB ? NA : NB) : NB == PG * PL && NA % PL == 0),
                "plane-resident mode: PL = max(NA, NB), or PG groups of PL planes");
  static constexpr int NACC = PL ? PG : SUM ? 1 : NB;
  static constexpr int NGA = PG > 1 ? NA / PL : 1;   // A operands of grouped plane products

  f32x16 acc[NACC][TM][TN];

  static __device__ __forceinline__ constexpr int ia(int p) {
    return NB0 >= 0 ? (p < NB0 ? 0 : 1) : NA == NB ? p : (NA == 2 && p == NB - 1) ? 1 : 0;
  }
  // A operand of plane group g (the same pairing over operands)
  static __device__ __forceinline__ constexpr int ga(int g) {
    return NB0 >= 0 ? (g < NB0 ? 0 : 1) : NGA == PG ? g : (NGA == 2 && g == PG - 1) ? 1 : 0;
  }

  // one 32 x 32 x 16 product of an A-tile fragment and a B-tile fragment into c
  static __device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    return SW ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0)
              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // row and column of element v of this lane's 32 x 32 tile, relative to the tile
  static __device__ __forceinline__ int elem_row(int v, int lane) {
    return SW ? (lane & 31) : 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
  }
  static __device__ __forceinline__ int elem_col(int v, int lane) {
    return SW ? 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3) : (lane & 31);
  }

  // origin of this wave's tile in the block tile
  // this wave's K group and its place in the WGM x WGN grid
  static __device__ __forceinline__ int wave_k() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) / (WGM * WGN));
  }
  static __device__ __forceinline__ int wave_mn() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) % (WGM * WGN));
  }
  static __device__ __forceinline__ int wm0() { return (wave_mn() / WGN) * WM; }
  static __device__ __forceinline__ int wn0() { return (wave_mn() % WGN) * WN; }
  // whether this wave holds the final value of run g (elements 4g .. 4g + 3) of its tile
  // (tm, tn) after reduce()
  static __device__ __forceinline__ bool owns(int tm, int tn, int g) {
    return WGK == 1 || ((tm * TN + tn) * 4 + g) % WGK == wave_k();
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int p = 0; p < NACC; ++p)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[p][i][j][v] = 0.f;
  }

  // A / B point at NA / NB consecutive operands (normally inside the kernel arguments).
  // st0 / st1: the two stage buffers, distinct __shared__ arrays.  Each K step's tiles
  // are loaded straight into LDS (buffer loads with the LDS flag) one step ahead: step t
  // computes from one buffer while step t + 1 lands in the other.  Every LDS access names
  // one of two distinct arrays, which lets the compiler see that the fragment reads never
  // touch the buffer being filled and wait for the loads only at the end of each step.
  //
  // krot rotates the K order: the steps cover k0 = krot, krot + BK, ... modulo K (the same
  // sum in another order).  A caller passing krot != 0 must have K a multiple of BK and one
  // plane segment.
  __device__ __forceinline__ void run(const Operand* __restrict__ A,
                                      const Operand* __restrict__ B, int m0, int n0, int z,
                                      int K, char* st0, char* st1, int krot = 0) {
    const int wm0 = this->wm0();
    const int wn0 = this->wn0();

    // plane-pair segments
    const int PA = A[0].planes, PB = B[0].planes;
    const int PM = PA > PB ? PA : PB;
    uint32_t segs = 0;  // 4 bits per segment: qa | qb << 2
    int nseg = 0;
#pragma unroll
    for (int qa = 0; qa < 3; ++qa)
#pragma unroll
      for (int qb = 0; qb < 3; ++qb)
        if (qa < PA && qb < PB && qa + qb < PM) {
          segs |= (uint32_t)(qa | (qb << 2)) << (4 * nseg);
          ++nseg;
        }
    const int nk = (K + BK - 1) / BK;
    const int total = nseg * nk;
    if (total == 0) return;

    TA la[NA];
    TB lb[NB];
    const u16* pa_[NA];
    const u16* pb_[NB];
    int na_[NA], nb_[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      la[i].init(A[i], m0, acol(i), i * (TA::CHUNKS / 64));
      pa_[i] = A[i].p + (int64_t)z * A[i].zstride;
      na_[i] = (int)(!acol(i) ? (int64_t)A[i].rows * A[i].ld * 2 : (int64_t)K * A[i].ld * 2);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      lb[i].init(B[i], n0, bcol(i), NA * (TA::CHUNKS / 64) + i * (TB::CHUNKS / 64));
      pb_[i] = B[i].p + (int64_t)z * B[i].zstride;
      nb_[i] = (int)(!bcol(i) ? (int64_t)B[i].rows * B[i].ld * 2 : (int64_t)K * B[i].ld * 2);
    }

    // Steps that lie wholly inside K move the buffer's base by the step's k offset (scalar
    // arithmetic only, no per-lane work); a partial last step checks each chunk against K.
    // The steps are loaded in order; (sg_n, k0_n) is the next one's segment and k offset.
    int sg_n = 0, k0_n = 0;
    auto issue = [&](char* st) __attribute__((always_inline)) {
      const int sg = sg_n;
      int k0 = k0_n + krot;
      if (k0 >= K) k0 -= K;
      k0_n += BK;
      if (k0_n >= K) {
        k0_n = 0;
        ++sg_n;
      }
      const int qa = (segs >> (4 * sg)) & 3, qb = (segs >> (4 * sg + 2)) & 3;
      if (k0 + BK <= K) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const uint32_t kb = (uint32_t)k0 * la[i].kstride;
          const char* base = reinterpret_cast<const char*>(pa_[i] + qa * A[i].pstride) + kb;
          const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
              (void*)base, (short)0, na_[i] - (int)kb, 0x00020000);
#pragma unroll
          for (int c = 0; c < TA::C; ++c)
            if (la[i].act)
              dma16(rk, (lds_void_t*)(st + i * A_TILE + c * NT * 16 + la[i].slice), la[i].off[c]);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint32_t kb = (uint32_t)k0 * lb[i].kstride;
          const char* base = reinterpret_cast<const char*>(pb_[i] + qb * B[i].pstride) + kb;
          const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
              (void*)base, (short)0, nb_[i] - (int)kb, 0x00020000);
#pragma unroll
          for (int c = 0; c < TB::C; ++c)
            if (lb[i].act)
              dma16(rk, (lds_void_t*)(st + NA * A_TILE + i * B_TILE + c * NT * 16 + lb[i].slice),
                    lb[i].off[c]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const uint32_t kb = (uint32_t)k0 * la[i].kstride;
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(pa_[i] + qa * A[i].pstride), (short)0, na_[i], 0x00020000);
#pragma unroll
          for (int c = 0; c < TA::C; ++c)
            if (la[i].act)
              dma16(rs, (lds_void_t*)(st + i * A_TILE + c * NT * 16 + la[i].slice),
                    (k0 + la[i].kk[c] < K) ? la[i].off[c] + kb : 0xFFFFFFF0u);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint32_t kb = (uint32_t)k0 * lb[i].kstride;
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(pb_[i] + qb * B[i].pstride), (short)0, nb_[i], 0x00020000);
#pragma unroll
          for (int c = 0; c < TB::C; ++c)
            if (lb[i].act)
              dma16(rs, (lds_void_t*)(st + NA * A_TILE + i * B_TILE + c * NT * 16 + lb[i].slice),
                    (k0 + lb[i].kk[c] < K) ? lb[i].off[c] + kb : 0xFFFFFFF0u);
        }
      }
    };
    auto compute = [&](const char* st) __attribute__((always_inline)) {
#pragma unroll
      for (int ss = 0; ss < SPW; ++ss) {
        const int s = wave_k() * SPW + ss;
        bf16x8 fa[NA][TM], fb[NB][TN];
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            fa[i][t] = acol(i) ? read_frag<true, BM, BK>(st + i * A_TILE, wm0 + t * 32, s)
                               : read_frag<false, BM, BK>(st + i * A_TILE, wm0 + t * 32, s);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int t = 0; t < TN; ++t)
            fb[i][t] = bcol(i) ? read_frag<true, BN, BK>(st + NA * A_TILE + i * B_TILE,
                                                        wn0 + t * 32, s)
                               : read_frag<false, BN, BK>(st + NA * A_TILE + i * B_TILE,
                                                         wn0 + t * 32, s);
        if constexpr (PL > 0 && PG > 1) {
#pragma unroll
          for (int g = 0; g < PG; ++g)
#pragma unroll
            for (int i = 0; i < PL; ++i)
#pragma unroll
              for (int j = 0; j < PL; ++j)
                if (i + j < PL) {
#pragma unroll
                  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                      acc[g][tm][tn] = mma(fa[ga(g) * PL + i][tm], fb[g * PL + j][tn],
                                           acc[g][tm][tn]);
                }
        } else if constexpr (PL > 0) {
#pragma unroll
          for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              if (i + j < PL) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                  for (int tn = 0; tn < TN; ++tn)
                    acc[0][tm][tn] = mma(fa[i][tm], fb[j][tn], acc[0][tm][tn]);
              }
        } else {
#pragma unroll
          for (int p = 0; p < NB; ++p)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
              for (int tn = 0; tn < TN; ++tn)
                acc[SUM ? 0 : p][tm][tn] =
                    mma(fa[ia(p)][tm], fb[p][tn], acc[SUM ? 0 : p][tm][tn]);
        }
      }
    };
    // end of a step: this thread's loads have landed and its LDS reads are done (wait for
    // every counter), then the whole block meets
    auto step_end = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };

    issue(st0);
    step_end();
    for (int t = 0; t < total; ++t) {
      char* cur = (t & 1) ? st1 : st0;
      char* nxt = (t & 1) ? st0 : st1;
      if (t + 1 < total) issue(nxt);
      compute(cur);
      step_end();
    }
  }

  // Swapped layout only: visit this thread's runs of four consecutive columns,
  //   f(tm, tn, g, row, col): elements 4g .. 4g + 3 of tile (tm, tn) at (row, col .. col + 3)
  // relative to the block tile origin.
  template <class F>
  __device__ __forceinline__ void for_each4(F f) const {
    static_assert(SW, "runs of columns need the swapped layout");
    const int lane = threadIdx.x & 63;
    const int wm0 = this->wm0();
    const int wn0 = this->wn0();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (owns(tm, tn, g))
            f(tm, tn, g, wm0 + tm * 32 + elem_row(4 * g, lane),
              wn0 + tn * 32 + elem_col(4 * g, lane));
  }

  // Visit every accumulator element owned by this thread:
  //   f(tm, tn, v, row, col)  with row/col relative to the block tile origin.
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    const int lane = threadIdx.x & 63;
    const int wm0 = this->wm0();
    const int wn0 = this->wn0();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (owns(tm, tn, v >> 2))
            f(tm, tn, v, wm0 + tm * 32 + elem_row(v, lane), wn0 + tn * 32 + elem_col(v, lane));
        }
  }

  // Sum the K groups' partial tiles (WGK > 1) into the owners of their runs, through red
  // (RED_LDS bytes of LDS that no wave still reads).  In the round that covers tile t (t
  // counted over the wave's TM x TN tiles), a non-owner of run g sends it to slot
  // ((wave_mn TPR + t mod TPR) 4 + g) (WGK - 1) + rank, 64 lanes x 16 bytes.
  // Contains barriers: call from every thread.
  __device__ __forceinline__ void reduce(char* red) {
    if constexpr (WGK > 1) {
      constexpr int TPR = TM * TN / RED_R;   // tiles per round
      const int lane = threadIdx.x & 63;
      const int wk = wave_k(), wmn = wave_mn();
#pragma unroll
      for (int p = 0; p < NACC; ++p)
#pragma unroll
        for (int rr = 0; rr < RED_R; ++rr) {
          if (p || rr) lds_barrier();   // the previous round's slots have been read
#pragma unroll
          for (int tt = 0; tt < TPR; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int t = rr * TPR + tt;
              const int owner = (t * 4 + g) % WGK;
              if (owner == wk) continue;
              const int rank = (wk - owner - 1 + WGK) % WGK;
              char* slot = red + (((wmn * TPR + tt) * 4 + g) * (WGK - 1) + rank) * 1024;
              const f32x16& a = acc[p][t / TN][t % TN];
              *reinterpret_cast<f32x4*>(slot + lane * 16) =
                  f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
            }
          lds_barrier();
#pragma unroll
          for (int tt = 0; tt < TPR; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int t = rr * TPR + tt;
              if ((t * 4 + g) % WGK != wk) continue;
#pragma unroll
              for (int rank = 0; rank < WGK - 1; ++rank) {
                const char* slot = red + (((wmn * TPR + tt) * 4 + g) * (WGK - 1) + rank) * 1024;
                const f32x4 x = *reinterpret_cast<const f32x4*>(slot + lane * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[p][t / TN][t % TN][4 * g + e] += x[e];
              }
            }
        }
      lds_barrier();
    }
  }
};

// The two stage buffers of a Gemm type G as distinct __shared__ arrays (distinct objects
// are what lets the compiler keep fragment reads of one buffer clear of the loads in
// flight into the other); `smem`, the first, is also the epilogue's staging area.
#define GEMM_LDS(G) GEMM_LDS_EPI(G, G::STORE_LDS)
// the same with the first buffer large enough for an epilogue that needs EPI bytes
#define GEMM_LDS_EPI(G, EPI)                                                                  \
  __shared__ __attribute__((aligned(1024)))                                                    \
  char gemm_st0_[(G::STAGE > G::RED_LDS ? G::STAGE : G::RED_LDS) > (EPI)                      \
                     ? (G::STAGE > G::RED_LDS ? G::STAGE : G::RED_LDS)                        \
                     : (EPI)];                                                                \
  __shared__ __attribute__((aligned(1024))) char gemm_st1_[G::STAGE];                         \
  char* const smem = gemm_st0_
// the stage buffers GEMM_LDS declares, as Gemm::run takes them
#define GEMM_STAGES gemm_st0_, gemm_st1_

// ------------------------------------------------------------------------ block order
// Workgroups of a launch are handed to the 8 XCDs round-robin by linear id, and each XCD
// has its own L2.  xcd_block() renumbers the launch so that XCD x runs a contiguous range
// of logical blocks: with logical ids ordered (problem, tile), the tiles that share a
// problem's operands run on one XCD and hit the same L2.
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int xcd_block(int id, int total) {
  const int q = total / NUM_XCD, r = total % NUM_XCD;
  const int x = id % NUM_XCD, j = id / NUM_XCD;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// Upper tile t (row-major over ti <= tj) of an nt x nt grid of tiles.
__device__ __forceinline__ void tri_tile(int t, int nt, int& ti, int& tj) {
  ti = 0;
  while (t >= nt - ti) {
    t -= nt - ti;
    ++ti;
  }
  tj = ti + t;
}

// ------------------------------------------------------------------------ tile stores
// Write one block tile of fp32 values (held in the MFMA accumulator layout of gemm G) as
// bf16 planes through LDS, so that global stores are 16-byte vectors along the buffer's
// contiguous dimension.
//   TILE_NORMAL: element (r, c) of the tile goes to row row0 + r, column col0 + c;
//   TILE_SYM   : square diagonal tile of a symmetric matrix: only elements with r <= c are
//                taken, each written to (r, c) and (c, r) (smem as for TILE_BOTH);
//   TILE_BOTH  : square tile written at (row0 + r, col0 + c) and, transposed, at
//                (col0 + c, row0 + r) (an off-diagonal tile of a symmetric matrix).
// Up to MAXP planes are staged per pass (each value is split once); more planes take more
// passes. rlim / clim bound the tile's rows / columns (relative to the tile origin); the
// limit of the buffer's contiguous dimension must be a multiple of 8. smem needs
// store_lds_bytes<G, MODE, MAXP>() bytes. Contains barriers: call from every thread.
enum TileMode { TILE_NORMAL = 0, TILE_SYM = 1, TILE_BOTH = 2 };

template <class G, int MODE, int MAXP>
constexpr int store_lds_bytes() {
  return MAXP * (MODE == TILE_BOTH ? 2 : 1) * G::TBM * (G::TBN + 8) * 2;
}

// store_planes with the plane count NP fixed, P planes per pass.
template <class G, int MODE, int NP, int P>
__device__ __forceinline__ void store_planes_n(const f32x16 (&v)[G::TM][G::TN], char* smem,
                                               const PlaneBuf& dst, int z, int row0, int col0,
                                               int rlim, int clim) {
  constexpr int TBM = G::TBM, TBN = G::TBN, LD = TBN + 8;
  constexpr int NO = MODE == TILE_BOTH ? 2 : 1;    // staged orientations
  constexpr int REG = TBM * LD;                    // elements per staged region
  constexpr int CPR = TBN / 8;                     // 16-byte chunks per staged row
  static_assert(MODE == TILE_NORMAL || TBM == TBN, "symmetric stores take square tiles");
  u16* t = reinterpret_cast<u16*>(smem);
  const int lane = threadIdx.x & 63;
  const int wm0 = G::wm0(), wn0 = G::wn0();
#pragma unroll
  for (int q0 = 0; q0 < NP; q0 += P) {
    const int nq = NP - q0 < P ? NP - q0 : P;
    lds_barrier();
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (!G::owns(tm, tn, g)) continue;
          // elements 4g .. 4g + 3: four consecutive columns of one row (SW) or four
          // consecutive rows of one column
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = v[tm][tn][4 * g + e];
            for (int i = 0; i < q0; ++i) x[e] -= bf2f(f2bf(x[e]));   // earlier passes' planes
          }
          const int r = wm0 + tm * 32 + G::elem_row(4 * g, lane);
          const int c = wn0 + tn * 32 + G::elem_col(4 * g, lane);
#pragma unroll
          for (int qq = 0; qq < P; ++qq) {
            if (qq >= nq) continue;
            u16 h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              h[e] = f2bf(x[e]);
              x[e] -= bf2f(h[e]);
            }
            u16* tq = t + qq * NO * REG;
            if constexpr (G::SW && MODE != TILE_SYM) {
              uint2 w;
              w.x = h[0] | ((uint32_t)h[1] << 16);
              w.y = h[2] | ((uint32_t)h[3] << 16);
              *reinterpret_cast<uint2*>(tq + r * LD + c) = w;
              if (MODE == TILE_BOTH) {
#pragma unroll
                for (int e = 0; e < 4; ++e) tq[REG + (c + e) * LD + r] = h[e];
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int re = G::SW ? r : r + e, ce = G::SW ? c + e : c;
                if (MODE == TILE_NORMAL) {
                  tq[re * LD + ce] = h[e];
                } else if (MODE == TILE_BOTH) {
                  tq[re * LD + ce] = h[e];
                  tq[REG + ce * LD + re] = h[e];
                } else {
                  // TILE_SYM: an element below the diagonal writes to this lane's scratch
                  // word instead (an address select, not a branch)
                  const bool up = re <= ce;
                  u16* const scr = t + P * REG + 2 * lane;
                  *(up ? tq + re * LD + ce : scr) = h[e];
                  *(up ? tq + ce * LD + re : scr) = h[e];
                }
              }
            }
          }
        }
    lds_barrier();
    const int total = nq * NO * TBM * CPR;
    for (int ch = threadIdx.x; ch < total; ch += G::NT) {
      const int qq = ch / (NO * TBM * CPR);
      int rem = ch - qq * (NO * TBM * CPR);
      const int o = rem / (TBM * CPR);
      rem -= o * (TBM * CPR);
      const int rr = rem / CPR, cc = (rem % CPR) * 8;
      const int rl = o ? clim : rlim, cl = o ? rlim : clim;
      if (rr < rl && cc < cl) {
        u16* out = dst.base + (q0 + qq) * dst.plane_stride + (int64_t)z * dst.zstride;
        const int gr = o ? col0 + rr : row0 + rr, gc = o ? row0 + cc : col0 + cc;
        *reinterpret_cast<uint4*>(out + (int64_t)gr * dst.ld + gc) =
            *reinterpret_cast<const uint4*>(t + (qq * NO + o) * REG + rr * LD + cc);
      }
    }
  }
  lds_barrier();
}

// The plane count of dst (the same for the whole block) picks the store_planes_n
// instance, whose per-element work then has no plane-count branches.
template <class G, int MODE, int MAXP>
__device__ __forceinline__ void store_planes(const f32x16 (&v)[G::TM][G::TN], char* smem,
                                             const PlaneBuf& dst, int z, int row0, int col0,
                                             int rlim, int clim) {
  if (dst.np == 1) store_planes_n<G, MODE, 1, 1>(v, smem, dst, z, row0, col0, rlim, clim);
  else if (dst.np == 2)
    store_planes_n<G, MODE, 2, (MAXP < 2 ? MAXP : 2)>(v, smem, dst, z, row0, col0, rlim, clim);
  else if (dst.np == 3)
    store_planes_n<G, MODE, 3, (MAXP < 3 ? MAXP : 3)>(v, smem, dst, z, row0, col0, rlim, clim);
}

// one plane per pass: the least LDS (the Gemm's STORE_LDS)
template <class G, int MODE>
__device__ __forceinline__ void store_tile_planes(const f32x16 (&v)[G::TM][G::TN], char* smem,
                                                  const PlaneBuf& dst, int z, int row0,
                                                  int col0, int rlim, int clim) {
  store_planes<G, MODE, 1>(v, smem, dst, z, row0, col0, rlim, clim);
}

}  // namespace ttt
