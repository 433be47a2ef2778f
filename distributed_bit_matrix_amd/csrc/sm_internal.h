// Internal declarations of libsignmuon: device helpers, the matrix-group
// descriptor every batched kernel receives by value, and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "signmuon.h"

namespace sm {

// Every batched launch carries up to this many matrix groups in its kernel
// arguments; more groups are split over several launches.
constexpr int kMaxGroups = 12;
// Padded operand layout: every matrix copy used by the matrix cores is
// stored with rows and columns rounded up to this multiple (zero filled).
constexpr int kPad = 128;
// Elements per block of the padded elementwise sweeps.
constexpr int kChunk = 2048;

typedef uint16_t bf16_t;   // raw bfloat16 bits

// A run of same-shaped matrices whose offsets advance by constant strides
// (for example the same projection in each of 12 transformer layers).
struct Group {
  int32_t count;          // matrices in the run
  int32_t rows, cols;     // original shape
  int32_t idx0, idx_stride;      // global matrix index (per-matrix scalars)
  int64_t elem0, elem_stride;    // flat G / W / Mom / U offset
  int64_t word0, word_stride;    // packed-sign offset
  int64_t x0, x_stride;          // padded operand offset (Mp x Np)
  int64_t r0, r_stride;          // padded Gram offset (Rp x Rp)
  int64_t v0, v_stride;          // power-iteration vector offset (Rp)
  int64_t u0_0, u0_stride;       // caller start vector offset (min dim)
  int64_t c0, c_stride;          // partial-sum chunk offset
  int64_t kp0, kp_stride;        // split-k partial tiles offset (floats)
  int32_t ksplit;                // k splits of the long-k symmetric GEMMs
  int32_t kslabs;                // k slabs per split (even), if ksplit > 1
  // Filled per launch: block range and per-matrix work shape.
  int32_t block0;         // first block of this group in the launch
  int32_t blocks_per_mat;
  int32_t gm, gn, gk;     // GEMM dims (padded) or sweep extents
  int32_t tiles_n;        // GEMM tiles along n
  int32_t ops;            // GEMM operand flags (sm_launch.h OPS_*)
  int32_t vec_ok;         // flat offsets allow 16-byte vector access
  int32_t tile;           // GEMM block tile width (columns), shared by a launch
};

struct Groups {
  Group g[kMaxGroups];
  int32_t n;
  int32_t total_blocks;
};

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) {
  return (x + m - 1) / m * m;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#ifdef __HIP_DEVICE_COMPILE__
#define SM_DEV __device__ __forceinline__
#else
#define SM_DEV __host__ __device__ inline
#endif

// Storage of the Newton-Schulz iterate: every matrix is kept as S with its
// short side as rows (S = X when rows <= cols, S = X^T for a tall X),
// zero padded to multiples of kPad.  Every Gram is then S S^T with k along
// the rows of S and every update is S <- a S + B S.
SM_DEV bool s_tall(const Group& g) { return g.rows > g.cols; }
SM_DEV int s_rows(const Group& g) { return g.rows > g.cols ? g.cols : g.rows; }
SM_DEV int s_cols(const Group& g) { return g.rows > g.cols ? g.rows : g.cols; }
// Offset in the padded S of the caller-layout element (row, col).
SM_DEV int64_t s_index(const Group& g, int64_t row, int64_t col) {
  const int64_t ld = round_up(s_cols(g), kPad);
  return g.rows > g.cols ? col * ld + row : row * ld + col;
}

// Locate the group and matrix of a block: linear scan over <= kMaxGroups.
__device__ __forceinline__ int find_group(const Groups& G, int b) {
  int gi = 0;
#pragma unroll 1
  for (int i = 1; i < G.n; ++i)
    if (b >= G.g[i].block0) gi = i;
  return gi;
}

// bfloat16 <-> float32.  Rounding to nearest even via the hardware
// conversion of gfx950 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}
// Split f into hi + lo bfloat16 parts with hi = rne(f), lo = rne(f - hi).
__device__ __forceinline__ void split_bf16(float f, bf16_t& hi, bf16_t& lo) {
  hi = f32_to_bf16(f);
  lo = f32_to_bf16(f - bf16_to_f32(hi));
}

// ---------------------------------------------------------------------------
// Workspace plan (host): per-matrix placement of the padded operand copies,
// Gram buffers, power vectors and partial sums, grouped for launches.
// ---------------------------------------------------------------------------
struct MatPlan {
  int64_t rows, cols, r;
  bool tall;
  int64_t Mp, Np, Rp;
  int64_t elem_off, word_off;
  int64_t x_off, r_off, v_off, u0_off, c_off;
  int64_t chunks;         // padded sweep chunks of kChunk elements
  int32_t idx;
  int32_t ks;             // k splits of its Gram (1 = none)
  int32_t kslabs;         // k slabs per split
  int64_t kp_off;         // its split-k partial tiles (floats), if ks > 1
};

enum Precision { P_F32 = 0, P_BF16 = 1, P_BF16X3 = 2 };

struct Plan {
  int nm = 0;
  int precision = P_BF16;
  bool quintic = false;
  bool spectral = false;
  // Newton-Schulz in Gram space (bfloat16 cubic, Frobenius scale):
  // X_K = Q_K X_0 with the iteration carried on Rp x Rp symmetric matrices
  bool gram_space = false;
  // bfloat16 symmetric Rp x Rp operands (Gram operands, the quintic square,
  // the Gram-space iterates) stored as their upper-triangular 128x128 tiles
  bool upper = false;
  int64_t x_total = 0, r_total = 0, v_total = 0, c_total = 0, kp_total = 0;
  // workspace byte offsets (0 = absent)
  size_t off_x[2][2] = {{0, 0}, {0, 0}};  // [pingpong][hi/lo] (or f32 in [p][0])
  size_t off_b[2] = {0, 0};   // Newton-Schulz right/left factor B (hi/lo)
  size_t off_a[2] = {0, 0};   // quintic: A (hi/lo)
  size_t off_araw = 0;        // spectral: raw float32 Gram
  size_t off_vec = 0;         // power vectors, 2 * v_total floats
  size_t off_tag = 0;         // one-launch power iteration: 2 * v_total tagged entries
  size_t off_part = 0;        // partial sums, c_total floats
  size_t off_kpart = 0;       // split-k partial Gram tiles, kp_total floats
  size_t off_gs = 0;          // Gram-space A, A', T, Q, Q' (bfloat16, r_total each)
  size_t off_scal = 0;        // per-matrix c = 1/(s+eps)
  size_t off_status = 0;      // int32 status word
  size_t total = 0;
};

}  // namespace sm
