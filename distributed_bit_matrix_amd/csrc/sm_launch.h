// Launch-side declarations of the kernels of libsignmuon.
#pragma once

#include "sm_internal.h"

namespace sm {

// Operand families of the batched GEMM: the padded copy of X (Mp x Np, row
// length Np) read with k along its rows (FAM_X) or with k down its columns
// (FAM_XK: the LDS tile holds k as rows and the fragments are read with the
// transposing LDS load), and the padded Gram-sized buffers (Rp x Rp, FAM_R,
// k along rows; FAM_R2 is a second such buffer, for products of two
// different symmetric matrices).
enum { FAM_X = 0, FAM_XK = 1, FAM_R = 2, FAM_R2 = 3 };
// Group.ops: A-operand family in bits 0-1, B-operand family in bits 2-3.
__host__ __device__ inline int gemm_ops(int a_fam, int b_fam) {
  return a_fam | (b_fam << 2);
}

enum Epi { E_RAW = 0, E_OP = 1, E_SQUARE = 2, E_UPDATE = 3 };
enum Out { O_X = 0, O_U = 1, O_BITS = 2, O_APPLY = 3, O_TERN = 4 };

// Source of the update's a X term on the first Newton-Schulz step: the
// caller's float32 matrix (XS_USER, full precision) or the bf16/f32 operand
// tiles as they pass through LDS (XS_OP).
enum XSrc { XS_USER = 0, XS_OP = 1 };

struct GemmArgs {
  Groups G;
  const void* x_hi; const void* x_lo;   // FAM_X operand buffers
  const void* r_hi; const void* r_lo;   // FAM_R operand buffers
  const void* r2_hi; const void* r2_lo; // FAM_R2 operand buffers
  int32_t epi, out, xsrc, scal_pow;
  // bfloat16 symmetric Rp x Rp operands and outputs (the R families; not
  // the raw Gram) are stored as their upper-triangular 128x128 tiles only:
  // symmetric outputs skip the mirror tile, and a product reading row
  // block t of such an operand takes its k-slabs left of the diagonal
  // (k < 128 t) from the stored tile above the diagonal, k-major.
  int32_t upper;
  float mul, ca, cb, cc;
  void* o_hi; void* o_lo;          // E_OP / E_SQUARE (R family), O_X (X family)
  // E_OP, unsplit launches: also o2 = o2_a I + o2_b (the Gram operand) in
  // bfloat16 (the Gram-space form's first factor), when o2_hi is set
  void* o2_hi; float o2_a, o2_b;
  float* o_raw;                    // E_RAW
  // E_RAW: when set, block 0 clears the tagged vector entries (two
  // buffers, tag_stride apart, at each matrix's vector offset) that the
  // one-launch power iteration after it exchanges
  uint64_t* tag; int64_t tag_stride;
  const void* sq_hi; const void* sq_lo;   // E_SQUARE: A for the b*A term
  const float* scal;               // per-matrix c = 1/(s+eps) or NULL
  const float* xs_user;            // XS_USER: float32 source in caller layout
  float* U;                        // O_U
  uint32_t* bits;                  // O_BITS (buffer of the local worker)
  int8_t* tern;                    // O_TERN: int8 signs, caller layout (local worker)
  void* W; int32_t w_bf16; float eta;   // O_APPLY
  const int32_t* status;           // O_APPLY is skipped when *status != 0
  float* kpart;                    // split-k partial tiles (groups with ksplit > 1)
  // Set by launch_gemm: blocks per XCD chunk (0: one contiguous range per
  // XCD).  Gram launches whose matrices all have C blocks give whole
  // matrices to the XCDs in turn, so that runs of long and short k mix.
  int32_t xcd_chunk;
};

// t0 / t1 (optional): events that take the start and stop time of the GEMM
// kernel itself (not of a split-k reduction that follows it)
hipError_t launch_gemm(int precision, const GemmArgs& args, hipStream_t s,
                       hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t gemm_set_attributes();
// Block tile (tm rows x tn columns) of a GEMM with output gm x gn and
// depth gk; every group of one launch must carry the same tn in
// Group::tile.
void gemm_tile(int precision, int epi, int64_t gm, int64_t gn, int64_t gk, int* tm, int* tn);
// k splits of a symmetric (Gram) GEMM of rp x rp output and depth gk over
// `count` matrices of one shape: 1 unless its upper-triangular tiles are too
// few to occupy the GPU and k is long.  *slabs receives the k slabs per
// split: even (the pipelined k-loop takes slabs in pairs), and the last
// split is shorter but not empty.
int gemm_sym_ksplit(int precision, int64_t rp, int64_t gk, int64_t count, int* slabs);
// Floats of split-k partial tiles per matrix for that split.
int64_t gemm_sym_kpart_floats(int64_t rp, int ksplit);

// ---- elementwise and small kernels (sm_elementwise.hip) ----
hipError_t launch_momentum_flat(const float* G, const void* W, int w_bf16,
                                float* Mom, int64_t n, float beta, float lam,
                                hipStream_t s);
hipError_t launch_sign_pack_flat(const float* U, uint32_t* bits, int64_t n,
                                 hipStream_t s);
// Ternary int8 sign buffers (sign with 0 kept) and their vote.
hipError_t launch_sign_ternary(const float* U, int8_t* S, int64_t n, hipStream_t s);
hipError_t launch_vote_ternary(const int8_t* S, int64_t stride, int M, int64_t n, int tie,
                               int8_t* D, int16_t* sums, hipStream_t s);
hipError_t launch_vote_flat(const uint32_t* bits, int64_t stride, int M,
                            int64_t n, int tie, int8_t* D, int16_t* sums,
                            hipStream_t s);
hipError_t launch_apply_flat(void* W, int w_bf16, const int8_t* D,
                             const float* Df, float eta, int64_t n,
                             hipStream_t s);

// Padded sweep over 64x64 tiles: writes the padded operand copy of each
// matrix (and the partial sums of squares per tile).
// ema = 1: Mom <- beta Mom + (1-beta)(G + lam W) first (G, W, Mom in caller
// layout), else the source is `src` (caller layout, float32).
struct SweepArgs {
  Groups G;
  int32_t ema, precision, w_bf16;
  float beta, lam;
  const float* src; const float* Gr; const void* W; float* Mom;
  void* o_hi; void* o_lo;
  float* part;          // partial sums per chunk, NULL to skip
  int32_t* status;      // non-finite flag, NULL to skip
};
// t0 / t1 (optional, here and for the vote): events that take the kernel's
// own start and stop times
hipError_t launch_sweep(const SweepArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);

// Momentum with the signs of the new momentum packed into `bits` (post-vote
// variant and K = 0).
struct MomSignArgs {
  Groups G;
  int32_t w_bf16;
  float beta, lam;
  const float* Gr; const void* W; float* Mom; uint32_t* bits;
  int8_t* tern;         // non-NULL: int8 signs (sign(0) = 0) instead of bits
  int32_t* status;
};
hipError_t launch_momentum_sign(const MomSignArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                                hipEvent_t t1 = nullptr);

// Vote over M buffers per matrix: mode VA_APPLY updates W, VA_SBAR writes
// the majority matrix into the padded operand (+ partial sums of squares).
enum { VA_APPLY = 0, VA_SBAR = 1 };
struct VoteArgs {
  Groups G;
  int32_t mode, M, tie, w_bf16, precision;
  const uint32_t* bits; int64_t stride;
  // non-NULL: int8 sign buffers (worker m at tern + m * stride bytes, a
  // matrix at its element offset) instead of the packed bits
  const int8_t* tern;
  void* W; float eta;
  // VA_APPLY: NULL, or per-matrix c (indexed as the matrices' scale
  // factors): W moves by eta c D (the normalized step, and the post-vote
  // step with K = 0)
  const float* scal;
  void* o_hi; void* o_lo; float* part;
  const int32_t* status;
};
hipError_t launch_vote_groups(const VoteArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                              hipEvent_t t1 = nullptr);
// Group::blocks_per_mat of a vote launch in mode `mode` over packed bits,
// and over int8 sign buffers (kTernChunk entries per block, or one 64 x 64
// tile of a tall matrix with whole 16-entry pieces per row in VA_SBAR);
// also the count of partial sums of squares a VA_SBAR vote leaves.
int vote_blocks_per_mat(int mode, int64_t rows, int64_t cols);
int tern_vote_blocks_per_mat(int mode, int64_t rows, int64_t cols);
constexpr int kTernChunk = 4096;

// Zero the padding of the padded operand copies.
hipError_t launch_zero_pad(const Groups& G, int precision, void* hi, void* lo,
                           hipStream_t s);

// c = 1 / (sqrt(sum of partials) + eps) per matrix (Frobenius).
hipError_t launch_fro_finalize(const Groups& G, const float* part, float eps,
                               float* scal, hipStream_t s);

// Power iteration on the padded raw Gram.
// first: src is ignored and the start vector (u0, or ones) is read instead.
hipError_t launch_power_step(const Groups& G, const float* araw,
                             const float* src, float* dst, const float* u0,
                             bool first, hipStream_t s);
// The P power steps and the scale of every matrix of a small set in one
// launch.  A block holds kPowerRows rows of the raw Gram in LDS for all P
// steps (blocks_per_mat = Rp / kPowerRows) and does the arithmetic of
// k_power_step; the blocks of a matrix exchange each step's vector as
// tagged entries (zero on entry: the raw Gram launch clears them) and wait
// for the whole vector before the next step.  The launch holds at most
// kPowerIterMaxBlocks blocks of at most (kPowerRows + 1) kPowerIterMaxRp
// floats of LDS each, which the GPU keeps resident together, and every
// wait is bounded: a block whose vector does not arrive sets bit 2 of both
// status words.
constexpr int kPowerRows = 16;
constexpr int kPowerIterMaxBlocks = 256;
constexpr int kPowerIterMaxRp = 768;
struct PowerIterArgs {
  Groups G;
  const float* araw;
  float* va; float* vb;      // step p reads (p odd ? vb : va), writes the other
  const float* u0;           // start vectors, or NULL for ones
  int32_t P;                 // power steps, >= 1
  int32_t scaled_op;         // 1: also write the scaled operand mul c^2 A to hi / lo
  int32_t precision;
  float mul, eps;
  float* scal;               // per-matrix c = 1 / (sqrt(|w|) + eps)
  void* hi; void* lo;
  uint64_t* tag;             // tagged vectors: 2 buffers of v_total entries,
  int64_t tag_stride;        //   tag_stride apart
  int32_t* status;           // the two status words
};
hipError_t launch_power_iter(const PowerIterArgs& a, int64_t rp_max, hipStream_t s);
hipError_t launch_power_finalize(const Groups& G, const float* w, float eps,
                                 float* scal, hipStream_t s);
// op = mul * c^2 * araw (padded Rp x Rp) in the operand precision; c is
// scal's entry, or (w non-null) the power-iteration scale of w, then stored.
hipError_t launch_prescale(const Groups& G, int precision, const float* araw,
                           float* scal, float mul, void* hi, void* lo,
                           const float* w, float eps, hipStream_t s);
// K = 0 output: v = c * x (x from caller-layout float32 or padded operand);
// writes U (caller layout) or applies W -= eta * v.
// PolarNS with K = 0: U = c X in the caller's layout (X float32).
struct ScaledOutArgs {
  Groups G;
  const float* x_user;
  const float* scal;
  float* U;
};
hipError_t launch_scaled_out(const ScaledOutArgs& a, hipStream_t s);

// Start of a step: status[0] = status[1] (flags of the worker pipelines
// enqueued since the last step), status[1] = 0.
hipError_t launch_begin_status(int32_t* status, hipStream_t s);
// Both status words to 0.
hipError_t launch_reset_status(int32_t* status, hipStream_t s);
// Q = a I + b A on each matrix's padded Rp x Rp bfloat16 buffer
// (blocks_per_mat = Rp * Rp / kChunk).
hipError_t launch_affine_ident(const Groups& G, const void* A, float a, float b, void* Q,
                               hipStream_t s);

}  // namespace sm
