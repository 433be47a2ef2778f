// Batched matrix-core GEMM for the Newton-Schulz products of PolarNS
// (SignMuon paper, section 4, Newton-Schulz paragraph).  Each iterate is
// kept as S, its short side as rows (S = X, or X^T for a tall X), so the
// products are the Gram matrix A = S S^T, the quintic square A*A, and the
// update a S + B S, with the epilogues that finish each step.
//
// One launch covers every matrix of a parameter set (up to kMaxGroups runs
// of same-shaped matrices).  Each block owns a 128x128 output tile and runs
// 4 waves (2x2), each wave a 64x64 sub-tile built from 16x16 MFMA tiles:
//   bf16 / split-bf16: v_mfma_f32_16x16x32_bf16
//   f32:               v_mfma_f32_16x16x4_f32
// Each k-slab of an operand tile is fetched with global_load_lds_dwordx4
// straight into LDS: lane l of a wave writes the 16 bytes at the wave's LDS
// base + 16 l, and the XOR swizzles of the LDS layouts (against bank
// conflicts of the fragment reads) are applied by permuting which global
// bytes each lane fetches.  Operands with k along their rows (S for the
// Gram, B for the update) land as 128-byte slab rows and are read with
// 16-byte loads; the update's S operand has k down its columns, lands as
// k-rows and is read with the transposing LDS load (ds_read_b64_tr_b16),
// so no transposed copy of S is ever stored.  bfloat16 symmetric operands
// (Gram operand, Gram-space iterates) are stored as their upper-triangular
// tiles: a product reads the slabs of a row block left of the diagonal
// k-major from the tiles above it, with the same transposing loads.  NSTG
// LDS stages form the prefetch pipeline; completion is tracked with
// explicit vmcnt waits and a bare s_barrier.  All operand copies are zero
// padded to multiples of 128, so no load is predicated and padding
// contributes exact zeros.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include <hip/hip_ext.h>

#include "sm_internal.h"
#include "sm_launch.h"

namespace sm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
// the kernel's helper lambdas take register arrays by reference: they must
// be inlined, or the arrays would live in scratch memory
#define SM_INLINE __attribute__((always_inline))

constexpr int BM = 128;          // block tile width (and height for WM = 2)

// LDS image of one k-slab of an operand tile: RB bytes per row (64 or 128),
// 16-byte chunks XOR-swizzled by row.  A fragment read is a ds_read_b128
// with 16 lanes on 16 consecutive rows and lane groups 16 apart on
// neighbouring chunks.  The LDS serves such a read per half-wave: it is
// free of bank conflicts when the 32 lanes of each half hit 32 distinct
// 16-byte units modulo 512 bytes (measured on gfx950 with the
// SQ_LDS_BANK_CONFLICT counter over several lane patterns; a swizzle that
// only separates groups of 8 or 16 lanes left a 2-way conflict).  Rows 4
// apart (128-byte rows) or 8 apart (64-byte rows) share a unit modulo 512
// bytes, so the swizzle separates exactly those.  It depends on row bits
// 0..3 only, so rows 16 apart share it and a fragment offset steps by a
// constant 16*RB bytes per 16-row tile.
template <int RB>
__host__ __device__ constexpr int swz(int row) {
  if constexpr (RB == 128) return (row >> 1) & 7;
  else return (((row >> 3) & 1) << 1) | ((row >> 2) & 1);
}
template <int RB>
__host__ __device__ constexpr int lds_off(int row, int chunk) {
  return row * RB + ((chunk ^ swz<RB>(row)) << 4);
}
// Compile-time checks of the layout: constant 16-row stride, a bijection of
// each row's chunks, and distinct 16-byte units modulo 512 bytes in each
// half-wave of a fragment read (lane l: row l % 16, chunk 4 kk + l / 16).
template <int RB>
constexpr bool slab_layout_ok() {
  constexpr int CPR = RB / 16;
  for (int r0 = 0; r0 < 256; r0 += 16) {
    for (int ch = 0; ch < CPR; ++ch)
      for (int r = 0; r < 16; ++r)
        if (lds_off<RB>(r0 + r, ch) != lds_off<RB>(r, ch) + r0 * RB) return false;
    for (int r = 0; r < 16; ++r) {
      unsigned seen = 0;
      for (int ch = 0; ch < CPR; ++ch) seen |= 1u << ((lds_off<RB>(r, ch) - r * RB) / 16);
      if (seen != (1u << CPR) - 1) return false;
    }
    for (int kk = 0; kk < CPR / 4; ++kk)
      for (int half = 0; half < 2; ++half) {
        unsigned seen = 0;
        for (int l = 32 * half; l < 32 * half + 32; ++l) {
          const int unit = (lds_off<RB>(r0 + (l & 15), 4 * kk + (l >> 4)) % 512) / 16;
          if (seen & (1u << unit)) return false;
          seen |= 1u << unit;
        }
      }
  }
  return true;
}
static_assert(slab_layout_ok<64>() && slab_layout_ok<128>(), "LDS slab swizzle");

// k-major operand tiles (an X block with k down its columns): LDS row = k
// within the slab, W * sizeof(T) bytes per row (the W output rows or columns
// of the tile), 32-byte chunks XOR-swizzled by row bits 0, 1 and 3.
// The 16 lanes of a transposing fragment read cover 4 consecutive rows of
// one chunk, and lane groups 16 apart read rows 8 apart; both then land in
// distinct bank groups.  The swizzle ignores row bit 2, so the second read
// of a fragment (4 rows down) is a constant offset away.
__host__ __device__ constexpr int km_swz(int row) { return (row & 3) ^ (((row >> 3) & 1) << 2); }
template <typename T, int W = 128>
__host__ __device__ constexpr int km_off(int row, int byte) {
  return row * (W * (int)sizeof(T)) + ((((byte >> 5) ^ km_swz(row)) << 5) | (byte & 31));
}
// Checks: a bijection of each row's chunks, and for the transposing read
// (lane j of a 16-lane group at row r0 + j/4, byte c*32 + 8*(j%4)) 16
// distinct 8-byte slots in 128 bytes, with lane groups 8 rows apart in the
// other half of 256 bytes.
constexpr bool km_layout_ok() {
  for (int r0 = 0; r0 < 64; r0 += 4)
    for (int c = 0; c < 8; ++c) {
      unsigned seen = 0, seen2 = 0;
      for (int j = 0; j < 16; ++j) {
        const int o = km_off<bf16_t>(r0 + j / 4, c * 32 + 8 * (j % 4));
        const int slot = (o % 128) / 8;
        if (seen & (1u << slot)) return false;
        seen |= 1u << slot;
        if (km_off<bf16_t>(r0 + 4 + j / 4, c * 32 + 8 * (j % 4)) != o + 4 * 256) {
          if ((r0 & 4) == 0) return false;
        }
        const int o8 = km_off<bf16_t>((r0 ^ 8) + j / 4, c * 32 + 8 * (j % 4));
        if ((o8 % 256) / 128 == (o % 256) / 128) return false;
        seen2 |= 1u << ((o8 % 128) / 8);
      }
      if (seen2 != 0xFFFFu) return false;
    }
  return true;
}
static_assert(km_layout_ok(), "k-major LDS swizzle");

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8 bytes addressed by lane
// 4 e + i / 4, for e = 0..3 (16-bit elements).
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) char*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

// A uniform pointer made opaque to the optimizer (an empty asm statement
// that keeps it in scalar registers), so that it cannot be folded with
// per-lane offsets into 64-bit vector addresses carried across the loop: a
// load then keeps the scalar-base + 32-bit vector-offset form.
__device__ __forceinline__ const char* scalar_ptr(const char* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<const char*>(v);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads (and scalar loads) have
// returned; the vector-memory and export counters are left alone.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int per16 = 8; };
template <> struct Elem<float>  { static constexpr int per16 = 4; };

// Per-matrix offset and row length of an operand family.
__device__ __forceinline__ int64_t fam_off(const Group& g, int fam, int mi) {
  return fam >= FAM_R ? g.r0 + (int64_t)mi * g.r_stride
                      : g.x0 + (int64_t)mi * g.x_stride;
}
__device__ __forceinline__ int64_t fam_ld(const Group& g, int fam) {
  return round_up(fam >= FAM_R ? s_rows(g) : s_cols(g), kPad);
}

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------
template <typename T, int SPLIT>
__device__ __forceinline__ float load_op(const void* hi, const void* lo,
                                         int64_t i) {
  if constexpr (sizeof(T) == 4) {
    return reinterpret_cast<const float*>(hi)[i];
  } else {
    float v = bf16_to_f32(reinterpret_cast<const bf16_t*>(hi)[i]);
    if constexpr (SPLIT == 2) v += bf16_to_f32(reinterpret_cast<const bf16_t*>(lo)[i]);
    return v;
  }
}
template <typename T, int SPLIT>
__device__ __forceinline__ void store_op(void* hi, void* lo, int64_t i, float v) {
  if constexpr (sizeof(T) == 4) {
    reinterpret_cast<float*>(hi)[i] = v;
  } else if constexpr (SPLIT == 2) {
    bf16_t h, l;
    split_bf16(v, h, l);
    reinterpret_cast<bf16_t*>(hi)[i] = h;
    reinterpret_cast<bf16_t*>(lo)[i] = l;
  } else {
    reinterpret_cast<bf16_t*>(hi)[i] = f32_to_bf16(v);
  }
}
// Four consecutive values (one column of a 16x16 accumulator tile, i.e. one
// row segment of the transposed copy) stored with one 8- or 16-byte store.
template <typename T, int SPLIT>
__device__ __forceinline__ void store_op4(void* hi, void* lo, int64_t i,
                                          const float (&v)[4]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(hi) + i) =
        f32x4_t{v[0], v[1], v[2], v[3]};
  } else {
    bf16_t h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (SPLIT == 2) split_bf16(v[k], h[k], l[k]);
      else h[k] = f32_to_bf16(v[k]);
    }
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(hi) + i) =
        u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    if constexpr (SPLIT == 2)
      *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(lo) + i) =
          u32x2_t{(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
  }
}

__device__ __forceinline__ void apply_one(void* W, int w_bf16, int64_t i,
                                          float eta, float u) {
#pragma clang fp contract(off)
  if (w_bf16) {
    bf16_t* w = reinterpret_cast<bf16_t*>(W);
    float t = eta * u;
    float r = bf16_to_f32(w[i]) - t;
    w[i] = f32_to_bf16(r);
  } else {
    float* w = reinterpret_cast<float*>(W);
    float t = eta * u;
    w[i] = w[i] - t;
  }
}


template <typename T>
__device__ __forceinline__ void* offset_ptr(void* p, int64_t off) {
  return p ? static_cast<void*>(reinterpret_cast<T*>(p) + off) : nullptr;
}

// Four consecutive operand values (8 or 16 bytes, aligned) as floats.
template <typename T, int SPLIT>
__device__ __forceinline__ void load_op4(const void* hi, const void* lo, int64_t i,
                                         float (&v)[4]) {
  if constexpr (sizeof(T) == 4) {
    f32x4_t x = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(hi) + i);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else {
    u32x2_t h = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(hi) + i);
    v[0] = __uint_as_float(h[0] << 16); v[1] = __uint_as_float(h[0] & 0xFFFF0000u);
    v[2] = __uint_as_float(h[1] << 16); v[3] = __uint_as_float(h[1] & 0xFFFF0000u);
    if constexpr (SPLIT == 2) {
      u32x2_t l = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(lo) + i);
      v[0] += __uint_as_float(l[0] << 16); v[1] += __uint_as_float(l[0] & 0xFFFF0000u);
      v[2] += __uint_as_float(l[1] << 16); v[3] += __uint_as_float(l[1] & 0xFFFF0000u);
    }
  }
}

// Store a BMT x BNT output tile (values in accumulator layout) row-major at
// dst (row length ld) through LDS: each wave writes its (16 TI) x (16 TJ)
// sub-tile into an LDS image of the tile, then every thread stores 16-byte
// row segments (rows at or past row_lim are skipped).  For split-bf16 the
// hi and lo images sit side by side.  The LDS row pitch is padded by 16
// bytes against bank conflicts.
// With TR the accumulators hold transposed tiles (4 consecutive columns of
// one row per register group) and each lane writes them as one 8- or
// 16-byte piece.
template <typename T, int SPLIT, int BMT, int BNT, int TI, int TJ, int NT, bool TR = false>
__device__ __forceinline__ void stage_store_tile(const f32x4_t (&v)[TI][TJ], char* smem,
                                                 void* dst_hi, void* dst_lo, int64_t ld,
                                                 int m0, int n0, int row_lim, int wm, int wn,
                                                 int lane, int tid) {
  constexpr int ES = sizeof(T);
  constexpr int PITCH = BNT * ES + 16;
  constexpr int IMG = BMT * PITCH;
  if constexpr (TR) {
    const int r0 = wm * TI * 16 + (lane & 15), c0 = wn * TJ * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        char* p = smem + (r0 + i * 16) * PITCH + (c0 + j * 16) * ES;
        if constexpr (ES == 4) {
          *reinterpret_cast<f32x4_t*>(p) = v[i][j];
        } else {
          bf16_t h[4], l[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (SPLIT == 2) split_bf16(v[i][j][r], h[r], l[r]);
            else h[r] = f32_to_bf16(v[i][j][r]);
          }
          *reinterpret_cast<u32x2_t*>(p) = u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                   (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
          if constexpr (SPLIT == 2)
            *reinterpret_cast<u32x2_t*>(p + IMG) = u32x2_t{(uint32_t)l[0] | ((uint32_t)l[1] << 16),
                                                           (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
        }
      }
  } else {
    const int r0 = wm * TI * 16 + 4 * (lane >> 4), c0 = wn * TJ * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          char* p = smem + (r0 + i * 16 + r) * PITCH + (c0 + j * 16) * ES;
          if constexpr (ES == 4) {
            *reinterpret_cast<float*>(p) = v[i][j][r];
          } else if constexpr (SPLIT == 2) {
            bf16_t h, l;
            split_bf16(v[i][j][r], h, l);
            *reinterpret_cast<bf16_t*>(p) = h;
            *reinterpret_cast<bf16_t*>(p + IMG) = l;
          } else {
            *reinterpret_cast<bf16_t*>(p) = f32_to_bf16(v[i][j][r]);
          }
        }
  }
  __syncthreads();
  constexpr int CH = BNT * ES / 16;         // 16-byte chunks per row
#pragma unroll
  for (int p = 0; p < BMT * CH / NT; ++p) {
    const int c = tid + NT * p;
    const int row = c / CH, ch = c % CH;
    if (m0 + row >= row_lim) continue;
    const char* src = smem + row * PITCH + ch * 16;
    const int64_t o = (int64_t)(m0 + row) * ld * ES + (int64_t)n0 * ES + ch * 16;
    *reinterpret_cast<u32x4_t*>(static_cast<char*>(dst_hi) + o) = *reinterpret_cast<const u32x4_t*>(src);
    if constexpr (SPLIT == 2)
      *reinterpret_cast<u32x4_t*>(static_cast<char*>(dst_lo) + o) =
          *reinterpret_cast<const u32x4_t*>(src + IMG);
  }
}

// Mirror tile of a symmetric output, through LDS: the transpose of the
// tile (rows n0.., columns m0..) is staged with the transposed-tile writes
// (the 4 rows of a register group become 4 consecutive columns; TRSRC:
// the accumulators hold transposed tiles, whose 4 columns become 4 rows) and stored
// as 16-byte row pieces.  Waits first for every thread to have read out the
// previous image.
template <typename T, int SPLIT, int BMT, int BNT, int TI, int TJ, int NT, bool TRSRC = false>
__device__ __forceinline__ void stage_store_mirror(const f32x4_t (&v)[TI][TJ], char* smem,
                                                   void* dst_hi, void* dst_lo, int64_t ld,
                                                   int m0, int n0, int row_lim, int wm, int wn,
                                                   int lane, int tid) {
  f32x4_t vt[TJ][TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) vt[j][i] = v[i][j];
  __syncthreads();
  stage_store_tile<T, SPLIT, BNT, BMT, TJ, TI, NT, !TRSRC>(vt, smem, dst_hi, dst_lo, ld, n0, m0,
                                                           row_lim, wn, wm, lane, tid);
}

// Tile of the symmetric outputs (Gram, raw Gram, quintic square).
constexpr int kTileSym = 128;

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// Template parameters: operand type and split (bf16 x2 = split-bf16), the
// epilogue, NSTG pipeline stages of RB-byte slab rows, WM x 2 waves of
// (16 TI) x (16 TJ) each, the waves per SIMD that the register allocation
// must leave room for, the software-pipelined k-loop and the transposed
// accumulator layout.
template <typename T, int SPLIT, int EPI, int NSTG, int WM, int TI, int TJ, int RB, int WPE,
          bool PIPE, bool TRACC>
__global__ __launch_bounds__(128 * WM, WPE) void k_gemm(GemmArgs A) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int WTM = 16 * TI, WTN = 16 * TJ;  // wave tile
  constexpr int BMT = WM * WTM, BNT = 2 * WTN; // block tile
  constexpr int NW = 2 * WM, NT = 64 * NW;
  constexpr int CPR = RB / 16;                 // 16-byte chunks per slab row
  constexpr int RPI = 1024 / RB;               // slab rows per wave-wide DMA load
  constexpr int NKK = CPR / 4;                 // MFMA k-steps per slab
  constexpr int QA = BMT * RB / 1024 / NW;     // A-operand loads per wave
  constexpr int QB = BNT * RB / 1024 / NW;     // B-operand loads per wave
  constexpr int ATILE = BMT * RB;              // A-operand bytes per split
  constexpr int BTILE = BNT * RB;
  constexpr int STAGEB = SPLIT * (ATILE + BTILE);
  constexpr int P = Elem<T>::per16;            // elements per 16 bytes
  constexpr int BK = RB / sizeof(T);           // k per slab
  static_assert(QA >= 1 && QB >= 1 && NKK >= 1, "tile / slab shape");
  static_assert(EPI == E_UPDATE || BMT == BNT, "symmetric outputs use square tiles");

  const int tid = threadIdx.x;
  if constexpr (EPI == E_RAW) {
    // clear the tagged vectors of the one-launch power iteration that reads
    // this Gram (gm = Rp entries per matrix, in both buffers)
    if (A.tag && blockIdx.x == 0) {
      for (int i = 0; i < A.G.n; ++i) {
        const Group& gz = A.G.g[i];
        for (int m = 0; m < gz.count; ++m) {
          uint64_t* t0 = A.tag + gz.v0 + (int64_t)m * gz.v_stride;
          for (int e = tid; e < gz.gm; e += NT) {
            t0[e] = 0;
            t0[A.tag_stride + e] = 0;
          }
        }
      }
    }
  }
  // the wave index is uniform: keep it (and everything derived from it) scalar
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- block -> (group, matrix, tile), XCD-aware: the 8 XCDs take blocks
  // round-robin, so consecutive logical tiles are given to one XCD: in
  // chunks of C = xcd_chunk logical blocks (whole matrices) dealt to the
  // XCDs in turn for as many full rounds of 8 C as fit, and the rest (or
  // everything, for C = 0) as one contiguous range per XCD.
  int b = blockIdx.x;
  {
    const int C = A.xcd_chunk;
    int x = b & 7, k = b >> 3, base = 0, nb = A.G.total_blocks;
    const int rounds = C > 0 ? nb / (8 * C) : 0;
    if (k < rounds * C) {
      b = (k / C) * 8 * C + x * C + k % C;
    } else {
      base = rounds * 8 * C;
      nb -= base;
      k -= rounds * C;
      const int per = nb >> 3, rem = nb & 7;
      b = base + (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
    }
  }
  const int gi = find_group(A.G, b);
  const Group& g = A.G.g[gi];
  const int lb = b - g.block0;
  const int mi = lb / g.blocks_per_mat;
  const int t = lb - mi * g.blocks_per_mat;
  // Symmetric outputs (Gram, raw Gram, symmetric products) are computed on
  // the upper-triangular tiles only; the epilogue also writes the mirror
  // tile unless the operand is stored upper-triangular.
  constexpr bool SYM = EPI != E_UPDATE;
  const int a_fam = g.ops & 3, b_fam = (g.ops >> 2) & 3;
  int tm, tn;
  // split-k (symmetric outputs with few tiles and long k): block t takes
  // triangular tile t % ntri over the slabs of split t / ntri
  int ks = 0, ttri = t;
  if constexpr (SYM) {
    const int ntri = g.tiles_n * (g.tiles_n + 1) / 2;
    ks = t / ntri;
    ttri = t - ks * ntri;
    tm = 0;
    int rem = ttri;
    while (rem >= g.tiles_n - tm) { rem -= g.tiles_n - tm; ++tm; }
    tn = tm + rem;
  } else if (a_fam == FAM_R) {
    // the small operand (B = b S S^T) is the A side: consecutive tiles walk
    // down m, so the tiles that share one column block of S run together on
    // one XCD and fetch it from HBM once
    const int tiles_m = (g.gm + BMT - 1) / BMT;
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
  } else {
    tm = t / g.tiles_n;
    tn = t - tm * g.tiles_n;
  }
  const int m0 = tm * BMT, n0 = tn * BNT;
  const int64_t lda = fam_ld(g, a_fam), ldb = fam_ld(g, b_fam);
  // Operand layouts are fixed by the product: only the update's S operand
  // (B) is read k-major.  (The host sets the operand families to match.)
  constexpr bool a_km = false, b_km = EPI == E_UPDATE;
  // Upper-triangular storage of the bfloat16 symmetric operands (A.upper):
  // row block t of a stored Rp x Rp operand has its k-slabs left of the
  // diagonal (k < 128 t) only in the tile above the diagonal, so those
  // slabs are fetched k-major from there.  The diagonal tile is itself
  // symmetric and may be read either way, so the k-major range includes
  // it: the A operand of the symmetric product and of the update (row block
  // tm) is k-major below slab sA = TPS (tm + 1), the B operand of the
  // symmetric product (row block tn) below sB = TPS (tn + 1), with TPS
  // slabs per 128-wide tile.  Every block then starts with both operands
  // k-major, meets the layouts in the same order, and reads k in natural
  // order (blocks sharing an operand block stay in step through L2).  With
  // mirrored storage (A.upper = 0) the same reads are valid, since every
  // tile is present and the operands are symmetric: A.upper only decides
  // whether symmetric outputs also write their mirror tiles.
  constexpr bool UPK = sizeof(T) == 2 && SPLIT == 1;
  constexpr bool UPR = UPK && (EPI == E_SQUARE || EPI == E_UPDATE) && BNT == kTileSym;
  const bool upper = UPK && A.upper != 0;
  constexpr int TPS = kTileSym / (RB / (int)sizeof(T));   // slabs per 128-wide tile
  const int sA = UPR ? (tm + 1) * TPS : 0;
  const int sB = UPR && EPI == E_SQUARE ? (tn + 1) * TPS : 0;
  // Accumulator layout.  Register r of lane l in tile (i, j) holds C(row, col):
  //   C tiles:       row = m0 + wm*WTM + 16 i + 4 (l/16) + r,  col = n0 + wn*WTN + 16 j + l % 16
  //   transposed:    row = m0 + wm*WTM + 16 i + l % 16,  col = n0 + wn*WTN + 16 j + 4 (l/16) + r
  // (4 consecutive rows of one column, or 4 consecutive columns of one row).
  // An update with TRACC runs its MFMAs with the operands swapped, which
  // gives the transposed tiles.
  constexpr bool SWAP = TRACC;
  static_assert(!TRACC || EPI == E_UPDATE || EPI == E_SQUARE,
                "transposed tiles: update and symmetric product");
  auto acc_row = [&](int i, int r) SM_INLINE {
    return m0 + wm * WTM + (SWAP ? (lane & 15) : 4 * (lane >> 4) + r) + 16 * i;
  };
  auto acc_col = [&](int j, int r) SM_INLINE {
    return n0 + wn * WTN + (SWAP ? 4 * (lane >> 4) + r : (lane & 15)) + 16 * j;
  };
  const void* a_hi = a_fam == FAM_R ? A.r_hi : A.x_hi;
  const void* b_hi = b_fam == FAM_R ? A.r_hi : b_fam == FAM_R2 ? A.r2_hi : A.x_hi;
  const void* a_lo = a_fam == FAM_R ? A.r_lo : A.x_lo;
  const void* b_lo = b_fam == FAM_R ? A.r_lo : b_fam == FAM_R2 ? A.r2_lo : A.x_lo;
  const T* a_src[SPLIT];
  const T* b_src[SPLIT];
  a_src[0] = reinterpret_cast<const T*>(a_hi) + fam_off(g, a_fam, mi);
  b_src[0] = reinterpret_cast<const T*>(b_hi) + fam_off(g, b_fam, mi);
  if constexpr (SPLIT == 2) {
    a_src[SPLIT - 1] = reinterpret_cast<const T*>(a_lo) + fam_off(g, a_fam, mi);
    b_src[SPLIT - 1] = reinterpret_cast<const T*>(b_lo) + fam_off(g, b_fam, mi);
  }

  // Per-lane source offsets of the loads per operand and slab; load q of
  // wave w fills the 1 KB piece c = QA w + q (B: QB w + q) of the tile and
  // lane l writes its bytes 16 l .. 16 l + 15.
  //  k along rows: LDS rows c*RPI .. +RPI-1; lane l writes row ..+l/CPR at
  //   chunk position l%CPR, so it fetches global chunk (l%CPR) ^ swz(row).
  //   Rows past the operand (a ragged last tile) read its last row instead;
  //   their results are never stored.
  //  k-major (tile width W): LDS rows (k) c*RPK .. +RPK-1 of W * sizeof(T)
  //   bytes, RPK = 1024 / (W * sizeof(T)); lane l writes 16 bytes of row
  //   ..+l/LPR (LPR lanes per row), fetched from the swizzled position.
  auto dma_off = [&](bool km, int c, int mn0, int lim, int64_t ld, int W) -> int64_t {
    if (km) {
      const int rowb = W * (int)sizeof(T), LPR = rowb / 16;
      const int row = c * (1024 / rowb) + lane / LPR;
      const int pb = (lane % LPR) * 16;                 // physical byte in the row
      const int lb = (((pb >> 5) ^ km_swz(row)) << 5) | (pb & 31);
      return (int64_t)row * ld + mn0 + lb / (int)sizeof(T);
    }
    const int row = c * RPI + lane / CPR;
    const int ch = (lane % CPR) ^ swz<RB>(row);
    const int r = mn0 + row < lim ? mn0 + row : lim - 1;
    return (int64_t)r * ld + ch * P;
  };
  // (element offsets within one matrix fit 32 bits: padded rows * cols of a
  // matrix is at most 2^31; the slab's uniform base pointer carries the rest)
  uint32_t aoff[QA], boff[QB];   // byte offsets
#pragma unroll
  for (int q = 0; q < QA; ++q) aoff[q] = (uint32_t)(dma_off(a_km, wave * QA + q, m0, g.gm, lda, BMT) * (int64_t)sizeof(T));
#pragma unroll
  for (int q = 0; q < QB; ++q) boff[q] = (uint32_t)(dma_off(b_km, wave * QB + q, n0, g.gn, ldb, BNT) * (int64_t)sizeof(T));
  // k-major offsets of the slabs taken from the tile above the diagonal,
  // one register per operand: load q of a wave fills LDS rows 4 (QA w + q)
  // .. +3 (256-byte rows), so loads q and q + 1 (q even) are 4 rows apart
  // with the same swizzle, and loads 2 apart are 8 rows apart with the
  // swizzle's row bit 3 flipped, i.e. bit 7 of the byte offset (rows start
  // at multiples of 256 bytes).  Holds for 128-wide tiles of 2-byte
  // elements with 2 or 4 loads per wave.
  constexpr bool UPB = UPR && EPI == E_SQUARE;
  // the update's S operand (always k-major) uses the same scheme when its
  // tile is 128 wide.  (The 128 x 256 update reads its A operand whole:
  // the host keeps mirrored storage for sets that use it.)
  constexpr bool BKC = sizeof(T) == 2 && b_km && BNT == 128;
  static_assert(!UPR || (BMT == 128 && (QA == 2 || QA == 4)), "k-major offset scheme");
  static_assert(!(UPB || BKC) || (BNT == 128 && (QB == 2 || QB == 4)), "k-major offset scheme");
  const uint32_t aoff_t = UPR ? (uint32_t)(dma_off(true, wave * QA, m0, g.gm, lda, BMT) * 2) : 0u;
  const uint32_t boff_t = UPB || BKC ? (uint32_t)(dma_off(true, wave * QB, n0, g.gn, ldb, BNT) * 2)
                                     : 0u;
  // elements between consecutive slabs
  const int64_t a_kst = a_km ? (int64_t)BK * lda : BK, b_kst = b_km ? (int64_t)BK * ldb : BK;

  // Per-lane LDS offsets of the fragment reads (k along rows): row within
  // the tile and 16-byte chunk (kk*4 + lane/16) of the slab row.  The
  // swizzle depends on row bits that i*16 does not touch, so one offset per
  // kk serves all i (j) with a constant stride.
  // (k-step kk is chunk 4 kk + lane/16: for kk < 2 that XORs bit 6 of the
  // k-step 0 offset, since the swizzle is below 8)
  static_assert(NKK <= 2, "fragment offsets");
  const int fa_off0 = lds_off<RB>(wm * WTM + (lane & 15), lane >> 4);
  const int fb_off0 = lds_off<RB>(wn * WTN + (lane & 15), lane >> 4);
  // A fragment of a k-major tile: MFMA tile columns c0 .. c0+15, k-step kk.
  //  bf16: two transposing reads, rows kk*32 + 8 (lane/16) + (lane%16)/4 and
  //   4 rows down, bytes 2 c0 + 8 (lane % 4): lane l gets k = 8 (l/16) .. +7
  //   of column c0 + l % 16, the MFMA operand layout.
  //  float32: the 16x16x4 MFMA takes k = 4 (kk*4 + l/16) + e, e = 0..3, of
  //   column c0 + l % 16 in register e (as the k-along-rows reads).
  // bf16: per-lane byte offset of the first transposing read of MFMA tile
  // i = 0, k-step 0 in a k-major tile of width W whose wave columns start
  // at cw; tile i and k-step kk are at (base ^ 32 i) + kk * 64 W (the
  // swizzle XORs the 32-byte chunk index, and 16 i columns are chunk i; 32
  // rows down leave it unchanged), the second read 4 rows (8 W bytes) down.
  auto km_base = [&](auto wc, int cw) SM_INLINE -> int {
    constexpr int W = decltype(wc)::value;
    return km_off<T, W>(8 * (lane >> 4) + ((lane & 15) >> 2), 2 * cw + 8 * (lane & 3));
  };
  int kmA = 0, kmB = 0;
  if constexpr (sizeof(T) == 2) {
    if constexpr (UPR) kmA = km_base(std::integral_constant<int, BMT>{}, wm * WTM);
    if constexpr (b_km || UPB) kmB = km_base(std::integral_constant<int, BNT>{}, wn * WTN);
  }
  auto km_frag2 = [&](auto wc, const char* tile, int base, int i, int kk) SM_INLINE -> u32x4_t {
    constexpr int W = decltype(wc)::value;
    const char* p = tile + (base ^ (i << 5)) + kk * 64 * W;
    const u32x2_t lo4 = lds_read_tr16(p);
    const u32x2_t hi4 = lds_read_tr16(p + 8 * W);
    return u32x4_t{lo4[0], lo4[1], hi4[0], hi4[1]};
  };
  auto km_frag = [&](auto wc, const char* tile, int c0, int kk) SM_INLINE -> u32x4_t {
    constexpr int W = decltype(wc)::value;
    if constexpr (sizeof(T) == 2) {
      const int row = kk * 32 + 8 * (lane >> 4) + ((lane & 15) >> 2);
      const int off = km_off<T, W>(row, 2 * c0 + 8 * (lane & 3));
      const u32x2_t lo4 = lds_read_tr16(tile + off);
      const u32x2_t hi4 = lds_read_tr16(tile + off + 4 * W * (int)sizeof(T));
      return u32x4_t{lo4[0], lo4[1], hi4[0], hi4[1]};
    } else {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * (kk * 4 + (lane >> 4)) + e;
        v[e] = *reinterpret_cast<const uint32_t*>(tile + km_off<T, W>(row, 4 * (c0 + (lane & 15))));
      }
      return v;
    }
  };

  // slabs of this block: all of k, or those of split ks (the host makes
  // every split non-empty and of an even slab count)
  int nslab = g.gk / BK;
  if (SYM && g.ksplit > 1) {
    const int per = g.kslabs;
    const int s0 = ks * per;
    nslab = nslab - s0 < per ? nslab - s0 : per;
#pragma unroll
    for (int sp = 0; sp < SPLIT; ++sp) {
      a_src[sp] += (int64_t)s0 * a_kst;
      b_src[sp] += (int64_t)s0 * b_kst;
    }
  }


  // LDS stage: [A split 0][A split 1..][B split 0][B split 1..]
  auto a_tile = [&](int st, int sp) -> char* { return smem + st * STAGEB + sp * ATILE; };
  auto b_tile = [&](int st, int sp) -> char* {
    return smem + st * STAGEB + SPLIT * ATILE + sp * BTILE;
  };
  // one slab of one operand, k along rows (offsets off[]) or k-major from
  // the tile above the diagonal (offset offt, base at row k of slab s)
  auto issue_op = [&](const T* src, const uint32_t* off, uint32_t offt, int64_t kst, int64_t ld,
                      bool km_slab, char* lds, int s, auto nq) SM_INLINE {
    constexpr int NQ = decltype(nq)::value;
    // (selects instead of branches: the fetch sits inside the MFMA sequence;
    // each load's base pointer is made opaque and scalar, so that the load
    // keeps the scalar-base + 32-bit offset form instead of per-lane 64-bit
    // addresses carried across the loop)
    const char* base = reinterpret_cast<const char*>(src + (km_slab ? (int64_t)s * BK * ld : s * kst));
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t dq = km_slab ? (int64_t)((q & 1) * 4 + (q >> 1) * 8) * ld * (int64_t)sizeof(T) : 0;
      const uint32_t o = km_slab ? ((q >> 1) ? (offt ^ 128u) : offt) : off[q];
      __builtin_amdgcn_global_load_lds((const void*)(scalar_ptr(base + dq) + o),
                                       (lds_void*)(lds + q * 1024), 16, 0, 0);
    }
  };
  auto issue = [&](int sq) SM_INLINE {
    const int st = sq % NSTG, s = sq;
#pragma unroll
    for (int sp = 0; sp < SPLIT; ++sp) {
      issue_op(a_src[sp], aoff, aoff_t, a_kst, lda, UPR && s < sA, a_tile(st, sp) + wave * QA * 1024,
               s, std::integral_constant<int, QA>{});
      if constexpr (BKC)   // (b_kst is the k-major slab stride)
        issue_op(b_src[sp], boff, boff_t, BK, ldb, true, b_tile(st, sp) + wave * QB * 1024, s,
                 std::integral_constant<int, QB>{});
      else
        issue_op(b_src[sp], boff, boff_t, b_kst, ldb, UPB && s < sB,
                 b_tile(st, sp) + wave * QB * 1024, s, std::integral_constant<int, QB>{});
    }
  };

  f32x4_t acc[TI][TJ];
  const bool ax_user = EPI == E_UPDATE && A.xsrc == XS_USER;
  if (ax_user) {
    // first step: a X from the caller's float32 source (entries past the
    // matrix are zero), loaded ahead of the k-loop.  (i, j) of S is (j, i)
    // of a tall X.  Addresses are clamped into the matrix so that every
    // load is issued unconditionally and all of them overlap; out-of-range
    // entries are replaced by zero afterwards.
    const int64_t eo = g.elem0 + (int64_t)mi * g.elem_stride;
    const int sr = s_rows(g), sc = s_cols(g);
    const bool tall = s_tall(g);
    if (tall != SWAP && g.vec_ok && g.cols % 4 == 0) {
      // the 4 registers of a tile are 4 consecutive entries of a row of X:
      // one 16-byte load (cols is a multiple of 4, so a group of 4 is
      // either inside the matrix or wholly past it)
      const int xrows = tall ? sc : sr;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int si = acc_row(i, 0), sj = acc_col(j, 0);
          const int xr = tall ? sj : si, xc = tall ? si : sj;
          const int rc = xr < xrows ? xr : xrows - 1, cc = xc < g.cols ? xc : g.cols - 4;
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(A.xs_user + eo + (int64_t)rc * g.cols + cc);
          const bool in = si < sr && sj < sc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = in ? A.ca * x[r] : 0.0f;
        }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int si = acc_row(i, r), sj = acc_col(j, r);
            const int ic = si < sr ? si : sr - 1, jc = sj < sc ? sj : sc - 1;
            const int64_t e = tall ? (int64_t)jc * g.cols + ic : (int64_t)ic * g.cols + jc;
            const float x = A.xs_user[eo + e];
            acc[i][j][r] = si < sr && sj < sc ? A.ca * x : 0.0f;
          }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Later steps read the update's a S term from the B operand tiles in LDS
  // while they pass through: S is read k-major, and the slab holding
  // k = m0 + wm*WTM + i*16 .. +15 contains S(m, n) for this wave's output
  // rows m and columns n.  Each k-block of 16 lies in one slab.
  const int ax_k0 = m0 + wm * WTM;  // first k of the a S block
  // a S for the 16-row block u of the wave tile from the stage holding it:
  // row k = m of the slab, 4 consecutive columns n per lane (one 8-byte
  // read for bf16, 16 bytes for float32)
  auto add_ax_block = [&](auto uc, int s, int stg) SM_INLINE {
    if constexpr (SWAP) {
      constexpr int u = decltype(uc)::value;
      const int row = ax_k0 + u * 16 - s * BK + (lane & 15);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int byte = (acc_col(j, 0) - n0) * (int)sizeof(T);
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp) {
          const char* p = b_tile(stg, sp) + km_off<T, BNT>(row, byte);
          if constexpr (sizeof(T) == 4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
            x[0] += v[0]; x[1] += v[1]; x[2] += v[2]; x[3] += v[3];
          } else {
            const u32x2_t h = *reinterpret_cast<const u32x2_t*>(p);
            x[0] += __uint_as_float(h[0] << 16); x[1] += __uint_as_float(h[0] & 0xFFFF0000u);
            x[2] += __uint_as_float(h[1] << 16); x[3] += __uint_as_float(h[1] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][j][r] += A.ca * x[r];
      }
    } else {
      constexpr int u = decltype(uc)::value;
      const int kb = ax_k0 + u * 16 - s * BK;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int c0 = wn * WTN + j * 16;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp) {
          const char* tile = b_tile(stg, sp);
          if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[r] += *reinterpret_cast<const float*>(
                  tile + km_off<T, BNT>(kb + 4 * (lane >> 4) + r, 4 * (c0 + (lane & 15))));
          } else {
            const u32x2_t h = lds_read_tr16(
                tile + km_off<T, BNT>(kb + 4 * (lane >> 4) + ((lane & 15) >> 2), 2 * c0 + 8 * (lane & 3)));
            x[0] += __uint_as_float(h[0] << 16); x[1] += __uint_as_float(h[0] & 0xFFFF0000u);
            x[2] += __uint_as_float(h[1] << 16); x[3] += __uint_as_float(h[1] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][j][r] += A.ca * x[r];
      }
    }
  };
  // every 16-row block of the a S term that lies in slab s
  auto add_ax = [&](int s, int stg) SM_INLINE {
    static_assert(TI <= 8, "a S blocks");
    auto one = [&](auto uc) SM_INLINE {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < TI)
        if ((ax_k0 + 16 * u) / BK == s) add_ax_block(uc, s, stg);
    };
    one(std::integral_constant<int, 0>{}); one(std::integral_constant<int, 1>{});
    one(std::integral_constant<int, 2>{}); one(std::integral_constant<int, 3>{});
    one(std::integral_constant<int, 4>{}); one(std::integral_constant<int, 5>{});
    one(std::integral_constant<int, 6>{}); one(std::integral_constant<int, 7>{});
  };

  constexpr int LOADS = SPLIT * (QA + QB);     // vector loads per thread per slab

  // MFMAs of one k-step on one accumulator tile.
  auto mfma_tile = [&](const u32x4_t* fa, const u32x4_t* fb, int i, int j) SM_INLINE {
    // C tile (SWAP: C^T tile) += A B over one k-step
    auto mm = [&](const u32x4_t& x, const u32x4_t& y) SM_INLINE {
      const u32x4_t& p = SWAP ? y : x;
      const u32x4_t& q = SWAP ? x : y;
      if constexpr (sizeof(T) == 2) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p),
                                                            __builtin_bit_cast(bf16x8_t, q),
                                                            acc[i][j], 0, 0, 0);
      } else {
        const f32x4_t pv = __builtin_bit_cast(f32x4_t, p), qv = __builtin_bit_cast(f32x4_t, q);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[e], qv[e], acc[i][j], 0, 0, 0);
      }
    };
    mm(fa[0], fb[0]);
    if constexpr (SPLIT == 2) {
      mm(fa[0], fb[TJ]);   // hi * lo
      mm(fa[TI], fb[0]);   // lo * hi
    }
  };

  // fragments of one slab: [kk][split * TI + i] (A) and [kk][split * TJ + j] (B)
  constexpr int NFA = SPLIT * TI, NFB = SPLIT * TJ, NF = NKK * (NFA + NFB);
  // fragment q of a slab (q = kk * (NFA + NFB) + A fragments, then B),
  // with the slab's operand layouts (k-major or k along rows) given as
  // compile-time constants akc, bkc
  auto read_one = [&](auto akc, auto bkc, u32x4_t (&fa)[NKK][NFA], u32x4_t (&fb)[NKK][NFB],
                      int stg, int q) SM_INLINE {
    constexpr bool AT = decltype(akc)::value, BT = decltype(bkc)::value;
    const int kk = q / (NFA + NFB), r = q % (NFA + NFB);
    if (r < NFA) {
      const int sp = r / TI, i = r % TI;
      if constexpr (AT && sizeof(T) == 2)
        fa[kk][r] = km_frag2(std::integral_constant<int, BMT>{}, a_tile(stg, sp), kmA, i, kk);
      else if constexpr (AT)
        fa[kk][r] = km_frag(std::integral_constant<int, BMT>{}, a_tile(stg, sp), wm * WTM + 16 * i, kk);
      else
        fa[kk][r] = *reinterpret_cast<const u32x4_t*>(a_tile(stg, sp) + (fa_off0 ^ (kk << 6)) + i * 16 * RB);
    } else {
      const int rb = r - NFA, sp = rb / TJ, j = rb % TJ;
      if constexpr (BT && sizeof(T) == 2)
        fb[kk][rb] = km_frag2(std::integral_constant<int, BNT>{}, b_tile(stg, sp), kmB, j, kk);
      else if constexpr (BT)
        fb[kk][rb] = km_frag(std::integral_constant<int, BNT>{}, b_tile(stg, sp), wn * WTN + 16 * j, kk);
      else
        fb[kk][rb] = *reinterpret_cast<const u32x4_t*>(b_tile(stg, sp) + (fb_off0 ^ (kk << 6)) + j * 16 * RB);
    }
  };
  using kTrue = std::true_type;
  using kFalse = std::false_type;
  auto ax_here = [&](int s) {
    if constexpr (EPI == E_UPDATE)
      return !ax_user && A.ca != 0.0f && s * BK < ax_k0 + 16 * TI && ax_k0 < (s + 1) * BK;
    else return false;
  };

  // The square kernel's term cb Y (out = cb Y + cc X Y, Y symmetric) is
  // taken from the B operand tiles while they pass through LDS: the B tile
  // holds rows n0.. of Y, and the slab holding k = m0 + wm*WTM + 16 i ..
  // holds Y(col, row) = Y(row, col) for this wave's output rows.  It is
  // added as (cb / cc) Y into the accumulators and the epilogue multiplies by
  // cc (cc != 0; otherwise the epilogue loads Y).
  const int sq_k0 = m0 + wm * WTM;
  const bool sq_lds = EPI == E_SQUARE && A.cc != 0.0f;
  const float sq_ratio = sq_lds ? A.cb / A.cc : 0.0f;
  auto sq_here = [&](int s) {
    if constexpr (EPI == E_SQUARE) return sq_lds && s * BK < sq_k0 + 16 * TI && sq_k0 < (s + 1) * BK;
    else return false;
  };
  auto add_sq = [&](auto bkc, int s, int stg) SM_INLINE {
    if constexpr (SWAP) {
      // transposed tiles: lane l holds row 16 i + l % 16 of the wave tile,
      // columns 16 j + 4 (l / 16) .. +3
      static_assert(sizeof(T) == 2 && SPLIT == 1, "transposed symmetric tiles are bf16");
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int kb = sq_k0 + 16 * i - s * BK;
        if (kb < 0 || kb >= BK) continue;
        const int kr = kb + (lane & 15);          // this lane's row k in the slab
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int cb0 = wn * WTN + 16 * j + 4 * (lane >> 4);   // first column - n0
          float y[4];
          if constexpr (decltype(bkc)::value) {
            // k-major slab: Y(k, n0 + c .. +3) is one 8-byte read
            const u32x2_t h = *reinterpret_cast<const u32x2_t*>(
                b_tile(stg, 0) + km_off<T, BNT>(kr, 2 * cb0));
            y[0] = __uint_as_float(h[0] << 16); y[1] = __uint_as_float(h[0] & 0xFFFF0000u);
            y[2] = __uint_as_float(h[1] << 16); y[3] = __uint_as_float(h[1] & 0xFFFF0000u);
          } else {
            // slab along rows (the diagonal tile): Y(k, col) = Y(col, k)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              y[r] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(
                  b_tile(stg, 0) + lds_off<RB>(cb0 + r, kr / P) + (kr % P) * 2));
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += sq_ratio * y[r];
        }
      }
      return;
    }
    if constexpr (EPI == E_SQUARE && decltype(bkc)::value) {
      // off the diagonal with upper-triangular storage the slab holds
      // Y(k, n0 + c) k-major: 4 consecutive k of one column per lane are
      // one transposing read
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int kb = sq_k0 + 16 * i - s * BK;
        if (kb < 0 || kb >= BK) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int c0 = wn * WTN + 16 * j;
          const u32x2_t h = lds_read_tr16(
              b_tile(stg, 0) + km_off<T, BNT>(kb + 4 * (lane >> 4) + ((lane & 15) >> 2),
                                              2 * c0 + 8 * (lane & 3)));
          acc[i][j][0] += sq_ratio * __uint_as_float(h[0] << 16);
          acc[i][j][1] += sq_ratio * __uint_as_float(h[0] & 0xFFFF0000u);
          acc[i][j][2] += sq_ratio * __uint_as_float(h[1] << 16);
          acc[i][j][3] += sq_ratio * __uint_as_float(h[1] & 0xFFFF0000u);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int kb = sq_k0 + 16 * i - s * BK;   // this 16-row block's k offset in the slab
      if (kb < 0 || kb >= BK) continue;
      const int kk = kb + 4 * (lane >> 4);      // 4 consecutive k (rows of the output)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int brow = wn * WTN + 16 * j + (lane & 15);   // output column - n0
        float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < SPLIT; ++sp) {
          const char* p = b_tile(stg, sp) + lds_off<RB>(brow, kk / P) + (kk % P) * (int)sizeof(T);
          if constexpr (sizeof(T) == 4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
            y[0] += v[0]; y[1] += v[1]; y[2] += v[2]; y[3] += v[3];
          } else {
            const u32x2_t h = *reinterpret_cast<const u32x2_t*>(p);
            y[0] += __uint_as_float(h[0] << 16); y[1] += __uint_as_float(h[0] & 0xFFFF0000u);
            y[2] += __uint_as_float(h[1] << 16); y[3] += __uint_as_float(h[1] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += sq_ratio * y[r];
      }
    }
  };

  if constexpr (!PIPE) {
#pragma unroll
    for (int s = 0; s < NSTG - 1; ++s)
      if (s < nslab) issue(s);

    // one slab with compile-time layouts; the layouts come in runs of the
    // slab order, one loop per run (as in the pipelined loop below)
    auto slab = [&](auto akc, auto bkc, int s) SM_INLINE {
      // the k-major read addresses derive from one register per operand;
      // redefining it opaquely here keeps the derived addresses from being
      // hoisted out of the loops and held in registers
      if constexpr (decltype(akc)::value && sizeof(T) == 2) asm volatile("" : "+v"(kmA));
      if constexpr (decltype(bkc)::value && sizeof(T) == 2) asm volatile("" : "+v"(kmB));
      // slab s has landed for this wave once at most the later slabs' loads
      // are outstanding; the barrier extends that to every wave and also
      // frees stage (s-1) % NSTG for the next fetch.
      if constexpr (NSTG >= 3) {
        if (s + NSTG - 2 < nslab) wait_vmcnt<(NSTG - 2) * LOADS>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");

      const int stg = s % NSTG;
      // every fragment read of the slab ahead of the MFMAs, so the waits
      // before them count down outstanding reads instead of draining them;
      // the reads also precede the next fetch, since a transposing LDS read
      // waits for every LDS DMA load issued before it
      u32x4_t fa[NKK][NFA], fb[NKK][NFB];
#pragma unroll
      for (int q = 0; q < NF; ++q) read_one(akc, bkc, fa, fb, stg, q);
      __builtin_amdgcn_sched_barrier(0);
      if (s + NSTG - 1 < nslab) issue(s + NSTG - 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) mfma_tile(&fa[kk][i], &fb[kk][j], i, j);
      if constexpr (EPI == E_UPDATE) {
        // after the slab's MFMAs, when the fragment registers are free again
        __builtin_amdgcn_sched_barrier(0);
        if (ax_here(s)) add_ax(s, stg);
      }
      if constexpr (EPI == E_SQUARE) {
        __builtin_amdgcn_sched_barrier(0);
        if (sq_here(s)) add_sq(bkc, s, stg);
      }
    };
    int s = 0;
    auto run = [&](auto akc, auto bkc, int end) SM_INLINE {
      for (; s < end; ++s) slab(akc, bkc, s);
    };
    if constexpr (UPR && EPI == E_SQUARE) {
      run(kTrue{}, kTrue{}, sA);
      run(kFalse{}, kTrue{}, sB);
      run(kFalse{}, kFalse{}, nslab);
    } else if constexpr (UPR) {
      run(kTrue{}, kTrue{}, sA);
      run(kFalse{}, kTrue{}, nslab);
    } else {
      run(std::integral_constant<bool, a_km>{}, std::integral_constant<bool, b_km>{}, nslab);
    }
  } else {
    // Software-pipelined k-loop: the fragments of slab s+1 are read into a
    // second register set while the MFMAs of slab s run, so no MFMA waits
    // for LDS.  Per slab s: wait for slab s+1's fetch and for this wave's
    // reads of slab s, barrier (then stage s % NSTG is free and slab s+1 is
    // in LDS for every wave), then the MFMAs of slab s interleaved with the
    // reads of slab s+1 and the fetch of slab s+NSTG into stage s % NSTG
    // (a slab read with plain loads only is fetched first; k-major
    // fragments are read before the fetch, see below).
    // After the last slab those reads hit a stale stage and are never used,
    // which keeps the MFMA sequence free of branches.  The slab count is
    // even (k is a multiple of 128).
    constexpr int NM = NKK * TI * TJ;                 // MFMA tiles per slab
    u32x4_t fa0[NKK][NFA], fb0[NKK][NFB], fa1[NKK][NFA], fb1[NKK][NFB];
    // (every launch has at least NSTG slabs: the host checks k)
#pragma unroll
    for (int p = 0; p < NSTG; ++p) issue(p);
    wait_vmcnt<(NSTG - 1) * LOADS>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The step's reads of slab s+1 use that slab's operand layouts (akc,
    // bkc).  The compiler makes a transposing LDS read wait for every LDS
    // DMA load issued before it (vmcnt(0)), which would wait for the fetch
    // just issued; plain reads get no such wait.  So with k-major fragments
    // those reads go with the first MFMAs, then the fetch, then the plain
    // reads; with none the fetch goes first and a read follows every second
    // MFMA.
    // (the last step, lastc = true, only runs the MFMAs of its slab)
    auto step = [&](auto akc, auto bkc, auto lastc, int s, u32x4_t (&ca)[NKK][NFA],
                    u32x4_t (&cb)[NKK][NFB], u32x4_t (&na)[NKK][NFA],
                    u32x4_t (&nb)[NKK][NFB]) SM_INLINE {
      constexpr bool AT = decltype(akc)::value, BT = decltype(bkc)::value;
      if constexpr (decltype(lastc)::value) {
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          const int kk = t / (TI * TJ), i = (t / TJ) % TI, j = t % TJ;
          mfma_tile(&ca[kk][i], &cb[kk][j], i, j);
        }
        return;
      }
      if (s + 1 < nslab) {
        // slab s+1 landed for this wave (later fetches may be in flight)
        if (s + NSTG - 1 < nslab) wait_vmcnt<(NSTG - 2) * LOADS>();
        else wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      const int nst = (s + 1) % NSTG;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!UPR && !AT && !BT) {
        if (s + 1 < nslab && s + NSTG < nslab) issue(s + NSTG);   // into stage s % NSTG, read out already
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          const int kk = t / (TI * TJ), i = (t / TJ) % TI, j = t % TJ;
          mfma_tile(&ca[kk][i], &cb[kk][j], i, j);
          if ((t & 1) && (t >> 1) < NF) read_one(akc, bkc, na, nb, nst, t >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = NM / 2; q < NF; ++q) read_one(akc, bkc, na, nb, nst, q);
      } else {
        // B's fragments, then A's, one with each of the first MFMAs, at the
        // same points whatever the slab's layouts (so that every layout
        // keeps the fragments in the same registers); the fetch goes after
        // the last k-major read, or first when there is none.
        constexpr int NB = NKK * NFB, NA = NKK * NFA;
        constexpr int NKM = (AT ? NA : 0) + (BT ? NB : 0);
        static_assert(NB + NA <= NM, "read schedule");
        static_assert(BT || !AT, "A k-major implies B k-major");
        auto qb = [&](int u) { return (u / NFB) * (NFA + NFB) + NFA + u % NFB; };
        auto qa = [&](int u) { return (u / NFA) * (NFA + NFB) + u % NFA; };
        if constexpr (NKM == 0) {
          if (s + 1 < nslab && s + NSTG < nslab) issue(s + NSTG);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < NM; ++t) {
          const int kk = t / (TI * TJ), i = (t / TJ) % TI, j = t % TJ;
          mfma_tile(&ca[kk][i], &cb[kk][j], i, j);
          if (t < NB) read_one(akc, bkc, na, nb, nst, qb(t));
          else if (t < NB + NA) read_one(akc, bkc, na, nb, nst, qa(t - NB));
          if (NKM > 0 && t == NKM - 1 && s + 1 < nslab && s + NSTG < nslab) {
            __builtin_amdgcn_sched_barrier(0);
            issue(s + NSTG);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (s + 1 < nslab && ax_here(s + 1)) {
        __builtin_amdgcn_sched_barrier(0);
        add_ax(s + 1, nst);
      }
      if (s + 1 < nslab && sq_here(s + 1)) {
        __builtin_amdgcn_sched_barrier(0);
        add_sq(bkc, s + 1, nst);
      }
    };
    // Step s reads slab s+1 with that slab's layouts, which change only at
    // even slabs (sA and sB are multiples of the slabs per tile, an even
    // number), and slabs 0 and 1 are k-major for both operands whenever
    // the operands are symmetric.  So the loop runs pairs of steps (s odd,
    // s+1), which read slabs s+1 and s+2 of one layout, one loop per layout,
    // each with a single schedule (a change of schedule from step to step
    // inside one loop made the register allocation spill).  Before them the
    // reads of slab 0 and step 0 (reading slab 1), after them the last step.
    // (Slab counts are even here: k is a multiple of 128 elements, and
    // split-k ranges are even.)
    using kBkm = std::integral_constant<bool, b_km>;
    using kA0 = std::integral_constant<bool, UPR || a_km>;
    using kB0 = std::integral_constant<bool, UPR || b_km>;
#pragma unroll
    for (int q = 0; q < NF; ++q) read_one(kA0{}, kB0{}, fa0, fb0, 0, q);
    if (ax_here(0)) add_ax(0, 0);
    if (sq_here(0)) add_sq(kB0{}, 0, 0);
    step(kA0{}, kB0{}, kFalse{}, 0, fa0, fb0, fa1, fb1);
    const int last = nslab - 1;
    int s = 1;
    auto pairs = [&](auto akc, auto bkc, int end) SM_INLINE {
      // pairs (s, s+1) with s + 1 < end (the first slab they read)
      for (; s < last && s + 1 < end; s += 2) {
        step(akc, bkc, kFalse{}, s, fa1, fb1, fa0, fb0);
        step(akc, bkc, kFalse{}, s + 1, fa0, fb0, fa1, fb1);
      }
    };
    if constexpr (UPR && EPI == E_SQUARE) {
      pairs(kTrue{}, kTrue{}, sA);      // k < 128 (tm + 1): both k-major
      pairs(kFalse{}, kTrue{}, sB);     // B k-major
      pairs(kFalse{}, kFalse{}, nslab);
    } else if constexpr (UPR) {
      pairs(kTrue{}, kTrue{}, sA);      // k < 128 (tm + 1): A k-major
      pairs(kFalse{}, kTrue{}, nslab);
    } else {
      pairs(std::integral_constant<bool, a_km>{}, kBkm{}, nslab);
    }
    step(kFalse{}, kBkm{}, kTrue{}, last, fa1, fb1, fa0, fb0);
  }

  // ---- epilogue (accumulator coordinates: acc_row / acc_col).  For the
  // update C is the new S: (row, col) of S is (col, row) of a tall X.
  const int idx = g.idx0 + mi * g.idx_stride;
  const float cs = A.scal ? A.scal[idx] : 1.0f;
  const int rows = g.rows, cols = g.cols;
  const int sr = s_rows(g), sc = s_cols(g);
  const bool tall = s_tall(g);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t Rp = round_up(sr, kPad);   // rows of S (padded)
  const int64_t Cp = round_up(sc, kPad);   // columns of S (padded)
  // every wave is done reading the operand stages: LDS is free for staging
  __syncthreads();

  if constexpr (EPI == E_OP || EPI == E_RAW) {   // (only Grams are split along k)
    if (g.ksplit > 1) {
      // split-k: the raw float32 tile of this split in accumulator order
      // (register group (i, j) of lane l of wave w at float4 index
      // ((w TI + i) TJ + j) 64 + l, one coalesced 16-byte store each); the
      // tile is summed over the splits and finished by k_split_reduce
      static_assert(!SWAP && NW == 4 && TI == 4 && TJ == 4, "split-k accumulator order");
      const int ntri = g.tiles_n * (g.tiles_n + 1) / 2;
      f32x4_t* dst = reinterpret_cast<f32x4_t*>(A.kpart + g.kp0 + (int64_t)mi * g.kp_stride +
                                                ((int64_t)ks * ntri + ttri) * (BMT * BNT));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) dst[((wave * TI + i) * TJ + j) * 64 + lane] = acc[i][j];
      return;
    }
  }
  if constexpr (EPI == E_RAW) {
    stage_store_tile<float, 1, BMT, BNT, TI, TJ, NT>(acc, smem, A.o_raw + roff, nullptr, Rp, m0,
                                                     n0, (int)Rp, wm, wn, lane, tid);
    if (tm != tn)
      stage_store_mirror<float, 1, BMT, BNT, TI, TJ, NT>(acc, smem, A.o_raw + roff, nullptr, Rp, m0,
                                                         n0, (int)Rp, wm, wn, lane, tid);
  } else if constexpr (EPI == E_OP) {
    const float m = A.mul * (A.scal_pow == 2 ? cs * cs : 1.0f);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] *= m;
    stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o_hi, roff),
                                                     offset_ptr<T>(A.o_lo, roff), Rp, m0, n0,
                                                     (int)Rp, wm, wn, lane, tid);
    if (tm != tn && !upper)
      stage_store_mirror<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o_hi, roff),
                                                         offset_ptr<T>(A.o_lo, roff), Rp, m0, n0,
                                                         (int)Rp, wm, wn, lane, tid);
    if constexpr (sizeof(T) == 2 && SPLIT == 1) {
      if (A.o2_hi) {
        // o2 = o2_a I + o2_b (this tile), the identity on the diagonal tile
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][r] = A.o2_b * acc[i][j][r] + (acc_row(i, r) == acc_col(j, r) ? A.o2_a : 0.0f);
        __syncthreads();   // the last image has been read out
        stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o2_hi, roff),
                                                         nullptr, Rp, m0, n0, (int)Rp, wm, wn,
                                                         lane, tid);
        if (tm != tn && !upper)
          stage_store_mirror<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o2_hi, roff),
                                                             nullptr, Rp, m0, n0, (int)Rp, wm, wn,
                                                             lane, tid);
      }
    }
  } else if constexpr (EPI == E_SQUARE) {
    // b A + c A^2; A is symmetric, so A(row..row+3, col) = A(col, row..row+3)
    // (combined tile by tile, so that the loaded values and the accumulator
    // never have to be held in registers side by side)
    if (sq_lds) {
      // cb Y was added from LDS as (cb / cc) Y
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] *= A.cc;
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // Y(row, col) of this upper tile (tm, tn), stored in every layout
            const float x = load_op<T, SPLIT>(
                A.sq_hi, A.sq_lo, roff + (int64_t)acc_row(i, r) * Rp + acc_col(j, r));
            acc[i][j][r] = A.cb * x + A.cc * acc[i][j][r];
          }
    }
    stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT, SWAP>(acc, smem, offset_ptr<T>(A.o_hi, roff),
                                                           offset_ptr<T>(A.o_lo, roff), Rp, m0, n0,
                                                           (int)Rp, wm, wn, lane, tid);
    if (tm != tn && !upper)
      stage_store_mirror<T, SPLIT, BMT, BNT, TI, TJ, NT, SWAP>(
          acc, smem, offset_ptr<T>(A.o_hi, roff), offset_ptr<T>(A.o_lo, roff), Rp, m0, n0, (int)Rp,
          wm, wn, lane, tid);
  } else {
    // E_UPDATE:  acc = a X + B X (first step: X = the unscaled source), and
    // the iterate is c^p * acc with c = 1/(s+eps) on the first step.
    const float gam = A.scal_pow == 1 ? cs : 1.0f;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] *= gam;

    if (A.out == O_X) {
      stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT, SWAP>(acc, smem, offset_ptr<T>(A.o_hi, xoff),
                                                             offset_ptr<T>(A.o_lo, xoff), Cp, m0,
                                                             n0, (int)Rp, wm, wn, lane, tid);
    } else if (A.out == O_U || A.out == O_APPLY || A.out == O_TERN) {
      if (A.out == O_APPLY && A.status && A.status[0] != 0) return;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int si = acc_row(i, r), sj = acc_col(j, r);
            if (si < sr && sj < sc) {
              const int64_t e = eoff + (tall ? (int64_t)sj * cols + si : (int64_t)si * cols + sj);
              const float u = acc[i][j][r];
              if (A.out == O_U) A.U[e] = u;
              else if (A.out == O_TERN) A.tern[e] = (int8_t)(u > 0.0f ? 1 : u < 0.0f ? -1 : 0);
              else apply_one(A.W, A.w_bf16, e, A.eta, u);
            }
          }
    } else {
      // O_BITS: entrywise sign packed into 32-bit words along the rows of
      // X: along the rows of S, or down its columns when X is tall.  With
      // cols % 32 == 0 a word covers two neighbouring tiles of one line.
      const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
      if (cols % 32 != 0) {
        // a word may take bits from two lines of X, and so from other
        // blocks: each entry sets or clears its own bit with an atomic
        // (bitwise, so the order does not matter), and the matrix's last
        // entry also clears the bits of its word past the end
        const int64_t last = (int64_t)rows * cols - 1;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int si = acc_row(i, r), sj = acc_col(j, r);
              if (si < sr && sj < sc) {
                const int64_t e = tall ? (int64_t)sj * cols + si : (int64_t)si * cols + sj;
                uint32_t* w = A.bits + woff + (e >> 5);
                const uint32_t bit = 1u << (e & 31);
                const uint32_t keep = e == last ? (bit << 1) - 1u : 0xFFFFFFFFu;
                if (acc[i][j][r] < 0.0f) {
                  atomicOr(w, bit);
                  if (keep != 0xFFFFFFFFu) atomicAnd(w, keep);
                } else {
                  atomicAnd(w, ~bit & keep);
                }
              }
            }
      } else if (tall == SWAP) {
        // lanes 0..15 of a tile run along the word: a wave ballot of
        // register r gives 4 x 16 sign bits, one 16-bit half-word for each
        // lane group q, and lane q < 4 writes the word of line 4 q + r
#pragma unroll
        for (int u = 0; u < (SWAP ? TI : TJ) / 2; ++u)
#pragma unroll
          for (int v = 0; v < (SWAP ? TJ : TI); ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const f32x4_t& t0 = SWAP ? acc[2 * u][v] : acc[v][2 * u];
              const f32x4_t& t1 = SWAP ? acc[2 * u + 1][v] : acc[v][2 * u + 1];
              const uint64_t b0 = __ballot(t0[r] < 0.0f);
              const uint64_t b1 = __ballot(t1[r] < 0.0f);
              if (lane < 4) {
                const uint32_t w = (uint32_t)((b0 >> (16 * lane)) & 0xFFFFu) |
                                   ((uint32_t)((b1 >> (16 * lane)) & 0xFFFFu) << 16);
                // the word's row of X and its first column
                const int line = 16 * v + 4 * lane + r, start = 32 * u;
                const int xrow = SWAP ? n0 + wn * WTN + line : m0 + wm * WTM + line;
                const int xcol = SWAP ? m0 + wm * WTM + start : n0 + wn * WTN + start;
                if (xrow < rows && xcol < cols)
                  A.bits[woff + ((int64_t)xrow * cols + xcol) / 32] = w;
              }
            }
      } else {
        // the 4 registers of a tile run along the word: lane 16 q + t holds
        // entries 4 q .. 4 q + 3 of line t of both tiles, whose signs go to
        // bits 4 q + r and 16 + 4 q + r; the 4 lanes of a line combine
        // theirs with two lane exchanges and lane t < 16 writes the word
#pragma unroll
        for (int u = 0; u < (SWAP ? TJ : TI) / 2; ++u)
#pragma unroll
          for (int v = 0; v < (SWAP ? TI : TJ); ++v) {
            const f32x4_t& t0 = SWAP ? acc[v][2 * u] : acc[2 * u][v];
            const f32x4_t& t1 = SWAP ? acc[v][2 * u + 1] : acc[2 * u + 1][v];
            uint32_t w = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              w |= (t0[r] < 0.0f ? 1u : 0u) << r | (t1[r] < 0.0f ? 1u : 0u) << (16 + r);
            w <<= 4 * (lane >> 4);
            w |= (uint32_t)__shfl_xor((int)w, 16);
            w |= (uint32_t)__shfl_xor((int)w, 32);
            const int line = 16 * v + (lane & 15), start = 32 * u;
            const int xrow = SWAP ? m0 + wm * WTM + line : n0 + wn * WTN + line;
            const int xcol = SWAP ? n0 + wn * WTN + start : m0 + wm * WTM + start;
            if (lane < 16 && xrow < rows && xcol < cols)
              A.bits[woff + ((int64_t)xrow * cols + xcol) / 32] = w;
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-k reduction of a symmetric output.  A block takes one 16-row block
// of an upper-triangular 128x128 tile: the partial tiles are stored in the
// GEMM's accumulator order, where the 16 rows 16 rb .. +15 (rb = 4 wm + i)
// are register groups (i, j) of the two waves (wm, wn), wn = 0, 1: 8 x 64
// float4 entries, float4 e of lane l holding rows 4 (l / 16) + 0..3 of
// column 64 wn + 16 j + l % 16.  The block sums them over the splits in
// split order (four splits in flight), transposes the sum through LDS into
// rows, and finishes as the unsplit epilogue does: the raw Gram (RAW), or
// the Gram operand scaled by mul (times c^2 for the first Gram), written in
// place and, off the diagonal, as the mirror rows.
// ---------------------------------------------------------------------------
constexpr int kReduceRows = 16;
template <typename T, int SPLIT, bool RAW>
__global__ __launch_bounds__(256) void k_split_reduce(GemmArgs A) {
  constexpr int TT = kTileSym, RR = kReduceRows, NRB = TT / RR;
  __shared__ float img[RR][TT + 1];
  const int gi = find_group(A.G, blockIdx.x);
  const Group& g = A.G.g[gi];
  const int lb = blockIdx.x - g.block0;
  const int mi = lb / g.blocks_per_mat;
  const int rest = lb - mi * g.blocks_per_mat;
  const int t = rest / NRB, rb = rest - t * NRB;   // triangular tile, row block
  int tm = 0, rem = t;
  while (rem >= g.tiles_n - tm) { rem -= g.tiles_n - tm; ++tm; }
  const int tn = tm + rem;
  const int ntri = g.tiles_n * (g.tiles_n + 1) / 2;
  const int64_t Rp = round_up(s_rows(g), kPad);
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const int64_t sstride = (int64_t)ntri * (TT * TT) / 4;    // float4 per split
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(
      A.kpart + g.kp0 + (int64_t)mi * g.kp_stride + (int64_t)t * (TT * TT));
  // this thread's two float4: lane l, groups q and q + 4 (q = wn * 4 + j)
  const int l = threadIdx.x & 63, q0 = threadIdx.x >> 6;
  const int wmb = rb >> 2, ib = rb & 3;
  int idx[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = q0 + 4 * h, wn = q >> 2, j = q & 3;
    idx[h] = (((wmb * 2 + wn) * 4 + ib) * 4 + j) * 64 + l;
  }
  f32x4_t s0 = src[idx[0]], s1 = src[idx[1]];
  int k = 1;
  for (; k + 3 < g.ksplit; k += 4) {
    f32x4_t u[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      u[p][0] = src[(k + p) * sstride + idx[0]];
      u[p][1] = src[(k + p) * sstride + idx[1]];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) { s0 += u[p][0]; s1 += u[p][1]; }
  }
  for (; k < g.ksplit; ++k) {
    s0 += src[k * sstride + idx[0]];
    s1 += src[k * sstride + idx[1]];
  }
  float mul = 1.0f;
  if constexpr (!RAW) {
    const float cs = A.scal ? A.scal[g.idx0 + mi * g.idx_stride] : 1.0f;
    mul = A.mul * (A.scal_pow == 2 ? cs * cs : 1.0f);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = q0 + 4 * h, wn = q >> 2, j = q & 3;
    const f32x4_t& sv = h ? s1 : s0;
    const int col = 64 * wn + 16 * j + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) img[4 * (l >> 4) + e][col] = sv[e] * mul;
  }
  __syncthreads();
  void* hi = RAW ? static_cast<void*>(A.o_raw) : A.o_hi;
  void* lo = RAW ? nullptr : A.o_lo;
  const int r = threadIdx.x >> 4, c8 = (threadIdx.x & 15) * 8;   // row of the block, 8 columns
  float v0[4], v1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { v0[e] = img[r][c8 + e]; v1[e] = img[r][c8 + 4 + e]; }
  const int64_t o = roff + (int64_t)(tm * TT + rb * RR + r) * Rp + tn * TT + c8;
  store_op4<T, SPLIT>(hi, lo, o, v0);
  store_op4<T, SPLIT>(hi, lo, o + 4, v1);
  // (bfloat16 Gram operands stored as upper-triangular tiles: no mirror)
  if (tm == tn || (!RAW && sizeof(T) == 2 && SPLIT == 1 && A.upper)) return;
  // mirror: output row tn*TT + cc, columns tm*TT + rb*RR .. +RR-1 (8 per thread)
  const int cc = threadIdx.x >> 1, e0 = (threadIdx.x & 1) * 8;
  float w0[4], w1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { w0[e] = img[e0 + e][cc]; w1[e] = img[e0 + 4 + e][cc]; }
  const int64_t om = roff + (int64_t)(tn * TT + cc) * Rp + tm * TT + rb * RR + e0;
  store_op4<T, SPLIT>(hi, lo, om, w0);
  store_op4<T, SPLIT>(hi, lo, om + 4, w1);
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------
// Launch configurations.
//   128x128 tiles, 4 waves of 64x64, two stages of 128-byte slab rows
//   (64 KB of LDS), so two blocks share a CU and one block's pipeline fill
//   and epilogue overlap the other's k-loop.  (Measured on the
//   Newton-Schulz shapes, where the outputs are only 768 wide: 64-byte slab
//   rows with four blocks per CU, and 256x256 tiles with one block per CU,
//   were all slower.)
//   The bf16 kernels whose accumulators and two slabs of fragments fit in
//   192 registers run the software-pipelined k-loop.
//   Long bf16 updates (k >= 2048, columns a multiple of 256): 128x256
//   tiles, 4 waves of 64x128, three stages of 64-byte slab rows (72 KB),
//   still two blocks per CU; per output they move a quarter fewer operand
//   bytes from L2 into LDS, which pays off on long k-loops (measured: the
//   4096-wide MLP set gains 2%, the nanoGPT set, with k = 768, runs 3%
//   faster with the pipelined 128x128 update).
#ifndef SM_GEMM_WIDE_UPDATE
#define SM_GEMM_WIDE_UPDATE 1
#endif
#ifndef SM_GEMM_PIPE
#define SM_GEMM_PIPE 1
#endif
// Pipeline of the bfloat16 128x128 kernels per epilogue (Gram and raw Gram,
// which share the split-k slab count; symmetric product; update): stages,
// slab row bytes and blocks per CU the register allocation leaves room for.
#ifndef SM_OP_NSTG
#define SM_OP_NSTG 2
#endif
#ifndef SM_OP_RB
#define SM_OP_RB 128
#endif
#ifndef SM_OP_WPE
#define SM_OP_WPE 2
#endif
#ifndef SM_SPLIT_MIN_SLABS
#define SM_SPLIT_MIN_SLABS 8
#endif
#ifndef SM_SPLIT_MIN_SLABS_F32
#define SM_SPLIT_MIN_SLABS_F32 2
#endif
#ifndef SM_DEAL_TILES
#define SM_DEAL_TILES 16
#endif
#ifndef SM_SQ_TRACC
#define SM_SQ_TRACC 1
#endif
#ifndef SM_SQ_NSTG
#define SM_SQ_NSTG 2
#endif
#ifndef SM_SQ_RB
#define SM_SQ_RB 128
#endif
#ifndef SM_SQ_WPE
#define SM_SQ_WPE 2
#endif
#ifndef SM_UP_NSTG
#define SM_UP_NSTG 2
#endif
#ifndef SM_UP_RB
#define SM_UP_RB 128
#endif
#ifndef SM_UP_WPE
#define SM_UP_WPE 2
#endif
template <typename T, int SPLIT, int EPI, bool WIDE = false, bool SMALL = false>
struct Cfg {
  static_assert(!SMALL || (sizeof(T) == 4 && EPI == E_UPDATE && !WIDE), "64x64: float32 update");
  static constexpr bool BF = sizeof(T) == 2 && SPLIT == 1 && !WIDE;
  static constexpr int WM = 2;
  static constexpr int TI = SMALL ? 2 : 4, TJ = WIDE ? 8 : SMALL ? 2 : 4;
  static constexpr int RB = WIDE ? 64
                          : !BF ? 128
                          : EPI == E_OP || EPI == E_RAW ? SM_OP_RB
                          : EPI == E_SQUARE ? SM_SQ_RB
                          : EPI == E_UPDATE ? SM_UP_RB : 128;
  static constexpr int NSTG = WIDE ? 3
                            : !BF ? 2
                            : EPI == E_OP || EPI == E_RAW ? SM_OP_NSTG
                            : EPI == E_SQUARE ? SM_SQ_NSTG
                            : EPI == E_UPDATE ? SM_UP_NSTG : 2;
  static constexpr int WPE = !BF ? 2
                           : EPI == E_OP || EPI == E_RAW ? SM_OP_WPE
                           : EPI == E_SQUARE ? SM_SQ_WPE
                           : EPI == E_UPDATE ? SM_UP_WPE : 2;
  // software pipelining holds two slabs of fragments: used where those and
  // the accumulators fit in 192 registers
  static constexpr bool PIPE = SM_GEMM_PIPE && sizeof(T) == 2 && SPLIT == 1 &&
                               TI * TJ * 4 + 2 * (RB / 64) * (TI + TJ) * 4 <= 192;
  // transposed accumulator tiles for the 128x128 update (measured: the
  // nanoGPT set gains 1.4%, the 128x256 update of the MLP set loses 0.6%)
  // and the bf16 symmetric product (8-byte staging writes of its output)
  static constexpr bool TRACC = (EPI == E_UPDATE && !WIDE) || (EPI == E_SQUARE && BF && SM_SQ_TRACC);
  static constexpr int BMT = WM * 16 * TI, BNT = 32 * TJ;
  static constexpr size_t lds() {
    size_t pipe = (size_t)NSTG * SPLIT * (BMT + BNT) * RB;
    size_t img = (size_t)SPLIT * BMT * (BNT * sizeof(T) + 16);
    size_t raw = (size_t)BMT * (BNT * sizeof(float) + 16);  // raw Gram is float32
    size_t m = pipe > img ? pipe : img;
    return EPI == E_RAW && m < raw ? raw : m;   // the raw Gram is float32
  }
};
using CfgWide = Cfg<bf16_t, 1, E_UPDATE, true>;
constexpr int kWideMinK = 2048;
// 64x64 tiles for the float32 update of small matrices: a 128x128 float32
// tile carries eight times the matrix-core time of a bfloat16 one per slab,
// so a matrix of a few such tiles leaves the GPU nearly idle for the
// length of one block; 64x64 tiles give four times the blocks at a quarter
// of the work each (matrices of at most kSmallMaxTiles 128x128 tiles).
using CfgSmall = Cfg<float, 1, E_UPDATE, false, true>;
constexpr int kSmallMaxTiles = 16;
constexpr int kTile = Cfg<bf16_t, 1, E_UPDATE>::BMT;
static_assert(Cfg<bf16_t, 1, E_UPDATE>::BNT == kTile, "square tile");
static_assert(CfgWide::BMT == kTile, "wide tiles keep the row height");

void gemm_tile(int precision, int epi, int64_t gm, int64_t gn, int64_t gk, int* tm, int* tn) {
  *tm = kTile;
  *tn = kTile;
  if (epi == E_UPDATE && precision == P_F32 && gm % CfgSmall::BMT == 0 &&
      gn % CfgSmall::BNT == 0 &&
      ((gm + kTile - 1) / kTile) * ((gn + kTile - 1) / kTile) <= kSmallMaxTiles) {
    *tm = CfgSmall::BMT;
    *tn = CfgSmall::BNT;
    return;
  }
  if (SM_GEMM_WIDE_UPDATE && epi == E_UPDATE && precision == P_BF16 && gm % kTile == 0 &&
      gn % CfgWide::BNT == 0 && gk >= kWideMinK)
    *tn = CfgWide::BNT;
}

template <typename T, int SPLIT, int EPI, bool WIDE = false, bool SMALL = false>
static hipError_t launch_one(const GemmArgs& args, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  using C = Cfg<T, SPLIT, EPI, WIDE, SMALL>;
  // the pipelined k-loop fills all NSTG stages before its first slab: every
  // block needs at least NSTG slabs (and, pipelined, an even count)
  constexpr int BK = C::RB / (int)sizeof(T);
  for (int i = 0; i < args.G.n; ++i) {
    const Group& g = args.G.g[i];
    if (g.gk % BK) return hipErrorInvalidValue;
    int64_t fewest = g.gk / BK;
    if (g.ksplit > 1) {
      const int64_t last = fewest - (int64_t)(g.ksplit - 1) * g.kslabs;
      fewest = std::min<int64_t>(g.kslabs, last);
    }
    if (fewest < C::NSTG || (C::PIPE && (fewest & 1))) return hipErrorInvalidValue;
  }
  auto kern = k_gemm<T, SPLIT, EPI, C::NSTG, C::WM, C::TI, C::TJ, C::RB, C::WPE, C::PIPE, C::TRACC>;
  if (t0 || t1)   // the events take the kernel's own start and stop times
    hipExtLaunchKernelGGL(kern, dim3(args.G.total_blocks), dim3(128 * C::WM), (uint32_t)C::lds(), s,
                          t0, t1, 0, args);
  else
    hipLaunchKernelGGL(kern, dim3(args.G.total_blocks), dim3(128 * C::WM), C::lds(), s, args);
  return hipGetLastError();
}

template <typename T, int SPLIT>
static hipError_t launch_epi(const GemmArgs& args, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  switch (args.epi) {
    case E_RAW: return launch_one<T, SPLIT, E_RAW>(args, s, t0, t1);
    case E_OP: return launch_one<T, SPLIT, E_OP>(args, s, t0, t1);
    case E_SQUARE: return launch_one<T, SPLIT, E_SQUARE>(args, s, t0, t1);
    default: return launch_one<T, SPLIT, E_UPDATE>(args, s, t0, t1);
  }
}

static_assert(Cfg<bf16_t, 1, E_OP>::BMT == kTileSym && Cfg<bf16_t, 2, E_OP>::BMT == kTileSym &&
                  Cfg<float, 1, E_OP>::BMT == kTileSym && Cfg<bf16_t, 1, E_OP>::BNT == kTileSym,
              "symmetric tile");

// Slabs of at least kSplitMinSlabs per split (float32: kSplitMinSlabsF32,
// since a float32 slab carries eight times the matrix-core time of a
// bfloat16 one: half the k at a sixteenth of the rate); splits only while
// the launch has fewer than kSplitBelow upper-triangular tiles, up to
// kSplitTarget blocks and kSplitMax splits.
constexpr int kSplitMinSlabs = SM_SPLIT_MIN_SLABS, kSplitMinSlabsF32 = SM_SPLIT_MIN_SLABS_F32,
              kSplitBelow = 128,
              kSplitTarget = 256, kSplitMax = 16;

static int64_t sym_slabs(int precision, int64_t gk) {
  return gk / (precision == P_F32 ? Cfg<float, 1, E_OP>::RB / 4 : Cfg<bf16_t, 1, E_OP>::RB / 2);
}

int gemm_sym_ksplit(int precision, int64_t rp, int64_t gk, int64_t count, int* slabs) {
  const int64_t T = rp / kTileSym, tiles = T * (T + 1) / 2 * count;
  const int64_t nslab = sym_slabs(precision, gk);
  *slabs = (int)nslab;
  const int64_t least = precision == P_F32 ? kSplitMinSlabsF32 : kSplitMinSlabs;
  if (tiles >= kSplitBelow || nslab < 2 * least) return 1;
  int64_t want = (kSplitTarget + tiles - 1) / tiles;
  want = std::min<int64_t>({want, nslab / least, (int64_t)kSplitMax});
  if (want < 2) return 1;
  // splits of `per` slabs, per even; the last one is shorter but not empty
  int64_t per = (nslab + want - 1) / want;
  per += per & 1;
  const int64_t ks = (nslab + per - 1) / per;
  if (ks < 2) return 1;
  *slabs = (int)per;
  return (int)ks;
}

int64_t gemm_sym_kpart_floats(int64_t rp, int ksplit) {
  if (ksplit <= 1) return 0;
  const int64_t T = rp / kTileSym;
  return T * (T + 1) / 2 * ksplit * (int64_t)kTileSym * kTileSym;
}

template <typename T, int SPLIT, bool RAW>
static hipError_t launch_reduce(const GemmArgs& args, hipStream_t s) {
  // the groups of the launch that were split: kTileSym / kReduceRows blocks
  // per triangular tile
  GemmArgs r = args;
  std::memset(&r.G, 0, sizeof(r.G));
  int64_t blocks = 0;
  for (int i = 0; i < args.G.n; ++i) {
    Group g = args.G.g[i];
    if (g.ksplit <= 1) continue;
    g.blocks_per_mat = g.tiles_n * (g.tiles_n + 1) / 2 * (kTileSym / kReduceRows);
    g.block0 = (int32_t)blocks;
    blocks += (int64_t)g.blocks_per_mat * g.count;
    r.G.g[r.G.n++] = g;
  }
  if (blocks == 0) return hipSuccess;
  r.G.total_blocks = (int32_t)blocks;
  hipLaunchKernelGGL((k_split_reduce<T, SPLIT, RAW>), dim3(r.G.total_blocks), dim3(256), 0, s, r);
  return hipGetLastError();
}

constexpr int kDealTiles = SM_DEAL_TILES;
// Whole matrices of a Gram launch go to the XCDs in turn unless the
// environment variable SIGNMUON_XCD_DEAL is "0" (read at every launch).
static bool xcd_deal_enabled() {
  const char* e = std::getenv("SIGNMUON_XCD_DEAL");
  return !(e && std::strcmp(e, "0") == 0);
}

hipError_t launch_gemm(int precision, const GemmArgs& args, hipStream_t s, hipEvent_t t0,
                       hipEvent_t t1) {
  if (args.G.total_blocks <= 0) return hipSuccess;
  // every group of a launch carries the same column tile (the host splits
  // launches by it)
  const int tile = args.G.g[0].tile;
  bool split = false;
  for (int i = 0; i < args.G.n; ++i) {
    const Group& g = args.G.g[i];
    int tm, tn;
    gemm_tile(precision, args.epi, g.gm, g.gn, g.gk, &tm, &tn);
    if (g.tile != tile || g.gk % 128 || g.tile != tn) return hipErrorInvalidValue;
    // the second Gram output: bfloat16 Grams that are not split along k
    if (args.o2_hi && (args.epi != E_OP || precision != P_BF16 || g.ksplit > 1))
      return hipErrorInvalidValue;
    if (g.ksplit > 1) {
      // only the Gram and the raw Gram split, into non-empty slab ranges
      const int64_t nslab = sym_slabs(precision, g.gk), per = g.kslabs;
      if ((args.epi != E_OP && args.epi != E_RAW) || !args.kpart || per < 2 || (per & 1) ||
          (int64_t)(g.ksplit - 1) * per >= nslab || (int64_t)g.ksplit * per < nslab ||
          g.blocks_per_mat != g.tiles_n * (g.tiles_n + 1) / 2 * g.ksplit)
        return hipErrorInvalidValue;
      split = true;
    }
  }
  // Grams (k = the long side, which differs between shapes): whole
  // matrices to the XCDs in turn when they all have the same block count.
  // When matrices of different k give less than a full round of whole
  // matrices, or their block counts differ, runs of kDealTiles blocks go
  // round instead, so that the long-k tiles spread over every XCD; equal k
  // keeps the contiguous split, which shares rows in each L2.
  GemmArgs a = args;
  a.xcd_chunk = 0;
  if ((args.epi == E_OP || args.epi == E_RAW) && xcd_deal_enabled()) {
    int c = args.G.g[0].blocks_per_mat;
    bool mixed_k = false;
    for (int i = 1; i < args.G.n; ++i) {
      if (args.G.g[i].blocks_per_mat != c) c = 0;
      if (args.G.g[i].gk != args.G.g[0].gk) mixed_k = true;
    }
    if (mixed_k && (c == 0 || 8 * c > args.G.total_blocks)) c = kDealTiles;
    a.xcd_chunk = c;
  }
  hipError_t e;
  if (tile == CfgWide::BNT) return launch_one<bf16_t, 1, E_UPDATE, true>(a, s, t0, t1);
  if (tile == CfgSmall::BNT) {
    if (precision != P_F32 || args.epi != E_UPDATE) return hipErrorInvalidValue;
    return launch_one<float, 1, E_UPDATE, false, true>(a, s, t0, t1);
  }
  if (precision == P_F32) e = launch_epi<float, 1>(a, s, t0, t1);
  else if (precision == P_BF16X3) e = launch_epi<bf16_t, 2>(a, s, t0, t1);
  else e = launch_epi<bf16_t, 1>(a, s, t0, t1);
  if (e != hipSuccess || !split) return e;
  if (args.epi == E_RAW) return launch_reduce<float, 1, true>(args, s);
  if (precision == P_F32) return launch_reduce<float, 1, false>(args, s);
  if (precision == P_BF16X3) return launch_reduce<bf16_t, 2, false>(args, s);
  return launch_reduce<bf16_t, 1, false>(args, s);
}

template <typename T, int SPLIT, int EPI, bool WIDE = false, bool SMALL = false>
static hipError_t set_lds() {
  using C = Cfg<T, SPLIT, EPI, WIDE, SMALL>;
  return hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<T, SPLIT, EPI, C::NSTG, C::WM, C::TI, C::TJ, C::RB, C::WPE, C::PIPE, C::TRACC>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::lds());
}
template <typename T, int SPLIT>
static hipError_t set_lds_all() {
  hipError_t e;
  if ((e = set_lds<T, SPLIT, E_RAW>()) != hipSuccess) return e;
  if ((e = set_lds<T, SPLIT, E_OP>()) != hipSuccess) return e;
  if ((e = set_lds<T, SPLIT, E_SQUARE>()) != hipSuccess) return e;
  return set_lds<T, SPLIT, E_UPDATE>();
}

hipError_t gemm_set_attributes() {
  hipError_t e;
  if ((e = set_lds_all<bf16_t, 1>()) != hipSuccess) return e;
  if ((e = set_lds_all<bf16_t, 2>()) != hipSuccess) return e;
  if ((e = set_lds_all<float, 1>()) != hipSuccess) return e;
  if ((e = set_lds<float, 1, E_UPDATE, false, true>()) != hipSuccess) return e;
  return set_lds<bf16_t, 1, E_UPDATE, true>();
}

}  // namespace sm
