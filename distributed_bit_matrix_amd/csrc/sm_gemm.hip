// Batched matrix-core GEMM for the Newton-Schulz products of PolarNS
// (SignMuon paper, section 4, Newton-Schulz paragraph): the Gram matrix
// A = X X^T (X^T X for a tall X), the quintic square A*A, and the update
// a X + B X (X B for a tall X), with the epilogues that finish each step.
//
// One launch covers every matrix of a parameter set (up to kMaxGroups runs
// of same-shaped matrices).  Each block owns a 128x128 output tile and runs
// 4 waves (2x2), each wave a 64x64 sub-tile built from 16x16 MFMA tiles:
//   bf16 / split-bf16: v_mfma_f32_16x16x32_bf16
//   f32:               v_mfma_f32_16x16x4_f32
// Every operand is read k-contiguous (the iterate is kept both as X and as
// X^T), so each 128-byte k-slab of a 128-row operand tile is fetched with
// global_load_lds_dwordx4 straight into LDS: lane l of a wave writes the 16
// bytes at the wave's LDS base + 16 l, and the XOR swizzle of 16-byte chunks
// (against bank conflicts of the fragment reads) is applied by permuting
// which global chunk each lane fetches.  NSTG LDS stages form the prefetch
// pipeline; completion is tracked with explicit vmcnt waits and a bare
// s_barrier.  All operand copies are zero padded to multiples of 128, so no
// load is predicated and padding contributes exact zeros.
#include <type_traits>

#include "sm_internal.h"
#include "sm_launch.h"

namespace sm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 128;          // block tile width (and height for WM = 2)

// LDS image of one k-slab of an operand tile: RB bytes per row (64 or 128),
// 16-byte chunks XOR-swizzled by row.  A fragment read (16 lanes on 16
// consecutive rows, one chunk) then touches every bank group once in each
// group of 8 lanes and in each group of 16 lanes.  The swizzle depends on
// row bits 0..3 only, so rows 16 apart share it and a fragment offset
// steps by a constant 16*RB bytes per 16-row tile.
template <int RB>
__host__ __device__ constexpr int swz(int row) {
  if constexpr (RB == 128) return (row ^ ((row >> 3) & 1)) & 7;
  else return ((row >> 1) & 3) ^ ((row >> 3) & 1);
}
template <int RB>
__host__ __device__ constexpr int lds_off(int row, int chunk) {
  return row * RB + ((chunk ^ swz<RB>(row)) << 4);
}
// Compile-time checks of the layout: constant 16-row stride, and distinct
// 16-byte bank groups for every 8 and every 16 lanes of a fragment read
// (banks repeat every 128 / 256 bytes).
template <int RB>
constexpr bool slab_layout_ok() {
  for (int r0 = 0; r0 < 256; r0 += 16)
    for (int ch = 0; ch < RB / 16; ++ch) {
      for (int r = 0; r < 16; ++r)
        if (lds_off<RB>(r0 + r, ch) != lds_off<RB>(r, ch) + r0 * RB) return false;
      for (int span = 8; span <= 16; span *= 2)
        for (int a = 0; a < 16; a += span) {
          unsigned seen = 0;
          for (int r = a; r < a + span; ++r) {
            const int unit = (lds_off<RB>(r0 + r, ch) % (16 * span)) / 16;
            if (seen & (1u << unit)) return false;
            seen |= 1u << unit;
          }
        }
    }
  return true;
}
static_assert(slab_layout_ok<64>() && slab_layout_ok<128>(), "LDS slab swizzle");

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int per16 = 8; };
template <> struct Elem<float>  { static constexpr int per16 = 4; };

// Per-matrix offset and row length of an operand family.
__device__ __forceinline__ int64_t fam_off(const Group& g, int fam, int mi) {
  return fam == FAM_R ? g.r0 + (int64_t)mi * g.r_stride
                      : g.x0 + (int64_t)mi * g.x_stride;
}
__device__ __forceinline__ int64_t fam_ld(const Group& g, int fam) {
  if (fam == FAM_X) return round_up(g.cols, kPad);
  if (fam == FAM_XT) return round_up(g.rows, kPad);
  return round_up(g.rows < g.cols ? g.rows : g.cols, kPad);
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
template <typename T, int SPLIT, int BMT, int BNT, int TI, int TJ, int NT>
__device__ __forceinline__ void stage_store_tile(const f32x4_t (&v)[TI][TJ], char* smem,
                                                 void* dst_hi, void* dst_lo, int64_t ld,
                                                 int m0, int n0, int row_lim, int wm, int wn,
                                                 int lane, int tid) {
  constexpr int ES = sizeof(T);
  constexpr int PITCH = BNT * ES + 16;
  constexpr int IMG = BMT * PITCH;
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

// Four consecutive values held in one accumulator register group.
template <typename T, int SPLIT>
__device__ __forceinline__ void store_acc4(void* hi, void* lo, int64_t i, const f32x4_t& a) {
  const float v[4] = {a[0], a[1], a[2], a[3]};
  store_op4<T, SPLIT>(hi, lo, i, v);
}

// Mirror tile of a symmetric output: C(row..row+3, col) goes to row `col`,
// columns row..row+3 (one 8- or 16-byte store per accumulator tile).
template <typename T, int SPLIT, int TI, int TJ>
__device__ __forceinline__ void store_mirror(const f32x4_t (&v)[TI][TJ], void* hi, void* lo,
                                             int64_t off, int64_t ld, int rbase, int cbase) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      store_acc4<T, SPLIT>(hi, lo, off + (int64_t)(cbase + j * 16) * ld + rbase + i * 16, v[i][j]);
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// Template parameters: operand type and split (bf16 x2 = split-bf16), the
// epilogue, NSTG pipeline stages of RB-byte slab rows, WM x 2 waves of
// (16 TI) x (16 TJ) each, and the waves per SIMD that the register
// allocation must leave room for.
template <typename T, int SPLIT, int EPI, int NSTG, int WM, int TI, int TJ, int RB, int WPE>
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
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- block -> (group, matrix, tile), XCD-aware: the 8 XCDs take blocks
  // round-robin, so consecutive logical tiles are given to one XCD.
  int nb = A.G.total_blocks;
  int b = blockIdx.x;
  {
    int per = nb >> 3, rem = nb & 7, x = b & 7, k = b >> 3;
    b = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
  }
  const int gi = find_group(A.G, b);
  const Group& g = A.G.g[gi];
  const int lb = b - g.block0;
  const int mi = lb / g.blocks_per_mat;
  const int t = lb - mi * g.blocks_per_mat;
  // Symmetric outputs (Gram, raw Gram, quintic square) are computed on the
  // upper-triangular tiles only; the epilogue also writes the mirror tile.
  constexpr bool SYM = EPI != E_UPDATE;
  const int a_fam = g.ops & 3, b_fam = (g.ops >> 2) & 3;
  int tm, tn;
  if constexpr (SYM) {
    tm = 0;
    int rem = t;
    while (rem >= g.tiles_n - tm) { rem -= g.tiles_n - tm; ++tm; }
    tn = tm + rem;
  } else if (a_fam == FAM_R) {
    // the small operand (B = b X X^T) is the A side: consecutive tiles walk
    // down m, so the tiles that share one X^T block run together on one XCD
    // and fetch it from HBM once
    const int tiles_m = (g.gm + BMT - 1) / BMT;
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
  } else {
    tm = t / g.tiles_n;
    tn = t - tm * g.tiles_n;
  }
  const int m0 = tm * BMT, n0 = tn * BNT;
  const int64_t lda = fam_ld(g, a_fam), ldb = fam_ld(g, b_fam);
  const void* a_hi = a_fam == FAM_X ? A.x_hi : (a_fam == FAM_XT ? A.xt_hi : A.r_hi);
  const void* b_hi = b_fam == FAM_X ? A.x_hi : (b_fam == FAM_XT ? A.xt_hi : A.r_hi);
  const void* a_lo = a_fam == FAM_X ? A.x_lo : (a_fam == FAM_XT ? A.xt_lo : A.r_lo);
  const void* b_lo = b_fam == FAM_X ? A.x_lo : (b_fam == FAM_XT ? A.xt_lo : A.r_lo);
  const T* a_src[SPLIT];
  const T* b_src[SPLIT];
  a_src[0] = reinterpret_cast<const T*>(a_hi) + fam_off(g, a_fam, mi);
  b_src[0] = reinterpret_cast<const T*>(b_hi) + fam_off(g, b_fam, mi);
  if constexpr (SPLIT == 2) {
    a_src[SPLIT - 1] = reinterpret_cast<const T*>(a_lo) + fam_off(g, a_fam, mi);
    b_src[SPLIT - 1] = reinterpret_cast<const T*>(b_lo) + fam_off(g, b_fam, mi);
  }

  // Per-lane source offsets of the loads per operand and slab: the A load q
  // of wave w fills LDS rows (QA w+q)*RPI .. +RPI-1 (B: (QB w+q)*RPI ..);
  // lane l writes row ..+l/CPR at chunk position l%CPR, so it fetches global
  // chunk (l%CPR) ^ swz(row).  Rows past the operand (a ragged last tile)
  // read its last row instead; their results are never stored.
  int64_t aoff[QA], boff[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    int row = (wave * QA + q) * RPI + lane / CPR;
    int ch = (lane % CPR) ^ swz<RB>(row);
    int arow = m0 + row < g.gm ? m0 + row : g.gm - 1;
    aoff[q] = (int64_t)arow * lda + ch * P;
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    int row = (wave * QB + q) * RPI + lane / CPR;
    int ch = (lane % CPR) ^ swz<RB>(row);
    int brow = n0 + row < g.gn ? n0 + row : g.gn - 1;
    boff[q] = (int64_t)brow * ldb + ch * P;
  }
  // Per-lane LDS offsets of the fragment reads: row within the tile and
  // 16-byte chunk (kk*4 + lane/16) of the slab row.  The swizzle depends
  // on row bits that i*16 does not touch, so one offset per kk serves all
  // i (j) with a constant stride.
  int fa_off[NKK], fb_off[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    fa_off[kk] = lds_off<RB>(wm * WTM + (lane & 15), kk * 4 + (lane >> 4));
    fb_off[kk] = lds_off<RB>(wn * WTN + (lane & 15), kk * 4 + (lane >> 4));
  }

  const int nslab = g.gk / BK;

  // LDS stage: [A split 0][A split 1..][B split 0][B split 1..]
  auto a_tile = [&](int st, int sp) -> char* { return smem + st * STAGEB + sp * ATILE; };
  auto b_tile = [&](int st, int sp) -> char* {
    return smem + st * STAGEB + SPLIT * ATILE + sp * BTILE;
  };
  auto issue = [&](int s) {
    const int st = s % NSTG;
    const int64_t k0 = (int64_t)s * BK;
#pragma unroll
    for (int sp = 0; sp < SPLIT; ++sp) {
      char* ta = a_tile(st, sp) + wave * QA * 1024;
      char* tb = b_tile(st, sp) + wave * QB * 1024;
#pragma unroll
      for (int q = 0; q < QA; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[sp] + aoff[q] + k0),
                                         (lds_void*)(ta + q * 1024), 16, 0, 0);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[sp] + boff[q] + k0),
                                         (lds_void*)(tb + q * 1024), 16, 0, 0);
    }
  };

  f32x4_t acc[TI][TJ];
  const bool ax_user = EPI == E_UPDATE && A.xsrc == XS_USER;
  if (ax_user) {
    // first step: a X from the caller's float32 source (rows past the
    // matrix are zero), loaded ahead of the k-loop
    const int rb = m0 + wm * WTM + 4 * (lane >> 4), cb = n0 + wn * WTN + (lane & 15);
    const int64_t eo = g.elem0 + (int64_t)mi * g.elem_stride;
    // (addresses clamped into the matrix so that every load is issued
    // unconditionally and all of them overlap; out-of-range entries are
    // replaced by zero afterwards)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rb + i * 16 + r, col = cb + j * 16;
          const int rc = row < g.rows ? row : g.rows - 1, cc = col < g.cols ? col : g.cols - 1;
          const float x = A.xs_user[eo + (int64_t)rc * g.cols + cc];
          acc[i][j][r] = row < g.rows && col < g.cols ? A.ca * x : 0.0f;
        }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Later steps read the update's a X term from the operand tiles in LDS
  // while they pass through: for a wide X (A = B, B operand = X^T) the slab holding
  // k = m0 + wm*WTM + i*16 .. +15 of the X^T block contains X(m, n) for this
  // wave's output rows m and columns n; for a tall X (A operand = X) the
  // slab holding k = n contains X(m, n).  Each k-block of 16 lies in one slab.
  const bool ax_wide = a_fam == FAM_R;
  const int ax_k0 = ax_wide ? m0 + wm * WTM : n0 + wn * WTN;  // first k of the a X block
  // a X for the 16-wide k-block u (acc row block u for a wide X, column
  // block u for a tall one) from the stage that holds it.
  auto add_ax_block = [&](auto uc, int s, int stg) {
    constexpr int u = decltype(uc)::value;
    const int kb = ax_k0 + u * 16 - s * BK;
    if (ax_wide) {
      if constexpr (u < TI) {
        // X^T rows n, 4 consecutive k = m: one 8- (bf16) or 16-byte (f32) read
        const int kk = kb + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wn * WTN + j * 16 + (lane & 15);
          const int off = lds_off<RB>(row, kk / P) + (kk % P) * (int)sizeof(T);
          float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sp = 0; sp < SPLIT; ++sp) {
            const char* p = b_tile(stg, sp) + off;
            if constexpr (sizeof(T) == 4) {
              f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
              x[0] += v[0]; x[1] += v[1]; x[2] += v[2]; x[3] += v[3];
            } else {
              u32x2_t h = *reinterpret_cast<const u32x2_t*>(p);
              x[0] += __uint_as_float(h[0] << 16); x[1] += __uint_as_float(h[0] & 0xFFFF0000u);
              x[2] += __uint_as_float(h[1] << 16); x[3] += __uint_as_float(h[1] & 0xFFFF0000u);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[u][j][r] += A.ca * x[r];
        }
      }
    } else if constexpr (u < TJ) {
      // X rows m (4 consecutive rows), one k = n each: element reads
      const int kk = kb + (lane & 15);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * WTM + i * 16 + 4 * (lane >> 4) + r;
          const int off = lds_off<RB>(row, kk / P) + (kk % P) * (int)sizeof(T);
          float x = 0.0f;
#pragma unroll
          for (int sp = 0; sp < SPLIT; ++sp) {
            const char* p = a_tile(stg, sp) + off;
            if constexpr (sizeof(T) == 4) x += *reinterpret_cast<const float*>(p);
            else x += bf16_to_f32(*reinterpret_cast<const bf16_t*>(p));
          }
          acc[i][u][r] += A.ca * x;
        }
    }
  };
  // every 16-wide k-block of the a X term that lies in slab s
  constexpr int NU = TI > TJ ? TI : TJ;
  const int ax_nu = ax_wide ? TI : TJ;
  auto add_ax = [&](int s, int stg) {
    static_assert(NU <= 8, "a X blocks");
    auto one = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < NU)
        if (u < ax_nu && (ax_k0 + 16 * u) / BK == s) add_ax_block(uc, s, stg);
    };
    one(std::integral_constant<int, 0>{}); one(std::integral_constant<int, 1>{});
    one(std::integral_constant<int, 2>{}); one(std::integral_constant<int, 3>{});
    one(std::integral_constant<int, 4>{}); one(std::integral_constant<int, 5>{});
    one(std::integral_constant<int, 6>{}); one(std::integral_constant<int, 7>{});
  };

  constexpr int LOADS = SPLIT * (QA + QB);     // vector loads per thread per slab

  // MFMAs of one k-step on one accumulator tile.
  auto mfma_tile = [&](const u32x4_t* fa, const u32x4_t* fb, int i, int j) {
    if constexpr (sizeof(T) == 2) {
      bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fa[0]);
      bf16x8_t bh = __builtin_bit_cast(bf16x8_t, fb[0]);
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[i][j], 0, 0, 0);
      if constexpr (SPLIT == 2) {
        bf16x8_t al = __builtin_bit_cast(bf16x8_t, fa[TI]);
        bf16x8_t bl = __builtin_bit_cast(bf16x8_t, fb[TJ]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[i][j], 0, 0, 0);
      }
    } else {
      f32x4_t av = __builtin_bit_cast(f32x4_t, fa[0]);
      f32x4_t bv = __builtin_bit_cast(f32x4_t, fb[0]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int s = 0; s < NSTG - 1; ++s)
    if (s < nslab) issue(s);

  for (int s = 0; s < nslab; ++s) {
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
    if (s + NSTG - 1 < nslab) issue(s + NSTG - 1);

    const int stg = s % NSTG;
    // fragments [kk][split * TI + i] (A) and [kk][split * TJ + j] (B)
    auto read_frags = [&](u32x4_t (&fa)[SPLIT * TI], u32x4_t (&fb)[SPLIT * TJ], int kk) {
#pragma unroll
      for (int sp = 0; sp < SPLIT; ++sp) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
          fa[sp * TI + i] =
              *reinterpret_cast<const u32x4_t*>(a_tile(stg, sp) + fa_off[kk] + i * 16 * RB);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          fb[sp * TJ + j] =
              *reinterpret_cast<const u32x4_t*>(b_tile(stg, sp) + fb_off[kk] + j * 16 * RB);
      }
    };
    // every fragment read of the slab ahead of the MFMAs, so the waits
    // before them count down outstanding reads instead of draining them
    u32x4_t fa[NKK][SPLIT * TI], fb[NKK][SPLIT * TJ];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) read_frags(fa[kk], fb[kk], kk);
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
      if (!ax_user && s * BK < ax_k0 + 16 * ax_nu && ax_k0 < (s + 1) * BK) add_ax(s, stg);
    }
  }

  // ---- epilogue.  acc[i][j][r] holds C(row, col) with
  //   row = m0 + wm*WTM + i*16 + 4*(lane/16) + r,  col = n0 + wn*WTN + j*16 + lane%16
  // i.e. the 4 registers of a tile are 4 consecutive rows of one column.
  const int idx = g.idx0 + mi * g.idx_stride;
  const float cs = A.scal ? A.scal[idx] : 1.0f;
  const int rows = g.rows, cols = g.cols;
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t Mp = round_up(rows, kPad);
  const int64_t Np = round_up(cols, kPad);
  const int64_t Rp = round_up(rows < cols ? rows : cols, kPad);
  const int rbase = m0 + wm * WTM + 4 * (lane >> 4);
  const int cbase = n0 + wn * WTN + (lane & 15);
  // every wave is done reading the operand stages: LDS is free for staging
  __syncthreads();

  if constexpr (EPI == E_RAW) {
    stage_store_tile<float, 1, BMT, BNT, TI, TJ, NT>(acc, smem, A.o_raw + roff, nullptr, Rp, m0,
                                                     n0, (int)Rp, wm, wn, lane, tid);
    if (tm != tn) store_mirror<float, 1, TI, TJ>(acc, A.o_raw, nullptr, roff, Rp, rbase, cbase);
  } else if constexpr (EPI == E_OP) {
    const float m = A.mul * (A.scal_pow == 2 ? cs * cs : 1.0f);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] *= m;
    stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o_hi, roff),
                                                     offset_ptr<T>(A.o_lo, roff), Rp, m0, n0,
                                                     (int)Rp, wm, wn, lane, tid);
    if (tm != tn) store_mirror<T, SPLIT, TI, TJ>(acc, A.o_hi, A.o_lo, roff, Rp, rbase, cbase);
  } else if constexpr (EPI == E_SQUARE) {
    // b A + c A^2; A is symmetric, so A(row..row+3, col) = A(col, row..row+3)
    // (combined tile by tile, so that the loaded values and the accumulator
    // never have to be held in registers side by side)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        float x[4];
        load_op4<T, SPLIT>(A.sq_hi, A.sq_lo, roff + (int64_t)(cbase + j * 16) * Rp + rbase + i * 16,
                           x);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = A.cb * x[r] + A.cc * acc[i][j][r];
      }
    stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o_hi, roff),
                                                     offset_ptr<T>(A.o_lo, roff), Rp, m0, n0,
                                                     (int)Rp, wm, wn, lane, tid);
    if (tm != tn) store_mirror<T, SPLIT, TI, TJ>(acc, A.o_hi, A.o_lo, roff, Rp, rbase, cbase);
  } else {
    // E_UPDATE:  acc = a X + B X (first step: X = the unscaled source), and
    // the iterate is c^p * acc with c = 1/(s+eps) on the first step.
    const float gam = A.scal_pow == 1 ? cs : 1.0f;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] *= gam;

    if (A.out == O_X) {
      // X^T rows directly (4 consecutive entries per tile), X rows via LDS
#pragma unroll
      for (int i = 0; i < TI; ++i)
        if (rbase + i * 16 < Mp) {
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            store_acc4<T, SPLIT>(A.ot_hi, A.ot_lo,
                                 xoff + (int64_t)(cbase + j * 16) * Mp + rbase + i * 16, acc[i][j]);
        }
      stage_store_tile<T, SPLIT, BMT, BNT, TI, TJ, NT>(acc, smem, offset_ptr<T>(A.o_hi, xoff),
                                                       offset_ptr<T>(A.o_lo, xoff), Np, m0, n0,
                                                       (int)Mp, wm, wn, lane, tid);
    } else if (A.out == O_U || A.out == O_APPLY) {
      if (A.out == O_APPLY && A.status && A.status[0] != 0) return;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r, col = cbase + j * 16;
            if (row < rows && col < cols) {
              const int64_t e = eoff + (int64_t)row * cols + col;
              if (A.out == O_U) A.U[e] = acc[i][j][r];
              else apply_one(A.W, A.w_bf16, e, A.eta, acc[i][j][r]);
            }
          }
    } else {
      // O_BITS: entrywise sign packed into 32-bit words (cols % 32 == 0).
      // For a 16x16 MFMA tile and accumulator register r, a wave ballot
      // gives 4 rows x 16 columns; two neighbouring tiles give 32 columns.
      const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int jp = 0; jp < TJ / 2; ++jp)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint64_t m0b = __ballot(acc[i][2 * jp][r] < 0.0f);
            uint64_t m1b = __ballot(acc[i][2 * jp + 1][r] < 0.0f);
            if (lane < 4) {
              uint32_t w = (uint32_t)((m0b >> (16 * lane)) & 0xFFFFu) |
                           ((uint32_t)((m1b >> (16 * lane)) & 0xFFFFu) << 16);
              int wrow = m0 + wm * WTM + i * 16 + 4 * lane + r;
              int wcol = n0 + wn * WTN + jp * 32;
              if (wrow < rows && wcol < cols)
                A.bits[woff + ((int64_t)wrow * cols + wcol) / 32] = w;
            }
          }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------
// Launch configuration: 128x128 tiles, 4 waves of 64x64, two stages of
// 128-byte slab rows (64 KB of LDS), so two blocks share a CU and one
// block's pipeline fill and epilogue overlap the other's k-loop.  (Measured
// on the Newton-Schulz shapes, where the outputs are only 768 wide: 64-byte
// slab rows with four blocks per CU, and 256x256 tiles with 4 waves of
// 128x128 or 8 waves of 64x128 and one block per CU, were all slower; the
// large tiles leave too few blocks per launch and expose each block's fill
// and epilogue.)
template <typename T, int SPLIT, int EPI>
struct Cfg {
  static constexpr int WM = 2;
  static constexpr int TI = 4, TJ = 4;
  static constexpr int RB = 128;
  static constexpr int NSTG = 2;
  static constexpr int WPE = 2;
  static constexpr int BMT = WM * 16 * TI, BNT = 32 * TJ;
  static constexpr size_t lds() {
    size_t pipe = (size_t)NSTG * SPLIT * (BMT + BNT) * RB;
    size_t img = (size_t)SPLIT * BMT * (BNT * sizeof(T) + 16);
    size_t raw = (size_t)BMT * (BNT * sizeof(float) + 16);  // raw Gram is float32
    size_t m = pipe > img ? pipe : img;
    return EPI == E_RAW && m < raw ? raw : m;
  }
};
constexpr int kTile = Cfg<bf16_t, 1, E_UPDATE>::BMT;
static_assert(Cfg<bf16_t, 1, E_UPDATE>::BNT == kTile, "square tile");

int gemm_tile(int /*precision*/, int /*epi*/, int64_t /*gm*/, int64_t /*gn*/) { return kTile; }

template <typename T, int SPLIT, int EPI>
static hipError_t launch_one(const GemmArgs& args, hipStream_t s) {
  using C = Cfg<T, SPLIT, EPI>;
  hipLaunchKernelGGL((k_gemm<T, SPLIT, EPI, C::NSTG, C::WM, C::TI, C::TJ, C::RB, C::WPE>),
                     dim3(args.G.total_blocks), dim3(128 * C::WM), C::lds(), s, args);
  return hipGetLastError();
}

template <typename T, int SPLIT>
static hipError_t launch_epi(const GemmArgs& args, hipStream_t s) {
  switch (args.epi) {
    case E_RAW: return launch_one<T, SPLIT, E_RAW>(args, s);
    case E_OP: return launch_one<T, SPLIT, E_OP>(args, s);
    case E_SQUARE: return launch_one<T, SPLIT, E_SQUARE>(args, s);
    default: return launch_one<T, SPLIT, E_UPDATE>(args, s);
  }
}

hipError_t launch_gemm(int precision, const GemmArgs& args, hipStream_t s) {
  if (args.G.total_blocks <= 0) return hipSuccess;
  for (int i = 0; i < args.G.n; ++i)
    if (args.G.g[i].tile != kTile || args.G.g[i].gk % 128) return hipErrorInvalidValue;
  if (precision == P_F32) return launch_epi<float, 1>(args, s);
  if (precision == P_BF16X3) return launch_epi<bf16_t, 2>(args, s);
  return launch_epi<bf16_t, 1>(args, s);
}

template <typename T, int SPLIT, int EPI>
static hipError_t set_lds() {
  using C = Cfg<T, SPLIT, EPI>;
  return hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<T, SPLIT, EPI, C::NSTG, C::WM, C::TI, C::TJ, C::RB, C::WPE>),
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
  return set_lds_all<float, 1>();
}

}  // namespace sm
