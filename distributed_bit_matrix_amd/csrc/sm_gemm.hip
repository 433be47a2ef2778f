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
#include "sm_internal.h"
#include "sm_launch.h"

namespace sm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 128;          // block tile (both dims)
constexpr int ROWB = 128;        // bytes per LDS row (one k-slab)
constexpr int TILEB = BM * ROWB; // bytes per operand tile per stage

#ifndef SM_GEMM_STAGES
#define SM_GEMM_STAGES 2
#endif

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
}

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

// Store a BMT x 128 output tile (values in accumulator layout) row-major at
// dst (row length ld) through LDS: each wave writes its 64x64 sub-tile into
// an LDS image of the tile, then every thread stores 16-byte row segments
// (rows at or past row_lim are skipped).  For split-bf16 the hi and lo
// images sit side by side.  The LDS row pitch is padded by 16 bytes
// against bank conflicts.
template <typename T, int SPLIT, int BMT, int NT>
__device__ __forceinline__ void stage_store_tile(const float (&v)[4][4][4], char* smem,
                                                 void* dst_hi, void* dst_lo, int64_t ld,
                                                 int m0, int n0, int row_lim, int wm, int wn,
                                                 int lane, int tid) {
  constexpr int ES = sizeof(T);
  constexpr int PITCH = BM * ES + 16;
  constexpr int IMG = BMT * PITCH;
  const int r0 = wm * 64 + 4 * (lane >> 4), c0 = wn * 64 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
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
  constexpr int CH = BM * ES / 16;          // 16-byte chunks per row
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

// Mirror tile of a symmetric output: C(row..row+3, col) goes to row `col`,
// columns row..row+3 (one 8- or 16-byte store per accumulator tile).
template <typename T, int SPLIT>
__device__ __forceinline__ void store_mirror(const float (&v)[4][4][4], void* hi, void* lo,
                                             int64_t off, int64_t ld, int rbase, int cbase) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_op4<T, SPLIT>(hi, lo, off + (int64_t)(cbase + j * 16) * ld + rbase + i * 16, v[i][j]);
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <typename T, int SPLIT, int EPI, int NSTG, int WM>
__global__ __launch_bounds__(128 * WM) void k_gemm(GemmArgs A) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // Block tile BMT x 128 with WM x 2 waves of 64x64.
  constexpr int BMT = 64 * WM;
  constexpr int NW = 2 * WM, NT = 64 * NW;
  constexpr int QB = 16 / NW;                 // B-operand loads per wave
  constexpr int ATILE = BMT * ROWB;           // A-operand bytes per split
  constexpr int STAGEB = SPLIT * (ATILE + TILEB);
  constexpr int P = Elem<T>::per16;           // elements per 16 bytes
  constexpr int BK = ROWB / sizeof(T);        // k per slab
  constexpr int LOADS = SPLIT * (4 + QB);     // vector loads per thread per slab
  static_assert(EPI == E_UPDATE || WM == 2, "symmetric outputs use square tiles");

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
  int tm, tn;
  if constexpr (SYM) {
    tm = 0;
    int rem = t;
    while (rem >= g.tiles_n - tm) { rem -= g.tiles_n - tm; ++tm; }
    tn = tm + rem;
  } else {
    tm = t / g.tiles_n;
    tn = t - tm * g.tiles_n;
  }
  const int m0 = tm * BMT, n0 = tn * BM;
  const int a_fam = g.ops & 3, b_fam = (g.ops >> 2) & 3;
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
  // of wave w fills LDS rows (4w+q)*8 .. +7 (B: (QB w+q)*8 ..); lane l writes
  // row ..+l/8 at chunk position l%8, so it fetches global chunk
  // (l%8) ^ swz(row).  A rows past the operand (a ragged last BMT-row tile)
  // read the last row instead; their results are never stored.
  int64_t aoff[4], boff[QB];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int row = (wave * 4 + q) * 8 + (lane >> 3);
    int ch = (lane & 7) ^ swz(row);
    int arow = m0 + row < g.gm ? m0 + row : g.gm - 1;
    aoff[q] = (int64_t)arow * lda + ch * P;
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    int row = (wave * QB + q) * 8 + (lane >> 3);
    int ch = (lane & 7) ^ swz(row);
    boff[q] = (int64_t)(n0 + row) * ldb + ch * P;
  }
  // Per-lane LDS offsets of the fragment reads: row within the tile and
  // 16-byte chunk (kk*4 + lane/16) of the 128-byte slab row.
  int fa_off[2][4], fb_off[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa_off[kk][i] = lds_off(wm * 64 + i * 16 + (lane & 15), kk * 4 + (lane >> 4));
      fb_off[kk][i] = lds_off(wn * 64 + i * 16 + (lane & 15), kk * 4 + (lane >> 4));
    }

  const int nslab = g.gk / BK;

  // LDS stage: [A split 0][A split 1..][B split 0][B split 1..]
  auto a_tile = [&](int st, int sp) -> char* { return smem + st * STAGEB + sp * ATILE; };
  auto b_tile = [&](int st, int sp) -> char* {
    return smem + st * STAGEB + SPLIT * ATILE + sp * TILEB;
  };
  auto issue = [&](int s) {
    const int st = s % NSTG;
    const int64_t k0 = (int64_t)s * BK;
#pragma unroll
    for (int sp = 0; sp < SPLIT; ++sp) {
      char* ta = a_tile(st, sp) + wave * 4096;
      char* tb = b_tile(st, sp) + wave * QB * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(a_src[sp] + aoff[q] + k0),
                                         (lds_void*)(ta + q * 1024), 16, 0, 0);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(b_src[sp] + boff[q] + k0),
                                         (lds_void*)(tb + q * 1024), 16, 0, 0);
    }
  };

  f32x4_t acc[4][4];
  if constexpr (EPI == E_UPDATE) {
    // a X + B X: start the accumulator at a * X so that its loads overlap
    // the k-loop.  X comes from the caller's float32 array (first step) or
    // from X^T (4 consecutive rows of a column are 4 consecutive entries).
    const int rb = m0 + wm * 64 + 4 * (lane >> 4), cb = n0 + wn * 64 + (lane & 15);
    const int64_t xo = g.x0 + (int64_t)mi * g.x_stride;
    const int64_t eo = g.elem0 + (int64_t)mi * g.elem_stride;
    const int64_t mp = round_up(g.rows, kPad);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x[4];
        if (A.xsrc == XS_USER) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb + i * 16 + r, col = cb + j * 16;
            x[r] = (row < g.rows && col < g.cols)
                       ? A.xs_user[eo + (int64_t)row * g.cols + col] : 0.0f;
          }
        } else if (rb + i * 16 < mp) {
          load_op4<T, SPLIT>(A.xs_hi, A.xs_lo, xo + (int64_t)(cb + j * 16) * mp + rb + i * 16, x);
        } else {
          x[0] = x[1] = x[2] = x[3] = 0.0f;
        }
        acc[i][j] = f32x4_t{A.ca * x[0], A.ca * x[1], A.ca * x[2], A.ca * x[3]};
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

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
    u32x4_t fa[2][SPLIT][4], fb[2][SPLIT][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int sp = 0; sp < SPLIT; ++sp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[kk][sp][i] = *reinterpret_cast<const u32x4_t*>(a_tile(stg, sp) + fa_off[kk][i]);
          fb[kk][sp][i] = *reinterpret_cast<const u32x4_t*>(b_tile(stg, sp) + fb_off[kk][i]);
        }
    // keep every fragment read of the slab ahead of the MFMAs, so the waits
    // before them count down outstanding reads instead of draining them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (sizeof(T) == 2) {
            bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fa[kk][0][i]);
            bf16x8_t bh = __builtin_bit_cast(bf16x8_t, fb[kk][0][j]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[i][j], 0, 0, 0);
            if constexpr (SPLIT == 2) {
              bf16x8_t al = __builtin_bit_cast(bf16x8_t, fa[kk][1][i]);
              bf16x8_t bl = __builtin_bit_cast(bf16x8_t, fb[kk][1][j]);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[i][j], 0, 0, 0);
            }
          } else {
            f32x4_t av = __builtin_bit_cast(f32x4_t, fa[kk][0][i]);
            f32x4_t bv = __builtin_bit_cast(f32x4_t, fb[kk][0][j]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[i][j], 0, 0, 0);
          }
        }
  }

  // ---- epilogue.  acc[i][j][r] holds C(row, col) with
  //   row = m0 + wm*64 + i*16 + 4*(lane/16) + r,  col = n0 + wn*64 + j*16 + lane%16
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
  const int rbase = m0 + wm * 64 + 4 * (lane >> 4);
  const int cbase = n0 + wn * 64 + (lane & 15);
  // every wave is done reading the operand stages: LDS is free for staging
  __syncthreads();

  float v[4][4][4];
  if constexpr (EPI == E_RAW) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][j][r] = acc[i][j][r];
    stage_store_tile<float, 1, BMT, NT>(v, smem, A.o_raw + roff, nullptr, Rp, m0, n0, (int)Rp, wm, wn, lane, tid);
    if (tm != tn) store_mirror<float, 1>(v, A.o_raw, nullptr, roff, Rp, rbase, cbase);
  } else if constexpr (EPI == E_OP) {
    const float m = A.mul * (A.scal_pow == 2 ? cs * cs : 1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][j][r] = m * acc[i][j][r];
    stage_store_tile<T, SPLIT, BMT, NT>(v, smem, offset_ptr<T>(A.o_hi, roff),
                                        offset_ptr<T>(A.o_lo, roff), Rp, m0, n0, (int)Rp, wm,
                                        wn, lane, tid);
    if (tm != tn) store_mirror<T, SPLIT>(v, A.o_hi, A.o_lo, roff, Rp, rbase, cbase);
  } else if constexpr (EPI == E_SQUARE) {
    // b A + c A^2; A is symmetric, so A(row..row+3, col) = A(col, row..row+3)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        load_op4<T, SPLIT>(A.sq_hi, A.sq_lo, roff + (int64_t)(cbase + j * 16) * Rp + rbase + i * 16,
                           v[i][j]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][j][r] = A.cb * v[i][j][r] + A.cc * acc[i][j][r];
    stage_store_tile<T, SPLIT, BMT, NT>(v, smem, offset_ptr<T>(A.o_hi, roff),
                                        offset_ptr<T>(A.o_lo, roff), Rp, m0, n0, (int)Rp, wm,
                                        wn, lane, tid);
    if (tm != tn) store_mirror<T, SPLIT>(v, A.o_hi, A.o_lo, roff, Rp, rbase, cbase);
  } else {
    // E_UPDATE:  acc = a X + B X (first step: X = the unscaled source), and
    // the iterate is c^p * acc with c = 1/(s+eps) on the first step.
    const float gam = A.scal_pow == 1 ? cs : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][j][r] = gam * acc[i][j][r];

    if (A.out == O_X) {
      // X^T rows directly (4 consecutive entries per tile), X rows via LDS
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (rbase + i * 16 < Mp) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_op4<T, SPLIT>(A.ot_hi, A.ot_lo,
                                xoff + (int64_t)(cbase + j * 16) * Mp + rbase + i * 16, v[i][j]);
        }
      stage_store_tile<T, SPLIT, BMT, NT>(v, smem, offset_ptr<T>(A.o_hi, xoff),
                                          offset_ptr<T>(A.o_lo, xoff), Np, m0, n0, (int)Mp, wm,
                                          wn, lane, tid);
    } else if (A.out == O_U || A.out == O_APPLY) {
      if (A.out == O_APPLY && A.status && A.status[0] != 0) return;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rbase + i * 16 + r, col = cbase + j * 16;
            if (row < rows && col < cols) {
              const int64_t e = eoff + (int64_t)row * cols + col;
              if (A.out == O_U) A.U[e] = v[i][j][r];
              else apply_one(A.W, A.w_bf16, e, A.eta, v[i][j][r]);
            }
          }
    } else {
      // O_BITS: entrywise sign packed into 32-bit words (cols % 32 == 0).
      // For a 16x16 MFMA tile and accumulator register r, a wave ballot
      // gives 4 rows x 16 columns; two neighbouring tiles give 32 columns.
      const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jp = 0; jp < 2; ++jp)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint64_t m0b = __ballot(v[i][2 * jp][r] < 0.0f);
            uint64_t m1b = __ballot(v[i][2 * jp + 1][r] < 0.0f);
            if (lane < 4) {
              uint32_t w = (uint32_t)((m0b >> (16 * lane)) & 0xFFFFu) |
                           ((uint32_t)((m1b >> (16 * lane)) & 0xFFFFu) << 16);
              int wrow = m0 + wm * 64 + i * 16 + 4 * lane + r;
              int wcol = n0 + wn * 64 + jp * 32;
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
// Launch configuration: 128x128 tiles, 4 waves, two stages, which lets two
// blocks share a CU so one block's pipeline fill and epilogue overlap the
// other's k-loop.  (The kernel also supports 256x128 tiles with 8 waves and
// three stages; on the Newton-Schulz shapes that measured slower, since one
// block per CU leaves those phases exposed.)
template <typename T, int SPLIT, int EPI>
struct Cfg {
  static constexpr int WM = 2;
  static constexpr int NSTG = 2;
  static constexpr int BMT = 64 * WM;
  static constexpr size_t lds() {
    size_t pipe = (size_t)NSTG * SPLIT * (BMT * ROWB + TILEB);
    size_t img = (size_t)SPLIT * BMT * (BM * sizeof(T) + 16);
    size_t raw = (size_t)BMT * (BM * sizeof(float) + 16);  // raw Gram is float32
    size_t m = pipe > img ? pipe : img;
    return m > raw ? m : raw;
  }
};

int gemm_update_tile_rows(int precision) {
  return precision == P_BF16X3 ? Cfg<bf16_t, 2, E_UPDATE>::BMT
                               : Cfg<bf16_t, 1, E_UPDATE>::BMT;
}

template <typename T, int SPLIT, int EPI>
static hipError_t launch_one(const GemmArgs& args, hipStream_t s) {
  using C = Cfg<T, SPLIT, EPI>;
  hipLaunchKernelGGL((k_gemm<T, SPLIT, EPI, C::NSTG, C::WM>), dim3(args.G.total_blocks),
                     dim3(128 * C::WM), C::lds(), s, args);
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
  if (precision == P_F32) return launch_epi<float, 1>(args, s);
  if (precision == P_BF16X3) return launch_epi<bf16_t, 2>(args, s);
  return launch_epi<bf16_t, 1>(args, s);
}

template <typename T, int SPLIT, int EPI>
static hipError_t set_lds() {
  using C = Cfg<T, SPLIT, EPI>;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<T, SPLIT, EPI, C::NSTG, C::WM>),
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
