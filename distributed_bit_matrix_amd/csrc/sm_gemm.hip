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
// Operands are staged through LDS in a [mn][k] layout (k contiguous) with
// 128-byte rows and an XOR swizzle of 16-byte chunks; operands whose k axis
// is strided in memory are transposed in registers on the way in (4 k-rows
// per thread, written as 8- or 16-byte k-vectors).  Two LDS stages: the
// next k-slab is fetched into registers while the current one is consumed.
// All operand copies are zero padded to multiples of 128, so no loads are
// predicated and padding contributes exact zeros.
#include "sm_internal.h"
#include "sm_launch.h"

namespace sm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = 128;          // block tile (both dims)
constexpr int ROWB = 128;        // bytes per LDS row (one k-slab)
constexpr int TILEB = BM * ROWB; // bytes per operand tile per stage

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int per16 = 8; };
template <> struct Elem<float>  { static constexpr int per16 = 4; };

// Per-matrix pointer offset of an operand family.
__device__ __forceinline__ int64_t fam_off(const Group& g, int fam, int mi) {
  return fam == FAM_X ? g.x0 + (int64_t)mi * g.x_stride
                      : g.r0 + (int64_t)mi * g.r_stride;
}
__device__ __forceinline__ int64_t fam_ld(const Group& g, int fam) {
  return fam == FAM_X ? round_up(g.cols, kPad)
                      : round_up(g.rows < g.cols ? g.rows : g.cols, kPad);
}

// Fetch of one operand slab (128 mn x 128 bytes of k) into registers.
// K-contiguous: 4 chunks of 16 bytes per thread (8 threads per row).
// MN-contiguous: one 4(k) x (16 bytes of mn) patch per thread.
template <typename T>
struct SlabRegs { u32x4_t v[4]; };

template <typename T>
__device__ __forceinline__ void fetch_slab(SlabRegs<T>& R, const T* base,
                                           int64_t ld, int kc, int mn0,
                                           int k0, int tid) {
  constexpr int P = Elem<T>::per16;           // elements per 16 bytes
  constexpr int BK = ROWB / sizeof(T);        // k per slab
  if (kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = tid + 256 * q;
      int row = c >> 3, ch = c & 7;
      const T* p = base + (int64_t)(mn0 + row) * ld + k0 + ch * P;
      R.v[q] = *reinterpret_cast<const u32x4_t*>(p);
    }
  } else {
    constexpr int NQ = BM / P;               // patches along mn (16 or 32)
    int mnq = tid % NQ, kq = tid / NQ;       // kq < BK/4
    (void)BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const T* p = base + (int64_t)(k0 + 4 * kq + q) * ld + mn0 + mnq * P;
      R.v[q] = *reinterpret_cast<const u32x4_t*>(p);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_slab(const SlabRegs<T>& R, char* lds,
                                           int kc, int tid) {
  if (kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = tid + 256 * q;
      int row = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(row, ch)) = R.v[q];
    }
  } else if constexpr (sizeof(T) == 2) {
    // patch: 4 k-rows x 8 mn; emit 8 k-vectors of 4 bf16 (8 bytes)
    int mnq = tid % 16, kq = tid / 16;       // kq in [0,16)
    int ch = kq >> 1, half = kq & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int w = e >> 1;
      uint32_t a0 = R.v[0][w], a1 = R.v[1][w], a2 = R.v[2][w], a3 = R.v[3][w];
      u32x2_t o;
      if (e & 1) {
        o[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
        o[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
      } else {
        o[0] = (a0 & 0xFFFFu) | (a1 << 16);
        o[1] = (a2 & 0xFFFFu) | (a3 << 16);
      }
      int row = mnq * 8 + e;
      *reinterpret_cast<u32x2_t*>(lds + lds_off(row, ch) + half * 8) = o;
    }
  } else {
    // patch: 4 k-rows x 4 mn floats; emit 4 k-vectors of 4 floats
    int mnq = tid % 32, kq = tid / 32;       // kq in [0,8)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4_t o;
      o[0] = R.v[0][e]; o[1] = R.v[1][e]; o[2] = R.v[2][e]; o[3] = R.v[3][e];
      int row = mnq * 4 + e;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(row, kq)) = o;
    }
  }
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

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <typename T, int SPLIT>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs A) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // smem layout: [stage 2][operand 2][split SPLIT][TILEB]
  auto tile = [&](int st, int op, int sp) -> char* {
    return smem + ((st * 2 + op) * SPLIT + sp) * TILEB;
  };

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
  const int tm = t / g.tiles_n, tn = t - tm * g.tiles_n;
  const int m0 = tm * BM, n0 = tn * BM;
  const int a_fam = g.ops & 1, a_kc = (g.ops >> 1) & 1;
  const int b_fam = (g.ops >> 2) & 1, b_kc = (g.ops >> 3) & 1;
  const int64_t a_off = fam_off(g, a_fam, mi), b_off = fam_off(g, b_fam, mi);
  const int64_t lda = fam_ld(g, a_fam), ldb = fam_ld(g, b_fam);
  const T* a_hi = reinterpret_cast<const T*>(a_fam == FAM_X ? A.x_hi : A.r_hi) + a_off;
  const T* b_hi = reinterpret_cast<const T*>(b_fam == FAM_X ? A.x_hi : A.r_hi) + b_off;
  const T* a_lo = SPLIT == 2
      ? reinterpret_cast<const T*>(a_fam == FAM_X ? A.x_lo : A.r_lo) + a_off : nullptr;
  const T* b_lo = SPLIT == 2
      ? reinterpret_cast<const T*>(b_fam == FAM_X ? A.x_lo : A.r_lo) + b_off : nullptr;

  constexpr int BK = ROWB / sizeof(T);
  const int nslab = g.gk / BK;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  SlabRegs<T> ra[SPLIT], rb[SPLIT];
  auto fetch = [&](int s) {
    int k0 = s * BK;
    fetch_slab<T>(ra[0], a_hi, lda, a_kc, m0, k0, tid);
    fetch_slab<T>(rb[0], b_hi, ldb, b_kc, n0, k0, tid);
    if constexpr (SPLIT == 2) {
      fetch_slab<T>(ra[1], a_lo, lda, a_kc, m0, k0, tid);
      fetch_slab<T>(rb[1], b_lo, ldb, b_kc, n0, k0, tid);
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int sp = 0; sp < SPLIT; ++sp) {
      store_slab<T>(ra[sp], tile(st, 0, sp), a_kc, tid);
      store_slab<T>(rb[sp], tile(st, 1, sp), b_kc, tid);
    }
  };

  if (nslab > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();

  for (int s = 0; s < nslab; ++s) {
    const int st = s & 1;
    if (s + 1 < nslab) fetch(s + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      u32x4_t fa[SPLIT][4], fb[SPLIT][4];
#pragma unroll
      for (int sp = 0; sp < SPLIT; ++sp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int ra_ = wm * 64 + i * 16 + (lane & 15);
          int rb_ = wn * 64 + i * 16 + (lane & 15);
          fa[sp][i] = *reinterpret_cast<const u32x4_t*>(tile(st, 0, sp) + lds_off(ra_, ch));
          fb[sp][i] = *reinterpret_cast<const u32x4_t*>(tile(st, 1, sp) + lds_off(rb_, ch));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (sizeof(T) == 2) {
            bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fa[0][i]);
            bf16x8_t bh = __builtin_bit_cast(bf16x8_t, fb[0][j]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[i][j], 0, 0, 0);
            if constexpr (SPLIT == 2) {
              bf16x8_t al = __builtin_bit_cast(bf16x8_t, fa[1][i]);
              bf16x8_t bl = __builtin_bit_cast(bf16x8_t, fb[1][j]);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[i][j], 0, 0, 0);
            }
          } else {
            f32x4_t av = __builtin_bit_cast(f32x4_t, fa[0][i]);
            f32x4_t bv = __builtin_bit_cast(f32x4_t, fb[0][j]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[i][j], 0, 0, 0);
          }
        }
    }
    if (s + 1 < nslab) stash(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  acc[i][j][r] holds C(row, col) with
  //   row = m0 + wm*64 + i*16 + 4*(lane/16) + r,  col = n0 + wn*64 + j*16 + lane%16
  const int idx = g.idx0 + mi * g.idx_stride;
  const float cs = A.scal ? A.scal[idx] : 1.0f;
  const int rows = g.rows, cols = g.cols;
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t Np = round_up(cols, kPad);
  const int64_t Rp = round_up(rows < cols ? rows : cols, kPad);
  const int rbase = m0 + wm * 64 + 4 * (lane >> 4);
  const int cbase = n0 + wn * 64 + (lane & 15);

  if (A.epi == E_RAW) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = rbase + i * 16 + r, col = cbase + j * 16;
          A.o_raw[roff + (int64_t)row * Rp + col] = acc[i][j][r];
        }
    return;
  }
  if (A.epi == E_OP) {
    float m = A.mul * (A.scal_pow == 2 ? cs * cs : 1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = rbase + i * 16 + r, col = cbase + j * 16;
          store_op<T, SPLIT>(A.o_hi, A.o_lo, roff + (int64_t)row * Rp + col,
                             m * acc[i][j][r]);
        }
    return;
  }
  if (A.epi == E_SQUARE) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = rbase + i * 16 + r, col = cbase + j * 16;
          int64_t o = roff + (int64_t)row * Rp + col;
          float a = load_op<T, SPLIT>(A.sq_hi, A.sq_lo, o);
          store_op<T, SPLIT>(A.o_hi, A.o_lo, o, A.cb * a + A.cc * acc[i][j][r]);
        }
    return;
  }

  // E_UPDATE:  v = (ca * c^p) * Xsrc + (c^p) * acc
  const float gam = A.scal_pow == 1 ? cs : 1.0f;
  const float alp = A.ca * gam;
  auto xsrc = [&](int row, int col) -> float {
    if (A.xsrc == XS_USER)
      return (row < rows && col < cols) ? A.xs_user[eoff + (int64_t)row * cols + col] : 0.0f;
    return load_op<T, SPLIT>(A.xs_hi, A.xs_lo, xoff + (int64_t)row * Np + col);
  };

  if (A.out == O_X) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = rbase + i * 16 + r, col = cbase + j * 16;
          float v = alp * xsrc(row, col) + gam * acc[i][j][r];
          store_op<T, SPLIT>(A.o_hi, A.o_lo, xoff + (int64_t)row * Np + col, v);
        }
    return;
  }
  if (A.out == O_U || A.out == O_APPLY) {
    if (A.out == O_APPLY && A.status && A.status[0] != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = rbase + i * 16 + r, col = cbase + j * 16;
          if (row < rows && col < cols) {
            float v = alp * xsrc(row, col) + gam * acc[i][j][r];
            int64_t e = eoff + (int64_t)row * cols + col;
            if (A.out == O_U) A.U[e] = v;
            else apply_one(A.W, A.w_bf16, e, A.eta, v);
          }
        }
    return;
  }
  // O_BITS: entrywise sign packed into 32-bit words (cols % 32 == 0).
  // For a 16x16 MFMA tile and accumulator register r, a wave ballot gives
  // 4 rows x 16 columns; two neighbouring tiles give 32 columns of a row.
  const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = rbase + i * 16 + r;
        int c0 = cbase + (2 * jp) * 16, c1 = c0 + 16;
        float v0 = alp * xsrc(row, c0) + gam * acc[i][2 * jp][r];
        float v1 = alp * xsrc(row, c1) + gam * acc[i][2 * jp + 1][r];
        uint64_t m0b = __ballot(v0 < 0.0f);
        uint64_t m1b = __ballot(v1 < 0.0f);
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

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------
hipError_t launch_gemm(int precision, const GemmArgs& args, hipStream_t s) {
  if (args.G.total_blocks <= 0) return hipSuccess;
  dim3 grid(args.G.total_blocks), block(256);
  if (precision == P_F32) {
    size_t lds = 2 * 2 * 1 * TILEB;
    hipLaunchKernelGGL((k_gemm<float, 1>), grid, block, lds, s, args);
  } else if (precision == P_BF16X3) {
    size_t lds = 2 * 2 * 2 * TILEB;
    hipLaunchKernelGGL((k_gemm<bf16_t, 2>), grid, block, lds, s, args);
  } else {
    size_t lds = 2 * 2 * 1 * TILEB;
    hipLaunchKernelGGL((k_gemm<bf16_t, 1>), grid, block, lds, s, args);
  }
  return hipGetLastError();
}

hipError_t gemm_set_attributes() {
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<bf16_t, 2>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 2 * 2 * 2 * TILEB);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<bf16_t, 1>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 2 * 2 * TILEB);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<float, 1>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 2 * 2 * TILEB);
}

}  // namespace sm
