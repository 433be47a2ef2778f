// HBM-bound passes of the Sign-Muon step: momentum EMA (Algorithm 1/2
// momentum lines), entrywise sign with 1-bit packing (section 3; section 6
// packing), majority vote over M packed worker buffers (Algorithm 2 sum and
// threshold, blog tie rule), the update of W (Algorithm 1/2 last line), and
// the small pre-scale kernels of PolarNS (section 4: Frobenius norm or power
// iteration).  No floating-point atomics: every reduction has a fixed order.
#include <hip/hip_ext.h>

#include "sm_internal.h"
#include "sm_launch.h"

namespace sm {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
// Loads and stores of data that a pass touches once (the gradient and W in
// the sweep, the sign buffers and W in the vote) carry the non-temporal
// hint: measured on the nanoGPT set, the sweep ran 9% faster with it.
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Sum over a 256-thread block in a fixed order; result valid in every thread.
__device__ __forceinline__ float block_sum(float v) {
  __shared__ float sh[4];
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__device__ __forceinline__ void group_of_block(const Groups& G, int b, int& gi,
                                               int& mi, int& q) {
  gi = find_group(G, b);
  int lb = b - G.g[gi].block0;
  mi = lb / G.g[gi].blocks_per_mat;
  q = lb - mi * G.g[gi].blocks_per_mat;
}

__device__ __forceinline__ float load_w(const void* W, int w_bf16, int64_t i) {
  return w_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(W)[i])
                : reinterpret_cast<const float*>(W)[i];
}

// Update of one parameter entry: product and difference each rounded to
// float32 (no contraction), then nearest-even to bfloat16 for a bf16 W.
__device__ __forceinline__ float apply_value(float w, float eta, float d) {
#pragma clang fp contract(off)
  float t = eta * d;
  return w - t;
}
__device__ __forceinline__ void apply_store(void* W, int w_bf16, int64_t i,
                                            float eta, float d) {
  if (w_bf16) {
    bf16_t* w = reinterpret_cast<bf16_t*>(W);
    w[i] = f32_to_bf16(apply_value(bf16_to_f32(w[i]), eta, d));
  } else {
    float* w = reinterpret_cast<float*>(W);
    w[i] = apply_value(w[i], eta, d);
  }
}

__device__ __forceinline__ float ema(float mom, float g, float w, float beta,
                                     float lam) {
  float gt = g + lam * w;
  return beta * mom + (1.0f - beta) * gt;
}

__device__ __forceinline__ void store_opv(int precision, void* hi, void* lo,
                                          int64_t i, float v) {
  if (precision == P_F32) {
    reinterpret_cast<float*>(hi)[i] = v;
  } else if (precision == P_BF16X3) {
    bf16_t h, l;
    split_bf16(v, h, l);
    reinterpret_cast<bf16_t*>(hi)[i] = h;
    reinterpret_cast<bf16_t*>(lo)[i] = l;
  } else {
    reinterpret_cast<bf16_t*>(hi)[i] = f32_to_bf16(v);
  }
}
// 8 consecutive operand values (16-byte aligned destination).
__device__ __forceinline__ void store_op8(int precision, void* hi, void* lo,
                                          int64_t i, const float (&v)[8]) {
  if (precision == P_F32) {
    f32x4_t a{v[0], v[1], v[2], v[3]}, b{v[4], v[5], v[6], v[7]};
    reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(hi) + i)[0] = a;
    reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(hi) + i)[1] = b;
    return;
  }
  u32x4_t h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bf16_t h0, h1, l0, l1;
    if (precision == P_BF16X3) {
      split_bf16(v[2 * k], h0, l0);
      split_bf16(v[2 * k + 1], h1, l1);
    } else {
      h0 = f32_to_bf16(v[2 * k]);
      h1 = f32_to_bf16(v[2 * k + 1]);
      l0 = l1 = 0;
    }
    h[k] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[k] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(hi) + i) = h;
  if (precision == P_BF16X3)
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(lo) + i) = l;
}

// ---------------------------------------------------------------------------
// Vote counting: vertical (bit-sliced) counters.  c[k] holds bit k of the
// count of set bits (negative votes) at each of the 32 positions of a word.
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ void add_vote(uint32_t (&c)[NB], uint32_t carry) {
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    uint32_t t = c[k] & carry;
    c[k] ^= carry;
    carry = t;
  }
}
// The words of 8 workers are loaded together (a word of zeros past the
// last worker adds nothing), so that 8 loads are in flight per lane.
template <int NB>
__device__ __forceinline__ void count_votes(const uint32_t* bits, int64_t stride,
                                            int M, int64_t w, uint32_t (&c)[NB]) {
#pragma unroll
  for (int k = 0; k < NB; ++k) c[k] = 0;
  for (int m = 0; m < M; m += 8) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = m + j < M ? ld_nt(bits + (int64_t)(m + j) * stride + w) : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) add_vote<NB>(c, v[j]);
  }
}
template <int NB>
__device__ __forceinline__ int vote_sum_at(const uint32_t (&c)[NB], int M, int b) {
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) cnt |= (int)((c[k] >> b) & 1u) << k;
  return M - 2 * cnt;
}
__device__ __forceinline__ int majority(int sum, int tie) {
  return sum > 0 ? 1 : (sum < 0 ? -1 : tie);
}

// ---------------------------------------------------------------------------
// ABI: momentum over a flat array
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_momentum_flat(
    const float* __restrict__ G, const void* __restrict__ W, int w_bf16,
    float* __restrict__ Mom, int64_t n, float beta, float lam, int vec) {
  int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= n) return;
  if (vec && i0 + 4 <= n) {
    f32x4_t g = *reinterpret_cast<const f32x4_t*>(G + i0);
    f32x4_t m = *reinterpret_cast<const f32x4_t*>(Mom + i0);
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = load_w(W, w_bf16, i0 + k);
    f32x4_t o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = ema(m[k], g[k], w[k], beta, lam);
    *reinterpret_cast<f32x4_t*>(Mom + i0) = o;
    return;
  }
  for (int64_t i = i0; i < n && i < i0 + 4; ++i)
    Mom[i] = ema(Mom[i], G[i], load_w(W, w_bf16, i), beta, lam);
}

hipError_t launch_momentum_flat(const float* G, const void* W, int w_bf16,
                                float* Mom, int64_t n, float beta, float lam,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int vec = ((uintptr_t)G % 16 == 0) && ((uintptr_t)Mom % 16 == 0);
  int64_t blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(k_momentum_flat, dim3((unsigned)blocks), dim3(256), 0, s,
                     G, W, w_bf16, Mom, n, beta, lam, vec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ABI: sign + 1-bit pack of a flat array.  One element per lane; a wave
// ballot yields two 32-bit words.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sign_pack_flat(
    const float* __restrict__ U, uint32_t* __restrict__ bits, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool neg = (i < n) && (U[i < n ? i : 0] < 0.0f);
  uint64_t m = __ballot(neg);
  int lane = threadIdx.x & 63;
  int64_t w0 = (i - lane) >> 5;
  int64_t nw = (n + 31) >> 5;
  if (lane < 2 && w0 + lane < nw)
    bits[w0 + lane] = (uint32_t)(m >> (32 * lane));
}

hipError_t launch_sign_pack_flat(const float* U, uint32_t* bits, int64_t n,
                                 hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_sign_pack_flat, dim3((unsigned)blocks), dim3(256), 0, s,
                     U, bits, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ABI: majority vote over a flat segment, one thread per 32-entry word.
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void k_vote_flat(
    const uint32_t* __restrict__ bits, int64_t stride, int M, int64_t n,
    int tie, int8_t* __restrict__ D, int16_t* __restrict__ sums, int vec) {
  int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t nw = (n + 31) >> 5;
  if (w >= nw) return;
  uint32_t c[NB];
  count_votes<NB>(bits, stride, M, w, c);
  int64_t e0 = w * 32;
  if (vec && e0 + 32 <= n) {
    u32x4_t d0, d1;
    uint32_t dw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int s = vote_sum_at<NB>(c, M, 4 * k + j);
        v |= ((uint32_t)(uint8_t)(int8_t)majority(s, tie)) << (8 * j);
      }
      dw[k] = v;
    }
    d0 = u32x4_t{dw[0], dw[1], dw[2], dw[3]};
    d1 = u32x4_t{dw[4], dw[5], dw[6], dw[7]};
    reinterpret_cast<u32x4_t*>(D + e0)[0] = d0;
    reinterpret_cast<u32x4_t*>(D + e0)[1] = d1;
    if (sums) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4_t v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int s0 = vote_sum_at<NB>(c, M, 8 * k + 2 * j);
          int s1 = vote_sum_at<NB>(c, M, 8 * k + 2 * j + 1);
          v[j] = (uint32_t)(uint16_t)(int16_t)s0 | ((uint32_t)(uint16_t)(int16_t)s1 << 16);
        }
        reinterpret_cast<u32x4_t*>(sums + e0)[k] = v;
      }
    }
    return;
  }
  for (int b = 0; b < 32 && e0 + b < n; ++b) {
    int s = vote_sum_at<NB>(c, M, b);
    D[e0 + b] = (int8_t)majority(s, tie);
    if (sums) sums[e0 + b] = (int16_t)s;
  }
}

hipError_t launch_vote_flat(const uint32_t* bits, int64_t stride, int M,
                            int64_t n, int tie, int8_t* D, int16_t* sums,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t nw = (n + 31) / 32;
  dim3 grid((unsigned)((nw + 255) / 256)), block(256);
  int vec = ((uintptr_t)D % 16 == 0) && (!sums || (uintptr_t)sums % 16 == 0);
  if (M <= 15)
    hipLaunchKernelGGL(k_vote_flat<4>, grid, block, 0, s, bits, stride, M, n, tie, D, sums, vec);
  else if (M <= 255)
    hipLaunchKernelGGL(k_vote_flat<8>, grid, block, 0, s, bits, stride, M, n, tie, D, sums, vec);
  else
    hipLaunchKernelGGL(k_vote_flat<16>, grid, block, 0, s, bits, stride, M, n, tie, D, sums, vec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ABI: apply over a flat array
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_apply_flat(
    void* __restrict__ W, int w_bf16, const int8_t* __restrict__ D,
    const float* __restrict__ Df, float eta, int64_t n) {
  int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  for (int64_t i = i0; i < n && i < i0 + 4; ++i) {
    float d = D ? (float)D[i] : Df[i];
    apply_store(W, w_bf16, i, eta, d);
  }
}

hipError_t launch_apply_flat(void* W, int w_bf16, const int8_t* D,
                             const float* Df, float eta, int64_t n,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(k_apply_flat, dim3((unsigned)blocks), dim3(256), 0, s, W,
                     w_bf16, D, Df, eta, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Padded sweep over 4096-entry tiles of the padded matrix: momentum (or a plain
// float32 source) -> padded operand copy S (X, or X^T for a tall matrix,
// transposed through LDS), partial sums of squares per tile, non-finite
// flag.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_op4v(int precision, void* hi, void* lo,
                                           int64_t i, const float (&v)[4]) {
  if (precision == P_F32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(hi) + i) = f32x4_t{v[0], v[1], v[2], v[3]};
    return;
  }
  bf16_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (precision == P_BF16X3) split_bf16(v[k], h[k], l[k]);
    else { h[k] = f32_to_bf16(v[k]); l[k] = 0; }
  }
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(hi) + i) =
      u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
  if (precision == P_BF16X3)
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(lo) + i) =
        u32x2_t{(uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
}

// Write the transpose of the 64x64 tile held in LDS (rows r0.., columns
// c0.. of X) into S = X^T with row length ld.
// Eight consecutive threads write one 64-entry row of S as 8-entry pieces,
// so each store instruction covers whole rows.
__device__ __forceinline__ void write_tile_t(const float (*tile)[65], int precision,
                                             void* hi, void* lo, int64_t xoff,
                                             int64_t ld, int r0, int c0) {
  const int ch = threadIdx.x & 7;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = (threadIdx.x >> 3) + 32 * pass;   // row of S = column of the tile
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[8 * ch + e][cc];
    store_op8(precision, hi, lo, xoff + (int64_t)(c0 + cc) * ld + r0 + 8 * ch, v);
  }
}

__global__ __launch_bounds__(256) void k_sweep(SweepArgs a) {
  __shared__ float tile[64][65];
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int rows = g.rows, cols = g.cols;
  const int64_t Mp = round_up(rows, kPad), Np = round_up(cols, kPad);
  const bool tall = s_tall(g);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  // A block covers 4096 entries: a 64x64 tile when X is tall (transposed
  // through LDS), else whole 256- or 128-column stretches of 16 or 32 rows,
  // so that a wave's accesses are one or two contiguous row pieces.
  // 2^lw threads share a row of the tile.
  const int lw = tall ? 4 : (Np % 256 == 0 ? 6 : 5);
  const int rstep = 256 >> lw;                     // rows per pass
  const int tiles_c = (int)(Np >> (lw + 2));
  const int r0 = (q / tiles_c) * 4 * rstep, c0 = (q % tiles_c) << (lw + 2);
  const int lr0 = threadIdx.x >> lw, lc = (threadIdx.x & ((1 << lw) - 1)) * 4;
  const int col = c0 + lc;
  // Each thread owns a 4-wide column strip in rows lr0 + rstep p (p < 4).
  // All loads are issued before any store (the momentum is read and
  // written).
  float gv[4][4], wv[4][4], mv[4][4];
  bool full[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = r0 + lr0 + rstep * p;
    const int64_t u = eoff + (int64_t)row * cols + col;
    full[p] = row < rows && col + 4 <= cols && g.vec_ok;
    if (full[p]) {
      if (a.ema) {
        f32x4_t gg = ld_nt(reinterpret_cast<const f32x4_t*>(a.Gr + u));
        f32x4_t mm = *reinterpret_cast<const f32x4_t*>(a.Mom + u);
        if (a.w_bf16) {
          typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
          u32x2_t wb = ld_nt(reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(a.W) + u));
          wv[p][0] = __uint_as_float(wb[0] << 16); wv[p][1] = __uint_as_float(wb[0] & 0xFFFF0000u);
          wv[p][2] = __uint_as_float(wb[1] << 16); wv[p][3] = __uint_as_float(wb[1] & 0xFFFF0000u);
        } else {
          f32x4_t wf = ld_nt(reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(a.W) + u));
#pragma unroll
          for (int k = 0; k < 4; ++k) wv[p][k] = wf[k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) { gv[p][k] = gg[k]; mv[p][k] = mm[k]; }
      } else {
        f32x4_t sv = *reinterpret_cast<const f32x4_t*>(a.src + u);
#pragma unroll
        for (int k = 0; k < 4; ++k) mv[p][k] = sv[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        gv[p][k] = 0.0f; wv[p][k] = 0.0f; mv[p][k] = 0.0f;
        if (row < rows && col + k < cols) {
          if (a.ema) {
            gv[p][k] = a.Gr[u + k];
            wv[p][k] = load_w(a.W, a.w_bf16, u + k);
            mv[p][k] = a.Mom[u + k];
          } else {
            mv[p][k] = a.src[u + k];
          }
        }
      }
    }
  }
  float ss = 0.0f;
  bool bad = false;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = r0 + lr0 + rstep * p;
    const int64_t u = eoff + (int64_t)row * cols + col;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool valid = row < rows && col + k < cols;
      v[k] = mv[p][k];
      if (a.ema && valid) {
        v[k] = ema(mv[p][k], gv[p][k], wv[p][k], a.beta, a.lam);
        bad |= !__builtin_isfinite(gv[p][k]) || !__builtin_isfinite(wv[p][k]) ||
               !__builtin_isfinite(v[k]);
      }
      ss += v[k] * v[k];
      if (tall) tile[lr0 + 16 * p][lc + k] = v[k];
    }
    if (a.ema) {
      if (full[p]) {
        *reinterpret_cast<f32x4_t*>(a.Mom + u) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (row < rows && col + k < cols) a.Mom[u + k] = v[k];
      }
    }
    if (!tall) store_op4v(a.precision, a.o_hi, a.o_lo, xoff + (int64_t)row * Np + col, v);
  }
  if (tall) {
    __syncthreads();
    write_tile_t(tile, a.precision, a.o_hi, a.o_lo, xoff, Mp, r0, c0);
  }
  if (bad && a.status) a.status[0] = 1;
  if (a.part) {
    float t = block_sum(ss);
    if (threadIdx.x == 0) a.part[g.c0 + (int64_t)mi * g.c_stride + q] = t;
  }
}

hipError_t launch_sweep(const SweepArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (a.G.total_blocks <= 0) return hipSuccess;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_sweep, dim3(a.G.total_blocks), dim3(256), 0, s, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_sweep, dim3(a.G.total_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Momentum + sign-pack of the new momentum (caller layout, per matrix).
// Block = 2048 consecutive entries of one matrix; one entry per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_momentum_sign(MomSignArgs a) {
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int64_t mn = (int64_t)g.rows * g.cols;
  const int64_t nw = (mn + 31) >> 5;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int IT = kChunk / 256;
  float gv[IT], wv[IT], mv[IT];
  // all loads first: the momentum is read and written
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t e = (int64_t)q * kChunk + (it * 4 + wave) * 64 + lane;
    gv[it] = wv[it] = mv[it] = 0.0f;
    if (e < mn) {
      gv[it] = a.Gr[eoff + e];
      wv[it] = load_w(a.W, a.w_bf16, eoff + e);
      mv[it] = a.Mom[eoff + e];
    }
  }
  bool bad = false;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t base = (int64_t)q * kChunk + (it * 4 + wave) * 64;
    const int64_t e = base + lane;
    bool neg = false;
    if (e < mn) {
      const float mk = ema(mv[it], gv[it], wv[it], a.beta, a.lam);
      a.Mom[eoff + e] = mk;
      bad |= !__builtin_isfinite(gv[it]) || !__builtin_isfinite(wv[it]) ||
             !__builtin_isfinite(mk);
      neg = mk < 0.0f;
      if (a.tern) a.tern[eoff + e] = (int8_t)(mk > 0.0f ? 1 : neg ? -1 : 0);
    }
    if (a.tern) continue;
    const uint64_t m = __ballot(neg);
    const int64_t w0 = base >> 5;
    if (lane < 2 && w0 + lane < nw) a.bits[woff + w0 + lane] = (uint32_t)(m >> (32 * lane));
  }
  if (bad && a.status) a.status[0] = 1;
}

hipError_t launch_momentum_sign(const MomSignArgs& a, hipStream_t s, hipEvent_t t0,
                                hipEvent_t t1) {
  if (a.G.total_blocks <= 0) return hipSuccess;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_momentum_sign, dim3(a.G.total_blocks), dim3(256), 0, s, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_momentum_sign, dim3(a.G.total_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Vote over the M resident buffers of each matrix: the majority matrix into
// the padded operand copy (VA_SBAR, a thread per packed word) or the update
// of W (VA_APPLY, k_vote_apply below).
// ---------------------------------------------------------------------------
// Majority masks from bit-sliced counts: the positions whose count of
// negative votes exceeds the constant K (0 <= K < 2^NB), compared from the
// most significant counter bit down.
template <int NB>
__device__ __forceinline__ uint32_t count_gt(const uint32_t (&c)[NB], int K) {
  uint32_t gt = 0, eq = 0xFFFFFFFFu;
#pragma unroll
  for (int k = NB - 1; k >= 0; --k) {
    if ((K >> k) & 1) {
      eq &= c[k];
    } else {
      gt |= eq & c[k];
      eq &= ~c[k];
    }
  }
  return gt;
}

// Vote value of bit k of a word's masks times c: +c (fewer than M/2
// negative votes), -c (more), else c times the tie value (c = 1 but for the
// normalized step).
__device__ __forceinline__ float vote_of(uint32_t pos, uint32_t neg, int k, int tie, float c) {
  return ((pos >> k) & 1u) ? c : (((neg >> k) & 1u) ? -c : c * (float)tie);
}

// Majority masks of one packed word: bit k of pos (neg) is set where fewer
// (more) than half of the M workers voted negative.
template <int NB>
__device__ __forceinline__ void vote_masks(const uint32_t (&c)[NB], int M, uint32_t& pos,
                                           uint32_t& neg) {
  neg = count_gt<NB>(c, M / 2);             // 2 cnt > M
  pos = ~count_gt<NB>(c, (M - 1) / 2);      // 2 cnt < M
}

// VA_SBAR of a tall matrix (stored transposed) whose rows are whole packed
// words: a block takes a tile of 64 rows x 128 columns of the matrix.  Each
// thread counts one word (a row, 32 columns) and leaves its masks in LDS;
// the block then writes the 128 rows of S the tile covers, 64 entries (128
// bytes in bfloat16) per row, 8 consecutive entries per lane.
constexpr int kVtRows = 64, kVtCols = 128;
template <int NB>
__device__ __forceinline__ float vote_sbar_tall(const VoteArgs& a, const Group& g, int mi,
                                                int q) {
  __shared__ uint32_t pm[4][64], nm[4][64];   // [word column][8 (row % 8) + row / 8]
  const int rows = g.rows, cols = g.cols;
  const int tiles_c = (cols + kVtCols - 1) / kVtCols;
  const int r0 = (q / tiles_c) * kVtRows, c0 = (q % tiles_c) * kVtCols;
  const int64_t wpr = cols >> 5;                       // packed words per row
  const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
  const int lr = threadIdx.x >> 2, wc = threadIdx.x & 3;
  const int row = r0 + lr, wcol = (c0 >> 5) + wc;
  uint32_t pos = 0, neg = 0;
  float ss = 0.0f;
  if (row < rows && wcol < wpr) {
    uint32_t c[NB];
    count_votes<NB>(a.bits, a.stride, a.M, woff + row * wpr + wcol, c);
    vote_masks<NB>(c, a.M, pos, neg);
    const int nz = __popc(pos) + __popc(neg);
    ss = (float)nz + (float)(a.tie * a.tie) * (float)(32 - nz);
  }
  pm[wc][8 * (lr & 7) + (lr >> 3)] = pos;
  nm[wc][8 * (lr & 7) + (lr >> 3)] = neg;
  __syncthreads();
  const int64_t ld = round_up(rows, kPad);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int ch = threadIdx.x & 7, bit = threadIdx.x >> 3;
  const int rr = r0 + 8 * ch;                         // first column of S (row of X)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int col = c0 + 32 * p + bit;                // row of S (column of X)
    if (col >= cols || rr >= rows) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = vote_of(pm[p][8 * j + ch], nm[p][8 * j + ch], bit, a.tie, 1.0f);
    const int64_t o = xoff + (int64_t)col * ld + rr;
    if (rr + 8 <= rows) {
      store_op8(a.precision, a.o_hi, a.o_lo, o, v);
    } else {
      for (int j = 0; j < 8 && rr + j < rows; ++j) store_opv(a.precision, a.o_hi, a.o_lo, o + j, v[j]);
    }
  }
  return ss;
}

template <int NB>
__global__ __launch_bounds__(256) void k_vote_groups(VoteArgs a) {
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int rows = g.rows, cols = g.cols;
  if (s_tall(g) && cols % 32 == 0) {
    const float ss = vote_sbar_tall<NB>(a, g, mi, q);
    if (a.part) {
      float t = block_sum(ss);
      if (threadIdx.x == 0) a.part[g.c0 + (int64_t)mi * g.c_stride + q] = t;
    }
    return;
  }
  const int64_t mn = (int64_t)rows * cols;
  const int64_t nw = (mn + 31) >> 5;
  const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
  const int64_t w = (int64_t)q * 256 + threadIdx.x;
  const int64_t Np = round_up(cols, kPad);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  float ss = 0.0f;
  if (cols % 32 == 0) {
    // S = X, rows of whole words: lane l counts word l of the wave's 2048
    // entries; the stores then run over the stretch in lane order, 8
    // entries (16 bytes in bfloat16) per lane, each lane taking the mask
    // bits of its entries from the lane that counted them.
    const int lane = threadIdx.x & 63;
    uint32_t pos = 0, neg = 0;
    if (w < nw) {
      uint32_t c[NB];
      count_votes<NB>(a.bits, a.stride, a.M, woff + w, c);
      vote_masks<NB>(c, a.M, pos, neg);
      const int nz = __popc(pos) + __popc(neg);
      ss = (float)nz + (float)(a.tie * a.tie) * (float)(32 - nz);
    }
    const uint32_t ew = (uint32_t)(w - lane) * 32u;   // entries < 2^31
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int src = 16 * j + (lane >> 2), sh = 8 * (lane & 3);
      const uint32_t pb = (uint32_t)__shfl((int)pos, src) >> sh;
      const uint32_t nb = (uint32_t)__shfl((int)neg, src) >> sh;
      const uint32_t e = ew + 512u * j + 8u * lane;
      if (e >= mn) continue;
      const uint32_t row = e / (uint32_t)cols, col = e - row * (uint32_t)cols;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = vote_of(pb, nb, k, a.tie, 1.0f);
      store_op8(a.precision, a.o_hi, a.o_lo, xoff + (int64_t)row * Np + col, v);
    }
  } else if (w < nw) {
    // rows that split packed words: one entry at a time
    uint32_t c[NB];
    count_votes<NB>(a.bits, a.stride, a.M, woff + w, c);
    const int64_t e0 = w * 32;
    for (int b = 0; b < 32 && e0 + b < mn; ++b) {
      int64_t e = e0 + b;
      int row = (int)(e / cols), col = (int)(e - (int64_t)row * cols);
      float v = (float)majority(vote_sum_at<NB>(c, a.M, b), a.tie);
      ss += v * v;
      store_opv(a.precision, a.o_hi, a.o_lo, xoff + s_index(g, row, col), v);
    }
  }
  if (a.part) {
    float t = block_sum(ss);
    if (threadIdx.x == 0) a.part[g.c0 + (int64_t)mi * g.c_stride + q] = t;
  }
}

// VA_APPLY: a wave takes 2048 consecutive entries of one matrix.  Lane l
// counts the votes of packed word l of the stretch (one coalesced 256-byte
// load per worker) and forms that word's majority masks; the W accesses then
// run over the stretch in lane order (16 bytes per lane and instruction),
// each lane taking the mask bits of its entries from the lane that counted
// them.
template <int NB>
__global__ __launch_bounds__(256) void k_vote_apply(VoteArgs a) {
  if (a.status && a.status[0] != 0) return;
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int64_t mn = (int64_t)g.rows * g.cols;
  const int64_t nw = (mn + 31) >> 5;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ew = ((int64_t)q * 4 + wave) * 2048;
  if (ew >= mn) return;                       // the whole wave
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t woff = g.word0 + (int64_t)mi * g.word_stride;
  const int64_t wi = (ew >> 5) + lane;
  // W moves by eta c D (c = 1 unless a per-matrix scale is given)
  const float c = a.scal ? a.scal[g.idx0 + mi * g.idx_stride] : 1.0f;
  auto masks = [&](uint32_t& pos, uint32_t& neg) {
    pos = neg = 0;
    if (wi < nw) {
      uint32_t c[NB];
      count_votes<NB>(a.bits, a.stride, a.M, woff + wi, c);
      vote_masks<NB>(c, a.M, pos, neg);
    }
  };
  uint32_t pos, neg;
  if (g.vec_ok && ew + 2048 <= mn) {
    // whole stretch, aligned: the W loads go out before the sign-word loads
    if (a.w_bf16) {
      u32x4_t* wp = reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(a.W) + eoff + ew) + lane;
      u32x4_t x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = ld_nt(wp + 64 * j);
      masks(pos, neg);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = 16 * j + (lane >> 2), sh = 8 * (lane & 3);
        const uint32_t pb = (uint32_t)__shfl((int)pos, src) >> sh;
        const uint32_t nb = (uint32_t)__shfl((int)neg, src) >> sh;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16_t r0 = f32_to_bf16(apply_value(__uint_as_float(x[j][k] << 16), a.eta,
                                                    vote_of(pb, nb, 2 * k, a.tie, c)));
          const bf16_t r1 = f32_to_bf16(apply_value(__uint_as_float(x[j][k] & 0xFFFF0000u),
                                                    a.eta, vote_of(pb, nb, 2 * k + 1, a.tie, c)));
          x[j][k] = (uint32_t)r0 | ((uint32_t)r1 << 16);
        }
        st_nt(wp + 64 * j, x[j]);
      }
    } else {
      f32x4_t* wp = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.W) + eoff + ew) + lane;
      f32x4_t x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = ld_nt(wp + 64 * j);
      masks(pos, neg);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int src = 8 * j + (lane >> 3), sh = 4 * (lane & 7);
        const uint32_t pb = (uint32_t)__shfl((int)pos, src) >> sh;
        const uint32_t nb = (uint32_t)__shfl((int)neg, src) >> sh;
#pragma unroll
        for (int k = 0; k < 4; ++k) x[j][k] = apply_value(x[j][k], a.eta, vote_of(pb, nb, k, a.tie, c));
        st_nt(wp + 64 * j, x[j]);
      }
    }
    return;
  }
  // the last, partial stretch of a matrix, or unaligned W
  masks(pos, neg);
  if (a.w_bf16) {
    bf16_t* W = reinterpret_cast<bf16_t*>(a.W);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // entries e .. e + 7 are bits 8 (lane % 4) .. of word 16 j + lane / 4
      const int src = 16 * j + (lane >> 2), sh = 8 * (lane & 3);
      const uint32_t pb = (uint32_t)__shfl((int)pos, src) >> sh;
      const uint32_t nb = (uint32_t)__shfl((int)neg, src) >> sh;
      const int64_t e = ew + 512 * j + 8 * lane;
      if (e >= mn) continue;
      if (g.vec_ok && e + 8 <= mn) {
        u32x4_t* wp = reinterpret_cast<u32x4_t*>(W + eoff + e);
        u32x4_t x = ld_nt(wp);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16_t r0 = f32_to_bf16(apply_value(__uint_as_float(x[k] << 16), a.eta,
                                                    vote_of(pb, nb, 2 * k, a.tie, c)));
          const bf16_t r1 = f32_to_bf16(apply_value(__uint_as_float(x[k] & 0xFFFF0000u), a.eta,
                                                    vote_of(pb, nb, 2 * k + 1, a.tie, c)));
          x[k] = (uint32_t)r0 | ((uint32_t)r1 << 16);
        }
        st_nt(wp, x);
      } else {
        for (int k = 0; k < 8 && e + k < mn; ++k)
          apply_store(a.W, 1, eoff + e + k, a.eta, vote_of(pb, nb, k, a.tie, c));
      }
    }
  } else {
    float* W = reinterpret_cast<float*>(a.W);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // entries e .. e + 3 are bits 4 (lane % 8) .. of word 8 j + lane / 8
      const int src = 8 * j + (lane >> 3), sh = 4 * (lane & 7);
      const uint32_t pb = (uint32_t)__shfl((int)pos, src) >> sh;
      const uint32_t nb = (uint32_t)__shfl((int)neg, src) >> sh;
      const int64_t e = ew + 256 * j + 4 * lane;
      if (e >= mn) continue;
      if (g.vec_ok && e + 4 <= mn) {
        f32x4_t* wp = reinterpret_cast<f32x4_t*>(W + eoff + e);
        f32x4_t x = ld_nt(wp);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = apply_value(x[k], a.eta, vote_of(pb, nb, k, a.tie, c));
        st_nt(wp, x);
      } else {
        for (int k = 0; k < 4 && e + k < mn; ++k)
          apply_store(a.W, 0, eoff + e + k, a.eta, vote_of(pb, nb, k, a.tie, c));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vote over M int8 sign buffers of each matrix (exact integer sums, a zero
// sign adds nothing): VA_APPLY updates W, VA_SBAR writes the majority matrix
// into the padded operand copy (+ partial sums of squares per block).  A
// thread takes 16 consecutive entries of one matrix (kTernChunk per block);
// the 16 signs of a worker are one 16-byte load when the buffers allow it.
// ---------------------------------------------------------------------------
// VA_SBAR over int8 buffers of a tall matrix (stored transposed) whose rows
// are whole 16-entry pieces: a block takes a tile of 64 rows x 64 columns.
// Each thread sums one piece (a row, 16 columns) over the M buffers and
// leaves its majority values in LDS (as bytes, transposed); the block then
// writes the 64 rows of S the tile covers, 64 entries (128 bytes in
// bfloat16) per row, 8 consecutive entries per lane.
constexpr int kTtRows = 64, kTtCols = 64;
__device__ __forceinline__ float vote_tern_sbar_tall(const VoteArgs& a, const Group& g, int mi,
                                                     int q) {
  __shared__ int8_t tv[kTtCols][kTtRows + 8];   // [column][row] of the tile
  const int rows = g.rows, cols = g.cols;
  const int tiles_c = (cols + kTtCols - 1) / kTtCols;
  const int r0 = (q / tiles_c) * kTtRows, c0 = (q % tiles_c) * kTtCols;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int lr = threadIdx.x >> 2, pc = (threadIdx.x & 3) * 16;
  const int row = r0 + lr, col = c0 + pc;
  float ss = 0.0f;
  if (row < rows && col < cols) {
    int acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0;
    const int8_t* src = a.tern + eoff + (int64_t)row * cols + col;
    const bool vec = (a.stride & 15) == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    for (int m = 0; m < a.M; ++m) {
      if (vec) {
        const u32x4_t w = ld_nt(reinterpret_cast<const u32x4_t*>(src + (int64_t)m * a.stride));
#pragma unroll
        for (int k = 0; k < 16; ++k)
          acc[k] += (int)(int8_t)((w[k >> 2] >> (8 * (k & 3))) & 0xFFu);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[k] += src[(int64_t)m * a.stride + k];
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int v = majority(acc[k], a.tie);
      ss += (float)(v * v);
      tv[pc + k][lr] = (int8_t)v;
    }
  }
  __syncthreads();
  const int64_t ld = round_up(rows, kPad);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int ch = threadIdx.x & 7, rr = r0 + 8 * ch;   // first column of S (row of X)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int cl = 32 * p + (threadIdx.x >> 3);
    const int scol = c0 + cl;                        // row of S (column of X)
    if (scol >= cols || rr >= rows) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)tv[cl][8 * ch + j];
    const int64_t o = xoff + (int64_t)scol * ld + rr;
    if (rr + 8 <= rows) {
      store_op8(a.precision, a.o_hi, a.o_lo, o, v);
    } else {
      for (int j = 0; j < 8 && rr + j < rows; ++j) store_opv(a.precision, a.o_hi, a.o_lo, o + j, v[j]);
    }
  }
  return ss;
}

__global__ __launch_bounds__(256) void k_vote_tern(VoteArgs a) {
  if (a.mode == VA_APPLY && a.status && a.status[0] != 0) return;
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int rows = g.rows, cols = g.cols;
  if (a.mode == VA_SBAR && s_tall(g) && cols % 16 == 0) {
    const float ss = vote_tern_sbar_tall(a, g, mi, q);
    if (a.part) {
      float t = block_sum(ss);
      if (threadIdx.x == 0) a.part[g.c0 + (int64_t)mi * g.c_stride + q] = t;
    }
    return;
  }
  const int64_t mn = (int64_t)rows * cols;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const int64_t e0 = (int64_t)q * kTernChunk + threadIdx.x * 16;
  float ss = 0.0f;
  if (e0 < mn) {
    const int cnt = mn - e0 < 16 ? (int)(mn - e0) : 16;
    int acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0;
    const int8_t* src = a.tern + eoff + e0;
    const bool vec = cnt == 16 && (a.stride & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    if (vec) {
      for (int m = 0; m < a.M; ++m) {
        const u32x4_t w = ld_nt(reinterpret_cast<const u32x4_t*>(src + (int64_t)m * a.stride));
#pragma unroll
        for (int k = 0; k < 16; ++k)
          acc[k] += (int)(int8_t)((w[k >> 2] >> (8 * (k & 3))) & 0xFFu);
      }
    } else {
      for (int m = 0; m < a.M; ++m) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (k < cnt) acc[k] += src[(int64_t)m * a.stride + k];
      }
    }
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = (float)majority(acc[k], a.tie);
    if (a.mode == VA_APPLY) {
      // W moves by eta c D (c = 1 unless a per-matrix scale is given)
      if (a.scal) {
        const float c = a.scal[g.idx0 + mi * g.idx_stride];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] *= c;
      }
      if (g.vec_ok && cnt == 16) {
        // e0 and the matrix offset are multiples of 8: 16-byte W accesses
        if (a.w_bf16) {
          u32x4_t* wp = reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(a.W) + eoff + e0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4_t x = ld_nt(wp + h);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const bf16_t r0 = f32_to_bf16(apply_value(__uint_as_float(x[k] << 16), a.eta,
                                                        v[8 * h + 2 * k]));
              const bf16_t r1 = f32_to_bf16(apply_value(__uint_as_float(x[k] & 0xFFFF0000u),
                                                        a.eta, v[8 * h + 2 * k + 1]));
              x[k] = (uint32_t)r0 | ((uint32_t)r1 << 16);
            }
            st_nt(wp + h, x);
          }
        } else {
          f32x4_t* wp = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.W) + eoff + e0);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            f32x4_t x = ld_nt(wp + h);
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = apply_value(x[k], a.eta, v[4 * h + k]);
            st_nt(wp + h, x);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (k < cnt) apply_store(a.W, a.w_bf16, eoff + e0 + k, a.eta, v[k]);
      }
    } else {
      // VA_SBAR: the majority matrix into the padded operand copy
      const int64_t Np = round_up(cols, kPad);
      const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < cnt) ss += v[k] * v[k];
      if (cnt == 16 && cols % 16 == 0 && !s_tall(g)) {
        const int row = (int)(e0 / cols), col = (int)(e0 - (int64_t)row * cols);
        float h0[8], h1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) { h0[k] = v[k]; h1[k] = v[8 + k]; }
        store_op8(a.precision, a.o_hi, a.o_lo, xoff + (int64_t)row * Np + col, h0);
        store_op8(a.precision, a.o_hi, a.o_lo, xoff + (int64_t)row * Np + col + 8, h1);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (k >= cnt) continue;
          const int64_t e = e0 + k;
          const int row = (int)(e / cols), col = (int)(e - (int64_t)row * cols);
          store_opv(a.precision, a.o_hi, a.o_lo, xoff + s_index(g, row, col), v[k]);
        }
      }
    }
  }
  if (a.mode == VA_SBAR && a.part) {
    float t = block_sum(ss);
    if (threadIdx.x == 0) a.part[g.c0 + (int64_t)mi * g.c_stride + q] = t;
  }
}

int tern_vote_blocks_per_mat(int mode, int64_t rows, int64_t cols) {
  if (mode == VA_SBAR && rows > cols && cols % 16 == 0)   // tiles of vote_tern_sbar_tall
    return (int)(((rows + kTtRows - 1) / kTtRows) * ((cols + kTtCols - 1) / kTtCols));
  return (int)((rows * cols + kTernChunk - 1) / kTernChunk);
}

int vote_blocks_per_mat(int mode, int64_t rows, int64_t cols) {
  const int64_t mn = rows * cols;
  if (mode == VA_APPLY) return (int)((mn + 8191) / 8192);
  if (rows > cols && cols % 32 == 0)   // tiles of vote_sbar_tall
    return (int)(((rows + kVtRows - 1) / kVtRows) * ((cols + kVtCols - 1) / kVtCols));
  return (int)(((mn + 31) / 32 + 255) / 256);
}

// Launches kernel K (grid, 256 threads) on s; with t0 / t1, events that take
// the kernel's own start and stop times.
template <typename K>
static void launch_timed(K kern, dim3 grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1,
                         const VoteArgs& a) {
  if (t0 || t1)
    hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, s, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, a);
}

hipError_t launch_vote_groups(const VoteArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (a.G.total_blocks <= 0) return hipSuccess;
  const dim3 grid(a.G.total_blocks);
  if (a.tern)
    launch_timed(k_vote_tern, grid, s, t0, t1, a);
  else if (a.mode == VA_APPLY)
    launch_timed(a.M <= 15 ? k_vote_apply<4> : a.M <= 255 ? k_vote_apply<8> : k_vote_apply<16>,
                 grid, s, t0, t1, a);
  else
    launch_timed(a.M <= 15 ? k_vote_groups<4> : a.M <= 255 ? k_vote_groups<8> : k_vote_groups<16>,
                 grid, s, t0, t1, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Zero the padding of padded operand copies S.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_zero_pad(Groups G, int precision,
                                                  void* hi, void* lo) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const int sr = s_rows(g), sc = s_cols(g);
  const int64_t ld = round_up(sc, kPad);
  const int64_t xoff = g.x0 + (int64_t)mi * g.x_stride;
  const int64_t p = (int64_t)q * kChunk + threadIdx.x * 8;
  const int row = (int)(p / ld), col = (int)(p - (int64_t)row * ld);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (row >= sr || col + k >= sc) store_opv(precision, hi, lo, xoff + p + k, 0.0f);
}

hipError_t launch_zero_pad(const Groups& G, int precision, void* hi, void* lo,
                           hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_pad, dim3(G.total_blocks), dim3(256), 0, s, G,
                     precision, hi, lo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pre-scale: Frobenius finalize, power iteration, scaled Gram operand.
// One block per matrix for the finalize kernels (blocks_per_mat = 1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fro_finalize(Groups G, const float* part,
                                                      float eps, float* scal) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const int64_t c0 = g.c0 + (int64_t)mi * g.c_stride;
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < g.gk; i += 256) s += part[c0 + i];
  s = block_sum(s);
  if (threadIdx.x == 0) scal[g.idx0 + mi * g.idx_stride] = 1.0f / (sqrtf(s) + eps);
}

hipError_t launch_fro_finalize(const Groups& G, const float* part, float eps,
                               float* scal, hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fro_finalize, dim3(G.total_blocks), dim3(256), 0, s, G,
                     part, eps, scal);
  return hipGetLastError();
}

// dst = A * (src / |src|) for 16 rows per block (4 per wave); each lane
// takes 4 consecutive entries per 256-entry stretch of a row.  With `first`
// set, src is the start vector itself: u0's r entries (ones when u0 is null)
// and zeros up to Rp.
__global__ __launch_bounds__(256) void k_power_step(Groups G, const float* araw,
                                                    const float* src, float* dst,
                                                    const float* u0, int first) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const int r = g.rows < g.cols ? g.rows : g.cols;
  const int64_t Rp = round_up(r, kPad);
  const int64_t voff = g.v0 + (int64_t)mi * g.v_stride;
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const float* x = src + voff;
  const float* u = u0 ? u0 + g.u0_0 + (int64_t)mi * g.u0_stride : nullptr;
  auto start = [&](int64_t i) -> float {
    return i < r ? (u ? u[i] : 1.0f) : 0.0f;
  };
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < Rp; i += 256) {
    const float xi = first ? start(i) : x[i];
    ss += xi * xi;
  }
  ss = block_sum(ss);
  const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t row0 = (int64_t)q * 16 + wave * 4;
  for (int64_t k = 4 * lane; k < Rp; k += 256) {
    f32x4_t xv;
    if (first) {
#pragma unroll
      for (int t = 0; t < 4; ++t) xv[t] = start(k + t);
    } else {
      xv = *reinterpret_cast<const f32x4_t*>(x + k);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4_t av = *reinterpret_cast<const f32x4_t*>(araw + roff + (row0 + rr) * Rp + k);
      acc[rr] += av[0] * (xv[0] * inv) + av[1] * (xv[1] * inv) + av[2] * (xv[2] * inv) +
                 av[3] * (xv[3] * inv);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float t = wave_sum(acc[rr]);
    if (lane == 0) dst[voff + row0 + rr] = t;
  }
}

hipError_t launch_power_step(const Groups& G, const float* araw,
                             const float* src, float* dst, const float* u0,
                             bool first, hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_power_step, dim3(G.total_blocks), dim3(256), 0, s, G,
                     araw, src, dst, u0, first ? 1 : 0);
  return hipGetLastError();
}

// 1 / (sqrt(|w|) + eps) for one matrix's final power-iteration vector w
// (|w| estimates the top eigenvalue of the raw Gram, so its square root is
// the top singular value); every thread of the block gets the value.
__device__ __forceinline__ float power_scale(const Group& g, int mi, const float* w,
                                             float eps) {
  const int r = g.rows < g.cols ? g.rows : g.cols;
  const int64_t Rp = round_up(r, kPad);
  const float* x = w + g.v0 + (int64_t)mi * g.v_stride;
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < Rp; i += 256) ss += x[i] * x[i];
  ss = block_sum(ss);
  const float lam = sqrtf(ss);
  return 1.0f / (sqrtf(lam) + eps);
}

// The one-launch power iteration.  The blocks of a matrix exchange each
// step's vector as tagged entries: one 8-byte word per entry holding the
// float and the number of the step that wrote it (zero: not yet written;
// the raw Gram launch before clears them), written and read with
// device-scope atomic accesses, which go to the device's coherence point
// rather than to an XCD's own L2.  A reader polls each entry until its tag
// is the step it waits for (bounded), so the vector's arrival is the
// barrier: no counter and no cache writeback or invalidation.  Step p
// writes tag p + 1 into buffer (p + 1) % 2; a writer can be at most one
// step ahead of any reader, so two buffers suffice.
constexpr int kTagSpins = 1 << 20;
__device__ __forceinline__ void put_tagged(uint64_t* t, float v, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
  __hip_atomic_store(t, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Entries i = threadIdx.x + 256 j (< n) of a tagged vector into xs, once
// each carries `tag`; false if any poll ran out (the same for every thread).
__device__ __forceinline__ bool get_tagged(const uint64_t* t, int64_t n, uint32_t tag,
                                           float* xs) {
  __shared__ int late;
  if (threadIdx.x == 0) late = 0;
  __syncthreads();
  constexpr int kMax = kPowerIterMaxRp / 256;
  uint64_t w[kMax];
#pragma unroll
  for (int j = 0; j < kMax; ++j) {
    const int64_t i = threadIdx.x + 256 * j;
    w[j] = i < n ? __hip_atomic_load(t + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : ((uint64_t)tag << 32);
  }
  bool ok = true;
#pragma unroll
  for (int j = 0; j < kMax; ++j) {
    const int64_t i = threadIdx.x + 256 * j;
    int spins = 0;
    while ((uint32_t)(w[j] >> 32) != tag && spins < kTagSpins) {
      __builtin_amdgcn_s_sleep(1);
      w[j] = __hip_atomic_load(t + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++spins;
    }
    if ((uint32_t)(w[j] >> 32) != tag) ok = false;
    if (i < n) xs[i] = __uint_as_float((uint32_t)w[j]);
  }
  if (!ok) late = 1;
  __syncthreads();
  return late == 0;
}

// The P power steps of k_power_step (same arithmetic, same order), with
// the block's kPowerRows rows of the raw Gram read once into LDS, then the
// scale (as power_scale) and, with scaled_op, the scaled operand of
// k_prescale for those rows.
__global__ __launch_bounds__(256) void k_power_iter(PowerIterArgs a) {
  extern __shared__ f32x4_t slab4[];
  float* slab = reinterpret_cast<float*>(slab4);   // kPowerRows x Rp, then x (Rp)
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int r = g.rows < g.cols ? g.rows : g.cols;
  const int64_t Rp = round_up(r, kPad);
  const int midx = g.idx0 + mi * g.idx_stride;
  const int64_t voff = g.v0 + (int64_t)mi * g.v_stride;
  const int64_t soff = g.r0 + (int64_t)mi * g.r_stride + (int64_t)q * kPowerRows * Rp;
  float* xs = slab + kPowerRows * Rp;
  uint64_t* tb[2] = {a.tag + voff, a.tag + a.tag_stride + voff};
  const float* u = a.u0 ? a.u0 + g.u0_0 + (int64_t)mi * g.u0_stride : nullptr;
  for (int64_t i = 4 * threadIdx.x; i < kPowerRows * Rp; i += 1024)
    *reinterpret_cast<f32x4_t*>(slab + i) = *reinterpret_cast<const f32x4_t*>(a.araw + soff + i);
  for (int64_t i = threadIdx.x; i < Rp; i += 256) xs[i] = i < r ? (u ? u[i] : 1.0f) : 0.0f;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int p = 0; p < a.P; ++p) {
    if (p > 0 && !get_tagged(tb[p & 1], Rp, (uint32_t)p, xs)) {
      if (threadIdx.x == 0) {
        atomicOr(a.status, 2);
        atomicOr(a.status + 1, 2);
      }
      return;
    }
    float ss = 0.0f;
    for (int64_t i = threadIdx.x; i < Rp; i += 256) ss += xs[i] * xs[i];
    ss = block_sum(ss);
    const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t k = 4 * lane; k < Rp; k += 256) {
      const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(xs + k);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4_t av = *reinterpret_cast<const f32x4_t*>(slab + (wave * 4 + rr) * Rp + k);
        acc[rr] += av[0] * (xv[0] * inv) + av[1] * (xv[1] * inv) + av[2] * (xv[2] * inv) +
                   av[3] * (xv[3] * inv);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float t = wave_sum(acc[rr]);
      if (lane == 0)
        put_tagged(tb[(p + 1) & 1] + (int64_t)q * kPowerRows + wave * 4 + rr, t, (uint32_t)(p + 1));
    }
  }
  // the scale of power_scale, from the final vector
  if (!get_tagged(tb[a.P & 1], Rp, (uint32_t)a.P, xs)) {
    if (threadIdx.x == 0) {
      atomicOr(a.status, 2);
      atomicOr(a.status + 1, 2);
    }
    return;
  }
  float ws = 0.0f;
  for (int64_t i = threadIdx.x; i < Rp; i += 256) ws += xs[i] * xs[i];
  ws = block_sum(ws);
  const float c = 1.0f / (sqrtf(sqrtf(ws)) + a.eps);
  if (q == 0 && threadIdx.x == 0) a.scal[midx] = c;
  if (a.scaled_op) {
    const float m = a.mul * c * c;
    for (int64_t i = 8 * threadIdx.x; i < kPowerRows * Rp; i += 2048) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = m * slab[i + k];
      store_op8(a.precision, a.hi, a.lo, soff + i, v);
    }
  }
}

hipError_t launch_power_iter(const PowerIterArgs& a, int64_t rp_max, hipStream_t s) {
  if (a.G.total_blocks <= 0) return hipSuccess;
  if (a.G.total_blocks > kPowerIterMaxBlocks || rp_max > kPowerIterMaxRp || a.P < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_power_iter, dim3(a.G.total_blocks), dim3(256),
                     (size_t)(kPowerRows + 1) * rp_max * sizeof(float), s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_power_finalize(Groups G, const float* w,
                                                        float eps, float* scal) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const float c = power_scale(g, mi, w, eps);
  if (threadIdx.x == 0) scal[g.idx0 + mi * g.idx_stride] = c;
}

hipError_t launch_power_finalize(const Groups& G, const float* w, float eps,
                                 float* scal, hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_power_finalize, dim3(G.total_blocks), dim3(256), 0, s, G,
                     w, eps, scal);
  return hipGetLastError();
}

// With w set, each block derives c from the final power vector itself (the
// same sum as the finalize kernel) and the matrix's first block stores it.
__global__ __launch_bounds__(256) void k_prescale(Groups G, int precision,
                                                  const float* araw,
                                                  float* scal, float mul,
                                                  void* hi, void* lo,
                                                  const float* w, float eps) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  float c;
  if (w) {
    c = power_scale(g, mi, w, eps);
    if (q == 0 && threadIdx.x == 0) scal[g.idx0 + mi * g.idx_stride] = c;
  } else {
    c = scal[g.idx0 + mi * g.idx_stride];
  }
  const float m = mul * c * c;
  const int64_t p = roff + (int64_t)q * kChunk + threadIdx.x * 8;
  float v[8];
  f32x4_t a0 = reinterpret_cast<const f32x4_t*>(araw + p)[0];
  f32x4_t a1 = reinterpret_cast<const f32x4_t*>(araw + p)[1];
#pragma unroll
  for (int k = 0; k < 4; ++k) { v[k] = m * a0[k]; v[4 + k] = m * a1[k]; }
  store_op8(precision, hi, lo, p, v);
}

hipError_t launch_prescale(const Groups& G, int precision, const float* araw,
                           float* scal, float mul, void* hi, void* lo,
                           const float* w, float eps, hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prescale, dim3(G.total_blocks), dim3(256), 0, s, G,
                     precision, araw, scal, mul, hi, lo, w, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q = a I + b A over each matrix's padded Gram-sized bfloat16 buffer (the
// first factor of the Gram-space Newton-Schulz form); 8 entries per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_affine_ident(Groups G, const bf16_t* A, float a,
                                                      float b, bf16_t* Q) {
  int gi, mi, q;
  group_of_block(G, blockIdx.x, gi, mi, q);
  const Group& g = G.g[gi];
  const int64_t Rp = round_up(s_rows(g), kPad);
  const int64_t roff = g.r0 + (int64_t)mi * g.r_stride;
  const int64_t p = (int64_t)q * kChunk + threadIdx.x * 8;
  const int64_t row = p / Rp, col0 = p - row * Rp;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(A + roff + p);
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float v0 = b * __uint_as_float(x[k] << 16);
    float v1 = b * __uint_as_float(x[k] & 0xFFFF0000u);
    if (row == col0 + 2 * k) v0 += a;
    if (row == col0 + 2 * k + 1) v1 += a;
    o[k] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  }
  *reinterpret_cast<u32x4_t*>(Q + roff + p) = o;
}

hipError_t launch_affine_ident(const Groups& G, const void* A, float a, float b, void* Q,
                               hipStream_t s) {
  if (G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_affine_ident, dim3(G.total_blocks), dim3(256), 0, s, G,
                     reinterpret_cast<const bf16_t*>(A), a, b, reinterpret_cast<bf16_t*>(Q));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// PolarNS with K = 0: U = c X (caller layout).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scaled_out(ScaledOutArgs a) {
  int gi, mi, q;
  group_of_block(a.G, blockIdx.x, gi, mi, q);
  const Group& g = a.G.g[gi];
  const int64_t mn = (int64_t)g.rows * g.cols;
  const int64_t eoff = g.elem0 + (int64_t)mi * g.elem_stride;
  const float c = a.scal[g.idx0 + mi * g.idx_stride];
  for (int k = 0; k < 8; ++k) {
    const int64_t e = (int64_t)q * kChunk + k * 256 + threadIdx.x;
    if (e >= mn) break;
    a.U[eoff + e] = c * a.x_user[eoff + e];
  }
}

hipError_t launch_scaled_out(const ScaledOutArgs& a, hipStream_t s) {
  if (a.G.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scaled_out, dim3(a.G.total_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ternary (int8) sign buffers: S = sign(U) in {-1, 0, +1} (NaN -> 0), and
// the vote over M such buffers, sum_j = sum_m S_m[j], D_j = sign(sum_j) with
// a tie (sum 0) mapped to tie.  Each thread takes 16 consecutive entries;
// 16-byte accesses when every buffer start is 16-byte aligned, else bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sign_ternary(const float* U, int8_t* S, int64_t n) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (e0 >= n) return;
  const int cnt = n - e0 < 16 ? (int)(n - e0) : 16;
  for (int k = 0; k < cnt; ++k) {
    const float u = U[e0 + k];
    S[e0 + k] = (int8_t)(u > 0.0f ? 1 : u < 0.0f ? -1 : 0);
  }
}

hipError_t launch_sign_ternary(const float* U, int8_t* S, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 16 * 256 - 1) / (16 * 256);
  hipLaunchKernelGGL(k_sign_ternary, dim3((unsigned)blocks), dim3(256), 0, s, U, S, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_vote_ternary(const int8_t* S, int64_t stride, int M,
                                                      int64_t n, int tie, int8_t* D,
                                                      int16_t* sums, int vec) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (e0 >= n) return;
  int acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0;
  if (vec && e0 + 16 <= n) {
    for (int m = 0; m < M; ++m) {
      const u32x4_t w = ld_nt(reinterpret_cast<const u32x4_t*>(S + (int64_t)m * stride + e0));
#pragma unroll
      for (int k = 0; k < 16; ++k)
        acc[k] += (int)(int8_t)((w[k >> 2] >> (8 * (k & 3))) & 0xFFu);
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int a = acc[4 * q + b];
        const int d = a > 0 ? 1 : a < 0 ? -1 : tie;
        v |= (uint32_t)(uint8_t)(int8_t)d << (8 * b);
      }
      o[q] = v;
    }
    *reinterpret_cast<u32x4_t*>(D + e0) = o;
    if (sums) {
#pragma unroll
      for (int k = 0; k < 16; ++k) sums[e0 + k] = (int16_t)acc[k];
    }
    return;
  }
  const int cnt = n - e0 < 16 ? (int)(n - e0) : 16;
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < cnt; ++k) acc[k] += S[(int64_t)m * stride + e0 + k];
  for (int k = 0; k < cnt; ++k) {
    const int a = acc[k];
    D[e0 + k] = (int8_t)(a > 0 ? 1 : a < 0 ? -1 : tie);
    if (sums) sums[e0 + k] = (int16_t)a;
  }
}

hipError_t launch_vote_ternary(const int8_t* S, int64_t stride, int M, int64_t n, int tie,
                               int8_t* D, int16_t* sums, hipStream_t s) {
  const int vec = (reinterpret_cast<uintptr_t>(S) % 16 == 0) &&
                  (M == 1 || stride % 16 == 0) && (reinterpret_cast<uintptr_t>(D) % 16 == 0);
  const int64_t blocks = (n + 16 * 256 - 1) / (16 * 256);
  hipLaunchKernelGGL(k_vote_ternary, dim3((unsigned)blocks), dim3(256), 0, s, S, stride, M, n,
                     tie, D, sums, vec);
  return hipGetLastError();
}

// Status words of a workspace: word 0 is the flag of the current step (the
// update of W is skipped while it is set), word 1 collects the flags of
// worker pipelines enqueued since the last step.  A step starts by moving
// word 1 into word 0 and clearing word 1.
__global__ void k_begin_status(int32_t* status) {
  if (threadIdx.x == 0) {
    status[0] = status[1];
    status[1] = 0;
  }
}
hipError_t launch_begin_status(int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_begin_status, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}
__global__ void k_reset_status(int32_t* status) {
  if (threadIdx.x < 2) status[threadIdx.x] = 0;
}
hipError_t launch_reset_status(int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_reset_status, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}

}  // namespace sm
