// C ABI of libsignmuon: argument validation, the workspace plan, grouping of
// matrices into launch runs, and the order of kernels of one step.
//
// Step order (SignMuon paper, Algorithm 2 and Figure 1, for the local
// worker; the other workers' buffers are already resident):
//   momentum sweep  -> padded operand copy of Mom, partial sums, status
//   pre-scale       -> c = 1/(s+eps) per matrix (Frobenius from the partial
//                      sums; spectral from P power steps on the raw Gram)
//   K Newton-Schulz steps, each a Gram GEMM and an update GEMM (the quintic
//   adds the A*A GEMM); the last update's epilogue packs sign(U) straight
//   into the local worker's buffer
//   vote over the M buffers fused with W <- W - eta * majority.
// Post-vote variant: momentum + sign-pack, vote -> majority matrix, PolarNS
// of the majority matrix whose last epilogue applies W <- W - eta * U.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "sm_internal.h"
#include "sm_launch.h"

using namespace sm;

namespace {

constexpr int32_t kAbiVersion = 2;
constexpr int64_t kMaxDim = 1 << 20;          // rows / cols
constexpr int64_t kMaxPadded = (int64_t)1 << 31;  // padded rows * cols

bool finite(float x) { return std::isfinite(x); }

sm_status check_hparams(const sm_hparams* hp, bool need_momentum) {
  if (!hp) return SM_EINVAL;
  if (!finite(hp->eps) || hp->eps <= 0.f) return SM_EINVAL;
  if (hp->K < 0 || hp->K > 64) return SM_EINVAL;
  if (hp->scale != SM_SCALE_FRO && hp->scale != SM_SCALE_SPECTRAL) return SM_EINVAL;
  if (hp->scale == SM_SCALE_SPECTRAL && (hp->P < 1 || hp->P > 256)) return SM_EINVAL;
  if (!finite(hp->ns_a) || !finite(hp->ns_b) || !finite(hp->ns_c)) return SM_EINVAL;
  if (hp->ns_precision < SM_NS_F32 || hp->ns_precision > SM_NS_BF16X3) return SM_EINVAL;
  if (hp->sign_encoding != SM_SIGNS_PACKED && hp->sign_encoding != SM_SIGNS_TERNARY)
    return SM_EINVAL;
  if (need_momentum) {
    if (!finite(hp->beta) || hp->beta < 0.f || hp->beta >= 1.f) return SM_EINVAL;
    if (!finite(hp->lambda) || hp->lambda < 0.f) return SM_EINVAL;
    if (!finite(hp->eta)) return SM_EINVAL;
    if (hp->tie_value != 0 && hp->tie_value != 1) return SM_EINVAL;
  }
  return SM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The Gram-space Newton-Schulz form is used for bfloat16 cubic steps with
// the Frobenius scale unless the environment variable SIGNMUON_NS_FORM is
// "iterate" (read at every call).
bool gram_space_enabled() {
  const char* e = std::getenv("SIGNMUON_NS_FORM");
  return !(e && std::strcmp(e, "iterate") == 0);
}

// One of the concurrent chains runs on the caller's stream unless the
// environment variable SIGNMUON_CALLER_CHAIN is "0" (read at every call).
bool caller_chain_enabled() {
  const char* e = std::getenv("SIGNMUON_CALLER_CHAIN");
  return !(e && std::strcmp(e, "0") == 0);
}

// The P power steps of small sets run in one launch unless the environment
// variable SIGNMUON_POWER_ITER is "steps" (one launch per step; read at
// every call).
bool power_iter_fused() {
  const char* e = std::getenv("SIGNMUON_POWER_ITER");
  return !(e && std::strcmp(e, "steps") == 0);
}

// bfloat16 symmetric operands are stored as their upper-triangular tiles
// unless the environment variable SIGNMUON_SYM_STORAGE is "full" (read at
// every call; then every symmetric output also writes its mirror tiles).
bool sym_upper_enabled() {
  const char* e = std::getenv("SIGNMUON_SYM_STORAGE");
  return !(e && std::strcmp(e, "full") == 0);
}

// Per-matrix placement.  Returns SM_OK or SM_EINVAL for unusable shapes.
sm_status build_plan(const sm_matrix* mats, int nm, const sm_hparams* hp,
                     int post_vote, Plan& P,
                     std::vector<MatPlan>& mp) {
  mp.assign(nm, MatPlan{});
  P = Plan{};
  P.nm = nm;
  P.precision = hp->ns_precision == SM_NS_F32 ? P_F32
              : hp->ns_precision == SM_NS_BF16X3 ? P_BF16X3 : P_BF16;
  P.quintic = hp->ns_c != 0.0f;
  P.spectral = hp->scale == SM_SCALE_SPECTRAL;
  // Gram space only with the Frobenius scale: with the spectral scale the top
  // singular values start near or above 1, where the Gram-space rounding
  // missed the sign gate on test matrices that the iterate form passes
  P.gram_space = P.precision == P_BF16 && !P.quintic && !P.spectral && hp->K > 0 &&
                 gram_space_enabled();
  P.upper = P.precision == P_BF16 && sym_upper_enabled();
  int64_t x = 0, r2 = 0, v = 0, c = 0, u0 = 0;
  for (int i = 0; i < nm; ++i) {
    const sm_matrix& m = mats[i];
    if (m.rows < 1 || m.cols < 1 || m.rows > kMaxDim || m.cols > kMaxDim) return SM_EINVAL;
    if (m.elem_off < 0 || m.word_off < 0) return SM_EINVAL;
    MatPlan& q = mp[i];
    q.rows = m.rows; q.cols = m.cols;
    q.r = std::min(m.rows, m.cols);
    q.tall = m.rows > m.cols;
    q.Mp = round_up(m.rows, kPad);
    q.Np = round_up(m.cols, kPad);
    q.Rp = round_up(q.r, kPad);
    // the GEMM addresses one operand matrix with 32-bit byte offsets
    if (q.Mp * q.Np >= (P.precision == P_F32 ? kMaxPadded / 2 : kMaxPadded)) return SM_EINVAL;
    q.elem_off = m.elem_off; q.word_off = m.word_off;
    q.x_off = x; x += q.Mp * q.Np;
    q.r_off = r2; r2 += q.Rp * q.Rp;
    q.v_off = v; v += q.Rp;
    q.u0_off = u0; u0 += q.r;
    // partial sums: one per sweep chunk or per vote block
    q.chunks = std::max<int64_t>({q.Mp * q.Np / kChunk,
                                  (int64_t)vote_blocks_per_mat(VA_SBAR, m.rows, m.cols),
                                  (int64_t)tern_vote_blocks_per_mat(VA_SBAR, m.rows, m.cols)});
    q.c_off = c; c += q.chunks;
    q.idx = i;
  }
  // split-k of the long-k Grams of shapes with few triangular tiles (the
  // decision counts every matrix of the shape, as one launch holds them)
  std::map<std::pair<int64_t, int64_t>, int64_t> shape_count;
  for (int i = 0; i < nm; ++i) ++shape_count[{mp[i].rows, mp[i].cols}];
  int64_t kp = 0;
  for (int i = 0; i < nm; ++i) {
    MatPlan& q = mp[i];
    const int64_t same = shape_count[{q.rows, q.cols}];
    int slabs = 0;
    q.ks = gemm_sym_ksplit(P.precision, q.Rp, q.tall ? q.Mp : q.Np, same, &slabs);
    q.kslabs = slabs;
    q.kp_off = kp;
    kp += gemm_sym_kpart_floats(q.Rp, q.ks);
  }
  // Upper-triangular storage needs every product that reads a symmetric
  // operand to take its slabs left of the diagonal k-major; the 128 x 256
  // update tile (long bfloat16 updates) reads whole rows, so a set with
  // such an update keeps mirrored storage.
  for (int i = 0; i < nm && P.upper; ++i) {
    const MatPlan& q = mp[i];
    int tm = 0, tn = 0;
    gemm_tile(P.precision, E_UPDATE, q.Rp, q.tall ? q.Mp : q.Np, q.Rp, &tm, &tn);
    if (tn != tm) P.upper = false;
  }
  P.x_total = x; P.r_total = r2; P.v_total = v; P.c_total = c; P.kp_total = kp;
  const size_t opb = P.precision == P_F32 ? 4 : 2;   // bytes per operand part
  const bool split = P.precision == P_BF16X3;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  take(256);                                  // status word (+ padding)
  P.off_status = 0;
  const bool ns = hp->K > 0;
  for (int pp = 0; pp < (ns ? 2 : 1); ++pp) {
    P.off_x[pp][0] = take(x * opb);
    if (split) P.off_x[pp][1] = take(x * opb);
  }
  if (ns) {
    P.off_b[0] = take(r2 * opb);
    if (split) P.off_b[1] = take(r2 * opb);
    if (P.quintic) {
      P.off_a[0] = take(r2 * opb);
      if (split) P.off_a[1] = take(r2 * opb);
    }
  }
  // the normalized sign step (post_vote 3) estimates ||D||_2 by power
  // iteration on the raw Gram of the majority matrix, whatever the scale
  const bool power = P.spectral || post_vote == 3;
  if (power) {
    P.off_araw = take(r2 * 4);
    P.off_vec = take(2 * v * 4);
    P.off_tag = take(2 * v * 8);
  }
  P.off_part = take(c * 4);
  if ((ns || power) && kp > 0) P.off_kpart = take(kp * 4);
  if (P.gram_space) P.off_gs = take(5 * r2 * 2);
  P.off_scal = take((size_t)nm * 4);
  P.total = off;
  return SM_OK;
}

// Split matrices (a subset, by index) into runs of equal shape and constant
// strides of every offset family.  Matrices are visited shape by shape (in
// their original order within a shape), so a layout that interleaves shapes,
// such as the projections of successive transformer layers, still gives one
// run per shape.
std::vector<Group> make_groups(const std::vector<MatPlan>& mp,
                               const std::vector<int>& sel_in) {
  std::vector<int> sel(sel_in);
  std::stable_sort(sel.begin(), sel.end(), [&](int a, int b) {
    if (mp[a].rows != mp[b].rows) return mp[a].rows < mp[b].rows;
    return mp[a].cols < mp[b].cols;
  });
  std::vector<Group> out;
  for (size_t t = 0; t < sel.size(); ++t) {
    const MatPlan& q = mp[sel[t]];
    if (!out.empty()) {
      Group& g = out.back();
      const MatPlan& f = mp[g.idx0];
      if (g.rows == q.rows && g.cols == q.cols) {
        int64_t k = g.count;
        if (g.count == 1) {
          int64_t de = q.elem_off - f.elem_off, dw = q.word_off - f.word_off;
          if (de > 0 && dw >= 0 && q.idx - f.idx > 0) {
            g.elem_stride = de; g.word_stride = dw;
            g.x_stride = q.x_off - f.x_off; g.r_stride = q.r_off - f.r_off;
            g.v_stride = q.v_off - f.v_off; g.u0_stride = q.u0_off - f.u0_off;
            g.c_stride = q.c_off - f.c_off; g.idx_stride = q.idx - f.idx;
            g.kp_stride = q.kp_off - f.kp_off;
            g.count = 2;
            continue;
          }
        } else if (q.elem_off == f.elem_off + k * g.elem_stride &&
                   q.word_off == f.word_off + k * g.word_stride &&
                   q.x_off == f.x_off + k * g.x_stride &&
                   q.r_off == f.r_off + k * g.r_stride &&
                   q.v_off == f.v_off + k * g.v_stride &&
                   q.u0_off == f.u0_off + k * g.u0_stride &&
                   q.c_off == f.c_off + k * g.c_stride &&
                   q.kp_off == f.kp_off + k * g.kp_stride &&
                   q.idx == f.idx + k * g.idx_stride) {
          g.count += 1;
          continue;
        }
      }
    }
    Group g;
    std::memset(&g, 0, sizeof(g));
    g.count = 1;
    g.rows = (int32_t)q.rows; g.cols = (int32_t)q.cols;
    g.idx0 = q.idx; g.idx_stride = 0;
    g.elem0 = q.elem_off; g.word0 = q.word_off;
    g.x0 = q.x_off; g.r0 = q.r_off; g.v0 = q.v_off; g.u0_0 = q.u0_off;
    g.c0 = q.c_off;
    g.kp0 = q.kp_off; g.ksplit = q.ks; g.kslabs = q.kslabs;
    out.push_back(g);
  }
  return out;
}

// Issue one kernel per chunk of at most kMaxGroups runs.  `fill` sets the
// per-group launch fields (blocks_per_mat, gm, gn, gk, tiles_n, ops) and
// returns false to drop a group; `go` launches.
template <class Fill, class Go>
hipError_t for_launches(const std::vector<Group>& groups, Fill fill, Go go,
                        int* launched = nullptr) {
  if (launched) *launched = 0;
  std::vector<Group> gs;
  for (const Group& g0 : groups) {
    Group g = g0;
    if (fill(g)) gs.push_back(g);
  }
  // launches hold at most kMaxGroups runs, all with the same GEMM tile
  std::stable_sort(gs.begin(), gs.end(),
                   [](const Group& a, const Group& b) { return a.tile < b.tile; });
  for (size_t s = 0, e = 0; s < gs.size(); s = e) {
    Groups G;
    std::memset(&G, 0, sizeof(G));
    int64_t blocks = 0;
    e = s;
    while (e < gs.size() && e - s < (size_t)kMaxGroups && gs[e].tile == gs[s].tile) ++e;
    for (size_t i = s; i < e; ++i) {
      Group g = gs[i];
      g.block0 = (int32_t)blocks;
      blocks += (int64_t)g.blocks_per_mat * g.count;
      G.g[G.n++] = g;
    }
    if (blocks == 0) continue;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    G.total_blocks = (int32_t)blocks;
    hipError_t err = go(G);
    if (err != hipSuccess) return err;
    if (launched) ++*launched;
  }
  return hipSuccess;
}

struct Bufs {
  char* base;
  int32_t* status;
  void* x[2][2];
  void* b[2];
  void* a[2];
  float* araw;
  float* vec;
  uint64_t* tag;   // tagged vectors of the one-launch power iteration
  float* part;
  float* kpart;
  void* gs[5];     // Gram-space A_even, A_odd, T, Q_even, Q_odd
  float* scal;
};

Bufs bind(const Plan& P, void* ws) {
  Bufs B;
  std::memset(&B, 0, sizeof(B));
  B.base = static_cast<char*>(ws);
  auto at = [&](size_t off) -> void* { return off ? B.base + off : nullptr; };
  B.status = reinterpret_cast<int32_t*>(B.base + P.off_status);
  for (int p = 0; p < 2; ++p)
    for (int h = 0; h < 2; ++h) {
      B.x[p][h] = at(P.off_x[p][h]);
    }
  B.b[0] = at(P.off_b[0]); B.b[1] = at(P.off_b[1]);
  B.a[0] = at(P.off_a[0]); B.a[1] = at(P.off_a[1]);
  B.araw = static_cast<float*>(at(P.off_araw));
  B.vec = static_cast<float*>(at(P.off_vec));
  B.tag = static_cast<uint64_t*>(at(P.off_tag));
  B.part = static_cast<float*>(at(P.off_part));
  B.kpart = static_cast<float*>(at(P.off_kpart));
  for (int j = 0; j < 5; ++j)
    B.gs[j] = P.off_gs ? B.base + P.off_gs + (size_t)j * P.r_total * 2 : nullptr;
  B.scal = static_cast<float*>(at(P.off_scal));
  return B;
}

std::once_flag g_attr_once[64];
hipError_t g_attr_err[64];

hipError_t ensure_attributes() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return gemm_set_attributes();
  std::call_once(g_attr_once[dev], [&] { g_attr_err[dev] = gemm_set_attributes(); });
  return g_attr_err[dev];
}

#define HIP_TRY(x)                         \
  do {                                     \
    hipError_t _e = (x);                   \
    if (_e != hipSuccess) return SM_EHIP;  \
  } while (0)

// Event after a phase (instrumented step only).
hipError_t mark(sm_profile* prof, int kind, hipStream_t s) {
  if (!prof || prof->count >= prof->capacity) return hipSuccess;
  hipError_t e = hipEventRecord(prof->events[prof->count], s);
  prof->kinds[prof->count++] = kind;
  return e;
}

// Start and stop events of one matrix-core launch (taken by the kernel
// itself): the interval up to its start is recorded as a gap, the kernel
// as `kind`.  Both null without a profile or room for two events.
struct KernelEvents { hipEvent_t t0 = nullptr, t1 = nullptr; };
KernelEvents kernel_events(sm_profile* prof, int kind) {
  KernelEvents k;
  if (!prof || prof->count + 2 > prof->capacity) return k;
  k.t0 = prof->events[prof->count];
  prof->kinds[prof->count++] = SM_PHASE_GAP;
  k.t1 = prof->events[prof->count];
  prof->kinds[prof->count++] = kind;
  return k;
}
hipError_t launch_gemm_timed(int precision, const GemmArgs& a, hipStream_t s, sm_profile* prof,
                             int kind) {
  const KernelEvents k = kernel_events(prof, kind);
  return launch_gemm(precision, a, s, k.t0, k.t1);
}

// ---------------------------------------------------------------------------
// PolarNS pipeline over all matrices of a plan, starting from the padded
// operand copies in x[0] with partial sums in part (Frobenius).
//   first: XS_USER (the first a X term from src_user, the caller's float32
//   source, e.g. the momentum) or XS_OP (from the operand copy, e.g. the
//   majority matrix, whose entries the operand holds exactly).
//   final: O_U (write U), O_BITS (pack into bits), O_TERN (int8 signs),
//   O_APPLY (update W).
// ---------------------------------------------------------------------------
struct NsIO {
  int first_xsrc;
  const float* src_user;
  int final_out;
  float* U;
  uint32_t* bits;         // local worker buffer base (packed signs)
  int8_t* tern;           // local worker buffer base (int8 signs, O_TERN)
  void* W; int w_bf16; float eta;
  const float* u0;
  const int32_t* status;
  sm_profile* prof;
};

// GEMM launch fields of a group whose gm / gn are set: the tile size, the
// tiles along n and the blocks per matrix (upper-triangular tiles of a
// symmetric output).
void set_gemm_tiles(Group& g, int prec, int epi) {
  int tm, tn;
  gemm_tile(prec, epi, g.gm, g.gn, g.gk, &tm, &tn);
  g.tile = tn;
  g.tiles_n = (g.gn + tn - 1) / tn;
  const int tiles_m = (g.gm + tm - 1) / tm;
  // only the Gram and the raw Gram (k = the long side) are split
  if (epi != E_OP && epi != E_RAW) g.ksplit = 1;
  g.blocks_per_mat = epi == E_UPDATE ? tiles_m * g.tiles_n
                                     : g.tiles_n * (g.tiles_n + 1) / 2 * (g.ksplit > 1 ? g.ksplit : 1);
}

// The enqueue of a PolarNS program is split into stages (one launch run
// each, plus its profiling mark), so that several independent programs can
// be enqueued interleaved: each stage is a closure over the program's
// arguments, which outlive the stage list.
using Stage = std::function<sm_status()>;
using Stages = std::vector<Stage>;

sm_status run_stages(const Stages& st) {
  for (const Stage& f : st) {
    const sm_status r = f();
    if (r != SM_OK) return r;
  }
  return SM_OK;
}

// Pre-scale: c = 1/(s+eps) per matrix, and (K > 0) the first Gram operand
// scaled by c^2.
// In the Gram-space form the first Gram also writes Q_1 = a I + b A_0 from
// its epilogue, unless one of the groups' Grams is split along k (then a
// separate elementwise pass makes Q_1).
bool gram_writes_q1(const Plan& P, const std::vector<Group>& groups) {
  if (!P.gram_space) return false;
  for (const Group& g : groups)
    if (g.ksplit > 1) return false;
  return true;
}

void pre_scale_stages(const Plan& P, const std::vector<MatPlan>& mp,
                      const std::vector<Group>& groups, const sm_hparams* hp, Bufs& B,
                      const NsIO& io, int part_kind, hipStream_t s, Stages& out) {
  const int prec = P.precision;
  const bool quin = P.quintic;
  // cubic folds b into B; the quintic and the Gram-space form keep A itself
  const float gram_mul = quin || P.gram_space ? 1.0f : hp->ns_b;
  // operand that receives the scaled first Gram
  void* dst_hi = P.gram_space ? B.gs[0] : quin ? B.a[0] : B.b[0];
  void* dst_lo = P.gram_space ? nullptr : quin ? B.a[1] : B.b[1];
  auto gram_fill = [&P, &mp, prec](Group& g) {
    const MatPlan& q = mp[g.idx0];
    g.gm = g.gn = (int32_t)q.Rp;
    g.gk = (int32_t)(q.tall ? q.Mp : q.Np);
    set_gemm_tiles(g, prec, P.spectral ? E_RAW : E_OP);
    g.ops = gemm_ops(FAM_X, FAM_X);   // S S^T
    return true;
  };
  if (!P.spectral) {
    out.push_back([&, hp, part_kind, s]() -> sm_status {
      HIP_TRY(for_launches(groups, [&](Group& g) {
        g.blocks_per_mat = 1;
        const int64_t mn = mp[g.idx0].rows * mp[g.idx0].cols;
        // partial sums per matrix: one per sweep tile (0), per packed vote
        // block (1) or per int8 vote block (2)
        g.gk = (int32_t)(part_kind == 0 ? mp[g.idx0].Mp * mp[g.idx0].Np / 4096
                         : part_kind == 1 ? vote_blocks_per_mat(VA_SBAR, mp[g.idx0].rows,
                                                                mp[g.idx0].cols)
                                          : tern_vote_blocks_per_mat(VA_SBAR, mp[g.idx0].rows,
                                                                     mp[g.idx0].cols));
        return true;
      }, [&](const Groups& G) { return launch_fro_finalize(G, B.part, hp->eps, B.scal, s); }));
      HIP_TRY(mark(io.prof, SM_PHASE_PRESCALE, s));
      return SM_OK;
    });
    if (hp->K == 0) return;
    out.push_back([&, hp, gram_fill, gram_mul, dst_hi, dst_lo, prec, s]() -> sm_status {
      HIP_TRY(for_launches(groups, gram_fill, [&](const Groups& G) {
        GemmArgs a;
        std::memset(&a, 0, sizeof(a));
        a.G = G;
        a.x_hi = B.x[0][0]; a.x_lo = B.x[0][1];
        a.epi = E_OP; a.upper = P.upper; a.mul = gram_mul; a.scal = B.scal; a.scal_pow = 2;
        a.kpart = B.kpart;
        a.o_hi = dst_hi; a.o_lo = dst_lo;
        if (gram_writes_q1(P, groups)) {
          a.o2_hi = B.gs[4]; a.o2_a = hp->ns_a; a.o2_b = hp->ns_b;
        }
        return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_GRAM);
      }));
      return SM_OK;
    });
    return;
  }
  // Small sets (few rows of raw Gram in all) run the P power steps and the
  // scale in one launch whose blocks keep their rows in LDS; the raw Gram
  // launch clears the tagged vectors they exchange.
  int64_t pblocks = 0, rp_max = 0;
  for (const Group& g : groups) {
    pblocks += mp[g.idx0].Rp / kPowerRows * g.count;
    rp_max = std::max<int64_t>(rp_max, mp[g.idx0].Rp);
  }
  const bool fused = power_iter_fused() && B.tag && pblocks <= kPowerIterMaxBlocks &&
                     rp_max <= kPowerIterMaxRp;
  out.push_back([&, hp, gram_fill, prec, fused, s]() -> sm_status {
    HIP_TRY(for_launches(groups, gram_fill, [&](const Groups& G) {
      GemmArgs a;
      std::memset(&a, 0, sizeof(a));
      a.G = G;
      a.x_hi = B.x[0][0]; a.x_lo = B.x[0][1];
      a.epi = E_RAW; a.o_raw = B.araw;
      a.kpart = B.kpart;
      if (fused) {
        a.tag = B.tag;
        a.tag_stride = P.v_total;
      }
      return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_GRAM);
    }));
    return SM_OK;
  });
  if (fused) {
    out.push_back([&, hp, gram_mul, dst_hi, dst_lo, prec, s]() -> sm_status {
      HIP_TRY(for_launches(groups, [&](Group& g) {
        g.blocks_per_mat = (int32_t)(mp[g.idx0].Rp / kPowerRows);
        return true;
      }, [&](const Groups& G) {
        PowerIterArgs pa;
        std::memset(&pa, 0, sizeof(pa));
        pa.G = G;
        pa.araw = B.araw; pa.va = B.vec; pa.vb = B.vec + P.v_total; pa.u0 = io.u0;
        pa.P = hp->P; pa.scaled_op = hp->K > 0 ? 1 : 0; pa.precision = prec;
        pa.mul = gram_mul; pa.eps = hp->eps; pa.scal = B.scal;
        pa.hi = dst_hi; pa.lo = dst_lo; pa.status = B.status;
        pa.tag = B.tag; pa.tag_stride = P.v_total;
        int64_t rpl = 0;
        for (int i = 0; i < G.n; ++i) rpl = std::max<int64_t>(rpl, mp[G.g[i].idx0].Rp);
        return launch_power_iter(pa, rpl, s);
      }));
      HIP_TRY(mark(io.prof, SM_PHASE_PRESCALE, s));
      return SM_OK;
    });
    return;
  }
  // power iteration: P >= 1 steps alternating va / vb (P is validated); the
  // first step reads the start vector (u0, or ones) directly, and with K > 0
  // the prescale launch derives the scale from the final vector itself, so a
  // separate finalize launch only runs for K = 0.
  float* va = B.vec;
  float* vb = B.vec + P.v_total;
  for (int p = 0; p < hp->P; ++p) {
    const bool first = p == 0;
    out.push_back([&, hp, va, vb, first, s]() -> sm_status {
      HIP_TRY(for_launches(groups, [&](Group& g) {
        g.blocks_per_mat = (int32_t)(mp[g.idx0].Rp / 16);
        return true;
      }, [&](const Groups& G) {
        return launch_power_step(G, B.araw, va, vb, io.u0, first, s);
      }));
      return SM_OK;
    });
    std::swap(va, vb);
  }
  if (hp->K == 0) {
    out.push_back([&, hp, va, s]() -> sm_status {
      HIP_TRY(for_launches(groups, [&](Group& g) { g.blocks_per_mat = 1; return true; },
                           [&](const Groups& G) {
                             return launch_power_finalize(G, va, hp->eps, B.scal, s);
                           }));
      HIP_TRY(mark(io.prof, SM_PHASE_PRESCALE, s));
      return SM_OK;
    });
    return;
  }
  out.push_back([&, hp, va, gram_mul, dst_hi, dst_lo, prec, s]() -> sm_status {
    HIP_TRY(for_launches(groups, [&](Group& g) {
      g.blocks_per_mat = (int32_t)(mp[g.idx0].Rp * mp[g.idx0].Rp / kChunk);
      return true;
    }, [&](const Groups& G) {
      return launch_prescale(G, prec, B.araw, B.scal, gram_mul, dst_hi, dst_lo, va,
                             hp->eps, s);
    }));
    HIP_TRY(mark(io.prof, SM_PHASE_PRESCALE, s));
    return SM_OK;
  });
}

sm_status run_pre_scale(const Plan& P, const std::vector<MatPlan>& mp,
                        const std::vector<Group>& groups, const sm_hparams* hp,
                        Bufs& B, const NsIO& io, int part_kind,
                        hipStream_t s) {
  Stages st;
  pre_scale_stages(P, mp, groups, hp, B, io, part_kind, s, st);
  return run_stages(st);
}

// B = b A + c A^2 from the operand A (quintic).
hipError_t run_square(const Plan& P, const std::vector<MatPlan>& mp,
                      const std::vector<Group>& groups, const sm_hparams* hp,
                      Bufs& B, hipStream_t s, sm_profile* prof) {
  return for_launches(groups, [&](Group& g) {
    const MatPlan& q = mp[g.idx0];
    g.gm = g.gn = g.gk = (int32_t)q.Rp;
    set_gemm_tiles(g, P.precision, E_SQUARE);
    g.ops = gemm_ops(FAM_R, FAM_R);
    return true;
  }, [&](const Groups& G) {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.G = G;
    a.r_hi = B.a[0]; a.r_lo = B.a[1];
    a.epi = E_SQUARE; a.upper = P.upper; a.cb = hp->ns_b; a.cc = hp->ns_c;
    a.sq_hi = B.a[0]; a.sq_lo = B.a[1];
    a.o_hi = B.b[0]; a.o_lo = B.b[1];
    return launch_gemm_timed(P.precision, a, s, prof, SM_PHASE_SQUARE);
  });
}

// The K Newton-Schulz steps in Gram space (bfloat16 cubic).  Every iterate
// is a polynomial in the first Gram A_0 = X_0 X_0^T times X_0: with
// P_k = a I + b A_k,
//   X_{k+1} = P_k X_k,  A_{k+1} = X_{k+1} X_{k+1}^T = P_k (P_k A_k),
// and the polynomials commute, so X_K = Q_K X_0 with Q_1 = P_0 and
// Q_{k+1} = P_k Q_k.  The steps run on Rp x Rp symmetric matrices
// (upper-triangular tiles, mirrored):
//   Q_{k+1} = a Q_k + b A_k Q_k,   T_k = a A_k + b A_k A_k,
//   A_{k+1} = a T_k + b A_k T_k,
// and one product Q_K S_0 gives the output (scaled by c, through the
// update kernel's epilogues).  A_0 comes from the pre-scale (c^2 S S^T).
// For a matrix m x n this executes about 2 m^2 n + 12 m^3 (upper-triangular)
// flops instead of 5 x 3 m^2 n for K = 5.
void gram_space_stages(const Plan& P, const std::vector<MatPlan>& mp,
                       const std::vector<Group>& groups,
                       const sm_hparams* hp, Bufs& B, const NsIO& io, hipStream_t s,
                       Stages& out) {
  const int prec = P.precision;
  const int K = hp->K;
  const float ca = hp->ns_a, cb = hp->ns_b;
  void* const Abuf[2] = {B.gs[0], B.gs[1]};
  void* const T = B.gs[2];
  void* const Qbuf[2] = {B.gs[3], B.gs[4]};
  // out = a Y + b X Y for symmetric, commuting X and Y
  auto product = [&](void* X, void* Y, void* O) {
    out.push_back([&, X, Y, O, prec, ca, cb, s]() -> sm_status {
      HIP_TRY(for_launches(groups, [&](Group& g) {
        const MatPlan& q = mp[g.idx0];
        g.gm = g.gn = g.gk = (int32_t)q.Rp;
        set_gemm_tiles(g, prec, E_SQUARE);
        g.ops = gemm_ops(FAM_R, FAM_R2);
        return true;
      }, [&](const Groups& G) {
        GemmArgs a;
        std::memset(&a, 0, sizeof(a));
        a.G = G;
        a.r_hi = X; a.r2_hi = Y;
        a.epi = E_SQUARE; a.upper = P.upper; a.cb = ca; a.cc = cb;
        a.sq_hi = Y;
        a.o_hi = O;
        return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_SQUARE);
      }));
      return SM_OK;
    });
  };
  // Q_1 = a I + b A_0 (unless the first Gram wrote it)
  if (!gram_writes_q1(P, groups)) out.push_back([&, prec, ca, cb, s]() -> sm_status {
    (void)prec;
    HIP_TRY(for_launches(groups, [&](Group& g) {
      const int64_t Rp = mp[g.idx0].Rp;
      g.blocks_per_mat = (int32_t)(Rp * Rp / kChunk);
      return true;
    }, [&](const Groups& G) { return launch_affine_ident(G, B.gs[0], ca, cb, B.gs[4], s); }));
    HIP_TRY(mark(io.prof, SM_PHASE_GEMM, s));
    return SM_OK;
  });
  for (int k = 0; k + 1 < K; ++k) {
    if (k >= 1) product(Abuf[k & 1], Qbuf[k & 1], Qbuf[(k + 1) & 1]);
    product(Abuf[k & 1], Abuf[k & 1], T);
    product(Abuf[k & 1], T, Abuf[(k + 1) & 1]);
  }
  if (K >= 2) product(Abuf[(K - 1) & 1], Qbuf[(K - 1) & 1], Qbuf[K & 1]);
  void* const QK = Qbuf[K & 1];
  // X_K = c Q_K S_0 into the requested output
  out.push_back([&, QK, prec, s]() -> sm_status {
    HIP_TRY(for_launches(groups, [&](Group& g) {
      const MatPlan& q = mp[g.idx0];
      g.gm = (int32_t)q.Rp; g.gn = (int32_t)(q.tall ? q.Mp : q.Np);
      g.gk = (int32_t)q.Rp;
      set_gemm_tiles(g, prec, E_UPDATE);
      g.ops = gemm_ops(FAM_R, FAM_XK);
      return true;
    }, [&](const Groups& G) {
      GemmArgs a;
      std::memset(&a, 0, sizeof(a));
      a.G = G;
      a.x_hi = B.x[0][0]; a.x_lo = B.x[0][1];
      a.r_hi = QK;
      a.epi = E_UPDATE; a.upper = P.upper; a.ca = 0.0f; a.xsrc = XS_OP;
      a.scal = B.scal; a.scal_pow = 1;
      a.out = io.final_out;
      a.U = io.U; a.bits = io.bits; a.tern = io.tern;
      a.W = io.W; a.w_bf16 = io.w_bf16; a.eta = io.eta;
      a.status = io.status;
      return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_UPDATE);
    }));
    return SM_OK;
  });
}

// The K Newton-Schulz steps: step k reads the iterate from x[(k-1) & 1]
// and writes x[k & 1] (the last one writes the final output instead).
void ns_stages(const Plan& P, const std::vector<MatPlan>& mp,
               const std::vector<Group>& groups,
               const sm_hparams* hp, Bufs& B, const NsIO& io, hipStream_t s, Stages& out) {
  if (P.gram_space) {
    gram_space_stages(P, mp, groups, hp, B, io, s, out);
    return;
  }
  const int prec = P.precision;
  const int K = hp->K;
  for (int k = 1; k <= K; ++k) {
    const int cur = (k - 1) & 1;
    if (k > 1) {
      // Gram of the current iterate: cubic -> B = b A, quintic -> A
      out.push_back([&, hp, cur, prec, s]() -> sm_status {
        HIP_TRY(for_launches(groups, [&](Group& g) {
          const MatPlan& q = mp[g.idx0];
          g.gm = g.gn = (int32_t)q.Rp;
          g.gk = (int32_t)(q.tall ? q.Mp : q.Np);
          set_gemm_tiles(g, prec, E_OP);
          g.ops = gemm_ops(FAM_X, FAM_X);   // S S^T
          return true;
        }, [&](const Groups& G) {
          GemmArgs a;
          std::memset(&a, 0, sizeof(a));
          a.G = G;
          a.x_hi = B.x[cur][0]; a.x_lo = B.x[cur][1];
          a.epi = E_OP; a.upper = P.upper; a.mul = P.quintic ? 1.0f : hp->ns_b; a.scal_pow = 0;
          a.kpart = B.kpart;
          a.o_hi = P.quintic ? B.a[0] : B.b[0];
          a.o_lo = P.quintic ? B.a[1] : B.b[1];
          return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_GRAM);
        }));
        return SM_OK;
      });
    }
    if (P.quintic) {
      out.push_back([&, hp, s]() -> sm_status {
        HIP_TRY(run_square(P, mp, groups, hp, B, s, io.prof));
        return SM_OK;
      });
    }
    // update: S <- a S + B S
    out.push_back([&, hp, k, K, cur, prec, s]() -> sm_status {
      const bool last = k == K;
      HIP_TRY(for_launches(groups, [&](Group& g) {
        const MatPlan& q = mp[g.idx0];
        g.gm = (int32_t)q.Rp; g.gn = (int32_t)(q.tall ? q.Mp : q.Np);
        g.gk = (int32_t)q.Rp;
        set_gemm_tiles(g, prec, E_UPDATE);
        g.ops = gemm_ops(FAM_R, FAM_XK);
        return true;
      }, [&](const Groups& G) {
        GemmArgs a;
        std::memset(&a, 0, sizeof(a));
        a.G = G;
        a.x_hi = B.x[cur][0]; a.x_lo = B.x[cur][1];
        a.r_hi = B.b[0]; a.r_lo = B.b[1];
        a.epi = E_UPDATE; a.upper = P.upper; a.ca = hp->ns_a;
        a.xsrc = k == 1 ? io.first_xsrc : XS_OP;
        a.xs_user = io.src_user;
        a.scal = B.scal; a.scal_pow = k == 1 ? 1 : 0;
        if (!last) {
          a.out = O_X;
          a.o_hi = B.x[cur ^ 1][0]; a.o_lo = B.x[cur ^ 1][1];
        } else {
          a.out = io.final_out;
          a.U = io.U; a.bits = io.bits; a.tern = io.tern;
          a.W = io.W; a.w_bf16 = io.w_bf16; a.eta = io.eta;
          a.status = io.status;
        }
        return launch_gemm_timed(prec, a, s, io.prof, SM_PHASE_UPDATE);
      }));
      return SM_OK;
    });
  }
}

sm_status run_ns(const Plan& P, const std::vector<MatPlan>& mp,
                 const std::vector<Group>& groups,
                 const sm_hparams* hp, Bufs& B, const NsIO& io, hipStream_t s) {
  Stages st;
  ns_stages(P, mp, groups, hp, B, io, s, st);
  return run_stages(st);
}

// ---------------------------------------------------------------------------
// PolarNS of all groups as up to kChains independent chains (pre-scale and
// the K Newton-Schulz steps of a subset of the groups each), run on the
// streams of a caller-owned executor, forked from and joined back into the
// caller's stream.
// A chain's launches depend only on its own matrices, so the GPU runs the
// chains side by side and one chain's next launch fills the tail of
// another's.  The chains' launches are enqueued interleaved, one stage of
// each chain in turn, so that no chain waits for the host to enqueue the
// others.  With one group everything runs on the caller's stream.
// Three chains: with the caller's stream they take four hardware queues,
// HIP's default per process; a fourth stream would share a queue with
// another chain and run behind it.
// ---------------------------------------------------------------------------
constexpr int kChains = 3;
#ifndef SM_CHAIN_MIN_GFLOP
#define SM_CHAIN_MIN_GFLOP 200
#endif
// Newton-Schulz flops per call below which one chain is used; the
// environment variable SIGNMUON_CHAIN_MIN_GFLOP (read at every call)
// overrides the default, e.g. 0 to always use the chains.
double chain_min_flop() {
  const char* e = std::getenv("SIGNMUON_CHAIN_MIN_GFLOP");
  if (e && *e) {
    char* end = nullptr;
    const double v = std::strtod(e, &end);
    if (end != e && v >= 0.0) return v * 1e9;
  }
  return SM_CHAIN_MIN_GFLOP * 1e9;
}
}  // namespace

// Caller-owned resources of the concurrent chains (signmuon_executor_create):
// the chains' streams, created on `device`, and for each of the (at most
// two) PolarNS passes of one step its own fork and join events, so no event
// is recorded twice within a step.  `mu` keeps two threads from
// enqueueing through one executor at the same time.
struct sm_executor {
  int device = -1;
  hipStream_t s[kChains] = {};
  hipEvent_t fork[2] = {};
  hipEvent_t join[2][kChains] = {};
  std::mutex mu;
};

namespace {

sm_status run_polar(const Plan& P, const std::vector<MatPlan>& mp,
                    const std::vector<Group>& groups,
                    const sm_hparams* hp, Bufs& B, const NsIO& io, int part_kind,
                    hipStream_t s, sm_executor* ex, int pass) {
  // Sets with little Newton-Schulz work are bound by the host's launch
  // rate: one chain puts all their groups into each launch (up to
  // kMaxGroups per launch), a third of the launches of three chains.
  // Without an executor, or while the caller's stream is being captured
  // into a graph, everything runs as one chain on the caller's stream.
  double ns_flop = 0.0;
  for (const Group& g : groups) {
    const double m = std::min(g.rows, g.cols), n = std::max(g.rows, g.cols);
    ns_flop += 4.0 * hp->K * g.count * m * m * n;
  }
  int nc = ns_flop < chain_min_flop() ? 1 : (int)std::min<size_t>(kChains, groups.size());
  if (nc > 1) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(s, &cap));
    if (!ex || cap != hipStreamCaptureStatusNone) nc = 1;
  }
  if (nc <= 1) {
    Stages st;
    pre_scale_stages(P, mp, groups, hp, B, io, part_kind, s, st);
    if (hp->K > 0) ns_stages(P, mp, groups, hp, B, io, s, st);
    return run_stages(st);
  }
  // longest-processing-time assignment of the groups to the chains, by
  // Newton-Schulz work count * m^2 * n
  std::vector<int> order(groups.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  auto work = [&](const Group& g) {
    const double m = std::min(g.rows, g.cols), n = std::max(g.rows, g.cols);
    return (double)g.count * m * m * n;
  };
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return work(groups[a]) > work(groups[b]); });
  std::vector<std::vector<Group>> chain(nc);
  std::vector<double> load(nc, 0.0);
  for (int i : order) {
    const int c = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    chain[c].push_back(groups[i]);
    load[c] += work(groups[i]);
  }
  // The chain with the most matrices runs on the caller's stream itself:
  // it starts right after the momentum pass without waiting on another
  // queue, and the vote after the join follows it on the same queue.  (Its
  // launches hold the most blocks and take the larger share of the CUs, so
  // on the nanoGPT-shaped set it ends before the other chains, and the vote
  // still waits for their join events.)
  int home = -1;
  if (caller_chain_enabled()) {
    int most = -1;
    for (int c = 0; c < nc; ++c) {
      int n = 0;
      for (const Group& g : chain[c]) n += g.count;
      if (n > most) { most = n; home = c; }
    }
  }
  sm_executor* R = ex;
  std::lock_guard<std::mutex> lock(R->mu);
  hipEvent_t* join_ev = R->join[pass];
  auto stream_of = [&](int c) { return c == home ? s : R->s[c]; };
  HIP_TRY(hipEventRecord(R->fork[pass], s));
  NsIO cio = io;
  cio.prof = nullptr;
  std::vector<Stages> prog(nc);
  for (int c = 0; c < nc; ++c) {
    hipStream_t cs = stream_of(c);
    pre_scale_stages(P, mp, chain[c], hp, B, cio, part_kind, cs, prog[c]);
    if (hp->K > 0) ns_stages(P, mp, chain[c], hp, B, cio, cs, prog[c]);
  }
  sm_status st = SM_OK;
  int forked = 0;
  for (int c = 0; c < nc && st == SM_OK; ++c) {
    if (c != home && hipStreamWaitEvent(R->s[c], R->fork[pass], 0) != hipSuccess) {
      st = SM_EHIP;
      break;
    }
    ++forked;
  }
  size_t longest = 0;
  for (const Stages& p : prog) longest = std::max(longest, p.size());
  for (size_t i = 0; i < longest && st == SM_OK; ++i)
    for (int c = 0; c < forked && st == SM_OK; ++c)
      if (i < prog[c].size()) st = prog[c][i]();
  // join every forked chain, also after an error, so that the caller's
  // stream orders after all work enqueued on the chains
  for (int c = 0; c < forked; ++c) {
    if (c == home) continue;
    if (hipEventRecord(join_ev[c], R->s[c]) != hipSuccess ||
        hipStreamWaitEvent(s, join_ev[c], 0) != hipSuccess)
      st = SM_EHIP;
  }
  if (st != SM_OK) return st;
  HIP_TRY(mark(io.prof, SM_PHASE_GEMM, s));
  return SM_OK;
}

void set_vec_ok(std::vector<Group>& groups, bool ptrs_aligned) {
  for (Group& g : groups)
    g.vec_ok = ptrs_aligned && g.elem0 % 8 == 0 && g.elem_stride % 8 == 0 &&
               g.cols % 8 == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// ===========================================================================
// Exported entry points
// ===========================================================================
extern "C" {

const char* signmuon_strerror(int status) {
  switch (status) {
    case SM_OK: return "ok";
    case SM_EINVAL: return "invalid argument";
    case SM_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SM_EHIP: return "HIP runtime or launch error";
    case SM_ENONFINITE: return "non-finite gradient, weight or momentum; update skipped";
    case SM_ERANGE: return "worker count or size out of range";
    case SM_EUNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

int32_t signmuon_abi_version(void) { return kAbiVersion; }

sm_status signmuon_momentum(const float* G, const void* W, int32_t w_dtype,
                            float* Mom, int64_t n, float beta, float lambda,
                            hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (w_dtype != SM_F32 && w_dtype != SM_BF16) return SM_EINVAL;
  if (!finite(beta) || beta < 0.f || beta >= 1.f) return SM_EINVAL;
  if (!finite(lambda) || lambda < 0.f) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!G || !W || !Mom) return SM_EINVAL;
  HIP_TRY(launch_momentum_flat(G, W, w_dtype == SM_BF16, Mom, n, beta, lambda, stream));
  return SM_OK;
}

sm_status signmuon_sign_pack(const float* U, uint32_t* bits, int64_t n,
                             hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!U || !bits) return SM_EINVAL;
  HIP_TRY(launch_sign_pack_flat(U, bits, n, stream));
  return SM_OK;
}

sm_status signmuon_majority_vote(const uint32_t* bits, int64_t worker_stride_words,
                                 int32_t M, int64_t n, int32_t tie_value, int8_t* D,
                                 int16_t* sums, hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (M < 1 || M > SM_MAX_WORKERS) return SM_ERANGE;
  if (tie_value != 0 && tie_value != 1) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!bits || !D) return SM_EINVAL;
  if (M > 1 && worker_stride_words < (n + 31) / 32) return SM_EINVAL;
  if (worker_stride_words < 0) return SM_EINVAL;
  HIP_TRY(launch_vote_flat(bits, worker_stride_words, M, n, tie_value, D, sums, stream));
  return SM_OK;
}

sm_status signmuon_sign_ternary(const float* U, int8_t* S, int64_t n, hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!U || !S) return SM_EINVAL;
  if (n > ((int64_t)1 << 36)) return SM_EINVAL;   // grid of n / 4096 blocks
  HIP_TRY(launch_sign_ternary(U, S, n, stream));
  return SM_OK;
}

sm_status signmuon_majority_vote_ternary(const int8_t* S, int64_t worker_stride, int32_t M,
                                         int64_t n, int32_t tie_value, int8_t* D,
                                         int16_t* sums, hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (M < 1 || M > SM_MAX_WORKERS) return SM_ERANGE;
  if (tie_value != 0 && tie_value != 1) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!S || !D) return SM_EINVAL;
  if (worker_stride < 0 || (M > 1 && worker_stride < n)) return SM_EINVAL;
  if (n > ((int64_t)1 << 36)) return SM_EINVAL;   // grid of n / 4096 blocks
  HIP_TRY(launch_vote_ternary(S, worker_stride, M, n, tie_value, D, sums, stream));
  return SM_OK;
}

sm_status signmuon_apply(void* W, int32_t w_dtype, const int8_t* D, const float* Df,
                         float eta, int64_t n, hipStream_t stream) {
  if (n < 0) return SM_EINVAL;
  if (w_dtype != SM_F32 && w_dtype != SM_BF16) return SM_EINVAL;
  if ((D == nullptr) == (Df == nullptr)) return SM_EINVAL;
  if (!finite(eta)) return SM_EINVAL;
  if (n == 0) return SM_OK;
  if (!W) return SM_EINVAL;
  HIP_TRY(launch_apply_flat(W, w_dtype == SM_BF16, D, Df, eta, n, stream));
  return SM_OK;
}

size_t signmuon_polar_ns_workspace(int64_t rows, int64_t cols, const sm_hparams* hp) {
  if (check_hparams(hp, false) != SM_OK) return 0;
  sm_matrix m{rows, cols, 0, 0};
  Plan P;
  std::vector<MatPlan> mp;
  if (build_plan(&m, 1, hp, 0, P, mp) != SM_OK) return 0;
  return P.total;
}

sm_status signmuon_polar_ns(const float* X, float* U, int64_t rows, int64_t cols,
                            const sm_hparams* hp, const float* u0, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  sm_status st = check_hparams(hp, false);
  if (st != SM_OK) return st;
  if (!X || !U || X == U) return SM_EINVAL;
  sm_matrix m{rows, cols, 0, 0};
  Plan P;
  std::vector<MatPlan> mp;
  st = build_plan(&m, 1, hp, 0, P, mp);
  if (st != SM_OK) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < P.total)
    return SM_EWORKSPACE;
  HIP_TRY(ensure_attributes());
  Bufs B = bind(P, ws);
  std::vector<Group> groups = make_groups(mp, {0});
  set_vec_ok(groups, aligned16(X));
  SweepArgs sw;
  std::memset(&sw, 0, sizeof(sw));
  sw.ema = 0; sw.precision = P.precision; sw.src = X;
  sw.o_hi = B.x[0][0]; sw.o_lo = B.x[0][1]; sw.part = B.part;
  HIP_TRY(for_launches(groups, [&](Group& g) {
    g.blocks_per_mat = (int32_t)(mp[g.idx0].Mp * mp[g.idx0].Np / 4096);
    return true;
  }, [&](const Groups& G) { sw.G = G; return launch_sweep(sw, stream); }));
  NsIO io;
  std::memset(&io, 0, sizeof(io));
  io.first_xsrc = XS_USER; io.src_user = X; io.final_out = O_U; io.U = U; io.u0 = u0;
  st = run_pre_scale(P, mp, groups, hp, B, io, 0, stream);
  if (st != SM_OK) return st;
  if (hp->K == 0) {
    ScaledOutArgs so;
    std::memset(&so, 0, sizeof(so));
    so.x_user = X; so.scal = B.scal; so.U = U;
    HIP_TRY(for_launches(groups, [&](Group& g) {
      g.blocks_per_mat = (int32_t)((rows * cols + kChunk - 1) / kChunk);
      return true;
    }, [&](const Groups& G) { so.G = G; return launch_scaled_out(so, stream); }));
    return SM_OK;
  }
  return run_ns(P, mp, groups, hp, B, io, stream);
}

}  // extern "C"

// Scratch memory of signmuon_polar_ns_static: one array per GPU, held from
// the library's load until the process ends and shared by every such call
// on that GPU.  In host code `scratch` names a host-side stand-in, not the
// device array: kernels and copies get the device address that
// hipGetSymbolAddress returns (scratch_on_device), never `scratch`.
static __device__ __align__(256) char scratch[SM_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device with that device current.
hipError_t scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}
}  // namespace

extern "C" {

sm_status signmuon_polar_ns_static(const float* X, float* U, int64_t rows, int64_t cols,
                                   const sm_hparams* hp, const float* u0,
                                   hipStream_t stream) {
  const sm_status st = check_hparams(hp, false);
  if (st != SM_OK) return st;
  if (!X || !U || X == U) return SM_EINVAL;
  const size_t need = signmuon_polar_ns_workspace(rows, cols, hp);
  if (need == 0) return SM_EINVAL;
  if (need > SM_STATIC_SCRATCH_BYTES) return SM_ERANGE;
  void* ws = nullptr;
  if (scratch_on_device(&ws) != hipSuccess || !ws) return SM_EHIP;
  return signmuon_polar_ns(X, U, rows, cols, hp, u0, ws, SM_STATIC_SCRATCH_BYTES, stream);
}

size_t signmuon_step_workspace(const sm_matrix* mats, int32_t n_mats,
                               const sm_hparams* hp, int32_t post_vote) {
  if (!mats || n_mats < 1 || n_mats > 65536) return 0;
  if (check_hparams(hp, true) != SM_OK) return 0;
  if (post_vote < 0 || post_vote > 3) return 0;
  if (post_vote == 3 && (hp->P < 1 || hp->P > 256)) return 0;
  Plan P;
  std::vector<MatPlan> mp;
  if (build_plan(mats, n_mats, hp, post_vote, P, mp) != SM_OK) return 0;
  return P.total;
}

}  // extern "C"

namespace {
sm_status step_impl(const sm_matrix* mats, int32_t n_mats, const sm_hparams* hp,
                    const float* G, void* W, int32_t w_dtype, float* Mom,
                    uint32_t* bits, int64_t worker_stride_words, int32_t M,
                    int32_t local_worker, int32_t post_vote, const float* u0,
                    void* ws, size_t ws_bytes, sm_profile* prof, sm_executor* ex,
                    hipStream_t stream, bool pipeline_only = false) {
  if (prof) {
    if (!prof->events || !prof->kinds || prof->capacity < 0) return SM_EINVAL;
    prof->count = 0;
  }
  if (!mats || n_mats < 1 || n_mats > 65536) return SM_EINVAL;
  sm_status st = check_hparams(hp, true);
  if (st != SM_OK) return st;
  if (M < 1 || M > SM_MAX_WORKERS) return SM_ERANGE;
  if (local_worker < 0 || local_worker >= M) return SM_EINVAL;
  if (post_vote < 0 || post_vote > 3) return SM_EINVAL;
  if (post_vote == 3 && (hp->P < 1 || hp->P > 256)) return SM_EINVAL;
  if (w_dtype != SM_F32 && w_dtype != SM_BF16) return SM_EINVAL;
  if (!G || !W || !Mom || !bits) return SM_EINVAL;
  if (worker_stride_words < 0) return SM_EINVAL;
  // int8 sign buffers: worker_stride_words counts bytes, and a matrix's
  // signs sit at its element offset
  const bool tern = hp->sign_encoding == SM_SIGNS_TERNARY;
  // shapes, offsets and overlap
  {
    std::vector<std::pair<int64_t, int64_t>> es, wsg;
    for (int i = 0; i < n_mats; ++i) {
      const sm_matrix& m = mats[i];
      if (m.rows < 1 || m.cols < 1 || m.rows > kMaxDim || m.cols > kMaxDim) return SM_EINVAL;
      if (m.elem_off < 0 || m.word_off < 0) return SM_EINVAL;
      int64_t mn = m.rows * m.cols, nw = (mn + 31) / 32;
      if (tern ? m.elem_off + mn > worker_stride_words : m.word_off + nw > worker_stride_words)
        return SM_EINVAL;
      es.push_back({m.elem_off, m.elem_off + mn});
      wsg.push_back(tern ? std::make_pair(m.elem_off, m.elem_off + mn)
                         : std::make_pair(m.word_off, m.word_off + nw));
    }
    std::sort(es.begin(), es.end());
    std::sort(wsg.begin(), wsg.end());
    for (int i = 1; i < n_mats; ++i)
      if (es[i].first < es[i - 1].second || wsg[i].first < wsg[i - 1].second) return SM_EINVAL;
  }
  // the signs (packed or int8) are written from the last epilogue for every
  // width (packed words that span two lines of X take their bits by atomics)
  Plan P;
  std::vector<MatPlan> mp;
  st = build_plan(mats, n_mats, hp, post_vote, P, mp);
  if (st != SM_OK) return st;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < P.total)
    return SM_EWORKSPACE;
  if (ex) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != ex->device) return SM_EINVAL;
  }
  HIP_TRY(ensure_attributes());
  Bufs B = bind(P, ws);
  std::vector<int> all(n_mats);
  for (int i = 0; i < n_mats; ++i) all[i] = i;
  std::vector<Group> groups = make_groups(mp, all);
  set_vec_ok(groups, aligned16(G) && aligned16(W) && aligned16(Mom));
  uint32_t* local_bits = tern ? nullptr : bits + (int64_t)local_worker * worker_stride_words;
  int8_t* const tern_bufs = tern ? reinterpret_cast<int8_t*>(bits) : nullptr;
  int8_t* local_tern = tern ? tern_bufs + (int64_t)local_worker * worker_stride_words : nullptr;
  const int w_bf16 = w_dtype == SM_BF16;
  HIP_TRY(mark(prof, SM_PHASE_START, stream));
  // A step takes over the flags of the worker pipelines enqueued since the
  // last step (word 1) as its own (word 0); a worker pipeline adds its flag
  // to word 1, so a non-finite value in any worker's pipeline of a step
  // skips that step's update.
  int32_t* const flag = pipeline_only ? B.status + 1 : B.status;
  if (!pipeline_only) HIP_TRY(launch_begin_status(B.status, stream));

  NsIO io;
  std::memset(&io, 0, sizeof(io));
  io.u0 = u0; io.status = B.status; io.prof = prof;
  io.W = W; io.w_bf16 = w_bf16; io.eta = hp->eta;

  VoteArgs va;
  std::memset(&va, 0, sizeof(va));
  va.M = M; va.tie = hp->tie_value; va.w_bf16 = w_bf16; va.precision = P.precision;
  va.bits = tern ? nullptr : bits; va.tern = tern_bufs; va.stride = worker_stride_words;
  va.W = W; va.eta = hp->eta; va.status = B.status;
  auto vote_blocks = [tern](int mode, const Group& g) {
    return tern ? (int32_t)tern_vote_blocks_per_mat(mode, g.rows, g.cols)
                : vote_blocks_per_mat(mode, g.rows, g.cols);
  };
  auto vote_fill = [&](Group& g) {
    g.blocks_per_mat = vote_blocks(va.mode, g);
    return true;
  };

  // post_vote 0, 2 and 3: the local worker's pre-sign pipeline (momentum,
  // PolarNS, signs); 0 then votes and applies the majority, 2 goes on to the
  // post-vote polar step below, 3 to the normalized sign step.
  if (post_vote != 1) {
    if (hp->K == 0) {
      // U = Mom/(s+eps) has the signs of Mom: pack them directly.
      MomSignArgs ms;
      std::memset(&ms, 0, sizeof(ms));
      ms.w_bf16 = w_bf16; ms.beta = hp->beta; ms.lam = hp->lambda;
      ms.Gr = G; ms.W = W; ms.Mom = Mom; ms.bits = local_bits; ms.tern = local_tern;
      ms.status = flag;
      HIP_TRY(for_launches(groups, [&](Group& g) {
        g.blocks_per_mat = (int32_t)(((int64_t)g.rows * g.cols + kChunk - 1) / kChunk);
        return true;
      }, [&](const Groups& Gs) {
        ms.G = Gs;
        const KernelEvents k = kernel_events(prof, SM_PHASE_MOMENTUM);
        return launch_momentum_sign(ms, stream, k.t0, k.t1);
      }));
    } else {
      SweepArgs sw;
      std::memset(&sw, 0, sizeof(sw));
      sw.ema = 1; sw.precision = P.precision; sw.w_bf16 = w_bf16;
      sw.beta = hp->beta; sw.lam = hp->lambda;
      sw.Gr = G; sw.W = W; sw.Mom = Mom;
      sw.o_hi = B.x[0][0]; sw.o_lo = B.x[0][1];
      sw.part = P.spectral ? nullptr : B.part;
      sw.status = flag;
      auto sweep_fill = [&](Group& g) {
        g.blocks_per_mat = (int32_t)(mp[g.idx0].Mp * mp[g.idx0].Np / 4096);
        return true;
      };
      io.first_xsrc = XS_USER; io.src_user = Mom;
      io.final_out = tern ? O_TERN : O_BITS; io.bits = local_bits; io.tern = local_tern;
      io.U = nullptr;
      // profiled: the sweep's own start and stop times (the interval before
      // it, with the status launch, closes as a gap)
      HIP_TRY(for_launches(groups, sweep_fill, [&](const Groups& Gs) {
        sw.G = Gs;
        const KernelEvents k = kernel_events(prof, SM_PHASE_MOMENTUM);
        return launch_sweep(sw, stream, k.t0, k.t1);
      }));
      st = run_polar(P, mp, groups, hp, B, io, 0, stream, ex, 0);
      if (st != SM_OK) return st;
    }
    if (pipeline_only) return SM_OK;
    if (post_vote == 0) {
      va.mode = VA_APPLY;
      HIP_TRY(for_launches(groups, vote_fill, [&](const Groups& Gs) {
        va.G = Gs;
        const KernelEvents k = kernel_events(prof, SM_PHASE_VOTE);
        return launch_vote_groups(va, stream, k.t0, k.t1);
      }));
      return SM_OK;
    }
  } else {
    // ---- post-vote variant: the local worker sends the momentum's signs
    MomSignArgs ms;
    std::memset(&ms, 0, sizeof(ms));
    ms.w_bf16 = w_bf16; ms.beta = hp->beta; ms.lam = hp->lambda;
    ms.Gr = G; ms.W = W; ms.Mom = Mom; ms.bits = local_bits; ms.tern = local_tern;
    ms.status = flag;
    HIP_TRY(for_launches(groups, [&](Group& g) {
      g.blocks_per_mat = (int32_t)(((int64_t)g.rows * g.cols + kChunk - 1) / kChunk);
      return true;
    }, [&](const Groups& Gs) {
      ms.G = Gs;
      const KernelEvents k = kernel_events(prof, SM_PHASE_MOMENTUM);
      return launch_momentum_sign(ms, stream, k.t0, k.t1);
    }));
    if (pipeline_only) return SM_OK;
  }

  // ---- post_vote 1 and 2: majority matrix, its polar factor, the update;
  // post_vote 3: majority matrix D, ||D||_2 by power iteration, and
  // W <- W - eta D / (||D||_2 + eps).
  // (The pre-sign pass of post_vote 2 and 3 has finished with the operand
  // and partial-sum buffers on this stream before the vote rewrites them.)
  // padding of the operand copy (only matrices with a ragged shape)
  HIP_TRY(for_launches(groups, [&](Group& g) {
    const MatPlan& q = mp[g.idx0];
    if (q.Mp == q.rows && q.Np == q.cols) return false;
    g.blocks_per_mat = (int32_t)(q.Mp * q.Np / kChunk);
    return true;
  }, [&](const Groups& Gs) {
    return launch_zero_pad(Gs, P.precision, B.x[0][0], B.x[0][1], stream);
  }));
  va.mode = VA_SBAR;
  va.o_hi = B.x[0][0]; va.o_lo = B.x[0][1];
  va.part = B.part;
  HIP_TRY(for_launches(groups, vote_fill, [&](const Groups& Gs) {
    va.G = Gs;
    const KernelEvents k = kernel_events(prof, SM_PHASE_VOTE);
    return launch_vote_groups(va, stream, k.t0, k.t1);
  }));
  io.first_xsrc = XS_OP; io.src_user = nullptr;
  io.final_out = O_APPLY;
  if (post_vote != 3 && hp->K > 0) {
    return run_polar(P, mp, groups, hp, B, io, tern ? 2 : 1, stream, ex,
                     post_vote == 2 ? 1 : 0);
  }
  // W <- W - eta c S with c = 1/(s + eps): the post-vote step with K = 0, or
  // the normalized sign step (a spectral pre-scale without Newton-Schulz
  // steps on the majority matrix, whose power vectors the plan holds)
  Plan Pn = P;
  sm_hparams hn = *hp;
  if (post_vote == 3) {
    Pn.spectral = true;
    Pn.gram_space = false;
    hn.scale = SM_SCALE_SPECTRAL;
    hn.K = 0;
  }
  st = run_pre_scale(Pn, mp, groups, &hn, B, io, tern ? 2 : 1, stream);
  if (st != SM_OK) return st;
  // the update votes again from the sign buffers (the M buffers cost M/8
  // (packed) or M bytes per entry, and are read in the caller's layout,
  // whereas the operand copy of a tall matrix is transposed), scaled by c
  va.mode = VA_APPLY;
  va.scal = B.scal;
  HIP_TRY(for_launches(groups, vote_fill, [&](const Groups& Gs) {
    va.G = Gs;
    const KernelEvents k = kernel_events(prof, SM_PHASE_VOTE);
    return launch_vote_groups(va, stream, k.t0, k.t1);
  }));
  return SM_OK;
}
}  // namespace

extern "C" {

sm_status signmuon_executor_create(sm_executor** out) {
  if (!out) return SM_EINVAL;
  *out = nullptr;
  sm_executor* ex = new (std::nothrow) sm_executor;
  if (!ex) return SM_EHIP;
  hipError_t e = hipGetDevice(&ex->device);
  for (int c = 0; c < kChains && e == hipSuccess; ++c)
    e = hipStreamCreateWithFlags(&ex->s[c], hipStreamNonBlocking);
  for (int p = 0; p < 2 && e == hipSuccess; ++p) {
    e = hipEventCreateWithFlags(&ex->fork[p], hipEventDisableTiming);
    for (int c = 0; c < kChains && e == hipSuccess; ++c)
      e = hipEventCreateWithFlags(&ex->join[p][c], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    signmuon_executor_destroy(ex);
    return SM_EHIP;
  }
  *out = ex;
  return SM_OK;
}

sm_status signmuon_executor_destroy(sm_executor* ex) {
  if (!ex) return SM_OK;
  int prev = 0;
  const bool have_prev = hipGetDevice(&prev) == hipSuccess;
  if (ex->device >= 0) (void)hipSetDevice(ex->device);
  sm_status st = SM_OK;
  for (int c = 0; c < kChains; ++c)
    if (ex->s[c] && hipStreamSynchronize(ex->s[c]) != hipSuccess) st = SM_EHIP;
  for (int p = 0; p < 2; ++p) {
    if (ex->fork[p]) (void)hipEventDestroy(ex->fork[p]);
    for (int c = 0; c < kChains; ++c)
      if (ex->join[p][c]) (void)hipEventDestroy(ex->join[p][c]);
  }
  for (int c = 0; c < kChains; ++c)
    if (ex->s[c]) (void)hipStreamDestroy(ex->s[c]);
  if (have_prev) (void)hipSetDevice(prev);
  delete ex;
  return st;
}

sm_status signmuon_step(const sm_matrix* mats, int32_t n_mats, const sm_hparams* hp,
                        const float* G, void* W, int32_t w_dtype, float* Mom,
                        uint32_t* bits, int64_t worker_stride_words, int32_t M,
                        int32_t local_worker, int32_t post_vote, const float* u0,
                        void* ws, size_t ws_bytes, sm_executor* ex, hipStream_t stream) {
  return step_impl(mats, n_mats, hp, G, W, w_dtype, Mom, bits, worker_stride_words, M,
                   local_worker, post_vote, u0, ws, ws_bytes, nullptr, ex, stream);
}

sm_status signmuon_worker_pipeline(const sm_matrix* mats, int32_t n_mats,
                                   const sm_hparams* hp, const float* G, const void* W,
                                   int32_t w_dtype, float* Mom, uint32_t* bits,
                                   int64_t worker_stride_words, int32_t M, int32_t worker,
                                   int32_t post_vote, const float* u0, void* ws,
                                   size_t ws_bytes, sm_executor* ex, hipStream_t stream) {
  // W is only read on this path
  return step_impl(mats, n_mats, hp, G, const_cast<void*>(W), w_dtype, Mom, bits,
                   worker_stride_words, M, worker, post_vote, u0, ws, ws_bytes, nullptr, ex,
                   stream, true);
}

sm_status signmuon_step_profiled(const sm_matrix* mats, int32_t n_mats,
                                 const sm_hparams* hp, const float* G, void* W,
                                 int32_t w_dtype, float* Mom, uint32_t* bits,
                                 int64_t worker_stride_words, int32_t M,
                                 int32_t local_worker, int32_t post_vote,
                                 const float* u0, void* ws, size_t ws_bytes,
                                 sm_profile* prof, sm_executor* ex, hipStream_t stream) {
  if (!prof) return SM_EINVAL;
  return step_impl(mats, n_mats, hp, G, W, w_dtype, Mom, bits, worker_stride_words, M,
                   local_worker, post_vote, u0, ws, ws_bytes, prof, ex, stream);
}

sm_status signmuon_reset_status(void* ws, hipStream_t stream) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return SM_EWORKSPACE;
  HIP_TRY(launch_reset_status(static_cast<int32_t*>(ws), stream));
  return SM_OK;
}

sm_status signmuon_get_status(const void* ws, hipStream_t stream) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return SM_EWORKSPACE;
  int32_t h[2] = {0, 0};
  if (hipMemcpyAsync(h, ws, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return SM_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SM_EHIP;
  if ((h[0] | h[1]) & 2) return SM_EHIP;
  return h[0] || h[1] ? SM_ENONFINITE : SM_OK;
}

}  // extern "C"
