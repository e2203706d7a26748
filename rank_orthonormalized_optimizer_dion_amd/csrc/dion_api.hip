// libdion host side: argument validation, workspace layout, grouped launch
// schedule and the C ABI declared in include/dion.h.
//
// One step (Orth-Dion page, equation block; Dion's rule from its closing
// remark) is enqueued as:
//   k_mv [+k_reduce]                 P = (G + R) V
//   CholeskyQR on P -> U             Gram (k_qmax, k_qslice, k_gram8 or
//                                    k_gram), k_chol_*, k_trmm; for
//                                    ill-conditioned P a shifted retry and a
//                                    second pass (k_gram, k_chol_one,
//                                    k_trmm64), gated on the device
//   k_mtu [+k_reduce]                W = (G + R)^T U
//   Orth-Dion: CholeskyQR on W -> V      Dion: k_colnorm, k_colscale -> V
//   k_epi                            X -= eta U V^T, R = beta (G + R - U W^T)
// Every kernel is one grouped launch over all matrices of the call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <list>
#include <mutex>
#include <vector>

#include "dion.h"
#include "dion_types.h"
#include "launchers.h"

#define DION_API extern "C" __attribute__((visibility("default")))

struct dion_plan;

namespace dion {
namespace {

constexpr size_t kAlign = 256;
constexpr int kTargetBlocks = 1024;   // split the reduction below this many tiles
// The same for launches of large split-bfloat16 tiles only, which hold one
// workgroup per CU: one round of workgroups (the 8192 x 28672 matrix at
// r = 512 takes 4 slices of M V instead of 16, 248 steps/s against 232).
constexpr int kTargetBigBlocks = 256;
constexpr int kMinSplitLen = 256;     // shortest reduction slice worth a split
constexpr int kBK = 32;
constexpr int kBlockThreads = 256;  // threads of every libdion workgroup
constexpr int kColnormRows = 512;   // fewest rows per column-norm slice

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

// The fused X / R update works on 128 x 64 tiles: its two accumulator sets
// then leave room for 3 wavefronts per SIMD, so that one block's X, G, R
// traffic overlaps another block's MFMAs.
constexpr int kEpiBN = 64;
constexpr int kFillTiles = 256;   // large tiles when a launch has this many (one per CU),
constexpr int kLongSlice = 1024;  // or reduction slices at least this long
constexpr int kWideTiles = 1024;  // 256 x 192 tiles: four per CU at least

// Rows of an M V / M^T U output tile of width bn: 256 for the
// split-bfloat16 256 x 256 and 256 x 192 tiles, 128 otherwise.
int big_rows(int bn) { return bn == 256 || bn == 192 ? 256 : 128; }

// Output tile width: 128 unless that wastes more than 10% of the tile.
int pick_bn(int cols) {
  const int t128 = cdiv(cols, 128) * 128;
  return cols * 10 >= t128 * 9 ? 128 : 64;
}

struct ClassRec {
  int m, n, r, rp;
  int first, count;
  int bn_r, bn_n, bg;
  int bn_mv;   // M V tile: bn_r, or 256 / 192 (256 x 256 / 256 x 192 split-bfloat16 tiles)
  int bn_mtu;  // M^T U tile, likewise
  int s_mv, kl_mv, s_mtu, kl_mtu, s_gp, kl_gp, s_gw, kl_gw;
  int s_cn, kl_cn;  // Dion column norms: row slices (<= 64, so the slices'
                    // float64 sums fit the Gram area, rp^2 >= 64 r) and rows per slice
  int small_rb;     // > 0: the whole step in one workgroup (k_small), with
                    // this rank block; such classes take no grouped launch
  bool small_res;   // k_small with M resident in LDS
};

// Whether a matrix takes the one-workgroup step (k_small): r <= 16, its
// factors fit that kernel's LDS, and each of its four products is at most
// 2^21 multiply-adds (about 15 us of one compute unit's float32 FMAs).
// Returns the rank block, or 0; resident: M fits in LDS as well.
int small_block(int64_t m, int64_t n, int64_t r, bool& resident) {
  resident = false;
  const int rb = small_rank_block(static_cast<int>(r));
  if (rb == 0) return 0;
  const int64_t n32 = (n + 31) / 32 * 32;
  if ((m + n + n32) * rb > kSmallFactorFloats) return 0;
  if (m * n * r > (int64_t{1} << 21)) return 0;
  resident = m * (n + 1) + (m + n32) * (rb + 1) <= kSmallResidentFloats;
  return rb;
}

}  // namespace
}  // namespace dion

struct dion_plan {
  int count = 0, variant = 0, gdtype = 0;
  int math = 0;                       // 0: float32 MFMA, 1: split-bfloat16
  bool gram8 = true;                  // sliced int8 Gram (else float64 MFMA)
  bool sharded = false;               // DION_SHARDED: staged step with exchanges
  bool vec = false;
  bool single = false;
  std::vector<dion::ClassRec> cls;
  std::vector<dion::MatDesc> table;   // grouped order
  size_t ws_bytes = 0, status_off = 0, table_off = 0;
  dion::MatDesc* pinned = nullptr;    // pinned copy of `table` (grouped calls)
  hipEvent_t ev = nullptr;
  bool ev_pending = false;
  std::vector<uint64_t> key;          // cache key (grouped calls)
  // Phase timing (dion_plan_timing_*): DION_PHASES + 1 events per step.
  std::vector<hipEvent_t> tev;
  int t_max = 0, t_count = 0;
};

namespace dion {
namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// sharded: a row shard of a larger matrix, whose rows may be fewer than r
// (the summed Gram matrix has the global row count).
int validate_matrix(const dion_matrix& a, int gdtype, bool sharded) {
  if (!a.X || !a.G || !a.R || !a.V) return DION_ERR_INVALID_ARG;
  if (a.m < 1 || a.n < 1 || a.m > DION_MAX_DIM || a.n > DION_MAX_DIM) return DION_ERR_INVALID_ARG;
  if (a.m * a.n > INT32_MAX) return DION_ERR_INVALID_ARG;
  if (a.r < 1 || a.r > (sharded ? a.n : std::min(a.m, a.n)) || a.r > DION_MAX_RANK)
    return DION_ERR_INVALID_ARG;
  const size_t eg = gdtype == DION_DTYPE_BF16 ? 2 : 4;
  auto misaligned = [](const void* p, size_t al) { return reinterpret_cast<uintptr_t>(p) % al != 0; };
  if (misaligned(a.X, 4) || misaligned(a.R, 4) || misaligned(a.V, 4) || misaligned(a.G, eg))
    return DION_ERR_INVALID_ARG;
  const size_t mn = static_cast<size_t>(a.m) * a.n, nr = static_cast<size_t>(a.n) * a.r;
  const void* p[4] = {a.X, a.G, a.R, a.V};
  const size_t s[4] = {mn * 4, mn * eg, mn * 4, nr * 4};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (ranges_overlap(p[i], s[i], p[j], s[j])) return DION_ERR_INVALID_ARG;
  return DION_OK;
}

bool vec_ok(const dion_matrix& a, int gdtype) {
  auto al = [](const void* p, size_t b) { return reinterpret_cast<uintptr_t>(p) % b == 0; };
  return a.n % 4 == 0 && a.r % 4 == 0 && al(a.X, 16) && al(a.R, 16) && al(a.V, 16) &&
         al(a.G, gdtype == DION_DTYPE_BF16 ? 8 : 16);
}

// Split count and slice length for a reduction of length K when the launch
// has `tiles` output tiles in total.
void pick_split(int64_t tiles, int K, int& s, int& klen, int target = kTargetBlocks) {
  s = 1;
  if (tiles < target / 2) {
    s = cdiv(target, tiles);
    s = std::max(1, std::min(s, K / kMinSplitLen));
  }
  klen = cdiv(cdiv(K, s), kBK) * kBK;
  s = cdiv(K, klen);
}

// Builds classes, split choices and the workspace layout.  Host only.
int build_plan(const dion_matrix* mats, int count, int variant, int gdtype, bool single,
               dion_plan& p) {
  if (!mats || count < 1) return DION_ERR_INVALID_ARG;
  if (variant & ~(DION_VARIANT_MASK | DION_MATH_MASK | DION_SHARDED | DION_GRAM_F64 |
                  DION_SCHED_GROUPED))
    return DION_ERR_INVALID_ARG;
  if ((variant & DION_SHARDED) && single) return DION_ERR_INVALID_ARG;
  // one matrix: its descriptor travels in the kernel arguments (no table in
  // the workspace, nothing copied from the host per step)
  single = single || count == 1;
  const int rule = variant & DION_VARIANT_MASK;
  if (rule != DION_VARIANT_DION && rule != DION_VARIANT_ORTH) return DION_ERR_INVALID_ARG;
  if (gdtype != DION_DTYPE_F32 && gdtype != DION_DTYPE_BF16) return DION_ERR_INVALID_ARG;
  p.count = count;
  p.variant = rule;
  p.math = (variant & DION_MATH_BF16X3) ? 1 : 0;
  p.sharded = (variant & DION_SHARDED) != 0;
  p.gram8 = (variant & DION_GRAM_F64) == 0;
  p.gdtype = gdtype;
  p.single = single;
  p.vec = true;
  for (int i = 0; i < count; ++i) {
    const int rc = validate_matrix(mats[i], gdtype, p.sharded);
    if (rc != DION_OK) return rc;
    p.vec = p.vec && vec_ok(mats[i], gdtype);
  }
  // Classes by shape, in order of first appearance.
  std::vector<int> cls_of(count, -1);
  for (int i = 0; i < count; ++i) {
    int c = 0;
    for (; c < static_cast<int>(p.cls.size()); ++c)
      if (p.cls[c].m == mats[i].m && p.cls[c].n == mats[i].n && p.cls[c].r == mats[i].r) break;
    if (c == static_cast<int>(p.cls.size())) {
      ClassRec k{};
      k.m = static_cast<int>(mats[i].m);
      k.n = static_cast<int>(mats[i].n);
      k.r = static_cast<int>(mats[i].r);
      k.rp = cdiv(k.r, kCholNB) * kCholNB;
      k.bn_r = pick_bn(k.r);
      // update tile: 256 x 128 split-bfloat16 tiles (bn_n = 256) when rows
      // fill them to 90%
      k.bn_n = p.math && k.m * 10 >= cdiv(k.m, 256) * 256 * 9 && k.n >= 128 ? 256 : kEpiBN;
      // Gram tiles: 64 wide unless the rank is large.  A diagonal tile
      // computes its lower half for nothing, so nt tiles per side reach at
      // most nt / (nt + 1) of the float64 matrix rate; 64-wide tiles halve
      // that loss and balance the grid better (r = 768: 1.5 ms less per
      // Gram than 128-wide tiles).
      // (The sliced Gram always works on 64-wide tiles.)
      k.bg = k.r > 1024 && !p.gram8 ? pick_bn(k.r) : 64;
      // large split-bfloat16 tiles: 256 wide when at most 10% of them
      // idle, else one 192-wide column tile for ranks 129 .. 192
      const bool big_r = k.r * 10 >= cdiv(k.r, 256) * 256 * 9;
      const int bn_big = big_r ? 256 : k.r > 128 && k.r <= 192 ? 192 : 0;
      k.bn_mv = p.math && k.m >= 256 && bn_big ? bn_big : k.bn_r;
      k.bn_mtu = p.math && k.n >= 256 && bn_big ? bn_big : k.bn_r;
      k.small_rb = p.sharded || (variant & DION_SCHED_GROUPED)
                       ? 0 : small_block(k.m, k.n, k.r, k.small_res);
      p.cls.push_back(k);
    }
    cls_of[i] = c;
    p.cls[c].count++;
  }
  // The large split-bfloat16 tiles pay off when a launch has enough of them
  // to give every CU one, or long reduction slices; with few tiles split
  // into short slices (a mid-size matrix on its own), the 128-row tiles keep
  // more CUs busy.  (The update kernel does not split its reduction.)  The
  // 256 x 192 tiles replace 128 x 64 ones, six to one: they need kWideTiles
  // of them in the launch (the 160M stack's 324 take 1.81 ms per step
  // against 1.70 with the small tiles; the 3B stack's 2,240 at r = 1/16
  // take M V from 6.4 to 4.7 ms).
  if (p.math) {
    int64_t big_mv = 0, big_mtu = 0, big_epi = 0, wide_mv = 0, wide_mtu = 0;
    for (const auto& k : p.cls) {
      if (k.small_rb > 0) continue;
      if (k.bn_mv == 256) big_mv += static_cast<int64_t>(k.count) * cdiv(k.m, 256) * cdiv(k.r, 256);
      if (k.bn_mtu == 256) big_mtu += static_cast<int64_t>(k.count) * cdiv(k.n, 256) * cdiv(k.r, 256);
      if (k.bn_mv == 192) wide_mv += static_cast<int64_t>(k.count) * cdiv(k.m, 256);
      if (k.bn_mtu == 192) wide_mtu += static_cast<int64_t>(k.count) * cdiv(k.n, 256);
      if (k.bn_n == 256) big_epi += static_cast<int64_t>(k.count) * cdiv(k.m, 256) * cdiv(k.n, 128);
    }
    auto short_slices = [](int64_t tiles, int K) {
      int sp, kl;
      pick_split(tiles, K, sp, kl);
      return kl < kLongSlice;
    };
    for (auto& k : p.cls) {
      if (big_mv < kFillTiles && k.bn_mv == 256 && short_slices(big_mv, k.n)) k.bn_mv = k.bn_r;
      if (big_mtu < kFillTiles && k.bn_mtu == 256 && short_slices(big_mtu, k.m)) k.bn_mtu = k.bn_r;
      if (wide_mv < kWideTiles && k.bn_mv == 192) k.bn_mv = k.bn_r;
      if (wide_mtu < kWideTiles && k.bn_mtu == 192) k.bn_mtu = k.bn_r;
      if (big_epi < kFillTiles && k.bn_n == 256) k.bn_n = kEpiBN;
    }
  }
  int first = 0;
  for (auto& k : p.cls) {
    k.first = first;
    first += k.count;
  }
  // Reduction splits, from the total tile count of each grouped launch.
  int64_t t_mv = 0, t_mtu = 0, t_gp = 0, t_gw = 0;
  for (auto& k : p.cls) {
    const int nt = cdiv(k.r, k.bg);
    t_mv += static_cast<int64_t>(k.count) * cdiv(k.m, big_rows(k.bn_mv)) * cdiv(k.r, k.bn_mv);
    t_mtu += static_cast<int64_t>(k.count) * cdiv(k.n, big_rows(k.bn_mtu)) * cdiv(k.r, k.bn_mtu);
    t_gp += static_cast<int64_t>(k.count) * nt * (nt + 1) / 2;
  }
  t_gw = t_gp;
  bool all_big_mv = true, all_big_mtu = true;
  for (const auto& k : p.cls) {
    if (k.small_rb > 0) continue;
    all_big_mv = all_big_mv && k.bn_mv >= 192;
    all_big_mtu = all_big_mtu && k.bn_mtu >= 192;
  }
  for (auto& k : p.cls) {
    pick_split(t_mv, k.n, k.s_mv, k.kl_mv, all_big_mv ? kTargetBigBlocks : kTargetBlocks);
    pick_split(t_mtu, k.m, k.s_mtu, k.kl_mtu, all_big_mtu ? kTargetBigBlocks : kTargetBlocks);
    pick_split(t_gp, k.m, k.s_gp, k.kl_gp);
    if (p.sharded) {   // the Gram exchange buffer is one plane of S
      k.s_gp = 1;
      k.kl_gp = cdiv(k.m, kBK) * kBK;
    }
    pick_split(t_gw, k.n, k.s_gw, k.kl_gw);
    k.s_cn = std::min(64, std::max(1, cdiv(k.n, kColnormRows)));
    k.kl_cn = cdiv(k.n, k.s_cn);
    k.s_cn = cdiv(k.n, k.kl_cn);
  }
  // Workspace: status words (one per matrix, then the union of the control
  // bits of the factorization in progress, then the dataflow
  // factorization's counters) | matrix table (grouped calls) | per-matrix
  // buffers.
  size_t off = 0;
  p.status_off = off;
  off = align_up(off + static_cast<size_t>(count + 1 + kFlowWords) * 4);
  p.table_off = off;
  if (!single) off = align_up(off + static_cast<size_t>(count) * sizeof(MatDesc));
  p.table.resize(count);
  std::vector<int> next(p.cls.size());
  for (size_t c = 0; c < p.cls.size(); ++c) next[c] = p.cls[c].first;
  std::vector<int> pos(count);
  for (int i = 0; i < count; ++i) pos[i] = next[cls_of[i]]++;
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) order[pos[i]] = i;
  for (int g = 0; g < count; ++g) {
    const int i = order[g];
    const ClassRec& k = p.cls[cls_of[i]];
    const dion_matrix& a = mats[i];
    MatDesc d{};
    d.X = a.X;
    d.G = a.G;
    d.R = a.R;
    d.V = a.V;
    d.m = k.m;
    d.n = k.n;
    d.r = k.r;
    d.rp = k.rp;
    d.slot = i;
    const size_t m = k.m, n = k.n, r = k.r, rp = k.rp;
    auto take = [&](size_t bytes) {
      const size_t o = off;
      off = align_up(off + bytes);
      return static_cast<int64_t>(o);
    };
    d.oP = take(m * r * 4);
    d.oB = take(m * r * 4);
    d.oW = take(n * r * 4);
    d.oS = take(static_cast<size_t>(std::max(k.s_gp, k.s_gw)) * rp * rp * 8);
    d.oA = take(rp * rp * 8);
    d.oY = take(rp * rp * 8);
    // diagonal-block inverse, diag(S), the trace partials of the first
    // pass (one per 64 x 64 block of T^{-T}), then the dataflow flags (one
    // word per 64 x 64 block)
    const size_t nbk = (rp / kCholNB) * (rp / kCholNB);
    d.oD = take((kCholNB * kCholNB + rp + nbk) * 8 + nbk * 4);
    d.oN = take(r * 4);
    const size_t kpart = std::max(k.s_mv > 1 ? k.s_mv * m * r : 0, k.s_mtu > 1 ? k.s_mtu * n * r : 0);
    d.oK = kpart ? take(kpart * 4) : 0;
    d.oH = p.math ? take(r * std::max(plane_pitch(k.m), plane_pitch(k.n)) * 4) : 0;
    d.oE = k.bn_n == 256 ? take((m + 2 * n) * plane_pitch(k.r) * 4) : 0;
    d.oQ = p.gram8 ? take(static_cast<size_t>(q_bytes(std::max(k.m, k.n), k.r))) : 0;
    // first-pass output of a two-pass orth: of P (m rows), and of W (n
    // rows) for Orth-Dion; last, so that the buffers every step uses keep
    // the offsets they have without it
    d.oC = take((p.variant == DION_VARIANT_ORTH ? std::max(m, n) : m) * r * 4);
    p.table[g] = d;
  }
  p.ws_bytes = off;
  return DION_OK;
}

// One grouped launch per batch of at most kMaxClasses classes.  `fill`
// sets the per-class work shape (returns false to leave a class out).
// Classes with the longest reduction per work item go first (longest job
// first), so that a launch does not end on a last round of its slowest
// blocks; classes of equal length keep their order.
// Classes of the one-workgroup step (small_rb > 0) take part only when
// `small` is set, and then alone.
template <class Fill, class Go>
hipError_t grouped(const dion_plan& p, const Launch& base, Fill fill, Go go, bool small = false) {
  std::vector<ClassInfo> todo;
  for (const ClassRec& c : p.cls) {
    if ((c.small_rb > 0) != small) continue;
    ClassInfo ci{};
    if (!fill(c, ci) || ci.tiles <= 0) continue;
    ci.first = c.first;
    ci.count = c.count;
    todo.push_back(ci);
  }
  std::stable_sort(todo.begin(), todo.end(),
                   [](const ClassInfo& a, const ClassInfo& b) { return a.klen > b.klen; });
  Launch L = base;
  L.nclass = 0;
  L.total = 0;
  for (ClassInfo ci : todo) {
    ci.base = L.total;
    L.cls[L.nclass++] = ci;
    L.total += ci.count * ci.tiles;
    if (L.nclass == kMaxClasses) {
      const hipError_t e = go(L);
      if (e != hipSuccess) return e;
      L.nclass = 0;
      L.total = 0;
    }
  }
  if (L.nclass > 0) return go(L);
  return hipSuccess;
}

#define DION_TRY(expr)                         \
  do {                                         \
    const hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return e_;           \
  } while (0)

// orth() of the P (which = 0) or W (which = 1) factor by one CholeskyQR
// pass with a float64 Gram matrix: S = Q^T Q (sliced int8 MFMA products,
// or float64 MFMA with DION_GRAM_F64), S = T^T T and
// Y = T^{-T} (float64, blocked), Q T^{-1} (float32 MFMA) into U (oB) or V.
// gram() writes the Gram partials into oS; factor() does the rest.
hipError_t gram(const dion_plan& p, Launch base, int which, hipStream_t st) {
  base.which = which;
  base.pass = 1;
  base.gate = kGateAll;
  base.flag = which == 0 ? DION_STATUS_ORTH_P : DION_STATUS_ORTH_W;
  if (p.gram8) {
    // column maxima over row slices (unless the kernel that wrote the
    // factor left them: then one slice per 256-row tile), digit planes,
    // int8 digit products.  A sharded plan's W is the caller's sum over
    // the shards, so its maxima are taken afresh.
    // (the region exists in every sliced-Gram plan: oQ != 0)
    constexpr int64_t kHasRegion = 1;
    auto fused = [&](const ClassRec& c) {
      return which == 0 ? c.bn_mv >= 192 && q_fused_max(kHasRegion, c.s_mv, cdiv(c.m, 256))
                        : c.bn_mtu >= 192 && !p.sharded && q_fused_max(kHasRegion, c.s_mtu, cdiv(c.n, 256));
    };
    auto qsplit = [&](const ClassRec& c, ClassInfo& ci) {
      const int rows = which == 0 ? c.m : c.n;
      if (fused(c)) {
        ci.splits = cdiv(rows, 256);
        ci.klen = 256;
        return rows;
      }
      ci.splits = std::min(kQMaxSplits, std::max(1, cdiv(rows, kQMaxRows)));
      ci.klen = cdiv(rows, ci.splits);
      ci.splits = cdiv(rows, ci.klen);
      return rows;
    };
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (fused(c)) return false;
      qsplit(c, ci);
      ci.tiles = ci.splits * cdiv(c.r, 256);
      return true;
    }, [&](const Launch& L) { return launch_qmax(L, st); }));
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      const int rows = qsplit(c, ci);
      ci.tiles = static_cast<int>(q_rows(rows) / 32) * cdiv(q_cols(c.r) / 32, 4);
      return true;
    }, [&](const Launch& L) { return launch_qslice(L, st); }));
    return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      const int nt = cdiv(c.r, 64);
      ci.tx = nt;
      ci.splits = which == 0 ? c.s_gp : c.s_gw;
      ci.klen = which == 0 ? c.kl_gp : c.kl_gw;
      ci.tiles = nt * (nt + 1) / 2 * ci.splits;
      return true;
    }, [&](const Launch& L) { return launch_gram8(L, st); });
  }
  for (int bg : {128, 64}) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (c.bg != bg) return false;
      const int nt = cdiv(c.r, bg);
      ci.tx = nt;
      ci.splits = which == 0 ? c.s_gp : c.s_gw;
      ci.klen = which == 0 ? c.kl_gp : c.kl_gw;
      ci.tiles = nt * (nt + 1) / 2 * ci.splits;
      return true;
    }, [&](const Launch& L) { return launch_gram(L, bg, p.vec, st); }));
  }
  return hipSuccess;
}

// The parts of orth() that only ill-conditioned factors take (gated on the
// device, see dion_types.h): the shifted first pass (float64 Gram matrix and
// the whole factorization of each matrix in one workgroup), and the float64
// triangular multiply of the first pass followed by the second pass.  Every
// launch runs a capped grid, so it costs little when no matrix needs it.
hipError_t rare_gram(const dion_plan& p, const Launch& base, int which, hipStream_t st) {
  return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    const int nt = cdiv(c.r, 64);
    ci.tx = nt;
    ci.splits = which == 0 ? c.s_gp : c.s_gw;
    ci.klen = which == 0 ? c.kl_gp : c.kl_gw;
    ci.tiles = nt * (nt + 1) / 2 * ci.splits;
    return true;
  }, [&](const Launch& L) { return launch_gram(L, 64, p.vec, st); });
}

hipError_t rare_chol(const dion_plan& p, const Launch& base, int which, hipStream_t st) {
  return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    ci.splits = which == 0 ? c.s_gp : c.s_gw;
    ci.tiles = 1;
    return true;
  }, [&](const Launch& L) { return launch_chol_one(L, st); });
}

hipError_t rare_trmm(const dion_plan& p, const Launch& base, int which, hipStream_t st) {
  return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    ci.tx = cdiv(which == 0 ? c.m : c.n, 64);
    ci.ty = cdiv(c.r, 64);
    ci.tiles = ci.tx * ci.ty;
    return true;
  }, [&](const Launch& L) { return launch_trmm64(L, st); });
}

hipError_t factor(const dion_plan& p, Launch base, int which, hipStream_t st) {
  base.which = which;
  base.pass = 1;
  base.flag = which == 0 ? DION_STATUS_ORTH_P : DION_STATUS_ORTH_W;
  // More passes need the whole factor here; the row-sharded P is a sum the
  // caller forms between stages, so its single pass is final.
  base.retry = p.sharded && which == 0 ? 0 : 1;
  base.gate = kGateAll;   // k_chol_init clears the control bits
  int blocks = 0;
  for (const ClassRec& c : p.cls) {
    const int nb = c.rp / kCholNB;
    if (c.small_rb == 0) blocks += c.count * nb * (nb + 1) / 2;
  }
  const int parts = blocks <= kCholInitSplit ? kCholInitParts : 1;
  DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    const int nb = c.rp / kCholNB;
    ci.splits = which == 0 ? c.s_gp : c.s_gw;
    ci.tiles = nb * (nb + 1) / 2 * parts;
    return true;
  }, [&](const Launch& L) { return launch_chol_init(L, parts, st); }));
  // Every block step in one dataflow launch (k_chol_flow) when its work
  // items, one workgroup per 64 x 64 block of T and of Y, all fit the chip
  // at once (its kernel holds one workgroup per CU); otherwise a launch per
  // step, each of which fills the chip.
  int flow_items = 0, max_nblk = 0;
  for (const ClassRec& c : p.cls) {
    if (c.small_rb > 0) continue;
    const int nb = c.rp / kCholNB;
    flow_items += c.count * nb * nb;
    max_nblk = std::max(max_nblk, nb);
  }
  base.gate = kGateFirst;
  if (flow_items <= kFlowItems) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      const int nb = c.rp / kCholNB;
      ci.tx = nb;
      ci.tiles = nb * nb;
      return true;
    }, [&](const Launch& L) { return launch_chol_flow(L, st); }));
  } else {
    // block steps in pairs (kb, kb + 1) with look-ahead: factor kb, bring
    // block row kb + 1 up to date, factor kb + 1, then one trailing pass
    // with both panels
    auto diag_panel = [&](int kb) -> hipError_t {
      base.kb = kb;
      DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
        ci.tiles = c.rp / kCholNB > kb ? 1 : 0;
        return true;
      }, [&](const Launch& L) { return launch_chol_diag(L, st); }));
      return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
        const int nb = c.rp / kCholNB;
        ci.tiles = nb > kb ? nb - 1 : 0;
        return true;
      }, [&](const Launch& L) { return launch_chol_panel(L, st); });
    };
    for (int kb = 0; kb < max_nblk; kb += 2) {
      DION_TRY(diag_panel(kb));
      if (kb + 1 >= max_nblk) break;
      base.kb = kb;
      base.mode = 1;
      DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
        const int nl = c.rp / kCholNB - kb - 1;
        ci.tiles = nl > 0 ? nl + kb + 1 : 0;
        return true;
      }, [&](const Launch& L) { return launch_chol_trail(L, st); }));
      DION_TRY(diag_panel(kb + 1));
      base.kb = kb;
      base.mode = 2;
      DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
        const int nl = c.rp / kCholNB - kb - 2;
        ci.tiles = nl > 0 ? nl * (nl + 1) / 2 + nl * (kb + 2) : 0;
        return true;
      }, [&](const Launch& L) { return launch_chol_trail(L, st); }));
    }
  }
  if (base.retry) {   // the decision whether more passes follow
    DION_TRY(grouped(p, base, [&](const ClassRec&, ClassInfo& ci) {
      ci.tiles = 1;
      return true;
    }, [&](const Launch& L) { return launch_orth_decide(L, st); }));
  }
  // the float32 triangular multiply of single-pass matrices
  base.gate = kGateOne;
  for (int bn : {128, 64}) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (c.bn_r != bn) return false;
      ci.tx = cdiv(which == 0 ? c.m : c.n, 128);
      ci.ty = cdiv(c.r, bn);
      ci.tiles = ci.tx * ci.ty;
      return true;
    }, [&](const Launch& L) { return launch_trmm(L, bn, p.vec, p.math, st); }));
  }
  if (base.retry) {
    Launch rl = base;   // ill-conditioned: the first pass again, shifted
    rl.gate = kGateRetry;
    DION_TRY(rare_gram(p, rl, which, st));
    DION_TRY(rare_chol(p, rl, which, st));
    Launch tl = base;   // the first pass's product in float64, then the second pass
    tl.gate = kGateTwo;
    DION_TRY(rare_trmm(p, tl, which, st));
    tl.pass = 2;
    DION_TRY(rare_gram(p, tl, which, st));
    DION_TRY(rare_chol(p, tl, which, st));
    DION_TRY(rare_trmm(p, tl, which, st));
  }
  return hipSuccess;
}

// Split-bfloat16 planes of V^T (which = 0) or U^T (which = 1).
hipError_t split_t(const dion_plan& p, Launch base, int which, hipStream_t st) {
  base.which = which;
  return grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    ci.tx = cdiv(which == 0 ? c.n : c.m, kSplitTile);
    ci.ty = cdiv(c.r, kSplitTile);
    ci.tiles = ci.tx * ci.ty;
    return true;
  }, [&](const Launch& L) { return launch_split_t(L, st); });
}

// Records the phase-boundary event `b` of the current timed step, if any.
struct Marker {
  hipEvent_t* ev = nullptr;
  hipError_t mark(int b, hipStream_t st) const {
    return ev ? hipEventRecord(ev[b], st) : hipSuccess;
  }
};

// Stages first..last of the step (the stages of DION_SHARDED; 0..2 is the
// whole step): 0 = P and its Gram partials, 1 = U and W, 2 = Vbar, X, R.
hipError_t run_step(const dion_plan& p, const MatDesc* dev_table, float eta, float beta,
                    char* ws, hipStream_t st, const Marker& mk = Marker{}, int first = 0,
                    int last = 2) {
  Launch base{};
  base.table = dev_table;
  if (p.single) base.inl = p.table[0];
  base.ws = ws;
  base.status = reinterpret_cast<int32_t*>(ws + p.status_off);
  base.any_slot = p.count;
  base.eta = eta;
  base.beta = beta;
  const int ept = elems_per_tile();

  if (first <= 0 && last >= 0) {
  DION_TRY(mk.mark(0, st));
  // small matrices: the whole step in one workgroup each
  for (int rb : {8, 16})
    for (bool res : {true, false}) {
      Launch sl = base;
      sl.mode = p.variant == DION_VARIANT_ORTH ? 1 : 0;
      DION_TRY(grouped(p, sl, [&](const ClassRec& c, ClassInfo& ci) {
        if (c.small_rb != rb || c.small_res != res) return false;
        ci.tiles = 1;
        return true;
      }, [&](const Launch& L) { return launch_small(L, p.gdtype, rb, res, st); }, true));
    }
  // P = M V (split-bfloat16: V^T split once into planes, read as whole cells
  // by every tile)
  if (p.math) DION_TRY(split_t(p, base, 0, st));
  for (int bn : {256, 192, 128, 64}) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (c.bn_mv != bn) return false;
      ci.tx = cdiv(c.m, big_rows(bn));
      ci.ty = cdiv(c.r, bn);
      ci.splits = c.s_mv;
      ci.klen = c.kl_mv;
      ci.tiles = ci.tx * ci.ty * ci.splits;
      return true;
    }, [&](const Launch& L) { return launch_mv(L, p.gdtype, bn, p.vec, p.math, st); }));
  }
  base.which = 0;
  DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    if (c.s_mv <= 1) return false;
    ci.splits = c.s_mv;
    ci.tiles = cdiv(static_cast<int64_t>(c.m) * c.r, ept);
    return true;
  }, [&](const Launch& L) { return launch_reduce(L, st); }));

  // U = orth(P): the Gram partials here, the rest in stage 1
  DION_TRY(mk.mark(1, st));
  DION_TRY(gram(p, base, 0, st));
  }

  if (first <= 1 && last >= 1) {
  DION_TRY(factor(p, base, 0, st));
  DION_TRY(mk.mark(2, st));

  // W = M^T U (split-bfloat16: U^T split once into planes, read as whole
  // cells by every tile)
  if (p.math) DION_TRY(split_t(p, base, 1, st));
  for (int bn : {256, 192, 128, 64}) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (c.bn_mtu != bn) return false;
      ci.tx = cdiv(c.n, big_rows(bn));
      ci.ty = cdiv(c.r, bn);
      ci.splits = c.s_mtu;
      ci.klen = c.kl_mtu;
      ci.tiles = ci.tx * ci.ty * ci.splits;
      return true;
    }, [&](const Launch& L) { return launch_mtu(L, p.gdtype, bn, p.vec, p.math, st); }));
  }
  base.which = 1;
  DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    if (c.s_mtu <= 1) return false;
    ci.splits = c.s_mtu;
    ci.tiles = cdiv(static_cast<int64_t>(c.n) * c.r, ept);
    return true;
  }, [&](const Launch& L) { return launch_reduce(L, st); }));

  }

  if (first <= 2 && last >= 2) {
  // Vbar into V
  DION_TRY(mk.mark(3, st));
  if (p.variant == DION_VARIANT_ORTH) {
    DION_TRY(gram(p, base, 1, st));
    DION_TRY(factor(p, base, 1, st));
  } else {
    base.flag = DION_STATUS_COLNORM;
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      ci.tiles = cdiv(c.r, 64) * c.s_cn;
      ci.splits = c.s_cn;
      ci.klen = c.kl_cn;
      return true;
    }, [&](const Launch& L) { return launch_colnorm(L, st); }));
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      ci.tiles = cdiv(c.r, kBlockThreads);
      ci.splits = c.s_cn;
      return true;
    }, [&](const Launch& L) { return launch_colnorm_fin(L, st); }));
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      ci.tiles = cdiv(static_cast<int64_t>(c.n) * c.r, ept);
      return true;
    }, [&](const Launch& L) { return launch_colscale(L, st); }));
  }

  // U, W and Vbar as split-bfloat16 planes for the large update tiles
  DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
    if (c.bn_n != 256) return false;
    const int cr = cdiv(c.r, kSplitTile);
    ci.tiles = (cdiv(c.m, kSplitTile) + 2 * cdiv(c.n, kSplitTile)) * cr;
    return true;
  }, [&](const Launch& L) { return launch_split_n(L, st); }));

  // X and R
  DION_TRY(mk.mark(4, st));
  for (int bn : {256, 128, 64}) {
    DION_TRY(grouped(p, base, [&](const ClassRec& c, ClassInfo& ci) {
      if (c.bn_n != bn) return false;
      ci.tx = cdiv(c.m, bn == 256 ? 256 : 128);
      ci.ty = cdiv(c.n, bn == 256 ? 128 : bn);
      ci.tiles = ci.tx * ci.ty;
      ci.klen = c.r;   // the update reduces over r; only orders the classes
      return true;
    }, [&](const Launch& L) { return launch_epi(L, p.gdtype, bn, p.vec, p.math, st); }));
  }
  DION_TRY(mk.mark(5, st));
  }
  return hipSuccess;
}

int check_call(const dion_plan& p, float eta, float beta, const void* ws, size_t bytes) {
  if (!std::isfinite(eta) || !std::isfinite(beta)) return DION_ERR_INVALID_ARG;
  if (!ws || bytes < p.ws_bytes) return DION_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return DION_ERR_WORKSPACE;
  return DION_OK;
}

void timing_free(dion_plan* p) {
  for (hipEvent_t e : p->tev) (void)hipEventDestroy(e);
  p->tev.clear();
  p->t_max = p->t_count = 0;
}

void plan_free(dion_plan* p) {
  if (!p) return;
  if (!p->tev.empty()) {
    (void)hipEventSynchronize(p->tev[p->t_count > 0 ? (p->t_count - 1) * (DION_PHASES + 1) + DION_PHASES : 0]);
    timing_free(p);
  }
  if (p->ev) {
    if (p->ev_pending) (void)hipEventSynchronize(p->ev);
    (void)hipEventDestroy(p->ev);
  }
  if (p->pinned) (void)hipHostFree(p->pinned);
  delete p;
}

int plan_alloc_host(dion_plan* p) {
  if (hipHostMalloc(reinterpret_cast<void**>(&p->pinned), sizeof(MatDesc) * p->count,
                    hipHostMallocDefault) != hipSuccess) {
    p->pinned = nullptr;
    return DION_ERR_HIP;
  }
  std::memcpy(p->pinned, p->table.data(), sizeof(MatDesc) * p->count);
  if (hipEventCreateWithFlags(&p->ev, hipEventDisableTiming) != hipSuccess) {
    p->ev = nullptr;
    return DION_ERR_HIP;
  }
  return DION_OK;
}

// Stages first..last of a grouped step (0..2: the whole step, timed when
// timing is enabled; a single stage: one stage of a sharded step).
int plan_step(dion_plan* p, float eta, float beta, void* ws, size_t bytes, hipStream_t st,
              int first = 0, int last = 2) {
  int rc = check_call(*p, eta, beta, ws, bytes);
  if (rc != DION_OK) return rc;
  char* w = static_cast<char*>(ws);
  MatDesc* dev_table = nullptr;
  if (!p->single) {
    dev_table = reinterpret_cast<MatDesc*>(w + p->table_off);
    if (hipMemcpyAsync(dev_table, p->pinned, sizeof(MatDesc) * p->count, hipMemcpyHostToDevice,
                       st) != hipSuccess)
      return DION_ERR_HIP;
    if (hipEventRecord(p->ev, st) != hipSuccess) return DION_ERR_HIP;
    p->ev_pending = true;
  }
  Marker mk;
  if (first == 0 && last == 2 && p->t_count < p->t_max)
    mk.ev = &p->tev[static_cast<size_t>(p->t_count++) * (DION_PHASES + 1)];
  return run_step(*p, dev_table, eta, beta, w, st, mk, first, last) == hipSuccess ? DION_OK
                                                                                  : DION_ERR_HIP;
}

// Cache of grouped plans keyed by the matrix list (most recent first).
// An evicted plan whose last table copy may still be in flight waits in
// g_retired until its event has completed (polled, never waited for), so
// that dion_step_batched does not block the host.
constexpr size_t kCacheSize = 8;
std::mutex g_cache_mu;
std::list<dion_plan*> g_cache;
std::list<dion_plan*> g_retired;

void retire(dion_plan* p) {
  if (p->ev_pending && hipEventQuery(p->ev) != hipSuccess) {
    g_retired.push_back(p);
    return;
  }
  p->ev_pending = false;
  plan_free(p);
}

void sweep_retired() {
  for (auto it = g_retired.begin(); it != g_retired.end();) {
    dion_plan* p = *it;
    if (hipEventQuery(p->ev) == hipSuccess) {
      p->ev_pending = false;
      plan_free(p);
      it = g_retired.erase(it);
    } else {
      ++it;
    }
  }
}

std::vector<uint64_t> make_key(const dion_matrix* mats, int count, int variant, int gdtype) {
  std::vector<uint64_t> k;
  k.reserve(3 + 7 * static_cast<size_t>(count));
  k.push_back(static_cast<uint64_t>(count));
  k.push_back(static_cast<uint64_t>(variant));
  k.push_back(static_cast<uint64_t>(gdtype));
  for (int i = 0; i < count; ++i) {
    k.push_back(reinterpret_cast<uintptr_t>(mats[i].X));
    k.push_back(reinterpret_cast<uintptr_t>(mats[i].G));
    k.push_back(reinterpret_cast<uintptr_t>(mats[i].R));
    k.push_back(reinterpret_cast<uintptr_t>(mats[i].V));
    k.push_back(static_cast<uint64_t>(mats[i].m));
    k.push_back(static_cast<uint64_t>(mats[i].n));
    k.push_back(static_cast<uint64_t>(mats[i].r));
  }
  return k;
}

// Scratch of dion_step_noalloc: the step's workspace in a file-scope device
// array, for callers that cannot allocate device memory.  Each GPU the
// library runs on holds its own copy until the process ends; its address on
// a device is taken once, with that device current, and kept per device.
// Calls on one GPU share it, so calls that overlap there race.
constexpr size_t kScratchBytes = size_t{32} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DION_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DION_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DION_OK;
}

}  // namespace
}  // namespace dion

using namespace dion;

DION_API int dion_version(void) { return 200; }

DION_API const char* dion_error_string(int code) {
  switch (code) {
    case DION_OK: return "success";
    case DION_ERR_INVALID_ARG: return "invalid argument";
    case DION_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DION_ERR_HIP: return "HIP runtime error";
    case DION_ERR_BREAKDOWN: return "numerical breakdown (rank-deficient or non-finite factor)";
    default: return "unknown error code";
  }
}

DION_API size_t dion_workspace_size(int64_t m, int64_t n, int64_t r, int variant, int g_dtype) {
  // Shape-only query: dummy, distinct, aligned addresses stand in for the
  // buffers so validation sees a well-formed call.
  dion_matrix a{};
  a.X = reinterpret_cast<float*>(uintptr_t{1} << 40);
  a.G = reinterpret_cast<const void*>(uintptr_t{2} << 40);
  a.R = reinterpret_cast<float*>(uintptr_t{3} << 40);
  a.V = reinterpret_cast<float*>(uintptr_t{4} << 40);
  a.m = m;
  a.n = n;
  a.r = r;
  dion_plan p;
  if (build_plan(&a, 1, variant, g_dtype, true, p) != DION_OK) return 0;
  return p.ws_bytes;
}

DION_API int dion_step(float* X, const void* G, float* R, float* V, int64_t m, int64_t n,
                       int64_t r, float eta, float beta, int variant, int g_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  dion_matrix a{X, G, R, V, m, n, r};
  dion_plan p;
  int rc = build_plan(&a, 1, variant, g_dtype, true, p);
  if (rc != DION_OK) return rc;
  rc = check_call(p, eta, beta, workspace, workspace_bytes);
  if (rc != DION_OK) return rc;
  const hipError_t e = run_step(p, nullptr, eta, beta, static_cast<char*>(workspace),
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DION_OK : DION_ERR_HIP;
}

DION_API int dion_step_noalloc(float* X, const void* G, float* R, float* V, int64_t m,
                               int64_t n, int64_t r, float eta, float beta, int variant,
                               int g_dtype, int* status_out, void* stream) {
  dion_matrix a{X, G, R, V, m, n, r};
  dion_plan p;
  int rc = build_plan(&a, 1, variant, g_dtype, true, p);
  if (rc != DION_OK) return rc;
  if (!std::isfinite(eta) || !std::isfinite(beta)) return DION_ERR_INVALID_ARG;
  if (p.ws_bytes > kScratchBytes) return DION_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != DION_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (run_step(p, nullptr, eta, beta, static_cast<char*>(ws), st) != hipSuccess) return DION_ERR_HIP;
  if (status_out &&
      hipMemcpyAsync(status_out, static_cast<char*>(ws) + p.status_off, sizeof(int32_t),
                     hipMemcpyDeviceToDevice, st) != hipSuccess)
    return DION_ERR_HIP;
  return DION_OK;
}

DION_API size_t dion_workspace_size_batched(const dion_matrix* mats, int count, int variant,
                                            int g_dtype) {
  if (variant & DION_SHARDED) return 0;   // sharded steps run through a plan
  dion_plan p;
  if (build_plan(mats, count, variant, g_dtype, false, p) != DION_OK) return 0;
  return p.ws_bytes;
}

DION_API int dion_plan_create(const dion_matrix* mats, int count, int variant, int g_dtype,
                              dion_plan** plan_out) {
  if (!plan_out) return DION_ERR_INVALID_ARG;
  *plan_out = nullptr;
  dion_plan* p = new (std::nothrow) dion_plan();
  if (!p) return DION_ERR_INVALID_ARG;
  int rc = build_plan(mats, count, variant, g_dtype, false, *p);
  if (rc == DION_OK) rc = plan_alloc_host(p);
  if (rc != DION_OK) {
    plan_free(p);
    return rc;
  }
  *plan_out = p;
  return DION_OK;
}

DION_API size_t dion_plan_workspace_size(const dion_plan* plan) {
  return plan ? plan->ws_bytes : 0;
}

DION_API int dion_plan_count(const dion_plan* plan) { return plan ? plan->count : 0; }

DION_API int dion_plan_step(dion_plan* plan, float eta, float beta, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!plan) return DION_ERR_INVALID_ARG;
  return plan_step(plan, eta, beta, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

DION_API void dion_plan_destroy(dion_plan* plan) { plan_free(plan); }

DION_API int dion_plan_shard_stage(dion_plan* plan, int stage, float eta, float beta,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !plan->sharded || stage < 0 || stage > 2) return DION_ERR_INVALID_ARG;
  return plan_step(plan, eta, beta, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                   stage, stage);
}

DION_API int dion_plan_shard_buffer(const dion_plan* plan, int which, int index, size_t* offset,
                                    size_t* bytes) {
  if (!plan || !plan->sharded || !offset || !bytes) return DION_ERR_INVALID_ARG;
  if (which != DION_SHARD_GRAM && which != DION_SHARD_W) return DION_ERR_INVALID_ARG;
  if (index < 0 || index >= plan->count) return DION_ERR_INVALID_ARG;
  for (const MatDesc& d : plan->table) {
    if (d.slot != index) continue;
    if (which == DION_SHARD_GRAM) {
      *offset = static_cast<size_t>(d.oS);
      *bytes = static_cast<size_t>(d.rp) * d.rp * 8;
    } else {
      *offset = static_cast<size_t>(d.oW);
      *bytes = static_cast<size_t>(d.n) * d.r * 4;
    }
    return DION_OK;
  }
  return DION_ERR_INVALID_ARG;
}

DION_API int dion_plan_buffer(const dion_plan* plan, int which, int index, size_t* offset,
                              size_t* bytes) {
  if (!plan || !offset || !bytes) return DION_ERR_INVALID_ARG;
  if (which != DION_BUF_P && which != DION_BUF_U && which != DION_BUF_W) return DION_ERR_INVALID_ARG;
  if (index < 0 || index >= plan->count) return DION_ERR_INVALID_ARG;
  for (const MatDesc& d : plan->table) {
    if (d.slot != index) continue;
    const int64_t off = which == DION_BUF_P ? d.oP : which == DION_BUF_U ? d.oB : d.oW;
    *offset = static_cast<size_t>(off);
    *bytes = static_cast<size_t>(which == DION_BUF_W ? d.n : d.m) * d.r * 4;
    return DION_OK;
  }
  return DION_ERR_INVALID_ARG;
}

DION_API int dion_plan_timing_enable(dion_plan* plan, int max_steps) {
  if (!plan || max_steps < 0 || max_steps > (1 << 20)) return DION_ERR_INVALID_ARG;
  if (!plan->tev.empty()) {
    if (plan->t_count > 0 &&
        hipEventSynchronize(plan->tev[(plan->t_count - 1) * (DION_PHASES + 1) + DION_PHASES]) !=
            hipSuccess)
      return DION_ERR_HIP;
    timing_free(plan);
  }
  if (max_steps == 0) return DION_OK;
  plan->tev.resize(static_cast<size_t>(max_steps) * (DION_PHASES + 1), nullptr);
  for (auto& e : plan->tev)
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      for (auto& f : plan->tev)
        if (f) (void)hipEventDestroy(f);
      plan->tev.clear();
      return DION_ERR_HIP;
    }
  plan->t_max = max_steps;
  plan->t_count = 0;
  return DION_OK;
}

DION_API int dion_plan_timing_read(dion_plan* plan, double* ms_per_phase, int* steps) {
  if (!plan || !ms_per_phase || !steps) return DION_ERR_INVALID_ARG;
  for (int ph = 0; ph < DION_PHASES; ++ph) ms_per_phase[ph] = 0.0;
  *steps = plan->t_count;
  if (plan->t_count == 0) return DION_OK;
  const int stride = DION_PHASES + 1;
  if (hipEventSynchronize(plan->tev[(plan->t_count - 1) * stride + DION_PHASES]) != hipSuccess)
    return DION_ERR_HIP;
  for (int s = 0; s < plan->t_count; ++s)
    for (int ph = 0; ph < DION_PHASES; ++ph) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, plan->tev[s * stride + ph], plan->tev[s * stride + ph + 1]) !=
          hipSuccess)
        return DION_ERR_HIP;
      ms_per_phase[ph] += ms;
    }
  plan->t_count = 0;
  return DION_OK;
}

DION_API int dion_step_batched(const dion_matrix* mats, int count, float eta, float beta,
                               int variant, int g_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!mats || count < 1 || (variant & DION_SHARDED)) return DION_ERR_INVALID_ARG;
  std::vector<uint64_t> key = make_key(mats, count, variant, g_dtype);
  std::lock_guard<std::mutex> lock(g_cache_mu);
  sweep_retired();
  dion_plan* hit = nullptr;
  for (auto it = g_cache.begin(); it != g_cache.end(); ++it)
    if ((*it)->key == key) {
      hit = *it;
      g_cache.erase(it);
      break;
    }
  if (!hit) {
    dion_plan* p = nullptr;
    const int rc = dion_plan_create(mats, count, variant, g_dtype, &p);
    if (rc != DION_OK) return rc;
    p->key = std::move(key);
    hit = p;
    if (g_cache.size() >= kCacheSize) {
      retire(g_cache.back());
      g_cache.pop_back();
    }
  }
  g_cache.push_front(hit);
  return plan_step(hit, eta, beta, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

DION_API int dion_status(const void* workspace, int count, void* stream, int* per_matrix) {
  if (!workspace || count < 1) return DION_ERR_INVALID_ARG;
  std::vector<int32_t> st(count);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(st.data(), workspace, sizeof(int32_t) * count, hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return DION_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DION_ERR_HIP;
  int rc = DION_OK;
  for (int i = 0; i < count; ++i) {
    const int flags = st[i] & kStatusMask;   // the breakdown flags, not the control bits
    if (per_matrix) per_matrix[i] = flags;
    if (flags != 0) rc = DION_ERR_BREAKDOWN;
  }
  return rc;
}
