// Device building blocks of libdion's gfx950 kernels: work lookup for
// grouped launches, XCD-aware block order, LDS tile loaders, and the float32
// MFMA main loop.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dion_types.h"

namespace dion {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;   // every kernel runs 4 wavefronts of 64

// Pointers into global memory, so that accesses compile to global_load /
// global_store (counted by vmcnt only) rather than flat accesses (which also
// count against lgkmcnt and would make LDS waits wait for HBM).
template <class T> using gptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return (gptr<T>)(p);
}

// Workgroups of a launch are handed to the 8 XCDs round-robin (block b goes
// to XCD b % 8), and each XCD has its own L2.  Renumber them so that each
// XCD works through chunks of kXcdChunk consecutive logical work items
// (neighbouring tiles share operand panels in that XCD's L2), with the
// chunks dealt to the XCDs in turn: at any time all XCDs work on nearby
// chunks, so a launch whose tiles differ in cost (different matrix shapes)
// stays balanced across XCDs.  Blocks of a last, partial round of chunks
// keep their own number.  The map is a bijection on [0, nb).  (On the 3B
// stack, chunks of 32 took up to 0.8 ms per step less than chunks of 64,
// level with 16; 8 and 128 were slower.)
constexpr int kXcdChunk = 32;
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int round = 8 * kXcdChunk;
  if (b >= nb / round * round) return b;
  const int x = b & 7, i = b >> 3;
  return ((i / kXcdChunk) * 8 + x) * kXcdChunk + i % kXcdChunk;
}

// Find the matrix and the local work item of logical item t.
__device__ __forceinline__ void locate(const Launch& L, int t, MatDesc& d,
                                       ClassInfo& ci, int& local) {
  ci = L.cls[0];
#pragma unroll
  for (int c = 1; c < kMaxClasses; ++c)
    if (c < L.nclass && t >= L.cls[c].base) ci = L.cls[c];
  const int rel = t - ci.base;
  const int mi = rel / ci.tiles;
  local = rel - mi * ci.tiles;
  d = L.table ? L.table[ci.first + mi] : L.inl;
}

// Whether a kernel leaves matrix d alone: it broke down earlier in the
// step, or the launch's gate excludes it (status word and gates: see
// dion_types.h).
__device__ __forceinline__ bool skipped(const Launch& L, const MatDesc& d) {
  const int32_t s = L.status[d.slot];
  if (s & kStatusMask) return true;
  switch (L.gate) {
    case kGateFirst: return (s & kCtlRetry) != 0;
    case kGateOne: return (s & kCtlTwo) != 0;
    case kGateRetry: return (s & kCtlRetry) == 0;
    case kGateTwo: return (s & kCtlTwo) == 0;
    default: return false;
  }
}

// A wave-uniform 64-bit field of a matrix descriptor as a plain value: a
// choice among several fields then stays a choice among values, where a
// choice among the fields themselves would become a load at a computed
// address and keep the whole descriptor copy in private memory.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The factor the first CholeskyQR pass reads: P (which = 0) or W
// (which = 1), and where a single-pass orth leaves its result: U (workspace
// oB) or Vbar (written into V).
__device__ __forceinline__ const float* first_src(const Launch& L, const MatDesc& d) {
  return reinterpret_cast<const float*>(L.ws + (L.which == 0 ? d.oP : d.oW));
}
__device__ __forceinline__ float* final_dst(const Launch& L, const MatDesc& d) {
  return L.which == 0 ? reinterpret_cast<float*>(L.ws + d.oB) : d.V;
}

// The factors of the kernels that also serve a two-pass orth: pass 1 reads
// the first pass's factor; when a second pass follows (kCtlTwo), the first
// writes oC and the second reads it and writes the final result.
__device__ __forceinline__ const float* orth_src(const Launch& L, const MatDesc& d) {
  const int64_t off = L.pass == 2 ? uniform64(d.oC) : L.which == 0 ? uniform64(d.oP) : uniform64(d.oW);
  return reinterpret_cast<const float*>(L.ws + off);
}
__device__ __forceinline__ float* orth_dst(const Launch& L, const MatDesc& d) {
  const bool to_c = L.pass == 1 && (L.status[d.slot] & kCtlTwo);
  const int64_t ws = reinterpret_cast<int64_t>(L.ws);
  const int64_t a = to_c ? ws + uniform64(d.oC)
                         : L.which == 0 ? ws + uniform64(d.oB)
                                        : uniform64(reinterpret_cast<int64_t>(d.V));
  return reinterpret_cast<float*>(a);
}

// Runs body(d, ci, local) over this workgroup's share of the launch's work
// items, for kernels launched with fewer workgroups than items (the gated
// launches of orth's extra passes): workgroup b takes one contiguous chunk
// of items, so a matrix the gate excludes is passed over with one look at
// its status word, not one per item.  With one workgroup per item it takes
// item xcd_remap(b) like every other kernel.  The body must be uniform over
// the workgroup (it may contain barriers).
template <class F>
__device__ __forceinline__ void for_items(const Launch& L, F&& body) {
  // no matrix of the factorization needs this gate: one load and done
  const int32_t any = L.status[L.any_slot];
  if ((L.gate == kGateRetry && !(any & kCtlRetry)) || (L.gate == kGateTwo && !(any & kCtlTwo)))
    return;
  if (static_cast<int>(gridDim.x) >= L.total) {
    MatDesc d;
    ClassInfo ci;
    int local;
    locate(L, xcd_remap(blockIdx.x, gridDim.x), d, ci, local);
    if (!skipped(L, d)) body(d, ci, local);
    return;
  }
  const int per = (L.total + gridDim.x - 1) / gridDim.x;
  int t = blockIdx.x * per;
  const int tend = min(L.total, t + per);
  while (t < tend) {
    MatDesc d;
    ClassInfo ci;
    int local;
    locate(L, t, d, ci, local);
    const int stop = min(tend, t - local + ci.tiles);   // the next matrix's first item
    if (skipped(L, d)) {
      t = stop;
      continue;
    }
    for (; t < stop; ++t, ++local) body(d, ci, local);
  }
}

// Workgroups of a launch whose kernel loops over its work items: launches
// that only some matrices need (gates kGateRetry and kGateTwo) run at most
// this many, so that they cost little when no matrix needs them.
constexpr int kGatedGrid = 256;
inline __host__ __device__ int gated_grid(int total) { return total < kGatedGrid ? total : kGatedGrid; }

// Grouped tile order inside one matrix's tx x ty tile grid: consecutive
// work items walk down GM tile rows of one tile column before moving to the
// next column, so the tiles resident at the same time share both operand
// panels in L2 (about GM row panels and a few column panels).  (GM = 4 took
// about 0.6 ms per step less than 8 on the 3B stack; 2 and 16 were slower.)
__device__ __forceinline__ void tile_order(int local, int tx, int ty, int& tm, int& tn) {
  constexpr int GM = 4;
  const int per_group = GM * ty;
  const int g = local / per_group;
  const int first = g * GM;
  const int gs = min(tx - first, GM);
  const int in = local - g * per_group;
  tm = first + in % gs;
  tn = in / gs;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// ---------------------------------------------------------------------------
// Element sources.  A loader keeps what it fetched from global memory in
// registers in the source's raw form (fetch4: 4 consecutive elements, one
// vector load; fetch4m: the same with per-element predicates, zero where
// false), and only converts it to float32 (fin) when it stores the tile to
// LDS, after the MFMAs of the current tile have been issued, so that the
// load latency hides behind them.
struct SrcF32 {
  using Raw = f32x4;
  gptr<const float> p;
  __device__ __forceinline__ explicit SrcF32(const float* q) : p(to_global(q)) {}
  __device__ __forceinline__ Raw fetch4(int64_t o) const {
    return *(gptr<const f32x4>)(p + o);
  }
  __device__ __forceinline__ Raw fetch4m(int64_t o, const bool (&ok)[4]) const {
    Raw v;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = ok[c] ? p[o + c] : 0.0f;
    return v;
  }
  __device__ __forceinline__ static f32x4 fin(const Raw& v) { return v; }
};

// The buffer M = G + R, formed on the fly (one float32 rounding, the same
// everywhere it is formed).
template <typename GT> struct SrcM;
template <> struct SrcM<float> {
  struct Raw {
    f32x4 g, r;
  };
  gptr<const float> g;
  gptr<const float> r;
  __device__ __forceinline__ SrcM(const float* g_, const float* r_)
      : g(to_global(g_)), r(to_global(r_)) {}
  __device__ __forceinline__ Raw fetch4(int64_t o) const {
    return {*(gptr<const f32x4>)(g + o), *(gptr<const f32x4>)(r + o)};
  }
  __device__ __forceinline__ Raw fetch4m(int64_t o, const bool (&ok)[4]) const {
    Raw v;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v.g[c] = ok[c] ? g[o + c] : 0.0f;
      v.r[c] = ok[c] ? r[o + c] : 0.0f;
    }
    return v;
  }
  __device__ __forceinline__ static f32x4 fin(const Raw& v) { return v.g + v.r; }
};
template <> struct SrcM<uint16_t> {
  struct Raw {
    u32x2 g;
    f32x4 r;
  };
  gptr<const uint16_t> g;
  gptr<const float> r;
  __device__ __forceinline__ SrcM(const uint16_t* g_, const float* r_)
      : g(to_global(g_)), r(to_global(r_)) {}
  __device__ __forceinline__ Raw fetch4(int64_t o) const {
    return {*(gptr<const u32x2>)(g + o), *(gptr<const f32x4>)(r + o)};
  }
  __device__ __forceinline__ Raw fetch4m(int64_t o, const bool (&ok)[4]) const {
    uint32_t h[4];
    Raw v;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h[c] = ok[c] ? g[o + c] : 0u;
      v.r[c] = ok[c] ? r[o + c] : 0.0f;
    }
    v.g.x = h[0] | (h[1] << 16);
    v.g.y = h[2] | (h[3] << 16);
    return v;
  }
  __device__ __forceinline__ static f32x4 fin(const Raw& v) {
    f32x4 a;
    a[0] = __uint_as_float(v.g.x << 16);
    a[1] = __uint_as_float(v.g.x & 0xffff0000u);
    a[2] = __uint_as_float(v.g.y << 16);
    a[3] = __uint_as_float(v.g.y & 0xffff0000u);
    return a + v.r;
  }
};

// float64 source rounded to float32 (the triangular inverse).
struct SrcF64 {
  struct Raw {
    f64x2 a, b;
  };
  gptr<const double> p;
  __device__ __forceinline__ explicit SrcF64(const double* q) : p(to_global(q)) {}
  __device__ __forceinline__ Raw fetch4(int64_t o) const {
    return {*(gptr<const f64x2>)(p + o), *(gptr<const f64x2>)(p + o + 2)};
  }
  __device__ __forceinline__ Raw fetch4m(int64_t o, const bool (&ok)[4]) const {
    Raw v;
    v.a.x = ok[0] ? p[o] : 0.0;
    v.a.y = ok[1] ? p[o + 1] : 0.0;
    v.b.x = ok[2] ? p[o + 2] : 0.0;
    v.b.y = ok[3] ? p[o + 3] : 0.0;
    return v;
  }
  __device__ __forceinline__ static f32x4 fin(const Raw& v) {
    f32x4 r;
    r[0] = static_cast<float>(v.a.x);
    r[1] = static_cast<float>(v.a.y);
    r[2] = static_cast<float>(v.b.x);
    r[3] = static_cast<float>(v.b.y);
    return r;
  }
};

// ---------------------------------------------------------------------------
// LDS tile layout: for an operand tile of BX rows (the output dimension it
// feeds) by BK reduction steps, LDS holds float4 cells cell[kg][x] =
// (e(x,4kg), e(x,4kg+1), e(x,4kg+2), e(x,4kg+3)), row pitch BX + PAD cells.
// A wavefront reads a fragment with one ds_read_b128 per lane: lane l takes
// cell[2q + l/32][x0 + l%32], i.e. 4 reduction steps at once; the MFMA loop
// then pairs lanes 0-31 (k = 8q + c) with lanes 32-63 (k = 8q + 4 + c).
// Both operands use the same k order, so the product is unchanged.
// Row padding 32 / BK and the row swizzle tile_swz make every store pattern
// (k-contiguous: 8 lanes on 8 rows of one x; x-contiguous: 8 lanes on x
// 4 apart) and every MFMA read (8 lanes on consecutive x of one row) touch
// 8 different 16-byte bank groups of the 32-bank LDS.
template <int BX, int BK> struct TileShape {
  static constexpr int PAD = 32 / BK;
  static constexpr int PITCH = BX + PAD;       // float4 cells per kg row
  static constexpr int CELLS = (BK / 4) * PITCH;
};
__device__ __forceinline__ int tile_swz(int x) { return x ^ ((x >> 3) & 3); }

// ---------------------------------------------------------------------------
// Split-bfloat16 tiles (float32 products as three bfloat16 MFMA products).
// Every float32 value x is stored as hi = bf16(x) and lo = bf16(x - hi)
// (round to nearest even; x - hi is exact), so x = hi + lo up to 2^-16 |x|,
// and a product a b is taken as ahi bhi + ahi blo + alo bhi (the dropped
// alo blo is below 2^-16 |a b|).  bfloat16 products are exact in the
// float32 accumulators.
//
// Layout per plane (hi, lo): cells of 16 bytes = 8 consecutive k of one
// row x; cell (k8, x) at k8 * PITCH + swz(x).  An MFMA 32x32x16 operand is
// one ds_read_b128 per lane: lane l reads cell (2q + l/32, x0 + l%32), i.e.
// k = 16q + 8(l/32) + e for its elements e = 0..7, the same for both
// operands.  The swizzle x ^ ((x >> 4) & 3) keeps the reads conflict-free
// and spreads the transposing stores of column-major sources over the
// banks.
template <int BX, int BK> struct BfShape {
  static constexpr int PITCH = BX + 4;           // cells per k8 row
  static constexpr int CELLS = (BK / 8) * PITCH; // 16-byte cells per plane
};
__device__ __forceinline__ int bf_swz(int x) { return x ^ ((x >> 4) & 3); }

__device__ __forceinline__ void bf_split4(const f32x4& v, u32x2& hi, u32x2& lo) {
  const bf16x2 h01 = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
  const bf16x2 h23 = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
  const unsigned a = __builtin_bit_cast(unsigned, h01), b = __builtin_bit_cast(unsigned, h23);
  const float r0 = v[0] - __uint_as_float(a << 16), r1 = v[1] - __uint_as_float(a & 0xffff0000u);
  const float r2 = v[2] - __uint_as_float(b << 16), r3 = v[3] - __uint_as_float(b & 0xffff0000u);
  const bf16x2 l01 = {static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
  const bf16x2 l23 = {static_cast<__bf16>(r2), static_cast<__bf16>(r3)};
  hi.x = a;
  hi.y = b;
  lo.x = __builtin_bit_cast(unsigned, l01);
  lo.y = __builtin_bit_cast(unsigned, l23);
}

// Store the quad (x, k = 4kq .. 4kq+3) as half cells of both planes
// (planes addressed in 8-byte units).
template <int BX>
__device__ __forceinline__ void bf_store_quad(u32x2* hi, u32x2* lo, int kq, int x, const f32x4& v) {
  u32x2 h, l;
  bf_split4(v, h, l);
  const int slot = ((kq >> 1) * (BX + 4) + bf_swz(x)) * 2 + (kq & 1);
  hi[slot] = h;
  lo[slot] = l;
}

// Cell (x, k8) (16 bytes: elements k = 8 k8 .. 8 k8 + 7 of row x) of a
// split-bfloat16 plane with `rows` rows in row-major cell
// order: the cells of one reduction column k8 of all rows are contiguous,
// so 64 consecutive rows of one k8 are one 1 KB run (one direct-to-LDS
// wavefront load).
__device__ __forceinline__ int64_t plane_cell_r(int64_t rows, int x, int k8) {
  return static_cast<int64_t>(k8) * rows + x;
}

// Direct-to-LDS loader of a plane pair (hi, lo) in plane_cell_r order:
// the BX rows x0 .. x0 + BX - 1 and BK / 8 reduction cells of one tile go
// straight into the BfShape LDS layout with global_load_lds_dwordx4, one
// wavefront instruction per 64 cells, no registers and no conversion.
// Lane l of a 64-cell chunk c fetches row bf_swz(64 c + l), which the
// swizzled layout keeps at LDS cell 64 c + l.  Rows past xmax read row
// xmax - 1: they only feed outputs that are never stored.
template <int BX, int BK, int NT>
struct LoadDma {
  static constexpr int K8 = BK / 8, CH = BX / 64;
  static constexpr int NI = 2 * K8 * CH;   // wavefront instructions per tile
  static constexpr int PER = NI / (NT / 64);
  static_assert(BX % 64 == 0 && NI % (NT / 64) == 0, "tile does not split over the wavefronts");
  const u32x4* hi;
  const u32x4* lo;
  int64_t rows;
  int x0, xmax;

  __device__ __forceinline__ void issue(int k0, u32x4* lds_hi, u32x4* lds_lo) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = wave * PER + j;
      const int plane = i / (K8 * CH), rem = i % (K8 * CH);
      const int k8 = rem / CH, c = rem % CH;
      const int x = min(x0 + bf_swz(64 * c + lane), xmax - 1);
      const u32x4* src = (plane ? lo : hi) + plane_cell_r(rows, x, k0 / 8 + k8);
      u32x4* dst = (plane ? lds_lo : lds_hi) + k8 * BfShape<BX, BK>::PITCH + 64 * c;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
    }
  }
};

// Three-way split for float32-accurate products on the bfloat16 matrix
// cores: x = hi + mid + lo with hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid) (both differences exact), 24 significant bits in
// all.  A product keeps the six terms of weight >= 2^-16 (hh, hm, mh, hl,
// lh, mm); the dropped ones are below 3 2^-24 |a b|, the order of float32
// rounding itself.
__device__ __forceinline__ void bf_split4x3(const f32x4& v, u32x2& hi, u32x2& mid, u32x2& lo) {
  u32x2 h, rest;
  bf_split4(v, h, rest);   // rest = bf16(x - hi): that is mid
  mid = rest;
  f32x4 r;
  r[0] = v[0] - __uint_as_float(h.x << 16) - __uint_as_float(mid.x << 16);
  r[1] = v[1] - __uint_as_float(h.x & 0xffff0000u) - __uint_as_float(mid.x & 0xffff0000u);
  r[2] = v[2] - __uint_as_float(h.y << 16) - __uint_as_float(mid.y << 16);
  r[3] = v[3] - __uint_as_float(h.y & 0xffff0000u) - __uint_as_float(mid.y & 0xffff0000u);
  const bf16x2 l01 = {static_cast<__bf16>(r[0]), static_cast<__bf16>(r[1])};
  const bf16x2 l23 = {static_cast<__bf16>(r[2]), static_cast<__bf16>(r[3])};
  hi = h;
  lo.x = __builtin_bit_cast(unsigned, l01);
  lo.y = __builtin_bit_cast(unsigned, l23);
}

// bf_store_quad for the three planes of bf_split4x3.
template <int BX>
__device__ __forceinline__ void bf_store_quad3(u32x2* hi, u32x2* mid, u32x2* lo, int kq, int x,
                                               const f32x4& v) {
  u32x2 h, m, l;
  bf_split4x3(v, h, m, l);
  const int slot = ((kq >> 1) * (BX + 4) + bf_swz(x)) * 2 + (kq & 1);
  hi[slot] = h;
  mid[slot] = m;
  lo[slot] = l;
}

// Loader of split-bfloat16 planes written ahead of time (hi and lo, zero
// past the reduction length) in plane_cell_r order, through registers: one
// 16-byte load per cell and plane (consecutive rows of one k8 are
// contiguous), stored to LDS in the BfShape layout.  FULL: every row x of
// the tile exists.
template <int BX, int BK, int NT = kThreads>
struct LoadPl {
  static_assert(BK == kPlaneK, "one plane block per reduction tile");
  static constexpr int K8 = BK / 8;
  static constexpr int NV = BX * K8 / NT;
  static_assert(NV >= 1 && BX * K8 % NT == 0, "tile too small");
  gptr<const u32x4> hi, lo;
  int64_t rows;
  int x0, xmax;
  u32x4 vh[NV], vl[NV];

  __device__ __forceinline__ LoadPl(const void* h, const void* l, int64_t rows_, int x0_, int xmax_)
      : hi(to_global(static_cast<const u32x4*>(h))), lo(to_global(static_cast<const u32x4*>(l))),
        rows(rows_), x0(x0_), xmax(xmax_) {}

  template <bool FULL>
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int k8 = idx % K8, x = idx / K8;
      const int64_t o = plane_cell_r(rows, x0 + x, k0 / 8 + k8);
      if (FULL || x0 + x < xmax) {
        vh[s] = hi[o];
        vl[s] = lo[o];
      } else {
        vh[s] = u32x4{0u, 0u, 0u, 0u};
        vl[s] = vh[s];
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* sh, u32x4* sl) const {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int k8 = idx % K8, x = idx / K8;
      const int c = k8 * BfShape<BX, BK>::PITCH + bf_swz(x);
      sh[c] = vh[s];
      sl[c] = vl[s];
    }
  }
  __device__ __forceinline__ void store_bf(u32x2* hi, u32x2* lo) const {
    store(reinterpret_cast<u32x4*>(hi), reinterpret_cast<u32x4*>(lo));
  }
};

// Loader for a source whose reduction index is contiguous:
// element (x, k) = src[x * ld + k].  Each row of the tile is read as BK/4
// consecutive float4 (full 128-byte lines for BK = 32).
// TRI: element is zero when k > x (reading the transpose of a lower
// triangle).
// FULL (load): the whole tile lies inside the operand, so loads are
// unconditional; otherwise every element is bounds-checked.
template <int BX, int BK, bool VEC, bool TRI, class Src, int NT = kThreads>
struct LoadKC {
  static constexpr int KQ = BK / 4;
  static constexpr int NV = BX * KQ / NT;
  static_assert(NV >= 1 && BX * KQ % NT == 0, "tile too small");
  Src src;
  int64_t ld;
  int x0, xmax, kmax, kcur;
  typename Src::Raw v[NV];

  __device__ __forceinline__ LoadKC(Src s, int64_t ld_, int x0_, int xmax_, int kmax_)
      : src(s), ld(ld_), x0(x0_), xmax(xmax_), kmax(kmax_), kcur(0) {}

  template <bool FULL>
  __device__ __forceinline__ void load(int k0) {
    kcur = k0;
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int kq = idx % KQ, x = idx / KQ;
      const int gx = x0 + x, gk = k0 + 4 * kq;
      const int64_t o = static_cast<int64_t>(gx) * ld + gk;
      if (FULL || (VEC && gx < xmax && gk + 3 < kmax)) {
        v[s] = src.fetch4(o);
      } else {
        bool ok[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) ok[c] = gx < xmax && gk + c < kmax;
        v[s] = src.fetch4m(o, ok);
      }
    }
  }
  __device__ __forceinline__ void store(f32x4* lds) const {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int kq = idx % KQ, x = idx / KQ;
      f32x4 val = Src::fin(v[s]);
      if constexpr (TRI) {
        const int gx = x0 + x, gk = kcur + 4 * kq;
#pragma unroll
        for (int c = 0; c < 4; ++c) val[c] = gk + c <= gx ? val[c] : 0.0f;
      }
      lds[kq * TileShape<BX, BK>::PITCH + tile_swz(x)] = val;
    }
  }
  // Three-plane store of bf_split4x3 (hi, mid, lo), otherwise as store_bf.
  __device__ __forceinline__ void store_bf3(u32x2* hi, u32x2* mid, u32x2* lo) const {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int kq = idx % KQ, x = idx / KQ;
      f32x4 val = Src::fin(v[s]);
      if constexpr (TRI) {
        const int gx = x0 + x, gk = kcur + 4 * kq;
#pragma unroll
        for (int c = 0; c < 4; ++c) val[c] = gk + c <= gx ? val[c] : 0.0f;
      }
      bf_store_quad3<BX>(hi, mid, lo, kq, x, val);
    }
  }
  // Split-bfloat16 store (see BfShape): each quad of 4 consecutive k is a
  // half cell of the hi and lo planes.
  __device__ __forceinline__ void store_bf(u32x2* hi, u32x2* lo) const {
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int idx = threadIdx.x + NT * s;
      const int kq = idx % KQ, x = idx / KQ;
      f32x4 val = Src::fin(v[s]);
      if constexpr (TRI) {
        const int gx = x0 + x, gk = kcur + 4 * kq;
#pragma unroll
        for (int c = 0; c < 4; ++c) val[c] = gk + c <= gx ? val[c] : 0.0f;
      }
      bf_store_quad<BX>(hi, lo, kq, x, val);
    }
  }
};

// Loader for a source whose output index is contiguous:
// element (x, k) = src[k * ld + x].  Each thread reads a 4 (k) x 4 (x)
// block as four float4 row pieces and transposes it in registers.
template <int BX, int BK, bool VEC, class Src, int NT = kThreads>
struct LoadXC {
  static constexpr int XQ = BX / 4;
  static constexpr int NB = XQ * (BK / 4);
  static constexpr int NPT = (NB + NT - 1) / NT;
  Src src;
  int64_t ld;
  int x0, xmax, kmax;
  typename Src::Raw v[NPT][4];

  __device__ __forceinline__ LoadXC(Src s, int64_t ld_, int x0_, int xmax_, int kmax_)
      : src(s), ld(ld_), x0(x0_), xmax(xmax_), kmax(kmax_) {}

  template <bool FULL>
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int s = 0; s < NPT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NB % NT != 0 && idx >= NB) continue;
      const int xq = idx % XQ, kg = idx / XQ;
      const int gx = x0 + 4 * xq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gk = k0 + 4 * kg + j;
        const int64_t o = static_cast<int64_t>(gk) * ld + gx;
        if (FULL || (VEC && gk < kmax && gx + 3 < xmax)) {
          v[s][j] = src.fetch4(o);
        } else {
          bool ok[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) ok[c] = gk < kmax && gx + c < xmax;
          v[s][j] = src.fetch4m(o, ok);
        }
      }
    }
  }
  __device__ __forceinline__ void store(f32x4* lds) const {
#pragma unroll
    for (int s = 0; s < NPT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NB % NT != 0 && idx >= NB) continue;
      const int xq = idx % XQ, kg = idx / XQ;
      f32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Src::fin(v[s][j]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x4 t;
        t[0] = w[0][c];
        t[1] = w[1][c];
        t[2] = w[2][c];
        t[3] = w[3][c];
        lds[kg * TileShape<BX, BK>::PITCH + tile_swz(4 * xq + c)] = t;
      }
    }
  }
  __device__ __forceinline__ void store_bf(u32x2* hi, u32x2* lo) const {
#pragma unroll
    for (int s = 0; s < NPT; ++s) {
      const int idx = threadIdx.x + NT * s;
      if (NB % NT != 0 && idx >= NB) continue;
      const int xq = idx % XQ, kg = idx / XQ;
      f32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Src::fin(v[s][j]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x4 t;
        t[0] = w[0][c];
        t[1] = w[1][c];
        t[2] = w[2][c];
        t[3] = w[3][c];
        bf_store_quad<BX>(hi, lo, kg, 4 * xq + c, t);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// float32 MFMA tile: BM x BN outputs per workgroup, 2 x 2 wavefronts, each
// wavefront FM x FN blocks of 32 x 32 accumulated with
// v_mfma_f32_32x32x2_f32.
template <int BM, int BN> struct Warps {
  static constexpr int TM = BM / 2, TN = BN / 2;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1, "tile too small");
};

template <int BM, int BN, int BK>
__device__ __forceinline__ void mma_tile(const f32x4* sA, const f32x4* sB,
                                         f32x16 (&acc)[Warps<BM, BN>::FM][Warps<BM, BN>::FN]) {
  using W = Warps<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int q = 0; q < BK / 8; ++q) {
    f32x4 a[W::FM], b[W::FN];
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
      a[fm] = sA[(2 * q + h) * TileShape<BM, BK>::PITCH + tile_swz(wm * W::TM + fm * 32 + i)];
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn)
      b[fn] = sB[(2 * q + h) * TileShape<BN, BK>::PITCH + tile_swz(wn * W::TN + fn * 32 + i)];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < W::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm][c], b[fn][c],
                                                             acc[fm][fn], 0, 0, 0);
  }
}

// Row / column (within the BM x BN tile) of accumulator register v of
// block (fm, fn) held by this lane (the 32x32 MFMA output layout: lane l
// holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4).
template <int BM, int BN>
__device__ __forceinline__ int acc_row(int fm, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * Warps<BM, BN>::TM + fm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
template <int BM, int BN>
__device__ __forceinline__ int acc_col(int fn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * Warps<BM, BN>::TN + fn * 32 + (lane & 31);
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;
}

// Double-buffered main loop over the K tiles starting at kbase: the loaders
// read tile kt into registers (global loads), store it to LDS, and
// mma_tile consumes it.  One barrier per K tile: the next tile's stores go
// to the other buffer, which every wavefront finished reading before the
// previous barrier.
template <int BM, int BN, int BK, bool FULL, class LA, class LB, class MMA>
__device__ __forceinline__ void pipeline(LA& la, LB& lb, int kbase, int nk, f32x4* smem, MMA&& mma) {
  constexpr int CA = TileShape<BM, BK>::CELLS, CB = TileShape<BN, BK>::CELLS;
  constexpr int STAGE = CA + CB;
  // Buffers are addressed by offset from the __shared__ array so that the
  // compiler keeps LDS addressing (ds_read / ds_write), not flat accesses.
  if (nk <= 0) return;
  la.template load<FULL>(kbase);
  lb.template load<FULL>(kbase);
  la.store(smem);
  lb.store(smem + CA);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * STAGE, nxt = STAGE - cur;
    const bool more = kt + 1 < nk;
    if (more) {
      la.template load<FULL>(kbase + (kt + 1) * BK);
      lb.template load<FULL>(kbase + (kt + 1) * BK);
    }
    mma(smem + cur, smem + cur + CA);
    if (more) {
      la.store(smem + nxt);
      lb.store(smem + nxt + CA);
    }
    __syncthreads();
  }
}

// Three-stage pipeline: LDS holds tile kt (being multiplied) and receives
// tile kt+1 from one register set while the other register set already has
// the global loads of tile kt+2 in flight, so every load has two MMA phases
// to arrive.  Register sets alternate, hence the 2-step unrolled loop.
template <int BM, int BN, int BK, bool FULL, class LA, class LB, class MMA>
__device__ __forceinline__ void pipeline2(LA& a0, LA& a1, LB& b0, LB& b1, int kbase, int nk,
                                          f32x4* smem, MMA&& mma) {
  constexpr int CA = TileShape<BM, BK>::CELLS, CB = TileShape<BN, BK>::CELLS;
  constexpr int STAGE = CA + CB;
  if (nk <= 0) return;
  a0.template load<FULL>(kbase);
  b0.template load<FULL>(kbase);
  if (nk > 1) {
    a1.template load<FULL>(kbase + BK);
    b1.template load<FULL>(kbase + BK);
  }
  a0.store(smem);
  b0.store(smem + CA);
  __syncthreads();
  const int pairs = nk >> 1;
  for (int p = 0; p < pairs; ++p) {
    const int kt = 2 * p;
    // tile kt is in LDS stage 0; set 1 holds tile kt+1; set 0 takes kt+2
    const bool more0 = kt + 2 < nk;
    if (more0) {
      a0.template load<FULL>(kbase + (kt + 2) * BK);
      b0.template load<FULL>(kbase + (kt + 2) * BK);
    }
    mma(smem, smem + CA);
    a1.store(smem + STAGE);
    b1.store(smem + STAGE + CA);
    __syncthreads();
    // tile kt+1 is in LDS stage 1; set 0 holds tile kt+2; set 1 takes kt+3
    if (kt + 3 < nk) {
      a1.template load<FULL>(kbase + (kt + 3) * BK);
      b1.template load<FULL>(kbase + (kt + 3) * BK);
    }
    mma(smem + STAGE, smem + STAGE + CA);
    if (more0) {
      a0.store(smem);
      b0.store(smem + CA);
    }
    __syncthreads();
  }
  if (nk & 1) mma(smem, smem + CA);   // last tile, already in stage 0
}

// Split-bfloat16 MFMA tile: BM x BN outputs, 2 x 2 wavefronts, each
// FM x FN blocks of 32 x 32 accumulated with 3 v_mfma_f32_32x32x16_bf16
// per 16 k (lo hi, hi lo, hi hi).  Planes: A hi, A lo, B hi, B lo.
template <int BM, int BN, int BK>
__device__ __forceinline__ void mma_tile_bf3(const u32x4* ah, const u32x4* al, const u32x4* bh,
                                             const u32x4* bl,
                                             f32x16 (&acc)[Warps<BM, BN>::FM][Warps<BM, BN>::FN]) {
  using W = Warps<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int q = 0; q < BK / 16; ++q) {
    bf16x8 a_hi[W::FM], a_lo[W::FM], b_hi[W::FN], b_lo[W::FN];
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm) {
      const int c = (2 * q + h) * BfShape<BM, BK>::PITCH + bf_swz(wm * W::TM + fm * 32 + i);
      a_hi[fm] = __builtin_bit_cast(bf16x8, ah[c]);
      a_lo[fm] = __builtin_bit_cast(bf16x8, al[c]);
    }
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int c = (2 * q + h) * BfShape<BN, BK>::PITCH + bf_swz(wn * W::TN + fn * 32 + i);
      b_hi[fn] = __builtin_bit_cast(bf16x8, bh[c]);
      b_lo[fn] = __builtin_bit_cast(bf16x8, bl[c]);
    }
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < W::FN; ++fn) {
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[fm], b_hi[fn], acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_lo[fn], acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_hi[fn], acc[fm][fn], 0, 0, 0);
      }
  }
}

// Wavefront grid of a BM x BN tile: GM x GN wavefronts (64 GM GN threads),
// wavefront (wm, wn) = (wave / GN, wave % GN) owning FM x FN blocks of
// 32 x 32 outputs.
template <int BM_, int BN_, int GM_, int GN_>
struct WGrid {
  static constexpr int BM = BM_, BN = BN_, GM = GM_, GN = GN_;
  static constexpr int NT = 64 * GM * GN;
  static constexpr int TM = BM / GM, TN = BN / GN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "tile too small");
  __device__ static int wm() { return (threadIdx.x >> 6) / GN; }
  __device__ static int wn() { return (threadIdx.x >> 6) % GN; }
  // row / column of accumulator register v of block (fm, fn) (32 x 32 MFMA
  // output layout: lane l holds column l % 32, rows 8(v/4) + 4(l/32) + v%4)
  __device__ static int row(int fm, int v) {
    return wm() * TM + fm * 32 + 8 * (v >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (v & 3);
  }
  __device__ static int col(int fn) { return wn() * TN + fn * 32 + (threadIdx.x & 31); }
};

// mma_tile_bf3 for any wavefront grid.
template <class W, int BK>
__device__ __forceinline__ void mma_tile_bf3w(const u32x4* ah, const u32x4* al, const u32x4* bh,
                                              const u32x4* bl, f32x16 (&acc)[W::FM][W::FN]) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, i = lane & 31;
  const int wm = W::wm(), wn = W::wn();
#pragma unroll
  for (int q = 0; q < BK / 16; ++q) {
    bf16x8 a_hi[W::FM], a_lo[W::FM], b_hi[W::FN], b_lo[W::FN];
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm) {
      const int c = (2 * q + h) * BfShape<W::BM, BK>::PITCH + bf_swz(wm * W::TM + fm * 32 + i);
      a_hi[fm] = __builtin_bit_cast(bf16x8, ah[c]);
      a_lo[fm] = __builtin_bit_cast(bf16x8, al[c]);
    }
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int c = (2 * q + h) * BfShape<W::BN, BK>::PITCH + bf_swz(wn * W::TN + fn * 32 + i);
      b_hi[fn] = __builtin_bit_cast(bf16x8, bh[c]);
      b_lo[fn] = __builtin_bit_cast(bf16x8, bl[c]);
    }
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < W::FN; ++fn) {
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[fm], b_hi[fn], acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_lo[fn], acc[fm][fn], 0, 0, 0);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_hi[fn], acc[fm][fn], 0, 0, 0);
      }
  }
}

// Two products sharing the left operand, A B^T and A C^T (the fused X / R
// update): A's fragments are read from LDS once per 16 k for both.
template <class W, int BK>
__device__ __forceinline__ void mma_tile_bf3w2(const u32x4* ah, const u32x4* al, const u32x4* bh,
                                               const u32x4* bl, const u32x4* ch, const u32x4* cl,
                                               f32x16 (&ab)[W::FM][W::FN],
                                               f32x16 (&ac)[W::FM][W::FN]) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, i = lane & 31;
  const int wm = W::wm(), wn = W::wn();
#pragma unroll
  for (int q = 0; q < BK / 16; ++q) {
    bf16x8 a_hi[W::FM], a_lo[W::FM], b_hi[W::FN], b_lo[W::FN], c_hi[W::FN], c_lo[W::FN];
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm) {
      const int c = (2 * q + h) * BfShape<W::BM, BK>::PITCH + bf_swz(wm * W::TM + fm * 32 + i);
      a_hi[fm] = __builtin_bit_cast(bf16x8, ah[c]);
      a_lo[fm] = __builtin_bit_cast(bf16x8, al[c]);
    }
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int c = (2 * q + h) * BfShape<W::BN, BK>::PITCH + bf_swz(wn * W::TN + fn * 32 + i);
      b_hi[fn] = __builtin_bit_cast(bf16x8, bh[c]);
      b_lo[fn] = __builtin_bit_cast(bf16x8, bl[c]);
      c_hi[fn] = __builtin_bit_cast(bf16x8, ch[c]);
      c_lo[fn] = __builtin_bit_cast(bf16x8, cl[c]);
    }
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < W::FN; ++fn) {
        ab[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[fm], b_hi[fn], ab[fm][fn], 0, 0, 0);
        ac[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[fm], c_hi[fn], ac[fm][fn], 0, 0, 0);
        ab[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_lo[fn], ab[fm][fn], 0, 0, 0);
        ac[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], c_lo[fn], ac[fm][fn], 0, 0, 0);
        ab[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], b_hi[fn], ab[fm][fn], 0, 0, 0);
        ac[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[fm], c_hi[fn], ac[fm][fn], 0, 0, 0);
      }
  }
}

// Float32-accurate product tile from three-way split operands: the six
// terms hh, hm, mh, hl, lh, mm of bf_split4x3 per 16 k.  Planes: A hi, mid,
// lo at ah, ah + CA, ah + 2 CA; B likewise from bh with stride CB.
template <int BM, int BN, int BK>
__device__ __forceinline__ void mma_tile_bf6(const u32x4* ah, const u32x4* bh,
                                             f32x16 (&acc)[Warps<BM, BN>::FM][Warps<BM, BN>::FN]) {
  using W = Warps<BM, BN>;
  constexpr int CA = BfShape<BM, BK>::CELLS, CB = BfShape<BN, BK>::CELLS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int q = 0; q < BK / 16; ++q) {
    bf16x8 a[3][W::FM], b[3][W::FN];
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm) {
      const int c = (2 * q + h) * BfShape<BM, BK>::PITCH + bf_swz(wm * W::TM + fm * 32 + i);
#pragma unroll
      for (int p = 0; p < 3; ++p) a[p][fm] = __builtin_bit_cast(bf16x8, ah[p * CA + c]);
    }
#pragma unroll
    for (int fn = 0; fn < W::FN; ++fn) {
      const int c = (2 * q + h) * BfShape<BN, BK>::PITCH + bf_swz(wn * W::TN + fn * 32 + i);
#pragma unroll
      for (int p = 0; p < 3; ++p) b[p][fn] = __builtin_bit_cast(bf16x8, bh[p * CB + c]);
    }
#pragma unroll
    for (int fm = 0; fm < W::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < W::FN; ++fn) {
        f32x16 t = acc[fm][fn];
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][fm], b[1][fn], t, 0, 0, 0);   // mm
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2][fm], b[0][fn], t, 0, 0, 0);   // lh
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][fm], b[2][fn], t, 0, 0, 0);   // hl
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][fm], b[0][fn], t, 0, 0, 0);   // mh
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][fm], b[1][fn], t, 0, 0, 0);   // hm
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][fm], b[0][fn], t, 0, 0, 0);
      }
  }
}

// LDS bytes of one split-bfloat16 stage (A and B, hi and lo planes).
template <int BM, int BN, int BK>
constexpr int bf_stage_cells() {
  return 2 * (BfShape<BM, BK>::CELLS + BfShape<BN, BK>::CELLS);
}

// Three-stage pipeline as pipeline2, storing split-bfloat16 planes.
// smem: 2 stages of bf_stage_cells() 16-byte cells.
template <int BM, int BN, int BK, bool FULL, class LA, class LB, class MMA>
__device__ __forceinline__ void pipeline2_bf(LA& a0, LA& a1, LB& b0, LB& b1, int kbase, int nk,
                                             u32x4* smem, MMA&& mma) {
  constexpr int CA = BfShape<BM, BK>::CELLS, CB = BfShape<BN, BK>::CELLS;
  constexpr int STAGE = 2 * (CA + CB);
  // plane offsets inside a stage: A hi, A lo, B hi, B lo
  auto store = [&](auto& la, auto& lb, int st) {
    u32x4* base = smem + st * STAGE;
    la.store_bf(reinterpret_cast<u32x2*>(base), reinterpret_cast<u32x2*>(base + CA));
    lb.store_bf(reinterpret_cast<u32x2*>(base + 2 * CA), reinterpret_cast<u32x2*>(base + 2 * CA + CB));
  };
  auto compute = [&](int st) {
    u32x4* base = smem + st * STAGE;
    mma(base, base + CA, base + 2 * CA, base + 2 * CA + CB);
  };
  if (nk <= 0) return;
  a0.template load<FULL>(kbase);
  b0.template load<FULL>(kbase);
  if (nk > 1) {
    a1.template load<FULL>(kbase + BK);
    b1.template load<FULL>(kbase + BK);
  }
  store(a0, b0, 0);
  __syncthreads();
  const int pairs = nk >> 1;
  for (int p = 0; p < pairs; ++p) {
    const int kt = 2 * p;
    const bool more0 = kt + 2 < nk;
    if (more0) {
      a0.template load<FULL>(kbase + (kt + 2) * BK);
      b0.template load<FULL>(kbase + (kt + 2) * BK);
    }
    compute(0);
    store(a1, b1, 1);
    __syncthreads();
    if (kt + 3 < nk) {
      a1.template load<FULL>(kbase + (kt + 3) * BK);
      b1.template load<FULL>(kbase + (kt + 3) * BK);
    }
    compute(1);
    if (more0) store(a0, b0, 0);
    __syncthreads();
  }
  if (nk & 1) compute(0);
}

// Two-stage split-bfloat16 pipeline for large tiles: LDS double-buffered,
// one barrier per tile.  The B operand (planes written ahead of time) is
// copied straight into LDS by LoadDma; A goes through registers (loaded
// before this tile's MFMAs, split and stored to the other stage after
// them).  The next tile's B copies run during this tile's MFMAs and are
// waited for at the barrier that ends the step.
// smem: 2 stages of bf_stage_cells() 16-byte cells.
template <int BM, int BN, int BK, bool FULL, class LA, class LB, class MMA>
__device__ __forceinline__ void pipeline_bf_dma(LA& a, const LB& b, int kbase, int nk, u32x4* smem,
                                                MMA&& mma) {
  constexpr int CA = BfShape<BM, BK>::CELLS, CB = BfShape<BN, BK>::CELLS;
  constexpr int STAGE = 2 * (CA + CB);
  if (nk <= 0) return;
  b.issue(kbase, smem + 2 * CA, smem + 2 * CA + CB);
  a.template load<FULL>(kbase);
  a.store_bf(reinterpret_cast<u32x2*>(smem), reinterpret_cast<u32x2*>(smem + CA));
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    u32x4* next = smem + ((kt + 1) & 1) * STAGE;
    if (more) {
      b.issue(kbase + (kt + 1) * BK, next + 2 * CA, next + 2 * CA + CB);
      a.template load<FULL>(kbase + (kt + 1) * BK);
    }
    const u32x4* cur = smem + (kt & 1) * STAGE;
    mma(cur, cur + CA, cur + 2 * CA, cur + 2 * CA + CB);
    if (more) a.store_bf(reinterpret_cast<u32x2*>(next), reinterpret_cast<u32x2*>(next + CA));
    __syncthreads();
  }
}

template <int BM, int BN, int BK, bool FULL, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(
    LA& la, LB& lb, int kbase, int nk, f32x4* smem,
    f32x16 (&acc)[Warps<BM, BN>::FM][Warps<BM, BN>::FN]) {
  pipeline<BM, BN, BK, FULL>(la, lb, kbase, nk, smem, [&](const f32x4* a, const f32x4* b) {
    mma_tile<BM, BN, BK>(a, b, acc);
  });
}

// float64 MFMA on a tile staged as float32 (v_mfma_f64_16x16x4_f64): the
// float32 products are exact in float64 and the sums are float64.  2 x 2
// wavefronts, each FB x FB blocks of 16 x 16.  Lane l reads the cell of k
// group 4q + l/16, row l%16, and feeds its 4 components to 4 MFMAs (the
// same k order for both operands).
template <int BG, int BK>
__device__ __forceinline__ void mma_tile_f64(const f32x4* sA, const f32x4* sB,
                                             f64x4 (&acc)[BG / 32][BG / 32]) {
  constexpr int WT = BG / 2, FB = WT / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, i = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int q = 0; q < BK / 16; ++q) {
    f32x4 a[FB], b[FB];
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      a[f] = sA[(4 * q + grp) * TileShape<BG, BK>::PITCH + tile_swz(wm * WT + f * 16 + i)];
      b[f] = sB[(4 * q + grp) * TileShape<BG, BK>::PITCH + tile_swz(wn * WT + f * 16 + i)];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int fm = 0; fm < FB; ++fm)
#pragma unroll
        for (int fn = 0; fn < FB; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(
              static_cast<double>(a[fm][c]), static_cast<double>(b[fn][c]), acc[fm][fn], 0, 0, 0);
  }
}

template <int BM, int BN, int BK>
constexpr int mainloop_cells() {
  return 2 * (TileShape<BM, BK>::CELLS + TileShape<BN, BK>::CELLS);
}

}  // namespace dion
