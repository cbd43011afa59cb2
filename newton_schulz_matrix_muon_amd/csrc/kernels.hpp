// Device kernels of the Muon step for gfx950 (CDNA4, wave64).
//
// Kernels, in launch order for one stacked pass ("chunk") of equal-shape NS
// units:
//   k_momentum      M <- mu*M + G, N = mu*M + G (or the EMA style with bias
//                   corrections: two coefficient pairs from the host, exact
//                   for the SGD style's 1s), per-block fp64 partial sums of
//                   N^2 (DeepSeek tech notes "Muon 优化器" section 1
//                   Algorithm 1; RFC-0023 方案 1).  N goes to the fp32
//                   buffer, or on the bf16 paths straight into the bf16
//                   iterate with its padding zeroed (k_momentum_t: units a
//                   pass holds transposed).
//   k_norm_finish   per unit: fixed-order fp64 sum of the partials, 1/||N||_F
//                   and the non-zero flag (notes section 2: Frobenius
//                   normalisation, a zero matrix stays zero).
//   k_normalize     fp32 path: X0 = N/||N||_F over the padded iterate (zeros
//                   in the padding) and X0^T, transposed through LDS.  The
//                   bf16 paths have no such pass: their first iteration
//                   reads N and scales the Gram by 1/nu^2, the apply by 1/nu.
//   ns_gemm<GRAM>   A = X X^T (or X^T X for a tall unit: the smaller side).
//   ns_gemm<POLY>   B' = a*I + b*A + c*A*A (on the bf16 path A is kept only
//                   as its bf16 operand copy, which the b*A term also
//                   reads; a*I carries the apply's a*X term).  Both outputs
//                   are symmetric: only the upper-triangle tiles are
//                   computed, each also written mirrored.
//   ns_gemm<APPLY>  X' = B'*X (or X*B'), written as its operand copy X' (and
//                   X'^T on the fp32 path).  On the bf16 path the iterate
//                   exists only in bf16.  In the last iteration the
//                   epilogue writes W <- W*(1 - lr*wd) - lr*scale*X' instead
//                   (Algorithm 1's decoupled update) or the NS output.
//   k_ns_small      the whole NS of a wide unit with at most 128 rows and
//                   more than 128 columns on chip: A and B' in the
//                   workgroup, one pass over X per iteration (bf16
//                   products); a few long units split over several
//                   workgroups that sum their partial Grams through memory.
//   k_ns_small_step the whole step (momentum to update) of a wide unit of
//                   at most 128 x 128 in one launch, the iterate in
//                   registers (bf16, or fp32 up to 64 rows).
//   ns_persistent   the three products of every iteration in one launch:
//                   workgroups claim tiles in order and wait on per-panel
//                   completion counts, so tiles of different units and
//                   phases overlap (no launch boundary between products).
//   ns_persistent2  the same over two passes of different unit shapes at
//                   once (a pass of one unit beside a stacked pass).
// The three products are the quintic step a*X + b*(X X^T)X + c*(X X^T)^2 X of
// the notes' section 2, grouped as (a*I + b*A + c*A^2)*X: the polynomial's
// epilogue adds a on the diagonal, so the apply is one plain product and
// reads nothing beside its operands.  Every product reads its operands
// K-contiguous or, on the bf16 path, K-major through the LDS transposing
// read: Gram X X^T reads X twice (X^T X reads X K-major twice), B'*X reads
// B' and X K-major, X*B' reads X and B' (B' is symmetric).  The fp32 path
// keeps X^T beside X instead.
//
// Padding: every iterate is stored as rows_pad x cols_pad with exact zeros
// outside rows x cols, and every Gram / polynomial matrix as s_pad x s_pad.
// Zero padding is invariant under all three products, so the GEMMs run on
// whole tiles with no bounds checks; only the final epilogue masks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxSeg = 48;
constexpr int kThreads = 256;

// A run of consecutive NS units inside one caller bank (unit stride =
// unit_elems elements in every caller buffer).
struct Seg {
  float* w;        // weights of the first unit (step) / NS output (NS only)
  const void* g;   // gradient of the first unit (step) / NS input (NS only)
  float* m;        // momentum of the first unit (step only)
  int32_t first;   // chunk-local index of the first unit
  int32_t count;   // number of units
  int32_t trans;   // 1: the units are stored transposed relative to the
                   // chunk's shape (wide units in a tall chunk, see below)
  float lr_scale;  // lr * the units' update scale (their own fan_out, fan_in)
};

// A chunk's units share one shape rows x cols.  Units whose caller
// matrices are that shape transposed (a wide unit, fan_out < fan_in, in a
// tall chunk: the tiled products always take the tall form, so that a unit's
// result does not depend on the other units of its batch) have `trans`
// set: their gradient, momentum and weight are caller matrices of cols x
// rows, the iterate holds N^T, and the update is written back transposed.
struct ChunkArgs {
  int32_t n_seg;
  int32_t n_units;
  int32_t rows, cols;          // unit shape in the chunk (fan_out x fan_in
                               // unless transposed)
  int32_t rows_pad, cols_pad;  // padded iterate shape
  int64_t unit_elems;          // rows * cols
  int64_t x_stride;            // rows_pad * cols_pad
  float ma, mb;                // M <- ma*M + mb*G
  float la, lb;                // N  = la*M + lb*G (on the updated M)
  float decay;                 // 1 - lr * weight_decay
  float lr_scale;              // lr * scale of units in the chunk's shape
                               // (each segment carries its own, Seg::lr_scale)
  int32_t pad0;
  Seg seg[kMaxSeg];
};

enum Phase { GRAM = 0, POLY = 1, APPLY = 2 };
enum FinalMode { FINAL_NONE = 0, FINAL_STEP = 1, FINAL_NSOUT = 2 };

struct GemmArgs {
  const void* a;        // operand A (unit 0)
  const void* b;        // operand B (unit 0)
  int64_t a_ustride, b_ustride;
  int32_t lda, ldb;
  int32_t M, N, K;      // padded sizes, multiples of the tile
  int32_t tiles_m, tiles_n;
  int32_t n_units;
  float* out32;         // fp32 output (unit 0) or nullptr
  void* out16;          // bf16 output (unit 0) or nullptr
  int64_t out_ustride;
  int32_t ldo;
  void* outt;           // APPLY, fp32 path: transposed operand copy of X' (T); else nullptr
  int32_t ldt;          // its leading dimension (rows of X')
  int32_t sym;          // GRAM/POLY: symmetric output; only tiles tm <= tn run
                        // and each off-diagonal tile also writes its mirror
  int32_t final_mode;
  const float* aux;     // POLY: fp32 A on the fp32 path, laid out like the output
  const void* aux16;    // POLY: bf16 A on the bf16 path
  int64_t aux_ustride;
  int32_t ldaux;
  float ca, cb, cc;     // quintic coefficients (POLY forms a*I + b*A + c*A^2)
  const int32_t* flag;  // per unit: nonzero = the unit has a nonzero norm
  const float* fold;    // per unit 1/nu when X holds N itself (first
                        // iteration of the folded bf16 path), or nullptr
};

// The segment holding chunk-local unit u.  Every table entry is read at a
// constant index (a dynamic index would copy the whole kernel-argument
// struct to scratch memory).
struct SegView {
  float* w;
  const void* g;
  float* m;
  int32_t first;
  int32_t trans;
  float lr_scale;
};

template <int NSEG>
__device__ __forceinline__ SegView find_seg_in(const Seg (&seg)[NSEG], int n_seg, int u) {
  SegView v{seg[0].w, seg[0].g, seg[0].m, seg[0].first, seg[0].trans, seg[0].lr_scale};
#pragma unroll
  for (int s = 1; s < NSEG; ++s) {
    if (s < n_seg && seg[s].first <= u) {
      v.w = seg[s].w;
      v.g = seg[s].g;
      v.m = seg[s].m;
      v.first = seg[s].first;
      v.trans = seg[s].trans;
      v.lr_scale = seg[s].lr_scale;
    }
  }
  return v;
}

__device__ __forceinline__ SegView find_seg(const ChunkArgs& ca, int u) {
  return find_seg_in(ca.seg, ca.n_seg, u);
}

// Where a final epilogue writes unit u: its weight (step) or NS output in
// the caller's layout, and the shape its stores are masked to.
struct UnitOut {
  float* w;          // the unit's first element
  int32_t trans;     // stored transposed relative to the shape below
  float lr_scale;    // lr * the unit's update scale
  int32_t rows, cols;
  float decay;
};

__device__ __forceinline__ UnitOut unit_out(const ChunkArgs& ca, int u) {
  const SegView sg = find_seg(ca, u);
  return UnitOut{sg.w + (int64_t)(u - sg.first) * ca.unit_elems, sg.trans, sg.lr_scale,
                 ca.rows, ca.cols, ca.decay};
}

// ----------------------------------------------------------------- utils ---
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Deterministic block sum (fixed shuffle tree, then waves in order).
__device__ __forceinline__ double block_sum(double v, double* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  }
  return t;
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

__device__ __forceinline__ void store_bf16x4(void* base, int64_t idx, float a, float b, float c,
                                             float d) {
  uint2 p;
  p.x = (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
  p.y = (uint32_t)to_bf16_bits(c) | ((uint32_t)to_bf16_bits(d) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = p;
}

// f rounded to bf16 (round to nearest even), as fp32.
__device__ __forceinline__ float bf16_round(float f) {
  return bf16_bits_to_f32(to_bf16_bits(f));
}

// ------------------------------------------------------------- momentum ----
// Streaming accesses to the caller's gradient and momentum.  With NT they
// carry the non-temporal hint, which the host picks for passes whose
// momentum is larger than the last-level cache (an MoE bank of 5.6G
// elements: 13.4 -> 12.9 ms on one machine, 13.0 -> 11.6 ms on another; on
// 32 x 1024^2, 134 MB of momentum, the hint was 5-10% slower).
typedef unsigned u32x2e __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint2 ld_u2(const void* p) {
  const u32x2e* q = static_cast<const u32x2e*>(p);
  u32x2e v;
  if constexpr (NT)
    v = __builtin_nontemporal_load(q);
  else
    v = *q;
  uint2 r;
  r.x = v.x;
  r.y = v.y;
  return r;
}
template <bool NT>
__device__ __forceinline__ float4 ld_f4(const float* p) {
  const f32x4v* q = reinterpret_cast<const f32x4v*>(p);
  f32x4v v;
  if constexpr (NT)
    v = __builtin_nontemporal_load(q);
  else
    v = *q;
  return make_float4(v.x, v.y, v.z, v.w);
}
template <bool NT>
__device__ __forceinline__ void st_f4(float* p, float a, float b, float c, float d) {
  const f32x4v v = {a, b, c, d};
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
  else
    *reinterpret_cast<f32x4v*>(p) = v;
}

// GK: 0 = bf16 gradient, 1 = fp32 gradient, 2 = NS-only (copy fp32 input).
// N goes to the fp32 buffer x32, or, when nb is given, to the bf16 iterate
// nb itself (the bf16 paths, which fold 1/nu into their first
// iteration), padding included: each block clears its rows' padded columns
// and a unit's last block its padded rows.
// Units u0, u0 + 1, ... (not transposed) take blocks_per_unit blocks each;
// a unit's partial sums fill slots 0 .. blocks_per_unit - 1 of its pp
// slots, and its last block zeroes the rest.
template <int GK, bool NT>
__global__ __launch_bounds__(kThreads) void k_momentum(ChunkArgs ca, float* __restrict__ x32,
                                                        uint16_t* __restrict__ nb,
                                                        double* __restrict__ partials,
                                                        int rows_per_block, int blocks_per_unit,
                                                        int u0, int pp) {
  __shared__ double sh[kThreads / 64];
  const int u = u0 + (int)(blockIdx.x / blocks_per_unit);
  const int bb = (int)blockIdx.x - (u - u0) * blocks_per_unit;
  const SegView sg = find_seg(ca, u);
  const int64_t uoff = (int64_t)(u - sg.first) * ca.unit_elems;
  const int cols = ca.cols;
  const int r0 = bb * rows_per_block;
  const int r1 = min(r0 + rows_per_block, ca.rows);
  const float ma = ca.ma, mb = ca.mb, la = ca.la, lb = ca.lb;
  float* xu = nb ? nullptr : x32 + (int64_t)u * ca.x_stride;  // x32 is null with nb
  uint16_t* const nbu = nb ? nb + (int64_t)u * ca.x_stride : nullptr;
  double ss = 0.0;
  const bool vec = (cols & 3) == 0;
  for (int r = r0; r < r1; ++r) {
    const int64_t base = uoff + (int64_t)r * cols;
    float* const xr = xu ? xu + (int64_t)r * ca.cols_pad : nullptr;
    uint16_t* const nr = nbu ? nbu + (int64_t)r * ca.cols_pad : nullptr;
    if (vec) {
      for (int c = threadIdx.x * 4; c < cols; c += kThreads * 4) {
        float g[4];
        if (GK == 0) {
          const uint2 raw = ld_u2<NT>(static_cast<const uint16_t*>(sg.g) + base + c);
          g[0] = bf16_bits_to_f32(raw.x & 0xffffu);
          g[1] = bf16_bits_to_f32(raw.x >> 16);
          g[2] = bf16_bits_to_f32(raw.y & 0xffffu);
          g[3] = bf16_bits_to_f32(raw.y >> 16);
        } else {
          const float4 v = ld_f4<NT>(static_cast<const float*>(sg.g) + base + c);
          g[0] = v.x; g[1] = v.y; g[2] = v.z; g[3] = v.w;
        }
        float n[4];
        if (GK == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) n[i] = g[i];
        } else {
          float* const mp = sg.m + base + c;
          const float4 mv = ld_f4<NT>(mp);
          float m[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m[i] = __builtin_fmaf(ma, m[i], mb * g[i]);
            n[i] = __builtin_fmaf(la, m[i], lb * g[i]);
          }
          st_f4<NT>(mp, m[0], m[1], m[2], m[3]);
        }
        if (nr)
          store_bf16x4(nr, c, n[0], n[1], n[2], n[3]);
        else
          *reinterpret_cast<float4*>(xr + c) = make_float4(n[0], n[1], n[2], n[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = __builtin_fma((double)n[i], (double)n[i], ss);
      }
    } else {
      for (int c = threadIdx.x; c < cols; c += kThreads) {
        float g;
        if (GK == 0)
          g = bf16_bits_to_f32(static_cast<const uint16_t*>(sg.g)[base + c]);
        else
          g = static_cast<const float*>(sg.g)[base + c];
        float n;
        if (GK == 2) {
          n = g;
        } else {
          float m = __builtin_fmaf(ma, sg.m[base + c], mb * g);
          sg.m[base + c] = m;
          n = __builtin_fmaf(la, m, lb * g);
        }
        if (nr)
          nr[c] = to_bf16_bits(n);
        else
          xr[c] = n;
        ss = __builtin_fma((double)n, (double)n, ss);
      }
    }
    if (nr)
      for (int c = cols + threadIdx.x; c < ca.cols_pad; c += kThreads) nr[c] = 0;
  }
  if (nbu && bb == blocks_per_unit - 1)
    for (int64_t e = (int64_t)ca.rows * ca.cols_pad + threadIdx.x; e < ca.x_stride; e += kThreads)
      nbu[e] = 0;
  const double t = block_sum(ss, sh);
  if (threadIdx.x == 0) partials[(int64_t)u * pp + bb] = t;
  if (bb == blocks_per_unit - 1)
    for (int i = blocks_per_unit + threadIdx.x; i < pp; i += kThreads) partials[(int64_t)u * pp + i] = 0.0;
}

// The same for transposed units (a tall chunk's wide units): the caller's
// matrices are cols x rows (chunk shape rows x cols), and N^T goes to the
// iterate.  One 64 x 64 tile of the caller matrix per workgroup, over its
// padded extent (cols_pad x rows_pad); the tile passes through LDS so that
// both the caller-side accesses and the iterate's rows are contiguous, and
// elements outside the matrix give the iterate's zero padding.  Partial
// sums: one per tile, the unit's remaining slots zeroed by its last tile.
template <int GK, bool NT>
__global__ __launch_bounds__(kThreads) void k_momentum_t(ChunkArgs ca, float* __restrict__ x32,
                                                          uint16_t* __restrict__ nb,
                                                          double* __restrict__ partials, int u0,
                                                          int pp) {
  __shared__ float tile[64][65];
  __shared__ double sh[kThreads / 64];
  const int tr = ca.cols_pad / 64, tc = ca.rows_pad / 64;  // tiles of the caller matrix
  const int per_unit = tr * tc;
  const int u = u0 + (int)(blockIdx.x / per_unit);
  const int bb = (int)blockIdx.x - (u - u0) * per_unit;
  const int ti = bb / tc, tj = bb - ti * tc;
  const SegView sg = find_seg(ca, u);
  const int64_t uoff = (int64_t)(u - sg.first) * ca.unit_elems;
  const int crow = ca.cols, ccol = ca.rows;  // caller matrix: crow x ccol
  const int i0 = ti * 64, j0 = tj * 64;
  const float ma = ca.ma, mb = ca.mb, la = ca.la, lb = ca.lb;
  const int t = threadIdx.x;
  double ss = 0.0;
  const bool vec = (ccol & 3) == 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = t / 16 + 16 * k, cc = (t % 16) * 4;
    const int i = i0 + rr, j = j0 + cc;
    float n[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < crow && j < ccol) {
      const int64_t e = uoff + (int64_t)i * ccol + j;
      float g[4] = {0.f, 0.f, 0.f, 0.f};
      float m[4] = {0.f, 0.f, 0.f, 0.f};
      const int w = vec ? 4 : min(4, ccol - j);
      if (vec) {
        if (GK == 0) {
          const uint2 raw = ld_u2<NT>(static_cast<const uint16_t*>(sg.g) + e);
          g[0] = bf16_bits_to_f32(raw.x & 0xffffu);
          g[1] = bf16_bits_to_f32(raw.x >> 16);
          g[2] = bf16_bits_to_f32(raw.y & 0xffffu);
          g[3] = bf16_bits_to_f32(raw.y >> 16);
        } else {
          const float4 v = ld_f4<NT>(static_cast<const float*>(sg.g) + e);
          g[0] = v.x;
          g[1] = v.y;
          g[2] = v.z;
          g[3] = v.w;
        }
        if (GK != 2) {
          const float4 v = ld_f4<NT>(sg.m + e);
          m[0] = v.x;
          m[1] = v.y;
          m[2] = v.z;
          m[3] = v.w;
        }
      } else {
        for (int q = 0; q < w; ++q) {
          g[q] = GK == 0 ? bf16_bits_to_f32(static_cast<const uint16_t*>(sg.g)[e + q])
                         : static_cast<const float*>(sg.g)[e + q];
          if (GK != 2) m[q] = sg.m[e + q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GK == 2) {
          n[q] = g[q];
        } else {
          m[q] = __builtin_fmaf(ma, m[q], mb * g[q]);
          n[q] = __builtin_fmaf(la, m[q], lb * g[q]);
        }
        if (q >= w) n[q] = 0.f;
      }
      if (GK != 2) {
        if (vec)
          st_f4<NT>(sg.m + e, m[0], m[1], m[2], m[3]);
        else
          for (int q = 0; q < w; ++q) sg.m[e + q] = m[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ss = __builtin_fma((double)n[q], (double)n[q], ss);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[rr][cc + q] = n[q];
  }
  __syncthreads();
  // iterate row j0 + jj (caller column), columns i0 .. i0 + 63 (caller rows)
  float* const xu = nb ? nullptr : x32 + (int64_t)u * ca.x_stride;
  uint16_t* const nbu = nb ? nb + (int64_t)u * ca.x_stride : nullptr;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int jj = t / 16 + 16 * k, ii = (t % 16) * 4;
    const int64_t o = (int64_t)(j0 + jj) * ca.cols_pad + i0 + ii;
    const float a = tile[ii][jj], b = tile[ii + 1][jj], c = tile[ii + 2][jj], d = tile[ii + 3][jj];
    if (nbu)
      store_bf16x4(nbu, o, a, b, c, d);
    else
      *reinterpret_cast<float4*>(xu + o) = make_float4(a, b, c, d);
  }
  const double tot = block_sum(ss, sh);
  if (threadIdx.x == 0) partials[(int64_t)u * pp + bb] = tot;
  if (bb == per_unit - 1)
    for (int i = per_unit + threadIdx.x; i < pp; i += kThreads) partials[(int64_t)u * pp + i] = 0.0;
}

// Folded normalisation: the bf16 iterate holds N itself and the first NS
// iteration applies 1/nu (Gram by 1/nu^2, apply by 1/nu).  Its fp32 Gram
// accumulators hold sums of products of N's entries, so the fold is taken
// for norms in [2^-40, 2^40] (entries' products stay normal, sums finite,
// for units of up to 2^31 elements); other units are scaled in place first.
constexpr double kFoldMin = 0x1p-80, kFoldMax = 0x1p80;  // bounds on nu^2

// Status header at the start of the workspace (32-bit words): word 0 is the
// current call's stop flag, which a persistent launch sets when a wait runs
// out and reads to stop early; word 1 is sticky, the OR of the stop flags of
// every call since the header was last read (muon_workspace_status clears
// both); words 2-3 hold kStatusMagic once the header has been initialised
// (a fresh workspace holds arbitrary bytes).
constexpr uint64_t kStatusMagic = 0x4e4f554d53544154ull;

// Start of a call (one thread of its first launch): the previous call's stop
// flag joins the sticky word and is cleared.
__device__ __forceinline__ void status_fold(uint32_t* err) {
  uint64_t* const magic = reinterpret_cast<uint64_t*>(err + 2);
  if (*magic != kStatusMagic) {
    err[1] = 0u;
    *magic = kStatusMagic;
  } else {
    err[1] |= err[0];
  }
  err[0] = 0u;
}

// One workgroup per unit: fixed-order sum of the partials.
// It also clears the persistent schedule's counts of the unit and claim
// counter (when given), and, on the first pass of a call (err given), moves
// the previous call's stop flag into the sticky word and clears it.  With nb (the
// folded path: unit iterates of x_stride bf16 elements holding N), inv_nu
// receives the first iteration's scale instead: 1/nu inside the fold's
// range, else 1 after the unit has been scaled by 1/nu here.
__global__ __launch_bounds__(kThreads) void k_norm_finish(const double* __restrict__ partials,
                                                          int blocks_per_unit,
                                                          float* __restrict__ inv_nu,
                                                          int32_t* __restrict__ flag,
                                                          uint32_t* __restrict__ sched_done,
                                                          int done_per_unit,
                                                          uint32_t* __restrict__ sched_queue,
                                                          int n_queue_words,
                                                          uint32_t* __restrict__ err,
                                                          uint16_t* __restrict__ nb,
                                                          int64_t x_stride) {
  __shared__ double total;
  __shared__ double sh[kThreads / 64];
  const int u = blockIdx.x;
  {
    // every thread a strided share (a long unit has thousands of partials),
    // then the fixed-order block sum
    double s = 0.0;
    for (int i = threadIdx.x; i < blocks_per_unit; i += kThreads)
      s += partials[(int64_t)u * blocks_per_unit + i];
    s = block_sum(s, sh);
    if (threadIdx.x == 0) total = s;
  }
  __syncthreads();
  const double s = total;
  // A NaN/Inf sum keeps the unit active so that it propagates.
  const bool zero = (s == 0.0);
  const float inv = zero ? 0.0f : (float)(1.0 / sqrt(s));
  const bool rescale = nb && !zero && !(s >= kFoldMin && s <= kFoldMax);
  if (threadIdx.x == 0) {
    flag[u] = zero ? 0 : 1;
    inv_nu[u] = rescale ? 1.0f : inv;
    if (u == 0 && sched_queue)
      for (int i = 0; i < n_queue_words; ++i) sched_queue[i] = 0u;
    if (u == 0 && err) status_fold(err);
  }
  if (sched_done)
    for (int i = threadIdx.x; i < done_per_unit; i += kThreads)
      sched_done[(int64_t)u * done_per_unit + i] = 0u;
  if (rescale) {
    uint4* xu = reinterpret_cast<uint4*>(nb + (int64_t)u * x_stride);
    for (int64_t e = threadIdx.x; e < x_stride / 8; e += kThreads) {
      uint4 v = xu[e];
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)to_bf16_bits(bf16_bits_to_f32(w[i] & 0xffffu) * inv) |
               ((uint32_t)to_bf16_bits(bf16_bits_to_f32(w[i] >> 16) * inv) << 16);
      xu[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// fp32 path: X0 = N * (1/nu) in place over the whole padded iterate (zeros
// in the padding), plus X0^T.  One 64x64 tile per workgroup; the transpose
// goes through LDS so that both the row-major and the transposed writes are
// coalesced.  (The bf16 products need no such pass: their first iteration
// reads N and applies 1/nu itself.)
__global__ __launch_bounds__(kThreads) void k_normalize(ChunkArgs ca, float* __restrict__ x32,
                                                         float* __restrict__ xt,
                                                         const float* __restrict__ inv_nu,
                                                         int tiles_c, int tiles_per_unit) {
  __shared__ float tile[64][65];
  const int u = blockIdx.x / tiles_per_unit;
  const int tt = blockIdx.x - u * tiles_per_unit;
  const int r0 = (tt / tiles_c) * 64, c0 = (tt - (tt / tiles_c) * tiles_c) * 64;
  const float s = inv_nu[u];
  const int cp = ca.cols_pad, rp = ca.rows_pad;
  float* xu = x32 + (int64_t)u * ca.x_stride;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = t / 16 + 16 * i, cc = (t % 16) * 4;
    const int r = r0 + rr, c = c0 + cc;
    const int64_t e = (int64_t)r * cp + c;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < ca.rows && c < ca.cols) {
      const float4 nv = *reinterpret_cast<const float4*>(xu + e);
      val.x = nv.x * s;
      val.y = (c + 1 < ca.cols) ? nv.y * s : 0.f;
      val.z = (c + 2 < ca.cols) ? nv.z * s : 0.f;
      val.w = (c + 3 < ca.cols) ? nv.w * s : 0.f;
    }
    *reinterpret_cast<float4*>(xu + e) = val;
    tile[rr][cc] = val.x;
    tile[rr][cc + 1] = val.y;
    tile[rr][cc + 2] = val.z;
    tile[rr][cc + 3] = val.w;
  }
  __syncthreads();
  // X^T (cols_pad x rows_pad): row c takes tile column c - c0.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = t / 16 + 16 * i, rr = (t % 16) * 4;
    const int64_t e = (int64_t)u * ca.x_stride + (int64_t)(c0 + cc) * rp + r0 + rr;
    const float a = tile[rr][cc], b = tile[rr + 1][cc], c = tile[rr + 2][cc], d = tile[rr + 3][cc];
    *reinterpret_cast<float4*>(xt + e) = make_float4(a, b, c, d);
  }
}

// ------------------------------------------------------------------ GEMM ---
// Batched C = A_op * B_op^T over padded units (both operands K-contiguous),
// one TILE x TILE output tile per workgroup.  256 tiles take 8 waves in a
// 4 x 2 grid (64 x 128 each), two per SIMD: a copy instruction holds up the
// issue of its wave for tens of cycles, and the other wave of the SIMD
// keeps the matrix core busy meanwhile (with one wave per SIMD the copies'
// issue time adds to the MFMA time).  128 tiles take 4 waves (2 x 2, 64 x
// 64 each).  Each wave's share is a grid of 32x32 MFMA blocks.
//
// LDS: a ring of kSlots half-stages; a half-stage holds TILE rows of one
// operand, a row being 128 bytes of K (64 bf16 or 32 fp32) in eight 16-byte
// chunks, XOR-swizzled by row so that the 32-row MFMA fragment reads spread
// over the banks.  Rows of 128 bytes make every global request a whole
// line: the L2 serves a fixed number of requests per clock, and with
// 64-byte rows the copies, not the matrix cores, set the pace.  Operands
// stream global -> LDS directly, 1.5 to 2.5 stages ahead of the MFMAs
// (buffer_load_dwordx4 ... lds: lane i of a wave lands at M0 + 16*i, so the
// swizzle is applied by choosing which global chunk each lane fetches).
// Fragments are double-buffered across the four K sub-steps of a stage, and
// the MFMA is issued as (B, A) so each lane accumulates C[m][n..n+3] for
// one row m and four consecutive columns: the epilogue moves 16-byte
// vectors.
template <typename T>
struct OpT;
template <>
struct OpT<__bf16> {
  static constexpr int kElems = 8;  // per 16-byte chunk
  static constexpr int kBK = 64;    // K per 128-byte LDS row (8 chunks)
};
template <>
struct OpT<float> {
  static constexpr int kElems = 4;
  static constexpr int kBK = 32;
};

constexpr int kRowChunks = 8;  // 16-byte chunks per 128-byte LDS row
constexpr int kSlots = 5;      // ring of half-stages (one operand each)

typedef __attribute__((address_space(3))) void* lds_vptr;

// Physical 16-byte chunk of logical chunk c in a 128-byte row: 16
// consecutive rows read at one logical chunk hit 16 distinct 4-bank groups
// (two rows per 256-byte bank line, eight chunk positions per parity).
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Buffer resource (4 SGPRs) for a raw buffer at `base`: stride 0, a 2 GiB
// range and the 32-bit data format of the gfx9 family.
// The base is uniform across the workgroup; readfirstlane keeps the
// descriptor in scalar registers whatever the compiler can prove.
__device__ __forceinline__ u32x4 tile_rsrc(const void* base) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return u32x4{lo, hi & 0xFFFFu, 0x7FFFFFFFu, 0x00020000u};
}

// Waves and threads of a GEMM workgroup.
template <int TILE>
constexpr int gemm_waves() { return TILE == 256 ? 8 : 4; }
template <int TILE>
constexpr int gemm_threads() { return 64 * gemm_waves<TILE>(); }

// Copy instructions per wave for one half-stage (TILE rows x 128 bytes).
template <int TILE>
constexpr int dma_per_wave() { return TILE * kRowChunks / (64 * gemm_waves<TILE>()); }

// One operand's share of a half-stage for this wave: TILE rows of the tile
// (resource based at its first row) x 128 bytes of K, eight lanes per row so
// that every request is a whole 128-byte line.  `voff` holds the
// stage-invariant per-lane byte offsets (row * ld + swizzled chunk), the K
// position comes in as the scalar offset `koff`, and lds_op is the LDS byte
// offset of the ring slot.  Lane i of each instruction lands at M0 + 16*i,
// so the swizzle is applied by choosing which global chunk each lane
// fetches.
//
// The copy is issued as inline assembly so that the compiler does not see an
// LDS writer: it cannot tell the slots apart and would otherwise wait for
// every copy in flight before each LDS read.  Completion is tracked with
// explicit vmcnt waits (vmcnt counts every vector-memory instruction in
// issue order) before the barrier that publishes a stage.
//
// K-major operands (KM, bf16 only) are stored with K along the rows (the
// iterate X read as the right operand of B'*X, or both sides of X^T X): a
// half-stage holds BK rows of K x TILE columns, a row being TILE * 2 bytes
// in 16-byte chunks, chunk c of row k stored at c ^ (4 * (k & 3)).  Each
// row is copied as whole 128-byte lines (the XOR keeps every aligned group
// of eight chunks together), and the MFMA fragments are read with the
// transposing LDS read (see read_km).
template <typename T, int TILE, bool KM = false>
struct DmaPlan {
  static constexpr int kN = dma_per_wave<TILE>();
  int voff[kN];
  __device__ __forceinline__ void init(int ld) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int sl = (w * kN + i) * 64 + lane;
      if constexpr (KM) {
        static_assert(sizeof(T) == 2, "K-major operands are bf16");
        constexpr int CPR = TILE / 8;      // 16-byte chunks per K row
        const int kr = sl / CPR, pc = sl % CPR;
        const int c = pc ^ (4 * (kr & 3));  // logical chunk stored at (kr, pc)
        voff[i] = (kr * ld + c * 8) * 2;
      } else {
        const int row = sl >> 3, pc = sl & 7;
        const int c = pc ^ ((row >> 1) & 7);  // logical chunk stored at (row, pc)
        voff[i] = (row * ld + c * OpT<T>::kElems) * (int)sizeof(T);
      }
    }
  }
  // Instruction i of this wave's share.
  __device__ __forceinline__ void issue_one(const u32x4& rs, uint32_t koff, uint32_t lds_op,
                                            int i) const {
    const int w = threadIdx.x >> 6;
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_op + (uint32_t)((w * kN + i) * 64) * 16u);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0v), "v"(voff[i]), "s"(rs), "s"(koff)
                 : "memory", "m0");
  }
};

// blockIdx -> logical tile so that each XCD (blocks are dealt round-robin to
// the 8 XCDs) works on one contiguous range of tiles, keeping a unit's
// operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int x = bid & 7, i = bid >> 3;
  const int q = nb >> 3, rem = nb & 7;
  return x * q + min(x, rem) + i;
}

// One 32x32 block over one 16-byte K chunk: a single bf16 MFMA, or four
// fp32 ones.  Issued as (B, A): the lane owning C row m receives 4
// consecutive columns.
template <typename T>
__device__ __forceinline__ void mfma_one(const u32x4& af, const u32x4& bf, f32x16& acc) {
  if constexpr (sizeof(T) == 2) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bf),
                                                  __builtin_bit_cast(bf16x8, af), acc, 0, 0, 0);
  } else {
    const f32x4v a4 = __builtin_bit_cast(f32x4v, af);
    const f32x4v b4 = __builtin_bit_cast(f32x4v, bf);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(b4[q], a4[q], acc, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Lanes of one wave exchanging data through LDS: the hardware runs a wave's
// LDS accesses in order, but the compiler reasons per lane and may reorder a
// lane's accesses to different addresses, or reuse a value the lane loaded
// before another lane overwrote it (a version of the epilogue whose staging
// writes were made by half of the lanes had its reads of the other lanes'
// rows replaced by the values loaded for the previous rows).  A compiler
// fence between the phases of such an exchange keeps them in program order.
__device__ __forceinline__ void wave_lds_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Workgroup barrier for LDS broadcasts: waits for this wave's LDS (and
// scalar) accesses only, not for its global stores and atomics in flight,
// which a __syncthreads() fence would drain first.  The signal fences keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The XCC (accelerator die, with its own L2) the workgroup runs on.
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg((3 << 11) | 20)) & 15;
}

// Atomic add of v at the wave-uniform address p, made by lane 0 alone: the
// execution mask is narrowed to lane 0 for that one instruction, so the
// wave makes exactly one request to the L2.  Left to the compiler, a
// wave's atomic is either rewritten into one atomic of the lanes' sum or
// issued by all 64 lanes (63 of them adding 0), and which of the two it
// does changed with unrelated edits elsewhere in the kernel; 64-lane
// atomics on the one queue line made the whole schedule about five times
// slower.  The leading s_nop covers an address the compiler has just
// moved into scalar registers from a vector one, the trailing one the
// execution-mask write the compiler does not see (an instruction that
// reads the mask through DPP must not follow it at once).  The returning
// form waits for its result (and so for every older vector-memory access
// of the wave) and gives every lane the old value; the other form does not
// wait.  Both are called in wave-uniform code with every lane active: lane
// 0 must hold v and the zero offset when the mask is narrowed.
__device__ __forceinline__ uint32_t lane0_atomic_add(uint32_t* p, uint32_t v) {
  uint32_t old;
  uint64_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b64 %[sv], exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %[old], %[zero], %[v], %[base] sc0\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_mov_b64 exec, %[sv]\n\t"
      "s_nop 4"
      : [old] "=&v"(old), [sv] "=&s"(saved)
      : [zero] "v"(0u), [v] "v"(v), [base] "s"(p)
      : "memory");
  return __builtin_amdgcn_readfirstlane(old);
}
__device__ __forceinline__ void lane0_atomic_add_noret(uint32_t* p, uint32_t v) {
  uint64_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b64 %[sv], exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %[zero], %[v], %[base]\n\t"
      "s_mov_b64 exec, %[sv]\n\t"
      "s_nop 4"
      : [sv] "=&s"(saved)
      : [zero] "v"(0u), [v] "v"(v), [base] "s"(p)
      : "memory");
}

// LDS of the GEMM tile: a ring of kSlots half-stages, each TILE rows of
// one operand x 128 bytes of K (160 KB at TILE 256).  Declared once per tile
// size, so a kernel that runs several tile phases holds a single ring; the
// epilogue stages its blocks in it too.
template <int TILE>
__shared__ u32x4 lds_ring[kSlots * TILE * kRowChunks];

// Zero unit in the last iteration: O' = 0, so the weight only decays (step)
// or the NS output is zero, over the TILE x TILE block at (m0, n0).
template <int TILE>
__device__ __forceinline__ void zero_unit_tile(const UnitOut& o, int final_mode, int m0, int n0) {
  for (int idx = threadIdx.x; idx < TILE * TILE; idx += gemm_threads<TILE>()) {
    // a transposed unit's caller element (nn, mm) is the chunk's (mm, nn);
    // walk the tile so that consecutive threads touch consecutive elements
    const int a = idx / TILE, b = idx % TILE;
    const int mm = m0 + (o.trans ? b : a), nn = n0 + (o.trans ? a : b);
    if (mm < o.rows && nn < o.cols) {
      float* p = o.w + (o.trans ? (int64_t)nn * o.rows + mm : (int64_t)mm * o.cols + nn);
      *p = (final_mode == FINAL_STEP) ? (*p) * o.decay : 0.0f;
    }
  }
}

// One TILE x TILE output tile (tm, tn) of unit u.  Every wave of the
// workgroup calls it; it starts by overwriting the LDS stage buffers, so the
// caller makes sure no wave still reads them (a barrier after the previous
// tile's epilogue).
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// `out_of()` gives the unit's UnitOut; the final apply epilogue calls it.
// `issued` runs once the prologue's first copies are in flight (the
// persistent schedule claims its next item there, so that the claim's round
// trip overlaps the copies' latency); `ready` runs after the prologue's
// barrier, when every wave's older memory accesses are complete.
//
// KM: bit 0 = the A operand is K-major, bit 1 = the B operand is.
template <int PHASE, typename T, int TILE, int KM = 0, bool FOLD = false, typename OutFn = NoHook,
          typename Hook = NoHook, typename Hook2 = NoHook>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const OutFn& out_of, int u, int tm,
                                          int tn, const Hook& issued = Hook(),
                                          const Hook2& ready = Hook2()) {
  constexpr int NW = gemm_waves<TILE>();
  constexpr int WM = TILE / (NW / 2);  // wave tile rows (waves in a (NW/2) x 2 grid)
  constexpr int WN = TILE / 2;         // wave tile columns
  constexpr int FA = WM / 32;          // 32x32 blocks per wave: FA rows x FB columns
  constexpr int FB = WN / 32;
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int BK = OpT<T>::kBK;
  constexpr int NI = dma_per_wave<TILE>();     // copies per wave per half-stage
  constexpr int kSlot = TILE * kRowChunks;     // 16-byte slots per ring slot
  u32x4* const ring = lds_ring<TILE>;
  const uint32_t ring_off = (uint32_t)(uintptr_t)(lds_vptr)lds_ring<TILE>;
  const int m0 = tm * TILE, n0 = tn * TILE;
  // Lane-dependent values are recomputed for every tile (see the copy
  // offsets below): an opaque copy of the lane index keeps the compiler
  // from hoisting each phase's per-lane addressing out of a persistent loop.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wid >> 1, wn = wid & 1;

  constexpr bool AKM = (KM & 1) != 0, BKM = (KM & 2) != 0;
  static_assert(KM == 0 || sizeof(T) == 2, "K-major operands are bf16");
  const T* A = static_cast<const T*>(g.a) + (int64_t)u * g.a_ustride;
  const T* B = static_cast<const T*>(g.b) + (int64_t)u * g.b_ustride;
  // a K-major operand's tile starts at its first column, a row-major one at its first row
  const u32x4 rsa = tile_rsrc(AKM ? A + m0 : A + (int64_t)m0 * g.lda);
  const u32x4 rsb = tile_rsrc(BKM ? B + n0 : B + (int64_t)n0 * g.ldb);

  f32x16 acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Stages of BK along K, each two half-stages: 2k holds A_op's rows, 2k+1
  // B_op's.  Half-stage h lives in ring slot h % kSlots.
  const int nk = g.K / BK;  // >= 2 (K is a multiple of 128)
  const int nh = 2 * nk;
  // The per-lane copy offsets are recomputed for every tile: an opaque copy
  // of the leading dimensions keeps the compiler from hoisting them out of
  // a persistent tile loop, where they would stay live for every phase.
  int lda = g.lda, ldb = g.ldb;
  asm volatile("" : "+s"(lda), "+s"(ldb));
  DmaPlan<T, TILE, AKM> pa;
  DmaPlan<T, TILE, BKM> pb;
  pa.init(lda);
  pb.init(ldb);
  auto issue_half = [&](int h, int i) {  // copy instruction i of half-stage h
    // K offset of the stage: along a row-major operand's rows, or whole rows
    // of a K-major one
    const uint32_t kst = (uint32_t)((h >> 1) * BK * (int)sizeof(T));
    const uint32_t so = ring_off + (uint32_t)((h % kSlots) * kSlot) * 16u;
    if (h & 1)
      pb.issue_one(rsb, BKM ? kst * (uint32_t)ldb : kst, so, i);
    else
      pa.issue_one(rsa, AKM ? kst * (uint32_t)lda : kst, so, i);
  };

  // Schedule of stage k (four K sub-steps kk0..kk3 of 16 bf16 / 8 fp32):
  //   sub-steps 0-2: read the fragments of kk(s+1) | MFMAs of kk(s), with
  //   the copies of half-stage 2k+4 (A of stage k+2) spread over sub-steps
  //   0 and 1 (as early as the slot allows, which gives them the most time
  //   to land; spread over all three they ran ~1% slower), into the slot of
  //   half 2k-1, which the previous stage's barrier released
  //   wait for this wave's copies of stage k+1 (half-stage 2k+4 may stay in
  //   flight); s_barrier: stage k+1 is complete and every wave is done
  //   reading stage k
  //   sub-step 3: copies of half-stage 2k+5 (B of stage k+2) into the slot
  //   of half 2k, interleaved with the reads of kk0(k+1) and the MFMAs of
  //   kk3(k)
  // A copy instruction holds up its wave's issue until the address unit
  // takes it, so the copies are spread over the whole stage rather than
  // bunched after the barrier.  The barrier sits between MFMA groups whose
  // operands are already in registers, so the fragment reads after it hide
  // under MFMAs.
  const int arow0 = wm * WM + (lane & 31);
  const int brow0 = wn * WN + (lane & 31);
  const int half = lane >> 5;
  // Waves w and w + 4 share a SIMD: the second one issues its copies half
  // a copy interval later, so that the two do not wait on the address unit
  // at the same time.
  const bool second = NW == 8 && wid >= 4;
  u32x4 af[2][FA], bf[2][FB];
  // Fragment of a K-major operand: lane (x, half) needs K rows 16kk + 8half
  // + 0..7 of column x.  Two transposing reads (ds_read_b64_tr_b16): in
  // each group of 16 lanes, lane 4r + q points at 4 elements of K row
  // k0 + r, columns 4q..4q+3 of the group's 16, and lane i receives column
  // i of those four rows.
  // The swizzle term depends on the lane only (16kk and +4 rows keep
  // k & 3), so each lane's byte offset within a slot is fixed per 32-column
  // block; the sub-step and the second read are immediate offsets.
  int kmoa[AKM ? FA : 1], kmob[BKM ? FB : 1];
  {
    const int gq = lane >> 4, gi = lane & 15;
    const int kr = 8 * (gq >> 1) + (gi >> 2);  // K row of the first read in sub-step 0
    const int x4 = 4 * (kr & 3);
    auto km_off = [&](int colbase) {
      const int col = colbase + 16 * (gq & 1) + 4 * (gi & 3);
      return (kr * TILE + ((((col >> 3) ^ x4) << 3) | (col & 7))) * 2;
    };
    if constexpr (AKM) {
#pragma unroll
      for (int i = 0; i < FA; ++i) kmoa[i] = km_off(wm * WM + i * 32);
    }
    if constexpr (BKM) {
#pragma unroll
      for (int j = 0; j < FB; ++j) kmob[j] = km_off(wn * WN + j * 32);
    }
  }
  auto read_km = [&](const u32x4* S, int kk, int off) -> u32x4 {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    __attribute__((address_space(3))) char* base =
        (__attribute__((address_space(3))) char*)(lds_vptr)S + off + kk * 16 * TILE * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)base);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(base + 4 * TILE * 2));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };
  auto read_a = [&](const u32x4* S, int kk, int slot, int i) {
    if constexpr (AKM) {
      af[slot][i] = read_km(S, kk, kmoa[i]);
    } else {
      const int r = arow0 + i * 32;
      af[slot][i] = S[r * kRowChunks + swz(r, 2 * kk + half)];
    }
  };
  auto read_b = [&](const u32x4* S, int kk, int slot, int i) {
    if constexpr (BKM) {
      bf[slot][i] = read_km(S, kk, kmob[i]);
    } else {
      const int r = brow0 + i * 32;
      bf[slot][i] = S[r * kRowChunks + swz(r, 2 * kk + half)];
    }
  };

  // Prologue: half-stages 0..3 (nh >= 4).  The scalar (kernel-argument)
  // loads are drained as well: one still in flight would turn every LDS
  // wait of the loop into a full wait.
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < NI; ++i) issue_half(h, i);
  issued();
#pragma unroll
  for (int h = 2; h < 4; ++h)
#pragma unroll
    for (int i = 0; i < NI; ++i) issue_half(h, i);
  wait_vmcnt<2 * NI>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  ready();
#pragma unroll
  for (int i = 0; i < FA; ++i) read_a(ring, 0, 0, i);
#pragma unroll
  for (int j = 0; j < FB; ++j) read_b(ring + kSlot, 0, 0, j);

  int sa = 0, sb = 1;  // ring slots of stage k
  for (int k = 0; k < nk; ++k) {
    const u32x4* SA = ring + sa * kSlot;
    const u32x4* SB = ring + sb * kSlot;
    const int na = sa + 2 >= kSlots ? sa + 2 - kSlots : sa + 2;
    const int nb = sb + 2 >= kSlots ? sb + 2 - kSlots : sb + 2;
    const int ha = 2 * k + 4;
    const bool more_a = ha < nh;
#pragma unroll
    for (int ss = 0; ss < 3; ++ss) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FA; ++i) read_a(SA, ss + 1, (ss + 1) & 1, i);
#pragma unroll
      for (int j = 0; j < FB; ++j) read_b(SB, ss + 1, (ss + 1) & 1, j);
      __builtin_amdgcn_sched_barrier(0);
      // this sub-step's share of the copies of half-stage ha (half of them
      // in sub-steps 0 and 1 each, none in 2), spread over its MFMA blocks
      constexpr int M = FA * FB;
      const int c0 = ss * NI / 2 < NI ? ss * NI / 2 : NI;
      const int c1 = (ss + 1) * NI / 2 < NI ? (ss + 1) * NI / 2 : NI;
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int c = c0; c < c1; ++c) {
          const int at = (c - c0) * M / (c1 - c0);
          const int later = at + M / (c1 - c0) / 2;
          if (more_a && ((!second && m == at) || (second && m == later))) issue_half(ha, c);
        }
        mfma_one<T>(af[ss & 1][m / FB], bf[ss & 1][m % FB], acc[m / FB][m % FB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Publish stage k+1 (for the last stage this only drains the copies;
    // the reads below then touch stale slots whose values go unused, which
    // keeps the MFMA block on a single control path).
    if (k + 3 <= nk)
      wait_vmcnt<NI>();
    else
      wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    {
      const int h0 = 2 * k + 5;
      const bool more0 = h0 < nh;
      const u32x4* NA = ring + na * kSlot;
      const u32x4* NB = ring + nb * kSlot;
      constexpr int C = NI;          // copy instructions
      constexpr int R = FA + FB;     // fragment reads
      constexpr int M = FA * FB;     // MFMA blocks
      static_assert(M >= C && M >= R, "at most one copy and one read per MFMA block");
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int at = c * M / C, later = at + M / C / 2;
          if (more0 && ((!second && m == at) || (second && m == later))) issue_half(h0, c);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (m == r * M / R) {
            if (r < FA)
              read_a(NA, 0, 0, r);
            else
              read_b(NB, 0, 0, r - FA);
          }
        }
        mfma_one<T>(af[1][m / FB], bf[1][m % FB], acc[m / FB][m % FB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    sa = na;
    sb = nb;
  }

  // ---- epilogue.  Each wave stages one 32-row block of its accumulators at
  // a time in its own LDS region (lane (m, half) holds C[m][n..n+3]), then
  // reads it back row-wise so that every global load and store covers whole
  // row segments (WN/4 lanes per row, 16 bytes per lane); the transposed
  // copy reads the staged block column-wise.
  constexpr int LDW = WN + 4;     // padded row stride (floats)
  constexpr int LPR = WN / 4;     // lanes per row
  constexpr int RPI = 64 / LPR;   // rows per instruction
  constexpr int NIT = 32 / RPI;   // row-wise iterations per block
  const int rl = lane / LPR;            // row within an instruction
  const int cl = (lane % LPR) * 4;      // first column of the lane
  const int ncol = n0 + wn * WN + cl;   // global column of the lane's first element
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  float* ep = reinterpret_cast<float*>(ring) + wid * (32 * LDW);
  UnitOut uo{nullptr, 0, 0.0f, 0, 0, 1.0f};
  if constexpr (PHASE == APPLY) {
    if (g.final_mode != FINAL_NONE) uo = out_of();
  }
  float* const wout = uo.w;
  const bool wtrans = uo.trans != 0;  // the unit's weight is the chunk shape transposed
  const float lrs = uo.lr_scale;      // lr * the unit's update scale
  const int wrows = uo.rows, wcols = uo.cols;
  const float wdecay = uo.decay;
  const bool vec_w = (wcols & 3) == 0;
  // FOLD (first iteration of the folded path): X = N, so A = (N N^T)/nu^2
  // and X' = (B' N)/nu; the accumulators take the scale as they are staged.
  // A separate instantiation, so that the other tiles' epilogues carry
  // neither the branch nor its registers.
  const float fs = FOLD ? g.fold[u] : 1.0f;
  const float acc_scale = PHASE == GRAM ? fs * fs : fs;
  // bf16 auxiliary input (A, for POLY's b*A term), row-wise, two blocks
  // ahead: blocks 0 and 1 are issued here and block i + 2 once block i has
  // taken its values, so the load latency is paid about once per tile.
  constexpr bool kAuxB = PHASE == POLY && kBF;
  uint2 auxr[kAuxB ? 2 : 1][NIT];
  const uint16_t* const aux_p =
      kAuxB ? static_cast<const uint16_t*>(g.aux16) + (int64_t)u * g.aux_ustride + ncol : nullptr;
  auto load_aux = [&](int i) {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      auxr[i & 1][it] = *reinterpret_cast<const uint2*>(
          aux_p + (int64_t)(m0 + wm * WM + i * 32 + it * RPI + rl) * g.ldaux);
  };
  if constexpr (kAuxB) {
    load_aux(0);
    if (FA > 1) load_aux(1);
  }
#pragma unroll
  for (int i = 0; i < FA; ++i) {
    const int mrow0 = m0 + wm * WM + i * 32;  // first global row of the block
    // auxiliary input of the block, row-wise (fp32: issued before the
    // staging; bf16: converted as the row pass uses it)
    float4 aux[(PHASE == POLY && !kBF) ? NIT : 1];
    auto aux_at = [&](int it) -> float4 {
      if constexpr (kAuxB) {
        const uint2 h = auxr[i & 1][it];
        return make_float4(bf16_bits_to_f32(h.x & 0xffffu), bf16_bits_to_f32(h.x >> 16),
                           bf16_bits_to_f32(h.y & 0xffffu), bf16_bits_to_f32(h.y >> 16));
      } else {
        return aux[(PHASE == POLY && !kBF) ? it : 0];
      }
    };
    if constexpr (PHASE == POLY && !kBF) {
      const float* ap = g.aux + (int64_t)u * g.aux_ustride + ncol;
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        aux[it] = *reinterpret_cast<const float4*>(ap + (int64_t)(mrow0 + it * RPI + rl) * g.ldaux);
    }
    if constexpr (FOLD && PHASE != POLY) {
#pragma unroll
      for (int j = 0; j < FB; ++j) acc[i][j] *= acc_scale;
    }
    // stage the block (after the previous block's reads)
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& c = acc[i][j];
        *reinterpret_cast<float4*>(ep + (lane & 31) * LDW + j * 32 + 8 * q + 4 * half) =
            make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
      }
    wave_lds_fence();
    // row-wise pass (a wave's LDS accesses complete in order)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + rl;
      const float4 cv = *reinterpret_cast<const float4*>(ep + r * LDW + cl);
      const int m = mrow0 + r;
      float v0 = cv.x, v1 = cv.y, v2 = cv.z, v3 = cv.w;
      const int64_t o = (int64_t)u * g.out_ustride + (int64_t)m * g.ldo + ncol;
      if constexpr (PHASE == GRAM || PHASE == POLY) {
        if constexpr (PHASE == POLY) {
          const float4 a = aux_at(it);
          v0 = g.cb * a.x + g.cc * v0;
          v1 = g.cb * a.y + g.cc * v1;
          v2 = g.cb * a.z + g.cc * v2;
          v3 = g.cb * a.w + g.cc * v3;
          if (tm == tn) {
            // B' = a*I + b*A + c*A^2: the apply's a*X term rides on the
            // diagonal (the padded diagonal too; X is zero there)
            const int d = m - ncol;
            v0 += d == 0 ? g.ca : 0.0f;
            v1 += d == 1 ? g.ca : 0.0f;
            v2 += d == 2 ? g.ca : 0.0f;
            v3 += d == 3 ? g.ca : 0.0f;
          }
          // the mirror pass below reads the final values
          *reinterpret_cast<float4*>(ep + r * LDW + cl) = make_float4(v0, v1, v2, v3);
        }
        if constexpr (kBF)
          store_bf16x4(g.out16, o, v0, v1, v2, v3);
        else
          *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v0, v1, v2, v3);
      } else {
        // X' = B' X (or X B'): the staged block is the result
        if (g.final_mode == FINAL_NONE) {
          if constexpr (kBF)
            store_bf16x4(g.out16, o, v0, v1, v2, v3);
          else
            *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v0, v1, v2, v3);
        } else if (!wtrans && m < wrows && ncol < wcols) {
          const int n = ncol;
          float* p = wout + (int64_t)m * wcols + n;
          const bool step = g.final_mode == FINAL_STEP;
          if (vec_w && n + 3 < wcols) {
            float4 wv = step ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
            if (step) {
              wv.x = __builtin_fmaf(-lrs, v0, wv.x * wdecay);
              wv.y = __builtin_fmaf(-lrs, v1, wv.y * wdecay);
              wv.z = __builtin_fmaf(-lrs, v2, wv.z * wdecay);
              wv.w = __builtin_fmaf(-lrs, v3, wv.w * wdecay);
            } else {
              wv = make_float4(v0, v1, v2, v3);
            }
            *reinterpret_cast<float4*>(p) = wv;
          } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (n + e < wcols)
                p[e] = step ? __builtin_fmaf(-lrs, vv[e], p[e] * wdecay) : vv[e];
            }
          }
        }
      }
    }
    if constexpr (kAuxB) {
      if (i + 2 < FA) load_aux(i + 2);  // the row pass has taken block i's values
    }
    wave_lds_fence();  // the column-wise passes read what other lanes wrote
    if constexpr (PHASE == GRAM || PHASE == POLY) {
      if (g.sym && tm != tn) {
        // mirror tile: rows n0 + wn*WN .. +WN, columns mrow0 .. +32, read
        // column-wise from the staged block (8 lanes per row, 4 columns each)
        const int cm = (lane & 7) * 4;
#pragma unroll
        for (int it = 0; it < WN / 8; ++it) {
          const int nn = it * 8 + (lane >> 3);
          const float a0 = ep[(cm + 0) * LDW + nn], a1 = ep[(cm + 1) * LDW + nn];
          const float a2 = ep[(cm + 2) * LDW + nn], a3 = ep[(cm + 3) * LDW + nn];
          const int64_t om = (int64_t)u * g.out_ustride + (int64_t)(n0 + wn * WN + nn) * g.ldo + mrow0 + cm;
          if constexpr (kBF)
            store_bf16x4(g.out16, om, a0, a1, a2, a3);
          else
            *reinterpret_cast<float4*>(g.out32 + om) = make_float4(a0, a1, a2, a3);
        }
      }
    }
    if constexpr (PHASE == APPLY) {
      if (wtrans) {
        // transposed unit: caller row n0 + wn*WN + nn holds the staged
        // block's column nn, caller columns mrow0 .. +32 its rows (8 lanes
        // per caller row, 4 consecutive elements each)
        const int cm = (lane & 7) * 4;
        const bool step = g.final_mode == FINAL_STEP;
        const bool vec_t = (wrows & 3) == 0;
#pragma unroll
        for (int it = 0; it < WN / 8; ++it) {
          const int nn = it * 8 + (lane >> 3);
          const int crow = n0 + wn * WN + nn, ccol = mrow0 + cm;
          if (crow < wcols && ccol < wrows) {
            const float vv[4] = {ep[(cm + 0) * LDW + nn], ep[(cm + 1) * LDW + nn],
                                 ep[(cm + 2) * LDW + nn], ep[(cm + 3) * LDW + nn]};
            float* p = wout + (int64_t)crow * wrows + ccol;
            if (vec_t && ccol + 3 < wrows) {
              float4 wv = step ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
              if (step) {
                wv.x = __builtin_fmaf(-lrs, vv[0], wv.x * wdecay);
                wv.y = __builtin_fmaf(-lrs, vv[1], wv.y * wdecay);
                wv.z = __builtin_fmaf(-lrs, vv[2], wv.z * wdecay);
                wv.w = __builtin_fmaf(-lrs, vv[3], wv.w * wdecay);
              } else {
                wv = make_float4(vv[0], vv[1], vv[2], vv[3]);
              }
              *reinterpret_cast<float4*>(p) = wv;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (ccol + e < wrows)
                  p[e] = step ? __builtin_fmaf(-lrs, vv[e], p[e] * wdecay) : vv[e];
            }
          }
        }
      }
      if (g.final_mode == FINAL_NONE && g.outt != nullptr) {
        // X'^T rows n0 + wn*WN .. +WN, columns mrow0 .. +32: 8 lanes per
        // row, 4 consecutive columns (staged rows) per lane.
        const int cm = (lane & 7) * 4;
#pragma unroll
        for (int it = 0; it < WN / 8; ++it) {
          const int nn = it * 8 + (lane >> 3);
          const float a0 = ep[(cm + 0) * LDW + nn], a1 = ep[(cm + 1) * LDW + nn];
          const float a2 = ep[(cm + 2) * LDW + nn], a3 = ep[(cm + 3) * LDW + nn];
          const int64_t ot = (int64_t)u * g.out_ustride + (int64_t)(n0 + wn * WN + nn) * g.ldt + mrow0 + cm;
          if constexpr (kBF)
            store_bf16x4(g.outt, ot, a0, a1, a2, a3);
          else
            *reinterpret_cast<float4*>(static_cast<float*>(g.outt) + ot) = make_float4(a0, a1, a2, a3);
        }
      }
    }
  }
}

// Tile orders that keep the tiles claimed together on few operand panels
// (32 CUs of an XCC run 32 consecutive tiles of a unit at once, and the L2
// serves a panel's K-slice to every tile reading it at about the same time).
// Upper triangle of a T x T grid in block rows of G tile rows: block row by
// block row, inside one column by column (rows r0 .. min(c, r0 + G - 1) of
// column c): 32 consecutive tiles read G row panels and about 32 / G column
// panels.
constexpr int kGroupRows = 8;
__device__ __forceinline__ void sym_tile_grouped(int t, int T, int& tm, int& tn) {
  int r0 = 0, h = min(kGroupRows, T);
  for (;;) {
    const int n = h * (h + 1) / 2 + h * (T - r0 - h);  // tiles of this block row
    if (t < n) break;
    t -= n;
    r0 += h;
    h = min(kGroupRows, T - r0);
  }
  if (t < h * (h + 1) / 2) {  // the block row's own triangle: column c has c + 1 tiles
    int c = 0;
    while (t > c) {
      t -= c + 1;
      ++c;
    }
    tm = r0 + t;
    tn = r0 + c;
  } else {  // full columns of h tiles
    t -= h * (h + 1) / 2;
    const int c = t / h;
    tm = r0 + (t - c * h);
    tn = r0 + h + c;
  }
}

// A full tiles_m x tiles_n grid in groups of kGroupRows tile rows, column by
// column inside a group.
__device__ __forceinline__ void grid_tile_grouped(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupRows * tiles_n;
  const int g = t / per_group;
  const int r0 = g * kGroupRows;
  const int h = min(kGroupRows, tiles_m - r0);
  const int w = t - g * per_group;
  tn = w / h;
  tm = r0 + (w - tn * h);
}

// One launch per product: workgroup -> (unit, tile), XCD-aware.
template <int PHASE, typename T, int TILE, int KM>
__global__ __launch_bounds__(gemm_threads<TILE>()) void ns_gemm(GemmArgs g, ChunkArgs ca) {
  const int tiles_per_unit = g.sym ? g.tiles_m * (g.tiles_m + 1) / 2 : g.tiles_m * g.tiles_n;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int u = logical / tiles_per_unit;
  const int tt = logical - u * tiles_per_unit;
  int tm, tn;
  if (g.sym)
    sym_tile_grouped(tt, g.tiles_m, tm, tn);
  else
    grid_tile_grouped(tt, g.tiles_m, g.tiles_n, tm, tn);
  if (!g.flag[u]) {
    if (PHASE == APPLY && g.final_mode != FINAL_NONE)
      zero_unit_tile<TILE>(unit_out(ca, u), g.final_mode, tm * TILE, tn * TILE);
    return;
  }
  auto out_of = [&]() { return unit_out(ca, u); };
  if (PHASE != POLY && g.fold)
    gemm_tile<PHASE, T, TILE, KM, PHASE != POLY>(g, out_of, u, tm, tn);
  else
    gemm_tile<PHASE, T, TILE, KM>(g, out_of, u, tm, tn);
}

// -------------------------------------------------------- small-s NS -------
// Wide units of at most 128 rows (split heads, small matrices), bf16
// products, on chip: the Gram A and B' = bA + cA^2 (128 x 128) never leave
// the workgroup, and each iteration makes one pass over X.
struct NsSmallArgs {
  uint16_t* xb[2];        // ping-pong bf16 iterates (unit 0), rows 128 x ldx
  int64_t x_stride;       // elements per unit
  int32_t ldx;            // padded columns (multiple of 128)
  int32_t n_iter;
  int32_t n_stages;
  int32_t stage_begin[4];
  float sa[4], sb[4], sc[4];
  int32_t final_mode;     // FINAL_STEP or FINAL_NSOUT
  const float* inv_nu;    // per unit: first-iteration scale (k_norm_finish)
  const int32_t* flag;    // per unit: nonzero norm
  // Split units (k_ns_small with groups > 1): each unit's column blocks are
  // shared by `groups` workgroups that sum their partial Grams through
  // memory once per iteration.
  int32_t groups;
  int32_t cnt_stride;     // words between the units' counters
  float* part;            // per unit: 2 x groups partial Grams of 128 x 128
  uint32_t* cnt;          // per unit: partial Grams published (cleared per call)
  uint32_t* err;          // the call's stop flag
  uint64_t timeout_ticks; // bound of one wait for the other workgroups
};

constexpr int kSmall = 128;  // padded rows (= Gram size) of the small path
constexpr int kSplitMax = 8;         // workgroups per split unit, at most
constexpr int kSplitWgMax = 256;     // workgroups of one split launch, at most

// Element (row, k) of a bf16 operand with 128-element rows in LDS: 16 chunks
// of 8 per row, the chunk index XOR-ed with a permutation of the row's low
// four bits.  16-byte reads of 16 consecutive rows at one k, and transposing
// reads of 4 consecutive rows (from a multiple of 4) x 16 columns, each touch
// distinct banks.
__device__ __forceinline__ int sb_at(int row, int k) {
  const int f = ((row & 7) << 1) | ((row >> 3) & 1);
  return row * kSmall + ((((k >> 3) ^ f) << 3) | (k & 7));
}

// MFMA fragment of rows r0 .. r0 + 31 of a row-major operand (K along the
// row): lane (x, half) gets k = 16kk + 8half .. +7 of row r0 + x.
__device__ __forceinline__ u32x4 sb_rows(const uint16_t* L, int r0, int kk, int lane) {
  const int r = r0 + (lane & 31);
  return *reinterpret_cast<const u32x4*>(L + sb_at(r, 16 * kk + 8 * (lane >> 5)));
}

// MFMA fragment of columns c0 .. c0 + 31 of a row-major operand whose K runs
// down the rows: lane (x, half) gets rows 16kk + 8half .. +7 of column
// c0 + x, by two transposing reads (ds_read_b64_tr_b16).  In each group of
// 16 lanes, lane 4r + q points at 4 elements of row k0 + r, columns
// 4q .. 4q + 3 of the group's 16, and lane i receives column i of the four
// rows.
__device__ __forceinline__ u32x4 sb_cols(const uint16_t* L, int c0, int kk, int lane) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const int g = lane >> 4, gi = lane & 15;
  const int k = 16 * kk + 8 * (g >> 1) + (gi >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (gi & 3);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(lds_vptr)(L + sb_at(k, col)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(lds_vptr)(L + sb_at(k + 4, col)));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// Accumulator-layout block (lane (x, half) holds row r0 + x, columns
// c0 + 8q + 4half + e for value 4q + e) into LDS as bf16, row-major.
__device__ __forceinline__ void sb_put(uint16_t* L, const float (&v)[16], int r0, int c0, int lane) {
  const int row = r0 + (lane & 31), half = lane >> 5;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint2 pk;
    pk.x = (uint32_t)to_bf16_bits(v[4 * q]) | ((uint32_t)to_bf16_bits(v[4 * q + 1]) << 16);
    pk.y = (uint32_t)to_bf16_bits(v[4 * q + 2]) | ((uint32_t)to_bf16_bits(v[4 * q + 3]) << 16);
    *reinterpret_cast<uint2*>(L + sb_at(row, c0 + 8 * q + 4 * half)) = pk;
  }
}

// Multi-block units (more than 128 columns), one workgroup per unit or, for
// a few long units, several (see below).  Per
// iteration the bf16 iterate streams through LDS in 128-column blocks X_j
// (row-major, the next block's loads in flight while one is used), and for
// each block
//   X'_j = B'*X_j                  (B' = a*I + b*A + c*A^2, its rows in
//                                   registers; X_j read K-major with the
//                                   transposing read)
//   A'  += X'_j X'_j^T             (the next iteration's Gram)
// so X makes one round trip through memory per iteration and the Gram,
// polynomial and apply of the notes' section 2 quintic step need no passes of
// their own.  Each wave owns a 64 x 64 quadrant of every 128 x 128 product.
// The iterate is the folded look-ahead on entry (k_momentum wrote bf16 N,
// padding zeroed; k_norm_finish left the first iteration's scale s = 1/nu,
// or 1 for a unit it rescaled): the first Gram is scaled by s^2 and the first
// X' by s.  Roundings as on the tiled bf16 path (bf16 operands, fp32
// accumulation, the iterate held in bf16) except that b*A takes A's fp32
// accumulator.
//
// A few long units (fewer than the CUs can keep busy) are split: workgroup
// g of a unit's `groups` takes column blocks [g nb / groups, (g + 1) nb /
// groups), and the Gram of the whole iterate is the sum of the groups'
// partial Grams.  Each workgroup publishes its partial (fp32, in its waves'
// accumulator layout) and a count, waits until every group of the unit has
// counted (bounded by a wall-clock limit, after which it reports through
// `err` and stops), and sums the partials in group order, so every
// workgroup of the unit holds the same A.  Partials alternate between two
// buffers: a group writes phase k + 1's partial only after every group has
// counted phase k, which each does after reading phase k - 1's.  The launch
// has at most as many workgroups as the CUs, one per CU, so all groups of a
// unit run at once.
__global__ __launch_bounds__(kThreads) void k_ns_small(NsSmallArgs p, ChunkArgs ca) {
  __shared__ __attribute__((aligned(16))) uint16_t LS[2][kSmall * kSmall];  // X_j, row-major
  __shared__ __attribute__((aligned(16))) uint16_t LR[kSmall * kSmall];     // A, B', then X'_j
  __shared__ int s_go;
  const int G = p.groups;
  const int u = blockIdx.x / G;
  const int g = blockIdx.x - u * G;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m = lane & 31, half = lane >> 5;
  const int nb = p.ldx / kSmall;
  const int j0 = g * nb / G, j1 = (g + 1) * nb / G;  // this workgroup's column blocks

  const SegView sg = find_seg(ca, u);
  float* const wout = sg.w + (int64_t)(u - sg.first) * ca.unit_elems;
  if (!p.flag[u]) {
    // Zero unit: O' = 0, so the weight only decays / the output is zero.
    const int64_t e0 = ca.unit_elems * g / G, e1 = ca.unit_elems * (g + 1) / G;
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kThreads)
      wout[e] = (p.final_mode == FINAL_STEP) ? wout[e] * ca.decay : 0.0f;
    return;
  }
  const float s0 = p.inv_nu[u];

  // Block j of an iterate into registers: 128 rows x 16 chunks of 8, chunk
  // t + 256 i of the block for thread t (16 threads per 256-byte row).
  u32x4 pf[8];
  auto fetch = [&](const uint16_t* X, int j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + kThreads * i, row = c >> 4, ch = c & 15;
      pf[i] = *reinterpret_cast<const u32x4*>(X + (int64_t)row * p.ldx + j * kSmall + ch * 8);
    }
  };
  auto stage = [&](uint16_t* L) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + kThreads * i, row = c >> 4, ch = c & 15;
      *reinterpret_cast<u32x4*>(L + sb_at(row, ch * 8)) = pf[i];
    }
  };
  auto zero = [](f32x16 (&a)[2][2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) a[i][j][r] = 0.0f;
  };
  // acc += rows of L (this wave's 64-row half) x rows of L (its 64-column half)
  auto gram = [&](const uint16_t* L, f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < kSmall / 16; ++kk) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = sb_rows(L, wm * 64 + i * 32, kk, lane);
        bf[i] = sb_rows(L, wn * 64 + i * 32, kk, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mfma_one<__bf16>(af[i], bf[j], acc[i][j]);
    }
  };

  f32x16 accA[2][2], accC[2][2];
  // Split units: publish this group's partial Gram of phase `ph` (accA),
  // wait for the unit's other groups, and replace accA by the sum of all
  // partials.  False when the wait gave up (the launch stops).
  uint32_t* const cnt = p.cnt ? p.cnt + (int64_t)u * p.cnt_stride : nullptr;
  auto reduce = [&](int ph) -> bool {
    float* const base = p.part + ((int64_t)u * 2 + (ph & 1)) * G * (kSmall * kSmall);
    float* const mine = base + (int64_t)g * (kSmall * kSmall);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[((w * 4 + i * 2 + jj) * 16 + r) * 64 + lane] = accA[i][jj][r];
    __syncthreads();  // every wave's stores are complete
    if (w == 0) {
      // The unit's other groups may run on other XCCs: write this L2 back
      // before the count.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      wait_vmcnt<0>();
      lane0_atomic_add_noret(cnt, 1u);
      const uint32_t need = (uint32_t)(G * (ph + 1));
      int go = 1;
      const uint64_t t0 = wall_clock64();
      for (;;) {
        const uint32_t c = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (c >= need) break;
        const uint32_t e = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (e != 0u || wall_clock64() - t0 > p.timeout_ticks) {
          __hip_atomic_store(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          go = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (go) {
        // drop this CU's L1 and this L2's copies of other XCCs' lines (one
        // acquire for every wave of the workgroup)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        wait_vmcnt<0>();
      }
      s_go = go;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_go) == 0) return false;
    // Sum the partials element-wise in group order into LDS (the two X
    // slots, free between passes: 64 KB), each thread 16 float4 positions
    // with every group's load in flight at once, then read this wave's
    // quadrant back.
    float4* const S = reinterpret_cast<float4*>(&LS[0][0]);
    const float4* const P = reinterpret_cast<const float4*>(base);
    constexpr int kQ = kSmall * kSmall / 4;  // float4 per partial
#pragma unroll 2
    for (int k = 0; k < kQ / kThreads; ++k) {
      const int idx = threadIdx.x + kThreads * k;
      float4 v[kSplitMax];
#pragma unroll
      for (int q = 0; q < kSplitMax; ++q) v[q] = P[(int64_t)(q < G ? q : 0) * kQ + idx];
      float4 t = v[0];
#pragma unroll
      for (int q = 1; q < kSplitMax; ++q)
        if (q < G) {
          t.x += v[q].x;
          t.y += v[q].y;
          t.z += v[q].z;
          t.w += v[q].w;
        }
      S[idx] = t;
    }
    lds_barrier();
    const float* const Sf = reinterpret_cast<const float*>(S);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) accA[i][jj][r] = Sf[((w * 4 + i * 2 + jj) * 16 + r) * 64 + lane];
    return true;
  };

  const uint16_t* const X0 = p.xb[0] + (int64_t)u * p.x_stride;
  // Gram of the entry iterate, scaled by s^2.
  zero(accA);
  fetch(X0, j0);
  for (int j = j0; j < j1; ++j) {
    stage(LS[j & 1]);
    if (j + 1 < j1) fetch(X0, j + 1);
    lds_barrier();  // block j staged; every wave is done with block j - 1
    gram(LS[j & 1], accA);
  }
  if (G > 1 && !reduce(0)) return;
  {
    const float s2 = s0 * s0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) accA[i][jj][r] *= s2;
  }

  const float lrs = sg.lr_scale;
  for (int it = 0; it < p.n_iter; ++it) {
    float ca_ = p.sa[0], cb = p.sb[0], cc = p.sc[0];
#pragma unroll
    for (int st = 1; st < 4; ++st)
      if (st < p.n_stages && it >= p.stage_begin[st]) {
        ca_ = p.sa[st];
        cb = p.sb[st];
        cc = p.sc[st];
      }
    const bool last = it == p.n_iter - 1;
    const float xs = it == 0 ? s0 : 1.0f;  // scale of this iteration's X'
    const uint16_t* const X = p.xb[it & 1] + (int64_t)u * p.x_stride;
    uint16_t* const Xn = p.xb[(it & 1) ^ 1] + (int64_t)u * p.x_stride;

    // B' = b*A + c*A*A (A symmetric), via LR; then this wave's rows of B'
    // into registers (the apply's first operand for every block).
    float av[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) av[i][jj][r] = accA[i][jj][r];
    // Every wave is done with LR and the last block, and the previous
    // iteration's stores of X (the barrier's fence drains them) are visible
    // to the whole workgroup before it reads X.
    __syncthreads();
    fetch(X, j0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) sb_put(LR, av[i][jj], wm * 64 + i * 32, wn * 64 + jj * 32, lane);
    lds_barrier();
    zero(accC);
    gram(LR, accC);
    // B' = a*I + b*A + c*A*A: the apply's a*X term rides on the diagonal.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          av[i][jj][r] = cb * av[i][jj][r] + cc * accC[i][jj][r];
          if (wm == wn && i == jj && m == 8 * (r >> 2) + 4 * half + (r & 3)) av[i][jj][r] += ca_;
        }
    lds_barrier();  // every wave has read A
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) sb_put(LR, av[i][jj], wm * 64 + i * 32, wn * 64 + jj * 32, lane);
    lds_barrier();
    u32x4 bfr[2][kSmall / 16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < kSmall / 16; ++kk) bfr[i][kk] = sb_rows(LR, wm * 64 + i * 32, kk, lane);

    zero(accA);
    for (int j = j0; j < j1; ++j) {
      stage(LS[j & 1]);
      if (j + 1 < j1) fetch(X, j + 1);
      lds_barrier();  // block j staged; every wave is done with LR and block j - 1
      // X'_j = a*X_j + B'*X_j over this wave's quadrant.
      zero(accC);
#pragma unroll
      for (int kk = 0; kk < kSmall / 16; ++kk) {
        u32x4 xf[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) xf[jj] = sb_cols(LS[j & 1], wn * 64 + jj * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) mfma_one<__bf16>(bfr[i][kk], xf[jj], accC[i][jj]);
      }
      float xv[2][2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) xv[i][jj][r] = xs * accC[i][jj][r];
      if (last) {
        // O' block: the decoupled update (or the NS output), masked.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = wm * 64 + i * 32 + m;
              const int c0 = j * kSmall + wn * 64 + jj * 32 + 8 * q + 4 * half;
              if (row >= ca.rows || c0 >= ca.cols) continue;
              float* const wp = wout + (int64_t)row * ca.cols + c0;
              const float o[4] = {xv[i][jj][4 * q], xv[i][jj][4 * q + 1], xv[i][jj][4 * q + 2],
                                  xv[i][jj][4 * q + 3]};
              if ((ca.cols & 3) == 0) {
                float4 wv = make_float4(o[0], o[1], o[2], o[3]);
                if (p.final_mode == FINAL_STEP) {
                  const float4 w0 = *reinterpret_cast<const float4*>(wp);
                  wv.x = __builtin_fmaf(-lrs, o[0], w0.x * ca.decay);
                  wv.y = __builtin_fmaf(-lrs, o[1], w0.y * ca.decay);
                  wv.z = __builtin_fmaf(-lrs, o[2], w0.z * ca.decay);
                  wv.w = __builtin_fmaf(-lrs, o[3], w0.w * ca.decay);
                }
                *reinterpret_cast<float4*>(wp) = wv;
              } else {
                const int ne = min(4, ca.cols - c0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (e < ne)
                    wp[e] = (p.final_mode == FINAL_STEP) ? __builtin_fmaf(-lrs, o[e], wp[e] * ca.decay) : o[e];
              }
            }
        continue;
      }
      // X'_j in bf16 into LR, for the next Gram and, in whole rows, for
      // memory (the next iteration's X).
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) sb_put(LR, xv[i][jj], wm * 64 + i * 32, wn * 64 + jj * 32, lane);
      lds_barrier();  // X'_j complete in LR
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + kThreads * i, row = c >> 4, ch = c & 15;
        *reinterpret_cast<u32x4*>(Xn + (int64_t)row * p.ldx + j * kSmall + ch * 8) =
            *reinterpret_cast<const u32x4*>(LR + sb_at(row, ch * 8));
      }
      gram(LR, accA);
    }
    if (!last && G > 1 && !reduce(it + 1)) return;
  }
}

// ------------------------------------------------ one-launch small step ----
// The whole step of units whose wide form fits one 128 x 128 block (at most
// 128 rows and 128 columns, rows <= columns; fp32 products: at most 64
// rows), one workgroup per unit and one launch per chunk: momentum and the
// look-ahead go straight into registers, the Frobenius norm is a block
// reduction, and every product of every iteration runs on chip over the
// unit's own extent rounded up to 32 (BS row blocks, BL column blocks of 32)
// rather than over 128 x 128.  Products are split into 32 x 32 output
// blocks, block b of a product going to wave b % 4; a wave keeps the
// iterate's blocks it updates, and the Gram blocks it later combines with
// A*A, in registers.  LDS holds the operands in the products' type T: X (two
// buffers: one read by this iteration's products, the other receiving X'),
// A and B, so an iteration needs three barriers.  The roundings are those of
// the other paths of the same type: operands in T, fp32 accumulation, and
// on the bf16 path the iterate rounded to bf16 between iterations.  gk: 0
// bf16 gradient, 1 fp32 gradient, 2 NS only.  err: the call's status words
// when this is its first launch, else null.

// Operand access of the one-launch kernel per product type.  bf16: rows of
// 128 elements swizzled by sb_at, K-major fragments by the transposing read,
// 16 K per fragment.  fp32: rows of 132 floats (the padding spreads 16
// consecutive rows over the banks), K-major fragments as four column reads,
// 8 K per fragment (lane half h holds k = 8kk + 4h .. +3, the order in which
// mfma_one<float> feeds its four K = 2 steps).
template <typename T>
struct SmallOps;

template <>
struct SmallOps<__bf16> {
  typedef uint16_t E;
  static constexpr int kPitch = kSmall;
  static constexpr int kK = 16;
  static __device__ __forceinline__ u32x4 rows(const E* L, int r0, int kk, int lane) {
    return sb_rows(L, r0, kk, lane);
  }
  static __device__ __forceinline__ u32x4 cols(const E* L, int c0, int kk, int lane) {
    return sb_cols(L, c0, kk, lane);
  }
  static __device__ __forceinline__ void put(E* L, const float (&v)[16], int r0, int c0, int lane) {
    sb_put(L, v, r0, c0, lane);
  }
  static __device__ __forceinline__ float iterate(float x) { return bf16_round(x); }
};

template <>
struct SmallOps<float> {
  typedef float E;
  static constexpr int kPitch = kSmall + 4;
  static constexpr int kK = 8;
  static __device__ __forceinline__ u32x4 rows(const E* L, int r0, int kk, int lane) {
    const int r = r0 + (lane & 31);
    return *reinterpret_cast<const u32x4*>(L + r * kPitch + 8 * kk + 4 * (lane >> 5));
  }
  static __device__ __forceinline__ u32x4 cols(const E* L, int c0, int kk, int lane) {
    const E* q = L + (8 * kk + 4 * (lane >> 5)) * kPitch + c0 + (lane & 31);
    return u32x4{__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[kPitch]),
                 __builtin_bit_cast(uint32_t, q[2 * kPitch]), __builtin_bit_cast(uint32_t, q[3 * kPitch])};
  }
  static __device__ __forceinline__ void put(E* L, const float (&v)[16], int r0, int c0, int lane) {
    const int row = r0 + (lane & 31), half = lane >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(L + row * kPitch + c0 + 8 * q + 4 * half) =
          make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  static __device__ __forceinline__ float iterate(float x) { return x; }
};

// acc[t] += the product of fragments fa(t, kk) and fb(t, kk) over kk < KS,
// t < NT: the fragments of the next D steps are read while a step's MFMAs
// run (a ring of registers, every index known at compile time), so LDS
// latency stays off the chain of dependent MFMAs.  D shrinks as a wave's
// blocks grow, to bound the registers the ring takes.
template <typename T, int NT, int KS, typename FA, typename FB>
__device__ __forceinline__ void small_product(f32x16* acc, const FA& fa, const FB& fb) {
  constexpr int D0 = NT >= 4 ? 1 : (NT >= 2 ? 2 : 4);
  constexpr int D = D0 < KS ? D0 : KS;
  u32x4 ra[D][NT], rb[D][NT];
#pragma unroll
  for (int k = 0; k < D; ++k)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ra[k][t] = fa(t, k);
      rb[k][t] = fb(t, k);
    }
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
    for (int t = 0; t < NT; ++t) mfma_one<T>(ra[kk % D][t], rb[kk % D][t], acc[t]);
    if (kk + D < KS) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        ra[kk % D][t] = fa(t, kk + D);
        rb[kk % D][t] = fb(t, kk + D);
      }
    }
  }
}

template <typename T, int BS, int BL>
__global__ __launch_bounds__(kThreads) void k_ns_small_step(NsSmallArgs p, ChunkArgs ca, int gk,
                                                             uint32_t* __restrict__ err) {
  typedef SmallOps<T> Op;
  typedef typename Op::E E;
  constexpr int R = 32 * BS;                // rows of every LDS operand
  constexpr int NA = BS * BS, NX = BS * BL;  // 32 x 32 blocks of A (and B), of X
  constexpr int TA = (NA + 3) / 4, TX = (NX + 3) / 4;  // blocks per wave, at most
  __shared__ __attribute__((aligned(16))) E LX[2][R * Op::kPitch];
  __shared__ __attribute__((aligned(16))) E LA[R * Op::kPitch];
  __shared__ __attribute__((aligned(16))) E LB[R * Op::kPitch];
  __shared__ double wsum[kThreads / 64];
  const int u = blockIdx.x;
  const int lane = threadIdx.x & 63;
  // wave-uniform, so that the per-block conditions below are scalar
  // branches and the products run as straight-line code
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 31, half = lane >> 5;
  if (err && u == 0 && threadIdx.x == 0) status_fold(err);

  const SegView sg = find_seg(ca, u);
  const int64_t uoff = (int64_t)(u - sg.first) * ca.unit_elems;
  float* const wout = sg.w + uoff;
  const int rows = ca.rows, cols = ca.cols;
  const bool vec = (cols & 3) == 0;

  // The old weights of this wave's blocks (step only), for the update at
  // the end: loaded with G and M when a wave holds at most two blocks (the
  // registers stay free enough), else at the end.
  const float lrs = sg.lr_scale;
  const bool step = p.final_mode == FINAL_STEP;
  constexpr bool kEarlyW = TX <= 2;
  float wo[TX][4][4];
  auto load_w = [&]() {
#pragma unroll
    for (int t = 0; t < TX; ++t) {
      const int b = w + 4 * t;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wo[t][q][e] = 0.0f;
        const int row = 32 * (b / BL) + m;
        const int c0 = 32 * (b % BL) + 8 * q + 4 * half;
        if (!step || b >= NX || row >= rows || c0 >= cols) continue;
        const float* const wp = wout + (int64_t)row * cols + c0;
        if (vec) {
          const float4 w0 = *reinterpret_cast<const float4*>(wp);
          wo[t][q][0] = w0.x; wo[t][q][1] = w0.y; wo[t][q][2] = w0.z; wo[t][q][3] = w0.w;
        } else {
          const int ne = min(4, cols - c0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < ne) wo[t][q][e] = wp[e];
        }
      }
    }
  };
  if constexpr (kEarlyW) load_w();

  // 1. M = ma*M + mb*G and N = la*M + lb*G for this wave's blocks of X
  // (block b: rows 32(b / BL) .., columns 32(b % BL) ..), zero outside the
  // matrix; gk == 2 takes the input itself as N.  Every group's G and M
  // are loaded before any is updated, so the loads are in flight together
  // (a store to M between them would hold each next load back).
  float xv[TX][16];
  float gv[TX][4][4], mv[TX][4][4];
  double ss = 0.0;
#pragma unroll
  for (int t = 0; t < TX; ++t) {
    const int b = w + 4 * t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) gv[t][q][e] = mv[t][q][e] = 0.0f;
      const int row = 32 * (b / BL) + m;
      const int c0 = 32 * (b % BL) + 8 * q + 4 * half;
      if (b < NX && row < rows && c0 < cols) {
        const int64_t base = uoff + (int64_t)row * cols + c0;
        if (vec) {
          if (gk == 0) {
            const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(sg.g) + base);
            gv[t][q][0] = bf16_bits_to_f32(raw.x & 0xffffu);
            gv[t][q][1] = bf16_bits_to_f32(raw.x >> 16);
            gv[t][q][2] = bf16_bits_to_f32(raw.y & 0xffffu);
            gv[t][q][3] = bf16_bits_to_f32(raw.y >> 16);
          } else {
            const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(sg.g) + base);
            gv[t][q][0] = v.x; gv[t][q][1] = v.y; gv[t][q][2] = v.z; gv[t][q][3] = v.w;
          }
          if (gk != 2) {
            const float4 v = *reinterpret_cast<const float4*>(sg.m + base);
            mv[t][q][0] = v.x; mv[t][q][1] = v.y; mv[t][q][2] = v.z; mv[t][q][3] = v.w;
          }
        } else {
          const int ne = min(4, cols - c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (e >= ne) continue;
            gv[t][q][e] = gk == 0 ? bf16_bits_to_f32(static_cast<const uint16_t*>(sg.g)[base + e])
                                  : static_cast<const float*>(sg.g)[base + e];
            if (gk != 2) mv[t][q][e] = sg.m[base + e];
          }
        }
        // lanes past the last column read nothing: g = 0, M = 0, N = 0
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TX; ++t) {
    const int b = w + 4 * t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float n[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      const int row = 32 * (b / BL) + m;
      const int c0 = 32 * (b % BL) + 8 * q + 4 * half;
      if (b < NX && row < rows && c0 < cols) {
        const int64_t base = uoff + (int64_t)row * cols + c0;
        const int ne = vec ? 4 : min(4, cols - c0);
        float* const mo = mv[t][q];
        const float* const g = gv[t][q];
        if (gk == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) n[e] = g[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mo[e] = __builtin_fmaf(ca.ma, mo[e], ca.mb * g[e]);
            n[e] = __builtin_fmaf(ca.la, mo[e], ca.lb * g[e]);
          }
          if (vec) {
            *reinterpret_cast<float4*>(sg.m + base) = make_float4(mo[0], mo[1], mo[2], mo[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (e < ne) sg.m[base + e] = mo[e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[t][4 * q + e] = n[e];
        ss = __builtin_fma((double)n[e], (double)n[e], ss);
      }
    }
  }

  // 2. ||N||_F^2: fixed shuffle tree per wave, then the waves in order (the
  // same value in every thread).
  ss = wave_sum(ss);
  if (lane == 0) wsum[w] = ss;
  __syncthreads();
  double s2 = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) s2 += wsum[i];

  if (s2 == 0.0) {
    // Zero look-ahead: O' = 0, so the weight only decays / the output is zero.
    for (int64_t e = threadIdx.x; e < ca.unit_elems; e += kThreads)
      wout[e] = (p.final_mode == FINAL_STEP) ? wout[e] * ca.decay : 0.0f;
    return;
  }
  // A NaN/Inf sum keeps the unit active so that it propagates.
  const float inv = (float)(1.0 / sqrt(s2));
#pragma unroll
  for (int t = 0; t < TX; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) xv[t][r] = Op::iterate(xv[t][r] * inv);
    const int b = w + 4 * t;
    if (b < NX) Op::put(LX[0], xv[t], 32 * (b / BL), 32 * (b % BL), lane);
  }
  __syncthreads();

  // 3. The iterations.
  float av[TA][16];
  f32x16 acc[TA > TX ? TA : TX];
  for (int it = 0; it < p.n_iter; ++it) {
    float ca_ = p.sa[0], cb = p.sb[0], cc = p.sc[0];
#pragma unroll
    for (int st = 1; st < 4; ++st)
      if (st < p.n_stages && it >= p.stage_begin[st]) {
        ca_ = p.sa[st];
        cb = p.sb[st];
        cc = p.sc[st];
      }
    const E* const X = LX[it & 1];
    // A = X X^T over K = 32 BL; block b: rows 32(b / BS), columns 32(b % BS).
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    // (A wave past the last block repeats the last one, in bounds, and
    // never stores it: no branch around the products, whose operand reads
    // then go ahead of the MFMAs.)
    small_product<T, TA, 32 * BL / Op::kK>(
        acc, [&](int t, int kk) { return Op::rows(X, 32 * (min(w + 4 * t, NA - 1) / BS), kk, lane); },
        [&](int t, int kk) { return Op::rows(X, 32 * (min(w + 4 * t, NA - 1) % BS), kk, lane); });
#pragma unroll
    for (int t = 0; t < TA; ++t) {
      const int b = w + 4 * t;
#pragma unroll
      for (int r = 0; r < 16; ++r) av[t][r] = acc[t][r];
      if (b < NA) Op::put(LA, av[t], 32 * (b / BS), 32 * (b % BS), lane);
    }
    __syncthreads();
    // B = b*A + c*A*A (A symmetric: both operands read rows of A).
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    small_product<T, TA, 32 * BS / Op::kK>(
        acc, [&](int t, int kk) { return Op::rows(LA, 32 * (min(w + 4 * t, NA - 1) / BS), kk, lane); },
        [&](int t, int kk) { return Op::rows(LA, 32 * (min(w + 4 * t, NA - 1) % BS), kk, lane); });
#pragma unroll
    for (int t = 0; t < TA; ++t) {
      const int b = w + 4 * t;
#pragma unroll
      for (int r = 0; r < 16; ++r) av[t][r] = cb * av[t][r] + cc * acc[t][r];
      if (b < NA) Op::put(LB, av[t], 32 * (b / BS), 32 * (b % BS), lane);
    }
    __syncthreads();
    // X' = a*X + B*X over K = 32 BS.
#pragma unroll
    for (int t = 0; t < TX; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    small_product<T, TX, 32 * BS / Op::kK>(
        acc, [&](int t, int kk) { return Op::rows(LB, 32 * (min(w + 4 * t, NX - 1) / BL), kk, lane); },
        [&](int t, int kk) { return Op::cols(X, 32 * (min(w + 4 * t, NX - 1) % BL), kk, lane); });
#pragma unroll
    for (int t = 0; t < TX; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xv[t][r] = __builtin_fmaf(ca_, xv[t][r], acc[t][r]);
    if (it == p.n_iter - 1) break;
#pragma unroll
    for (int t = 0; t < TX; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xv[t][r] = Op::iterate(xv[t][r]);
      const int b = w + 4 * t;
      if (b < NX) Op::put(LX[(it & 1) ^ 1], xv[t], 32 * (b / BL), 32 * (b % BL), lane);
    }
    __syncthreads();
  }

  // 4. The decoupled update (or the NS output) of this wave's blocks, from
  // the old weights loaded with G and M (or, for a wave of more blocks,
  // all loaded now, in flight together).
  if constexpr (!kEarlyW) load_w();
#pragma unroll
  for (int t = 0; t < TX; ++t) {
    const int b = w + 4 * t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 32 * (b / BL) + m;
      const int c0 = 32 * (b % BL) + 8 * q + 4 * half;
      if (b >= NX || row >= rows || c0 >= cols) continue;
      float* const wp = wout + (int64_t)row * cols + c0;
      float o[4] = {xv[t][4 * q], xv[t][4 * q + 1], xv[t][4 * q + 2], xv[t][4 * q + 3]};
      if (step) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(-lrs, o[e], wo[t][q][e] * ca.decay);
      }
      if (vec) {
        *reinterpret_cast<float4*>(wp) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        const int ne = min(4, cols - c0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < ne) wp[e] = o[e];
      }
    }
  }
}

// ------------------------------------------------------ persistent NS ------
// All Newton-Schulz iterations of a chunk in one launch.  Work items, in
// claim order: for each iteration, the Gram tiles of every unit, then the
// polynomial tiles, then the apply tiles (unit-major within a phase).  A
// workgroup claims the next item from an atomic counter, waits until the
// tile panels it reads are final (counts of finished tiles per panel, see
// below), runs the tile and adds one to the counts of its panels.  An
// item only waits for items that precede it in claim order, and those were
// claimed by running workgroups, so the schedule always makes progress; the
// wait is still bounded by a wall-clock limit, after which the launch stops
// and reports through `err`.
//
// A launch may carry a second pass (ns_persistent2): units of another
// shape with the same tile size and operand layout, with their own buffers
// and completion counts.  Its items follow the first pass's within each
// phase (Gram of the first pass, Gram of the second, polynomial of the
// first, ...), so every item still waits only for earlier ones; the second
// pass's tiles fill the CUs that the first pass leaves idle.
//
// Queues.  With one queue any workgroup may run any tile, so a tile's
// results are published at agent scope (the L2 written back before the
// count).  With one queue per XCC, unit u of a pass belongs to queue
// u % n_queues and only workgroups running on that XCC claim from it:
// every tile of a unit is then produced and consumed through the same L2,
// so publishing only needs the stores to have completed.  Before a tile's
// first load, wave 0 of the reading workgroup acquires at agent scope once
// for all its waves (in both cases).  The last workgroup to leave runs, on
// its own, any queue that no workgroup ever claimed from (an XCC that
// received none).

// One pass: the products of its units and where their tiles are counted.
struct NsPass {
  GemmArgs gram, poly, apply;     // cur-independent fields of each product
  const void* gram_op[2];         // Gram operand (both sides) for X in buffer cur
  const void* app_a[2];           // apply operands for X in buffer cur
  const void* app_b[2];
  float* app_out32[2];            // apply outputs (buffer cur ^ 1)
  void* app_out16[2];
  void* app_outt[2];
  uint32_t* done;                 // per unit: finished tiles per small-side
                                  // panel, for each of the three products
  int32_t n_units;
  int32_t tg;                     // tiles per unit of a symmetric product
  int32_t ta;                     // tiles per unit of the apply product
  int32_t apply_s_m;              // 1: an apply tile's small-side panel is its
                                  // row (wide units), 0: its column (tall)
};

struct NsSched {
  NsPass a;                       // the first pass (its units: the ChunkArgs)
  int32_t final_mode;             // of the last iteration's apply
  int32_t n_iter;
  int32_t n_stages;
  int32_t stage_begin[4];         // first iteration of each stage
  float sa[4], sb[4], sc[4];      // coefficients of each stage
  int32_t n_queues;               // 1, or one queue per XCC (see above)
  uint32_t* queue;                // per queue: next item to claim; then the
                                  // count of workgroups that have left
  uint32_t* err;                  // set when a wait timed out
  uint64_t timeout_ticks;         // wall-clock ticks
};

// The second pass of a two-pass launch, with what its final epilogue needs
// of its chunk (the first pass takes that from the kernel's ChunkArgs).
constexpr int kMaxSegB = 4;
struct NsPassB {
  NsPass b;
  int32_t rows, cols;             // unit shape
  int64_t unit_elems;
  float decay;
  int32_t n_seg;
  Seg seg[kMaxSegB];
};

// The pass an item belongs to, picked field by field as values: sel()
// takes both fields by value, so each pick selects between two loaded
// kernel-argument values.  (c ? x.f : y.f on two lvalues is itself an
// lvalue: the compiler selects the addresses and loads through them, and
// then keeps both kernel arguments in scratch memory and loads every field
// per lane.)
template <typename V>
__device__ __forceinline__ V sel(bool c, V x, V y) {
  return c ? x : y;
}

__device__ __forceinline__ GemmArgs pick(bool c, const GemmArgs& x, const GemmArgs& y) {
  static_assert(sizeof(GemmArgs) == 176, "every GemmArgs field is picked below");
  GemmArgs g;
  g.a = sel(c, x.a, y.a);
  g.b = sel(c, x.b, y.b);
  g.a_ustride = sel(c, x.a_ustride, y.a_ustride);
  g.b_ustride = sel(c, x.b_ustride, y.b_ustride);
  g.lda = sel(c, x.lda, y.lda);
  g.ldb = sel(c, x.ldb, y.ldb);
  g.M = sel(c, x.M, y.M);
  g.N = sel(c, x.N, y.N);
  g.K = sel(c, x.K, y.K);
  g.tiles_m = sel(c, x.tiles_m, y.tiles_m);
  g.tiles_n = sel(c, x.tiles_n, y.tiles_n);
  g.n_units = sel(c, x.n_units, y.n_units);
  g.out32 = sel(c, x.out32, y.out32);
  g.out16 = sel(c, x.out16, y.out16);
  g.out_ustride = sel(c, x.out_ustride, y.out_ustride);
  g.ldo = sel(c, x.ldo, y.ldo);
  g.outt = sel(c, x.outt, y.outt);
  g.ldt = sel(c, x.ldt, y.ldt);
  g.sym = sel(c, x.sym, y.sym);
  g.final_mode = sel(c, x.final_mode, y.final_mode);
  g.aux = sel(c, x.aux, y.aux);
  g.aux16 = sel(c, x.aux16, y.aux16);
  g.aux_ustride = sel(c, x.aux_ustride, y.aux_ustride);
  g.ldaux = sel(c, x.ldaux, y.ldaux);
  g.ca = sel(c, x.ca, y.ca);
  g.cb = sel(c, x.cb, y.cb);
  g.cc = sel(c, x.cc, y.cc);
  g.flag = sel(c, x.flag, y.flag);
  g.fold = sel(c, x.fold, y.fold);
  return g;
}

__device__ __forceinline__ UnitOut unit_out(const NsPassB& pb, int u) {
  const SegView sg = find_seg_in(pb.seg, pb.n_seg, u);
  return UnitOut{sg.w + (int64_t)(u - sg.first) * pb.unit_elems, sg.trans, sg.lr_scale,
                 pb.rows, pb.cols, pb.decay};
}

// KMODE: 0 = every operand row-major (fp32 path: X^T is kept); 1 = wide
// bf16 units, B'*X reads X K-major; 2 = tall bf16 units, X^T X reads X
// K-major on both sides.  TWO: the launch carries a second pass (`second`).
template <typename T, int TILE, int KMODE, bool TWO>
__device__ __forceinline__ void ns_persistent_run(const NsSched& p, const ChunkArgs& ca,
                                                  const NsPassB* second) {
  // Every branch below is uniform across the workgroup or across a wave:
  // the scheduling work (claim, completion count, dependency wait) is done
  // by all of wave 0, whose atomics lane 0 makes alone (lane0_atomic_add),
  // never under a per-lane condition.  A per-lane branch around it lets the
  // compiler thread the tail of one iteration into the head of the next for
  // that lane alone, and the other lanes would then reach the barriers on
  // stale state.
  // Broadcast words live in the tile ring (which fills the LDS).  They are
  // written only after the barrier that ends a tile, and the barrier that
  // follows their last read comes before the next tile's first copy.
  int& s_item = reinterpret_cast<int*>(lds_ring<TILE>)[0];
  int& s_go = reinterpret_cast<int*>(lds_ring<TILE>)[1];
  const int per_unit_a = 2 * p.a.tg + p.a.ta;
  const int per_unit_b = TWO ? 2 * second->b.tg + second->b.ta : 0;
  const int nq = p.n_queues;
  const bool local = nq > 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* const left = p.queue + nq;                    // workgroups that have left
  // units of a pass of n units in queue qq: qq, qq + nq, ...
  auto units_of = [&](int qq, int n) { return n > qq ? (n - qq + nq - 1) / nq : 0; };
  const int na = p.a.n_units;
  const int nb = TWO ? second->b.n_units : 0;
  int q = local ? xcc_id() % nq : 0;
  int uqa = units_of(q, na);
  int uqb = TWO ? units_of(q, nb) : 0;
  // Completion counts, per unit three arrays of ts words (Gram, polynomial,
  // apply), indexed by tile panel on the small side: a Gram or polynomial
  // tile (r, c) counts in panels r and c (once when r == c), an apply tile
  // in its small-side panel.  Each iteration adds ts to every Gram and
  // polynomial panel and tl to every apply panel.  A tile waits only for
  // the panels it reads:
  //   Gram (r, c) of iteration it > 0: apply panels r and c at it * tl;
  //   polynomial (r, c): Gram panels r and c at (it + 1) * ts;
  //   apply with small-side panel i: polynomial panel i at (it + 1) * ts.
  // Each of these points to items earlier in claim order.  The buffers that
  // are rewritten every iteration (A, B', the two iterates) cannot be
  // overwritten while still read: every such write depends, through those
  // chains, on the whole earlier phase that reads them.
  // A finished tile is counted once every wave's stores of it are
  // complete.  With XCC-local queues the count is deferred into the next
  // tile's prologue, whose in-order copy wait covers the stores; it is
  // made at once (a flush) before any wait that could block, before an
  // item that runs no tile and on every exit, so no workgroup ever blocks
  // while holding an uncounted tile.  With one queue the release also
  // writes the L2 back, and tiles are flushed as they end.
  uint32_t* pend_a = nullptr;  // counts of the finished tile not yet made
  uint32_t* pend_b = nullptr;
  bool alone = false;  // running unclaimed queues after every other workgroup left
  auto count_pending = [&]() {  // wave 0; every wave's stores of the tile are complete
    if (wave == 0 && pend_a) {
      if (!local) {
        // Other XCCs read the tile from memory: write this L2 back and wait
        // for the write-back before the count can be seen.  The compiler
        // drops its own wait after the write-back when the tile's stores
        // are already complete, as they are here.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        wait_vmcnt<0>();
      }
      lane0_atomic_add_noret(pend_a, 1u);
      if (pend_b) lane0_atomic_add_noret(pend_b, 1u);
    }
    pend_a = pend_b = nullptr;
  };
  auto flush = [&]() {  // every wave
    if (pend_a) {
      wait_vmcnt<0>();
      __syncthreads();
      count_pending();
    }
  };
  // Wave 0 claims the next item (and reads the error word) right after the
  // current tile's first copies are issued.  The claim's result is read at
  // once, and as the vector-memory counter completes in order that read
  // also waits for those copies, which the prologue waits for in any case
  // (claiming after the tile's last copies had landed measured no faster).
  // Holding one claimed item ahead cannot stall the schedule: the earliest
  // unfinished item in claim order is always some workgroup's current one
  // (a held item comes after its holder's current, unfinished item).
  // The claimed item is kept as a scalar (-1 after an error), so that the
  // next head reads it without waiting on memory accesses issued since.
  bool have_next = false;
  int next_item = 0;
  auto claim = [&]() {  // wave 0
    const uint32_t raw = lane0_atomic_add(p.queue + q, 1u);
    const uint32_t err = __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    next_item = __builtin_amdgcn_readfirstlane(err) != 0u ? -1 : (int)raw;
  };
  for (;;) {
    if (wave == 0) {
      if (!have_next) claim();
      s_item = next_item;  // every lane writes the same value
    }
    have_next = false;
    lds_barrier();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    const int per_iter = uqa * per_unit_a + uqb * per_unit_b;
    if (item < 0 || item >= p.n_iter * per_iter) flush();
    if (item < 0) break;  // stopped
    if (item >= p.n_iter * per_iter) {
      // This queue is drained.
      if (!local) break;
      if (!alone) {
        // Count this workgroup out; the last one continues alone.
        __syncthreads();
        if (wave == 0)
          s_go = (int)lane0_atomic_add(left, 1u) == (int)gridDim.x - 1;
        __syncthreads();
        if (!__builtin_amdgcn_readfirstlane(s_go)) break;
        alone = true;
      }
      // Every other workgroup has left, so a queue that nobody claimed from
      // has no workgroup on its XCC: run it here, one tile after another.
      int next = -1;
      for (int qq = 0; qq < nq; ++qq) {
        const uint32_t head = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p.queue + qq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (next < 0 && head == 0u && units_of(qq, na) + (TWO ? units_of(qq, nb) : 0) > 0)
          next = qq;
      }
      if (next < 0) break;
      q = next;
      uqa = units_of(q, na);
      uqb = TWO ? units_of(q, nb) : 0;
      continue;
    }
    // Within an iteration: Gram of pass a, Gram of pass b, polynomial of
    // a, of b, apply of a, of b.
    const int ga = uqa * p.a.tg;
    const int gb = TWO ? uqb * second->b.tg : 0;
    const int it = item / per_iter;
    int r = item - it * per_iter;
    int phase;
    bool in_b = false;
    if (r < ga) {
      phase = GRAM;
    } else if (TWO && r < ga + gb) {
      phase = GRAM;
      in_b = true;
      r -= ga;
    } else if (r < 2 * ga + gb) {
      phase = POLY;
      r -= ga + gb;
    } else if (TWO && r < 2 * ga + 2 * gb) {
      phase = POLY;
      in_b = true;
      r -= 2 * ga + gb;
    } else {
      phase = APPLY;
      r -= 2 * ga + 2 * gb;
      if (TWO && r >= uqa * p.a.ta) {
        in_b = true;
        r -= uqa * p.a.ta;
      }
    }
    // the item's pass (b: the second one; always the first without TWO)
    const NsPass& PB = TWO ? second->b : p.a;
    const bool b = TWO && in_b;
    const int tg = sel(b, PB.tg, p.a.tg);
    const int ta = sel(b, PB.ta, p.a.ta);
    const int tpu = phase == APPLY ? ta : tg;
    int u = r / tpu;
    const int t = r - u * tpu;
    u = q + nq * u;
    const int32_t* const flag = sel(b, PB.gram.flag, p.a.gram.flag);
    const bool live = __builtin_amdgcn_readfirstlane(flag[u]) != 0;
    const int ts = sel(b, PB.gram.tiles_m, p.a.gram.tiles_m);
    const int tl = ta / ts;
    int tm, tn;
    if (phase == APPLY)
      grid_tile_grouped(t, sel(b, PB.apply.tiles_m, p.a.apply.tiles_m),
                        sel(b, PB.apply.tiles_n, p.a.apply.tiles_n), tm, tn);
    else
      sym_tile_grouped(t, ts, tm, tn);
    // Small-side panels the tile reads and completes, and the counts it
    // waits for (a zero unit computes nothing, so its items wait for
    // nothing).
    const int apply_s_m = sel(b, PB.apply_s_m, p.a.apply_s_m);
    const int pa = phase == APPLY ? (apply_s_m ? tm : tn) : tm;
    const int pb = phase == APPLY ? pa : tn;
    uint32_t* const cnt = sel(b, PB.done, p.a.done) + (int64_t)u * 3 * ts;  // Gram | polynomial | apply
    uint32_t* dep = nullptr;  // the counts waited for: dep[pa] and dep[pb]
    uint32_t need = 0;
    if (phase == GRAM) {
      if (it > 0) {
        dep = cnt + 2 * ts;
        need = (uint32_t)(it * tl);
      }
    } else if (phase == POLY) {
      dep = cnt;
      need = (uint32_t)((it + 1) * ts);
    } else {
      dep = cnt + ts;
      need = (uint32_t)((it + 1) * ts);
    }
    auto deps_met = [&]() -> bool {  // wave 0
      if (!dep) return true;
      // both loads in flight at once (the same word twice when pb == pa)
      const uint32_t da = __hip_atomic_load(dep + pa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t db = __hip_atomic_load(dep + pb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t d = __builtin_amdgcn_readfirstlane(da < db ? da : db);
      return d >= need;
    };
    // One look at the completion counts; if the item must wait, the pending
    // tile is counted first (it may be what the wait is for).  Wave 0 makes
    // the producers' results visible to the whole workgroup before the
    // barrier that releases the other waves to load them: an acquire at
    // agent scope (it drops the CU's L1, which every wave shares, and this
    // L2's copies of lines other XCCs wrote), waited for in full.  One
    // invalidate per tile rather than one per wave.
    auto acquire = [&]() {  // wave 0
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      wait_vmcnt<0>();
    };
    if (wave == 0) {
      int ready = 1;
      if (live) ready = deps_met();
      if (ready && live) acquire();
      s_go = ready;
    }
    lds_barrier();
    const bool ready = __builtin_amdgcn_readfirstlane(s_go) != 0;
    lds_barrier();  // every wave has read s_go
    if (!ready || !live) flush();
    if (!ready) {
      if (wave == 0) {
        int go = 1;
        const uint64_t t0 = wall_clock64();
        while (!deps_met()) {
          const uint32_t e = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (e != 0u || wall_clock64() - t0 > p.timeout_ticks) {
            __hip_atomic_store(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            go = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (go) acquire();
        s_go = go;
      }
      lds_barrier();
      const int go = __builtin_amdgcn_readfirstlane(s_go);
      lds_barrier();  // every wave has read the broadcast words
      if (!go) {
        flush();
        break;
      }
    }
    // Wave 0 claims the next item once the tile's first copies are in
    // flight (a zero unit's item runs no tile; the next head claims).
    auto claim_next = [&]() {
      if (wave == 0) {
        claim();
        have_next = true;
      }
    };
    // the final epilogue's view of the unit, from its own pass's chunk
    auto out_of = [&]() {
      if constexpr (TWO) {
        if (in_b) return unit_out(*second, u);
      }
      return unit_out(ca, u);
    };
    const int cur = it & 1;
    if (phase == GRAM) {
      if (live) {
        GemmArgs g = pick(b, PB.gram, p.a.gram);
        g.a = g.b = sel(cur != 0, sel(b, PB.gram_op[1], p.a.gram_op[1]),
                        sel(b, PB.gram_op[0], p.a.gram_op[0]));
        if (it == 0 && g.fold)
          gemm_tile<GRAM, T, TILE, KMODE == 2 ? 3 : 0, true>(g, out_of, u, tm, tn, claim_next,
                                                            count_pending);
        else
          gemm_tile<GRAM, T, TILE, KMODE == 2 ? 3 : 0>(g, out_of, u, tm, tn, claim_next,
                                                       count_pending);
      }
    } else if (phase == POLY) {
      if (live) {
        GemmArgs g = pick(b, PB.poly, p.a.poly);
        float a = p.sa[0], cb = p.sb[0], cc = p.sc[0];
#pragma unroll
        for (int s = 1; s < 4; ++s)
          if (s < p.n_stages && it >= p.stage_begin[s]) {
            a = p.sa[s];
            cb = p.sb[s];
            cc = p.sc[s];
          }
        g.ca = a;
        g.cb = cb;
        g.cc = cc;
        gemm_tile<POLY, T, TILE, 0>(g, out_of, u, tm, tn, claim_next, count_pending);
      }
    } else {
      const int fm = it == p.n_iter - 1 ? p.final_mode : (int)FINAL_NONE;
      if (live) {
        GemmArgs g = pick(b, PB.apply, p.a.apply);
        g.final_mode = fm;
        const NsPass& PA = p.a;
        const bool c1 = cur != 0;
        g.a = sel(c1, sel(b, PB.app_a[1], PA.app_a[1]), sel(b, PB.app_a[0], PA.app_a[0]));
        g.b = sel(c1, sel(b, PB.app_b[1], PA.app_b[1]), sel(b, PB.app_b[0], PA.app_b[0]));
        g.out32 = sel(c1, sel(b, PB.app_out32[1], PA.app_out32[1]), sel(b, PB.app_out32[0], PA.app_out32[0]));
        g.out16 = sel(c1, sel(b, PB.app_out16[1], PA.app_out16[1]), sel(b, PB.app_out16[0], PA.app_out16[0]));
        g.outt = sel(c1, sel(b, PB.app_outt[1], PA.app_outt[1]), sel(b, PB.app_outt[0], PA.app_outt[0]));
        if (it == 0 && g.fold)
          gemm_tile<APPLY, T, TILE, KMODE == 1 ? 2 : 0, true>(g, out_of, u, tm, tn, claim_next,
                                                             count_pending);
        else
          gemm_tile<APPLY, T, TILE, KMODE == 1 ? 2 : 0>(g, out_of, u, tm, tn, claim_next,
                                                       count_pending);
      } else if (fm != FINAL_NONE) {
        zero_unit_tile<TILE>(out_of(), fm, tm * TILE, tn * TILE);
      }
    }
    if (live) {
      pend_a = cnt + (phase == GRAM ? 0 : phase == POLY ? ts : 2 * ts) + pa;
      pend_b = pb != pa ? pend_a + (pb - pa) : nullptr;
    }
    if (!local) flush();
    // The next tile's first copies overwrite the LDS that this tile's
    // epilogue staged through; the barrier after the next claim orders them.
  }
  // Every exit flushes the pending tile first.
}

template <typename T, int TILE, int KMODE>
__global__ __launch_bounds__(gemm_threads<TILE>()) void ns_persistent(NsSched p, ChunkArgs ca) {
  ns_persistent_run<T, TILE, KMODE, false>(p, ca, nullptr);
}

template <typename T, int TILE, int KMODE>
__global__ __launch_bounds__(gemm_threads<TILE>()) void ns_persistent2(NsSched p, ChunkArgs ca,
                                                                       NsPassB second) {
  ns_persistent_run<T, TILE, KMODE, true>(p, ca, &second);
}

}  // namespace muon_dev
