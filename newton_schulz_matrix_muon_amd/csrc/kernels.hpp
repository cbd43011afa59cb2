// Device kernels of the Muon step for gfx950 (CDNA4, wave64).
//
// Kernels, in launch order for one stacked pass ("chunk") of equal-shape NS
// units:
//   k_momentum      M <- mu*M + G, N = mu*M + G into the fp32 iterate buffer,
//                   per-block fp64 partial sums of N^2 (DeepSeek tech notes
//                   "Muon 优化器" section 1 Algorithm 1; RFC-0023 方案 1).
//   k_norm_finish   per unit: fixed-order fp64 sum of the partials, 1/||N||_F
//                   and the non-zero flag (notes section 2: Frobenius
//                   normalisation, a zero matrix stays zero).
//   k_normalize     X0 = N/||N||_F over the padded iterate (zeros in the
//                   padding), plus the bf16 operand copy.
//   ns_gemm<GRAM>   A = X X^T (or X^T X for a tall unit: the smaller side).
//   ns_gemm<POLY>   B = b*A + c*A*A (on the bf16 path A is kept only as its
//                   bf16 operand copy, which the b*A term also reads).
//   ns_gemm<APPLY>  X' = a*X + B*X (or X*B); in the last iteration the
//                   epilogue writes W <- W*(1 - lr*wd) - lr*scale*X' instead
//                   (Algorithm 1's decoupled update) or the NS output.
// The three products are the quintic step a*X + b*(X X^T)X + c*(X X^T)^2 X of
// the notes' section 2, grouped as (b*A + c*A^2)*X.
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
};

struct ChunkArgs {
  int32_t n_seg;
  int32_t n_units;
  int32_t rows, cols;          // unit shape (fan_out x fan_in)
  int32_t rows_pad, cols_pad;  // padded iterate shape
  int64_t unit_elems;          // rows * cols
  int64_t x_stride;            // rows_pad * cols_pad
  float mu;
  float decay;                 // 1 - lr * weight_decay
  float lr_scale;              // lr * scale
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
  int32_t final_mode;
  const float* aux;     // fp32 A (POLY, fp32 path) or X (APPLY), laid out like the output
  const void* aux16;    // bf16 A (POLY, bf16 path)
  int64_t aux_ustride;
  int32_t ldaux;
  float ca, cb, cc;     // quintic coefficients
  const int32_t* flag;  // per unit: nonzero = the unit has a nonzero norm
};

// The segment holding chunk-local unit u.  Every table entry is read at a
// constant index (a dynamic index would copy the whole kernel-argument
// struct to scratch memory).
struct SegView {
  float* w;
  const void* g;
  float* m;
  int32_t first;
};

__device__ __forceinline__ SegView find_seg(const ChunkArgs& ca, int u) {
  SegView v{ca.seg[0].w, ca.seg[0].g, ca.seg[0].m, ca.seg[0].first};
#pragma unroll
  for (int s = 1; s < kMaxSeg; ++s) {
    if (s < ca.n_seg && ca.seg[s].first <= u) {
      v.w = ca.seg[s].w;
      v.g = ca.seg[s].g;
      v.m = ca.seg[s].m;
      v.first = ca.seg[s].first;
    }
  }
  return v;
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

// ------------------------------------------------------------- momentum ----
// GK: 0 = bf16 gradient, 1 = fp32 gradient, 2 = NS-only (copy fp32 input).
template <int GK>
__global__ __launch_bounds__(kThreads) void k_momentum(ChunkArgs ca, float* __restrict__ x32,
                                                        double* __restrict__ partials,
                                                        int rows_per_block, int blocks_per_unit) {
  __shared__ double sh[kThreads / 64];
  const int u = blockIdx.x / blocks_per_unit;
  const int bb = blockIdx.x - u * blocks_per_unit;
  const SegView sg = find_seg(ca, u);
  const int64_t uoff = (int64_t)(u - sg.first) * ca.unit_elems;
  const int cols = ca.cols;
  const int r0 = bb * rows_per_block;
  const int r1 = min(r0 + rows_per_block, ca.rows);
  const float mu = ca.mu;
  float* xu = x32 + (int64_t)u * ca.x_stride;
  double ss = 0.0;
  const bool vec = (cols & 3) == 0;
  for (int r = r0; r < r1; ++r) {
    const int64_t base = uoff + (int64_t)r * cols;
    float* xr = xu + (int64_t)r * ca.cols_pad;
    if (vec) {
      for (int c = threadIdx.x * 4; c < cols; c += kThreads * 4) {
        float g[4];
        if (GK == 0) {
          const uint2 raw = *reinterpret_cast<const uint2*>(
              static_cast<const uint16_t*>(sg.g) + base + c);
          g[0] = bf16_bits_to_f32(raw.x & 0xffffu);
          g[1] = bf16_bits_to_f32(raw.x >> 16);
          g[2] = bf16_bits_to_f32(raw.y & 0xffffu);
          g[3] = bf16_bits_to_f32(raw.y >> 16);
        } else {
          const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(sg.g) + base + c);
          g[0] = v.x; g[1] = v.y; g[2] = v.z; g[3] = v.w;
        }
        float n[4];
        if (GK == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) n[i] = g[i];
        } else {
          float4* mp = reinterpret_cast<float4*>(sg.m + base + c);
          const float4 mv = *mp;
          float m[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m[i] = __builtin_fmaf(mu, m[i], g[i]);
            n[i] = __builtin_fmaf(mu, m[i], g[i]);
          }
          *mp = make_float4(m[0], m[1], m[2], m[3]);
        }
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
          float m = __builtin_fmaf(mu, sg.m[base + c], g);
          sg.m[base + c] = m;
          n = __builtin_fmaf(mu, m, g);
        }
        xr[c] = n;
        ss = __builtin_fma((double)n, (double)n, ss);
      }
    }
  }
  const double t = block_sum(ss, sh);
  if (threadIdx.x == 0) partials[(int64_t)u * blocks_per_unit + bb] = t;
}

// One wave per unit: fixed-order sum of the partials.
__global__ __launch_bounds__(64) void k_norm_finish(const double* __restrict__ partials,
                                                    int blocks_per_unit, float* __restrict__ inv_nu,
                                                    int32_t* __restrict__ flag) {
  const int u = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < blocks_per_unit; i += 64)
    s += partials[(int64_t)u * blocks_per_unit + i];
  s = wave_sum(s);
  if (threadIdx.x == 0) {
    // A NaN/Inf sum keeps the unit active so that it propagates.
    const bool zero = (s == 0.0);
    flag[u] = zero ? 0 : 1;
    inv_nu[u] = zero ? 0.0f : (float)(1.0 / sqrt(s));
  }
}

// X0 = N * (1/nu) over the whole padded iterate; zeros in the padding.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_normalize(ChunkArgs ca, float* __restrict__ x32,
                                                         uint16_t* __restrict__ xb,
                                                         const float* __restrict__ inv_nu,
                                                         int64_t vec_per_block, int blocks_per_unit) {
  const int u = blockIdx.x / blocks_per_unit;
  const int bb = blockIdx.x - u * blocks_per_unit;
  const float s = inv_nu[u];
  const int64_t nvec = ca.x_stride >> 2;
  const int64_t v0 = (int64_t)bb * vec_per_block;
  const int64_t v1 = min(v0 + vec_per_block, nvec);
  float* xu = x32 + (int64_t)u * ca.x_stride;
  uint16_t* xbu = BF16 ? xb + (int64_t)u * ca.x_stride : nullptr;
  const int cp = ca.cols_pad;
  for (int64_t v = v0 + threadIdx.x; v < v1; v += kThreads) {
    const int64_t e = v << 2;
    const int r = (int)(e / cp);
    const int c = (int)(e - (int64_t)r * cp);
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < ca.rows && c < ca.cols) {
      const float4 nv = *reinterpret_cast<const float4*>(xu + e);
      val.x = nv.x * s;
      val.y = (c + 1 < ca.cols) ? nv.y * s : 0.f;
      val.z = (c + 2 < ca.cols) ? nv.z * s : 0.f;
      val.w = (c + 3 < ca.cols) ? nv.w * s : 0.f;
    }
    *reinterpret_cast<float4*>(xu + e) = val;
    if (BF16) {
      uint2 packed;
      packed.x = (uint32_t)to_bf16_bits(val.x) | ((uint32_t)to_bf16_bits(val.y) << 16);
      packed.y = (uint32_t)to_bf16_bits(val.z) | ((uint32_t)to_bf16_bits(val.w) << 16);
      *reinterpret_cast<uint2*>(xbu + e) = packed;
    }
  }
}

// ------------------------------------------------------------------ GEMM ---
// Batched C = A_op * B_op over padded units, one TILE x TILE output tile per
// workgroup of 4 waves (2 x 2, each TILE/2 x TILE/2 as 32x32 MFMA blocks).
//
// LDS holds, per stage, TILE rows of A_op and TILE rows of B_op, each row
// 128 bytes of K (64 bf16 or 32 fp32) in eight 16-byte chunks, XOR-swizzled
// (chunk ^ row%8 ^ (row/8)%8) so that 8 consecutive rows read at one logical
// chunk hit distinct banks.  Two stages live in two separate LDS arrays.
//  - A K-contiguous global operand is copied global -> LDS directly
//    (buffer_load_dwordx4 ... lds: lane i of a wave lands at M0 + 16*i, so
//    the swizzle is applied by choosing which global chunk each lane fetches).
//  - An MN-contiguous operand is loaded into registers, transposed there in
//    8x8 (bf16) or 4x4 (fp32) blocks and written to LDS.
// MFMA fragments are double-buffered across the four K sub-steps of a tile.
// The MFMA is issued as (B fragment, A fragment), so each lane accumulates
// C[m][n..n+3] for one row m and 4 consecutive columns: the epilogue moves
// 16-byte vectors.
template <typename T>
struct OpT;
template <>
struct OpT<__bf16> {
  static constexpr int kElems = 8;  // per 16-byte chunk
  static constexpr int kBK = 64;    // K per LDS row
};
template <>
struct OpT<float> {
  static constexpr int kElems = 4;
  static constexpr int kBK = 32;
};

typedef __attribute__((address_space(3))) void* lds_vptr;

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ (row & 7) ^ ((row >> 3) & 7);
}

// K-contiguous operand: TILE rows x 8 chunks, straight into LDS through a
// buffer resource whose base is the tile's first row (so 32-bit offsets
// cover TILE rows).  The MUBUF form (buffer_load ... lds) is used rather
// than global_load_lds: the latter is a FLAT-encoded LDS writer, which makes
// the compiler wait for all LDS reads at once while it is in flight.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  // raw buffer, stride 0, 2 GiB range, 32-bit data format (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

template <typename T, int TILE>
__device__ __forceinline__ void issue_direct(__amdgpu_buffer_rsrc_t rs, int ld, int k0,
                                             u32x4* lds_stage) {
  constexpr int kPerWave = TILE / 32;  // 64-lane instructions per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int slot0 = (w * kPerWave + i) * 64;  // first 16-byte slot of this instruction
    const int s = slot0 + lane;
    const int row = s >> 3, pc = s & 7;
    const int c = pc ^ (row & 7) ^ ((row >> 3) & 7);  // logical chunk stored at (row, pc)
    const int voff = (row * ld + k0 + c * OpT<T>::kElems) * (int)sizeof(T);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_vptr)(lds_stage + slot0), 16, voff, 0, 0, 0);
  }
}

// MN-contiguous operand: registers, transposed on the way to LDS.
template <typename T, int TILE>
struct TransLoader {
  static constexpr bool kBF = sizeof(T) == 2;
  static constexpr int kBlocks = kBF ? TILE : 2 * TILE;  // 8x8 bf16 or 4x4 fp32 blocks
  static constexpr int kIters = (kBlocks + kThreads - 1) / kThreads;
  static constexpr int kRegs = kIters * (kBF ? 8 : 4);
  u32x4 r[kRegs];

  __device__ __forceinline__ void load(const T* __restrict__ base, int ld, int mn0, int k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int blk = t + kThreads * i;
      if (kBlocks % kThreads == 0 || blk < kBlocks) {
        if constexpr (kBF) {
          const int mb = blk % (TILE / 8), kb = blk / (TILE / 8);
#pragma unroll
          for (int rr = 0; rr < 8; ++rr)
            r[i * 8 + rr] = *reinterpret_cast<const u32x4*>(
                base + (int64_t)(k0 + kb * 8 + rr) * ld + mn0 + mb * 8);
        } else {
          const int mb = blk % (TILE / 4), kb = blk / (TILE / 4);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            r[i * 4 + rr] = *reinterpret_cast<const u32x4*>(
                base + (int64_t)(k0 + kb * 4 + rr) * ld + mn0 + mb * 4);
        }
      }
    }
  }

  __device__ __forceinline__ void store(u32x4* __restrict__ lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int blk = t + kThreads * i;
      if (kBlocks % kThreads == 0 || blk < kBlocks) {
        if constexpr (kBF) {
          const int mb = blk % (TILE / 8), kb = blk / (TILE / 8);
          const u32x4* v = &r[i * 8];
          // v[rr] holds mn = mb*8 + 0..7 at k = kb*8 + rr; LDS row
          // mn = mb*8 + e takes k = kb*8 + 0..7 (dword j packs k = 2j, 2j+1).
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              d[j] = __builtin_amdgcn_perm(v[2 * j + 1][e >> 1], v[2 * j][e >> 1], sel);
            const int row = mb * 8 + e;
            lds[row * 8 + swz(row, kb)] = u32x4{d[0], d[1], d[2], d[3]};
          }
        } else {
          const int mb = blk % (TILE / 4), kb = blk / (TILE / 4);
          const u32x4* v = &r[i * 4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = mb * 4 + e;
            lds[row * 8 + swz(row, kb)] = u32x4{v[0][e], v[1][e], v[2][e], v[3][e]};
          }
        }
      }
    }
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

template <typename T, int FM>
__device__ __forceinline__ void mfma_block(const u32x4 (&af)[FM], const u32x4 (&bf)[FM],
                                           f32x16 (&acc)[FM][FM]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      // (B, A): the lane owning C row m receives 4 consecutive columns.
      if constexpr (sizeof(T) == 2) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, bf[j]), __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0, 0, 0);
      } else {
        const f32x4v a4 = __builtin_bit_cast(f32x4v, af[i]);
        const f32x4v b4 = __builtin_bit_cast(f32x4v, bf[j]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(b4[q], a4[q], acc[i][j], 0, 0, 0);
      }
    }
}

__device__ __forceinline__ void store_bf16x4(void* base, int64_t idx, float a, float b, float c,
                                             float d) {
  uint2 p;
  p.x = (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
  p.y = (uint32_t)to_bf16_bits(c) | ((uint32_t)to_bf16_bits(d) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = p;
}

template <int PHASE, typename T, int TILE, bool AKC, bool BKC>
__global__ __launch_bounds__(kThreads) void ns_gemm(GemmArgs g, ChunkArgs ca) {
  constexpr int WT = TILE / 2;   // wave tile
  constexpr int FM = WT / 32;    // 32x32 blocks per wave side
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int kOp = TILE * 8;  // 16-byte slots of one operand in one stage
  __shared__ u32x4 lds0[2 * kOp];
  __shared__ u32x4 lds1[2 * kOp];

  const int tiles_per_unit = g.tiles_m * g.tiles_n;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int u = logical / tiles_per_unit;
  const int tt = logical - u * tiles_per_unit;
  const int tm = tt / g.tiles_n, tn = tt - (tt / g.tiles_n) * g.tiles_n;
  const int m0 = tm * TILE, n0 = tn * TILE;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  if (!g.flag[u]) {
    if (PHASE == APPLY && g.final_mode != FINAL_NONE) {
      // Zero unit: O' = 0, so the weight only decays / the output is zero.
      const SegView sg = find_seg(ca, u);
      float* wout = sg.w + (int64_t)(u - sg.first) * ca.unit_elems;
      for (int idx = threadIdx.x; idx < TILE * TILE; idx += kThreads) {
        const int mm = m0 + idx / TILE, nn = n0 + idx % TILE;
        if (mm < ca.rows && nn < ca.cols) {
          float* p = wout + (int64_t)mm * ca.cols + nn;
          *p = (g.final_mode == FINAL_STEP) ? (*p) * ca.decay : 0.0f;
        }
      }
    }
    return;
  }

  const T* A = static_cast<const T*>(g.a) + (int64_t)u * g.a_ustride;
  const T* B = static_cast<const T*>(g.b) + (int64_t)u * g.b_ustride;

  f32x16 acc[FM][FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  TransLoader<T, TILE> ta, tb;
  constexpr int BK = OpT<T>::kBK;
  const int nk = g.K / BK;

  const __amdgpu_buffer_rsrc_t rsa = tile_rsrc(A + (int64_t)m0 * g.lda);
  const __amdgpu_buffer_rsrc_t rsb = tile_rsrc(B + (int64_t)n0 * g.ldb);
  auto issue = [&](int kt, u32x4* stage) {
    if constexpr (AKC) issue_direct<T, TILE>(rsa, g.lda, kt * BK, stage);
    else ta.load(A, g.lda, m0, kt * BK);
    if constexpr (BKC) issue_direct<T, TILE>(rsb, g.ldb, kt * BK, stage + kOp);
    else tb.load(B, g.ldb, n0, kt * BK);
  };
  auto finish = [&](u32x4* stage) {
    if constexpr (!AKC) ta.store(stage);
    if constexpr (!BKC) tb.store(stage + kOp);
  };

  issue(0, lds0);
  finish(lds0);
  // Drain the scalar (kernel-argument) loads before the K loop: a scalar
  // load still in flight would force every LDS wait in the loop to wait for
  // everything, since scalar loads can return out of order.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  const int arow0 = wm * WT + (lane & 31);
  const int brow0 = wn * WT + (lane & 31);
  const int half = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    u32x4* cur = (kt & 1) ? lds1 : lds0;
    u32x4* nxt = (kt & 1) ? lds0 : lds1;
    if (kt + 1 < nk) issue(kt + 1, nxt);
    const u32x4* As = cur;
    const u32x4* Bs = cur + kOp;
    u32x4 af[2][FM], bf[2][FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int ra = arow0 + i * 32, rb = brow0 + i * 32;
      af[0][i] = As[ra * 8 + swz(ra, half)];
      bf[0][i] = Bs[rb * 8 + swz(rb, half)];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // One scheduling region per sub-step: the fragment reads of sub-step
      // kk+1 and the MFMAs of sub-step kk (which only read registers loaded
      // in the previous region), so LDS latency hides under the MFMAs.
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) {
        const int ch = 2 * (kk + 1) + half;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int ra = arow0 + i * 32, rb = brow0 + i * 32;
          af[(kk + 1) & 1][i] = As[ra * 8 + swz(ra, ch)];
          bf[(kk + 1) & 1][i] = Bs[rb * 8 + swz(rb, ch)];
        }
      }
      mfma_block<T, FM>(af[kk & 1], bf[kk & 1], acc);
      // Within the region: every fragment read first, then the MFMAs, so
      // the reads have the whole region to land.
      if (kk < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FM * (kBF ? 1 : 4), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) finish(nxt);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m][n + 0..3] for m = .. + lane%32 and
  // n = .. + 8*q + 4*(lane/32), q = r/4, within each 32x32 block.
  float* wout = nullptr;
  if (PHASE == APPLY && g.final_mode != FINAL_NONE) {
    const SegView sg = find_seg(ca, u);
    wout = sg.w + (int64_t)(u - sg.first) * ca.unit_elems;
  }
  const bool vec_w = (ca.cols & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WT + i * 32 + (lane & 31);
    float4 aux[FM][4];
    if constexpr (PHASE == POLY && kBF) {
      // bf16 path: A exists only as the bf16 operand copy.
      const uint16_t* ap = static_cast<const uint16_t*>(g.aux16) + (int64_t)u * g.aux_ustride +
                           (int64_t)m * g.ldaux;
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 h = *reinterpret_cast<const uint2*>(ap + n0 + wn * WT + j * 32 + 8 * q + 4 * half);
          aux[j][q] = make_float4(bf16_bits_to_f32(h.x & 0xffffu), bf16_bits_to_f32(h.x >> 16),
                                  bf16_bits_to_f32(h.y & 0xffffu), bf16_bits_to_f32(h.y >> 16));
        }
    } else if constexpr (PHASE != GRAM) {
      const float* ap = g.aux + (int64_t)u * g.aux_ustride + (int64_t)m * g.ldaux;
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          aux[j][q] = *reinterpret_cast<const float4*>(ap + n0 + wn * WT + j * 32 + 8 * q + 4 * half);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WT + j * 32 + 8 * q + 4 * half;
        const f32x16& c = acc[i][j];
        float v0 = c[4 * q], v1 = c[4 * q + 1], v2 = c[4 * q + 2], v3 = c[4 * q + 3];
        const int64_t o = (int64_t)u * g.out_ustride + (int64_t)m * g.ldo + n;
        if constexpr (PHASE == GRAM) {
          if constexpr (kBF)
            store_bf16x4(g.out16, o, v0, v1, v2, v3);
          else
            *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v0, v1, v2, v3);
        } else if constexpr (PHASE == POLY) {
          const float4 a = aux[j][q];
          v0 = g.cb * a.x + g.cc * v0;
          v1 = g.cb * a.y + g.cc * v1;
          v2 = g.cb * a.z + g.cc * v2;
          v3 = g.cb * a.w + g.cc * v3;
          if constexpr (kBF)
            store_bf16x4(g.out16, o, v0, v1, v2, v3);
          else
            *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v0, v1, v2, v3);
        } else {
          const float4 a = aux[j][q];
          v0 = __builtin_fmaf(g.ca, a.x, v0);
          v1 = __builtin_fmaf(g.ca, a.y, v1);
          v2 = __builtin_fmaf(g.ca, a.z, v2);
          v3 = __builtin_fmaf(g.ca, a.w, v3);
          if (g.final_mode == FINAL_NONE) {
            *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v0, v1, v2, v3);
            if constexpr (kBF) store_bf16x4(g.out16, o, v0, v1, v2, v3);
          } else if (m < ca.rows && n < ca.cols) {
            float* p = wout + (int64_t)m * ca.cols + n;
            const bool step = g.final_mode == FINAL_STEP;
            if (vec_w && n + 3 < ca.cols) {
              float4 wv = step ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
              if (step) {
                wv.x = __builtin_fmaf(-ca.lr_scale, v0, wv.x * ca.decay);
                wv.y = __builtin_fmaf(-ca.lr_scale, v1, wv.y * ca.decay);
                wv.z = __builtin_fmaf(-ca.lr_scale, v2, wv.z * ca.decay);
                wv.w = __builtin_fmaf(-ca.lr_scale, v3, wv.w * ca.decay);
              } else {
                wv = make_float4(v0, v1, v2, v3);
              }
              *reinterpret_cast<float4*>(p) = wv;
            } else {
              const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (n + e < ca.cols)
                  p[e] = step ? __builtin_fmaf(-ca.lr_scale, vv[e], p[e] * ca.decay) : vv[e];
              }
            }
          }
        }
      }
  }
}

}  // namespace muon_dev
