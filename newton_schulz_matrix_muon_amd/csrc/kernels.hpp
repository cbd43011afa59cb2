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
//   ns_gemm<POLY>   B = b*A + c*A*A.
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
  const float* aux;     // A (POLY) or X (APPLY), fp32, same layout as the output
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
// Operands are staged through LDS with 128-byte rows (64 bf16 or 32 fp32 of
// K), always K-contiguous in LDS; a K-contiguous global operand is copied
// 16 bytes at a time, an MN-contiguous one is transposed in registers on the
// way in.  16-byte chunks are XOR-swizzled so that both the row-wise stores
// and the 32-row MFMA fragment reads avoid bank conflicts.  Two LDS stages:
// the global loads of tile k+1 are in flight while tile k is multiplied.
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

__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ (row & 7) ^ ((row >> 3) & 7);
}

// Global -> registers for one operand tile (TILE rows of the M or N side,
// kBK of K).  KC: the operand is K-contiguous in global memory.
template <typename T, int TILE, bool KC>
struct TileLoader {
  static constexpr int kChunks = TILE / 32;  // 16-byte chunks per thread (K-contiguous)
  // Registers per thread: K-contiguous TILE/32 chunks; transposed bf16 one
  // 8x8 block (8 chunks) per thread, fewer blocks than threads at TILE 128;
  // transposed fp32 2*TILE/256 blocks of 4 chunks.
  static constexpr int kRegs =
      KC ? kChunks : (sizeof(T) == 2 ? 8 * ((TILE + kThreads - 1) / kThreads) : kChunks);
  u32x4 r[kRegs];

  __device__ __forceinline__ void load(const T* __restrict__ base, int ld, int mn0, int k0) {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = t + kThreads * i;
        const int row = c >> 3, kc = c & 7;
        r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)(mn0 + row) * ld + k0 +
                                                kc * OpT<T>::kElems);
      }
    } else if constexpr (sizeof(T) == 2) {
      // 8 (k) x 8 (mn) bf16 blocks; TILE blocks per tile.
      constexpr int kBlocks = TILE;
#pragma unroll
      for (int i = 0; i < (kBlocks + kThreads - 1) / kThreads; ++i) {
        const int blk = t + kThreads * i;
        if (kBlocks % kThreads == 0 || blk < kBlocks) {
          const int mb = blk % (TILE / 8), kb = blk / (TILE / 8);
#pragma unroll
          for (int rr = 0; rr < 8; ++rr)
            r[i * 8 + rr] = *reinterpret_cast<const u32x4*>(
                base + (int64_t)(k0 + kb * 8 + rr) * ld + mn0 + mb * 8);
        }
      }
    } else {
      // 4 (k) x 4 (mn) fp32 blocks; 2*TILE blocks per tile.
      constexpr int kBlocks = 2 * TILE;
#pragma unroll
      for (int i = 0; i < kBlocks / kThreads; ++i) {
        const int blk = t + kThreads * i;
        const int mb = blk % (TILE / 4), kb = blk / (TILE / 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          r[i * 4 + rr] = *reinterpret_cast<const u32x4*>(
              base + (int64_t)(k0 + kb * 4 + rr) * ld + mn0 + mb * 4);
      }
    }
  }

  // Registers -> LDS stage (TILE rows x 8 chunks of 16 bytes).
  __device__ __forceinline__ void store(u32x4* __restrict__ lds) const {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = t + kThreads * i;
        const int row = c >> 3, kc = c & 7;
        lds[row * 8 + swz(row, kc)] = r[i];
      }
    } else if constexpr (sizeof(T) == 2) {
      constexpr int kBlocks = TILE;
#pragma unroll
      for (int i = 0; i < (kBlocks + kThreads - 1) / kThreads; ++i) {
        const int blk = t + kThreads * i;
        if (kBlocks % kThreads == 0 || blk < kBlocks) {
          const int mb = blk % (TILE / 8), kb = blk / (TILE / 8);
          const u32x4* v = &r[i * 8];
          // v[rr] holds mn = mb*8 + 0..7 at k = kb*8 + rr.  Output row
          // mn = mb*8 + e gets k = kb*8 + 0..7: dword j packs k = 2j, 2j+1.
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            uint32_t d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t lo = v[2 * j][e >> 1];
              const uint32_t hi = v[2 * j + 1][e >> 1];
              d[j] = __builtin_amdgcn_perm(hi, lo, sel);
            }
            const int row = mb * 8 + e;
            lds[row * 8 + swz(row, kb)] = u32x4{d[0], d[1], d[2], d[3]};
          }
        }
      }
    } else {
      constexpr int kBlocks = 2 * TILE;
#pragma unroll
      for (int i = 0; i < kBlocks / kThreads; ++i) {
        const int blk = t + kThreads * i;
        const int mb = blk % (TILE / 4), kb = blk / (TILE / 4);
        const u32x4* v = &r[i * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = mb * 4 + e;
          const u32x4 o = u32x4{v[0][e], v[1][e], v[2][e], v[3][e]};
          lds[row * 8 + swz(row, kb)] = o;
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

template <int PHASE, typename T, int TILE, bool AKC, bool BKC>
__global__ __launch_bounds__(kThreads) void ns_gemm(GemmArgs g, ChunkArgs ca) {
  constexpr int WT = TILE / 2;   // wave tile
  constexpr int FM = WT / 32;    // 32x32 blocks per wave side
  constexpr bool kBF = sizeof(T) == 2;
  __shared__ u32x4 lds[2 * 2 * TILE * 8];

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
      const int64_t uoff = (int64_t)(u - sg.first) * ca.unit_elems;
      for (int idx = threadIdx.x; idx < TILE * TILE; idx += kThreads) {
        const int mm = m0 + idx / TILE, nn = n0 + idx % TILE;
        if (mm < ca.rows && nn < ca.cols) {
          float* p = sg.w + uoff + (int64_t)mm * ca.cols + nn;
          *p = (g.final_mode == FINAL_STEP) ? (*p) * ca.decay : 0.0f;
        }
      }
    }
    return;
  }

  const T* A = static_cast<const T*>(g.a) + (int64_t)u * g.a_ustride;
  const T* B = static_cast<const T*>(g.b) + (int64_t)u * g.b_ustride;
  // Stage st: A rows at lds + st*2*TILE*8, B rows right after them.
  constexpr int kStage = 2 * TILE * 8;

  f32x16 acc[FM][FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  TileLoader<T, TILE, AKC> la;
  TileLoader<T, TILE, BKC> lb;
  constexpr int BK = OpT<T>::kBK;
  const int nk = g.K / BK;

  la.load(A, g.lda, m0, 0);
  lb.load(B, g.ldb, n0, 0);
  la.store(lds);
  lb.store(lds + TILE * 8);
  __syncthreads();

  const int arow0 = wm * WT + (lane & 31);
  const int brow0 = wn * WT + (lane & 31);
  const int half = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, g.lda, m0, (kt + 1) * BK);
      lb.load(B, g.ldb, n0, (kt + 1) * BK);
    }
    const u32x4* As = lds + cur * kStage;
    const u32x4* Bs = As + TILE * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + half;
      u32x4 af[FM], bfr[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int ra = arow0 + i * 32;
        af[i] = As[ra * 8 + swz(ra, ch)];
        const int rb = brow0 + i * 32;
        bfr[i] = Bs[rb * 8 + swz(rb, ch)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          if constexpr (kBF) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j],
                0, 0, 0);
          } else {
            const f32x4v a4 = __builtin_bit_cast(f32x4v, af[i]);
            const f32x4v b4 = __builtin_bit_cast(f32x4v, bfr[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[q], b4[q], acc[i][j], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) {
      la.store(lds + (cur ^ 1) * kStage);
      lb.store(lds + (cur ^ 1) * kStage + TILE * 8);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m][n] for n = lane%32 and
  // m = 8*(r/4) + 4*(lane/32) + r%4 within each 32x32 block.
  const int ncol = lane & 31;
  const int mrow = 4 * half;
  float* wout = nullptr;
  if (PHASE == APPLY && g.final_mode != FINAL_NONE) {
    const SegView sg = find_seg(ca, u);
    wout = sg.w + (int64_t)(u - sg.first) * ca.unit_elems;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WT + i * 32 + 8 * (r >> 2) + mrow + (r & 3);
        const int n = n0 + wn * WT + j * 32 + ncol;
        const float v = acc[i][j][r];
        const int64_t o = (int64_t)u * g.out_ustride + (int64_t)m * g.ldo + n;
        if constexpr (PHASE == GRAM) {
          g.out32[o] = v;
          if constexpr (kBF) static_cast<uint16_t*>(g.out16)[o] = to_bf16_bits(v);
        } else if constexpr (PHASE == POLY) {
          const float bv =
              g.cb * g.aux[(int64_t)u * g.aux_ustride + (int64_t)m * g.ldaux + n] + g.cc * v;
          if constexpr (kBF)
            static_cast<uint16_t*>(g.out16)[o] = to_bf16_bits(bv);
          else
            g.out32[o] = bv;
        } else {
          const float xv = __builtin_fmaf(
              g.ca, g.aux[(int64_t)u * g.aux_ustride + (int64_t)m * g.ldaux + n], v);
          if (g.final_mode == FINAL_NONE) {
            g.out32[o] = xv;
            if constexpr (kBF) static_cast<uint16_t*>(g.out16)[o] = to_bf16_bits(xv);
          } else if (m < ca.rows && n < ca.cols) {
            float* p = wout + (int64_t)m * ca.cols + n;
            if (g.final_mode == FINAL_STEP)
              *p = __builtin_fmaf(-ca.lr_scale, xv, (*p) * ca.decay);
            else
              *p = xv;
          }
        }
      }
}

}  // namespace muon_dev
