// fa_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// Matrix-core fragments.  All contractions use v_mfma_f32_32x32x16_bf16 (bf16)
// or eight v_mfma_f32_32x32x2f32 (fp32) per 16-wide chunk of the contraction.
// Lane l of a 64-wide wave is described by (l32 = l % 32, g = l / 32):
//   A operand (32 x 16): lane (i = l32, g) supplies 8 values of row i,
//   B operand (16 x 32): lane (j = l32, g) supplies 8 values of column j,
//   C (32 x 32 fp32, 16 registers): register r of lane (j = l32, g) holds
//     row 8*(r/4) + 4*g + (r%4), column j.
// The hardware pairs item e of lane-half g of A with item e of lane-half g of
// B, so any fixed assignment "contraction index = pi(g, e)" that both operands
// follow gives the right sum.  Two assignments are used:
//   natural  : pi(g, e) = 8g + e                 (d-contractions; operands read
//                                                  straight from row-major tiles)
//   C-shaped : pi(g, e) = 8*(e/4) + 4g + (e%4)   (contractions over the row
//                                                  index of a C tile, so that
//                                                  registers 8t..8t+7 of C are
//                                                  directly an operand chunk)
// Tiles that feed the C-shaped side are stored transposed in LDS with each
// 16-group of the contraction index permuted (bits 2 and 3 swapped), so a
// lane's 8 values are one contiguous 16-byte (bf16) read.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaskBlock = 128;
constexpr int kThreads = 256;   // 4 waves per work-group

// Exponent coefficient c = scale * log2(e), clamped to at least FLT_MIN so
// that c > 0: a masked score (-inf) then always gives 2^(-inf * c) = 0.  For
// scale = 0 every kept exponent is 2^(s * FLT_MIN - m) with |s * FLT_MIN| far
// below half an ulp of 1, i.e. exactly the values scale = 0 gives.
inline float score_coef(float scale) {
  const float c = scale * kLog2e;
  return c < 1.17549435e-38f ? 1.17549435e-38f : c;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

// Position of contraction index x inside its 16-group in a transposed tile.
__device__ __forceinline__ constexpr int perm16(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// ---------------------------------------------------------------------------
// Element traits
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  struct frag { bf16x8 v; };
  static constexpr int kPerChunk = 8;      // elements per 16-byte chunk
  __device__ static frag zero() { frag f; f.v = bf16x8{}; return f; }
  __device__ static frag load(const __bf16* p) {   // 16-byte aligned
    frag f; f.v = *reinterpret_cast<const bf16x8*>(p); return f;
  }
  __device__ static f32x16 mma(const frag& a, const frag& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
  }
  // Registers 8t..8t+7 of a C tile as an operand chunk (rounded to nearest even).
  __device__ static frag from_c(const f32x16& c, int t) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (__bf16)c[8 * t + e];
    return f;
  }
  __device__ static void store4(__bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v; v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
  }
  __device__ static float to_f32(__bf16 x) { return (float)x; }
};

template <> struct Elem<float> {
  struct frag { f32x4 lo, hi; };
  static constexpr int kPerChunk = 4;
  __device__ static frag zero() { frag f; f.lo = f32x4{}; f.hi = f32x4{}; return f; }
  __device__ static frag load(const float* p) {    // 16-byte aligned
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
  }
  __device__ static f32x16 mma(const frag& a, const frag& b, f32x16 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], c, 0, 0, 0);
    return c;
  }
  __device__ static frag from_c(const f32x16& c, int t) {
    frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.lo[e] = c[8 * t + e]; f.hi[e] = c[8 * t + 4 + e]; }
    return f;
  }
  __device__ static void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
  __device__ static float to_f32(float x) { return x; }
};

// ---------------------------------------------------------------------------
// Global loads through raw buffer descriptors.  A descriptor covers [base,
// base + bytes); a load whose offset falls outside returns zeros, so tile
// tails need no branches (and the waitcnt bookkeeping of the loads stays
// exact, which a branch around each load would defeat).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Wait until every outstanding global load of this wave has landed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maximum).  Issued
// unconditionally at the top of each tile iteration: the LDS stores need the
// prefetched tile anyway, and it tells the compiler that older loads (the
// fragments loaded before the loop) are complete.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One operand fragment (8 contraction values) read straight from global memory.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag gload_frag(rsrc_t r, uint32_t off) {
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    f.v = __builtin_bit_cast(bf16x8, buf_load16(r, off));
  } else {
    f.lo = __builtin_bit_cast(f32x4, buf_load16(r, off));
    f.hi = __builtin_bit_cast(f32x4, buf_load16(r, off + 16));
  }
  return f;
}

// ---------------------------------------------------------------------------
// Tile staging: global [rows x D] row-major (row stride D) -> LDS.
//
// A "quad task" covers 4 consecutive rows x one 16-byte column chunk.  It is
// loaded with four 16-byte buffer loads (rows outside the descriptor read as
// zero) and can be written to LDS row-major and/or transposed
// (contraction-permuted).
// ---------------------------------------------------------------------------
template <typename T, int D>
struct QuadTask {
  static constexpr int E = Elem<T>::kPerChunk;   // elements per chunk
  static constexpr uint32_t kRowBytes = D * sizeof(T);
  u32x4 r[4];

  // `off`: byte offset, inside the descriptor, of (row0, col).
  __device__ void load(rsrc_t rs, uint32_t off) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = buf_load16(rs, off + i * kRowBytes);
  }
  // Row-major: lds[(row0+i) * ld + col .. +E]
  __device__ void store_rows(T* lds, int ld, int row0, int col) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(lds + (row0 + i) * ld + col) = r[i];
  }
  // Transposed: ldsT[(col+e) * ldt + perm16(row0) .. +4]; row0 % 4 == 0.
  __device__ void store_transposed(T* ldsT, int ldt, int row0, int col) const;
};

template <typename T, int D>
__device__ __forceinline__ void QuadTask<T, D>::store_transposed(T* ldsT, int ldt, int row0,
                                                                 int col) const {
  const int p = perm16(row0);
  if constexpr (sizeof(T) == 2) {
    // r[i] holds 8 bf16 of row i: element e sits in dword e/2, half e%2.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
      } else {
        lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
      }
      *reinterpret_cast<u32x2*>(ldsT + (col + e) * ldt + p) = u32x2{lo, hi};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<u32x4*>(ldsT + (col + e) * ldt + p) =
          u32x4{r[0][e], r[1][e], r[2][e], r[3][e]};
  }
}

// ---------------------------------------------------------------------------
// Work-group -> (head, block) mapping.
//
// Blocks are handed to the 8 XCDs round-robin by work-group id, and each XCD
// has its own L2.  When the head count is a multiple of 8, head h is pinned to
// XCD h % 8 so all blocks of a head share one L2 (they re-read the same K/V or
// Q/dO tiles).  Within an XCD, blocks are ordered by decreasing work when
// `heavy_first_desc` (causal query blocks: the last block has the most keys)
// or `heavy_first_asc` (causal key blocks: the first block has the most
// queries).
// ---------------------------------------------------------------------------
struct BlockCoord { int bh; int blk; };

__device__ __forceinline__ BlockCoord map_block(int wg, int nblk, int BH, bool causal,
                                                bool heavy_is_last) {
  int rank, bh;
  if ((BH & 7) == 0) {
    const int xcd = wg & 7;
    const int s = wg >> 3;
    const int hpx = BH >> 3;          // heads per XCD
    rank = s / hpx;
    bh = (s - rank * hpx) * 8 + xcd;
  } else {
    rank = wg / BH;
    bh = wg - rank * BH;
  }
  int blk = rank;
  if (causal && heavy_is_last) blk = nblk - 1 - rank;
  return BlockCoord{bh, blk};
}

}  // namespace fa
