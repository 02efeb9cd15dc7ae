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
// Operands of the C-shaped side that come from LDS are read from row-major
// tiles with the transposing LDS load (trans_frag below).

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
// The forward moves its reference max only when a row max grows by more than
// this many doublings (see fa_fwd.hip); probabilities stay <= 2^kLazy.
constexpr float kLazy = 8.0f;

// Exponent coefficient handed to the kernels: |c| = |scale| * log2(e),
// clamped to at least FLT_MIN, carrying the sign of scale.  The forward
// kernels set masked scores to -inf before the row max, so they split it with
// split_coef and work with the positive |c| (then 2^(-inf * |c|) = 0 and |c|
// times the row max of the kept scores is the row max of S * |c|); for
// scale < 0 they flip the sign of Q in registers, which is exact, so they form
// -S and -S * |c| = scale * log2(e) * S.  The backward kernels mask P with a
// select after the exponential and use the signed c as it is; their final dQ
// and dK multiplications use the signed scale.  For scale = 0 every kept
// exponent is 2^(s * FLT_MIN - m) with |s * FLT_MIN| far below half an ulp of
// 1, i.e. exactly the values scale = 0 gives.
inline float score_coef(float scale) {
  float c = (scale < 0.f ? -scale : scale) * kLog2e;
  c = c < 1.17549435e-38f ? 1.17549435e-38f : c;
  return scale < 0.f ? -c : c;
}

// Kernel side of score_coef: returns |c| and whether the scores must be negated.
__device__ __forceinline__ float split_coef(float c, bool& negate_scores) {
  negate_scores = c < 0.f;
  return negate_scores ? -c : c;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

// Compile-time tags for generic lambdas.
template <int V> struct IntTag {
  static constexpr int value = V;
  __device__ constexpr operator int() const { return V; }
};
template <bool V> struct BoolTag {
  static constexpr bool value = V;
  __device__ constexpr operator bool() const { return V; }
};

// Double-buffered LDS tiles are two distinct __shared__ arrays, and loops
// that alternate between them are unrolled by two so the buffer is a
// compile-time choice (pick with an IntTag).  Then the compiler can tell that
// an LDS read of one buffer does not touch the other buffer, which the
// direct-to-LDS loads of the next tile are filling: with a single array (or a
// runtime choice) it makes each transposing LDS read wait until all of those
// loads have landed.
template <int V>
__device__ __forceinline__ unsigned char* pick(IntTag<V>, unsigned char* b0, unsigned char* b1) {
  return V == 0 ? b0 : b1;
}
__device__ __forceinline__ unsigned char* pick(int v, unsigned char* b0, unsigned char* b1) {
  return v ? b1 : b0;
}
template <int V> __device__ __forceinline__ constexpr IntTag<V ^ 1> other(IntTag<V>) { return {}; }
__device__ __forceinline__ int other(int v) { return v ^ 1; }
// The same for a ring of three arrays.
template <int V>
__device__ __forceinline__ unsigned char* pick3(IntTag<V>, unsigned char* a, unsigned char* b,
                                                unsigned char* c) {
  return V == 0 ? a : (V == 1 ? b : c);
}
template <int V>
__device__ __forceinline__ unsigned char* pick4(IntTag<V>, unsigned char* a, unsigned char* b,
                                                unsigned char* c, unsigned char* d) {
  return V == 0 ? a : (V == 1 ? b : (V == 2 ? c : d));
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), written from the paper's
// definition: each round multiplies words 0 and 2 by the two round constants,
// keeps the low halves as the new words 3 and 1 and XORs the high halves with
// the other two words and the key into the new words 0 and 2; the key
// advances by the two Weyl constants between rounds.  A counter-based
// generator: the dropout keep mask is recomputed wherever it is needed
// instead of being stored.
struct Philox4 { uint32_t w[4]; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    // one 32 x 32 -> 64-bit multiply each (a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Dropout parameters as the kernels receive them (unused unless the kernel
// is instantiated with dropout).
struct DropParams {
  uint32_t key0, key1, thresh;
  float inv_keep;
};

// Value of lane l ^ 32 exchanged without a trip through LDS:
// v_permlane32_swap_b32 swaps the upper 32 lanes of its first register with
// the lower 32 lanes of its second, so with both holding x the pair becomes
// (x of lanes 0-31 twice, x of lanes 32-63 twice).  The leading s_nop covers
// the wait states the swap needs after a VALU write of its sources.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
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

// Every caller passes a wave-uniform base and size.  Saying so explicitly
// keeps the descriptor in scalar registers: if the compiler cannot prove the
// values uniform it wraps each buffer load in a per-lane loop over distinct
// descriptors.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
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

// Keeps the compiler's scheduler from moving instructions across this point
// (used to issue a batch of LDS operand reads before the MFMAs that consume
// them, so their latency overlaps the matrix work).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Scheduling hint for one straight-line region: issue the region's first
// `READS` LDS reads, then alternate one MFMA with up to `VPM` VALU
// instructions, `MFMAS` times.  Instructions the pattern does not claim are
// placed freely by the scheduler; dependencies always win.
template <int MFMAS, int READS, int VPM>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);   // DS read
#pragma unroll
  for (int i = 0; i < MFMAS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);   // VALU
  }
}

// Flip the sign of every value of an operand fragment (a sign-bit XOR: exact,
// and -x of a finite value is always representable).
__device__ __forceinline__ void negate(Elem<__bf16>::frag& f) {
  f.v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f.v) ^ 0x80008000u);
}
__device__ __forceinline__ void negate(Elem<float>::frag& f) {
  f.lo = -f.lo;
  f.hi = -f.hi;
}
// Pin an MFMA operand fragment to the accumulation registers (AGPRs).  The
// empty asm reads the value, so the compiler waits for the load that produced
// it at this point: call it just before the MFMA that consumes the fragment.
template <typename F>
__device__ __forceinline__ void to_agpr(F& f) {
  if constexpr (sizeof(f) == 16) {
    asm("" : "+a"(f.v));
  } else {
    asm("" : "+a"(f.lo));
    asm("" : "+a"(f.hi));
  }
}

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
// LDS tiles.
//
// A tile holds R rows of a [*, D] row-major tensor, unpadded (D * sizeof(T)
// bytes per row), with the 16-byte chunks of row r stored at chunk position
// c ^ swz(r).  The swizzles were chosen against the gfx950 LDS, which serves
// ds_read_b128 in four groups of 16 lanes (256 bytes), grouped by bit 5 and by
// the parity of bits 2..4 of the lane index (measured with the bank-conflict
// counter), and ds_read_b64_tr_b16 32 lanes at a time:
//   * operand reads along a row (ds_read_b128, lane l32 of each half-wave on
//     row l32 at one chunk; rows r and r + 16 fall in different groups) need
//     swz to be a bijection over 16 consecutive rows;
//   * transposed reads (ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes per
//     32 lanes) need those 4 rows to land in 4 different 64-byte segments of
//     the 256-byte bank window.
// bf16, D = 128: swz(r) = 4 (r % 4) + (r / 4) % 4 satisfies both; bf16, D = 64
// (two rows per bank window): swz(r) = 4 ((r / 2) % 2) + (r / 4) % 4.  The
// fp32 path reads transposed operands with scalar loads and uses r % 16.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Tile {
  static constexpr int RB = D * (int)sizeof(T);    // bytes per row
  __device__ static constexpr int swz(int r) {
    if constexpr (sizeof(T) == 2) {
      if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
      else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    } else {
      return r & 15;
    }
  }
  // Byte offset of logical 16-byte chunk c of row r.
  __device__ static constexpr uint32_t off(int r, int c) {
    return (uint32_t)(r * RB + ((c ^ swz(r)) << 4));
  }
};

typedef __attribute__((address_space(3))) unsigned char lds_byte;
__device__ __forceinline__ lds_byte* as_lds(unsigned char* p) { return (lds_byte*)p; }

// Copy R rows of a row-major global tile into an LDS tile (layout Tile<T, D>)
// with direct buffer->LDS loads: every lane moves one 16-byte chunk, lane l of
// a wave landing at LDS byte 16 l of the wave's 1 KiB block, so each lane
// fetches the global chunk that the swizzle puts there.  `src` starts at the
// tile's first row; rows outside it arrive as zeros.  The WAVES waves of the
// work-group take 1 KiB blocks round-robin.  Completion: wait_global_loads() in each wave, then a barrier.
template <typename T, int D, int R, int WAVES = 4>
__device__ __forceinline__ void stage_tile(rsrc_t src, unsigned char* tile, int w, int lane) {
  using L = Tile<T, D>;
  constexpr int NB = R * L::RB / 1024;
  static_assert(NB % WAVES == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NB / WAVES; ++i) {
    const int blk = w + WAVES * i;
    const int pos = blk * 1024 + lane * 16;
    const int r = pos / L::RB, pc = (pos % L::RB) >> 4;
    const uint32_t goff = (uint32_t)(r * L::RB + ((pc ^ L::swz(r)) << 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, as_lds(tile + blk * 1024), 16, goff, 0, 0, 0);
  }
}

// Natural-order operand: 8 contraction values of row `row` starting at
// element 16 t + 8 g (A operand of a d-contraction with rows as MFMA rows,
// or B operand with rows as MFMA columns).
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag row_frag(const unsigned char* tile, int row,
                                                            int t, int g) {
  using L = Tile<T, D>;
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(tile + L::off(row, 2 * t + g));
  } else {
    f.lo = *reinterpret_cast<const f32x4*>(tile + L::off(row, 4 * t + 2 * g));
    f.hi = *reinterpret_cast<const f32x4*>(tile + L::off(row, 4 * t + 2 * g + 1));
  }
  return f;
}

// Precomputed per-lane LDS offsets for the operand reads of one kernel.  The
// swizzle depends only on (row mod 16), so for a lane the offsets of the
// natural reads differ only per d-chunk t, and those of the transposed reads
// only per (output block b, row group h); row-block, 16-row chunk and
// tensor offsets are compile-time and go into the instruction's immediate.
template <typename T, int D>
struct LaneOffsets {
  static constexpr int NT = D / 16, ND = D / 32;
  uint32_t row[NT];        // row l32, chunk 2t + g (bf16)
  uint32_t tr[ND][2];      // transposed reads: rows rl + 8h, columns of block b

  __device__ void init(int lane) {
    using L = Tile<T, D>;
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int t = 0; t < NT; ++t) row[t] = L::off(l32, 2 * t + g);
    if constexpr (sizeof(T) == 2) {
      const int q = lane >> 4, j = lane & 15;
      const int rl = 4 * (q >> 1) + (j >> 2);
#pragma unroll
      for (int b = 0; b < ND; ++b) {
        const int col = 32 * b + 16 * (q & 1) + 4 * (j & 3);
#pragma unroll
        for (int h = 0; h < 2; ++h) tr[b][h] = L::off(rl + 8 * h, col >> 3) + ((col & 7) << 1);
      }
    }
  }
};

// Natural-order bf16 operand at a precomputed lane offset (see row_frag).
// (fp32 operands span two swizzled chunks and use row_frag.)
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag row_frag_at(const unsigned char* p) {
  static_assert(sizeof(T) == 2, "bf16 only");
  typename Elem<T>::frag f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}

// C-shaped transposed operand: the A operand of a contraction over the tile's
// rows, for output rows 32 b .. 32 b + 31 (= tile columns) and contraction
// rows 16 cc .. 16 cc + 15.  Lane (l32, g) gets, for item e, the element at
// tile row 16 cc + 8 (e / 4) + 4 g + e % 4, column 32 b + l32.
//
// bf16: two ds_read_b64_tr_b16.  Within each 16-lane group the instruction
// gives lane i element (i % 4) of the 8 bytes read by lane 4 k + i / 4, as
// its k-th value; so source lane j = 4 k + m reads tile row (base + k),
// columns 4 m .. 4 m + 3 of the group's 16 columns, and lane i receives
// column i of those 4 rows.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag trans_frag(const unsigned char* tile, int b,
                                                              int cc, int lane) {
  using L = Tile<T, D>;
  typename Elem<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const int q = lane >> 4, j = lane & 15;
    const int col = 32 * b + 16 * (q & 1) + 4 * (j & 3);
    const int row0 = 16 * cc + 4 * (q >> 1) + (j >> 2);
    const uint32_t o0 = L::off(row0, col >> 3) + ((col & 7) << 1);
    const uint32_t o1 = L::off(row0 + 8, col >> 3) + ((col & 7) << 1);
    lds_byte* t3 = as_lds(const_cast<unsigned char*>(tile));
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(t3 + o0));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(t3 + o1));
    const v8i16 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    f.v = __builtin_bit_cast(bf16x8, x);
  } else {
    const int l32 = lane & 31, g = lane >> 5;
    const int col = 32 * b + l32;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = 16 * cc + 4 * g + e;
      f.lo[e] = *reinterpret_cast<const float*>(tile + L::off(r0, col >> 2) + ((col & 3) << 2));
      f.hi[e] = *reinterpret_cast<const float*>(tile + L::off(r0 + 8, col >> 2) + ((col & 3) << 2));
    }
  }
  return f;
}

// Transposed operand (bf16) at precomputed offsets: p0/p1 address the two
// 4-row groups (see trans_frag).
__device__ __forceinline__ Elem<__bf16>::frag trans_frag_at(const unsigned char* p0,
                                                            const unsigned char* p1) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)as_lds(const_cast<unsigned char*>(p0)));
  const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)as_lds(const_cast<unsigned char*>(p1)));
  Elem<__bf16>::frag f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

// Kept tiles along one row (stride 1) or one column (stride = row length) of
// the 128 x 128 block mask, for tiles TILE wide (TILE divides 128).  The wave
// fetches the mask 64 blocks at a time, one byte per lane, and keeps the
// 64-bit ballot, so the tile loop touches global memory for the mask once
// per 64 blocks instead of once per tile.
template <int TILE>
struct KeptTiles {
  static_assert(kMaskBlock % TILE == 0, "tiles must divide the mask block");
  static constexpr int TPB = kMaskBlock / TILE;
  const uint8_t* p;
  size_t stride;
  int blocks;
  int base = -64;          // first block of the cached ballot
  uint64_t bits = 0;

  __device__ KeptTiles(const uint8_t* p_, size_t stride_, int blocks_)
      : p(p_), stride(stride_), blocks(blocks_) {}

  // First kept tile >= j; blocks * TPB (past every tile) when none is left.
  __device__ int next(int j, int lane) {
    const int b0 = j / TPB;
    for (int b = b0; b < blocks;) {
      const int chunk = b & ~63;
      if (chunk != base) {
        base = chunk;
        const int idx = chunk + lane;
        bits = __ballot(idx < blocks && p[(size_t)idx * stride] != 0);
      }
      const uint64_t m = bits >> (b - chunk);
      if (m) {
        b += __builtin_ctzll(m);
        return b == b0 ? j : b * TPB;
      }
      b = chunk + 64;
    }
    return blocks * TPB;
  }
};

// Waves per SIMD each kernel is compiled for (two waves let one wave's
// softmax arithmetic overlap the other's matrix work; the fp32 path at
// d = 128 needs the full register file of one wave).  bf16 at d = 64 fits a
// third wave (168 VGPRs) in the forward and in the dQ pass without dropout,
// except the plain non-causal forward, which would spill; a third
// work-group per compute unit also lets every block of a 96-head, 1K-row
// launch be resident at once.
template <typename T, int D, bool CAUSAL = true, bool MASKED = false, bool DROP = false>
struct Occupancy {
  static constexpr bool narrow = sizeof(T) == 2 && D == 64;
  static constexpr int fwd = narrow && (CAUSAL || MASKED || DROP) ? 3
                             : (sizeof(T) == 2 || D == 64)        ? 2
                                                                  : 1;
  static constexpr int dq = narrow && !DROP ? 3 : (sizeof(T) == 2 || D == 64) ? 2 : 1;
};

// ---------------------------------------------------------------------------
// Work-group -> (head, block) mapping.
//
// Blocks are handed to the 8 XCDs round-robin by work-group id, and each XCD
// has its own L2.  When the head count is a multiple of 8, head h is pinned to
// XCD h % 8 so all blocks of a head share one L2 (they re-read the same K/V or
// Q/dO tiles).  Under the causal mask, blocks are ordered by decreasing work
// (`heavy_is_last`: causal query blocks, the last has the most keys; else
// causal key blocks, the first has the most queries), so that work-groups
// dispatched as compute units free up take the longest blocks first.
//
// When every work-group of the launch is resident at once (`wgs_per_cu`
// work-groups per CU, 32 CUs per XCD), each CU's work is fixed at dispatch:
// consecutive work-groups of an XCD land on consecutive CUs, so in that
// order CU j would take blocks j, j + 32, j + 64, all heavy for small j and
// all light for large j.  There every second round of 32 is reversed, and
// each CU takes a heavy, a middle and a light block.
// ---------------------------------------------------------------------------
struct BlockCoord { int bh; int blk; };

__device__ __forceinline__ BlockCoord map_block(int wg, int nblk, int BH, bool causal,
                                                bool heavy_is_last, int wgs_per_cu = 0) {
  int rank, bh;
  if ((BH & 7) == 0) {
    const int xcd = wg & 7;
    int s = wg >> 3;
    const int hpx = BH >> 3;          // heads per XCD
    const int per = nblk * hpx;       // work-groups on this XCD
    if (causal && per <= 32 * wgs_per_cu && ((s >> 5) & 1)) {
      const int base = s & ~31;
      s = base + min(32, per - base) - 1 - (s & 31);
    }
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
