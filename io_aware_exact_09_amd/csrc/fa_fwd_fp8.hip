// fa_fwd_fp8.hip -- attention forward on FP8 (OCP E4M3) inputs for gfx950.
//
// FlashAttention-3 runs its forward in FP8 (the pages note this for FA3:
// aivaro.ru/en/answers/474, the list of versions; snula.amonoc.com/course/
// ru/week-13.html, the note on FA2 and FA3).  Here both products run on the
// gfx950 FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3
// operands, unit block scales, fp32 accumulation), which has twice the
// throughput of the bf16 one:
//
//   S^T = K_j Q_i^T       one MFMA per 64-wide d chunk and 32 keys
//   P~  = 2^(8 + S c_j - m), rounded to E4M3 (P~ <= 2^8.75 < 448)
//   O^T += V_j^T P~^T     one MFMA per 32-wide d block and 64 keys
//
// Inputs are quantized per block: Q and K carry one fp32 scale per 128-row
// block, V one per head; a tile's score coefficient is c_j = scale log2(e)
// sQ_i sK_j, and sV multiplies O at the end.  V arrives transposed
// ([B, H, d, N]), so the P V contraction reads consecutive bytes.  Work-group
// layout, online softmax, masking and tile walk follow fa_fwd.hip (S^T
// orientation: one query row per lane pair); the row sum uses the unrounded
// P~ so that LSE carries no FP8 rounding.
//
// Operand layouts.  For a contraction the instruction pairs item e of lane
// half g of A with item e of lane half g of B, 32 one-byte items per lane,
// so any assignment of contraction indices to (g, e) that both operands
// follow gives the product:
//   S^T: natural order, d = 64 t + 32 g + e (A from the K tile, B from Q);
//   P V: key = 32 h + 8 a + 4 g + x for item e = 16 h + 4 a + x -- the order
//        in which the S^T accumulators of the tile's two 32-key halves
//        (register 4a + x of half h) hold P~ -- so lane (d row i, g) of the
//        V^T tile needs the key dwords 2 m + g, m = 4 h + a.  The V^T tile
//        is therefore staged with each row's even key dwords first and its
//        odd ones second (dword-sized direct-to-LDS loads pick the source
//        dword per lane), and a lane reads its 32 bytes with two 16-byte
//        reads.
//
// Online softmax: the reference max m moves only when a row's tile max
// exceeds it by more than kLazy8 = 0.75 (log2 units), so P~ <= 2^8.75 stays
// below the E4M3 maximum (448) and most tiles skip the rescale of O; the key
// that set m keeps P~ = 2^8, so the row sum stays >= 2^8.

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kFp8Fmt = 0;          // E4M3 operand format of the f8f6f4 MFMA
constexpr int kUnitScale = 127;     // E8M0 block scale 2^0

__device__ __forceinline__ f32x16 mma_fp8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFp8Fmt, kFp8Fmt, 0,
                                                        kUnitScale, 0, kUnitScale);
}

// Four fp32 values -> four E4M3 bytes (round to nearest even) in one dword.
// The first conversion writes the low half over the bits of `a` (dead after
// this), which spares a register clear.
__device__ __forceinline__ int pack_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// K tile: 64 rows of D bytes, 16-byte chunks XOR-swizzled per row so that the
// 16 rows one ds_read_b128 serves at a time hit 16 different 16-byte slots of
// the 256-byte bank window (two rows per window at D = 128, four at D = 64).
template <int D>
struct KTile {
  static constexpr int RB = D;
  __device__ static constexpr int swz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  __device__ static constexpr uint32_t off(int r, int c) {
    return (uint32_t)(r * RB + ((c ^ swz(r)) << 4));
  }
};

// V^T tile: D rows (d index) of 64 key bytes.  Logical row layout: the 8
// even key dwords (keys 8 m .. 8 m + 3), then the 8 odd ones (8 m + 4 ..);
// its four 16-byte chunks are XOR-swizzled by (r / 4) % 4, so the 16 rows
// that one ds_read_b128 serves at a time hit 16 different slots of the
// 256-byte bank window.
struct VtTile {
  static constexpr int RB = 64;
  __device__ static constexpr int swz(int r) { return (r >> 2) & 3; }
  __device__ static constexpr uint32_t off(int r, int c) {
    return (uint32_t)(r * RB + ((c ^ swz(r)) << 4));
  }
  // Key dword of the global row held by LDS dword slot q (0 .. 15) of row r.
  __device__ static constexpr int key_dword(int r, int q) {
    const int lq = (((q >> 2) ^ swz(r)) << 2) | (q & 3);   // logical dword
    return lq < 8 ? 2 * lq : 2 * (lq - 8) + 1;
  }
};

}  // namespace

template <int D, bool CAUSAL, bool MASKED>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(3, 3)))
fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                  const uint8_t* __restrict__ Vt, const float* __restrict__ sQ,
                  const float* __restrict__ sK, const float* __restrict__ sV,
                  __bf16* __restrict__ O, float* __restrict__ LSE,
                  const uint8_t* __restrict__ mask, int BH, int N, int T_tiles,
                  float c /* score_coef(scale) */) {
  constexpr int BR = 128, BC = 64;
  constexpr int NT = D / 64;               // 64-wide d chunks (S^T MFMAs per 32 keys)
  constexpr int ND = D / 32;               // 32-wide d blocks of O^T
  constexpr int KB = BC * D;               // bytes of the K tile
  constexpr int VB = D * BC;               // bytes of the V^T tile
  constexpr float kShift = 8.0f;           // P~ = 2^(kShift + s c - m)
  constexpr float kLazy8 = 0.75f;          // P~ <= 2^(kShift + kLazy8) < 448

  __shared__ __attribute__((aligned(1024))) unsigned char lds0[KB + VB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[KB + VB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int nqb = (N + BR - 1) / BR;
  const BlockCoord bc = map_block(blockIdx.x, nqb, BH, CAUSAL, true);
  const int bh = bc.bh, q0 = bc.blk * BR;
  const size_t head = (size_t)bh * N * D;
  const uint8_t* Kh = K + head;
  const uint8_t* Vth = Vt + head;          // [D][N]
  const int qrow = q0 + 32 * w + l32;

  // Query fragments (B operand): Q[qrow][64 t + 32 g .. +31]; rows past N are zero.
  const rsrc_t rq = make_rsrc(Q + head, (uint32_t)N * D);
  i32x8 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t off = (uint32_t)qrow * D + 64 * t + 32 * g;
    const u32x4 a = buf_load16(rq, off), b = buf_load16(rq, off + 16);
    qf[t] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                  (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }
  bool negs;
  c = split_coef(c, negs);   // c = |scale| log2(e); Q negated when scale < 0
  if (negs) {              // E4M3: bit 7 of each code is its sign
#pragma unroll
    for (int t = 0; t < NT; ++t) qf[t] ^= (int)0x80808080u;
  }
  const int T = (N + kMaskBlock - 1) / kMaskBlock;
  const float cq = c * sQ[(size_t)bh * T + q0 / kMaskBlock];
  const float* sKh = sK + (size_t)bh * T;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  KeptTiles<BC> kept(MASKED ? mask + (size_t)(q0 / kMaskBlock) * T_tiles : nullptr, 1, T_tiles);
  auto next_kept = [&](int j) {
    if constexpr (MASKED) return kept.next(j, lane);
    return j;
  };

  // Direct-to-LDS staging: K rows kv0.. (rows past N read as zero) and the
  // 64-key column block kv0.. of every V^T row (bytes past the head read as
  // zero; within the head, columns past N hold the next row's first keys,
  // which meet P~ = 0).
  auto stage = [&](int j, auto buf) {
    const int kv0 = j * BC;
    unsigned char* base = pick(buf, lds0, lds1);
    const rsrc_t rk = make_rsrc(Kh + (size_t)kv0 * D, (uint32_t)(N - kv0) * D);
#pragma unroll
    for (int i = 0; i < KB / 1024 / 4; ++i) {
      const int blk = w + 4 * i;
      const int pos = blk * 1024 + lane * 16;
      const int r = pos / D, pc = (pos % D) >> 4;
      const uint32_t goff = (uint32_t)(r * D + ((pc ^ KTile<D>::swz(r)) << 4));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, as_lds(base + blk * 1024), 16, goff, 0, 0, 0);
    }
    const rsrc_t rv = make_rsrc(Vth + kv0, (uint32_t)((size_t)D * N - kv0));
#pragma unroll
    for (int i = 0; i < VB / 256 / 4; ++i) {   // one dword per lane, 256 bytes per load
      const int blk = w + 4 * i;
      const int pos = blk * 256 + lane * 4;
      const int r = pos / 64, q = (pos % 64) >> 2;
      const uint32_t goff = (uint32_t)r * (uint32_t)N + 4 * VtTile::key_dword(r, q);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, as_lds(base + KB + blk * 256), 4, goff, 0,
                                               0, 0);
    }
  };

  // Per-lane LDS offsets (computed once, so every read names one buffer).
  uint32_t koff[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int x = 0; x < 2; ++x) koff[t][x] = KTile<D>::off(l32, 4 * t + 2 * g + x);
  uint32_t voff[2];          // row l32, logical chunks 2 g and 2 g + 1 (dwords 2 m + g)
#pragma unroll
  for (int x = 0; x < 2; ++x) voff[x] = VtTile::off(l32, 2 * g + x);

  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) oacc[b] = f32x16{};
  float m_run = neg_inf();   // running max of S*c_j (log2 domain)
  float l_run = 0.f;

  auto tile = [&](auto buf_tag, int kv0) {
    const unsigned char* sKt = pick(buf_tag, lds0, lds1);
    const unsigned char* sVt = sKt + KB;
    // (kept > 0 so that a masked score, -inf, always maps to P~ = 0)
    const float cj = fmaxf(cq * sKh[kv0 / kMaskBlock], 1.17549435e-38f);

    // ---- S^T = K_j Q^T (two 32-key halves) -------------------------------
    f32x16 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x8 ak[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sKt + koff[t][0] + 32 * h * D);
        const u32x4 b = *reinterpret_cast<const u32x4*>(sKt + koff[t][1] + 32 * h * D);
        ak[t] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                      (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
      }
      sched_fence();
      s[h] = f32x16{};
#pragma unroll
      for (int t = 0; t < NT; ++t) s[h] = mma_fp8(ak[t], qf[t], s[h]);
    }

    // ---- mask (diagonal / tail tiles) ---------------------------------------
    const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > q0 + 32 * w);
    if (need_mask) {
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - kv0 - 4 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * h + 8 * (r >> 2) + (r & 3) >= lim) s[h][r] = neg_inf();
    }

    // ---- online softmax (exact running max) -----------------------------------
    float mx = neg_inf();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[h][r]);
    const float m_tile = max_xor32(mx) * cj;
    const bool grow = m_tile > m_run + kLazy8;
    if (__any(grow)) {   // wave-uniform branch
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;   // 0 at first
#pragma unroll
      for (int b = 0; b < ND; ++b) oacc[b] *= alpha;
      l_run *= alpha;
      m_run = grow ? m_tile : m_run;
    }
    const float m_use = (m_run == neg_inf() ? 0.f : m_run) - kShift;
    float psum[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[h][r] = __builtin_amdgcn_exp2f(fmaf(s[h][r], cj, -m_use));
        psum[r & 3] = (h == 0 && r < 4) ? s[h][r] : psum[r & 3] + s[h][r];
      }
    l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

    // ---- O^T += V^T P~^T ------------------------------------------------------
    i32x8 pf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        pf[4 * h + a] = pack_fp8(s[h][4 * a], s[h][4 * a + 1], s[h][4 * a + 2], s[h][4 * a + 3]);
#pragma unroll
    for (int b = 0; b < ND; ++b) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(sVt + voff[0] + 32 * b * VtTile::RB);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(sVt + voff[1] + 32 * b * VtTile::RB);
      const i32x8 av = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      oacc[b] = mma_fp8(av, pf, oacc[b]);
    }
  };

  // One loop body with a run-time buffer index: unrolled over the two
  // buffers, the compiler gave each copy its own registers for the O
  // accumulators and copied all 64 of them before every P V product; one
  // body also fits three waves per SIMD (~162 VGPRs at d = 128).
  int j = next_kept(0);
  auto step = [&](auto buf_tag) {
    wait_global_loads();
    __syncthreads();
    const int jn = next_kept(j + 1);
    if (jn < ntiles) stage(jn, other(buf_tag));
    tile(buf_tag, j * BC);
    j = jn;
  };
  if (j < ntiles) stage(j, IntTag<0>{});
  int buf = 0;
  while (j < ntiles) {
    step(buf);
    buf ^= 1;
  }

  // ---- epilogue ------------------------------------------------------------------
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot != 0.f ? sV[bh] / l_tot : 0.f;
  if (qrow < N) {
    __bf16* Orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        Elem<__bf16>::store4(Orow + 32 * b + 8 * a + 4 * g, oacc[b][4 * a] * inv,
                             oacc[b][4 * a + 1] * inv, oacc[b][4 * a + 2] * inv,
                             oacc[b][4 * a + 3] * inv);
    if (g == 0)
      LSE[(size_t)bh * N + qrow] =
          l_tot != 0.f ? (m_run - kShift + __builtin_amdgcn_logf(l_tot)) * kLn2 : neg_inf();
  }
}

template <int D, bool CAUSAL, bool MASKED>
static hipError_t launch_fp8_t(const Fp8FwdArgs& a) {
  const int nqb = (a.N + 127) / 128;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, MASKED>), dim3(nqb * a.BH), dim3(kThreads), 0,
                     a.stream, a.q, a.k, a.vt, a.sq, a.sk, a.sv, static_cast<__bf16*>(a.o),
                     a.lse, a.mask, a.BH, a.N, a.T, score_coef(a.scale));
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fp8_d(const Fp8FwdArgs& a) {
  const bool mk = a.mask != nullptr;
  if (a.causal) return mk ? launch_fp8_t<D, true, true>(a) : launch_fp8_t<D, true, false>(a);
  return mk ? launch_fp8_t<D, false, true>(a) : launch_fp8_t<D, false, false>(a);
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a) {
  return a.d == 64 ? launch_fp8_d<64>(a) : launch_fp8_d<128>(a);
}

}  // namespace fa
