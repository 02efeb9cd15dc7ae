// fa_fwd.hip -- tiled exact-attention forward for gfx950.
//
// One work-group (4 waves) owns 128 query rows of one (batch, head); wave w
// owns rows 32w..32w+31 and each lane-pair (l32, l32+32) owns one query row.
// The work-group walks the kept key/value tiles of BC keys:
//
//   S^T = K_j Q_i^T      (MFMA; K from LDS, Q held in registers)
//   mask causal / tail / nothing, running max m, P~ = 2^(S*c - m),
//   rescale l and O by 2^(m_old - m_new) when the max moved,
//   O^T += V_j^T P~^T    (MFMA; V stored transposed in LDS, P~ from registers)
//
// and writes O = O_acc / l and LSE = (m + log2 l) ln 2 at the end.  K and V
// tiles go straight from global memory into double-buffered LDS (one barrier
// per tile); V^T operands are read with the transposing LDS load.  This is
// the per-block update of the FlashAttention reading guide (xyznot.com/tr/
// paper/2205.14135, "Yöntem" steps 1-4, with the two-part rule of "Artımsal
// Softmax Takibi") in its deferred-normalisation form (snula.amonoc.com/
// course/ru/week-13.html, Step 2: keep (m, d, o) per query block, scale the
// old d and o by e^(m_old - m_new) on a new maximum).  Scores live in the
// log2 domain: c = |scale| * log2(e), so every exponential is one v_exp_f32
// (a negative scale flips the sign of Q in registers instead; score_coef).
// A row whose running max is still -inf uses 0 as the subtrahend, so no
// 2^(-inf - (-inf)) is formed (week-13 page, "Типичные ошибки").
//
// Computing S^T (keys as the MFMA rows) puts one query row in each lane:
// the row max needs one cross-lane exchange (lane l with l^32), the row sum
// stays per lane until the end, and the C registers of S^T are already the B
// operand of the P V product (C-shaped contraction order, see fa_common.hpp).

#include "fa_common.hpp"
#include "fa_launch.hpp"
#include "fa_rows.hpp"

namespace fa {

template <typename T>
struct FwdCfg {
  static constexpr int BR = 128;                          // query rows per work-group
  static constexpr int BC = sizeof(T) == 2 ? 64 : 32;     // keys per tile
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Occupancy<T, D, CAUSAL, MASKED, DROP>::fwd,
                                   Occupancy<T, D, CAUSAL, MASKED, DROP>::fwd)))
fa_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              T* __restrict__ O, float* __restrict__ LSE, const uint8_t* __restrict__ mask,
              int BH, int kv_group, int N, int T_tiles, float c /* score_coef(scale) */,
              DropParams dp, int fsplit, float* __restrict__ opart, float* __restrict__ lpart) {
  using E = Elem<T>;
  using frag = typename E::frag;
  using Cfg = FwdCfg<T>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC;
  constexpr int NH = BC / 32;              // 32-key halves per tile
  constexpr int NT = D / 16;               // 16-wide d chunks
  constexpr int ND = D / 32;               // 32-wide d blocks of O^T
  constexpr uint32_t RB = Tile<T, D>::RB;  // bytes per row
  constexpr int TB = BC * RB;              // bytes per K or V tile

  // Two buffers of [K, V] tiles (distinct arrays, see pick()).
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[2 * TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[2 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int nqb = (N + BR - 1) / BR;
  // fsplit > 1: runs of key tiles per query block, as in the ping-pong kernel.
  const BlockCoord bc = map_block(blockIdx.x, nqb, BH * fsplit, CAUSAL, true,
                                  Occupancy<T, D, CAUSAL, MASKED, DROP>::fwd);
  const int bh = bc.bh / fsplit, run = bc.bh - bh * fsplit, q0 = bc.blk * BR;
  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = (size_t)(bh / kv_group) * N * D;    // shared key/value head
  const T* Kh = K + kvhead;
  const T* Vh = V + kvhead;
  const int qrow = q0 + 32 * w + l32;
  // Dropout: this lane's 16-bit half of a Philox word is the low one for an
  // even query row (w & 0xFFFF >= T), the high one for an odd row
  // (w >= T << 16).
  const int odd = l32 & 1;
  const uint32_t hmask = odd ? 0xFFFFFFFFu : 0xFFFFu;
  const uint32_t hthr = odd ? dp.thresh << 16 : dp.thresh;

  // Query fragments (B operand, natural order): Q[qrow][16t + 8g .. +7];
  // rows past N read as zero.
  const rsrc_t rq = make_rsrc(Q + head, (uint32_t)N * RB);
  frag qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qf[t] = gload_frag<T>(rq, (uint32_t)qrow * RB + (16 * t + 8 * g) * sizeof(T));
  bool negs;
  c = split_coef(c, negs);   // from here on c = |scale| log2(e) > 0
  if (negs) {
#pragma unroll
    for (int t = 0; t < NT; ++t) negate(qf[t]);
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles_all = (kv_end + BC - 1) / BC;
  const int jbeg = (int)((long long)run * ntiles_all / fsplit);
  const int ntiles = (int)((long long)(run + 1) * ntiles_all / fsplit);   // end of this run
  KeptTiles<BC> kept(MASKED ? mask + (size_t)(q0 / kMaskBlock) * T_tiles : nullptr, 1, T_tiles);
  auto next_kept = [&](int j) {
    if constexpr (MASKED) return kept.next(j, lane);
    return j;
  };
  auto stage = [&](int j, auto buf) {
    const int kv0 = j * BC;
    const uint32_t left = (uint32_t)(N - kv0) * RB;
    unsigned char* base = pick(buf, lds0, lds1);
    stage_tile<T, D, BC>(make_rsrc(Kh + (size_t)kv0 * D, left), base, w, lane);
    stage_tile<T, D, BC>(make_rsrc(Vh + (size_t)kv0 * D, left), base + TB, w, lane);
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) oacc[b] = f32x16{};
  float m_run = neg_inf();   // running max of S*c (log2 domain), same in both lane halves
  float l_run = 0.f;         // this lane's partial row sum

  // bf16, d = 64: compile-time LDS buffers (loop unrolled by two) and
  // precomputed operand offsets.  d = 128 keeps a runtime buffer index: at
  // two waves per SIMD its registers have no room for either, and measured
  // slower with them.
  constexpr bool kCt = sizeof(T) == 2 && D == 64;
  LaneOffsets<T, D> lo;
  if constexpr (kCt) lo.init(lane);

  // One kept tile in LDS buffer `buf` (an IntTag where compile-time).
  // `first`: no earlier kept tile, so O and l are still zero and need no
  // rescaling.
  auto tile = [&](auto buf_tag, int kv0, bool first) {
    const unsigned char* sK = pick(buf_tag, lds0, lds1);
    const unsigned char* sV = sK + TB;

    // ---- S^T = K_j Q^T -------------------------------------------------
    // Operands are read into registers a batch ahead of their MFMAs so the
    // LDS latency overlaps the matrix work.
    f32x16 s[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      frag ak[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (kCt) ak[t] = row_frag_at<T>(sK + lo.row[t] + 32 * h * RB);
        else ak[t] = row_frag<T, D>(sK, 32 * h + l32, t, g);
      }
      sched_fence();
      s[h] = f32x16{};
#pragma unroll
      for (int t = 0; t < NT; ++t) s[h] = E::mma(ak[t], qf[t], s[h]);
    }

    // ---- mask (diagonal / tail tiles only) -------------------------------
    // Register r of half h holds key kv0 + 4g + off, off = 32h + 8(r/4) + r%4;
    // it is kept iff off < lim.
    const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > q0 + 32 * w);
    if (need_mask) {
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - kv0 - 4 * g;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * h + 8 * (r >> 2) + (r & 3) >= lim) s[h][r] = neg_inf();
    }

    // ---- online softmax ----------------------------------------------------
    // c > 0, so a masked score gives 2^(-inf) = 0 and c times the row max of
    // the kept scores is the max of S*c.  The reference m_run moves only when
    // a row's tile max exceeds it by more than kLazy (log2 units): P stays
    // <= 2^kLazy, numerator and denominator share the same reference, and the
    // O/l rescale (one multiply per accumulator) is skipped on most tiles.
    float mx = neg_inf();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[h][r]);
    const float m_tile = max_xor32(mx) * c;
    const bool grow = m_tile > m_run + kLazy;          // always true on a row's first kept key
    if (__any(grow)) {
      if (!first) {
        // alpha = 1 on rows whose reference stays (also rows with nothing
        // kept yet, whose m_run and m_tile are both -inf); 2^(-inf) = 0 on a
        // row's first kept keys.
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
#pragma unroll
        for (int b = 0; b < ND; ++b) oacc[b] *= alpha;
        l_run *= alpha;
      }
      m_run = grow ? m_tile : m_run;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    // Row sum in fp32 from the unrounded probabilities (the log-sum-exp the
    // backward relies on must not carry the bf16 rounding of P).
    float psum[NH][4] = {};
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[h][r] = __builtin_amdgcn_exp2f(fmaf(s[h][r], c, -m_use));
        psum[h][r & 3] += s[h][r];
      }
#pragma unroll
    for (int h = 0; h < NH; ++h) l_run += (psum[h][0] + psum[h][1]) + (psum[h][2] + psum[h][3]);

    // ---- dropout: zero the dropped probabilities (the row sum above keeps
    // them: softmax statistics are those of the undropped P; the 1/(1-p) of
    // the kept ones is applied to O at the end).  Registers 4a..4a+3 of half h
    // are keys kv0 + 32h + 8a + 4g + x.  A Philox call covers four keys of a
    // query pair (2y, 2y + 1), i.e. of lanes l32 and l32 ^ 1: the even lane
    // draws the calls of groups a = 0, 1, the odd lane those of a = 2, 3, and
    // both read each group's words from the lane that drew them (DPP quad
    // broadcasts), each keeping its own 16-bit half.
    if constexpr (DROP) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {   // groups c2 (even lane's call), 2 + c2 (odd lane's)
          const Philox4 z = philox4x32_10((uint32_t)((kv0 + 32 * h + 8 * (2 * odd + c2)) >> 2) + g,
                                          (uint32_t)qrow >> 1, (uint32_t)bh, 0u, dp.key0, dp.key1);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t we = (uint32_t)__builtin_amdgcn_mov_dpp((int)z.w[x], 0xA0, 0xF, 0xF, true);
            const uint32_t wo = (uint32_t)__builtin_amdgcn_mov_dpp((int)z.w[x], 0xF5, 0xF, 0xF, true);
            if ((we & hmask) < hthr) s[h][4 * c2 + x] = 0.f;
            if ((wo & hmask) < hthr) s[h][4 * (2 + c2) + x] = 0.f;
          }
        }
    }

    // ---- O^T += V_j^T P^T ----------------------------------------------------
    frag pf[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      pf[h][0] = E::from_c(s[h], 0);
      pf[h][1] = E::from_c(s[h], 1);
    }
#pragma unroll
    for (int b = 0; b < ND; ++b) {
      frag av[2 * NH];
#pragma unroll
      for (int cc = 0; cc < 2 * NH; ++cc) {
        if constexpr (kCt)
          av[cc] = trans_frag_at(sV + lo.tr[b][0] + 16 * cc * RB, sV + lo.tr[b][1] + 16 * cc * RB);
        else
          av[cc] = trans_frag<T, D>(sV, b, cc, lane);
      }
      sched_fence();
#pragma unroll
      for (int cc = 0; cc < 2 * NH; ++cc) oacc[b] = E::mma(av[cc], pf[cc >> 1][cc & 1], oacc[b]);
    }
  };

  // Wait for kept tile j (buffer buf_tag), prefetch the next kept tile into
  // the other buffer, then run the tile.
  int j = next_kept(jbeg);
  bool first = true;
  auto step = [&](auto buf_tag) {
    wait_global_loads();             // this wave's part of tile j has landed
    __syncthreads();                 // all of tile j is in LDS; the other buffer is free
    const int jn = next_kept(j + 1);
    if (jn < ntiles) stage(jn, other(buf_tag));   // in flight while this tile is computed
    tile(buf_tag, j * BC, first);
    first = false;
    j = jn;
  };
  if (j < ntiles) stage(j, IntTag<0>{});
  if constexpr (kCt) {
    while (j < ntiles) {   // two tiles per trip: the buffer index is compile-time
      step(IntTag<0>{});
      if (j >= ntiles) break;
      step(IntTag<1>{});
    }
  } else {
    for (int buf = 0; j < ntiles; buf ^= 1) step(buf);
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot != 0.f ? (DROP ? dp.inv_keep : 1.0f) / l_tot : 0.f;
  const float lse = l_tot != 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : neg_inf();
  if (fsplit > 1) {
    if (qrow < N) {
      const size_t r = ((size_t)run * BH + bh) * N + qrow;
      if (g == 0) lpart[r] = lse;
      float* po = opart + r * D;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<f32x4*>(po + 32 * b + 8 * a + 4 * g) =
              f32x4{oacc[b][4 * a], oacc[b][4 * a + 1], oacc[b][4 * a + 2],
                    oacc[b][4 * a + 3]} * inv;
    }
    return;
  }
  if (qrow < N && g == 0) LSE[(size_t)bh * N + qrow] = lse;
  if constexpr (sizeof(T) == 2) {
    // O through LDS (fa_rows.hpp; padded rows would not fit).
    static_assert(BR * D * (int)sizeof(T) <= 2 * TB, "O rows must fit a staging array");
    __syncthreads();                                  // every wave is done with the tiles
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        put_row4<T, D, false>(lds0, 32 * w + l32, 32 * b + 8 * a + 4 * g, oacc[b][4 * a] * inv,
                              oacc[b][4 * a + 1] * inv, oacc[b][4 * a + 2] * inv,
                              oacc[b][4 * a + 3] * inv);
    __syncthreads();
    write_rows<T, D, false, BR, kThreads>(lds0, O + head + (size_t)q0 * D, N - q0, tid);
  } else if (qrow < N) {
    T* Orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        E::store4(Orow + 32 * b + 8 * a + 4 * g, oacc[b][4 * a] * inv, oacc[b][4 * a + 1] * inv,
                  oacc[b][4 * a + 2] * inv, oacc[b][4 * a + 3] * inv);
  }
}

template <typename T, int D>
static hipError_t launch_fwd_combine(const FwdArgs& a);

template <typename T, int D, bool CAUSAL, bool MASKED>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  const int nqb = (a.N + FwdCfg<T>::BR - 1) / FwdCfg<T>::BR;
  const dim3 grid(nqb * a.BH * a.fsplit), block(kThreads);
  const DropParams dp{a.drop.key0, a.drop.key1, a.drop.thresh, a.drop.inv_keep};
  if (a.drop.on)
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, MASKED, true>), grid, block, 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, a.mask, a.BH,
                       a.G, a.N, a.T, score_coef(a.scale), dp, a.fsplit, a.opart, a.lpart);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, MASKED, false>), grid, block, 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, a.mask, a.BH,
                       a.G, a.N, a.T, score_coef(a.scale), dp, a.fsplit, a.opart, a.lpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.fsplit == 1) return e;
  return launch_fwd_combine<T, D>(a);
}

// ---------------------------------------------------------------------------
// Ping-pong forward: bf16 without a block mask.
//
// Eight waves, two per SIMD.  Group G = w / 4 owns query rows q0 + 128 G ..
// q0 + 128 G + 127 (wave w % 4 owns 32 of them, laid out as above), and both
// groups walk the same K/V tiles, kept in a ring of three LDS slots.  Time is
// cut into phases by work-group barriers.  In each phase one group runs its
// matrix work (S^T of tile t, and O^T += V^T P^T of tile t - 1) while the
// other runs the softmax of its latest scores on the VALU; the roles swap
// every phase, so each SIMD has one wave feeding the matrix cores while the
// other does the exponentials.  Step s (phases 2s and 2s+1):
//   group 0:  matrix(s)     | softmax(s)
//   group 1:  softmax(s-1)  | matrix(s)
// At the start of step s every wave issues its part of the loads of tile s+1
// into slot (s+1) % 3, whose previous tile (s-2) was last read in step s-1,
// and waits for them at the end of the step, before the barrier after which
// tile s+1 is first read.  The loop is unrolled by three steps so the slots
// are compile-time choices of three distinct arrays (see pick()).
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(2 * kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_pp_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                 T* __restrict__ O, float* __restrict__ LSE, int BH, int kv_group, int N,
                 float c /* score_coef(scale) */, int fsplit, float* __restrict__ opart,
                 float* __restrict__ lpart) {
  static_assert(sizeof(T) == 2, "bf16 only");
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int BR = 256, BC = 64;
  constexpr int NH = BC / 32, NT = D / 16, ND = D / 32;
  constexpr uint32_t RB = Tile<T, D>::RB;
  constexpr int TB = BC * RB;              // bytes per K or V tile

  __shared__ __attribute__((aligned(1024))) unsigned char slot0[2 * TB];   // [K, V]
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[2 * TB];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[2 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int G = w >> 2, wg = w & 3;
  const int nqb = (N + BR - 1) / BR;
  // With fsplit > 1 each query block's key tiles are cut into fsplit runs
  // of equal length, one per work-group (the runs of one block count as
  // separate heads in the block order); a run writes its normalised O and
  // its LSE in fp32 (opart [fsplit][BH * N][D], lpart [fsplit][BH * N]) and a
  // combine kernel merges the runs.
  const BlockCoord bc = map_block(blockIdx.x, nqb, BH * fsplit, CAUSAL, true);
  const int bh = bc.bh / fsplit, run = bc.bh - bh * fsplit, q0 = bc.blk * BR;
  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = (size_t)(bh / kv_group) * N * D;    // shared key/value head
  const T* Kh = K + kvhead;
  const T* Vh = V + kvhead;
  const int row0 = q0 + 128 * G + 32 * wg;     // this wave's first row
  const int qrow = row0 + l32;

  const rsrc_t rq = make_rsrc(Q + head, (uint32_t)N * RB);
  frag qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qf[t] = gload_frag<T>(rq, (uint32_t)qrow * RB + (16 * t + 8 * g) * sizeof(T));
  bool negs;
  c = split_coef(c, negs);   // from here on c = |scale| log2(e) > 0
  if (negs) {
#pragma unroll
    for (int t = 0; t < NT; ++t) negate(qf[t]);
  }

  // Tiles of the work-group's run [tb, tb + ntiles), and the end of this
  // wave's group's tiles within it (causal: the first group's rows end 128
  // keys earlier); the walk below counts tiles from tb.
  const int ntiles_all = ((CAUSAL ? min(N, q0 + BR) : N) + BC - 1) / BC;
  const int tb = (int)((long long)run * ntiles_all / fsplit);
  const int ntiles = (int)((long long)(run + 1) * ntiles_all / fsplit) - tb;
  const int gtiles = max(0, min(((CAUSAL ? min(N, q0 + 128 * (G + 1)) : N) + BC - 1) / BC,
                                tb + ntiles) - tb);

  auto stage = [&](int t, auto sl) {
    const int kv0 = (tb + t) * BC;
    const uint32_t left = (uint32_t)(N - kv0) * RB;
    unsigned char* base = pick3(sl, slot0, slot1, slot2);
    stage_tile<T, D, BC, 8>(make_rsrc(Kh + (size_t)kv0 * D, left), base, w, lane);
    stage_tile<T, D, BC, 8>(make_rsrc(Vh + (size_t)kv0 * D, left), base + TB, w, lane);
  };

  LaneOffsets<T, D> lo;
  lo.init(lane);
  f32x16 oacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) oacc[b] = f32x16{};
  f32x16 sc[NH];             // scores of the tile between its matrix and softmax phases
  frag pf[NH][2];            // probabilities of the tile between its softmax and P V
  float m_run = neg_inf();   // running reference max of S*c (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum

  // V^T operands of the tile whose P was produced last: blocks 0 .. NBP-1
  // are read during the softmax phase, so the next matrix phase starts on
  // MFMAs instead of LDS latency; the rest are read behind those MFMAs.
  constexpr int NBP = ND / 2;
  frag vpre[NBP][2 * NH];
  auto read_v = [&](auto vs) {
    const unsigned char* sV = pick3(vs, slot0, slot1, slot2) + TB;
#pragma unroll
    for (int b = 0; b < NBP; ++b)
#pragma unroll
      for (int cc = 0; cc < 2 * NH; ++cc)
        vpre[b][cc] =
            trans_frag_at(sV + lo.tr[b][0] + 16 * cc * RB, sV + lo.tr[b][1] + 16 * cc * RB);
  };

  // Matrix phase of step s: O^T += V^T P^T of tile s - 1 (from slot VS),
  // then S^T of tile s (from slot KS); each batch of LDS operands is read
  // in full before its MFMAs.
  auto matrix = [&](auto ks, auto vs, int s) {
    const unsigned char* sK = pick3(ks, slot0, slot1, slot2);
    const unsigned char* sV = pick3(vs, slot0, slot1, slot2) + TB;
    if (s >= 1 && s - 1 < gtiles) {
      frag vr[ND - NBP][2 * NH];
#pragma unroll
      for (int b = NBP; b < ND; ++b)
#pragma unroll
        for (int cc = 0; cc < 2 * NH; ++cc)
          vr[b - NBP][cc] =
              trans_frag_at(sV + lo.tr[b][0] + 16 * cc * RB, sV + lo.tr[b][1] + 16 * cc * RB);
      sched_fence();
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int cc = 0; cc < 2 * NH; ++cc)
          oacc[b] = E::mma(b < NBP ? vpre[b][cc] : vr[b - NBP][cc], pf[cc >> 1][cc & 1], oacc[b]);
    }
    if (s < gtiles) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        frag ak[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) ak[t] = row_frag_at<T>(sK + lo.row[t] + 32 * h * RB);
        sched_fence();   // all reads of the batch first, then its MFMA chain
        sc[h] = f32x16{};
#pragma unroll
        for (int t = 0; t < NT; ++t) sc[h] = E::mma(ak[t], qf[t], sc[h]);
      }
    }
  };

  // Softmax phase for tile t: mask, lazy reference max, O/l rescale, P.
  // Register r of half h holds key kv0 + 4g + 32h + 8(r/4) + r%4.
  auto softmax = [&](int t, auto vs) {
    if (t < 0 || t >= gtiles) return;
    read_v(vs);
    const int kv0 = (tb + t) * BC;
    if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > row0)) {
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - kv0 - 4 * g;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * h + 8 * (r >> 2) + (r & 3) >= lim) sc[h][r] = neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[h][r]);
    const float m_tile = max_xor32(mx) * c;
    const bool grow = m_tile > m_run + kLazy;
    if (__any(grow)) {
      if (t > 0) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
#pragma unroll
        for (int b = 0; b < ND; ++b) oacc[b] *= alpha;
        l_run *= alpha;
      }
      m_run = grow ? m_tile : m_run;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    // The four partial sums of a half start from its first four terms: an
    // addition to a zero start is not folded (it would turn -0 into +0), and
    // the probabilities are never -0, so the sums are the same (1% off this
    // kernel's time; the d = 64 kernel above measured slower with it).
    float psum[NH][4];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[h][r] = __builtin_amdgcn_exp2f(fmaf(sc[h][r], c, -m_use));
        psum[h][r & 3] = r < 4 ? sc[h][r] : psum[h][r & 3] + sc[h][r];
      }
      pf[h][0] = E::from_c(sc[h], 0);
      pf[h][1] = E::from_c(sc[h], 1);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) l_run += (psum[h][0] + psum[h][1]) + (psum[h][2] + psum[h][3]);
  };

  // Step s with slot of tile s = KS (compile-time); the softmax phase of tile
  // t also reads the V operands of tile t, so it takes that tile's slot.
  auto step = [&](auto ks, int s) {
    constexpr int KS = decltype(ks)::value;
    constexpr IntTag<(KS + 2) % 3> vs{};    // slot of tile s - 1
    constexpr IntTag<(KS + 1) % 3> ns{};    // slot of tile s + 1
    if (s + 1 < ntiles) stage(s + 1, ns);
    if (G == 0) matrix(ks, vs, s); else softmax(s - 1, vs);
    // Phase boundary only: no data changes hands here, so a bare barrier
    // (__syncthreads would first wait for the tile loads just issued).
    __builtin_amdgcn_s_barrier();
    if (G == 0) softmax(s, ks); else matrix(ks, vs, s);
    wait_global_loads();
    __syncthreads();
  };

  if (ntiles > 0) stage(0, IntTag<0>{});
  wait_global_loads();
  __syncthreads();
  for (int s = 0; s <= ntiles;) {
    step(IntTag<0>{}, s++);
    if (s > ntiles) break;
    step(IntTag<1>{}, s++);
    if (s > ntiles) break;
    step(IntTag<2>{}, s++);
  }

  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot != 0.f ? 1.0f / l_tot : 0.f;
  const float lse = l_tot != 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : neg_inf();
  if (fsplit > 1) {
    if (qrow < N) {
      const size_t r = ((size_t)run * BH + bh) * N + qrow;
      if (g == 0) lpart[r] = lse;
      float* po = opart + r * D;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<f32x4*>(po + 32 * b + 8 * a + 4 * g) =
              f32x4{oacc[b][4 * a], oacc[b][4 * a + 1], oacc[b][4 * a + 2],
                    oacc[b][4 * a + 3]} * inv;
    }
    return;
  }
  if (qrow < N && g == 0) LSE[(size_t)bh * N + qrow] = lse;
  // O through LDS (fa_rows.hpp, unpadded): group G's 128 rows in slot G.
  static_assert(128 * D * (int)sizeof(T) <= 2 * TB, "O rows must fit a ring slot");
  __syncthreads();                                    // every wave is done with the ring
  unsigned char* so = G == 0 ? slot0 : slot1;
#pragma unroll
  for (int b = 0; b < ND; ++b)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      put_row4<T, D, false>(so, 32 * wg + l32, 32 * b + 8 * a + 4 * g, oacc[b][4 * a] * inv,
                            oacc[b][4 * a + 1] * inv, oacc[b][4 * a + 2] * inv,
                            oacc[b][4 * a + 3] * inv);
  __syncthreads();
  const int g0 = q0 + 128 * G;
  write_rows<T, D, false, 128, kThreads>(so, O + head + (size_t)g0 * D, N - g0,
                                         tid & (kThreads - 1));
}

// Merge of the runs of a split forward, per row, in run order: with M the
// largest run LSE and w_r = e^(LSE_r - M), LSE = M + ln sum_r w_r and
// O = sum_r w_r O_r / sum_r w_r (the two-part merge rule of the reading
// guide's "Artımsal Softmax Takibi", each run's statistics carried as its
// LSE).  32 lanes per row (4 columns each at d = 128, 2 at d = 64).
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
fa_fwd_combine_kernel(const float* __restrict__ opart, const float* __restrict__ lpart,
                      T* __restrict__ O, float* __restrict__ LSE, int rows, int fsplit) {
  constexpr int CPL = D / 32;              // columns per lane
  const int row = blockIdx.x * (kThreads / 32) + (threadIdx.x >> 5);
  const int c0 = (threadIdx.x & 31) * CPL;
  if (row >= rows) return;
  float M = neg_inf();
  for (int r = 0; r < fsplit; ++r) M = fmaxf(M, lpart[(size_t)r * rows + row]);
  float acc[CPL] = {};
  float wsum = 0.f;
  if (M != neg_inf()) {
    for (int r = 0; r < fsplit; ++r) {
      const float lr = lpart[(size_t)r * rows + row];
      const float wr = __builtin_amdgcn_exp2f((lr - M) * kLog2e);
      const float* po = opart + ((size_t)r * rows + row) * D + c0;
      wsum += wr;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = fmaf(wr, po[e], acc[e]);
    }
  }
  const float inv = wsum != 0.f ? 1.0f / wsum : 0.f;
  T* out = O + (size_t)row * D + c0;
#pragma unroll
  for (int e = 0; e < CPL; e += 2) {
    out[e] = (T)(acc[e] * inv);
    out[e + 1] = (T)(acc[e + 1] * inv);
  }
  if ((threadIdx.x & 31) == 0)
    LSE[row] = wsum != 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : neg_inf();
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_pp(const FwdArgs& a) {
  const int nqb = (a.N + 255) / 256;
  hipLaunchKernelGGL((fa_fwd_pp_kernel<T, D, CAUSAL>), dim3(nqb * a.BH * a.fsplit),
                     dim3(2 * kThreads), 0, a.stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<T*>(a.o), a.lse, a.BH, a.G, a.N, score_coef(a.scale), a.fsplit,
                     a.opart, a.lpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.fsplit == 1) return e;
  return launch_fwd_combine<T, D>(a);
}

template <typename T, int D>
static hipError_t launch_fwd_combine(const FwdArgs& a) {
  const int rows = a.BH * a.N;
  hipLaunchKernelGGL((fa_fwd_combine_kernel<T, D>), dim3((rows + kThreads / 32 - 1) / (kThreads / 32)),
                     dim3(kThreads), 0, a.stream, a.opart, a.lpart, static_cast<T*>(a.o), a.lse,
                     rows, a.fsplit);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  if (a.causal) return a.mask ? launch_fwd_t<T, D, true, true>(a) : launch_fwd_t<T, D, true, false>(a);
  return a.mask ? launch_fwd_t<T, D, false, true>(a) : launch_fwd_t<T, D, false, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  // d = 128 without a block mask: the ping-pong kernel.  (At d = 64 the
  // four-wave kernel runs three waves per SIMD and measured faster.)
  if (a.bf16 && !a.mask && a.d == 128 && !a.drop.on)
    return a.causal ? launch_fwd_pp<__bf16, 128, true>(a) : launch_fwd_pp<__bf16, 128, false>(a);
  if (a.bf16) return a.d == 64 ? launch_fwd_d<__bf16, 64>(a) : launch_fwd_d<__bf16, 128>(a);
  return a.d == 64 ? launch_fwd_d<float, 64>(a) : launch_fwd_d<float, 128>(a);
}

}  // namespace fa
