// fa_bwd.hip -- exact-attention training backward for gfx950.
//
// The backward never reads a stored P: it recomputes S and P tile by tile
// from Q, K and the per-row log-sum-exp saved by the forward, as the
// recomputation scheme of the aivaro.ru answer on FlashAttention training
// (§3 and §3.1) and the week-13 course page (snula.amonoc.com/course/ru/
// week-13.html, Step 2) describe.  The gradients follow the chain rule
// through softmax (the closed form that the page's garbled dQ/dK stand for):
//
//   D_i = sum_k dO_ik O_ik
//   P_ij = 2^(S_ij * c - LSE_i * log2 e)      (c = scale * log2 e, of either
//                                              sign: the backward masks P by
//                                              a select after the exponential,
//                                              so it needs no c > 0)
//   dV_j = sum_i P_ij dO_i,   dP_ij = <dO_i, V_j>,   dS_ij = P_ij (dP_ij - D_i)
//   dK_j = scale * sum_i dS_ij Q_i,   dQ_i = scale * sum_j dS_ij K_j
//
// Three kernels run in order on one stream:
//   1. fa_bwd_delta: D = rowsum(dO * O) into the caller's workspace.
//   2. fa_bwd_dkdv:  one work-group per 128 keys; walks the kept query tiles,
//                    accumulates dK, dV on chip, writes them once.  Q and dO
//                    tiles are staged row-major; their transposes are read
//                    with the transposing LDS load.
//   3. fa_bwd_dq:    one work-group per 128 queries; walks the kept key tiles,
//                    accumulates dQ on chip, writes it once.
// Splitting dQ into its own pass recomputes S and dP once more but needs no
// atomics, so the result is deterministic.

#include <algorithm>

#include "fa_common.hpp"
#include "fa_launch.hpp"
#include "fa_rows.hpp"

namespace fa {

// The dot product of one 16-byte chunk of an O row with the same chunk of
// its dO row: one fma chain from zero, in element order.  Both places that
// form D (the preprocess kernel and the dQ pass) build on it and then add the
// chunk results in the same pairwise tree, so they give bit-identical D.
template <typename T, int CH>
__device__ __forceinline__ float chunk_dot(const T* a, const T* b) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < CH; ++e) acc = fmaf(Elem<T>::to_f32(a[e]), Elem<T>::to_f32(b[e]), acc);
  return acc;
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO_ik O_ik  (HBM-bound; one 16-byte chunk per lane)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
fa_bwd_delta_kernel(const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ delta,
                    int rows) {
  using E = Elem<T>;
  constexpr int CH = E::kPerChunk;
  constexpr int LPR = D / CH;                      // lanes per row
  constexpr int RPB = kThreads / LPR;              // rows per block
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int col = (tid % LPR) * CH;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + (size_t)row * D + col);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + (size_t)row * D + col);
    acc = chunk_dot<T, CH>(reinterpret_cast<const T*>(&a), reinterpret_cast<const T*>(&b));
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && (tid % LPR) == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV: work-group = 128 keys (wave w: keys 32w..32w+31, lane l32 one
//    key).  Per kept query tile of BQ = 64 rows:
//      S   = Q_i K_j^T      (A = Q rows from LDS, B = K in registers)
//      dP  = dO_i V_j^T     (A = dO rows from LDS, B = V in registers)
//      P, dS elementwise in the C layout (query index per register)
//      dV^T += dO_i^T P     (A = dO^T by transposing LDS reads, B = P registers)
//      dK^T += Q_i^T dS     (A = Q^T by transposing LDS reads, B = dS registers)
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvCfg {
  static constexpr int BK = 128;                         // keys per work-group
  // query rows per compute tile: 64 for bf16 at d = 128 (the software-
  // pipelined tile body); 32 for fp32 and for bf16 at d = 64, whose two
  // waves per SIMD leave registers for a simpler body only
  static constexpr int BQ = (sizeof(T) == 2 && D == 128) ? 64 : 32;
  static constexpr int SQ = sizeof(T) == 2 ? 128 : 64;   // query rows per staged tile
};

// Waves per SIMD of the dK/dV pass: one at d = 128 (the tile needs ~436
// registers); two for bf16 at d = 64 (about half of that), so that two
// work-groups share a compute unit and one's prologue and epilogue overlap
// the other's tiles.  The two-wave build keeps operands in VGPRs (no AGPR
// pins, see to_agpr).
template <typename T, int D>
struct DkdvOcc {
  static constexpr int waves = (sizeof(T) == 2 && D == 64) ? 2 : 1;
  static constexpr bool pin_agpr = waves == 1;
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DkdvOcc<T, D>::waves, DkdvOcc<T, D>::waves)))
fa_bwd_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                   const T* __restrict__ dO, const float* __restrict__ LSE,
                   const float* __restrict__ delta, T* __restrict__ dK, T* __restrict__ dV,
                   float* __restrict__ part, int gsplit,
                   const uint8_t* __restrict__ mask, int BH, int kv_group, int N, int T_tiles,
                   float c, float scale, DropParams drp) {
  using E = Elem<T>;
  using frag = typename E::frag;
  using Cfg = DkdvCfg<T, D>;
  constexpr int BK = Cfg::BK, BQ = Cfg::BQ, SQ = Cfg::SQ;
  constexpr int NQH = BQ / 32;            // 32-row query halves per tile
  constexpr int NT = D / 16, ND = D / 32;
  constexpr uint32_t RB = Tile<T, D>::RB;
  constexpr int TB = BQ * RB;             // bytes per compute tile of Q or dO
  constexpr int STB = SQ * RB;            // bytes per staged tile of Q or dO

  // Two buffers of [Q, dO] tiles (distinct arrays, see pick()), plus per-row
  // LSE*log2e and D.
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[2 * STB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[2 * STB];
  __shared__ __attribute__((aligned(16))) float sL[2][SQ];   // +inf: no keys / past N
  __shared__ __attribute__((aligned(16))) float sD[2][SQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int nkb = (N + BK - 1) / BK;
  // BH counts (key/value head, split) pairs here: query heads
  // bh*kv_group .. +kv_group-1 share head bh, and their contributions to dK,
  // dV are summed on chip.  With gsplit > 1 the group's query heads are
  // divided among gsplit work-groups (more work-groups when there are few key
  // blocks), each writing an fp32 partial that a reduction kernel adds up.
  const BlockCoord bc = map_block(blockIdx.x, nkb, BH, CAUSAL, false);
  const int bh = bc.bh / gsplit, sp = bc.bh - bh * gsplit;
  const int kb = bc.blk, k0 = kb * BK;
  const size_t head = (size_t)bh * N * D;   // K, V, dK, dV of this key/value head
  const int kw = k0 + 32 * w;            // this wave's first key
  const int krow = kw + l32;             // this lane's key

  // K and V rows of this lane as B operands (natural d order); rows past N
  // read as zero.
  const rsrc_t rk = make_rsrc(K + head, (uint32_t)N * RB);
  const rsrc_t rv = make_rsrc(V + head, (uint32_t)N * RB);
  frag kf[NT], vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t off = (uint32_t)krow * RB + (16 * t + 8 * g) * sizeof(T);
    kf[t] = gload_frag<T>(rk, off);
    vf[t] = gload_frag<T>(rv, off);
    if constexpr (DkdvOcc<T, D>::pin_agpr) {
      to_agpr(kf[t]);
      to_agpr(vf[t]);
    }
  }

  // Staged tiles of SQ query rows, each run as two compute tiles of BQ rows
  // (one barrier and one round of loads per SQ rows).
  const int ntiles = (N + SQ - 1) / SQ;
  const int first = CAUSAL ? k0 / SQ : 0;
  // Column kb of the block mask: mask[qi][kb], stride T.
  KeptTiles<SQ> kept(MASKED ? mask + kb : nullptr, (size_t)T_tiles, T_tiles);
  auto next_kept = [&](int i) {
    if constexpr (MASKED) return kept.next(i, lane);
    return i;
  };

  // The walk covers (query head of the group, staged tile) pairs u =
  // gq * ntiles + i, tiles from the causal start `first` on, kept tiles only.
  // With gsplit > 1 the kv_group * (ntiles - first) pairs are cut into
  // gsplit equal runs, one per work-group: whole query heads when gsplit
  // divides kv_group, else runs of one head's query tiles.
  const int nt = ntiles - first;
  const int tot = kv_group * nt;
  auto u_at = [&](int idx) {
    return idx >= tot ? kv_group * ntiles : (idx / nt) * ntiles + first + idx % nt;
  };
  const int U0 = u_at((int)((long long)sp * tot / gsplit));
  const int NU = u_at((int)((long long)(sp + 1) * tot / gsplit));
  auto next_u = [&](int u) {
    while (u < NU) {
      const int gq = u / ntiles;
      const int k = next_kept(max(u - gq * ntiles, first));
      if (k < ntiles) return gq * ntiles + k;
      u = (gq + 1) * ntiles;
    }
    return NU;
  };

  float lpre = 0.f, dpre = 0.f;     // row statistics of the tile in flight (threads < SQ)
  int lrow_pre = 0;
  auto stage = [&](int u, auto buf) {
    const int gq = u / ntiles;
    const int q0 = (u - gq * ntiles) * SQ;
    const size_t hq = (size_t)bh * kv_group + gq;      // query head
    const T* Qh = Q + hq * N * D;
    const T* dOh = dO + hq * N * D;
    const rsrc_t rl = make_rsrc(LSE + hq * N, (uint32_t)N * 4);
    const rsrc_t rd = make_rsrc(delta + hq * N, (uint32_t)N * 4);
    const uint32_t left = (uint32_t)(N - q0) * RB;
    unsigned char* base = pick(buf, lds0, lds1);
    stage_tile<T, D, SQ>(make_rsrc(Qh + (size_t)q0 * D, left), base, w, lane);
    stage_tile<T, D, SQ>(make_rsrc(dOh + (size_t)q0 * D, left), base + STB, w, lane);
    if (tid < SQ) {
      lpre = buf_load_f32(rl, (uint32_t)(q0 + tid) * 4);   // raw; transformed when stored
      dpre = buf_load_f32(rd, (uint32_t)(q0 + tid) * 4);
      lrow_pre = q0 + tid;
    }
  };

  f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) { dkacc[b] = f32x16{}; dvacc[b] = f32x16{}; }
  LaneOffsets<T, D> lo;
  lo.init(lane);
  int bhq = bh * kv_group;   // query head of the tile being computed

  // One tile iteration.  MASKED_TILE (the tile crosses this wave's causal
  // diagonal) is compile-time, so unmasked tiles carry no mask arithmetic.
  auto tile = [&](auto mask_tag, auto buf_sel, int sub, int q0) {
    const int BUF = buf_sel;
    constexpr bool MASKED_TILE = decltype(mask_tag)::value;
    const unsigned char* sQ = pick(buf_sel, lds0, lds1) + sub * TB;
    const unsigned char* sdO = sQ + STB;
    const float* sLt = &sL[BUF][sub * BQ];
    const float* sDt = &sD[BUF][sub * BQ];
      // The tile is processed as a pipeline of MFMA blocks:
      //   S/dP of query half 0 (NT/SB blocks of 2*SB MFMAs), S/dP of half 1,
      //   dV/dK of half 0 (2 blocks of 2*ND MFMAs), dV/dK of half 1.
      // Each block's LDS operands are read while the previous block's MFMAs run,
      // and the P/dS arithmetic of a half is spread over the blocks that follow
      // it, between their MFMAs.
      constexpr int SB = NT >= 8 ? 4 : NT;          // d-chunks per S/dP block
      constexpr int NSB = NT / SB;                  // S/dP blocks per half

      // S/dP block (half qh, d-chunks t0 .. t0+SB-1)
      auto sdp_read = [&](int qh, int t0, frag* aq, frag* ao) {
#pragma unroll
        for (int t = 0; t < SB; ++t) {
          if constexpr (sizeof(T) == 2) {
            const unsigned char* p = sQ + lo.row[t0 + t] + 32 * qh * RB;
            aq[t] = row_frag_at<T>(p);
            ao[t] = row_frag_at<T>(p + STB);
          } else {
            aq[t] = row_frag<T, D>(sQ, 32 * qh + l32, t0 + t, g);
            ao[t] = row_frag<T, D>(sdO, 32 * qh + l32, t0 + t, g);
          }
        }
      };
      auto sdp_mma = [&](int t0, const frag* aq, const frag* ao, f32x16& sv, f32x16& dpv) {
#pragma unroll
        for (int t = 0; t < SB; ++t) {
          frag a = aq[t], o = ao[t];
          if constexpr (DkdvOcc<T, D>::pin_agpr) {
            to_agpr(a);    // at the consumer: a pin right after the read
            to_agpr(o);    // would make the read wait for its data there
          }
          sv = E::mma(a, kf[t0 + t], sv);
          dpv = E::mma(o, vf[t0 + t], dpv);
        }
      };
      // Dropout keep bits of query half qh: bit r for register r (query
      // 32qh + 8(r/4) + 4g + r%4, key krow).  A Philox call yields the words of
      // four consecutive keys, i.e. of the four lanes of a lane quad, for a
      // query pair (low 16 bits for the even query, high for the odd one), so
      // lane m of the quad draws the two calls of registers 4m..4m+3 for the
      // whole quad and the quad exchanges the 16 keep bits each lane drew (DPP
      // broadcasts): 2 calls per lane instead of 16.
      uint32_t kbits[NQH];
      auto drop_bits = [&](int qh) -> uint32_t {
        const int m = l32 & 3;
        uint32_t mine = 0;      // bit 4x + k: register 4m + x, key of quad lane k
#pragma unroll
        for (int y = 0; y < 2; ++y) {   // registers 4m + 2y (low halves), 4m + 2y + 1 (high)
          const Philox4 z = philox4x32_10((uint32_t)krow >> 2,
                                          (uint32_t)(q0 + 32 * qh + 8 * m + 4 * g + 2 * y) >> 1,
                                          (uint32_t)bhq, 0u, drp.key0, drp.key1);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            mine |= (uint32_t)((z.w[k] & 0xFFFFu) >= drp.thresh) << (8 * y + k);
            mine |= (uint32_t)((z.w[k] >> 16) >= drp.thresh) << (8 * y + 4 + k);
          }
        }
        // this lane's bits (k = m) of quad lane src's draws -> registers 4src..4src+3
        auto mine_of = [&](auto src_tag) {
          constexpr int src = decltype(src_tag)::value;
          const uint32_t v =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)mine, src * 0x55, 0xF, 0xF, true) >> m;
          return ((v & 1u) | ((v >> 3) & 2u) | ((v >> 6) & 4u) | ((v >> 9) & 8u)) << (4 * src);
        };
        return mine_of(IntTag<0>{}) | mine_of(IntTag<1>{}) | mine_of(IntTag<2>{}) |
               mine_of(IntTag<3>{});
      };
      // d = 128: the LSE and D rows a P/dS part needs are read one MFMA
      // block ahead (read in the same block they queue behind that block's
      // operand reads, and the arithmetic waits for all of them), and each
      // part's results are anchored in its block (see pds_part).  At d = 64
      // the blocks are too short for either and both measured slower.
      constexpr bool LOOK = D == 128 && NQH == 2;
      auto stat_load = [&](int qh, int a0, int a1, f32x4* lv, f32x4* dv) {
#pragma unroll
        for (int a = a0; a < a1; ++a) {
          const int qi = 32 * qh + 8 * a + 4 * g;
          lv[a - a0] = *reinterpret_cast<const f32x4*>(sLt + qi);
          if constexpr (DROP) dv[a - a0] = *reinterpret_cast<const f32x4*>(sDt + qi);
        }
      };
      // LDS reads per register group in stat_load (LSE, and D for dropout)
      constexpr int NSTAT = DROP ? 2 : 1;
      // The dP accumulators of query half qh start at the LDS D row values,
      // -D (times 1 - p under dropout; see step), so the matrix cores return
      // dP - D and pds_part needs no subtraction.
      auto dinit = [&](int qh) {
        f32x16 v;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(sDt + 32 * qh + 8 * a + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * a + e] = x[e];
        }
        return v;
      };
      // P = 2^(S c - LSE log2 e), dS = P (dP - D) for register groups
      // a0 .. a1-1 (register r holds query 32qh + 8(r/4) + 4g + r%4), with the
      // statistics from stat_load (LOOK) or read here.
      auto pds_part = [&](int qh, int a0, int a1, f32x16& sv, f32x16& dpv,
                          const f32x4* lvs = nullptr, const f32x4* dvs = nullptr) {
        if constexpr (DROP) {
          if (a0 == 0) kbits[qh] = drop_bits(qh);
        }
#pragma unroll
        for (int a = a0; a < a1; ++a) {
          const int qi = 32 * qh + 8 * a + 4 * g;
          const f32x4 lv = LOOK ? lvs[a - a0] : *reinterpret_cast<const f32x4*>(sLt + qi);
          f32x4 dv = f32x4{};
          if constexpr (DROP) dv = LOOK ? dvs[a - a0] : *reinterpret_cast<const f32x4*>(sDt + qi);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * a + x;
            float p = __builtin_amdgcn_exp2f(fmaf(sv[r], c, -lv[x]));
            if (MASKED_TILE && krow > q0 + qi + x) p = 0.f;
            if constexpr (DROP) {
              // dV takes the dropped probabilities (its 1/(1-p) is applied at
              // the end); dS = P (dP M - D) with M = Z / (1-p).
              const bool keep = (kbits[qh] >> r) & 1u;
              sv[r] = keep ? p : 0.f;
              // dpv = dP - D (1-p): kept, (dP - D (1-p)) / (1-p) = dP M - D;
              // dropped, -D = (-D (1-p)) / (1-p) from the LDS row value.
              dpv[r] = p * (keep ? dpv[r] : dv[x]) * drp.inv_keep;
            } else {
              sv[r] = p;
              dpv[r] = p * dpv[r];
            }
          }
        }
        // The arithmetic is pure and its results are next used blocks later,
        // so instruction selection would place it there, past this block's
        // scheduling fence (leaving this block's MFMAs without VALU work and
        // a later block with too much); an empty asm use keeps it here.
        if constexpr (LOOK) {
#pragma unroll
          for (int r = 4 * a0; r < 4 * a1; ++r) asm volatile("" ::"v"(sv[r]), "v"(dpv[r]));
        }
      };
      auto pds_pack = [&](const f32x16& sv, const f32x16& dpv, frag* pf, frag* df) {
        pf[0] = E::from_c(sv, 0);
        pf[1] = E::from_c(sv, 1);
        df[0] = E::from_c(dpv, 0);
        df[1] = E::from_c(dpv, 1);
      };
      // dV/dK block (half qh, 16-row chunk t of the half)
      auto dvdk_read = [&](int qh, int t, frag* ot, frag* qt) {
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          if constexpr (sizeof(T) == 2) {
            const unsigned char* p0 = sQ + lo.tr[b][0] + 16 * (2 * qh + t) * RB;
            const unsigned char* p1 = sQ + lo.tr[b][1] + 16 * (2 * qh + t) * RB;
            ot[b] = trans_frag_at(p0 + STB, p1 + STB);
            qt[b] = trans_frag_at(p0, p1);
          } else {
            ot[b] = trans_frag<T, D>(sdO, b, 2 * qh + t, lane);
            qt[b] = trans_frag<T, D>(sQ, b, 2 * qh + t, lane);
          }
        }
      };
      auto dvdk_mma = [&](const frag* ot, const frag* qt, const frag& pf, const frag& df) {
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          frag o = ot[b], q = qt[b];
          if constexpr (DkdvOcc<T, D>::pin_agpr) {
            to_agpr(o);
            to_agpr(q);
          }
          dvacc[b] = E::mma(o, pf, dvacc[b]);
          dkacc[b] = E::mma(q, df, dkacc[b]);
        }
      };

      f32x16 s0 = f32x16{}, dp0 = dinit(0);
      frag pf0[2], df0[2];
      frag xa[SB], xb[SB];        // operand set of the block being issued
      frag ya[SB], yb[SB];        // operand set prefetched for the next block
      if constexpr (NQH == 2) {
        f32x16 s1 = f32x16{}, dp1 = f32x16{};
        frag pf1[2], df1[2];
        frag ta[ND], tb[ND], ua[ND], ub[ND];
        constexpr int GP = 4 / NSB;             // register groups of P/dS per S/dP block
        f32x4 lc[GP], dc[GP], ln[GP], dn[GP];   // LOOK: statistics in use / being read
        auto stat_next = [&]() {
#pragma unroll
          for (int t = 0; t < GP; ++t) { lc[t] = ln[t]; dc[t] = dn[t]; }
        };
        sdp_read(0, 0, xa, xb);
        sched_fence();
        // S/dP, half 0
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
          if (k + 1 < NSB) sdp_read(0, (k + 1) * SB, ya, yb);
          else sdp_read(1, 0, ya, yb);
          if (LOOK && k + 1 == NSB) stat_load(0, 0, GP, lc, dc);
          if (k + 1 == NSB) dp1 = dinit(1);
          sdp_mma(k * SB, xa, xb, s0, dp0);
          if (LOOK && k + 1 == NSB) interleave<2 * SB, 2 * SB + NSTAT * GP + 4, 0>();
          else if (k + 1 == NSB) interleave<2 * SB, 2 * SB + 4, 0>();
          else interleave<2 * SB, 2 * SB, 0>();
          sched_fence();
#pragma unroll
          for (int t = 0; t < SB; ++t) { xa[t] = ya[t]; xb[t] = yb[t]; }
        }
        // S/dP, half 1, with P/dS of half 0 in between
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
          if (k + 1 < NSB) sdp_read(1, (k + 1) * SB, ya, yb);
          else dvdk_read(0, 0, ta, tb);
          if constexpr (LOOK) {
            if (k + 1 < NSB) stat_load(0, (k + 1) * GP, (k + 2) * GP, ln, dn);
            else stat_load(1, 0, 2, ln, dn);
          }
          sdp_mma(k * SB, xa, xb, s1, dp1);
          pds_part(0, k * GP, (k + 1) * GP, s0, dp0, lc, dc);
          if (k + 1 == NSB) pds_pack(s0, dp0, pf0, df0);
          if (k + 1 < NSB) interleave<2 * SB, 2 * SB + NSTAT * GP, 5>();
          else interleave<2 * SB, 4 * ND + (LOOK ? 2 * NSTAT : NSTAT * GP), 5>();
          sched_fence();
#pragma unroll
          for (int t = 0; t < SB; ++t) { xa[t] = ya[t]; xb[t] = yb[t]; }
          if constexpr (LOOK) stat_next();
        }
        // dV/dK, half 0, with P/dS of half 1 in between
        dvdk_read(0, 1, ua, ub);
        if constexpr (LOOK) stat_load(1, 2, 4, ln, dn);
        dvdk_mma(ta, tb, pf0[0], df0[0]);
        pds_part(1, 0, 2, s1, dp1, lc, dc);
        interleave<2 * ND, 4 * ND + 2 * NSTAT, 6>();
        sched_fence();
        if constexpr (LOOK) stat_next();
        dvdk_read(1, 0, ta, tb);
        dvdk_mma(ua, ub, pf0[1], df0[1]);
        pds_part(1, 2, 4, s1, dp1, lc, dc);
        pds_pack(s1, dp1, pf1, df1);
        interleave<2 * ND, 4 * ND + (LOOK ? 0 : 2 * NSTAT), 6>();
        sched_fence();
        // dV/dK, half 1
        dvdk_read(1, 1, ua, ub);
        dvdk_mma(ta, tb, pf1[0], df1[0]);
        interleave<2 * ND, 4 * ND, 0>();
        sched_fence();
        dvdk_mma(ua, ub, pf1[1], df1[1]);
      } else {
        frag ta[ND], tb[ND];
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
          sdp_read(0, k * SB, xa, xb);
          sdp_mma(k * SB, xa, xb, s0, dp0);
        }
        pds_part(0, 0, 4, s0, dp0);
        pds_pack(s0, dp0, pf0, df0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          dvdk_read(0, t, ta, tb);
          dvdk_mma(ta, tb, pf0[t], df0[t]);
        }
      }
  };
  // Wait for tile i (buffer BUF), publish its row statistics, prefetch the
  // next kept tile into the other buffer, then run the tile.
  auto step = [&](auto buf_sel, int u, int un) {
    const int BUF = buf_sel;
    const int gq = u / ntiles;
    const int i = u - gq * ntiles;
    bhq = bh * kv_group + gq;
    wait_global_loads();
    if (tid < SQ) {
      // Rows past N, and rows that keep no key (LSE = -inf), get P = 0.
      sL[BUF][tid] = (lrow_pre < N && lpre != neg_inf()) ? lpre * kLog2e : pos_inf();
      // -D, the dP accumulators' starting value (see dinit); under dropout
      // -D (1-p), exactly -D at p = 0.
      sD[BUF][tid] = DROP ? -dpre * (1.0f / drp.inv_keep) : -dpre;
    }
    __syncthreads();
    if (un < NU) stage(un, other(buf_sel));
#pragma unroll 1
    for (int sub = 0; sub < SQ / BQ; ++sub) {
      const int q0 = i * SQ + sub * BQ;
      if (q0 >= N) break;
      if constexpr (sizeof(T) == 4) {
        tile(BoolTag<CAUSAL>{}, buf_sel, sub, q0);   // one body: the fp32 path needs every register
      } else {
        if (CAUSAL && q0 < kw + 31) tile(BoolTag<true>{}, buf_sel, sub, q0);
        else tile(BoolTag<false>{}, buf_sel, sub, q0);
      }
    }
  };

  int u = next_u(U0);
  if (u < NU) stage(u, IntTag<0>{});
  if constexpr (sizeof(T) == 2) {
    // Two iterations per trip with the buffer index a compile-time constant,
    // so the LDS offsets are immediates.
    while (u < NU) {
      int un = next_u(u + 1);
      step(IntTag<0>{}, u, un);
      u = un;
      if (u >= NU) break;
      un = next_u(u + 1);
      step(IntTag<1>{}, u, un);
      u = un;
    }
  } else {
    int buf = 0;
    while (u < NU) {
      const int un = next_u(u + 1);
      step(buf, u, un);
      buf ^= 1;
      u = un;
    }
  }

  // dV^T / dK^T C layout: lane (key l32, g), register r -> d = 32b + 8(r/4) + 4g + r%4.
  if (gsplit > 1) {
    if (krow < N) {
      const size_t E = (size_t)(BH / gsplit) * N * D;     // elements of dK
      float* pk = part + (size_t)sp * E + head + (size_t)krow * D;
      float* pv = part + (size_t)(gsplit + sp) * E + head + (size_t)krow * D;
      const float vs = DROP ? drp.inv_keep : 1.0f;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d0 = 32 * b + 8 * a + 4 * g;
          *reinterpret_cast<f32x4*>(pv + d0) =
              f32x4{dvacc[b][4 * a], dvacc[b][4 * a + 1], dvacc[b][4 * a + 2],
                    dvacc[b][4 * a + 3]} * vs;
          *reinterpret_cast<f32x4*>(pk + d0) =
              f32x4{dkacc[b][4 * a], dkacc[b][4 * a + 1], dkacc[b][4 * a + 2],
                    dkacc[b][4 * a + 3]} * scale;
        }
    }
    return;
  }
  if constexpr (sizeof(T) == 2) {
    // Results through LDS (fa_rows.hpp, padded rows): dV in lds0, dK in lds1.
    static_assert(BK * RowTile<T, D, true>::RS <= 2 * STB, "result rows must fit a staging array");
    __syncthreads();                                  // every wave is done with the tiles
    const float vs = DROP ? drp.inv_keep : 1.0f;
    const int lr = 32 * w + l32;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = 32 * b + 8 * a + 4 * g;
        put_row4<T, D, true>(lds0, lr, col, dvacc[b][4 * a] * vs, dvacc[b][4 * a + 1] * vs,
                             dvacc[b][4 * a + 2] * vs, dvacc[b][4 * a + 3] * vs);
        put_row4<T, D, true>(lds1, lr, col, dkacc[b][4 * a] * scale, dkacc[b][4 * a + 1] * scale,
                             dkacc[b][4 * a + 2] * scale, dkacc[b][4 * a + 3] * scale);
      }
    __syncthreads();
    write_rows<T, D, true, BK, kThreads>(lds0, dV + head + (size_t)k0 * D, N - k0, tid);
    write_rows<T, D, true, BK, kThreads>(lds1, dK + head + (size_t)k0 * D, N - k0, tid);
    return;
  }
  if (krow < N) {
    T* dKr = dK + head + (size_t)krow * D;
    T* dVr = dV + head + (size_t)krow * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * b + 8 * a + 4 * g;
        const float vs = DROP ? drp.inv_keep : 1.0f;
        E::store4(dVr + d0, dvacc[b][4 * a] * vs, dvacc[b][4 * a + 1] * vs,
                  dvacc[b][4 * a + 2] * vs, dvacc[b][4 * a + 3] * vs);
        E::store4(dKr + d0, dkacc[b][4 * a] * scale, dkacc[b][4 * a + 1] * scale,
                  dkacc[b][4 * a + 2] * scale, dkacc[b][4 * a + 3] * scale);
      }
  }
}

// dK, dV = the sum of the gsplit fp32 partials of the dK/dV pass (element
// order of dK; partials laid out [2][gsplit][E], dK first).
template <typename T>
__global__ void __launch_bounds__(kThreads)
fa_bwd_dkdv_reduce_kernel(const float* __restrict__ part, T* __restrict__ dK,
                          T* __restrict__ dV, size_t E4 /* elements / 4 */, int gsplit) {
  const f32x4* p = reinterpret_cast<const f32x4*>(part);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < E4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4 k = f32x4{}, v = f32x4{};
    for (int sp = 0; sp < gsplit; ++sp) {
      k += p[(size_t)sp * E4 + i];
      v += p[(size_t)(gsplit + sp) * E4 + i];
    }
    Elem<T>::store4(dK + 4 * i, k[0], k[1], k[2], k[3]);
    Elem<T>::store4(dV + 4 * i, v[0], v[1], v[2], v[3]);
  }
}

// dQ = the sum of the ksplit fp32 partials of the dQ pass, in split order.
template <typename T>
__global__ void __launch_bounds__(kThreads)
fa_bwd_dq_reduce_kernel(const float* __restrict__ part, T* __restrict__ dQ,
                        size_t E4 /* elements / 4 */, int ksplit) {
  const f32x4* p = reinterpret_cast<const f32x4*>(part);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < E4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4 q = p[i];
    for (int sp = 1; sp < ksplit; ++sp) q += p[(size_t)sp * E4 + i];
    Elem<T>::store4(dQ + 4 * i, q[0], q[1], q[2], q[3]);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: work-group = 128 queries (wave w: rows 32w..32w+31, lane pair one
//    row), same walk over key tiles as the forward:
//      S^T  = K_j Q_i^T     (A = K rows from LDS, B = Q registers)
//      dP^T = V_j dO_i^T    (A = V rows from LDS, B = dO registers)
//      P^T, dS^T elementwise with this lane's own LSE_i and D_i
//      dQ^T += K_j^T dS^T   (A = K^T via transposing LDS reads, B = dS^T)
//    D_i comes from the preprocess kernel, or (given O) the pass forms it
//    from the O and dO rows in its registers and writes it for the dK/dV
//    pass, which then runs after it.
// ---------------------------------------------------------------------------
// D_i for the row that lane pair (l32, l32 + 32) holds in the dQ layout:
// lane (l32, g) has the 8-element operand chunk at column 16t + 8g of O (o)
// and dO (d), t = 0..D/16-1, i.e. 16-byte chunks 2t + g (bf16) or 4t + 2g
// and 4t + 2g + 1 (fp32).  The chunk results are added in the preprocess
// kernel's tree (partners at chunk-index distance LPR/2, ..., 2, 1): strides
// inside a lane's own chunks add in registers, the stride between g = 0 and
// g = 1 takes one cross-lane swap.  Both lanes of the pair return D_i.
template <typename T, int D>
__device__ __forceinline__ float pair_row_delta(const typename Elem<T>::frag* o,
                                                const typename Elem<T>::frag* d) {
  constexpr int CH = Elem<T>::kPerChunk, LPR = D / CH, NJ = LPR / 2, NT = D / 16;
  constexpr int GSTRIDE = sizeof(T) == 2 ? 1 : 2;   // chunk-index distance between g = 0, 1
  float a[NJ];                                      // a[j]: this lane's j-th chunk
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if constexpr (sizeof(T) == 2) {
      a[t] = chunk_dot<T, CH>(reinterpret_cast<const T*>(&o[t].v),
                              reinterpret_cast<const T*>(&d[t].v));
    } else {
      a[2 * t] = chunk_dot<T, CH>(reinterpret_cast<const T*>(&o[t].lo),
                                  reinterpret_cast<const T*>(&d[t].lo));
      a[2 * t + 1] = chunk_dot<T, CH>(reinterpret_cast<const T*>(&o[t].hi),
                                      reinterpret_cast<const T*>(&d[t].hi));
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) {
    if (off == GSTRIDE) {
      // Chunks still live here: j < GSTRIDE (wider strides already folded).
#pragma unroll
      for (int j = 0; j < GSTRIDE; ++j) a[j] += __shfl_xor(a[j], 32);
    } else {
      const int jo = off > GSTRIDE ? off / 2 : off;   // the same distance in j
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (!(j & jo)) a[j] += a[j ^ jo];
    }
  }
  return a[0];
}

template <typename T>
struct DqCfg {
  static constexpr int BR = 128;
  static constexpr int BC = sizeof(T) == 2 ? 64 : 32;
};

template <typename T, int D, bool CAUSAL, bool MASKED, bool DROP>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Occupancy<T, D, CAUSAL, MASKED, DROP>::dq,
                                   Occupancy<T, D, CAUSAL, MASKED, DROP>::dq)))
fa_bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                 const T* __restrict__ dO, const T* __restrict__ O, const float* __restrict__ LSE,
                 float* __restrict__ delta, T* __restrict__ dQ,
                 const uint8_t* __restrict__ mask, int BH, int kv_group, int N, int T_tiles,
                 float c, float scale, DropParams drp, int ksplit, float* __restrict__ qpart) {
  using E = Elem<T>;
  using frag = typename E::frag;
  using Cfg = DqCfg<T>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC;
  constexpr int NH = BC / 32, NT = D / 16, ND = D / 32;
  constexpr uint32_t RB = Tile<T, D>::RB;
  constexpr int TB = BC * RB;

  // Two buffers of [K, V] tiles (distinct arrays, see pick()).
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[2 * TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[2 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int nqb = (N + BR - 1) / BR;
  // With ksplit > 1 each query block's key tiles are cut into ksplit runs
  // of equal length, one per work-group, which write scale * their dQ
  // partial in fp32 (qpart, [ksplit][BH * N * D]) for a reduction kernel;
  // the runs of one block count as separate heads in the block order.
  const BlockCoord bc = map_block(blockIdx.x, nqb, BH * ksplit, CAUSAL, true,
                                  Occupancy<T, D, CAUSAL, MASKED, DROP>::dq);
  const int bh = bc.bh / ksplit, ksp = bc.bh - bh * ksplit, q0 = bc.blk * BR;
  const size_t head = (size_t)bh * N * D;
  const size_t kvhead = (size_t)(bh / kv_group) * N * D;    // shared key/value head
  const T* Kh = K + kvhead;
  const T* Vh = V + kvhead;
  const int qrow = q0 + 32 * w + l32;
  // Dropout: the low 16-bit half of a Philox word for an even query row,
  // the high half for an odd one.
  const int odd = l32 & 1;
  const uint32_t hmask = odd ? 0xFFFFFFFFu : 0xFFFFu;
  const uint32_t hthr = odd ? drp.thresh << 16 : drp.thresh;

  const rsrc_t rq = make_rsrc(Q + head, (uint32_t)N * RB);
  const rsrc_t ro = make_rsrc(dO + head, (uint32_t)N * RB);
  frag qf[NT], of[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t off = (uint32_t)qrow * RB + (16 * t + 8 * g) * sizeof(T);
    qf[t] = gload_frag<T>(rq, off);
    of[t] = gload_frag<T>(ro, off);
  }
  // Rows past N, and rows that keep no key (LSE = -inf), get P = 0.
  const float lrow = buf_load_f32(make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4), (uint32_t)qrow * 4);
  // D_i: formed here from O (when given, which the pass then writes for the
  // dK/dV pass), else read from what the preprocess kernel wrote.
  const rsrc_t rd = make_rsrc(delta + (size_t)bh * N, (uint32_t)N * 4);
  frag oo[NT];
  float dval = 0.f;
  if (O) {
    const rsrc_t rO = make_rsrc(O + head, (uint32_t)N * RB);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      oo[t] = gload_frag<T>(rO, (uint32_t)qrow * RB + (16 * t + 8 * g) * sizeof(T));
  } else {
    dval = buf_load_f32(rd, (uint32_t)qrow * 4);
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles_all = (kv_end + BC - 1) / BC;
  const int jbeg = (int)((long long)ksp * ntiles_all / ksplit);
  const int ntiles = (int)((long long)(ksp + 1) * ntiles_all / ksplit);   // end of this run
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

  f32x16 dqacc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) dqacc[b] = f32x16{};

  // bf16: precomputed per-lane operand offsets and compile-time LDS buffers
  // (loop unrolled by two), so every LDS read is a lane offset plus an
  // immediate.  fp32 forms addresses per read (register budget).
  constexpr bool USE_LO = sizeof(T) == 2;
  LaneOffsets<T, D> lo;
  if constexpr (USE_LO) lo.init(lane);
  int j = next_kept(jbeg);
  if (j < ntiles) stage(j, IntTag<0>{});
  wait_global_loads();
  const float lse2 = (qrow < N && lrow != neg_inf()) ? lrow * kLog2e : pos_inf();
  if (O) {
    dval = pair_row_delta<T, D>(oo, of);
    if (ksp == 0 && g == 0 && qrow < N) delta[(size_t)bh * N + qrow] = dval;
  }
  // Starting value of every dP accumulator: -D (times 1 - p under dropout),
  // so the matrix cores return dP - D and the tile needs no subtraction.
  // Under dropout a kept entry is (dP - D (1-p)) / (1-p) = dP M - D; at
  // p = 0 both paths do the same operations.
  f32x16 dinit;
  {
    const float d0 = DROP ? -dval * (1.0f / drp.inv_keep) : -dval;
#pragma unroll
    for (int r = 0; r < 16; ++r) dinit[r] = d0;
  }

  // One key tile.  MASKED_TILE: the tile crosses this wave's causal diagonal
  // or the end of the sequence (a compile-time tag where a second body fits
  // the register budget, so other tiles carry no mask arithmetic).
  auto tile = [&](auto mask_sel, auto buf_sel, int kv0) {
    const bool MASKED_TILE = mask_sel;
    const unsigned char* sK = pick(buf_sel, lds0, lds1);
    const unsigned char* sV = sK + TB;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      // Operands in sub-batches of SB chunks (register budget of two waves
      // per SIMD); the other wave on the SIMD covers the LDS latency.
      constexpr int SB = NT >= 8 ? 4 : NT;
      f32x16 s = f32x16{}, dp = dinit;
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += SB) {
        frag ak[SB], av[SB];
#pragma unroll
        for (int t = 0; t < SB; ++t) {
          if constexpr (USE_LO) {
            const unsigned char* p = sK + lo.row[t0 + t] + 32 * h * RB;
            ak[t] = row_frag_at<T>(p);
            av[t] = row_frag_at<T>(p + TB);
          } else {
            ak[t] = row_frag<T, D>(sK, 32 * h + l32, t0 + t, g);
            av[t] = row_frag<T, D>(sV, 32 * h + l32, t0 + t, g);
          }
        }
#pragma unroll
        for (int t = 0; t < SB; ++t) {
          s = E::mma(ak[t], qf[t0 + t], s);
          dp = E::mma(av[t], of[t0 + t], dp);
        }
        if constexpr (USE_LO) sched_fence();
      }
      // Register r holds key kv0 + 4g + 32h + 8(r/4) + r%4.
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - kv0 - 4 * g - 32 * h;
      if constexpr (DROP) {
        // dS = P (dP M - D), M = Z / (1-p); registers 4a..4a+3 are keys
        // kv0 + 32h + 8a + 4g + x.  As in the forward, lanes l32 and l32 ^ 1
        // (a query pair) share the Philox calls: the even lane draws groups
        // a = 0, 1, the odd lane a = 2, 3, each reads the other's words over
        // DPP and keeps its own 16-bit half.
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {   // groups c2 (even lane's call), 2 + c2 (odd lane's)
          const Philox4 z = philox4x32_10((uint32_t)((kv0 + 32 * h + 8 * (2 * odd + c2)) >> 2) + g,
                                          (uint32_t)qrow >> 1, (uint32_t)bh, 0u, drp.key0, drp.key1);
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const int r = 4 * (2 * e + c2) + x;
              const uint32_t wv = (uint32_t)(e == 0
                  ? __builtin_amdgcn_mov_dpp((int)z.w[x], 0xA0, 0xF, 0xF, true)
                  : __builtin_amdgcn_mov_dpp((int)z.w[x], 0xF5, 0xF, 0xF, true));
              const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
              dp[r] = p * ((wv & hmask) >= hthr ? dp[r] * drp.inv_keep : -dval);
            }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
          dp[r] = p * dp[r];
        }
      }
      // Keys this row does not keep get dS = 0 (a select, so an overflowed P
      // of a masked key leaves nothing behind).  The flag is uniform over the
      // wave, so tiles off the diagonal branch past this.
      if (__builtin_expect(MASKED_TILE, 0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) >= lim) dp[r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const frag df = E::from_c(dp, t);
        const int cc = 2 * h + t;
        frag kt[ND];
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          if constexpr (USE_LO)
            kt[b] = trans_frag_at(sK + lo.tr[b][0] + 16 * cc * RB, sK + lo.tr[b][1] + 16 * cc * RB);
          else
            kt[b] = trans_frag<T, D>(sK, b, cc, lane);
        }
#pragma unroll
        for (int b = 0; b < ND; ++b) dqacc[b] = E::mma(kt[b], df, dqacc[b]);
        if constexpr (USE_LO) sched_fence();
      }
    }
  };
  auto step = [&](auto buf_sel, int j, int jn) {
    wait_global_loads();
    __syncthreads();
    const int kv0 = j * BC;
    if (jn < ntiles) stage(jn, other(buf_sel));
    const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > q0 + 32 * w);
    if constexpr (sizeof(T) == 2 && !(DROP && !CAUSAL && D == 128)) {
      // Separate masked / unmasked bodies where the registers allow it.
      if (need_mask) tile(BoolTag<true>{}, buf_sel, kv0);
      else tile(BoolTag<false>{}, buf_sel, kv0);
    } else {
      // One body with the mask under a wave-uniform branch: the fp32 path
      // and the non-causal dropout path at d = 128 have no registers for two.
      tile(need_mask, buf_sel, kv0);
    }
  };
  if constexpr (sizeof(T) == 2 && !CAUSAL && !DROP) {
    // Without the causal mask only the sequence's last tile can need the
    // masked body.  With both bodies in one loop the register allocator
    // kept both live and spilled at d = 128, so the walk runs as two loops,
    // unmasked tiles then the rest, each with one body; two tiles per trip,
    // buffer index compile-time (`odd`: the next tile is in buffer 1).
    // (The causal walk below, with the same two bodies chosen per tile,
    // compiles free of spills; the dropout bodies do not fit either way.)
    auto step_as = [&](auto buf_sel, auto mask_sel, int j, int jn) {
      wait_global_loads();
      __syncthreads();
      if (jn < ntiles) stage(jn, other(buf_sel));
      tile(mask_sel, buf_sel, j * BC);
    };
    bool odd = false;
    auto walk = [&](auto mask_sel) {
      constexpr bool MT = decltype(mask_sel)::value;
      auto more = [&](int jj) { return jj < ntiles && (MT || jj * BC + BC <= N); };
      if (odd && more(j)) {
        const int jn = next_kept(j + 1);
        step_as(IntTag<1>{}, mask_sel, j, jn);
        j = jn;
        odd = false;
      }
      while (more(j)) {
        int jn = next_kept(j + 1);
        step_as(IntTag<0>{}, mask_sel, j, jn);
        j = jn;
        if (!more(j)) { odd = true; break; }
        jn = next_kept(j + 1);
        step_as(IntTag<1>{}, mask_sel, j, jn);
        j = jn;
      }
    };
    walk(BoolTag<false>{});
    walk(BoolTag<true>{});
  } else if constexpr (sizeof(T) == 2) {
    while (j < ntiles) {   // two tiles per trip, buffer index compile-time
      int jn = next_kept(j + 1);
      step(IntTag<0>{}, j, jn);
      j = jn;
      if (j >= ntiles) break;
      jn = next_kept(j + 1);
      step(IntTag<1>{}, j, jn);
      j = jn;
    }
  } else {
    int buf = 0;
    while (j < ntiles) {
      const int jn = next_kept(j + 1);
      step(buf, j, jn);
      buf ^= 1;
      j = jn;
    }
  }

  if (ksplit > 1) {
    if (qrow < N) {
      float* pr = qpart + (size_t)ksp * BH * N * D + head + (size_t)qrow * D;
#pragma unroll
      for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<f32x4*>(pr + 32 * b + 8 * a + 4 * g) =
              f32x4{dqacc[b][4 * a], dqacc[b][4 * a + 1], dqacc[b][4 * a + 2],
                    dqacc[b][4 * a + 3]} * scale;
    }
    return;
  }
  if constexpr (sizeof(T) == 2) {
    // Results through LDS (fa_rows.hpp; padded rows would not fit).
    static_assert(BR * D * (int)sizeof(T) <= 2 * TB, "result rows must fit a staging array");
    __syncthreads();                                  // every wave is done with the tiles
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        put_row4<T, D, false>(lds0, 32 * w + l32, 32 * b + 8 * a + 4 * g, dqacc[b][4 * a] * scale,
                              dqacc[b][4 * a + 1] * scale, dqacc[b][4 * a + 2] * scale,
                              dqacc[b][4 * a + 3] * scale);
    __syncthreads();
    write_rows<T, D, false, BR, kThreads>(lds0, dQ + head + (size_t)q0 * D, N - q0, tid);
    return;
  }
  if (qrow < N) {
    T* dQr = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        E::store4(dQr + 32 * b + 8 * a + 4 * g, dqacc[b][4 * a] * scale,
                  dqacc[b][4 * a + 1] * scale, dqacc[b][4 * a + 2] * scale,
                  dqacc[b][4 * a + 3] * scale);
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_pre_t(const BwdArgs& a) {
  constexpr int RPB = kThreads / (D / Elem<T>::kPerChunk);
  const int rows = a.BH * a.N;
  hipLaunchKernelGGL((fa_bwd_delta_kernel<T, D>), dim3((rows + RPB - 1) / RPB), dim3(kThreads),
                     0, a.stream, static_cast<const T*>(a.o), static_cast<const T*>(a.dout),
                     a.delta, rows);
  return hipGetLastError();
}

static DropParams drop_params(const BwdArgs& a) {
  return DropParams{a.drop.key0, a.drop.key1, a.drop.thresh, a.drop.inv_keep};
}

template <typename T, int D, bool CAUSAL, bool MASKED>
static hipError_t launch_dkdv_t(const BwdArgs& a) {
  const int nkb = (a.N + DkdvCfg<T, D>::BK - 1) / DkdvCfg<T, D>::BK;
  auto go = [&](auto kernel) {
    // one work-group row per (key/value head, split of its query heads)
    const int rows = a.BH / a.G * a.gsplit;
    hipLaunchKernelGGL(kernel, dim3(nkb * rows), dim3(kThreads), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                       static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.part, a.gsplit, a.mask,
                       rows, a.G, a.N, a.T, score_coef(a.scale), a.scale, drop_params(a));
  };
  if (a.drop.on) go(fa_bwd_dkdv_kernel<T, D, CAUSAL, MASKED, true>);
  else go(fa_bwd_dkdv_kernel<T, D, CAUSAL, MASKED, false>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.gsplit == 1) return e;
  const size_t E4 = (size_t)(a.BH / a.G) * a.N * D / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((E4 + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL((fa_bwd_dkdv_reduce_kernel<T>), dim3(blocks), dim3(kThreads), 0, a.stream,
                     a.part, static_cast<T*>(a.dk), static_cast<T*>(a.dv), E4, a.gsplit);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool MASKED>
static hipError_t launch_dq_t(const BwdArgs& a) {
  const int nqb = (a.N + DqCfg<T>::BR - 1) / DqCfg<T>::BR;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(nqb * a.BH * a.ksplit), dim3(kThreads), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<const T*>(a.dout),
                       a.dq_forms_delta ? static_cast<const T*>(a.o) : nullptr, a.lse, a.delta,
                       static_cast<T*>(a.dq), a.mask, a.BH, a.G, a.N, a.T, score_coef(a.scale),
                       a.scale, drop_params(a), a.ksplit, a.qpart);
  };
  if (a.drop.on) go(fa_bwd_dq_kernel<T, D, CAUSAL, MASKED, true>);
  else go(fa_bwd_dq_kernel<T, D, CAUSAL, MASKED, false>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1) return e;
  const size_t E4 = (size_t)a.BH * a.N * D / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((E4 + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL((fa_bwd_dq_reduce_kernel<T>), dim3(blocks), dim3(kThreads), 0, a.stream,
                     a.qpart, static_cast<T*>(a.dq), E4, a.ksplit);
  return hipGetLastError();
}

// Dispatch on (dtype, d, causal, masked) to a kernel instance.
#define FA_DISPATCH(LAUNCH, a)                                                       \
  do {                                                                               \
    const bool cz = (a).causal, mk = (a).mask != nullptr;                            \
    if ((a).bf16) {                                                                  \
      if ((a).d == 64) {                                                             \
        if (cz) return mk ? LAUNCH<__bf16, 64, true, true>(a) : LAUNCH<__bf16, 64, true, false>(a); \
        return mk ? LAUNCH<__bf16, 64, false, true>(a) : LAUNCH<__bf16, 64, false, false>(a);       \
      }                                                                              \
      if (cz) return mk ? LAUNCH<__bf16, 128, true, true>(a) : LAUNCH<__bf16, 128, true, false>(a); \
      return mk ? LAUNCH<__bf16, 128, false, true>(a) : LAUNCH<__bf16, 128, false, false>(a);       \
    }                                                                                \
    if ((a).d == 64) {                                                               \
      if (cz) return mk ? LAUNCH<float, 64, true, true>(a) : LAUNCH<float, 64, true, false>(a);     \
      return mk ? LAUNCH<float, 64, false, true>(a) : LAUNCH<float, 64, false, false>(a);           \
    }                                                                                \
    if (cz) return mk ? LAUNCH<float, 128, true, true>(a) : LAUNCH<float, 128, true, false>(a);     \
    return mk ? LAUNCH<float, 128, false, true>(a) : LAUNCH<float, 128, false, false>(a);           \
  } while (0)

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.bf16) return a.d == 64 ? launch_pre_t<__bf16, 64>(a) : launch_pre_t<__bf16, 128>(a);
  return a.d == 64 ? launch_pre_t<float, 64>(a) : launch_pre_t<float, 128>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) { FA_DISPATCH(launch_dkdv_t, a); }

hipError_t launch_bwd_dq(const BwdArgs& a) { FA_DISPATCH(launch_dq_t, a); }

}  // namespace fa
