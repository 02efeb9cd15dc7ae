// fa_decode.hip -- split-KV attention of a few new query rows against a long
// key/value cache, with grouped key/value heads (inference decode).
//
// In decode each request reads its whole cache to produce one (or a few)
// output rows, so the work is bound by HBM bandwidth, not by the matrix
// cores: the cache has to stream through once at full rate, and a cache
// head has to serve all G = Hq / Hkv query heads that share it from that one
// read (the week-13 page's note on decode intensity and GQA,
// snula.amonoc.com/course/ru/week-13.html).  The R = G * Nq query rows of a
// (batch, cache head) pair are contiguous in Q ([B, Hq, Nq, d]: heads
// kvh*G .. kvh*G+G-1), so they form one 32-column query tile (more tiles when
// R > 32).
//
// fa_decode_split_kernel: one work-group per (batch, cache head, query tile,
// key chunk).  Its waves stream the chunk's K/V tiles (32 keys per wave per
// tile) through a ring of LDS buffers with direct-to-LDS loads, a few tiles
// ahead, and each wave keeps its own running (max, sum, O^T) over its keys:
//   S^T = K_w Q^T (MFMA, keys as rows, one query per lane),
//   online softmax in the log2 domain, O^T += V_w^T P^T (MFMA).
// At the end the waves' states are merged through LDS with the two-part rule
// of the FlashAttention reading guide (xyznot.com/tr/paper/2205.14135,
// "Artımsal Softmax Takibi"); the work-group writes either the final O and
// LSE (one chunk) or the chunk's normalised O and its LSE (several chunks).
//
// fa_decode_combine_kernel: one wave per output row merges the chunks'
// (LSE_s, O_s) with the same rule: M = max_s LSE_s,
// O = sum_s e^(LSE_s - M) O_s / sum_s e^(LSE_s - M), LSE = M + ln(sum ...).
//
// Masking: sequence b has L_b valid cache rows; with causal masking the Nq
// new tokens are the last Nq positions, so query row nq sees keys
// j <= L_b - Nq + nq.  A row that sees no key gets O = 0, LSE = -inf.

#include <algorithm>

#include "fa_common.hpp"
#include "fa_decode.hpp"

namespace fa {

// WAVES waves per work-group (32 keys each per tile), a ring of NBUF [K, V]
// tile buffers.
template <typename T, int D, int WAVES, int NBUF>
struct DecCfg {
  static constexpr int RB = D * (int)sizeof(T);
  static constexpr int KT = 32 * WAVES;                       // keys per tile
  static constexpr int TB = KT * RB;                          // bytes of K (or V) per tile
  static constexpr int LOADS = 2 * TB / 1024 / WAVES;        // buffer loads per wave per tile
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of 2 to 4 buffers");
  static_assert(2 * TB * NBUF <= 160 * 1024, "ring must fit in LDS");
  static_assert((NBUF - 2) * LOADS <= 63, "vmcnt immediate is 6 bits");
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

template <typename T, int D, bool CAUSAL, int WAVES, int NBUF>
__global__ void __launch_bounds__(64 * WAVES)
fa_decode_split_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                       const T* __restrict__ V, const int32_t* __restrict__ seqlens,
                       T* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart,
                       float* __restrict__ Lpart, int Hkv, int Nq, int R, int RG, int Nkv,
                       int S, int chunk, int P, float c /* score_coef(scale) */) {
  using E = Elem<T>;
  using frag = typename E::frag;
  using Cfg = DecCfg<T, D, WAVES, NBUF>;
  constexpr int RB = Cfg::RB, KT = Cfg::KT, TB = Cfg::TB;
  constexpr int NT = D / 16, ND = D / 32;

  __shared__ __attribute__((aligned(1024))) unsigned char buf0[2 * TB];   // [K, V]
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[2 * TB];
  __shared__ __attribute__((aligned(1024))) unsigned char buf2[NBUF > 2 ? 2 * TB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char buf3[NBUF > 3 ? 2 * TB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  // Work-group order: blocks of P (batch, cache head, query tile) groups,
  // about one device-full of work-groups per block; within a block, chunk
  // index slowest.  So every group's first chunk is dispatched before any
  // second chunk of its block (the chunks that are empty or short, past the
  // end of shorter sequences, come last and fill in the tail), while the
  // work-groups in flight at any time stay within a few blocks of groups.
  const int PG = (int)(gridDim.x / S);
  const int blk = blockIdx.x / (P * S);
  const int pb0 = blk * P;
  const int Pb = min(P, PG - pb0);
  const int within = blockIdx.x - pb0 * S;
  const int s = within / Pb;
  const int rest = pb0 + (within - s * Pb);
  const int rg = rest % RG;
  const int bkv = rest / RG;                 // b * Hkv + kvh
  const int b = bkv / Hkv;

  int L = seqlens ? seqlens[b] : Nkv;
  L = min(max(L, 0), Nkv);
  const int kb = s * chunk;
  const int ke = min(L, kb + chunk);
  const int ntiles = ke > kb ? (ke - kb + KT - 1) / KT : 0;

  // This lane's query row r of the (batch, cache head) group and the keys it sees.
  const int r = 32 * rg + l32;
  const int nq = r % Nq;
  const int lim = min(ke, CAUSAL ? L - Nq + nq + 1 : L);     // keys < lim are visible
  const int min_lim = min(ke, CAUSAL ? L - Nq + 1 : L);       // over all rows

  const size_t head = (size_t)bkv * Nkv * D;
  const T* Kh = K + head;
  const T* Vh = V + head;

  // Query fragments (B operand, natural order): rows past R read as zero.
  const rsrc_t rq = make_rsrc(Q + (size_t)bkv * R * D, (uint32_t)R * RB);
  frag qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qf[t] = gload_frag<T>(rq, (uint32_t)r * RB + (16 * t + 8 * g) * sizeof(T));
  bool negs;
  c = split_coef(c, negs);   // c = |scale| log2(e); Q negated when scale < 0
  if (negs) {
#pragma unroll
    for (int t = 0; t < NT; ++t) negate(qf[t]);
  }

  auto stage = [&](int i, auto slot) {
    const int kv0 = kb + i * KT;
    const uint32_t left = (uint32_t)(ke - kv0) * RB;
    unsigned char* base = pick4(slot, buf0, buf1, buf2, buf3);
    stage_tile<T, D, KT, WAVES>(make_rsrc(Kh + (size_t)kv0 * D, left), base, w, lane);
    stage_tile<T, D, KT, WAVES>(make_rsrc(Vh + (size_t)kv0 * D, left), base + TB, w, lane);
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int bb = 0; bb < ND; ++bb) oacc[bb] = f32x16{};
  float m_run = neg_inf();   // running max of S*c over this wave's keys (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum

  // bf16: per-lane operand offsets computed once (the compiler then sees
  // every LDS read as an offset into one named buffer).
  constexpr bool kBf16 = sizeof(T) == 2;
  LaneOffsets<T, D> lo;
  if constexpr (kBf16) lo.init(lane);

  auto compute = [&](auto slot, int kv0) {
    const unsigned char* sK = pick4(slot, buf0, buf1, buf2, buf3) + 32 * w * RB;
    const unsigned char* sV = sK + TB;

    frag ak[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (kBf16) ak[t] = row_frag_at<T>(sK + lo.row[t]);
      else ak[t] = row_frag<T, D>(sK, l32, t, g);
    }
    sched_fence();
    f32x16 st = f32x16{};
#pragma unroll
    for (int t = 0; t < NT; ++t) st = E::mma(ak[t], qf[t], st);

    // Register e of this lane is key kv0 + 32 w + 4 g + 8 (e / 4) + e % 4.
    if (kv0 + KT > min_lim) {
      const int off = lim - (kv0 + 32 * w + 4 * g);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) >= off) st[e] = neg_inf();
    }

    float mx = neg_inf();
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[e]);
    const float m_new = fmaxf(m_run, max_xor32(mx) * c);
    if (m_new > m_run) {     // first visible key of the row included: 2^(-inf) = 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int bb = 0; bb < ND; ++bb) oacc[bb] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == neg_inf() ? 0.f : m_run;
    float ps[4] = {};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      st[e] = __builtin_amdgcn_exp2f(fmaf(st[e], c, -m_use));
      ps[e & 3] += st[e];
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    const frag p0 = E::from_c(st, 0), p1 = E::from_c(st, 1);
#pragma unroll
    for (int bb = 0; bb < ND; ++bb) {
      frag a0, a1;
      if constexpr (kBf16) {
        a0 = trans_frag_at(sV + lo.tr[bb][0], sV + lo.tr[bb][1]);
        a1 = trans_frag_at(sV + lo.tr[bb][0] + 16 * RB, sV + lo.tr[bb][1] + 16 * RB);
      } else {
        a0 = trans_frag<T, D>(sV, bb, 0, lane);
        a1 = trans_frag<T, D>(sV, bb, 1, lane);
      }
      oacc[bb] = E::mma(a0, p0, oacc[bb]);
      oacc[bb] = E::mma(a1, p1, oacc[bb]);
    }
  };

  // Ring of NBUF slots, tiles staged NBUF - 1 ahead.  At the top of tile i
  // this wave's loads of tiles i+1 .. i+NBUF-2 may still be in flight; wait
  // for the rest (vmcnt counts the direct-to-LDS loads until their data is
  // in LDS), then a barrier: all of tile i is in LDS and every wave has
  // finished tile i-1, whose slot receives tile i+NBUF-1.
  int i = 0;
  auto step = [&](auto slot) -> bool {
    constexpr int SL = decltype(slot)::value;
    if (i >= ntiles) return false;
    const int after = min(NBUF - 2, ntiles - 1 - i);
    if constexpr (NBUF >= 4) {
      if (after >= 2) wait_vmcnt<2 * Cfg::LOADS>();
      else if (after == 1) wait_vmcnt<Cfg::LOADS>();
      else wait_vmcnt<0>();
    } else if constexpr (NBUF == 3) {
      if (after >= 1) wait_vmcnt<Cfg::LOADS>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    // A plain barrier: __syncthreads() would also wait for the tiles still
    // in flight.  The clobber keeps LDS accesses on their side of it.
    asm volatile("s_barrier" ::: "memory");
    if (i + NBUF - 1 < ntiles) stage(i + NBUF - 1, IntTag<(SL + NBUF - 1) % NBUF>{});
    compute(slot, kb + i * KT);
    ++i;
    return true;
  };
  if (0 < ntiles) stage(0, IntTag<0>{});
  if constexpr (NBUF > 2) { if (1 < ntiles) stage(1, IntTag<1>{}); }
  if constexpr (NBUF > 3) { if (2 < ntiles) stage(2, IntTag<2>{}); }
  while (true) {
    if (!step(IntTag<0>{})) break;
    if (!step(IntTag<1>{})) break;
    if constexpr (NBUF > 2) { if (!step(IntTag<2 % NBUF>{})) break; }
    if constexpr (NBUF > 3) { if (!step(IntTag<3 % NBUF>{})) break; }
  }

  // ---- merge the waves' states -------------------------------------------
  // buf0 holds O^T of every wave as [w][query j][d] fp32 (16-byte chunks of a
  // row XOR-swizzled by j); buf1 the per-wave (m, l) of each query.
  __syncthreads();                            // every wave is done with the ring
  constexpr int NC = D / 4;                   // 16-byte chunks per row
  float* so = reinterpret_cast<float*>(buf0);
  float* sm = reinterpret_cast<float*>(buf1);
  float* sl = sm + WAVES * 32;
  const float l_tot = sum_xor32(l_run);
#pragma unroll
  for (int bb = 0; bb < ND; ++bb)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = (32 * bb + 8 * a + 4 * g) >> 2;
      *reinterpret_cast<f32x4*>(so + ((w * 32 + l32) * NC + (ch ^ (l32 & (NC - 1)))) * 4) =
          f32x4{oacc[bb][4 * a], oacc[bb][4 * a + 1], oacc[bb][4 * a + 2], oacc[bb][4 * a + 3]};
    }
  if (g == 0) {
    sm[w * 32 + l32] = m_run;
    sl[w * 32 + l32] = l_tot;
  }
  __syncthreads();

  const size_t row0 = (size_t)bkv * R + 32 * rg;
  for (int u = tid; u < 32 * NC; u += 64 * WAVES) {
    const int j = u / NC, ch = u % NC;
    if (32 * rg + j >= R) continue;
    float M = neg_inf();
#pragma unroll
    for (int x = 0; x < WAVES; ++x) M = fmaxf(M, sm[x * 32 + j]);
    float lsum = 0.f;
    f32x4 acc = f32x4{};
    if (M != neg_inf()) {
#pragma unroll
      for (int x = 0; x < WAVES; ++x) {
        const float e = __builtin_amdgcn_exp2f(sm[x * 32 + j] - M);   // 0 for an empty wave
        lsum += e * sl[x * 32 + j];
        acc += e * *reinterpret_cast<const f32x4*>(so + ((x * 32 + j) * NC + (ch ^ (j & (NC - 1)))) * 4);
      }
    }
    const float inv = lsum != 0.f ? 1.0f / lsum : 0.f;
    const float lse = lsum != 0.f ? (M + __builtin_amdgcn_logf(lsum)) * kLn2 : neg_inf();
    const size_t row = row0 + j;
    if (S == 1) {
      E::store4(O + row * D + 4 * ch, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      if (ch == 0) LSE[row] = lse;
    } else {
      *reinterpret_cast<f32x4*>(Opart + (row * S + s) * D + 4 * ch) = acc * inv;
      if (ch == 0) Lpart[row * S + s] = lse;
    }
  }
}

// One wave per output row: merge the S chunk results (module comment).
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
fa_decode_combine_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                         T* __restrict__ O, float* __restrict__ LSE, int rows, int S) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;                    // whole waves; no barriers below
  const float* lp = Lpart + (size_t)row * S;
  float M = neg_inf();
  for (int x = lane; x < S; x += 64) M = fmaxf(M, lp[x]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
  constexpr int PER = D / 64;
  float acc[PER] = {};
  float den = 0.f;
  if (M != neg_inf()) {
    const float* op = Opart + (size_t)row * S * D + lane;
    for (int x = 0; x < S; ++x) {
      const float e = __builtin_amdgcn_exp2f((lp[x] - M) * kLog2e);   // 0 for an empty chunk
      den += e;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = fmaf(e, op[(size_t)x * D + 64 * k], acc[k]);
    }
  }
  const float inv = den != 0.f ? 1.0f / den : 0.f;
  T* orow = O + (size_t)row * D + lane;
#pragma unroll
  for (int k = 0; k < PER; ++k) orow[64 * k] = (T)(acc[k] * inv);
  if (lane == 0) LSE[row] = den != 0.f ? M + __builtin_amdgcn_logf(den) * kLn2 : neg_inf();
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  constexpr int WAVES = 2;
  constexpr int NBUF = 2;
  const int RG = (a.R + 31) / 32;
  const dim3 grid((unsigned)a.pairs * RG * a.S), block(64 * WAVES);
  // Groups per ordering block: about 512 work-groups (two per compute unit).
  const int P = std::max(1, 512 / a.S);
  hipLaunchKernelGGL((fa_decode_split_kernel<T, D, CAUSAL, WAVES, NBUF>), grid, block, 0, a.stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.seqlens, static_cast<T*>(a.o), a.lse,
                     a.opart, a.lpart, a.Hkv, a.Nq, a.R, RG, a.Nkv, a.S, a.chunk, P,
                     score_coef(a.scale));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  const int rows = a.pairs * a.R;
  const int per = kThreads / 64;
  hipLaunchKernelGGL((fa_decode_combine_kernel<T, D>), dim3((rows + per - 1) / per),
                     dim3(kThreads), 0, a.stream, a.opart, a.lpart, static_cast<T*>(a.o), a.lse,
                     rows, a.S);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  return a.causal ? launch_decode_t<T, D, true>(a) : launch_decode_t<T, D, false>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.bf16) return a.d == 64 ? launch_decode_d<__bf16, 64>(a) : launch_decode_d<__bf16, 128>(a);
  return a.d == 64 ? launch_decode_d<float, 64>(a) : launch_decode_d<float, 128>(a);
}

}  // namespace fa
