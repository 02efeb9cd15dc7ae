// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation
// (pure host code that runs before anything is enqueued) and dispatch to the
// kernel launchers.  Check order: NULL pointers, shape/dtype/scale,
// alignment, workspace, overlaps.

#include <climits>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include <algorithm>

#include "../../include/fa.h"
#include "fa_decode.hpp"
#include "fa_launch.hpp"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

struct Buf {
  const void* p;
  uintptr_t bytes;
  uintptr_t align;
};

bool overlaps(const Buf& a, const Buf& b) {
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

struct Shape {
  int B, H, N, d;
  fa_dtype dtype;
  uintptr_t tensor_bytes() const { return (uintptr_t)B * H * N * d * (dtype == FA_BF16 ? 2 : 4); }
  uintptr_t row_bytes() const { return (uintptr_t)B * H * N * 4; }
  uintptr_t mask_bytes() const { const uintptr_t t = (N + 127) / 128; return t * t; }
};

// The kernels address the rows of one head through 32-bit byte offsets into
// a buffer descriptor (rows up to the next multiple of 256 past N are formed,
// and read as zeros), so one head's rows, rounded up to 256, must span fewer
// than 2^32 bytes.
bool head_fits_u32(long long rows, int d, unsigned elem) {
  const unsigned long long padded = ((unsigned long long)rows + 255) / 256 * 256;
  return padded * (unsigned long long)d * elem <= 0xFFFFFFFFull;
}

fa_status check_shape(const Shape& s, float scale) {
  if (s.dtype != FA_BF16 && s.dtype != FA_FP32) return FA_ERR_DTYPE;
  if (s.B < 1 || s.H < 1 || s.N < 1) return FA_ERR_SHAPE;
  if (s.d != 64 && s.d != 128) return FA_ERR_HEAD_DIM;
  const long long bh = (long long)s.B * s.H;
  const long long tiles = (s.N + 127LL) / 128;
  if (bh > INT_MAX || (long long)s.N * s.d > INT_MAX || bh * tiles > INT_MAX ||
      bh * s.N > INT_MAX || !head_fits_u32(s.N, s.d, s.dtype == FA_BF16 ? 2 : 4))
    return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  return FA_OK;
}

// ins/outs: every listed buffer must be non-NULL (callers list the optional
// block mask only when present); the workspace is checked separately.
fa_status check_buffers(std::initializer_list<Buf> ins, std::initializer_list<Buf> outs) {
  for (const Buf& b : ins)
    if (!b.p) return FA_ERR_NULL;
  for (const Buf& b : outs)
    if (!b.p) return FA_ERR_NULL;
  return FA_OK;
}

fa_status check_layout(std::initializer_list<Buf> ins, std::initializer_list<Buf> outs,
                       const Buf* ws, bool ws_is_output, size_t ws_need) {
  for (const Buf& b : ins)
    if ((uintptr_t)b.p % b.align) return FA_ERR_ALIGN;
  for (const Buf& b : outs)
    if ((uintptr_t)b.p % b.align) return FA_ERR_ALIGN;
  if (ws && (!ws->p || ws->bytes < ws_need || (uintptr_t)ws->p % 16)) return FA_ERR_WORKSPACE;
  for (const Buf& o : outs) {
    for (const Buf& i : ins)
      if (overlaps(o, i)) return FA_ERR_ALIAS;
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return FA_ERR_ALIAS;
    if (ws && overlaps(o, *ws)) return FA_ERR_ALIAS;
  }
  if (ws && ws_is_output)
    for (const Buf& i : ins)
      if (overlaps(*ws, i)) return FA_ERR_ALIAS;
  return FA_OK;
}

fa::BwdArgs bwd_args(const Shape& s, float scale, int causal, const unsigned char* mask,
                     void* stream) {
  fa::BwdArgs a{};
  a.mask = mask;
  a.BH = s.B * s.H; a.N = s.N; a.d = s.d; a.T = (s.N + 127) / 128;
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = s.dtype == FA_BF16;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

#define FA_TRY(expr)                 \
  do {                               \
    const fa_status st_ = (expr);    \
    if (st_ != FA_OK) return st_;    \
  } while (0)

// Dropout probability p in [0, 1) and seed -> kernel parameters.
fa_status dropout_params(float p, unsigned long long seed, fa::Dropout* out) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return FA_ERR_ARG;
  const double t = std::floor((double)p * 65536.0);
  out->on = true;
  out->key0 = (uint32_t)(seed & 0xFFFFFFFFull);
  out->key1 = (uint32_t)(seed >> 32);
  out->thresh = t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
  out->inv_keep = (float)(1.0 / (1.0 - (double)p));
  return FA_OK;
}

fa_status fwd_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                   int H, int Hkv, int N, int d, float scale, int causal,
                   const unsigned char* block_mask, fa_dtype dtype, const fa::Dropout& drop,
                   void* stream, void* workspace = nullptr, size_t workspace_bytes = 0);

fa_status bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, const unsigned char* block_mask,
                   fa_dtype dtype, void* workspace, size_t workspace_bytes,
                   const fa::Dropout& drop, void* stream, bool seq_splits = true);

// Key/value head count: >= 1 and dividing the query head count.
fa_status check_kv_heads(int H, int Hkv) {
  if (Hkv < 1 || H < 1 || H % Hkv) return FA_ERR_SHAPE;
  return FA_OK;
}

// Work-groups per key/value head and key block in the grouped dK/dV pass:
// with fewer than two work-groups per compute unit (about 512 on the 256-CU
// MI355X) the group's query heads are divided among several work-groups.
int gqa_split(int B, int H, int Hkv, int N) {
  const int G = H / Hkv;
  if (G <= 1) return 1;
  const long long groups = (long long)B * Hkv * ((N + 127) / 128);
  if (groups >= 512) return 1;
  return (int)std::min<long long>(G, (512 + groups - 1) / groups);
}

// Sequence splits (bf16 only): a shape whose query or key blocks would fill
// fewer than the 256 compute units of the MI355X (one GPU's share of a long
// sequence, e.g. one head of 16K rows) gets more work-groups by cutting each
// key block's query tiles (dK/dV) and each query block's key tiles (dQ) into
// runs; a run's work-group writes an fp32 partial and a reduction kernel adds
// the partials in a fixed order, so results stay deterministic.  The split
// count aims at `target` work-groups, at most 8 runs and at least `min_run`
// tiles per run.
constexpr int kCUs = 256;

int run_split(long long blocks, long long target, int tiles, int min_run) {
  if (blocks >= kCUs) return 1;
  long long sp = std::min<long long>((target + blocks - 1) / blocks, 8);
  sp = std::min<long long>(sp, std::max(1, tiles / min_run));
  return (int)std::max<long long>(1, sp);
}

// Backward work split and workspace layout: D (4 bytes per query row,
// rounded up to 256 bytes), then the dK/dV partials, then the dQ partials.
struct BwdPlan {
  int kv = 1, q = 1;            // dK/dV split (grouped heads or query tiles), dQ split
  size_t kv_off = 0, q_off = 0;
  size_t bytes = 0;             // workspace needed
};

BwdPlan bwd_plan(const Shape& s, int Hkv, bool seq_splits) {
  BwdPlan p;
  p.kv = gqa_split(s.B, s.H, Hkv, s.N);
  if (seq_splits && s.dtype == FA_BF16) {
    const int nb = (s.N + 127) / 128;
    if (Hkv == s.H)             // one query head per key/value head
      p.kv = run_split((long long)s.B * s.H * nb, 2LL * kCUs * (s.d == 64 ? 2 : 1), nb, 4);
    p.q = run_split((long long)s.B * s.H * nb, 4LL * kCUs, (s.N + 63) / 64, 8);
  }
  const size_t rows = ((size_t)s.row_bytes() + 255) / 256 * 256;
  p.kv_off = rows;
  p.q_off = rows + (p.kv > 1 ? (size_t)2 * p.kv * s.B * Hkv * s.N * s.d * 4 : 0);
  const size_t qb = p.q > 1 ? (size_t)p.q * s.B * s.H * s.N * s.d * 4 : 0;
  p.bytes = (p.kv == 1 && p.q == 1) ? (size_t)s.row_bytes() : p.q_off + qb;
  return p;
}

// Forward split (bf16, no dropout): with fewer than 256 query blocks (of 256
// rows in the ping-pong kernel, d = 128 without a block mask; of 128 rows in
// the four-wave kernel otherwise), each block's key tiles are cut into runs
// (at most 8, at least 8 tiles of 64 keys each), aiming at 512 work-groups
// for the ping-pong kernel (one per CU) and 1024 for the four-wave kernel
// (two per CU); the runs' fp32 O and LSE go to the workspace (O first, then
// LSE) and a combine kernel merges them in run order.
struct FwdPlan {
  int runs = 1;
  size_t lse_off = 0, bytes = 0;   // bytes = 0: no split
};

FwdPlan fwd_plan(const Shape& s, bool masked, bool dropout) {
  FwdPlan p;
  if (s.dtype != FA_BF16 || dropout) return p;
  const bool pp = s.d == 128 && !masked;
  const int br = pp ? 256 : 128;
  p.runs = run_split((long long)s.B * s.H * ((s.N + br - 1) / br), (pp ? 2LL : 4LL) * kCUs,
                     (s.N + 63) / 64, 8);
  if (p.runs == 1) return p;
  const size_t rows = (size_t)s.B * s.H * s.N;
  p.lse_off = (size_t)p.runs * rows * s.d * 4;
  p.bytes = p.lse_off + (size_t)p.runs * rows * 4;
  return p;
}

}  // namespace

FA_EXPORT fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int B, int H, int N, int d, float scale, int causal,
                           const unsigned char* block_mask, fa_dtype dtype, void* stream) {
  return fwd_impl(Q, K, V, O, LSE, B, H, H, N, d, scale, causal, block_mask, dtype,
                  fa::Dropout{}, stream);
}

FA_EXPORT size_t fa_fwd_workspace_bytes(int B, int H, int N, int d) {
  const Shape s{B, H, N, d, FA_BF16};
  if (check_shape(s, 1.0f) != FA_OK) return 0;
  return std::max(fwd_plan(s, false, false).bytes, fwd_plan(s, true, false).bytes);
}

FA_EXPORT fa_status fa_fwd_ws(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int B, int H, int N, int d, float scale, int causal,
                              const unsigned char* block_mask, fa_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!workspace && workspace_bytes) return FA_ERR_WORKSPACE;
  return fwd_impl(Q, K, V, O, LSE, B, H, H, N, d, scale, causal, block_mask, dtype,
                  fa::Dropout{}, stream, workspace, workspace_bytes);
}

FA_EXPORT fa_status fa_fwd_dropout(const void* Q, const void* K, const void* V, void* O,
                                   float* LSE, int B, int H, int N, int d, float scale,
                                   int causal, const unsigned char* block_mask, float dropout_p,
                                   unsigned long long seed, fa_dtype dtype, void* stream) {
  fa::Dropout drop;
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}}, {{O, 0, 0}, {LSE, 0, 0}}));
  FA_TRY(check_shape(Shape{B, H, N, d, dtype}, scale));
  FA_TRY(dropout_params(dropout_p, seed, &drop));
  return fwd_impl(Q, K, V, O, LSE, B, H, H, N, d, scale, causal, block_mask, dtype, drop,
                  stream);
}

namespace {

fa_status fwd_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                   int H, int Hkv, int N, int d, float scale, int causal,
                   const unsigned char* block_mask, fa_dtype dtype, const fa::Dropout& drop,
                   void* stream, void* workspace, size_t workspace_bytes) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}}, {{O, 0, 0}, {LSE, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  FA_TRY(check_kv_heads(H, Hkv));
  const uintptr_t tb = s.tensor_bytes(), lb = s.row_bytes();
  const uintptr_t kvb = tb / H * Hkv;
  const Buf q{Q, tb, 16}, k{K, kvb, 16}, v{V, kvb, 16}, o{O, tb, 16}, l{LSE, lb, 4};
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  // A workspace, when given, is checked like any output (alignment, no
  // overlap); the run split is used when it is large enough.
  const Buf ws{workspace, workspace_bytes, 16};
  FA_TRY(check_layout({q, k, v, m}, {o, l}, workspace ? &ws : nullptr, true, 0));
  const FwdPlan plan = fwd_plan(s, block_mask != nullptr, drop.on);
  const bool split = workspace && plan.bytes && workspace_bytes >= plan.bytes;

  fa::FwdArgs a{};
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
  a.mask = block_mask;
  a.BH = B * H; a.N = N; a.d = d; a.T = (N + 127) / 128;
  a.G = H / Hkv;
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = dtype == FA_BF16;
  a.drop = drop;
  a.stream = static_cast<hipStream_t>(stream);
  if (split) {
    a.fsplit = plan.runs;
    a.opart = static_cast<float*>(workspace);
    a.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.lse_off);
  }
  return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

FA_EXPORT size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  const Shape s{B, H, N, d, FA_BF16};
  if (check_shape(s, 1.0f) != FA_OK) return 0;
  return bwd_plan(s, H, true).bytes;
}

FA_EXPORT fa_status fa_bwd_splits(int B, int Hq, int Hkv, int N, int d, fa_dtype dtype,
                                  int* dkdv_split, int* dq_split) {
  if (!dkdv_split || !dq_split) return FA_ERR_NULL;
  const Shape s{B, Hq, N, d, dtype};
  FA_TRY(check_shape(s, 1.0f));
  FA_TRY(check_kv_heads(Hq, Hkv));
  const BwdPlan p = bwd_plan(s, Hkv, true);
  *dkdv_split = p.kv;
  *dq_split = p.q;
  return FA_OK;
}

FA_EXPORT fa_status fa_bwd_preprocess(const void* O, const void* dO, int B, int H, int N, int d,
                                      fa_dtype dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  FA_TRY(check_buffers({{O, 0, 0}, {dO, 0, 0}}, {}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, 1.0f));
  const uintptr_t tb = s.tensor_bytes();
  const Buf ws{workspace, workspace_bytes, 16};
  FA_TRY(check_layout({{O, tb, 16}, {dO, tb, 16}}, {}, &ws, true, s.row_bytes()));
  fa::BwdArgs a = bwd_args(s, 1.0f, 0, nullptr, stream);
  a.o = O; a.dout = dO; a.delta = static_cast<float*>(workspace);
  return fa::launch_bwd_preprocess(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

FA_EXPORT fa_status fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, void* dK, void* dV, int B, int H, int N, int d,
                                float scale, int causal, const unsigned char* block_mask,
                                fa_dtype dtype, const void* workspace, size_t workspace_bytes,
                                void* stream) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dK, 0, 0}, {dV, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  const uintptr_t tb = s.tensor_bytes(), lb = s.row_bytes();
  const Buf ws{workspace, workspace_bytes, 16};
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  FA_TRY(check_layout({{Q, tb, 16}, {K, tb, 16}, {V, tb, 16}, {dO, tb, 16}, {LSE, lb, 4}, m},
                      {{dK, tb, 16}, {dV, tb, 16}}, &ws, false, lb));
  fa::BwdArgs a = bwd_args(s, scale, causal, block_mask, stream);
  a.q = Q; a.k = K; a.v = V; a.dout = dO; a.lse = LSE; a.dk = dK; a.dv = dV;
  a.delta = static_cast<float*>(const_cast<void*>(workspace));
  return fa::launch_bwd_dkdv(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

FA_EXPORT fa_status fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                              const float* LSE, void* dQ, int B, int H, int N, int d, float scale,
                              int causal, const unsigned char* block_mask, fa_dtype dtype,
                              const void* workspace, size_t workspace_bytes, void* stream) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dQ, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  const uintptr_t tb = s.tensor_bytes(), lb = s.row_bytes();
  const Buf ws{workspace, workspace_bytes, 16};
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  FA_TRY(check_layout({{Q, tb, 16}, {K, tb, 16}, {V, tb, 16}, {dO, tb, 16}, {LSE, lb, 4}, m},
                      {{dQ, tb, 16}}, &ws, false, lb));
  fa::BwdArgs a = bwd_args(s, scale, causal, block_mask, stream);
  a.q = Q; a.k = K; a.v = V; a.dout = dO; a.lse = LSE; a.dq = dQ;
  a.delta = static_cast<float*>(const_cast<void*>(workspace));
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

FA_EXPORT fa_status fa_bwd_dq_and_d(const void* Q, const void* K, const void* V, const void* O,
                                    const void* dO, const float* LSE, void* dQ, int B, int H,
                                    int N, int d, float scale, int causal,
                                    const unsigned char* block_mask, fa_dtype dtype,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {O, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dQ, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  const uintptr_t tb = s.tensor_bytes(), lb = s.row_bytes();
  const Buf ws{workspace, workspace_bytes, 16};
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  FA_TRY(check_layout(
      {{Q, tb, 16}, {K, tb, 16}, {V, tb, 16}, {O, tb, 16}, {dO, tb, 16}, {LSE, lb, 4}, m},
      {{dQ, tb, 16}}, &ws, true, lb));
  fa::BwdArgs a = bwd_args(s, scale, causal, block_mask, stream);
  a.q = Q; a.k = K; a.v = V; a.o = O; a.dout = dO; a.lse = LSE; a.dq = dQ;
  a.delta = static_cast<float*>(workspace);
  a.dq_forms_delta = true;
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

FA_EXPORT fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                           int B, int H, int N, int d, float scale, int causal,
                           const unsigned char* block_mask, fa_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, scale, causal, block_mask,
                  dtype, workspace, workspace_bytes, fa::Dropout{}, stream);
}

FA_EXPORT fa_status fa_bwd_static(const void* Q, const void* K, const void* V, const void* O,
                                  const void* dO, const float* LSE, void* dQ, void* dK,
                                  void* dV, int B, int H, int N, int d, float scale, int causal,
                                  const unsigned char* block_mask, fa_dtype dtype,
                                  void* stream) {
  // The argument checks of fa_bwd come first, then the size limit, then the
  // (once per device) lookup of the static array's device address.
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {O, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dQ, 0, 0}, {dK, 0, 0}, {dV, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  if (s.row_bytes() > (uintptr_t)FA_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (fa::static_scratch(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, scale, causal, block_mask,
                  dtype, ws, FA_STATIC_SCRATCH_BYTES, fa::Dropout{}, stream,
                  /*seq_splits=*/false);
}

FA_EXPORT fa_status fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* LSE, void* dQ, void* dK,
                                   void* dV, int B, int H, int N, int d, float scale, int causal,
                                   const unsigned char* block_mask, float dropout_p,
                                   unsigned long long seed, fa_dtype dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  fa::Dropout drop;
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {O, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dQ, 0, 0}, {dK, 0, 0}, {dV, 0, 0}}));
  FA_TRY(check_shape(Shape{B, H, N, d, dtype}, scale));
  FA_TRY(dropout_params(dropout_p, seed, &drop));
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, scale, causal, block_mask,
                  dtype, workspace, workspace_bytes, drop, stream);
}

FA_EXPORT size_t fa_bwd_gqa_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  const Shape s{B, Hq, N, d, FA_BF16};
  if (check_shape(s, 1.0f) != FA_OK || check_kv_heads(Hq, Hkv) != FA_OK) return 0;
  return bwd_plan(s, Hkv, true).bytes;
}

FA_EXPORT fa_status fa_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                               const unsigned char* block_mask, fa_dtype dtype, void* stream) {
  return fwd_impl(Q, K, V, O, LSE, B, Hq, Hkv, N, d, scale, causal, block_mask, dtype,
                  fa::Dropout{}, stream);
}

FA_EXPORT fa_status fa_bwd_gqa(const void* Q, const void* K, const void* V, const void* O,
                               const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                               int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                               const unsigned char* block_mask, fa_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, Hq, Hkv, N, d, scale, causal, block_mask,
                  dtype, workspace, workspace_bytes, fa::Dropout{}, stream);
}

namespace {

fa_status bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, const unsigned char* block_mask,
                   fa_dtype dtype, void* workspace, size_t workspace_bytes,
                   const fa::Dropout& drop, void* stream, bool seq_splits) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}, {O, 0, 0}, {dO, 0, 0}, {LSE, 0, 0}},
                       {{dQ, 0, 0}, {dK, 0, 0}, {dV, 0, 0}}));
  const Shape s{B, H, N, d, dtype};
  FA_TRY(check_shape(s, scale));
  FA_TRY(check_kv_heads(H, Hkv));
  const uintptr_t tb = s.tensor_bytes(), lb = s.row_bytes();
  const uintptr_t kvb = tb / H * Hkv;
  // The sequence splits are used when the workspace holds their partials
  // (fa_bwd_workspace_bytes and fa_bwd_gqa_workspace_bytes include them);
  // with less, down to D alone, the passes run unsplit.  The grouped-head
  // split of dK/dV is required.
  BwdPlan plan = bwd_plan(s, Hkv, seq_splits);
  if (seq_splits && workspace_bytes < plan.bytes) plan = bwd_plan(s, Hkv, false);
  const size_t need = plan.bytes;
  const Buf ws{workspace, workspace_bytes, 16};
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  FA_TRY(check_layout(
      {{Q, tb, 16}, {K, kvb, 16}, {V, kvb, 16}, {O, tb, 16}, {dO, tb, 16}, {LSE, lb, 4}, m},
      {{dQ, tb, 16}, {dK, kvb, 16}, {dV, kvb, 16}}, &ws, true, need));

  fa::BwdArgs a = bwd_args(s, scale, causal, block_mask, stream);
  a.G = H / Hkv;
  a.gsplit = plan.kv;
  if (plan.kv > 1) a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.kv_off);
  a.ksplit = plan.q;
  if (plan.q > 1) a.qpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.q_off);
  a.q = Q; a.k = K; a.v = V; a.o = O; a.dout = dO; a.lse = LSE;
  a.dq = dQ; a.dk = dK; a.dv = dV;
  a.delta = static_cast<float*>(workspace);
  a.drop = drop;
  // The dQ pass forms D itself (bit-identical to the preprocess kernel's) and
  // writes it for the dK/dV pass, so it runs first and no preprocess runs.
  a.dq_forms_delta = true;
  if (fa::launch_bwd_dq(a) != hipSuccess) return FA_ERR_LAUNCH;
  if (fa::launch_bwd_dkdv(a) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// FP8 forward
// ---------------------------------------------------------------------------

FA_EXPORT fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8,
                               const float* q_scale, const float* k_scale,
                               const float* v_scale, void* O, float* LSE, int B, int H, int N,
                               int d, float scale, int causal, const unsigned char* block_mask,
                               void* stream) {
  FA_TRY(check_buffers({{Q8, 0, 0}, {K8, 0, 0}, {Vt8, 0, 0}, {q_scale, 0, 0}, {k_scale, 0, 0},
                        {v_scale, 0, 0}},
                       {{O, 0, 0}, {LSE, 0, 0}}));
  const Shape s{B, H, N, d, FA_BF16};
  FA_TRY(check_shape(s, scale));
  if (N % 16) return FA_ERR_SHAPE;      // V^T rows must start on 16-byte boundaries
  const uintptr_t cb = s.tensor_bytes() / 2, ob = s.tensor_bytes(), lb = s.row_bytes();
  const uintptr_t T = (N + 127) / 128;
  const uintptr_t sb = (uintptr_t)B * H * T * 4;
  const Buf m{block_mask, block_mask ? s.mask_bytes() : 0, 1};
  FA_TRY(check_layout({{Q8, cb, 16}, {K8, cb, 16}, {Vt8, cb, 16}, {q_scale, sb, 4},
                       {k_scale, sb, 4}, {v_scale, (uintptr_t)B * H * 4, 4}, m},
                      {{O, ob, 16}, {LSE, lb, 4}}, nullptr, false, 0));
  fa::Fp8FwdArgs a{};
  a.q = static_cast<const uint8_t*>(Q8);
  a.k = static_cast<const uint8_t*>(K8);
  a.vt = static_cast<const uint8_t*>(Vt8);
  a.sq = q_scale; a.sk = k_scale; a.sv = v_scale;
  a.o = O; a.lse = LSE; a.mask = block_mask;
  a.BH = B * H; a.N = N; a.d = d; a.T = (int)T;
  a.scale = scale;
  a.causal = causal != 0;
  a.stream = static_cast<hipStream_t>(stream);
  return fa::launch_fwd_fp8(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------

namespace fa {

DecodePlan decode_plan(int B, int Hkv, int R, int Nkv, int num_splits) {
  constexpr int kTile = 128;               // keys per tile (bf16 kernels)
  constexpr int kMinChunk = 512;           // automatic chunks span at least 4 tiles
  constexpr long long kMaxAuto = 128;
  // About 8 work-groups per compute unit of the 256-CU MI355X, so chunks of
  // sequences of different lengths balance over the device.
  constexpr long long kTargetGroups = 2048;
  const long long pairs = (long long)B * Hkv * ((R + 31) / 32);
  const int tiles = (Nkv + kTile - 1) / kTile;
  long long S = num_splits;
  if (S <= 0) {
    S = std::min(kMaxAuto, (kTargetGroups + pairs - 1) / pairs);
    S = std::min<long long>(S, std::max(1, (Nkv + kMinChunk - 1) / kMinChunk));
  }
  S = std::max<long long>(1, std::min<long long>(S, tiles));
  const int per = (int)((Nkv + S - 1) / S);
  const int chunk = (per + kTile - 1) / kTile * kTile;
  return DecodePlan{(Nkv + chunk - 1) / chunk, chunk};
}

}  // namespace fa

namespace {

struct DecShape {
  int B, Hq, Hkv, Nq, Nkv, d;
  fa_dtype dtype;
  long long R() const { return (long long)(Hq / Hkv) * Nq; }   // call once Hq % Hkv == 0
  uintptr_t elem() const { return dtype == FA_BF16 ? 2 : 4; }
  uintptr_t q_bytes() const { return (uintptr_t)B * Hq * Nq * d * elem(); }
  uintptr_t kv_bytes() const { return (uintptr_t)B * Hkv * Nkv * d * elem(); }
  uintptr_t rows() const { return (uintptr_t)B * Hq * Nq; }
};

fa_status check_decode_shape(const DecShape& s, int num_splits) {
  if (s.dtype != FA_BF16 && s.dtype != FA_FP32) return FA_ERR_DTYPE;
  if (s.B < 1 || s.Hq < 1 || s.Hkv < 1 || s.Nq < 1 || s.Nkv < 1) return FA_ERR_SHAPE;
  if (s.Hq % s.Hkv) return FA_ERR_SHAPE;
  if (s.d != 64 && s.d != 128) return FA_ERR_HEAD_DIM;
  // Each product is formed only once its factors are known to be small
  // enough not to overflow 64 bits.
  const long long bq = (long long)s.B * s.Hq;
  if (bq > INT_MAX || bq * s.Nq > INT_MAX || bq * s.Nq * s.d > INT_MAX) return FA_ERR_SHAPE;
  const long long pairs = (long long)s.B * s.Hkv;            // <= B * Hq
  const long long qgroups = pairs * ((s.R() + 31) / 32);     // R <= Hq * Nq
  if (qgroups > INT_MAX || qgroups * ((s.Nkv + 127LL) / 128) > INT_MAX ||
      (long long)s.Nkv * s.d > INT_MAX || !head_fits_u32(s.Nkv, s.d, (unsigned)s.elem()) ||
      !head_fits_u32(s.R(), s.d, (unsigned)s.elem()))
    return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
  return FA_OK;
}

size_t decode_workspace(const DecShape& s, const fa::DecodePlan& p) {
  return p.S > 1 ? (size_t)s.rows() * p.S * (s.d + 1) * 4 : 0;
}

}  // namespace

FA_EXPORT int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                                   int num_splits) {
  const DecShape s{B, Hq, Hkv, Nq, Nkv, d, FA_BF16};
  if (check_decode_shape(s, num_splits) != FA_OK) return 0;
  return fa::decode_plan(B, Hkv, (int)s.R(), Nkv, num_splits).S;
}

FA_EXPORT size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                                           int num_splits) {
  const DecShape s{B, Hq, Hkv, Nq, Nkv, d, FA_BF16};
  if (check_decode_shape(s, num_splits) != FA_OK) return 0;
  return decode_workspace(s, fa::decode_plan(B, Hkv, (int)s.R(), Nkv, num_splits));
}

FA_EXPORT fa_status fa_decode(const void* Q, const void* K, const void* V, const int* seqlens,
                              void* O, float* LSE, int B, int Hq, int Hkv, int Nq, int Nkv,
                              int d, float scale, int causal, int num_splits, fa_dtype dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  FA_TRY(check_buffers({{Q, 0, 0}, {K, 0, 0}, {V, 0, 0}}, {{O, 0, 0}, {LSE, 0, 0}}));
  const DecShape s{B, Hq, Hkv, Nq, Nkv, d, dtype};
  FA_TRY(check_decode_shape(s, num_splits));
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  const fa::DecodePlan plan = fa::decode_plan(B, Hkv, (int)s.R(), Nkv, num_splits);
  const size_t need = decode_workspace(s, plan);
  const Buf q{Q, s.q_bytes(), 16}, k{K, s.kv_bytes(), 16}, v{V, s.kv_bytes(), 16};
  const Buf o{O, s.q_bytes(), 16}, l{LSE, s.rows() * 4, 4};
  const Buf sl{seqlens, seqlens ? (uintptr_t)B * 4 : 0, 4};
  const Buf ws{workspace, workspace_bytes, 16};
  FA_TRY(check_layout({q, k, v, sl}, {o, l}, need ? &ws : nullptr, true, need));

  fa::DecodeArgs a{};
  a.q = Q; a.k = K; a.v = V;
  a.seqlens = reinterpret_cast<const int32_t*>(seqlens);
  a.o = O; a.lse = LSE;
  a.opart = need ? static_cast<float*>(workspace) : nullptr;
  a.lpart = need ? static_cast<float*>(workspace) + s.rows() * plan.S * d : nullptr;
  a.pairs = B * Hkv;
  a.Hkv = Hkv; a.Nq = Nq; a.R = (int)s.R(); a.Nkv = Nkv; a.d = d;
  a.S = plan.S; a.chunk = plan.chunk;
  a.scale = scale;
  a.causal = causal != 0;
  a.bf16 = dtype == FA_BF16;
  a.stream = static_cast<hipStream_t>(stream);
  return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

FA_EXPORT const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE:
      return "invalid shape (sizes must be >= 1 and fit int32, one head's rows must span "
             "under 4 GiB; Hq a multiple of Hkv)";
    case FA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_ALIGN: return "misaligned tensor pointer (16 bytes; LSE 4 bytes)";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ARG:
      return "scale must be finite; dropout probability in [0, 1); num_splits in [0, 1024]";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_SCRATCH:
      return "the sizes need more than the library's static scratch (FA_STATIC_SCRATCH_BYTES)";
    case FA_STATUS_INT_MIN_:
    case FA_STATUS_INT_MAX_: break;
  }
  return "unknown status";
}
