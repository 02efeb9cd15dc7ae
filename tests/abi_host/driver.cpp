// Drives every entry point of the C ABI (include/fa.h) through its argument
// validation, built together with fa_api.cpp and the host-only launcher stubs
// (stub_launch.cpp) under the address and undefined-behaviour sanitizers.
// Invalid calls must return their status without reaching a launcher; valid
// calls (including the largest accepted sizes) must reach the launchers with
// the arguments the header documents.  Pointers are fake and never
// dereferenced: they only feed the alignment and overlap checks.
//
// Prints "ok <cases>" and exits 0 when every expectation holds.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa.h"
#include "fa_decode.hpp"
#include "fa_launch.hpp"

namespace fa {
extern int g_launches;
extern int g_scratch_lookups;
extern FwdArgs g_fwd;
extern BwdArgs g_bwd;
extern BwdArgs g_dq;   // the last dQ-pass launch
extern Fp8FwdArgs g_fp8;
extern DecodeArgs g_dec;
}  // namespace fa

static int g_cases = 0, g_fails = 0;

#define EXPECT(cond)                                                          \
  do {                                                                        \
    ++g_cases;                                                                \
    if (!(cond)) {                                                            \
      ++g_fails;                                                              \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
    }                                                                         \
  } while (0)

// Fake device pointers 64 GiB apart (so even the largest accepted tensors do
// not overlap), plus a byte offset for misalignment and overlap cases.
static void* P(int i, uintptr_t off = 0) {
  return reinterpret_cast<void*>(0x100000000000ull + (uintptr_t)i * (1ull << 36) + off);
}
static float* F(int i, uintptr_t off = 0) { return static_cast<float*>(P(i, off)); }
static const unsigned char* M(int i, uintptr_t off = 0) {
  return static_cast<const unsigned char*>(P(i, off));
}

// A call that must be rejected with `want` before any launch.
#define REJECT(want, call)                                                    \
  do {                                                                        \
    const int before = fa::g_launches;                                        \
    const fa_status st = (call);                                              \
    EXPECT(st == (want));                                                     \
    EXPECT(fa::g_launches == before);                                         \
  } while (0)

// A call that must pass validation and reach `n` launchers.
#define ACCEPT(n, call)                                                       \
  do {                                                                        \
    const int before = fa::g_launches;                                        \
    const fa_status st = (call);                                              \
    EXPECT(st == FA_OK);                                                      \
    EXPECT(fa::g_launches == before + (n));                                   \
  } while (0)

static fa_status fwd(int B, int H, int N, int d, float scale, fa_dtype dt,
                     const unsigned char* mask = nullptr, void* q = P(0), void* o = P(3)) {
  return fa_fwd(q, P(1), P(2), o, F(4), B, H, N, d, scale, 1, mask, dt, nullptr);
}

static fa_status bwd(int B, int H, int N, int d, float scale, fa_dtype dt, void* ws,
                     size_t wsb, void* dk = P(7)) {
  return fa_bwd(P(0), P(1), P(2), P(3), P(4), F(5), P(6), dk, P(8), B, H, N, d, scale, 0,
                nullptr, dt, ws, wsb, nullptr);
}

static void forward_cases() {
  ACCEPT(1, fwd(2, 16, 4096, 128, 0.0883883f, FA_BF16));
  EXPECT(fa::g_fwd.BH == 32 && fa::g_fwd.N == 4096 && fa::g_fwd.d == 128 && fa::g_fwd.T == 32);
  EXPECT(fa::g_fwd.G == 1 && fa::g_fwd.causal && fa::g_fwd.bf16 && !fa::g_fwd.drop.on);
  ACCEPT(1, fwd(1, 3, 1, 64, -0.5f, FA_FP32));               // any finite scale
  EXPECT(fa::g_fwd.scale == -0.5f && !fa::g_fwd.bf16);
  ACCEPT(1, fwd(1, 1, 8388352, 128, 0.1f, FA_FP32));         // largest fp32 head at d = 128
  REJECT(FA_ERR_SHAPE, fwd(1, 1, 8388353, 128, 0.1f, FA_FP32));
  ACCEPT(1, fwd(1, 1, 16776960, 128, 0.1f, FA_BF16));        // largest bf16 head at d = 128
  REJECT(FA_ERR_SHAPE, fwd(1, 1, 16776961, 128, 0.1f, FA_BF16));
  REJECT(FA_ERR_SHAPE, fwd(1, 65536, 32768, 64, 0.1f, FA_BF16));   // B*H*N > INT_MAX
  REJECT(FA_ERR_SHAPE, fwd(0, 1, 128, 64, 0.1f, FA_BF16));
  REJECT(FA_ERR_SHAPE, fwd(1, 1, -5, 64, 0.1f, FA_BF16));
  REJECT(FA_ERR_HEAD_DIM, fwd(1, 1, 128, 96, 0.1f, FA_BF16));
  REJECT(FA_ERR_DTYPE, fwd(1, 1, 128, 64, 0.1f, (fa_dtype)7));
  REJECT(FA_ERR_ARG, fwd(1, 1, 128, 64, NAN, FA_BF16));
  REJECT(FA_ERR_ARG, fwd(1, 1, 128, 64, -INFINITY, FA_BF16));
  REJECT(FA_ERR_ALIGN, fwd(1, 1, 128, 64, 0.1f, FA_BF16, nullptr, P(0, 8)));
  REJECT(FA_ERR_ALIAS, fwd(1, 1, 128, 64, 0.1f, FA_BF16, nullptr, P(0), P(0, 64)));
  REJECT(FA_ERR_ALIAS, fwd(1, 1, 256, 64, 0.1f, FA_BF16, M(3, 16)));   // mask inside O
  REJECT(FA_ERR_NULL, fa_fwd(nullptr, P(1), P(2), P(3), F(4), 1, 1, 128, 64, 0.1f, 0, nullptr,
                             FA_BF16, nullptr));
  ACCEPT(1, fa_fwd_dropout(P(0), P(1), P(2), P(3), F(4), 1, 2, 300, 64, 0.1f, 1, nullptr, 0.25f,
                           0x123456789abcull, FA_BF16, nullptr));
  EXPECT(fa::g_fwd.drop.on && fa::g_fwd.drop.key0 == 0x56789abcu && fa::g_fwd.drop.key1 == 0x1234u);
  EXPECT(fa::g_fwd.drop.thresh == 16384u);   // floor(0.25 * 2^16)
  ACCEPT(1, fa_fwd_dropout(P(0), P(1), P(2), P(3), F(4), 1, 2, 300, 64, 0.1f, 1, nullptr,
                           0.99999f, 1, FA_BF16, nullptr));
  EXPECT(fa::g_fwd.drop.thresh == 65535u);   // clamped below 2^16
  for (float p : {-0.1f, 1.0f, NAN, INFINITY})
    REJECT(FA_ERR_ARG, fa_fwd_dropout(P(0), P(1), P(2), P(3), F(4), 1, 2, 300, 64, 0.1f, 1,
                                      nullptr, p, 1, FA_BF16, nullptr));
  ACCEPT(1, fa_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 16, 4, 4096, 128, 0.1f, 1, nullptr,
                       FA_BF16, nullptr));
  EXPECT(fa::g_fwd.G == 4 && fa::g_fwd.BH == 32);
  REJECT(FA_ERR_SHAPE, fa_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 16, 3, 4096, 128, 0.1f, 1,
                                  nullptr, FA_BF16, nullptr));
}

static void backward_cases() {
  const size_t need = fa_bwd_workspace_bytes(2, 16, 4096, 128);
  EXPECT(need == 4ull * 2 * 16 * 4096);
  ACCEPT(2, bwd(2, 16, 4096, 128, 0.1f, FA_BF16, P(9), need));
  EXPECT(fa::g_bwd.delta == F(9) && fa::g_bwd.gsplit == 1 && fa::g_bwd.part == nullptr);
  EXPECT(fa::g_dq.dq_forms_delta && fa::g_dq.o == P(3) && fa::g_dq.delta == F(9));
  ACCEPT(2, bwd(2, 16, 4096, 128, -0.1f, FA_BF16, P(9), need));
  REJECT(FA_ERR_WORKSPACE, bwd(2, 16, 4096, 128, 0.1f, FA_BF16, P(9), need - 1));
  REJECT(FA_ERR_WORKSPACE, bwd(2, 16, 4096, 128, 0.1f, FA_BF16, nullptr, need));
  REJECT(FA_ERR_WORKSPACE, bwd(2, 16, 4096, 128, 0.1f, FA_BF16, P(9, 4), need));
  REJECT(FA_ERR_ALIAS, bwd(2, 16, 4096, 128, 0.1f, FA_BF16, P(5), need));   // over LSE
  REJECT(FA_ERR_ALIGN, bwd(1, 1, 128, 64, 0.1f, FA_BF16, P(9), 4096, P(7, 8)));
  ACCEPT(2, bwd(1, 1, 8388352, 128, 0.1f, FA_FP32, P(9), 4ull * 8388352));
  REJECT(FA_ERR_SHAPE, bwd(1, 1, 8388353, 128, 0.1f, FA_FP32, P(9), 1ull << 30));
  EXPECT(fa_bwd_workspace_bytes(0, 1, 1, 64) == 0);
  EXPECT(fa_bwd_workspace_bytes(1, 1, 1, 96) == 0);
  EXPECT(fa_bwd_workspace_bytes(65536, 65536, 65536, 64) == 0);
  EXPECT(fa_bwd_workspace_bytes(1, 1, 2147483647, 64) == 0);
  // grouped heads: 256 work-groups are split in two, partials after D
  const size_t gneed = fa_bwd_gqa_workspace_bytes(2, 16, 4, 4096, 128);
  EXPECT(gneed == 4ull * 2 * 16 * 4096 + 2ull * 2 * 2 * 4 * 4096 * 128 * 4);
  ACCEPT(2, fa_bwd_gqa(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 2, 16, 4, 4096, 128,
                       0.1f, 1, nullptr, FA_BF16, P(9), gneed, nullptr));
  EXPECT(fa::g_bwd.gsplit == 2 && fa::g_bwd.G == 4);
  EXPECT((char*)fa::g_bwd.part == (char*)P(9) + 4 * 2 * 16 * 4096);
  REJECT(FA_ERR_WORKSPACE, fa_bwd_gqa(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 2,
                                      16, 4, 4096, 128, 0.1f, 1, nullptr, FA_BF16, P(9),
                                      gneed - 16, nullptr));
  ACCEPT(2, fa_bwd_dropout(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 1, 2, 300, 64,
                           0.1f, 1, nullptr, 0.5f, 7, FA_BF16, P(9), 4096, nullptr));
  EXPECT(fa::g_bwd.drop.on && fa::g_bwd.drop.inv_keep == 2.0f);
  // the phases one by one
  ACCEPT(1, fa_bwd_preprocess(P(3), P(4), 2, 16, 4096, 128, FA_BF16, P(9), need, nullptr));
  REJECT(FA_ERR_ALIAS, fa_bwd_preprocess(P(3), P(4), 2, 16, 4096, 128, FA_BF16, P(4, 64), need,
                                         nullptr));
  ACCEPT(1, fa_bwd_dkdv(P(0), P(1), P(2), P(4), F(5), P(7), P(8), 2, 16, 4096, 128, 0.1f, 1,
                        nullptr, FA_BF16, P(9), need, nullptr));
  REJECT(FA_ERR_ALIAS, fa_bwd_dkdv(P(0), P(1), P(2), P(4), F(5), P(9), P(8), 2, 16, 4096, 128,
                                   0.1f, 1, nullptr, FA_BF16, P(9), need, nullptr));
  ACCEPT(1, fa_bwd_dq(P(0), P(1), P(2), P(4), F(5), P(6), 2, 16, 4096, 128, 0.1f, 1, M(10),
                      FA_BF16, P(9), need, nullptr));
  EXPECT(!fa::g_dq.dq_forms_delta);
  ACCEPT(1, fa_bwd_dq_and_d(P(0), P(1), P(2), P(3), P(4), F(5), P(6), 2, 16, 4096, 128, 0.1f,
                            1, nullptr, FA_BF16, P(9), need, nullptr));
  EXPECT(fa::g_dq.dq_forms_delta && fa::g_dq.o == P(3) && fa::g_dq.delta == F(9));
  REJECT(FA_ERR_ALIAS, fa_bwd_dq_and_d(P(0), P(1), P(2), P(3), P(4), F(5), P(6), 2, 16, 4096,
                                       128, 0.1f, 1, nullptr, FA_BF16, P(3, 64), need, nullptr));
  REJECT(FA_ERR_NULL, fa_bwd_dq_and_d(P(0), P(1), P(2), nullptr, P(4), F(5), P(6), 2, 16, 4096,
                                      128, 0.1f, 1, nullptr, FA_BF16, P(9), need, nullptr));
  REJECT(FA_ERR_DTYPE, fa_bwd_dq(P(0), P(1), P(2), P(4), F(5), P(6), 2, 16, 4096, 128, 0.1f, 1,
                                 nullptr, (fa_dtype)3, P(9), need, nullptr));
}

static void static_scratch_cases() {
  const int rows = FA_STATIC_SCRATCH_BYTES / 4;
  ACCEPT(2, fa_bwd_static(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 2, 16, 4096,
                          128, 0.1f, 1, nullptr, FA_BF16, nullptr));
  EXPECT((uintptr_t)fa::g_bwd.delta == 0x7e0000000000ull && fa::g_bwd.gsplit == 1);
  ACCEPT(2, fa_bwd_static(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 1, 1, rows, 64,
                          -0.1f, 0, nullptr, FA_FP32, nullptr));
  const int looked = fa::g_scratch_lookups;
  REJECT(FA_ERR_SCRATCH, fa_bwd_static(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 1,
                                       1, rows + 1, 64, 0.1f, 0, nullptr, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_bwd_static(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(7), P(8), 0, 1,
                                     128, 64, 0.1f, 0, nullptr, FA_BF16, nullptr));
  REJECT(FA_ERR_NULL, fa_bwd_static(P(0), P(1), P(2), P(3), nullptr, F(5), P(6), P(7), P(8), 1,
                                    1, 128, 64, 0.1f, 0, nullptr, FA_BF16, nullptr));
  EXPECT(fa::g_scratch_lookups == looked);      // rejected calls never look the buffer up
  REJECT(FA_ERR_ALIAS, fa_bwd_static(P(0), P(1), P(2), P(3), P(4), F(5), P(6), P(6, 64), P(8),
                                     1, 1, 128, 64, 0.1f, 0, nullptr, FA_BF16, nullptr));
}

static void fp8_cases() {
  ACCEPT(1, fa_fwd_fp8(P(0), P(1), P(2), F(3), F(4), F(5), P(6), F(7), 2, 16, 4096, 128, 0.1f,
                       1, nullptr, nullptr));
  EXPECT(fa::g_fp8.BH == 32 && fa::g_fp8.T == 32 && fa::g_fp8.scale == 0.1f);
  ACCEPT(1, fa_fwd_fp8(P(0), P(1), P(2), F(3), F(4), F(5), P(6), F(7), 1, 1, 16, 64, -2.0f, 0,
                       nullptr, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_fp8(P(0), P(1), P(2), F(3), F(4), F(5), P(6), F(7), 1, 1, 250,
                                  128, 0.1f, 1, nullptr, nullptr));
  REJECT(FA_ERR_ALIGN, fa_fwd_fp8(P(0), P(1), P(2, 4), F(3), F(4), F(5), P(6), F(7), 1, 1, 256,
                                  128, 0.1f, 1, nullptr, nullptr));
  REJECT(FA_ERR_ARG, fa_fwd_fp8(P(0), P(1), P(2), F(3), F(4), F(5), P(6), F(7), 1, 1, 256, 128,
                                NAN, 1, nullptr, nullptr));
}

static void decode_cases() {
  EXPECT(fa_decode_num_splits(64, 32, 8, 1, 8192, 128, 0) == 4);
  const size_t need = fa_decode_workspace_bytes(64, 32, 8, 1, 8192, 128, 0);
  EXPECT(need == 64ull * 32 * 4 * 129 * 4);
  ACCEPT(1, fa_decode(P(0), P(1), P(2), (const int*)P(3), P(4), F(5), 64, 32, 8, 1, 8192, 128,
                      0.1f, 0, 0, FA_BF16, P(9), need, nullptr));
  EXPECT(fa::g_dec.S == 4 && fa::g_dec.chunk == 2048 && fa::g_dec.R == 4 && fa::g_dec.pairs == 512);
  EXPECT(fa::g_dec.opart == F(9));
  EXPECT(fa::g_dec.lpart == F(9) + 64ull * 32 * 4 * 128);
  REJECT(FA_ERR_WORKSPACE, fa_decode(P(0), P(1), P(2), nullptr, P(4), F(5), 64, 32, 8, 1, 8192,
                                     128, 0.1f, 0, 0, FA_BF16, P(9), need - 1, nullptr));
  ACCEPT(1, fa_decode(P(0), P(1), P(2), nullptr, P(4), F(5), 2, 8, 2, 3, 5000, 64, -0.3f, 1, 1,
                      FA_FP32, nullptr, 0, nullptr));        // one chunk: no workspace
  EXPECT(fa::g_dec.S == 1 && fa::g_dec.opart == nullptr);
  EXPECT(fa_decode_num_splits(1, 1, 1, 1, 8388352, 128, 1) == 1);
  ACCEPT(1, fa_decode(P(0), P(1), P(2), nullptr, P(4), F(5), 1, 1, 1, 1, 8388352, 128, 0.1f, 0, 1,
                      FA_FP32, nullptr, 0, nullptr));
  REJECT(FA_ERR_SHAPE, fa_decode(P(0), P(1), P(2), nullptr, P(4), F(5), 1, 1, 1, 1, 8388608, 128,
                                 0.1f, 0, 1, FA_FP32, nullptr, 0, nullptr));
  EXPECT(fa_decode_num_splits(1, 6, 4, 1, 64, 64, 0) == 0);
  EXPECT(fa_decode_num_splits(1, 4, 4, 1, 64, 64, 1025) == 0);
  EXPECT(fa_decode_workspace_bytes(2147483647, 2147483647, 1, 2147483647, 2147483647, 128, 0) == 0);
  REJECT(FA_ERR_ARG, fa_decode(P(0), P(1), P(2), nullptr, P(4), F(5), 1, 1, 1, 1, 64, 64, 0.1f, 0,
                               -1, FA_BF16, nullptr, 0, nullptr));
  REJECT(FA_ERR_ALIGN, fa_decode(P(0), P(1), P(2), (const int*)P(3, 2), P(4), F(5), 1, 1, 1, 1,
                                 64, 64, 0.1f, 0, 1, FA_BF16, nullptr, 0, nullptr));
}

static void status_cases() {
  for (int s = 0; s <= 10; ++s) {
    const char* str = fa_status_str((fa_status)s);
    EXPECT(str != nullptr && std::strcmp(str, "unknown status") != 0);
  }
  EXPECT(std::strcmp(fa_status_str((fa_status)42), "unknown status") == 0);
  EXPECT(std::strcmp(fa_status_str((fa_status)-1), "unknown status") == 0);
}

// Shapes whose blocks fill few compute units (one head of 16K rows) run
// split: the forward's runs land in its workspace (O, then LSE), the
// backward's partials after D (dK/dV, then dQ); smaller workspaces run unsplit.
static void split_cases() {
  const int N = 16384;
  const unsigned long long orun = 8ull * N * 128 * 4;
  const size_t fneed = fa_fwd_workspace_bytes(1, 1, N, 128);
  EXPECT(fneed == orun + 8ull * N * 4);
  auto fws = [&](void* ws, size_t wsb, fa_dtype dt = FA_BF16, void* o = P(3)) {
    return fa_fwd_ws(P(0), P(1), P(2), o, F(4), 1, 1, N, 128, 0.1f, 1, nullptr, dt, ws, wsb,
                     nullptr);
  };
  ACCEPT(1, fws(P(9), fneed));
  EXPECT(fa::g_fwd.fsplit == 8 && fa::g_fwd.opart == F(9) && fa::g_fwd.lpart == F(9, orun));
  ACCEPT(1, fws(P(9), fneed - 1));
  EXPECT(fa::g_fwd.fsplit == 1 && fa::g_fwd.opart == nullptr);
  ACCEPT(1, fws(nullptr, 0));
  EXPECT(fa::g_fwd.fsplit == 1);
  ACCEPT(1, fws(P(9), fneed, FA_FP32));
  EXPECT(fa::g_fwd.fsplit == 1);
  REJECT(FA_ERR_WORKSPACE, fws(nullptr, 16));
  REJECT(FA_ERR_WORKSPACE, fws(P(9, 8), fneed));
  REJECT(FA_ERR_ALIAS, fws(P(3), fneed));
  REJECT(FA_ERR_ALIAS, fws(P(9), fneed, FA_BF16, P(9, orun)));
  EXPECT(fa_fwd_workspace_bytes(2, 16, 4096, 128) == 0);

  int kv = 0, q = 0;
  EXPECT(fa_bwd_splits(1, 1, 1, N, 128, FA_BF16, &kv, &q) == FA_OK && kv == 4 && q == 8);
  EXPECT(fa_bwd_splits(1, 1, 1, N, 128, FA_BF16, nullptr, &q) == FA_ERR_NULL);
  EXPECT(fa_bwd_splits(1, 6, 4, N, 128, FA_BF16, &kv, &q) == FA_ERR_SHAPE);
  const unsigned long long d_bytes = 4ull * N, kv_bytes = 2ull * 4 * N * 128 * 4;
  const size_t bneed = fa_bwd_workspace_bytes(1, 1, N, 128);
  EXPECT(bneed == d_bytes + kv_bytes + 8ull * N * 128 * 4);
  ACCEPT(2, bwd(1, 1, N, 128, 0.1f, FA_BF16, P(9), bneed));
  EXPECT(fa::g_bwd.gsplit == 4 && fa::g_bwd.part == F(9, d_bytes));
  EXPECT(fa::g_dq.ksplit == 8 && fa::g_dq.qpart == F(9, d_bytes + kv_bytes));
  ACCEPT(2, bwd(1, 1, N, 128, 0.1f, FA_BF16, P(9), d_bytes));
  EXPECT(fa::g_bwd.gsplit == 1 && fa::g_dq.ksplit == 1 && fa::g_dq.qpart == nullptr);
}

int main() {
  forward_cases();
  backward_cases();
  split_cases();
  static_scratch_cases();
  fp8_cases();
  decode_cases();
  status_cases();
  if (g_fails) {
    std::printf("%d of %d expectations failed\n", g_fails, g_cases);
    return 1;
  }
  std::printf("ok %d\n", g_cases);
  return 0;
}
