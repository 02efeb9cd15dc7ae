// fa_launch.hpp -- internal launch interface between the C-ABI layer and the
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Dropout on the attention probabilities (see philox4x32_10 in
// fa_common.hpp): element (i, j) of head bh is kept iff the 16-bit half
// i % 2 (0 low, 1 high) of word j % 4 of Philox4x32-10(counter
// (j / 4, i / 2, bh, 0), key (key0, key1)) is >= thresh (< 2^16); kept
// probabilities are scaled by inv_keep = 1 / (1 - p).
struct Dropout {
  bool on = false;
  uint32_t key0 = 0, key1 = 0;
  uint32_t thresh = 0;
  float inv_keep = 1.f;
};

struct FwdArgs {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  const uint8_t* mask;     // nullptr = dense
  int BH, N, d, T;         // BH = B * (query heads); T = ceil(N / 128) (mask side)
  int G = 1;               // query heads per key/value head (K, V have BH / G heads)
  float scale;
  bool causal, bf16;
  Dropout drop;
  hipStream_t stream;
  int fsplit = 1;          // work-groups sharing one query block's key tiles (ping-pong
                           // forward only)
  float* opart = nullptr;  // fp32 run outputs [fsplit][BH * N][d] (fsplit > 1)
  float* lpart = nullptr;  // fp32 run LSE [fsplit][BH * N] (fsplit > 1)
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;
  void* dq; void* dk; void* dv;
  float* delta;            // workspace: D_i = rowsum(dO * O), [BH * N] fp32
  bool dq_forms_delta = false;  // the dQ pass forms D from O and writes delta
  const uint8_t* mask;
  int BH, N, d, T;         // BH = B * (query heads)
  int G = 1;               // query heads per key/value head (K, V, dK, dV have BH / G heads)
  int gsplit = 1;          // work-groups sharing one key/value head's (query head, query
                           // tile) pairs in dK/dV
  float* part = nullptr;   // fp32 dK, dV partials, [2][gsplit][BH / G * N * d] (gsplit > 1)
  int ksplit = 1;          // work-groups sharing one query block's key tiles in dQ
  float* qpart = nullptr;  // fp32 dQ partials, [ksplit][BH * N * d] (ksplit > 1)
  float scale;
  bool causal, bf16;
  Dropout drop;
  hipStream_t stream;
};

// FP8 (E4M3) forward: Q, K [BH][N][d] and V^T [BH][d][N] codes; scales sQ,
// sK [BH][ceil(N/128)], sV [BH]; O bf16 [BH][N][d], LSE fp32 [BH][N].
struct Fp8FwdArgs {
  const uint8_t* q; const uint8_t* k; const uint8_t* vt;
  const float* sq; const float* sk; const float* sv;
  void* o; float* lse;
  const uint8_t* mask;
  int BH, N, d, T;
  float scale;
  bool causal;
  hipStream_t stream;
};

// Device address of the library's static scratch (FA_STATIC_SCRATCH_BYTES
// bytes) on the current device, looked up once per device (fa_static.hip).
hipError_t static_scratch(void** ptr);

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa
