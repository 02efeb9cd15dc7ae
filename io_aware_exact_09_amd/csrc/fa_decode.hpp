// fa_decode.hpp -- internal launch interface of the split-KV decode kernels.
// Arguments arrive here already validated (fa_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Key-chunk plan of one decode call: the keys of every (batch, cache head)
// are cut into S chunks of `chunk` keys (a multiple of the 128-key tile).
struct DecodePlan {
  int S;
  int chunk;
};

// num_splits = 0 picks the plan for the shape; otherwise the keys are cut
// into at most num_splits chunks.
DecodePlan decode_plan(int B, int Hkv, int R, int Nkv, int num_splits);

struct DecodeArgs {
  const void* q; const void* k; const void* v;
  const int32_t* seqlens;  // device, [B], or nullptr (every sequence Nkv long)
  void* o; float* lse;
  float* opart;            // workspace: [pairs * R][S][d] fp32 (S > 1 only)
  float* lpart;            // workspace: [pairs * R][S] fp32
  int pairs;               // B * Hkv
  int Hkv, Nq, R, Nkv, d;  // R = (Hq / Hkv) * Nq query rows per pair
  int S, chunk;
  float scale;
  bool causal, bf16;
  hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);

}  // namespace fa
