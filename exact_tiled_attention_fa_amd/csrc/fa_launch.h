// Internal host-side launch interface between the C ABI (fa_api.hip) and the
// kernel translation units. Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr float kLog2eHost = 1.4426950408889634f;

// Forward pass: one work-group per (batch, query head, 128-row query block).
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, N;
  float c;   // scale * log2(e): scores are handled in base 2
  int nqb;   // query blocks per head
  int nwg;   // total work-groups
};
constexpr int kFwdRows = 128;     // query rows per work-group (4 waves x 32)
constexpr int kFwdKeys = 64;      // keys per K/V tile
constexpr int kFwdThreads = 256;

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream);

// Split-KV decode: one work-group per (batch, KV head, head group, chunk).
struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_part;    // [B, Hq, S, d]
  float* lse_part;  // [B, Hq, S]
  int B, Hq, Hkv, L;
  int chunk;        // keys per chunk
  int S;            // number of non-empty chunks
  int G;            // query heads per KV head
  int n_hg;         // head groups per KV head (heads per group <= 16)
  float c;          // scale * log2(e)
};
constexpr int kDecThreads = 256;

hipError_t launch_decode_split(const DecArgs& a, int d, int heads_per_group, hipStream_t stream);

// Log-sum-exp merge of S normalised partials per row into BF16 O and FP32 lse.
hipError_t launch_combine(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                          int rows, int S, int d, hipStream_t stream);

}  // namespace fa
