// Internal host-side launch interface between the C ABI (fa_api.hip) and the
// kernel translation units. Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr float kLog2eHost = 1.4426950408889634f;

// Forward pass: one work-group per (batch, query head, key split, 128-row
// query block). With n_splits == 1 each work-group sweeps all keys of its
// block and writes O and lse; otherwise split s covers key tiles
// [s * split_tiles, (s + 1) * split_tiles) and writes its normalised partial
// O_s (BF16) and lse_s (FP32) to o_part [B*Hq*N, n_splits, d] and
// lse_part [B*Hq*N, n_splits] for fa_fwd_combine_kernel.
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, N;
  float c;   // scale * log2(e): scores are handled in base 2
  int rows;  // query rows per block: 32 x waves per work-group
  int nqb;   // query blocks per head
  int nwg;   // total work-groups
  int n_splits;
  int split_tiles;
  uint16_t* o_part;  // [B*Hq*N, n_splits, d] BF16 normalised partial outputs
  float* lse_part;   // [B*Hq*N, n_splits] FP32
  float v_scale;  // FP8 pass: the factor of V's codes (O = v_scale P V / l)
  int head_group;  // heads whose blocks interleave in the grid order (one XCD's share; 1 = head by head)
};
constexpr int kFwdKeys = 64;      // keys per K/V tile
constexpr int kFwdWaveRows = 32;  // query rows per wave

// Waves per forward work-group: 8 (256 rows, one work-group per CU, every K/V
// tile it loads serves twice the rows) except for causal sweeps shorter than
// 8K keys, where 4 (128 rows, two work-groups per CU) waste less on the
// diagonal (every wave of a block takes every tile of the block) and balance
// the short, unequal blocks better; also 4 for causal sweeps shorter than 16K
// whose 256-row blocks would not fill the CUs (the key-split path).
// One exception in BF16: from 4K keys, when the 256-row blocks make exactly two
// per CU, the heaviest-first order hands every CU that frees up the heaviest
// block left, so each CU's two blocks add up to about the same work and 8
// waves win (32 causal heads at 4K: 137.7 -> 131.8 us at d = 128, 85.4 -> 81.6
// at d = 64; with one, three or four blocks per CU 8 waves lose 1-15%, and the
// FP8 pass loses 1-3% at two).
inline int fwd_waves(bool causal, int N, int64_t blocks256, int cus, bool fp8) {
  if (!causal) return 8;
  if (N < 8192) return !fp8 && N >= 4096 && blocks256 == 2 * (int64_t)cus ? 8 : 4;
  return N < 16384 && blocks256 < cus ? 4 : 8;
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream);
// FP8 E4M3 inputs (q, k, v point at bytes), d = 64 or 128; c folds scale * q_scale * k_scale.
hipError_t launch_fwd_fp8(const FwdArgs& a, int d, bool causal, hipStream_t stream);
// Merge the key-split partials of a split forward into O (BF16) and lse.
hipError_t launch_fwd_combine(const FwdArgs& a, int d, bool causal, hipStream_t stream);

// Backward pass (d = 64 or 128): a row pass (lse2 = lse log2 e and delta = rowsum(dO O),
// both padded to Npad rows with zeros), then dK/dV with one work-group per
// (batch, KV head, 64-key block) sweeping the query tiles of every query head
// of its group, and dQ with one work-group per (batch, query head, 128-row
// block) sweeping the key tiles. Scores and weights are recomputed from Q, K
// and lse; nothing N x N reaches memory.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* lse2;   // [B * Hq, Npad]
  float* delta;  // [B * Hq, Npad]
  int B, Hq, Hkv, N, Npad;
  float c;       // scale * log2(e)
  float scale;
  int nkb;       // 64-key blocks per KV head
  int nqb;       // 128-row query blocks per head
  int hg_kv;     // KV heads whose key blocks interleave in the dK/dV grid order (1 = head by head)
  int hg_q;      // query heads whose row blocks interleave in the dQ grid order
};
constexpr int kBwdKeyBlock = 64;
constexpr int kBwdRowBlock = 128;
constexpr int kBwdTile = 64;  // rows per Q/dO tile (dK/dV) and per K/V tile (dQ)

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t stream);

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
  const int* lens;  // per-sequence key counts (clamped to [0, L]), or null: all L
};
constexpr int kDecThreads = 256;

hipError_t launch_decode_split(const DecArgs& a, int d, int heads_per_group, hipStream_t stream);

// Log-sum-exp merge of S normalised partials per row into BF16 O and FP32 lse.
hipError_t launch_combine(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                          int rows, int S, int d, hipStream_t stream);

}  // namespace fa
