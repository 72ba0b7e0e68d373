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
  // Causal key split sized per query block (0 = off): block qb, whose keys
  // below the diagonal fill vis(qb) tiles, takes ns(qb) = ceil(vis / split_target)
  // splits of ceil(vis / ns) tiles each, so no split holds more than
  // split_target tiles and the light blocks take fewer splits; n_splits is
  // then the largest ns (the partials' row stride) and per_head the
  // work-groups of one head. A block with one split writes O and lse itself.
  int split_target;
  int per_head;
};

// Key tiles of causal query block qb (rows qb * rows ..) at or below the diagonal.
__host__ __device__ inline int causal_block_tiles(int qb, int rows, int N, int keys_per_tile) {
  const int end = (qb + 1) * rows < N ? (qb + 1) * rows : N;
  return (end + keys_per_tile - 1) / keys_per_tile;
}
constexpr int kFwdKeys = 64;      // keys per K/V tile
constexpr int kFwdWaveRows = 32;  // query rows per wave

// Forward grid order: logical work-group id (after the XCD-contiguous remap)
// -> query block qb, key split, (batch * Hq + head) bh, the split's key tiles
// per split and the block's split count. Groups of head_group heads, then
// query blocks (heaviest first when causal), then splits, then the head
// within the group. Shared by the kernel and host-side checks of the mapping.
__host__ __device__ inline void fwd_block_map(int lid, const FwdArgs& a, bool causal, int& qb, int& split,
                                              int& bh, int& split_tiles, int& block_splits) {
  if (causal && a.split_target > 0) {
    // Splits sized per block, blocks heaviest first, each taking (its splits)
    // x (heads in the group) consecutive ids. The last block sees every key
    // tile; a full block qb < nqb - 1 sees u R tiles (u = qb + 1, R = rows /
    // 64) and takes ceil(u R / T) splits, which equals k exactly for u in
    // [floor((k - 1) T / R) + 1, floor(k T / R)]. So the walk goes over the
    // split counts k (at most the largest count, about 16) instead of over the
    // blocks, with no division inside: every wave of the work-group runs it on
    // the CU's one scalar unit, and a walk over 64 blocks had held the last
    // work-groups of a 16K head up by 8 us.
    const int T = a.split_target;
    const int R = a.rows / kFwdKeys;  // 2 or 4: a shift below
    const int rs = 31 - __builtin_clz((unsigned)R);
    const int per_group = a.head_group * a.per_head;
    const int grp = lid / per_group;
    int r = lid - grp * per_group;
    const int left = a.B * a.Hq - grp * a.head_group;
    const int gh = a.head_group < left ? a.head_group : left;
    int vis = causal_block_tiles(a.nqb - 1, a.rows, a.N, kFwdKeys);
    int ns = (vis + T - 1) / T;
    qb = a.nqb - 1;
    if (r >= ns * gh && a.nqb > 1) {
      r -= ns * gh;
      const int u_top = a.nqb - 1;  // full blocks: u = 1 .. u_top
      int k = (u_top * R + T - 1) / T;
      int u_hi = u_top;
      for (; k > 1; --k) {
        const int u_lo = (((k - 1) * T) >> rs) + 1;  // first u with ceil(u R / T) = k
        const int span = (u_hi - u_lo + 1) * k * gh;
        if (u_lo <= u_hi) {
          if (r < span) break;
          r -= span;
          u_hi = u_lo - 1;
        }
      }
      // Here the block is in the run of split count k ending at u_hi.
      const int p = r / (k * gh);
      r -= p * k * gh;
      qb = u_hi - p - 1;
      ns = k;
      vis = (qb + 1) * R;
    }
    split = r / gh;
    bh = grp * a.head_group + (r - split * gh);
    block_splits = ns;
    split_tiles = (vis + ns - 1) / ns;
  } else {
    const int per_head = a.nqb * a.n_splits;
    const int grp = lid / (a.head_group * per_head);
    const int rem_g = lid - grp * a.head_group * per_head;
    const int left = a.B * a.Hq - grp * a.head_group;
    const int gh = a.head_group < left ? a.head_group : left;  // heads in this group
    const int qs = rem_g / gh;
    bh = grp * a.head_group + (rem_g - qs * gh);
    qb = qs / a.n_splits;
    split = qs - qb * a.n_splits;
    if (causal) qb = a.nqb - 1 - qb;
    block_splits = a.n_splits;
    split_tiles = a.split_tiles;
  }
}

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

// Fewest key tiles a split may hold: shorter splits spend too much of their
// time in the prologue and the partial-result write.
constexpr int kMinSplitTiles = 8;
// Causal BF16 forward with its keys split per block (see plan_fwd): 8-wave
// work-groups, at least 4 key tiles per split, and only for calls of at least
// 8192 query rows; below that the fixed cost of the partial results and the
// merge outweighs the balance, and the uniform split of 4-wave blocks is
// faster (one head of 4K keys: 17.0 against 22.7 us; two heads: 24.6 against
// 23.7; one head of 8K: 37.5 against 31.7).
constexpr int kCausalSplitWaves = 8;
constexpr int kCausalSplitMinTiles = 4;
constexpr int64_t kCausalSplitMinRows = 8192;

struct FwdPlan {
  int rows, nqb, n_splits, split_tiles;
  int head_group;    // see FwdArgs::head_group
  int split_target;  // see FwdArgs::split_target (0: uniform splits)
  int per_head;      // work-groups per head when split_target > 0
  int64_t nwg;       // work-groups of the forward launch
  size_t ws_bytes;   // partial-result buffer for a split, 0 otherwise
};

// Key split for grids that would leave CUs idle: aim at as many work-groups
// as fit on the CUs at once (one of 8 waves or two of 4 per CU), never fewer
// than kMinSplitTiles key tiles per split.
//
// Causal (BF16): the blocks see different numbers of keys, so the splits are
// sized per block. With T key tiles at most per split, block qb takes
// ceil(vis(qb) / T) splits; T is the smallest value (>= kCausalSplitMinTiles)
// whose splits all fit on the CUs at once, so every work-group holds about the
// average share of the work below the diagonal. (Uniform splits of every
// block's full key range left a quarter to a half of the work-groups empty and
// the heaviest with twice the average: one head of 8K keys went 37.5 -> 31.7 us,
// of 16K 106.8 -> 78.3 us, of 32K 401 -> 286 us.)
inline FwdPlan plan_fwd(int B, int Hq, int N, int d, bool causal, bool fp8, int cus) {
  FwdPlan p;
  const int64_t blocks256 = (int64_t)B * Hq * ((N + 255) / 256);
  const int tiles = (N + kFwdKeys - 1) / kFwdKeys;
  const bool causal_split = causal && !fp8 && blocks256 < cus && tiles >= 2 * kMinSplitTiles &&
                            (int64_t)B * Hq * N >= kCausalSplitMinRows;
  const int waves = causal_split ? kCausalSplitWaves : fwd_waves(causal, N, blocks256, cus, fp8);
  p.rows = kFwdWaveRows * waves;
  p.split_target = 0;
  p.per_head = 0;
  // Causal blocks differ in work (heaviest first). Each of the 8 XCDs takes a
  // contiguous range of the grid; when that range is a whole number (>= 2) of
  // heads, their blocks interleave so the XCD starts all its heaviest blocks
  // first instead of one head's after another's lightest.
  const int64_t nbh = (int64_t)B * Hq;
  p.head_group = causal && nbh % 8 == 0 && nbh >= 16 ? (int)(nbh / 8) : 1;
  p.nqb = (N + p.rows - 1) / p.rows;
  const int64_t base = (int64_t)B * Hq * p.nqb;
  p.n_splits = 1;
  p.split_tiles = tiles;
  const int64_t target = (waves == 8 ? 1 : 2) * (int64_t)cus;
  const int64_t nbh_all = (int64_t)B * Hq;
  if (causal_split && base < target) {
    // base < target <= 2 * CUs bounds nqb, so these sums are short.
    int64_t vis_sum = 0;
    for (int qb = 0; qb < p.nqb; ++qb) vis_sum += causal_block_tiles(qb, p.rows, N, kFwdKeys);
    int64_t T = (vis_sum * nbh_all + target - 1) / target;
    if (T < kCausalSplitMinTiles) T = kCausalSplitMinTiles;
    int64_t per_head = 0;
    for (;; ++T) {
      per_head = 0;
      for (int qb = 0; qb < p.nqb; ++qb)
        per_head += (causal_block_tiles(qb, p.rows, N, kFwdKeys) + T - 1) / T;
      if (per_head * nbh_all <= target) break;
    }
    const int most = (int)((causal_block_tiles(p.nqb - 1, p.rows, N, kFwdKeys) + T - 1) / T);
    if (most > 1) {
      p.split_target = (int)T;
      p.per_head = (int)per_head;
      p.n_splits = most;
      p.split_tiles = (int)T;
    }
  } else if (base < target && tiles >= 2 * kMinSplitTiles) {
    const int64_t want = (target + base - 1) / base;
    p.n_splits = (int)(want < tiles / kMinSplitTiles ? want : tiles / kMinSplitTiles);
    p.split_tiles = (tiles + p.n_splits - 1) / p.n_splits;
    p.n_splits = (tiles + p.split_tiles - 1) / p.split_tiles;
  }
  p.nwg = p.split_target > 0 ? nbh_all * p.per_head : base * p.n_splits;
  const size_t rows = (size_t)B * Hq * N;
  // BF16 partial outputs, then FP32 partial lse values.
  const size_t bytes = p.n_splits > 1 ? rows * p.n_splits * ((size_t)d * 2 + sizeof(float)) : 0;
  p.ws_bytes = (bytes + 255) & ~(size_t)255;
  return p;
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
  float* ndelta;  // [B * Hq, Npad]: -delta (the products start from it)
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
