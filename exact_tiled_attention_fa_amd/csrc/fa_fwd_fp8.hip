// Exact tiled attention forward pass with FP8 inputs, for gfx950.
//
// What it computes: the attention of the dequantised inputs q_scale Q,
// k_scale K, v_scale V, where Q, K, V hold OCP FP8 E4M3 codes (the FP8 low
// precision the memory-bound page names for the third FlashAttention version,
// "What does FlashAttention-2 change?"), with the same online softmax and the
// same outputs as the BF16 pass: O in BF16, lse in FP32.
//
// Mapping onto CDNA4 (the BF16 kernel's plan, at twice the product rate):
//   * Scores transposed, S^T = K Q^T, with v_mfma_f32_32x32x64_f8f6f4 (both
//     operands E4M3): A = 32 keys x 64 d bytes of K from LDS, B = Q^T held in
//     registers. Each lane holds 16 keys of one query row, as in BF16.
//   * p = 2^(t - m + 6) is rounded to E4M3 (v_cvt_pk_fp8_f32, nearest even)
//     and used as the B operand P^T of O^T = V^T P^T; the factor 2^6 keeps
//     p up to 2^8 (within E4M3's 448) and moves small weights out of the
//     subnormal range; it cancels in O / l and is removed from lse. The row
//     max moves only when a tile's max exceeds it by more than 2.
//   * V^T operands come from LDS with ds_read_b64_tr_b8 (transposed 8-bit
//     reads): lane i of a 16-lane block receives byte i % 8 of the 8-byte runs
//     named by lanes i / 8 + 2 e, e = 0..7.
//   * K/V tiles of 64 keys (8 KiB each) go HBM -> LDS with direct loads,
//     double buffered; causal tile skipping, key splits and the grid order
//     are those of the BF16 pass, and its combine kernel merges split partials.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// O^T or S^T (32 x 32, FP32) += A (32 x 64 E4M3) B (64 x 32 E4M3). Lane l
// holds row (A) or column (B) l % 32 and 32 bytes of the contraction index
// for its half l / 32; A and B assign those bytes the same way.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const void* lds_byte_ptr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_byte_ptr));
}

// Four FP32 values -> four E4M3 bytes (nearest even), first value lowest.
// Both halves of the word are written, so `prev` (the word this one replaces)
// only names the register: no zeroing move per word.
__device__ __forceinline__ int pack_fp8x4(int prev, float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, prev, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

constexpr float kRescaleSlack8 = 2.f;
constexpr float kPBias8 = 6.f;        // p = 2^(t - m + kPBias8) <= 2^8

template <int D>
struct Fp8Cfg {
  static constexpr int CH = D / 16;             // 16-byte chunks per K/V row (D bytes)
  static constexpr int TILE = kFwdKeys * D;     // bytes per K or V tile
  static constexpr int KK = D / 64;             // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  static constexpr int BLOCKS = TILE / 1024;    // 1 KiB direct-load blocks per tile
  static constexpr int RPB = 1024 / D;          // rows per block
};

// LDS chunk swizzles (16-byte chunk index within a D-byte row).
// K (fragment reads: 16 consecutive rows at one chunk column): D = 128 has
// 128-byte rows, two per 64 banks, so chunk ^ ((r >> 1) & 7); D = 64 has
// four rows per 64 banks, so chunk ^ ((r >> 2) & 3). Either way the 16 rows
// land on 16 distinct 16-byte bank slots.
template <int D>
__device__ __forceinline__ int kswz8(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
// V (transposed reads: one 16-lane block takes 8 keys x two 8-byte halves of
// one chunk column, its partner block the next chunk column).
//   D = 128: column chunk c is stored at ((c & 1) << 2 | c >> 1) ^ f(r), f
//   taking bits 1 and 3 of the key, so the two blocks cover 32 distinct
//   8-byte slots.
//   D = 64: chunk c is stored at c ^ (2 * bit 3 of the key): the 8 keys of a
//   block (two runs of 4 consecutive keys, 8 apart) fill 8 distinct 16-byte
//   slots and the partner block's column the other 8.
__device__ __forceinline__ int vf8(int r) { return ((r >> 1) & 1) | ((r >> 2) & 2); }
template <int D>
__device__ __forceinline__ int vphys8(int c, int r) {
  if (D == 128) return (((c & 1) << 2) | (c >> 1)) ^ vf8(r);
  return c ^ (((r >> 3) & 1) << 1);
}
template <int D>
__device__ __forceinline__ int vlogical8(int p, int r) {
  if (D == 128) {
    const int x = p ^ vf8(r);
    return ((x & 3) << 1) | (x >> 2);
  }
  return p ^ (((r >> 3) & 1) << 1);
}
// BF16 staging of the output rows: 8-byte unit e of row r is stored at unit
// e ^ ostw(r) (as the BF16 pass).
template <int D>
__device__ __forceinline__ int ostw(int r) { return D == 128 ? r : ((r >> 1) & 15); }

}  // namespace

template <int D, bool CAUSAL, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(FwdArgs a) {
  using C = Fp8Cfg<D>;
  constexpr int ROWS = kFwdWaveRows * W;
  // 1 KiB direct-load blocks per wave per tile; with fewer blocks than waves
  // (d = 64, 8 waves) the first C::BLOCKS waves load one each.
  constexpr int BPW = C::BLOCKS >= W ? C::BLOCKS / W : 1;
  constexpr int RPB = C::RPB;
  constexpr int DT = C::DT;
  constexpr int kD8 = D;
  constexpr int kTile8 = C::TILE;
  constexpr int kChunks8 = C::CH;
  // K buffers 0, 1 then V buffers 0, 1; after the sweep the epilogue stages
  // each wave's 32 BF16 rows over the whole array.
  constexpr int STAGE_BYTES = W * 32 * kD8 * 2 > 4 * kTile8 ? W * 32 * kD8 * 2 : 4 * kTile8;
  __shared__ uint4 smem[STAGE_BYTES / 16];
  // Q rows staged in LDS by direct loads (as the BF16 pass) at d = 128 where
  // LDS allows: one work-group per CU (8 waves), or two with room for both.
  // (At d = 64 the direct operand loads are only two per lane and staging
  // measured 1.5% slower.)
  constexpr int Q_BYTES = W * 32 * kD8;
  constexpr bool kStageQ = D == 128 && (W == 8 || 2 * (STAGE_BYTES + Q_BYTES) <= 160 * 1024);
  __shared__ uint4 q_lds[kStageQ ? Q_BYTES / 16 : 1];
  char* const lds = reinterpret_cast<char*>(smem);
  auto k_lds = [&](int i) { return lds + i * kTile8; };
  auto v_lds = [&](int i) { return lds + (2 + i) * kTile8; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int li = lane & 31;

  // ---- grid order (as the BF16 pass): XCD-contiguous, groups of head_group
  // heads, then query block (heaviest first when causal), then head within
  // the group, then key split.
  const int lid = xcd_contiguous(blockIdx.x, a.nwg);
  const int per_head = a.nqb * a.n_splits;
  const int grp = lid / (a.head_group * per_head);
  const int rem_g = lid - grp * a.head_group * per_head;
  const int gh = min(a.head_group, a.B * a.Hq - grp * a.head_group);  // heads in this group
  const int qs = rem_g / gh;
  const int bh = grp * a.head_group + (rem_g - qs * gh);
  int qb = qs / a.n_splits;
  const int split = qs - qb * a.n_splits;
  if (CAUSAL) qb = a.nqb - 1 - qb;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int N = a.N;
  const int q0 = qb * ROWS;
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q);
  const size_t kv_row0 = (size_t)(b * a.Hkv + hk) * (size_t)N;
  const int t_begin = split * a.split_tiles;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.k) + (kv_row0 + (size_t)t_begin * kFwdKeys) * kD8;
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(a.v) + (kv_row0 + (size_t)t_begin * kFwdKeys) * kD8;
  const int n_keys = N - t_begin * kFwdKeys;

  const int kv_end = CAUSAL ? min(N, q0 + ROWS) : N;
  const int n_tiles = min((kv_end + kFwdKeys - 1) / kFwdKeys, t_begin + a.split_tiles) - t_begin;
  if (n_tiles <= 0) return;
  const int wave_q0 = q0 + wave * 32;

  // ---- direct loads: lane l fills physical chunk l % 8 of tile row
  // (block row) + l / 8 with the logical chunk the swizzle puts there; rows
  // past the last key are clamped to it (finite data, masked scores).
  const int dma_row = lane / kChunks8;
  const int dma_p = lane % kChunks8;
  uint32_t kdo[BPW], vdo[BPW];
#pragma unroll
  for (int x = 0; x < BPW; ++x) {
    const int r = (wave * BPW + x) * RPB + dma_row;
    kdo[x] = (uint32_t)(r * kD8 + 16 * (dma_p ^ kswz8<D>(r)));
    vdo[x] = (uint32_t)(r * kD8 + 16 * vlogical8<D>(dma_p, r));
  }
  auto issue = [&](const uint8_t* src, const uint32_t* offs, bool is_v, int tile, char* dst) {
    const uint8_t* base = src + (size_t)tile * kTile8;
    const int rows = n_keys - tile * kFwdKeys;
    const uint32_t l0 = lds_addr(dst) + 1024u * (uint32_t)(wave * BPW);
    if (C::BLOCKS < W && wave >= C::BLOCKS) return;
    if (rows >= kFwdKeys) {
#pragma unroll
      for (int x = 0; x < BPW; ++x) dma16(base, offs[x], l0 + 1024u * x);
    } else {
#pragma unroll
      for (int x = 0; x < BPW; ++x) {
        const int r = (wave * BPW + x) * RPB + dma_row;
        const int lc = is_v ? vlogical8<D>(dma_p, r) : (dma_p ^ kswz8<D>(r));
        dma16(base, (uint32_t)(min(r, rows - 1) * kD8 + 16 * lc), l0 + 1024u * x);
      }
    }
  };

  // As in the BF16 pass, steps whose K(t+1) and V(t) tiles are both full
  // place their direct loads among the matrix products (block x of K before
  // k-step kx(x) of the scores, block x of V before d tile vx(x) of the PV
  // products) when every wave loads a block; t + 1 < full_tiles marks them.
  constexpr bool kSpread = C::BLOCKS >= W;
  auto kx = [](int x) { return C::KK == 1 ? 0 : (BPW == 1 ? 1 : x); };
  auto vx = [](int x) { return BPW == 1 ? DT / 2 : 2 * x + 1; };
  const int full_tiles = kSpread ? min(n_tiles, n_keys / kFwdKeys) : 0;

  issue(kg, kdo, false, 0, k_lds(0));

  // ---- Q^T operand: lane (row li, half g) holds bytes 64 kk + 32 g .. + 31 of
  // its row. A negative scale product flips the sign bits (exact); a zero one
  // becomes the smallest normal float (every visible key then gets the same
  // weight, as with scale 0).
  const int qi = q0 + wave * 32 + li;
  const int sign = a.c < 0.f ? (int)0x80808080u : 0;
  const float c = fmaxf(fabsf(a.c), 1.17549435e-38f);
  i32x8 qf[C::KK];
  if constexpr (kStageQ) {
    // Rows past N repeat row N - 1 (finite; their results are never stored).
    const int wrow0 = min(q0 + wave * 32, N - 1);
    const uint8_t* qsrc = q8 + ((size_t)(b * a.Hq + h) * N + wrow0) * kD8;
    const uint32_t ql0 = lds_addr(q_lds) + (uint32_t)(wave * 32 * kD8);
#pragma unroll
    for (int x = 0; x < 32 / RPB; ++x) {
      const int r = x * RPB + dma_row;
      const int rel = min(q0 + wave * 32 + r, N - 1) - wrow0;
      dma16(qsrc, (uint32_t)(rel * kD8 + 16 * (dma_p ^ kswz8<D>(r))), ql0 + 1024u * x);
    }
  } else {
    const uint4* qrow = reinterpret_cast<const uint4*>(q8 + ((size_t)(b * a.Hq + h) * N + (qi < N ? qi : 0)) * kD8);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      uint4 w0 = qi < N ? qrow[4 * kk + 2 * g] : make_uint4(0u, 0u, 0u, 0u);
      uint4 w1 = qi < N ? qrow[4 * kk + 2 * g + 1] : make_uint4(0u, 0u, 0u, 0u);
      qf[kk] = i32x8{(int)w0.x ^ sign, (int)w0.y ^ sign, (int)w0.z ^ sign, (int)w0.w ^ sign,
                     (int)w1.x ^ sign, (int)w1.y ^ sign, (int)w1.z ^ sign, (int)w1.w ^ sign};
    }
  }
  // Staged Q: this lane's operand (row li, chunks 4 kk + 2 g + {0, 1}) once
  // step 0's wait and barrier have passed.
  auto read_q = [&]() {
    const char* qb = reinterpret_cast<const char*>(q_lds) + wave * 32 * kD8 + li * kD8;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const uint4 w0 = *reinterpret_cast<const uint4*>(qb + 16 * ((4 * kk + 2 * g) ^ kswz8<D>(li)));
      const uint4 w1 = *reinterpret_cast<const uint4*>(qb + 16 * ((4 * kk + 2 * g + 1) ^ kswz8<D>(li)));
      qf[kk] = i32x8{(int)w0.x ^ sign, (int)w0.y ^ sign, (int)w0.z ^ sign, (int)w0.w ^ sign,
                     (int)w1.x ^ sign, (int)w1.y ^ sign, (int)w1.z ^ sign, (int)w1.w ^ sign};
    }
  };

  // ---- per-lane LDS byte offsets. K: row li, logical chunks 4 kk + 2 g + {0, 1}
  // (rows 32 + li add 4 KiB). V^T: as a source lane, lane i of 16-lane block
  // beta names the run of key 8 (e / 4) + 4 g + e % 4 (e = i / 2; + 16 n for
  // read n) at column 32 dt + 16 (beta % 2) + 8 (i % 2).
  int koff[C::KK][2];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) koff[kk][hh] = li * kD8 + 16 * ((4 * kk + 2 * g + hh) ^ kswz8<D>(li));
  const int i16 = lane & 15;
  const int beta2 = (lane >> 4) & 1;
  const int e8 = i16 >> 1;
  const int vkey = 8 * (e8 >> 2) + 4 * g + (e8 & 3);
  int voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) voff[dt] = vkey * kD8 + 16 * vphys8<D>(2 * dt + beta2, vkey) + 8 * (i16 & 1);

  float m_run = -INFINITY;
  float l_run = 0.f;  // running sum of 2^(t - m_run + kPBias8)
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  f32x16 pp0, pp1;  // p of the previous tile (FP32)
  i32x8 pf = {};    // its P^T operand (E4M3): dword 4 jt + q holds keys 32 jt + 8 q + 4 g + 0..3

  auto scores = [&](const char* kb, f32x16& s0, f32x16& s1, bool valu, bool dma, const uint8_t* kbase,
                    uint32_t kl0) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (kSpread && dma) {
#pragma unroll
        for (int x = 0; x < BPW; ++x)
          if (kk == kx(x)) dma16(kbase, kdo[x], kl0 + 1024u * x);
      }
      const uint4 a0 = *reinterpret_cast<const uint4*>(kb + koff[kk][0]);
      const uint4 a1 = *reinterpret_cast<const uint4*>(kb + koff[kk][1]);
      const uint4 b0 = *reinterpret_cast<const uint4*>(kb + koff[kk][0] + 32 * kD8);
      const uint4 b1 = *reinterpret_cast<const uint4*>(kb + koff[kk][1] + 32 * kD8);
      s0 = mfma_fp8(i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w},
                    qf[kk], s0);
      s1 = mfma_fp8(i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w},
                    qf[kk], s1);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::KK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 2 < 2 * C::KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (valu) __builtin_amdgcn_sched_group_barrier(0x002, 24 / C::KK, 0);
    }
  };

  auto apply_mask = [&](int kv0, f32x16& s0, f32x16& s1) {
    const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 4 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 8 * (r >> 2) + (r & 3);
      if (o > lim) s0[r] = -INFINITY;
      if (o + 32 > lim) s1[r] = -INFINITY;
    }
  };

  auto finish_p = [&](const f32x16& p0, const f32x16& p1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pf[q] = pack_fp8x4(pf[q], p0[4 * q], p0[4 * q + 1], p0[4 * q + 2], p0[4 * q + 3]);
      pf[4 + q] = pack_fp8x4(pf[4 + q], p1[4 * q], p1[4 * q + 1], p1[4 * q + 2], p1[4 * q + 3]);
    }
    float ra = p0[0] + p1[0];
    float rb = p0[1] + p1[1];
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      ra += p0[r] + p1[r];
      rb += p0[r + 1] + p1[r + 1];
    }
    l_run += ra + rb;
  };

  // O^T += V^T P^T: the V^T operand of lane l is column 32 dt + l % 32 at the
  // 32 keys of its P^T bytes, gathered with four transposed reads of 8 keys.
  auto pv = [&](const char* vb, bool dma, const uint8_t* vbase, uint32_t vl0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (kSpread && dma) {
#pragma unroll
        for (int x = 0; x < BPW; ++x)
          if (dt == vx(x)) dma16(vbase, vdo[x], vl0 + 1024u * x);
      }
      const i32x2 r0 = lds_read_tr8(vb + voff[dt]);
      const i32x2 r1 = lds_read_tr8(vb + voff[dt] + 16 * kD8);
      const i32x2 r2 = lds_read_tr8(vb + voff[dt] + 32 * kD8);
      const i32x2 r3 = lds_read_tr8(vb + voff[dt] + 48 * kD8);
      oacc[dt] = mfma_fp8(i32x8{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y}, pf, oacc[dt]);
    }
  };

  auto tile_max = [&](const f32x16& s0, const f32x16& s1) {
    float ma = fmax_ieee(s0[0], s1[0]);
    float mb = fmax_ieee(s0[1], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      ma = fmax_ieee(fmax_ieee(ma, s0[r]), s1[r]);
      mb = fmax_ieee(fmax_ieee(mb, s0[r + 1]), s1[r + 1]);
    }
    return max_xor32(fmax_ieee(ma, mb));
  };

  auto exps = [&](f32x16& s0, f32x16& s1) {
    const float nm = (m_run == -INFINITY ? 0.f : -m_run) + kPBias8;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = exp2_hw(fmaf(s0[r], c, nm));
      s1[r] = exp2_hw(fmaf(s1[r], c, nm));
    }
  };

  auto softmax_pv = [&](int kv0, f32x16& s0, f32x16& s1, const char* vb, bool with_pv, bool dma,
                        const uint8_t* vbase, uint32_t vl0) {
    if ((kv0 + kFwdKeys > N) || (CAUSAL && kv0 + kFwdKeys - 1 > wave_q0)) apply_mask(kv0, s0, s1);
    // Branch-free reference update (alpha = 1 where it stays), so the max,
    // the exponentials and the PV products share one scheduling region.
    const float mt = tile_max(s0, s1) * c;
    const bool grow = mt > m_run + kRescaleSlack8;
    const float alpha = grow ? exp2_hw(m_run - mt) : 1.f;
    m_run = grow ? mt : m_run;
    l_run *= alpha;
    const bool any_grow = __any(grow);
    exps(s0, s1);
    if (with_pv) {
      pv(vb, dma, vbase, vl0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + 1 < DT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 22, 0);
      }
    }
    asm volatile("" : "+v"(s0), "+v"(s1));
    pp0 = s0;
    pp1 = s1;
    if (any_grow) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
  };

  auto step = [&](auto kb_c, int t, bool with_pv, bool spread) {
    constexpr int KB = decltype(kb_c)::value;
    spread = spread && !kSyncCheck;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!spread) {
      if (t + 1 < n_tiles) issue(kg, kdo, false, t + 1, k_lds(KB ^ 1));
      issue(vg, vdo, true, t, v_lds(KB));
    }
    sync_check_group();
    if (kStageQ && !with_pv) read_q();
    const uint8_t* kbase = kg + (size_t)(t + 1) * kTile8;
    const uint32_t kl0 = lds_addr(k_lds(KB ^ 1)) + 1024u * (uint32_t)(wave * BPW);
    const uint8_t* vbase = vg + (size_t)t * kTile8;
    const uint32_t vl0 = lds_addr(v_lds(KB)) + 1024u * (uint32_t)(wave * BPW);
    __builtin_amdgcn_sched_barrier(0);
    if (with_pv) finish_p(pp0, pp1);
    f32x16 s0, s1;
    scores(k_lds(KB), s0, s1, with_pv, spread, kbase, kl0);
    sync_check_group();
    if (with_pv) asm volatile("" : "+v"(pf), "+v"(l_run));
    softmax_pv((t_begin + t) * kFwdKeys, s0, s1, v_lds(KB ^ 1), with_pv, spread, vbase, vl0);
    sync_check_group();
  };
  auto last = [&](auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    finish_p(pp0, pp1);
    pv(v_lds(KB ^ 1), false, nullptr, 0u);
    sync_check_group();
  };

  step(IC<0>{}, 0, false, false);
  int t = 1;
  for (; t + 2 < full_tiles; t += 2) {
    step(IC<1>{}, t, true, true);
    step(IC<0>{}, t + 1, true, true);
  }
  if (!kSpread) {
    for (; t + 1 < n_tiles; t += 2) {
      step(IC<1>{}, t, true, false);
      step(IC<0>{}, t + 1, true, false);
    }
  }
  // At most three steps remain (t + 2 >= full_tiles >= n_tiles - 1 when the
  // loads spread; at most one otherwise).
  if (t < n_tiles) {
    step(IC<1>{}, t, true, false);
    if (t + 1 < n_tiles) {
      step(IC<0>{}, t + 1, true, false);
      if (t + 2 < n_tiles) {
        step(IC<1>{}, t + 2, true, false);
        last(IC<0>{});
      } else {
        last(IC<1>{});
      }
    } else {
      last(IC<0>{});
    }
  } else {
    last(IC<1>{});
  }

  // ---- epilogue (as the BF16 pass): O = v_scale O / l, lse = (m - 6 + log2 l) ln 2;
  // O rounded to BF16 to the output or, with key splits, to the split's partial.
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? a.v_scale / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run - kPBias8 + log2_hw(l_tot)) * kLn2 : -INFINITY;
  const size_t head_row0 = (size_t)(b * a.Hq + h) * N;
  const size_t qo_base = head_row0 * kD8;
  if (qi < N && g == 0) {
    if (a.n_splits == 1) a.lse[head_row0 + qi] = lse_v;
    else a.lse_part[(head_row0 + qi) * a.n_splits + split] = lse_v;
  }
  __syncthreads();  // every wave is done with the K/V buffers
  char* stage = lds + wave * (32 * kD8 * 2);
  // 8-byte units: unit e = 8 dt + 2 rq + g of row li (columns 4 e .. 4 e + 3).
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e = 8 * dt + 2 * rq + g;
      *reinterpret_cast<uint2*>(stage + li * (kD8 * 2) + 8 * (e ^ ostw<D>(li))) =
          pack_bf16x4(oacc[dt][4 * rq + 0] * inv, oacc[dt][4 * rq + 1] * inv,
                      oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
    }
  wave_sync_lds();
  sync_check_group();
  constexpr int C16 = kD8 / 8;  // 16-byte chunks per BF16 row
  constexpr int RPI = 64 / C16;
  const int c16 = lane % C16;
  uint16_t* const dst = a.n_splits == 1 ? a.o + qo_base : a.o_part + (head_row0 * a.n_splits + split) * kD8;
  const size_t row_stride = (size_t)a.n_splits * kD8;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / C16;
    const int sw = ostw<D>(r);
    uint4 w = *reinterpret_cast<const uint4*>(stage + r * (kD8 * 2) + 16 * (c16 ^ (sw >> 1)));
    if (sw & 1) w = make_uint4(w.z, w.w, w.x, w.y);
    const int row = q0 + wave * 32 + r;
    if (row < N) *reinterpret_cast<uint4*>(dst + (size_t)row * row_stride + 8 * c16) = w;
  }
}

template <int D, bool CAUSAL, int W>
static hipError_t launch_fp8_t(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, W>), dim3(a.nwg), dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fp8_d(const FwdArgs& a, bool causal, hipStream_t stream) {
  if (a.rows == kFwdWaveRows * 8)
    return causal ? launch_fp8_t<D, true, 8>(a, stream) : launch_fp8_t<D, false, 8>(a, stream);
  return causal ? launch_fp8_t<D, true, 4>(a, stream) : launch_fp8_t<D, false, 4>(a, stream);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_fp8_d<128>(a, causal, stream) : launch_fp8_d<64>(a, causal, stream);
}

}  // namespace fa
