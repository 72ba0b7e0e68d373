// Exact tiled attention forward pass for gfx950.
//
// What it computes: O = softmax(scale Q K^T) V and lse = ln sum exp(scale q.k),
// tiled with the online softmax ("Flash Attention Mechanics: How Tiled
// Attention Fits in SRAM", section "The Tiling Algorithm"; "Why is standard
// attention memory-bound, and how does FlashAttention fix it?", "Step 3"). The
// query-outer loop order follows the FA2 schedule described in "FlashAttention
// HBM bytes, one head, 8K" ("A strong answer"): each work-group owns one query
// block, streams every K/V tile of its head, and writes its O tile once.
//
// Mapping onto CDNA4:
//   * 256 threads = 4 waves; each wave owns 32 query rows (128 per work-group).
//     Registers are budgeted for two work-groups per CU (two waves per SIMD),
//     so one wave's softmax arithmetic overlaps the other's matrix products.
//   * K/V tiles of 64 keys go HBM -> LDS with direct loads
//     (global_load_lds_dwordx4: lane l of a wave fills bytes 16 l .. 16 l + 15
//     of a 1 KiB block), double buffered; the loads of K(t+1) and V(t) are
//     placed among the matrix products of step t (each one holds up its
//     wave's issue for a while) and waited for at the next step's barrier.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (A = K from LDS, B = Q^T held in registers for the whole sweep). In the
//     result each lane holds 16 keys of ONE query row, so the row max and row
//     sum are in-lane reductions plus one permlane32 swap, and the same
//     registers, rounded to BF16, are directly the B operand (P^T) of the
//     second product O^T = V^T P^T -- no LDS round trip for P.
//   * V^T operands come from LDS with ds_read_b64_tr_b16 (transposed reads).
//   * Softmax in base 2: t = s * scale * log2(e); p = 2^(t - m). A row's
//     reference max m moves (and O and l are rescaled by 2^(m_old - m_new))
//     only when a tile's max exceeds it by more than 8, so most tiles skip the
//     rescale; the result is the same for any reference.
//   * Causal: K/V tiles past the block's last row are never loaded; every
//     wave takes every tile of its block, and only the diagonal tiles (and a
//     ragged tail) take the masked path.
//   * Grid: logical id -> (batch, head, query block, key split) with the
//     query blocks of a head adjacent (heaviest first when causal), and
//     logical ids laid out so that each XCD gets one contiguous range: a
//     head's K/V is then shared in one XCD's L2.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int W>
struct FwdCfg {
  static constexpr int CPR = D / 8;                       // 16-byte chunks per K/V row
  static constexpr int RPB = 64 / CPR;                    // rows per 1 KiB direct-load block
  static constexpr int BLOCKS = kFwdKeys / RPB;           // 1 KiB blocks per K (or V) tile
  static constexpr int BPW = BLOCKS / W;                  // blocks per wave per tile
  static constexpr int ROWS = kFwdWaveRows * W;           // query rows per work-group
  static constexpr int TILE_CHUNKS = kFwdKeys * CPR;
  static constexpr int KK = D / 16;                       // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;                       // 32-wide d tiles of O^T
};

// XOR swizzles of the 16-byte chunk index within a tile row (in LDS). They keep
// the two read patterns free of bank conflicts: K fragment reads (32 rows, one
// chunk column) and V transposed reads (4 rows x 4 chunks per half wave).
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }


// The reference max of a row moves only when a tile's max exceeds it by more
// than this many base-2 units; until then p = 2^(t - m) <= 2^8, and O and l are
// rescaled together when it does move, so O / l and m + log2 l are unchanged.
constexpr float kRescaleSlack = 8.f;

template <int D, bool CAUSAL, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D, W>;
  // K buffers 0, 1 then V buffers 0, 1; after the sweep each wave stages its
  // output rows here for coalesced stores (one wave's 32 BF16 rows take half
  // a tile, so eight waves fit).
  __shared__ uint4 smem[4][C::TILE_CHUNKS];
  // With 8 waves (one work-group per CU, so LDS is to spare) each wave stages
  // its 32 Q rows here by direct loads (rows XOR-swizzled as K) and reads its
  // operand from them: loading the operand layout straight from HBM takes 32
  // bytes of 32 rows per load, and at the start of every work-group those
  // requests held up step 0 by about a microsecond (3% of the 1-head 8K call).
  constexpr bool kStageQ = W == 8;
  __shared__ uint4 q_lds[kStageQ ? W * 32 * C::CPR : 1];
  uint4 (*k_lds)[C::TILE_CHUNKS] = smem;
  uint4 (*v_lds)[C::TILE_CHUNKS] = smem + 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;    // half of the wave (k-slot group)
  const int li = lane & 31;   // query row within the wave / column of S^T

  // ---- grid order: XCD-contiguous; groups of head_group heads, then query
  // block (heaviest first when causal), then head within the group, then key
  // split. A group is one XCD's range when causal grids allow it, so each XCD
  // starts all its heaviest blocks first (one head after another left the
  // light blocks of the first head ahead of the heavy blocks of the next: 7%
  // on 32 causal heads of 4K); otherwise head_group = 1 and a head's blocks
  // sit together on one XCD and share its K/V in that L2. With splits each
  // XCD takes all splits of a few blocks, so it reads only those blocks' Q
  // when every work-group starts at once (8 XCDs reading all of Q cost the
  // 1-head 8K call 4%), while K/V chunks are streamed once per XCD.
  const int lid = xcd_contiguous(blockIdx.x, a.nwg);
  int qb, split, bh;
  int split_tiles;   // key tiles per split of this block
  int block_splits;  // splits of this block (1: it writes O and lse itself)
  fwd_block_map(lid, a, CAUSAL, qb, split, bh, split_tiles, block_splits);
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int N = a.N;
  const int q0 = qb * C::ROWS;
  const size_t qo_base = (size_t)(b * a.Hq + h) * (size_t)N * D;
  const int t_begin = split * split_tiles;
  const uint16_t* kg = a.k + ((size_t)(b * a.Hkv + hk) * (size_t)N + (size_t)t_begin * kFwdKeys) * D;
  const uint16_t* vg = a.v + ((size_t)(b * a.Hkv + hk) * (size_t)N + (size_t)t_begin * kFwdKeys) * D;
  const int n_keys = N - t_begin * kFwdKeys;  // keys from the split's first one to the end

  const int kv_end = CAUSAL ? min(N, q0 + C::ROWS) : N;
  const int n_tiles = min((kv_end + kFwdKeys - 1) / kFwdKeys, t_begin + split_tiles) - t_begin;
  if (n_tiles <= 0) return;  // this split lies past the block's last visible key

  // Every wave takes every tile of its block; with causal masking the last
  // tile of a block can be wholly above the rows of its first waves, whose
  // scores there are all masked (p = 0).
  const int wave_q0 = q0 + wave * 32;

  // ---- direct HBM -> LDS loads of one K or V tile. Lane l fills physical chunk
  // l % CPR of tile row r, which holds logical chunk (l % CPR) ^ swizzle(r); the
  // byte offsets from the tile's first row are fixed per lane. In a tile that
  // runs past the last key, rows past it are clamped to it: finite data whose
  // scores are masked.
  const int dma_row = lane / C::CPR;
  const int dma_p = lane % C::CPR;
  uint32_t kdo[C::BPW], vdo[C::BPW];
#pragma unroll
  for (int x = 0; x < C::BPW; ++x) {
    const int r = (wave * C::BPW + x) * C::RPB + dma_row;
    kdo[x] = 2u * (uint32_t)(r * D + 8 * (dma_p ^ kswz<D>(r)));
    vdo[x] = 2u * (uint32_t)(r * D + 8 * (dma_p ^ vswz<D>(r)));
  }
  auto issue = [&](const uint16_t* src, const uint32_t* offs, bool is_v, int tile, uint4* dst) {
    const uint16_t* base = src + (size_t)tile * kFwdKeys * D;
    const int rows = n_keys - tile * kFwdKeys;
    const uint32_t l0 = lds_addr(dst) + 1024u * (uint32_t)(wave * C::BPW);
    if (rows >= kFwdKeys) {
#pragma unroll
      for (int x = 0; x < C::BPW; ++x) dma16(base, offs[x], l0 + 1024u * x);
    } else {
#pragma unroll
      for (int x = 0; x < C::BPW; ++x) {
        const int r = (wave * C::BPW + x) * C::RPB + dma_row;
        const int sw = is_v ? vswz<D>(r) : kswz<D>(r);
        dma16(base, 2u * (uint32_t)(min(r, rows - 1) * D + 8 * (dma_p ^ sw)), l0 + 1024u * x);
      }
    }
  };

  // Steps whose K(t+1) and V(t) tiles are both full place their loads among
  // the matrix products (block x of K before k-step kx(x) of the scores,
  // block x of V before key group vx(x) of the PV products) instead of all at
  // the start of the step: every direct load holds up its wave's instruction
  // issue for a while, and spread out these stalls overlap the products.
  auto kx = [](int x) {
    return C::BPW == 2 ? (x == 0 ? C::KK / 4 : 5 * C::KK / 8) : (2 * x + 1) * C::KK / (2 * C::BPW);
  };
  auto vx = [](int x) { return C::BPW >= 4 ? x : (C::BPW == 2 ? 1 + x : 2); };
  // Tiles from the split's first key that hold 64 keys (n_tiles or, when the
  // last tile of the sequence is partial, n_tiles - 1). Step t spreads its
  // loads iff t + 1 < full_tiles: K(t+1) exists and both tiles are full.
  const int full_tiles = min(n_tiles, n_keys / kFwdKeys);

  issue(kg, kdo, false, 0, k_lds[0]);

  // ---- Q^T operand of this lane's row, kept in registers for the whole sweep.
  // A negative scale is folded into Q (sign flip is exact), so the kernel
  // works with c = |scale| log2(e) > 0 and max(t) = c max(s). For scale 0 it
  // uses the smallest normal float: every finite score then gives exactly
  // p = 2^0 = 1, as scale 0 does, while masked (-inf) scores still give 0.
  const int qi = q0 + wave * 32 + li;
  const uint32_t sign = a.c < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.c), 1.17549435e-38f);
  bf16x8 qf[C::KK];
  if constexpr (kStageQ) {
    // Rows past N repeat row N - 1 (finite; their results are never stored).
    const int wrow0 = min(q0 + wave * 32, N - 1);
    const uint16_t* qsrc = a.q + qo_base + (size_t)wrow0 * D;
    const uint32_t ql0 = lds_addr(q_lds) + (uint32_t)(wave * 32 * D * 2);
#pragma unroll
    for (int x = 0; x < 32 / C::RPB; ++x) {
      const int r = x * C::RPB + dma_row;
      const int rel = min(q0 + wave * 32 + r, N - 1) - wrow0;
      dma16(qsrc, 2u * (uint32_t)(rel * D + 8 * (dma_p ^ kswz<D>(r))), ql0 + 1024u * x);
    }
  } else {
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + qo_base + (size_t)(qi < N ? qi : 0) * D);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      uint4 w = qi < N ? qrow[2 * kk + g] : make_uint4(0u, 0u, 0u, 0u);
      w.x ^= sign; w.y ^= sign; w.z ^= sign; w.w ^= sign;
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // Staged Q: this lane's operand (row li, chunks 2 kk + g) once step 0's
  // wait and barrier have passed.
  auto read_q = [&]() {
    const char* qb = reinterpret_cast<const char*>(q_lds) + wave * 32 * D * 2 + li * D * 2;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qb + 16 * ((2 * kk + g) ^ kswz<D>(li)));
      w.x ^= sign; w.y ^= sign; w.z ^= sign; w.w ^= sign;
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  };

  // ---- per-lane LDS byte offsets (tile-relative). K: row li, chunk 2 kk + g.
  // V^T: lane t16 of each 16-lane block names row t16 / 4 of a 4-key group and
  // 4 columns at 32 dt + 16 vch + 4 (t16 % 4).
  int koff[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) koff[kk] = 16 * (li * C::CPR + ((2 * kk + g) ^ kswz<D>(li)));
  const int t16 = lane & 15;
  const int vch = (lane >> 4) & 1;
  const int vrow = 4 * g + (t16 >> 2);  // + 32 jt + 16 hh (+ 8): multiples of 4 keep vswz fixed
  int voff[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int chunk = (32 * dt + 16 * vch + 4 * (t16 & 3)) >> 3;
    voff[dt] = 16 * (vrow * C::CPR + (chunk ^ vswz<D>(vrow))) + 8 * (t16 & 1);
  }

  float m_run = -INFINITY;  // reference max of t (base-2 scaled scores) for row qi
  float l_run = 0.f;        // running sum of 2^(t - m_run) over this lane's keys
  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  f32x16 pp0, pp1;          // p of the previous tile (FP32), packed and summed one step later
  bf16x8 pb[2][2];          // that tile's P^T operands (BF16)

  // S^T = K Q^T for two 32-key sub-tiles; the two accumulation chains
  // interleave. With valu, the products also carry the packing and summing of
  // the previous tile's p (issued in the same region).
  auto scores = [&](const char* kb, f32x16& s0, f32x16& s1, bool valu, bool dma, const uint16_t* kbase,
                    uint32_t kl0) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (dma) {
#pragma unroll
        for (int x = 0; x < C::BPW; ++x)
          if (kk == kx(x)) dma16(kbase, kdo[x], kl0 + 1024u * x);
      }
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kb + koff[kk]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kb + koff[kk] + 32 * C::CPR * 16);
      s0 = mfma32(k0, qf[kk], s0);
      s1 = mfma32(k1, qf[kk], s1);
    }
    // Reads run two k-steps ahead of the products.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (kk + 2 < C::KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (valu) __builtin_amdgcn_sched_group_barrier(0x002, 56 / C::KK, 0);
    }
  };

  // Keys outside the mask become -inf (only diagonal and ragged tiles need it).
  // Key kv0 + o + 4 g (o = 32 jt + 8 (r/4) + r%4, a constant) is visible iff
  // it is <= min(N-1, qi) (causal) or <= N-1, i.e. iff o <= lim.
  auto apply_mask = [&](int kv0, f32x16& s0, f32x16& s1) {
    const int lim = (CAUSAL ? min(N - 1, qi) : N - 1) - kv0 - 4 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 8 * (r >> 2) + (r & 3);
      if (o > lim) s0[r] = -INFINITY;
      if (o + 32 > lim) s1[r] = -INFINITY;
    }
  };

  // P^T operands of a tile, rounded to BF16: registers 8 hh .. 8 hh + 7 of
  // sub-tile jt hold keys 32 jt + 16 hh + 8 (e/4) + 4 g + e%4, e = 0..7. The
  // row sum (of the FP32 values) joins l.
  auto finish_p = [&](const f32x16& p0, const f32x16& p1) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      pb[0][hh] = pack_bf16x8(p0[8 * hh + 0], p0[8 * hh + 1], p0[8 * hh + 2], p0[8 * hh + 3],
                              p0[8 * hh + 4], p0[8 * hh + 5], p0[8 * hh + 6], p0[8 * hh + 7]);
      pb[1][hh] = pack_bf16x8(p1[8 * hh + 0], p1[8 * hh + 1], p1[8 * hh + 2], p1[8 * hh + 3],
                              p1[8 * hh + 4], p1[8 * hh + 5], p1[8 * hh + 6], p1[8 * hh + 7]);
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

  // O^T += V^T P^T. The V^T operand of lane l is column d = 32 dt + l%32 at the
  // same 8 keys as its P^T registers, gathered with two transposed reads of 4 keys.
  auto pv = [&](const char* vb, bool dma, const uint16_t* vbase, uint32_t vl0) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (dma) {
#pragma unroll
          for (int x = 0; x < C::BPW; ++x)
            if (2 * jt + hh == vx(x)) dma16(vbase, vdo[x], vl0 + 1024u * x);
        }
        const int rowoff = (32 * jt + 16 * hh) * C::CPR * 16;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const i16x4 lo = lds_read_tr(vb + voff[dt] + rowoff);
          const i16x4 hi = lds_read_tr(vb + voff[dt] + rowoff + 8 * C::CPR * 16);
          oacc[dt] = mfma32(join_bf16x8(lo, hi), pb[jt][hh], oacc[dt]);
        }
      }
  };

  // Row max of a tile (keys kv0 + 32 jt + 8 (r/4) + 4 g + r%4 of row qi): two
  // chains of three-input maxima, then the other half-wave's value.
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

  // p = 2^(s c - m) in place; with c > 0 a -inf score gives p = 0.
  auto exps = [&](f32x16& s0, f32x16& s1) {
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = exp2_hw(fmaf(s0[r], c, nm));
      s1[r] = exp2_hw(fmaf(s1[r], c, nm));
    }
  };

  // Softmax of tile t (its scores in s0, s1) alongside O += V(t-1)^T P(t-1)
  // from the V buffer vb: the matrix cores and the vector ALUs of one wave
  // work at the same time. When a row's reference max moves, l is rescaled at
  // once and O after P(t-1) V(t-1) has joined it (both were formed at the old
  // reference). On return pp0, pp1 hold p of tile t.
  auto softmax_pv = [&](int kv0, f32x16& s0, f32x16& s1, const char* vb, bool with_pv, bool dma,
                        const uint16_t* vbase, uint32_t vl0) {
    if ((kv0 + kFwdKeys > N) || (CAUSAL && kv0 + kFwdKeys - 1 > wave_q0)) apply_mask(kv0, s0, s1);
    // The row max, the reference update and the exponentials form one
    // branch-free block with the products of P(t-1), so the products run
    // while the max is reduced. alpha = 1 exactly where the reference stays
    // (the select also keeps -inf - -inf out).
    const float mt = tile_max(s0, s1) * c;
    const bool grow = mt > m_run + kRescaleSlack;
    const float alpha = grow ? exp2_hw(m_run - mt) : 1.f;  // 0 where m was -inf
    m_run = grow ? mt : m_run;
    l_run *= alpha;
    const bool any_grow = __any(grow);
    exps(s0, s1);
    if (with_pv) {
      pv(vb, dma, vbase, vl0);
      // Each product of P(t-1) with its two V^T reads and a share of the max
      // reduction and this tile's exponentials.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 4 * C::DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);
      }
    }
    // Keep the exponentials in this step: without this the compiler sinks
    // them into the next one, past the barrier, next to their first use.
    asm volatile("" : "+v"(s0), "+v"(s1));
    pp0 = s0;
    pp1 = s1;
    if (any_grow) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
  };

  // One step of the sweep. Step t < n_tiles: the loads of K(t+1) and V(t) are
  // issued, S(t) = K(t) Q^T is formed, then the softmax of tile t runs with
  // O += V(t-1)^T P(t-1). Step n_tiles only adds V^T P of the last tile. KB =
  // t & 1 is a compile-time constant, so every LDS address is a per-lane
  // register plus an immediate.
  // spread: the loads go among the products (t + 1 < full_tiles); otherwise
  // they are issued at the start.
  auto step = [&](auto kb_c, int t, bool with_pv, bool spread) {
    constexpr int KB = decltype(kb_c)::value;
    spread = spread && !kSyncCheck;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!spread) {
      if (t + 1 < n_tiles) issue(kg, kdo, false, t + 1, k_lds[KB ^ 1]);
      issue(vg, vdo, true, t, v_lds[KB]);
    }
    sync_check_group();
    if (kStageQ && !with_pv) read_q();
    const uint16_t* kbase = kg + (size_t)(t + 1) * kFwdKeys * D;
    const uint32_t kl0 = lds_addr(k_lds[KB ^ 1]) + 1024u * (uint32_t)(wave * C::BPW);
    const uint16_t* vbase = vg + (size_t)t * kFwdKeys * D;
    const uint32_t vl0 = lds_addr(v_lds[KB]) + 1024u * (uint32_t)(wave * C::BPW);
    __builtin_amdgcn_sched_barrier(0);
    if (with_pv) finish_p(pp0, pp1);
    f32x16 s0, s1;
    scores(reinterpret_cast<const char*>(k_lds[KB]), s0, s1, with_pv, spread, kbase, kl0);
    sync_check_group();
    // Keep the packing and summing beside the score products: without this
    // the compiler sinks them past the mask branch, next to their first use.
    if (with_pv) asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]), "+v"(l_run));
    softmax_pv((t_begin + t) * kFwdKeys, s0, s1, reinterpret_cast<const char*>(v_lds[KB ^ 1]), with_pv, spread,
               vbase, vl0);
    sync_check_group();
  };
  auto last = [&](auto kb_c) {
    constexpr int KB = decltype(kb_c)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    finish_p(pp0, pp1);
    pv(reinterpret_cast<const char*>(v_lds[KB ^ 1]), false, nullptr, 0u);
    sync_check_group();
  };

  // ---- the sweep: step 0 has no product to overlap; the steps in between go
  // two per trip; the last product follows the last step.
  step(IC<0>{}, 0, false, false);
  int t = 1;
  for (; t + 2 < full_tiles; t += 2) {
    step(IC<1>{}, t, true, true);
    step(IC<0>{}, t + 1, true, true);
  }
  // At most three steps remain: t + 2 >= full_tiles >= n_tiles - 1.
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

  // ---- epilogue: O = O / l, lse = (m + log2 l) ln 2. O is rounded to BF16
  // (nearest even), to the output or, with key splits, to the split's
  // normalised partial. Each wave stages its 32 rows in LDS (row-major, 8-byte
  // units XOR-swizzled by row so that both the fragment-order writes and the
  // row-order reads are free of bank conflicts), then stores whole rows: every
  // store instruction writes 1 KiB of contiguous row segments.
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
  const size_t head_row0 = (size_t)(b * a.Hq + h) * N;
  if (qi < N && g == 0) {
    if (block_splits == 1) a.lse[head_row0 + qi] = lse_v;
    else a.lse_part[(head_row0 + qi) * a.n_splits + split] = lse_v;
  }
  __syncthreads();  // every wave is done with the K/V buffers
  char* stage = reinterpret_cast<char*>(smem) + wave * (32 * D * 2);
  // 8-byte units: unit e = 8 dt + 2 rq + g of row li (columns 4 e .. 4 e + 3).
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e = 8 * dt + 2 * rq + g;
      const int pe = e ^ (D == 128 ? li : ((li >> 1) & 15));
      *reinterpret_cast<uint2*>(stage + li * (D * 2) + 8 * pe) =
          pack_bf16x4(oacc[dt][4 * rq + 0] * inv, oacc[dt][4 * rq + 1] * inv,
                      oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
    }
  wave_sync_lds();
  sync_check_group();
  // Row order: lane l takes 16-byte chunk l % (D / 8) of row l / (D / 8) + RPI i,
  // to the output or (split) to the split's partial row.
  constexpr int CPR16 = D / 8;
  constexpr int RPI = 64 / CPR16;
  const int c16 = lane % CPR16;
  uint16_t* const dst = block_splits == 1 ? a.o + qo_base : a.o_part + (head_row0 * a.n_splits + split) * D;
  const size_t row_stride = block_splits == 1 ? (size_t)D : (size_t)a.n_splits * D;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR16;
    const int sw = D == 128 ? r : ((r >> 1) & 15);
    uint4 w = *reinterpret_cast<const uint4*>(stage + r * (D * 2) + 16 * (c16 ^ (sw >> 1)));
    if (sw & 1) w = make_uint4(w.z, w.w, w.x, w.y);
    const int row = q0 + wave * 32 + r;
    if (row < N) *reinterpret_cast<uint4*>(dst + (size_t)row * row_stride + 8 * c16) = w;
  }
}

// Merge each row's non-empty key splits with the log-sum-exp combine; D / 8
// lanes take one row, eight columns each, so every partial of a row is one
// 16-byte load per lane. The work-groups take the query blocks in the forward
// grid's order (without its key-split level) through the same XCD-contiguous
// mapping, a block's rows in a.rows / RPG consecutive work-groups: each XCD
// then merges the blocks whose partials its own forward work-groups wrote.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kMergeThreads) void fa_fwd_combine_kernel(FwdArgs a) {
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPG = kMergeThreads / LPR;   // rows per work-group
  const int chunks = a.rows / RPG;           // work-groups per query block
  const int lid = xcd_contiguous(blockIdx.x, a.B * a.Hq * a.nqb * chunks);
  const int blk = lid / chunks;
  const int grp = blk / (a.head_group * a.nqb);
  const int rem_g = blk - grp * a.head_group * a.nqb;
  const int gh = min(a.head_group, a.B * a.Hq - grp * a.head_group);
  const int qs = rem_g / gh;
  const int bh = grp * a.head_group + (rem_g - qs * gh);
  const int qb = CAUSAL ? a.nqb - 1 - qs : qs;
  const int n = qb * a.rows + (lid - blk * chunks) * RPG + (int)threadIdx.x / LPR;
  if (n >= a.N) return;
  const size_t row = (size_t)bh * a.N + n;
  const int col = 8 * (threadIdx.x % LPR);
  const int kv_end = CAUSAL ? min(a.N, qb * a.rows + a.rows) : a.N;
  const int tiles = (kv_end + kFwdKeys - 1) / kFwdKeys;
  int S;
  if (CAUSAL && a.split_target > 0) {
    S = (tiles + a.split_target - 1) / a.split_target;
    if (S == 1) return;  // the block's only split wrote O and lse itself
  } else {
    S = min(a.n_splits, (tiles + a.split_tiles - 1) / a.split_tiles);
  }
  merge_splits8<D>(a.o_part + row * a.n_splits * D + col, a.lse_part + row * a.n_splits, S, a.o + row * D + col,
                   a.lse + row, col == 0);
}

template <int D, bool CAUSAL, int W>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, W>), dim3(a.nwg), dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, hipStream_t stream) {
  if (a.rows == kFwdWaveRows * 8)
    return causal ? launch_fwd_t<D, true, 8>(a, stream) : launch_fwd_t<D, false, 8>(a, stream);
  return causal ? launch_fwd_t<D, true, 4>(a, stream) : launch_fwd_t<D, false, 4>(a, stream);
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_fwd_d<128>(a, causal, stream) : launch_fwd_d<64>(a, causal, stream);
}

// One work-group per (query block, RPG-row chunk of it). Key splits are only
// planned for grids of fewer query blocks than twice the CU count, so the
// grid stays far below the int range the kernel indexes it with.
template <int D, bool CAUSAL>
static hipError_t launch_combine_t(const FwdArgs& a, hipStream_t stream) {
  const int chunks = a.rows / (kMergeThreads / (D / 8));
  const size_t nwg = (size_t)a.B * a.Hq * a.nqb * chunks;
  if (a.rows % (kMergeThreads / (D / 8)) != 0 || nwg > (size_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fa_fwd_combine_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_combine_t<128, true>(a, stream) : launch_combine_t<128, false>(a, stream);
  return causal ? launch_combine_t<64, true>(a, stream) : launch_combine_t<64, false>(a, stream);
}

}  // namespace fa
