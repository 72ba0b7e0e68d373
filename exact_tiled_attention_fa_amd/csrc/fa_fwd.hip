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
//     of a 1 KiB block), double buffered; the loads of tile t+1 are issued
//     before the math of tile t and waited for at the next tile's barrier.
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
//   * Causal: K/V tiles past the block's last row are never loaded; a wave
//     skips the math of tiles wholly above its rows; only the diagonal tiles
//     (and a ragged tail) take the masked path.
//   * Grid: logical id -> (batch, head, query block) with the query blocks of
//     a head adjacent (heaviest first when causal), and logical ids laid out so
//     that each XCD gets one contiguous range: a head's K/V is then shared in
//     one XCD's L2.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int CPR = D / 8;                       // 16-byte chunks per K/V row
  static constexpr int RPB = 64 / CPR;                    // rows per 1 KiB direct-load block
  static constexpr int BLOCKS = kFwdKeys / RPB;           // 1 KiB blocks per K (or V) tile
  static constexpr int BPW = BLOCKS / 4;                  // blocks per wave per tile
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

__device__ __forceinline__ uint2 pack_bf16x4(float a0, float a1, float a2, float a3) {
  __bf16 b0 = (__bf16)a0, b1 = (__bf16)a1, b2 = (__bf16)a2, b3 = (__bf16)a3;
  uint2 r;
  r.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
  r.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
  return r;
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// fills bytes 16 l .. 16 l + 15 of the 1 KiB block at lds_dst, whose LDS
// address goes in M0. Issued through inline assembly so that the compiler's
// wait-count pass, which cannot tell which LDS buffer a direct load writes,
// does not make the current tile's LDS reads wait for the next tile's loads;
// the kernel waits for them itself (s_waitcnt vmcnt(0)) before the barrier
// that hands the buffer to its readers. M0 is saved and restored around it.
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// The reference max of a row moves only when a tile's max exceeds it by more
// than this many base-2 units; until then p = 2^(t - m) <= 2^8, and O and l are
// rescaled together when it does move, so O / l and m + log2 l are unchanged.
constexpr float kRescaleSlack = 8.f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ uint4 k_lds[2][C::TILE_CHUNKS];
  __shared__ uint4 v_lds[2][C::TILE_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;    // half of the wave (k-slot group)
  const int li = lane & 31;   // query row within the wave / column of S^T

  // ---- grid order: XCD-contiguous; head-major, then key split, then query
  // block (heaviest first when causal), so the blocks sharing one K/V chunk sit
  // together on one XCD.
  const int lid = xcd_contiguous(blockIdx.x, a.nwg);
  const int per_head = a.nqb * a.n_splits;
  const int bh = lid / per_head;
  const int rem = lid - bh * per_head;
  const int split = rem / a.nqb;
  int qb = rem - split * a.nqb;
  if (CAUSAL) qb = a.nqb - 1 - qb;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int N = a.N;
  const int q0 = qb * kFwdRows;
  const size_t qo_base = (size_t)(b * a.Hq + h) * (size_t)N * D;
  const uint16_t* kg = a.k + (size_t)(b * a.Hkv + hk) * (size_t)N * D;
  const uint16_t* vg = a.v + (size_t)(b * a.Hkv + hk) * (size_t)N * D;

  const int kv_end = CAUSAL ? min(N, q0 + kFwdRows) : N;
  const int t_begin = split * a.split_tiles;
  const int n_tiles = min((kv_end + kFwdKeys - 1) / kFwdKeys, t_begin + a.split_tiles) - t_begin;
  if (n_tiles <= 0) return;  // this split lies past the block's last visible key

  // ---- direct HBM -> LDS loads of one K or V tile. Lane l fills physical chunk
  // l % CPR of tile row r, which holds logical chunk (l % CPR) ^ swizzle(r).
  // Rows past N are clamped to row N-1: finite data whose scores are masked.
  const int dma_row = lane / C::CPR;
  const int dma_p = lane % C::CPR;
  auto issue_k = [&](int tile, uint4* dst) {
#pragma unroll
    for (int x = 0; x < C::BPW; ++x) {
      const int blk = wave * C::BPW + x;
      const int r = blk * C::RPB + dma_row;
      const int key = min((t_begin + tile) * kFwdKeys + r, N - 1);
      dma16(kg + (size_t)key * D + 8 * (dma_p ^ kswz<D>(r)), dst + blk * 64);
    }
  };
  auto issue_v = [&](int tile, uint4* dst) {
#pragma unroll
    for (int x = 0; x < C::BPW; ++x) {
      const int blk = wave * C::BPW + x;
      const int r = blk * C::RPB + dma_row;
      const int key = min((t_begin + tile) * kFwdKeys + r, N - 1);
      dma16(vg + (size_t)key * D + 8 * (dma_p ^ vswz<D>(r)), dst + blk * 64);
    }
  };

  // Tile 0's loads go out first; the Q fragments load while they fly.
  issue_k(0, k_lds[0]);
  issue_v(0, v_lds[0]);

  // ---- Q^T operand of this lane's row, kept in registers for the whole sweep.
  // A negative scale is folded into Q (sign flip is exact), so the kernel
  // works with c = |scale| log2(e) > 0 and max(t) = c max(s). For scale 0 it
  // uses the smallest normal float: every finite score then gives exactly
  // p = 2^0 = 1, as scale 0 does, while masked (-inf) scores still give 0.
  const int qi = q0 + wave * 32 + li;
  const uint32_t sign = a.c < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.c), 1.17549435e-38f);
  bf16x8 qf[C::KK];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + qo_base + (size_t)(qi < N ? qi : 0) * D);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      uint4 w = qi < N ? qrow[2 * kk + g] : make_uint4(0u, 0u, 0u, 0u);
      w.x ^= sign; w.y ^= sign; w.z ^= sign; w.w ^= sign;
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

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

  const int wave_q0 = q0 + wave * 32;
  const int wave_q1 = wave_q0 + 31;

  // S^T = K Q^T for two 32-key sub-tiles; the two accumulation chains interleave.
  auto scores = [&](const uint4* kbuf, f32x16& s0, f32x16& s1) {
    const char* kb = reinterpret_cast<const char*>(kbuf);
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kb + koff[kk]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kb + koff[kk] + 32 * C::CPR * 16);
      s0 = mfma32(k0, qf[kk], s0);
      s1 = mfma32(k1, qf[kk], s1);
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

  // Online softmax of one tile (lane holds keys kv0 + 32 jt + 8 (r/4) + 4 g + r%4
  // of row qi), then O^T += V^T P^T. With c > 0, a -inf score gives p = 0.
  auto softmax_pv = [&](const uint4* vbuf, f32x16& s0, f32x16& s1) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = max_xor32(mx);
    const float mt = mx * c;
    const bool grow = mt > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = exp2_hw(m_run - m_new);  // 1 for rows that keep their reference
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = exp2_hw(fmaf(s0[r], c, nm));
      const float p1 = exp2_hw(fmaf(s1[r], c, nm));
      s0[r] = p0;
      s1[r] = p1;
      rs += p0 + p1;
    }
    l_run += rs;

    // P^T operands: registers 8 hh .. 8 hh + 7 of sub-tile jt hold keys
    // 32 jt + 16 hh + 8 (e/4) + 4 g + e%4, e = 0..7.
    bf16x8 pb[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      pb[0][hh] = pack_bf16x8(s0[8 * hh + 0], s0[8 * hh + 1], s0[8 * hh + 2], s0[8 * hh + 3],
                              s0[8 * hh + 4], s0[8 * hh + 5], s0[8 * hh + 6], s0[8 * hh + 7]);
      pb[1][hh] = pack_bf16x8(s1[8 * hh + 0], s1[8 * hh + 1], s1[8 * hh + 2], s1[8 * hh + 3],
                              s1[8 * hh + 4], s1[8 * hh + 5], s1[8 * hh + 6], s1[8 * hh + 7]);
    }
    // The V^T operand of lane l is column d = 32 dt + l%32 at the same 8 keys,
    // gathered with two transposed reads of 4 keys each.
    const char* vb = reinterpret_cast<const char*>(vbuf);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rowoff = (32 * jt + 16 * hh) * C::CPR * 16;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const i16x4 lo = lds_read_tr(vb + voff[dt] + rowoff);
          const i16x4 hi = lds_read_tr(vb + voff[dt] + rowoff + 8 * C::CPR * 16);
          oacc[dt] = mfma32(join_bf16x8(lo, hi), pb[jt][hh], oacc[dt]);
        }
      }
  };

  // ---- main loop: the next tile streams into the other buffer during this tile's math.
  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = (t_begin + t) * kFwdKeys;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < n_tiles) {
      issue_k(t + 1, k_lds[(t + 1) & 1]);
      issue_v(t + 1, v_lds[(t + 1) & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (CAUSAL && kv0 > wave_q1) continue;  // every key of the tile is above this wave's rows
    f32x16 s0, s1;
    scores(k_lds[t & 1], s0, s1);
    if ((kv0 + kFwdKeys > N) || (CAUSAL && kv0 + kFwdKeys - 1 > wave_q0)) apply_mask(kv0, s0, s1);
    softmax_pv(v_lds[t & 1], s0, s1);
  }

  // ---- epilogue: O = O / l, lse = (m + log2 l) ln 2. Unsplit: O rounded to
  // BF16 (nearest even) straight to the output. Split: FP32 partials.
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
  if (qi < N) {
    const size_t row = (size_t)(b * a.Hq + h) * N + qi;
    if (a.n_splits == 1) {
      uint16_t* orow = a.o + qo_base + (size_t)qi * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const uint2 w = pack_bf16x4(oacc[dt][4 * rq + 0] * inv, oacc[dt][4 * rq + 1] * inv,
                                      oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * rq + 4 * g) = w;
        }
      if (g == 0) a.lse[row] = lse_v;
    } else {
      float* prow = a.o_part + (row * a.n_splits + split) * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float4 w = make_float4(oacc[dt][4 * rq + 0] * inv, oacc[dt][4 * rq + 1] * inv,
                                       oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
          *reinterpret_cast<float4*>(prow + 32 * dt + 8 * rq + 4 * g) = w;
        }
      if (g == 0) a.lse_part[row * a.n_splits + split] = lse_v;
    }
  }
}

// One wave per row: merge the row's non-empty key splits with the
// log-sum-exp combine.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fa_fwd_combine_kernel(FwdArgs a) {
  const size_t row = blockIdx.x;
  const int n = (int)(row % (size_t)a.N);
  const int qb = n / kFwdRows;
  const int kv_end = CAUSAL ? min(a.N, qb * kFwdRows + kFwdRows) : a.N;
  const int tiles = (kv_end + kFwdKeys - 1) / kFwdKeys;
  const int S = min(a.n_splits, (tiles + a.split_tiles - 1) / a.split_tiles);
  combine_row<D>(a.o_part + row * a.n_splits * D, a.lse_part + row * a.n_splits, S, a.o + row * D, a.lse + row);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3(a.nwg), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
  return causal ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_combine_t(const FwdArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)((size_t)a.B * a.Hq * a.N);
  hipLaunchKernelGGL((fa_fwd_combine_kernel<D, CAUSAL>), dim3(rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_combine_t<128, true>(a, stream) : launch_combine_t<128, false>(a, stream);
  return causal ? launch_combine_t<64, true>(a, stream) : launch_combine_t<64, false>(a, stream);
}

}  // namespace fa
