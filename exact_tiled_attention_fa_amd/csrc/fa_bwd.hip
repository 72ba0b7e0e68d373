// Backward pass of exact attention for gfx950 (head dims 64 and 128).
//
// What it computes: with P = softmax(scale Q K^T) (masked when causal) and the
// upstream gradient dO, the chain rule through O = P V gives
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta_i = sum_t dO_it O_it,
//   dQ = scale dS K,  dK = scale dS^T Q,
// and for GQA a KV head's dK, dV sum over the query heads that read it. As the
// pages describe for training ("Why is standard attention memory-bound, and
// how does FlashAttention fix it?", "Step 4: The result is exact, and the
// backward pass recomputes"), the scores are recomputed tile by tile from Q, K
// and the per-row statistic lse the forward pass saved; no N x N matrix is
// stored.
//
// Three launches:
//   * row pass: lse2 = lse log2(e) and -delta = -rowsum(dO O) per query row
//     (the forward's O; sum_j P_ij dP_ij = sum_t dO_it O_it); the dP products
//     start their accumulation from -delta, so they yield dP - delta at once;
//   * dK/dV: one work-group of 4 waves per (batch, KV head, 64-key block);
//     each wave owns 16 keys and keeps K^T and V^T of them in registers as
//     v_mfma_f32_16x16x32_bf16 B operands. It sweeps 64-row tiles of Q and dO
//     (double-buffered in LDS by direct loads) of every query head of the
//     group: S = Q K^T and dP = dO V^T (lane = key, four query rows per
//     register group), P = 2^(S c - lse2), dS = P (dP - delta), then
//     dV += P^T dO and dK += dS^T Q with the P / dS registers as A operands
//     and dO / Q gathered by transposed LDS reads;
//   * dQ: one work-group of 4 waves per (batch, query head, 128-row block),
//     the forward's layout: S^T = K Q^T and dP^T = V dO^T (lane = query row),
//     dS^T packed to BF16 as the B operand of dQ^T += K^T dS^T with K^T
//     gathered by transposed reads.
// Tiles that hold both row reads and transposed reads use a swizzle that keeps
// both patterns free of bank conflicts (sw2, swq below).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

template <int D>
struct BwdCfg {
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE_CHUNKS = kBwdTile * CPR;  // 64-row tiles (16 or 8 KiB)
  static constexpr int KK32 = D / 16;              // k-steps of a 32x32x16 product over d
  static constexpr int DT = D / 32;                // 32-wide d tiles
  static constexpr int KK16 = D / 32;              // k-steps of a 16x16x32 product over d
  static constexpr int TT = D / 16;                // 16-wide d tiles
  static constexpr int RPB = 512 / D;              // rows per 1 KiB direct-load block
  static constexpr int BPW = D / 32;               // blocks per wave per tile (4 waves)
};

// XOR swizzle of the 16-byte chunk index of tile row r, for tiles read both
// by rows (16 consecutive rows at one chunk) and transposed (4 rows from a
// 4-aligned start, two adjacent chunks); rows 16 apart share it, so row
// offsets that are multiples of 16 stay immediates.
//   d = 128 (16 chunks, a row spans the 64 banks): bijective on r & 15 and
//   8-valued on a transposed read's rows.
//   d = 64 (8 chunks, two rows per 64 banks, so row parity separates them):
//   a bit permutation of t = (r >> 1) & 7 (t0 -> bit 1, t1 -> bit 2, t2 ->
//   bit 0), bijective on t, and rows r, r + 2 of a transposed read differ in
//   bit 1, so their two-chunk pairs do not collide.
template <int D>
__device__ __forceinline__ int sw2(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 1) | (((r >> 2) & 1) << 2) | ((r >> 3) & 1);
}

// Swizzle of the dK/dV pass's Q and dO tiles, read by rows (16 rows at one
// chunk) and transposed with rows 4 b + (lane / 4) % 4 for 16-lane block b.
// Two 16-lane blocks share an LDS cycle of those 8-byte reads: measured, sw2
// (conflict-free within one block) still cost 134 M bank-conflict cycles, a
// third of the pass, and a swizzle built for blocks (0, 1) and (2, 3) sharing
// a cycle 67 M. This one gives distinct chunk pairs to the 8 rows of blocks
// (0, 1), (2, 3), (0, 2) and (1, 3) alike, and distinct chunks to 16 rows:
//   d = 128 (16 chunks per row): bits 1-2 = r & 3, bit 3 = bit 2 ^ bit 3 of r,
//     bit 0 = bit 3 of r;
//   d = 64 (8 chunks, two rows per bank line, parity separating them): the same
//     construction on t = (r >> 1) & 7 in 3 bits.
// (Checked on the CPU against a 64-bank model under both pairings.)
template <int D>
__device__ __forceinline__ int swq(int r) {
  if (D == 128) {
    const int f = (r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
    return (f << 1) | ((r >> 3) & 1);
  }
  const int t = (r >> 1) & 7;
  const int h = (t & 1) | ((((t >> 1) ^ (t >> 2)) & 1) << 1);
  return (h << 1) | ((t >> 2) & 1);
}

// Swizzle kinds of a tile: sw2 (dQ's K and V tiles), swq (dK/dV's Q, dO).
enum { kSw2 = 1, kSwQ = 2 };
template <int D, int SW>
__device__ __forceinline__ int swz(int r) {
  return SW == kSwQ ? swq<D>(r) : sw2<D>(r);
}

// Direct loads of the 64-row tile starting at row row0 of a row-major
// [rows, D] BF16 matrix into LDS: wave w fills the 1 KiB blocks
// BPW w .. BPW w + BPW - 1; lane l writes physical chunk l % CPR of its row
// with logical chunk (l % CPR) ^ sw. The base moves to the tile's first row in
// 64-bit arithmetic, so each lane's 32-bit byte offset spans one tile (at most
// 16 KiB) whatever the sequence length.
//
// The per-lane byte offsets within a full tile are computed once per
// work-group and kept in registers for the sweep: a load's offset register
// must not be overwritten while the load is in flight, so offsets computed
// afresh for every tile made the compiler wait for the next tile's loads
// before the current tile's first LDS reads (which reused those registers),
// undoing the double buffering.
// The only ragged tile of a sweep is the last one, whose rows past the end
// read row (rows - 1) % 64 of the tile (finite data the caller masks); its
// clamped offsets are precomputed the same way.
template <int D, int SW>
struct TileOffsets {
  uint32_t full[BwdCfg<D>::BPW];
  uint32_t tail[BwdCfg<D>::BPW];
  __device__ __forceinline__ TileOffsets(int wave, int lane, int rows) {
    using C = BwdCfg<D>;
    const int pc = lane % C::CPR;
    const int last = (rows - 1) % kBwdTile;
#pragma unroll
    for (int x = 0; x < C::BPW; ++x) {
      const int r = C::RPB * (C::BPW * wave + x) + lane / C::CPR;
      const int sw = swz<D, SW>(r);
      full[x] = 2u * (uint32_t)(r * D + 8 * (pc ^ sw));
      tail[x] = 2u * (uint32_t)(min(r, last) * D + 8 * (pc ^ sw));
    }
  }
};

// load_tile with the precomputed offsets (row0 a multiple of 64 below `rows`).
template <int D, int SW>
__device__ __forceinline__ void load_tile_at(const uint16_t* src, int row0, int rows, const TileOffsets<D, SW>& t,
                                             uint4* dst, int wave) {
  using C = BwdCfg<D>;
  const uint16_t* base = src + (size_t)row0 * D;
  const uint32_t l0 = lds_addr(dst) + 1024u * (uint32_t)(C::BPW * wave);
  // Two branches, each passing its precomputed registers as they are: a
  // select would put the offsets in fresh registers again. The ragged branch
  // issues the same instruction through a differently worded asm statement, so
  // the compiler cannot merge the branches into one load fed by a select.
  if (row0 + kBwdTile <= rows) {
#pragma unroll
    for (int x = 0; x < C::BPW; ++x) dma16(base, t.full[x], l0 + 1024u * x);
  } else {
#pragma unroll
    for (int x = 0; x < C::BPW; ++x) {
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "global_load_lds_dwordx4 %2, %3 ; ragged tile\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(l0 + 1024u * x), "v"(t.tail[x]), "s"(base)
          : "memory");
    }
  }
}

// s_waitcnt vmcnt(0) through the builtin (expcnt and lgkmcnt left at their
// maxima, 0x0F70 in the gfx9 encoding): unlike the same instruction in inline
// assembly, the compiler's wait-count pass sees it, so it knows that the loads
// issued before the loop (K^T, V^T, Q^T, dO^T held in registers) are complete
// inside the loop. With the inline-asm wait it did not, and made each tile's
// first products wait, load by load, for the next tile's direct loads.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace

// ---------------------------------------------------------------- row pass
// D / 8 lanes per row (8 columns each): -delta = -sum_t dO O in FP32, lse2 =
// lse log2(e); rows N .. Npad - 1 of each head get zeros.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_rows_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  const size_t row = (size_t)blockIdx.x * (256 / LPR) + (threadIdx.x / LPR);
  const int c16 = threadIdx.x % LPR;
  const size_t rows = (size_t)a.B * a.Hq * a.Npad;
  if (row >= rows) return;
  const size_t bh = row / a.Npad;
  const int n = (int)(row - bh * a.Npad);
  float s = 0.f;
  if (n < a.N) {
    const size_t src = (bh * a.N + n) * D + 8 * c16;
    const uint4 x = *reinterpret_cast<const uint4*>(a.o + src);
    const uint4 y = *reinterpret_cast<const uint4*>(a.dout + src);
    s = bf16_lo(x.x) * bf16_lo(y.x) + bf16_hi(x.x) * bf16_hi(y.x) + bf16_lo(x.y) * bf16_lo(y.y) +
        bf16_hi(x.y) * bf16_hi(y.y) + bf16_lo(x.z) * bf16_lo(y.z) + bf16_hi(x.z) * bf16_hi(y.z) +
        bf16_lo(x.w) * bf16_lo(y.w) + bf16_hi(x.w) * bf16_hi(y.w);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += shfl_xor(s, m);
  if (c16 == 0) {
    a.ndelta[row] = -s;
    a.lse2[row] = n < a.N ? a.lse[bh * a.N + n] * kLog2e : 0.f;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdArgs a, int nwg) {
  using C = BwdCfg<D>;
  __shared__ uint4 q_lds[2][C::TILE_CHUNKS];
  __shared__ uint4 do_lds[2][C::TILE_CHUNKS];
  __shared__ float4 st_lds[2][2][kBwdTile / 4];  // [buffer][lse2 | -delta][rows / 4]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b16 = lane >> 4;  // 16-lane block
  const int j16 = lane & 15;

  // Grid: XCD-contiguous; groups of hg_kv KV heads, then key blocks (the
  // first key blocks have the most query tiles when causal, so they start
  // first), then head within the group: a causal XCD range of several heads
  // starts all their heaviest blocks first.
  const int lid = xcd_contiguous(blockIdx.x, nwg);
  const int grp = lid / (a.hg_kv * a.nkb);
  const int rem_g = lid - grp * a.hg_kv * a.nkb;
  const int gh = min(a.hg_kv, a.B * a.Hkv - grp * a.hg_kv);  // KV heads in this group
  const int kb = rem_g / gh;
  const int bhk = grp * a.hg_kv + (rem_g - kb * gh);
  const int b = bhk / a.Hkv;
  const int hk = bhk - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int N = a.N;
  const int j0 = kb * kBwdKeyBlock;
  const int key = j0 + 16 * wave + j16;  // this lane's key (S columns, P^T rows)
  const size_t kv_base = (size_t)(b * a.Hkv + hk) * (size_t)N * D;

  // K^T and V^T as B operands: lane holds row `key`, columns 32 kk + 8 b16 .. + 7.
  bf16x8 kf[C::KK16], vf[C::KK16];
  {
    const int kr = min(key, N - 1);
    const uint4* krow = reinterpret_cast<const uint4*>(a.k + kv_base + (size_t)kr * D);
    const uint4* vrow = reinterpret_cast<const uint4*>(a.v + kv_base + (size_t)kr * D);
#pragma unroll
    for (int kk = 0; kk < C::KK16; ++kk) {
      kf[kk] = __builtin_bit_cast(bf16x8, krow[4 * kk + b16]);
      vf[kk] = __builtin_bit_cast(bf16x8, vrow[4 * kk + b16]);
    }
  }

  // Query tiles: for each query head of the group, tiles u_begin .. n_u - 1
  // (causal: none above the key block).
  const int n_u = (N + kBwdTile - 1) / kBwdTile;
  const int u_begin = CAUSAL ? j0 / kBwdTile : 0;
  const int per_head = n_u - u_begin;
  const int n_t = G * per_head;

  const TileOffsets<D, kSwQ> toff(wave, lane, N);
  const uint32_t st_off = 16u * (uint32_t)lane;
  // Tile t is query tile u of query head hk G + gq; (gq, u) step through the
  // tiles in order, without a division per tile.
  auto issue = [&](int gq, int u, int buf) {
    const size_t rb = (size_t)(b * a.Hq + hk * G + gq);
    load_tile_at<D, kSwQ>(a.q + rb * N * D, u * kBwdTile, N, toff, q_lds[buf], wave);
    load_tile_at<D, kSwQ>(a.dout + rb * N * D, u * kBwdTile, N, toff, do_lds[buf], wave);
    if (wave == 0 && lane < 16) {  // lse2 and -delta of the tile's 64 rows (256 B each)
      const size_t off = rb * a.Npad + (size_t)u * kBwdTile;
      dma16(a.lse2 + off, st_off, lds_addr(&st_lds[buf][0][0]));
      dma16(a.ndelta + off, st_off, lds_addr(&st_lds[buf][1][0]));
    }
  };

  // Per-lane LDS byte offsets. A fragments (rows): row 16 qt + j16, chunk 4 kk + b16.
  int aoff[C::KK16];
#pragma unroll
  for (int kk = 0; kk < C::KK16; ++kk) aoff[kk] = 16 * (j16 * C::CPR + ((4 * kk + b16) ^ swq<D>(j16)));
  // Transposed reads: lane names row 4 b16 + j16 / 4 (+ 32 u2, + 16 for the
  // second half) and 4 columns at 16 tt + 4 (j16 % 4); lane l receives column
  // 16 tt + j16 of rows 4 b16 .. 4 b16 + 3.
  int troff[C::TT];
  {
    const int r0 = 4 * b16 + (j16 >> 2);
#pragma unroll
    for (int tt = 0; tt < C::TT; ++tt)
      troff[tt] = 16 * (r0 * C::CPR + ((2 * tt + ((j16 & 3) >> 1)) ^ swq<D>(r0))) + 8 * (j16 & 1);
  }

  f32x4 dk[C::TT], dv[C::TT];
#pragma unroll
  for (int tt = 0; tt < C::TT; ++tt) dk[tt] = dv[tt] = f32x4{};

  const float c = a.c;
  issue(0, u_begin, 0);  // n_t >= 1: the key block lies below N
  int u_cur = u_begin;                                     // query tile of tile t
  int u_next = u_begin + 1 < n_u ? u_begin + 1 : u_begin;  // query tile and head of tile t + 1
  int gq_next = u_begin + 1 < n_u ? 0 : 1;
  // One query tile; the buffer index is a compile-time constant (the loop
  // takes two tiles per trip), so every LDS address is a register plus an
  // immediate: with a run-time index each of the tile's 96 reads took an
  // address add.
  // The products and weights of one query tile, MASKED for the tiles that hold
  // keys past N, rows past N or (causal) keys above a row: the last key
  // block, the last query tile and the diagonal tile. The others take no mask
  // (a mask in every tile turned into a branch per weight).
  auto tile_body = [&](auto buf_c, auto mask_c, int i0) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool MASKED = decltype(mask_c)::value != 0;
    const char* qb = reinterpret_cast<const char*>(q_lds[buf]);
    const char* db = reinterpret_cast<const char*>(do_lds[buf]);

    // S = Q K^T and dP = dO V^T for the group of 16 query rows qt, from
    // fragments read one group ahead into alternating register sets. A
    // scheduling barrier after each set's reads keeps them where they are
    // written (left to itself the compiler read every fragment right before
    // its product, one read in flight); the wait for the data stays at its
    // first use. (An empty asm statement naming the registers would also hold
    // the reads in place, but as a use of the data it made the wave wait for
    // every read right there.)
    f32x4 s[4], dp[4];
    bf16x8 fq[2][C::KK16], fd[2][C::KK16];
    auto read_a = [&](int qt) {
#pragma unroll
      for (int kk = 0; kk < C::KK16; ++kk) {
        fq[qt & 1][kk] = *reinterpret_cast<const bf16x8*>(qb + aoff[kk] + qt * 16 * C::CPR * 16);
        fd[qt & 1][kk] = *reinterpret_cast<const bf16x8*>(db + aoff[kk] + qt * 16 * C::CPR * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // dP starts from -delta of its rows, so the products leave dP - delta.
    auto sdp = [&](int qt) {
      s[qt] = f32x4{};
      dp[qt] = __builtin_bit_cast(f32x4, st_lds[buf][1][4 * qt + b16]);
#pragma unroll
      for (int kk = 0; kk < C::KK16; ++kk) {
        s[qt] = mfma16(fq[qt & 1][kk], kf[kk], s[qt]);
        dp[qt] = mfma16(fd[qt & 1][kk], vf[kk], dp[qt]);
      }
    };
    // P and dS of group qt: lane holds key `key`, query rows i0 + 16 qt + 4 b16 + r.
    auto pds = [&](int qt) {
      const float4 l4 = st_lds[buf][0][4 * qt + b16];
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qrow = i0 + 16 * qt + 4 * b16 + r;
        const bool vis = qrow < N && key < N && (!CAUSAL || key <= qrow);
        const float e = exp2_hw(fmaf(s[qt][r], c, -lv[r]));
        const float p = MASKED ? (vis ? e : 0.f) : e;
        s[qt][r] = p;
        dp[qt][r] = p * dp[qt][r];
      }
    };
    // dV += P^T dO and dK += dS^T Q over the 32-row half u2: the A operand is
    // rows 32 u2 + 4 b16 + (0..3) and 32 u2 + 16 + 4 b16 + (0..3). The
    // transposed B fragments are read one 16-column step ahead (held in place
    // as the A fragments are).
    i16x4 tr[2][4];
    auto read_tr = [&](int u2, int tt) {
      const int ro = u2 * 32 * C::CPR * 16;
      tr[tt & 1][0] = lds_read_tr(db + troff[tt] + ro);
      tr[tt & 1][1] = lds_read_tr(db + troff[tt] + ro + 16 * C::CPR * 16);
      tr[tt & 1][2] = lds_read_tr(qb + troff[tt] + ro);
      tr[tt & 1][3] = lds_read_tr(qb + troff[tt] + ro + 16 * C::CPR * 16);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto dvdk = [&](int u2) {
      const bf16x8 pa = pack_bf16x8(s[2 * u2][0], s[2 * u2][1], s[2 * u2][2], s[2 * u2][3],
                                    s[2 * u2 + 1][0], s[2 * u2 + 1][1], s[2 * u2 + 1][2], s[2 * u2 + 1][3]);
      const bf16x8 sa = pack_bf16x8(dp[2 * u2][0], dp[2 * u2][1], dp[2 * u2][2], dp[2 * u2][3],
                                    dp[2 * u2 + 1][0], dp[2 * u2 + 1][1], dp[2 * u2 + 1][2], dp[2 * u2 + 1][3]);
      read_tr(u2, 0);
#pragma unroll
      for (int tt = 0; tt < C::TT; ++tt) {
        if (tt + 1 < C::TT) read_tr(u2, tt + 1);
        dv[tt] = mfma16(pa, join_bf16x8(tr[tt & 1][0], tr[tt & 1][1]), dv[tt]);
        dk[tt] = mfma16(sa, join_bf16x8(tr[tt & 1][2], tr[tt & 1][3]), dk[tt]);
      }
    };
    // The weights of groups 0 and 1 are computed while the products of groups
    // 2 and 3 run, those of groups 2 and 3 while the dV/dK products of rows
    // 0..31 run (each call's instructions are independent of the other's).
    read_a(0);
    read_a(1);
    sdp(0);
    read_a(2);
    sdp(1);
    read_a(3);
    sdp(2);
    pds(0);
    pds(1);
    sdp(3);
    dvdk(0);
    pds(2);
    pds(3);
    dvdk(1);
  };
  auto tile = [&](auto buf_c, int t) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < n_t) issue(gq_next, u_next, buf ^ 1);
    sync_check_group();
    const int i0 = u_cur * kBwdTile;
    u_cur = u_next;
    if (++u_next == n_u) {
      u_next = u_begin;
      ++gq_next;
    }
    if (j0 + kBwdKeyBlock > N || i0 + kBwdTile > N || (CAUSAL && i0 < j0 + kBwdKeyBlock))
      tile_body(buf_c, IC<1>{}, i0);
    else
      tile_body(buf_c, IC<0>{}, i0);
    sync_check_group();
  };
  int t = 0;
  for (; t + 1 < n_t; t += 2) {
    tile(IC<0>{}, t);
    tile(IC<1>{}, t + 1);
  }
  if (t < n_t) tile(IC<0>{}, t);

  // Epilogue: lane holds keys j0 + 16 wave + 4 b16 + r, column 16 tt + j16.
  const float sc = a.scale;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kr = j0 + 16 * wave + 4 * b16 + r;
    if (kr < N) {
      uint16_t* dkrow = a.dk + kv_base + (size_t)kr * D;
      uint16_t* dvrow = a.dv + kv_base + (size_t)kr * D;
#pragma unroll
      for (int tt = 0; tt < C::TT; ++tt) {
        dkrow[16 * tt + j16] = __builtin_bit_cast(uint16_t, (__bf16)(dk[tt][r] * sc));
        dvrow[16 * tt + j16] = __builtin_bit_cast(uint16_t, (__bf16)dv[tt][r]);
      }
    }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdArgs a, int nwg) {
  using C = BwdCfg<D>;
  __shared__ uint4 k_lds[2][C::TILE_CHUNKS];
  __shared__ uint4 v_lds[2][C::TILE_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int li = lane & 31;

  const int lid = xcd_contiguous(blockIdx.x, nwg);
  const int grp = lid / (a.hg_q * a.nqb);
  const int rem_g = lid - grp * a.hg_q * a.nqb;
  const int gh = min(a.hg_q, a.B * a.Hq - grp * a.hg_q);  // query heads in this group
  int qb = rem_g / gh;
  const int bh = grp * a.hg_q + (rem_g - qb * gh);
  if (CAUSAL) qb = a.nqb - 1 - qb;  // heaviest first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int N = a.N;
  const int q0 = qb * kBwdRowBlock;
  const int qi = q0 + 32 * wave + li;
  const size_t q_base = (size_t)(b * a.Hq + h) * (size_t)N * D;
  const uint16_t* kg = a.k + (size_t)(b * a.Hkv + hk) * (size_t)N * D;
  const uint16_t* vg = a.v + (size_t)(b * a.Hkv + hk) * (size_t)N * D;
  const int kv_end = CAUSAL ? min(N, q0 + kBwdRowBlock) : N;
  const int n_tiles = (kv_end + kBwdTile - 1) / kBwdTile;

  const TileOffsets<D, kSw2> koffs(wave, lane, N);  // K and V tiles alike
  load_tile_at<D, kSw2>(kg, 0, N, koffs, k_lds[0], wave);
  load_tile_at<D, kSw2>(vg, 0, N, koffs, v_lds[0], wave);

  // Q^T and dO^T as B operands (lane = query row qi), lse2 and -delta of qi.
  bf16x8 qf[C::KK32], df[C::KK32];
  {
    const size_t r = q_base + (size_t)(qi < N ? qi : 0) * D;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + r);
    const uint4* drow = reinterpret_cast<const uint4*>(a.dout + r);
#pragma unroll
    for (int kk = 0; kk < C::KK32; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8, qrow[2 * kk + g]);
      df[kk] = __builtin_bit_cast(bf16x8, drow[2 * kk + g]);
    }
  }
  const size_t st = (size_t)(b * a.Hq + h) * a.Npad + (qi < N ? qi : 0);
  const float lse2 = a.lse2[st];
  const float ndl_v = a.ndelta[st];

  // LDS offsets of the row reads: row li, chunk 2 kk + g. The V tiles take the
  // K tiles' swizzle (sw2, conflict-free for these reads too), so one set of
  // offsets serves both; the 16 registers this saves hold the fragments read
  // one k-step ahead.
  int koff[C::KK32];
#pragma unroll
  for (int kk = 0; kk < C::KK32; ++kk) koff[kk] = 16 * (li * C::CPR + ((2 * kk + g) ^ sw2<D>(li)));
  // K^T transposed reads (as the forward's V^T): lane t16 names row
  // 4 g + t16 / 4 (+ 32 jt + 16 hh, + 8 for the upper 4 keys) and 4 columns at
  // 32 dt + 16 vch + 4 (t16 % 4). sw2 of those rows depends on the +8 only.
  const int t16 = lane & 15;
  const int vch = (lane >> 4) & 1;
  const int vrow = 4 * g + (t16 >> 2);
  int klo[C::DT], khi[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int chunk = (32 * dt + 16 * vch + 4 * (t16 & 3)) >> 3;
    klo[dt] = 16 * (vrow * C::CPR + (chunk ^ sw2<D>(vrow))) + 8 * (t16 & 1);
    khi[dt] = 16 * ((vrow + 8) * C::CPR + (chunk ^ sw2<D>(vrow + 8))) + 8 * (t16 & 1);
  }

  f32x16 dq[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dq[dt] = f32x16{};
  const float c = a.c;

  // One key tile. MASKED for the tiles that hold keys past N or (causal) keys
  // above a row of the block: the tail of the sweep, from t_edge on (below,
  // the loop splits there so that the other tiles take no compare per weight,
  // a quarter of a tile's vector instructions; a branch inside the tile body
  // instead made the d = 128 kernel spill). Rows past N need no mask: their
  // dQ columns are never stored, and the products keep columns apart.
  auto tile = [&](int t, auto mask_c) {
    constexpr bool MASKED = decltype(mask_c)::value != 0;
    const int buf = t & 1;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < n_tiles) {
      load_tile_at<D, kSw2>(kg, (t + 1) * kBwdTile, N, koffs, k_lds[buf ^ 1], wave);
      load_tile_at<D, kSw2>(vg, (t + 1) * kBwdTile, N, koffs, v_lds[buf ^ 1], wave);
    }
    sync_check_group();
    const int kv0 = t * kBwdTile;
    const char* kb = reinterpret_cast<const char*>(k_lds[buf]);
    const char* vb = reinterpret_cast<const char*>(v_lds[buf]);

    // S^T = K Q^T and dP^T = V dO^T for two 32-key halves, the K and V
    // fragments of k-step kk + 1 read while the products of step kk run
    // (alternating register sets; a scheduling barrier keeps each step's reads
    // in place, the waits stay at the first use).
    // Every register of dP^T holds row qi: the products start from a tile of
    // -delta and leave dP^T - delta. At d = 128 the tile is rebuilt per key
    // tile (held over the sweep, its 16 registers made the kernel spill).
    f32x16 ndl;
    {
      float v = ndl_v;
      if constexpr (D == 128) asm volatile("" : "+v"(v));
#pragma unroll
      for (int r = 0; r < 16; ++r) ndl[r] = v;
    }
    f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = ndl, p1 = ndl;
    bf16x8 fk[2][2], fv[2][2];
    auto read_kv = [&](int kk) {
      fk[kk & 1][0] = *reinterpret_cast<const bf16x8*>(kb + koff[kk]);
      fk[kk & 1][1] = *reinterpret_cast<const bf16x8*>(kb + koff[kk] + 32 * C::CPR * 16);
      fv[kk & 1][0] = *reinterpret_cast<const bf16x8*>(vb + koff[kk]);
      fv[kk & 1][1] = *reinterpret_cast<const bf16x8*>(vb + koff[kk] + 32 * C::CPR * 16);
      __builtin_amdgcn_sched_barrier(0);
    };
    read_kv(0);
#pragma unroll
    for (int kk = 0; kk < C::KK32; ++kk) {
      if (kk + 1 < C::KK32) read_kv(kk + 1);
      s0 = mfma32(fk[kk & 1][0], qf[kk], s0);
      s1 = mfma32(fk[kk & 1][1], qf[kk], s1);
      p0 = mfma32(fv[kk & 1][0], df[kk], p0);
      p1 = mfma32(fv[kk & 1][1], df[kk], p1);
    }
    // dS^T = P^T (dP^T - delta); lane holds keys kv0 + 32 jt + 8 (r / 4) + 4 g + r % 4.
    // Key kv0 + 4 g + o (o a compile-time offset) is visible to row qi iff
    // o <= lim: one compare per weight (rows past N get lim = -1).
    const int lim = (qi < N ? min(N - 1, CAUSAL ? qi : N - 1) : -1) - kv0 - 4 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 8 * (r >> 2) + (r & 3);
      const float ea = exp2_hw(fmaf(s0[r], c, -lse2));
      const float eb = exp2_hw(fmaf(s1[r], c, -lse2));
      const float pa = MASKED ? (o <= lim ? ea : 0.f) : ea;
      const float pb = MASKED ? (o + 32 <= lim ? eb : 0.f) : eb;
      s0[r] = pa * p0[r];
      s1[r] = pb * p1[r];
    }
    bf16x8 sb[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sb[0][hh] = pack_bf16x8(s0[8 * hh + 0], s0[8 * hh + 1], s0[8 * hh + 2], s0[8 * hh + 3],
                              s0[8 * hh + 4], s0[8 * hh + 5], s0[8 * hh + 6], s0[8 * hh + 7]);
      sb[1][hh] = pack_bf16x8(s1[8 * hh + 0], s1[8 * hh + 1], s1[8 * hh + 2], s1[8 * hh + 3],
                              s1[8 * hh + 4], s1[8 * hh + 5], s1[8 * hh + 6], s1[8 * hh + 7]);
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ro = (32 * jt + 16 * hh) * C::CPR * 16;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const i16x4 lo = lds_read_tr(kb + klo[dt] + ro);
          const i16x4 hi = lds_read_tr(kb + khi[dt] + ro);
          dq[dt] = mfma32(join_bf16x8(lo, hi), sb[jt][hh], dq[dt]);
        }
      }
    sync_check_group();
  };
  // Tiles below t_edge hold only keys below N and (causal) below the block's
  // first row q0 (a multiple of the tile), so every key is visible to every row.
  const int t_edge = CAUSAL ? min(q0, N) / kBwdTile : N / kBwdTile;
  int t = 0;
  for (; t < t_edge && t < n_tiles; ++t) tile(t, IC<0>{});
  for (; t < n_tiles; ++t) tile(t, IC<1>{});

  // Epilogue: lane holds row qi, columns 32 dt + 8 rq + 4 g + (0..3).
  if (qi < N) {
    uint16_t* row = a.dq + q_base + (size_t)qi * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<uint2*>(row + 32 * dt + 8 * rq + 4 * g) =
            pack_bf16x4(dq[dt][4 * rq + 0] * sc, dq[dt][4 * rq + 1] * sc, dq[dt][4 * rq + 2] * sc,
                        dq[dt][4 * rq + 3] * sc);
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.Hq * a.Npad;
  const size_t per_wg = 256 / (D / 8);
  hipLaunchKernelGGL(fa_bwd_rows_kernel<D>, dim3((unsigned)((rows + per_wg - 1) / per_wg)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nwg_kv = a.B * a.Hkv * a.nkb;
  const int nwg_q = a.B * a.Hq * a.nqb;
  if (causal) {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true>), dim3(nwg_kv), dim3(256), 0, stream, a, nwg_kv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true>), dim3(nwg_q), dim3(256), 0, stream, a, nwg_q);
  } else {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false>), dim3(nwg_kv), dim3(256), 0, stream, a, nwg_kv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false>), dim3(nwg_q), dim3(256), 0, stream, a, nwg_q);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  return d == 128 ? launch_bwd_d<128>(a, causal, stream) : launch_bwd_d<64>(a, causal, stream);
}

}  // namespace fa
