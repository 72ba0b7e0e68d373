// Split-KV decode attention and the log-sum-exp combine for gfx950.
//
// Decode is one query token per (sequence, query head) against a KV cache:
// bandwidth-bound, since each K/V byte feeds only the query heads of its GQA
// group ("FlashAttention HBM bytes, one head, 8K", "What interviewers probe
// next"); to keep the GPU busy the key sequence is split across work-groups
// ("Why is standard attention memory-bound...", "Does FlashAttention help when
// generating one token at a time?"). Each work-group owns one (sequence, KV
// head, head group, chunk) and reads that chunk of K and V exactly once for
// all query heads of the group; a second kernel merges the chunks with the
// log-sum-exp combine, which is the online-softmax merge step ("Flash Attention
// Mechanics", "The Tiling Algorithm") applied to whole chunks.
//
// Mapping onto CDNA4:
//   * 4 waves; per step each wave takes 32 keys of the chunk (a step is 128).
//   * Scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16: K is loaded straight
//     from HBM into the A-operand layout (16 keys x 64 contiguous bytes per
//     instruction); Q^T of up to 16 grouped heads is the B operand, kept in
//     registers. Lane l then holds head l%16 at 4 keys per 16-key tile.
//   * Online softmax per head in base 2, reduced over the 4 lanes of a head.
//   * K and V are read once; V (whole 128-byte lines per load) with the
//     non-temporal hint, K (half lines per load) without it.
//   * P V on the vector ALUs: V is loaded with fully coalesced 16-byte reads
//     (one row per 16 lanes at d = 128), each lane keeps FP32 partial outputs
//     for its 8 columns and every head of the group; the weights p[key][head]
//     pass through a small per-wave LDS buffer.
//   * At the end the 4 waves' (m, l, O) are merged in LDS and the chunk's
//     normalised O_c (FP32) and lse_c are written to the workspace.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += shfl_xor(x, m);
  return x;
}

// Log-sum-exp merge of S normalised partial results of one row, by one wave:
// M = max_s lse_s, w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s,
// lse = M + ln sum_s w_s. Partial s of the row is o_part[s * D ..]; its lse is
// lse_part[s]. Lanes load the lse values in parallel (with up to 16 partials,
// together with all partial rows); the weights are then broadcast with
// readlane while each lane accumulates D / 64 columns.
template <int D>
__device__ __forceinline__ void combine_row(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                            int S, uint16_t* __restrict__ o_row, float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  const int lane = __lane_id();
  if (S <= 16) {
    // One round trip: the partial rows do not depend on the lse values, so
    // their loads go out with them.
    const float l = lane < S ? lse_part[lane] : -INFINITY;
    float v[16][PER];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int j = 0; j < PER; ++j) v[u][j] = u < S ? o_part[(size_t)u * D + lane * PER + j] : 0.f;
    const float M = wave_max(l);
    const float Ms = M == -INFINITY ? 0.f : M;
    const float wl = lane < S ? exp2_hw((l - Ms) * kLog2e) : 0.f;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, v[u][j], acc[j]);
    }
    const float wsum = wave_sum(wl);
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) o_row[lane * PER + j] = __builtin_bit_cast(uint16_t, (__bf16)(acc[j] * inv));
    if (lane == 0) *lse_out = wsum > 0.f ? M + log2_hw(wsum) * kLn2 : -INFINITY;
    return;
  }
  float M = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 64) M = fmaxf(M, s0 + lane < S ? lse_part[s0 + lane] : -INFINITY);
  M = wave_max(M);
  const float Ms = M == -INFINITY ? 0.f : M;
  float wsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int cnt = min(64, S - s0);
    const float wl = lane < cnt ? exp2_hw((lse_part[s0 + lane] - Ms) * kLog2e) : 0.f;
    wsum += wl;
    int s = 0;
    for (; s + 4 <= cnt; s += 4) {
      float v[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < PER; ++j) v[u][j] = o_part[(size_t)(s0 + s + u) * D + lane * PER + j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s + u));
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, v[u][j], acc[j]);
      }
    }
    for (; s < cnt; ++s) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] = fmaf(w, o_part[(size_t)(s0 + s) * D + lane * PER + j], acc[j]);
    }
  }
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const __bf16 bv = (__bf16)(acc[j] * inv);
    o_row[lane * PER + j] = __builtin_bit_cast(uint16_t, bv);
  }
  if (lane == 0) *lse_out = wsum > 0.f ? M + log2_hw(wsum) * kLn2 : -INFINITY;
}

constexpr int kDecWaveKeys = 32;
constexpr int kDecRankedSeqs = kDecThreads;  // varlen batches ranked by length in the grid order
constexpr int kDecStepKeys = 4 * kDecWaveKeys;

template <int D>
struct DecCfg {
  static constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  static constexpr int RPI = 64 / CPR;       // rows covered by one wave-wide 16-byte load
  static constexpr int NV = kDecWaveKeys / RPI;  // V loads per lane per step
  static constexpr int KK = D / 32;          // k-steps of the 16x16x32 MFMA
};

// Up to 4 query heads per group the kernel fits 128 VGPRs: four work-groups
// per CU, so the workload's 2048 work-groups run in exactly two rounds.
template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(GM <= 4 ? 4 : 2)))
void fa_decode_split_kernel(DecArgs a) {
  using C = DecCfg<D>;
  __shared__ float p_lds[4][kDecWaveKeys][GM];
  __shared__ float alpha_lds[4][GM];
  __shared__ float wm_lds[4][GM];
  __shared__ float wl_lds[4][GM];
  __shared__ float wo_lds[4][GM][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Grid order. All caches of one length: chunk index slowest, so consecutive
  // work-groups (dealt round-robin to the 8 XCDs) take the same chunk of
  // different sequences and heads. Caches of their own lengths (up to
  // kDecRankedSeqs sequences): sequences longest first, each with all its
  // chunks and heads, so the longest chunks start first and the short ones
  // fill in behind them; every work-group ranks the lengths itself.
  int rest = blockIdx.x;
  const int hg = rest % a.n_hg; rest /= a.n_hg;
  const int hk = rest % a.Hkv; rest /= a.Hkv;
  int b, split;
  if (a.lens && a.B <= kDecRankedSeqs) {
    __shared__ int by_rank[kDecRankedSeqs];
    if (tid < a.B) {
      const int mine = min(max(a.lens[tid], 0), a.L);
      int r = 0;
      for (int j = 0; j < a.B; ++j) {
        const int lj = min(max(a.lens[j], 0), a.L);
        r += (lj > mine) || (lj == mine && j < tid);
      }
      by_rank[r] = tid;
    }
    __syncthreads();
    split = rest % a.S;
    b = by_rank[rest / a.S];
  } else {
    b = rest % a.B;
    split = rest / a.B;
  }
  // Keys of this sequence and its chunk: with per-sequence lengths the S
  // chunks cut each sequence's own keys, so the work follows the lengths, in
  // chunks of at least one step (a short sequence then takes fewer than S
  // chunks, and its other work-groups write empty partials: 7% faster on
  // lengths 1..1024, larger minimums cut the parallelism of mid-length ones).
  const int len = a.lens ? min(max(a.lens[b], 0), a.L) : a.L;
  const int chunk = a.lens ? max((len + a.S - 1) / a.S, kDecStepKeys) : a.chunk;
  const int key_begin = split * chunk;
  const int key_end = min(len, key_begin + chunk);  // an empty chunk writes O_c = 0, lse_c = -inf
  const int h_first = hk * a.G + hg * GM;
  const int gv = min(GM, a.G - hg * GM);  // valid heads in this work-group
  const float c = a.c;
  const size_t kv_base = (size_t)(b * a.Hkv + hk) * (size_t)a.L * D;

  // Q^T operand: lane l holds head n = l%16 (zero if n >= gv), dims 32 kk + 8 (l/16) + e.
  const int n = lane & 15;
  const int quad = lane >> 4;
  bf16x8 qf[C::KK];
  {
    const bool ok = n < gv;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + (size_t)(b * a.Hq + h_first + (ok ? n : 0)) * D);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const uint4 w = ok ? qrow[4 * kk + quad] : make_uint4(0u, 0u, 0u, 0u);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // PV ownership: lane holds columns 8 cl .. 8 cl + 7 of rows l / CPR + RPI x.
  const int cl = lane % C::CPR;
  const int rl = lane / C::CPR;

  float m_run = -INFINITY;  // per head n (same in the 4 lanes of that head)
  float l_run = 0.f;        // partial over this lane's keys
  float o[GM][8];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;

  for (int kb = key_begin; kb < key_end; kb += kDecStepKeys) {
    const int kw = kb + wave * kDecWaveKeys;
    // ---- loads: K in MFMA A layout, V coalesced. Rows past the chunk read the
    // chunk's last key instead (finite data): their scores become -inf, p = 0.
    // K takes plain loads: a K load fetches 64 bytes of each of 16 rows, the
    // other half of each 128-byte line comes with the next k-step's load, and
    // with the non-temporal hint that second half missed again (streaming the
    // decode's loads alone: 6.3 TB/s with the hint on K, 7.4 without). V loads
    // take whole lines and keep the hint.
    bf16x8 kf[2][C::KK];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int key = min(kw + tt * 16 + n, key_end - 1);
      const uint4* krow = reinterpret_cast<const uint4*>(a.k + kv_base + (size_t)key * D);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) kf[tt][kk] = __builtin_bit_cast(bf16x8, krow[4 * kk + quad]);
    }
    uint4 vr[C::NV];
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int key = min(kw + rl + C::RPI * x, key_end - 1);
      vr[x] = load_nt(a.v + kv_base + (size_t)key * D + cl * 8);
    }

    // ---- S^T tiles: lane holds head n, keys kw + 16 tt + 4 quad + r
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) s[tt] = mfma16(kf[tt][kk], qf[kk], s[tt]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kw + 16 * tt + 4 * quad + r;
        const float tv = key < key_end ? s[tt][r] * c : -INFINITY;
        s[tt][r] = tv;
        tmax = fmaxf(tmax, tv);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = max_xor32(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2_hw(s[tt][r] - m_use);
        rs += p;
        if (n < GM) p_lds[wave][16 * tt + 4 * quad + r][n] = p;
      }
    l_run = fmaf(l_run, alpha, rs);
    if (lane < GM) alpha_lds[wave][lane] = alpha;
    wave_sync_lds();
    sync_check_wave();

    // ---- O = alpha O + P V on the vector ALUs
    float al[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) al[hh] = alpha_lds[wave][hh];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= al[hh];
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int kl = rl + C::RPI * x;
      float pv[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) pv[hh] = p_lds[wave][kl][hh];
      const uint4 w = vr[x];
      const float vv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pv[hh], vv[e], o[hh][e]);
    }
    wave_sync_lds();
    sync_check_wave();
  }

  // ---- per-wave totals: l over the 4 lanes of a head; O over the lanes sharing columns
  float l_head = l_run + shfl_xor(l_run, 16);
  l_head = sum_xor32(l_head);
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[hh][e];
#pragma unroll
      for (int msk = C::CPR; msk < 64; msk <<= 1) x += shfl_xor(x, msk);
      o[hh][e] = x;
    }
  if (lane < GM) {
    wm_lds[wave][lane] = m_run;
    wl_lds[wave][lane] = l_head;
  }
  if (rl == 0) {
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) wo_lds[wave][hh][8 * cl + e] = o[hh][e];
  }
  __syncthreads();

  // ---- merge the 4 waves and write the chunk's normalised partial result
  for (int idx = tid; idx < gv * D; idx += kDecThreads) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm_lds[w][hh]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2_hw(wm_lds[w][hh] - Ms);
      lsum = fmaf(wt, wl_lds[w][hh], lsum);
      acc = fmaf(wt, wo_lds[w][hh][d], acc);
    }
    const size_t row = (size_t)(b * a.Hq + h_first + hh);
    a.o_part[(row * a.S + split) * D + d] = lsum > 0.f ? acc / lsum : 0.f;
    if (d == 0) a.lse_part[row * a.S + split] = lsum > 0.f ? (M + log2_hw(lsum)) * kLn2 : -INFINITY;
  }
}

// One wave per (sequence, query head): merge the chunks' partial results.
template <int D>
__global__ __launch_bounds__(64) void fa_combine_kernel(const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        uint16_t* __restrict__ o, float* __restrict__ lse,
                                                        int S) {
  const size_t row = blockIdx.x;
  combine_row<D>(o_part + row * S * D, lse_part + row * S, S, o + row * D, lse + row);
}

template <int D, int GM>
static hipError_t launch_split_t(const DecArgs& a, hipStream_t stream) {
  const unsigned nwg = (unsigned)a.B * a.Hkv * a.n_hg * a.S;
  hipLaunchKernelGGL((fa_decode_split_kernel<D, GM>), dim3(nwg), dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_split_d(const DecArgs& a, int gm, hipStream_t stream) {
  switch (gm) {
    case 1: return launch_split_t<D, 1>(a, stream);
    case 2: return launch_split_t<D, 2>(a, stream);
    case 4: return launch_split_t<D, 4>(a, stream);
    case 8: return launch_split_t<D, 8>(a, stream);
    default: return launch_split_t<D, 16>(a, stream);
  }
}

hipError_t launch_decode_split(const DecArgs& a, int d, int heads_per_group, hipStream_t stream) {
  return d == 128 ? launch_split_d<128>(a, heads_per_group, stream) : launch_split_d<64>(a, heads_per_group, stream);
}

hipError_t launch_combine(const float* o_part, const float* lse_part, uint16_t* o, float* lse,
                          int rows, int S, int d, hipStream_t stream) {
  if (d == 128)
    hipLaunchKernelGGL((fa_combine_kernel<128>), dim3(rows), dim3(64), 0, stream, o_part, lse_part, o, lse, S);
  else
    hipLaunchKernelGGL((fa_combine_kernel<64>), dim3(rows), dim3(64), 0, stream, o_part, lse_part, o, lse, S);
  return hipGetLastError();
}

}  // namespace fa
