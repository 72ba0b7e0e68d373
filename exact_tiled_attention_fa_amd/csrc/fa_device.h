// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers, LDS transpose reads, cross-lane exchanges and BF16 packing.
//
// Register layouts (CDNA4 MFMA, wave64; lane l, element/register index e/r):
//   v_mfma_f32_32x32x16_bf16  D[32x32] = A[32x16] B[16x32] + C
//     A: lane l holds A[l%32][8*(l/32) + e], e = 0..7
//     B: lane l holds B[8*(l/32) + e][l%32]
//     C: lane l reg r holds C[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15
//   v_mfma_f32_16x16x32_bf16  D[16x16] = A[16x32] B[32x16] + C
//     A: lane l holds A[l%16][8*(l/16) + e]
//     B: lane l holds B[8*(l/16) + e][l%16]
//     C: lane l reg r holds C[4*(l/16) + r][l%16], r = 0..3
// Only the pairing of A's and B's k-slots matters for a contraction, so the
// kernels are free to choose which k index lives in which slot, as long as A
// and B agree.
//
//   ds_read_b64_tr_b16: within each block of 16 lanes, lane t names an 8-byte
//   run of 4 b16 values; lane i receives element (i%4) of the runs named by
//   lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4. With lane t pointing at row t/4,
//   columns 4*(t%4)..+3 of a row-major b16 matrix, lane i gets column i of
//   those 4 rows: a transposed 4x16 read.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// LDS writes of some lanes of a wave made visible to reads by other lanes of
// the same wave.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Race-check build (compiled with -DFA_SYNC_CHECK=1): every phase of a kernel
// that hands data through LDS, or fills LDS with direct loads, is closed by a
// wait for all of the wave's outstanding memory operations (s_waitcnt 0) and,
// where the whole work-group runs the phase, a work-group barrier; the
// forward kernels also issue every direct load at the start of its step. The
// arithmetic and its order do not change, so the race-check library must
// reproduce the normal one bit for bit: a difference means that some read
// met data that was not yet, or no longer, there.
#ifndef FA_SYNC_CHECK
#define FA_SYNC_CHECK 0
#endif
constexpr bool kSyncCheck = FA_SYNC_CHECK != 0;

// Wave-level form: allowed anywhere, also in code the waves of a work-group
// run a different number of times.
__device__ __forceinline__ void sync_check_wave() {
  if constexpr (kSyncCheck) {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
}

// Work-group form: only where every wave of the work-group passes the same
// number of times (beside the kernels' own __syncthreads()).
__device__ __forceinline__ void sync_check_group() {
  if constexpr (kSyncCheck) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// 16-byte global load with the non-temporal hint: for data read exactly once
// (a KV cache in decode), so it does not displace reusable lines in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// IEEE 754-2019 maximum (NaN-propagating). Unlike fmaxf it needs no quieting
// of its operands, and chains max(max(a, b), c) become one v_maximum3_f32.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Value of x in the lane 32 away (l ^ 32), combined with the own value.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x from lane l ^ mask (any mask < 64), through the LDS crossbar.
__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Round-to-nearest-even FP32 -> BF16 of 8 values (v_cvt_pk_bf16_f32 pairs).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Transposed 4x16 read of b16 values from LDS (see the header comment).
__device__ __forceinline__ i16x4 lds_read_tr(const void* lds_byte_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte_ptr));
}

__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 lo, i16x4 hi) {
  i16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four floats to four BF16 (nearest even), packed little-end first.
// Built as a vector so that each pair becomes one v_cvt_pk_bf16_f32 (assembled
// from 16-bit halves, the compiler converted one value per instruction and
// shifted and merged the halves).
__device__ __forceinline__ uint2 pack_bf16x4(float a0, float a1, float a2, float a3) {
  bf16x4 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  return __builtin_bit_cast(uint2, r);
}

// Log-sum-exp merge of one row's S key-split partials (BF16 normalised
// outputs O_s and FP32 lse_s, natural log) for eight columns: M = max_s lse_s,
// w_s = e^(lse_s - M), O = sum_s w_s O_s / sum_s w_s and lse = M + ln sum_s w_s.
// op points at column col of partial 0 (partials D values apart, col a
// multiple of 8, so each partial is one 16-byte load), lp at the row's S lse
// values. With S <= 16 all loads go out together (the partials do not depend
// on the lse values); otherwise eight partials at a time after a first pass
// for M. O goes to o8 (eight BF16, nearest even); lse is written when
// write_lse.
template <int D>
__device__ __forceinline__ void merge_splits8(const uint16_t* __restrict__ op, const float* __restrict__ lp, int S,
                                              uint16_t* __restrict__ o8, float* __restrict__ lse_out,
                                              bool write_lse) {
  auto part = [&](int s, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(op + (size_t)s * D);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  float M = -INFINITY;
  if (S <= 8) {
    float l[8];
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = u < S;
      l[u] = in ? lp[u] : -INFINITY;
      if (in) {
        part(u, v[u]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[u][c] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, l[u]);
    const float Ms = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = u < S ? exp2_hw((l[u] - Ms) * kLog2e) : 0.f;
      wsum += w;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(w, v[u][c], acc[c]);
    }
  } else if (S <= 16) {
    // Every load in one round trip: partial u reads partial min(u, S - 1)
    // (no branch per load) and the copies past S - 1 get weight 0.
    float l[16];
    uint4 w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int su = u < S ? u : S - 1;
      l[u] = lp[su];
      w[u] = *reinterpret_cast<const uint4*>(op + (size_t)su * D);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) M = fmaxf(M, l[u]);
    const float Ms = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wt = u < S ? exp2_hw((l[u] - Ms) * kLog2e) : 0.f;
      wsum += wt;
      const float v[8] = {bf16_lo(w[u].x), bf16_hi(w[u].x), bf16_lo(w[u].y), bf16_hi(w[u].y),
                          bf16_lo(w[u].z), bf16_hi(w[u].z), bf16_lo(w[u].w), bf16_hi(w[u].w)};
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(wt, v[c], acc[c]);
    }
  } else {
    for (int s0 = 0; s0 < S; s0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, s0 + u < S ? lp[s0 + u] : -INFINITY);
    }
    const float Ms = M == -INFINITY ? 0.f : M;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float v[8][8];
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = s0 + u < S;
        if (in) {
          part(s0 + u, v[u]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) v[u][c] = 0.f;
        }
        w[u] = in ? exp2_hw((lp[s0 + u] - Ms) * kLog2e) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        wsum += w[u];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(w[u], v[u][c], acc[c]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const uint2 lo = pack_bf16x4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  const uint2 hi = pack_bf16x4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(o8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  if (write_lse) *lse_out = wsum > 0.f ? M + log2_hw(wsum) * kLn2 : -INFINITY;
}

// Threads per work-group of the forward merge kernel (D / 8 lanes per row).
constexpr int kMergeThreads = 256;

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// fills bytes 16 l .. 16 l + 15 of the 1 KiB block whose LDS address goes in
// M0; the global address is the uniform base plus the lane's 32-bit offset.
// Issued through inline assembly so that the compiler's wait-count pass, which
// cannot tell which LDS buffer a direct load writes, does not make LDS reads of
// the other buffer wait for it; the kernel waits for its loads itself
// (s_waitcnt vmcnt(0)) before the barrier that hands a buffer to its readers.
// M0 is saved and restored around it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

template <int V>
using IC = std::integral_constant<int, V>;

// Work-group id -> logical id such that each XCD (work-groups are handed to
// the 8 XCDs round-robin) receives one contiguous range of logical ids.
__device__ __forceinline__ int xcd_contiguous(int wg, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int x = wg & 7, k = wg >> 3;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace fa
