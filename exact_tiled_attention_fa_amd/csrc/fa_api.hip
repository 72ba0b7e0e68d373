// C ABI of libfa: argument checks (host only, before any HIP call), launch
// configuration and dispatch to the kernel translation units.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Elements of a [B, H, N, d] tensor, or -1 if it does not fit in int64.
int64_t elems(int64_t B, int64_t H, int64_t N, int64_t d) {
  const int64_t lim = INT64_MAX / 4;
  int64_t x = B;
  for (int64_t f : {H, N, d}) {
    if (f != 0 && x > lim / f) return -1;
    x *= f;
  }
  return x;
}

// Longest sequence (N or L) accepted: keeps every in-head index expression of
// the kernels and planners (a row or key plus one block, L + num_splits - 1)
// inside int. One head's Q at that length and d = 64 is already 128 GiB.
constexpr int kMaxSeq = 1 << 30;

int decode_chunk(int L, int num_splits) { return (L + num_splits - 1) / num_splits; }
int decode_splits_used(int L, int num_splits) {
  const int chunk = decode_chunk(L, num_splits);
  return (L + chunk - 1) / chunk;
}

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int next_pow2_le16(int g) {
  int p = 1;
  while (p < g && p < 16) p <<= 1;
  return p;
}

}  // namespace

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is out of range";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: d must be 64 or 128";
    case FA_ERR_GQA: return "FA_ERR_GQA: Hq must be a multiple of Hkv";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensors must be 16-byte aligned (lse 4-byte)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: a HIP launch failed";
    case FA_ERR_ARG: return "FA_ERR_ARG: causal must be 0 or 1 and the scales finite";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the key-split partials of these sizes exceed fa_fwd_noalloc's static scratch "
             "(fa_fwd_noalloc_max_scratch_bytes())";
    default: return "unknown fa_status";
  }
}

namespace {

// Checks shared by the forward entry points; FA_OK or the failing status.
int check_fwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ALIGN;
  return FA_OK;
}

// Sizes only: FA_OK or FA_ERR_SHAPE. The work-group count (also after a key
// split, which targets at most two per CU beyond it) and the combine's
// one-wave-per-row grid must fit a launch.
int check_fwd_sizes(int B, int Hq, int N, int d) {
  if (B <= 0 || Hq <= 0 || N <= 0 || N > kMaxSeq || (d != 64 && d != 128)) return FA_ERR_SHAPE;
  if (elems(B, Hq, N, d) < 0) return FA_ERR_SHAPE;
  const int64_t nqb = (N + fa::kFwdWaveRows * 4 - 1) / (fa::kFwdWaveRows * 4);  // the smaller blocks
  if ((int64_t)B * Hq * nqb > INT32_MAX / 4 || (int64_t)B * Hq * N > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

using fa::FwdPlan;

FwdPlan plan_fwd(int B, int Hq, int N, int d, bool causal, bool fp8) {
  return fa::plan_fwd(B, Hq, N, d, causal, fp8, device_cu_count());
}

int launch_fwd_planned(const FwdPlan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* ws,
                       hipStream_t s, hipEvent_t after_attention = nullptr) {
  fa::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N;
  a.c = scale * fa::kLog2eHost;
  a.rows = p.rows;
  a.nqb = p.nqb;
  a.nwg = (int)p.nwg;
  a.n_splits = p.n_splits;
  a.split_tiles = p.split_tiles;
  a.head_group = p.head_group;
  a.split_target = p.split_target;
  a.per_head = p.per_head;
  a.o_part = static_cast<uint16_t*>(ws);
  a.lse_part = ws ? reinterpret_cast<float*>(a.o_part + (size_t)B * Hq * N * p.n_splits * d) : nullptr;
  a.v_scale = 1.f;
  hipError_t e = fa::launch_fwd(a, d, causal != 0, s);
  if (e == hipSuccess && after_attention) e = hipEventRecord(after_attention, s);
  if (e == hipSuccess && p.n_splits > 1) e = fa::launch_fwd_combine(a, d, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fwd_ws_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
                int d, int causal, float scale, void* workspace, size_t workspace_bytes, hipStream_t s,
                hipEvent_t after_attention) {
  int st = check_fwd_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  if ((st = check_fwd_sizes(B, Hq, N, d)) != FA_OK) return st;
  const FwdPlan p = plan_fwd(B, Hq, N, d, causal != 0, false);
  if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  return launch_fwd_planned(p, q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale,
                            p.ws_bytes > 0 ? workspace : nullptr, s, after_attention);
}

}  // namespace

extern "C" size_t fa_fwd_workspace_bytes(int B, int Hq, int N, int d) {
  if (check_fwd_sizes(B, Hq, N, d) != FA_OK) return 0;
  // Enough for either mask and either input type (the plan depends on both).
  size_t most = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (int fp8 = 0; fp8 < 2; ++fp8) {
      const size_t b = plan_fwd(B, Hq, N, d, causal != 0, fp8 != 0).ws_bytes;
      if (b > most) most = b;
    }
  return most;
}

extern "C" int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  return fwd_ws_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, workspace, workspace_bytes,
                     reinterpret_cast<hipStream_t>(stream), nullptr);
}

extern "C" int fa_fwd_ws_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                               void* workspace, size_t workspace_bytes, fa_stream_t stream,
                               fa_event_t after_attention) {
  if (!after_attention) return FA_ERR_NULL;
  return fwd_ws_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, workspace, workspace_bytes,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(after_attention));
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      fa_stream_t stream) {
  int st = check_fwd_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  if ((st = check_fwd_sizes(B, Hq, N, d)) != FA_OK) return st;
  const FwdPlan p = plan_fwd(B, Hq, N, d, causal != 0, false);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.ws_bytes == 0) return launch_fwd_planned(p, q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, nullptr, s);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, p.ws_bytes, s) != hipSuccess || !ws) return FA_ERR_LAUNCH;
  st = launch_fwd_planned(p, q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, ws, s);
  const hipError_t ef = hipFreeAsync(ws, s);
  return (st == FA_OK && ef == hipSuccess) ? FA_OK : (st != FA_OK ? st : FA_ERR_LAUNCH);
}

// ---- fa_fwd_noalloc: the key-split partials live in a static device array.
namespace {

// Largest key-split partial buffer that plan_fwd makes on a 256-CU part is
// 32.4 MiB (one head of 65,280 keys at d = 128, two splits of 256-row blocks);
// the array covers it with room to spare.
constexpr size_t kScratchBytes = (size_t)34 << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, kept until the process ends. In host code this name is a
// host-side stand-in, not a device address: host code uses only the address
// hipGetSymbolAddress returns for the current device (scratch_on_device).
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call for that device (null if the lookup fails).
void* scratch_on_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t fa_fwd_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

extern "C" int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              fa_stream_t stream) {
  int st = check_fwd_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  if ((st = check_fwd_sizes(B, Hq, N, d)) != FA_OK) return st;
  const FwdPlan p = plan_fwd(B, Hq, N, d, causal != 0, false);
  if (p.ws_bytes > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (p.ws_bytes > 0 && !(ws = scratch_on_device())) return FA_ERR_LAUNCH;
  // Every non-empty split writes all of its partial rows before the combine
  // reads them, and the combine reads no other split, so the array needs no
  // clearing between calls.
  return launch_fwd_planned(p, q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, ws,
                            reinterpret_cast<hipStream_t>(stream));
}

namespace {

int check_fp8_args(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale,
                   void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
  int st = check_fwd_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  if (!isfinite(q_scale) || !isfinite(k_scale) || !isfinite(v_scale) ||
      !isfinite((double)scale * q_scale * k_scale * fa::kLog2eHost) ||
      !isfinite((float)((double)scale * q_scale * k_scale * fa::kLog2eHost)))
    return FA_ERR_ARG;
  return check_fwd_sizes(B, Hq, N, d);
}

int launch_fwd_fp8_planned(const FwdPlan& p, const void* q, const void* k, const void* v, float q_scale,
                           float k_scale, float v_scale, void* o, float* lse, int B, int Hq, int Hkv, int N,
                           int d, int causal, float scale, void* ws, hipStream_t s) {
  fa::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);  // E4M3 bytes; the kernel reads them as such
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N;
  a.c = (float)((double)scale * q_scale * k_scale * fa::kLog2eHost);
  a.rows = p.rows;
  a.nqb = p.nqb;
  a.nwg = (int)p.nwg;
  a.n_splits = p.n_splits;
  a.split_tiles = p.split_tiles;
  a.head_group = p.head_group;
  a.split_target = 0;  // the FP8 kernel takes uniform splits only
  a.per_head = 0;
  a.o_part = static_cast<uint16_t*>(ws);
  a.lse_part = ws ? reinterpret_cast<float*>(a.o_part + (size_t)B * Hq * N * p.n_splits * d) : nullptr;
  a.v_scale = v_scale;
  hipError_t e = fa::launch_fwd_fp8(a, d, causal != 0, s);
  if (e == hipSuccess && p.n_splits > 1) e = fa::launch_fwd_combine(a, d, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa_fwd_fp8_ws(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                             float v_scale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                             int causal, float scale, void* workspace, size_t workspace_bytes,
                             fa_stream_t stream) {
  const int st = check_fp8_args(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  const FwdPlan p = plan_fwd(B, Hq, N, d, causal != 0, true);
  if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  return launch_fwd_fp8_planned(p, q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale,
                                p.ws_bytes > 0 ? workspace : nullptr, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                          float v_scale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, fa_stream_t stream) {
  int st = check_fp8_args(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  const FwdPlan p = plan_fwd(B, Hq, N, d, causal != 0, true);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.ws_bytes == 0)
    return launch_fwd_fp8_planned(p, q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale,
                                  nullptr, s);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, p.ws_bytes, s) != hipSuccess || !ws) return FA_ERR_LAUNCH;
  st = launch_fwd_fp8_planned(p, q, k, v, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, N, d, causal, scale, ws, s);
  const hipError_t ef = hipFreeAsync(ws, s);
  return (st == FA_OK && ef == hipSuccess) ? FA_OK : (st != FA_OK ? st : FA_ERR_LAUNCH);
}

namespace {

int64_t bwd_npad(int N) { return ((int64_t)N + fa::kBwdTile - 1) / fa::kBwdTile * fa::kBwdTile; }

}  // namespace

extern "C" size_t fa_bwd_workspace_bytes(int B, int Hq, int N, int d) {
  if (check_fwd_sizes(B, Hq, N, d) != FA_OK) return 0;
  const size_t bytes = (size_t)2 * B * Hq * (size_t)bwd_npad(N) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                      int causal, float scale, void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  if (!o || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_fwd_args(q, k, v, dq, lse, B, Hq, Hkv, N, d, causal, scale);
  if (st != FA_OK) return st;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return FA_ERR_ALIGN;
  if ((st = check_fwd_sizes(B, Hq, N, d)) != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(B, Hq, N, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const int64_t npad = bwd_npad(N);
  const int64_t nkb = (N + fa::kBwdKeyBlock - 1) / fa::kBwdKeyBlock;
  const int64_t nqb = (N + fa::kBwdRowBlock - 1) / fa::kBwdRowBlock;
  if ((int64_t)B * Hkv * nkb > INT32_MAX || (int64_t)B * Hq * nqb > INT32_MAX ||
      (int64_t)B * Hq * npad / 16 > INT32_MAX)
    return FA_ERR_SHAPE;

  fa::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.lse2 = static_cast<float*>(workspace);
  a.ndelta = a.lse2 + (size_t)B * Hq * npad;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.Npad = (int)npad;
  a.c = scale * fa::kLog2eHost;
  a.scale = scale;
  a.nkb = (int)nkb;
  a.nqb = (int)nqb;
  // Causal blocks differ in work; when one XCD's range of the grid is a whole
  // number (>= 2) of heads, their blocks interleave (heaviest of all first),
  // as in the forward.
  const auto head_group = [&](int64_t heads) {
    return causal && heads % 8 == 0 && heads >= 16 ? (int)(heads / 8) : 1;
  };
  a.hg_kv = head_group((int64_t)B * Hkv);
  a.hg_q = head_group((int64_t)B * Hq);
  const hipError_t e = fa::launch_bwd(a, d, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" size_t fa_decode_workspace_bytes(int B, int Hq, int L, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || L <= 0 || L > kMaxSeq || (d != 64 && d != 128) || num_splits < 1 || num_splits > L)
    return 0;
  const int S = decode_splits_used(L, num_splits);
  const int64_t rows = (int64_t)B * Hq;
  const int64_t floats = rows * S * (int64_t)d + rows * S;
  const size_t bytes = (size_t)floats * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

namespace {

int decode_impl(const void* q, const void* k, const void* v, void* o, float* lse, const int* lens,
                int B, int Hq, int Hkv, int L, int d, int num_splits, float scale,
                void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || L > kMaxSeq) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if (num_splits < 1 || num_splits > L) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ALIGN;
  if (elems(B, Hkv, L, d) < 0 || elems(B, Hq, 1, d) < 0) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, Hq, L, d, num_splits);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;

  const int G = Hq / Hkv;
  const int gm = G <= 16 ? next_pow2_le16(G) : 16;
  const int n_hg = (G + gm - 1) / gm;
  const int S = decode_splits_used(L, num_splits);
  const int64_t nwg = (int64_t)B * Hkv * n_hg * S;
  if (nwg > INT32_MAX || (int64_t)B * Hq > INT32_MAX) return FA_ERR_SHAPE;

  fa::DecArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o_part = static_cast<float*>(workspace);
  a.lse_part = a.o_part + (size_t)B * Hq * S * d;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L;
  a.chunk = decode_chunk(L, num_splits);
  a.S = S;
  a.G = G;
  a.n_hg = n_hg;
  a.c = scale * fa::kLog2eHost;
  a.lens = lens;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = fa::launch_decode_split(a, d, gm, s);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  e = fa::launch_combine(a.o_part, a.lse_part, static_cast<uint16_t*>(o), lse, B * Hq, S, d, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int L, int d, int num_splits, float scale,
                         void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  return decode_impl(q, k, v, o, lse, nullptr, B, Hq, Hkv, L, d, num_splits, scale, workspace, workspace_bytes,
                     stream);
}

extern "C" int fa_decode_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* seq_lens, int B, int Hq, int Hkv, int L, int d, int num_splits,
                                float scale, void* workspace, size_t workspace_bytes, fa_stream_t stream) {
  if (!seq_lens) return FA_ERR_NULL;
  if (!aligned4(seq_lens)) return FA_ERR_ALIGN;
  return decode_impl(q, k, v, o, lse, seq_lens, B, Hq, Hkv, L, d, num_splits, scale, workspace, workspace_bytes,
                     stream);
}
