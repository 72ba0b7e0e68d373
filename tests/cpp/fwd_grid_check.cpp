// Host-side check of the forward's work decomposition (no GPU needed): for
// many shapes, the planner's grid and the kernels' index mapping (the same
// header functions the kernels call) cover every visible key tile of every
// query block exactly once, keep every partial-result index inside the
// workspace the planner sized, and give the combine kernel the number of
// partials each block's rows received.
//
// Build and run: tests/test_grid_plan.py (g++ with the ROCm headers).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa_launch.h"

namespace {

int failures = 0;

void fail(const char* what, int B, int Hq, int N, int d, int causal, int fp8, int cus, long detail) {
  if (failures < 20)
    std::printf("FAIL %s: B=%d Hq=%d N=%d d=%d causal=%d fp8=%d cus=%d (%ld)\n", what, B, Hq, N, d, causal, fp8,
                cus, detail);
  ++failures;
}

void check(int B, int Hq, int N, int d, bool causal, bool fp8, int cus) {
  const fa::FwdPlan p = fa::plan_fwd(B, Hq, N, d, causal, fp8, cus);
  fa::FwdArgs a{};
  a.B = B; a.Hq = Hq; a.Hkv = 1; a.N = N;
  a.rows = p.rows; a.nqb = p.nqb; a.nwg = (int)p.nwg;
  a.n_splits = p.n_splits; a.split_tiles = p.split_tiles; a.head_group = p.head_group;
  a.split_target = fp8 ? 0 : p.split_target;
  a.per_head = fp8 ? 0 : p.per_head;
  const int tiles_all = (N + fa::kFwdKeys - 1) / fa::kFwdKeys;
  const long nblocks = (long)B * Hq * p.nqb;
  std::vector<int> cover((size_t)nblocks * tiles_all, 0);
  std::vector<int> parts((size_t)nblocks, 0), direct((size_t)nblocks, 0), max_split((size_t)nblocks, -1);
  const size_t rows = (size_t)B * Hq * N;
  if (p.n_splits > 1 && p.ws_bytes < rows * p.n_splits * ((size_t)d * 2 + 4))
    fail("workspace smaller than the partials", B, Hq, N, d, causal, fp8, cus, (long)p.ws_bytes);
  const int per_cu = (p.rows == 256 ? 1 : 2) * cus;
  if (p.split_target > 0 && p.nwg > per_cu) fail("causal split grid takes more than one round", B, Hq, N, d, causal, fp8, cus, p.nwg);
  for (int lid = 0; lid < p.nwg; ++lid) {
    int qb, split, bh, st, ns;
    fa::fwd_block_map(lid, a, causal, qb, split, bh, st, ns);
    if (qb < 0 || qb >= p.nqb || bh < 0 || bh >= B * Hq) {
      fail("block out of range", B, Hq, N, d, causal, fp8, cus, lid);
      continue;
    }
    // The kernel's tile range of this work-group.
    const int q0 = qb * p.rows;
    const int kv_end = causal ? (q0 + p.rows < N ? q0 + p.rows : N) : N;
    const int t_begin = split * st;
    const int vis = (kv_end + fa::kFwdKeys - 1) / fa::kFwdKeys;
    const int t_end = vis < t_begin + st ? vis : t_begin + st;
    if (t_end <= t_begin) continue;  // an empty split returns at once
    const size_t blk = (size_t)bh * p.nqb + qb;
    for (int t = t_begin; t < t_end; ++t) cover[blk * tiles_all + t]++;
    if (ns == 1) {
      direct[blk]++;
    } else {
      if (split >= p.n_splits) fail("partial index past the workspace", B, Hq, N, d, causal, fp8, cus, split);
      parts[blk]++;
      if (split > max_split[blk]) max_split[blk] = split;
    }
  }
  for (long blk = 0; blk < nblocks; ++blk) {
    const int qb = (int)(blk % p.nqb);
    const int q0 = qb * p.rows;
    const int kv_end = causal ? (q0 + p.rows < N ? q0 + p.rows : N) : N;
    const int vis = (kv_end + fa::kFwdKeys - 1) / fa::kFwdKeys;
    for (int t = 0; t < tiles_all; ++t) {
      const int want = t < vis ? 1 : 0;
      if (cover[blk * tiles_all + t] != want) {
        fail("tile covered a wrong number of times", B, Hq, N, d, causal, fp8, cus, blk * 100000L + t);
        break;
      }
    }
    // What the combine kernel reads for this block's rows.
    int S;
    bool skip = false;
    if (causal && a.split_target > 0) {
      S = (vis + a.split_target - 1) / a.split_target;
      skip = S == 1;
    } else {
      S = p.n_splits < (vis + p.split_tiles - 1) / p.split_tiles ? p.n_splits
                                                                 : (vis + p.split_tiles - 1) / p.split_tiles;
    }
    if (p.n_splits == 1) {
      if (direct[blk] != 1 || parts[blk] != 0) fail("unsplit block not written once", B, Hq, N, d, causal, fp8, cus, blk);
    } else if (skip) {
      if (direct[blk] != 1 || parts[blk] != 0) fail("one-split block not written directly", B, Hq, N, d, causal, fp8, cus, blk);
    } else {
      if (direct[blk] != 0 || parts[blk] != S || max_split[blk] != S - 1)
        fail("combine reads other partials than were written", B, Hq, N, d, causal, fp8, cus, blk);
    }
  }
}

}  // namespace

int main() {
  long shapes = 0;
  const int Ns[] = {1, 17, 64, 100, 129, 300, 500, 960, 1000, 1023, 1024, 1025, 1100, 2000, 2048, 2500, 3000,
                    4096, 4100, 6000, 7937, 8000, 8191, 8192, 8200, 12345, 16384, 20000, 32768, 65280};
  const int Hs[] = {1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 40, 64};
  for (int cus : {256, 304, 80}) {
    for (int B : {1, 2, 3})
      for (int H : Hs)
        for (int N : Ns)
          for (int d : {64, 128})
            for (int causal = 0; causal < 2; ++causal)
              for (int fp8 = 0; fp8 < 2; ++fp8) {
                if ((long)B * H * N > (1L << 22)) continue;
                check(B, H, N, d, causal != 0, fp8 != 0, cus);
                ++shapes;
              }
  }
  std::printf("%ld shapes checked, %d failures\n", shapes, failures);
  return failures == 0 ? 0 : 1;
}
