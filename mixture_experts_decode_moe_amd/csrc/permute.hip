// Token-by-expert permutation: histogram, exclusive prefix scan and a stable
// scatter, all on the device (the pages moved this "grouping" off a single
// host or device thread: "Strata on an Intel Arc", Decode round 2, and
// "Models and backends", What was tuned).
//
// Pass 1 (one block per tile of 1024 (token, slot) pairs): within each wave
// the pairs that share an expert are found with ballots; each group's size
// goes to an LDS table [wave][expert], which gives every pair its rank among
// the tile's earlier pairs of the same expert, and the tile's histogram.
// Pass 2 (one block per tile): every block re-derives the expert totals and
// their exclusive prefix sum from the (small) tile histograms, adds the
// counts of earlier tiles, and scatters its pairs.  Order inside an expert is
// the pair order t*K + k; no atomic whose order could change a value is used.
#include "common.h"

namespace moe {

constexpr int kWaves = kPermuteTile / 64;  // 16

MOE_DEV uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__global__ void __launch_bounds__(kPermuteTile) permute_tile_kernel(const int32_t *__restrict__ ids, int32_t TK,
                                                                    int32_t E, int32_t *__restrict__ tile_hist,
                                                                    int32_t *__restrict__ rank) {
  extern __shared__ uint16_t wcnt[];  // [kWaves][E]
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  for (int i = tid; i < kWaves * E; i += kPermuteTile) wcnt[i] = 0;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kPermuteTile + tid;
  int e = -1;
  if (p < TK) {
    e = ids[p];
    if (e < 0 || e >= E) e = -1;  // out-of-range ids are dropped
  }
  const bool valid = e >= 0;
  lds_barrier();
  uint64_t todo = __ballot(valid);
  uint64_t peers = 0;
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int v = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == v);
    if (valid && e == v) peers = m;
    todo &= ~m;
  }
  const int rank_w = __popcll(peers & lanemask_lt());
  if (valid && rank_w == 0) wcnt[wave * E + e] = static_cast<uint16_t>(__popcll(peers));
  lds_barrier();
  if (valid) {
    int r = rank_w;
    for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
    rank[p] = r;
  }
  for (int x = tid; x < E; x += kPermuteTile) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += wcnt[w * E + x];
    tile_hist[static_cast<size_t>(blockIdx.x) * E + x] = s;
  }
}

// Exclusive scan of one value per thread over a 1024-thread block.
MOE_DEV int block_exclusive_scan(int v, int *scratch /* >= kWaves ints */, int &total) {
  const int lane = __lane_id();
  const int wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int s = scratch[w];
    if (w < wave) before += s;
    all += s;
  }
  lds_barrier();
  total = all;
  return before + inc - v;
}

__global__ void __launch_bounds__(kPermuteTile) permute_scatter_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int32_t TK, int32_t K, int32_t E,
    int32_t n_tiles, const int32_t *__restrict__ tile_hist, const int32_t *__restrict__ rank,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ row_tok,
    float *__restrict__ row_w, int32_t *__restrict__ inv_pos, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active) {
  extern __shared__ int32_t base[];  // [E]
  __shared__ int scan_scratch[kWaves];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  // E <= 1024: thread tid owns expert tid.
  int tot = 0, pre = 0;
  if (tid < E) {
    for (int tl = 0; tl < n_tiles; ++tl) {
      const int h = tile_hist[static_cast<size_t>(tl) * E + tid];
      tot += h;
      if (tl < tile) pre += h;
    }
  }
  int total = 0;
  const int excl = block_exclusive_scan(tot, scan_scratch, total);
  int n_act = 0;
  const int act_pos = block_exclusive_scan(tot > 0 ? 1 : 0, scan_scratch, n_act);
  if (tid < E) base[tid] = excl + pre;
  if (tile == 0) {
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = excl;
      if (tot > 0) active[act_pos] = tid;
    }
    if (tid == 0) {
      offsets[E] = total;
      *n_active = n_act;
    }
  }
  lds_barrier();
  const int64_t p = static_cast<int64_t>(tile) * kPermuteTile + tid;
  if (p < TK) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int pos = base[e] + rank[p];
      row_tok[pos] = static_cast<int32_t>(p / K);
      row_w[pos] = w ? w[p] : 1.0f;
      inv_pos[p] = pos;
    } else {
      inv_pos[p] = -1;
    }
  }
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s) {
  const int32_t TK = a.T * a.K;
  const int32_t n_tiles = (TK + kPermuteTile - 1) / kPermuteTile;
  permute_tile_kernel<<<n_tiles, kPermuteTile, kWaves * a.E * sizeof(uint16_t), s>>>(a.ids, TK, a.E, a.tile_hist,
                                                                                  a.rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter_kernel<<<n_tiles, kPermuteTile, a.E * sizeof(int32_t), s>>>(
      a.ids, a.w, TK, a.K, a.E, n_tiles, a.tile_hist, a.rank, a.counts, a.offsets, a.row_tok, a.row_w, a.inv_pos,
      a.active, a.n_active);
  return hipGetLastError();
}

}  // namespace moe
