// Device helpers of the routing: the wavefront top-k shared by the router
// kernels and the decode gate/up kernel (which routes a decode batch itself).
#pragma once

#include <math.h>

#include "common.h"

namespace moe {


template <int CTRL>
MOE_DEV uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// Maximum over each 16-lane row, left in every lane of the row.
MOE_DEV uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  return max(v, dpp_u32<0x140>(v));  // row_mirror
}

// Wave-wide maximum (uniform result).
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Wave-wide maximum left in every lane, on the vector unit only: row
// maxima through DPP, then the four rows through the gfx950 permlane swaps
// (no lane reads, so no round trip through scalar registers).
MOE_DEV uint32_t wave_max_all_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(static_cast<uint32_t>(p[0]), static_cast<uint32_t>(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(static_cast<uint32_t>(q[0]), static_cast<uint32_t>(q[1]));
}

// Wave-wide minimum (uniform result).
MOE_DEV uint32_t wave_min_u32(uint32_t v) {
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Softmax of the K selected logits (renorm) or over all E, the largest
// logit subtracted for range; sums in a fixed order.  Lane k < K holds
// round k's logit in my_v.
template <int NPL>
MOE_DEV float topk_weight(const float (&v)[NPL], int32_t E, int32_t K, int32_t renorm, float my_v, float top_v) {
  const int lane = __lane_id();
  const float mine = (lane < K) ? expf(my_v - top_v) : 0.f;
  float denom;
  if (renorm) {
    denom = 0.f;
    for (int k = 0; k < K; ++k) denom += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), k));
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (lane + 64 * j < E) part += expf(v[j] - top_v);
    denom = sum64(part);
  }
  return mine / denom;
}

// Top-k of one token's logits held by a whole wave: lane l holds experts
// l, l+64, ... in v[] (NaN already replaced by -inf, absent experts -inf).
// Lane k < K receives round k's expert and routing weight.
//
// NPL <= 4: each lane first sorts its NPL (key, expert) pairs, larger key
// first and the lower expert on equal keys.  A round is then one wave-wide
// maximum of the lanes' first keys; when one lane holds it (the usual case)
// its first pair wins, else the lowest expert among the lanes holding it
// (each lane's first pair is its lowest expert of that key).  The winning
// lane drops its first pair.  Results are those of the rule "largest
// logit, lower index on equal logits", round by round.
// The K rounds over per-lane lists sorted by (key desc, expert asc) (key 0:
// used or absent).  Each round: the maximum in every lane, the winning lane
// (the lowest expert among equal keys, rare), the winner's expert by one
// lane read, and the winner's list shifted with selects (no branch, no
// exec-mask copies); lane k keeps round k's key and expert.
template <int NPL>
MOE_DEV void wave_topk_rounds(uint32_t (&key)[NPL], int (&idx)[NPL], int32_t K, uint32_t &my_key, int &my_e) {
  const int lane = __lane_id();
  my_key = 0u;
  my_e = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_all_u32(key[0]);
    bool win = key[0] == m;
    uint64_t hit = __ballot(win);
    if (__popcll(hit) != 1) {
      const uint32_t lo = wave_min_u32(win ? static_cast<uint32_t>(idx[0]) : 0xFFFFFFFFu);
      win = win && static_cast<uint32_t>(idx[0]) == lo;
      hit = __ballot(win);
    }
    const int sel = __builtin_amdgcn_readlane(idx[0], __builtin_ctzll(hit));
#pragma unroll
    for (int j = 0; j + 1 < NPL; ++j) {
      key[j] = win ? key[j + 1] : key[j];
      idx[j] = win ? idx[j + 1] : idx[j];
    }
    key[NPL - 1] = win ? 0u : key[NPL - 1];
    const bool mine = lane == k;
    my_key = mine ? m : my_key;
    my_e = mine ? sel : my_e;
  }
}

template <int NPL>
MOE_DEV void wave_topk(const float (&v)[NPL], int32_t E, int32_t K, int32_t renorm, int &my_e, float &my_w) {
  const int lane = __lane_id();
  if constexpr (NPL <= 4) {
    uint32_t key[NPL];  // 0 = used or absent
    int idx[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      key[j] = (lane + 64 * j < E) ? float_key(v[j]) : 0u;
      idx[j] = lane + 64 * j;
    }
    // sorting network, comparing (key desc, expert asc)
    auto cswap = [&](int a, int b) {
      const bool sw = key[b] > key[a] || (key[b] == key[a] && idx[b] < idx[a]);
      const uint32_t ka = key[a], kb = key[b];
      const int ia = idx[a], ib = idx[b];
      key[a] = sw ? kb : ka;
      key[b] = sw ? ka : kb;
      idx[a] = sw ? ib : ia;
      idx[b] = sw ? ia : ib;
    };
    if constexpr (NPL >= 2) cswap(0, 1);
    if constexpr (NPL == 4) {
      cswap(2, 3);
      cswap(0, 2);
      cswap(1, 3);
      cswap(1, 2);
    }
    uint32_t my_key;
    wave_topk_rounds<NPL>(key, idx, K, my_key, my_e);
    const float top_v = key_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(my_key, 0)));
    my_w = topk_weight<NPL>(v, E, K, renorm, key_float(my_key), top_v);
    return;
  }
  uint32_t key[NPL];  // 0 = used or absent
#pragma unroll
  for (int j = 0; j < NPL; ++j) key[j] = (lane + 64 * j < E) ? float_key(v[j]) : 0u;
  float top_v = 0.f;
  float my_v = 0.f;  // lane k keeps round k's value and index
  my_e = 0;
  for (int k = 0; k < K; ++k) {
    // the largest remaining key, then the lowest expert index holding it
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) m = max(m, key[j]);
    m = wave_max_u32(m);
    int sel = 0;
#pragma unroll
    for (int j = NPL - 1; j >= 0; --j) {
      const uint64_t hit = __ballot(key[j] == m);
      if (hit) sel = 64 * j + __builtin_ctzll(hit);
    }
    if ((sel & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == (sel >> 6)) key[j] = 0u;
    }
    const float sel_v = key_float(m);
    if (k == 0) top_v = sel_v;
    if (lane == k) {
      my_v = sel_v;
      my_e = sel;
    }
  }
  my_w = topk_weight<NPL>(v, E, K, renorm, my_v, top_v);
}

// ------------------------------------------------------------------------
// Routing of a decode batch (T <= kFusedTokens) inside one block: logits
// from the router's partial sums (slices added in order, then the bias),
// top-k per token (one wave per token), and the permutation, all in LDS.
// With `publish` the block also writes the routing to global memory (ids,
// weights, counts, offsets, active list, rows, inverse positions).

constexpr int kRouteMaxPairs = 1024;  // T * K for T <= 16, K <= 64
constexpr int kRouteMaxExperts = 1024;

struct RouteLds {
  uint32_t mask[16][kRouteMaxExperts / 32];   // experts chosen by each token
  uint32_t early[16][kRouteMaxExperts / 32];  // tail-skip: experts each token ranks among its first N
  int ids[kRouteMaxPairs];
  float w[kRouteMaxPairs];
  int row_tok[kRouteMaxPairs];  // token of each permuted row
  int cnt[kRouteMaxExperts];    // rows per expert
  int off[kRouteMaxExperts];    // first row per expert
  int active[kRouteMaxExperts];
  int scan[16];
  int n_active;
  __attribute__((aligned(16))) uint2 lists[16 * 16 * kSortedKeep];  // sorted groups: (token, group) lists of (key, expert)
};

// Exclusive scan of one value per thread over the block (up to 16 waves);
// also returns the block total.
MOE_DEV int block_scan(int v, int *scratch, int &total) {
  const int lane = __lane_id();
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = scratch[w];
    before += w < wave ? x : 0;
    all += x;
  }
  total = all;
  lds_barrier();
  return before + inc - v;
}

// The shared gate of token t from the partials of row E (slices added in
// order, as the logits are): every lane gets sigmoid(logit).
MOE_DEV float route_gate(const RouteFusedArgs &a, int t) {
  float z = 0.f;
  for (int s0 = 0; s0 < a.S; ++s0) z += a.part[(static_cast<size_t>(s0) * a.T + t) * a.Ep + a.E];
  return 1.f / (1.f + expf(-z));
}

// Tail-skip: whether some token of the call ranks expert ex among its first
// N picks (always true without tail-skip).
MOE_DEV bool route_kept(const RouteFusedArgs &a, const RouteLds &L, int ex) {
  if (a.tail_skip <= 0) return true;
  uint32_t any = 0;
  for (int q = 0; q < a.T; ++q) any |= L.early[q][ex >> 5];
  return (any >> (ex & 31)) & 1u;
}

template <int NPL>
MOE_DEV void route_in_block(const RouteFusedArgs &a, RouteLds &L, bool publish) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int nw = nthr >> 6;
  const int T = a.T, E = a.E, S = a.S, K = a.K, Ep = a.Ep;
  const int TK = T * K;
  const int mwords = (E + 31) / 32;
  const int N = a.tail_skip > 0 ? min(a.tail_skip, K) : 0;
  for (int i = tid; i < E; i += nthr) L.cnt[i] = 0;
  for (int i = tid; i < T * mwords; i += nthr) {
    L.mask[i / mwords][i % mwords] = 0u;
    L.early[i / mwords][i % mwords] = 0u;
  }
  for (int t = wave; t < T; t += nw) {
    // the partials of four slices at a time as independent loads, then
    // their sums in slice order
    const float *__restrict__ part = a.part;
    float acc[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[j] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
      float pv[NPL][4];
#pragma unroll
      for (int j = 0; j < NPL; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ex = lane + 64 * j;
          pv[j][q] = (ex < E && s0 + q < S) ? part[(static_cast<size_t>(s0 + q) * T + t) * Ep + ex] : 0.f;
        }
#pragma unroll
      for (int j = 0; j < NPL; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (s0 + q < S) acc[j] += pv[j][q];
    }
    float v[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int ex = lane + 64 * j;
      const float sum = acc[j] + (a.router_bias && ex < E ? a.router_bias[ex] : 0.f);
      v[j] = (ex < E && sum == sum) ? sum : -INFINITY;  // NaN never outranks a number
      if (publish && a.logits && ex < E) a.logits[static_cast<size_t>(t) * E + ex] = sum;
    }
    int my_e;
    float my_w;
    wave_topk<NPL>(v, E, K, a.renorm, my_e, my_w);
    if (lane < K) {
      const int p = t * K + lane;
      L.ids[p] = my_e;
      L.w[p] = my_w;
      if (publish) {
        a.ids[p] = my_e;
        a.w[p] = my_w;
      }
    }
    if (a.gate_w) {
      const float gv = route_gate(a, t);
      if (publish && lane == 0) a.gate[t] = gv;
    }
  }
  lds_barrier();
  for (int p = tid; p < TK; p += nthr) {
    const int ex = L.ids[p];
    atomicAdd(&L.cnt[ex], 1);
    atomicOr(&L.mask[p / K][ex >> 5], 1u << (ex & 31));
    if (p % K < N) atomicOr(&L.early[p / K][ex >> 5], 1u << (ex & 31));
  }
  lds_barrier();
  // thread tid owns the experts [tid * ept, tid * ept + ept)
  const int ept = (E + nthr - 1) / nthr;  // <= 4
  // an active unit is an expert with rows that tail-skip keeps
  int c4[4], act4[4], n_here = 0, nz_here = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = tid * ept + i;
    c4[i] = (i < ept && ex < E) ? L.cnt[ex] : 0;
    act4[i] = c4[i] > 0 && route_kept(a, L, ex);
    n_here += c4[i];
    nz_here += act4[i];
  }
  int total = 0, n_act = 0;
  int base = block_scan(n_here, L.scan, total);
  int abase = block_scan(nz_here, L.scan, n_act);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = tid * ept + i;
    if (i < ept && ex < E) {
      L.off[ex] = base;
      if (act4[i]) L.active[abase] = ex;
      if (publish) {
        a.counts[ex] = c4[i];
        a.offsets[ex] = base;
        if (act4[i]) {
          a.active[abase] = ex;
          if (a.units) reinterpret_cast<int4 *>(a.units)[abase] = make_int4(ex, base, c4[i], 0);
        }
      }
      abase += act4[i];
    }
    base += c4[i];
  }
  if (tid == 0) {
    L.n_active = n_act;
    if (publish) {
      a.offsets[E] = total;
      *a.n_active = n_act;
    }
  }
  lds_barrier();
  for (int p = tid; p < TK; p += nthr) {
    // a token picks an expert at most once, so the pair's rank inside its
    // expert is the number of earlier tokens that picked the expert
    const int ex = L.ids[p];
    const int t = p / K;
    int r = 0;
    for (int q = 0; q < t; ++q) r += (L.mask[q][ex >> 5] >> (ex & 31)) & 1u;
    const int pos = L.off[ex] + r;
    L.row_tok[pos] = p / K;
    if (publish) {
      a.row_tok[pos] = p / K;
      a.row_w[pos] = L.w[p];
      a.inv_pos[p] = route_kept(a, L, ex) ? pos : -1;  // a left-out slot adds nothing
    }
  }
  lds_barrier();
}

// Inclusive sum over the wave: four row shifts give each 16-lane row's
// running sum, two row broadcasts carry the sums of the earlier rows.
MOE_DEV int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// The same routing for E <= 256 (NPL <= 4) in three phases with fewer
// block-wide steps: each token's wave (four tokens a wave when the
// previous launch left sorted groups) takes the token's top-k and builds
// its expert bitmask (route_small_topk); wave 0 derives the counts,
// offsets and active list from the masks (route_small_scan); every thread
// then places pairs (route_small_rows).  The phases are separated by block
// barriers, so a caller can start work that needs only the active list
// before the rows are placed.  Results are identical to route_in_block's.
// `stage` runs once per wave, after the wave's first partial-logit (or
// sorted-group) requests are out and before they are used (the gate/up
// kernel stages its x rows there, so their wait overlaps that round trip).
struct NoStage {
  MOE_DEV void operator()() const {}
};

// The top-k from the previous launch's sorted groups (route_sorted_ok:
// renormalised weights, K <= 8, E <= 256), four tokens a wave: 16-lane row
// r holds token 4 (wave + nw j) + r, and lane i of the row merges the (up
// to) eight pairs of group i (experts 16 i .. 16 i + 15), ranked by (key
// desc, expert asc) and staged in LDS.  Every selected expert is among its
// group's first eight, and the groups are in expert order, so each round is
// the row's largest head key, won by the lowest lane that holds it (the
// lowest expert of that key across groups, the group's lowest within one);
// the winner's list advances by one pair.
// The weights are the softmax over the K selections with the sum in round
// order, the arithmetic of topk_weight with renormalisation.
template <class Stage>
MOE_DEV void route_sorted_rows(const RouteFusedArgs &a, RouteLds &L, bool publish, const Stage &stage, bool &staged) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int T = a.T, E = a.E, K = a.K;
  const int mwords = (E + 31) / 32;  // <= 8
  const int N = a.tail_skip > 0 ? min(a.tail_skip, K) : 0;
  const int G = route_sorted_groups(E);  // <= 16
  const int r = lane >> 4, i = lane & 15;
  for (int t0 = 4 * wave; t0 < T; t0 += 4 * nw) {
    const int t = t0 + r;
    const bool tv = t < T;
    // the four tokens' lists (contiguous in the sorted array) into LDS,
    // 16 bytes a lane a request; each lane then holds its own list's head
    // and the pair after it, and reads the next pair ahead of each round
    const int n16 = T * G * (kSortedKeep / 2);  // 16-byte pieces of the array
    const int p0 = t0 * G * (kSortedKeep / 2);
    uint4 pc[kSortedKeep / 2];
#pragma unroll
    for (int q = 0; q < kSortedKeep / 2; ++q)
      pc[q] = reinterpret_cast<const uint4 *>(a.sorted)[min(p0 + lane + 64 * q, n16 - 1)];
    if (!staged) {
      stage();
      staged = true;
    }
#pragma unroll
    for (int q = 0; q < kSortedKeep / 2; ++q)
      if (p0 + lane + 64 * q < n16) reinterpret_cast<uint4 *>(L.lists)[p0 + lane + 64 * q] = pc[q];
    const bool gv = tv && i < G;
    const uint2 *my = L.lists + ((tv ? t : t0) * G + (i < G ? i : G - 1)) * kSortedKeep;
    const uint2 h0 = my[0], n0 = my[1];
    uint32_t hk = gv ? h0.x : 0u, nk = gv ? n0.x : 0u;  // 0: used or absent
    int hi = static_cast<int>(h0.y), ni = static_cast<int>(n0.y);
    int c = 1;  // list position of (nk, ni)
    // the row's own LDS operations run in order: clear, then (below) set the bits
    if (tv && i < mwords) {
      L.mask[t][i] = 0u;
      L.early[t][i] = 0u;
    }
    uint32_t my_key = 0u, top_key = 0u;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      // the pair after (nk, ni), read ahead by every lane (a winner takes it)
      const uint2 nx = my[c + 1 < kSortedKeep ? c + 1 : kSortedKeep - 1];
      const uint32_t m = row_max_u32(hk);
      bool win = hk == m;
      // the row's lanes holding m (at least one: m is one of their keys)
      const uint32_t rowbits = static_cast<uint32_t>(__ballot(win) >> (lane & 48)) & 0xFFFFu;
      win = win && i == __builtin_ctz(rowbits);
      if (win && tv) L.ids[t * K + k] = hi;
      my_key = i == k ? m : my_key;
      top_key = k == 0 ? m : top_key;
      hk = win ? nk : hk;
      hi = win ? ni : hi;
      nk = win ? (c + 1 < kSortedKeep && gv ? nx.x : 0u) : nk;
      ni = win ? static_cast<int>(nx.y) : ni;
      c += win ? 1 : 0;
    }
    const bool sel = tv && i < K;
    const int p = (tv ? t : 0) * K + i;
    const float mine = i < K ? expf(key_float(my_key) - key_float(top_key)) : 0.f;
    if (sel) L.w[p] = mine;
    float denom = 0.f;
    for (int k = 0; k < K; ++k) denom += L.w[(tv ? t : 0) * K + k];
    if (sel) {
      const float my_w = mine / denom;
      const int my_e = L.ids[p];
      L.w[p] = my_w;
      if (publish) {
        a.ids[p] = my_e;
        a.w[p] = my_w;
      }
      atomicOr(&L.mask[t][my_e >> 5], 1u << (my_e & 31));
      if (i < N) atomicOr(&L.early[t][my_e >> 5], 1u << (my_e & 31));
    }
    if (a.gate_w && tv) {
      const float gv2 = route_gate(a, t);
      if (publish && i == 0) a.gate[t] = gv2;
    }
  }
}

template <int NPL, class Stage = NoStage>
MOE_DEV void route_small_topk(const RouteFusedArgs &a, RouteLds &L, bool publish, const Stage &stage = Stage()) {
  static_assert(NPL <= 4, "E <= 256");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int T = a.T, E = a.E, S = a.S, K = a.K, Ep = a.Ep;
  const int mwords = (E + 31) / 32;  // <= 8
  const int N = a.tail_skip > 0 ? min(a.tail_skip, K) : 0;
  // the bias (when there is one) requested with the first partials
  float bias[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) bias[j] = a.router_bias && !a.sorted ? a.router_bias[min(lane + 64 * j, E - 1)] : 0.f;
  bool staged = false;
  if (a.sorted) route_sorted_rows(a, L, publish, stage, staged);
  for (int t = wave; !a.sorted && t < T; t += nw) {
    int my_e;
    float my_w;
    {
      const float *__restrict__ part = a.part;
      float acc[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] = 0.f;
      if (S == 1) {
        // whole logits (the previous launch formed them): one request each
        float pv[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) pv[j] = part[static_cast<size_t>(t) * Ep + min(lane + 64 * j, E - 1)];
        if (!staged) {
          stage();
          staged = true;
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j) acc[j] += pv[j];
      }
      for (int s0 = 0; S > 1 && s0 < S; s0 += 4) {
        // every request of the batch at once (clamped, unconditional), then
        // the slices added in order
        float pv[NPL][4];
#pragma unroll
        for (int j = 0; j < NPL; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ex = min(lane + 64 * j, E - 1);
            const int sl = min(s0 + q, S - 1);
            pv[j][q] = part[(static_cast<size_t>(sl) * T + t) * Ep + ex];
          }
        if (!staged) {
          stage();
          staged = true;
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[j] += (s0 + q < S) ? pv[j][q] : 0.f;
      }
      float v[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int ex = lane + 64 * j;
        const float sum = acc[j] + (a.router_bias && ex < E ? bias[j] : 0.f);
        v[j] = (ex < E && sum == sum) ? sum : -INFINITY;  // NaN never outranks a number
        if (publish && a.logits && ex < E) a.logits[static_cast<size_t>(t) * E + ex] = sum;
      }
      wave_topk<NPL>(v, E, K, a.renorm, my_e, my_w);
    }
    // the wave's own LDS operations run in order: clear, then set the bits
    if (lane < mwords) {
      L.mask[t][lane] = 0u;
      L.early[t][lane] = 0u;
    }
    if (lane < K) {
      const int p = t * K + lane;
      L.ids[p] = my_e;
      L.w[p] = my_w;
      if (publish) {
        a.ids[p] = my_e;
        a.w[p] = my_w;
      }
      atomicOr(&L.mask[t][my_e >> 5], 1u << (my_e & 31));
      if (lane < N) atomicOr(&L.early[t][my_e >> 5], 1u << (my_e & 31));
    }
    if (a.gate_w) {
      const float gv = route_gate(a, t);
      if (publish && lane == 0) a.gate[t] = gv;
    }
  }
  if (!staged) stage();
}

// Wave 0 only, after route_small_topk and a block barrier.
MOE_DEV void route_small_scan(const RouteFusedArgs &a, RouteLds &L, bool publish) {
  const int lane = threadIdx.x & 63;
  const int T = a.T, E = a.E;
  // lane l owns the experts 4l .. 4l+3 (one mask word)
  int c[4] = {0, 0, 0, 0};
  const int word = (4 * lane) >> 5, sh = (4 * lane) & 31;
  if (4 * lane < E) {
    for (int t = 0; t < T; ++t) {
      const uint32_t m = L.mask[t][word] >> sh;
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += (m >> i) & 1u;
    }
  }
  // an active unit is an expert with rows that tail-skip keeps
  int n_here = 0, nz_here = 0, act[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * lane + i >= E) c[i] = 0;
    act[i] = c[i] > 0 && route_kept(a, L, 4 * lane + i);
    n_here += c[i];
    nz_here += act[i];
  }
  const int inc = wave_incl_sum(n_here), incz = wave_incl_sum(nz_here);
  int base = inc - n_here, abase = incz - nz_here;
  const int total = __builtin_amdgcn_readlane(inc, 63), n_act = __builtin_amdgcn_readlane(incz, 63);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = 4 * lane + i;
    if (ex < E) {
      L.cnt[ex] = c[i];
      L.off[ex] = base;
      if (act[i]) L.active[abase] = ex;
      if (publish) {
        a.counts[ex] = c[i];
        a.offsets[ex] = base;
        if (act[i]) {
          a.active[abase] = ex;
          if (a.units) reinterpret_cast<int4 *>(a.units)[abase] = make_int4(ex, base, c[i], 0);
        }
      }
      abase += act[i];
    }
    base += c[i];
  }
  if (lane == 0) {
    L.n_active = n_act;
    if (publish) {
      a.offsets[E] = total;
      *a.n_active = n_act;
    }
  }
}

// Every thread, after route_small_scan and a block barrier.
MOE_DEV void route_small_rows(const RouteFusedArgs &a, RouteLds &L, bool publish) {
  const int K = a.K, TK = a.T * a.K;
  for (int p = threadIdx.x; p < TK; p += blockDim.x) {
    // rank inside the expert = earlier tokens that picked it
    const int ex = L.ids[p];
    const int t = p / K;
    int r = 0;
    for (int q = 0; q < t; ++q) r += (L.mask[q][ex >> 5] >> (ex & 31)) & 1u;
    const int pos = L.off[ex] + r;
    L.row_tok[pos] = t;
    if (publish) {
      a.row_tok[pos] = t;
      a.row_w[pos] = L.w[p];
      a.inv_pos[p] = route_kept(a, L, ex) ? pos : -1;  // a left-out slot adds nothing
    }
  }
}

template <int NPL, class Stage = NoStage>
MOE_DEV void route_in_block_small(const RouteFusedArgs &a, RouteLds &L, bool publish, const Stage &stage = Stage()) {
  route_small_topk<NPL>(a, L, publish, stage);
  lds_barrier();
  if ((threadIdx.x >> 6) == 0) route_small_scan(a, L, publish);
  lds_barrier();
  route_small_rows(a, L, publish);
  lds_barrier();
}

}  // namespace moe
