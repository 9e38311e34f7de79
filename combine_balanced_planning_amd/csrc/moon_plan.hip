// moon_plan.hip — the online balancing planner for gfx950 (wave64).
//
// Four launches on the caller's stream ("MoonEP Public API Visual Guide",
// Buffer.dispatch: planning turns the S*K routes of every rank into a compact
// dst map, local offsets, E+B padded groups and duplicate-route metadata):
//
//   k_plan_hist     one workgroup per tile of tokens: per-(expert, tile) route
//                   counts in LDS, id validation.
//   k_plan_balance  one workgroup: per-expert scan over tiles (one lane per
//                   tile), per-home-rank stream offsets, the alias balance
//                   (every rank gets exactly S*K routes, overflow from at most
//                   one remote home rank: MoonEP README, "Perfect balance" and
//                   "How to set B"), slots, padded layout (cu_seqlens,
//                   zero_fill_ranges), experts_to_copy, remote_stats, status.
//   k_plan_place    one workgroup per tile: stable within-tile rank of every
//                   route by a ballot multisplit over the expert id bits and
//                   per-wave running counters in LDS, then stream position ->
//                   (destination rank, group, row); primary/duplicate by
//                   lane shuffles inside each token; signed dst.
//   k_plan_dups     one workgroup per tile: duplicate records in token order
//                   (ballot multisplit over destination-rank bits).
//
// Nothing depends on the order of atomics: LDS atomics only add counts, so
// the plan is bit-reproducible.  Tiles never span two source ranks, every
// wave owns a contiguous token range of its tile, and routes are processed in
// chunks of whole tokens (floor(64/K) tokens per chunk) so a token's K routes
// sit in adjacent lanes of one wave.
#include "moon_internal.h"

namespace moon {
namespace {

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanes_below() {
  return (lane_id() == 0) ? 0ull : ((~0ull) >> (kWave - lane_id()));
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Lanes of `set` whose `key` equals this lane's key (ballot over key bits).
__device__ __forceinline__ uint64_t match_key(uint64_t set, int key, int bits) {
  uint64_t peers = set;
  for (int b = 0; b < bits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Order LDS traffic of one wave between consecutive chunks.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

struct TileRange {
  int r, s0, s1;  // source rank, token range [s0, s1) of that rank
};

__device__ __forceinline__ TileRange tile_range(const Dims& d, int t) {
  TileRange tr;
  tr.r = t / d.tiles_per_rank;
  const int ti = t % d.tiles_per_rank;
  tr.s0 = ti * d.tile_tok;
  tr.s1 = min(d.S, tr.s0 + d.tile_tok);
  return tr;
}

// Contiguous token range of wave w inside a tile.
__device__ __forceinline__ void wave_tokens(const TileRange& tr, int w, int& ws0, int& ws1) {
  const int nt = tr.s1 - tr.s0;
  const int per = (nt + kPlanWaves - 1) / kPlanWaves;
  ws0 = min(tr.s1, tr.s0 + w * per);
  ws1 = min(tr.s1, ws0 + per);
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPlanThreads)
    k_plan_hist(Dims d, const int32_t* __restrict__ topk, int32_t* __restrict__ tile_cnt,
                int32_t* __restrict__ tile_bad) {
  __shared__ int hist[kMaxE];
  const int t = blockIdx.x;
  const TileRange tr = tile_range(d, t);
  for (int e = threadIdx.x; e < d.E; e += kPlanThreads) hist[e] = 0;
  __syncthreads();
  int bad = 0;
  const int64_t i0 = ((int64_t)tr.r * d.S + tr.s0) * d.K;
  const int64_t i1 = ((int64_t)tr.r * d.S + tr.s1) * d.K;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kPlanThreads) {
    const int e = topk[i];
    if ((unsigned)e < (unsigned)d.E) atomicAdd(&hist[e], 1);
    else bad = 1;
  }
  bad = __syncthreads_or(bad);
  for (int e = threadIdx.x; e < d.E; e += kPlanThreads) tile_cnt[e * d.ntiles + t] = hist[e];
  if (threadIdx.x == 0) tile_bad[t] = bad;
}

// ---------------------------------------------------------------------------
constexpr int kEPerWave = kMaxE / kPlanWaves;

__global__ void __launch_bounds__(kPlanThreads)
    k_plan_balance(Dims d, const int32_t* __restrict__ tpe, Scratch sc, PlanArrays pa) {
  __shared__ int sT[kMaxE], sPe[kMaxE];
  __shared__ int sL[kMaxR], sKeep[kMaxR], sDonor[kMaxR], sSegA[kMaxR], sSegB[kMaxR];
  __shared__ int sNslot[kMaxSlotsTotal];
  __shared__ int sAlias[6 * kMaxR];
  __shared__ int sFlags;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int E = d.E, R = d.R, Eg = d.Eg, B = d.B, EB = d.EB;

  if (threadIdx.x == 0) sFlags = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < d.ntiles; t += kPlanThreads)
    if (sc.tile_bad[t]) atomicOr(&sFlags, kBadExpert);
  __syncthreads();
  if (sFlags & kBadExpert) {
    if (threadIdx.x == 0) pa.status[0] = sFlags;
    return;
  }

  // Per-expert exclusive scan over tiles (tiles in global route order).  All
  // loads of a wave are issued before the first scan.
  {
    int vals[kEPerWave];
#pragma unroll
    for (int j = 0; j < kEPerWave; ++j) {
      const int e = wave + j * kPlanWaves;
      vals[j] = (e < E && lane < d.ntiles) ? sc.tile_cnt[e * d.ntiles + lane] : 0;
    }
#pragma unroll
    for (int j = 0; j < kEPerWave; ++j) {
      const int e = wave + j * kPlanWaves;
      if (e >= E) break;
      const int c = vals[j];
      const int incl = wave_incl_scan(c);
      if (lane < d.ntiles) sc.base[e * d.ntiles + lane] = incl - c;
      const int tot = __shfl(incl, kWave - 1, kWave);
      if (lane == 0) sT[e] = tot;
      if (tpe != nullptr) {
        // routes of e from source rank r = sum over that rank's tiles
        const int tpr = d.tiles_per_rank;
        const int before = __shfl(incl, max(lane - tpr, 0), kWave);
        const int cnt_r = incl - (lane >= tpr ? before : 0);
        const bool last = lane < d.ntiles && (lane % tpr) == tpr - 1;
        if (last && tpe[(lane / tpr) * E + e] != cnt_r) atomicOr(&sFlags, kHistogram);
      }
    }
  }
  __syncthreads();

  // Stream offsets: home rank h's stream is its experts in ascending id.
  for (int h = wave; h < R; h += kPlanWaves) {
    int carry = 0;
    for (int j0 = 0; j0 < Eg; j0 += kWave) {
      const int j = j0 + lane;
      const int v = j < Eg ? sT[h * Eg + j] : 0;
      const int incl = wave_incl_scan(v);
      if (j < Eg) {
        sPe[h * Eg + j] = carry + incl - v;
        sc.Pe[h * Eg + j] = carry + incl - v;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) sL[h] = carry;
  }
  __syncthreads();

  // Balance: alias fill on the R rank loads (R <= 32, one lane; the queues
  // live in LDS).
  if (threadIdx.x == 0) {
    const int C = d.S * d.K;
    int* rem = sAlias;
    int* take = sAlias + kMaxR;
    int* off = sAlias + 2 * kMaxR;
    int* given = sAlias + 3 * kMaxR;
    int* small = sAlias + 4 * kMaxR;
    int* large = sAlias + 5 * kMaxR;
    int sh = 0, st = 0, lh = 0, lt = 0;
    for (int h = 0; h < R; ++h) {
      rem[h] = sL[h];
      sDonor[h] = -1;
      take[h] = 0;
      off[h] = 0;
      given[h] = 0;
      if (rem[h] < C) small[st++] = h;
    }
    for (int h = 0; h < R; ++h)
      if (rem[h] > C) large[lt++] = h;
    while (sh < st) {
      const int u = small[sh++];
      if (lh >= lt) {  // cannot happen: the loads sum to R*C
        sFlags |= kInternal;
        break;
      }
      const int o = large[lh];
      const int f = C - rem[u];
      sDonor[u] = o;
      take[u] = f;
      off[u] = given[o];
      given[o] += f;
      rem[o] -= f;
      if (rem[o] < C) {
        ++lh;
        if (st < kMaxR) small[st++] = o;
      } else if (rem[o] == C) {
        ++lh;
      }
    }
    for (int h = 0; h < R; ++h) sKeep[h] = rem[h];
    for (int u = 0; u < R; ++u) {
      const int o = sDonor[u];
      sSegA[u] = o >= 0 ? sKeep[o] + off[u] : 0;
      sSegB[u] = o >= 0 ? sKeep[o] + off[u] + take[u] : 0;
    }
    for (int h = 0; h < R; ++h) {
      sc.keep[h] = sKeep[h];
      sc.donor[h] = sDonor[h];
      sc.seg_a[h] = sSegA[h];
      sc.seg_b[h] = sSegB[h];
    }
  }
  __syncthreads();

  // Slots: a receiver's pieces are its donor's experts overlapping its
  // segment, in ascending expert id, numbered from slot 0.
  for (int u = wave; u < R; u += kPlanWaves) {
    const int o = sDonor[u];
    int count = 0, routed = 0;
    for (int j0 = 0; j0 < Eg; j0 += kWave) {
      const int j = j0 + lane;
      bool piece = false;
      int len = 0;
      if (o >= 0 && j < Eg) {
        const int e = o * Eg + j;
        const int lo = max(sPe[e], sSegA[u]);
        const int hi = min(sPe[e] + sT[e], sSegB[u]);
        piece = sT[e] > 0 && lo < hi;
        len = hi - lo;
      }
      const uint64_t m = __ballot(piece);
      const int slot = count + __popcll(m & lanes_below());
      if (j < Eg) sc.slot_of[u * Eg + j] = (piece && slot < B) ? slot : -1;
      if (piece) {
        if (slot < B) {
          pa.etc[u * B + slot] = o * Eg + j;
          sNslot[u * B + slot] = len;
          routed += len;
        } else {
          atomicOr(&sFlags, kSlotBudget);
        }
      }
      count += __popcll(m);
    }
    routed = wave_sum(routed);
    for (int j = count + lane; j < B; j += kWave) {
      pa.etc[u * B + j] = -1;
      sNslot[u * B + j] = 0;
    }
    if (lane == 0) {
      pa.rstats[u * 2 + 0] = min(count, B);
      pa.rstats[u * 2 + 1] = routed;
    }
  }
  __syncthreads();

  // Layout: inclusive padded end offsets of the E+B groups of every rank.
  if ((sFlags & (kSlotBudget | kHistogram | kInternal)) == 0) {
    const int P = d.P;
    for (int u = wave; u < R; u += kPlanWaves) {
      int carry = 0;
      for (int g0 = 0; g0 < EB; g0 += kWave) {
        const int g = g0 + lane;
        int n = 0;
        if (g < E) {
          if (g / Eg == u) n = min(max(sKeep[u] - sPe[g], 0), sT[g]);
        } else if (g < EB) {
          n = sNslot[u * B + (g - E)];
        }
        const int pad = n == 0 ? 0 : (n + P - 1) / P * P;
        const int incl = wave_incl_scan(pad);
        if (g < EB) {
          const int end = carry + incl;
          pa.cu[u * EB + g] = end;
          pa.zfr[(u * EB + g) * 2 + 0] = end - pad + n;
          pa.zfr[(u * EB + g) * 2 + 1] = end;
        }
        carry += __shfl(incl, kWave - 1, kWave);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) pa.status[0] = sFlags;
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPlanThreads)
    k_plan_place(Dims d, const int32_t* __restrict__ topk, Scratch sc, PlanArrays pa) {
  if (pa.status[0] != 0) return;
  __shared__ int cnt[kPlanWaves * kMaxE];
  __shared__ int sBase[kMaxE], sPe[kMaxE], sSlot[kMaxE];
  __shared__ int sKeep[kMaxR], sDonor[kMaxR], sSegA[kMaxR], sSegB[kMaxR];
  __shared__ int sDup[kMaxR * 2];
  __shared__ int sFlags;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int E = d.E, R = d.R, K = d.K, Eg = d.Eg, EB = d.EB, NvS = d.NvS;
  const int t = blockIdx.x;
  const TileRange tr = tile_range(d, t);

  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    sBase[e] = sc.base[e * d.ntiles + t];
    sPe[e] = sc.Pe[e];
    sSlot[e] = sc.slot_of[e];
  }
  for (int x = threadIdx.x; x < kPlanWaves * E; x += kPlanThreads) cnt[x] = 0;
  for (int h = threadIdx.x; h < R; h += kPlanThreads) {
    sKeep[h] = sc.keep[h];
    sDonor[h] = sc.donor[h];
    sSegA[h] = sc.seg_a[h];
    sSegB[h] = sc.seg_b[h];
  }
  for (int x = threadIdx.x; x < R * 2; x += kPlanThreads) sDup[x] = 0;
  if (threadIdx.x == 0) sFlags = 0;
  __syncthreads();

  int ws0, ws1;
  wave_tokens(tr, wave, ws0, ws1);
  const int64_t rowbase = (int64_t)tr.r * d.S;
  // Pass 1: per-wave expert counts.
  for (int64_t i = (rowbase + ws0) * K + lane; i < (rowbase + ws1) * K; i += kWave)
    atomicAdd(&cnt[wave * E + topk[i]], 1);
  __syncthreads();
  // Exclusive prefix over waves: routes of e in earlier waves of this tile.
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    int run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();

  // Pass 2: chunks of whole tokens.
  const int ctok = kWave / K;
  const int k = lane % K;
  for (int tok = ws0; tok < ws1; tok += ctok) {
    const int nl = min(ctok, ws1 - tok) * K;
    const bool act = lane < nl;
    const int64_t i = (rowbase + tok) * K + lane;
    const int e = act ? topk[i] : 0;
    const uint64_t peers = match_key(__ballot(act), e, d.ebits);
    const int rank = __popcll(peers & lanes_below());
    const int tot = __popcll(peers);
    int u = 0, G = 0;
    if (act) {
      const int pos = sBase[e] + cnt[wave * E + e] + rank;  // position among e's routes
      const int h = e / Eg;
      const int q = sPe[e] + pos;                            // position in h's stream
      int g, idx;
      if (q < sKeep[h]) {
        u = h;
        g = e;
        idx = q - sPe[e];
      } else {
        u = -1;
        for (int v = 0; v < R; ++v)
          if (sDonor[v] == h && sSegA[v] <= q && q < sSegB[v]) u = v;
        const int slot = u >= 0 ? sSlot[u * Eg + (e - h * Eg)] : -1;
        if (u < 0 || slot < 0) {  // cannot happen for a consistent plan
          atomicOr(&sFlags, kInternal);
          u = 0;
          g = 0;
          idx = 0;
        } else {
          g = E + slot;
          idx = q - max(sPe[e], sSegA[u]);
        }
      }
      const int start = g == 0 ? 0 : pa.cu[u * EB + g - 1];
      G = u * NvS + start + idx;
    }
    wave_lds_fence();
    if (act && rank == 0) cnt[wave * E + e] += tot;
    wave_lds_fence();
    // Primary = first route of the token to its destination rank.
    bool dup = false, has_later = false;
    for (int j = 1; j < K; ++j) {
      const int ub = __shfl(u, (lane - j) & (kWave - 1), kWave);
      const int ua = __shfl(u, (lane + j) & (kWave - 1), kWave);
      if (j <= k && ub == u) dup = true;
      if (j < K - k && ua == u) has_later = true;
    }
    if (act) {
      pa.dst[i] = dup ? -(G + 1) : G;
      if (dup) atomicAdd(&sDup[u * 2 + 1], 1);
      else if (has_later) atomicAdd(&sDup[u * 2 + 0], 1);
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < R * 2; x += kPlanThreads) sc.tile_dup[t * R * 2 + x] = sDup[x];
  if (threadIdx.x == 0 && sFlags) atomicOr(&pa.status[0], sFlags);
}

// ---------------------------------------------------------------------------
__device__ __forceinline__ int dst_row(int v) { return v >= 0 ? v : -v - 1; }

__global__ void __launch_bounds__(kPlanThreads) k_plan_dups(Dims d, Scratch sc, PlanArrays pa) {
  if (pa.status[0] != 0) return;
  __shared__ int wc[kPlanWaves * kMaxR * 2];
  __shared__ int sBaseD[kMaxR * 2];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int R = d.R, K = d.K, NvS = d.NvS;
  const int t = blockIdx.x;
  const TileRange tr = tile_range(d, t);

  // Duplicate groups / rows of earlier tiles, per destination rank.
  for (int x = threadIdx.x; x < R * 2; x += kPlanThreads) {
    int acc = 0;
    for (int tt = 0; tt < t; ++tt) acc += sc.tile_dup[tt * R * 2 + x];
    sBaseD[x] = acc;
    if (t == d.ntiles - 1) pa.dup_counts[x] = acc + sc.tile_dup[t * R * 2 + x];
  }
  for (int x = threadIdx.x; x < kPlanWaves * R * 2; x += kPlanThreads) wc[x] = 0;
  __syncthreads();

  int ws0, ws1;
  wave_tokens(tr, wave, ws0, ws1);
  const int64_t rowbase = (int64_t)tr.r * d.S;
  const int ctok = kWave / K;
  const int k = lane % K;

  // Pass 1: per-wave counts of groups (owners) and duplicates per rank.
  for (int tok = ws0; tok < ws1; tok += ctok) {
    const int nl = min(ctok, ws1 - tok) * K;
    const bool act = lane < nl;
    const int v = act ? pa.dst[(rowbase + tok) * K + lane] : 0;
    const int u = dst_row(v) / NvS;
    const bool dup = act && v < 0;
    bool owner = false;
    for (int j = 1; j < K; ++j) {
      const int ua = __shfl(u, (lane + j) & (kWave - 1), kWave);
      if (act && !dup && j < K - k && ua == u) owner = true;
    }
    if (owner) atomicAdd(&wc[(wave * R + u) * 2 + 0], 1);
    if (dup) atomicAdd(&wc[(wave * R + u) * 2 + 1], 1);
  }
  __syncthreads();
  for (int x = threadIdx.x; x < R * 2; x += kPlanThreads) {
    int run = sBaseD[x];
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = wc[w * R * 2 + x];
      wc[w * R * 2 + x] = run;
      run += c;
    }
  }
  __syncthreads();

  // Pass 2: records.  Within a wave, owners (and duplicates) of one rank are
  // ranked by lane order, i.e. token order then ascending k.
  for (int tok = ws0; tok < ws1; tok += ctok) {
    const int nl = min(ctok, ws1 - tok) * K;
    const bool act = lane < nl;
    const int v = act ? pa.dst[(rowbase + tok) * K + lane] : 0;
    const int G = dst_row(v);
    const int u = G / NvS;
    const int row = G - u * NvS;
    const bool dup = act && v < 0;
    bool owner = false;
    for (int j = 1; j < K; ++j) {
      const int ua = __shfl(u, (lane + j) & (kWave - 1), kWave);
      if (act && !dup && j < K - k && ua == u) owner = true;
    }
    const uint64_t dpeers = match_key(__ballot(dup), u, d.rbits);
    const uint64_t gpeers = match_key(__ballot(owner), u, d.rbits);
    const int drank = __popcll(dpeers & lanes_below());
    const int grank = __popcll(gpeers & lanes_below());
    int didx = -1;
    if (dup) {
      didx = wc[(wave * R + u) * 2 + 1] + drank;
      pa.dup_loffs[(int64_t)u * NvS + didx] = row;
    }
    int first = -1, m = 0;
    for (int j = 1; j < K; ++j) {
      const int ua = __shfl(u, (lane + j) & (kWave - 1), kWave);
      const int da = __shfl(didx, (lane + j) & (kWave - 1), kWave);
      if (owner && j < K - k && ua == u) {
        if (first < 0) first = da;
        ++m;
      }
    }
    if (owner) {
      const int gidx = wc[(wave * R + u) * 2 + 0] + grank;
      int32_t* rec = pa.dup_groups + ((int64_t)u * NvS + gidx) * 3;
      rec[0] = row;
      rec[1] = first;
      rec[2] = m;
    }
    wave_lds_fence();
    if (dup && drank == 0) wc[(wave * R + u) * 2 + 1] += __popcll(dpeers);
    if (owner && grank == 0) wc[(wave * R + u) * 2 + 0] += __popcll(gpeers);
    wave_lds_fence();
  }
}

}  // namespace

hipError_t launch_plan(const Dims& d, const Scratch& sc, const PlanArrays& pa, const int32_t* topk,
                       const int32_t* tpe, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_hist, dim3(d.ntiles), dim3(kPlanThreads), 0, s, d, topk, sc.tile_cnt,
                     sc.tile_bad);
  hipLaunchKernelGGL(k_plan_balance, dim3(1), dim3(kPlanThreads), 0, s, d, tpe, sc, pa);
  hipLaunchKernelGGL(k_plan_place, dim3(d.ntiles), dim3(kPlanThreads), 0, s, d, topk, sc, pa);
  hipLaunchKernelGGL(k_plan_dups, dim3(d.ntiles), dim3(kPlanThreads), 0, s, d, sc, pa);
  return hipGetLastError();
}

}  // namespace moon
