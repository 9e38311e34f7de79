// moon_plan.hip — the online balancing planner for gfx950 (wave64).
//
// ("MoonEP Public API Visual Guide", Buffer.dispatch: the planner maps each
//  of a rank's S*K routes to a destination row, lays out E+B padded groups
//  and records which routes are duplicates; MoonEP README, Perfect balance
//  and How to set B: each rank ends with S*K routes, the excess going to
//  redundant-expert slots whose experts all come from one remote home rank.)
//
// Two launches on the caller's stream.  A tile is a token range of one
// source rank (at most one tile per compute unit, sized by a cost model on
// the host) and one workgroup of 16 waves; wave w owns a contiguous token
// range of its tile and walks it in chunks of whole tokens (floor(64/K)
// tokens), so a token's K routes sit in adjacent lanes.
//
//   k_plan_count    per tile: expert counts (LDS atomics) -> one column of
//                   the [E][tiles] count matrix.
//   k_plan_place    per tile, in LDS:
//                   - balance, recomputed by every tile from the count
//                     matrix (identical in all of them, so no tile waits for
//                     another): expert totals and the tile's own base (routes
//                     of each expert in earlier tiles), home stream offsets,
//                     the alias fill over the R rank loads (one wave, one lane
//                     per rank), then per rank its slots and the start rows of
//                     its padded groups; tile u also writes rank u's
//                     experts_to_copy (with each slot's owner rank and row,
//                     the prefetch index), remote_stats, cu_seqlens and
//                     zero_fill_ranges;
//                   - placement: stable rank of every route = tile base + wave
//                     prefix + running per-wave counter + rank inside the chunk
//                     (ballot match over the expert-id bits); stream position
//                     -> (destination rank, group, row); primary or duplicate
//                     by a ballot match over (token, destination rank); signed
//                     dst;
//                   - duplicate records: each tile publishes its duplicate
//                     counts per rank and reads those of the earlier tiles
//                     (never of later ones, so the wait always ends).
//
// The few words tiles pass to each other inside k_plan_place are relaxed
// atomics at agent scope carrying the call's tag in their high half: coherent
// across the XCDs' L2 caches without fences, and a reader waits for the tag.
// Bulk data crosses kernel boundaries only.  LDS atomics only add counts, so
// plans are bit-reproducible.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kBatch = 16;            // chunks a wave stages in LDS at once
static_assert(kMaxE <= kPlanThreads, "one thread per expert in the table passes");
static_assert(kMaxE / kPlanWaves <= 32, "checked expert groups form a 32-bit mask");
constexpr int kScanBatch = 8;         // experts whose tile counts a wave loads at once
constexpr int kTilesPerLane = kMaxTiles / kWave;
static_assert(kTilesPerLane == 4, "a lane holds four tiles of a count row (one 16-byte load)");
constexpr uint32_t kSpinLimit = 1u << 24;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index as a scalar, so ranges derived from it stay uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ uint64_t below_lane(int l) {
  return l <= 0 ? 0ull : ((~0ull) >> (kWave - l));
}

__device__ __forceinline__ uint64_t lanes_below() { return below_lane(lane_id()); }

__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, kWave - 1); }

__device__ __forceinline__ int wave_sum(int v) { return lane63(wave_incl_scan(v)); }

__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order the LDS traffic of one wave between consecutive chunks: the LDS
// executes a wave's operations in issue order, so it is enough to keep the
// compiler from moving them and to wait for the wave's own LDS operations
// (not for its global stores).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
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
    k_plan_count(Dims d, const int32_t* __restrict__ topk, Scratch sc, PlanArrays pa) {
  __shared__ int cnt[kMaxE];
  __shared__ int sBad;
  const int E = d.E;
  const int t = blockIdx.x;
  const TileRange tr = tile_range(d, t);
  for (int x = threadIdx.x; x < E; x += kPlanThreads) cnt[x] = 0;
  if (threadIdx.x == 0) sBad = 0;
  __syncthreads();
  const int64_t i0 = ((int64_t)tr.r * d.S + tr.s0) * d.K, i1 = ((int64_t)tr.r * d.S + tr.s1) * d.K;
  int bad = 0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 8 * kPlanThreads) {
    int e[8];
    bool in[8];  // the slot holds a route of the tile (every id value is checked)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      in[j] = i + j * kPlanThreads < i1;
      e[j] = in[j] ? topk[i + j * kPlanThreads] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!in[j]) continue;
      if ((unsigned)e[j] < (unsigned)E) atomicAdd(&cnt[e[j]], 1);
      else bad = 1;
    }
  }
  if (bad) atomicOr(&sBad, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPlanThreads) sc.tile_cnt[e * d.ntiles_pad + t] = cnt[e];
  if (threadIdx.x == 0) sc.tile_cnt[E * d.ntiles_pad + t] = sBad;
  // The scratch may hold an earlier call's data of another shape: the last
  // tile zeroes the padding columns of the count matrix (read in whole
  // 16-byte groups), and every tile resets its words of the duplicate-count
  // exchange to tag 0, which no call uses, so no word left by an earlier call
  // can pass for one of this call's.
  const int npad = d.ntiles_pad - d.ntiles;
  if (t == d.ntiles - 1)
    for (int x = threadIdx.x; x < (E + 1) * npad; x += kPlanThreads)
      sc.tile_cnt[(x / npad) * d.ntiles_pad + d.ntiles + x % npad] = 0;
  for (int u = threadIdx.x; u < d.R; u += kPlanThreads) sc.tile_agg[t * d.R + u] = 0;
  if (t == 0 && threadIdx.x == 0) {
    pa.status[0] = 0;  // k_plan_place ORs in what it finds
    uint32_t next = sc.epoch[0] + 1u;  // tag of this call's words in k_plan_place
    if ((next & 0xFFFFu) == 0u) next += 1u;  // tag 0 marks a reset word
    sc.epoch[0] = next;
  }
}

// ---------------------------------------------------------------------------
__device__ __forceinline__ int dst_row(int v) { return v >= 0 ? v : -v - 1; }

// v of the lane j places below (wave_shr) or above (wave_shl); `fill` where
// that lane does not exist.
__device__ __forceinline__ int from_below(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x138, 0xF, 0xF, false);  // wave_shr:1
}
__device__ __forceinline__ int from_above(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x130, 0xF, 0xF, false);  // wave_shl:1
}

// Lanes of `set` whose key equals this lane's (ballot per key bit), with the
// bit loop unrolled to a compile-time bound.
template <int kMaxBits>
__device__ __forceinline__ uint64_t match_bits(uint64_t set, int key, int bits) {
  uint64_t peers = set;
#pragma unroll
  for (int b = 0; b < kMaxBits; ++b) {
    if (b < bits) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
  }
  return peers;
}

struct PlanLds {
  int run[kPlanWaves * kMaxE];             // per-wave counts, then running positions
  int stage[kPlanWaves * kBatch * kWave];  // a wave's staged expert ids, then dst
  int T[kMaxE];     // routes of expert e over all source ranks
  int base[kMaxE];  // routes of e in tiles before this one
  int Pe[kMaxE];    // start of e in its home rank's stream
  int hst[kMaxE];   // start row of home group e on its owner
  int sst[kMaxE];   // [u*Eg + j]: start row of the slot group of receiver u that
                    // holds its donor's j-th expert, -1 if none
  int Lh[kMaxR], keep[kMaxR], donor[kMaxR], segA[kMaxR], segB[kMaxR];
  int recv[kMaxR], rfirst[kMaxR], rcnt[kMaxR];
  int wflags[kPlanWaves];
  int wc[kPlanWaves * kMaxR * 2];          // per-wave duplicate groups / rows per rank
  int baseD[kMaxR * 2], tot[kMaxR * 2];
  int flags;
};

// Status bits that leave the plan without a layout: every tile finds them
// from the same data, so all tiles stop together.
constexpr int kFatal = kBadExpert | kSlotBudget | kInternal;

// Duplicate groups and rows of tile-group word w for rank field x.
__device__ __forceinline__ int word_field(uint64_t w, int f) {
  return f == 0 ? (int)((w >> 24) & 0xFFFFFFu) : (int)(w & 0xFFFFFFu);
}

// Tile counts of a batch of experts e0, e0 + 16, ..: lane l holds tiles
// 4l..4l+3 (one 16-byte load).  Expert e = w + 16i is checked against the
// given histogram by wave w of the tiles t = i mod tiles (bit i of `chk`);
// there lanes r < R also fetch tokens_per_expert[r][e].
__device__ __forceinline__ void load_count_batch(const Dims& d, const Scratch& sc,
                                                 const int32_t* __restrict__ tpe, uint32_t chk,
                                                 int e0, int (&c)[kScanBatch][kTilesPerLane],
                                                 int (&given)[kScanBatch]) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) {
    const int e = e0 + j * kPlanWaves;
    int4 v = {0, 0, 0, 0};
    if (e < d.E && lane * 4 < d.ntiles)
      v = *reinterpret_cast<const int4*>(sc.tile_cnt + e * d.ntiles_pad + lane * 4);
    c[j][0] = v.x;
    c[j][1] = v.y;
    c[j][2] = v.z;
    c[j][3] = v.w;
    const bool want = e < d.E && ((chk >> (e / kPlanWaves)) & 1u) && lane < d.R;
    given[j] = want ? tpe[lane * d.E + e] : 0;
  }
}

// Expert totals and this tile's bases from a loaded batch; the checking tile
// compares each rank's count of e (a rank's tiles are consecutive) with the
// given histogram.  Returns status bits found.
__device__ __forceinline__ int reduce_count_batch(const Dims& d, PlanLds& L, uint32_t chk,
                                                  int e0, int t,
                                                  const int (&c)[kScanBatch][kTilesPerLane],
                                                  const int (&given)[kScanBatch]) {
  const int lane = lane_id();
  const int tl = t >> 2, sub_t = t & 3;
  int bits = 0;
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) {
    const int e = e0 + j * kPlanWaves;
    if (e >= d.E) break;
    const int sum4 = c[j][0] + c[j][1] + c[j][2] + c[j][3];
    const int incl = wave_incl_scan(sum4);
    const int ex0 = incl - sum4;  // routes of e in tiles before 4*lane
    const int part = (sub_t > 0 ? c[j][0] : 0) + (sub_t > 1 ? c[j][1] : 0) +
                     (sub_t > 2 ? c[j][2] : 0);
    const int bse = __builtin_amdgcn_readlane(ex0 + part, tl);
    const int total = lane63(incl);
    if (lane == 0) {
      L.T[e] = total;
      L.base[e] = bse;
    }
    if ((chk >> (e / kPlanWaves)) & 1u) {
      // Lane x <= R fetches the prefix at tile x * tiles_per_rank.
      const int tile = min(lane, d.R) * d.tiles_per_rank;
      const int src = min(tile / kTilesPerLane, kWave - 1), sub = tile % kTilesPerLane;
      const int v0 = __shfl(ex0, src, kWave);
      const int v1 = __shfl(ex0 + c[j][0], src, kWave);
      const int v2 = __shfl(ex0 + c[j][0] + c[j][1], src, kWave);
      const int v3 = __shfl(ex0 + c[j][0] + c[j][1] + c[j][2], src, kWave);
      int pre = sub == 0 ? v0 : sub == 1 ? v1 : sub == 2 ? v2 : v3;
      if (tile >= d.ntiles) pre = total;
      const int next = __shfl_down(pre, 1, kWave);
      if (__ballot(lane < d.R && next - pre != given[j])) bits |= kHistogram;
    }
  }
  return bits;
}

// The alias fill (one wave, lane = rank).  Under-loaded ranks, in ascending
// order, take what they lack from the lowest over-loaded rank; a donor pushed
// below S*K joins the back of the receiver queue.  Donors are used up in
// ascending order, so the appended receivers come after all initial ones and
// in ascending order too: both queues are bit masks.
__device__ __forceinline__ void alias_fill(const Dims& d, PlanLds& L) {
  const int lane = lane_id();
  const int R = d.R;
  const int C = d.S * d.K;
  int rem = lane < R ? L.Lh[lane] : C;
  int donor = -1, take = 0, off = 0, given = 0;
  int recv = 0, rfirst = 0, rcnt = 0;  // lane j: j-th receiver served; lane o: donor o's range
  uint64_t small = __ballot(rem < C), large = __ballot(rem > C), appended = 0;
  int served = 0;
  bool broken = false;
  while (small | appended) {
    int u;
    if (small) {
      u = __ffsll((unsigned long long)small) - 1;
      small &= small - 1;
    } else {
      u = __ffsll((unsigned long long)appended) - 1;
      appended &= appended - 1;
    }
    if (!large) {  // cannot happen: the loads sum to R*C
      broken = true;
      break;
    }
    const int o = __ffsll((unsigned long long)large) - 1;
    // u and o are uniform (taken from ballot masks): read their lanes directly
    const int f = C - __builtin_amdgcn_readlane(rem, u);
    const int g_o = __builtin_amdgcn_readlane(given, o);
    const int rem_o = __builtin_amdgcn_readlane(rem, o) - f;
    const int cnt_o = __builtin_amdgcn_readlane(rcnt, o);
    if (lane == u) {
      donor = o;
      take = f;
      off = g_o;
    }
    if (lane == o) {
      given = g_o + f;
      rem = rem_o;
      if (cnt_o == 0) rfirst = served;
      rcnt = cnt_o + 1;
    }
    if (lane == served) recv = u;
    ++served;
    if (rem_o < C) {
      large &= large - 1;
      appended |= 1ull << o;
    } else if (rem_o == C) {
      large &= large - 1;
    }
  }
  if (broken && lane == 0) atomicOr(&L.flags, kInternal);
  const int keep = rem;
  const int dk = __shfl(keep, donor < 0 ? 0 : donor, kWave);
  if (lane < R) {
    L.keep[lane] = keep;
    L.donor[lane] = donor;
    L.segA[lane] = donor >= 0 ? dk + off : 0;
    L.segB[lane] = donor >= 0 ? dk + off + take : 0;
    L.recv[lane] = recv;
    L.rfirst[lane] = rfirst;
    L.rcnt[lane] = rcnt;
  }
}

// Rank u's padded groups (one wave): its home experts u*Eg.. in ascending id,
// then its slots (the donor's experts overlapping its segment, ascending id,
// from slot 0).  Every other expert group of u is empty.  Start rows go to
// LDS; when `writer`, the rank's plan arrays are written as well.
__device__ __forceinline__ void rank_layout(const Dims& d, const PlanArrays& pa, PlanLds& L, int u,
                                            bool writer) {
  const int lane = lane_id();
  const int E = d.E, Eg = d.Eg, B = d.B, EB = d.EB, P = d.P;
  int32_t* cu = pa.cu + u * EB;
  int32_t* zfr = pa.zfr + u * EB * 2;
  int carry = 0;
  for (int j0 = 0; j0 < Eg; j0 += kWave) {
    const int j = j0 + lane, g = u * Eg + j;
    int n = 0;
    if (j < Eg) n = min(max(L.keep[u] - L.Pe[g], 0), L.T[g]);
    const int pad = n == 0 ? 0 : (n + P - 1) / P * P;
    const int incl = wave_incl_scan(pad);
    if (j < Eg) {
      const int end = carry + incl;
      L.hst[g] = end - pad;
      if (writer) {
        cu[g] = end;
        zfr[g * 2 + 0] = end - pad + n;
        zfr[g * 2 + 1] = end;
      }
    }
    carry += lane63(incl);
  }
  if (writer) {
    for (int g = lane; g < E; g += kWave) {
      if (g / Eg == u) continue;
      const int end = g < u * Eg ? 0 : carry;
      cu[g] = end;
      zfr[g * 2 + 0] = end;
      zfr[g * 2 + 1] = end;
    }
  }
  const int o = L.donor[u];
  int count = 0, routed = 0, bits = 0;
  for (int j0 = 0; j0 < Eg; j0 += kWave) {
    const int j = j0 + lane;
    bool piece = false;
    int len = 0;
    if (o >= 0 && j < Eg) {
      const int e = o * Eg + j;
      const int lo = max(L.Pe[e], L.segA[u]);
      const int hi = min(L.Pe[e] + L.T[e], L.segB[u]);
      piece = L.T[e] > 0 && lo < hi;
      len = hi - lo;
    }
    const uint64_t m = __ballot(piece);
    const int slot = count + __popcll(m & lanes_below());
    const bool kept = piece && slot < B;
    const int n = kept ? len : 0;
    const int pad = n == 0 ? 0 : (n + P - 1) / P * P;
    const int incl = wave_incl_scan(pad);
    const int end = carry + incl;
    if (j < Eg) L.sst[u * Eg + j] = kept ? end - pad : -1;
    if (writer && kept) {
      pa.etc[u * B + slot] = o * Eg + j;
      pa.pidx[(u * B + slot) * 2 + 0] = o;  // owner rank and row of the expert
      pa.pidx[(u * B + slot) * 2 + 1] = j;
      cu[E + slot] = end;
      zfr[(E + slot) * 2 + 0] = end - pad + n;
      zfr[(E + slot) * 2 + 1] = end;
    }
    if (__ballot(piece && !kept)) bits |= kSlotBudget;
    routed += n;
    count += __popcll(m);
    carry += lane63(incl);
  }
  if (bits && lane == 0) atomicOr(&L.flags, bits);
  if (writer) {
    routed = wave_sum(routed);
    const int used = min(count, B);
    for (int j = used + lane; j < B; j += kWave) {
      pa.etc[u * B + j] = -1;
      pa.pidx[(u * B + j) * 2 + 0] = -1;
      pa.pidx[(u * B + j) * 2 + 1] = -1;
      cu[E + j] = carry;
      zfr[(E + j) * 2 + 0] = carry;
      zfr[(E + j) * 2 + 1] = carry;
    }
    if (lane == 0) {
      pa.rstats[u * 2 + 0] = used;
      pa.rstats[u * 2 + 1] = routed;
    }
  }
}

// Publish zero duplicate counts for tile t (so that no later tile waits on
// it) and report the tile's status bits.
__device__ __forceinline__ void stop_tile(const Dims& d, const Scratch& sc, const PlanArrays& pa,
                                          uint32_t tag, int flags) {
  for (int u = threadIdx.x; u < d.R; u += kPlanThreads)
    __hip_atomic_store(sc.tile_agg + blockIdx.x * d.R + u, pack_word(tag, 0, 0), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0 && flags != 0) atomicOr(&pa.status[0], flags);
}

__device__ void place_tile(const Dims& d, const int32_t* __restrict__ topk,
                           const int32_t* __restrict__ tpe, const Scratch& sc,
                           const PlanArrays& pa, PlanLds& L, uint32_t tag) {
  const int lane = lane_id(), wave = wave_id();
  const int E = d.E, R = d.R, K = d.K, Eg = d.Eg, NvS = d.NvS, nt = d.ntiles;
  const int t = blockIdx.x;
  const TileRange tr = tile_range(d, t);
  int ws0, ws1;
  wave_tokens(tr, wave, ws0, ws1);
  const int64_t rowbase = (int64_t)tr.r * d.S;
  const int ctok = d.ctok;
  const int nchunks = (ws1 - ws0 + ctok - 1) / ctok;
  const int k = lane % K;
  int* st = L.stage + wave * kBatch * kWave;
  int* run = L.run + wave * E;
  int* wc = L.wc + wave * R * 2;
  const bool staged = nchunks <= kBatch;

  // ---- This wave's first batch of routes, the first batch of its experts'
  // tile counts and (wave 0) the out-of-range flags of all tiles: all loads
  // in flight together.
  int tc[kScanBatch][kTilesPerLane], given[kScanBatch];
  int wbits = 0;
  // Groups of 16 experts this tile checks against the given histogram.
  uint32_t chk = 0;
  if (tpe != nullptr)
    for (int i = t; i < kMaxE / kPlanWaves; i += nt) chk |= 1u << i;
  {
    int v[kBatch];
#pragma unroll
    for (int cc = 0; cc < kBatch; ++cc) {
      const int tok = ws0 + cc * ctok;
      const int nl = (cc < nchunks) ? min(ctok, ws1 - tok) * K : 0;
      v[cc] = lane < nl ? topk[(rowbase + tok) * K + lane] : -1;
    }
    load_count_batch(d, sc, tpe, chk, wave, tc, given);
    int4 bad = {0, 0, 0, 0};
    if (wave == 0 && lane * 4 < nt)
      bad = *reinterpret_cast<const int4*>(sc.tile_cnt + E * d.ntiles_pad + lane * 4);
    // The wave's own LDS regions: no other wave touches them before the
    // next barrier.
    for (int x = lane; x < E; x += kWave) run[x] = 0;
    for (int x = lane; x < R * 2; x += kWave) wc[x] = 0;
#pragma unroll
    for (int cc = 0; cc < kBatch; ++cc) st[cc * kWave + lane] = v[cc];
    if (__ballot((bad.x | bad.y | bad.z | bad.w) != 0)) wbits |= kBadExpert;
  }
  // Per-wave expert counts of the tile (recounted from the routes).
  wave_lds_fence();
  // (separate loops for LDS and global reads: a read through a pointer to
  // either becomes a flat load, which waits for every outstanding access)
  if (staged) {
    for (int cc = 0; cc < nchunks; ++cc) {
      const int e = st[cc * kWave + lane];
      if ((unsigned)e < (unsigned)E) atomicAdd(&run[e], 1);
    }
  } else {
    for (int cc = 0; cc < nchunks; ++cc) {
      const int tok = ws0 + cc * ctok;
      const int nl = min(ctok, ws1 - tok) * K;
      const int e = lane < nl ? topk[(rowbase + tok) * K + lane] : -1;
      if ((unsigned)e < (unsigned)E) atomicAdd(&run[e], 1);
    }
  }
  // Expert totals and this tile's bases.
  for (int e0 = wave; e0 < E; e0 += kScanBatch * kPlanWaves) {
    if (e0 != wave) load_count_batch(d, sc, tpe, chk, e0, tc, given);
    wbits |= reduce_count_batch(d, L, chk, e0, t, tc, given);
  }
  if (lane == 0) L.wflags[wave] = wbits;
  __syncthreads();

  // ---- Running positions = tile base + counts of earlier waves; home stream
  // offsets (home rank h's stream is its experts in ascending id).
  if (threadIdx.x == 0) {
    int f = 0;
    for (int w = 0; w < kPlanWaves; ++w) f |= L.wflags[w];
    L.flags = f;
  }
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    int acc = L.base[e];
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int cnt = L.run[w * E + e];
      L.run[w * E + e] = acc;
      acc += cnt;
    }
  }
  for (int h = wave; h < R; h += kPlanWaves) {
    int carry = 0;
    for (int j0 = 0; j0 < Eg; j0 += kWave) {
      const int j = j0 + lane;
      const int v = j < Eg ? L.T[h * Eg + j] : 0;
      const int incl = wave_incl_scan(v);
      if (j < Eg) L.Pe[h * Eg + j] = carry + incl - v;
      carry += lane63(incl);
    }
    if (lane == 0) L.Lh[h] = carry;
  }
  __syncthreads();
  if (L.flags & kBadExpert) {
    stop_tile(d, sc, pa, tag, L.flags);
    return;
  }

  // ---- Balance and layout.
  if (wave == 0) alias_fill(d, L);
  __syncthreads();
  for (int u = wave; u < R; u += kPlanWaves) rank_layout(d, pa, L, u, t == u);
  __syncthreads();
  if (L.flags & kFatal) {
    stop_tile(d, sc, pa, tag, L.flags);
    return;
  }

  // ---- Placement.
  for (int b0 = 0; b0 < nchunks; b0 += kBatch) {
    if (b0 > 0) {  // later batches (long wave ranges only)
      int v[kBatch];
#pragma unroll
      for (int c = 0; c < kBatch; ++c) {
        const int tok = ws0 + (b0 + c) * ctok;
        const int nl = (b0 + c < nchunks) ? min(ctok, ws1 - tok) * K : 0;
        v[c] = lane < nl ? topk[(rowbase + tok) * K + lane] : -1;
      }
#pragma unroll
      for (int c = 0; c < kBatch; ++c) st[c * kWave + lane] = v[c];
    }
    const int cend = min(kBatch, nchunks - b0);
    for (int c = 0; c < cend; ++c) {
      const int tok = ws0 + (b0 + c) * ctok;
      const int e = st[c * kWave + lane];
      const bool act = e >= 0;
      const uint64_t peers = match_bits<10>(__ballot(act), act ? e : 0, d.ebits);
      const int rank = __popcll(peers & lanes_below());
      int u = -1, G = 0;
      if (act) {
        const int pos = run[e] + rank;  // position among e's routes
        const int h = e / Eg;
        const int q = L.Pe[e] + pos;    // position in h's stream
        int start, idx;
        if (q < L.keep[h]) {
          u = h;
          start = L.hst[e];
          idx = q - L.Pe[e];
        } else {
          const int f0 = L.rfirst[h], nr = L.rcnt[h];
          for (int j = 0; j < nr; ++j) {
            const int v = L.recv[f0 + j];
            if (q < L.segB[v]) {
              u = v;
              break;
            }
          }
          const int s0 = u >= 0 ? L.sst[u * Eg + (e - h * Eg)] : -1;
          if (s0 < 0) {  // cannot happen for a consistent plan
            atomicOr(&L.flags, kInternal);
            u = 0;
            start = 0;
            idx = 0;
          } else {
            start = s0;
            idx = q - max(L.Pe[e], L.segA[u]);
          }
        }
        G = u * NvS + start + idx;
      }
      wave_lds_fence();
      if (act && rank == 0) run[e] += __popcll(peers);
      // Primary = first route of its token to its destination rank; lanes
      // j places away hold routes of the same token when j <= k (below) or
      // j < K - k (above).
      bool dup = false, later = false;
      int sb = u, sa = u;
      for (int j = 1; j < K; ++j) {
        sb = from_below(sb, -1);
        sa = from_above(sa, -1);
        if (j <= k && sb == u) dup = true;
        if (j < K - k && sa == u) later = true;
      }
      dup = dup && act;
      const bool owner = act && !dup && later;
      const int v = dup ? -(G + 1) : G;
      if (act) pa.dst[(rowbase + tok) * K + lane] = v;
      st[c * kWave + lane] = act ? v : INT32_MIN;
      const int uk = act ? u : 0;
      const uint64_t gpeers = match_bits<5>(__ballot(owner), uk, d.rbits);
      const uint64_t dpeers = match_bits<5>(__ballot(dup), uk, d.rbits);
      if (owner && (gpeers & lanes_below()) == 0) wc[uk * 2 + 0] += __popcll(gpeers);
      if (dup && (dpeers & lanes_below()) == 0) wc[uk * 2 + 1] += __popcll(dpeers);
      wave_lds_fence();
    }
  }
  __syncthreads();

  // ---- Per-rank duplicate counts: wave prefixes and the tile's totals.
  for (int x = threadIdx.x; x < R * 2; x += kPlanThreads) {
    int acc = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = L.wc[w * R * 2 + x];
      L.wc[w * R * 2 + x] = acc;
      acc += c;
    }
    L.tot[x] = acc;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < R; u += kPlanThreads)
    __hip_atomic_store(sc.tile_agg + t * R + u, pack_word(tag, L.tot[u * 2], L.tot[u * 2 + 1]),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- Counts of earlier tiles: for each rank, lane l reads tiles l,
  // l+64, .. below this one (one packed word each, all in flight together).
  // Every wait is on a lower tile, which publishes before it waits; the
  // hardware starts workgroups in index order, so a lower tile is already
  // running or done when a higher one waits for it, even when other kernels
  // share the device.
  bool timeout = false;
  const uint32_t tag16 = tag & 0xFFFFu;
  for (int u = wave; u < R; u += kPlanWaves) {
    uint64_t w[kTilesPerLane];
#pragma unroll
    for (int j = 0; j < kTilesPerLane; ++j) {
      const int tp = j * kWave + lane;
      w[j] = tp < t ? get_word(sc.tile_agg + tp * R + u) : pack_word(tag, 0, 0);
    }
    int sg = 0, sd = 0;
#pragma unroll
    for (int j = 0; j < kTilesPerLane; ++j) {
      const int tp = j * kWave + lane;
      uint32_t spins = 0;
      while ((uint32_t)(w[j] >> 48) != tag16) {
        if (++spins > kSpinLimit) {
          timeout = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w[j] = get_word(sc.tile_agg + tp * R + u);
      }
      sg += word_field(w[j], 0);
      sd += word_field(w[j], 1);
    }
    sg = wave_sum(sg);
    sd = wave_sum(sd);
    if (lane == 0) {
      L.baseD[u * 2 + 0] = sg;
      L.baseD[u * 2 + 1] = sd;
    }
  }
  if (timeout) atomicOr(&L.flags, kInternal);
  __syncthreads();
  if (threadIdx.x == 0 && L.flags != 0) atomicOr(&pa.status[0], L.flags);
  if (L.flags & kFatal) return;
  for (int x = threadIdx.x; x < kPlanWaves * R * 2; x += kPlanThreads)
    L.wc[x] += L.baseD[x % (R * 2)];
  if (t == nt - 1)
    for (int x = threadIdx.x; x < R * 2; x += kPlanThreads)
      pa.dup_counts[x] = L.baseD[x] + L.tot[x];
  __syncthreads();

  // ---- Duplicate records.  Owners (first route of a token to a rank that
  // has later routes there) and duplicates of one rank are ranked by lane
  // order, i.e. token order then ascending k.
  for (int c = 0; c < nchunks; ++c) {
    const int tok = ws0 + c * ctok;
    const int nl = min(ctok, ws1 - tok) * K;
    const bool act = lane < nl;
    int v = 0;
    if (staged) {  // (two reads, not one through a selected pointer: see above)
      if (act) v = st[c * kWave + lane];
    } else {
      if (act) v = pa.dst[(rowbase + tok) * K + lane];
    }
    const int G = dst_row(v);
    const int u = act ? G / NvS : -1;
    const int uk = act ? u : 0;
    const int row = G - uk * NvS;
    const bool dup = act && v < 0;
    const uint64_t dpeers = match_bits<5>(__ballot(dup), uk, d.rbits);
    const int didx = dup ? wc[uk * 2 + 1] + __popcll(dpeers & lanes_below()) : -1;
    // later routes of the same token to the same rank: count and first index
    bool owner_cand = act && !dup;
    int m = 0, first = -1, sa = u, da = didx;
    for (int j = 1; j < K; ++j) {
      sa = from_above(sa, -1);
      da = from_above(da, -1);
      if (j < K - k && sa == u && owner_cand) {
        if (first < 0) first = da;
        ++m;
      }
    }
    const bool owner = owner_cand && m > 0;
    const uint64_t gpeers = match_bits<5>(__ballot(owner), uk, d.rbits);
    if (dup) pa.dup_loffs[(int64_t)uk * NvS + didx] = row;
    if (owner) {
      const int gidx = wc[uk * 2 + 0] + __popcll(gpeers & lanes_below());
      int32_t* rec = pa.dup_groups + ((int64_t)uk * NvS + gidx) * 3;
      rec[0] = row;
      rec[1] = first;
      rec[2] = m;
    }
    wave_lds_fence();
    if (dup && (dpeers & lanes_below()) == 0) wc[uk * 2 + 1] += __popcll(dpeers);
    if (owner && (gpeers & lanes_below()) == 0) wc[uk * 2 + 0] += __popcll(gpeers);
    wave_lds_fence();
  }
}

__global__ void __launch_bounds__(kPlanThreads)
    k_plan_place(Dims d, const int32_t* __restrict__ topk, const int32_t* __restrict__ tpe,
                 Scratch sc, PlanArrays pa) {
  __shared__ PlanLds L;
  place_tile(d, topk, tpe, sc, pa, L, sc.epoch[0]);
}

}  // namespace

hipError_t launch_plan(const Dims& d, const Scratch& sc, const PlanArrays& pa, const int32_t* topk,
                       const int32_t* tpe, hipStream_t s) {
  hipLaunchKernelGGL(k_plan_count, dim3(d.ntiles), dim3(kPlanThreads), 0, s, d, topk, sc, pa);
  hipLaunchKernelGGL(k_plan_place, dim3(d.ntiles), dim3(kPlanThreads), 0, s, d, topk, tpe, sc, pa);
  return hipGetLastError();
}

}  // namespace moon
