// moon_oracle.cpp — plain CPU oracle (test infrastructure only; see header).
//
// Every step is written the slow, obvious way, in the order the pages give:
//   planning  = histogram -> per-home-rank streams -> balance -> slots ->
//               padded layout -> placement -> dedup + dst + duplicate records
//   ("MoonEP Public API Visual Guide", section Buffer.dispatch, high-level
//    description of planning; section MoonEPCommPlan, field table)
//   dispatch  = copy every route's token row to its physical row, every route
//               weight to its row, zero the padding (same page, Buffer.dispatch)
//   combine   = per token, sum the K routed rows (weighted or not) back into
//               token-major order (same page, Buffer.combine)
//   prefetch  = split a slot's expert id into (owner rank, local row) and
//               copy that expert's weight rows into the slot
//               (same page, Buffer.prefetch_weight)
//   reduce    = add every slot gradient back into its expert's gradient row
//               and clear the consumed slots (same page, Buffer.reduce_grad)
// Arithmetic on values happens in combine (float32, ascending k, with an
// optional float64 counterpart as the exact reference) and in the gradient
// reduction (float32, as the pages' gradient tensors are).

#include "moon_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <deque>
#include <vector>

namespace {

const int32_t ST_OK = 0, ST_INVALID = -1, ST_BAD_EXPERT = -7, ST_SLOT_BUDGET = -8,
              ST_HISTOGRAM = -9;

int64_t round_up(int64_t n, int64_t p) { return (n + p - 1) / p * p; }

// Padded size of a group: non-empty groups are padded to a multiple of the
// token padding; empty groups stay empty (Visual Guide, Buffer(...): the
// token padding is the row alignment of groups that hold a route).
int64_t padded(int64_t n, int64_t p) { return n == 0 ? 0 : round_up(n, p); }

float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Physical row of a route from its signed dst entry.
int64_t decode_row(int32_t d) { return d >= 0 ? (int64_t)d : -(int64_t)d - 1; }

// One token: sum its K routed rows in ascending k, optionally scaled by the
// route weight stored at the route's own row (Visual Guide, Buffer.combine:
// each token's K contributions are reduced back into its row; the weights are
// read back through the signed dst entries, both signs alike).  The pages
// state fp32 accumulation for the duplicate prologue's fold; the main K-sum
// is held to the same fp32 precision as the target stated for this path, and
// its order and rounding are a reading: `out` is the fp32 sum -- each product
// and each addition rounded to fp32 in turn, ascending k -- rounded once to
// bf16.  When `acc` is given it receives the float64 sum of the same terms,
// the exact reference (the fp32 result does not depend on it).
template <class RowFn, class WFn>
void combine_token(int32_t K, int32_t H, const int32_t* d, RowFn row, WFn wat, int32_t weighted,
                   uint16_t* out, float* wsk, double* acc) {
  std::vector<float> sum32(H, 0.0f);
  std::vector<double> sum(acc != nullptr ? H : 0, 0.0);
  for (int k = 0; k < K; ++k) {
    int64_t G = decode_row(d[k]);
    const uint16_t* y = row(G);
    float wk = wat(G);
    float c32 = weighted ? wk : 1.0f;
    double c = (double)c32;
    for (int h = 0; h < H; ++h) {
      float yv = bf16_to_float(y[h]);
      float prod = c32 * yv;
      sum32[h] = sum32[h] + prod;
    }
    if (acc != nullptr)
      for (int h = 0; h < H; ++h) sum[h] += c * (double)bf16_to_float(y[h]);
    if (wsk != nullptr) wsk[k] = wk;
  }
  for (int h = 0; h < H; ++h) {
    out[h] = orc_bf16_from_double((double)sum32[h]);
    if (acc != nullptr) acc[h] = sum[h];
  }
}


// Combine with a duplicate prologue (Visual Guide, Buffer.combine: before the
// gather, the rows of a token's duplicate routes on one destination rank are
// summed into that rank's primary row in fp32; the gather then reads primary
// rows only).  Per token and destination rank with m >= 2 routes, the folded
// row is bf16(sum over those routes, ascending k, of c_k * y) with the fp32
// arithmetic the pages fix (separate multiply and add); it stands for all m
// routes with coefficient 1.  The outer sum over primaries, ascending k, is
// fp32 as in the plain combine (`out`), with its float64 counterpart in
// `acc`.  `fold(G, bits)` receives every folded primary row.
template <class RowFn, class WFn, class FoldFn>
void combine_token_prologue(int32_t K, int32_t H, int64_t NvS, const int32_t* d, RowFn row, WFn wat,
                            int32_t weighted, uint16_t* out, float* wsk, double* acc, FoldFn fold) {
  std::vector<double> sum(H, 0.0);
  std::vector<float> sum32(H, 0.0f);
  std::vector<float> part(H);
  std::vector<uint16_t> bits(H);
  for (int k = 0; k < K; ++k) {
    int64_t G = decode_row(d[k]);
    if (wsk != nullptr) wsk[k] = wat(G);
    if (d[k] < 0) continue;  // a duplicate: folded into its primary below
    std::vector<int> members{k};
    for (int k2 = k + 1; k2 < K; ++k2)
      if (d[k2] < 0 && decode_row(d[k2]) / NvS == G / NvS) members.push_back(k2);
    if (members.size() == 1) {
      float c32 = weighted ? wat(G) : 1.0f;
      const uint16_t* y = row(G);
      for (int h = 0; h < H; ++h) {
        float yv = bf16_to_float(y[h]);
        float prod = c32 * yv;
        sum32[h] = sum32[h] + prod;
        sum[h] += (double)c32 * (double)yv;
      }
      continue;
    }
    std::fill(part.begin(), part.end(), 0.0f);
    for (int m : members) {
      int64_t Gm = decode_row(d[m]);
      float c = weighted ? wat(Gm) : 1.0f;
      const uint16_t* y = row(Gm);
      for (int h = 0; h < H; ++h) {
        float prod = c * bf16_to_float(y[h]);
        part[h] = part[h] + prod;
      }
    }
    for (int h = 0; h < H; ++h) {
      bits[h] = orc_bf16_from_double((double)part[h]);
      float yv = bf16_to_float(bits[h]);
      float prod = 1.0f * yv;
      sum32[h] = sum32[h] + prod;
      sum[h] += (double)yv;
    }
    fold(G, bits.data());
  }
  for (int h = 0; h < H; ++h) {
    out[h] = orc_bf16_from_double((double)sum32[h]);
    if (acc != nullptr) acc[h] = sum[h];
  }
}

}  // namespace

extern "C" {

// Capacity.  The pages define NvS as room for the S*K routes plus the
// padding of every group (README, Integration notation), without a formula.  A rank holds at most Eg
// home groups and at most B slot groups, and padding adds fewer than P rows to
// each non-empty group, so S*K + (Eg+B)*(P-1) rounded up to P always suffices.
int32_t orc_nvs(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B, int32_t P) {
  if (R <= 0 || E <= 0 || E % R != 0 || K <= 0 || S <= 0 || B < 0 || P <= 0) return ST_INVALID;
  int64_t Eg = E / R;
  int64_t v = round_up((int64_t)S * K + (Eg + B) * (int64_t)(P - 1), P);
  if (v > INT32_MAX) return ST_INVALID;
  return (int32_t)v;
}

// Balance (reading): every rank must end with exactly C routes (README,
// Perfect balance), and the overflow a rank takes in must all come from a
// single other rank's home experts, so it needs at most E/R slots (README,
// How to set B).
// Under-loaded ranks are served in ascending rank order from the lowest
// over-loaded rank; a rank keeps its own routes first (home-first); a donor
// pushed below C becomes a receiver itself and joins the back of the queue.
// This is the Walker/Vose alias-table construction applied to integer loads.
// `served` receives the receivers in the order they were served.
static int32_t alias_core(int32_t R, int64_t C, const int64_t* L, int64_t* keep,
                          int32_t* donor, int64_t* take, std::vector<int>* served) {
  if (R <= 0 || C < 0) return ST_INVALID;
  int64_t total = 0;
  for (int h = 0; h < R; ++h) {
    if (L[h] < 0) return ST_INVALID;
    total += L[h];
  }
  if (total != (int64_t)R * C) return ST_INVALID;

  std::vector<int64_t> rem(L, L + R);
  std::deque<int> small, large;
  for (int h = 0; h < R; ++h) {
    donor[h] = -1;
    take[h] = 0;
    if (rem[h] < C) small.push_back(h);
    if (rem[h] > C) large.push_back(h);
  }
  while (!small.empty()) {
    int u = small.front();
    small.pop_front();
    if (large.empty()) return ST_INVALID;  // cannot happen when sum(L) == R*C
    int o = large.front();
    int64_t f = C - rem[u];  // u keeps all it still has and takes the rest from o
    donor[u] = o;
    take[u] = f;
    if (served != nullptr) served->push_back(u);
    rem[o] -= f;
    if (rem[o] < C) {
      large.pop_front();
      small.push_back(o);
    } else if (rem[o] == C) {
      large.pop_front();
    }
  }
  for (int h = 0; h < R; ++h) keep[h] = rem[h];
  return ST_OK;
}

int32_t orc_alias(int32_t R, int64_t C, const int64_t* L, int64_t* keep, int32_t* donor,
                  int64_t* take) {
  return alias_core(R, C, L, keep, donor, take, nullptr);
}

int32_t orc_plan(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B, int32_t P,
                 const int32_t* topk, const int32_t* tpe, int32_t* dst, int32_t* etc,
                 int32_t* zfr, int32_t* rstats, int32_t* dup_groups, int32_t* dup_loffs,
                 int32_t* dup_counts, int32_t* cu, int64_t* dbg) {
  const int32_t NvS = orc_nvs(R, E, K, S, B, P);
  if (NvS < 0) return ST_INVALID;
  const int Eg = E / R;
  const int EB = E + B;
  const int64_t C = (int64_t)S * K;
  const int64_t NR = (int64_t)R * S * K;  // all routes, global order (r, s, k)

  // ---- Histogram: routes per (source rank, expert) and per expert.
  // (Visual Guide, dispatch table: the planner's input tokens_per_expert is
  //  this count per source rank.)  Ids outside [0, E) are an error: the
  // planner has no sentinel id.
  std::vector<int64_t> cnt((size_t)R * E, 0), T(E, 0);
  for (int64_t i = 0; i < NR; ++i) {
    int32_t e = topk[i];
    if (e < 0 || e >= E) return ST_BAD_EXPERT;
    int64_t r = i / C;
    cnt[r * E + e] += 1;
    T[e] += 1;
  }
  if (tpe != nullptr) {
    for (int64_t j = 0; j < (int64_t)R * E; ++j)
      if ((int64_t)tpe[j] != cnt[j]) return ST_HISTOGRAM;
  }

  // ---- Streams.  The routes of expert e, in global route order, get
  // positions 0..T[e]-1.  A home rank's stream is its experts in ascending id,
  // each expert's routes in global order; Pe[e] is where e starts in it.
  std::vector<int64_t> pos(NR), seen(E, 0), Pe(E, 0), L(R, 0);
  for (int64_t i = 0; i < NR; ++i) pos[i] = seen[topk[i]]++;
  for (int h = 0; h < R; ++h) {
    int64_t acc = 0;
    for (int e = h * Eg; e < (h + 1) * Eg; ++e) {
      Pe[e] = acc;
      acc += T[e];
    }
    L[h] = acc;
  }

  // ---- Balance.
  std::vector<int64_t> keep(R), take(R);
  std::vector<int32_t> donor(R);
  std::vector<int> served;
  if (alias_core(R, C, L.data(), keep.data(), donor.data(), take.data(), &served) != ST_OK)
    return ST_INVALID;
  // A donor's stream: [0, keep) stays home, then one segment per receiver in
  // the order the receivers were served.
  std::vector<int64_t> seg_a(R, 0), seg_b(R, 0), next_a(keep);
  for (int u : served) {
    int o = donor[u];
    seg_a[u] = next_a[o];
    seg_b[u] = next_a[o] + take[u];
    next_a[o] += take[u];
  }

  // ---- Pieces and slots.  A receiver's pieces are the donor's experts that
  // overlap its segment, in ascending expert id; slot j holds the j-th piece
  // (Visual Guide, prefetch_weight: experts_to_copy maps a slot to a global
  // expert, -1 = unused).  n[u][g] = routes in group g of rank u.
  std::vector<int64_t> n((size_t)R * EB, 0);
  std::vector<int32_t> slot_of((size_t)R * E, -1);  // (receiver, expert) -> slot
  bool over_budget = false;
  for (int u = 0; u < R; ++u) {
    for (int j = 0; j < B; ++j) etc[(size_t)u * B + j] = -1;
    if (donor[u] < 0) continue;
    int o = donor[u];
    int j = 0;
    for (int e = o * Eg; e < (o + 1) * Eg; ++e) {
      int64_t lo = std::max(Pe[e], seg_a[u]);
      int64_t hi = std::min(Pe[e] + T[e], seg_b[u]);
      if (T[e] > 0 && lo < hi) {
        if (j >= B) {
          over_budget = true;
        } else {
          etc[(size_t)u * B + j] = e;
          n[(size_t)u * EB + E + j] = hi - lo;
          slot_of[(size_t)u * E + e] = j;
        }
        ++j;
      }
    }
  }
  if (over_budget) return ST_SLOT_BUDGET;
  for (int h = 0; h < R; ++h)
    for (int e = h * Eg; e < (h + 1) * Eg; ++e)
      n[(size_t)h * EB + e] = std::min(std::max(keep[h] - Pe[e], (int64_t)0), T[e]);
  for (int u = 0; u < R; ++u) {
    int64_t used = 0, routed = 0;
    for (int j = 0; j < B; ++j)
      if (etc[(size_t)u * B + j] >= 0) {
        used += 1;
        routed += n[(size_t)u * EB + E + j];
      }
    rstats[u * 2 + 0] = (int32_t)used;
    rstats[u * 2 + 1] = (int32_t)routed;
  }

  // ---- Layout: cu holds inclusive padded end offsets of the E+B groups
  // (Visual Guide, dispatch tensor table: cu_seqlens holds the padded end of
  // every group); zero_fill_ranges is the padding tail [start+n, end) of each.
  std::vector<int64_t> start((size_t)R * EB, 0);
  for (int u = 0; u < R; ++u) {
    int64_t acc = 0;
    for (int g = 0; g < EB; ++g) {
      size_t ug = (size_t)u * EB + g;
      start[ug] = acc;
      acc += padded(n[ug], P);
      cu[ug] = (int32_t)acc;
      zfr[ug * 2 + 0] = (int32_t)(start[ug] + n[ug]);
      zfr[ug * 2 + 1] = (int32_t)acc;
    }
    if (acc > NvS) return ST_INVALID;  // cannot happen: capacity bound
  }

  // ---- Placement: stream position q of a route decides rank, group, index.
  std::vector<int64_t> G(NR);
  for (int64_t i = 0; i < NR; ++i) {
    int e = topk[i];
    int h = e / Eg;
    int64_t q = Pe[e] + pos[i];
    int u = -1, g = -1;
    int64_t idx = -1;
    if (q < keep[h]) {
      u = h;
      g = e;
      idx = q - Pe[e];
    } else {
      for (int v = 0; v < R; ++v)
        if (donor[v] == h && seg_a[v] <= q && q < seg_b[v]) u = v;
      if (u < 0) return ST_INVALID;  // cannot happen
      g = E + slot_of[(size_t)u * E + e];
      idx = q - std::max(Pe[e], seg_a[u]);
    }
    G[i] = (int64_t)u * NvS + start[(size_t)u * EB + g] + idx;
  }

  // ---- Dedup and dst.  Within a token, the first route (lowest k) to each
  // destination rank is the primary and carries the row copy; later routes of
  // the same token to the same rank are local duplicates (Visual Guide,
  // Buffer.dispatch: one row copy per destination rank, duplicates filled on
  // the receiving rank afterwards; Buffer.combine: the sign of a dst entry
  // tells the two kinds apart).
  for (int64_t t = 0; t < (int64_t)R * S; ++t) {
    for (int k = 0; k < K; ++k) {
      int64_t i = t * K + k;
      int64_t u = G[i] / NvS;
      bool dup = false;
      for (int k2 = 0; k2 < k; ++k2)
        if (G[t * K + k2] / NvS == u) dup = true;
      dst[i] = dup ? (int32_t)(-(G[i] + 1)) : (int32_t)G[i];
    }
  }
  // Duplicate records per destination rank, tokens in global order.
  for (int u = 0; u < R; ++u) {
    int64_t ng = 0, nd = 0;
    for (int64_t t = 0; t < (int64_t)R * S; ++t) {
      int64_t prim = -1, m = 0;
      for (int k = 0; k < K; ++k) {
        int64_t i = t * K + k;
        if (G[i] / NvS != u) continue;
        if (dst[i] >= 0) prim = G[i] - (int64_t)u * NvS;
        else ++m;
      }
      if (m == 0) continue;
      int32_t* rec = dup_groups + ((size_t)u * NvS + ng) * 3;
      rec[0] = (int32_t)prim;
      rec[1] = (int32_t)nd;
      rec[2] = (int32_t)m;
      for (int k = 0; k < K; ++k) {
        int64_t i = t * K + k;
        if (G[i] / NvS == u && dst[i] < 0)
          dup_loffs[(size_t)u * NvS + nd++] = (int32_t)(G[i] - (int64_t)u * NvS);
      }
      ++ng;
    }
    dup_counts[u * 2 + 0] = (int32_t)ng;
    dup_counts[u * 2 + 1] = (int32_t)nd;
  }

  if (dbg != nullptr) {
    int64_t* p = dbg;
    for (int64_t j = 0; j < (int64_t)R * E; ++j) *p++ = cnt[j];
    for (int e = 0; e < E; ++e) *p++ = T[e];
    for (int e = 0; e < E; ++e) *p++ = Pe[e];
    for (int h = 0; h < R; ++h) *p++ = L[h];
    for (int h = 0; h < R; ++h) *p++ = keep[h];
    for (int h = 0; h < R; ++h) *p++ = donor[h];
    for (int h = 0; h < R; ++h) *p++ = take[h];
    for (int h = 0; h < R; ++h) *p++ = seg_a[h];
  }
  return ST_OK;
}


int32_t orc_dispatch(int32_t R, int32_t E, int32_t K, int32_t S, int32_t H, int32_t B,
                     int32_t NvS, const int32_t* dst, const int32_t* zfr,
                     const uint16_t* hidden, const float* w, uint16_t* win, float* wwin) {
  const int EB = E + B;
  for (int64_t t = 0; t < (int64_t)R * S; ++t) {
    for (int k = 0; k < K; ++k) {
      int64_t G = decode_row(dst[t * K + k]);
      if (H > 0) std::memcpy(win + G * H, hidden + t * H, (size_t)H * 2);
      if (w != nullptr) wwin[G] = w[t * K + k];
    }
  }
  for (int u = 0; u < R; ++u)
    for (int g = 0; g < EB; ++g) {
      const int32_t* zr = zfr + ((size_t)u * EB + g) * 2;
      for (int64_t row = zr[0]; row < zr[1]; ++row) {
        int64_t G = (int64_t)u * NvS + row;
        if (H > 0) std::memset(win + G * H, 0, (size_t)H * 2);
        if (w != nullptr) wwin[G] = 0.0f;
      }
    }
  return ST_OK;
}

int32_t orc_row_sources(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B, int32_t NvS,
                        const int32_t* dst, const int32_t* zfr, const int32_t* cu,
                        int64_t* src) {
  (void)cu;
  const int EB = E + B;
  for (int64_t j = 0; j < (int64_t)R * NvS; ++j) src[j] = -2;
  for (int u = 0; u < R; ++u)
    for (int g = 0; g < EB; ++g) {
      const int32_t* zr = zfr + ((size_t)u * EB + g) * 2;
      for (int64_t row = zr[0]; row < zr[1]; ++row) src[(int64_t)u * NvS + row] = -1;
    }
  for (int64_t i = 0; i < (int64_t)R * S * K; ++i) src[decode_row(dst[i])] = i;
  return ST_OK;
}

// Nearest bf16 of a double, ties to even, by exact scaling: bf16 keeps 8
// significant bits for normal numbers and a fixed quantum of 2^-133 below
// 2^-126.  Overflow past the largest finite bf16 gives infinity; any NaN gives
// the quiet NaN 0x7FC0 (a reading: the pages say nothing of non-finite values).
uint16_t orc_bf16_from_double(double v) {
  if (std::isnan(v)) return 0x7FC0;
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
  int ex;
  std::frexp(v, &ex);  // |v| = m * 2^ex, 0.5 <= m < 1
  int qexp = std::max(ex, -125) - 8;
  double scaled = std::ldexp(v, -qexp);  // exact: power-of-two scaling
  double r = std::nearbyint(scaled);     // default rounding mode: ties to even
  double res = std::ldexp(r, qexp);
  float f = (float)res;                  // exact unless it overflows
  if (std::fabs(res) >= 0x1.0p128 || std::isinf(f)) return res > 0 ? 0x7F80 : 0xFF80;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int32_t orc_combine(int32_t R, int32_t K, int32_t S, int32_t H, int32_t NvS,
                    const int32_t* dst, const uint16_t* y, const float* wnvs,
                    int32_t weighted, uint16_t* out, float* wsk_out, double* acc) {
  (void)NvS;
  if (weighted && wnvs == nullptr) return ST_INVALID;
  for (int64_t t = 0; t < (int64_t)R * S; ++t) {
    combine_token(
        K, H, dst + t * K, [&](int64_t G) { return y + G * H; },
        [&](int64_t G) { return wnvs != nullptr ? wnvs[G] : 0.0f; }, weighted, out + t * H,
        wsk_out != nullptr ? wsk_out + t * K : nullptr, acc != nullptr ? acc + t * H : nullptr);
  }
  return ST_OK;
}

int32_t orc_combine_rows(int32_t n, int32_t K, int32_t H, const int32_t* dst_tok, int64_t M,
                         const int64_t* rows, const uint16_t* yrows, const float* wrows,
                         int32_t weighted, uint16_t* out, float* wsk_out, double* acc) {
  if (weighted && wrows == nullptr) return ST_INVALID;
  auto find = [&](int64_t G) -> int64_t {
    const int64_t* p = std::lower_bound(rows, rows + M, G);
    return (p != rows + M && *p == G) ? (int64_t)(p - rows) : -1;
  };
  for (int64_t t = 0; t < n; ++t)
    for (int k = 0; k < K; ++k)
      if (find(decode_row(dst_tok[t * K + k])) < 0) return ST_INVALID;
  for (int64_t t = 0; t < n; ++t) {
    combine_token(
        K, H, dst_tok + t * K, [&](int64_t G) { return yrows + find(G) * H; },
        [&](int64_t G) { return wrows != nullptr ? wrows[find(G)] : 0.0f; }, weighted,
        out + t * H, wsk_out != nullptr ? wsk_out + t * K : nullptr,
        acc != nullptr ? acc + t * H : nullptr);
  }
  return ST_OK;
}

int32_t orc_combine_prologue(int32_t R, int32_t K, int32_t S, int32_t H, int32_t NvS,
                             const int32_t* dst, const uint16_t* y, const float* wnvs,
                             int32_t weighted, uint16_t* out, float* wsk_out, double* acc,
                             uint16_t* folded) {
  if (weighted && wnvs == nullptr) return ST_INVALID;
  if (folded != nullptr) std::memcpy(folded, y, (size_t)R * NvS * H * 2);
  for (int64_t t = 0; t < (int64_t)R * S; ++t) {
    combine_token_prologue(
        K, H, NvS, dst + t * K, [&](int64_t G) { return y + G * H; },
        [&](int64_t G) { return wnvs != nullptr ? wnvs[G] : 0.0f; }, weighted, out + t * H,
        wsk_out != nullptr ? wsk_out + t * K : nullptr, acc != nullptr ? acc + t * H : nullptr,
        [&](int64_t G, const uint16_t* b) {
          if (folded != nullptr) std::memcpy(folded + G * H, b, (size_t)H * 2);
        });
  }
  return ST_OK;
}

int32_t orc_combine_prologue_rows(int32_t n, int32_t K, int32_t H, int32_t NvS,
                                  const int32_t* dst_tok, int64_t M, const int64_t* rows,
                                  const uint16_t* yrows, const float* wrows, int32_t weighted,
                                  uint16_t* out, float* wsk_out, double* acc,
                                  uint16_t* folded_rows) {
  if (weighted && wrows == nullptr) return ST_INVALID;
  auto find = [&](int64_t G) -> int64_t {
    const int64_t* p = std::lower_bound(rows, rows + M, G);
    return (p != rows + M && *p == G) ? (int64_t)(p - rows) : -1;
  };
  for (int64_t t = 0; t < n; ++t)
    for (int k = 0; k < K; ++k)
      if (find(decode_row(dst_tok[t * K + k])) < 0) return ST_INVALID;
  if (folded_rows != nullptr) std::memcpy(folded_rows, yrows, (size_t)M * H * 2);
  for (int64_t t = 0; t < n; ++t) {
    combine_token_prologue(
        K, H, NvS, dst_tok + t * K, [&](int64_t G) { return yrows + find(G) * H; },
        [&](int64_t G) { return wrows != nullptr ? wrows[find(G)] : 0.0f; }, weighted,
        out + t * H, wsk_out != nullptr ? wsk_out + t * K : nullptr,
        acc != nullptr ? acc + t * H : nullptr, [&](int64_t G, const uint16_t* b) {
          if (folded_rows != nullptr) std::memcpy(folded_rows + find(G) * H, b, (size_t)H * 2);
        });
  }
  return ST_OK;
}

// Prefetch index: a slot's global expert id names the rank that homes the
// expert and the expert's row among that rank's experts (Visual Guide,
// Buffer.prefetch_weight).
int32_t orc_prefetch_index(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t* out) {
  if (R <= 0 || E % R != 0) return ST_INVALID;
  int Eg = E / R;
  for (int64_t j = 0; j < (int64_t)R * B; ++j) {
    int32_t e = etc[j];
    out[j * 2 + 0] = e >= 0 ? e / Eg : -1;
    out[j * 2 + 1] = e >= 0 ? e % Eg : -1;
  }
  return ST_OK;
}

// Weight prefetch (Visual Guide, Buffer.prefetch_weight): every used slot j
// of rank u receives a copy of the weights of expert experts_to_copy[u][j],
// taken from the authoritative expert rows [0, E); a -1 slot is left as it
// is.  The copy moves bytes, so it is the same for bf16, fp32 or packed
// formats.  The tensors (gate, up, down and optional scales) are treated one
// after another.  experts[t] is [E, row_bytes[t]], slots[t] is
// [R, B, row_bytes[t]].
int32_t orc_prefetch_weight(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t n,
                            const uint8_t* const* experts, uint8_t* const* slots,
                            const int64_t* row_bytes) {
  for (int t = 0; t < n; ++t) {
    for (int u = 0; u < R; ++u) {
      for (int j = 0; j < B; ++j) {
        int32_t e = etc[u * B + j];
        if (e < 0) continue;
        if (e >= E) return ST_INVALID;
        uint8_t* dst = slots[t] + ((int64_t)u * B + j) * row_bytes[t];
        std::memcpy(dst, experts[t] + (int64_t)e * row_bytes[t], (size_t)row_bytes[t]);
      }
    }
  }
  return ST_OK;
}

// Gradient reduction (Visual Guide, Buffer.reduce_grad): for every expert e
// (each owner handles its own experts), the accumulator starts from the
// authoritative gradient row e, then adds the slot gradients of every slot
// that held e, visiting ranks in ascending order (on one rank e occupies at
// most one slot; slots ascending if it were more), in fp32 as the gradient
// tensors are fp32 (a plain a + b per element).  The sum is written back to
// row e, and every consumed slot (every used slot) is cleared to +0.0.
// Experts that no slot held keep their row unchanged.  grads[t] is
// [E, row_elems[t]], slot_grads[t] is [R, B, row_elems[t]].
int32_t orc_reduce_grad(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t n,
                        float* const* grads, float* const* slot_grads, const int64_t* row_elems) {
  for (int i = 0; i < R * B; ++i)
    if (etc[i] >= E) return ST_INVALID;
  for (int t = 0; t < n; ++t) {
    const int64_t L = row_elems[t];
    for (int e = 0; e < E; ++e) {
      float* g = grads[t] + (int64_t)e * L;
      for (int u = 0; u < R; ++u) {
        for (int j = 0; j < B; ++j) {
          if (etc[u * B + j] != e) continue;
          const float* sg = slot_grads[t] + ((int64_t)u * B + j) * L;
          for (int64_t x = 0; x < L; ++x) g[x] = g[x] + sg[x];
        }
      }
    }
    for (int u = 0; u < R; ++u)
      for (int j = 0; j < B; ++j)
        if (etc[u * B + j] >= 0)
          std::fill(slot_grads[t] + ((int64_t)u * B + j) * L,
                    slot_grads[t] + ((int64_t)u * B + j + 1) * L, 0.0f);
  }
  return ST_OK;
}

}  // extern "C"
