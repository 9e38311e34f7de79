// moon_api.hip — host side of the C ABI declared in include/moon.h.
//
// Validation happens here, before anything is launched; kernels only see
// shapes that fit their grids and LDS tables.  Context = the pages' Buffer
// ("MoonEP Public API Visual Guide", Buffer(...): the constructor checks the
// topology, fixes the capacities and owns the persistent windows); plan = the
// MoonEPCommPlan arrays plus cu_seqlens and a status word.
#include <new>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "moon_internal.h"

// The largest planner scratch moon_plan_noalloc serves (the count matrix,
// the exchange words and the call tag): 512 KB holds every shape up to
// E = 384 with 256 planner tiles; the largest ones (E = 512 with more than
// about 220 tiles) are refused.
constexpr size_t kNoAllocScratchBytes = 512u << 10;

// Planner scratch of moon_plan_noalloc: one block on every GPU the library
// runs on, held until the process ends.  Host code reaches it only through
// the device address that hipGetSymbolAddress gives for the current device
// (noalloc_scratch); the array's name is not a device address on the host.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

using moon::Dims;

constexpr uint32_t kCtxMagic = 0x43584E4Du, kPlanMagic = 0x504C4E4Du, kDead = 0u;

int64_t round_up(int64_t n, int64_t p) { return (n + p - 1) / p * p; }

int bits_for(int n) {  // bits of the values 0..n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
      changed = hipSetDevice(dev) == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// Most planner tiles per call (never above kMaxTiles, nor the compute units).
constexpr int kPlanTileCap = moon::kMaxTiles;
// Cost of one more chunk per planner wave, in units of one expert count
// reduced for one tile (fitted on MI355X over five workload shapes: a chunk
// costs about 3 us, a tile's share of the count matrix very little).
constexpr double kChunkWeight = 300000.0;

moon_status make_dims(const moon_config* c, Dims* d) {
  if (c == nullptr || c->flags != 0) return MOON_ERR_INVALID_ARG;
  if (c->R < 1 || c->E < 1 || c->K < 1 || c->S < 1 || c->H < 1 || c->token_padding < 1)
    return MOON_ERR_INVALID_ARG;
  if (c->E % c->R != 0) return MOON_ERR_TOPOLOGY;
  if (c->R > moon::kMaxR || c->E > moon::kMaxE || c->K > moon::kMaxK || c->H % 8 != 0 ||
      c->H > 65536 || c->H < 8)
    return MOON_ERR_UNSUPPORTED;
  const int Eg = c->E / c->R;
  const int B = c->B <= 0 ? Eg : c->B;
  if ((int64_t)c->R * B > moon::kMaxSlotsTotal) return MOON_ERR_UNSUPPORTED;
  const int64_t routes = (int64_t)c->R * c->S * c->K;
  const int64_t nvs =
      round_up((int64_t)c->S * c->K + (int64_t)(Eg + B) * (c->token_padding - 1), c->token_padding);
  if (routes >= (int64_t)1 << 31 || (int64_t)c->R * nvs >= (int64_t)1 << 31)
    return MOON_ERR_UNSUPPORTED;
  d->R = c->R;
  d->E = c->E;
  d->K = c->K;
  d->S = c->S;
  d->H = c->H;
  d->B = B;
  d->P = c->token_padding;
  d->Eg = Eg;
  d->EB = c->E + B;
  d->NvS = (int32_t)nvs;
  // Planner tiles, never across a rank boundary, at most one per compute
  // unit and kMaxTiles in all.  Every tile reduces the E x tiles count
  // matrix, and each of its kPlanWaves waves walks its share of the tile in
  // chunks of floor(64/K) tokens, so plan time is about
  // E*tiles + kChunkWeight*chunks (weight fitted on MI355X).  Tiles are a
  // whole number of chunks per wave; the cheapest count is taken.
  int max_tiles = kPlanTileCap;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0 && cus < max_tiles)
    max_tiles = cus;
  const int ctok = moon::kWave / c->K;
  const int64_t round_tok = (int64_t)moon::kPlanWaves * ctok;  // tokens per chunk round
  int tt = 0;
  double best = 0.0;
  for (int64_t m = 1; m <= (c->S + round_tok - 1) / round_tok; ++m) {
    const int cand = (int)std::min<int64_t>(round_tok * m, c->S);
    const int64_t tiles = (int64_t)c->R * ((c->S + cand - 1) / cand);
    if (tiles > max_tiles) continue;
    const double cost = (double)c->E * tiles + kChunkWeight * m;
    if (tt == 0 || cost < best) {
      tt = cand;
      best = cost;
    }
  }
  if (tt == 0) tt = c->S;  // more ranks than compute units: one tile per rank
  const int tpr = (c->S + tt - 1) / tt;
  tt = (c->S + tpr - 1) / tpr;  // even out the tiles of a rank
  d->tile_tok = tt;
  d->tiles_per_rank = tpr;
  d->ntiles = c->R * tpr;
  d->ntiles_pad = (d->ntiles + 3) / 4 * 4;
  if ((int64_t)tt * c->K >= (int64_t)1 << 24) return MOON_ERR_UNSUPPORTED;  // 24-bit tile counts
  d->ctok = moon::kWave / c->K;
  d->tbits = bits_for(d->ctok);
  d->ebits = bits_for(c->E);
  d->rbits = bits_for(c->R);
  d->ncu = cus > 0 ? cus : 256;
  return MOON_OK;
}

bool ctx_ok(const moon_ctx* c) { return c != nullptr && c->magic == kCtxMagic; }
bool plan_ok(const moon_comm_plan* p) { return p != nullptr && p->magic == kPlanMagic && ctx_ok(p->ctx); }

size_t carve(size_t& off, size_t bytes) {
  size_t at = (off + 255) & ~(size_t)255;
  off = at + bytes;
  return at;
}

moon::Scratch scratch_at(char* base, const moon::ScratchLayout& sl) {
  moon::Scratch sc;
  sc.tile_cnt = reinterpret_cast<int32_t*>(base + sl.cnt);
  sc.tile_agg = reinterpret_cast<uint64_t*>(base + sl.agg);
  sc.epoch = reinterpret_cast<uint32_t*>(base + sl.epoch);
  return sc;
}

// Offsets of the plan arrays inside one allocation.
struct PlanOffsets {
  size_t dst, etc, zfr, rstats, dup_groups, dup_loffs, dup_counts, cu, status, pidx, total;
};

PlanOffsets plan_offsets(const Dims& d) {
  PlanOffsets o;
  size_t off = 0;
  const size_t i4 = sizeof(int32_t);
  o.dst = carve(off, (size_t)d.R * d.S * d.K * i4);
  o.etc = carve(off, (size_t)d.R * d.B * i4);
  o.zfr = carve(off, (size_t)d.R * d.EB * 2 * i4);
  o.rstats = carve(off, (size_t)d.R * 2 * i4);
  o.dup_groups = carve(off, (size_t)d.R * d.NvS * 3 * i4);
  o.dup_loffs = carve(off, (size_t)d.R * d.NvS * i4);
  o.dup_counts = carve(off, (size_t)d.R * 2 * i4);
  o.cu = carve(off, (size_t)d.R * d.EB * i4);
  o.status = carve(off, i4);
  o.pidx = carve(off, (size_t)d.R * d.B * 2 * i4);
  o.total = (off + 255) & ~(size_t)255;
  return o;
}

moon::PlanArrays plan_arrays(void* mem, const PlanOffsets& o) {
  char* b = static_cast<char*>(mem);
  moon::PlanArrays a;
  a.dst = reinterpret_cast<int32_t*>(b + o.dst);
  a.etc = reinterpret_cast<int32_t*>(b + o.etc);
  a.zfr = reinterpret_cast<int32_t*>(b + o.zfr);
  a.rstats = reinterpret_cast<int32_t*>(b + o.rstats);
  a.dup_groups = reinterpret_cast<int32_t*>(b + o.dup_groups);
  a.dup_loffs = reinterpret_cast<int32_t*>(b + o.dup_loffs);
  a.dup_counts = reinterpret_cast<int32_t*>(b + o.dup_counts);
  a.cu = reinterpret_cast<int32_t*>(b + o.cu);
  a.status = reinterpret_cast<int32_t*>(b + o.status);
  a.pidx = reinterpret_cast<int32_t*>(b + o.pidx);
  return a;
}

moon_status new_plan(moon_ctx* ctx, moon_comm_plan** out) {
  const PlanOffsets o = plan_offsets(ctx->d);
  void* mem = nullptr;
  if (hipMalloc(&mem, o.total) != hipSuccess) return MOON_ERR_OOM;
  moon_comm_plan* p = new (std::nothrow) moon_comm_plan;
  if (p == nullptr) {
    (void)hipFree(mem);
    return MOON_ERR_OOM;
  }
  p->magic = kPlanMagic;
  p->ctx = ctx;
  p->mem = mem;
  p->bytes = o.total;
  p->a = plan_arrays(mem, o);
  *out = p;
  return MOON_OK;
}

// Device address of this GPU's planner scratch block, taken once per device
// with that device current; nullptr if the runtime refuses.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* noalloc_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace moon {

ScratchLayout scratch_layout(const Dims& d) {
  ScratchLayout sl;
  size_t off = 0;
  sl.cnt = carve(off, (size_t)(d.E + 1) * d.ntiles_pad * sizeof(int32_t));
  sl.agg = carve(off, (size_t)d.ntiles * d.R * 8);
  sl.epoch = carve(off, sizeof(uint32_t));
  sl.total = (off + 255) & ~(size_t)255;
  return sl;
}

}  // namespace moon

extern "C" {

moon_status moon_ctx_create(const moon_config* cfg, moon_ctx** out) {
  if (out == nullptr) return MOON_ERR_INVALID_ARG;
  *out = nullptr;
  Dims d;
  moon_status st = make_dims(cfg, &d);
  if (st != MOON_OK) return st;

  moon_ctx* c = new (std::nothrow) moon_ctx;
  if (c == nullptr) return MOON_ERR_OOM;
  c->magic = kCtxMagic;
  c->d = d;
  c->hidden_win = nullptr;
  c->w_win = nullptr;
  c->scratch_mem = nullptr;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return MOON_ERR_HIP;
  }
  const size_t rows = (size_t)d.R * d.NvS;
  const moon::ScratchLayout sl = moon::scratch_layout(d);
  size_t off = sl.total;
  const size_t i4 = sizeof(int32_t);
  const size_t o_used = carve(off, (size_t)d.R * d.B * i4);
  const size_t o_acte = carve(off, (size_t)d.E * i4);
  const size_t o_actm = carve(off, (size_t)d.E * d.R * i4);
  const size_t o_scnt = carve(off, 2 * i4);
  if (hipMalloc(&c->hidden_win, rows * d.H * 2) != hipSuccess ||
      hipMalloc(reinterpret_cast<void**>(&c->w_win), rows * 4) != hipSuccess ||
      hipMalloc(&c->scratch_mem, off) != hipSuccess) {
    moon_ctx_destroy(&c);
    return MOON_ERR_OOM;
  }
  if (hipMemset(c->hidden_win, 0, rows * d.H * 2) != hipSuccess ||
      hipMemset(c->w_win, 0, rows * 4) != hipSuccess ||
      hipMemset(c->scratch_mem, 0, off) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    moon_ctx_destroy(&c);
    return MOON_ERR_HIP;
  }
  char* b = static_cast<char*>(c->scratch_mem);
  c->sc = scratch_at(b, sl);
  c->si.used = reinterpret_cast<int32_t*>(b + o_used);
  c->si.act_e = reinterpret_cast<int32_t*>(b + o_acte);
  c->si.act_match = reinterpret_cast<int32_t*>(b + o_actm);
  c->si.counts = reinterpret_cast<int32_t*>(b + o_scnt);
  *out = c;
  return MOON_OK;
}

moon_status moon_ctx_layout(const moon_ctx* ctx, moon_layout* out) {
  if (!ctx_ok(ctx) || out == nullptr) return MOON_ERR_INVALID_ARG;
  out->N = ctx->d.S * ctx->d.K;
  out->NvS = ctx->d.NvS;
  out->NvS_padded = ctx->d.NvS;
  out->E_plus_B = ctx->d.EB;
  out->B = ctx->d.B;
  out->hidden_windows = ctx->hidden_win;
  out->weight_windows = ctx->w_win;
  return MOON_OK;
}

void moon_ctx_destroy(moon_ctx** ctx) {
  if (ctx == nullptr || *ctx == nullptr) return;
  moon_ctx* c = *ctx;
  if (c->magic == kCtxMagic) {
    DeviceGuard g(c->device);
    (void)hipDeviceSynchronize();
    if (c->hidden_win) (void)hipFree(c->hidden_win);
    if (c->w_win) (void)hipFree(c->w_win);
    if (c->scratch_mem) (void)hipFree(c->scratch_mem);
    c->magic = kDead;
    delete c;
  }
  *ctx = nullptr;
}

moon_status moon_plan_create(moon_ctx* ctx, moon_comm_plan** out) {
  if (out == nullptr) return MOON_ERR_INVALID_ARG;
  *out = nullptr;
  if (!ctx_ok(ctx)) return MOON_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  moon_comm_plan* p = nullptr;
  moon_status st = new_plan(ctx, &p);
  if (st != MOON_OK) return st;
  const int32_t init = moon::kNotPlanned;
  if (hipMemcpy(p->a.status, &init, sizeof(init), hipMemcpyHostToDevice) != hipSuccess) {
    moon_plan_destroy(&p);
    return MOON_ERR_HIP;
  }
  *out = p;
  return MOON_OK;
}

moon_status moon_plan_clone(const moon_comm_plan* src, moon_comm_plan** out, hipStream_t stream) {
  if (out == nullptr) return MOON_ERR_INVALID_ARG;
  *out = nullptr;
  if (!plan_ok(src)) return MOON_ERR_INVALID_ARG;
  DeviceGuard g(src->ctx->device);
  moon_comm_plan* p = nullptr;
  moon_status st = new_plan(src->ctx, &p);
  if (st != MOON_OK) return st;
  if (hipMemcpyAsync(p->mem, src->mem, src->bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
    moon_plan_destroy(&p);
    return MOON_ERR_HIP;
  }
  *out = p;
  return MOON_OK;
}

void moon_plan_destroy(moon_comm_plan** plan) {
  if (plan == nullptr || *plan == nullptr) return;
  moon_comm_plan* p = *plan;
  if (p->magic == kPlanMagic) {
    if (p->mem) (void)hipFree(p->mem);
    p->magic = kDead;
    delete p;
  }
  *plan = nullptr;
}

moon_status moon_plan_view(const moon_comm_plan* plan, moon_plan_arrays* out) {
  if (!plan_ok(plan) || out == nullptr) return MOON_ERR_INVALID_ARG;
  const Dims& d = plan->ctx->d;
  out->dst = plan->a.dst;
  out->experts_to_copy = plan->a.etc;
  out->zero_fill_ranges = plan->a.zfr;
  out->remote_stats = plan->a.rstats;
  out->dup_groups = plan->a.dup_groups;
  out->dup_loffs = plan->a.dup_loffs;
  out->dup_counts = plan->a.dup_counts;
  out->cu_seqlens = plan->a.cu;
  out->status = plan->a.status;
  out->prefetch_index = plan->a.pidx;
  out->N = d.S * d.K;
  out->R = d.R;
  out->E = d.E;
  out->B = d.B;
  out->NvS = d.NvS;
  out->K = d.K;
  return MOON_OK;
}

moon_status moon_plan_status(const moon_comm_plan* plan, hipStream_t stream) {
  if (!plan_ok(plan)) return MOON_ERR_INVALID_ARG;
  DeviceGuard g(plan->ctx->device);
  int32_t bits = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOON_ERR_HIP;
  if (hipMemcpy(&bits, plan->a.status, sizeof(bits), hipMemcpyDeviceToHost) != hipSuccess)
    return MOON_ERR_HIP;
  if (bits & moon::kBadExpert) return MOON_ERR_BAD_EXPERT;
  if (bits & moon::kHistogram) return MOON_ERR_HISTOGRAM;
  if (bits & moon::kSlotBudget) return MOON_ERR_SLOT_BUDGET;
  if (bits & moon::kInternal) return MOON_ERR_INTERNAL;
  if (bits & moon::kNotPlanned) return MOON_ERR_NOT_PLANNED;
  return bits == 0 ? MOON_OK : MOON_ERR_INTERNAL;
}

moon_status moon_debug_tile_counts(const moon_ctx* ctx, int32_t* counts_dev, int32_t* tile_tokens,
                                   int32_t* tiles_per_rank, hipStream_t stream) {
  if (!ctx_ok(ctx) || !aligned(counts_dev, 4)) return MOON_ERR_INVALID_ARG;
  const Dims& d = ctx->d;
  if (tile_tokens != nullptr) *tile_tokens = d.tile_tok;
  if (tiles_per_rank != nullptr) *tiles_per_rank = d.tiles_per_rank;
  if (counts_dev == nullptr) return MOON_OK;
  DeviceGuard g(ctx->device);
  // the count matrix rows are ntiles_pad wide; the copy drops the padding
  const size_t w = (size_t)d.ntiles * sizeof(int32_t);
  if (hipMemcpy2DAsync(counts_dev, w, ctx->sc.tile_cnt, (size_t)d.ntiles_pad * sizeof(int32_t), w,
                       (size_t)d.E + 1, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_plan(moon_ctx* ctx, const int32_t* topk_rsk, const int32_t* tokens_per_expert_re,
                      moon_comm_plan* plan, hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || topk_rsk == nullptr) return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  if (!aligned(topk_rsk, 4) || !aligned(tokens_per_expert_re, 4)) return MOON_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (moon::launch_plan(ctx->d, ctx->sc, plan->a, topk_rsk, tokens_per_expert_re, stream) !=
      hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_plan_noalloc(const moon_config* cfg, const int32_t* topk_rsk,
                              const int32_t* tokens_per_expert_re, const moon_plan_arrays* plan,
                              hipStream_t stream) {
  if (plan == nullptr || topk_rsk == nullptr) return MOON_ERR_INVALID_ARG;
  Dims d;
  moon_status st = make_dims(cfg, &d);
  if (st != MOON_OK) return st;
  const moon_plan_arrays& p = *plan;
  if (p.N != d.S * d.K || p.R != d.R || p.E != d.E || p.B != d.B || p.NvS != d.NvS || p.K != d.K)
    return MOON_ERR_INVALID_ARG;
  const int32_t* arrays[] = {p.dst, p.experts_to_copy, p.zero_fill_ranges, p.remote_stats,
                             p.dup_groups, p.dup_loffs, p.dup_counts, p.cu_seqlens, p.status,
                             p.prefetch_index, topk_rsk};
  for (const int32_t* a : arrays)
    if (a == nullptr || !aligned(a, 4)) return MOON_ERR_INVALID_ARG;
  if (!aligned(tokens_per_expert_re, 4)) return MOON_ERR_INVALID_ARG;
  const moon::ScratchLayout sl = moon::scratch_layout(d);
  if (sl.total > kNoAllocScratchBytes) return MOON_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOON_ERR_HIP;
  void* base = noalloc_scratch(dev);
  if (base == nullptr) return MOON_ERR_HIP;
  moon::PlanArrays pa;
  pa.dst = p.dst;
  pa.etc = p.experts_to_copy;
  pa.zfr = p.zero_fill_ranges;
  pa.rstats = p.remote_stats;
  pa.dup_groups = p.dup_groups;
  pa.dup_loffs = p.dup_loffs;
  pa.dup_counts = p.dup_counts;
  pa.cu = p.cu_seqlens;
  pa.status = p.status;
  pa.pidx = p.prefetch_index;
  if (moon::launch_plan(d, scratch_at(static_cast<char*>(base), sl), pa, topk_rsk,
                        tokens_per_expert_re, stream) != hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_dispatch(moon_ctx* ctx, const moon_comm_plan* plan, const void* hidden_rsh,
                          const float* weights_rsk, void* hidden_out, float* weights_out,
                          uint32_t flags, hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || hidden_rsh == nullptr) return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  if ((flags & ~(MOON_DISPATCH_FUSED_DUPS | MOON_DISPATCH_DEDUP_EPILOGUE)) != 0 ||
      ((flags & MOON_DISPATCH_FUSED_DUPS) != 0 && (flags & MOON_DISPATCH_DEDUP_EPILOGUE) != 0))
    return MOON_ERR_INVALID_ARG;
  void* hout = hidden_out != nullptr ? hidden_out : ctx->hidden_win;
  float* wout = weights_out != nullptr ? weights_out : ctx->w_win;
  if (!aligned(hidden_rsh, 16) || !aligned(hout, 16) || !aligned(weights_rsk, 4) ||
      !aligned(wout, 4))
    return MOON_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (moon::launch_dispatch(ctx->d, plan->a, static_cast<const uint16_t*>(hidden_rsh), weights_rsk,
                            static_cast<uint16_t*>(hout), wout,
                            (flags & MOON_DISPATCH_DEDUP_EPILOGUE) != 0, stream) != hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_combine(moon_ctx* ctx, const moon_comm_plan* plan, const void* y_nvsh,
                         const float* w_nvs, uint32_t flags, void* out_rsh, float* w_rsk_out,
                         hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || y_nvsh == nullptr || out_rsh == nullptr)
    return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  if ((flags & ~(MOON_COMBINE_WEIGHTED | MOON_COMBINE_DUP_PROLOGUE)) != 0)
    return MOON_ERR_INVALID_ARG;
  const bool weighted = (flags & MOON_COMBINE_WEIGHTED) != 0;
  // the prologue folds into the persistent shard: the context's hidden window
  uint16_t* fold = (flags & MOON_COMBINE_DUP_PROLOGUE) != 0
                       ? static_cast<uint16_t*>(ctx->hidden_win) : nullptr;
  if ((weighted || w_rsk_out != nullptr) && w_nvs == nullptr) return MOON_ERR_INVALID_ARG;
  if (!aligned(y_nvsh, 16) || !aligned(out_rsh, 16) || !aligned(w_nvs, 4) || !aligned(w_rsk_out, 4))
    return MOON_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (moon::launch_combine(ctx->d, plan->a, static_cast<const uint16_t*>(y_nvsh), w_nvs, weighted,
                           fold, static_cast<uint16_t*>(out_rsh), w_rsk_out, stream) != hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_prefetch_weight(moon_ctx* ctx, const moon_comm_plan* plan,
                                 const moon_weight_tensor* tensors, int32_t n_tensors,
                                 hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || tensors == nullptr || n_tensors < 1 ||
      n_tensors > moon::kMaxWeightTensors)
    return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  const void* src[moon::kMaxWeightTensors];
  void* dst[moon::kMaxWeightTensors];
  int64_t bytes[moon::kMaxWeightTensors];
  for (int t = 0; t < n_tensors; ++t) {
    const moon_weight_tensor& w = tensors[t];
    if (w.experts == nullptr || w.slots == nullptr || w.row_bytes <= 0 || w.row_bytes % 16 != 0 ||
        !aligned(w.experts, 16) || !aligned(w.slots, 16))
      return MOON_ERR_INVALID_ARG;
    src[t] = w.experts;
    dst[t] = w.slots;
    bytes[t] = w.row_bytes;
  }
  DeviceGuard g(ctx->device);
  if (moon::launch_prefetch_weight(ctx->d, plan->a, ctx->si, n_tensors, src, dst, bytes, stream) !=
      hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_reduce_grad(moon_ctx* ctx, const moon_comm_plan* plan,
                             const moon_grad_tensor* tensors, int32_t n_tensors,
                             hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || tensors == nullptr || n_tensors < 1 ||
      n_tensors > moon::kMaxWeightTensors)
    return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  float* grads[moon::kMaxWeightTensors];
  float* slots[moon::kMaxWeightTensors];
  int64_t bytes[moon::kMaxWeightTensors];
  for (int t = 0; t < n_tensors; ++t) {
    const moon_grad_tensor& w = tensors[t];
    if (w.expert_grads == nullptr || w.slot_grads == nullptr || w.row_elems <= 0 ||
        w.row_elems % 4 != 0 || w.row_elems > (INT64_MAX / 4) || !aligned(w.expert_grads, 16) ||
        !aligned(w.slot_grads, 16))
      return MOON_ERR_INVALID_ARG;
    grads[t] = w.expert_grads;
    slots[t] = w.slot_grads;
    bytes[t] = w.row_elems * 4;
  }
  DeviceGuard g(ctx->device);
  if (moon::launch_reduce_grad(ctx->d, plan->a, ctx->si, n_tensors, grads, slots, bytes, stream) !=
      hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

moon_status moon_prefetch_index(moon_ctx* ctx, const moon_comm_plan* plan, int32_t* src_rb2,
                                hipStream_t stream) {
  if (!ctx_ok(ctx) || !plan_ok(plan) || src_rb2 == nullptr || !aligned(src_rb2, 4))
    return MOON_ERR_INVALID_ARG;
  if (plan->ctx != ctx) return MOON_ERR_PLAN_MISMATCH;
  DeviceGuard g(ctx->device);
  if (moon::launch_prefetch_index(ctx->d, plan->a, src_rb2, stream) != hipSuccess)
    return MOON_ERR_HIP;
  return MOON_OK;
}

const char* moon_status_str(moon_status s) {
  switch (s) {
    case MOON_OK: return "ok";
    case MOON_ERR_INVALID_ARG: return "invalid argument";
    case MOON_ERR_TOPOLOGY: return "E is not divisible by R";
    case MOON_ERR_UNSUPPORTED: return "sizes beyond the supported limits";
    case MOON_ERR_OOM: return "device allocation failed";
    case MOON_ERR_HIP: return "HIP runtime error";
    case MOON_ERR_PLAN_MISMATCH: return "plan belongs to another context";
    case MOON_ERR_BAD_EXPERT: return "expert id out of range";
    case MOON_ERR_SLOT_BUDGET: return "prefetch slot budget exceeded";
    case MOON_ERR_HISTOGRAM: return "tokens_per_expert disagrees with the routes";
    case MOON_ERR_NOT_PLANNED: return "plan not filled yet";
    case MOON_ERR_INTERNAL: return "internal consistency check failed";
  }
  return "unknown status";
}

}  // extern "C"
