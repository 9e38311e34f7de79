/*
 * A C11 program that drives libmoon through its C ABI alone: device memory
 * from hipMalloc, copies with hipMemcpy, no Python and no torch.  It plans,
 * dispatches and combines a small routing in which every third token sends
 * all its routes to rank 0's experts (so rank 0 donates routes to slots),
 * then checks closed forms that the method fixes exactly:
 *   - the default B is E/R and NvS = round_up(S*K + (E/R + B)*(P - 1), P);
 *   - every rank receives S*K routes (cu_seqlens and zero_fill_ranges agree);
 *   - with y = the dispatched windows, the plain combine returns K*x and the
 *     weighted combine with every route weight 1/K returns x, bit for bit
 *     (x are small integers and K = 4, so every product and sum is exact);
 *   - the prefetch index of every used slot names the slot expert's owner
 *     rank and local row, and (-1, -1) for an unused slot;
 *   - the plan's own prefetch_index array holds the same;
 *   - moon_plan_noalloc, given caller-allocated arrays and no context,
 *     writes the same plan as moon_plan, field for field;
 *   - an expert id out of range sets MOON_ERR_BAD_EXPERT without a launch
 *     error, and a plan of another context is refused on the host.
 * Prints "c abi ok" and exits 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moon.h"

#define R 4
#define E 16
#define K 4
#define S 100
#define H 64
#define P 8

static int failures = 0;

#define HIP_OK(x)                                                            \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);  \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

#define MOON_OK_(x)                                                          \
  do {                                                                       \
    moon_status s_ = (x);                                                    \
    if (s_ != MOON_OK) {                                                     \
      printf("moon error %s at line %d\n", moon_status_str(s_), __LINE__);   \
      exit(3);                                                               \
    }                                                                        \
  } while (0)

#define EXPECT(c, ...)         \
  do {                         \
    if (!(c)) {                \
      printf(__VA_ARGS__);     \
      printf("\n");            \
      ++failures;              \
    }                          \
  } while (0)

/* bf16 bits of a small integer (exact: the low half of its fp32 bits is 0) */
static uint16_t bf16_of_int(int v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes));
  return p;
}

int main(void) {
  const int Eg = E / R;
  static int32_t topk[R * S * K];
  static uint16_t hidden[R * S * H];
  static float w[R * S * K];
  for (int r = 0; r < R; ++r)
    for (int s = 0; s < S; ++s)
      for (int k = 0; k < K; ++k) {
        const int e = (s % 3 == 0) ? k : (r * 7 + s * 3 + k * 5) % E;
        topk[(r * S + s) * K + k] = e;
        w[(r * S + s) * K + k] = 1.0f / K;
      }
  for (int i = 0; i < R * S * H; ++i) hidden[i] = bf16_of_int((i * 7 + i / H * 3) % 15 - 7);

  moon_config cfg = {R, E, K, S, H, 0, P, 0};
  moon_ctx* ctx = NULL;
  MOON_OK_(moon_ctx_create(&cfg, &ctx));
  moon_layout lay;
  MOON_OK_(moon_ctx_layout(ctx, &lay));
  const int B = lay.B, NvS = lay.NvS_padded;
  EXPECT(B == Eg && NvS == (S * K + (Eg + B) * (P - 1) + P - 1) / P * P && lay.N == S * K,
         "layout: B %d NvS %d N %d", B, NvS, lay.N);

  int32_t* d_topk = dev_alloc(sizeof topk);
  uint16_t* d_hidden = dev_alloc(sizeof hidden);
  float* d_w = dev_alloc(sizeof w);
  uint16_t* d_out = dev_alloc(sizeof hidden);
  int32_t* d_pidx = dev_alloc((size_t)R * B * 2 * sizeof(int32_t));
  HIP_OK(hipMemcpy(d_topk, topk, sizeof topk, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_hidden, hidden, sizeof hidden, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  moon_comm_plan* plan = NULL;
  MOON_OK_(moon_plan_create(ctx, &plan));
  EXPECT(moon_plan_status(plan, st) == MOON_ERR_NOT_PLANNED, "a new plan must read NOT_PLANNED");
  MOON_OK_(moon_plan(ctx, d_topk, NULL, plan, st));
  MOON_OK_(moon_dispatch(ctx, plan, d_hidden, d_w, NULL, NULL, 0, st));
  MOON_OK_(moon_prefetch_index(ctx, plan, d_pidx, st));
  MOON_OK_(moon_plan_status(plan, st));

  /* balance: S*K routes per rank; rank 0 donated */
  moon_plan_arrays pa;
  MOON_OK_(moon_plan_view(plan, &pa));
  static int32_t cu[R * (E + E)], etc[R * E], rstats[R * 2];
  HIP_OK(hipMemcpy(cu, pa.cu_seqlens, (size_t)R * (E + B) * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(etc, pa.experts_to_copy, (size_t)R * B * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(rstats, pa.remote_stats, (size_t)R * 2 * 4, hipMemcpyDeviceToHost));
  static int32_t zfr[R * (E + E) * 2];
  HIP_OK(hipMemcpy(zfr, pa.zero_fill_ranges, (size_t)R * (E + B) * 2 * 4, hipMemcpyDeviceToHost));
  int slots_used = 0;
  for (int u = 0; u < R; ++u) {
    int routes = 0;
    for (int g = 0; g < E + B; ++g) {
      const int a = zfr[(u * (E + B) + g) * 2], b = zfr[(u * (E + B) + g) * 2 + 1];
      const int begin = g == 0 ? 0 : cu[u * (E + B) + g - 1];
      routes += a - begin;       /* rows before the padding are routes */
      EXPECT(b == cu[u * (E + B) + g], "rank %d group %d: padding must end at cu_seqlens", u, g);
    }
    EXPECT(routes == S * K, "rank %d holds %d routes, not S*K = %d", u, routes, S * K);
    slots_used += rstats[u * 2];
  }
  EXPECT(slots_used > 0, "the skewed routing must use slots");

  /* prefetch index */
  static int32_t pidx[R * E * 2];
  HIP_OK(hipMemcpy(pidx, d_pidx, (size_t)R * B * 2 * 4, hipMemcpyDeviceToHost));
  for (int i = 0; i < R * B; ++i) {
    const int e = etc[i];
    EXPECT(pidx[2 * i] == (e >= 0 ? e / Eg : -1) && pidx[2 * i + 1] == (e >= 0 ? e % Eg : -1),
           "slot %d: prefetch index (%d, %d) for expert %d", i, pidx[2 * i], pidx[2 * i + 1], e);
  }

  static int32_t pidx_plan[R * E * 2];
  HIP_OK(hipMemcpy(pidx_plan, pa.prefetch_index, (size_t)R * B * 2 * 4, hipMemcpyDeviceToHost));
  EXPECT(memcmp(pidx_plan, pidx, (size_t)R * B * 2 * 4) == 0,
         "the plan's prefetch_index differs from moon_prefetch_index");

  /* planning without a context into caller-owned arrays */
  {
    moon_plan_arrays na = pa;  /* same sizes; fresh device arrays */
    const size_t n_dst = (size_t)R * S * K, n_eb = (size_t)R * (E + B);
    na.dst = dev_alloc(n_dst * 4);
    na.experts_to_copy = dev_alloc((size_t)R * B * 4);
    na.zero_fill_ranges = dev_alloc(n_eb * 2 * 4);
    na.remote_stats = dev_alloc((size_t)R * 2 * 4);
    na.dup_groups = dev_alloc((size_t)R * NvS * 3 * 4);
    na.dup_loffs = dev_alloc((size_t)R * NvS * 4);
    na.dup_counts = dev_alloc((size_t)R * 2 * 4);
    na.cu_seqlens = dev_alloc(n_eb * 4);
    na.status = dev_alloc(4);
    na.prefetch_index = dev_alloc((size_t)R * B * 2 * 4);
    MOON_OK_(moon_plan_noalloc(&cfg, d_topk, NULL, &na, st));
    HIP_OK(hipStreamSynchronize(st));
    int32_t status = -1;
    HIP_OK(hipMemcpy(&status, na.status, 4, hipMemcpyDeviceToHost));
    EXPECT(status == 0, "moon_plan_noalloc: status word %d", status);
    struct { const char* name; int32_t* a; int32_t* b; size_t n; } f[] = {
        {"dst", pa.dst, na.dst, n_dst},
        {"experts_to_copy", pa.experts_to_copy, na.experts_to_copy, (size_t)R * B},
        {"zero_fill_ranges", pa.zero_fill_ranges, na.zero_fill_ranges, n_eb * 2},
        {"remote_stats", pa.remote_stats, na.remote_stats, (size_t)R * 2},
        {"dup_counts", pa.dup_counts, na.dup_counts, (size_t)R * 2},
        {"cu_seqlens", pa.cu_seqlens, na.cu_seqlens, n_eb},
        {"prefetch_index", pa.prefetch_index, na.prefetch_index, (size_t)R * B * 2},
        {"dup_groups", pa.dup_groups, na.dup_groups, (size_t)R * NvS * 3},
        {"dup_loffs", pa.dup_loffs, na.dup_loffs, (size_t)R * NvS}};
    static int32_t ha[R * S * K * 4], hb[R * S * K * 4], cnt[R * 2];
    HIP_OK(hipMemcpy(cnt, pa.dup_counts, sizeof cnt, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < sizeof f / sizeof f[0]; ++i) {
      HIP_OK(hipMemcpy(ha, f[i].a, f[i].n * 4, hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(hb, f[i].b, f[i].n * 4, hipMemcpyDeviceToHost));
      int differ = 0;
      for (size_t j = 0; j < f[i].n; ++j) {
        /* duplicate records: the valid prefix of each rank only */
        if (i == 7 && (int)(j % ((size_t)NvS * 3)) >= cnt[(j / ((size_t)NvS * 3)) * 2] * 3) continue;
        if (i == 8 && (int)(j % (size_t)NvS) >= cnt[(j / (size_t)NvS) * 2 + 1]) continue;
        differ += ha[j] != hb[j];
      }
      EXPECT(differ == 0, "moon_plan_noalloc: %d entries of %s differ from moon_plan", differ,
             f[i].name);
    }
    int32_t* ptrs[] = {na.dst, na.experts_to_copy, na.zero_fill_ranges, na.remote_stats,
                       na.dup_groups, na.dup_loffs, na.dup_counts, na.cu_seqlens, na.status,
                       na.prefetch_index};
    for (size_t i = 0; i < sizeof ptrs / sizeof ptrs[0]; ++i) HIP_OK(hipFree(ptrs[i]));
  }

  /* combine over the dispatched windows: K*x unweighted, x weighted by 1/K */
  static uint16_t out[R * S * H];
  MOON_OK_(moon_combine(ctx, plan, lay.hidden_windows, NULL, 0, d_out, NULL, st));
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  int bad = 0;
  for (int i = 0; i < R * S * H; ++i) {
    const int x = (i * 7 + i / H * 3) % 15 - 7;
    bad += out[i] != bf16_of_int(K * x);
  }
  EXPECT(bad == 0, "plain combine: %d of %d values differ from K*x", bad, R * S * H);
  MOON_OK_(moon_combine(ctx, plan, lay.hidden_windows, lay.weight_windows, MOON_COMBINE_WEIGHTED,
                        d_out, NULL, st));
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  bad = 0;
  for (int i = 0; i < R * S * H; ++i) bad += out[i] != hidden[i];
  EXPECT(bad == 0, "weighted combine: %d of %d values differ from x", bad, R * S * H);

  /* a device-detected error and a host-detected one */
  topk[5] = E;
  HIP_OK(hipMemcpy(d_topk, topk, sizeof topk, hipMemcpyHostToDevice));
  MOON_OK_(moon_plan(ctx, d_topk, NULL, plan, st));
  EXPECT(moon_plan_status(plan, st) == MOON_ERR_BAD_EXPERT, "expert id E must be reported");
  moon_ctx* other = NULL;
  MOON_OK_(moon_ctx_create(&cfg, &other));
  EXPECT(moon_dispatch(other, plan, d_hidden, d_w, NULL, NULL, 0, st) == MOON_ERR_PLAN_MISMATCH,
         "a plan of another context must be refused");

  moon_plan_destroy(&plan);
  EXPECT(plan == NULL, "moon_plan_destroy must clear the handle");
  moon_ctx_destroy(&other);
  moon_ctx_destroy(&ctx);
  moon_ctx_destroy(&ctx); /* idempotent */
  EXPECT(ctx == NULL, "moon_ctx_destroy must clear the handle");
  HIP_OK(hipStreamDestroy(st));
  HIP_OK(hipFree(d_topk));
  HIP_OK(hipFree(d_hidden));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_pidx));
  if (failures) {
    printf("%d check(s) failed\n", failures);
    return 1;
  }
  printf("c abi ok (slots used %d)\n", slots_used);
  return 0;
}
