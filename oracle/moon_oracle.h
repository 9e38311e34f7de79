/*
 * moon_oracle.h — plain, single-threaded CPU oracle for balanced MoE
 * expert-parallel planning, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may use it.  It shares no source, header, table or
 * helper with the GPU library; the two are compared on identical seeded
 * inputs.
 *
 * What it computes follows the "MoonEP Public API Visual Guide"
 * (sections Buffer.dispatch, Buffer.combine, Buffer.prefetch_weight,
 * Buffer.reduce_grad, MoonEPCommPlan) and the MoonEP README (Performance: maxvio equation;
 * Integration: How to set B).  Where the pages state only guarantees
 * (perfect balance, slot experts from one remote home rank) the oracle takes
 * one deterministic reading, written out in the .cpp next to each step.
 *
 * Conventions (all arrays C-contiguous, caller-owned host memory):
 *   R ranks, E experts (E % R == 0, Eg = E/R experts homed per rank,
 *   expert e is homed on rank e / Eg), K routes per token, S tokens per rank,
 *   H hidden width, B prefetch slots per rank, P = token_padding.
 *   C = S*K routes per rank; NvS = per-rank dispatched-row capacity.
 *   topk       [R,S,K] int32     expert id of route (r,s,k)
 *   dst        [R,S*K] int32     +G primary, -(G+1) locally deduplicated;
 *                                 G = u*NvS + local row on destination rank u
 *   etc        [R,B]   int32     experts_to_copy (-1 = unused slot)
 *   zfr        [R,E+B,2] int32   zero_fill_ranges, half-open local rows
 *   rstats     [R,2]   int32     remote_stats (slots used, routes in slots)
 *   dup_groups [R,NvS,3] int32   (primary local row, first dup_loffs index, m)
 *   dup_loffs  [R,NvS] int32     duplicate local rows
 *   dup_counts [R,2]   int32     (groups, duplicates) valid prefix sizes
 *   cu         [R,E+B] int32     inclusive padded end offset per group
 *   bf16 values are passed as their uint16 bit patterns.
 *
 * Status codes (returned; outputs are undefined unless 0):
 *    0 ok, -1 invalid argument, -7 expert id out of range,
 *   -8 slot budget exceeded, -9 tokens_per_expert disagrees with the routes.
 *   Priority when several apply: -7, then -9, then -8.
 */
#ifndef MOON_ORACLE_H
#define MOON_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-rank dispatched-row capacity NvS (reading of the capacity rule). */
int32_t orc_nvs(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B, int32_t P);

/* Balancing step alone on integer rank loads L[R] with target C per rank.
 * Outputs keep[R], donor[R] (-1 if none), take[R]. Returns 0, or -1 if
 * sum(L) != R*C or any L < 0. */
int32_t orc_alias(int32_t R, int64_t C, const int64_t* L,
                  int64_t* keep, int32_t* donor, int64_t* take);

/* Full plan.  tpe [R,E] may be NULL.  dbg (may be NULL) receives, in order:
 * cnt[R*E], T[E], Pe[E], L[R], keep[R], donor[R], take[R], seg_a[R] as int64. */
int32_t orc_plan(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B, int32_t P,
                 const int32_t* topk, const int32_t* tpe,
                 int32_t* dst, int32_t* etc, int32_t* zfr, int32_t* rstats,
                 int32_t* dup_groups, int32_t* dup_loffs, int32_t* dup_counts,
                 int32_t* cu, int64_t* dbg);

/* Dispatch with a plan: win [R*NvS,H] bf16 bits, wwin [R*NvS] fp32.
 * w may be NULL (then wwin is not touched). Rows past the last group of a
 * rank are not written. */
int32_t orc_dispatch(int32_t R, int32_t E, int32_t K, int32_t S, int32_t H, int32_t B,
                     int32_t NvS, const int32_t* dst, const int32_t* zfr,
                     const uint16_t* hidden, const float* w,
                     uint16_t* win, float* wwin);

/* For every window row: the route id r*S*K + s*K + k that lands there,
 * -1 for a zero-filled padding row, -2 for a row no group covers. */
int32_t orc_row_sources(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B,
                        int32_t NvS, const int32_t* dst, const int32_t* zfr,
                        const int32_t* cu, int64_t* src);

/* Combine over all tokens.  y [R*NvS,H] bf16 bits; wnvs [R*NvS] (needed when
 * weighted != 0).  out [R,S,H] bf16 bits: the fp32 sum of c_k * y_k, ascending
 * k, every product and addition rounded to fp32, rounded once to bf16 (fp32
 * is the precision the target for this path fixes for the K-sum; the pages
 * state fp32 for the duplicate prologue's fold only, and the order and the
 * single rounding are a reading).  wsk_out [R,S,K] and acc [R,S,H] (the
 * float64 sum of the same terms, the exact reference, computed only when
 * given) may be NULL. */
int32_t orc_combine(int32_t R, int32_t K, int32_t S, int32_t H, int32_t NvS,
                    const int32_t* dst, const uint16_t* y, const float* wnvs,
                    int32_t weighted, uint16_t* out, float* wsk_out, double* acc);

/* Combine for a sample of tokens whose needed rows are supplied compactly:
 * dst_tok [n,K] are the tokens' dst entries, rows [M] the sorted global rows
 * present in yrows [M,H] and wrows [M].  Returns -1 if a needed row is absent. */
int32_t orc_combine_rows(int32_t n, int32_t K, int32_t H, const int32_t* dst_tok,
                         int64_t M, const int64_t* rows, const uint16_t* yrows,
                         const float* wrows, int32_t weighted,
                         uint16_t* out, float* wsk_out, double* acc);

/* Combine with the duplicate prologue: for every token and destination rank
 * holding m >= 2 of its routes, the m rows are first summed in fp32
 * (ascending k, c_k = w_nvs[row] when weighted, else 1) and rounded to bf16
 * into the primary row; the main sum then takes primary routes only, a
 * folded primary with coefficient 1, in fp32 as orc_combine (acc: float64),
 * rounded once.  folded (may be NULL) [R*NvS,H] receives y with the folded
 * primary rows. */
int32_t orc_combine_prologue(int32_t R, int32_t K, int32_t S, int32_t H, int32_t NvS,
                             const int32_t* dst, const uint16_t* y, const float* wnvs,
                             int32_t weighted, uint16_t* out, float* wsk_out, double* acc,
                             uint16_t* folded);

/* The same for n sampled tokens, like orc_combine_rows; folded_rows [M,H]
 * receives yrows with the folded primary rows. */
int32_t orc_combine_prologue_rows(int32_t n, int32_t K, int32_t H, int32_t NvS,
                                  const int32_t* dst_tok, int64_t M, const int64_t* rows,
                                  const uint16_t* yrows, const float* wrows, int32_t weighted,
                                  uint16_t* out, float* wsk_out, double* acc,
                                  uint16_t* folded_rows);

/* Prefetch index: out [R,B,2] = (owner rank, rank-local row) or (-1,-1). */
int32_t orc_prefetch_index(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t* out);

/* Weight prefetch for n tensors: slots[t] [R,B,row_bytes[t]] bytes, slot
 * (u,j) <- experts[t] row etc[u][j] ([E,row_bytes[t]]); unused slots keep
 * their bytes. */
int32_t orc_prefetch_weight(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t n,
                            const uint8_t* const* experts, uint8_t* const* slots,
                            const int64_t* row_bytes);

/* Gradient reduction for n fp32 tensors: grads[t] [E,L] row e <- row e +
 * slot gradients of the slots holding e (ranks ascending, fp32 adds);
 * slot_grads[t] [R,B,L] used slots <- 0. */
int32_t orc_reduce_grad(int32_t R, int32_t E, int32_t B, const int32_t* etc, int32_t n,
                        float* const* grads, float* const* slot_grads, const int64_t* row_elems);

/* Nearest bf16 (ties to even) of a double, as bits.  Exposed for tests. */
uint16_t orc_bf16_from_double(double v);

#ifdef __cplusplus
}
#endif
#endif
