/*
 * oracle.h -- fp64 CPU reference for the Gated DeltaNet (GDN) core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code, header, table or helper.
 *
 * Sources (pages, cited by title and section):
 *   [P1] RL-Kernel pull request #469, "C6: GDN decode-step goldens and
 *        recurrent/conv state contract": sections "Summary", "How the golden
 *        relates to the kernel, and where it is not a transcription",
 *        "State ABI: index validation and the two NULL_BLOCK_ID contracts",
 *        "The conv half: coverage and the two mismatch mechanisms".
 *   [P4] vLLM pull request #53864 (CuteDSL GDN prefill, Newton-Schulz 3 -> 4
 *        rounds), section "Numerical root cause and fix".
 *   The gated delta rule itself, S_t = exp(g_t) S_{t-1} (I - b_t k_t k_t^T)
 *   + b_t v_t k_t^T and o_t = S_t q_t, is the standard form of the method the
 *   pages' kernels implement; no page prints it, so it is taken as written.
 *
 * Every array is a dense C-order fp64 array owned by the caller.  Caches are
 * updated in place.  All functions validate every index BEFORE they touch any
 * cache, and return a nonzero code (a bit set) without mutating anything when
 * an index is bad, mirroring the goldens that raise in [P1] "State ABI".
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error bits returned by every entry point (0 = success). */
#define ORACLE_ERR_SLOT_RANGE   1  /* an active slot index >= num_slots        */
#define ORACLE_ERR_SLOT_REPEAT  2  /* an active slot index appears twice        */
#define ORACLE_ERR_SEQLENS      4  /* cu_seqlens not monotone / last != total   */
#define ORACLE_ERR_ARGS         8  /* null pointer or nonsensical size          */

/* Flag bits (same meaning as the product's flags, defined independently). */
#define ORACLE_FLAG_SILU        1
#define ORACLE_FLAG_QK_L2NORM   2

/*
 * Causal depthwise conv1d update over runs of tokens, with per-slot left
 * context ([P1] "Summary", conv state [num_blocks, dim, W-1]; "The conv half").
 *
 *   x          [total_tokens, dim]
 *   cu_seqlens [n_seqs + 1] token offsets, or NULL: then n_seqs == total_tokens
 *              and row b is one token of sequence b (decode).
 *   slot_idx   [n_seqs]; <= 0 means inactive: zero output, cache untouched.
 *   conv_state [num_slots, dim, width-1], oldest tap first; rolled in place to
 *              the last width-1 raw inputs of the sequence.
 *   weight     [dim, width]; tap j multiplies X[t + j] where X is the state
 *              followed by the tokens, so tap width-1 is the current token.
 *   bias       [dim] or NULL.
 *   out        [total_tokens, dim]
 */
int oracle_conv_update(const double* x, int64_t total_tokens,
                       const int32_t* cu_seqlens, int32_t n_seqs,
                       const int32_t* slot_idx,
                       double* conv_state, int32_t num_slots,
                       const double* weight, const double* bias,
                       double* out, int32_t dim, int32_t width, int32_t flags);

/*
 * One decode token per row: conv update -> SiLU -> split [q | k | v] ->
 * L2-normalise q, k -> scale q -> gated delta rule on rec_state[slot] -> o.
 *
 *   mixed_qkv  [batch, 2*H*dk + HV*dv], channel order q, k, v, head-major.
 *   g, beta    [batch, HV]: log-decay (alpha = exp(g)) and write strength.
 *   rec_state  [num_slots, HV, dv, dk]  (S[v, k], k fastest).
 *   out        [batch, HV, dv]
 */
int oracle_decode_step(const double* mixed_qkv, const double* g, const double* beta,
                       const int32_t* slot_idx, int32_t batch,
                       double* conv_state, const double* conv_weight,
                       const double* conv_bias,
                       double* rec_state, int32_t num_slots, double* out,
                       int32_t num_k_heads, int32_t num_v_heads,
                       int32_t head_k_dim, int32_t head_v_dim, int32_t conv_width,
                       double scale, int32_t flags);

/*
 * Prefill on post-conv q, k, v, token by token (no chunking at all).
 *
 *   q, k       [total_tokens, H, dk]; v [total_tokens, HV, dv]
 *   g, beta    [total_tokens, HV]
 *   cu_seqlens [n_seqs + 1]; slot_idx [n_seqs] (<= 0: inactive sequence,
 *              zero outputs, state untouched).
 *   rec_state  [num_slots, HV, dv, dk]: read at the start of each sequence,
 *              final state written back.
 *   out        [total_tokens, HV, dv]
 */
int oracle_prefill(const double* q, const double* k, const double* v,
                   const double* g, const double* beta,
                   const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                   const int32_t* slot_idx,
                   double* rec_state, int32_t num_slots, double* out,
                   int32_t num_k_heads, int32_t num_v_heads,
                   int32_t head_k_dim, int32_t head_v_dim,
                   double scale, int32_t flags);

/*
 * Fused gating ([P1] "How the golden relates to the kernel", item 1): for
 * each row r and value head h,
 *   x = a[r, h] + dt_bias[h]
 *   softplus(x) = log(1 + exp(x)) for x <= 20, and x itself above 20 (the
 *                 kernel's threshold branch)
 *   g[r, h]    = -exp(A_log[h]) * softplus(x)
 *   beta[r, h] = 1 / (1 + exp(-b[r, h]))           (sigmoid)
 *
 *   a, b       [rows, HV]; A_log, dt_bias [HV]; g, beta [rows, HV] (outputs)
 */
int oracle_gating(const double* a, const double* b, const double* A_log,
                  const double* dt_bias, int64_t rows, int32_t num_v_heads,
                  double* g, double* beta);

/*
 * Gated RMSNorm of the GDN block's output ([P1] "Latest Status": zero-centred
 * and gated RMSNorm operators with SiLU or sigmoid gating and a weight
 * offset; the pages print no formula, so the plain definition is taken):
 * for each row r of `dim` values,
 *   rms     = sqrt(sum_j x[r, j]^2 / dim + eps)
 *   out[r, j] = (x[r, j] / rms) * w'[j] * act(z[r, j])
 * with w' = weight + 1 under ORACLE_NORM_ZERO_CENTRED (else weight), act =
 * SiLU (y / (1 + e^-y)) or, under ORACLE_NORM_GATE_SIGMOID, 1 / (1 + e^-y);
 * z == NULL means no gate (act = 1).  The norm comes before the gate.
 */
#define ORACLE_NORM_GATE_SIGMOID 1
#define ORACLE_NORM_ZERO_CENTRED 2
int oracle_gated_rmsnorm(const double* x, const double* z, const double* weight,
                         int64_t rows, int32_t dim, double eps, int32_t flags, double* out);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
