/*
 * Oracle (test infrastructure only; never linked into the product library).
 *
 * Router logits of a top-K MoE layer in float32, in the canonical order.
 *
 * The router is a linear map followed by a softmax over the experts
 * (Lensa ML explainer "Mixture of Experts", Step 2 of 6: The Router; Curionode
 * "Mixture of Experts." Plate VII.4, section "Parameters you hold, parameters
 * you use"), and it is kept in float32 (Arjun Jaggi, "Mixture of Experts in
 * LLMs: How Sparse Models Scale", section "Switch Transformers").
 *
 * The pages do not fix a summation order. Expert selection must agree bit for
 * bit between implementations, so the layer's numeric contract fixes one:
 *   acc = +0.0f;  for k = 0 .. d-1 ascending:  acc = fmaf(h[t][k], W_r[k][e], acc);
 *   logit[t][e] = acc (+ b_r[e], one separate float32 addition, if a bias is given).
 * fmaf is correctly rounded, so this defines every bit of every logit.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math, no
 * contraction: every rounding is the one written here).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

void oracle_router_logits_f32(const float* h, const float* W_r, const float* b_r,
                              int64_t T, int64_t d, int64_t E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    float* acc = logits + t * E;
    for (int64_t e = 0; e < E; ++e) acc[e] = 0.0f;
    const float* ht = h + t * d;
    /* k outermost so that each (t, e) chain still runs k = 0, 1, 2, ... in order. */
    for (int64_t k = 0; k < d; ++k) {
      const float hk = ht[k];
      const float* wk = W_r + k * E;
      for (int64_t e = 0; e < E; ++e) acc[e] = fmaf(hk, wk[e], acc[e]);
    }
    if (b_r != NULL) {
      for (int64_t e = 0; e < E; ++e) acc[e] = acc[e] + b_r[e];
    }
  }
}
