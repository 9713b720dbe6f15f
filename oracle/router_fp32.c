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
 * bit between implementations, so the layer's numeric contract fixes one. The
 * reduction index k is cut into groups of four consecutive values; group g =
 * k / 4 belongs to chain j = g mod 4. Each chain starts at +0 and takes its
 * terms in ascending k:
 *   c[j] = fmaf(h[t][k], W_r[k][e], c[j])   for every k with (k / 4) mod 4 == j
 *   logit[t][e] = (c[0] + c[1]) + (c[2] + c[3])   (float32 additions)
 *   (+ b_r[e], one more float32 addition, if a bias is given).
 * fmaf and the additions are correctly rounded, so this defines every bit of
 * every logit.
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
    float* out = logits + t * E;
    const float* ht = h + t * d;
    for (int64_t e = 0; e < E; ++e) {
      float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int64_t k = 0; k < d; ++k) {
        const int j = (int)((k / 4) % 4);
        c[j] = fmaf(ht[k], W_r[k * E + e], c[j]);
      }
      float l = (c[0] + c[1]) + (c[2] + c[3]);
      if (b_r != NULL) l = l + b_r[e];
      out[e] = l;
    }
  }
}
