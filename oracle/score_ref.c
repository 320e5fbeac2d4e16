/*
 * score_ref.c - a second fp64 implementation of the window attention score,
 * written independently of oracle/kvs.py (TEST INFRASTRUCTURE ONLY: only the
 * test suite loads it, to check the NumPy oracle against it).
 *
 * The definition is the one the ClusterAttn note gives for feature aggregation
 * ("Background and key observations": window logits, causal window mask,
 * softmax over the keys, column sum over the window rows) and the CLAA post
 * for the FastKV / per-layer window score ("Three representative token-ranking
 * methods", "Three design decisions": summed over heads); the DELTA note's
 * maximum over heads ("Key design 2") is GROUP_MAX.  Plain loops, one row at
 * a time: the row's logits in fp64 (dot products accumulated in ascending
 * channel order), its maximum, the sum of exp(s - max), then every visible
 * column receives exp(s - max) / sum.
 *
 * Q: bf16 bits [H_q][W][d_k]; K: bf16 bits [H_kv][L][d_k]; query head h reads
 * KV head h / (H_q / H_kv); row j sits at position q_pos0 + j and sees keys
 * t <= q_pos0 + j.  heads: 0 per query head [H_q][L], 1 sum over each group's
 * heads [H_kv][L], 2 maximum over them [H_kv][L], 3 sum over every head [1][L].
 * Returns 0, or -1 on bad arguments or when memory runs out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int kvs_ref_score(const uint16_t* Q, const uint16_t* K, int L, int W, int d_k, int H_q, int H_kv,
                  long long q_pos0, int heads, double scale, double* out) {
  if (L < 1 || W < 1 || d_k < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || q_pos0 < 0) return -1;
  if (heads < 0 || heads > 3) return -1;
  const int G = H_q / H_kv;
  double* col = (double*)malloc(sizeof(double) * (size_t)L);    /* one head's column sums */
  double* logit = (double*)malloc(sizeof(double) * (size_t)L);  /* one row's logits */
  if (!col || !logit) {
    free(col);
    free(logit);
    return -1;
  }
  const int rows_out = heads == 0 ? H_q : heads == 3 ? 1 : H_kv;
  for (size_t i = 0; i < (size_t)rows_out * L; ++i) out[i] = heads == 2 ? -INFINITY : 0.0;
  for (int h = 0; h < H_q; ++h) {
    const int g = h / G;
    for (int t = 0; t < L; ++t) col[t] = 0.0;
    for (int j = 0; j < W; ++j) {
      long long last = q_pos0 + j;              /* last visible key */
      int vis = last >= L - 1 ? L : (int)last + 1;
      const uint16_t* q = Q + ((size_t)h * W + j) * d_k;
      double mx = -INFINITY;
      for (int t = 0; t < vis; ++t) {
        const uint16_t* k = K + ((size_t)g * L + t) * d_k;
        double dot = 0.0;
        for (int c = 0; c < d_k; ++c) dot += bf16_value(q[c]) * bf16_value(k[c]);
        logit[t] = scale * dot;
        if (logit[t] > mx) mx = logit[t];
      }
      double z = 0.0;
      for (int t = 0; t < vis; ++t) z += exp(logit[t] - mx);
      for (int t = 0; t < vis; ++t) col[t] += exp(logit[t] - mx) / z;
    }
    double* o = out + (size_t)(heads == 0 ? h : heads == 3 ? 0 : g) * L;
    for (int t = 0; t < L; ++t) {
      if (heads == 2)
        o[t] = col[t] > o[t] ? col[t] : o[t];
      else
        o[t] += col[t];
    }
  }
  free(col);
  free(logit);
  return 0;
}
