/*
 * CPU fp64 oracle for absorbed multi-head latent attention (MLA) decode over a
 * paged latent KV cache.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and
 * the CPU-baseline leg of the benchmark may call it; the product path never
 * does.  It shares no code, header or table with the HIP library.
 *
 * What it computes (plain loops, fp64, no blocking, no fusion):
 *
 *   The pages describe decode for DeepSeek-R1-shaped MLA as multi-query
 *   attention over one shared latent per cached token ("MQA" decode:
 *   vLLM PR #46819 digest, "Implementation" item 1 and "Key files";
 *   vLLM PR #47327 digest, "Motivation").  Each cached token j of sequence b
 *   is one 576-wide vector: a 512-wide latent c_j followed by a 64-wide rope
 *   part r_j (kv_lora_rank + 1 is the partial width in the Triton workspace,
 *   vLLM PR #46819 digest, "Key code excerpt").  The token lives in page
 *   block_table[b][j / P], slot j % P.  For query row (b, t, h):
 *
 *     s_j   = scale * ( <q_nope[b,t,h], c_j> + <q_pe[b,t,h], r_j> )
 *     m     = max_j s_j ;  Z = sum_j exp(s_j - m)
 *     out   = sum_j exp(s_j - m) * c_j / Z      (values are the latent itself)
 *     lse   = m + ln Z                          (natural log, scale included)
 *
 *   over the visible list of row (b, t):
 *     dense : j = 0 .. L_b - T + t  (query t of a T-token draft sees the
 *             cache up to and including its own position; causal inside the
 *             draft; MTP decode, vLLM PR #41778 digest, "Motivation")
 *     sparse: the entries of topk_indices[b, t, 0..K) that lie in [0, L_b),
 *             in the order given (index_topk per token, vLLM PR #47327
 *             digest, "Key code excerpt"); -1 padding and any other
 *             out-of-range entry is skipped.
 *   An empty visible list gives out = 0 and lse = -inf.
 *
 *   Inputs are dequantized first: bf16 values exactly; OCP e4m3fn bytes by
 *   the format definition (1 sign, 4 exponent bits with bias 7, 3 mantissa
 *   bits, subnormals m * 2^-9, 0x7F / 0xFF NaN, no infinities) times the
 *   per-tensor scale (q_scale for q_nope and q_pe, kv_scale for the cache).
 *   FP8 decode needs dequant scales passed in (vLLM PR #41778 digest,
 *   "Implementation" item 1 and "Risks" item 3).
 *
 *   Optional split mode (num_splits > 0): the visible list is cut into
 *   num_splits contiguous chunks of ceil(n / num_splits) entries; each chunk
 *   gives a normalized partial (O_s, lse_s) and the partials are merged by
 *   log-sum-exp:  lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) O_s
 *   (two-stage split-KV with a kv_lora_rank + 1 wide partial, vLLM PR #46819
 *   digest, "Implementation" items 1-3).  It exists to check the merge.
 *
 * Every input index is bounds-checked; a bad one returns an error code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D_LATENT 512
#define ORC_D_ROPE 64
#define ORC_D_TOKEN 576

enum { ORC_BF16 = 0, ORC_E4M3FN = 1, ORC_F64 = 2 };
enum {
  ORC_OK = 0,
  ORC_BAD_ARG = -1,
  ORC_BAD_BLOCK = -2,
  ORC_NO_MEMORY = -3
};

/* OCP FP8 E4M3 ("fn": finite, no infinities) decoded from its definition. */
double orc_e4m3fn_to_double(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int exp_bits = (byte >> 3) & 0xF;
  int man_bits = byte & 0x7;
  double mag;
  if (exp_bits == 0xF && man_bits == 0x7) return NAN; /* S.1111.111 */
  if (exp_bits == 0)
    mag = ldexp((double)man_bits, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + man_bits / 8.0, exp_bits - 7);
  return sign ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t idx, double scale) {
  switch (dtype) {
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
    case ORC_E4M3FN: return orc_e4m3fn_to_double(((const uint8_t*)base)[idx]) * scale;
    default: return ((const double*)base)[idx];
  }
}

/* Softmax-weighted latent sum of one row over list[0..n): writes the
 * normalized output and the log-sum-exp.  Two passes over the list: logits
 * and their maximum first, then the exponentials. */
static void attend_list(const void* q_nope, const void* q_pe, int q_dtype, double q_scale,
                        int64_t q_row, const void* kv, int kv_dtype, double kv_scale,
                        const int64_t* tok_off, int64_t n, double scale, double* logits,
                        double* out, double* lse) {
  double qn[ORC_D_LATENT], qp[ORC_D_ROPE];
  for (int d = 0; d < ORC_D_LATENT; d++) qn[d] = load_elem(q_nope, q_dtype, q_row * ORC_D_LATENT + d, q_scale);
  for (int d = 0; d < ORC_D_ROPE; d++) qp[d] = load_elem(q_pe, q_dtype, q_row * ORC_D_ROPE + d, q_scale);
  for (int d = 0; d < ORC_D_LATENT; d++) out[d] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t i = 0; i < n; i++) {
    double dot = 0.0;
    for (int d = 0; d < ORC_D_LATENT; d++) dot += qn[d] * load_elem(kv, kv_dtype, tok_off[i] + d, kv_scale);
    for (int d = 0; d < ORC_D_ROPE; d++)
      dot += qp[d] * load_elem(kv, kv_dtype, tok_off[i] + ORC_D_LATENT + d, kv_scale);
    logits[i] = scale * dot;
    if (logits[i] > m) m = logits[i];
  }
  double z = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double p = exp(logits[i] - m);
    z += p;
    for (int d = 0; d < ORC_D_LATENT; d++) out[d] += p * load_elem(kv, kv_dtype, tok_off[i] + d, kv_scale);
  }
  for (int d = 0; d < ORC_D_LATENT; d++) out[d] /= z;
  *lse = m + log(z);
}

/*
 * Evaluate rows of the decode.  Row id = (b * T + t) * H + h, the memory
 * order of q_nope [B, T, H, 512].  rows == NULL means all B*T*H rows in order.
 * out: [n_rows, 512] fp64, lse: [n_rows] fp64.
 * topk_indices == NULL selects the dense causal visible list.
 */
int mla_oracle_decode(const void* q_nope, const void* q_pe, int q_dtype, double q_scale,
                      const void* kv, int kv_dtype, double kv_scale, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* topk_indices, int K, int B, int T,
                      int H, int NB, int P, int MB, double softmax_scale, int num_splits,
                      const int64_t* rows, int64_t n_rows, double* out, double* lse,
                      int n_threads) {
  if (B < 0 || T < 1 || H < 1 || NB < 0 || P < 1 || MB < 0 || num_splits < 0) return ORC_BAD_ARG;
  if (q_dtype < ORC_BF16 || q_dtype > ORC_F64 || kv_dtype < ORC_BF16 || kv_dtype > ORC_F64) return ORC_BAD_ARG;
  if (topk_indices != NULL && K < 0) return ORC_BAD_ARG;
  const int64_t total_rows = (int64_t)B * T * H;
  if (rows == NULL) n_rows = total_rows;
  for (int64_t i = 0; rows != NULL && i < n_rows; i++)
    if (rows[i] < 0 || rows[i] >= total_rows) return ORC_BAD_ARG;
  int status = ORC_OK;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
  {
    int64_t cap = 0;
    int64_t* tok_off = NULL;
    double* logits = NULL;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; i++) {
      int64_t row = rows ? rows[i] : i;
      int t = (int)((row / H) % T);
      int b = (int)(row / ((int64_t)H * T));
      int L = seq_lens[b];
      int64_t n_cand = topk_indices ? K : (int64_t)L - T + t + 1;
      if (n_cand < 0) n_cand = 0;
      if (n_cand > cap) {
        free(tok_off);
        free(logits);
        cap = n_cand;
        tok_off = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
        logits = (double*)malloc(sizeof(double) * (size_t)cap);
        if (!tok_off || !logits) {
#pragma omp atomic write
          status = ORC_NO_MEMORY;
          cap = 0;
          continue;
        }
      }
      /* Visible list -> element offsets of each token vector in the cache. */
      int64_t n = 0;
      int bad = 0;
      for (int64_t c = 0; c < n_cand; c++) {
        int64_t j;
        if (topk_indices) {
          j = topk_indices[((int64_t)b * T + t) * K + c];
          if (j < 0 || j >= L) continue;
        } else {
          j = c;
        }
        int64_t page_slot = j / P;
        if (page_slot >= MB) { bad = 1; break; }
        int64_t page = block_table[(int64_t)b * MB + page_slot];
        if (page < 0 || page >= NB) { bad = 1; break; }
        tok_off[n++] = (page * P + j % P) * ORC_D_TOKEN;
      }
      if (bad) {
#pragma omp atomic write
        status = ORC_BAD_BLOCK;
        continue;
      }
      double* o = out + i * ORC_D_LATENT;
      if (num_splits <= 0) {
        attend_list(q_nope, q_pe, q_dtype, q_scale, row, kv, kv_dtype, kv_scale, tok_off, n,
                    softmax_scale, logits, o, &lse[i]);
        continue;
      }
      /* Split mode: contiguous chunks, each normalized, merged by LSE. */
      int64_t chunk = (n + num_splits - 1) / num_splits;
      double* parts = (double*)malloc(sizeof(double) * (size_t)num_splits * (ORC_D_LATENT + 1));
      if (!parts) {
#pragma omp atomic write
        status = ORC_NO_MEMORY;
        continue;
      }
      double* lse_s = parts + (size_t)num_splits * ORC_D_LATENT;
      double lse_max = -INFINITY;
      for (int s = 0; s < num_splits; s++) {
        int64_t lo = (int64_t)s * chunk, hi = lo + chunk;
        if (lo > n) lo = n;
        if (hi > n) hi = n;
        attend_list(q_nope, q_pe, q_dtype, q_scale, row, kv, kv_dtype, kv_scale, tok_off + lo,
                    hi - lo, softmax_scale, logits, parts + (size_t)s * ORC_D_LATENT, &lse_s[s]);
        if (lse_s[s] > lse_max) lse_max = lse_s[s];
      }
      for (int d = 0; d < ORC_D_LATENT; d++) o[d] = 0.0;
      double lse_all = -INFINITY;
      if (lse_max != -INFINITY) {
        double zsum = 0.0;
        for (int s = 0; s < num_splits; s++) zsum += exp(lse_s[s] - lse_max);
        lse_all = lse_max + log(zsum);
        for (int s = 0; s < num_splits; s++) {
          if (lse_s[s] == -INFINITY) continue;
          double w = exp(lse_s[s] - lse_all);
          for (int d = 0; d < ORC_D_LATENT; d++) o[d] += w * parts[(size_t)s * ORC_D_LATENT + d];
        }
      }
      free(parts);
      lse[i] = lse_all;
    }
    free(tok_off);
    free(logits);
  }
  return status;
}
