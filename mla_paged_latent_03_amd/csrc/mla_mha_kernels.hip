// Dense un-absorbed MHA over the paged latent cache, for gfx950.
//
// The route the pages take for sparse-MLA batches whose sequences all fit in
// top-k (vLLM PR #47327 digest, "Summary" and "Implementation" item 2): the
// top-k list then holds every position, so the attention is dense, and
// un-absorbed multi-head attention replaces the absorbed MQA form.  With
// the DeepSeek-R1 head dims (128 no-rope + 64 rope for keys, 128 for
// values; vLLM PR #41778 digest, "Risks and impact" item 4) and per-head
// up-projections W_UK[h], W_UV[h] (128 x 512 each), cached latent c_j and
// rope r_j:
//     k_{h,j} = [ W_UK[h] c_j ; r_j ]     v_{h,j} = W_UV[h] c_j
//     out[b,t,h] = sum_j softmax_j(scale * <q[b,t,h], k_{h,j}>) v_{h,j}
// over the tokens query t sees (causal: positions 0 .. L_b - T + t).
//
// Two kernels:
//  * mha_expand_kernel: per (sequence, head, 32 tokens) a GEMM of the
//    gathered latents with [W_UK[h]; W_UV[h]] (256 x 512) on bf16 MFMA,
//    writing K_nope as [token][128] and V transposed as [128][token] into
//    the workspace, so that the attention reads both as contiguous rows;
//  * mha_attn_kernel: per (sequence, head, 32 queries) a flash-attention
//    loop over 32-key tiles: S^T = K Q^T (keys on the MFMA A side, the
//    192-wide query in registers on the B side), online softmax in the log2
//    domain with bf16 P, O^T += V^T P^T.  The S^T accumulator holds per lane
//    one query and 16 keys, which is directly P's B-operand layout; V^T's A
//    operand takes the keys in the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_mha_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ inline bf16x8_t load8(const __bf16* p) { return *(const bf16x8_t*)p; }

__device__ inline bf16x8_t zero8() { return bf16x8_t{}; }

// Physical address of token j's 576-wide cache row, or null past the
// sequence or for an out-of-range page.
__device__ inline const __bf16* token_row(const MhaParams& p, int b, int j, int L) {
  if (j >= L) return nullptr;
  const int pg = p.block_table[(int64_t)b * p.MB + (j >> 6)];
  if (pg < 0 || pg >= p.NB) return nullptr;
  return p.kv + ((int64_t)pg * 64 + (j & 63)) * 576;
}

// Sequence length clamped to the block table and to max_seq_len (the
// workspace holds Lpad >= max_seq_len tokens per sequence).
__device__ inline int seq_len(const MhaParams& p, int b) {
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.MB * 64 ? p.MB * 64 : L);
  return L > p.max_len ? p.max_len : L;
}

// ---------------------------------------------------------------------------
// Expansion.  Block (tile, head, sequence) of 4 waves; wave w computes output
// rows [64 w, 64 w + 64) of [W_UK[h]; W_UV[h]] times the 32 latents of the
// tile: D[m][token] = sum_k W[m][k] c_token[k], m on the MFMA A side, the
// tokens on the B side.  D's lane layout: token column l % 32, rows
// 8 (i / 4) + 4 (l / 32) + i % 4 of register i.
__global__ void __launch_bounds__(256) mha_expand_kernel(const MhaParams p) {
  const int b = blockIdx.z, h = blockIdx.y, j0 = blockIdx.x * 32;
  const int L = seq_len(p, b);
  if (j0 >= L) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int j = j0 + l32;
  const __bf16* x = token_row(p, b, j, L);
  const __bf16* wrow[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int m = 64 * wave + 32 * c + l32;
    wrow[c] = (m < 128 ? p.w_uk + ((int64_t)h * 128 + m) * 512 : p.w_uv + ((int64_t)h * 128 + (m - 128)) * 512);
  }
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll 4
  for (int ks = 0; ks < 32; ks++) {
    const int k = 16 * ks + 8 * hh;
    const bf16x8_t bx = x ? load8(x + k) : zero8();
#pragma unroll
    for (int c = 0; c < 2; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(wrow[c] + k), bx, acc[c], 0, 0, 0);
  }
  // Tokens past the sequence in this tile are stored as zeros: the
  // attention multiplies their V by zero weights, and stale workspace bytes
  // could be NaN.
  const bool real = j < L;
  const int64_t bh = (int64_t)b * p.H + h;
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int m0 = 64 * wave + 32 * c;
    if (m0 < 128) {
      __bf16* k_out = p.ws_k + (bh * p.Lpad + j) * 128 + m0;
#pragma unroll
      for (int a = 0; a < 4; a++) {
        const bf16x4_t v = {(__bf16)(real ? acc[c][4 * a] : 0.f), (__bf16)(real ? acc[c][4 * a + 1] : 0.f),
                            (__bf16)(real ? acc[c][4 * a + 2] : 0.f), (__bf16)(real ? acc[c][4 * a + 3] : 0.f)};
        *(bf16x4_t*)(k_out + 8 * a + 4 * hh) = v;
      }
    } else {
      __bf16* vt = p.ws_vt + (bh * 128 + (m0 - 128)) * p.Lpad + j;
#pragma unroll
      for (int i = 0; i < 16; i++)
        vt[(int64_t)(8 * (i / 4) + 4 * hh + i % 4) * p.Lpad] = (__bf16)(real ? acc[c][i] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention.  One wave per (32-query block, head, sequence).
__global__ void __launch_bounds__(64) mha_attn_kernel(const MhaParams p) {
  const int b = blockIdx.z, h = blockIdx.y, t0 = blockIdx.x * 32;
  const int L = seq_len(p, b);
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int t = t0 + l32;
  const bool t_ok = t < p.T;
  const int n_vis = t_ok ? max(0, L - p.T + t + 1) : 0;   // keys this lane's query sees
  int nv_max = n_vis;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) nv_max = max(nv_max, __shfl_xor(nv_max, d));

  // Query operand: B side, column = query, 8 features per lane half and step.
  bf16x8_t qreg[12];
  {
    const int64_t qr = ((int64_t)b * p.T + (t_ok ? t : 0)) * p.H + h;
#pragma unroll
    for (int ks = 0; ks < 12; ks++) {
      const int k = 16 * ks + 8 * hh;
      const bf16x8_t v = ks < 8 ? load8(p.q_nope + qr * 128 + k) : load8(p.q_pe + qr * 64 + (k - 128));
      qreg[ks] = t_ok ? v : zero8();
    }
  }
  const float c_qk = p.qk_scale;   // softmax scale * log2(e)
  float m = -INFINITY;             // running maximum (log2 domain), per query
  float l = 0.f;                   // this half's sum of the rounded weights
  f32x16_t o[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};   // O^T, dims 32 f .. 32 f + 31
  const int64_t bh = (int64_t)b * p.H + h;
  const __bf16* ks_base = p.ws_k + bh * p.Lpad * 128;
  const __bf16* vt_base = p.ws_vt + bh * 128 * p.Lpad;
  const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};

  for (int j0 = 0; j0 < nv_max; j0 += 32) {
    // K tile on the A side: row = key j0 + l32; K_nope from the workspace,
    // the rope part from the cache.
    const int j = j0 + l32;
    const __bf16* rope = token_row(p, b, j, L);
    const bool j_ok = j < L;
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 12; ks++) {
      const int k = 16 * ks + 8 * hh;
      bf16x8_t a;
      if (ks < 8) a = j_ok ? load8(ks_base + (int64_t)j * 128 + k) : zero8();
      else a = rope ? load8(rope + 512 + (k - 128)) : zero8();
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s, 0, 0, 0);
    }
    // Register i holds key j0 + 8 (i / 4) + 4 hh + i % 4 of this lane's query.
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = j0 + 8 * (i / 4) + 4 * hh + (i % 4);
      x[i] = key < n_vis ? s[i] * c_qk : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
    const float sh = m_new == -INFINITY ? 0.f : m_new;
    bf16x8_t pb[2];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const bf16x2_t pr = {(__bf16)__builtin_amdgcn_exp2f(x[i] - sh), (__bf16)__builtin_amdgcn_exp2f(x[i + 1] - sh)};
      ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
      pb[i / 8][i % 8] = pr[0];
      pb[i / 8][i % 8 + 1] = pr[1];
    }
    l = l * alpha + ls;
    m = m_new;
#pragma unroll
    for (int f = 0; f < 4; f++)
#pragma unroll
      for (int i = 0; i < 16; i++) o[f][i] *= alpha;
    // V^T on the A side: row = dim 32 f + l32; step s2 takes keys
    // 16 s2 + 4 hh + {0..3} and 16 s2 + 8 + 4 hh + {0..3}, the order of pb.
#pragma unroll
    for (int f = 0; f < 4; f++) {
      const __bf16* vrow = vt_base + (int64_t)(32 * f + l32) * p.Lpad + j0;
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) {
        const i32x2_t lo = *(const i32x2_t*)(vrow + 16 * s2 + 4 * hh);
        const i32x2_t hi = *(const i32x2_t*)(vrow + 16 * s2 + 8 + 4 * hh);
        const i32x4_t cat = {lo[0], lo[1], hi[0], hi[1]};
        o[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cat), pb[s2], o[f], 0, 0, 0);
      }
    }
  }

  const float l_tot = l + __shfl_xor(l, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (!t_ok) return;
  const int64_t orow = ((int64_t)b * p.T + t) * p.H + h;
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int a = 0; a < 4; a++) {
      const int d = 32 * f + 8 * a + 4 * hh;
      if (p.out_f32) {
        float* op = (float*)p.out + orow * 128 + d;
        *(float4*)op = float4{o[f][4 * a] * inv, o[f][4 * a + 1] * inv, o[f][4 * a + 2] * inv, o[f][4 * a + 3] * inv};
      } else {
        __bf16* op = (__bf16*)p.out + orow * 128 + d;
        const bf16x4_t v = {(__bf16)(o[f][4 * a] * inv), (__bf16)(o[f][4 * a + 1] * inv),
                            (__bf16)(o[f][4 * a + 2] * inv), (__bf16)(o[f][4 * a + 3] * inv)};
        *(bf16x4_t*)op = v;
      }
    }
  if (hh == 0 && p.lse) p.lse[orow] = empty ? -INFINITY : (m + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_mha(const MhaParams& p, hipStream_t stream) {
  void* args[] = {(void*)&p};
  if (p.Lpad > 0) {   // no cached token at all: the attention alone writes the empty rows
    const dim3 ge((unsigned)(p.Lpad / 32), (unsigned)p.H, (unsigned)p.B);
    const hipError_t e = hipLaunchKernel((const void*)&mha_expand_kernel, ge, dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 ga((unsigned)((p.T + 31) / 32), (unsigned)p.H, (unsigned)p.B);
  return hipLaunchKernel((const void*)&mha_attn_kernel, ga, dim3(64), args, 0, stream);
}

}  // namespace mla
