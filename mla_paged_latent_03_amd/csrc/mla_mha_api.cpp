// C ABI of the dense un-absorbed MHA route: argument checks, workspace
// sizing and the two launches.  Declarations and contracts: mla_decode.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/mla_decode.h"
#include "mla_mha_internal.h"

namespace {

bool mha_dims_ok(int B, int T, int H, int max_seq_len) {
  return B >= 0 && B <= 65535 && T >= 1 && T <= MLA_MHA_MAX_Q_LEN && H >= 1 && H <= 1024 && max_seq_len >= 0 &&
         max_seq_len <= (1 << 24);
}

int64_t padded_len(int max_seq_len) {
  return ((int64_t)max_seq_len + mla::kMhaTokPad - 1) / mla::kMhaTokPad * mla::kMhaTokPad;
}

// Workgroups of each launch (one per 128 tokens or 128 queries of every
// (sequence, head)) must fit a 32-bit grid.
bool grid_ok(int B, int T, int H, int max_seq_len) {
  const int64_t pairs = (int64_t)B * H;
  const int64_t lim = (int64_t)1 << 30;
  return pairs * (padded_len(max_seq_len) / mla::kMhaTokPad) <= lim && pairs * ((T + 127) / 128) <= lim;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

}  // namespace

extern "C" {

size_t mla_dense_mha_workspace_size(int batch, int num_heads, int max_seq_len) {
  if (!mha_dims_ok(batch, 1, num_heads, max_seq_len)) return 0;
  return (size_t)2 * batch * num_heads * padded_len(max_seq_len) * 128 * sizeof(uint16_t);
}

mla_status_t mla_dense_mha(const void* q_nope, const void* q_pe, const void* kv_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const void* w_uk, const void* w_uv, int batch, int q_len,
                           int num_heads, int num_blocks, int block_size, int max_blocks_per_seq, int max_seq_len,
                           float softmax_scale, void* out, int out_dtype, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  if (!mha_dims_ok(batch, q_len, num_heads, max_seq_len)) return MLA_ERR_INVALID_ARGUMENT;
  if (!grid_ok(batch, q_len, num_heads, max_seq_len)) return MLA_ERR_UNSUPPORTED;
  if (num_blocks < 0 || max_blocks_per_seq < 1 || (int64_t)num_blocks * MLA_BLOCK_SIZE > INT32_MAX)
    return MLA_ERR_INVALID_ARGUMENT;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !block_table || !seq_lens || !w_uk || !w_uv || !out || (num_blocks > 0 && !kv_cache))
    return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_cache) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(out))
    return MLA_ERR_INVALID_ARGUMENT;
  const size_t need = mla_dense_mha_workspace_size(batch, num_heads, max_seq_len);
  if (need > 0) {
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARGUMENT;
  }
  mla::MhaParams p{};
  p.q_nope = (const __bf16*)q_nope;
  p.q_pe = (const __bf16*)q_pe;
  p.kv = (const __bf16*)kv_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.w_uk = (const __bf16*)w_uk;
  p.w_uv = (const __bf16*)w_uv;
  p.B = batch;
  p.T = q_len;
  p.H = num_heads;
  p.NB = num_blocks;
  p.MB = max_blocks_per_seq;
  p.max_len = max_seq_len;
  p.Lpad = (int)padded_len(max_seq_len);
  p.qk_scale = softmax_scale * 1.4426950408889634f;
  const size_t half = need / 2;
  p.ws_k = need ? (__bf16*)workspace : nullptr;
  p.ws_vt = need ? (__bf16*)((uint8_t*)workspace + half) : nullptr;
  p.out = out;
  p.out_f32 = out_dtype == MLA_OUT_F32;
  p.lse = lse;
  if (mla::launch_mha(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
