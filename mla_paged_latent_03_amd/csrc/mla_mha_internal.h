// Internal declarations of the dense un-absorbed MHA route (host launcher and
// its two gfx950 kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Tokens per expansion block; the workspace pads each sequence to a multiple.
constexpr int kMhaTokPad = 128;

struct MhaParams {
  const __bf16* q_nope;        // [B, T, H, 128]
  const __bf16* q_pe;          // [B, T, H, 64]
  const __bf16* kv;            // [NB, 64, 576]
  const int32_t* block_table;  // [B, MB]
  const int32_t* seq_lens;     // [B]
  const __bf16* w_uk;          // [H, 128, 512]
  const __bf16* w_uv;          // [H, 128, 512]
  int B, T, H, NB, MB;
  int max_len;                 // max_seq_len (lengths are clamped to it)
  int Lpad;                    // max_len rounded up to kMhaTokPad: tokens per (sequence, head) in the workspace
  float qk_scale;              // softmax_scale * log2(e)
  __bf16* ws_k;                // [B, H, Lpad, 128]  K_nope = W_UK c
  __bf16* ws_vt;               // [B, H, 128, Lpad]  V^T = (W_UV c)^T, keys of each group of 16 in the
                               // order 0-3, 8-11, 4-7, 12-15 (the order a lane holds P in)
  void* out;                   // [B, T, H, 128] bf16 / f32
  int out_f32;
  float* lse;                  // [B, T, H] or null
};

// Both kernels of one call, in order, on `stream`.
hipError_t launch_mha(const MhaParams& p, hipStream_t stream);

}  // namespace mla
