// Internal declarations shared by the host launcher and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatentDim = 512;
constexpr int kRopeDim = 64;
constexpr int kTokenDim = 576;
constexpr int kPage = 64;
constexpr int kPartialWidth = kLatentDim + 1;   // normalized outputs, then the chunk's lse
constexpr int kSparseChunkMax = 1024;           // top-k entries one workgroup handles
constexpr int kDensePagesMax = 1024;            // pages one workgroup handles (65536 tokens)
constexpr int kDefaultCUs = 256;                // MI355X compute units (when no device can be asked)
constexpr int kBalanceMaxBatch = 1024;          // largest batch whose split lengths are balanced on the device

struct PartialParams {
  const uint8_t* q_nope;        // [B, T, H, 512] bf16 or e4m3 bytes
  const uint8_t* q_pe;          // [B, T, H, 64]
  const uint8_t* kv;            // [NB, 64, 576]
  const int32_t* block_table;   // [B, MB]
  const int32_t* seq_lens;      // [B]
  const int32_t* topk;          // [B, T, K] (sparse) or null
  int B, T, H, R, NB, MB, K;
  int n_rb;                     // row blocks per (sequence, split)
  int n_hb;                     // sparse: head blocks per draft token
  int chunk;                    // dense: pages per split; sparse: indices per split
  int S;                        // splits (partial slots per sequence)
  int n_units;                  // B * S * n_rb
  int balance;                  // dense, S > 1: length-balanced pieces instead of fixed chunks
  int n_target;                 // balanced: pieces the batch may be cut into (one round of workgroups)
  int lpt;                      // balanced, B <= 64: number pieces longest first (two rounds)
  int max_pages;                // balanced: pages of max_seq_len (longer sequences are cut there)
  float qk_scale;               // softmax_scale * log2(e) [* q_scale * kv_scale]
  float out_scale;              // kv_scale (fp8) or 1
  void* out;                    // [B, T, H, 512] bf16 / f32 (one split)
  int out_f32;
  float* lse;                   // [B, T, H] or null (one split)
  float* ws;                    // [B, R, S, 513] (more than one split)
  // Single launch (more than one split, every unit resident at once): the
  // units of a (sequence, row block) meet at two words of `sync` and then
  // merge the group's rows themselves.  sync: [groups][2] words of
  // (epoch << 16 | count); epoch: this call's number (48 bits).
  unsigned long long* sync;
  unsigned long long epoch;
  int fused;
};

struct MergeParams {
  const float* ws;              // [n_rows, S, 513]
  int64_t n_rows;               // B * R
  int S;
  void* out;
  int out_f32;
  float* lse;
};

// fp8 work units planned at most this many tokens long use the residual
// product from the start.  (Without it, units a little over 8192 tokens
// measured row errors up to 0.025 against the oracle on N(0,1) data, close
// to the 3e-2 bound; from about 16000 tokens on, 0.006.)  Longer units run
// without it and rerun a unit with it when its weights need it.
constexpr int kFp8ResidualMaxUnitTokens = 16384;

// Size of the static split workspace behind mla_decode_fp8_noalloc.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

// Device address of this GPU's static workspace (looked up once per device).
hipError_t static_scratch(void** ptr);

// Workgroups of the partial-kernel variant (fp8, sparse, waves, residual
// product) that one compute unit of the current device holds at once, as
// the runtime reports it; 0 when it cannot be asked.
int partial_kernel_occupancy(bool fp8, bool sparse, int rg, bool resid);

hipError_t launch_partial_kernel(const PartialParams& p, bool fp8, bool sparse, int rg, bool resid, int grid,
                                 hipStream_t stream);
hipError_t launch_merge_kernel(const MergeParams& p, hipStream_t stream);

}  // namespace mla
