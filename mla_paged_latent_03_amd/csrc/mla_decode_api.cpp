// C ABI of libmla_decode.so: argument checks, the split planner, workspace
// sizing and the two launches.  Declarations and contracts: mla_decode.h.
#include "../../include/mla_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "mla_decode_internal.h"

namespace {

using mla::kPartialWidth;
using mla::kDensePagesMax;
using mla::kSparseChunkMax;

struct Plan {
  int R = 0;        // query rows per sequence, T * H
  int rg = 1;       // waves per workgroup (32 rows each)
  int n_rb = 1;     // row blocks per (sequence, split)
  int n_hb = 1;     // sparse: head blocks per draft token
  int S = 1;        // KV splits (partial slots per sequence)
  int chunk = 1;    // dense: pages per split; sparse: indices per split
  bool balance = false;   // dense, S > 1: length-balanced pieces (cut on the device)
  bool lpt = false;       // balanced over two rounds of workgroups, pieces numbered longest first
  int n_target = 0;       // balanced: pieces one round of workgroups holds
  int max_pages = 0;      // dense: pages of max_seq_len
  int unit_pages = 0;     // dense: a work unit's pages when every sequence is max_seq_len long
  int64_t grid_units = 0; // work units the launch covers
  bool fused = false;     // one launch: the units merge their partials themselves
  int64_t groups = 0;     // (sequence, row block) groups that merge together
  size_t ws_bytes = 0;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// The single-launch form (the split units merge their partials themselves)
// is chosen only when the environment variable MLA_SINGLE_LAUNCH is "1".
// Measured against the two launches it is slower on every workload here:
// its units live on different XCDs, whose L2 caches are not coherent, so
// the partials go through device-scope stores and loads and the units meet
// at device-scope atomics, several round trips of a few microseconds each,
// more than the merge kernel and the launch gap it saves.  Read on every
// plan, so the sizing queries and the decode call agree within a process
// that does not change it in between.
bool single_launch_requested() {
  const char* v = std::getenv("MLA_SINGLE_LAUNCH");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

// Compute units of the current device, looked up once per device and
// cached (the library's only cache).  A partitioned MI355X or a CU-masked
// process shows fewer, and every plan follows what the device reports.
// Without a usable device (host-only queries) the MI355X's 256 are assumed.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cached[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return mla::kDefaultCUs;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = mla::kDefaultCUs;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

int rg_for_rows(int rows) { return rows <= 32 ? 1 : (rows <= 64 ? 2 : 4); }

// Resident workgroups per CU for a row-group width, from the LDS each
// variant takes out of the CU's 160 KiB: four waves ring 4 x 36 KiB (one
// workgroup); one or two waves ring 2 x 36 KiB plus their table (two
// workgroups dense, where the page table is 4 KiB; one sparse, where the
// 8-byte row addresses of 1024 indices make it 82 KiB).
int wg_per_cu(int rg, bool sparse) { return rg == 4 || sparse ? 1 : 2; }

bool dims_ok(int B, int T, int H, int max_seq_len, int topk) {
  return B >= 0 && B <= (1 << 20) && T >= 1 && T <= MLA_MAX_Q_LEN && H >= 1 && H <= 1024 &&
         max_seq_len >= 0 && max_seq_len <= (1 << 26) && topk >= 0 && topk <= (1 << 24);
}

// The piece length (pages) the device picks for a batch whose sequences are
// all n_pages long: the smallest c >= ceil(n_pages / S), capped by the LDS
// page table, for which B * ceil(n_pages / c) <= n_target (the largest when
// none qualifies).  Used to choose the kernel variant for the pieces' length.
int balanced_length(int B, int n_pages, int S, int n_target) {
  const int lo = std::max(1, ceil_div(n_pages, S));
  const int hi = std::max(lo, std::min(n_pages, kDensePagesMax));
  for (int c = lo; c <= hi; c++)
    if ((int64_t)B * std::max(1, ceil_div(n_pages, c)) <= n_target) return c;
  return hi;
}

// Split planning.  Work unit = (sequence, row block, split).  Every
// candidate (row-block width, split count) is costed as the bytes it moves
// divided by how well its units fill the chip's resident workgroup slots
// (whole rounds of units, so a last partial round counts as idle slots):
//   bytes = KV bytes x row blocks (each row block reads its sequence's KV)
//         + fp32 partials written and read back (when split).
// The cheapest candidate wins; ties go to fewer splits, then wider blocks.
bool make_plan(int B, int T, int H, int max_seq_len, int topk, bool fp8, int req_splits, Plan* pl) {
  if (!dims_ok(B, T, H, max_seq_len, topk) || req_splits < 0 || req_splits > MLA_MAX_KV_SPLITS) return false;
  const int n_cu = device_cu_count();
  Plan p;
  p.R = T * H;
  const bool sparse = topk > 0;
  const int rows_blk = sparse ? H : p.R;                    // rows sharing one token list
  const int64_t lists = (int64_t)B * (sparse ? T : 1);      // token lists (one per sequence or per draft token)
  const double kv_token_bytes = MLA_TOKEN_DIM * (fp8 ? 1.0 : 2.0);
  const int64_t tokens = sparse ? (int64_t)topk : (int64_t)max_seq_len;
  const double kv_bytes = (double)lists * (double)tokens * kv_token_bytes;
  const double part_bytes = (double)B * p.R * kPartialWidth * 4.0 * 2.0;   // per split: write + read
  // A split's index / page table lives in LDS, which bounds its length from
  // below; a split holds at least one page (dense) or one tile of indices.
  const int max_pages = ceil_div(max_seq_len, MLA_BLOCK_SIZE);
  const int s_min = sparse ? ceil_div(topk, kSparseChunkMax) : ceil_div(max_pages, kDensePagesMax);
  int s_max = sparse ? ceil_div(topk, 64) : max_pages;
  if (s_max > MLA_MAX_KV_SPLITS) s_max = MLA_MAX_KV_SPLITS;
  if (s_max < 1) s_max = 1;

  // Dense blocks of at most 32 rows start from two waves: the second wave
  // has no rows, but it takes half of each tile's DMA instructions (R1-shaped
  // batch, B=128 with 16 rows per sequence: 149.6 against 153.6 us per call
  // with the DMA spread over the QK products; with the DMA issued in one
  // burst, as now, the two widths measure the same).  One wave is costed the
  // same and so never replaces it there.
  const int g_first = std::max(rg_for_rows(rows_blk), (!sparse && rows_blk <= 32) ? 2 : 1);
  int rg = g_first, S = 1;
  double best = -1.0;
  for (int g = g_first; g >= 1; g >>= 1) {
    const int64_t n_blk = ceil_div(rows_blk, 32 * g);
    const int64_t slots = (int64_t)n_cu * wg_per_cu(g, sparse);
    for (int s = s_min < 1 ? 1 : s_min; s <= (s_max > s_min ? s_max : s_min); s++) {
      const int64_t units = lists * n_blk * s;
      if (units <= 0) break;
      const double fill = (double)units / (double)(slots * ((units + slots - 1) / slots));
      const double cost = (kv_bytes * (double)n_blk + (s > 1 ? part_bytes * s : 0.0)) / fill;
      if (best < 0.0 || cost < best * 0.98) {   // a new choice must be clearly cheaper
        best = cost;
        rg = g;
        S = s;
      }
    }
  }
  const int S_model = S;
  if (req_splits > 0) S = req_splits;
  if (S < s_min) {
    if (req_splits > 0) return false;   // the split would exceed the LDS table
    S = s_min;
  }
  p.rg = rg;
  const int rb_rows = 32 * rg;
  if (sparse) {
    p.n_hb = ceil_div(H, rb_rows);
    p.n_rb = T * p.n_hb;
    int c = ceil_div(topk, S);
    c = ceil_div(c, 64) * 64;
    if (c > kSparseChunkMax) return false;
    p.chunk = c;
    p.grid_units = (int64_t)B * S * p.n_rb;
  } else {
    p.n_rb = ceil_div(p.R, rb_rows);
    p.max_pages = max_pages;
    // With more than one split, the device cuts the actual lengths into
    // near-equal pieces (balanced_piece in the kernels).  That pays off when
    // the batch has fewer sequences than one round of workgroups holds
    // (otherwise every sequence stays one piece).  The split count costed
    // above assumes every sequence is max_seq_len long; in a mixed batch a
    // long sequence may need more pieces than that, so the library's own
    // choice gives each sequence twice the slots.
    const int64_t slots = (int64_t)n_cu * wg_per_cu(rg, sparse);
    const int n_target = (int)std::max<int64_t>(1, slots / p.n_rb);
    p.balance = S > 1 && B <= mla::kBalanceMaxBatch && B < n_target;
    if (p.balance && req_splits == 0) S = std::max(S, std::min(2 * S, s_max));
    // One round of whole sequences (S = 1) is as long as the longest
    // sequence.  When the row blocks make the work matrix-bound (at least
    // four per sequence) and the batch fills one round but not two, the
    // library's own plan instead cuts the batch into pieces for two rounds
    // and numbers them longest first: the workgroup slots that finish their
    // first piece early take the shortest pieces, so the slots end close to
    // the mean length (for lengths spread over a factor of two, about 0.84
    // of the longest).  The cost is the partials of two splits per row,
    // small next to the products over the piece.  An explicit split count
    // of 2 (what the library reports for such a call) takes the same plan.
    if (!p.balance && S_model == 1 && (req_splits == 0 || req_splits == 2) && p.n_rb >= 4 && B >= n_target &&
        B < 2 * n_target && B <= 64 && max_pages >= 2 && s_max >= 2) {
      p.balance = p.lpt = true;
      S = 2;
    }
    p.chunk = max_pages > 0 ? ceil_div(max_pages, S) : 1;
    if (p.chunk > kDensePagesMax) return false;
    p.unit_pages = p.chunk;
    p.grid_units = (int64_t)B * S * p.n_rb;
    if (p.balance) {
      p.n_target = p.lpt ? 2 * n_target : n_target;
      p.unit_pages = balanced_length(B, max_pages, S, p.n_target);
      // Pieces never exceed B * S; they stay within n_target whenever one
      // piece per sequence (at the largest length the page table holds)
      // already does.
      const int top = std::max(1, std::min(max_pages, kDensePagesMax));
      const int64_t worst = (int64_t)B * ceil_div(std::max(max_pages, 1), top);
      const int64_t pieces = worst <= p.n_target ? std::min<int64_t>(p.n_target, (int64_t)B * S) : (int64_t)B * S;
      p.grid_units = ceil_div(pieces, 8) * 8 * (int64_t)p.n_rb;
    }
  }
  p.S = S;
  p.ws_bytes = S > 1 ? (size_t)B * p.R * S * kPartialWidth * sizeof(float) : 0;
  // Single launch (opt-in, single_launch_requested): when every unit of the
  // launch is resident at once (one round of workgroup slots), the units of
  // each (sequence, row block) wait for each other and merge the block's
  // rows themselves, so there is no second kernel and no launch gap.  Two
  // 8-byte words per group follow the partials in the workspace.
  const int64_t launched = (p.grid_units + 7) / 8 * 8;
  p.groups = (int64_t)B * p.n_rb;
  // Residency is what the runtime reports for the variant (the LDS model
  // above when it cannot be asked): the single launch waits on it.
  const bool resid_kernel = fp8 && (sparse || (int64_t)p.unit_pages * MLA_BLOCK_SIZE <= mla::kFp8ResidualMaxUnitTokens);
  const int occ = mla::partial_kernel_occupancy(fp8, sparse, p.rg, resid_kernel);
  const int64_t resident = (int64_t)n_cu * (occ > 0 ? occ : wg_per_cu(p.rg, sparse));
  p.fused = single_launch_requested() && S > 1 && S <= 64 && launched <= resident;
  if (p.fused) p.ws_bytes = (p.ws_bytes + 15) / 16 * 16 + (size_t)p.groups * 16;
  *pl = p;
  return true;
}

// Number of this call among the library's calls in this process (48 bits);
// marks the group words of a single-launch call, so that words left by an
// earlier call (or never written) count as zero and need no clearing.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{1};
  return counter.fetch_add(1, std::memory_order_relaxed) & ((1ull << 48) - 1);
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

enum class Kind { kBf16, kFp8, kSparse, kSparseFp8 };

mla_status_t run(Kind kind, const void* q_nope, const void* q_pe, const void* kv_cache,
                 const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk_indices,
                 int topk, int B, int T, int H, int NB, int block_size, int MB, int max_seq_len,
                 float softmax_scale, float q_scale, float kv_scale, void* out, int out_dtype, float* lse,
                 void* workspace, size_t workspace_bytes, int num_kv_splits, void* stream) {
  const bool fp8 = kind == Kind::kFp8 || kind == Kind::kSparseFp8;
  const bool sparse = kind == Kind::kSparse || kind == Kind::kSparseFp8;
  if (block_size != MLA_BLOCK_SIZE) return MLA_ERR_UNSUPPORTED;
  if (!dims_ok(B, T, H, max_seq_len, sparse ? topk : 0)) return MLA_ERR_INVALID_ARGUMENT;
  if (sparse && topk < 1) return MLA_ERR_INVALID_ARGUMENT;
  if (NB < 0 || MB < 1 || (int64_t)NB * MLA_BLOCK_SIZE > INT32_MAX) return MLA_ERR_INVALID_ARGUMENT;
  if (num_kv_splits < 0 || num_kv_splits > MLA_MAX_KV_SPLITS) return MLA_ERR_INVALID_ARGUMENT;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_INVALID_ARGUMENT;
  // The kernels take each row's softmax reference from the maximum of the
  // raw scores, which is the maximum of the scaled ones only for a positive
  // scale (a zero scale would also turn masked scores, -inf * 0, into NaN).
  if (!std::isfinite(softmax_scale) || !std::isfinite(q_scale) || !std::isfinite(kv_scale) || softmax_scale <= 0.f ||
      q_scale <= 0.f || kv_scale <= 0.f)
    return MLA_ERR_INVALID_ARGUMENT;
  if (B == 0) return MLA_OK;
  const bool stage1_only = out == nullptr && lse == nullptr;
  if (out == nullptr && lse != nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (stage1_only && num_kv_splits < 2) return MLA_ERR_INVALID_ARGUMENT;
  if (!q_nope || !q_pe || !block_table || !seq_lens || (NB > 0 && !kv_cache) || (sparse && !topk_indices))
    return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_cache) || !aligned16(out))
    return MLA_ERR_INVALID_ARGUMENT;
  Plan pl;
  if (!make_plan(B, T, H, max_seq_len, sparse ? topk : 0, fp8, num_kv_splits, &pl)) return MLA_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0) {
    if (workspace_bytes < pl.ws_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned16(workspace)) return MLA_ERR_INVALID_ARGUMENT;
  }

  mla::PartialParams p{};
  p.q_nope = (const uint8_t*)q_nope;
  p.q_pe = (const uint8_t*)q_pe;
  p.kv = (const uint8_t*)kv_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.topk = sparse ? topk_indices : nullptr;
  p.B = B;
  p.T = T;
  p.H = H;
  p.R = pl.R;
  p.NB = NB;
  p.MB = MB;
  p.K = sparse ? topk : 0;
  p.n_rb = pl.n_rb;
  p.n_hb = pl.n_hb;
  p.chunk = pl.chunk;
  p.S = pl.S;
  p.balance = pl.balance ? 1 : 0;
  p.n_target = pl.n_target;
  p.lpt = pl.lpt ? 1 : 0;
  p.max_pages = pl.max_pages;
  const int64_t units = pl.grid_units;
  if (units > (int64_t)1 << 30) return MLA_ERR_INVALID_ARGUMENT;
  p.n_units = (int)units;
  const float log2e = 1.4426950408889634f;
  p.qk_scale = fp8 ? softmax_scale * log2e * q_scale * kv_scale : softmax_scale * log2e;
  p.out_scale = fp8 ? kv_scale : 1.0f;
  p.out = out;
  p.out_f32 = out_dtype == MLA_OUT_F32;
  p.lse = lse;
  p.ws = pl.S > 1 ? (float*)workspace : nullptr;
  p.fused = pl.fused && !stage1_only ? 1 : 0;
  p.sync = p.fused ? (unsigned long long*)((uint8_t*)workspace +
                                           ((size_t)B * pl.R * pl.S * kPartialWidth * sizeof(float) + 15) / 16 * 16)
                   : nullptr;
  p.epoch = p.fused ? next_epoch() : 0;
  const int grid = (int)((units + 7) / 8 * 8);
  hipStream_t st = (hipStream_t)stream;
  // fp8: units planned at most kFp8ResidualMaxUnitTokens long take the
  // residual-product kernel.  The others run without it and rerun a unit
  // with it when a few tokens carry most of a row's weight (a short
  // sequence in a batch of long ones, or a peaked softmax).
  const int64_t unit_tokens = (int64_t)(sparse ? pl.chunk : pl.unit_pages * MLA_BLOCK_SIZE);
  const bool resid = fp8 && unit_tokens <= mla::kFp8ResidualMaxUnitTokens;
  if (mla::launch_partial_kernel(p, fp8, sparse, pl.rg, resid, grid, st) != hipSuccess) return MLA_ERR_HIP;
  if (pl.S > 1 && !stage1_only && !p.fused) {
    mla::MergeParams m{};
    m.ws = (const float*)workspace;
    m.n_rows = (int64_t)B * pl.R;
    m.S = pl.S;
    m.out = out;
    m.out_f32 = p.out_f32;
    m.lse = lse;
    if (mla::launch_merge_kernel(m, st) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP launch failure";
    case MLA_ERR_SCRATCH_LIMIT: return "call needs more split workspace than the static 64 MiB buffer";
  }
  return "unknown status";
}

int mla_num_kv_splits(int batch, int q_len, int num_heads, int max_seq_len, int topk, int kv_fp8) {
  Plan pl;
  if (!make_plan(batch, q_len, num_heads, max_seq_len, topk, kv_fp8 != 0, 0, &pl)) return 0;
  return pl.S;
}

int mla_launch_waves(int batch, int q_len, int num_heads, int max_seq_len, int topk, int kv_fp8) {
  Plan pl;
  if (!make_plan(batch, q_len, num_heads, max_seq_len, topk, kv_fp8 != 0, 0, &pl)) return 0;
  return pl.rg;
}

size_t mla_workspace_size(int batch, int q_len, int num_heads, int max_seq_len, int topk, int kv_fp8,
                          int num_kv_splits) {
  Plan pl;
  if (!make_plan(batch, q_len, num_heads, max_seq_len, topk, kv_fp8 != 0, num_kv_splits, &pl)) return 0;
  return pl.ws_bytes;
}

mla_status_t mla_decode(const void* q_nope, const void* q_pe, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int q_len, int num_heads, int num_blocks,
                        int block_size, int max_blocks_per_seq, int max_seq_len, float softmax_scale, void* out,
                        int out_dtype, float* lse, void* workspace, size_t workspace_bytes, int num_kv_splits,
                        void* stream) {
  return run(Kind::kBf16, q_nope, q_pe, kv_cache, block_table, seq_lens, nullptr, 0, batch, q_len, num_heads,
             num_blocks, block_size, max_blocks_per_seq, max_seq_len, softmax_scale, 1.0f, 1.0f, out, out_dtype,
             lse, workspace, workspace_bytes, num_kv_splits, stream);
}

mla_status_t mla_decode_fp8(const void* q_nope, const void* q_pe, const void* kv_cache, const int32_t* block_table,
                            const int32_t* seq_lens, int batch, int q_len, int num_heads, int num_blocks,
                            int block_size, int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                            float q_scale, float kv_scale, void* out, int out_dtype, float* lse, void* workspace,
                            size_t workspace_bytes, int num_kv_splits, void* stream) {
  return run(Kind::kFp8, q_nope, q_pe, kv_cache, block_table, seq_lens, nullptr, 0, batch, q_len, num_heads,
             num_blocks, block_size, max_blocks_per_seq, max_seq_len, softmax_scale, q_scale, kv_scale, out,
             out_dtype, lse, workspace, workspace_bytes, num_kv_splits, stream);
}

mla_status_t mla_decode_fp8_noalloc(const void* q_nope, const void* q_pe, const void* kv_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, int batch, int q_len,
                                    int num_heads, int num_blocks, int block_size, int max_blocks_per_seq,
                                    int max_seq_len, float softmax_scale, float q_scale, float kv_scale, void* out,
                                    int out_dtype, float* lse, int num_kv_splits, void* stream) {
  // Sizes the plan first: a call whose partials do not fit the static buffer
  // is refused before anything is looked up or enqueued.  Invalid arguments
  // fall through to run(), which reports them.
  Plan pl;
  void* ws = nullptr;
  if (batch > 0 && make_plan(batch, q_len, num_heads, max_seq_len, 0, true, num_kv_splits, &pl)) {
    if (pl.ws_bytes > mla::kStaticScratchBytes) return MLA_ERR_SCRATCH_LIMIT;
    if (pl.ws_bytes > 0 && mla::static_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
  }
  return run(Kind::kFp8, q_nope, q_pe, kv_cache, block_table, seq_lens, nullptr, 0, batch, q_len, num_heads,
             num_blocks, block_size, max_blocks_per_seq, max_seq_len, softmax_scale, q_scale, kv_scale, out,
             out_dtype, lse, ws, ws ? mla::kStaticScratchBytes : 0, num_kv_splits, stream);
}

mla_status_t mla_sparse_decode(const void* q_nope, const void* q_pe, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk_indices,
                               int topk, int batch, int q_len, int num_heads, int num_blocks, int block_size,
                               int max_blocks_per_seq, int max_seq_len, float softmax_scale, void* out,
                               int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                               int num_kv_splits, void* stream) {
  return run(Kind::kSparse, q_nope, q_pe, kv_cache, block_table, seq_lens, topk_indices, topk, batch, q_len,
             num_heads, num_blocks, block_size, max_blocks_per_seq, max_seq_len, softmax_scale, 1.0f, 1.0f, out,
             out_dtype, lse, workspace, workspace_bytes, num_kv_splits, stream);
}

mla_status_t mla_sparse_decode_fp8(const void* q_nope, const void* q_pe, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* topk_indices, int topk, int batch, int q_len, int num_heads,
                                   int num_blocks, int block_size, int max_blocks_per_seq, int max_seq_len,
                                   float softmax_scale, float q_scale, float kv_scale, void* out, int out_dtype,
                                   float* lse, void* workspace, size_t workspace_bytes, int num_kv_splits,
                                   void* stream) {
  return run(Kind::kSparseFp8, q_nope, q_pe, kv_cache, block_table, seq_lens, topk_indices, topk, batch, q_len,
             num_heads, num_blocks, block_size, max_blocks_per_seq, max_seq_len, softmax_scale, q_scale, kv_scale,
             out, out_dtype, lse, workspace, workspace_bytes, num_kv_splits, stream);
}

mla_status_t mla_merge_partials(const float* workspace, int64_t rows, int num_kv_splits, void* out, int out_dtype,
                                float* lse, void* stream) {
  if (rows < 0 || rows > ((int64_t)1 << 40) || num_kv_splits < 1 || num_kv_splits > MLA_MAX_KV_SPLITS)
    return MLA_ERR_INVALID_ARGUMENT;
  if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_F32) return MLA_ERR_INVALID_ARGUMENT;
  if (rows == 0) return MLA_OK;
  if (!workspace || !out || !aligned16(workspace) || !aligned16(out)) return MLA_ERR_INVALID_ARGUMENT;
  mla::MergeParams m{};
  m.ws = workspace;
  m.n_rows = rows;
  m.S = num_kv_splits;
  m.out = out;
  m.out_f32 = out_dtype == MLA_OUT_F32;
  m.lse = lse;
  if (mla::launch_merge_kernel(m, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
