// MLA decode kernels for gfx950 (MI355X / CDNA4).
//
// Two kernels implement absorbed multi-head latent attention decode over a
// paged latent KV cache (one 576-wide token vector = 512 latent + 64 rope,
// shared by every head; DeepSeek-R1 dims from the vLLM PR #41778 digest,
// "Risks and impact" item 4):
//
//  * mla_partial_kernel: one workgroup per (sequence, row block, KV split).
//    Its pages stream from HBM straight into an LDS ring with 16-byte
//    global->LDS DMA loads; every wave owns 32 query rows (rows = H * q_len
//    packed together, row = t * H + h) and, per tile of KV tokens, runs
//    S^T = K Q^T on MFMA, the online softmax in registers, and
//    O^T += V^T P^T on MFMA.  It writes either the final output and LSE
//    (one split) or an fp32 partial [512 outputs | lse] per (row, split),
//    the two-stage split-KV scheme of the Triton MLA decode (vLLM PR #46819
//    digest, "Implementation" items 1-3, partial width kv_lora_rank + 1 in
//    its "Key code excerpt").
//  * mla_merge_kernel: one wave per output row; combines the split partials
//    by log-sum-exp with wavefront shuffles.
//
// Layout choices that matter on CDNA4:
//  * Keys/values sit on the MFMA "A" side (M = tokens) and queries on the
//    "B" side (N = rows).  The QK accumulator then holds, per lane, one row
//    and a set of tokens - exactly the operand layout the PV product wants
//    for P, so P never leaves registers.  V^T is read from LDS with the
//    gfx950 transpose loads (ds_read_b64_tr_b16 / _b8).
//  * The LDS copy of a tile keeps the token-major order of the cache, with
//    16-byte units XOR-swizzled per token so that both the row reads of the
//    QK operand and the transposed reads of the PV operand are free of bank
//    conflicts.  The swizzle is applied on the global side of the DMA: the
//    lane that fills LDS unit (t, c) fetches global unit (t, c ^ f(t)).
//  * fp8: both products use v_mfma_scale_f32_32x32x64_f8f6f4.  P is
//    quantized to e4m3 per tile relative to the tile's own (integer,
//    log2-domain) row maximum times 2^8, and the MFMA's per-row E8M0 scale
//    on the P operand restores the common reference, so the O accumulator
//    is rescaled only when a row maximum jumps by more than 2^64.
//  * bf16: P is bf16 relative to a running row maximum that is raised lazily
//    (only when a row grows by more than 2^16), which keeps O rescaling rare.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "mla_decode_internal.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define LDS_AS __attribute__((address_space(3)))
// Wave-uniform metadata (block table entries, sequence lengths) is read
// through the constant address space so it becomes a scalar (SMEM) load: a
// vector load would share vmcnt with the in-flight tile DMA and force a full
// drain before its use.
#define CONST_AS __attribute__((address_space(4)))

constexpr float kLn2 = 0.6931471805599453f;
// fp8 without the residual product: a unit is rerun with it when some row's
// bound of sum_j w_j^2 (w the normalized softmax weights) exceeds this.
constexpr float kFp8RedoSumSq = 0x1p-7f;
constexpr float kNegBig = -1.0e30f;  // running-max sentinel: finite, below any logit
constexpr int kE4m3OnesX4 = 0x38383838;  // four e4m3 1.0 bytes

// A zero token row: DMA source for tokens past the end of a sequence, padded
// or out-of-range top-k entries and out-of-range page numbers, so that no
// stale (possibly NaN) cache bytes reach the PV product.
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[kTokenDim * 2];

template <bool FP8>
struct Kv;
template <>
struct Kv<false> {                         // bf16 cache
  static constexpr int kRowBytes = 1152;   // 576 * 2
  static constexpr int kUnits = 72;        // 16-byte units per token
  static constexpr int kTileTok = 32;      // tokens per LDS tile (36 KiB)
  static constexpr int kQkSteps = 36;      // 576 / 16 (32x32x16 MFMA)
  static constexpr int kTokBlocks = 1;     // 32-token MFMA blocks per tile
  static constexpr int kPeriodInstr = 18;  // DMA instructions per swizzle period (16 tokens)
  // Swizzle: t bits (1, 3:2) -> 3-bit XOR on the unit index.
  __device__ static inline int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
};
template <>
struct Kv<true> {                          // e4m3 cache
  static constexpr int kRowBytes = 576;
  static constexpr int kUnits = 36;
  static constexpr int kTileTok = 64;
  static constexpr int kQkSteps = 9;       // 576 / 64 (32x32x64 MFMA)
  static constexpr int kTokBlocks = 2;
  static constexpr int kPeriodInstr = 9;
  __device__ static inline int swz(int t) { return (t >> 2) & 3; }
};

constexpr int kTileBytes = 36864;          // both dtypes
constexpr int kInstrPerTile = kTileBytes / 1024;

__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses have completed.
__device__ inline void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
}

// Combine the two halves of a wave (lanes l and l ^ 32 hold the same row)
// with v_permlane32_swap.  Issued from inline asm: the builtin applied to
// one value twice gets folded away by the compiler.
__device__ inline float other_half(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  // a = [x_lo, x_lo], b = [x_hi, x_hi]: each lane takes the half it lacks.
  return (__lane_id() < 32) ? b : a;
}
__device__ inline float max_across_halves(float x) { return fmaxf(x, other_half(x)); }

__device__ inline float sum_across_halves(float x) { return x + other_half(x); }

// 16-byte global -> LDS DMA: lane i writes LDS bytes [m0 + 16 i, m0 + 16 i + 16).
// Both DMA helpers load with the non-temporal hint (nt): cache lines are
// streamed, so they do not push out what is reused (query rows, tables,
// partials).  Each workgroup reads its tiles once, and row blocks sharing a
// piece run side by side.  Measured against the same kernels without the
// hint (alternating calls on one GPU): R1-shaped batch 143.9 -> 129.2 us,
// MTP-3 fp8 716 -> 704 us, sparse bf16 77.5 -> 71.4 us, sparse fp8 61.7 ->
// 57.5 us, MTP-7 unchanged.
// Issued from inline asm so the compiler does not treat it as an LDS store
// (it would otherwise drain every in-flight DMA before each LDS read it
// cannot prove disjoint); completion is tracked explicitly with vmcnt.
//
// The compiler inserts no hazard wait states before an inline-asm memory
// instruction, so the DMA helpers carry their own: an LDS DMA reading M0
// needs one after the SALU write of M0 placed just before it.  A vector
// memory instruction reading an SGPR needs five after a VALU write of that
// SGPR; buffer_rsrc() provides those once per descriptor.  The build scans
// the compiled kernels for both cases (asm_hazards.py).
__device__ inline void dma16(const void* gsrc, uint32_t lds_byte_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gsrc), "{m0}"(lds_byte_addr) : "memory");
}

// 16-byte buffer -> LDS DMA: lane i reads rsrc.base + voff_i + soff and
// writes LDS bytes [m0 + 16 i, m0 + 16 i + 16).  An offset at or past the
// descriptor's size reads zeros (no memory access), which is how missing
// tokens of a tile become zero vectors.  Inline asm for the same reason as
// dma16().
__device__ inline void dma16_buf(int voff, i32x4_t rsrc, int soff, uint32_t lds_byte_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "{m0}"(lds_byte_addr)
               : "memory");
}
// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, size in bytes.
// Its words come from v_readfirstlane (VALU writes of SGPRs); the s_nop 4
// after them gives the five wait states a vector memory read of those SGPRs
// needs, and as an asm output the descriptor is not re-derived after it.
__device__ inline i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
  asm volatile("s_nop 4" : "+s"(r));
  return r;
}

// MFMAs whose accumulator must stay in VGPRs.  The output accumulator O
// fills all 256 AGPRs; the compiler would otherwise give the score and
// row-sum accumulators AGPRs too and shuttle two O tiles through VGPRs on
// every tile.  Being inline asm, these carry their own hazard padding: three
// wait states before the product (a VALU write of an operand needs two), and
// callers end a chain with mfma_drain(acc) before any VALU reads the result
// (an XDL result needs about 18).  Back-to-back products on one accumulator
// need no padding (the compiler emits none for such chains either).
__device__ inline void mfma_f8_acc(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b, int sa, int sb) {
  asm volatile("s_nop 2\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// The same fp8 product without block scales (both 2^0), for the QK chain:
// one 8-byte instruction instead of the 16-byte scaled form.
__device__ inline void mfma_f8_first_plain(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_f8_acc_plain(f32x16_t& acc, const i32x8_t& a, const i32x8_t& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_first(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_bf16_acc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// Keeps the computation of a value at this point of the program: an empty
// inline-asm use.  Softmax stages produce values that are only consumed at
// the end of a loop step; without this, IR-level sinking moves their
// arithmetic down to that use, past the scheduling barriers that are meant
// to interleave it with matrix products.
__device__ inline void pin(int& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }

// 24 wait states after the last product of a chain.  The accumulators are
// in/out operands: code that reads them then depends on this statement and
// cannot be scheduled above the padding (with no operands the compiler is
// free to hoist such reads above it, right behind the product).
__device__ inline void mfma_drain(f32x16_t& a) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a)); }
__device__ inline void mfma_drain(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// ---------------------------------------------------------------------------
// Length-balanced pieces (dense calls with more than one split).
//
// The host knows only a bound of the sequence lengths, so every workgroup
// derives the cut from the lengths themselves (the same result in each):
//  * a sequence of n pages is cut into k = max(1, ceil(n / c)) pieces; piece
//    i covers pages [i n / k, (i+1) n / k), so its pieces differ by at most a
//    page and none is longer than c;
//  * c is the smallest length for which the whole batch needs at most
//    n_target pieces, n_target being the workgroups the chip holds at once
//    divided by the row blocks per piece: the pieces then run in one round
//    and are about equally long, whatever the spread of the lengths.  c is
//    at least ceil(longest / S) (a sequence has S partial slots) and at most
//    the LDS page table's capacity; when no length qualifies, the largest
//    one is taken;
//  * pieces are numbered sequence after sequence, or, for a batch of at most
//    64 sequences cut for two rounds of workgroups (lpt), longest piece
//    first, which is the longest-processing-time-first order for the
//    hardware's in-order dispatch of workgroups to free slots.
// Lengths are clamped as the kernel clamps them, and to max_pages.
struct Piece {
  int b;          // sequence
  int k;          // piece of that sequence, which is its partial slot
  int n;          // pieces of that sequence
  int pg0, pg1;   // pages [pg0, pg1) of the sequence
};

// Row (16-lane) sums and maxima through DPP; a lane then holds its row's
// result and four lane reads combine the rows.
__device__ __attribute__((always_inline)) inline int row16_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);   // row_mirror
  return v;
}
__device__ __attribute__((always_inline)) inline int wave_sum_i(int v) {
  v = row16_sum(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
__device__ __attribute__((always_inline)) inline int wave_max_i(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// ceil(x / c) for 0 <= x < 2^21 and 1 <= c <= 2^11, rc being 1/c rounded to
// float: the float quotient is then within 1/4 of the exact one, so a single
// correction of the truncated value makes it exact.
__device__ __attribute__((always_inline)) inline int ceil_div_small(int x, int c, float rc) {
  const int y = x + c - 1;
  int q = (int)((float)y * rc);
  const int r = y - q * c;
  q += r >= c ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
}

// Lane l holds sequences [l M', l M' + M') with M' = ceil(B / 64) <= M.
template <int M>
__device__ __attribute__((always_inline)) inline bool balanced_piece_m(const PartialParams& p, int j, Piece* pc) {
  const int lane = threadIdx.x & 63;
  const int m = (p.B + 63) >> 6;
  const int first = lane * m;
  const int nv = max(0, min(m, p.B - first));       // sequences of this lane
  const int cap = p.MB * 64;
  int pg[M];
  int tot = 0, mx = 0;
#pragma unroll
  for (int e = 0; e < M; e++) {
    int n = 0;
    if (e < nv) {
      int L = p.seq_lens[first + e];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      n = min((L + 63) >> 6, p.max_pages);
    }
    pg[e] = n;
    tot += n;
    mx = max(mx, n);
  }
  tot = wave_sum_i(tot);
  mx = wave_max_i(mx);

  auto count = [&](int c) {
    const float rc = 1.0f / (float)c;
    int s = 0;
#pragma unroll
    for (int e = 0; e < M; e++) s += e < nv ? max(1, ceil_div_small(pg[e], c, rc)) : 0;
    return wave_sum_i(s);
  };
  const int S = p.S, NT = p.n_target;
  int lo = max(1, (mx + S - 1) / S);
  lo = max(lo, min((tot + NT - 1) / NT, kDensePagesMax));
  int hi = max(lo, min(mx, kDensePagesMax));
  // sum max(1, ceil(n / c)) <= tot / c + B, so c >= tot / (NT - B) qualifies
  if (NT > p.B) hi = max(lo, min(hi, (tot + (NT - p.B) - 1) / (NT - p.B)));
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (count(mid) <= NT) hi = mid;
    else lo = mid + 1;
  }
  const int c = lo;

  // Pieces per sequence, their running count over the lanes, and the lane
  // that holds piece j.
  const float rc = 1.0f / (float)c;
  int kb[M];
  int ls = 0;
#pragma unroll
  for (int e = 0; e < M; e++) {
    kb[e] = e < nv ? max(1, ceil_div_small(pg[e], c, rc)) : 0;
    ls += kb[e];
  }
  if constexpr (M == 1) {
    if (p.lpt) {
      // Longest first: piece slots go to the sequences in decreasing order
      // of their piece length (ties: lower sequence first), so the longest
      // pieces start in the first round of workgroups and the slots that
      // free up early take the shortest ones.  Lane b holds sequence b.
      const int len = nv > 0 ? (pg[0] + kb[0] - 1) / kb[0] : -1;
      int rank = 0;
      for (int o = 0; o < p.B; o++) {
        const int len_o = __builtin_amdgcn_readlane(len, o);
        const int kb_o = __builtin_amdgcn_readlane(kb[0], o);
        rank += (len_o > len || (len_o == len && o < lane)) ? kb_o : 0;
      }
      const uint64_t own1 = __builtin_amdgcn_ballot_w64(nv > 0 && j >= rank && j < rank + kb[0]);
      if (own1 == 0) return false;
      const int owner1 = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(own1));
      pc->b = owner1;
      pc->k = j - __builtin_amdgcn_readlane(rank, owner1);
      pc->n = __builtin_amdgcn_readlane(kb[0], owner1);
      const int n_pg1 = __builtin_amdgcn_readlane(pg[0], owner1);
      pc->pg0 = pc->k * n_pg1 / pc->n;
      pc->pg1 = (pc->k + 1) * n_pg1 / pc->n;
      return true;
    }
  }
  int inc = ls;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d);
    if (lane >= d) inc += t;
  }
  const int total = __builtin_amdgcn_readlane(inc, 63);
  if (j >= total) return false;
  const int excl = inc - ls;
  const uint64_t own = __builtin_amdgcn_ballot_w64(j >= excl && j < inc);
  const int owner = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(own));
  int rem = j - excl, fb = 0, fk = 0, fn = 1, fp = 0;
  bool found = false;
#pragma unroll
  for (int e = 0; e < M; e++) {
    if (!found && e < nv) {
      if (rem < kb[e]) {
        found = true;
        fb = first + e;
        fk = rem;
        fn = kb[e];
        fp = pg[e];
      } else {
        rem -= kb[e];
      }
    }
  }
  pc->b = __builtin_amdgcn_readlane(fb, owner);
  pc->k = __builtin_amdgcn_readlane(fk, owner);
  pc->n = __builtin_amdgcn_readlane(fn, owner);
  const int n_pg = __builtin_amdgcn_readlane(fp, owner);
  pc->pg0 = pc->k * n_pg / pc->n;
  pc->pg1 = (pc->k + 1) * n_pg / pc->n;
  return true;
}

__device__ __attribute__((always_inline)) inline bool balanced_piece(const PartialParams& p, int j, Piece* pc) {
  const int m = (p.B + 63) >> 6;
  if (m <= 1) return balanced_piece_m<1>(p, j, pc);
  if (m <= 2) return balanced_piece_m<2>(p, j, pc);
  if (m <= 4) return balanced_piece_m<4>(p, j, pc);
  if (m <= 8) return balanced_piece_m<8>(p, j, pc);
  return balanced_piece_m<kBalanceMaxBatch / 64>(p, j, pc);
}

// A device-scope load: reads what other XCDs wrote with device-scope stores,
// whatever this XCD's L2 held.
__device__ inline float coherent_load(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// LSE merge of NR rows by one wave (lane l: outputs 8l .. 8l+7), all rows'
// loads issued before any is used; at most 64 splits.  The arithmetic of
// each row is that of mla_merge_kernel, so both give the same bits.
template <int NR>
__device__ __attribute__((always_inline)) inline void merge_rows(const float* ws, const int64_t (&rows)[NR],
                                                                 const bool (&valid)[NR], int S, void* out,
                                                                 int out_f32, float* lse) {
  const int lane = threadIdx.x & 63;
  float mx[NR], w[NR], z[NR];
#pragma unroll
  for (int i = 0; i < NR; i++)
    mx[i] = (valid[i] && lane < S) ? coherent_load(ws + (rows[i] * S + lane) * (int64_t)kPartialWidth + 512)
                                    : -INFINITY;
#pragma unroll
  for (int i = 0; i < NR; i++) {
    w[i] = mx[i];    // this lane's split lse
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], d));
  }
#pragma unroll
  for (int i = 0; i < NR; i++) {
    w[i] = (mx[i] != -INFINITY && lane < S) ? __expf(w[i] - mx[i]) : 0.f;
    float zs = w[i];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) zs += __shfl_xor(zs, d);
    z[i] = 0.f + zs;
  }
  float acc[NR][8];
#pragma unroll
  for (int i = 0; i < NR; i++)
#pragma unroll
    for (int c = 0; c < 8; c++) acc[i][c] = 0.f;
  for (int k0 = 0; k0 < S; k0 += 8) {
    float wk[NR][8];
    float v[NR][8][8];
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
      for (int k = 0; k < 8; k++) wk[i][k] = __shfl(w[i], (k0 + k) & 63);   // 0 past S
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (wk[i][k] != 0.f) {
          const float* src = ws + (rows[i] * S + k0 + k) * (int64_t)kPartialWidth + 8 * lane;
#pragma unroll
          for (int c = 0; c < 8; c++) v[i][k][c] = coherent_load(src + c);
        }
#pragma unroll
    for (int i = 0; i < NR; i++)
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (wk[i][k] != 0.f) {
#pragma unroll
          for (int c = 0; c < 8; c++) acc[i][c] += wk[i][k] * v[i][k][c];
        }
  }
#pragma unroll
  for (int i = 0; i < NR; i++) {
    if (!valid[i]) continue;
    float lse_out = -INFINITY;
    if (mx[i] != -INFINITY) {
      const float inv = 1.f / z[i];
#pragma unroll
      for (int c = 0; c < 8; c++) acc[i][c] *= inv;
      lse_out = mx[i] + __logf(z[i]);
    }
    if (out_f32) {
      float* o = (float*)out + rows[i] * 512 + 8 * lane;
      *(float4*)o = float4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      *(float4*)(o + 4) = float4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
    } else {
      typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));
      bf16x8s_t bv;
#pragma unroll
      for (int c = 0; c < 8; c++) bv[c] = (__bf16)acc[i][c];
      *(bf16x8s_t*)((__bf16*)out + rows[i] * 512 + 8 * lane) = bv;
    }
    if (lane == 0 && lse) lse[rows[i]] = lse_out;
  }
}

// Arrival at a group word (epoch << 16 | count): a word of another epoch
// counts as zero.  Returns the count after this arrival, or 0 if the word
// could not be updated within the bound.
__device__ inline int sync_arrive(unsigned long long* word, unsigned long long e) {
  unsigned long long cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; it < (1 << 20); it++) {
    const unsigned long long base = (cur >> 16) == (e >> 16) ? cur : e;
    if (__hip_atomic_compare_exchange_strong(word, &cur, base + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return (int)((base + 1) & 0xffff);
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Split-KV partial kernel.
//   FP8    : e4m3 cache and query (else bf16)
//   SPARSE : visible tokens from top-k index lists (else dense causal)
//   RG     : waves per workgroup; each owns 32 rows of the row block
//   NS     : LDS ring stages (tiles of 36 KiB)
//   RESID  : fp8 only - also multiply V by the e4m3 rounding residual of P
//            (a second fp8 product), so each softmax weight is carried to
//            about 2^-8 instead of 2^-4; chosen for short work units, where
//            a few tokens can dominate a row.  Without it, a row whose
//            weight concentrates on a few tokens gets the residual product
//            of its heaviest tile added afterwards, or its unit reruns with
//            the residual product (see "the passes" below)
//
// With four waves (RG = 4) the tile loop is software-pipelined: the QK
// products of tile i+1 are issued interleaved with the PV products of tile
// i, so the two dependent QK accumulator chains never stall the matrix pipe.
template <bool FP8, bool SPARSE, int RG, int NS, bool RESID, bool FS>
__global__ void __launch_bounds__(64 * RG) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_partial_kernel(const PartialParams p) {
  using K = Kv<FP8>;
  constexpr int NI = kInstrPerTile / RG;          // DMA instructions per wave per tile
  constexpr int NPRE = NI <= 18 ? NI : K::kPeriodInstr;
  static_assert(NI % NPRE == 0, "DMA offset period");
  constexpr bool PIPE = RG == 4;
  static_assert(!PIPE || NS >= 3, "the pipelined loop keeps two tiles resident");
  static_assert(!FS || (FP8 && !SPARSE && RG == 4 && !RESID), "feature split: dense fp8, four waves");
  constexpr int kTableCap = SPARSE ? kSparseChunkMax : kDensePagesMax;
  // Dense: int32 page per page of the unit.  Sparse: the 64-bit address of
  // each index's token row (the zero row for a skipped entry), then one
  // tile's worth of zero-row addresses that tiles past the end read.
  constexpr int kTableBytes = SPARSE ? (kTableCap + K::kTileTok) * 8 : kTableCap * 4;
  constexpr int kPBytes = FS ? 4 * 2048 : 0;      // FS: P tile of each row block (64 lanes x 32 B)
  constexpr int kScBytes = FS ? 4 * 64 * 4 : 0;   // FS: E8M0 scales of each row block (per lane)
  constexpr bool kFixTiles = FP8 && !SPARSE && !RESID;   // pass 0 without the residual product
  constexpr int kFixWords = kFixTiles ? kDensePagesMax / 32 : 0;   // bitmap of tiles to fix (one page each)

  // LDS: [ring of NS tiles][unit table: int32 x kTableCap][FS: P tiles][FS: scales][redo flag]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * kTileBytes + kTableBytes + kPBytes + kScBytes + 16 +
                                                         4 * kFixWords];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;
  LDS_AS int* table = (LDS_AS int*)(lds + NS * kTileBytes);
  LDS_AS uint64_t* table64 = (LDS_AS uint64_t*)(lds + NS * kTileBytes);
  LDS_AS uint8_t* pbuf = lds + NS * kTileBytes + kTableBytes;
  LDS_AS int* scbuf = (LDS_AS int*)(pbuf + kPBytes);
  LDS_AS int* redo_flag = (LDS_AS int*)(pbuf + kPBytes + kScBytes);
  LDS_AS uint32_t* fix_map = (LDS_AS uint32_t*)(pbuf + kPBytes + kScBytes + 16);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;       // which half of the wave
  const int l32 = lane & 31;     // MFMA column = query row within the wave

  // ---- work unit.  Consecutive workgroup ids land on consecutive XCDs
  // (eight, each with its own L2); the row blocks of one (sequence, split)
  // read the same KV and are kept on one XCD.
  int rb, split, b, n_split, bal_pg0 = 0, bal_pg1 = 0;
  if (!SPARSE && p.balance) {
    // Length-balanced pieces, dealt round-robin to the XCDs: piece j runs on
    // XCD j mod 8, so every XCD gets an equal share of near-equal pieces.
    const int i = blockIdx.x >> 3;
    rb = i % p.n_rb;
    const int j = (i / p.n_rb) * 8 + (blockIdx.x & 7);
    Piece pc;
    if (!balanced_piece(p, j, &pc)) return;
    b = pc.b;
    split = pc.k;
    n_split = pc.n;
    bal_pg0 = pc.pg0;
    bal_pg1 = pc.pg1;
  } else {
    // Fixed chunks: unit u = (sequence, split, row block), renumbered so that
    // consecutive units share an XCD.
    const int nwg = gridDim.x;     // multiple of 8
    const int u = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    rb = u % p.n_rb;
    const int bs = u / p.n_rb;
    split = bs % p.S;
    b = bs / p.S;
    n_split = p.S;
  }

  int L = ((const CONST_AS int32_t*)p.seq_lens)[b];
  L = L < 0 ? 0 : (L > p.MB * 64 ? p.MB * 64 : L);

  // ---- rows of this lane
  int row, t_row;
  bool row_ok;
  if (SPARSE) {
    const int t_blk = rb / p.n_hb;
    const int hrow = (rb % p.n_hb) * (32 * RG) + wave * 32 + l32;
    row_ok = hrow < p.H;
    t_row = t_blk;
    row = t_blk * p.H + hrow;
  } else {
    row = rb * (32 * RG) + wave * 32 + l32;
    row_ok = row < p.R;
    t_row = row_ok ? row / p.H : 0;
  }
  const int64_t qrow = (int64_t)b * p.R + row;

  // ---- token range of the unit
  int n_tiles, tok_begin = 0, idx_begin = 0, idx_count = 0, page0 = 0, n_unit_pages = 0;
  if (SPARSE) {
    idx_begin = split * p.chunk;
    idx_count = min(p.chunk, p.K - idx_begin);
    if (idx_count < 0) idx_count = 0;
    n_tiles = (idx_count + K::kTileTok - 1) / K::kTileTok;
  } else {
    const int n_pages = (L + 63) >> 6;
    page0 = p.balance ? bal_pg0 : split * p.chunk;
    const int p1 = p.balance ? bal_pg1 : min(page0 + p.chunk, n_pages);
    n_unit_pages = p1 > page0 ? p1 - page0 : 0;
    tok_begin = page0 * 64;
    const int tok_end = n_unit_pages > 0 ? min(p1 * 64, L) : tok_begin;
    n_tiles = (tok_end - tok_begin + K::kTileTok - 1) / K::kTileTok;
    if (n_tiles < 0) n_tiles = 0;
  }
  const int n_vis = L - p.T + t_row + 1;  // dense: visible tokens of this row

  // ---- query operand registers.  Dense: filled after the first DMAs are
  // issued, so that the two latencies overlap.  Sparse: filled first, under
  // the latency of the index-table loads (the DMAs need the table).
  constexpr int QREGS = FP8 ? 8 * K::kQkSteps : 4 * K::kQkSteps;
  int qreg[QREGS];
  // ---- query operand in registers (B side: lane holds row l32, a K slice)
  // bf16: step k covers features 16k .. 16k+15; lane half h holds 8 of them.
  // fp8 : step k covers features 64k .. 64k+63; lane half h holds 32 of them.
  auto load_q = [&]() __attribute__((always_inline)) {
    // Rows past the end read row 0 of the sequence (always present) and are zeroed.
    const int64_t qsafe = row_ok ? qrow : (int64_t)b * p.R;
    const uint8_t* qn = p.q_nope + qsafe * (512 * (FP8 ? 1 : 2));
    const uint8_t* qp = p.q_pe + qsafe * (64 * (FP8 ? 1 : 2));
    const int keep = row_ok ? -1 : 0;
    if (FP8) {
#pragma unroll
      for (int k = 0; k < K::kQkSteps; k++) {
        const uint8_t* src = k < 8 ? qn + 64 * k + 32 * h : qp + 32 * h;
        const i32x4_t a = *(const i32x4_t*)src;
        const i32x4_t c = *(const i32x4_t*)(src + 16);
#pragma unroll
        for (int i = 0; i < 4; i++) { qreg[8 * k + i] = a[i] & keep; qreg[8 * k + 4 + i] = c[i] & keep; }
      }
    } else {
#pragma unroll
      for (int k = 0; k < K::kQkSteps; k++) {
        const uint8_t* src = k < 32 ? qn + 2 * (16 * k + 8 * h) : qp + 2 * (16 * (k - 32) + 8 * h);
        const i32x4_t a = *(const i32x4_t*)src;
#pragma unroll
        for (int i = 0; i < 4; i++) qreg[4 * k + i] = a[i] & keep;
      }
    }
  };

  if constexpr (SPARSE) load_q();

  // ---- unit table in LDS.  Dense: physical page of each page of the unit
  // (-1 if out of range).  Sparse: address of each index's token row, or of
  // the zero row for padding / out-of-range entries.
  const uint64_t zero_row = (uint64_t)(uintptr_t)g_zero_row;
  if (SPARSE) {
    const int32_t* idx = p.topk + ((int64_t)b * p.T + (rb / p.n_hb)) * p.K + idx_begin;
    const int n_ent = n_tiles * K::kTileTok;
    // A thread's entries (at most kTableCap / (64 RG)): every index load is
    // issued before any is used, then every block-table load, so the two
    // dependent latencies are paid once, not once per entry.
    constexpr int EPT = (kTableCap + 64 * RG - 1) / (64 * RG);
    int jv[EPT], pgv[EPT];
#pragma unroll
    for (int k = 0; k < EPT; k++) {
      const int e = threadIdx.x + k * 64 * RG;
      jv[k] = e < idx_count ? idx[e] : -1;
    }
#pragma unroll
    for (int k = 0; k < EPT; k++) {
      const int j = jv[k];
      pgv[k] = (j >= 0 && j < L) ? p.block_table[(int64_t)b * p.MB + (j >> 6)] : -1;
    }
#pragma unroll
    for (int k = 0; k < EPT; k++) {
      const int e = threadIdx.x + k * 64 * RG;
      const int j = jv[k], pg = pgv[k];
      const uint64_t a = (j >= 0 && j < L && pg >= 0 && pg < p.NB)
                             ? (uint64_t)(uintptr_t)(p.kv + ((int64_t)pg * 64 + (j & 63)) * K::kRowBytes)
                             : zero_row;
      if (e < n_ent) table64[e] = a;
    }
    if (threadIdx.x < K::kTileTok) table64[kTableCap + threadIdx.x] = zero_row;
  } else {
    const int32_t* bt = p.block_table + (int64_t)b * p.MB + page0;
    for (int e = threadIdx.x; e < n_unit_pages; e += 64 * RG) {
      const int pg = bt[e];
      table[e] = (pg >= 0 && pg < p.NB) ? pg : -1;
    }
  }
  __syncthreads();


  // ---- DMA source offsets.  Wave w fills tile units [w*NI*64, (w+1)*NI*64):
  // instruction j writes LDS units pos = (w*NI + j)*64 + lane, i.e. token
  // t = pos / kUnits, swizzled unit c' = pos % kUnits, and so fetches global
  // unit (t, c' ^ swz(t)).  The pattern repeats every NPRE instructions (16
  // tokens) when NI > 18.  Kept per lane as token | (byte in token) << 8.
  int dma_tc[NPRE];
#pragma unroll
  for (int j = 0; j < NPRE; j++) {
    const int pos = (wave * NI + j) * 64 + lane;
    const int t = pos / K::kUnits;
    const int c = (pos % K::kUnits) ^ K::swz(t);
    dma_tc[j] = SPARSE ? (t | (16 * c) << 8) : t * K::kRowBytes + 16 * c;   // dense: byte offset in the tile
  }
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;

  // Source of one tile's DMA.  Dense: a buffer descriptor over the tile's
  // existing tokens (past the sequence, a bad page or a tile past the end
  // of the unit: fewer or no bytes, so those reads return zeros).  Sparse:
  // the tile's slice of the row table (n_valid = 0 for a tile past the end).
  struct DmaSrc {
    i32x4_t rsrc;
    LDS_AS const uint64_t* rows;   // sparse: the tile's token-row addresses
    int n_valid;
  };
  // Page of tile i (dense; the same LDS word in every lane).  Split from
  // dma_prepare so that the pipelined steps can read the next step's page
  // early and build its descriptor late, off the step's critical start.
  auto dma_page = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) {
      return 0;
    } else {
      const int tok0 = tok_begin + (i < n_tiles ? i : 0) * K::kTileTok;
      return n_tiles > 0 ? table[(tok0 >> 6) - page0] : -1;
    }
  };
  auto dma_prepare_pg = [&](int i, int pg_v) __attribute__((always_inline)) -> DmaSrc {
    DmaSrc d;
    const bool real = i < n_tiles;
    if (SPARSE) {
      d.rsrc = i32x4_t{0, 0, 0, 0};
      d.rows = table64 + (real ? i * K::kTileTok : kTableCap);   // past the end: zero rows
      d.n_valid = real ? K::kTileTok : 0;
    } else {
      const int tok0 = tok_begin + (real ? i : 0) * K::kTileTok;
      // Taken into a scalar register at once so that the descriptor
      // arithmetic below stays on the scalar unit.
      const int pg = n_tiles > 0 ? __builtin_amdgcn_readfirstlane(pg_v) : -1;
      const int n_valid = (real && pg >= 0) ? min(K::kTileTok, L - tok0) : 0;
      d.rsrc = buffer_rsrc(p.kv + ((int64_t)(pg >= 0 ? pg : 0) * 64 + (tok0 & 63)) * K::kRowBytes,
                           (uint32_t)(n_valid * K::kRowBytes));
      d.rows = table64;
      d.n_valid = n_valid;
    }
    return d;
  };
  auto dma_prepare = [&](int i) __attribute__((always_inline)) -> DmaSrc { return dma_prepare_pg(i, dma_page(i)); };
  // DMA instruction j of a tile into ring slot `slot`.
  auto dma_issue = [&](const DmaSrc& d, int slot, int j) __attribute__((always_inline)) {
    const uint32_t dst = lds_u32 + slot * kTileBytes + (wave * NI + j) * 1024;
    if (SPARSE) {
      const int tc = dma_tc[j % NPRE];
      const int t = (tc & 255) + (j / NPRE) * 16;
      const int cb = tc >> 8;
      dma16((const void*)(uintptr_t)(d.rows[t] + cb), dst);
    } else {
      dma16_buf(dma_tc[j % NPRE], d.rsrc, (j / NPRE) * 16 * K::kRowBytes, dst);
    }
  };
  auto issue_tile = [&](int i, int slot) __attribute__((always_inline)) {
    const DmaSrc d = dma_prepare(i);
#pragma unroll
    for (int j = 0; j < NI; j++) dma_issue(d, slot, j);
  };

  // Pass 0's first tiles go out before the query loads, so that the two
  // latencies overlap.  (A second pass issues them again at its start.)
  auto issue_first_tiles = [&]() __attribute__((always_inline)) {
    if (n_tiles > 0) {
      if constexpr (PIPE) {
#pragma unroll
        for (int i = 0; i < NS - 1; i++) issue_tile(i, i);
      } else {
        issue_tile(0, 0);
      }
    }
  };
  issue_first_tiles();

  if constexpr (!SPARSE) load_q();

  // ---- per-lane LDS read offsets (within a tile)
  // QK operand A = K tile rows: token 32*tb + l32, unit(s) for step k.
  int a_off[FP8 ? 2 : 4];
  if (FP8) {
    const int f = K::swz(l32);
#pragma unroll
    for (int e = 0; e < 2; e++) a_off[e] = l32 * K::kRowBytes + 16 * ((2 * h + e) ^ f);
  } else {
    const int x = h ^ K::swz(l32);
#pragma unroll
    for (int m = 0; m < 4; m++) a_off[m] = l32 * K::kRowBytes + 16 * ((2 * m) ^ x);
  }
  // PV operand A = V^T via transpose reads; [read r][fb parity].
  // fp8: read r covers tokens 16 r + (lane's token), so only read 0's
  // offsets are kept and read r adds the compile-time 16 r rows.
  constexpr int NRD = FP8 ? 4 : 2;
  int v_off[NRD][2];
  {
    const int i = lane & 15, g = lane >> 4, e = g & 1;
    if (FP8) {
      const int sp = i >> 1, q = i & 1, sig = sp >> 2;
      const int t = 8 * sig + 4 * h + (sp & 3);
      const int base = t * K::kRowBytes + 16 * (e ^ h) + 8 * q;
      v_off[0][0] = base + 32 * sig;   // even feature block: fb ^ sig = fb + sig
      v_off[0][1] = base - 32 * sig;   // odd feature block : fb ^ sig = fb - sig
    } else {
      const int sp = i >> 2, q = i & 3, sig = sp >> 1;
#pragma unroll
      for (int r = 0; r < NRD; r++) {
        const int t = 8 * r + 4 * h + sp;
        const int base = t * K::kRowBytes + 16 * ((2 * e + (q >> 1)) ^ (h | (r << 1))) + 8 * (q & 1);
        v_off[r][0] = base + 64 * sig;
        v_off[r][1] = base - 64 * sig;
      }
    }
  }

  // ---- operand loaders
  // QK product n: fp8 -> step n/2 of token block n%2; bf16 -> step n.
  constexpr int NQK = FP8 ? 2 * K::kQkSteps : K::kQkSteps;     // 18 | 36
  constexpr int NPV = FP8 ? 16 : 32;                            // fp8: block fb; bf16: 2 fb + kk
  typedef typename std::conditional<FP8, i32x8_t, bf16x8_t>::type opnd_t;
  auto ld_qk = [&](const LDS_AS uint8_t* tile, int n) -> opnd_t {
    if constexpr (FP8) {
      const LDS_AS uint8_t* base = tile + (n / K::kQkSteps) * 32 * K::kRowBytes + 64 * (n % K::kQkSteps);
      const i32x4_t lo = *(const LDS_AS i32x4_t*)(base + a_off[0]);
      const i32x4_t hi = *(const LDS_AS i32x4_t*)(base + a_off[1]);
      return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return __builtin_bit_cast(bf16x8_t, *(const LDS_AS i32x4_t*)(tile + a_off[n & 3] + 128 * (n >> 2)));
    }
  };
  auto ld_pv = [&](const LDS_AS uint8_t* tile, int n) -> opnd_t {
    if constexpr (FP8) {
      i32x8_t a;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const i32x2_t d = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS_AS i32x2_t*)(tile + v_off[0][n & 1] + 16 * r * K::kRowBytes + 32 * n));
        a[2 * r] = d[0];
        a[2 * r + 1] = d[1];
      }
      return a;
    } else {
      const int fb = n >> 1, kk = n & 1;
      const i16x4_t d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(tile + v_off[0][fb & 1] + 64 * fb + 16 * kk * K::kRowBytes));
      const i16x4_t d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4_t*)(tile + v_off[1][fb & 1] + 64 * fb + 16 * kk * K::kRowBytes));
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const i16x8_t cat = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      return __builtin_bit_cast(bf16x8_t, cat);
    }
  };

  // ---- accumulators and softmax state (per lane: row l32, its half of tokens)
  //
  // Each row accumulates O and l relative to a fixed reference m_ref (log2
  // domain), set at the first tile where the row sees any token; later
  // tiles add their contributions scaled by 2^(tile max - m_ref).  So the
  // accumulators are never rescaled inside the loop.  Only if a row's tile
  // maximum ever exceeds m_ref by more than 2^64 (fp32 headroom for O) is the
  // whole unit run a second time with m_ref = that row's true maximum.
  f32x16_t oacc[16];
  // fp8: ones x P^T, the row sum of the rounded weights, normalizes O, so
  // that the up to 2^-4 rounding of each weight cancels.  bf16 weights are
  // rounded to 2^-9; their row sum l_r comes from dot products of the
  // packed weights with ones (fp32 accumulation), so that for bf16 too the
  // numerator and the denominator of O hold the same rounded weights.
  f32x16_t lsum;
  float m_ref = kNegBig;
  float m_seen = -INFINITY;        // running lane maximum, for the second pass
  float l_f = 0.f;                 // this half's sum of the unrounded weights (gives lse)
  float l_r = 0.f;                 // bf16: this half's sum of the rounded weights (normalizes O)
  float l_q2 = 0.f;                // fp8 without residual: bound of this half's sum of squared weights
  int top_sc = -1;                 // fp8 without residual: highest block exponent of a tile so far,
  int top_tile = 0;                //   the first tile that reached it,
  float top_q2 = 0.f;              //   and that tile's share of l_q2
  const float c_qk = p.qk_scale;   // softmax_scale * log2(e) [* q_scale * kv_scale]
  const int e8m0_one = 127;        // E8M0 scale 2^0 (a VGPR operand of the inline-asm products)

  // Softmax output of one tile, consumed by its PV products.
  struct PTile {
    i32x8_t pb, pbl;    // fp8: e4m3 weights (and residual); bf16: two bf16x8 packed
    int sc, scl;        // fp8: E8M0 scales of pb / pbl
  };

  // QK product n on accumulator sacc (VGPR chain).
  auto qk_mfma = [&](f32x16_t (&sacc)[K::kTokBlocks], int n, const opnd_t& a) {
    if constexpr (FP8) {
      const int k = n % K::kQkSteps, tb = n / K::kQkSteps;   // token block 0's chain first
      const i32x8_t bq = {qreg[8 * k], qreg[8 * k + 1], qreg[8 * k + 2], qreg[8 * k + 3],
                          qreg[8 * k + 4], qreg[8 * k + 5], qreg[8 * k + 6], qreg[8 * k + 7]};
      if (k == 0) mfma_f8_first_plain(sacc[tb], a, bq);
      else mfma_f8_acc_plain(sacc[tb], a, bq);
    } else {
      const i32x4_t bq = {qreg[4 * n], qreg[4 * n + 1], qreg[4 * n + 2], qreg[4 * n + 3]};
      if (n == 0) mfma_bf16_first(sacc[0], a, __builtin_bit_cast(bf16x8_t, bq));
      else mfma_bf16_acc(sacc[0], a, __builtin_bit_cast(bf16x8_t, bq));
    }
  };
  // PV product n of a tile with softmax output pt (resid_c: also the
  // residual weights, fp8 only).
  auto pv_mfma = [&](int n, const opnd_t& a, const PTile& pt, auto resid_c) {
    if constexpr (FP8) {
      oacc[n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pt.pb, oacc[n], 0, 0, 0, 127, 0, pt.sc);
      if constexpr (decltype(resid_c)::value)
        oacc[n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pt.pbl, oacc[n], 0, 0, 0, 127, 0, pt.scl);
    } else {
      const i32x4_t half = n & 1 ? i32x4_t{pt.pb[4], pt.pb[5], pt.pb[6], pt.pb[7]}
                                 : i32x4_t{pt.pb[0], pt.pb[1], pt.pb[2], pt.pb[3]};
      oacc[n >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, half), oacc[n >> 1], 0,
                                                             0, 0);
    }
  };
  auto row_sum_mfma = [&](const PTile& pt, auto resid_c) {
    // The all-ones operand is rebuilt at each use rather than held live.
    const i32x8_t ones8 = {kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4,
                           kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4};
    const bf16x8_t ones16 = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                             (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    if constexpr (FP8) {
      mfma_f8_acc(lsum, ones8, pt.pb, e8m0_one, pt.sc);
      if constexpr (decltype(resid_c)::value) mfma_f8_acc(lsum, ones8, pt.pbl, e8m0_one, pt.scl);
    }
    (void)ones16;
  };

  // Padding after a tile's QK chain, tied to its score accumulators.
  auto drain_scores = [&](f32x16_t (&sacc)[K::kTokBlocks]) {
    if constexpr (K::kTokBlocks == 2) mfma_drain(sacc[0], sacc[1]);
    else mfma_drain(sacc[0]);
  };

  // ---- softmax of one tile, in stages, token block by token block.  The
  // pipelined loops place the stages of token block 0 between the QK
  // products of block 1 and those of block 1 between the PV products of the
  // previous tile, so that their VALU work runs while the matrix core is busy.
  //
  // Register v of token block tb holds token 32*tb + 8*(v/4) + 4*h + v%4.
  // fp8: each token block carries its own E8M0 scale.  In the P operand,
  // bytes 0-15 of both wave halves are token block 0 and bytes 16-31 token
  // block 1, and the MFMA applies lane j's B scale to the first of those
  // K-blocks of column j and lane j+32's to the second.
  constexpr int NEXP = 4;                // exponent stages per token block, four scores each
  struct SmState {
    float ml[K::kTokBlocks];     // this lane's maximum of the block's scores
    float mr[K::kTokBlocks];     // the row's maximum (feature-split stages)
    float shift[K::kTokBlocks];  // exponent offset applied to the block's scaled scores
    float psum[K::kTokBlocks];   // this lane's sum of the block's unrounded weights
    float prsum[K::kTokBlocks];  // bf16: this lane's sum of the block's rounded weights
    int sc[K::kTokBlocks];       // fp8: E8M0 scale of the block's weights
  };

  // Mask of token block tb: compare each register's compile-time token
  // offset (without the 4*h) against one per-lane limit.  Selects, not
  // branches: a branch here splits the loop body and costs registers.
  auto sm_mask = [&](f32x16_t (&sacc)[K::kTokBlocks], int i, int tb) {
    if (SPARSE) {
      const uint64_t a = lane < K::kTileTok ? table64[i * K::kTileTok + lane] : zero_row;
      const uint64_t valid = __builtin_amdgcn_ballot_w64(a != zero_row) | (K::kTileTok == 64 ? 0ull : ~0ull << 32);
      const uint64_t mine = valid >> (4 * h);
#pragma unroll
      for (int v = 0; v < 16; v++)
        sacc[tb][v] = (mine >> (32 * tb + 8 * (v >> 2) + (v & 3))) & 1 ? sacc[tb][v] : -INFINITY;
    } else {
      const int lim = n_vis - (tok_begin + i * K::kTileTok) - 4 * h;   // offsets at or past lim are masked
#pragma unroll
      for (int v = 0; v < 16; v++)
        sacc[tb][v] = 32 * tb + 8 * (v >> 2) + (v & 3) < lim ? sacc[tb][v] : -INFINITY;
    }
  };
  // Stage "lane maximum of token block tb".
  auto sm_max = [&](f32x16_t (&sacc)[K::kTokBlocks], int tb, SmState& st) {
    float m = sacc[tb][0];
#pragma unroll
    for (int v = 1; v < 16; v++) m = fmaxf(m, sacc[tb][v]);
    st.ml[tb] = m;
  };
  // Stage "row maximum of token block tb": the reference (set by the first
  // block a row sees), the block's shift and (fp8) its scale.
  auto sm_row = [&](int tb, bool& jumped, SmState& st) {
    const float ml = st.ml[tb] * c_qk;   // this lane's maximum, scaled (-inf if all masked)
    m_seen = fmaxf(m_seen, ml);
    // A jump is measured against a reference already set by an earlier block.
    jumped |= m_ref != kNegBig && ml > m_ref + 64.f;
    const float mrow = max_across_halves(ml);
    if constexpr (FP8) {
      // P' = 2^(x - mi + 8) in [0, 256] -> e4m3, with mi the integer ceiling
      // of the row's block maximum; the PV MFMA multiplies it by 2^(mi - m_ref)
      // through the block's E8M0 scale.
      if (m_ref == kNegBig && mrow != -INFINITY) m_ref = ceilf(mrow);
      const float mi = mrow == -INFINITY ? m_ref : ceilf(mrow);
      st.shift[tb] = 8.f - mi;
      // E8M0 biased exponent of 2^(mi - m_ref), clamped to the format
      // (0 = 2^-127: the block's weights are negligible there).
      const float dexp = fminf(mi - m_ref, 64.f);
      st.sc[tb] = dexp < -126.f ? 0 : (int)dexp + 127;
      pin(st.sc[tb]);
      pin(st.shift[tb]);
    } else {
      if (m_ref == kNegBig && mrow != -INFINITY) m_ref = mrow;
      st.shift[tb] = -m_ref;
      st.sc[tb] = 0;
    }
    st.psum[tb] = 0.f;
    st.prsum[tb] = 0.f;
  };
  // Stage "exponents of registers 4d .. 4d+3 of token block tb".
  auto sm_exp = [&](f32x16_t (&sacc)[K::kTokBlocks], int tb, int d, SmState& st, PTile& pt, auto resid_c) {
    const int v = 4 * d;
    const float sh = st.shift[tb];
    const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v], c_qk, sh));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 1], c_qk, sh));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 2], c_qk, sh));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 3], c_qk, sh));
    st.psum[tb] += (e0 + e1) + (e2 + e3);
    pin(st.psum[tb]);
    if constexpr (FP8) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
      pin(w);
      pt.pb[4 * tb + d] = w;
      if constexpr (decltype(resid_c)::value) {
        // lo = e4m3(16 (P' - hi)): hi + lo/16 holds P' to about 2^-8.
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        int wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (e0 - h01[0]), 16.f * (e1 - h01[1]), 0, false);
        wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (e2 - h23[0]), 16.f * (e3 - h23[1]), wl, true);
        pin(wl);
        pt.pbl[4 * tb + d] = wl;
      } else {
        pt.pbl[4 * tb + d] = 0;
      }
    } else {
      // P operand: registers 8*kk .. 8*kk+7 form k-step kk; two bf16 per dword.
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t lo = {(__bf16)e0, (__bf16)e1};
      const bf16x2_t hi = {(__bf16)e2, (__bf16)e3};
      int wlo = __builtin_bit_cast(int, lo), whi = __builtin_bit_cast(int, hi);
      pin(wlo);
      pin(whi);
      const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
      st.prsum[tb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, whi), one2,
                                                     __builtin_amdgcn_fdot2_f32_bf16(
                                                         __builtin_bit_cast(bf16x2_t, wlo), one2, st.prsum[tb],
                                                         false),
                                                     false);
      pin(st.prsum[tb]);
      pt.pb[2 * d] = wlo;
      pt.pb[2 * d + 1] = whi;
    }
  };
  // Stage "finish": the P operand's scales (lane half h carries token
  // block h's) and this half's unrounded weights join l_f.
  auto sm_finish = [&](const SmState& st, PTile& pt, int tile) {
    if constexpr (FP8) {
      pt.sc = h == 0 ? st.sc[0] : st.sc[1];
      pt.scl = pt.sc > 4 ? pt.sc - 4 : 0;
      l_f += st.psum[0] * __builtin_amdgcn_ldexpf(1.0f, st.sc[0] - 127) +
             st.psum[1] * __builtin_amdgcn_ldexpf(1.0f, st.sc[1] - 127);
      if constexpr (!RESID) {
        // A block's weights are psum * 2^e (e = sc - 127) in l_f's units and
        // none exceeds 2^(8 + e), so their squares sum to at most
        // psum * 2^(2e + 8); kept scaled by 2^-64 (e <= 64, so no overflow).
        const float t2 = __builtin_amdgcn_ldexpf(st.psum[0], 2 * st.sc[0] - 310) +
                         __builtin_amdgcn_ldexpf(st.psum[1], 2 * st.sc[1] - 310);
        l_q2 += t2;
        // The tile holding the row's heaviest block (by its exponent; the
        // same in both halves of the row, so both pick the same tile).
        const int tsc = max(st.sc[0], st.sc[1]);
        const bool up = tsc > top_sc;
        top_sc = up ? tsc : top_sc;
        top_tile = up ? tile : top_tile;
        top_q2 = up ? t2 : top_q2;
      }
    } else {
      pt.sc = pt.scl = 0;
      l_f += st.psum[0];
      l_r += st.prsum[0];
    }
  };
  // Stage k of token block tb's softmax (compile-time k once loops are
  // unrolled): [mask], max, row, NEXP exponent stages; no-op past the end.
  constexpr int NSTAGE_BLOCK = 2 + NEXP;
  auto sm_block_stage = [&](int k, bool mask, f32x16_t (&sacc)[K::kTokBlocks], int i, int tb, bool& jumped,
                            SmState& st, PTile& pt, auto resid_c) {
    if (mask) {
      if (k == 0) { sm_mask(sacc, i, tb); return; }
      k -= 1;
    }
    if (k == 0) sm_max(sacc, tb, st);
    else if (k == 1) sm_row(tb, jumped, st);
    else if (k < 2 + NEXP) sm_exp(sacc, tb, k - 2, st, pt, resid_c);
  };
  auto softmax_all = [&](f32x16_t (&sacc)[K::kTokBlocks], int i, bool& jumped, PTile& pt, auto resid_c) {
    SmState st;
#pragma unroll
    for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
      for (int k = 0; k < NSTAGE_BLOCK + 1; k++) sm_block_stage(k, true, sacc, i, tb, jumped, st, pt, resid_c);
    sm_finish(st, pt, i);
  };

  // Finer stages for the feature-split step, whose schedule gives each one
  // a matrix product of its own: [mask], max, row (two halves), and eight
  // exponent stages of two scores each.
  constexpr int FS_NEXP = 8;
  constexpr int FS_NSTAGE = 3 + FS_NEXP;
  // Unmasked stages (`clean`) run only on tiles after tile 0, which every
  // row sees in full, so m_ref is set and the scores are finite: the
  // sentinel and -inf cases drop out.
  auto fs_row_a = [&](int tb, bool& jumped, SmState& st, bool clean) {
    const float ml = st.ml[tb] * c_qk;
    m_seen = fmaxf(m_seen, ml);
    jumped |= (clean || m_ref != kNegBig) && ml > m_ref + 64.f;
    st.mr[tb] = max_across_halves(ml);
  };
  auto fs_row_b = [&](int tb, SmState& st, bool clean) {
    const float mrow = st.mr[tb];
    if (!clean && m_ref == kNegBig && mrow != -INFINITY) m_ref = ceilf(mrow);
    const float mi = (clean || mrow != -INFINITY) ? ceilf(mrow) : m_ref;
    st.shift[tb] = 8.f - mi;
    const float dexp = fminf(mi - m_ref, 64.f);
    st.sc[tb] = dexp < -126.f ? 0 : (int)dexp + 127;
    pin(st.sc[tb]);
    pin(st.shift[tb]);
  };
  // Scores 2d and 2d+1 of token block tb: byte pair d & 1 of P word 4 tb + d / 2.
  auto fs_exp = [&](f32x16_t (&sacc)[K::kTokBlocks], int tb, int d, SmState& st, PTile& pt) {
    const float sh = st.shift[tb];
    const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][2 * d], c_qk, sh));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][2 * d + 1], c_qk, sh));
    st.psum[tb] = d == 0 ? e0 + e1 : st.psum[tb] + (e0 + e1);
    pin(st.psum[tb]);
    // The first pair fills the low half; the high half is written by the
    // second pair, so the word's earlier contents do not matter: the spent
    // bits of e0 serve, which spares a register clear.
    int w;
    if (d & 1) w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, pt.pb[4 * tb + d / 2], true);
    else w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, __builtin_bit_cast(int, e0), false);
    pin(w);
    pt.pb[4 * tb + d / 2] = w;
  };
  auto fs_stage = [&](int k, bool mask, f32x16_t (&sacc)[K::kTokBlocks], int i, int tb, bool& jumped,
                      SmState& st, PTile& pt) {
    if (mask) {
      if (k == 0) { sm_mask(sacc, i, tb); return; }
      k -= 1;
    }
    if (k == 0) sm_max(sacc, tb, st);
    else if (k == 1) fs_row_a(tb, jumped, st, !mask);
    else if (k == 2) fs_row_b(tb, st, !mask);
    else if (k < FS_NSTAGE) fs_exp(sacc, tb, k - 3, st, pt);
  };

  // ---- tiles [0, n_clean) need no mask: every row sees all their tokens
  // (dense: the tile ends at or before the first draft row's causal limit).
  // The tiles after them take the masked softmax.
  int n_clean = 0;
  if (!SPARSE) {
    const int lim0 = L - p.T + 1 - tok_begin;
    n_clean = lim0 > 0 ? min(n_tiles, lim0 / K::kTileTok) : 0;
  }

  // ---- one step of the pipelined loop (four waves, fp8): QK of tile i+1
  // (token block 0, then block 1) with the DMA of tile i+NS-1 spread between
  // its products and token block 0's softmax between block 1's products;
  // then the PV products of tile i with block 1's softmax between them.
  auto pipe_step = [&](int i, f32x16_t (&sacc)[K::kTokBlocks], PTile& pt, bool& jumped, DmaSrc& src, int& pg_nx,
                       auto mask_c, auto resid_c) __attribute__((always_inline)) {
    constexpr bool mask = decltype(mask_c)::value;
    constexpr int KS = K::kQkSteps;
    // Tile i+1 resident (one tile may still be in flight behind it); every
    // wave is done with tile i-1, whose slot the DMA below refills.
    wait_vmcnt<NI * (NS - 3)>();
    lds_barrier();
    const LDS_AS uint8_t* tv = lds + (i % NS) * kTileBytes;
    const LDS_AS uint8_t* tq = lds + ((i + 1) % NS) * kTileBytes;
    const int nxt = i + NS - 1;   // past the end: a zero fill of a free slot; src covers it
    constexpr int DSTRIDE = NQK / NI;
    static_assert(NQK % NI == 0, "DMA spread");
    opnd_t qa[3], va[3];
    PTile pn;
    SmState st;
    qa[0] = ld_qk(tq, 0);
    qa[1] = ld_qk(tq, 1);
#pragma unroll
    for (int n = 0; n < NQK; n++) {
      if (n + 2 < NQK) qa[(n + 2) % 3] = ld_qk(tq, n + 2);
      if (n == NQK - 2) va[0] = ld_pv(tv, 0);
      if (n == NQK - 1) va[1] = ld_pv(tv, 1);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfma(sacc, n, qa[n % 3]);
      if (n == KS) mfma_drain(sacc[0]);          // block 0's chain ended one product ago
      if (n > KS) sm_block_stage(n - KS - 1, mask, sacc, i + 1, 0, jumped, st, pn, resid_c);
      if (n % DSTRIDE == DSTRIDE - 1) dma_issue(src, nxt % NS, n / DSTRIDE);
      if (n == 1) pg_nx = dma_page(nxt + 1);     // consumed at the end of the step
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(NSTAGE_BLOCK + 1 <= KS - 1, "block 0's stages fit between block 1's products");
#pragma unroll
    for (int n = 0; n < NPV; n++) {
      if (n + 2 < NPV) va[(n + 2) % 3] = ld_pv(tv, n + 2);
      __builtin_amdgcn_sched_barrier(0);
      pv_mfma(n, va[n % 3], pt, resid_c);
      if (n == 0) mfma_drain(sacc[1]);
      if (n > 0) sm_block_stage(n - 1, mask, sacc, i + 1, 1, jumped, st, pn, resid_c);
      if (n == NSTAGE_BLOCK + 2) sm_finish(st, pn, i + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(NSTAGE_BLOCK + 3 <= NPV, "block 1's stages fit between the PV products");
    row_sum_mfma(pt, resid_c);
    src = dma_prepare_pg(nxt + 1, pg_nx);        // the next step's DMA source
    pt = pn;
  };

  // ---- feature split (FS): wave w accumulates O for all four row blocks
  // of the workgroup over output features [128 w, 128 w + 128), so every
  // byte of V is read from LDS by one wave instead of four.  The P tile
  // (fp8, in the B-operand layout) and the E8M0 scales of each row block
  // pass from the wave that computed them to the others through LDS.
  // oacc[4 * r + fs]: row block (w + r) mod 4 (r = 0 is the wave's own),
  // feature block 4 w + fs; r and fs are compile-time indices.
  // A P tile's two 16-byte halves per lane sit in separate 1 KiB halves of
  // the wave's 2 KiB slot, lane-contiguous, so that 16 lanes of a 16-byte
  // LDS access hit 16 distinct bank quads.
  auto fs_write_p = [&](const PTile& pt) {
    LDS_AS i32x4_t* dst = (LDS_AS i32x4_t*)(pbuf + wave * 2048 + lane * 16);
    dst[0] = i32x4_t{pt.pb[0], pt.pb[1], pt.pb[2], pt.pb[3]};
    dst[64] = i32x4_t{pt.pb[4], pt.pb[5], pt.pb[6], pt.pb[7]};
    scbuf[wave * 64 + lane] = pt.sc;       // lane half h: token block h's scale
  };
  auto fs_read_p = [&](int rq, i32x8_t& pb, int& sc) {
    const LDS_AS i32x4_t* src = (const LDS_AS i32x4_t*)(pbuf + rq * 2048 + lane * 16);
    const i32x4_t a = src[0], c = src[64];
    pb = i32x8_t{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    sc = scbuf[rq * 64 + lane];
  };
  auto fs_pv_mfma = [&](int r, int fs, const i32x8_t& vt, const i32x8_t& pb, int sc) {
    oacc[4 * r + fs] =
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vt, pb, oacc[4 * r + fs], 0, 0, 0, 127, 0, sc);
  };
  // V^T operand of this wave's feature block fs.
  auto fs_ld_v = [&](const LDS_AS uint8_t* tile, int fs) -> i32x8_t {
    if constexpr (FS) return ld_pv(tile, 4 * wave + fs);
    else return i32x8_t{};
  };
  // PV of a whole tile (the last one): own row block from registers, the
  // others from the P tiles in LDS; vt holds the tile's Vᵀ operands.
  auto fs_pv_tile = [&](const i32x8_t (&vt)[4], const PTile& pt) {
    i32x8_t pbq[2];
    int scq[2];
    fs_read_p((wave + 1) & 3, pbq[0], scq[0]);
#pragma unroll
    for (int f = 0; f < 4; f++) fs_pv_mfma(0, f, vt[f], pt.pb, pt.sc);
#pragma unroll
    for (int n = 0; n < 12; n++) {
      const int j = n >> 2, f = n & 3;
      if (f == 0 && j + 1 < 3) fs_read_p((wave + 2 + j) & 3, pbq[(j + 1) & 1], scq[(j + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      fs_pv_mfma(1 + j, f, vt[f], pbq[j & 1], scq[j & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One step of the pipelined loop with the feature split: QK of tile i+1
  // and PV of tile i in three phases around two barriers.  A tile's softmax
  // spans two steps, so that its VALU work sits between matrix products in
  // every phase (one product hides only part of a stage):
  //  A  QK of tile i+1, token block 0 (9 products), with the last four
  //     exponent stages of tile i's block 1 and tile i's finish between
  //     them; then tile i's P tile is published.
  //  -- barrier: every row block's P tile of tile i is in LDS.
  //  B  QK of tile i+1, token block 1 (9 products), with the first stages
  //     of tile i+1's block 0 between them; Vᵀ of tile i is loaded.
  //  C  PV of tile i: own row block (4 products, P from registers), then
  //     the other three (12, P from LDS), with the first stages of tile
  //     i+1's block 1 and the last four of its block 0 between them.
  // The DMA of tile i+NS-1 is spread over A and B.  Entering, st / pt hold
  // tile i's softmax state and P tile with all but block 1's last four
  // exponent stages and the finish done, and sacc[1] holds tile i's block-1
  // scores; leaving, the same holds for tile i+1.
  auto pipe_step_fs = [&](int i, f32x16_t (&sacc)[K::kTokBlocks], PTile& pt, SmState& st, bool& jumped, DmaSrc& src,
                          int& pg_nx, auto mask_c) __attribute__((always_inline)) {
    constexpr bool mask = decltype(mask_c)::value;     // tile i+1's softmax takes the mask
    constexpr int HEAD = FS_NSTAGE - 4 + (mask ? 1 : 0);   // stages before the last four exponent stages
    constexpr int KS = K::kQkSteps;
    static_assert(NI == 9 && KS == 9 && NQK == 18, "schedule of the feature-split step");
    wait_vmcnt<NI * (NS - 3)>();
    lds_barrier();     // tile i+1 resident; slot i-1 free; every wave done with tile i-1's P tiles
    const LDS_AS uint8_t* tq = lds + ((i + 1) % NS) * kTileBytes;
    const LDS_AS uint8_t* tv = lds + (i % NS) * kTileBytes;
    const int nxt = i + NS - 1;   // src (built by the previous step) covers this tile
    opnd_t qa[3];
    qa[0] = ld_qk(tq, 0);
    qa[1] = ld_qk(tq, 1);
    // A: tile i's block-1 exponent stages 4..7 at a = 0, 2, 4, 6, finish at 7,
    // publish at 8; DMA instructions 0..3 at a = 1, 3, 5, 7.
#pragma unroll
    for (int a = 0; a < KS; a++) {
      qa[(a + 2) % 3] = ld_qk(tq, a + 2);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfma(sacc, a, qa[a % 3]);
      if (a % 2 == 0 && a < 8) fs_exp(sacc, 1, 4 + a / 2, st, pt);
      if (a == 7) sm_finish(st, pt, i);
      if (a == 8) fs_write_p(pt);
      if (a % 2 == 1) dma_issue(src, nxt % NS, a / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
    lds_barrier();     // every P tile of tile i published
    // B: tile i+1's block-0 stages 0..HEAD-1 at b = 1..HEAD; Vᵀ of tile i at
    // b = 0, 2, 4, 6; DMA instructions 4..8 at b = 0, 2, 4, 6, 8.
    SmState sn;
    PTile pn;
    i32x8_t vt[4];
#pragma unroll
    for (int b = 0; b < KS; b++) {
      const int n = KS + b;
      if (n + 2 < NQK) qa[(n + 2) % 3] = ld_qk(tq, n + 2);
      if (b % 2 == 0 && b < 8) vt[b / 2] = fs_ld_v(tv, b / 2);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfma(sacc, n, qa[n % 3]);
      if (b == 0) mfma_drain(sacc[0]);           // block 0's chain ended one product ago
      if (b >= 1 && b - 1 < HEAD) fs_stage(b - 1, mask, sacc, i + 1, 0, jumped, sn, pn);
      if (b % 2 == 0) dma_issue(src, nxt % NS, 4 + b / 2);
      if (b == 1) pg_nx = dma_page(nxt + 1);     // consumed at the end of phase C
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(FS_NSTAGE - 4 + 1 <= KS - 1, "block 0's first stages fit phase B");
    // C: PV of tile i (own row block at m = 0..3, the others at m = 4..15);
    // tile i+1's block-1 stages 0..HEAD-1 at odd m, block-0 exponent stages
    // 4..7 at m = 2, 6, 10, 14.
    i32x8_t pbq[2];
    int scq[2];
#pragma unroll
    for (int m = 0; m < 16; m++) {
      const int n = m - 4, j = n >> 2, f = n & 3;
      if (m == 2) fs_read_p((wave + 1) & 3, pbq[0], scq[0]);
      if (m >= 4 && f == 0 && j + 1 < 3) fs_read_p((wave + 2 + j) & 3, pbq[(j + 1) & 1], scq[(j + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (m < 4) fs_pv_mfma(0, m, vt[m], pt.pb, pt.sc);
      else fs_pv_mfma(1 + j, f, vt[f], pbq[j & 1], scq[j & 1]);
      if (m == 0) mfma_drain(sacc[1]);           // block 1's chain ended one product ago
      if (m % 2 == 1 && m / 2 < HEAD) fs_stage(m / 2, mask, sacc, i + 1, 1, jumped, sn, pn);
      if (m % 4 == 2) fs_exp(sacc, 0, 4 + m / 4, sn, pn);
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(FS_NSTAGE - 4 + 1 <= 8, "block 1's first stages fit phase C");
    row_sum_mfma(pt, std::false_type{});
    src = dma_prepare_pg(nxt + 1, pg_nx);        // the next step's DMA source
    pt = pn;
    st = sn;
  };

  // bf16 step: the QK chain of tile i+1 (one token block of 32, 36 products)
  // with the DMA of tile i+NS-1 spread between its products, then the 32 PV
  // products of tile i with the softmax stages of tile i+1 between them.
  // Operands are loaded QD products ahead.
  auto pipe_step_bf16 = [&](int i, f32x16_t (&sacc)[K::kTokBlocks], PTile& pt, bool& jumped, DmaSrc& src,
                            int& pg_nx, auto mask_c) __attribute__((always_inline)) {
    constexpr bool mask = decltype(mask_c)::value;
    constexpr int QD = 2;
    wait_vmcnt<NI * (NS - 3)>();
    lds_barrier();
    const LDS_AS uint8_t* tv = lds + (i % NS) * kTileBytes;
    const LDS_AS uint8_t* tq = lds + ((i + 1) % NS) * kTileBytes;
    const int nxt = i + NS - 1;   // src covers this tile
    constexpr int DSTRIDE = NQK / NI;
    static_assert(NQK % NI == 0, "DMA spread");
    opnd_t qa[QD + 1], va[QD + 1];
#pragma unroll
    for (int n = 0; n < QD; n++) qa[n] = ld_qk(tq, n);
#pragma unroll
    for (int n = 0; n < NQK; n++) {
      if (n + QD < NQK) qa[(n + QD) % (QD + 1)] = ld_qk(tq, n + QD);
      if (n + QD >= NQK) va[n + QD - NQK] = ld_pv(tv, n + QD - NQK);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfma(sacc, n, qa[n % (QD + 1)]);
      if (n % DSTRIDE == DSTRIDE - 1) dma_issue(src, nxt % NS, n / DSTRIDE);
      if (n == 1) pg_nx = dma_page(nxt + 1);     // consumed at the end of the step
      __builtin_amdgcn_sched_barrier(0);
    }
    PTile pn;
    SmState st;
    constexpr int NSB = NSTAGE_BLOCK + (mask ? 1 : 0);
#pragma unroll
    for (int n = 0; n < NPV; n++) {
      if (n + QD < NPV) va[(n + QD) % (QD + 1)] = ld_pv(tv, n + QD);
      __builtin_amdgcn_sched_barrier(0);
      pv_mfma(n, va[n % (QD + 1)], pt, std::false_type{});
      if (n == 0) mfma_drain(sacc[0]);           // the QK chain ended one product ago
      // stages at every third product from n = 1, then the finish
      if (n >= 1 && (n - 1) % 3 == 0 && (n - 1) / 3 < NSB)
        sm_block_stage((n - 1) / 3, mask, sacc, i + 1, 0, jumped, st, pn, std::false_type{});
      if (n == 3 * NSB + 1) sm_finish(st, pn, i + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(3 * (NSTAGE_BLOCK + 1) + 1 < NPV, "the bf16 softmax stages fit between the PV products");
    src = dma_prepare_pg(nxt + 1, pg_nx);        // the next step's DMA source
    pt = pn;
  };


  // bf16 dense step with the barrier between its two phases: QK of tile i+1
  // on operands whose first QD were loaded at the end of the previous step,
  // then (tile i+2 resident for every wave; every wave done with tile i-1)
  // the PV products of tile i with tile i+1's softmax stages and the DMA of
  // tile i+3 between them, and the first QK operands of tile i+2.  So the
  // first QK product of a step does not wait on an LDS read issued after a
  // barrier (MTP-7 batch: 1630 -> 1600 us; B=64, H=128, 16k tokens: 324 ->
  // 319 us; same bits).  A tile's DMA then has one step to land instead of
  // about two, which the sparse gather does not afford (it keeps
  // pipe_step_bf16: 74.7 against 75.3 us).
  auto pipe_step_mid = [&](int i, f32x16_t (&sacc)[K::kTokBlocks], PTile& pt, bool& jumped, DmaSrc& src,
                           int& pg_nx, opnd_t (&qpre)[2], auto mask_c) __attribute__((always_inline)) {
    constexpr bool mask = decltype(mask_c)::value;
    constexpr int QD = 2;
    const LDS_AS uint8_t* tv = lds + (i % NS) * kTileBytes;
    const LDS_AS uint8_t* tq = lds + ((i + 1) % NS) * kTileBytes;
    const LDS_AS uint8_t* tn = lds + ((i + 2) % NS) * kTileBytes;
    const int nxt = i + NS - 1;   // src covers this tile
    opnd_t qa[QD + 1], va[QD + 1];
    qa[0] = qpre[0];
    qa[1] = qpre[1];
#pragma unroll
    for (int n = 0; n < NQK; n++) {
      if (n + QD < NQK) qa[(n + QD) % (QD + 1)] = ld_qk(tq, n + QD);
      if (n + QD >= NQK) va[n + QD - NQK] = ld_pv(tv, n + QD - NQK);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfma(sacc, n, qa[n % (QD + 1)]);
      if (n == 1) pg_nx = dma_page(nxt + 1);     // consumed at the end of the step
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();
    lds_barrier();
    PTile pn;
    SmState st;
    constexpr int NSB = NSTAGE_BLOCK + (mask ? 1 : 0);
    constexpr int DSTRIDE2 = NPV / NI >= 1 ? NPV / NI : 1;
#pragma unroll
    for (int n = 0; n < NPV; n++) {
      if (n + QD < NPV) va[(n + QD) % (QD + 1)] = ld_pv(tv, n + QD);
      if (n == NPV - 4) qpre[0] = ld_qk(tn, 0);
      if (n == NPV - 3) qpre[1] = ld_qk(tn, 1);
      __builtin_amdgcn_sched_barrier(0);
      pv_mfma(n, va[n % (QD + 1)], pt, std::false_type{});
      if (n == 0) mfma_drain(sacc[0]);
      if (n >= 1 && (n - 1) % 3 == 0 && (n - 1) / 3 < NSB)
        sm_block_stage((n - 1) / 3, mask, sacc, i + 1, 0, jumped, st, pn, std::false_type{});
      if (n == 3 * NSB + 1) sm_finish(st, pn, i + 1);
      if (n % DSTRIDE2 == DSTRIDE2 - 1 && n / DSTRIDE2 < NI) dma_issue(src, nxt % NS, n / DSTRIDE2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = (NPV / DSTRIDE2 < NI ? NPV / DSTRIDE2 : NI); j < NI; j++) dma_issue(src, nxt % NS, j);
    src = dma_prepare_pg(nxt + 1, pg_nx);
    pt = pn;
  };

  // ---- the tile loop of one pass.  fs_c: the feature-split step (else
  // every wave owns its rows' whole output); resid_c: fp8 weights also
  // carry their e4m3 residual.
  auto tile_loop = [&](bool& jumped, auto fs_c, auto resid_c) __attribute__((always_inline)) {
    constexpr bool fs = decltype(fs_c)::value;
    // Step-variant tags that depend on this lambda's arguments, so that only
    // the steps a variant uses are instantiated.
    using clean_t = std::integral_constant<bool, fs && !fs>;
    using masked_t = std::integral_constant<bool, fs || !fs>;
    if constexpr (PIPE) {
      if (n_tiles > 0) {
        // Prologue: NS-1 tiles in flight (zero fills past the end keep the
        // count uniform), then QK and softmax of tile 0.
        wait_vmcnt<NI * (NS - 2)>();
        lds_barrier();
        f32x16_t sacc[K::kTokBlocks];
        {
          opnd_t qa[3];
          qa[0] = ld_qk(lds, 0);
          qa[1] = ld_qk(lds, 1);
#pragma unroll
          for (int n = 0; n < NQK; n++) {
            if (n + 2 < NQK) qa[(n + 2) % 3] = ld_qk(lds, n + 2);
            __builtin_amdgcn_sched_barrier(0);
            qk_mfma(sacc, n, qa[n % 3]);
            __builtin_amdgcn_sched_barrier(0);
          }
          drain_scores(sacc);
        }
        PTile pt;
        int i = 0;
        if constexpr (fs) {
          // Tile 0's softmax up to the hand-over point of the step (block 1's
          // last two exponent stages and the finish come in step 0).
          SmState st;
#pragma unroll
          for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
            for (int k = 0; k < FS_NSTAGE + 1 - (tb == 1 ? 4 : 0); k++)
              fs_stage(k, true, sacc, 0, tb, jumped, st, pt);
          DmaSrc src = dma_prepare(NS - 1);
          int pg_nx = 0;
          for (; i + 1 < n_clean; i++) pipe_step_fs(i, sacc, pt, st, jumped, src, pg_nx, clean_t{});
          for (; i + 1 < n_tiles; i++) pipe_step_fs(i, sacc, pt, st, jumped, src, pg_nx, masked_t{});
          // Last tile: the rest of its softmax, publish, PV.
#pragma unroll
          for (int d = 4; d < FS_NEXP; d++) fs_exp(sacc, 1, d, st, pt);
          sm_finish(st, pt, n_tiles - 1);
          fs_write_p(pt);
        } else {
          softmax_all(sacc, 0, jumped, pt, resid_c);
          DmaSrc src = dma_prepare(NS - 1);
          int pg_nx = 0;
          if constexpr (FP8) {
            for (; i + 1 < n_clean; i++) pipe_step(i, sacc, pt, jumped, src, pg_nx, clean_t{}, resid_c);
            for (; i + 1 < n_tiles; i++) pipe_step(i, sacc, pt, jumped, src, pg_nx, masked_t{}, resid_c);
          } else if constexpr (!SPARSE) {
            // tile 1 resident for every wave before the first step's QK
            wait_vmcnt<NI * (NS - 3)>();
            lds_barrier();
            opnd_t qpre[2];
            qpre[0] = ld_qk(lds + (1 % NS) * kTileBytes, 0);
            qpre[1] = ld_qk(lds + (1 % NS) * kTileBytes, 1);
            for (; i + 1 < n_clean; i++) pipe_step_mid(i, sacc, pt, jumped, src, pg_nx, qpre, clean_t{});
            for (; i + 1 < n_tiles; i++) pipe_step_mid(i, sacc, pt, jumped, src, pg_nx, qpre, masked_t{});
          } else {
            for (; i + 1 < n_clean; i++) pipe_step_bf16(i, sacc, pt, jumped, src, pg_nx, clean_t{});
            for (; i + 1 < n_tiles; i++) pipe_step_bf16(i, sacc, pt, jumped, src, pg_nx, masked_t{});
          }
        }

        // Last tile: PV only.
        if constexpr (fs) {
          wait_lgkm0();
          lds_barrier();   // every P tile of the last tile published
          const LDS_AS uint8_t* tv = lds + ((n_tiles - 1) % NS) * kTileBytes;
          i32x8_t vt[4];
#pragma unroll
          for (int f = 0; f < 4; f++) vt[f] = fs_ld_v(tv, f);
          fs_pv_tile(vt, pt);
          row_sum_mfma(pt, clean_t{});
        } else {
          const LDS_AS uint8_t* tv = lds + ((n_tiles - 1) % NS) * kTileBytes;
          opnd_t va[3];
          va[0] = ld_pv(tv, 0);
          va[1] = ld_pv(tv, 1);
#pragma unroll
          for (int n = 0; n < NPV; n++) {
            if (n + 2 < NPV) va[(n + 2) % 3] = ld_pv(tv, n + 2);
            __builtin_amdgcn_sched_barrier(0);
            pv_mfma(n, va[n % 3], pt, resid_c);
            __builtin_amdgcn_sched_barrier(0);
          }
          row_sum_mfma(pt, resid_c);
        }
        wait_vmcnt<0>();   // the zero fills past the end must land before the LDS is reused
      }
    } else {
      // Two-slot loop (one or two waves): tile i+1 streams into the other
      // slot while tile i is computed; its DMA instructions go out right
      // after the first QK product (a wave can keep at most 63
      // vector-memory instructions in flight, so a one-wave workgroup holds
      // one tile in flight at a time).  Past the end the slot gets a zero
      // fill, which keeps the wait a constant.
      static_assert(NS == 2, "two-slot loop");
      // The DMA source of the next tile is built at the end of the previous
      // iteration from a page read early in it, off the iteration's start.
      DmaSrc src = dma_prepare(1);
      int pg_nx = 0;
      // A wave whose rows are all past the block's end (the second wave of a
      // two-wave block over at most 32 rows) only moves its share of each
      // tile: its products would be discarded, and they cost power.
      // (A separate loop: a branch inside the computing loop makes the
      // compiler spill the accumulators around it.)
      const bool wave_busy = __builtin_amdgcn_ballot_w64(row_ok) != 0;
      if (RG > 1 && !wave_busy) {
        for (int i = 0; i < n_tiles; i++) {
          wait_vmcnt<0>();
          lds_barrier();   // the same barriers as the computing waves
#pragma unroll
          for (int j = 0; j < NI; j++) dma_issue(src, (i + 1) % NS, j);
          pg_nx = dma_page(i + 2);
          src = dma_prepare_pg(i + 2, pg_nx);
        }
      } else
      for (int i = 0; i < n_tiles; i++) {
        wait_vmcnt<0>();
        if (RG > 1) lds_barrier();   // tile i complete; every wave is done with tile i-1's slot
        const LDS_AS uint8_t* tile = lds + (i % NS) * kTileBytes;
        f32x16_t sacc[K::kTokBlocks];
        {
          opnd_t qa[3];
          qa[0] = ld_qk(tile, 0);
          qa[1] = ld_qk(tile, 1);
#pragma unroll
          for (int n = 0; n < NQK; n++) {
            if (n + 2 < NQK) qa[(n + 2) % 3] = ld_qk(tile, n + 2);
            __builtin_amdgcn_sched_barrier(0);
            qk_mfma(sacc, n, qa[n % 3]);
            // All of the next tile's DMA instructions follow the first
            // product, so its data has the whole tile's compute to arrive
            // (R1-shaped batch: 130.6 -> 124.1 us per call against spreading
            // them over the QK products, alternating on one GPU).
            if (n == 0) {
#pragma unroll
              for (int j = 0; j < NI; j++) dma_issue(src, (i + 1) % NS, j);
            }
            if (n == 1) pg_nx = dma_page(i + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
          drain_scores(sacc);
        }
        PTile pt;
        softmax_all(sacc, i, jumped, pt, resid_c);
        opnd_t va[3];
        va[0] = ld_pv(tile, 0);
        va[1] = ld_pv(tile, 1);
#pragma unroll
        for (int n = 0; n < NPV; n++) {
          if (n + 2 < NPV) va[(n + 2) % 3] = ld_pv(tile, n + 2);
          __builtin_amdgcn_sched_barrier(0);
          pv_mfma(n, va[n % 3], pt, resid_c);
          __builtin_amdgcn_sched_barrier(0);
        }
        row_sum_mfma(pt, resid_c);
        src = dma_prepare_pg(i + 2, pg_nx);
      }
      wait_vmcnt<0>();   // the zero fill past the end must land before the LDS is reused
    }
  };

  // ---- one tile of the fix pass: its DMA into ring slot 0, QK, the
  // softmax weights against the unchanged m_ref, then only the products of
  // the residual weights (PV and the row sum).
  auto fix_tile = [&](int t) __attribute__((always_inline)) {
    if constexpr (kFixTiles) {
      issue_tile(t, 0);
      wait_vmcnt<0>();
      lds_barrier();
      f32x16_t sacc[K::kTokBlocks];
      {
        opnd_t qa[3];
        qa[0] = ld_qk(lds, 0);
        qa[1] = ld_qk(lds, 1);
#pragma unroll
        for (int n = 0; n < NQK; n++) {
          if (n + 2 < NQK) qa[(n + 2) % 3] = ld_qk(lds, n + 2);
          __builtin_amdgcn_sched_barrier(0);
          qk_mfma(sacc, n, qa[n % 3]);
          __builtin_amdgcn_sched_barrier(0);
        }
        drain_scores(sacc);
      }
      PTile pt;
      SmState st;
      bool no_jump = false;   // pass 0 already judged these scores
#pragma unroll
      for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
        for (int k = 0; k < NSTAGE_BLOCK + 1; k++)
          sm_block_stage(k, true, sacc, t, tb, no_jump, st, pt, std::true_type{});
      const int sc = h == 0 ? st.sc[0] : st.sc[1];
      pt.scl = sc > 4 ? sc - 4 : 0;
      const i32x8_t ones8 = {kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4,
                             kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4, kE4m3OnesX4};
      mfma_f8_acc(lsum, ones8, pt.pbl, e8m0_one, pt.scl);
      if constexpr (FS) {
        // Publish this row block's residual tile; every wave then applies
        // all four to its feature quarter.
        LDS_AS i32x4_t* dst = (LDS_AS i32x4_t*)(pbuf + wave * 2048 + lane * 16);
        dst[0] = i32x4_t{pt.pbl[0], pt.pbl[1], pt.pbl[2], pt.pbl[3]};
        dst[64] = i32x4_t{pt.pbl[4], pt.pbl[5], pt.pbl[6], pt.pbl[7]};
        scbuf[wave * 64 + lane] = pt.scl;
        wait_lgkm0();
        lds_barrier();
        i32x8_t vt[4];
#pragma unroll
        for (int f = 0; f < 4; f++) vt[f] = fs_ld_v(lds, f);
#pragma unroll
        for (int r = 0; r < 4; r++) {
          i32x8_t pb = pt.pbl;
          int scq = pt.scl;
          if (r > 0) fs_read_p((wave + r) & 3, pb, scq);
#pragma unroll
          for (int f = 0; f < 4; f++) fs_pv_mfma(r, f, vt[f], pb, scq);
        }
      } else {
#pragma unroll
        for (int n = 0; n < NPV; n++)
          oacc[n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ld_pv(lds, n), pt.pbl, oacc[n], 0, 0, 0, 127,
                                                                    0, pt.scl);
      }
      mfma_drain(lsum);
      lds_barrier();   // every wave is done with slot 0 and the P buffer
    }
  };

  // ---- the passes.  Pass 0 uses the kernel's own step.  A second pass
  // reruns the unit when a row's weights need more than pass 0 gave them:
  //  * a row's block maximum rose more than 2^64 above its reference (the
  //    O accumulator's headroom): the rerun takes the exact row maximum;
  //  * fp8 without the residual product: the rounding of each weight to
  //    e4m3 (up to 2^-4 relative) stays far below the output tolerance
  //    while the weight is spread over many tokens, but not when a few
  //    tokens carry most of it.  Pass 0 bounds sum_j w_j^2 (w the
  //    normalized weights) from each block's sums; above 2^-7 the unit is
  //    rerun with the residual product (each weight to about 2^-8), in the
  //    plain four-wave step when pass 0 was the feature split.
  // Rows of N(0,1) data in units of more than 16384 tokens stay near 2^-9.
  constexpr bool kRedoResid = FP8 && !RESID;
  bool fs_layout = FS;             // O is held in the feature-split layout
  bool redone = false;             // pass 1 ran
  for (int pass = 0; pass < 2; pass++) {
#pragma unroll
    for (int fb = 0; fb < 16; fb++) oacc[fb] = f32x16_t{};
    lsum = f32x16_t{};
    l_f = 0.f;
    l_r = 0.f;
    l_q2 = 0.f;
    if (pass == 1) {
      const float mrow = max_across_halves(m_seen);
      m_ref = mrow == -INFINITY ? kNegBig : (FP8 ? ceilf(mrow) : mrow);
    }
    bool jumped = false;
    if (pass > 0) issue_first_tiles();
    if constexpr (kRedoResid) {
      if (pass == 0) {
        tile_loop(jumped, std::integral_constant<bool, FS>{}, std::false_type{});
      } else {
        fs_layout = false;
        redone = true;
        tile_loop(jumped, std::false_type{}, std::true_type{});
      }
    } else {
      tile_loop(jumped, std::integral_constant<bool, FS>{}, std::integral_constant<bool, RESID>{});
    }
    if constexpr (FP8) mfma_drain(lsum);

    // ---- second pass needed?  (workgroup-uniform: all waves share the DMA)
    if (pass == 1) break;
    bool need = jumped;
    bool fix = false;
    if constexpr (kRedoResid) {
      // sum_j w_j^2 <= q2 / l^2 with both in the units of sm_finish.  Most
      // rows above the bound owe it to one heavy tile: adding the residual
      // product of that tile alone (the fix pass below) is enough when the
      // rest of the row stays under the bound; otherwise the unit reruns.
      const float lt = sum_across_halves(l_f) * 0x1p-32f;
      const float q2 = sum_across_halves(l_q2);
      const float q2_top = sum_across_halves(top_q2);
      const float lim = kFp8RedoSumSq * lt * lt;
      need |= q2 - q2_top > lim;
      fix = q2 > lim;
    }
    const bool wave_jump = __builtin_amdgcn_ballot_w64(need && row_ok) != 0;
    if (threadIdx.x == 0) *redo_flag = 0;
    if constexpr (kFixTiles) {
      if (threadIdx.x < kFixWords) fix_map[threadIdx.x] = 0u;
    }
    __syncthreads();
    if (wave_jump && lane == 0) *redo_flag = 1;
    if constexpr (kFixTiles) {
      if (fix && row_ok && h == 0) __hip_atomic_fetch_or(&fix_map[top_tile >> 5], 1u << (top_tile & 31),
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    const int redo = *redo_flag;
    __syncthreads();
    if (!redo) break;
  }

  // ---- fix pass (fp8 without the residual product): the residual product
  // of each marked tile, added to what pass 0 accumulated.  Pass 0 reached
  // every mark with the same reference m_ref, so recomputing the tile gives
  // the same scores and the same e4m3 weights, and the residual completes
  // them to about 2^-8 exactly as a residual-product pass would.  Rare:
  // N(0,1) data marks about one row in 400, one tile each.
  if constexpr (kFixTiles) {
    if (!redone && n_tiles > 0) {
      for (int wd = 0; wd < (n_tiles + 31) / 32; wd++) {
        uint32_t bits = __builtin_amdgcn_readfirstlane(fix_map[wd]);
        while (bits != 0u) {
          const int t = wd * 32 + __builtin_ctz(bits);
          bits &= bits - 1u;
          fix_tile(t);
        }
      }
    }
  }

  // ---- epilogue: normalize, write final output or the split partial
  const float off = FP8 ? 8.f : 0.f;
  l_f = sum_across_halves(l_f);
  // fp8: every element of a lane's lsum holds its row's sum of rounded weights.
  const float l_q = FP8 ? lsum[0] : sum_across_halves(l_r);
  const bool empty = !(l_f > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_q;
  const float lse_v = empty ? -INFINITY : (m_ref - off + __builtin_amdgcn_logf(l_f)) * kLn2;

  // This lane's 16 values of output feature block fb of query row qr (the
  // C layout: register 4a+c holds feature 32 fb + 8a + 4h + c).
  // A float of a split partial.  A single-launch call writes its partials
  // with device-scope stores (through to the device's coherence point), so
  // that the units merging them on other XCDs read them without any cache
  // write-back or invalidation.
  auto put = [&](float* a, float v) __attribute__((always_inline)) {
    if (p.fused) __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *a = v;
  };
  auto store_block = [&](int64_t qr, int fb, const f32x16_t& acc, float iv) {
    if (p.S == 1) {
      if (p.out_f32) {
        float* o = (float*)p.out + qr * 512;
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
          const float4 w = {acc[4 * a4] * iv, acc[4 * a4 + 1] * iv, acc[4 * a4 + 2] * iv, acc[4 * a4 + 3] * iv};
          *(float4*)(o + 32 * fb + 8 * a4 + 4 * h) = w;
        }
      } else {
        __bf16* o = (__bf16*)p.out + qr * 512;
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
          const bf16x4_t w = {(__bf16)(acc[4 * a4] * iv), (__bf16)(acc[4 * a4 + 1] * iv),
                              (__bf16)(acc[4 * a4 + 2] * iv), (__bf16)(acc[4 * a4 + 3] * iv)};
          *(bf16x4_t*)(o + 32 * fb + 8 * a4 + 4 * h) = w;
        }
      }
    } else {
      float* w = p.ws + (qr * p.S + split) * (int64_t)kPartialWidth + 32 * fb + 4 * h;
#pragma unroll
      for (int a4 = 0; a4 < 4; a4++)
#pragma unroll
        for (int c = 0; c < 4; c++) put(&w[8 * a4 + c], acc[4 * a4 + c] * iv);
    }
  };
  // Split partials of four-wave blocks leave through LDS.  In the
  // accumulator layout one store instruction would touch 32 rows (two
  // 16-byte pieces each); staged as [32 rows][128 features] in the (now
  // idle) tile ring, each wave then writes every row's 128 features as two
  // fully coalesced 256-byte stores.  `acc` holds one lane's four feature
  // blocks [fbase, fbase + 128) of row qr0 + l32, and `iv` is that row's
  // normalizer; rows whose bit is clear in `ok` are not written.
  constexpr int kStgStride = 132;   // floats per staged row (128 + 4 against bank conflicts)
  static_assert(RG * 32 * kStgStride * 4 <= NS * kTileBytes, "staging fits the tile ring");
  LDS_AS float* stg = (LDS_AS float*)lds + wave * 32 * kStgStride;
  auto stage_partial = [&](const f32x16_t* acc, int64_t qr0, int fbase, float iv, uint32_t ok) {
#pragma unroll
    for (int f = 0; f < 4; f++)
#pragma unroll
      for (int a4 = 0; a4 < 4; a4++) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t v = {acc[f][4 * a4] * iv, acc[f][4 * a4 + 1] * iv, acc[f][4 * a4 + 2] * iv,
                           acc[f][4 * a4 + 3] * iv};
        *(LDS_AS f32x4_t*)(stg + l32 * kStgStride + 32 * f + 8 * a4 + 4 * h) = v;
      }
    if (!FS && !p.fused) {
      // Two rows per store instruction, 16 bytes per lane: lane l writes
      // features 4 (l % 32) .. + 3 of row 2 k + l / 32 of each group of
      // eight.  A partial row starts 4-byte aligned (513 floats), which the
      // 16-byte global stores accept; the LDS reads are 16-byte aligned.
      typedef float f32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      const int hr = lane >> 5, c4 = 4 * (lane & 31);
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += 8) {
        f32x4_t v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = *(const LDS_AS f32x4_t*)(stg + (r0 + 2 * k + hr) * kStgStride + c4);
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const int r = r0 + 2 * k + hr;
          if ((ok >> r) & 1u) {
            f32x4a4_t* w = (f32x4a4_t*)(p.ws + ((qr0 + r) * p.S + split) * (int64_t)kPartialWidth + fbase + c4);
            *w = f32x4a4_t{v[k][0], v[k][1], v[k][2], v[k][3]};
          }
        }
      }
    } else {
      // Eight rows at a time: their sixteen LDS reads go out together, so the
      // read latency is paid once per group rather than once per row.
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += 8) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 8; k++) {
          v[2 * k] = stg[(r0 + k) * kStgStride + lane];
          v[2 * k + 1] = stg[(r0 + k) * kStgStride + 64 + lane];
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if ((ok >> (r0 + k)) & 1u) {
            float* w = p.ws + ((qr0 + r0 + k) * p.S + split) * (int64_t)kPartialWidth + fbase;
            put(&w[lane], v[2 * k]);
            put(&w[64 + lane], v[2 * k + 1]);
          }
        }
      }
    }
  };
  auto store_lse = [&]() {
    if (h != 0 || !row_ok) return;
    if (p.S == 1) {
      if (p.lse) p.lse[qrow] = lse_v;
    } else {
      float* wl = p.ws + qrow * p.S * (int64_t)kPartialWidth + 512;
      put(&wl[split * (int64_t)kPartialWidth], lse_v);
      // A sequence cut into fewer pieces than it has slots: its last piece
      // marks the remaining slots empty (lse -inf; their outputs are left
      // unwritten and the merge does not read them).
      if (split == n_split - 1)
        for (int s = n_split; s < p.S; s++) put(&wl[s * (int64_t)kPartialWidth], -INFINITY);
    }
  };

  if (FS && fs_layout) {
    // Row block rq's normalizer lives in wave rq; pass them through LDS
    // (the P tiles are dead by now).
    LDS_AS float* invbuf = (LDS_AS float*)pbuf;
    if (h == 0) invbuf[wave * 32 + l32] = inv;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int rq = (wave + r) & 3;
      const int rrow0 = rb * (32 * RG) + rq * 32;          // the row block's first row
      const int rrow = rrow0 + l32;
      const float iv = invbuf[rq * 32 + l32];
      if (p.S > 1) {
        const int n_ok = min(32, p.R - rrow0);
        if (n_ok > 0)
          stage_partial(&oacc[4 * r], (int64_t)b * p.R + rrow0, 128 * wave, iv,
                        n_ok >= 32 ? 0xffffffffu : (1u << n_ok) - 1u);
        continue;
      }
      if (rrow >= p.R) continue;
      const int64_t qr = (int64_t)b * p.R + rrow;
#pragma unroll
      for (int f = 0; f < 4; f++) store_block(qr, 4 * wave + f, oacc[4 * r + f], iv);
    }
    store_lse();
  } else {
    // Staging pays off for four-wave blocks (128 rows of partials each);
    // narrower blocks write few rows, and there the extra LDS round trips
    // cost more latency than the coalescing saves.
    if (RG == 4 && p.S > 1) {
      // Every wave is done with the tile ring before any stages into it.
      __syncthreads();
      const uint32_t ok = (uint32_t)__builtin_amdgcn_ballot_w64(row_ok);   // lanes 0-31: rows l32
      const int64_t qr0 = qrow - l32;
#pragma unroll
      for (int c = 0; c < 4; c++) stage_partial(&oacc[4 * c], qr0, 128 * c, inv, ok);
      store_lse();
    } else if (row_ok) {
#pragma unroll
      for (int fb = 0; fb < 16; fb++) store_block(qrow, fb, oacc[fb], inv);
      store_lse();
    }
  }

  // ---- single launch: the units of this (sequence, row block) wait for
  // each other, then each merges its share of the block's rows.  Every unit
  // of the launch is resident at once (the host plans this form only then),
  // so the wait ends; it is bounded all the same.
  if (p.fused && p.S > 1) {
    unsigned long long* word = p.sync + 2 * ((int64_t)b * p.n_rb + rb);
    const unsigned long long e = p.epoch << 16;
    wait_vmcnt<0>();            // this wave's partial stores have reached the device
    __syncthreads();
    if (threadIdx.x == 0) {
      sync_arrive(word, e);
      // Device-scope reads of the word; the partials are read the same way,
      // so no fence (an L2 write-back or invalidation) is needed anywhere.
      for (int it = 0; it < (1 << 22); it++) {
        if (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (e | (unsigned)n_split)) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    // Rows of the block: dense rb covers rows [32 RG rb, ...) of the
    // sequence; sparse rb is (draft token, head block).
    int row0, nrows;
    if (SPARSE) {
      const int hb = rb % p.n_hb;
      row0 = (rb / p.n_hb) * p.H + hb * (32 * RG);
      nrows = min(32 * RG, p.H - hb * (32 * RG));
    } else {
      row0 = rb * (32 * RG);
      nrows = min(32 * RG, p.R - row0);
    }
    const int r_beg = split * nrows / n_split, r_end = (split + 1) * nrows / n_split;
    for (int r = r_beg + wave; r < r_end; r += 2 * RG) {
      const int64_t rows2[2] = {(int64_t)b * p.R + row0 + r, (int64_t)b * p.R + row0 + r + RG};
      const bool ok2[2] = {true, r + RG < r_end};
      merge_rows<2>(p.ws, rows2, ok2, p.S, p.out, p.out_f32, p.lse);
    }
    __syncthreads();
    if (threadIdx.x == 0 && sync_arrive(word + 1, e) == n_split) {
      // every unit of the group is past its wait: both words back to zero
      __hip_atomic_store(word, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word + 1, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// LSE merge: one wave per (sequence, row); lane i owns outputs 8i .. 8i+7.
__global__ void __launch_bounds__(256) mla_merge_kernel(const MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.n_rows) return;
  const float* base = p.ws + r * p.S * (int64_t)kPartialWidth;
  // Maximum partial LSE across splits (lanes hold splits s, s+64, ...).
  float mx = -INFINITY;
  for (int s = lane; s < p.S; s += 64) mx = fmaxf(mx, base[(int64_t)s * kPartialWidth + 512]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float lse_out = -INFINITY;
  if (mx != -INFINITY) {
    float z = 0.f;
    for (int s0 = 0; s0 < p.S; s0 += 64) {
      const int s = s0 + lane;
      const float w = s < p.S ? __expf(base[(int64_t)s * kPartialWidth + 512] - mx) : 0.f;
      float zs = w;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) zs += __shfl_xor(zs, d);
      z += zs;
      // Eight splits at a time: all of a group's loads are issued before any
      // is used, so their latencies overlap.  A split of weight zero (an
      // empty one, lse -inf) is not read: its outputs may be undefined.
      // Rows of 513 floats are only 4-byte aligned; the 16-byte global loads
      // accept that.
      const int ns = min(64, p.S - s0);
      for (int k0 = 0; k0 < ns; k0 += 8) {
        float wk[8];
#pragma unroll
        for (int k = 0; k < 8; k++) wk[k] = __shfl(w, (k0 + k) & 63);   // w is 0 past ns
        float v[8][8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if (wk[k] != 0.f) {
            typedef float f32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
            const f32x4a4_t* src = (const f32x4a4_t*)(base + (int64_t)(s0 + k0 + k) * kPartialWidth + 8 * lane);
            const f32x4a4_t lo = src[0], hi = src[1];
#pragma unroll
            for (int c = 0; c < 4; c++) {
              v[k][c] = lo[c];
              v[k][4 + c] = hi[c];
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if (wk[k] != 0.f) {
#pragma unroll
            for (int c = 0; c < 8; c++) acc[c] += wk[k] * v[k][c];
          }
        }
      }
    }
    const float inv = 1.f / z;
#pragma unroll
    for (int c = 0; c < 8; c++) acc[c] *= inv;
    lse_out = mx + __logf(z);
  }
  if (p.out_f32) {
    float* o = (float*)p.out + r * 512 + 8 * lane;
    *(float4*)o = float4{acc[0], acc[1], acc[2], acc[3]};
    *(float4*)(o + 4) = float4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));
    bf16x8s_t v;
#pragma unroll
    for (int c = 0; c < 8; c++) v[c] = (__bf16)acc[c];
    *(bf16x8s_t*)((__bf16*)p.out + r * 512 + 8 * lane) = v;
  }
  if (lane == 0 && p.lse) p.lse[r] = lse_out;
}

// ---------------------------------------------------------------------------
// Launchers.
template <bool FP8, bool SPARSE, int RG, int NS, bool RESID = false, bool FS = false>
static hipError_t launch_partial(const PartialParams& p, int grid, hipStream_t stream) {
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)&mla_partial_kernel<FP8, SPARSE, RG, NS, RESID, FS>, dim3(grid), dim3(64 * RG),
                         args, 0, stream);
}

hipError_t launch_partial_kernel(const PartialParams& p, bool fp8, bool sparse, int rg, bool resid, int grid,
                                 hipStream_t stream) {
  if (fp8 && !sparse) {
    if (resid) {
      switch (rg) {
        case 1: return launch_partial<true, false, 1, 2, true>(p, grid, stream);
        case 2: return launch_partial<true, false, 2, 2, true>(p, grid, stream);
        case 4: return launch_partial<true, false, 4, 4, true>(p, grid, stream);
      }
    } else {
      switch (rg) {
        case 1: return launch_partial<true, false, 1, 2>(p, grid, stream);
        case 2: return launch_partial<true, false, 2, 2>(p, grid, stream);
        case 4: return launch_partial<true, false, 4, 4, false, true>(p, grid, stream);
      }
    }
  } else if (!fp8 && !sparse) {
    switch (rg) {
      case 1: return launch_partial<false, false, 1, 2>(p, grid, stream);
      case 2: return launch_partial<false, false, 2, 2>(p, grid, stream);
      case 4: return launch_partial<false, false, 4, 4>(p, grid, stream);
    }
  } else if (!fp8 && sparse) {
    switch (rg) {
      case 1: return launch_partial<false, true, 1, 2>(p, grid, stream);
      case 2: return launch_partial<false, true, 2, 2>(p, grid, stream);
      case 4: return launch_partial<false, true, 4, 4>(p, grid, stream);
    }
  } else if (fp8 && sparse && resid) {
    // A sparse unit holds at most 1024 indices, always short enough for the
    // residual product.
    switch (rg) {
      case 1: return launch_partial<true, true, 1, 2, true>(p, grid, stream);
      case 2: return launch_partial<true, true, 2, 2, true>(p, grid, stream);
      case 4: return launch_partial<true, true, 4, 4, true>(p, grid, stream);
    }
  }
  return hipErrorInvalidValue;
}

// Workgroups of a partial-kernel variant that one compute unit holds at
// once, as the runtime reports it for the current device (cached per
// device and variant); 0 if it cannot be asked.
template <bool FP8, bool SPARSE, int RG, int NS, bool RESID = false, bool FS = false>
static int occupancy_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mla_partial_kernel<FP8, SPARSE, RG, NS, RESID, FS>, 64 * RG,
                                                   0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

int partial_kernel_occupancy(bool fp8, bool sparse, int rg, bool resid) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cached[kMaxDevices][2][2][3][2] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  const int gi = rg == 4 ? 2 : rg - 1;
  std::lock_guard<std::mutex> lock(mu);
  int& c = cached[dev][fp8][sparse][gi][resid];
  if (c == 0) {
    int n = 0;
    if (fp8 && !sparse) {
      if (resid) n = rg == 1 ? occupancy_of<true, false, 1, 2, true>() : rg == 2 ? occupancy_of<true, false, 2, 2, true>()
                                                                         : occupancy_of<true, false, 4, 4, true>();
      else n = rg == 1 ? occupancy_of<true, false, 1, 2>() : rg == 2 ? occupancy_of<true, false, 2, 2>()
                                                           : occupancy_of<true, false, 4, 4, false, true>();
    } else if (!fp8 && !sparse) {
      n = rg == 1 ? occupancy_of<false, false, 1, 2>() : rg == 2 ? occupancy_of<false, false, 2, 2>()
                                                       : occupancy_of<false, false, 4, 4>();
    } else if (!fp8 && sparse) {
      n = rg == 1 ? occupancy_of<false, true, 1, 2>() : rg == 2 ? occupancy_of<false, true, 2, 2>()
                                                      : occupancy_of<false, true, 4, 4>();
    } else {
      n = rg == 1 ? occupancy_of<true, true, 1, 2, true>() : rg == 2 ? occupancy_of<true, true, 2, 2, true>()
                                                           : occupancy_of<true, true, 4, 4, true>();
    }
    c = n > 0 ? n : -1;
  }
  return c > 0 ? c : 0;
}

hipError_t launch_merge_kernel(const MergeParams& p, hipStream_t stream) {
  const int64_t blocks = (p.n_rows + 3) / 4;
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)&mla_merge_kernel, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

// ---------------------------------------------------------------------------
// Static split workspace of the allocation-free entry point.  One copy per
// GPU, at that GPU's own address, held until the process ends.  Host code
// must not use the array's name as a device address: it is a host-side
// stand-in.  The device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
