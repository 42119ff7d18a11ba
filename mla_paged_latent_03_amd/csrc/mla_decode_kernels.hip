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
constexpr float kNegBig = -1.0e30f;  // running-max sentinel: finite, below any logit

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

template <int NI, int MAXR>
__device__ inline void wait_tiles_after(int remaining) {
  // Wait until at most `remaining` tiles (NI loads each) are still in flight.
  if constexpr (MAXR >= 2) {
    if (remaining >= 2) { wait_vmcnt<2 * NI>(); return; }
  }
  if constexpr (MAXR >= 1) {
    if (remaining >= 1) { wait_vmcnt<NI>(); return; }
  }
  wait_vmcnt<0>();
}

// Combine the two halves of a wave (lanes l and l ^ 32 hold the same row).
// (v_permlane32_swap of a value with itself gets folded to a no-op by the
// compiler, so the exchange goes through ds_bpermute.)
__device__ inline float max_across_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

__device__ inline float sum_across_halves(float x) { return x + __shfl_xor(x, 32); }

// 16-byte global -> LDS DMA: lane i writes LDS bytes [m0 + 16 i, m0 + 16 i + 16).
// Issued from inline asm so the compiler does not treat it as an LDS store
// (it would otherwise drain every in-flight DMA before each LDS read it
// cannot prove disjoint); completion is tracked explicitly with vmcnt.
__device__ inline void dma16(const void* gsrc, uint32_t lds_byte_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(lds_byte_addr) : "memory");
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
//            a few tokens can dominate a row
template <bool FP8, bool SPARSE, int RG, int NS, bool RESID>
__global__ void __launch_bounds__(64 * RG) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_partial_kernel(const PartialParams p) {
  using K = Kv<FP8>;
  constexpr int NI = kInstrPerTile / RG;          // DMA instructions per wave per tile
  constexpr int NPRE = NI <= 18 ? NI : K::kPeriodInstr;
  static_assert(NI % NPRE == 0, "DMA offset period");
  constexpr int kSparseCap = SPARSE ? kSparseChunkMax : 0;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * kTileBytes + kSparseCap * 4 + 16];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;       // which half of the wave
  const int l32 = lane & 31;     // MFMA column = query row within the wave

  // ---- work unit: XCD-aware renumbering of the linear workgroup id so that
  // consecutive units (row blocks of one (sequence, split)) share an XCD.
  const int nwg = gridDim.x;     // multiple of 8
  const int u = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (u >= p.n_units) return;
  const int rb = u % p.n_rb;
  const int bs = u / p.n_rb;
  const int split = bs % p.S;
  const int b = bs / p.S;

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
  int n_tiles, tok_begin = 0, idx_begin = 0, idx_count = 0;
  if (SPARSE) {
    idx_begin = split * p.chunk;
    idx_count = min(p.chunk, p.K - idx_begin);
    if (idx_count < 0) idx_count = 0;
    n_tiles = (idx_count + K::kTileTok - 1) / K::kTileTok;
  } else {
    const int n_pages = (L + 63) >> 6;
    const int p0 = split * p.chunk;
    const int p1 = min(p0 + p.chunk, n_pages);
    tok_begin = p0 * 64;
    const int tok_end = p1 > p0 ? min(p1 * 64, L) : tok_begin;
    n_tiles = (tok_end - tok_begin + K::kTileTok - 1) / K::kTileTok;
    if (n_tiles < 0) n_tiles = 0;
  }
  // Highest position any row of this sequence may see (dense causal limit of
  // the last draft token); tiles fully below the first row's limit skip masks.
  const int n_vis = L - p.T + t_row + 1;  // dense: visible tokens of this row

  // ---- sparse: physical row table for this unit's index range, in LDS
  LDS_AS int* sp_rows = (LDS_AS int*)(lds + NS * kTileBytes);
  if (SPARSE) {
    const int32_t* idx = p.topk + ((int64_t)b * p.T + (rb / p.n_hb)) * p.K + idx_begin;
    const int n_ent = n_tiles * K::kTileTok;
    for (int e = threadIdx.x; e < n_ent; e += 64 * RG) {
      int phys = -1;
      if (e < idx_count) {
        const int j = idx[e];
        if (j >= 0 && j < L) {
          const int pg = p.block_table[(int64_t)b * p.MB + (j >> 6)];
          if (pg >= 0 && pg < p.NB) phys = pg * 64 + (j & 63);
        }
      }
      sp_rows[e] = phys;
    }
    __syncthreads();
  }

  // ---- query operand in registers (B side: lane holds row l32, a K slice)
  // bf16: step k covers features 16k .. 16k+15; lane half h holds 8 of them.
  // fp8 : step k covers features 64k .. 64k+63; lane half h holds 32 of them.
  constexpr int QREGS = FP8 ? 8 * K::kQkSteps : 4 * K::kQkSteps;
  int qreg[QREGS];
  {
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
  }

  // ---- DMA source offsets.  Wave w fills tile units [w*NI*64, (w+1)*NI*64):
  // instruction j writes LDS units pos = (w*NI + j)*64 + lane, i.e. token
  // t = pos / kUnits, swizzled unit c' = pos % kUnits, and so fetches global
  // unit (t, c' ^ swz(t)).
  int dma_off[NPRE];   // byte offset inside the tile's global rows
#pragma unroll
  for (int j = 0; j < NPRE; j++) {
    const int pos = (wave * NI + j) * 64 + lane;
    const int t = pos / K::kUnits;
    const int c = (pos % K::kUnits) ^ K::swz(t);
    dma_off[j] = t * K::kRowBytes + 16 * c;
  }
  // Period: NPRE instructions cover exactly 16 tokens when NI > 18.
  constexpr int kPeriodBytes = 16 * K::kRowBytes;

  auto issue_tile = [&](int i, int slot) {
    const uint32_t dst = (uint32_t)(uintptr_t)(lds + slot * kTileBytes + wave * NI * 1024);
    if (SPARSE) {
      LDS_AS const int* rows_tab = sp_rows + i * K::kTileTok;
#pragma unroll
      for (int j = 0; j < NI; j++) {
        const int off = dma_off[j % NPRE] + (j / NPRE) * kPeriodBytes;
        const int t = off / K::kRowBytes;
        const int cb = off - t * K::kRowBytes;
        const int phys = rows_tab[t];
        const uint8_t* src = phys >= 0 ? p.kv + (int64_t)phys * K::kRowBytes + cb : g_zero_row + cb;
        dma16(src, dst + j * 1024);
      }
    } else {
      const int tok0 = tok_begin + i * K::kTileTok;     // first token of the tile
      const int pg = ((const CONST_AS int32_t*)p.block_table)[(int64_t)b * p.MB + (tok0 >> 6)];
      const bool page_ok = pg >= 0 && pg < p.NB;
      const uint8_t* base = p.kv + ((int64_t)(page_ok ? pg : 0) * 64 + (tok0 & 63)) * K::kRowBytes;
      const int n_valid = page_ok ? min(K::kTileTok, L - tok0) : 0;
      if (n_valid == K::kTileTok) {
#pragma unroll
        for (int j = 0; j < NI; j++) {
          const int off = dma_off[j % NPRE] + (j / NPRE) * kPeriodBytes;
          dma16(base + off, dst + j * 1024);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NI; j++) {
          const int off = dma_off[j % NPRE] + (j / NPRE) * kPeriodBytes;
          const int t = off / K::kRowBytes;
          const uint8_t* src = t < n_valid ? base + off : g_zero_row + (off - t * K::kRowBytes);
          dma16(src, dst + j * 1024);
        }
      }
    }
  };

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
  constexpr int NRD = FP8 ? 4 : 2;
  int v_off[NRD][2];
  {
    const int i = lane & 15, g = lane >> 4, e = g & 1;
    if (FP8) {
      const int sp = i >> 1, q = i & 1, sig = sp >> 2;
#pragma unroll
      for (int r = 0; r < NRD; r++) {
        const int t = 32 * (r >> 1) + 16 * (r & 1) + 8 * sig + 4 * h + (sp & 3);
        const int base = t * K::kRowBytes + 16 * (e ^ h) + 8 * q;
        v_off[r][0] = base + 32 * sig;   // even feature block: fb ^ sig = fb + sig
        v_off[r][1] = base - 32 * sig;   // odd feature block : fb ^ sig = fb - sig
      }
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

  // ---- accumulators and softmax state (per lane: row l32, its half of tokens)
  //
  // Each row accumulates O and l relative to a fixed reference m_ref (log2
  // domain), set at the first tile where the row sees any token; later
  // tiles add their contributions scaled by 2^(tile max - m_ref).  So the
  // accumulators are never rescaled inside the loop.  Only if a row's tile
  // maximum ever exceeds m_ref by more than 2^64 (fp32 headroom for O) is the
  // whole unit run a second time with m_ref = that row's true maximum.
  f32x16_t oacc[16];
  float m_ref = kNegBig;
  float m_seen = -INFINITY;        // running row maximum, for the second pass
  float l_q = 0.f;                 // row sum of the rounded weights (normalizes out)
  float l_f = 0.f;                 // row sum of the unrounded weights (gives lse)
  const float c_qk = p.qk_scale;   // softmax_scale * log2(e) [* q_scale * kv_scale]
  LDS_AS int* redo_flag = (LDS_AS int*)(lds + NS * kTileBytes + kSparseCap * 4);

  for (int pass = 0; pass < 2; pass++) {
#pragma unroll
    for (int fb = 0; fb < 16; fb++) oacc[fb] = f32x16_t{};
    l_q = 0.f;
    l_f = 0.f;
    if (pass == 1) m_ref = m_seen == -INFINITY ? kNegBig : (FP8 ? ceilf(m_seen) : m_seen);
    bool jumped = false;

    // ---- prologue
#pragma unroll
    for (int i = 0; i < NS - 1; i++)
      if (i < n_tiles) issue_tile(i, i);

    for (int i = 0; i < n_tiles; i++) {
      wait_tiles_after<NI, NS - 2>(min(NS - 2, n_tiles - 1 - i));
      if (RG > 1) lds_barrier();
      if (i + NS - 1 < n_tiles) issue_tile(i + NS - 1, (i + NS - 1) % NS);
      const LDS_AS uint8_t* tile = lds + (i % NS) * kTileBytes;

      // ---- S^T = K Q^T
      f32x16_t sacc[K::kTokBlocks];
#pragma unroll
      for (int tb = 0; tb < K::kTokBlocks; tb++) {
        sacc[tb] = f32x16_t{};
        const LDS_AS uint8_t* tb_base = tile + tb * 32 * K::kRowBytes;
#pragma unroll
        for (int k = 0; k < K::kQkSteps; k++) {
          if (FP8) {
            const i32x4_t lo = *(const LDS_AS i32x4_t*)(tb_base + a_off[0] + 64 * k);
            const i32x4_t hi = *(const LDS_AS i32x4_t*)(tb_base + a_off[1] + 64 * k);
            const i32x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const i32x8_t bq = {qreg[8 * k], qreg[8 * k + 1], qreg[8 * k + 2], qreg[8 * k + 3],
                                qreg[8 * k + 4], qreg[8 * k + 5], qreg[8 * k + 6], qreg[8 * k + 7]};
            sacc[tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq, sacc[tb], 0, 0, 0, 127, 0, 127);
          } else {
            const i32x4_t a = *(const LDS_AS i32x4_t*)(tb_base + a_off[k & 3] + 128 * (k >> 2));
            const i32x4_t bq = {qreg[4 * k], qreg[4 * k + 1], qreg[4 * k + 2], qreg[4 * k + 3]};
            sacc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                               __builtin_bit_cast(bf16x8_t, bq), sacc[tb], 0, 0, 0);
          }
        }
      }

      // ---- masks.  Register v of token block tb holds token 32*tb + 8*(v/4) + 4*h + v%4.
      if (SPARSE) {
        const int phys = lane < K::kTileTok ? sp_rows[i * K::kTileTok + lane] : 0;
        const uint64_t valid =
            __builtin_amdgcn_ballot_w64(phys >= 0) | (K::kTileTok == 64 ? 0ull : ~0ull << 32);
        if (valid != ~0ull) {
#pragma unroll
          for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
              const int tok = 32 * tb + 8 * (v >> 2) + 4 * h + (v & 3);
              if (!((valid >> tok) & 1)) sacc[tb][v] = -INFINITY;
            }
        }
      } else {
        const int tok0 = tok_begin + i * K::kTileTok;
        if (tok0 + K::kTileTok > L - p.T + 1) {   // some token may lie past a row's causal limit
#pragma unroll
          for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
              const int tok = tok0 + 32 * tb + 8 * (v >> 2) + 4 * h + (v & 3);
              if (tok >= n_vis) sacc[tb][v] = -INFINITY;
            }
        }
      }

      // ---- online softmax (log2 domain)
      float mt = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < K::kTokBlocks; tb++)
#pragma unroll
        for (int v = 0; v < 16; v++) mt = fmaxf(mt, sacc[tb][v]);
      mt = max_across_halves(mt) * c_qk;   // tile row maximum, scaled (-inf if all masked)
      m_seen = fmaxf(m_seen, mt);
      if (FP8) {
        // Integer tile reference keeps every scale an exact power of two.
        const float mi = ceilf(mt);
        if (m_ref == kNegBig && mt != -INFINITY) m_ref = mi;
        jumped |= mi > m_ref + 64.f;
        // P' = 2^(x - mi + 8) in [0, 256] -> e4m3; the PV MFMA multiplies it by
        // 2^(mi - m_ref) through the E8M0 scale of its P operand.
        const float mref = mt == -INFINITY ? m_ref : mi;
        const float shift = 8.f - mref;
        // hi = e4m3(P'), lo = e4m3(16 (P' - hi)): the pair holds P' to ~2^-8.
        float psum_f = 0.f, psum_q = 0.f, psum_lo = 0.f;
        int pk[8], pl[8];
#pragma unroll
        for (int d = 0; d < 8; d++) {
          const int tb = d >> 2, v = 4 * (d & 3);
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v], c_qk, shift));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 1], c_qk, shift));
          const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 2], c_qk, shift));
          const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[tb][v + 3], c_qk, shift));
          psum_f += (e0 + e1) + (e2 + e3);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
          pk[d] = w;
          const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
          psum_q += (h01[0] + h01[1]) + (h23[0] + h23[1]);
          if constexpr (RESID) {
            int wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (e0 - h01[0]), 16.f * (e1 - h01[1]), 0, false);
            wl = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (e2 - h23[0]), 16.f * (e3 - h23[1]), wl, true);
            pl[d] = wl;
            const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8(wl, false);
            const auto l23 = __builtin_amdgcn_cvt_pk_f32_fp8(wl, true);
            psum_lo += (l01[0] + l01[1]) + (l23[0] + l23[1]);
          } else {
            pl[d] = 0;
          }
        }
        psum_q = sum_across_halves(psum_q);
        psum_f = sum_across_halves(psum_f);
        // E8M0 biased exponent of 2^(mref - m_ref); below 2^-122 the tile is dropped.
        const float dexp = fminf(mref - m_ref, 64.f);
        const int sc = dexp < -122.f ? 0 : (int)dexp + 127;
        const float pscale = sc > 0 ? __builtin_amdgcn_ldexpf(1.0f, sc - 127) : 0.f;
        if (RESID) psum_q += sum_across_halves(psum_lo) * 0.0625f;
        l_q += psum_q * pscale;
        l_f += psum_f * pscale;
        const i32x8_t pz = {0, 0, 0, 0, 0, 0, 0, 0};
        const i32x8_t pop = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
        const i32x8_t pb = sc > 0 ? pop : pz;
        const int scl = sc > 4 ? sc - 4 : 0;
        const i32x8_t plo = {pl[0], pl[1], pl[2], pl[3], pl[4], pl[5], pl[6], pl[7]};
        const i32x8_t pbl = sc > 4 ? plo : pz;
        // ---- O^T += V^T P^T  (+ V^T Plo^T 2^-4)
#pragma unroll
        for (int fb = 0; fb < 16; fb++) {
          i32x8_t a;
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const i32x2_t d =
                __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)(tile + v_off[r][fb & 1] + 32 * fb));
            a[2 * r] = d[0];
            a[2 * r + 1] = d[1];
          }
          oacc[fb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[fb], 0, 0, 0, 127, 0, sc);
          if constexpr (RESID)
            oacc[fb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pbl, oacc[fb], 0, 0, 0, 127, 0, scl);
        }
      } else {
        if (m_ref == kNegBig && mt != -INFINITY) m_ref = mt;
        jumped |= mt > m_ref + 64.f;
        const float shift = -m_ref;
        float psum_f = 0.f, psum_q = 0.f;
        // P operand: k-step kk holds the tokens of registers 8*kk .. 8*kk+7.
        bf16x8_t pop[2];
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
          for (int s = 0; s < 8; s++) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sacc[0][8 * kk + s], c_qk, shift));
            const __bf16 eb = (__bf16)e;
            psum_f += e;
            psum_q += (float)eb;      // the rounded weight the PV product uses
            pop[kk][s] = eb;
          }
        l_q += sum_across_halves(psum_q);
        l_f += sum_across_halves(psum_f);
        // ---- O^T += V^T P^T
#pragma unroll
        for (int fb = 0; fb < 16; fb++) {
#pragma unroll
          for (int kk = 0; kk < 2; kk++) {
            const i16x4_t d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS i16x4_t*)(tile + v_off[0][fb & 1] + 64 * fb + 16 * kk * K::kRowBytes));
            const i16x4_t d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS i16x4_t*)(tile + v_off[1][fb & 1] + 64 * fb + 16 * kk * K::kRowBytes));
            typedef short i16x8_t __attribute__((ext_vector_type(8)));
            const i16x8_t cat = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
            oacc[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cat), pop[kk],
                                                               oacc[fb], 0, 0, 0);
          }
        }
      }
    }

    // ---- second pass needed?  (workgroup-uniform: all waves share the DMA)
    if (pass == 1) break;
    const bool wave_jump = __builtin_amdgcn_ballot_w64(jumped && row_ok) != 0;
    if (threadIdx.x == 0) *redo_flag = 0;
    __syncthreads();
    if (wave_jump && lane == 0) *redo_flag = 1;
    __syncthreads();
    const int redo = *redo_flag;
    __syncthreads();
    if (!redo) break;
  }

  // ---- epilogue: normalize, write final output or the split partial
  const float off = FP8 ? 8.f : 0.f;
  const bool empty = !(l_f > 0.f);
  const float inv = empty ? 0.f : p.out_scale / l_q;
  const float lse_v = empty ? -INFINITY : (m_ref - off + __builtin_amdgcn_logf(l_f)) * kLn2;
  if (!row_ok) return;
  if (p.S == 1) {
    if (p.out_f32) {
      float* o = (float*)p.out + qrow * 512;
#pragma unroll
      for (int fb = 0; fb < 16; fb++)
#pragma unroll
        for (int a = 0; a < 4; a++) {
          const int f0 = 32 * fb + 8 * a + 4 * h;
          float4 w = {oacc[fb][4 * a] * inv, oacc[fb][4 * a + 1] * inv, oacc[fb][4 * a + 2] * inv,
                      oacc[fb][4 * a + 3] * inv};
          *(float4*)(o + f0) = w;
        }
    } else {
      __bf16* o = (__bf16*)p.out + qrow * 512;
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int fb = 0; fb < 16; fb++)
#pragma unroll
        for (int a = 0; a < 4; a++) {
          const int f0 = 32 * fb + 8 * a + 4 * h;
          bf16x4_t w = {(__bf16)(oacc[fb][4 * a] * inv), (__bf16)(oacc[fb][4 * a + 1] * inv),
                        (__bf16)(oacc[fb][4 * a + 2] * inv), (__bf16)(oacc[fb][4 * a + 3] * inv)};
          *(bf16x4_t*)(o + f0) = w;
        }
    }
    if (h == 0 && p.lse) p.lse[qrow] = lse_v;
  } else {
    float* w = p.ws + (qrow * p.S + split) * (int64_t)kPartialWidth;
#pragma unroll
    for (int fb = 0; fb < 16; fb++)
#pragma unroll
      for (int a = 0; a < 4; a++) {
        const int f0 = 32 * fb + 8 * a + 4 * h;
#pragma unroll
        for (int c = 0; c < 4; c++) w[f0 + c] = oacc[fb][4 * a + c] * inv;
      }
    if (h == 0) w[512] = lse_v;
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
      const int ns = min(64, p.S - s0);
      for (int k = 0; k < ns; k++) {
        const float wk = __shfl(w, k);
        if (wk == 0.f) continue;
        const float* src = base + (int64_t)(s0 + k) * kPartialWidth + 8 * lane;
#pragma unroll
        for (int c = 0; c < 8; c++) acc[c] += wk * src[c];
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
template <bool FP8, bool SPARSE, int RG, int NS, bool RESID = false>
static hipError_t launch_partial(const PartialParams& p, int grid, hipStream_t stream) {
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)&mla_partial_kernel<FP8, SPARSE, RG, NS, RESID>, dim3(grid), dim3(64 * RG),
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
        case 4: return launch_partial<true, false, 4, 4>(p, grid, stream);
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
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge_kernel(const MergeParams& p, hipStream_t stream) {
  const int64_t blocks = (p.n_rows + 3) / 4;
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)&mla_merge_kernel, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace mla
