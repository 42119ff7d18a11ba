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
//  * mha_expand_kernel: per (sequence, head, 128 tokens) the GEMM of the
//    gathered latents with [W_UK[h]; W_UV[h]] (256 x 512) on bf16 MFMA,
//    K-chunks of 64 staged through LDS; the result goes through LDS once
//    more so that K_nope is stored as [token][128] and V transposed as
//    [128][token], both with 16-byte coalesced stores;
//  * mha_attn_kernel: per (sequence, head, 128 queries) a flash-attention
//    loop over 64-key tiles staged in LDS and shared by the four waves (32
//    queries each): S^T = K Q^T (keys on the MFMA A side, the 192-wide
//    query in registers on the B side), online softmax in the log2 domain
//    with bf16 P, O^T += V^T P^T.  The S^T accumulator holds per lane one
//    query and 16 keys, which is directly P's B-operand layout; V^T is
//    stored with its keys permuted inside each group of 16 (vt_pos) so that
//    a lane's A operand is one contiguous 16-byte read in the same order.
// Blocks are numbered so that each XCD (every eighth workgroup id) takes a
// contiguous range of work: the blocks of one (sequence, head) run on one
// XCD together and share its L2 for the head's K, V and weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_mha_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ inline i32x4_t ld16(const void* p) { return *(const i32x4_t*)p; }
__device__ inline void st16(void* p, const i32x4_t& v) { *(i32x4_t*)p = v; }
__device__ inline bf16x8_t lds8(const __bf16* p) { return *(const bf16x8_t*)p; }

// Sixteen zero bytes: the source of DMA lanes with nothing to load.
__device__ __attribute__((aligned(16))) uint8_t g_mha_zero16[16];

// LDS DMA: lane i copies 16 bytes from gsrc_i to LDS bytes [m0 + 16 i,
// m0 + 16 i + 16).  Issued from inline asm, so the compiler neither waits
// for it nor counts it; the kernels wait on the vector-memory counter
// themselves before the barrier that publishes a tile.  The s_nop gives the one wait state an LDS DMA
// needs after the SALU write of M0 that precedes it (the compiler adds none
// before inline asm); the build scans the compiled kernels for it.
__device__ inline void dma16(const void* gsrc, uint32_t lds_byte_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(lds_byte_addr) : "memory");
}

__device__ inline void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ inline void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ inline f32x16_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key k in the stored V^T rows: inside each group of 16 keys,
// keys 4e..4e+3 of the first half and 8+4e..8+4e+3 of the second half sit
// next to each other (e = 0, 1), the order in which a lane holds P.
__device__ inline int vt_pos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

// Sequence length clamped to the block table and to max_seq_len (the
// workspace holds Lpad >= max_seq_len tokens per sequence).
__device__ inline int seq_len(const MhaParams& p, int b) {
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.MB * 64 ? p.MB * 64 : L);
  return L > p.max_len ? p.max_len : L;
}

// Work item of this workgroup: XCD x = blockIdx % 8 takes the contiguous
// range [x * n, (x + 1) * n) of work ids, n = gridDim / 8.
__device__ inline int64_t xcd_work_id() {
  return (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
}

// ---------------------------------------------------------------------------
// Expansion.  Work id = ((b * H + h) * tiles + tile): block = 128 tokens of
// sequence b times the 256 outputs of head h.  Wave (wm, wn) computes
// outputs [128 wm, 128 wm + 128) (K_nope for wm = 0, V for wm = 1) of
// tokens [64 wn, 64 wn + 64): D[m][token] = sum_k W[m][k] c_token[k], the
// weights on the A side, the latents on the B side.  D's lane layout:
// token column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4 of register i.
constexpr int EX_TOK = kMhaTokPad;       // tokens per block
constexpr int EX_KC = 64;                // K chunk
constexpr int EX_P = EX_KC + 8;          // LDS row pitch of a chunk (bf16)
constexpr int EX_OP = EX_TOK + 8;        // LDS row pitch of the epilogue tiles (bf16)
constexpr int EX_LDS_CHUNK = (256 + EX_TOK) * EX_P;   // bf16
constexpr int EX_LDS_OUT = 2 * 128 * EX_OP;           // bf16
constexpr int EX_LDS = EX_LDS_CHUNK > EX_LDS_OUT ? EX_LDS_CHUNK : EX_LDS_OUT;

__global__ void __launch_bounds__(256, 2) mha_expand_kernel(const MhaParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[EX_LDS];
  const int n_tiles = p.Lpad / EX_TOK;
  const int64_t w = xcd_work_id();
  if (w >= (int64_t)p.B * p.H * n_tiles) return;
  const int tile = (int)(w % n_tiles);
  const int64_t bh = w / n_tiles;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int L = seq_len(p, b);
  const int n0 = tile * EX_TOK;
  if (n0 >= L) return;   // the attention never reads a tile past the sequence

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  __bf16* w_l = lds;                   // [256][EX_P]
  __bf16* x_l = lds + 256 * EX_P;      // [128][EX_P]

  // Staging: weight rows (tid >> 3) + 32 k, latent rows (tid >> 3) + 32 k,
  // 16 bytes at column 8 (tid & 7) of the chunk.  Latent rows past the
  // sequence, or on a page out of range, read as zeros, so their outputs
  // are exactly zero.
  const int sr = tid >> 3, sc = 8 * (tid & 7);
  const __bf16* wrow[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int m = sr + 32 * k;
    wrow[k] = m < 128 ? p.w_uk + ((int64_t)h * 128 + m) * 512 : p.w_uv + ((int64_t)h * 128 + (m - 128)) * 512;
  }
  const __bf16* xrow[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int j = n0 + sr + 32 * k;
    const int pg = j < L ? p.block_table[(int64_t)b * p.MB + (j >> 6)] : -1;
    xrow[k] = (pg >= 0 && pg < p.NB) ? p.kv + ((int64_t)pg * 64 + (j & 63)) * 576 : nullptr;
  }
  i32x4_t wst[8], xst[4];
  auto fetch = [&](int kc) {
#pragma unroll
    for (int k = 0; k < 8; k++) wst[k] = ld16(wrow[k] + EX_KC * kc + sc);
#pragma unroll
    for (int k = 0; k < 4; k++) xst[k] = xrow[k] ? ld16(xrow[k] + EX_KC * kc + sc) : i32x4_t{0, 0, 0, 0};
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int im = 0; im < 4; im++)
#pragma unroll
    for (int in = 0; in < 2; in++) acc[im][in] = f32x16_t{};
  fetch(0);
  for (int kc = 0; kc < 512 / EX_KC; kc++) {
    __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int k = 0; k < 8; k++) st16(w_l + (sr + 32 * k) * EX_P + sc, wst[k]);
#pragma unroll
    for (int k = 0; k < 4; k++) st16(x_l + (sr + 32 * k) * EX_P + sc, xst[k]);
    __syncthreads();
    if (kc + 1 < 512 / EX_KC) fetch(kc + 1);
#pragma unroll
    for (int ks = 0; ks < EX_KC / 16; ks++) {
      bf16x8_t bx[2];
#pragma unroll
      for (int in = 0; in < 2; in++) bx[in] = lds8(x_l + (64 * wn + 32 * in + l32) * EX_P + 16 * ks + 8 * hh);
#pragma unroll
      for (int im = 0; im < 4; im++) {
        const bf16x8_t a = lds8(w_l + (128 * wm + 32 * im + l32) * EX_P + 16 * ks + 8 * hh);
#pragma unroll
        for (int in = 0; in < 2; in++) acc[im][in] = mfma16(a, bx[in], acc[im][in]);
      }
    }
  }

  // Epilogue: K_nope to k_l[token][dim], V to v_l[dim][vt_pos(token)], then
  // 16-byte rows out.
  __syncthreads();
  __bf16* k_l = lds;                   // [128 tokens][EX_OP]
  __bf16* v_l = lds + 128 * EX_OP;     // [128 dims][EX_OP]
#pragma unroll
  for (int im = 0; im < 4; im++)
#pragma unroll
    for (int in = 0; in < 2; in++) {
      const int n = 64 * wn + 32 * in + l32;
      if (wm == 0) {
#pragma unroll
        for (int a = 0; a < 4; a++) {
          const bf16x4_t v = {(__bf16)acc[im][in][4 * a], (__bf16)acc[im][in][4 * a + 1],
                              (__bf16)acc[im][in][4 * a + 2], (__bf16)acc[im][in][4 * a + 3]};
          *(bf16x4_t*)(k_l + n * EX_OP + 32 * im + 8 * a + 4 * hh) = v;
        }
      } else {
        const int pos = vt_pos(n);
#pragma unroll
        for (int i = 0; i < 16; i++) v_l[(32 * im + 8 * (i / 4) + 4 * hh + i % 4) * EX_OP + pos] = (__bf16)acc[im][in][i];
      }
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int q = tid + 256 * k, r = q >> 4, c = 8 * (q & 15);
    st16(p.ws_k + ((bh * p.Lpad) + n0 + r) * 128 + c, ld16(k_l + r * EX_OP + c));
    st16(p.ws_vt + (bh * 128 + r) * p.Lpad + n0 + c, ld16(v_l + r * EX_OP + c));
  }
}

// ---------------------------------------------------------------------------
// Attention.  Work id = (b * H + h) * chunks + (chunks - 1 - chunk): the
// blocks of one (sequence, head) run together on one XCD, the longest
// (last) query chunk first.  Wave w takes queries q0 + 32 w + (lane % 32).
// Two tile buffers in LDS.  A tile's K rows and its V^T rows are refilled
// separately: the K part of tile kt+2 goes out as soon as every wave is done
// with tile kt's QK products (second barrier of the step), the V^T part of
// tile kt+1 as soon as every wave is done with tile kt-1's PV products
// (first barrier), so each part has about one and a half steps to land
// instead of one.  A buffer holds
// the tile's K_nope rows (64 x 256 B), rope rows (64 x 128 B) and V^T rows
// (128 x 128 B), unpadded, their 16-byte pieces XOR-swizzled (swz16 for the
// 16-piece rows, swz8 for the 8-piece ones) so that the 16 lanes of a
// 16-byte LDS read always hit 16 distinct bank quads.
constexpr int AT_Q = 128;                // queries per block
constexpr int AT_KT = 64;                // keys per tile
constexpr int AT_NOPE = AT_KT * 128;     // bf16 of the K_nope rows
constexpr int AT_ROPE = AT_KT * 64;      // bf16 of the rope rows
constexpr int AT_VT = 128 * AT_KT;       // bf16 of the V^T rows
constexpr int AT_BUF = AT_NOPE + AT_ROPE + AT_VT;   // one tile buffer (40 KiB)

__device__ inline int swz16(int row, int c) { return c ^ (row & 15); }
__device__ inline int swz8(int row, int c) { return c ^ ((row >> 1) & 7); }

__global__ void __launch_bounds__(256, 2) mha_attn_kernel(const MhaParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 tbuf[2 * AT_BUF];
  const int n_qc = (p.T + AT_Q - 1) / AT_Q;
  const int64_t w = xcd_work_id();
  if (w >= (int64_t)p.B * p.H * n_qc) return;
  const int qc = n_qc - 1 - (int)(w % n_qc);
  const int64_t bh = w / n_qc;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int L = seq_len(p, b);
  const int q0 = qc * AT_Q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int t = q0 + 32 * wave + l32;
  const bool t_ok = t < p.T;
  const int n_vis = t_ok ? max(0, L - p.T + t + 1) : 0;   // keys this lane's query sees
  // Keys the wave needs at most, and the fewest any of its real queries
  // sees (tiles below that need no mask).
  int nv_max = n_vis, nv_min = t_ok ? n_vis : 0x7fffffff;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    nv_max = max(nv_max, __shfl_xor(nv_max, d));
    nv_min = min(nv_min, __shfl_xor(nv_min, d));
  }
  const int t_last = min(q0 + AT_Q, p.T) - 1;
  const int n_blk = max(0, L - p.T + t_last + 1);   // keys the block needs
  const int n_kt = (n_blk + AT_KT - 1) / AT_KT;

  // Query operand: B side, column = query, 8 features per lane half and step.
  bf16x8_t qreg[12];
  {
    const int64_t qr = ((int64_t)b * p.T + (t_ok ? t : 0)) * p.H + h;
#pragma unroll
    for (int ks = 0; ks < 12; ks++) {
      const int k = 16 * ks + 8 * hh;
      const bf16x8_t v = ks < 8 ? lds8(p.q_nope + qr * 128 + k) : lds8(p.q_pe + qr * 64 + (k - 128));
      qreg[ks] = t_ok ? v : bf16x8_t{};
    }
  }

  // One tile goes from HBM into a buffer by 40 LDS-DMA instructions of 64
  // lanes; instruction g fills 16-byte slots [64 g, 64 g + 64) of the
  // buffer: g < 16 the K_nope rows, g < 24 the rope rows (from the cache),
  // the rest the V^T rows.  Wave w issues K_nope instructions 4 w .. 4 w + 3,
  // rope 16 + 2 w, 17 + 2 w and V^T 24 + 4 w .. 27 + 4 w, so the kind of its
  // i-th instruction is fixed at compile time.  A slot's logical piece is
  // its swizzled position (each swizzle is its own inverse), so every lane's
  // source offset within a tile is fixed and only the tile start moves.
  // The tile's keys all lie on one cache page, looked up one tile ahead (a
  // page out of range reads zeros).  Every tile read starts below L, inside
  // a 128-token block the expansion wrote (zeros past L), so the workspace
  // reads need no bounds; rope rows past L are read from their page and
  // masked out of the softmax.
  const __bf16* ks_base = p.ws_k + bh * p.Lpad * 128;
  const __bf16* vt_base = p.ws_vt + bh * 128 * p.Lpad;
  const int32_t* bt = p.block_table + (int64_t)b * p.MB;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int src_off[10];    // element offset of this lane's piece within the tile's source
  uint32_t dst[10];   // LDS byte offset of the instruction within a buffer
#pragma unroll
  for (int i = 0; i < 10; i++) {
    if (i < 4) {
      const int g = 4 * wv + i, sl = 64 * g + lane, r = sl >> 4;
      src_off[i] = r * 128 + 8 * swz16(r, sl & 15);
      dst[i] = g * 1024;
    } else if (i < 6) {
      const int g = 16 + 2 * wv + (i - 4), sl = 64 * (g - 16) + lane, r = sl >> 3;
      src_off[i] = r * 576 + 512 + 8 * swz8(r, sl & 7);
      dst[i] = g * 1024;
    } else {
      const int g = 24 + 4 * wv + (i - 6), sl = 64 * (g - 24) + lane, d = sl >> 3;
      src_off[i] = d * p.Lpad + 8 * swz8(d, sl & 7);
      dst[i] = g * 1024;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)tbuf;
  // The block table is read with scalar loads (uniform index), so that the
  // only vector-memory instructions in flight in the loop are the DMAs and
  // the waits below can count them.
  const __attribute__((address_space(4))) int32_t* btc = (const __attribute__((address_space(4))) int32_t*)bt;
  int pg = n_kt > 0 ? btc[0] : -1;   // page of the next tile whose keys are fetched
  // K part of a tile (6 DMA instructions per wave: K_nope, rope).
  auto fetch_k = [&](int j0, int buf) {
    const bool pg_ok = pg >= 0 && pg < p.NB;
    const uint32_t lb = lds0 + (uint32_t)(buf * AT_BUF * 2);
#pragma unroll
    for (int i = 0; i < 6; i++) {
      const void* src;
      if (i < 4) src = ks_base + (int64_t)j0 * 128 + src_off[i];
      else src = pg_ok ? (const void*)(p.kv + (int64_t)pg * 64 * 576 + src_off[i]) : (const void*)g_mha_zero16;
      dma16(src, lb + dst[i]);
    }
    pg = j0 + AT_KT < n_blk ? btc[(j0 + AT_KT) >> 6] : -1;
  };
  // V part of a tile (4 DMA instructions per wave).
  auto fetch_v = [&](int j0, int buf) {
    const uint32_t lb = lds0 + (uint32_t)(buf * AT_BUF * 2);
#pragma unroll
    for (int i = 6; i < 10; i++) dma16(vt_base + j0 + src_off[i], lb + dst[i]);
  };

  const float c_qk = p.qk_scale;   // softmax scale * log2(e)
  float m = -INFINITY;             // running maximum (log2 domain), per query
  float l = 0.f;                   // this half's sum of the rounded weights (normalizes O)
  float lx = 0.f;                  // this half's sum of the unrounded weights (the LSE)
  f32x16_t o[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};   // O^T, dims 32 f .. 32 f + 31
  const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};

  // Per wave, DMAs go out in the order K(0) V(0) K(1), then in tile kt
  // V(kt+1) after the first barrier and K(kt+2) after the second, so that
  // K(kt) is followed by V(kt) and K(kt+1), and V(kt) by K(kt+1) and V(kt+1).
  if (n_kt > 0) { fetch_k(0, 0); fetch_v(0, 0); }
  if (n_kt > 1) fetch_k(AT_KT, 1);
  for (int kt = 0; kt < n_kt; kt++) {
    const int j0 = kt * AT_KT;
    if (kt + 1 < n_kt) wait_vmcnt<10>();
    else wait_vmcnt<4>();
    __syncthreads();   // K(kt) in LDS; every wave is done with tile kt-1's V^T
    if (kt + 1 < n_kt) fetch_v(j0 + AT_KT, (kt + 1) & 1);
    const __bf16* kn_l = tbuf + (kt & 1) * AT_BUF;   // K_nope rows
    const __bf16* kr_l = kn_l + AT_NOPE;               // rope rows
    const __bf16* vb_l = kr_l + AT_ROPE;               // V^T rows
    bf16x8_t pb[2][2];   // this tile's weights (P^T operand)
    if (j0 < nv_max) {   // some query of this wave sees the tile
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int ks = 0; ks < 12; ks++)
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
          const int r = 32 * kb + l32;
          const __bf16* a = ks < 8 ? kn_l + (r * 16 + swz16(r, 2 * ks + hh)) * 8
                                   : kr_l + (r * 8 + swz8(r, 2 * (ks - 8) + hh)) * 8;
          s[kb] = mfma16(lds8(a), qreg[ks], s[kb]);
        }

      // Register i of block kb holds key j0 + 32 kb + 8 (i / 4) + 4 hh + i % 4.
      // The row maximum is taken on the raw scores (the scale is positive),
      // and the scale and shift enter each exponent in one fma.
      if (j0 + AT_KT > nv_min) {   // some key of the tile is past some query's causal limit
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int i = 0; i < 16; i++)
            if (j0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4) >= n_vis) s[kb][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(s[kb][i], s[kb][i + 1]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m, tmax == -INFINITY ? -INFINITY : tmax * c_qk);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      const float nsh = m_new == -INFINITY ? 0.f : -m_new;
      float ls = 0.f, lsx = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c_qk, nsh));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], c_qk, nsh));
          const bf16x2_t pr = {(__bf16)e0, (__bf16)e1};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
          lsx += e0 + e1;
          pb[kb][i / 8][i % 8] = pr[0];
          pb[kb][i / 8][i % 8 + 1] = pr[1];
        }
      l = l * alpha + ls;
      lx = lx * alpha + lsx;
      m = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int f = 0; f < 4; f++)
#pragma unroll
          for (int i = 0; i < 16; i++) o[f][i] *= alpha;
      }
    }
    if (kt + 1 < n_kt) wait_vmcnt<10>();
    else wait_vmcnt0();
    __syncthreads();   // V(kt) in LDS; every wave is done with tile kt's K rows
    if (kt + 2 < n_kt) fetch_k(j0 + 2 * AT_KT, kt & 1);
    if (j0 < nv_max) {
      // V^T on the A side: row = dim 32 f + l32, keys 16 s + [8 hh, 8 hh + 8)
      // in stored order, which is the order of P's group s (block s / 2,
      // registers 8 (s % 2) ..).
#pragma unroll
      for (int f = 0; f < 4; f++)
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) {
          const int d = 32 * f + l32;
          o[f] = mfma16(lds8(vb_l + (d * 8 + swz8(d, 2 * s4 + hh)) * 8), pb[s4 >> 1][s4 & 1], o[f]);
        }
    }
  }

  const float l_tot = l + __shfl_xor(l, 32);
  const float lx_tot = lx + __shfl_xor(lx, 32);
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
  if (hh == 0 && p.lse) p.lse[orow] = empty ? -INFINITY : (m + __builtin_amdgcn_logf(lx_tot)) * kLn2;
}

unsigned grid_of(int64_t work) { return (unsigned)((work + 7) / 8 * 8); }

}  // namespace

hipError_t launch_mha(const MhaParams& p, hipStream_t stream) {
  void* args[] = {(void*)&p};
  if (p.Lpad > 0) {   // no cached token at all: the attention alone writes the empty rows
    const int64_t work = (int64_t)p.B * p.H * (p.Lpad / EX_TOK);
    const hipError_t e = hipLaunchKernel((const void*)&mha_expand_kernel, dim3(grid_of(work)), dim3(256), args, 0,
                                         stream);
    if (e != hipSuccess) return e;
  }
  const int64_t work = (int64_t)p.B * p.H * ((p.T + AT_Q - 1) / AT_Q);
  return hipLaunchKernel((const void*)&mha_attn_kernel, dim3(grid_of(work)), dim3(256), args, 0, stream);
}

}  // namespace mla
