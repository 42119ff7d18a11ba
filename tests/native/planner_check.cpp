// Host-only check of the library's C ABI layer (argument checks, split
// planner, workspace sizing, launch parameters) built with AddressSanitizer
// and UndefinedBehaviorSanitizer, no GPU involved.
//
// The HIP runtime calls the host layer makes and the kernel launchers are
// replaced by stubs: the launchers check what the kernels assume of their
// parameters (grid covers the units, chunk fits the LDS tables, splits
// cover the sequence, the workspace holds the partials) and never touch the
// (fake) device pointers.  The device reports MLA_CHECK_CUS compute units
// (default 256).  Exit status 0 when every call behaved; a sanitizer report
// or a failed check exits non-zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "mla_decode.h"
#include "../../mla_paged_latent_03_amd/csrc/mla_decode_internal.h"
#include "../../mla_paged_latent_03_amd/csrc/mla_mha_internal.h"

static int g_failures = 0;
static long g_partial_launches = 0, g_merge_launches = 0, g_mha_launches = 0;

#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      if (g_failures < 20) {                                          \
        std::fprintf(stderr, "check failed: %s: ", #cond);            \
        std::fprintf(stderr, __VA_ARGS__);                            \
        std::fprintf(stderr, "\n");                                   \
      }                                                               \
      g_failures++;                                                   \
    }                                                                 \
  } while (0)

// ---------------------------------------------------------------- HIP runtime stubs
extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  const char* e = std::getenv("MLA_CHECK_CUS");
  *v = attr == hipDeviceAttributeMultiprocessorCount ? (e ? std::atoi(e) : 256) : 0;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

// ---------------------------------------------------------------- launcher stubs
struct Expect {
  int B, T, H, max_len, topk;
  bool fp8;
  size_t ws_bytes;
  int req_splits;
} g_expect;

namespace mla {

static unsigned char g_static[64];

hipError_t static_scratch(void** ptr) {
  *ptr = g_static;
  return hipSuccess;
}

int partial_kernel_occupancy(bool, bool sparse, int rg, bool) { return rg == 4 || sparse ? 1 : 2; }

hipError_t launch_partial_kernel(const PartialParams& p, bool fp8, bool sparse, int rg, bool resid, int grid,
                                 hipStream_t) {
  g_partial_launches++;
  const Expect& e = g_expect;
  CHECK(p.B == e.B && p.T == e.T && p.H == e.H && p.R == e.T * e.H, "shape B=%d T=%d H=%d", e.B, e.T, e.H);
  CHECK(fp8 == e.fp8 && sparse == (e.topk > 0), "kind");
  CHECK(rg == 1 || rg == 2 || rg == 4, "rg=%d", rg);
  CHECK(!resid || fp8, "residual product on bf16");
  CHECK(p.S >= 1 && p.S <= MLA_MAX_KV_SPLITS, "S=%d", p.S);
  CHECK(e.req_splits == 0 || p.S == e.req_splits, "requested %d splits, got %d", e.req_splits, p.S);
  CHECK(p.n_units >= 1 && grid >= p.n_units && grid % 8 == 0, "grid %d units %d", grid, p.n_units);
  CHECK((p.S > 1) == (p.ws != nullptr), "workspace pointer with S=%d", p.S);
  if (p.S > 1 && e.ws_bytes > 0)
    CHECK(e.ws_bytes >= (size_t)p.B * p.R * p.S * kPartialWidth * sizeof(float), "workspace %zu short", e.ws_bytes);
  if (sparse) {
    CHECK(p.K == e.topk, "K");
    CHECK(p.chunk >= 64 && p.chunk % 64 == 0 && p.chunk <= kSparseChunkMax, "sparse chunk %d", p.chunk);
    CHECK((int64_t)p.chunk * p.S >= p.K, "splits of %d cover %d of %d indices", p.chunk, p.chunk * p.S, p.K);
    CHECK((int64_t)p.n_hb * 32 * rg >= p.H && p.n_rb == p.T * p.n_hb, "head blocks");
    CHECK((int64_t)p.n_units == (int64_t)p.B * p.S * p.n_rb, "sparse units");
  } else {
    CHECK(p.chunk >= 1 && p.chunk <= kDensePagesMax, "dense chunk %d", p.chunk);
    CHECK((int64_t)p.n_rb * 32 * rg >= p.R, "row blocks %d x %d rows < %d", p.n_rb, 32 * rg, p.R);
    const int max_pages = (e.max_len + kPage - 1) / kPage;
    if (!p.balance) {
      CHECK((int64_t)p.chunk * p.S >= max_pages, "fixed chunks %d x %d < %d pages", p.chunk, p.S, max_pages);
      CHECK((int64_t)p.n_units == (int64_t)p.B * p.S * p.n_rb, "dense units");
    } else {
      CHECK(p.S > 1 && p.max_pages == max_pages && p.n_target >= 1, "balance params");
      CHECK(p.n_units % p.n_rb == 0, "balanced units");
    }
  }
  if (p.fused) CHECK(p.sync != nullptr && p.S > 1 && p.S <= 64, "fused");
  return hipSuccess;
}

hipError_t launch_merge_kernel(const MergeParams& m, hipStream_t) {
  g_merge_launches++;
  CHECK(m.S >= 2 && m.n_rows == (int64_t)g_expect.B * g_expect.T * g_expect.H && m.ws != nullptr, "merge");
  return hipSuccess;
}

hipError_t launch_mha(const MhaParams& p, hipStream_t) {
  g_mha_launches++;
  CHECK(p.Lpad % kMhaTokPad == 0 && p.Lpad >= p.max_len && p.Lpad < p.max_len + kMhaTokPad, "Lpad %d for %d",
        p.Lpad, p.max_len);
  CHECK(p.Lpad == 0 || (p.ws_k != nullptr && p.ws_vt != nullptr), "mha workspace");
  CHECK((char*)p.ws_vt - (char*)p.ws_k == (ptrdiff_t)((size_t)p.B * p.H * p.Lpad * 128 * 2), "V^T offset");
  return hipSuccess;
}

}  // namespace mla

// ---------------------------------------------------------------- the sweep
static void* fake(size_t k) { return (void*)(uintptr_t)(0x100000 + 0x1000 * k); }

static void call_all(int B, int T, int H, int L, int topk, int req) {
  const int NB = 16, MB = (L + 63) / 64 > 0 ? (L + 63) / 64 : 1;
  for (int fp8 = 0; fp8 < 2; fp8++) {
    const size_t ws = mla_workspace_size(B, T, H, L, topk, fp8, req);
    const int S = mla_num_kv_splits(B, T, H, L, topk, fp8);
    const int waves = mla_launch_waves(B, T, H, L, topk, fp8);
    CHECK(S >= 0 && S <= MLA_MAX_KV_SPLITS, "splits %d", S);
    CHECK(waves == 0 || waves == 1 || waves == 2 || waves == 4, "waves %d", waves);
    g_expect = Expect{B, T, H, L, topk, fp8 != 0, ws, req};
    const int32_t* bt = (const int32_t*)fake(3);
    const int32_t* sl = (const int32_t*)fake(4);
    void* out = fake(6);
    float* lse = (float*)fake(7);
    void* w = ws ? fake(8) : nullptr;
    auto invoke = [&](size_t bytes) {
      if (topk > 0) {
        const int32_t* idx = (const int32_t*)fake(5);
        return fp8 ? mla_sparse_decode_fp8(fake(0), fake(1), fake(2), bt, sl, idx, topk, B, T, H, NB, 64, MB, L,
                                           0.07f, 0.5f, 0.25f, out, MLA_OUT_BF16, lse, w, bytes, req, nullptr)
                   : mla_sparse_decode(fake(0), fake(1), fake(2), bt, sl, idx, topk, B, T, H, NB, 64, MB, L, 0.07f,
                                       out, MLA_OUT_F32, lse, w, bytes, req, nullptr);
      }
      return fp8 ? mla_decode_fp8(fake(0), fake(1), fake(2), bt, sl, B, T, H, NB, 64, MB, L, 0.07f, 0.5f, 0.25f, out,
                                  MLA_OUT_BF16, lse, w, bytes, req, nullptr)
                 : mla_decode(fake(0), fake(1), fake(2), bt, sl, B, T, H, NB, 64, MB, L, 0.07f, out, MLA_OUT_F32, lse,
                              w, bytes, req, nullptr);
    };
    const mla_status_t st = invoke(ws);
    CHECK(st == MLA_OK || st == MLA_ERR_UNSUPPORTED, "status %d (B=%d T=%d H=%d L=%d K=%d req=%d fp8=%d)", st, B, T, H,
          L, topk, req, fp8);
    if (fp8 && topk == 0) {
      const mla_status_t s2 = mla_decode_fp8_noalloc(fake(0), fake(1), fake(2), bt, sl, B, T, H, NB, 64, MB, L, 0.07f,
                                                     0.5f, 0.25f, out, MLA_OUT_BF16, lse, req, nullptr);
      CHECK(s2 == st || (st == MLA_OK && s2 == MLA_ERR_SCRATCH_LIMIT), "noalloc status %d against %d", s2, st);
      CHECK(s2 != MLA_ERR_SCRATCH_LIMIT || ws > mla::kStaticScratchBytes, "refused %zu bytes", ws);
    }
    if (st == MLA_OK && B > 0 && ws > 0) {   // one byte short is refused before any launch
      const long before = g_partial_launches;
      CHECK(invoke(ws - 1) == MLA_ERR_WORKSPACE_TOO_SMALL, "short workspace accepted");
      CHECK(g_partial_launches == before, "launched with a short workspace");
    }
  }
}

int main() {
  const int Bs[] = {0, 1, 2, 3, 7, 64, 128, 255, 1000, 4097};
  const int Ts[] = {1, 2, 4, 8};
  const int Hs[] = {1, 16, 32, 33, 64, 128, 1024};
  const int Ls[] = {0, 1, 63, 64, 65, 300, 8192, 80000, 1 << 20};
  const int Ks[] = {0, 64, 100, 2048};
  const int reqs[] = {0, 1, 2, 3, 17, 256};
  for (int B : Bs)
    for (int T : Ts)
      for (int H : Hs)
        for (int L : Ls)
          for (int K : Ks)
            for (int r : reqs) {
              if ((long)B * T * H > (1L << 22) && (r != 0 || K != 0)) continue;   // keep the sweep short
              call_all(B, T, H, L, K, r);
            }
  // The dense MHA route's host layer.
  for (int B : {0, 1, 3, 64})
    for (int H : {1, 16, 128})
      for (int L : {0, 1, 31, 32, 33, 2048}) {
        const size_t need = mla_dense_mha_workspace_size(B, H, L);
        g_expect = Expect{B, 1, H, L, 0, false, need, 0};
        const mla_status_t st =
            mla_dense_mha(fake(0), fake(1), fake(2), (const int32_t*)fake(3), (const int32_t*)fake(4), fake(5),
                          fake(6), B, 4, H, 16, 64, 40, L, 0.07f, fake(7), MLA_OUT_BF16, (float*)fake(8),
                          need ? fake(9) : nullptr, need, nullptr);
        CHECK(st == MLA_OK, "mha status %d", st);
      }
  std::printf("partial launches %ld, merge launches %ld, mha launches %ld, failures %d\n", g_partial_launches,
              g_merge_launches, g_mha_launches, g_failures);
  return g_failures == 0 && g_partial_launches > 0 ? 0 : 1;
}
