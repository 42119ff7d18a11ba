// Streaming-read reference for the decode benchmark (libmla_stream_ref.so).
//
// Reads a buffer once from HBM into LDS through the same path the decode
// kernels use for KV tiles: 16-byte buffer_load ... lds DMAs with the
// non-temporal hint, 36 KiB tiles, a ring of four tiles with three in
// flight, four waves per workgroup, one workgroup per compute unit.  It
// does no arithmetic on the data, so its rate is what the decode's tile
// stream could reach with nothing else to do: the practical ceiling the
// decode's HBM roofline fraction is read against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = 36864;          // one fp8 page of 64 tokens x 576 bytes
constexpr int kRing = 4;
constexpr int kWaves = 4;
constexpr int kInstrPerWave = kTileBytes / 1024 / kWaves;   // 16-byte DMAs per lane per tile

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Buffer descriptor over [base, base + bytes); the s_nop gives the five wait
// states a vector memory read of VALU-written SGPRs needs (the compiler adds
// none before inline asm).
__device__ inline i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
  asm volatile("s_nop 4" : "+s"(r));
  return r;
}

// One 16-byte-per-lane DMA into LDS at m0 (one wait state after the M0 write).
__device__ inline void dma16_buf(int voff, i32x4_t rsrc, int soff, uint32_t lds_byte_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "{m0}"(lds_byte_addr)
               : "memory");
}

// Workgroup g streams tiles [g * n / G, (g + 1) * n / G) of the buffer.
__global__ void __launch_bounds__(64 * kWaves) stream_read_kernel(const uint8_t* src, int64_t n_tiles,
                                                                  uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * n_tiles / gridDim.x;
  const int64_t t1 = (int64_t)(blockIdx.x + 1) * n_tiles / gridDim.x;
  const uint32_t lds0 = (uint32_t)(uintptr_t)ring;
  auto issue = [&](int64_t t, int slot) __attribute__((always_inline)) {
    // past the range: a zero-size descriptor (reads zeros, no memory access)
    const bool real = t < t1;
    const i32x4_t rsrc = buffer_rsrc(src + (real ? t : t0) * kTileBytes, real ? kTileBytes : 0);
#pragma unroll
    for (int j = 0; j < kInstrPerWave; j++) {
      const int unit = (wave * kInstrPerWave + j) * 64;
      dma16_buf(16 * lane, rsrc, 16 * unit, lds0 + slot * kTileBytes + 16 * unit);
    }
  };
  if (t1 > t0) {
    for (int k = 0; k < kRing - 1; k++) issue(t0 + k, k);
    for (int64_t t = t0; t < t1; t++) {
      wait_vmcnt<kInstrPerWave * (kRing - 2)>();     // tile t landed (two more in flight)
      __builtin_amdgcn_s_barrier();                  // every wave is past tile t-1's slot
      issue(t + kRing - 1, (int)((t - t0 + kRing - 1) % kRing));
    }
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = ring[(blockIdx.x * 64) % sizeof(ring)];
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 36864, 16-byte aligned device memory) once
// into LDS with `grid` workgroups; writes one byte per workgroup to `sink`
// (device, grid uint32 values).  Returns 0 on success, 1 on invalid
// arguments, 2 on a launch failure.
int mla_stream_read_reference(const void* src, int64_t bytes, int grid, uint32_t* sink, void* stream) {
  if (!src || !sink || grid < 1 || bytes <= 0 || bytes % kTileBytes != 0 || ((uintptr_t)src & 15) != 0) return 1;
  const int64_t n_tiles = bytes / kTileBytes;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(64 * kWaves), 0, (hipStream_t)stream,
                     (const uint8_t*)src, n_tiles, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
