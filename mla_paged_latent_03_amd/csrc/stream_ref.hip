// Streaming-read and LDS read-rate references for the decode benchmark
// (libmla_stream_ref.so).
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


// LDS read-rate reference.  Each lane reads 16 bytes per ds_read_b128 from a
// 64 KiB LDS array: INFLIGHT independent reads per iteration, all issued
// before any is used and all used before the next iteration's, folded into
// one value so that none is dropped.  Index
// lane + 64 k with k in [0, 64) stays inside the 4096 16-byte slots.  Thread
// 0 records the shader clock (s_memtime) and the constant-rate wall clock
// around the loop, so the host gets bytes per shader clock per workgroup and
// the clock frequency itself.
template <int WAVES, int INFLIGHT>
__global__ void __launch_bounds__(64 * WAVES) lds_read_rate_kernel(int iters, int* sink, long long* clocks) {
  __shared__ i32x4_t buf[4096];
  for (int i = threadIdx.x; i < 4096; i += 64 * WAVES) buf[i] = (i32x4_t){i, i + 1, i + 2, i + 3};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  i32x4_t acc = {0, 0, 0, 0};
  const long long c0 = clock64();
  const long long w0 = wall_clock64();
  for (int it = 0; it < iters; it++) {
    i32x4_t v[INFLIGHT];
#pragma unroll
    for (int j = 0; j < INFLIGHT; j++) v[j] = buf[lane + 64 * ((it * INFLIGHT + j + 7 * wv) & 63)];
#pragma unroll
    for (int j = 0; j < INFLIGHT; j++) acc ^= v[j];
    // The next round's reads stay behind this round's (no overlap across
    // iterations), so INFLIGHT is the number in flight.
    asm volatile("" : "+v"(acc)::"memory");
  }
  __syncthreads();
  const long long c1 = clock64();
  const long long w1 = wall_clock64();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = w1 - w0;
  }
  sink[blockIdx.x * 64 * WAVES + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

template <int WAVES, int INFLIGHT>
hipError_t launch_rate(int grid, int iters, int* sink, long long* clocks, hipStream_t stream) {
  hipLaunchKernelGGL((lds_read_rate_kernel<WAVES, INFLIGHT>), dim3(grid), dim3(64 * WAVES), 0, stream, iters, sink,
                     clocks);
  return hipGetLastError();
}

template <int WAVES>
hipError_t launch_rate_w(int inflight, int grid, int iters, int* sink, long long* clocks, hipStream_t stream) {
  switch (inflight) {
    case 2: return launch_rate<WAVES, 2>(grid, iters, sink, clocks, stream);
    case 4: return launch_rate<WAVES, 4>(grid, iters, sink, clocks, stream);
    case 8: return launch_rate<WAVES, 8>(grid, iters, sink, clocks, stream);
    default: return launch_rate<WAVES, 16>(grid, iters, sink, clocks, stream);
  }
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

// LDS read-rate reference: `grid` workgroups of `waves` waves (1, 2, 4, 8 or
// 16), each lane keeping `inflight` (2, 4, 8 or 16) 16-byte LDS reads in
// flight for `iters` iterations.  Writes 64 * waves ints per workgroup to
// `sink` (device) and, per workgroup, its shader-clock cycles and wall-clock
// ticks around the loop to `clocks` (device, 2 * grid int64); the wall
// clock's rate in kHz goes to *wall_khz (host).  Returns 0 on success, 1 on
// invalid arguments, 2 on a launch or device-query failure.
int mla_lds_read_rate_reference(int waves, int inflight, int grid, int iters, int* sink, long long* clocks,
                                int* wall_khz, void* stream) {
  const bool w_ok = waves == 1 || waves == 2 || waves == 4 || waves == 8 || waves == 16;
  const bool f_ok = inflight == 2 || inflight == 4 || inflight == 8 || inflight == 16;
  if (!w_ok || !f_ok || grid < 1 || iters < 1 || !sink || !clocks || !wall_khz) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return 2;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (waves) {
    case 1: e = launch_rate_w<1>(inflight, grid, iters, sink, clocks, st); break;
    case 2: e = launch_rate_w<2>(inflight, grid, iters, sink, clocks, st); break;
    case 4: e = launch_rate_w<4>(inflight, grid, iters, sink, clocks, st); break;
    case 8: e = launch_rate_w<8>(inflight, grid, iters, sink, clocks, st); break;
    default: e = launch_rate_w<16>(inflight, grid, iters, sink, clocks, st); break;
  }
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
