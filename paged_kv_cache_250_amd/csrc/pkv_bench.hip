// Measurement helpers: a cache-evicting fill, a 128-bit streaming read that
// measures the achievable HBM read bandwidth, and a plain copy of known
// traffic for calibrating hardware byte counters.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int BENCH_THREADS = 256;
constexpr int BENCH_MAX_GROUPS = 8192;

__global__ __launch_bounds__(BENCH_THREADS) void bench_fill_kernel(u32x4* __restrict__ p,
                                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * BENCH_THREADS;
  const u32x4 pat = {0x9E3779B9u, 0x7F4A7C15u, 0x85EBCA6Bu, 0xC2B2AE35u};
  for (int64_t i = (int64_t)blockIdx.x * BENCH_THREADS + threadIdx.x; i < n16; i += stride)
    p[i] = pat ^ (uint32_t)i;
}

// Each wave reads its own range of whole 1 KB runs (one 128-bit load per
// lane covers a run) and keeps READ_DEPTH loads in flight: in the steady
// state a load is issued, unconditionally, as soon as the one READ_DEPTH
// runs before it has been consumed (a conditional load would make the
// compiler wait for it at once).  Runs past the last multiple of READ_DEPTH
// are read one at a time, and wave 0 also reads the last partial run.
constexpr int READ_DEPTH = 4;

__global__ __launch_bounds__(BENCH_THREADS) void bench_read_kernel(const u32x4* __restrict__ p,
                                                                   int64_t n16, int64_t per_wave,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (BENCH_THREADS / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t runs = n16 / 64;
  const int64_t lo = wave * per_wave < runs ? wave * per_wave : runs;
  const int64_t cnt = (lo + per_wave < runs ? lo + per_wave : runs) - lo;
  const u32x4* q = p + lo * 64 + lane;
  u32x4 acc = {0, 0, 0, 0};
  int64_t i = 0;
  if (cnt >= READ_DEPTH) {
    u32x4 r[READ_DEPTH];
#pragma unroll
    for (int k = 0; k < READ_DEPTH; ++k) r[k] = __builtin_nontemporal_load(q + (int64_t)k * 64);
    for (; i + 2 * READ_DEPTH <= cnt; i += READ_DEPTH) {
#pragma unroll
      for (int k = 0; k < READ_DEPTH; ++k) {
        acc ^= r[k];
        r[k] = __builtin_nontemporal_load(q + (i + k + READ_DEPTH) * 64);
        __builtin_amdgcn_sched_barrier(0);  // keep each load beside its use
      }
    }
#pragma unroll
    for (int k = 0; k < READ_DEPTH; ++k) acc ^= r[k];
    i += READ_DEPTH;
  }
  for (; i < cnt; ++i) acc ^= __builtin_nontemporal_load(q + i * 64);
  if (wave == 0 && runs * 64 + lane < n16) acc ^= __builtin_nontemporal_load(p + runs * 64 + lane);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t red[BENCH_THREADS / 64];
  if (lane == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int w = 0; w < BENCH_THREADS / 64; ++w) v ^= red[w];
    sink[blockIdx.x] = v;
  }
}

__global__ __launch_bounds__(BENCH_THREADS) void bench_copy_kernel(u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src,
                                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * BENCH_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * BENCH_THREADS + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

static unsigned bench_groups(int64_t n16) {
  int64_t g = (n16 + BENCH_THREADS - 1) / BENCH_THREADS;
  if (g > BENCH_MAX_GROUPS) g = BENCH_MAX_GROUPS;
  return (unsigned)(g < 1 ? 1 : g);
}

static pkv_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_bench_flush(void* buf, size_t bytes, pkv_stream_t stream) {
  if (!buf || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return fail(PKV_ERR_INVALID_ARG, "buffer must be 16-byte aligned, size a multiple of 16");
  if (bytes == 0) return PKV_OK;
  const int64_t n16 = (int64_t)(bytes / 16);
  (void)hipGetLastError();  // report only this call's launch errors
  hipLaunchKernelGGL(bench_fill_kernel, dim3(bench_groups(n16)), dim3(BENCH_THREADS), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<u32x4*>(buf), n16);
  return check_launch("flush");
}

extern "C" pkv_status pkv_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                            pkv_stream_t stream) {
  if (!buf || !sink || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return fail(PKV_ERR_INVALID_ARG, "buffer must be 16-byte aligned, size a multiple of 16");
  if (bytes == 0) return PKV_OK;
  const int64_t n16 = (int64_t)(bytes / 16);
  // four workgroups of four waves per compute unit, all resident at once
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "stream read: %s", hipGetErrorString(e));
  constexpr int WAVES = BENCH_THREADS / 64;
  const int64_t runs = n16 / 64;
  int64_t groups = 4 * (int64_t)(cus > 0 ? cus : 1);
  if (groups > BENCH_MAX_GROUPS) groups = BENCH_MAX_GROUPS;
  if (groups * WAVES > runs) groups = runs > WAVES ? runs / WAVES : 1;
  const int64_t per_wave = (runs + groups * WAVES - 1) / (groups * WAVES);
  (void)hipGetLastError();  // report only this call's launch errors
  hipLaunchKernelGGL(bench_read_kernel, dim3((unsigned)groups), dim3(BENCH_THREADS), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), n16,
                     per_wave, sink);
  return check_launch("stream read");
}

extern "C" pkv_status pkv_bench_copy(void* dst, const void* src, size_t bytes,
                                     pkv_stream_t stream) {
  if (!dst || !src || (bytes & 15) || ((reinterpret_cast<uintptr_t>(dst) |
                                        reinterpret_cast<uintptr_t>(src)) & 15))
    return fail(PKV_ERR_INVALID_ARG, "buffers must be 16-byte aligned, size a multiple of 16");
  if (bytes == 0) return PKV_OK;
  const int64_t n16 = (int64_t)(bytes / 16);
  (void)hipGetLastError();  // report only this call's launch errors
  hipLaunchKernelGGL(bench_copy_kernel, dim3(bench_groups(n16)), dim3(BENCH_THREADS), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n16);
  return check_launch("copy");
}
