// Probes, built as their own small library (not part of the AWQ C ABI).
//
// Streaming-read probe:
// reads a device buffer once with 16-byte nontemporal loads, one contiguous 16 KiB
// chunk per workgroup, and stores a word only if the XOR of all data equals a magic
// value (practically never).  Timed by the benchmark next to awq_gemm on the same
// byte count, it gives the per-launch time of a plain read of those bytes on this
// device: launch and memory latency included, no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int64_t kChunk = 16384;  // bytes per workgroup

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (kChunk / 16);
  uint32_t acc = 0u;
#pragma unroll
  for (int r = 0; r < (int)(kChunk / 16 / kThreads); ++r) {
    const int64_t i = base + threadIdx.x + (int64_t)r * kThreads;
    if (i < n16) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Launch-floor probe: a grid of workgroups that do nothing.  Replayed back to back from a
// graph, its per-launch time is what every dependent launch costs on this device before
// any work: dispatch, wave launch and retirement, the end-of-kernel release.
__global__ void empty_kernel(uint32_t* __restrict__ sink, int never) {
  if (never == 1 && threadIdx.x == 0) sink[blockIdx.x] = 0u;  // the host passes 0
}

}  // namespace

// bytes: multiple of 16; sink: at least ceil(bytes / 16384) words of device memory.
// Returns the hipError_t of the launch.
extern "C" int awq_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  const int64_t blocks = (bytes + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

// blocks x threads workgroups of the empty kernel; sink: at least `blocks` words.
extern "C" int awq_probe_empty(int64_t blocks, int threads, uint32_t* sink, hipStream_t stream) {
  if (sink == nullptr || blocks <= 0 || blocks >= (int64_t(1) << 31) || threads <= 0 || threads > 1024)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, sink, 0);
  return (int)hipGetLastError();
}
