// awq_dequant / awq_dequant_f16: packed AWQ GEMM weight -> float32 or fp16 [K, N].
//
// W[k, n] = (float)(q[k, n] - z[k / g, n]) * (float)s[k / g, n]
// (tensref.org "AWQ" format page, Reader; rule AWQ-005: the zero is subtracted as
// stored).  The product of a 4-bit difference and an fp16 scale is exact in fp32,
// so the float32 output is the unique correct bit pattern, and the fp16 output is
// that value rounded once to nearest even (the weight a dequantize-then-matmul path
// feeds to a dense fp16 GEMM: vLLM article, section 5.3).
//
// Bandwidth-bound: per packed word it reads 4 B of qweight (+ the group's zero word
// and 16 B of scales, mostly L2 hits) and writes 32 B (float32) or 16 B (fp16).  One
// thread per word, eight consecutive outputs written as 16-byte stores; consecutive
// threads own consecutive words of a row, so both loads and stores are coalesced.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

template <typename T>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint32_t* __restrict__ qzeros,
                                                      const _Float16* __restrict__ scales, int K,
                                                      int N, int g, T* __restrict__ out) {
  const int NW = N >> 3;
  const int64_t total = (int64_t)K * NW;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
  const int k = (int)(idx / NW);
  const int c = (int)(idx - (int64_t)k * NW);
  const int gi = k / g;
  const uint32_t w = qweight[idx];
  const uint32_t zw = qzeros[(int64_t)gi * NW + c];
  const u32x4 sv = *reinterpret_cast<const u32x4*>(scales + (int64_t)gi * N + 8 * c);
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = (int)((w >> (4 * nibble_of_col(j))) & 0xFu);
    const int z = (int)zero_code(zw, j);
    const uint32_t sbits = (sv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
    o[j] = (float)(q - z) * s;
  }
  if constexpr (sizeof(T) == 4) {
    float4* dst = reinterpret_cast<float4*>(out + (int64_t)k * N + 8 * c);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else {
    half8v h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)o[j];  // one rounding of the exact product
    *reinterpret_cast<half8v*>(out + (int64_t)k * N + 8 * c) = h;
  }
  }
}

hipError_t launch_dequant(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                          int K, int N, int g, void* out, bool f16, hipStream_t stream) {
  const int64_t words = (int64_t)K * (N / 8);
  int64_t blocks = (words + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond ~268M words
  const auto* qw = reinterpret_cast<const uint32_t*>(qweight);
  const auto* qz = reinterpret_cast<const uint32_t*>(qzeros);
  const auto* sc = reinterpret_cast<const _Float16*>(scales);
  if (f16)
    hipLaunchKernelGGL(dequant_kernel<_Float16>, dim3((unsigned)blocks), dim3(256), 0, stream, qw, qz, sc, K, N,
                       g, static_cast<_Float16*>(out));
  else
    hipLaunchKernelGGL(dequant_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, qw, qz, sc, K, N, g,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace awq
