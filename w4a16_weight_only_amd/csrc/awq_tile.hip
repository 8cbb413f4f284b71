// MFMA tile family of awq_gemm (large M): compute-bound.
//
// y = x . dequant(W) + bias with fp16 MFMA and fp32 accumulation (GPTQModel wiki
// "AWQ", section "Native GEMM": fp32 accumulation; GPU LLM serving-stack blog,
// section 1.2: large batches are compute-bound, so dequant work must hide under
// the matrix products).
//
// Workgroup tile 128 (M) x 128 (N), k-tile 32, 256 threads as 2 x 2 waves, each
// wave 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_f16.
// Per k-tile:
//   A: 128 x 32 fp16 of x staged into LDS (two 16-byte loads per thread).
//   B: 32 rows x 16 packed words; each thread takes two rows of one word column,
//      interleaves their bytes (v_perm_b32), expands each nibble pair to exact fp16
//      with the 0x6400 mantissa trick, subtracts the zero exactly, multiplies by the
//      fp16 scale (one rounding: fp16((q - z) s)) and writes the eight (k, k+1)
//      pairs of its eight columns to LDS in [n][k] order, un-permuting the AWQ
//      column order on the way.  Each weight is dequantised once per workgroup.
//   Waves read 16-byte A and B fragments from LDS and issue 2 k16 steps x 4 MFMAs.
// The next k-tile's global loads are issued before the current tile's MFMAs.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {
constexpr int LDK = kTileK + 8;  // padded LDS row (halves) to spread banks
}

__global__ __launch_bounds__(kTileThreads) void tile_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint32_t* __restrict__ qzeros, const _Float16* __restrict__ scales,
    const _Float16* __restrict__ bias, int M, int K, int N, int g, int n_tiles,
    _Float16* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) _Float16 As[kTileM][LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[kTileN][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile_n = blockIdx.x % n_tiles;
  const int tile_m = blockIdx.x / n_tiles;
  const int m0 = tile_m * kTileM, n0 = tile_n * kTileN;
  const int NW = N >> 3;
  const int wc0 = n0 >> 3;

  // Global -> register mapping.
  const int ar = tid >> 1, ap = (tid & 1) * 16;  // A: row, half offset
  const int bp = tid >> 4, bw = tid & 15;         // B: row pair, word column
  const bool a_ok = m0 + ar < M;
  const bool b_ok = wc0 + bw < NW;
  const _Float16* aptr = x + (int64_t)(m0 + ar) * K + ap;
  const uint32_t* bptr = qweight + (int64_t)(2 * bp) * NW + wc0 + bw;

  u32x4 areg0, areg1, sreg;
  uint32_t bra, brb, zreg;
  auto load = [&](int k0) {
    areg0 = areg1 = u32x4{0u, 0u, 0u, 0u};
    if (a_ok) {
      areg0 = *reinterpret_cast<const u32x4*>(aptr + k0);
      areg1 = *reinterpret_cast<const u32x4*>(aptr + k0 + 8);
    }
    bra = brb = zreg = 0u;
    sreg = u32x4{0u, 0u, 0u, 0u};
    if (b_ok) {
      const int gi = k0 / g;
      bra = bptr[(int64_t)k0 * NW];
      brb = bptr[(int64_t)(k0 + 1) * NW];
      zreg = qzeros[(int64_t)gi * NW + wc0 + bw];
      sreg = *reinterpret_cast<const u32x4*>(scales + (int64_t)gi * N + 8 * (wc0 + bw));
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const UnpackConsts uk = unpack_consts();
  load(0);
  for (int k0 = 0; k0 < K; k0 += kTileK) {
    __syncthreads();  // previous k-tile's fragments have been read
    *reinterpret_cast<u32x4*>(&As[ar][ap]) = areg0;
    *reinterpret_cast<u32x4*>(&As[ar][ap + 8]) = areg1;
    {
      uint32_t pb[4] = {pair_byte<0>(bra, brb), pair_byte<1>(bra, brb), pair_byte<2>(bra, brb),
                        pair_byte<3>(bra, brb)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int jl = lo_col(t), jh = hi_col(t);
        const _Float16 sl = __builtin_bit_cast(_Float16, (uint16_t)((sreg[jl >> 1] >> (16 * (jl & 1))) & 0xFFFFu));
        const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)((sreg[jh >> 1] >> (16 * (jh & 1))) & 0xFFFFu));
        const half2v zl = splat(-(_Float16)(float)(1024u + zero_code(zreg, jl)));
        const half2v zh = splat(-(_Float16)(float)(64u + zero_code(zreg, jh)));
        const half2v wl = lo_minus_zero(pb[t], zl, uk) * splat(sl);
        const half2v wh = hi_minus_zero(pb[t], zh, uk) * splat(sh);
        *reinterpret_cast<uint32_t*>(&Bs[8 * bw + jl][2 * bp]) = as_u32(wl);
        *reinterpret_cast<uint32_t*>(&Bs[8 * bw + jh][2 * bp]) = as_u32(wh);
      }
    }
    __syncthreads();
    if (k0 + kTileK < K) load(k0 + kTileK);

#pragma unroll
    for (int kk = 0; kk < kTileK; kk += 16) {
      const int kc = kk + 8 * (lane >> 5);
      half8v af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8v*>(&As[wm * 64 + i * 32 + (lane & 31)][kc]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8v*>(&Bs[wn * 64 + j * 32 + (lane & 31)][kc]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  32x32 MFMA output: lane l, register r holds row 8(r/4) + 4(l/32) + r%4,
  // column l%32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= N) continue;
    const float b = bias ? (float)bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) y[(int64_t)row * N + n] = (_Float16)(acc[i][j][r] + b);
      }
  }
}

hipError_t launch_tile(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                       const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                       uint16_t* y, hipStream_t stream) {
  const int n_tiles = (N + kTileN - 1) / kTileN;
  const int m_tiles = (M + kTileM - 1) / kTileM;
  const int64_t blocks = (int64_t)n_tiles * m_tiles;
  hipLaunchKernelGGL(tile_kernel, dim3((unsigned)blocks), dim3(kTileThreads), 0, stream,
                     reinterpret_cast<const _Float16*>(x), reinterpret_cast<const uint32_t*>(qweight),
                     reinterpret_cast<const uint32_t*>(qzeros), reinterpret_cast<const _Float16*>(scales),
                     reinterpret_cast<const _Float16*>(bias), M, K, N, g, n_tiles,
                     reinterpret_cast<_Float16*>(y));
  return hipGetLastError();
}

}  // namespace awq
