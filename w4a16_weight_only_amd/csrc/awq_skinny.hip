// Skinny family of awq_gemm (small M): bandwidth-bound streaming of the packed weight.
//
// What it computes: y[m, n] = sum_k x[m, k] * (q[k, n] - z[k/g, n]) * s[k/g, n] + bias[n]
// (tensref.org "AWQ" format page, Reader; GPU LLM serving-stack blog, section 1.2:
// small-batch decode is limited by weight bandwidth, so the packed weight is read
// once and expanded only in registers).
//
// Per workgroup (256 threads, 4 waves): 32 packed word-columns (256 output columns,
// 128 contiguous bytes of every qweight row) times a contiguous run of 32-row
// k-steps.  Each wave takes a contiguous sub-run of those k-steps.
//
// Per wave and k-step, on v_mfma_f32_16x16x32_f16 (x rows padded to 16):
//   lane l: q = l / 16 picks rows 8q..8q+7 of the k-step, c = l % 16 picks word
//   columns 2c, 2c+1 of the tile.  The lane loads 8 rows x 8 bytes (one 8-byte
//   load per row; 16 lanes cover 128 contiguous bytes of a row).
//   From each pair of rows, v_perm_b32 interleaves byte t of both words, and the
//   0x6400 mantissa trick turns each nibble pair into an exact fp16 pair
//   (code + 1024) or (16 code + 1024); one packed add / fma subtracts the zero,
//   leaving the exact integers (q - z) for rows (r, r+1) of one column.  Four such
//   pairs form the B operand (8 consecutive k of one column) of one MFMA.
//   Each lane's 16 columns give 16 MFMAs; lane c of the MFMA is column
//   8 (tile_wc + 2c + w) + j.  The A operand is x[m = l % 16][8q..8q+7].
//   Products fp16 x integer are exact in fp32; the MFMA sums in fp32.
// Groups: the MFMA accumulates sum_k x (q - z) per group in `part`; at the end of
// each group it is scaled by s (fp32) into `acc`.  Group boundaries fall on
// k-step boundaries (g % 32 == 0).
// Reduction: waves -> LDS (fixed order), then across the K splits of a column tile
// through a workspace: each workgroup stores its partial, the last to arrive (device
// counter) sums all splits in split order, adds bias, rounds once to fp16 and
// stores y, then resets the counter.  The result does not depend on timing.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {

struct WordPair {
  uint32_t w0, w1;
};

__device__ __forceinline__ WordPair load_pair(const uint32_t* p, bool ok) {
  if (!ok) return WordPair{0u, 0u};
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return WordPair{v.x, v.y};
}

__device__ __forceinline__ half8v pack4(half2v a, half2v b, half2v c, half2v d) {
  return half8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Run the 16 MFMAs of one k-step for one lane's 2 word-columns.
__device__ __forceinline__ void kstep_mfma(const WordPair (&v)[8], half8v a, const half2v (&zlo)[2][4],
                                           const half2v (&zhi)[2][4], floatx4 (&part)[2][8]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half2v lo[4], hi[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t ra = w ? v[2 * p].w1 : v[2 * p].w0;
        const uint32_t rb = w ? v[2 * p + 1].w1 : v[2 * p + 1].w0;
        uint32_t pb;
        if (t == 0) pb = pair_byte<0>(ra, rb);
        else if (t == 1) pb = pair_byte<1>(ra, rb);
        else if (t == 2) pb = pair_byte<2>(ra, rb);
        else pb = pair_byte<3>(ra, rb);
        lo[p] = lo_minus_zero(pb, zlo[w][t]);
        hi[p] = hi_minus_zero(pb, zhi[w][t]);
      }
      part[w][lo_col(t)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pack4(lo[0], lo[1], lo[2], lo[3]),
                                                                  part[w][lo_col(t)], 0, 0, 0);
      part[w][hi_col(t)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pack4(hi[0], hi[1], hi[2], hi[3]),
                                                                  part[w][hi_col(t)], 0, 0, 0);
    }
  }
}

}  // namespace

template <int MROWS>
__global__ __launch_bounds__(kSkinnyThreads) void skinny_kernel(
    const _Float16* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint32_t* __restrict__ qzeros, const _Float16* __restrict__ scales,
    const _Float16* __restrict__ bias, int M, int K, int N, int g, int splits,
    float* __restrict__ partial, uint32_t* __restrict__ counters, _Float16* __restrict__ y) {
  __shared__ float red[4][MROWS][kSkinnyCols];
  __shared__ int is_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int NW = N >> 3;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int wc = tile * kSkinnyWordCols + 2 * c;
  const bool col_ok = wc < NW;  // NW % 4 == 0, so wc + 1 < NW as well

  // k-steps of this workgroup, then of this wave (contiguous runs).
  const int T = K / kKStep;
  const int s0 = (int)((int64_t)T * split / splits);
  const int s1 = (int)((int64_t)T * (split + 1) / splits);
  const int L = s1 - s0;
  const int kb = s0 + (L * wave) / 4;
  const int ke = s0 + (L * (wave + 1)) / 4;

  const int m = lane & 15;
  const bool row_ok = m < M;
  const _Float16* xrow = x + (int64_t)m * K + 8 * q;
  const uint32_t* wbase = qweight + (int64_t)(8 * q) * NW + wc;

  floatx4 acc[2][8];
  floatx4 part[2][8];
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[w][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      part[w][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  half2v zlo[2][4], zhi[2][4];
  int cur_g = -1;

  auto flush = [&](int gi) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      u32x4 sv = u32x4{0u, 0u, 0u, 0u};
      if (col_ok) sv = *reinterpret_cast<const u32x4*>(scales + (int64_t)gi * N + 8 * (wc + w));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)((sv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
        acc[w][j] += s * part[w][j];
        part[w][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto load_zeros = [&](int gi) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t zw = col_ok ? qzeros[(int64_t)gi * NW + wc + w] : 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        zlo[w][t] = splat(-(_Float16)(float)(1024u + zero_code(zw, lo_col(t))));
        zhi[w][t] = splat(-(_Float16)(float)(64u + zero_code(zw, hi_col(t))));
      }
    }
  };

  WordPair v[8];
  half8v a = half8v{0, 0, 0, 0, 0, 0, 0, 0};
  if (kb < ke) {
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = load_pair(wbase + (int64_t)(kb * kKStep + r) * NW, col_ok);
    if (row_ok) a = *reinterpret_cast<const half8v*>(xrow + kb * kKStep);
  }
  for (int ks = kb; ks < ke; ++ks) {
    const int gi = (ks * kKStep) / g;
    if (gi != cur_g) {
      if (cur_g >= 0) flush(cur_g);
      load_zeros(gi);
      cur_g = gi;
    }
    // Issue the next k-step's loads before this step's arithmetic.
    WordPair vn[8];
    half8v an = half8v{0, 0, 0, 0, 0, 0, 0, 0};
    const bool more = ks + 1 < ke;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      vn[r] = load_pair(wbase + (int64_t)((ks + 1) * kKStep + r) * NW, col_ok && more);
    if (row_ok && more) an = *reinterpret_cast<const half8v*>(xrow + (ks + 1) * kKStep);

    kstep_mfma(v, a, zlo, zhi, part);

#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = vn[r];
    a = an;
  }
  if (cur_g >= 0) flush(cur_g);

  // Wave partials -> LDS.  MFMA 16x16 output: lane l holds rows 4(l/16)+i, column l%16.
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * q + i;
        if (row < MROWS) red[wave][row][8 * (2 * c + w) + j] = acc[w][j][i];
      }
  __syncthreads();

  const int t = threadIdx.x;  // output column within the tile
  const int n = tile * kSkinnyCols + t;
  const int rows = M < MROWS ? M : MROWS;
  if (splits == 1) {
    if (n < N) {
      const float b = bias ? (float)bias[n] : 0.f;
      for (int row = 0; row < rows; ++row) {
        const float s = ((red[0][row][t] + red[1][row][t]) + red[2][row][t]) + red[3][row][t];
        y[(int64_t)row * N + n] = (_Float16)(s + b);
      }
    }
    return;
  }

  float* my_part = partial + ((int64_t)tile * splits + split) * MROWS * kSkinnyCols;
  for (int row = 0; row < rows; ++row)
    my_part[row * kSkinnyCols + t] = ((red[0][row][t] + red[1][row][t]) + red[2][row][t]) + red[3][row][t];

  // Publish the partial device-wide, then count arrivals for this column tile.
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Last arrival: sum the splits in split order (deterministic), add bias, round once.
  if (n < N) {
    const float b = bias ? (float)bias[n] : 0.f;
    const float* base = partial + (int64_t)tile * splits * MROWS * kSkinnyCols;
    for (int row = 0; row < rows; ++row) {
      float s = 0.f;
      for (int sp = 0; sp < splits; ++sp)
        s += __builtin_nontemporal_load(base + ((int64_t)sp * MROWS + row) * kSkinnyCols + t);
      y[(int64_t)row * N + n] = (_Float16)(s + b);
    }
  }
  if (t == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_skinny(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                         const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                         int splits, float* partial, uint32_t* counters, uint16_t* y,
                         hipStream_t stream) {
  const int n_tiles = (N + kSkinnyCols - 1) / kSkinnyCols;
  const dim3 grid(n_tiles, splits);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kSkinnyThreads), 0, stream,
                       reinterpret_cast<const _Float16*>(x), reinterpret_cast<const uint32_t*>(qweight),
                       reinterpret_cast<const uint32_t*>(qzeros), reinterpret_cast<const _Float16*>(scales),
                       reinterpret_cast<const _Float16*>(bias), M, K, N, g, splits, partial, counters,
                       reinterpret_cast<_Float16*>(y));
  };
  if (M <= 4) args(skinny_kernel<4>);
  else args(skinny_kernel<16>);
  return hipGetLastError();
}

}  // namespace awq
