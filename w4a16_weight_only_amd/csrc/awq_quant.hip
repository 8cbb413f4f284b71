// awq_quantize_rtn: fp16 weight [K, N] -> AWQ GEMM pack (qweight, qzeros, scales).
//
// Round-to-nearest group quantization (GPTQModel wiki "AWQ", section "Group
// quantization and zero points"), per group of g input rows and per column n:
//   asymmetric: s = fp16(max(max - min, 1e-5) / 15), z = clamp(-rint(min / s), 0, 15),
//               q = clamp(rint(w / s) + z, 0, 15)
//   symmetric:  s = fp16(max(max |w|, 1e-5) / 7),   z = 8,
//               q = clamp(rint(w / s), -8, 7) + 8
// The scale is computed in fp32 and rounded once to the stored fp16 value; every
// later division uses that stored value, in fp32, correctly rounded, and rint rounds
// half to even.  Codes are packed with nibble i of word c holding column
// 8c + ORDER[i], ORDER = {0,2,4,6,1,3,5,7} (tensref.org "AWQ" format page, Reader).
//
// Bandwidth-bound: 2 bytes read per weight, half a byte written, plus 2.5 bytes per
// (group, column) for scales and zeros.  Thread layout: a thread owns one packed
// word column c (8 weights wide) and a strided slice of the group's rows; the
// lanes of a wave cover CL adjacent word columns and 64 / CL row slices, so every
// row load is a contiguous 16*CL-byte run.  The rows of a group are read once into
// registers, reduced to the per-column min and max (lane shuffles, then LDS across
// the waves), and coded from the registers; groups longer than the register cache
// are read a second time for the coding pass.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {

struct ColStats {
  float mn[8], mx[8];
};

__device__ __forceinline__ void unpack8(const u32x4& v, float f[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    f[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
}

__device__ __forceinline__ void accumulate(ColStats& st, const u32x4& v) {
  float f[8];
  unpack8(v, f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    st.mn[j] = fminf(st.mn[j], f[j]);
    st.mx[j] = fmaxf(st.mx[j], f[j]);
  }
}

// Codes of one row (8 columns) packed into one word.
__device__ __forceinline__ uint32_t code_word(const u32x4& v, const float sf[8], const float zf[8], bool sym) {
  float f[8];
  unpack8(v, f);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = rintf(f[j] / sf[j]);
    const float q = sym ? fminf(fmaxf(r, -8.0f), 7.0f) + 8.0f : fminf(fmaxf(r + zf[j], 0.0f), 15.0f);
    word |= (uint32_t)(int)q << (4 * nibble_of_col(j));
  }
  return word;
}

}  // namespace

// CL word columns per wave, WAVES waves per workgroup, CACHE rows kept in registers
// per thread.  Workgroup b handles group b / ncb and word columns
// (b % ncb) * CL .. + CL - 1.
template <int CL, int WAVES, int CACHE>
__global__ __launch_bounds__(64 * WAVES) void rtn_kernel(const u32x4* __restrict__ w, int K, int N8, int g,
                                                        int ncb, int sym, uint32_t* __restrict__ qweight,
                                                        uint32_t* __restrict__ qzeros,
                                                        u32x4* __restrict__ scales) {
  constexpr int RL = 64 / CL;     // row slices per wave
  constexpr int S = WAVES * RL;   // row slices per workgroup
  __shared__ float red[2][WAVES][CL][8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = lane % CL;
  const int slice = wave * RL + lane / CL;
  const int grp = blockIdx.x / ncb;
  const int c = (blockIdx.x % ncb) * CL + cl;
  const bool cvalid = c < N8;
  const int64_t row0 = (int64_t)grp * g;
  const bool resident = g <= S * CACHE;

  ColStats st;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    st.mn[j] = __builtin_inff();
    st.mx[j] = -__builtin_inff();
  }
  u32x4 buf[CACHE];
  for (int base = slice; base < g; base += S * CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      const int r = base + S * i;
      if (cvalid && r < g) buf[i] = w[(row0 + r) * N8 + c];
    }
#pragma unroll
    for (int i = 0; i < CACHE; ++i)
      if (cvalid && base + S * i < g) accumulate(st, buf[i]);
  }

  // Min / max across the row slices of a wave (lanes cl, cl + CL, ...), then across waves.
#pragma unroll
  for (int off = CL; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st.mn[j] = fminf(st.mn[j], __shfl_xor(st.mn[j], off));
      st.mx[j] = fmaxf(st.mx[j], __shfl_xor(st.mx[j], off));
    }
  }
  if (lane < CL) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      red[0][wave][cl][j] = st.mn[j];
      red[1][wave][cl][j] = st.mx[j];
    }
  }
  __syncthreads();
  float mn[8], mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mn[j] = red[0][0][cl][j];
    mx[j] = red[1][0][cl][j];
  }
#pragma unroll
  for (int v = 1; v < WAVES; ++v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mn[j] = fminf(mn[j], red[0][v][cl][j]);
      mx[j] = fmaxf(mx[j], red[1][v][cl][j]);
    }
  }
  if (!cvalid) return;

  float sf[8], zf[8];
  uint32_t zword = 0;
  u32x4 sbits;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s32;
    if (sym) {
      s32 = fmaxf(fmaxf(mx[j], -mn[j]), 1e-5f) / 7.0f;
    } else {
      s32 = fmaxf(mx[j] - mn[j], 1e-5f) / 15.0f;
    }
    const _Float16 s16 = (_Float16)s32;  // the stored scale, rounded once
    sf[j] = (float)s16;
    zf[j] = sym ? 8.0f : fminf(fmaxf(-rintf(mn[j] / sf[j]), 0.0f), 15.0f);
    zword |= (uint32_t)(int)zf[j] << (4 * nibble_of_col(j));
    const uint32_t b = __builtin_bit_cast(uint16_t, s16);
    if (j & 1) sbits[j >> 1] |= b << 16;
    else sbits[j >> 1] = b;
  }
  if (slice == 0) {
    qzeros[(int64_t)grp * N8 + c] = zword;
    scales[(int64_t)grp * N8 + c] = sbits;
  }

  const bool s = sym != 0;
  if (resident) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      const int r = slice + S * i;
      if (r < g) qweight[(row0 + r) * N8 + c] = code_word(buf[i], sf, zf, s);
    }
  } else {
    for (int r = slice; r < g; r += S) qweight[(row0 + r) * N8 + c] = code_word(w[(row0 + r) * N8 + c], sf, zf, s);
  }
}

namespace {
constexpr int kSmallCL = 64, kSmallWaves = 4, kSmallCache = 32;  // groups of up to 128 rows
constexpr int kLargeCL = 8, kLargeWaves = 8, kLargeCache = 16;   // resident up to 1024 rows
}  // namespace

int rtn_plan(int g, int N, int* block, int* cols_per_block) {
  const bool small = g <= kSmallWaves * (64 / kSmallCL) * kSmallCache;
  *block = 64 * (small ? kSmallWaves : kLargeWaves);
  *cols_per_block = 8 * (small ? kSmallCL : kLargeCL);
  (void)N;
  return small ? 0 : 1;
}

hipError_t launch_quantize_rtn(const uint16_t* w, int K, int N, int g, bool sym, int32_t* qweight,
                               int32_t* qzeros, uint16_t* scales, hipStream_t stream) {
  int block, cols;
  const int variant = rtn_plan(g, N, &block, &cols);
  const int N8 = N / 8;
  const int ncb = (N + cols - 1) / cols;
  const int64_t blocks = (int64_t)(K / g) * ncb;
  const auto* src = reinterpret_cast<const u32x4*>(w);
  auto* qw = reinterpret_cast<uint32_t*>(qweight);
  auto* qz = reinterpret_cast<uint32_t*>(qzeros);
  auto* sc = reinterpret_cast<u32x4*>(scales);
  if (variant == 0)
    hipLaunchKernelGGL((rtn_kernel<kSmallCL, kSmallWaves, kSmallCache>), dim3((unsigned)blocks), dim3(block), 0,
                       stream, src, K, N8, g, ncb, (int)sym, qw, qz, sc);
  else
    hipLaunchKernelGGL((rtn_kernel<kLargeCL, kLargeWaves, kLargeCache>), dim3((unsigned)blocks), dim3(block), 0,
                       stream, src, K, N8, g, ncb, (int)sym, qw, qz, sc);
  return hipGetLastError();
}

}  // namespace awq
