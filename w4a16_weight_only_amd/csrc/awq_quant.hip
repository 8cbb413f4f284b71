// awq_quantize_rtn: fp16 weight [K, N] -> AWQ GEMM pack (qweight, qzeros, scales).
//
// Round-to-nearest group quantization (GPTQModel wiki "AWQ", section "Group
// quantization and zero points"), per group of g input rows and per column n:
//   asymmetric: s = fp16(max(max - min, 1e-5) / 15), z = clamp(-rint(min / s), 0, 15),
//               q = clamp(rint(w / s) + z, 0, 15)
//   symmetric:  s = fp16(max(max |w|, 1e-5) / 7),   z = 8,
//               q = clamp(rint(w / s), -8, 7) + 8 = clamp(rint(w / s) + 8, 0, 15)
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
// registers, reduced to the per-column min and max (packed fp16, exact: the inputs
// are fp16), across lanes by shuffles and across waves through LDS, and coded from
// the registers.  Small workgroups let several groups share a CU at different
// phases, so one group's coding overlaps another's loads.  Groups longer than the
// register cache are read a second time for the coding pass.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {

// Packed fp16 min / max.  The NaN-propagating forms need no canonicalising of
// their inputs (the inputs are finite), and chains of two fold into gfx950's
// three-operand v_pk_minimum3_f16 / v_pk_maximum3_f16.  They order -0 below +0,
// which changes no output: a zero min or max only enters max(range, 1e-5),
// max(|w|, 1e-5) and a zero point rounded from +-0.
__device__ __forceinline__ half2v hmin2(half2v a, half2v b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ half2v hmax2(half2v a, half2v b) { return __builtin_elementwise_maximum(a, b); }

// Per-thread running min / max of 8 columns as 4 packed fp16 pairs (column pairs
// (0,1), (2,3), (4,5), (6,7) of the 16-byte row chunk).
struct PairStats {
  half2v mn[4], mx[4];
};

__device__ __forceinline__ void accumulate(PairStats& st, const u32x4& v) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    st.mn[p] = hmin2(st.mn[p], as_h2(v[p]));
    st.mx[p] = hmax2(st.mx[p], as_h2(v[p]));
  }
}

__device__ __forceinline__ void accumulate2(PairStats& st, const u32x4& v, const u32x4& u) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    st.mn[p] = hmin2(hmin2(st.mn[p], as_h2(v[p])), as_h2(u[p]));
    st.mx[p] = hmax2(hmax2(st.mx[p], as_h2(v[p])), as_h2(u[p]));
  }
}

__device__ __forceinline__ float col_of(const u32x4& v, int j) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
}

// Codes of one row (8 columns) packed into one word.  q = rint(fl32(w / s)) needs
// the division rounded as IEEE fp32 division.
//
// Fast path.  With P = w * rcp(s) (exact product): v_rcp_f32 is within 1 ulp, so P
// is within about 1.5 * 2^-23 |w / s| of w / s, and fl32(w / s) within 2^-24 |w / s|:
// together less than 2^-18 while |w / s| < 16.  One fma, x = fl32(P + (M + z)) with
// M = 1.5 * 2^23, rounds P + z to an integer held in the low mantissa bits of x
// (values in [2^23, 2^24) are spaced 1 apart); the clamp to [M, M + 15] and
// bits(x) - bits(M) then give the code.  A second fma measures d = P - (x - M - z).
// If |d| < 1/2 - 2^-16, P is not near a half-integer, so x - M - z = rint(P) =
// rint(w / s) = rint(fl32(w / s)).  If |w / s| >= 16, both the fast and the exact
// value of rint(w / s) + z lie beyond the clamp range on the same side (z is in
// 0..15; x is monotone in P), so the clamped code agrees whatever d is.  A row in
// which some |d| reaches 1/2 - 2^-16 (ties included) is flagged, and the caller
// redoes it with correctly rounded divisions (code_word_exact).  zf holds z (8
// when symmetric), mzf holds M + z.
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

__device__ __forceinline__ uint32_t code_word_exact(const u32x4& v, const float sf[8], const float zf[8]) {
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = __builtin_amdgcn_fmed3f(rintf(col_of(v, j) / sf[j]) + zf[j], 0.0f, 15.0f);
    word |= (uint32_t)q << (4 * nibble_of_col(j));
  }
  return word;
}

__device__ __forceinline__ uint32_t code_word_fast(const u32x4& v, const float rf[8], const float mzf[8],
                                                   bool& near) {
  uint32_t word = 0;
  float dmax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float wj = col_of(v, j);
    const float x = __builtin_fmaf(wj, rf[j], mzf[j]);
    const float d = __builtin_fmaf(wj, rf[j], mzf[j] - x);
    dmax = fmaxf(dmax, fabsf(d));
    const float y = __builtin_amdgcn_fmed3f(x, kMagic, kMagic + 15.0f);
    word |= (__builtin_bit_cast(uint32_t, y) - kMagicBits) << (4 * nibble_of_col(j));
  }
  near = dmax >= 0.5f - 0x1p-16f;
  return word;
}

}  // namespace

// Work item = (span of rows, block of CL word columns).  A span is a whole group
// (kFused) or one chunk of up to S * CACHE rows of a group (kStats, kCode; cpg
// chunks per group).  Workgroup b takes item b / ncb and word columns
// (b % ncb) * CL .. + CL - 1; CACHE rows per thread stay in registers.
//   kFused  min / max of the group, then scales, zeros and codes: one pass.
//   kStats  min / max of the chunk, stored to part (packed fp16, 2 x 16 bytes per
//           word column and chunk: part[(item * 2 + {0: min, 1: max}) * N8 + c]).
//   kCode   min / max of the group from its chunks' part entries, then scales and
//           zeros (first chunk only) and the chunk's codes.
enum RtnMode { kFused = 0, kStats = 1, kCode = 2 };

template <int CL, int WAVES, int CACHE, int MODE>
__global__ __launch_bounds__(64 * WAVES) void rtn_kernel(const u32x4* __restrict__ w, int N8, int g, int cpg,
                                                        int ncb, int sym, uint32_t* __restrict__ qweight,
                                                        uint32_t* __restrict__ qzeros, u32x4* __restrict__ scales,
                                                        u32x4* __restrict__ part) {
  constexpr int RL = 64 / CL;     // row slices per wave
  constexpr int S = WAVES * RL;   // row slices per workgroup
  constexpr int CH = S * CACHE;   // rows per chunk (kStats, kCode)
  __shared__ u32x4 red[2][WAVES][CL];  // per-wave min / max, packed fp16

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = lane % CL;
  const int slice = wave * RL + lane / CL;
  const int item = blockIdx.x / ncb;
  const int grp = item / cpg;
  const int chunk = item - grp * cpg;
  const int c = (blockIdx.x % ncb) * CL + cl;
  const bool cvalid = c < N8;
  const int rows = MODE == kFused ? g : min(CH, g - chunk * CH);  // 1 <= rows <= S * CACHE
  const int64_t row0 = (int64_t)grp * g + (int64_t)chunk * CH;

  // Loads are unconditional so that they issue back to back (a load under a branch
  // waits for the previous one): a row index past the span is clamped to the
  // span's last row, whose repeat leaves min and max unchanged, and a column past
  // N to the last column, whose lanes never store.
  const int cc = cvalid ? c : N8 - 1;
  u32x4 buf[CACHE];
#pragma unroll
  for (int i = 0; i < CACHE; ++i) buf[i] = w[(row0 + min(slice + S * i, rows - 1)) * N8 + cc];

  u32x4 mnw, mxw;
  if constexpr (MODE == kCode) {
    const _Float16 inf = (_Float16)__builtin_inff();
    const uint32_t pinf = as_u32(half2v{inf, inf}), ninf = as_u32(half2v{-inf, -inf});
    mnw = u32x4{pinf, pinf, pinf, pinf};
    mxw = u32x4{ninf, ninf, ninf, ninf};
    const u32x4* pg = part + (int64_t)grp * cpg * 2 * N8 + cc;
    for (int k = 0; k < cpg; ++k) {
      const u32x4 a = pg[(int64_t)(2 * k) * N8], b = pg[(int64_t)(2 * k + 1) * N8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        mnw[p] = as_u32(hmin2(as_h2(mnw[p]), as_h2(a[p])));
        mxw[p] = as_u32(hmax2(as_h2(mxw[p]), as_h2(b[p])));
      }
    }
  } else {
    PairStats st;
    const _Float16 inf = (_Float16)__builtin_inff();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      st.mn[p] = half2v{inf, inf};
      st.mx[p] = half2v{-inf, -inf};
    }
#pragma unroll
    for (int i = 0; i + 1 < CACHE; i += 2) accumulate2(st, buf[i], buf[i + 1]);
    if constexpr (CACHE % 2 == 1) accumulate(st, buf[CACHE - 1]);

    // Min / max across the row slices of a wave (lanes cl, cl + CL, ...), then across waves.
#pragma unroll
    for (int off = CL; off < 64; off <<= 1) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        st.mn[p] = hmin2(st.mn[p], as_h2(__shfl_xor(as_u32(st.mn[p]), off)));
        st.mx[p] = hmax2(st.mx[p], as_h2(__shfl_xor(as_u32(st.mx[p]), off)));
      }
    }
    if (lane < CL) {
      red[0][wave][cl] = u32x4{as_u32(st.mn[0]), as_u32(st.mn[1]), as_u32(st.mn[2]), as_u32(st.mn[3])};
      red[1][wave][cl] = u32x4{as_u32(st.mx[0]), as_u32(st.mx[1]), as_u32(st.mx[2]), as_u32(st.mx[3])};
    }
    __syncthreads();
    mnw = red[0][0][cl];
    mxw = red[1][0][cl];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) {
      const u32x4 a = red[0][v][cl], b = red[1][v][cl];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        mnw[p] = as_u32(hmin2(as_h2(mnw[p]), as_h2(a[p])));
        mxw[p] = as_u32(hmax2(as_h2(mxw[p]), as_h2(b[p])));
      }
    }
  }
  if (!cvalid) return;
  if constexpr (MODE == kStats) {
    if (slice == 0) {
      part[(int64_t)(2 * item) * N8 + c] = mnw;
      part[(int64_t)(2 * item + 1) * N8 + c] = mxw;
    }
    return;
  }

  float sf[8], rf[8], zf[8], mzf[8];
  uint32_t zword = 0;
  u32x4 sbits;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float mn = col_of(mnw, j), mx = col_of(mxw, j);
    const float s32 = sym ? fmaxf(fmaxf(mx, -mn), 1e-5f) / 7.0f : fmaxf(mx - mn, 1e-5f) / 15.0f;
    const _Float16 s16 = (_Float16)s32;  // the stored scale, rounded once
    sf[j] = (float)s16;
    rf[j] = __builtin_amdgcn_rcpf(sf[j]);
    zf[j] = sym ? 8.0f : __builtin_amdgcn_fmed3f(-rintf(mn / sf[j]), 0.0f, 15.0f);
    mzf[j] = kMagic + zf[j];
    zword |= (uint32_t)zf[j] << (4 * nibble_of_col(j));
    const uint32_t b = __builtin_bit_cast(uint16_t, s16);
    if (j & 1) sbits[j >> 1] |= b << 16;
    else sbits[j >> 1] = b;
  }
  if (slice == 0 && chunk == 0) {
    qzeros[(int64_t)grp * N8 + c] = zword;
    scales[(int64_t)grp * N8 + c] = sbits;
  }

  uint32_t redo = 0;  // rows i whose fast codes must be recomputed exactly
#pragma unroll
  for (int i = 0; i < CACHE; ++i) {
    const int r = slice + S * i;
    bool near = false;
    const uint32_t word = code_word_fast(buf[i], rf, mzf, near);
    if (r < rows) {
      qweight[(row0 + r) * N8 + c] = word;
      redo |= (uint32_t)near << i;
    }
  }
  // Rare: the row is read again (an L2 hit) so that buf needs no runtime index;
  // the exact word overwrites the fast one written above by this same thread.
  while (redo) {
    const int i = __builtin_ctz(redo);
    redo &= redo - 1;
    const int64_t idx = (row0 + slice + S * i) * N8 + c;
    qweight[idx] = code_word_exact(w[idx], sf, zf);
  }
}

namespace {
constexpr int kCL = kRtnWordCols, kWaves = kRtnWaves;
constexpr int kChunkCache = kRtnChunkCache;
}  // namespace

hipError_t launch_quantize_rtn(const uint16_t* w, int K, int N, int g, bool sym, int32_t* qweight,
                               int32_t* qzeros, uint16_t* scales, void* scratch, hipStream_t stream) {
  const RtnPlan p = rtn_plan(K, N, g);
  const int N8 = N / 8;
  const int ncb = (N + p.cols - 1) / p.cols;
  const dim3 grid((unsigned)p.grid), block(p.block);
  const auto* src = reinterpret_cast<const u32x4*>(w);
  auto* qw = reinterpret_cast<uint32_t*>(qweight);
  auto* qz = reinterpret_cast<uint32_t*>(qzeros);
  auto* sc = reinterpret_cast<u32x4*>(scales);
  auto* part = static_cast<u32x4*>(scratch);
  const int sy = sym ? 1 : 0;
  if (p.two_pass) {
    hipLaunchKernelGGL((rtn_kernel<kCL, kWaves, kChunkCache, kStats>), grid, block, 0, stream, src, N8, g, p.cpg,
                       ncb, sy, qw, qz, sc, part);
    hipLaunchKernelGGL((rtn_kernel<kCL, kWaves, kChunkCache, kCode>), grid, block, 0, stream, src, N8, g, p.cpg,
                       ncb, sy, qw, qz, sc, part);
    return hipGetLastError();
  }
  switch (p.cache) {
#define AWQ_RTN_FUSED(C)                                                                                    \
  case C:                                                                                                   \
    hipLaunchKernelGGL((rtn_kernel<kCL, kWaves, C, kFused>), grid, block, 0, stream, src, N8, g, 1, ncb, sy, \
                       qw, qz, sc, part);                                                                   \
    break;
    AWQ_RTN_FUSED(1)
    AWQ_RTN_FUSED(2)
    AWQ_RTN_FUSED(4)
    AWQ_RTN_FUSED(8)
    AWQ_RTN_FUSED(16)
#undef AWQ_RTN_FUSED
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace awq
