// Decode family of awq_gemm (fp16 activations, 1 <= M <= 4): bandwidth-bound streaming
// of the packed weight.
//
// What it computes: y[m, n] = sum_k x[m, k] * (q[k, n] - z[k/g, n]) * s[k/g, n] + bias[n]
// (tensref.org "AWQ" format page, Reader; GPU LLM serving-stack blog, section 1.2:
// small-batch decode is limited by weight bandwidth, so the packed weight is read once,
// expanded only in registers, and the arithmetic hides under the stream).
//
// Work split.  A workgroup of WAVES waves owns a column tile of 64 packed word-columns
// (256 contiguous bytes of every qweight row, 512 output columns), or 32 (HALF: 128
// bytes, 256 columns), and WAVES * KS k-steps of 32 rows; wave w takes KS consecutive
// k-steps, all in one quantization group (the host guarantees it).  The K splits of a
// tile meet in 64-bit fixed-point accumulators (awq_device.h): one returning atomic per
// output element and split, and the add that completes an element writes y.
//
// Per wave and k-step, on v_mfma_f32_16x16x16_f16 (x rows padded to 16), for full tiles:
//   lane l: c = l % 16 picks the 16-byte chunk (words 4c .. 4c+3) of the tile's 256-byte
//   row segment, q = l / 16 picks rows 8q .. 8q+7 of the k-step; one 16-byte load per
//   row (16 lanes cover a row's 256 bytes, one wave instruction covers 4 rows).  Every
//   load of the wave is requested before any arithmetic.  From each pair of rows,
//   v_perm_b32 interleaves byte t of both words, the 0x6400 mantissa trick makes each
//   nibble pair an exact fp16 pair (1024 + code, or 1024 + 16 code), and one packed add
//   (or fma by 1/16) with the column's -(1024 + z) (or -(64 + z)) leaves the exact
//   integers (q - z) of rows (r, r + 1).  Two pairs are one B operand: 4 consecutive k
//   of one column, rows 8q .. 8q+3 or 8q+4 .. 8q+7 (the two halves of the k-step).  The
//   32 (word, byte, nibble) choices of the lane's chunk give 32 MFMAs per half; MFMA
//   column c is chunk c.  The A operand is x[m = l % 16][8q .. 8q+7] of the k-step, one
//   contiguous 16-byte load.  fp16 x times a small integer is
//   exact in fp32 and the MFMA accumulates in fp32; the wave's group sum is then scaled
//   by s in fp32, so the weight is never rounded.
// HALF tiles: lane l takes chunk l % 8 of the 128-byte segment and only nibble half
// (l / 8) % 2 of each byte, so MFMA column l % 16 is (nibble half, chunk) and a k-step is
// 16 MFMAs.  Lanes l and l ^ 8 load the two rows of each row pair (every 16-byte chunk is
// loaded once) and trade words with a DPP row rotation, so each holds both rows.
// Reduction: the waves' sums meet in LDS (only the live rows of each MFMA entry, in
// rounds), each thread sums a few (row block, column) entries over the waves in wave
// order, then adds them to the fixed-point words.
#include <type_traits>

#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {

constexpr int kDppRowRor8 = 0x128;  // DPP row_ror:8: lane l reads lane l ^ 8 of its 16-lane row

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Column within a word of MFMA entry u = 2 t + h (byte t, nibble h of the byte).
__device__ __forceinline__ constexpr int entry_col(int u) { return (u & 1) ? hi_col(u >> 1) : lo_col(u >> 1); }

// Column within the tile of MFMA entry v in lane l (output column l % 16 of the MFMA).
template <bool HALF>
__device__ __forceinline__ int out_col(int v, int l) {
  if constexpr (HALF) {
    const int c = l & 7, h = (l >> 3) & 1, t = v & 3;
    return 8 * (4 * c + (v >> 2)) + (h ? hi_col(t) : lo_col(t));
  } else {
    return 8 * (4 * (l & 15) + (v >> 3)) + entry_col(v & 7);
  }
}

// Byte t of each 16-bit half of a word, replicated: [b.t, 0, b.t, 0].
template <int t>
__device__ __forceinline__ uint32_t splat_byte(uint32_t b) {
  return pair_byte<t>(b, b);
}

}  // namespace

// MP: rows padded to 1, 2, 4, 8 or 16; KS: k-steps per wave; WAVES: 4 or 8 waves per
// workgroup (two waves per SIMD either way).  LG: how the group scales are applied.
// LG = 0: each wave scales its own sums (the 32 scales of its lane's chunk, 64 bytes per
// lane).  LG = 1, 2, 4: the workgroup's waves form LG equal parts, each inside one
// quantization group; the wave reduction sums each part apart and scales it once (LG
// 2-byte scales per output entry).
// HALF: a column tile of 32 word-columns (256 outputs, 128 bytes of a row): lane l
// takes chunk c = l % 8 and nibble half h = (l / 8) % 2 of every byte (MFMA column
// l % 16 is the pair (h, c)), the two lanes of a chunk load one row each of every row
// pair and trade words, and a k-step is 16 MFMAs (word w, byte t) instead of 32.  Half the columns per workgroup
// means half the K splits for the same grid, so half the fixed-point adds, and half
// as many of them meet at each address.
template <int MP, int KS, int WAVES, int LG, bool HALF = false>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void decode_kernel(const uint16_t* __restrict__ x,
                                                        const uint32_t* __restrict__ qweight,
                                                        const uint32_t* __restrict__ qzeros,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ bias, int M, int K, int N,
                                                        int g, int splits, uint64_t* __restrict__ accum,
                                                        float* __restrict__ side, uint16_t* __restrict__ y) {
  // MFMA output: lane l holds rows 4 (l / 16) .. +3 of column l % 16, so rows < MP live
  // in the first LIVE lanes, RREG registers each.
  constexpr int LIVE = MP <= 4 ? 16 : 16 * (MP / 4);
  constexpr int RREG = MP < 4 ? MP : 4;
  constexpr int THREADS = 64 * WAVES;
  constexpr int WORDS = HALF ? kDecodeWords / 2 : kDecodeWords;  // packed words of a column tile
  constexpr int COLS = 8 * WORDS;
  constexpr int NV = HALF ? 16 : 32;     // MFMA entries (accumulators) per k-step
  constexpr int ROUNDS = LIVE / 16;      // LDS rounds of the wave reduction
  constexpr int VR = NV / ROUNDS;        // MFMA entries per round
  constexpr int PAIRS = VR * LIVE;       // (entry, lane) pairs per round: the tile's columns
  constexpr int EPR = PAIRS / THREADS;   // reduced pairs per thread and round
  constexpr int EPT = EPR * ROUNDS;      // reduced pairs per thread
  static_assert(PAIRS == COLS && EPR * THREADS == PAIRS, "one round is one (entry, lane) pair per column");
  __shared__ float red[WAVES][VR][LIVE][RREG];  // only the live rows of each entry

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = HALF ? (lane & 7) : (lane & 15);
  const int hsel = HALF ? ((lane >> 3) & 1) : 0;  // HALF: this lane's nibble of each byte
  const int q = lane >> 4;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int NW = N >> 3;
  const int T = K >> 5;
  // Lanes of a partial last tile read the last valid chunk (N % 32 == 0, so NW % 4 == 0)
  // and never store.
  const int wc_raw = tile * WORDS + 4 * c;
  const int wc = wc_raw < NW ? wc_raw : NW - 4;
  const int kb = (split * WAVES + wave) * KS;  // first k-step of this wave
  const int nks = min(max(T - kb, 0), KS);      // k-steps this wave multiplies (uniform)
  const int gi = (min(kb, T - 1) * kKStep) / g;  // the wave's group

  // ---- Loads, in the order they are consumed.
  const u32x4 zw = *reinterpret_cast<const u32x4*>(qzeros + (int64_t)gi * NW + wc);
  const int xr = c < M ? c : M - 1;  // A row; rows >= M are copies, never stored
  half8v a[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ks = min(kb + s, T - 1);
    a[s] = *reinterpret_cast<const half8v*>(x + (int64_t)xr * K + ks * kKStep + 8 * q);
  }
  // Packed weights: buffer loads, one VGPR offset per lane, the row in a scalar offset.
  const uint32_t row_bytes = (uint32_t)NW * 4u;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(qweight), (short)0, (int)(row_bytes * (uint32_t)K), 0x00020000);
  // Full tiles: rows 8q + j, j = 0..7.  HALF: rows 8q + 2j + hsel, j = 0..3 (lanes l and
  // l ^ 8 take the two rows of each pair; every 16-byte chunk is loaded once).
  constexpr int LPS = HALF ? 4 : 8;  // weight loads per lane and k-step
  const uint32_t voff = ((uint32_t)(8 * q + hsel) * (uint32_t)NW + (uint32_t)wc) * 4u;
  u32x4 wv[KS][LPS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t r0 = (uint32_t)min(kb + s, T - 1) * kKStep;
#pragma unroll
    for (int j = 0; j < LPS; ++j)
      wv[s][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, voff, (r0 + (HALF ? 2 * j : j)) * row_bytes, 2));
  }
  // Scales of the lane's 32 columns (8 wc .. 8 wc + 31), when each wave scales its own sums.
  constexpr bool LATE = LG > 0;
  static_assert(LG == 0 || LG == 1 || (LG == 2 && WAVES % 2 == 0) || (LG == 4 && WAVES % 4 == 0), "parts");
  u32x4 sv[LATE ? 1 : 4];
  if constexpr (!LATE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = *reinterpret_cast<const u32x4*>(scales + (int64_t)gi * N + 8 * wc + 8 * i);
  }
  // This thread's epilogue entries: bias prefetch, branch-free (a load under a per-lane
  // branch would be waited for before the weight loads go out).  Entry k: round k / EPR,
  // pair index tid + THREADS (k % EPR) of the round = (MFMA entry v, lane l).  Without a
  // bias every lane reads x[0] and selects 0.
  const bool has_bias = bias != nullptr;
  const uint16_t* bsrc = has_bias ? bias : x;
  // The group of each part of the waves (a part past K reads the last group; its sums
  // are zero).
  constexpr int LGN = LG > 0 ? LG : 1;
  int gpart[LGN];
#pragma unroll
  for (int j = 0; j < LGN; ++j) gpart[j] = (min((split * WAVES + j * (WAVES / LGN)) * KS, T - 1) * kKStep) / g;
  uint16_t braw[EPT], sraw[LGN][EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int le = tid + THREADS * (k % EPR);
    const int v = (k / EPR) * VR + le / LIVE, l = le % LIVE;
    const int n = min(tile * COLS + out_col<HALF>(v, l), N - 1);
    braw[k] = bsrc[has_bias ? n : 0];
    if constexpr (LATE) {
#pragma unroll
      for (int j = 0; j < LG; ++j) sraw[j][k] = scales[(int64_t)gpart[j] * N + n];
    }
  }
  // Every load is issued before any arithmetic waits on one.
  __builtin_amdgcn_sched_barrier(0);
  // The kernel arguments past the preloaded ones are fetched here, under the loads, not
  // when the split sum first needs them.
  asm volatile("" ::"s"(splits), "s"(accum), "s"(side), "s"(y));

  // ---- Zero splats of the group: entry v = 8 w + 2 t + h holds -(1024 + z) (h = 0) or
  // -(64 + z) (h = 1) in both fp16 halves.
  // HALF: entry v = 4 w + t holds the lane's own nibble half: -(1024 + z) or -(64 + z).
  const UnpackConsts uk = unpack_consts();
  uint32_t zneg_lo = 0xE400E400u, zneg_hi = 0xD400D400u;
  asm volatile("" : "+v"(zneg_lo), "+v"(zneg_hi));
  const uint32_t hmask = hsel ? uk.mhi : uk.mlo;           // HALF: the lane's nibble mask
  const uint32_t zneg_h = hsel ? zneg_hi : zneg_lo;
  const half2v hmult = hsel ? half2v{(_Float16)0.0625f, (_Float16)0.0625f} : half2v{(_Float16)1.f, (_Float16)1.f};
  // HALF: v_perm_b32 selectors that put byte t of row 8q + 2j in the low half and of row
  // 8q + 2j + 1 in the high half, from (the partner lane's word, this lane's word): the
  // lane holding the odd row takes the even row from its partner.
  const uint32_t psel0 = 0x0C000C00u | (hsel ? 0x00000004u : 0x00040000u);
  uint32_t zs[HALF ? 16 : 32];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t b[4] = {splat_byte<0>(zw[w]), splat_byte<1>(zw[w]), splat_byte<2>(zw[w]), splat_byte<3>(zw[w])};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (HALF) {
        zs[4 * w + t] = (b[t] & hmask) | zneg_h;
      } else {
        zs[8 * w + 2 * t] = (b[t] & uk.mlo) | zneg_lo;
        zs[8 * w + 2 * t + 1] = (b[t] & uk.mhi) | zneg_hi;
      }
    }
  }

  // ---- Multiply, in halves of a k-step (rows 8q .. 8q+3, then 8q+4 .. 8q+7) on
  // v_mfma_f32_16x16x16_f16, so the first half runs while the second half's loads are
  // still arriving.
  floatx4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // Each half's MFMAs stay after its own loads only (the scheduler would otherwise
        // interleave the halves and wait for every load first).
        __builtin_amdgcn_sched_barrier(0);
        // A k-step past K (the last split's idle waves) multiplies zeros: (q - z) is finite.
        const half8v as = s < nks ? a[s] : half8v{};
        const half4v ah = half4v{as[4 * hh], as[4 * hh + 1], as[4 * hh + 2], as[4 * hh + 3]};
        // HALF: the partner lane's (l ^ 8) words of this half's two row pairs.
        uint32_t oth[2][4];
        if constexpr (HALF) {
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              oth[p][w] = (uint32_t)__builtin_amdgcn_mov_dpp((int)wv[s][2 * hh + p][w], kDppRowRor8, 0xF, 0xF, false);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            uint32_t lo[2], hi[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              uint32_t pb;
              if constexpr (HALF) {
                pb = __builtin_amdgcn_perm(oth[p][w], wv[s][2 * hh + p][w], psel0 + 0x00010001u * (uint32_t)t);
              } else {
                const uint32_t ra = wv[s][4 * hh + 2 * p][w], rb = wv[s][4 * hh + 2 * p + 1][w];
                if (t == 0) pb = pair_byte<0>(ra, rb);
                else if (t == 1) pb = pair_byte<1>(ra, rb);
                else if (t == 2) pb = pair_byte<2>(ra, rb);
                else pb = pair_byte<3>(ra, rb);
              }
              if constexpr (HALF) {
                lo[p] = as_u32(__builtin_elementwise_fma(as_h2((pb & hmask) | uk.magic), hmult, as_h2(zs[4 * w + t])));
              } else {
                lo[p] = as_u32(as_h2((pb & uk.mlo) | uk.magic) + as_h2(zs[8 * w + 2 * t]));
                hi[p] = as_u32(__builtin_elementwise_fma(as_h2((pb & uk.mhi) | uk.magic), sixteenth,
                                                         as_h2(zs[8 * w + 2 * t + 1])));
              }
            }
            if constexpr (HALF) {
              const int vl = 4 * w + t;
              acc[vl] = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, __builtin_bit_cast(half4v, u32x2{lo[0], lo[1]}),
                                                              acc[vl], 0, 0, 0);
            } else {
              const int vl = 8 * w + 2 * t;
              acc[vl] = __builtin_amdgcn_mfma_f32_16x16x16f16(ah, __builtin_bit_cast(half4v, u32x2{lo[0], lo[1]}),
                                                              acc[vl], 0, 0, 0);
              acc[vl + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                  ah, __builtin_bit_cast(half4v, u32x2{hi[0], hi[1]}), acc[vl + 1], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float bb[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) bb[k] = has_bias ? (float)__builtin_bit_cast(_Float16, braw[k]) : 0.f;
  // Scale the group's sums (fp32, exact dequant).
  if constexpr (!LATE) {
    const _Float16* sh = reinterpret_cast<const _Float16*>(sv);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float sc = HALF ? (float)sh[8 * (v >> 2) + (hsel ? hi_col(v & 3) : lo_col(v & 3))]
                            : (float)sh[8 * (v >> 3) + entry_col(v & 7)];
#pragma unroll
      for (int r = 0; r < RREG; ++r) acc[v][r] *= sc;
    }
  }

  // ---- Waves -> LDS, in rounds; each thread sums EPR (entry, lane) pairs per round.
  floatx4 ent[LGN][EPT];
#pragma unroll
  for (int b = 0; b < ROUNDS; ++b) {
    if (b > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // previous round read
    if (lane < LIVE) {
#pragma unroll
      for (int vl = 0; vl < VR; ++vl)
#pragma unroll
        for (int r = 0; r < RREG; ++r) red[wave][vl][lane][r] = acc[b * VR + vl][r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < EPR; ++k) {
      const int le = tid + THREADS * k;
      constexpr int WP = WAVES / LGN;  // waves per part
#pragma unroll
      for (int j = 0; j < LGN; ++j) {
        floatx4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv2 = j * WP; wv2 < (j + 1) * WP; ++wv2)
#pragma unroll
          for (int r = 0; r < RREG; ++r) sum[r] += red[wv2][le / LIVE][le % LIVE][r];
        ent[j][EPR * b + k] = sum;
      }
    }
  }

  if constexpr (LATE) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
#pragma unroll
      for (int r = 0; r < RREG; ++r) {
        float v = ent[0][k][r] * (float)__builtin_bit_cast(_Float16, sraw[0][k]);
#pragma unroll
        for (int j = 1; j < LG; ++j) v += ent[j][k][r] * (float)__builtin_bit_cast(_Float16, sraw[j][k]);
        ent[0][k][r] = v;
      }
    }
  }

  // ---- Split-K: fixed-point adds, all issued before any is waited for.  Thread entry k
  // is MFMA entry v, lane l: column cl of the tile, rows rb .. rb + RREG - 1.  Its
  // accumulator slots are ((tile * 32 + v) * RREG + r) * LIVE + l: consecutive threads
  // take consecutive 8-byte slots, so one wave's adds touch four 128-byte lines.  An add
  // outside the layer (row >= M or column >= N) adds 0 to its own slot, which no
  // workgroup ever completes: harmless, and branch-free.
  int e0[EPT], nrow[EPT], ncol[EPT], row0[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int le = tid + THREADS * (k % EPR);
    const int v = (k / EPR) * VR + le / LIVE, l = le % LIVE;
    row0[k] = 4 * (l >> 4);
    ncol[k] = tile * COLS + out_col<HALF>(v, l);
    e0[k] = (tile * NV + v) * RREG * LIVE + l;
    nrow[k] = ncol[k] < N ? min(max(M - row0[k], 0), RREG) : 0;
  }
  if (splits == 1) {  // K <= 128: the workgroup holds the whole sum
#pragma unroll
    for (int k = 0; k < EPT; ++k)
#pragma unroll
      for (int r = 0; r < RREG; ++r)
        if (r < nrow[k])
          y[(int64_t)(row0[k] + r) * N + ncol[k]] = __builtin_bit_cast(uint16_t, (_Float16)(ent[0][k][r] + bb[k]));
    return;
  }
  bool exc = false;
#pragma unroll
  for (int k = 0; k < EPT; ++k)
#pragma unroll
    for (int r = 0; r < RREG; ++r) exc |= r < nrow[k] && !fx_normal(ent[0][k][r]);
  if (__builtin_amdgcn_ballot_w64(exc) != 0) {  // rare: NaN, +-inf or huge partials
#pragma unroll
    for (int k = 0; k < EPT; ++k)
#pragma unroll
      for (int r = 0; r < RREG; ++r)
        if (r < nrow[k] && !fx_normal(ent[0][k][r])) fx_side_add(side + e0[k] + r * LIVE, ent[0][k][r]);
    fx_release();
  }
  uint64_t ret[EPT][RREG];
#pragma unroll
  for (int k = 0; k < EPT; ++k)
#pragma unroll
    for (int r = 0; r < RREG; ++r) ret[k][r] = fx_add(accum + e0[k] + r * LIVE, r < nrow[k] ? fx_word(ent[0][k][r]) : 0ull);
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
#pragma unroll
    for (int r = 0; r < RREG; ++r) {
      const FxSum sm = fx_decode(ret[k][r]);
      if (r < nrow[k] && sm.arrivals == (uint32_t)splits) {
        const float v = fx_total(sm, side + e0[k] + r * LIVE) + bb[k];
        fx_clear(accum + e0[k] + r * LIVE);
        y[(int64_t)(row0[k] + r) * N + ncol[k]] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

hipError_t launch_decode(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         const uint16_t* bias, int M, int K, int N, int g, const DecodePlan& p, uint64_t* accum,
                         float* side, uint16_t* y, hipStream_t stream) {
  const dim3 grid(p.n_tiles, p.splits);
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, x, reinterpret_cast<const uint32_t*>(qweight),
                       reinterpret_cast<const uint32_t*>(qzeros), scales, bias, M, K, N, g, p.splits, accum, side, y);
  };
  auto by_shape = [&](auto mp) {
    constexpr int MP = decltype(mp)::value;
    if (p.words != kDecodeWords) {  // half-width tiles: 4 waves, scaled after the reduction
      auto by_lg = [&](auto ks) {
        constexpr int KS = decltype(ks)::value;
        if (p.late == 1) go(decode_kernel<MP, KS, 4, 1, true>, 256);
        else if (p.late == 2) go(decode_kernel<MP, KS, 4, 2, true>, 256);
        else go(decode_kernel<MP, KS, 4, 4, true>, 256);
      };
      if (p.ks == 2) by_lg(std::integral_constant<int, 2>{});
      else by_lg(std::integral_constant<int, 1>{});
    } else if (p.waves == 8) {
      if (p.ks == 2) p.late ? go(decode_kernel<MP, 2, 8, 1>, 512) : go(decode_kernel<MP, 2, 8, 0>, 512);
      else p.late ? go(decode_kernel<MP, 1, 8, 1>, 512) : go(decode_kernel<MP, 1, 8, 0>, 512);
    } else {
      if (p.ks == 2) p.late ? go(decode_kernel<MP, 2, 4, 1>, 256) : go(decode_kernel<MP, 2, 4, 0>, 256);
      else p.late ? go(decode_kernel<MP, 1, 4, 1>, 256) : go(decode_kernel<MP, 1, 4, 0>, 256);
    }
  };
  if (p.mp == 1) by_shape(std::integral_constant<int, 1>{});
  else if (p.mp == 2) by_shape(std::integral_constant<int, 2>{});
  else by_shape(std::integral_constant<int, 4>{});
  return hipGetLastError();
}

}  // namespace awq
