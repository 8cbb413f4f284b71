// Skinny family of awq_gemm (small M): bandwidth-bound streaming of the packed weight.
//
// What it computes: y[m, n] = sum_k x[m, k] * (q[k, n] - z[k/g, n]) * s[k/g, n] + bias[n]
// (tensref.org "AWQ" format page, Reader; GPU LLM serving-stack blog, section 1.2:
// small-batch decode is limited by weight bandwidth, so the packed weight is read
// once and expanded only in registers).
//
// Work split.  A workgroup (4 or 8 waves) owns a column tile of 32 packed word-columns
// (256 output columns = 128 contiguous bytes of every qweight row) and a run of
// WAVES*L 32-row k-steps; wave w takes L consecutive k-steps of that run.  The host
// picks L and the number of K splits S (about one resident round of workgroups on
// small layers, shorter one-group runs on large ones) and the plan's rows: 4-row
// plans (one or two rows of x; three or four on large layers), 8-row plans (five to
// eight on large layers) or 16-row plans (up to 16).
// At a few microseconds per call the kernel is latency-bound, so every input is
// requested up front: each wave issues the weight loads of its first two k-steps,
// and the workgroup turns the zero words and scales of every group it touches into
// per-lane LDS tables (fp16 zero splats, fp32 scales) in the same round trip.
//
// Per wave and k-step, on v_mfma_f32_16x16x32_f16 (x rows padded to 16):
//   lane l: q = l / 16 picks rows 8q..8q+7 of the k-step, c = l % 16 picks word
//   columns 2c, 2c+1 of the tile; one 8-byte load per row (16 lanes cover 128
//   contiguous bytes of a row).  From each pair of rows, v_perm_b32 interleaves byte
//   t of both words, the 0x6400 mantissa trick turns each nibble pair into an exact
//   fp16 pair (code + 1024) or (16 code + 1024), and one packed add / fma removes the
//   zero, leaving the exact integers (q - z) of rows (r, r+1) of one column.  Four
//   pairs form one B operand (8 consecutive k of one column).  The lane's 16 columns
//   give 16 MFMAs; MFMA column c is output column 8 (tile_wc + 2c + w) + j.  The A
//   operand is x[m = l % 16][8q..8q+7].  fp16 x times a small integer is exact in
//   fp32 and the MFMA accumulates in fp32.
// Groups: the MFMA accumulates sum_k x (q - z) per group; at the end of a group the
// sum is scaled by s in fp32 (exact dequant, no fp16 weight rounding).
// Reduction: the waves' accumulators meet in LDS in register order (conflict-free
// 16-byte accesses) and are summed in wave order.  With S > 1 splits, the plans of
// three or more rows (and bfloat16) store fp32 partials that are summed in split order,
// by a second kernel or, on grids of several rounds (`fused`), by the workgroup of each
// tile that arrives last; in fp16 plans of one or two rows (ATOMIC) the splits of an output
// element meet in one 64-bit accumulator in the workspace: each workgroup
// adds, with one relaxed atomic fetch-add, its partial as a fixed-point integer
// (24 fractional bits) plus 2^56, i.e. one arrival in the top byte.  Integer
// addition does not depend on order, so the sum is bit-reproducible; the add that
// brings the arrival count to S returns the complete sum to its workgroup, which
// converts it, adds bias, rounds once to fp16, stores y and resets the accumulator
// to zero for the next call (graph replays included).  One round trip to the
// atomic units and no cross-workgroup reads or fences.
// Fixed point: every fp16 value is a multiple of 2^-24, so a single exact product
// (an identity input row, an integer weight) survives unchanged; sums are kept to
// 2^-24 absolute, finer than fp32's rounding for |partial| > 1.  Partials are
// clamped to +-2^23 so up to 128 splits can never carry into the count byte; a
// partial that large would already exceed fp16's range by a factor of 128.
#include <type_traits>

#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Step {
  u32x2 v[8];  // rows 8q..8q+7, words (2c, 2c+1)
  half8v a;    // x[m][8q..8q+7] of this k-step
};

__device__ __forceinline__ half8v pack4(half2v a, half2v b, half2v c, half2v d) {
  return half8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Entry v of a lane's 16-entry tables and accumulators: word w = v / 8, byte
// t = (v / 2) % 4, nibble half h = v % 2 (0: low nibble, column lo_col(t);
// 1: high nibble, column hi_col(t)).
__host__ __device__ constexpr int tab_idx(int w, int t, int h) { return w * 8 + 2 * t + h; }
__host__ __device__ constexpr int tab_col(int v) {  // column within the word
  return (v & 1) ? hi_col((v >> 1) & 3) : lo_col((v >> 1) & 3);
}

// The 16 MFMAs of one k-step for one lane's 2 word-columns.
// fp16 x: zs holds, per entry, the fp16 splat to add: -(1024 + z) for low-nibble
// columns, -(64 + z) for high-nibble columns, so B = (q - z) exactly.
// bfloat16 x (no packed bfloat16 add on this chip): B = 128 + q, exact in
// bfloat16, and one more MFMA against a B of ones adds the k-step's sum of x per row
// to sx; the group's sum is then corrected by -(128 + z) sx in fp32 (flush).
template <bool BF16>
__device__ __forceinline__ void kstep_mfma(const Step& st, const uint32_t (&zs)[16], const UnpackConsts& uk,
                                           floatx4 (&part)[16], floatx4& sx) {
  if constexpr (BF16) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, st.a);
    const uint32_t one2 = 0x3F803F80u;  // bfloat16 pair (1, 1)
    sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2}), sx,
                                                 0, 0, 0);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t ra = st.v[2 * p][w];
          const uint32_t rb = st.v[2 * p + 1][w];
          uint32_t pb;
          if (t == 0) pb = pair_byte<0>(ra, rb);
          else if (t == 1) pb = pair_byte<1>(ra, rb);
          else if (t == 2) pb = pair_byte<2>(ra, rb);
          else pb = pair_byte<3>(ra, rb);
          lo[p] = lo_magic_bf16(pb, uk);
          hi[p] = hi_magic_bf16(pb, uk);
        }
        const int il = tab_idx(w, t, 0), ih = tab_idx(w, t, 1);
        part[il] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]}), part[il], 0, 0, 0);
        part[ih] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]}), part[ih], 0, 0, 0);
      }
    }
    return;
  }
  (void)sx;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      half2v lo[4], hi[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t ra = st.v[2 * p][w];
        const uint32_t rb = st.v[2 * p + 1][w];
        uint32_t pb;
        if (t == 0) pb = pair_byte<0>(ra, rb);
        else if (t == 1) pb = pair_byte<1>(ra, rb);
        else if (t == 2) pb = pair_byte<2>(ra, rb);
        else pb = pair_byte<3>(ra, rb);
        lo[p] = lo_minus_zero(pb, as_h2(zs[tab_idx(w, t, 0)]), uk);
        hi[p] = hi_minus_zero(pb, as_h2(zs[tab_idx(w, t, 1)]), uk);
      }
      const int il = tab_idx(w, t, 0), ih = tab_idx(w, t, 1);
      part[il] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.a, pack4(lo[0], lo[1], lo[2], lo[3]), part[il], 0, 0, 0);
      part[ih] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st.a, pack4(hi[0], hi[1], hi[2], hi[3]), part[ih], 0, 0, 0);
    }
  }
}

// LDS tables: per group and lane column c, 16 entries padded to 20 words (spreads
// the 16-byte reads of the 16 column lanes over the banks).
constexpr int kTabStride = 20;

// red: per wave, accumulator and lane; with at most 4 (8) rows only lanes 0..15
// (0..31) hold rows that are stored, so RL = 16 (32) lanes are kept, which lets a
// third 4-wave workgroup share a compute unit.
template <int WAVES, int RL>
struct SkinnyLds {
  union {
    struct {
      uint32_t zsplat[kSkinnyMaxGroups][16][kTabStride];
      float scale[kSkinnyMaxGroups][16][kTabStride];
    } meta;
    floatx4 red[WAVES][16][RL];  // [wave][accumulator][lane]
    uint16_t ys[16][kSkinnyCols + 8];  // rounded outputs of the last split, in output order
  } u;
};

}  // namespace

// Routed experts: bit t of the result is set when token t (t < T <= 64) sends a
// slot to `expert`.  Lanes 0..T-1 of the calling wave each test one token; every wave
// of a workgroup gets the same mask.
__device__ __forceinline__ uint64_t routed_tokens(const SkinnyExperts& ex, int T, int expert, int lane) {
  bool r = false;
  if (lane < T)
    for (int j = 0; j < ex.topk; ++j) r |= ex.ids[lane * ex.topk + j] == expert;
  return (uint64_t)__ballot(r);
}

// Index of the n-th set bit of mask (n < popcount(mask)).
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int n) {
  for (int i = 0; i < n; ++i) mask &= mask - 1;
  return __builtin_ctzll(mask);
}

// Block x of the routed-expert grid: chunk-major (every expert's first 16 routed
// tokens first; the later chunks, empty for most experts, come last and exit at
// once), then expert, then column tile.
struct ExpertBlock {
  int expert, chunk, tile;
};
__device__ __forceinline__ ExpertBlock expert_block(const SkinnyExperts& ex, int b, int experts) {
  const int per_chunk = experts * ex.tiles;
  const int c = b / per_chunk;
  const int r = b - c * per_chunk;
  return ExpertBlock{r / ex.tiles, c, r % ex.tiles};
}

// Workspace: per tile, 64-bit accumulator 4 * slot + i holds row 4 (slot / 256) + i
// of the slot's column, slot = q * 256 + accumulator * 16 + c.  All zero between calls.
// EXPERTS: routed experts (SkinnyExperts); M is the token count on entry, there is
// no bias.  The block's rows are then only its chunk of the tokens routed to its
// expert, in token order (row m = routed token 16 chunk + m), and M becomes their
// count: the MFMA rows, the split accumulators or partials and the reduction cover
// just those rows.
template <int WAVES, int MROWS, bool SINGLE, bool BF16, bool EXPERTS = false, bool ATOMIC = MROWS == 4 && !BF16>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void skinny_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint32_t* __restrict__ qzeros, const _Float16* __restrict__ scales, int M, int K, int N, int g,
    int L, int splits, const uint16_t* __restrict__ bias, int fused, uint64_t* __restrict__ accum,
    float* __restrict__ partial, uint16_t* __restrict__ y, SkinnyExperts ex) {
  // Argument order: everything the k loop needs first, so that it falls in the 14 dwords
  // the dispatcher preloads into SGPRs (the rest is fetched from memory).
  constexpr int THREADS = 64 * WAVES;
  constexpr int TILE_ENTRIES = MROWS * kSkinnyCols;  // (slot, row) entries of a tile
  // k-steps in flight per wave: two, so a wave multiplies one k-step while the next is
  // in flight.  Deeper rings issue more loads before the first multiply, and on a
  // saturated memory system issuing itself stalls: up_proj 16 x 4096 x 11008 13.3 ->
  // 12.9 us and down_proj 8 x 11008 x 4096 12.4 -> 12.2 us with two instead of four on
  // 8-wave one-group plans.  How K splits meet: ATOMIC (4-row fp16 plans of one or two
  // rows) combines splits with fixed-point atomics; the other plans (the atomic count
  // M * N * S gets large) store fp32 partials.  bfloat16 always takes the partials: the
  // fixed-point format relies on fp16's range and resolution (every fp16 value a
  // multiple of 2^-24, |x| < 2^16).
  constexpr int PF = 2;
  static_assert(!ATOMIC || (MROWS == 4 && !BF16), "fixed-point atomics: 4-row fp16 plans only");
  static_assert(MROWS == 4 || MROWS == 8 || MROWS == 16, "4, 8 or 16 rows");
  __shared__ SkinnyLds<WAVES, 4 * MROWS> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int q = lane >> 4;
  const int c = lane & 15;
  const int NW = N >> 3;
  // Column tile; with EXPERTS, block x also names the expert.  Accumulators and
  // partials belong to the block.
  const ExpertBlock eb = EXPERTS ? expert_block(ex, blockIdx.x, ex.experts) : ExpertBlock{0, 0, (int)blockIdx.x};
  const int expert = eb.expert;
  const int tile = eb.tile;
  const int split = blockIdx.y;
  uint64_t tokens = 0;  // EXPERTS: the routed-token mask of this block's expert
  const int row0 = kSkinnyMaxM * eb.chunk;  // EXPERTS: first routed token of the chunk
  const uint32_t x_bytes = (uint32_t)M * (uint32_t)K * 2u;  // x rows (tokens with EXPERTS)
  if constexpr (EXPERTS) {
    tokens = routed_tokens(ex, M, expert, lane);
    M = min(__builtin_popcountll(tokens) - row0, kSkinnyMaxM);
    if (M <= 0) return;  // uniform: no routed token in this chunk
    qweight += expert * ex.w_stride;
    qzeros += expert * ex.z_stride;
    scales += expert * ex.s_stride;
  }
  // Store of output row `row`, column n: row `row` of y, or every slot of the
  // row's token routed to this block's expert.
  auto put = [&](int row, int n, float v) {
    if constexpr (EXPERTS) {
      const int tok = nth_set_bit(tokens, row0 + row);
      for (int j = 0; j < ex.topk; ++j)
        if (ex.ids[tok * ex.topk + j] == expert) y[((int64_t)tok * ex.topk + j) * N + n] = float_to_act<BF16>(v);
    } else {
      y[(int64_t)row * N + n] = float_to_act<BF16>(v);
    }
  };
  const int wc = tile * kSkinnyWordCols + 2 * c;
  const bool col_ok = wc < NW;  // NW % 4 == 0, so wc + 1 < NW as well

  // k-steps: workgroup run [s0, s1), wave run [kb, ke).
  const int T = K / kKStep;
  const int s0 = split * WAVES * L;
  const int s1 = min(T, s0 + WAVES * L);
  const int kb = min(s1, s0 + wave * L);
  const int ke = min(s1, kb + L);
  const int gsteps = g / kKStep;
  const int g0 = s0 / gsteps;

  // Loads address the uniform base pointers with 32-bit byte offsets (the host
  // keeps qweight under 4 GiB).  Lanes of x rows >= M or of columns >= N read a
  // valid clamped address instead of being masked: an MFMA output row depends only
  // on its own x row, and rows >= M and columns >= N are never stored.
  const int m = lane & 15;
  const int xrow = EXPERTS ? nth_set_bit(tokens, row0 + (m < M ? m : 0)) : (m < M ? m : 0);
  const uint32_t x_off = ((uint32_t)xrow * (uint32_t)K + 8u * q) * 2u;
  const uint32_t w_off = ((uint32_t)(8 * q) * (uint32_t)NW + (uint32_t)(col_ok ? wc : 0)) * 4u;
  const uint32_t row_bytes = (uint32_t)NW * 4u;
  // Buffer loads: the lane's offset stays in one VGPR and the row moves in the scalar
  // offset, so the loads cost no vector address arithmetic.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(qweight), (short)0, (int)(row_bytes * (uint32_t)K), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, (int)x_bytes, 0x00020000);

  // Loads of k-step ks (ks < ke, uniform across the wave).
  auto issue = [&](Step& st, int ks) {
    const uint32_t r0 = (uint32_t)ks * (uint32_t)kKStep;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      st.v[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wrs, w_off, (r0 + r) * row_bytes, 2));
    st.a = __builtin_bit_cast(half8v, __builtin_amdgcn_raw_buffer_load_b128(xrs, x_off, r0 * 2u, 0));
  };

  // 1. Group data and weight loads.
  //   One group per wave (SINGLE): every lane loads the zero words and fp16 scales of
  //   its two word columns for its wave's group straight into registers, before the
  //   weights, so that nothing waits for the weights but the multiply itself and no
  //   workgroup barrier is needed.
  //   Several groups: the workgroup turns the zero words and scales of every group
  //   it touches into per-lane LDS tables while the weights are in flight.
  u32x2 gz = {0u, 0u};
  half8v gs0 = {}, gs1 = {};
  if constexpr (SINGLE) {
    const int gw = min(kb, T - 1) / gsteps;  // a wave without k-steps loads a valid group
    const int wcc = col_ok ? wc : 0;
    gz = *reinterpret_cast<const u32x2*>(qzeros + (int64_t)gw * NW + wcc);
    const _Float16* sp = scales + (int64_t)gw * N + 8 * wcc;
    gs0 = *reinterpret_cast<const half8v*>(sp);
    gs1 = *reinterpret_cast<const half8v*>(sp + 8);
  }
  Step ring[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (kb + j < ke) issue(ring[j], kb + j);
  if constexpr (!SINGLE) {
    const int ng = (s1 > s0) ? (s1 - 1) / gsteps - g0 + 1 : 0;  // <= kSkinnyMaxGroups (host)
    // Every table entry's loads are issued before any is used (one round trip to
    // memory, not one per entry a thread fills); entries past the tables load entry 0.
    constexpr int TAB_IT = (kSkinnyMaxGroups * 256 + THREADS - 1) / THREADS;
    uint32_t zr[TAB_IT];
    uint16_t sr[TAB_IT];
    const uint16_t* sbits = reinterpret_cast<const uint16_t*>(scales);
#pragma unroll
    for (int it = 0; it < TAB_IT; ++it) {
      const int i = tid + it * THREADS;
      const int gl = i >> 8, cc = (i >> 4) & 15, v = i & 15;
      const int wcol = tile * kSkinnyWordCols + 2 * cc + (v >> 3);
      const bool ok = i < ng * 256 && wcol < NW;
      zr[it] = qzeros[ok ? (int64_t)(g0 + gl) * NW + wcol : 0];
      sr[it] = sbits[ok ? (int64_t)(g0 + gl) * N + 8 * wcol + tab_col(v) : 0];
    }
#pragma unroll
    for (int it = 0; it < TAB_IT; ++it) {
      const int i = tid + it * THREADS;
      if (i >= ng * 256) break;
      const int gl = i >> 8, cc = (i >> 4) & 15, v = i & 15;
      const int wcol = tile * kSkinnyWordCols + 2 * cc + (v >> 3);
      const int col = tab_col(v);
      const uint32_t zw = wcol < NW ? zr[it] : 0u;
      const float sv = wcol < NW ? (float)__builtin_bit_cast(_Float16, sr[it]) : 0.f;
      const uint32_t z = zero_code(zw, col);
      if constexpr (BF16) {
        sh.u.meta.zsplat[gl][cc][v] = __builtin_bit_cast(uint32_t, 128.0f + (float)z);  // 128 + z, fp32
      } else {
        // fp16 bits of -(1024 + z) (low nibble) or -(64 + z) (high nibble), splatted.
        const uint32_t h = (v & 1) ? (0xD400u | (z << 4)) : (0xE400u | z);
        sh.u.meta.zsplat[gl][cc][v] = h | (h << 16);
      }
      sh.u.meta.scale[gl][cc][v] = sv;
    }
    __syncthreads();
  }

  floatx4 part[16];
  floatx4 acc[16];
  floatx4 sx = floatx4{0.f, 0.f, 0.f, 0.f};  // bfloat16: sum of x over the group's k, per row
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    part[v] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (!SINGLE) acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto load_tab = [&](const uint32_t* row, uint32_t (&dst)[16]) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + 4 * k4);
      dst[4 * k4 + 0] = v[0];
      dst[4 * k4 + 1] = v[1];
      dst[4 * k4 + 2] = v[2];
      dst[4 * k4 + 3] = v[3];
    }
  };
  uint32_t zs[16];
  // Scale this group's sums into acc (several groups); bfloat16 first subtracts
  // (128 + z) times the group's sum of x (zs holds 128 + z as fp32 bits).
  auto flush = [&](int gl) {
    uint32_t sb[16];
    load_tab(reinterpret_cast<const uint32_t*>(sh.u.meta.scale[gl][c]), sb);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      floatx4 pv = part[v];
      if constexpr (BF16) pv -= __builtin_bit_cast(float, zs[v]) * sx;
      acc[v] += __builtin_bit_cast(float, sb[v]) * pv;
      part[v] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    sx = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  const UnpackConsts uk = unpack_consts();
  if constexpr (SINGLE) {
    // Entry v: word w = v / 8, column tab_col(v) of it; zero term as in the tables.
    const uint32_t zw[2] = {gz[0], gz[1]};
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const uint32_t z = zero_code(zw[v >> 3], tab_col(v));
      if constexpr (BF16) {
        zs[v] = __builtin_bit_cast(uint32_t, 128.0f + (float)z);
      } else {
        const uint32_t h = (v & 1) ? (0xD400u | (z << 4)) : (0xE400u | z);
        zs[v] = h | (h << 16);
      }
    }
  }
  int cur_g = -1;
  // Ring of PF k-steps in flight: after step ks is consumed its slot loads ks + PF.
  for (int base = kb; base < ke; base += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int ks = base + j;
      if (ks < ke) {
        if constexpr (!SINGLE) {
          const int gl = ks / gsteps - g0;
          if (gl != cur_g) {
            if (cur_g >= 0) flush(cur_g);
            load_tab(sh.u.meta.zsplat[gl][c], zs);
            cur_g = gl;
          }
        }
        kstep_mfma<BF16>(ring[j], zs, uk, part, sx);
        if (ks + PF < ke) issue(ring[j], ks + PF);
      }
    }
  }
  if constexpr (SINGLE) {
    // Scale the group's sums (all four rows of each entry: a per-entry branch on M == 1
    // compiled to 32 branches here, on the path to the wave reduction).
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float sv = (float)((v >> 3) ? gs1[tab_col(v)] : gs0[tab_col(v)]);
      if constexpr (BF16) {
        const float zc = __builtin_bit_cast(float, zs[v]);
        part[v] = (part[v] - zc * sx) * sv;
      } else {
        part[v] *= sv;
      }
    }
  } else {
    if (cur_g >= 0) flush(cur_g);
    __syncthreads();  // the tables are dead; their LDS becomes the reduction buffer
  }

  // Output column of a slot.
  auto slot_n = [&](int s) {
    const int sv = (s >> 4) & 15, sc = s & 15;
    return tile * kSkinnyCols + 8 * (2 * sc + (sv >> 3)) + tab_col(sv);
  };
  constexpr int SLOTS = 1024 / THREADS;  // slots per thread when all 16 rows are live
  // The bias of this thread's slots, requested now so that it arrives under the wave
  // reduction: each epilogue below would otherwise wait for it after its own memory round
  // trip (partials or fixed-point adds).  Without a bias the loads read x and are unused.
  uint16_t braw[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int n = slot_n(tid + k * THREADS);
    braw[k] = (bias != nullptr ? bias : x)[bias != nullptr ? min(n, N - 1) : 0];
  }

  // 2. Waves -> LDS in register order, then sums over waves per slot.  Only the
  // lanes q < MROWS / 4 (rows 0 .. MROWS - 1) hold rows that are ever stored.
  if (q < MROWS / 4) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sh.u.red[wave][v][lane] = SINGLE ? part[v] : acc[v];
  }
  __syncthreads();

  // Slots in q-major order so that M <= 4 touches only q = 0 (one slot per thread).
  const int rows = M < MROWS ? M : MROWS;
  const int nslots = 256 * ((rows + 3) / 4);
  floatx4 sum[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int s = tid + k * THREADS;
    sum[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (s < nslots) {
#pragma unroll
      for (int wv = 0; wv < WAVES; ++wv) sum[k] += sh.u.red[wv][(s >> 4) & 15][(s >> 8) * 16 + (s & 15)];
    }
  }
  if (splits == 1) {
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      const int s = tid + k * THREADS;
      const int n = slot_n(s);
      if (s < nslots && n < N) {
        const float b = bias ? act_to_float<BF16>(braw[k]) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * (s >> 8) + i;
          if (row < rows) put(row, n, sum[k][i] + b);
        }
      }
    }
    return;
  }

  if (!ATOMIC) {
    if constexpr (!EXPERTS) {
      if (fused) {
        // 3'. fp32 partials [tile][split][entry], summed in split order by whichever
        // workgroup of the tile arrives last.  Partials are stored and read at device
        // scope (each XCD has its own L2); every wave waits for its stores to complete
        // before the workgroup's single arrival on the tile's counter, so the workgroup
        // that brings the count to `splits` reads complete partials.  It resets the
        // counter for the next call.
        const uint32_t entry_bytes = (uint32_t)TILE_ENTRIES * 4u;
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            partial + (int64_t)blockIdx.x * splits * TILE_ENTRIES, (short)0, (int)((uint32_t)splits * entry_bytes),
            0x00020000);
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
          const int s = tid + k * THREADS;
          if (s < nslots)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sum[k]), prs,
                                                   (uint32_t)split * entry_bytes + 16u * (uint32_t)s, 0, kCpolDevice);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ uint32_t last_arrival;
        if (tid == 0) {
          uint32_t* ctr = reinterpret_cast<uint32_t*>(accum) + blockIdx.x;
          const bool last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                            (uint32_t)splits - 1u;
          if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last_arrival = last;
        }
        __syncthreads();
        if (!last_arrival) return;
        // Every slot's loads of a batch are issued before any is added (a slot whose
        // entries lie past the live rows reads slot tid's, in bounds, and is dropped).
        floatx4 tot[SLOTS];
        auto gather = [&](auto bc) {
          constexpr int B = decltype(bc)::value;
          auto ld = [&](int k, int sp) {
            const int sl = tid + k * THREADS < nslots ? tid + k * THREADS : tid;
            const uint32_t off = (uint32_t)min(sp, splits - 1) * entry_bytes + 16u * (uint32_t)sl;
            return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, kCpolDevice));
          };
          floatx4 v[SLOTS][B];
#pragma unroll
          for (int k = 0; k < SLOTS; ++k)
#pragma unroll
            for (int j = 0; j < B; ++j) v[k][j] = ld(k, j);
#pragma unroll
          for (int k = 0; k < SLOTS; ++k) {
            tot[k] = v[k][0];
#pragma unroll
            for (int j = 1; j < B; ++j)
              if (j < splits) tot[k] += v[k][j];
          }
          for (int s0 = B; s0 < splits; s0 += 8) {
            floatx4 w[SLOTS][8];
#pragma unroll
            for (int k = 0; k < SLOTS; ++k)
#pragma unroll
              for (int j = 0; j < 8; ++j) w[k][j] = ld(k, s0 + j);
#pragma unroll
            for (int k = 0; k < SLOTS; ++k)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                if (s0 + j < splits) tot[k] += w[k][j];
          }
        };
        if (splits <= 4) gather(std::integral_constant<int, 4>{});
        else if (splits <= 8) gather(std::integral_constant<int, 8>{});
        else gather(std::integral_constant<int, 16>{});
        // Rounded outputs meet in LDS in output order; y is written as 16-byte row pieces.
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
          const int s = tid + k * THREADS;
          if (s >= nslots) continue;
          const int sv = (s >> 4) & 15, sc = s & 15;
          const int ct = 8 * (2 * sc + (sv >> 3)) + tab_col(sv);  // column within the tile
          const int n = tile * kSkinnyCols + ct;
          const float b = (bias != nullptr && n < N) ? act_to_float<BF16>(braw[k]) : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) sh.u.ys[4 * (s >> 8) + i][ct] = float_to_act<BF16>(tot[k][i] + b);
        }
        __syncthreads();
        for (int i = tid; i < rows * (kSkinnyCols / 8); i += THREADS) {
          const int row = i / (kSkinnyCols / 8), pc = i % (kSkinnyCols / 8);
          const int n0 = tile * kSkinnyCols + 8 * pc;
          if (n0 < N)
            *reinterpret_cast<u32x4*>(y + (int64_t)row * N + n0) =
                *reinterpret_cast<const u32x4*>(&sh.u.ys[row][8 * pc]);
        }
        return;
      }
    }
    // 3'. Plain fp32 partial stores [block][split][entry]; skinny_reduce_kernel sums
    // them in split order after this kernel completes.
    float* tile_part = partial + ((int64_t)blockIdx.x * splits + split) * TILE_ENTRIES;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      const int s = tid + k * THREADS;
      if (s < nslots) *reinterpret_cast<floatx4*>(tile_part + 4 * s) = sum[k];
    }
    return;
  }

  // 3. Fixed-point accumulation across splits (awq_device.h); the add that completes an
  // element finishes it.  For these plans `partial` holds the float side words, one per
  // accumulator word.  Adds outside the layer (rows >= M, columns >= N) add 0 to their own
  // slot, which never completes.
  uint64_t* tile_acc = accum + (int64_t)blockIdx.x * TILE_ENTRIES;
  float* tile_side = partial + (int64_t)blockIdx.x * TILE_ENTRIES;
  bool exc = false;
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int s = tid + k * THREADS;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      exc |= s < nslots && slot_n(s) < N && 4 * (s >> 8) + i < rows && !fx_normal(sum[k][i]);
  }
  if (__builtin_amdgcn_ballot_w64(exc) != 0) {  // rare: NaN, +-inf or huge partials
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      const int s = tid + k * THREADS;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (s < nslots && slot_n(s) < N && 4 * (s >> 8) + i < rows && !fx_normal(sum[k][i]))
          fx_side_add(tile_side + 4 * s + i, sum[k][i]);
    }
    fx_release();
  }
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int s = tid + k * THREADS;
    if (s >= nslots) continue;
    const int n = slot_n(s);
    uint64_t ret[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = n < N && 4 * (s >> 8) + i < rows;
      ret[i] = fx_add(tile_acc + 4 * s + i, live ? fx_word(sum[k][i]) : 0ull);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (s >> 8) + i;
      const FxSum fs = fx_decode(ret[i]);
      if (n < N && row < rows && fs.arrivals == (uint32_t)splits) {
        const float b = bias ? act_to_float<BF16>(braw[k]) : 0.f;
        const float v = fx_total(fs, tile_side + 4 * s + i) + b;
        fx_clear(tile_acc + 4 * s + i);
        put(row, n, v);
      }
    }
  }
}

// Sums the fp32 partials of the skinny kernel in split order, adds bias, rounds once
// to fp16 or bfloat16.  One workgroup per (tile, group of 4 rows): thread t reads the
// 4 rows of slot 256 q + t (16 contiguous bytes per split), and the rounded values
// meet in LDS in output order so that y is written as whole 16-byte row pieces.
// tile_entries: rows kept per tile (4 or 16) x 256.
// EXPERTS: partials of block b = (expert, chunk, column tile), whose rows are the
// chunk's tokens routed to the expert in token order (row m = routed token
// 16 chunk + m); row m goes to that token's slots of the expert.  Blocks without
// rows wrote no partials and store nothing.
template <bool BF16, bool EXPERTS = false, int B = 8>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ partial,
                                                            const uint16_t* __restrict__ bias, int M, int N,
                                                            int splits, int tile_entries, uint16_t* __restrict__ y,
                                                            SkinnyExperts ex) {
  const int TILE_ENTRIES = tile_entries;
  __shared__ __attribute__((aligned(16))) uint16_t ys[4][kSkinnyCols + 8];
  const int block = blockIdx.x / 4, q = blockIdx.x % 4;
  const ExpertBlock eb = EXPERTS ? expert_block(ex, block, ex.experts) : ExpertBlock{0, 0, block};
  const int expert = eb.expert;
  const int tile = eb.tile;
  const int row0 = kSkinnyMaxM * eb.chunk;
  uint64_t tokens = 0;
  if constexpr (EXPERTS) {
    tokens = routed_tokens(ex, M, expert, threadIdx.x & 63);
    M = min(__builtin_popcountll(tokens) - row0, kSkinnyMaxM);  // rows of the block (<= 0: none)
  }
  if (4 * q >= M) return;  // whole workgroup: rows beyond M
  const int t = threadIdx.x;
  const int slot = q * 256 + t;
  const int sv = (t >> 4) & 15, sc = t & 15;
  const int ct = 8 * (2 * sc + (sv >> 3)) + tab_col(sv);  // column within the tile
  const int n = tile * kSkinnyCols + ct;
  // The bias is requested first, so that it arrives with the partials: one memory round
  // trip, not two (without a bias the load reads the first partial and is not used).
  const uint16_t* bsrc = bias != nullptr ? bias : reinterpret_cast<const uint16_t*>(partial);
  const uint16_t braw = bsrc[bias != nullptr ? min(n, N - 1) : 0];
  __builtin_amdgcn_sched_barrier(0);
  const floatx4 a = sum_splits<B>(partial + (int64_t)block * splits * TILE_ENTRIES + 4 * slot, TILE_ENTRIES, splits);
  const float b = (bias != nullptr && n < N) ? act_to_float<BF16>(braw) : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) ys[i][ct] = float_to_act<BF16>(a[i] + b);
  __syncthreads();
  if (t < 4 * (kSkinnyCols / 8)) {
    const int i = t / (kSkinnyCols / 8), pc = t % (kSkinnyCols / 8);
    const int row = 4 * q + i, n0 = tile * kSkinnyCols + 8 * pc;
    if (row < M && n0 < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&ys[i][8 * pc]);
      if constexpr (EXPERTS) {
        const int tok = nth_set_bit(tokens, row0 + row);
        for (int j = 0; j < ex.topk; ++j)
          if (ex.ids[tok * ex.topk + j] == expert)
            *reinterpret_cast<u32x4*>(y + ((int64_t)tok * ex.topk + j) * N + n0) = v;
      } else {
        *reinterpret_cast<u32x4*>(y + (int64_t)row * N + n0) = v;
      }
    }
  }
}

template <bool BF16>
static hipError_t launch_skinny_t(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                                  const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                                  const SkinnyPlan& p, uint64_t* accum, float* partial, uint16_t* y,
                                  hipStream_t stream) {
  const dim3 grid(p.n_tiles, p.splits);
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, x, reinterpret_cast<const uint32_t*>(qweight),
                       reinterpret_cast<const uint32_t*>(qzeros), reinterpret_cast<const _Float16*>(scales), M, K,
                       N, g, p.L, p.splits, bias, (int)p.fused, accum, partial, y, SkinnyExperts{});
  };
  if (p.mrows == 4 && p.atomic && !BF16) {
    if (p.single_group) go(skinny_kernel<4, 4, true, false, false, true>, 256);
    else go(skinny_kernel<4, 4, false, false, false, true>, 256);
  } else if (p.mrows == 4) {
    if (p.single_group) go(skinny_kernel<4, 4, true, BF16, false, false>, 256);
    else go(skinny_kernel<4, 4, false, BF16, false, false>, 256);
  } else if (p.mrows == 8) {
    if (p.single_group) go(skinny_kernel<4, 8, true, BF16>, 256);
    else go(skinny_kernel<4, 8, false, BF16>, 256);
  } else if (p.waves == 4) {
    if (p.single_group) go(skinny_kernel<4, 16, true, BF16>, 256);
    else go(skinny_kernel<4, 16, false, BF16>, 256);
  } else {
    if (p.single_group) go(skinny_kernel<8, 16, true, BF16>, 512);
    else go(skinny_kernel<8, 16, false, BF16>, 512);
  }
  // Partials of unfused plans (all but the atomic ones) are summed by the reduce kernel.
  if (p.splits > 1 && !p.fused && !(p.mrows == 4 && p.atomic && !BF16)) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto red = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(p.n_tiles * 4), dim3(256), 0, stream, partial, bias, M, N, p.splits,
                         p.mrows * kSkinnyCols, y, SkinnyExperts{});
    };
    const int b = split_batch(p.splits);
    if (b == 4) red(skinny_reduce_kernel<BF16, false, 4>);
    else if (b == 8) red(skinny_reduce_kernel<BF16, false, 8>);
    else red(skinny_reduce_kernel<BF16, false, 16>);
  }
  return hipGetLastError();
}

// Routed experts (fp16): p.n_tiles = chunks x experts x column tiles per expert.
hipError_t launch_skinny_experts(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                                 const uint16_t* scales, int T, int K, int N, int g, const SkinnyPlan& p,
                                 const SkinnyExperts& ex, uint64_t* accum, float* partial, uint16_t* y,
                                 hipStream_t stream) {
  const dim3 grid(p.n_tiles, p.splits);
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, x, reinterpret_cast<const uint32_t*>(qweight),
                       reinterpret_cast<const uint32_t*>(qzeros), reinterpret_cast<const _Float16*>(scales), T, K,
                       N, g, p.L, p.splits, nullptr, 0, accum, partial, y, ex);
  };
  if (p.mrows == 4 && p.atomic) {
    if (p.single_group) go(skinny_kernel<4, 4, true, false, true, true>, 256);
    else go(skinny_kernel<4, 4, false, false, true, true>, 256);
  } else if (p.mrows == 4) {
    if (p.single_group) go(skinny_kernel<4, 4, true, false, true, false>, 256);
    else go(skinny_kernel<4, 4, false, false, true, false>, 256);
  } else if (p.mrows == 8) {
    if (p.single_group) go(skinny_kernel<4, 8, true, false, true>, 256);
    else go(skinny_kernel<4, 8, false, false, true>, 256);
  } else if (p.waves == 4) {
    if (p.single_group) go(skinny_kernel<4, 16, true, false, true>, 256);
    else go(skinny_kernel<4, 16, false, false, true>, 256);
  } else {
    if (p.single_group) go(skinny_kernel<8, 16, true, false, true>, 512);
    else go(skinny_kernel<8, 16, false, false, true>, 512);
  }
  if (p.splits > 1 && !(p.mrows == 4 && p.atomic)) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((skinny_reduce_kernel<false, true>), dim3(p.n_tiles * 4), dim3(256), 0, stream, partial,
                       nullptr, T, N, p.splits, p.mrows * kSkinnyCols, y, ex);
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                         const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                         const SkinnyPlan& p, bool bf16, uint64_t* accum, float* partial, uint16_t* y,
                         hipStream_t stream) {
  return bf16 ? launch_skinny_t<true>(x, qweight, qzeros, scales, bias, M, K, N, g, p, accum, partial, y, stream)
              : launch_skinny_t<false>(x, qweight, qzeros, scales, bias, M, K, N, g, p, accum, partial, y, stream);
}

}  // namespace awq
