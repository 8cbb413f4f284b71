// Internal launch interface between the C ABI (awq_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

// Skinny (small-M) family geometry: a workgroup owns 32 packed word-columns
// (256 output columns) and a contiguous run of 32-row k-steps.
constexpr int kSkinnyThreads = 256;
constexpr int kSkinnyWordCols = 32;
constexpr int kSkinnyCols = 8 * kSkinnyWordCols;
constexpr int kKStep = 32;
constexpr int kSkinnyMaxM = 16;
constexpr int kSkinnyMaxGroups = 16;  // quantization groups one workgroup may touch
constexpr int kFxMaxSplits = 127;     // arrivals a fixed-point split-K word can count
constexpr int kSkinnyMaxSplits = kFxMaxSplits;

// Launch plan of the skinny family (chosen on the host, see awq_api.hip).
struct SkinnyPlan {
  int n_tiles;       // column tiles of kSkinnyCols
  int splits;        // K splits across workgroups (grid y)
  int L;             // k-steps per wave
  int waves;         // 4 or 8 waves per workgroup (8 only for 16-row plans)
  int mrows;         // rows kept per tile: 4, 8 or 16 (8 only on 4 waves)
  bool single_group; // every wave's k-steps lie in one quantization group
  bool atomic;       // 4-row fp16 plans: splits meet in fixed-point atomics (else fp32 partials)
};

// Decode family (fp16 activations, 1 <= M <= 2): a workgroup of `waves` waves owns a
// column tile of 64 packed word-columns (512 output columns, 256 contiguous bytes of a
// row) and waves * ks k-steps of 32 rows, all of one wave's ks k-steps in one
// quantization group.  The K splits meet in fixed-point accumulators: n_tiles * 512 * mp
// 64-bit words, then as many float side words, zero before the call and left zero by it.
constexpr int kDecodeWords = 64;
constexpr int kDecodeCols = 8 * kDecodeWords;
constexpr int kDecodeMaxM = 2;
struct DecodePlan {
  int n_tiles;  // column tiles of kDecodeCols
  int splits;   // K splits (grid y), at most kFxMaxSplits
  int ks;       // k-steps per wave: 1 or 2
  int waves;    // waves per workgroup: 4 or 8
  int mp;       // rows: 1 or 2
  bool late;    // the workgroup's rows lie in one group: scale after the wave reduction
};
hipError_t launch_decode(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         const uint16_t* bias, int M, int K, int N, int g, const DecodePlan& p, uint64_t* accum,
                         float* side, uint16_t* y, hipStream_t stream);

// MFMA tile family.  Variants (rows x columns per workgroup, threads):
// 0: 256 x 128 (512: two k-groups of 4 waves), 1: 64 x 128 (256), 2: 32 x 128 (256).
// With splits > 1 each workgroup covers kps k-tiles of 64 and
// writes fp32 sums to partial, [splits][M][N]; a second kernel adds the splits and
// the bias.
constexpr int kTileVariants = 3;
constexpr int kTileBM[kTileVariants] = {256, 64, 32};
constexpr int kTileBN[kTileVariants] = {128, 128, 128};
constexpr int kTileThreads[kTileVariants] = {512, 256, 256};
constexpr int kTileBK = 64;
// Blocks of a tile grid with row_units row tiles (or table entries): whole runs of
// 8 * (256 / bn) blocks, so that the column tiles sharing 128-byte weight lines
// fall on one XCD (the block order of tile_kernel); padding blocks exit at once.
int64_t tile_blocks(int64_t row_units, int64_t N, int bn);
struct TilePlan {
  int variant;
  int splits;  // K splits (1: direct fp16 output)
  int kps;     // k-tiles of kTileBK per split
};

// Routed experts: the tile kernel's grouped mode.  Each workgroup takes one table
// entry and one column tile (in the block order of tile_kernel, with entries
// slowest, so that the unused entries at the end of the table take the last blocks);
// an entry is (expert, first sorted row, rows, 0), with expert < 0 for an unused
// entry (the workgroup exits).  Row r of the entry
// is routed slot sorted_slots[first + r], which reads x row slot / topk and writes
// y row slot.  Expert e's weights start e * w_stride words into qweight (and
// likewise for qzeros and scales).
struct MoeTiles {
  const int32_t* sorted_slots;
  const int32_t* table;
  int topk;
  int tiles;
  int64_t w_stride, z_stride, s_stride;
  // Set per launch: the launch takes the entries of lo <= rows < hi, each as sub
  // row tiles of the kernel's BM rows (sub * BM covers the table's block rows or
  // the entries' rows).
  int sub = 1;
  int lo = 0, hi = 1 << 30;
};
// Tile rows of the grouped variant picked for an average of `avg_rows` slots per
// expert, and the variant itself.
int moe_tile_variant(int64_t avg_rows, int* block_rows);
// Counting sort of S slots by expert into offsets [E + 1], sorted_slots [S] and the
// tile table [tiles][4] (tiles = ceil(S / block_rows) + E), one workgroup.
hipError_t launch_moe_align(const int32_t* expert_ids, int S, int E, int block_rows, int tiles,
                            int32_t* offsets, int32_t* sorted_slots, int32_t* table, hipStream_t stream);
hipError_t launch_tile_grouped(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                               const uint16_t* scales, int K, int N, int g, int variant, const MoeTiles& moe,
                               uint16_t* y, hipStream_t stream);

// out: float32 [K, N] (f16 = false) or fp16 [K, N] (f16 = true).
hipError_t launch_dequant(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                          int K, int N, int g, void* out, bool f16, hipStream_t stream);

// RTN writer: fp16 w [K, N] -> qweight [K, N/8], qzeros [K/g, N/8], scales fp16 [K/g, N].
// Groups of up to 256 rows take one fused pass (cache = rows per thread); longer
// groups take two passes over chunks of 128 rows (cpg chunks per group) and need
// scratch_bytes of device scratch for the chunks' min / max, fully written by the
// first pass before the second reads it.  grid = workgroups per launch.
struct RtnPlan {
  int cache = 1, block = 0, cols = 0, cpg = 1;
  bool two_pass = false;
  int64_t grid = 0, scratch_bytes = 0;
};
RtnPlan rtn_plan(int64_t K, int64_t N, int g);
hipError_t launch_quantize_rtn(const uint16_t* w, int K, int N, int g, bool sym, int32_t* qweight,
                               int32_t* qzeros, uint16_t* scales, void* scratch, hipStream_t stream);

// With p.splits > 1: atomic plans use accum, [n_tiles][4 * 256] 64-bit
// accumulators that are zero before the call and left zero by it; the others use
// partial, [n_tiles][splits][mrows * 256] fp32 scratch, and a second reduce kernel.
// x, bias and y are fp16 or (bf16 = true) bfloat16 bit patterns; scales are fp16.
// bfloat16 skinny plans with splits > 1 always use partial (fp32 partials and the
// reduce kernel), never accum.
// Routed experts on the skinny family, for at most kSkinnyExpertsMaxT tokens: block x
// is (chunk * experts + expert) * tiles + column tile.  The rows of a block are the
// tokens routed to its expert (those with some ids[t * topk + j] == e), in token
// order, from the (16 chunk)-th on, at most 16; row m goes to each slot t * topk + j
// of its token t with ids[t * topk + j] == e.  A block without rows exits before any
// load.  Expert e's weights start e * w_stride words into qweight (likewise qzeros
// and scales).  Accumulators and partials are per block.
constexpr int kSkinnyExpertsMaxT = 64;
struct SkinnyExperts {
  const int32_t* ids;  // [T * topk]
  int topk;
  int tiles;           // column tiles per expert
  int chunks;          // 16-row chunks of routed tokens per expert: ceil(T / 16)
  int experts;
  int64_t w_stride, z_stride, s_stride;
};
hipError_t launch_skinny_experts(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                                 const uint16_t* scales, int T, int K, int N, int g, const SkinnyPlan& p,
                                 const SkinnyExperts& ex, uint64_t* accum, float* partial, uint16_t* y,
                                 hipStream_t stream);

hipError_t launch_skinny(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                         const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                         const SkinnyPlan& p, bool bf16, uint64_t* accum, float* partial, uint16_t* y,
                         hipStream_t stream);

hipError_t launch_tile(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                       const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                       const TilePlan& p, bool bf16, float* partial, uint16_t* y, hipStream_t stream);

}  // namespace awq
