// Internal launch interface between the C ABI (awq_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "awq_plan.h"

namespace awq {

hipError_t launch_decode(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         const uint16_t* bias, int M, int K, int N, int g, const DecodePlan& p, uint64_t* accum,
                         float* side, uint16_t* y, hipStream_t stream);

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
