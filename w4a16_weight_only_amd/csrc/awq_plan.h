// Host-only launch planning of the AWQ W4A16 library: argument and size checks, the
// choice of kernel family and launch shape for each product, and the workspace each
// plan needs.  Plain C++ (no HIP types), so that it also builds and runs on its own
// on the CPU, where a sweep over shapes checks every plan against the kernels' limits
// under the address and undefined-behaviour sanitizers.  Status codes are those of
// include/awq_w4a16.h.
#pragma once

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
constexpr int kSkinnyExpertsMaxT = 64;  // routed experts: most tokens on the skinny family

// Launch plan of the skinny family (chosen by plan_skinny below).
struct SkinnyPlan {
  int n_tiles;       // column tiles of kSkinnyCols
  int splits;        // K splits across workgroups (grid y)
  int L;             // k-steps per wave
  int waves;         // 4 or 8 waves per workgroup (8 only for 16-row plans)
  int mrows;         // rows kept per tile: 4, 8 or 16 (8 only on 4 waves)
  bool single_group; // every wave's k-steps lie in one quantization group
  bool atomic;       // 4-row fp16 plans: splits meet in fixed-point atomics (else fp32 partials)
  bool fused;        // fp32 partials summed by each tile's last workgroup (else a reduce kernel)
};

// Decode family (fp16 activations, 1 <= M <= 4): a workgroup of `waves` waves owns a
// column tile of `words` packed word-columns (64: 512 output columns, 256 contiguous
// bytes of a row; 32: 256 columns, 128 bytes, 4 waves only) and waves * ks k-steps of 32
// rows, all of one wave's ks k-steps in one quantization group.  The K splits meet in
// fixed-point accumulators: n_tiles * 8 * words * mp 64-bit words, then as many float
// side words, zero before the call and left zero by it.
constexpr int kDecodeWords = 64;
constexpr int kDecodeMaxM = 4;
struct DecodePlan {
  int n_tiles;  // column tiles of 8 * words columns
  int words;    // packed word-columns per tile: 64, or 32 (half-width tiles)
  int splits;   // K splits (grid y), at most kFxMaxSplits
  int ks;       // k-steps per wave: 1 or 2
  int waves;    // waves per workgroup: 4 or 8
  int mp;       // rows kept: 1, 2 or 4 (three rows padded to 4)
  int late;     // 1, 2 or 4: the workgroup's waves form that many equal parts, each in
                // one group, scaled after the wave reduction; 0: each wave scales its sums
};
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

// Tile rows of the grouped variant picked for an average of `avg_rows` slots per
// expert, and the variant itself.
int moe_tile_variant(int64_t avg_rows, int* block_rows);

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
// Geometry of the RTN writer's workgroups: 4 waves of 4 row slices x 16 word columns
// (every row load is a 256-byte run).
constexpr int kRtnWordCols = 16;
constexpr int kRtnWaves = 4;
constexpr int kRtnSlices = kRtnWaves * (64 / kRtnWordCols);  // row slices per workgroup
constexpr int kRtnMaxFusedCache = 16;  // fused pass for groups of up to 256 rows
constexpr int kRtnChunkCache = 8;      // longer groups: chunks of 128 rows
RtnPlan rtn_plan(int64_t K, int64_t N, int g);
// awq_quantize_rtn's checks and plan (sym 0 or 1).
int plan_rtn(int64_t K, int64_t N, int64_t group_size, int sym, RtnPlan& p);


// Largest K, N and M the library accepts.
constexpr int64_t kMaxDim = int64_t(1) << 24;

// Quantization groups along K (group_size -1: one group spanning K).
int64_t groups_of(int64_t K, int64_t group_size);
// Group length passed to kernels: K for group_size -1.
int eff_group(int64_t K, int64_t group_size);
// The format's own rules (the AWQ GEMM pack): K >= 1, N >= 1 and N % 8 == 0, group_size
// -1 or a positive divisor of K.
int format_check(int64_t K, int64_t N, int64_t group_size);
// format_check plus the kernels' limits: M >= 0, K % 32 == 0, N % 32 == 0, group_size
// -1 or a multiple of 32, sizes <= kMaxDim.
int limits_check(int64_t M, int64_t K, int64_t N, int64_t group_size);
// Tensor shapes against (K, N, group_size); bias_len -1 for no bias.
int validate_pack(int64_t K, int64_t N, int64_t group_size, int64_t qweight_rows, int64_t qweight_cols,
                  int64_t qzeros_rows, int64_t qzeros_cols, int64_t scales_rows, int64_t scales_cols,
                  int64_t bias_len);

// One launch of the tile family.
struct TileLaunch {
  TilePlan tp{};   // splits 0: no launch
  int64_t grid_x = 0;
  int block = 0;
  int64_t workgroups = 0;  // working workgroups (tiles x splits)
  // Rounds of 256 x 128 workgroups, one per compute unit at a time.
  int64_t rounds(int cus) const { return (workgroups + cus - 1) / cus; }
};

struct Plan {
  int family = 0;  // 0 skinny, 1 tile, 2 decode
  SkinnyPlan sk{};
  DecodePlan dp{};
  TilePlan tp{};
  // Tile family: the launch over rows [0, rows1), and over rows [rows1, M) when
  // rows1 < M (the last, partly filled 256-row tile in a launch of its own).
  int64_t rows1 = 0;
  TileLaunch tile{}, tail{};
  int64_t grid_x = 0;
  int grid_y = 0, block = 0;
  int64_t accum_bytes = 0;    // zero-maintained fixed-point words + side words
  int64_t partial_bytes = 0;  // scratch fp32 partials (skinny partial plans, split tile plans)
  int64_t workspace_bytes() const { return accum_bytes + partial_bytes; }
};

bool plan_skinny(int64_t M, int64_t K, int64_t N, int64_t g, int cus, SkinnyPlan& s);
bool plan_decode(int64_t M, int64_t K, int64_t N, int64_t g, DecodePlan& d);
// Fixed-point entries of a decode plan: one 64-bit word and one float side word per
// (tile, column, row).
int64_t decode_entries(const DecodePlan& d);
// Fixed-point entries of an atomic skinny plan, likewise.
int64_t skinny_accum_entries(const SkinnyPlan& s);
TileLaunch plan_tile(int64_t M, int64_t K, int64_t N, int cus);
// The plan of y = x . dequant(W) + bias for M rows (g resolved: K for one group) on a
// device of `cus` compute units; bf16 activations never take the decode family.
Plan make_plan(int64_t M, int64_t K, int64_t N, int64_t g, int cus, bool bf16 = false);
// limits_check, make_plan, and the check that every launch of the plan fits the
// hardware's grid limits and the kernels' 32-bit offsets (AWQ_ERR_UNSUPPORTED where
// not).  M = 0 gives an empty plan.
int plan_gemm(int64_t M, int64_t K, int64_t N, int64_t group_size, int cus, bool bf16, Plan& p);

// Routed experts, awq_moe_gemm: T tokens, topk slots each, E experts.
struct MoePlan {
  bool skinny = false;  // few tokens: the skinny kernel batched over experts
  SkinnyPlan sk{};
  int64_t tiles_e = 0, chunks = 0;  // skinny: column tiles per expert, 16-token chunks
  int64_t accum_bytes = 0, partial_bytes = 0;
  int variant = 0, block_rows = 0;  // grouped tiles: tile variant, rows per table entry
  int64_t tiles = 0;                // grouped tiles: table entries
  int64_t scratch_bytes = 0;        // grouped tiles: table, offsets, sorted slots
};
// Table entries of the grouped tiles: ceil(S / block_rows) + E, -1 for invalid
// arguments (or sizes of 2^40 and more).
int64_t moe_tiles(int64_t S, int64_t E, int64_t block_rows);
// Every check of awq_moe_gemm's sizes and, for T > 0, its plan.
int plan_moe(int64_t T, int64_t topk, int64_t E, int64_t K, int64_t N, int64_t group_size, int cus, MoePlan& mp);

}  // namespace awq
