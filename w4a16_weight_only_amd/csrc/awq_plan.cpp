// Host-only launch planning of the AWQ W4A16 library (declarations and the plan
// structures in awq_plan.h).  Every choice below is measured on MI355X; the comments
// give the measurements that decided it.
#include "awq_plan.h"

#include "../../include/awq_w4a16.h"

namespace awq {

int64_t groups_of(int64_t K, int64_t group_size) { return group_size == -1 ? 1 : K / group_size; }

// Effective group length passed to kernels: -1 means one group spanning K.
int eff_group(int64_t K, int64_t group_size) { return (int)(group_size == -1 ? K : group_size); }

int format_check(int64_t K, int64_t N, int64_t group_size) {
  if (K < 1 || N < 1 || N % 8 != 0) return AWQ_ERR_SHAPE;
  if (group_size == -1) return AWQ_OK;
  if (group_size <= 0 || K % group_size != 0) return AWQ_ERR_GROUP;
  return AWQ_OK;
}

int limits_check(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  int st = format_check(K, N, group_size);
  if (st != AWQ_OK) return st;
  if (M < 0) return AWQ_ERR_SHAPE;
  if (K % 32 != 0 || N % 32 != 0) return AWQ_ERR_UNSUPPORTED;
  if (group_size != -1 && group_size % 32 != 0) return AWQ_ERR_UNSUPPORTED;
  if (K > kMaxDim || N > kMaxDim || M > kMaxDim) return AWQ_ERR_UNSUPPORTED;
  // The tile family's 1-D grid must stay below 2^31 workgroups.
  if (((M + 127) / 128) * ((N + 63) / 64) >= (int64_t(1) << 31)) return AWQ_ERR_UNSUPPORTED;
  return AWQ_OK;
}

constexpr int kSkinnyWgPer2Cu = 4;  // 4-wave skinny workgroups counted per two compute units

// Skinny plan for M <= kSkinnyMaxM, or false when no launch shape fits the
// kernel's limits (at most kSkinnyMaxSplits splits, at most kSkinnyMaxGroups
// quantization groups per workgroup).
bool plan_skinny(int64_t M, int64_t K, int64_t N, int64_t g, int cus, SkinnyPlan& s) {
  // The kernel addresses qweight with 32-bit byte offsets.
  if (K * (N / 2) >= (int64_t(1) << 32) - 4096) return false;
  const int64_t T = K / kKStep;
  const int64_t gsteps = g / kKStep;  // g already resolved (-1 -> K)
  s.n_tiles = (int)((N + kSkinnyCols - 1) / kSkinnyCols);
  // One or two rows: 4-row plans (4 waves, splits meet in fixed-point atomics).
  // From three rows the atomics cost more than fp32 partials and the reduce kernel
  // (every split costs one returning atomic per row and column; M = 3, 4: 10-25%
  // faster with partials; M = 2 mixed, within 7% either way).  Three or four rows
  // on a layer whose 8-wave grid would take more than four rounds (above ~32 MB of
  // packed weights) take 4-row plans with partials: their smaller LDS reduction
  // buffer lets more workgroups share a compute unit (4096 x 114688: 69.5 -> 62.8
  // us; 8192 x 28672: 37.3 -> 33.3 us; routed experts at 3-4 tokens 6-10%); on
  // smaller layers they measured 0-3% slower than the 16-row plans.  Five to eight
  // rows on those layers take 8-row plans for the same reason (32 KB of LDS
  // reduction buffer instead of 64 KB; 4096 x 114688 M = 8: 73.8 -> 68.2 us;
  // 8192 x 28672 M = 6: 38.6 -> 35.6 us).  16-row plans
  // take 8 waves, or 4 waves (two per CU, shorter workgroups overlapping each
  // other's fixed phases) on those large layers: measured 8-15% faster on
  // 8192 x 28672, 28672 x 8192 and 4096 x 114688, 10-25% slower on layers of up
  // to 22 MB.
  const bool large = T * s.n_tiles > (int64_t)8 * cus * 4;
  s.mrows = (M <= 2 || (M <= 4 && large)) ? 4 : ((M <= 8 && large) ? 8 : 16);
  s.atomic = M <= 2;
  s.waves = (s.mrows == 4 || large) ? 4 : 8;
  const int64_t W = s.waves;
  // Whole grid resident in one round, counting two 4-wave workgroups per CU (three
  // fit when every wave stays inside one group; counting three gives more splits,
  // which measured slower at four rows) and one 8-wave workgroup (large LDS
  // reduction buffer).
  const int64_t cap = s.waves == 4 ? (int64_t)cus * kSkinnyWgPer2Cu / 2 : (int64_t)cus;
  int64_t L = (T * s.n_tiles + W * cap - 1) / (W * cap);
  const int64_t l_min = (T + W * kSkinnyMaxSplits - 1) / (W * kSkinnyMaxSplits);
  if (L < l_min) L = l_min;
  // At least two k-steps per wave, so that each wave's second step is in flight
  // while its first is multiplied (measured faster than one step per wave even
  // at half the workgroups); four for two rows, whose splits each cost one atomic
  // per row and column (half the splits measured faster).
  const int64_t l_floor = M == 2 ? 4 : 2;
  if (L < l_floor) L = l_floor;
  if (L > T) L = T;
  // 4-row plans on a grid of more than two rounds: keep each wave's run inside one
  // group (at most 4 k-steps).  Such waves need no per-group LDS tables and fewer
  // registers, so three workgroups share a compute unit, and the extra splits cost
  // one atomic (or partial) per output element each; on 16-row plans the extra
  // splits outweigh the gain (measured on 4096 x 114688, 8192 x 28672 and
  // 28672 x 8192 layers).
  if (s.mrows == 4 && gsteps < T && L > gsteps && T * s.n_tiles > W * cap * 2) L = gsteps < 4 ? gsteps : 4;
  auto splits_of = [&](int64_t l) { return (T + W * l - 1) / (W * l); };
  if (gsteps >= T) {
    s.single_group = true;  // one group spans K
  } else if (L <= gsteps) {
    while (gsteps % L != 0) ++L;  // stays <= gsteps: each wave's run in one group
    s.single_group = true;
  } else {
    s.single_group = false;
    // A workgroup's run of W*L steps may touch at most kSkinnyMaxGroups groups.
    if ((W * L - 1) / gsteps + 2 > kSkinnyMaxGroups) {
      int64_t l2 = ((int64_t)(kSkinnyMaxGroups - 2) * gsteps + 1) / W;
      if (l2 < 1) l2 = 1;
      if (l2 <= gsteps) {
        while (gsteps % l2 != 0) --l2;
        s.single_group = true;
      }
      L = l2;
    }
  }
  // 8- and 16-row plans whose waves span several groups: take one-group runs of at most 4
  // k-steps instead when that lowers (rounds of resident workgroups) x (k-steps
  // per wave + 2); the 2 stands for a workgroup's fixed cost (group data, the
  // reduction, the partial stores).  The round count decides it: 5.25 rounds of
  // 7-step waves lose to 7 full rounds of 4-step waves (4096 x 114688), while
  // 1 or 2 full rounds beat 2 or 3.5 (11008 x 4096, 28672 x 8192); measured.
  if (s.mrows >= 8 && !s.single_group) {
    int64_t l1 = gsteps < 4 ? gsteps : 4;
    while (gsteps % l1 != 0) --l1;
    auto cost = [&](int64_t l) { return (s.n_tiles * splits_of(l) + cap - 1) / cap * (l + 2); };
    if (splits_of(l1) <= kSkinnyMaxSplits && cost(l1) < cost(L)) {
      L = l1;
      s.single_group = true;
    }
  }
  if (splits_of(L) > kSkinnyMaxSplits) return false;
  s.L = (int)L;
  s.splits = (int)splits_of(L);
  // fp32 partials: the workgroup of a tile that arrives last sums them when the grid takes
  // two or more rounds of resident workgroups (its tail then overlaps the next round's
  // loads), and for 16-row plans only from five rounds (their partials are twice the
  // 8-row plans'); otherwise a reduce kernel does.  Measured, µs per call: 4 x 8192 x
  // 28672 34.2 -> 31.5, 3 / 8 / 16 x 4096 x 114688 61.3 / 67.4 / 77.9 -> 56.0 / 60.8 /
  // 75.0; 16 x 8192 x 28672 (four rounds) 43.9 -> 44.5; one-round grids 2-15% slower
  // fused (16 x 4096 x 11008 13.2 -> 13.6, 8 x 11008 x 4096 14.0 -> 16.3), where the
  // write-through of the partials, the arrival and the partial loads sit on the
  // critical path instead of the reduce launch.
  const int64_t per_cu = s.waves == 8 ? 1 : (s.mrows == 16 ? 2 : 3);
  const int64_t rounds = ((int64_t)s.n_tiles * s.splits + per_cu * cus - 1) / (per_cu * cus);
  s.fused = s.splits > 1 && rounds >= 2 && (s.mrows <= 8 || rounds >= 5);
  return true;
}

// Decode plan (fp16, 1 <= M <= 16), or false when the layer is outside its limits: a
// wave's k-steps must lie in one quantization group, the splits fit the fixed-point
// format, and qweight stays below 4 GiB (32-bit buffer offsets).  One workgroup per
// (512-column tile, K split) of waves * ks k-steps.
bool plan_decode(int64_t M, int64_t K, int64_t N, int64_t g, DecodePlan& d) {
  // Up to four rows: the returning fixed-point adds (M x N x splits of them) stay cheap
  // enough.  From five rows they cost more than the skinny family's fp32 partials (M = 8
  // on 11008 x 4096: 15.6 / 17.9 us for g-1 / g64 against 12.3 / 14.2), which keeps those.
  if (M < 1 || M > kDecodeMaxM) return false;
  if (K * (N / 2) >= (int64_t(1) << 32) - 4096) return false;
  const int64_t T = K / kKStep;
  d.mp = M <= 2 ? (int)M : 4;
  auto splits_of = [&](int ks, int waves) { return (T + (int64_t)ks * waves - 1) / ((int64_t)ks * waves); };
  auto ok = [&](int ks, int waves) {
    return (g == K || g % (kKStep * ks) == 0) && splits_of(ks, waves) <= kFxMaxSplits;
  };
  // Half-width tiles (256 columns, 4 waves): two k-steps per wave when g is K or a
  // multiple of 64, else one; the workgroup's waves then form 1, 2 or 4 parts that each
  // lie in one quantization group, summed and scaled apart after the wave reduction.
  // Half the columns per workgroup halves the K splits for the same grid, and with them
  // the fixed-point adds and how many meet at each address.  Measured, us per call, full
  // tiles -> half: 1 x 4096 x 4096 g128 6.38 -> 5.39, g64 6.88 -> 5.49, g32 6.97 -> 5.61;
  // 2 x 4096 x 4096 g128 8.00 -> 6.04; 1 x 4096 x 11008 g128 10.15 -> 8.33; 1 x 11008 x
  // 4096 g-1 9.02 -> 8.25, g32 11.18 -> 9.90; 2 x 11008 x 4096 g64 10.48 -> 9.42; 1 x 8192
  // x 28672 g128 35.9 -> 27.6.  Beyond 127 splits, full tiles: two k-steps per wave on 8
  // waves (one on 4 waves up to 128 k-steps), each wave scaling its own sums unless the
  // workgroup lies in one group.
  const int hks = (g == K || g % (2 * kKStep) == 0) ? 2 : 1;
  if (splits_of(hks, 4) <= kFxMaxSplits) {
    d.words = kDecodeWords / 2;
    d.ks = hks;
    d.waves = 4;
  } else {
    d.words = kDecodeWords;
    const int pref_ks = T <= 128 ? 1 : 2, pref_w = T <= 128 ? 4 : 8;
    const int cand[4][2] = {{pref_ks, pref_w}, {1, 4}, {1, 8}, {2, 8}};
    d.ks = 0;
    for (const auto& c : cand)
      if (ok(c[0], c[1])) {
        d.ks = c[0];
        d.waves = c[1];
        break;
      }
    if (d.ks == 0) return false;
  }
  d.n_tiles = (int)((N / 8 + d.words - 1) / d.words);
  d.splits = (int)splits_of(d.ks, d.waves);
  // Three or four rows: only while the grid stays within two rounds of three workgroups
  // per CU (1536 workgroups) or N <= 8192, and N <= 32768 (the adds' words stay under
  // 1.5 MB).  Measured against the skinny family, us per call: 3 x 2048 x 4096 8.90 ->
  // 5.91, 3 x 4096 x 4096 9.49 -> 6.95, 4 x 4096 x 4096 9.36 -> 7.39, 4 x 11008 x 4096
  // g64 13.68 -> 10.93, 4 x 4096 x 22016 17.46 -> 16.01, 4 x 28672 x 8192 35.8 -> 32.9;
  // kept on the skinny family: 3 x 8192 x 16384 20.5 (21.2 here), 4 x 8192 x 28672 32.3
  // (34.6), 3 x 4096 x 114688 56.0 (60.1).
  if (M > 2) {
    const int64_t grid = (int64_t)d.n_tiles * d.splits;
    if (N > 32768 || (grid > 1536 && N > 8192)) return false;
  }
  const int64_t span = (int64_t)kKStep * d.ks * d.waves;
  d.late = (g == K || g % span == 0) ? 1 : d.words == kDecodeWords ? 0 : (g % (span / 2) == 0 ? 2 : 4);
  return true;
}

int64_t decode_entries(const DecodePlan& d) { return (int64_t)d.n_tiles * 8 * d.words * d.mp; }

int64_t skinny_accum_entries(const SkinnyPlan& s) { return (int64_t)s.n_tiles * s.mrows * kSkinnyCols; }

// One launch of the tile family over M rows.
TileLaunch plan_tile(int64_t M, int64_t K, int64_t N, int cus) {
  auto tiles = [&](int v) {
    return ((M + kTileBM[v] - 1) / kTileBM[v]) * ((N + kTileBN[v] - 1) / kTileBN[v]);
  };
  // Row tile by M: 256 x 128 above 128 rows, 64 x 128 above 32, 32 x 128 below (a
  // tile taller than M wastes MFMA rows and x loads: 32 x 128 against 64 x 128 at
  // 17-32 rows measured 6-25% faster; at 65-128 rows two 64 x 128 row tiles beat
  // one 128 x 64 tile by 4-13%, and at 33-64 one 64 x 128 tile beats two 32 x 128).
  // Above 128 rows the product is MFMA-bound: K is split only while the tiles
  // leave compute units idle.  At or below 128 rows the weight stream dominates
  // and K is split to about two workgroups per compute unit (rounded down;
  // measured best over 1 to 4 per unit on 4096- to 28672-wide layers).  Every
  // split keeps at least 8 k-tiles.
  const int64_t fill = (int64_t)cus * 3 / 4;
  int v = M > 128 ? 0 : (M > 32 ? 1 : 2);
  // 129-192 rows with K <= 4096, where the 256-row tiles would be split over K: up to
  // three 64 x 128 row tiles instead (M = 130 on 4096 x 4096: 28.7 -> 21.8 us; M = 176
  // on 4096 x 11008: 61.1 -> 57.6 us).  With longer K (each weight dequantised by up
  // to three workgroups: M = 144 on 8192 x 8192 52.5 -> 69.6 us) or an unsplit grid
  // (M = 192 on 4096 x 28672: 83.8 -> 115.6 us) the 256-row tiles stay.
  if (v == 0 && M <= 192 && K <= 4096 && tiles(0) < fill) v = 1;
  const int64_t KT = (K + kTileBK - 1) / kTileBK;
  int64_t splits = 1;
  if (v == 0) {
    if (tiles(v) < fill) splits = ((int64_t)cus + tiles(v) - 1) / tiles(v);
  } else {
    splits = 2 * (int64_t)cus / tiles(v);
    if (splits < 1) splits = 1;
  }
  const int64_t max_splits = KT / 8 > 1 ? KT / 8 : 1;
  if (splits > max_splits) splits = max_splits;
  const int64_t kps = (KT + splits - 1) / splits;
  splits = (KT + kps - 1) / kps;
  TileLaunch t;
  t.tp.variant = v;
  t.tp.splits = (int)splits;
  t.tp.kps = (int)kps;
  t.block = kTileThreads[v];
  t.grid_x = tile_blocks((M + kTileBM[v] - 1) / kTileBM[v], N, kTileBN[v]);
  t.workgroups = tiles(v) * splits;
  return t;
}

Plan make_plan(int64_t M, int64_t K, int64_t N, int64_t g, int cus, bool bf16) {
  Plan p;
  if (!bf16 && plan_decode(M, K, N, g, p.dp)) {
    p.family = 2;
    p.grid_x = p.dp.n_tiles;
    p.grid_y = p.dp.splits;
    p.block = 64 * p.dp.waves;
    if (p.dp.splits > 1) p.accum_bytes = decode_entries(p.dp) * 12;  // word + side word
    return p;
  }
  if (M <= kSkinnyMaxM && plan_skinny(M, K, N, g, cus, p.sk)) {
    p.family = 0;
    p.grid_x = p.sk.n_tiles;
    p.grid_y = p.sk.splits;
    p.block = 64 * p.sk.waves;
    // 4-row fp16 plans: 64-bit fixed-point accumulators per tile entry; 16-row
    // plans and every bfloat16 plan: fp32 partials per (tile, split, entry).
    if (p.sk.splits > 1) {
      if (p.sk.atomic && !bf16) {
        p.accum_bytes = skinny_accum_entries(p.sk) * 12;
      } else {
        p.partial_bytes = (int64_t)p.sk.n_tiles * p.sk.splits * p.sk.mrows * kSkinnyCols * 4;
        if (p.sk.fused) p.accum_bytes = (int64_t)p.sk.n_tiles * 4;  // one arrival counter per column tile
      }
    }
  } else {
    p.family = 1;
    // A partly filled last 256-row tile whose workgroups would take one more round of
    // the compute units (one 256 x 128 workgroup per unit) goes to a second launch with
    // its own row tile and K splits: M = 2100 on 4096 x 4096, 137 -> 104 us; M = 1100,
    // 97 -> 77 us.  Where the round count stays, one launch is faster (M = 300 or
    // 600: the second launch's fixed cost and its reduce).
    const TileLaunch all = plan_tile(M, K, N, cus);
    p.rows1 = M;
    p.tile = all;
    const int64_t r = M % kTileBM[0];
    if (all.tp.variant == 0 && M > kTileBM[0] && r != 0) {
      const TileLaunch main = plan_tile(M - r, K, N, cus);
      if (main.rounds(cus) < all.rounds(cus)) {
        p.rows1 = M - r;
        p.tile = main;
        p.tail = plan_tile(r, K, N, cus);
      }
    }
    p.tp = p.tile.tp;
    p.block = p.tile.block;
    p.grid_x = p.tile.grid_x;
    p.grid_y = p.tile.tp.splits;
    const int64_t b1 = p.tile.tp.splits > 1 ? p.tile.tp.splits * p.rows1 * N * 4 : 0;
    const int64_t b2 = p.tail.tp.splits > 1 ? p.tail.tp.splits * (M - p.rows1) * N * 4 : 0;
    p.partial_bytes = b1 > b2 ? b1 : b2;  // the launches run in stream order
  }
  return p;
}

// Blocks of the tile grid (see the block order in tile_kernel): row_units units per
// run of 256 / bn column tiles, in whole runs of 8 (256 / bn) blocks.
int64_t tile_blocks(int64_t row_units, int64_t N, int bn) {
  const int64_t ct = 256 / bn;
  const int64_t n_tiles = (N + bn - 1) / bn;
  const int64_t units = row_units * ((n_tiles + ct - 1) / ct);
  return 8 * ct * ((units + 7) / 8);
}

// Grouped variants by slots per expert: 256 x 128 from 192, 64 x 128 above 32, and
// 32 x 128 for the few rows per expert of decode-sized batches, where the weights
// dominate and a smaller x tile lets four workgroups share a CU.  Below 192 rows two
// or three 64 x 128 row tiles beat one 256 x 128 tile that leaves rows idle; from
// 192 the larger tile wins (768 tokens over 8 experts, top-2: 300 against 390 us).
int moe_tile_variant(int64_t avg_rows, int* block_rows) {
  const int v = avg_rows >= 192 ? 0 : (avg_rows > 32 ? 1 : 2);
  *block_rows = kTileBM[v];
  return v;
}

RtnPlan rtn_plan(int64_t K, int64_t N, int g) {
  RtnPlan p;
  p.block = 64 * kRtnWaves;
  p.cols = 8 * kRtnWordCols;
  const int64_t ncb = (N + p.cols - 1) / p.cols;
  const int64_t G = K / g;
  if (g <= kRtnSlices * kRtnMaxFusedCache) {
    int cache = 1;
    while (kRtnSlices * cache < g) cache *= 2;
    p.cache = cache;
    p.two_pass = false;
    p.cpg = 1;
    p.scratch_bytes = 0;
  } else {
    p.cache = kRtnChunkCache;
    p.two_pass = true;
    p.cpg = (g + kRtnSlices * kRtnChunkCache - 1) / (kRtnSlices * kRtnChunkCache);
    p.scratch_bytes = G * p.cpg * 2 * (N / 8) * 16;
  }
  p.grid = G * p.cpg * ncb;
  return p;
}

int validate_pack(int64_t K, int64_t N, int64_t group_size, int64_t qweight_rows, int64_t qweight_cols,
                  int64_t qzeros_rows, int64_t qzeros_cols, int64_t scales_rows, int64_t scales_cols,
                  int64_t bias_len) {
  const int st = format_check(K, N, group_size);
  if (st != AWQ_OK) return st;
  const int64_t G = groups_of(K, group_size);
  if (qweight_rows != K || qweight_cols != N / 8) return AWQ_ERR_SHAPE;
  if (qzeros_rows != G || qzeros_cols != N / 8) return AWQ_ERR_SHAPE;
  if (scales_rows != G || scales_cols != N) return AWQ_ERR_SHAPE;
  if (bias_len != -1 && bias_len != N) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

namespace {

constexpr int64_t k2p32 = int64_t(1) << 32;

// HIP takes a launch's size in 32-bit work-item counts per dimension; grid y stays
// below 2^16 workgroups.
bool grid_fits(int64_t gx, int64_t gy, int64_t block) { return gx >= 1 && gy >= 1 && gx * block < k2p32 && gy < 65536; }

// One tile launch over `rows` rows: its grid, the 32-bit byte offsets of a tile's x
// rows from the tile's first row, and the grid of its split reduce (one thread per
// four outputs).
bool tile_launch_fits(const TileLaunch& t, int64_t rows, int64_t K, int64_t N) {
  if (!grid_fits(t.grid_x, t.tp.splits, t.block)) return false;
  if ((int64_t)kTileBM[t.tp.variant] * K * 2 >= k2p32) return false;
  if (t.tp.splits > 1 && rows * N / 4 + 256 >= k2p32) return false;
  return true;
}

}  // namespace

int plan_gemm(int64_t M, int64_t K, int64_t N, int64_t group_size, int cus, bool bf16, Plan& p) {
  p = Plan{};
  const int st = limits_check(M, K, N, group_size);
  if (st != AWQ_OK) return st;
  if (M == 0) return AWQ_OK;
  p = make_plan(M, K, N, eff_group(K, group_size), cus < 1 ? 1 : cus, bf16);
  bool ok;
  if (p.family == 1)
    ok = tile_launch_fits(p.tile, p.rows1, K, N) && (p.rows1 == M || tile_launch_fits(p.tail, M - p.rows1, K, N));
  else
    ok = grid_fits(p.grid_x, p.grid_y, p.block);
  return ok ? AWQ_OK : AWQ_ERR_UNSUPPORTED;
}

int64_t moe_tiles(int64_t S, int64_t E, int64_t block_rows) {
  const int64_t big = int64_t(1) << 40;
  if (S < 0 || E < 1 || block_rows < 1 || S >= big || E >= big) return -1;
  return (S + block_rows - 1) / block_rows + E;
}

int plan_moe(int64_t T, int64_t topk, int64_t E, int64_t K, int64_t N, int64_t group_size, int cus, MoePlan& mp) {
  mp = MoePlan{};
  if (T < 0 || topk < 1 || E < 1) return AWQ_ERR_SHAPE;
  if (T > kMaxDim || topk > kMaxDim) return AWQ_ERR_UNSUPPORTED;
  int st = limits_check(T * topk, K, N, group_size);
  if (st != AWQ_OK) return st;
  if (E > 1024 || T * topk >= (int64_t(1) << 30)) return AWQ_ERR_UNSUPPORTED;
  if (T * K * 2 >= k2p32) return AWQ_ERR_UNSUPPORTED;  // gathered rows use 32-bit offsets
  if (T == 0) return AWQ_OK;
  if (cus < 1) cus = 1;
  const int64_t S = T * topk;
  const int g = eff_group(K, group_size);
  // Few tokens: the skinny family batched over experts, each block taking up to 16
  // of its expert's routed tokens as rows, no alignment pass.  Up to 16 tokens always;
  // up to 64 when the experts average at most 8 slots (most experts then need one
  // 16-row chunk and stream their weights once) and each expert's packed weight is at
  // least 2 MB (shorter streams lose to the grouped tiles: per-block fixed costs and
  // the empty later chunks weigh more).  Measured, 4096 -> 2048 layers, 64 experts
  // top-2: 17 tokens 81.9 -> 47.2 us, 64 tokens 111.6 -> 85.5 us; 2048 -> 1024, 128
  // experts top-8, 64 tokens: 70.8 on the tiles against 94.6.
  mp.tiles_e = (N + kSkinnyCols - 1) / kSkinnyCols;
  mp.chunks = (T + kSkinnyMaxM - 1) / kSkinnyMaxM;
  const bool few = T <= kSkinnyMaxM || (T <= kSkinnyExpertsMaxT && S <= 8 * E && K * (N / 2) >= (int64_t(1) << 21));
  const int64_t blocks = E * mp.chunks * mp.tiles_e;
  if (few && blocks < (int64_t(1) << 31) &&
      plan_skinny(T < kSkinnyMaxM ? T : kSkinnyMaxM, K, blocks * kSkinnyCols, g, cus, mp.sk) &&
      grid_fits(mp.sk.n_tiles, mp.sk.splits, 64 * mp.sk.waves)) {
    mp.skinny = true;
    if (mp.sk.splits > 1) {
      if (mp.sk.atomic) mp.accum_bytes = skinny_accum_entries(mp.sk) * 12;
      else mp.partial_bytes = (int64_t)mp.sk.n_tiles * mp.sk.splits * mp.sk.mrows * kSkinnyCols * 4;
    }
    return AWQ_OK;
  }
  mp.sk = SkinnyPlan{};
  mp.variant = moe_tile_variant(S / E, &mp.block_rows);
  mp.tiles = moe_tiles(S, E, mp.block_rows);
  // Grids of the launches: 256-row tables take a second launch of two 64-row parts
  // per entry on 256 threads.
  const int bn = kTileBN[mp.variant];
  if (!grid_fits(tile_blocks(mp.tiles, N, bn), 1, kTileThreads[mp.variant])) return AWQ_ERR_UNSUPPORTED;
  if (mp.variant == 0 && !grid_fits(tile_blocks(mp.tiles * 2, N, bn), 1, kTileThreads[1])) return AWQ_ERR_UNSUPPORTED;
  // Scratch: tile table (16-byte entries), offsets, sorted slots.
  mp.scratch_bytes = mp.tiles * 16 + (E + 1 + S + 4) * 4;
  return AWQ_OK;
}

int plan_rtn(int64_t K, int64_t N, int64_t group_size, int sym, RtnPlan& p) {
  p = RtnPlan{};
  const int st = format_check(K, N, group_size);
  if (st != AWQ_OK) return st;
  if (sym != 0 && sym != 1) return AWQ_ERR_SHAPE;
  if (K > kMaxDim || N > kMaxDim) return AWQ_ERR_UNSUPPORTED;
  p = rtn_plan(K, N, eff_group(K, group_size));
  return grid_fits(p.grid, 1, p.block) ? AWQ_OK : AWQ_ERR_UNSUPPORTED;
}

}  // namespace awq
