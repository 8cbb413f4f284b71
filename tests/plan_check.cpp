// Sweep of the host planner (w4a16_weight_only_amd/csrc/awq_plan.cpp) over shapes,
// built on the CPU with the address and undefined-behaviour sanitizers.  Every plan is
// checked against what the kernels rely on, stated here from the kernels' contracts
// rather than from the planner's own formulas:
//   - the launch fits HIP's limits (under 2^32 work-items along x, 2^16 workgroups
//     along y) and covers every output tile and every k-step exactly once;
//   - split counts fit the fixed-point word (127 arrivals);
//   - a skinny wave's k-steps lie in one quantization group when the plan says so, and
//     a skinny workgroup never touches more than 16 groups otherwise (counted exactly
//     over every split);
//   - the 32-bit offsets the kernels use (qweight bytes for skinny and decode, a
//     tile's x rows for the tile family) stay below 2^32;
//   - the workspace matches the kernels' buffers;
//   - the status codes follow the documented argument rules.
// Prints "plans checked: <n>" and exits 0, or prints the first failures and exits 1.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../include/awq_w4a16.h"
#include "../w4a16_weight_only_amd/csrc/awq_plan.h"

using namespace awq;

namespace {

long g_checked = 0, g_failed = 0, g_rejected = 0;
char g_ctx[256];

void fail(const char* what, int line) {
  std::fprintf(stderr, "FAIL line %d: %s  [%s]\n", line, what, g_ctx);
  if (++g_failed >= 20) std::exit(1);
}
#define CHECK(c) \
  do {           \
    if (!(c)) fail(#c, __LINE__); \
  } while (0)

constexpr int64_t k2p32 = int64_t(1) << 32;
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool format_ok(int64_t K, int64_t N, int64_t gs) {
  return K >= 1 && N >= 1 && N % 8 == 0 && (gs == -1 || (gs > 0 && K % gs == 0));
}
bool limits_ok(int64_t M, int64_t K, int64_t N, int64_t gs) {
  const int64_t D = int64_t(1) << 24;
  return format_ok(K, N, gs) && M >= 0 && K % 32 == 0 && N % 32 == 0 && (gs == -1 || gs % 32 == 0) && K <= D &&
         N <= D && M <= D;
}

void check_grid(int64_t gx, int64_t gy, int64_t block) {
  CHECK(gx >= 1 && gy >= 1);
  CHECK(gx * block < k2p32);
  CHECK(gy < 65536);
}

// Skinny plan over M rows of an N-column product (N: all columns the grid covers).
void check_skinny(const SkinnyPlan& s, int64_t M, int64_t K, int64_t N, int64_t g) {
  const int64_t T = K / 32, gsteps = g / 32;
  CHECK(M >= 1 && M <= 16);
  CHECK(s.mrows == 4 || s.mrows == 8 || s.mrows == 16);
  CHECK(s.mrows >= M);
  CHECK(s.waves == 4 || s.waves == 8);
  CHECK(s.waves == 4 || s.mrows == 16);
  CHECK(s.n_tiles == cdiv(N, 256));
  CHECK(s.L >= 1);
  const int64_t span = (int64_t)s.waves * s.L;  // k-steps per workgroup
  CHECK(s.splits == cdiv(T, span));
  CHECK(s.splits >= 1 && s.splits <= 127);
  CHECK(K * (N / 2) < k2p32 - 4096);  // qweight byte offsets
  CHECK(s.atomic == (M <= 2));
  CHECK(!s.fused || s.splits > 1);
  CHECK((int64_t)s.splits * s.mrows * 256 * 4 < k2p32);  // a tile's partials: 32-bit buffer offsets
  if (s.single_group) {
    CHECK(gsteps >= T || gsteps % s.L == 0);  // waves start at multiples of L
  } else {
    for (int64_t sp = 0; sp < s.splits; ++sp) {
      const int64_t a = sp * span, b = (a + span < T ? a + span : T) - 1;
      CHECK(b / gsteps - a / gsteps + 1 <= 16);
    }
  }
}

void check_gemm(int64_t M, int64_t K, int64_t N, int64_t gs, int cus, bool bf16) {
  std::snprintf(g_ctx, sizeof g_ctx, "gemm M=%" PRId64 " K=%" PRId64 " N=%" PRId64 " g=%" PRId64 " cus=%d bf16=%d", M,
                K, N, gs, cus, (int)bf16);
  ++g_checked;
  Plan p;
  const int st = plan_gemm(M, K, N, gs, cus, bf16, p);
  const int lim = limits_check(M, K, N, gs);
  if (!format_ok(K, N, gs)) {
    CHECK(st == AWQ_ERR_SHAPE || st == AWQ_ERR_GROUP);
    CHECK(st == lim);
    return;
  }
  if (M < 0) {
    CHECK(st == AWQ_ERR_SHAPE);
    return;
  }
  if (!limits_ok(M, K, N, gs)) {
    CHECK(st == AWQ_ERR_UNSUPPORTED);
    return;
  }
  if (st != AWQ_OK) {
    CHECK(st == AWQ_ERR_UNSUPPORTED);  // a launch beyond the grid or offset limits
    ++g_rejected;
    return;
  }
  if (M == 0) {
    CHECK(p.workspace_bytes() == 0);
    return;
  }
  const int64_t g = gs == -1 ? K : gs, T = K / 32;
  CHECK(p.block == 256 || p.block == 512);
  CHECK(p.accum_bytes >= 0 && p.partial_bytes >= 0);
  if (p.family == 2) {
    const DecodePlan& d = p.dp;
    CHECK(!bf16 && M <= 4 && d.mp == (M <= 2 ? M : 4));
    // three or four rows: grids of up to two rounds of three workgroups per CU, or N <= 8192
    CHECK(M <= 2 || (N <= 32768 && (d.n_tiles * d.splits <= 1536 || N <= 8192)));
    CHECK(d.ks == 1 || d.ks == 2);
    CHECK(d.waves == 4 || d.waves == 8);
    CHECK(p.block == 64 * d.waves);
    const int64_t span = (int64_t)d.ks * d.waves;
    CHECK(d.splits == cdiv(T, span));
    CHECK(d.splits >= 1 && d.splits <= 127);
    CHECK(g == K || (g / 32) % d.ks == 0);             // a wave's k-steps in one group
    CHECK(d.late == 0 || d.late == 1 || d.late == 2 || d.late == 4);
    // late > 0: the workgroup's waves form `late` equal parts, each inside one group
    CHECK(d.late == 0 || g == K || (g / 32) % (span / d.late) == 0);
    CHECK(d.late <= 1 || d.words == 32);
    CHECK(d.words == 64 || (d.words == 32 && d.waves == 4 && d.late >= 1));
    CHECK(d.words == 32 || d.splits > 0);
    CHECK(d.n_tiles == cdiv(N / 8, d.words));
    CHECK(p.grid_x == d.n_tiles && p.grid_y == d.splits);
    CHECK(K * (N / 2) < k2p32 - 4096);
    CHECK(p.accum_bytes == (d.splits > 1 ? (int64_t)d.n_tiles * 8 * d.words * d.mp * 12 : 0));
    CHECK(p.partial_bytes == 0);
    check_grid(p.grid_x, p.grid_y, p.block);
  } else if (p.family == 0) {
    const SkinnyPlan& s = p.sk;
    check_skinny(s, M, K, N, g);
    CHECK(p.block == 64 * s.waves);
    CHECK(p.grid_x == s.n_tiles && p.grid_y == s.splits);
    check_grid(p.grid_x, p.grid_y, p.block);
    const int64_t acc = s.splits == 1 ? 0
                        : (s.atomic && !bf16) ? (int64_t)s.n_tiles * s.mrows * 256 * 12
                                              : (s.fused ? (int64_t)s.n_tiles * 4 : 0);  // arrival counters
    const int64_t part = (s.splits > 1 && !(s.atomic && !bf16)) ? (int64_t)s.n_tiles * s.splits * s.mrows * 256 * 4 : 0;
    CHECK(p.accum_bytes == acc && p.partial_bytes == part);
  } else {
    CHECK(p.family == 1);
    CHECK(p.rows1 >= 1 && p.rows1 <= M);
    CHECK(p.accum_bytes == 0);
    const int64_t KT = cdiv(K, 64);
    auto check_launch = [&](const TileLaunch& t, int64_t rows) {
      const int v = t.tp.variant;
      CHECK(v >= 0 && v <= 2);
      const int64_t bm = v == 0 ? 256 : (v == 1 ? 64 : 32), threads = v == 0 ? 512 : 256;
      CHECK(t.block == threads);
      CHECK(t.tp.kps >= 1 && t.tp.splits == cdiv(KT, t.tp.kps));
      CHECK(t.tp.splits == 1 || t.tp.kps >= 8);
      const int64_t tiles = cdiv(rows, bm) * cdiv(N, 128);
      CHECK(t.grid_x >= tiles && t.grid_x % 16 == 0 && t.grid_x < tiles + 16 * cdiv(rows, bm) + 16);
      check_grid(t.grid_x, t.tp.splits, t.block);
      CHECK(bm * K * 2 < k2p32);  // 32-bit byte offsets of a tile's x rows
      if (t.tp.splits > 1) {
        CHECK(p.partial_bytes >= t.tp.splits * rows * N * 4);
        CHECK(rows * N / 4 + 256 < k2p32);  // the reduce launch
      }
    };
    check_launch(p.tile, p.rows1);
    CHECK(p.grid_x == p.tile.grid_x && p.grid_y == p.tile.tp.splits && p.block == p.tile.block);
    if (p.rows1 < M) {
      CHECK(p.tile.tp.variant == 0 && p.rows1 % 256 == 0);
      check_launch(p.tail, M - p.rows1);
    }
    if (p.tile.tp.splits == 1 && (p.rows1 == M || p.tail.tp.splits == 1)) CHECK(p.partial_bytes == 0);
  }
}

void check_moe(int64_t T, int64_t topk, int64_t E, int64_t K, int64_t N, int64_t gs, int cus) {
  std::snprintf(g_ctx, sizeof g_ctx, "moe T=%" PRId64 " topk=%" PRId64 " E=%" PRId64 " K=%" PRId64 " N=%" PRId64
                " g=%" PRId64 " cus=%d", T, topk, E, K, N, gs, cus);
  ++g_checked;
  MoePlan mp;
  const int st = plan_moe(T, topk, E, K, N, gs, cus, mp);
  if (T < 0 || topk < 1 || E < 1) {
    CHECK(st == AWQ_ERR_SHAPE);
    return;
  }
  if (st != AWQ_OK || T == 0) return;
  const int64_t S = T * topk, g = gs == -1 ? K : gs;
  CHECK(E <= 1024 && S < (int64_t(1) << 30) && T * K * 2 < k2p32);
  if (mp.skinny) {
    CHECK(T <= 64);
    const int64_t cols = E * mp.chunks * mp.tiles_e * 256;
    CHECK(mp.tiles_e == cdiv(N, 256) && mp.chunks == cdiv(T, 16));
    check_skinny(mp.sk, T < 16 ? T : 16, K, cols, g);
    check_grid(mp.sk.n_tiles, mp.sk.splits, 64 * mp.sk.waves);
    if (mp.sk.splits > 1 && mp.sk.atomic) CHECK(mp.accum_bytes == (int64_t)mp.sk.n_tiles * mp.sk.mrows * 256 * 12);
    if (mp.sk.splits > 1 && !mp.sk.atomic)
      CHECK(mp.partial_bytes == (int64_t)mp.sk.n_tiles * mp.sk.splits * mp.sk.mrows * 256 * 4);
  } else {
    CHECK(mp.variant >= 0 && mp.variant <= 2);
    CHECK(mp.block_rows == (mp.variant == 0 ? 256 : (mp.variant == 1 ? 64 : 32)));
    CHECK(mp.tiles == cdiv(S, mp.block_rows) + E);
    // Enough table entries: every expert's rows in tiles of block_rows.
    CHECK(mp.tiles >= cdiv(S, mp.block_rows));
    CHECK(mp.scratch_bytes == mp.tiles * 16 + (E + 1 + S + 4) * 4);
    const int64_t threads = mp.variant == 0 ? 512 : 256;
    CHECK(tile_blocks(mp.tiles, N, 128) * threads < k2p32);
    if (mp.variant == 0) CHECK(tile_blocks(mp.tiles * 2, N, 128) * 256 < k2p32);
  }
}

void check_rtn_plan(int64_t K, int64_t N, int64_t gs, int sym) {
  std::snprintf(g_ctx, sizeof g_ctx, "rtn K=%" PRId64 " N=%" PRId64 " g=%" PRId64 " sym=%d", K, N, gs, sym);
  ++g_checked;
  RtnPlan p;
  const int st = plan_rtn(K, N, gs, sym, p);
  if (!format_ok(K, N, gs)) {
    CHECK(st == AWQ_ERR_SHAPE || st == AWQ_ERR_GROUP);
    return;
  }
  if (sym != 0 && sym != 1) {
    CHECK(st == AWQ_ERR_SHAPE);
    return;
  }
  if (st != AWQ_OK) {
    CHECK(st == AWQ_ERR_UNSUPPORTED);
    return;
  }
  const int64_t g = gs == -1 ? K : gs, G = K / g;
  CHECK(p.block == 256 && p.cols == 128);
  CHECK(p.grid * p.block < k2p32);
  CHECK(p.grid == G * p.cpg * cdiv(N, 128));
  if (!p.two_pass) {
    CHECK(p.cache == 1 || p.cache == 2 || p.cache == 4 || p.cache == 8 || p.cache == 16);
    CHECK(16 * p.cache >= g && p.cpg == 1 && p.scratch_bytes == 0);  // 16 row slices x cache rows
  } else {
    CHECK(g > 256 && p.cache == 8 && (int64_t)p.cpg * 128 >= g && (int64_t)(p.cpg - 1) * 128 < g);
    CHECK(p.scratch_bytes == G * p.cpg * 2 * (N / 8) * 16);
  }
}

void check_pack(int64_t K, int64_t N, int64_t gs, int64_t qr, int64_t qc, int64_t zr, int64_t zc, int64_t sr, int64_t sc,
                int64_t bl) {
  std::snprintf(g_ctx, sizeof g_ctx, "pack K=%" PRId64 " N=%" PRId64 " g=%" PRId64, K, N, gs);
  ++g_checked;
  const int st = validate_pack(K, N, gs, qr, qc, zr, zc, sr, sc, bl);
  if (!format_ok(K, N, gs)) {
    CHECK(st == AWQ_ERR_SHAPE || st == AWQ_ERR_GROUP);
    CHECK(st == (K >= 1 && N >= 1 && N % 8 == 0 ? AWQ_ERR_GROUP : AWQ_ERR_SHAPE));
    return;
  }
  const int64_t G = gs == -1 ? 1 : K / gs;
  const bool shapes = qr == K && qc * 8 == N && zr == G && zc * 8 == N && sr == G && sc == N && (bl == -1 || bl == N);
  CHECK(st == (shapes ? AWQ_OK : AWQ_ERR_SHAPE));
}

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (g_rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int64_t pick(const std::vector<int64_t>& v) { return v[next() % v.size()]; }
// Log-uniform multiple of 32 in [32, 2^bits].
int64_t log_mult32(int bits) {
  const int e = 5 + (int)(next() % (uint64_t)(bits - 4));
  int64_t v = (int64_t)(next() % (uint64_t(1) << e)) + 1;
  return cdiv(v, 32) * 32;
}

}  // namespace

int main() {
  const int64_t D = int64_t(1) << 24, BIG = INT64_MAX, SMALL = INT64_MIN;
  const std::vector<int64_t> Ms = {SMALL, -1, 0, 1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
                                   129, 191, 192, 193, 255, 256, 257, 300, 511, 512, 513, 1000, 2047, 2048, 2100,
                                   4095, 8192, 65536, 1 << 20, D - 1, D, D + 1, BIG};
  const std::vector<int64_t> Ks = {SMALL, -32, 0, 8, 32, 64, 96, 128, 4096, 4128, 11008, 14336, 28672, 131072,
                                   1 << 22, (1 << 23) - 32, 1 << 23, (1 << 23) + 32, D, D + 32, BIG};
  const std::vector<int64_t> Ns = {SMALL, 0, 8, 32, 64, 544, 4096, 11008, 114688, 1 << 20, D, D + 32, BIG};
  const std::vector<int64_t> gfix = {SMALL, -2, -1, 0, 16, 32, 48, 64, 96, 128, 256, 1024, BIG};
  const int cuss[] = {1, 80, 256, 304};
  for (int64_t M : Ms)
    for (int64_t K : Ks)
      for (int64_t N : Ns) {
        std::vector<int64_t> gs = gfix;
        gs.push_back(K);
        for (int64_t g : gs)
          for (int cus : cuss)
            for (int bf16 = 0; bf16 < 2; ++bf16) check_gemm(M, K, N, g, cus, bf16 != 0);
      }
  // Random shapes in range, with groups that divide K.
  for (int i = 0; i < 400000; ++i) {
    const int64_t K = log_mult32(24), N = log_mult32(24);
    int64_t M = (int64_t)(next() % 4) == 0 ? (int64_t)(next() % 17) : (int64_t)(next() % (uint64_t)(1 + (next() % 3 == 0 ? D : 4096)));
    int64_t g = pick({-1, 32, 64, 128, 256, K});
    if (g != -1 && K % g != 0) g = 32;
    check_gemm(M, K, N, g, cuss[next() % 4], next() % 2 == 0);
  }
  // Routed experts.
  const std::vector<int64_t> Ts = {-1, 0, 1, 2, 3, 15, 16, 17, 40, 64, 65, 150, 768, 4096, 1 << 20, D, D + 1, BIG};
  const std::vector<int64_t> topks = {0, 1, 2, 8, 64, D + 1, BIG};
  const std::vector<int64_t> Es = {0, 1, 2, 8, 64, 128, 1024, 1025, BIG};
  const std::vector<int64_t> Kms = {32, 256, 2048, 4096, 7168, 1 << 20, D};
  const std::vector<int64_t> Nms = {32, 224, 1024, 2048, 14336, 1 << 20};
  for (int64_t T : Ts)
    for (int64_t tk : topks)
      for (int64_t E : Es)
        for (int64_t K : Kms)
          for (int64_t N : Nms)
            for (int64_t g : {int64_t(-1), int64_t(32), int64_t(128)})
              for (int cus : {1, 256}) check_moe(T, tk, E, K, N, g, cus);
  for (int i = 0; i < 200000; ++i) {
    const int64_t K = log_mult32(16), N = log_mult32(16);
    const int64_t g = K % 128 == 0 ? 128 : -1;
    check_moe((int64_t)(next() % 300), 1 + (int64_t)(next() % 8), 1 + (int64_t)(next() % 256), K, N, g, 256);
  }
  // RTN writer.
  for (int64_t K : Ks)
    for (int64_t N : Ns) {
      std::vector<int64_t> gs = gfix;
      gs.push_back(K);
      for (int64_t g : gs)
        for (int sym : {-1, 0, 1, 2}) check_rtn_plan(K, N, g, sym);
    }
  for (int i = 0; i < 100000; ++i) {
    const int64_t K = log_mult32(24), N = cdiv(log_mult32(24), 8) * 8;
    int64_t g = pick({-1, 32, 64, 128, 256, 512, K});
    if (g != -1 && K % g != 0) g = -1;
    check_rtn_plan(K, N, g, (int)(next() % 2));
  }
  // Pack validation: right shapes, and each one off in turn.
  for (int64_t K : Ks)
    for (int64_t N : Ns)
      for (int64_t g : gfix) {
        const int64_t G = g == -1 ? 1 : (g > 0 ? K / g : 1);
        const int64_t base[7] = {K, N / 8, G, N / 8, G, N, N};
        check_pack(K, N, g, base[0], base[1], base[2], base[3], base[4], base[5], base[6]);
        check_pack(K, N, g, base[0], base[1], base[2], base[3], base[4], base[5], -1);
        for (int j = 0; j < 7; ++j) {
          int64_t a[7];
          for (int t = 0; t < 7; ++t) a[t] = base[t];
          a[j] = a[j] == BIG ? 0 : a[j] + 1;
          check_pack(K, N, g, a[0], a[1], a[2], a[3], a[4], a[5], a[6]);
        }
      }
  if (g_failed) return 1;
  std::printf("plans checked: %ld (rejected for launch limits: %ld)\n", g_checked, g_rejected);
  return 0;
}
