// C ABI of the AWQ W4A16 library: argument checks, launch planning, workspace.
// The declarations and their contracts are in include/awq_w4a16.h.
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/awq_w4a16.h"
#include "awq_kernels.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int64_t kMaxDim = int64_t(1) << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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

struct TileLaunch {
  awq::TilePlan tp{};   // splits 0: no launch
  int grid_x = 0, block = 0;
  int64_t workgroups = 0;  // working workgroups (tiles x splits)
  // Rounds of 256 x 128 workgroups, one per compute unit at a time.
  int64_t rounds(int cus) const { return (workgroups + cus - 1) / cus; }
};

struct Plan {
  int family = 0;  // 0 skinny, 1 tile, 2 decode
  awq::SkinnyPlan sk{};
  awq::DecodePlan dp{};
  awq::TilePlan tp{};
  // Tile family: the launch over rows [0, rows1), and over rows [rows1, M) when
  // rows1 < M (the last, partly filled 256-row tile in a launch of its own).
  int64_t rows1 = 0;
  TileLaunch tile{}, tail{};
  int grid_x = 0, grid_y = 0, block = 0;
  int64_t accum_bytes = 0;    // zero-maintained fixed-point words + side words
  int64_t partial_bytes = 0;  // scratch fp32 partials (8-wave skinny plans, split tile plans)
  int64_t workspace_bytes() const { return accum_bytes + partial_bytes; }
};

// Compute units of the current device (cached per device ordinal).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

constexpr int kSkinnyWgPer2Cu = 4;  // 4-wave skinny workgroups counted per two compute units

// Skinny plan for M <= kSkinnyMaxM, or false when no launch shape fits the
// kernel's limits (at most kSkinnyMaxSplits splits, at most kSkinnyMaxGroups
// quantization groups per workgroup).
bool plan_skinny(int64_t M, int64_t K, int64_t N, int64_t g, int cus, awq::SkinnyPlan& s) {
  // The kernel addresses qweight with 32-bit byte offsets.
  if (K * (N / 2) >= (int64_t(1) << 32) - 4096) return false;
  const int64_t T = K / awq::kKStep;
  const int64_t gsteps = g / awq::kKStep;  // g already resolved (-1 -> K)
  s.n_tiles = (int)((N + awq::kSkinnyCols - 1) / awq::kSkinnyCols);
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
  const int64_t l_min = (T + W * awq::kSkinnyMaxSplits - 1) / (W * awq::kSkinnyMaxSplits);
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
    if ((W * L - 1) / gsteps + 2 > awq::kSkinnyMaxGroups) {
      int64_t l2 = ((int64_t)(awq::kSkinnyMaxGroups - 2) * gsteps + 1) / W;
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
    if (splits_of(l1) <= awq::kSkinnyMaxSplits && cost(l1) < cost(L)) {
      L = l1;
      s.single_group = true;
    }
  }
  if (splits_of(L) > awq::kSkinnyMaxSplits) return false;
  s.L = (int)L;
  s.splits = (int)splits_of(L);
  return true;
}

// Decode plan (fp16, 1 <= M <= 16), or false when the layer is outside its limits: a
// wave's k-steps must lie in one quantization group, the splits fit the fixed-point
// format, and qweight stays below 4 GiB (32-bit buffer offsets).  One workgroup per
// (512-column tile, K split) of waves * ks k-steps.
bool plan_decode(int64_t M, int64_t K, int64_t N, int64_t g, awq::DecodePlan& d) {
  // One or two rows: the returning fixed-point adds (M x N x splits of them) stay cheap.
  // From three rows they cost more than the older skinny family's fp32 partials (M = 16
  // on 4096 x 11008: 27.6 us at best against 13.9; M = 8 on 11008 x 4096: 17.2 against
  // 12.9), which keeps those.
  if (M < 1 || M > awq::kDecodeMaxM) return false;
  if (K * (N / 2) >= (int64_t(1) << 32) - 4096) return false;
  const int64_t T = K / awq::kKStep;
  d.n_tiles = (int)((N / 8 + awq::kDecodeWords - 1) / awq::kDecodeWords);
  d.mp = (int)M;
  auto splits_of = [&](int ks, int waves) { return (T + (int64_t)ks * waves - 1) / ((int64_t)ks * waves); };
  auto ok = [&](int ks, int waves) {
    return (g == K || g % (awq::kKStep * ks) == 0) && splits_of(ks, waves) <= awq::kFxMaxSplits;
  };
  // Up to 128 k-steps (K <= 4096): one k-step per wave, 4 waves (4096 x 4096: 6.2 us
  // against 6.6-8.2 for the other shapes).  Longer K: two k-steps per wave on 8-wave
  // workgroups (11008 x 4096: 8.9 us against 9.7-12.8).
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
  d.splits = (int)splits_of(d.ks, d.waves);
  d.late = g == K || g % ((int64_t)awq::kKStep * d.ks * d.waves) == 0;
  return true;
}

// Zero-maintained fixed-point workspace of a decode plan: 64-bit words, then float
// side words, one of each per (tile, column, padded row).
int64_t decode_entries(const awq::DecodePlan& d) { return (int64_t)d.n_tiles * awq::kDecodeCols * d.mp; }

// One launch of the tile family over M rows.
TileLaunch plan_tile(int64_t M, int64_t K, int64_t N, int cus) {
  auto tiles = [&](int v) {
    return ((M + awq::kTileBM[v] - 1) / awq::kTileBM[v]) * ((N + awq::kTileBN[v] - 1) / awq::kTileBN[v]);
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
  const int64_t KT = (K + awq::kTileBK - 1) / awq::kTileBK;
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
  t.block = awq::kTileThreads[v];
  t.grid_x = (int)awq::tile_blocks((M + awq::kTileBM[v] - 1) / awq::kTileBM[v], N, awq::kTileBN[v]);
  t.workgroups = tiles(v) * splits;
  return t;
}

Plan make_plan(int64_t M, int64_t K, int64_t N, int64_t g, int cus, bool bf16 = false) {
  Plan p;
  if (!bf16 && plan_decode(M, K, N, g, p.dp)) {
    p.family = 2;
    p.grid_x = p.dp.n_tiles;
    p.grid_y = p.dp.splits;
    p.block = 64 * p.dp.waves;
    if (p.dp.splits > 1) p.accum_bytes = decode_entries(p.dp) * 12;
    return p;
  }
  if (M <= awq::kSkinnyMaxM && plan_skinny(M, K, N, g, cus, p.sk)) {
    p.family = 0;
    p.grid_x = p.sk.n_tiles;
    p.grid_y = p.sk.splits;
    p.block = 64 * p.sk.waves;
    // 4-row fp16 plans: 64-bit fixed-point accumulators per tile entry; 16-row
    // plans and every bfloat16 plan: fp32 partials per (tile, split, entry).
    if (p.sk.splits > 1) {
      if (p.sk.atomic && !bf16) p.accum_bytes = (int64_t)p.sk.n_tiles * p.sk.mrows * awq::kSkinnyCols * 12;
      else p.partial_bytes = (int64_t)p.sk.n_tiles * p.sk.splits * p.sk.mrows * awq::kSkinnyCols * 4;
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
    const int64_t r = M % awq::kTileBM[0];
    if (all.tp.variant == 0 && M > awq::kTileBM[0] && r != 0) {
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

// Library-owned split-K workspace, one per (device, stream), in two buffers:
//   accum    fixed-point words and their float side words; zeroed once at allocation
//            and left zero by every call that uses them, so they never hold anything
//            else between calls;
//   partial  fp32 scratch, fully written before it is read in each call.
// A buffer that must grow is replaced, and the old one is retired, never freed while
// the library is loaded (a graph captured earlier may still hold its address and replay
// into it); awq_release_workspace() frees retired and current buffers on request.  A
// stream that is being captured cannot grow its workspace: that call fails with
// AWQ_ERR_UNSUPPORTED before enqueueing anything.
struct Buffer {
  void* ptr = nullptr;
  int64_t bytes = 0;
};
struct Workspace {
  Buffer accum, partial;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;  // (device, buffer) replaced by a larger one

int ensure(int dev, Buffer& b, int64_t need, bool zero, hipStream_t stream) {
  if (need <= 0 || (b.ptr && need <= b.bytes)) return AWQ_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return AWQ_ERR_HIP;
  if (cap != hipStreamCaptureStatusNone) return AWQ_ERR_UNSUPPORTED;
  const int64_t bytes = need + need / 4;  // headroom against frequent regrowth
  void* ptr = nullptr;
  if (hipMalloc(&ptr, (size_t)bytes) != hipSuccess) return AWQ_ERR_HIP;
  // Zeroed in stream order, before any kernel of this stream can use the buffer.
  if (zero && hipMemsetAsync(ptr, 0, (size_t)bytes, stream) != hipSuccess) {
    (void)hipFree(ptr);
    return AWQ_ERR_HIP;
  }
  if (b.ptr) g_retired.emplace_back(dev, b.ptr);
  b.ptr = ptr;
  b.bytes = bytes;
  return AWQ_OK;
}

int get_workspace(const Plan& p, hipStream_t stream, uint64_t** accum, float** partial) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AWQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& ws = g_ws[{dev, stream}];
  int st = ensure(dev, ws.accum, p.accum_bytes, true, stream);
  if (st != AWQ_OK) return st;
  st = ensure(dev, ws.partial, p.partial_bytes, false, stream);
  if (st != AWQ_OK) return st;
  *accum = reinterpret_cast<uint64_t*>(ws.accum.ptr);
  *partial = reinterpret_cast<float*>(ws.partial.ptr);
  return AWQ_OK;
}

// Scratch that is fully written before it is read within one call: the partial
// buffer of the same (device, stream) workspace.
int get_scratch(int64_t bytes, hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AWQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& ws = g_ws[{dev, stream}];
  const int st = ensure(dev, ws.partial, bytes, false, stream);
  if (st != AWQ_OK) return st;
  *out = ws.partial.ptr;
  return AWQ_OK;
}

// Allocation-free workspace for awq_gemm_noalloc: one file-scope device array per GPU
// (each device that runs the library holds its own copy until the process ends).  The
// first kScratchWordBytes hold fixed-point words and their side words, zero between
// calls like the workspace above (a fill kernel clears them on the device's first call);
// the rest holds fp32 partials, fully written before they are read in each call.  The
// two regions never trade places, so neither kind of plan can break the other's
// invariant.  In host code `scratch` only names the symbol: kernels get the address
// hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchWordBytes = int64_t(2) << 20;
constexpr int64_t kScratchPartialBytes = int64_t(62) << 20;
__device__ __align__(256) unsigned char scratch[kScratchWordBytes + kScratchPartialBytes];

__global__ void zero_words_kernel(u32x4_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;  // device -> address of `scratch` on that device

int get_static_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AWQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return AWQ_ERR_HIP;
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream, static_cast<u32x4_t*>(ptr),
                       kScratchWordBytes / 16);
    if (hipGetLastError() != hipSuccess) return AWQ_ERR_HIP;
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return AWQ_OK;
}

// The split-K buffers of plan p: the stream's grown workspace, or (noalloc) the static
// scratch, AWQ_ERR_UNSUPPORTED when the plan needs more than it holds.
int workspace_for(const Plan& p, hipStream_t stream, bool noalloc, uint64_t** accum, float** partial) {
  if (!noalloc) return get_workspace(p, stream, accum, partial);
  if (p.accum_bytes > kScratchWordBytes || p.partial_bytes > kScratchPartialBytes) return AWQ_ERR_UNSUPPORTED;
  void* base = nullptr;
  const int st = get_static_scratch(stream, &base);
  if (st != AWQ_OK) return st;
  *accum = static_cast<uint64_t*>(base);
  *partial = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + kScratchWordBytes);
  return AWQ_OK;
}

}  // namespace

extern "C" {

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_NULL: return "AWQ_ERR_NULL: a required pointer is NULL";
    case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE: tensor shapes disagree with K, N, group_size (or N % 8 != 0)";
    case AWQ_ERR_GROUP: return "AWQ_ERR_GROUP: group_size must be -1 or a positive divisor of K";
    case AWQ_ERR_ALIGN: return "AWQ_ERR_ALIGN: tensor base pointers must be 16-byte aligned";
    case AWQ_ERR_UNSUPPORTED:
      return "AWQ_ERR_UNSUPPORTED: needs K % 32 == 0, N % 32 == 0, group_size -1 or a multiple of 32, sizes <= 2^24";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP: the HIP runtime reported an error";
    default: return "AWQ: unknown status";
  }
}

int awq_validate_pack(int64_t K, int64_t N, int64_t group_size, int64_t qweight_rows,
                      int64_t qweight_cols, int64_t qzeros_rows, int64_t qzeros_cols,
                      int64_t scales_rows, int64_t scales_cols, int64_t bias_len) {
  const int st = format_check(K, N, group_size);
  if (st != AWQ_OK) return st;
  const int64_t G = groups_of(K, group_size);
  if (qweight_rows != K || qweight_cols != N / 8) return AWQ_ERR_SHAPE;
  if (qzeros_rows != G || qzeros_cols != N / 8) return AWQ_ERR_SHAPE;
  if (scales_rows != G || scales_cols != N) return AWQ_ERR_SHAPE;
  if (bias_len != -1 && bias_len != N) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

int awq_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return AWQ_ERR_HIP;
  int st = AWQ_OK;
  auto release = [&](int dev, void* ptr) {
    if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess || hipFree(ptr) != hipSuccess)
      st = AWQ_ERR_HIP;
  };
  for (auto& r : g_retired) release(r.first, r.second);
  g_retired.clear();
  for (auto& w : g_ws) {
    if (w.second.accum.ptr) release(w.first.first, w.second.accum.ptr);
    if (w.second.partial.ptr) release(w.first.first, w.second.partial.ptr);
  }
  g_ws.clear();
  if (hipSetDevice(cur) != hipSuccess) st = AWQ_ERR_HIP;
  return st;
}

int awq_check_limits(int64_t M, int64_t K, int64_t N, int64_t group_size) {
  return limits_check(M, K, N, group_size);
}

int awq_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t group_size, int* family, int* splits,
                  int* grid_x, int* grid_y, int* block, int64_t* workspace_bytes) {
  const int st = limits_check(M, K, N, group_size);
  if (st != AWQ_OK) return st;
  // Planning uses a 256-CU device when no device is visible (host-only callers).
  int cus = 256;
  int count = 0;
  if (hipGetDeviceCount(&count) == hipSuccess && count > 0) cus = device_cus();
  else (void)hipGetLastError();
  const Plan p = make_plan(M, K, N, eff_group(K, group_size), cus);
  if (family) *family = p.family;
  if (splits) *splits = p.family == 2 ? p.dp.splits : (p.family == 0 ? p.sk.splits : p.tp.splits);
  if (grid_x) *grid_x = p.grid_x;
  if (grid_y) *grid_y = p.grid_y;
  if (block) *block = p.block;
  if (workspace_bytes) *workspace_bytes = p.workspace_bytes();
  return AWQ_OK;
}

int awq_gemm_plan_tail(int64_t M, int64_t K, int64_t N, int64_t group_size, int64_t* rows, int* splits,
                       int* grid_x, int* grid_y, int* block) {
  const int st = limits_check(M, K, N, group_size);
  if (st != AWQ_OK) return st;
  int cus = 256;
  int count = 0;
  if (hipGetDeviceCount(&count) == hipSuccess && count > 0) cus = device_cus();
  else (void)hipGetLastError();
  const Plan p = make_plan(M, K, N, eff_group(K, group_size), cus);
  const bool tail = p.family == 1 && p.rows1 < M;
  if (rows) *rows = tail ? M - p.rows1 : 0;
  if (splits) *splits = tail ? p.tail.tp.splits : 0;
  if (grid_x) *grid_x = tail ? p.tail.grid_x : 0;
  if (grid_y) *grid_y = tail ? p.tail.tp.splits : 0;
  if (block) *block = tail ? p.tail.block : 0;
  return AWQ_OK;
}

namespace {
int dequant_common(const int32_t* qweight, const int32_t* qzeros, const void* scales_f16, int64_t K, int64_t N,
                   int64_t group_size, void* out, bool f16, hipStream_t stream) {
  const int st = limits_check(0, K, N, group_size);
  if (st != AWQ_OK) return st;
  if (!qweight || !qzeros || !scales_f16 || !out) return AWQ_ERR_NULL;
  if (!aligned16(qweight) || !aligned16(qzeros) || !aligned16(scales_f16) || !aligned16(out))
    return AWQ_ERR_ALIGN;
  hipError_t e = awq::launch_dequant(qweight, qzeros, static_cast<const uint16_t*>(scales_f16), (int)K,
                                     (int)N, eff_group(K, group_size), out, f16, stream);
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}
}  // namespace

int awq_dequant(const int32_t* qweight, const int32_t* qzeros, const void* scales_f16, int64_t K,
                int64_t N, int64_t group_size, float* out, struct ihipStream_t* stream) {
  return dequant_common(qweight, qzeros, scales_f16, K, N, group_size, out, false, stream);
}

int awq_dequant_f16(const int32_t* qweight, const int32_t* qzeros, const void* scales_f16, int64_t K,
                    int64_t N, int64_t group_size, void* out_f16, struct ihipStream_t* stream) {
  return dequant_common(qweight, qzeros, scales_f16, K, N, group_size, out_f16, true, stream);
}

int awq_quantize_rtn(const void* w_f16, int64_t K, int64_t N, int64_t group_size, int sym, int32_t* qweight,
                     int32_t* qzeros, void* scales_f16, struct ihipStream_t* stream) {
  int st = format_check(K, N, group_size);
  if (st != AWQ_OK) return st;
  if (sym != 0 && sym != 1) return AWQ_ERR_SHAPE;
  if (K > kMaxDim || N > kMaxDim) return AWQ_ERR_UNSUPPORTED;
  const int g = eff_group(K, group_size);
  const awq::RtnPlan p = awq::rtn_plan(K, N, g);
  if (p.grid >= (int64_t(1) << 31)) return AWQ_ERR_UNSUPPORTED;
  if (!w_f16 || !qweight || !qzeros || !scales_f16) return AWQ_ERR_NULL;
  if (!aligned16(w_f16) || !aligned16(qweight) || !aligned16(qzeros) || !aligned16(scales_f16))
    return AWQ_ERR_ALIGN;
  void* scratch = nullptr;
  if (p.scratch_bytes > 0) {
    st = get_scratch(p.scratch_bytes, stream, &scratch);
    if (st != AWQ_OK) return st;
  }
  hipError_t e = awq::launch_quantize_rtn(static_cast<const uint16_t*>(w_f16), (int)K, (int)N, g, sym != 0, qweight,
                                          qzeros, static_cast<uint16_t*>(scales_f16), scratch, stream);
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}

namespace {
int gemm_common(const void* x_f16, const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                const void* bias_f16, int64_t M, int64_t K, int64_t N, int64_t group_size, void* y_f16,
                bool bf16, hipStream_t stream, bool noalloc = false) {
  const int st = limits_check(M, K, N, group_size);
  if (st != AWQ_OK) return st;
  if (M == 0) return AWQ_OK;
  if (!x_f16 || !qweight || !qzeros || !scales_f16 || !y_f16) return AWQ_ERR_NULL;
  if (!aligned16(x_f16) || !aligned16(qweight) || !aligned16(qzeros) || !aligned16(scales_f16) ||
      !aligned16(y_f16) || (bias_f16 && !aligned16(bias_f16)))
    return AWQ_ERR_ALIGN;
  const int g = eff_group(K, group_size);
  const Plan p = make_plan(M, K, N, g, device_cus(), bf16);
  const auto* x = static_cast<const uint16_t*>(x_f16);
  const auto* sc = static_cast<const uint16_t*>(scales_f16);
  const auto* b = static_cast<const uint16_t*>(bias_f16);
  auto* y = static_cast<uint16_t*>(y_f16);
  hipError_t e;
  if (p.family == 2) {
    uint64_t* accum = nullptr;
    float* partial = nullptr;
    if (p.dp.splits > 1) {
      const int ws = workspace_for(p, stream, noalloc, &accum, &partial);
      if (ws != AWQ_OK) return ws;
    }
    float* side = accum ? reinterpret_cast<float*>(accum + decode_entries(p.dp)) : nullptr;
    e = awq::launch_decode(x, qweight, qzeros, sc, b, (int)M, (int)K, (int)N, g, p.dp, accum, side, y, stream);
  } else if (p.family == 0) {
    uint64_t* accum = nullptr;
    float* partial = nullptr;
    if (p.sk.splits > 1) {
      const int ws = workspace_for(p, stream, noalloc, &accum, &partial);
      if (ws != AWQ_OK) return ws;
    }
    // Fixed-point plans: the float side words follow the accumulator words.
    if (p.sk.splits > 1 && p.sk.atomic && !bf16)
      partial = reinterpret_cast<float*>(accum + (int64_t)p.sk.n_tiles * p.sk.mrows * awq::kSkinnyCols);
    e = awq::launch_skinny(x, qweight, qzeros, sc, b, (int)M, (int)K, (int)N, g, p.sk, bf16, accum, partial, y,
                           stream);
  } else {
    uint64_t* accum = nullptr;
    float* partial = nullptr;
    if (p.tp.splits > 1 || p.tail.tp.splits > 1) {
      const int ws = workspace_for(p, stream, noalloc, &accum, &partial);
      if (ws != AWQ_OK) return ws;
    }
    e = awq::launch_tile(x, qweight, qzeros, sc, b, (int)p.rows1, (int)K, (int)N, g, p.tp, bf16, partial, y,
                         stream);
    if (e == hipSuccess && p.rows1 < M)
      e = awq::launch_tile(x + p.rows1 * K, qweight, qzeros, sc, b, (int)(M - p.rows1), (int)K, (int)N, g,
                           p.tail.tp, bf16, partial, y + p.rows1 * N, stream);
  }
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}
}  // namespace

int64_t awq_moe_tiles(int64_t S, int64_t E, int64_t block_rows) {
  if (S < 0 || E < 1 || block_rows < 1) return -1;
  return (S + block_rows - 1) / block_rows + E;
}

int awq_moe_align(const int32_t* expert_ids, int64_t S, int64_t E, int64_t block_rows, int32_t* offsets,
                  int32_t* sorted_slots, int32_t* tile_table, struct ihipStream_t* stream) {
  if (S < 0 || E < 1 || block_rows < 1) return AWQ_ERR_SHAPE;
  if (E > 1024 || S >= (int64_t(1) << 30)) return AWQ_ERR_UNSUPPORTED;
  if (!offsets || !tile_table || (S > 0 && (!expert_ids || !sorted_slots))) return AWQ_ERR_NULL;
  if (!aligned16(tile_table)) return AWQ_ERR_ALIGN;
  const int64_t tiles = awq_moe_tiles(S, E, block_rows);
  hipError_t e = awq::launch_moe_align(expert_ids, (int)S, (int)E, (int)block_rows, (int)tiles, offsets, sorted_slots,
                                       tile_table, stream);
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}

int awq_moe_gemm(const void* x_f16, const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                 const int32_t* expert_ids, int64_t T, int64_t topk, int64_t E, int64_t K, int64_t N,
                 int64_t group_size, void* y_f16, struct ihipStream_t* stream) {
  if (T < 0 || topk < 1 || E < 1) return AWQ_ERR_SHAPE;
  int st = limits_check(T * topk, K, N, group_size);
  if (st != AWQ_OK) return st;
  if (E > 1024 || T * topk >= (int64_t(1) << 30)) return AWQ_ERR_UNSUPPORTED;
  if (T * K * 2 >= (int64_t(1) << 32)) return AWQ_ERR_UNSUPPORTED;  // gathered rows use 32-bit offsets
  if (T == 0) return AWQ_OK;
  if (!x_f16 || !qweight || !qzeros || !scales_f16 || !expert_ids || !y_f16) return AWQ_ERR_NULL;
  if (!aligned16(x_f16) || !aligned16(qweight) || !aligned16(qzeros) || !aligned16(scales_f16) || !aligned16(y_f16))
    return AWQ_ERR_ALIGN;
  const int64_t S = T * topk;
  const int g = eff_group(K, group_size);
  const int64_t G = K / g;
  // Few tokens: the skinny family batched over experts, each block taking up to 16
  // of its expert's routed tokens as rows, no alignment pass.  Up to 16 tokens always;
  // up to 64 when the experts average at most 8 slots (most experts then need one
  // 16-row chunk and stream their weights once) and each expert's packed weight is at
  // least 2 MB (shorter streams lose to the grouped tiles: per-block fixed costs and
  // the empty later chunks weigh more).  Measured, 4096 -> 2048 layers, 64 experts
  // top-2: 17 tokens 81.9 -> 47.2 us, 64 tokens 111.6 -> 85.5 us; 2048 -> 1024, 128
  // experts top-8, 64 tokens: 70.8 on the tiles against 94.6.
  awq::SkinnyPlan sk{};
  const int64_t tiles_e = (N + awq::kSkinnyCols - 1) / awq::kSkinnyCols;
  const int64_t chunks = (T + awq::kSkinnyMaxM - 1) / awq::kSkinnyMaxM;
  const bool few = T <= awq::kSkinnyMaxM ||
                   (T <= awq::kSkinnyExpertsMaxT && S <= 8 * E && K * (N / 2) >= (int64_t(1) << 21));
  if (few && E * chunks * tiles_e < (int64_t(1) << 31) &&
      plan_skinny(T < awq::kSkinnyMaxM ? T : awq::kSkinnyMaxM, K, E * chunks * tiles_e * awq::kSkinnyCols, g,
                  device_cus(), sk)) {
    Plan p;
    if (sk.splits > 1) {
      if (sk.atomic) p.accum_bytes = (int64_t)sk.n_tiles * sk.mrows * awq::kSkinnyCols * 12;
      else p.partial_bytes = (int64_t)sk.n_tiles * sk.splits * sk.mrows * awq::kSkinnyCols * 4;
    }
    uint64_t* accum = nullptr;
    float* partial = nullptr;
    if (sk.splits > 1) {
      st = get_workspace(p, stream, &accum, &partial);
      if (st != AWQ_OK) return st;
      if (sk.atomic) partial = reinterpret_cast<float*>(accum + (int64_t)sk.n_tiles * sk.mrows * awq::kSkinnyCols);
    }
    const awq::SkinnyExperts ex{expert_ids, (int)topk, (int)tiles_e, (int)chunks, (int)E, K * (N / 8), G * (N / 8),
                                G * N};
    hipError_t e = awq::launch_skinny_experts(static_cast<const uint16_t*>(x_f16), qweight, qzeros,
                                              static_cast<const uint16_t*>(scales_f16), (int)T, (int)K, (int)N, g,
                                              sk, ex, accum, partial, static_cast<uint16_t*>(y_f16), stream);
    return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
  }
  int block_rows = 0;
  const int variant = awq::moe_tile_variant(S / E, &block_rows);
  const int64_t tiles = awq_moe_tiles(S, E, block_rows);
  const int64_t bn = awq::kTileBN[variant];
  // Grid of the launches (256-row tables also take a launch of two 64-row parts per entry).
  if (awq::tile_blocks(tiles * (variant == 0 ? 2 : 1), N, (int)bn) >= (int64_t(1) << 31)) return AWQ_ERR_UNSUPPORTED;
  // Scratch: tile table (16-byte entries), offsets, sorted slots; written by the
  // alignment kernel before the product reads it, on the same stream.
  void* scratch = nullptr;
  st = get_scratch(tiles * 16 + (E + 1 + S + 4) * 4, stream, &scratch);
  if (st != AWQ_OK) return st;
  int32_t* table = static_cast<int32_t*>(scratch);
  int32_t* offsets = table + 4 * tiles;
  int32_t* sorted = offsets + E + 1;
  hipError_t e = awq::launch_moe_align(expert_ids, (int)S, (int)E, block_rows, (int)tiles, offsets, sorted, table,
                                       stream);
  if (e != hipSuccess) return AWQ_ERR_HIP;
  awq::MoeTiles moe{sorted, table, (int)topk, (int)tiles, K * (N / 8), G * (N / 8), G * N};
  e = awq::launch_tile_grouped(static_cast<const uint16_t*>(x_f16), qweight, qzeros,
                               static_cast<const uint16_t*>(scales_f16), (int)K, (int)N, g, variant, moe,
                               static_cast<uint16_t*>(y_f16), stream);
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}

int awq_gemm(const void* x_f16, const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
             const void* bias_f16, int64_t M, int64_t K, int64_t N, int64_t group_size, void* y_f16,
             struct ihipStream_t* stream) {
  return gemm_common(x_f16, qweight, qzeros, scales_f16, bias_f16, M, K, N, group_size, y_f16, false, stream);
}

int awq_gemm_noalloc(const void* x_f16, const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                     const void* bias_f16, int64_t M, int64_t K, int64_t N, int64_t group_size, void* y_f16,
                     struct ihipStream_t* stream) {
  return gemm_common(x_f16, qweight, qzeros, scales_f16, bias_f16, M, K, N, group_size, y_f16, false, stream, true);
}

int awq_gemm_bf16(const void* x_bf16, const int32_t* qweight, const int32_t* qzeros, const void* scales_f16,
                  const void* bias_bf16, int64_t M, int64_t K, int64_t N, int64_t group_size, void* y_bf16,
                  struct ihipStream_t* stream) {
  return gemm_common(x_bf16, qweight, qzeros, scales_f16, bias_bf16, M, K, N, group_size, y_bf16, true, stream);
}

}  // extern "C"
