// MFMA tile family of awq_gemm (large M): compute-bound.
//
// y = x . dequant(W) + bias with fp16 MFMA and fp32 accumulation (GPTQModel wiki
// "AWQ", section "Native GEMM": fp32 accumulation; GPU LLM serving-stack blog,
// section 1.2: large batches are compute-bound, so the dequant work must hide under
// the matrix products).
//
// Workgroup: KG groups of 4 waves as WM (M) x 4/WM (N); wave tile (32 FM) x (32 FN)
// of v_mfma_f32_32x32x16_f16 accumulators.  Instantiations, chosen by M alone:
// FM = 8, FN = 1, WM = 1, KG = 2 (256 x 128, 8 waves; each B column is dequantised
// by one wave of a k-group) above 128 rows; FM = 2, FN = 1 with 1 x 4 waves
// (64 x 128) from 33; FM = 1 (32 x 128) below.
//
// Staging, per k-tile of 64 rows, in a ring of kStages LDS buffers: x (BM x 64
// fp16), the workgroup's packed qweight (64 rows x BN / 8 words, row-major as
// stored) and the zero words + fp16 scales of the k-tile's two 32-row halves (g is
// a multiple of 32, so no other group boundary can occur) go from global memory
// straight into LDS (global_load_lds_dwordx4, no register round trip), kStages - 1
// k-tiles ahead of the multiply; layouts are XOR-swizzled so that both the direct
// loads and the fragment reads are conflict-free.
// k loop: software-pipelined (the B operand of the next k16 step dequantised while the
// MFMAs of the current one run, across the k-tile barrier too) for the 256-row and the
// 32-row tiles; the 64-row tiles, two workgroups per CU whose waves already overlap
// each other, go step by step (pipelining them measured 2-4% slower).
// B operand, dequantised in registers: in a 32x32x16 B operand lane l supplies 8
// consecutive k of column n = l % 32.  A wave's 32 FN columns are its packed word
// columns x nibble positions: lane l takes word column l % 8 (FN = 2) or l % 4
// (FN = 1) and extracts the nibble(s) of its own column(s), for FN = 2 nibbles p and
// p + 4 (bytes t and t + 2, same half).  Per pair of rows: one v_perm_b32 gathers the
// needed bytes of both rows, one v_and_or_b32 per column makes exact fp16
// (1024 + q) or (1024 + 16 q) (0x6400 mantissa trick), one packed fma with per-lane
// constants gives (q - z) exactly (x 1 or x 1/16, plus -(1024 + z) or -(64 + z)),
// and one packed multiply by the fp16 scale rounds once: B = fp16((q - z) s).
// Output columns are un-permuted at the store: MFMA column i of N-tile f is packed
// word column (base + i % 8 or i % 4) at nibble position ((i / 8) % 4 + 4 f) or
// (i / 4) % 8, i.e. output column 8 wc + ORDER[nibble].
// Grid order: XCD-aware (see the block order in the kernel): the column tiles that
// share 128-byte weight lines run on one XCD, and M tiles (or table entries) are
// fastest within a run, so each XCD's L2 also keeps one slab of x.
#include <type_traits>

#include "awq_device.h"
#include "awq_kernels.h"


namespace awq {

namespace {

constexpr int kBK = 64;            // k-tile of the x staging
constexpr int kStages = 4;  // LDS buffers of the k loop

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's data lands at lds + 16 l; lds must be the same for the whole wave.  Issued
// as inline assembly, so the compiler does not track these loads: the kernel waits for
// them itself (vmcnt) before anyone reads what they wrote.  M0 takes the LDS byte
// address (the low 32 bits of the generic address of a __shared__ object).
__device__ __forceinline__ void load_lds16(const void* src, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}

// The same load from a wave-uniform 64-bit base (scalar registers) plus a 32-bit
// per-lane byte offset: the base advances with scalar adds, so the per-load address
// math stays off the vector ALU.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// ORDER[p]: column within a packed word held by nibble p.
__device__ __forceinline__ int order_of(int p) { return (p & 4) ? 2 * (p & 3) + 1 : 2 * p; }

}  // namespace

// MFMA of one 32x32x16 block; a and b hold fp16 or (BF16) bfloat16 bit patterns.
template <bool BF16>
__device__ __forceinline__ floatx16 mfma32(const half8v& a, const half8v& b, const floatx16& c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// One B pair (rows k, k + 1 of a column) from the magic form: fp16 x gets
// fp16((q - z) s), rounded once; bfloat16 x gets bf16((q - z) s), rounded once from
// the exact fp32 product ((q - z) has at most 5 significant bits and s 11).
template <bool BF16>
__device__ __forceinline__ uint32_t b_pair(uint32_t magic_pair, half2v mult, half2v off, half2v sc) {
  const half2v qz = __builtin_elementwise_fma(as_h2(magic_pair), mult, off);  // (q - z) exactly
  if constexpr (BF16) return pack_bf16x2((float)qz[0] * (float)sc[0], (float)qz[1] * (float)sc[1]);
  else return as_u32(qz * sc);
}

// GROUPED: routed-expert mode (MoeTiles): each workgroup takes BM rows (one row
// tile of moe.sub) of one table entry, i.e. of one expert, gathers their x rows and
// scatters its y rows; no bias, no K splits.
template <int FM, int FN, int WM, int KG, bool BF16, bool GROUPED = false>
__global__ __launch_bounds__(256 * KG, 1) void tile_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint32_t* __restrict__ qzeros, const _Float16* __restrict__ scales, int M, int K, int N,
    int g, int m_tiles, int kps, const uint16_t* __restrict__ bias, float* __restrict__ partial,
    uint16_t* __restrict__ y, MoeTiles moe) {
  // Argument order: everything the prologue needs first, so that it falls in the 14
  // dwords the dispatcher preloads into SGPRs (the rest is fetched from memory).
  constexpr int THREADS = 256 * KG;   // KG groups of 4 waves; group kg takes k16 steps of its share
  constexpr int WN = 4 / WM;          // waves along N
  constexpr int BM = WM * 32 * FM;    // workgroup rows
  constexpr int BN = WN * 32 * FN;    // workgroup columns
  constexpr int BW = BN / 8;          // packed word columns per workgroup (16 or 8)
  constexpr int WW = 32 * FN / 8;     // packed word columns per wave (8 or 4)
  // Group data of one k-tile, per 32-row half: the zero words of the BW word columns
  // then the BN fp16 scales, in 16-byte pieces.
  constexpr int ZP = BW / 4, SP = BN / 8, GP = ZP + SP;  // pieces: zeros, scales, per half
  constexpr int ACC = FM * FN * 16;   // accumulator registers per lane
  constexpr int YLD = BN + 16;        // staged output row (halves); rows 4 apart in opposite bank halves
  // x tile: rows of 64 halves (128 B); 16-byte chunk c of row r sits at position
  // c ^ ((r / 2) % 8).  A 16-byte fragment read serves 16 lanes (16 consecutive rows)
  // per pass from the 64 banks (256 B): rows of one parity share a bank half, and the
  // swizzle gives the 8 rows of each parity 8 distinct positions, so the pass is
  // conflict-free; a direct-to-LDS load still writes 8 whole rows (1 KB) per wave.  It is
  // its own LDS object: the compiler then knows that the register-staged stores below
  // cannot overlap the direct loads still in flight, and does not wait for them.
  // After the k loop it holds the second k-group's sums (KG = 2), then the fp16
  // output tile.
  __shared__ __attribute__((aligned(16))) _Float16 As[kStages][BM * kBK];
  // Packed weights of a k-tile: 64 rows of BW words, row-major as stored, in groups
  // of 4 words (16 bytes) XOR-swizzled by bit 3 of the row, so that the rows r and
  // r + 8 a 32-bit fragment read touches at once fall in different banks.  Group data:
  // 64 slots of 16 bytes, of which 2 GP are used.  sink: target of the padding loads
  // that keep every wave's count of direct loads equal.
  constexpr int NG = BW / 4;          // 16-byte groups per weight row
  struct Staging {
    uint32_t Bs[kStages][kBK * BW];
    u32x4 Gs[kStages][64];
    u32x4 sink[64];
  };
  __shared__ __attribute__((aligned(16))) Staging stg;
  auto& Bs = stg.Bs;
  auto& Gs = stg.Gs;
  static_assert(2 * GP <= 64, "group data must fit one wave load");
  static_assert(BM * YLD <= kStages * BM * kBK, "staged output tile must fit in the x buffers");
  static_assert(KG == 1 || 4 * (ACC / 2) * 64 * 4 <= kStages * BM * kBK * 2, "half of the k-group exchange must fit");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int kg = wave >> 2;           // k-group
  const int w4 = wave & 3;            // wave within the group
  const int wm = w4 / WN, wn = w4 % WN;
  // Block order.  Workgroups go to the 8 XCDs in turn (block b to XCD b % 8), each
  // XCD with its own L2; the CT = 256 / BN column tiles whose weights share the
  // 128-byte lines of a row get blocks 8 apart, so that one XCD reads each line once
  // for all of them, at about the same time.  Block b is unit u (row tile, or table
  // entry, and a run of CT column tiles) and part p of the run; the grid is whole
  // runs of 8 CT blocks, and blocks past the units or the columns leave at once.
  constexpr int CT = 256 / BN;
  const int bx = blockIdx.x;
  const int u = (bx & 7) + 8 * (bx / (8 * CT));
  const int n_tiles = (N + BN - 1) / BN;
  int tile_m, tile_n;
  if constexpr (GROUPED) {
    // Entries slowest: the unused entries at the end of the table (expert < 0) then
    // take the last blocks of the grid, which exit at once, instead of slots among
    // the working ones.
    const int runs = (n_tiles + CT - 1) / CT;
    tile_m = u / runs;
    tile_n = CT * (u - tile_m * runs) + (bx >> 3) % CT;
    if (tile_m >= moe.tiles * moe.sub || tile_n >= n_tiles) return;
  } else {
    tile_m = u % m_tiles;
    tile_n = CT * (u / m_tiles) + (bx >> 3) % CT;
    if (tile_n >= n_tiles) return;  // also every unit past the last (its tile_n is larger still)
  }
  int first = 0;  // grouped: first sorted row of this workgroup's entry
  if constexpr (GROUPED) {
    const int ti = tile_m / moe.sub;
    const int part = tile_m - ti * moe.sub;  // row tile within the entry
    tile_m = 0;
    const int* ent = moe.table + 4 * ti;
    const int e = ent[0];
    if (e < 0) return;  // an unused entry: the whole workgroup leaves before any barrier
    const int rows = ent[2];
    if (rows < moe.lo || rows >= moe.hi) return;  // the other launch's entry
    first = ent[1] + part * BM;
    M = min(rows - part * BM, BM);  // rows of this tile; rows are tile-local from here on
    if (M <= 0) return;
    qweight += e * moe.w_stride;
    qzeros += e * moe.z_stride;
    scales += e * moe.s_stride;
  }
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  // Grouped mode multiplies every 32-row block of the tile, also those past the
  // tile's rows (their x rows are clamped copies and their sums are never stored).
  const int NW = N >> 3;
  const int wc0 = n0 / 8;

  // ---- Staging of one k-tile.  Every thread runs the same code (no divergent
  // branches).  Loads are a uniform base, advanced per k-tile, plus a per-lane 32-bit
  // byte offset fixed for the whole kernel; out-of-range rows and columns are clamped
  // into those offsets and never stored to y.  A partial last k-tile (K % 64 = 32) is
  // loaded as the full k-tile ending at K, i.e. starting 32 rows early, and only its
  // upper half is multiplied; when K = 32 (the only k-tile is partial) the lanes of the
  // upper half re-read the lower half instead.
  // x goes straight from global memory to LDS (global_load_lds_dwordx4): each wave
  // instruction fills 8 rows; lane l writes position l % 8 of row r = l / 8 (of the
  // group) and so fetches chunk (l % 8) ^ ((r / 2) % 8).
  constexpr int A_GROUPS = BM / 8;              // 8-row groups of the x tile
  constexpr int IPW = A_GROUPS / (4 * KG);      // direct loads per wave per k-tile
  static_assert(IPW >= 1 && A_GROUPS % (4 * KG) == 0, "x tile must split evenly over the waves");
  const int lrow = lane >> 3;
  const char* xb = reinterpret_cast<const char*>(x);
  int a_row0[IPW];              // wave-uniform first row of each 8-row group (clamped)
  uint32_t a_off[IPW];          // lane's byte offset from that row
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int grp = wave * IPW + j;
    const int lch = (lane & 7) ^ (((8 * grp + lrow) >> 1) & 7);
    const int a_ch = K < kBK ? (lch & 3) : lch;
    if constexpr (GROUPED) {
      // Gathered: row r of the entry is token sorted_slots[first + r] / topk (x below
      // 4 GiB, checked by the host).
      const int r = min(8 * grp + lrow, M - 1);
      const int tok = moe.sorted_slots[first + r] / moe.topk;
      a_row0[j] = 0;
      a_off[j] = ((uint32_t)tok * (uint32_t)K + 8u * (uint32_t)a_ch) * 2u;
    } else {
      a_row0[j] = min(m0 + 8 * grp, M - 1);
      const int t = min(lrow, M - 1 - a_row0[j]);
      a_off[j] = ((uint32_t)t * (uint32_t)K + 8u * (uint32_t)a_ch) * 2u;
    }
  }
  // Packed weights and group data also go straight to LDS: NB wave loads of 16 rows
  // (BW = 16) or 32 rows (BW = 8) for the weights, one for the group data, spread over
  // the waves; waves with fewer real loads issue padding loads into sink, so that every
  // wave issues IPW + XPW direct loads per k-tile (the barrier counts them).
  constexpr int RPI = 256 / BW;                // weight rows per wave load
  constexpr int NB = kBK / RPI;                // weight loads per k-tile
  constexpr int NWAVES = 4 * KG;
  constexpr int XPW = (NB + 1 + NWAVES - 1) / NWAVES;  // extra loads per wave
  constexpr int DPW = IPW + XPW;               // direct loads per wave per k-tile
  const char* wb = reinterpret_cast<const char*>(qweight);
  const char* sb = reinterpret_cast<const char*>(scales);
  // Weight load: lane l covers row l / NG of the load's RPI rows and position l % NG,
  // which holds word group (l % NG) ^ swz(row).
  auto swz = [](int r) { return ((r >> 3) & 1) * (NG / 2); };
  const int b_rl = lane / NG;
  // Per-lane byte offset of each extra weight load from the k-tile's first row.
  uint32_t w_off[XPW];
#pragma unroll
  for (int xs = 0; xs < XPW; ++xs) {
    const int e = min(wave + NWAVES * xs, NB - 1);
    const int row = e * RPI + b_rl;                 // row within the k-tile
    const int grp = (lane % NG) ^ swz(row);
    const int r = K < kBK ? (row & 31) : row;       // K = 32: re-read the real half
    w_off[xs] = ((uint32_t)r * (uint32_t)NW + (uint32_t)min(wc0 + 4 * grp, NW - 4)) * 4u;
  }
  // Group data: lane l < 2 GP loads piece l % GP of half l / GP (others repeat piece 0).
  const int g_lane = lane < 2 * GP ? lane : 0;
  const int g_half = g_lane < GP ? 0 : 1;
  const int g_u = g_lane - g_half * GP;
  // The piece of group gi sits at g_base + gi * g_stride: four zero words of a qzeros
  // row (NW words long) or eight scales of a scales row (N halves long).
  const bool g_zero = g_u < ZP;
  const char* g_base = g_zero ? reinterpret_cast<const char*>(qzeros) + 4 * (int64_t)min(wc0 + 4 * g_u, NW - 4)
                              : sb + 2 * (int64_t)min(n0 + 8 * (g_u - ZP), N - 8);
  const uint32_t g_stride = g_zero ? 4u * (uint32_t)NW : 2u * (uint32_t)N;
  // Group of the 32-row block u: floor(u / gk), gk = g / 32, as floor((u + 0.5) * (1 / gk))
  // in fp32.  (u + 0.5) / gk lies at least 0.5 / gk from an integer; for u < 2^19 (K <=
  // 2^24) the two roundings move it by less than 2^-4 / gk, so the floor is exact.
  const float g_rcp = 1.0f / (float)(g >> 5);
  // First row loaded for the k-tile starting at k0 (see above).
  auto tile_row = [&](int k0) { return (K - k0 < kBK && K >= kBK) ? k0 - kBK / 2 : k0; };
  auto load_tile = [&](int buf, int k0) {
    const int kl = tile_row(k0);
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      load_lds16_s(xb + ((int64_t)a_row0[j] * K + kl) * 2, a_off[j], &As[buf][(wave * IPW + j) * 8 * kBK]);
#pragma unroll
    for (int xs = 0; xs < XPW; ++xs) {
      const int e = wave + NWAVES * xs;  // wave-uniform: which extra load this is
      if (e < NB) {
        load_lds16_s(wb + (int64_t)kl * NW * 4, w_off[xs], &Bs[buf][e * RPI * BW]);
      } else if (e == NB) {
        // Groups of the two 32-row halves; g is a multiple of 32, so a group boundary
        // inside the k-tile can only fall between the halves.
        const uint32_t u = (uint32_t)min(kl + g_half * (kBK / 2), K - 1) >> 5;
        const uint32_t gi = (uint32_t)(((float)u + 0.5f) * g_rcp);
        load_lds16(g_base + (uint64_t)gi * g_stride, &Gs[buf][0]);
      } else {
        load_lds16_s(xb + ((int64_t)a_row0[0] * K + kl) * 2, a_off[0], &stg.sink[0]);
      }
    }
  };

  // ---- This lane's column(s) of the B operand.
  const int lc = lane & 31;                    // MFMA column slot
  const int wsub = FN == 2 ? (lc & 7) : (lc & 3);
  const int p0 = FN == 2 ? ((lc >> 3) & 3) : ((lc >> 2) & 7);  // nibble of N-tile 0
  const int wloc = wn * WW + wsub;             // word column within the workgroup tile
  const int kq = 8 * (lane >> 5);              // this lane's k offset within a k16 step
  // v_perm_b32 selector: [a.t0, a.t1, b.t0, b.t1], t0 = byte of nibble p0, t1 = t0 + 2.
  const int byte0 = p0 >> 1;
  const uint32_t sel = FN == 2 ? ((uint32_t)byte0 | ((uint32_t)(byte0 + 2) << 8) | ((uint32_t)(4 + byte0) << 16) |
                                  ((uint32_t)(6 + byte0) << 24))
                               : ((uint32_t)byte0 | (0x0Cu << 8) | ((uint32_t)(4 + byte0) << 16) | (0x0Cu << 24));
  const bool hi_nib = p0 & 1;
  const UnpackConsts uk = unpack_consts();
  const uint32_t mask = hi_nib ? uk.mhi : uk.mlo;
  const half2v mult = hi_nib ? half2v{(_Float16)0.0625f, (_Float16)0.0625f} : half2v{(_Float16)1.f, (_Float16)1.f};
  const int c0 = 8 * wloc + order_of(p0);      // column within the workgroup tile, N-tile 0
  const int c1 = 8 * wloc + order_of(p0 + 4);  // N-tile 1 (FN = 2)
  // -(1024 + z) (low nibble) and -(64 + z) (high nibble) as fp16 bit patterns: 1024 + z
  // and 64 + z (z <= 15) are exact, with z in the low mantissa bits (ulp 1) or above them
  // (ulp 1/16).
  const uint32_t zpat = hi_nib ? 0xD400u : 0xE400u;
  const uint32_t zsh = hi_nib ? 4u : 0u;
  auto zsplat = [&](uint32_t z) {
    const uint32_t h = zpat | (z << zsh);
    return __builtin_bit_cast(half2v, h | (h << 16));
  };

  half2v off0, off1, sc0, sc1;
  // Group data of half h of k-tile buf.  keep = false zeroes the scales (the unused half
  // of a partial last k-tile, whose MFMAs are skipped anyway).
  auto apply_group = [&](int buf, int h, bool keep) {
    const uint32_t* gz = reinterpret_cast<const uint32_t*>(&Gs[buf][h * GP]);
    const _Float16* gs = reinterpret_cast<const _Float16*>(&Gs[buf][h * GP + ZP]);
    const uint32_t zw = gz[wloc];
    // Loads first, then a select: a conditional load would split the loop body.
    const _Float16 s0v = gs[c0];
    off0 = zsplat((zw >> (4 * p0)) & 0xFu);
    sc0 = splat(keep ? s0v : (_Float16)0.f);
    if (FN == 2) {
      const _Float16 s1v = gs[c1];
      off1 = zsplat((zw >> (4 * (p0 + 4))) & 0xFu);
      sc1 = splat(keep ? s1v : (_Float16)0.f);
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Multiply the k-tile staged in LDS buffer buf: k16 steps S0..S1-1 (all four, or
  // the half holding a partial last k-tile's rows).  Straight-line code with the fragments of step s + 1
  // read from LDS while step s is dequantised and multiplied; the group data of
  // half h is applied before steps 2h and 2h + 1.
  struct Frag {
    half8v a[FM];
    u32x4 wlo, whi;
  };
  // kh: this wave's first 32-row half of the k-tile (0, or 1 for the second k-group).
  const int rx = (lc >> 1) & 7;  // (row / 2) % 8 of every x row this lane reads
  auto read_frag = [&](Frag& f, int buf, int s, int kh) {
    const int k = 16 * s + 32 * kh + kq;
    // Word wloc of rows k..k+7; swz(row) is the same for all 8 (k % 8 == 0).
    const uint32_t* brow = &Bs[buf][k * BW + (((wloc >> 2) ^ swz(k)) << 2) + (wloc & 3)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.wlo[j] = brow[j * BW];
      f.whi[j] = brow[(4 + j) * BW];
    }
    const int pos = (k >> 3) ^ rx;  // swizzled 16-byte position of chunk k / 8
#pragma unroll
    for (int i = 0; i < FM; ++i)
      f.a[i] = *reinterpret_cast<const half8v*>(&As[buf][(wm * 32 * FM + 32 * i + lc) * kBK + 8 * pos]);
  };
  // With one wave per SIMD (KG = 1) the fragments of step s + 1 are read while step s
  // is multiplied; with two (KG = 2) the other wave covers that latency and the
  // registers go to the second wave instead.
  constexpr bool kPrefetch = KG == 1;
  auto compute = [&](auto s0_c, auto s1_c, int buf, int kh, bool keep) {
    constexpr int S0 = decltype(s0_c)::value, S1 = decltype(s1_c)::value;
    Frag fr[kPrefetch ? 2 : 1];
    if (kPrefetch) read_frag(fr[S0 & 1], buf, S0, kh);
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      if (!kPrefetch) read_frag(fr[0], buf, s, kh);
      const Frag& f = fr[kPrefetch ? (s & 1) : 0];
      if (kPrefetch && s + 1 < S1) read_frag(fr[(s + 1) & 1], buf, s + 1, kh);
      if (s % 2 == 0) apply_group(buf, s / 2 + kh, keep);
      const uint32_t w[8] = {f.wlo[0], f.wlo[1], f.wlo[2], f.wlo[3], f.whi[0], f.whi[1], f.whi[2], f.whi[3]};
      u32x4 b0w, b1w;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t pb = __builtin_amdgcn_perm(w[2 * pr + 1], w[2 * pr], sel);
        b0w[pr] = b_pair<BF16>((pb & mask) | uk.magic, mult, off0, sc0);
        if (FN == 2) b1w[pr] = b_pair<BF16>(((pb >> 8) & mask) | uk.magic, mult, off1, sc1);
      }
      half8v bf[2];
      bf[0] = __builtin_bit_cast(half8v, b0w);
      if (FN == 2) bf[1] = __builtin_bit_cast(half8v, b1w);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32<BF16>(f.a[i], bf[j], acc[i][j]);
      }
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C2 = std::integral_constant<int, 2>;
  // This wave's share of k-tile buf: both 32-row halves (KG = 1) or the half of its
  // k-group (KG = 2: group kg takes half kg, with that half's group data).  A partial
  // last k-tile holds its 32 rows in the upper half (K >= 64) or the lower one
  // (K = 32); the other half is multiplied with zero scales.
  const int part_half = K >= kBK ? 1 : 0;
  // The other half of a partial last k-tile is not multiplied at all (a uniform branch):
  // zero weights would still turn an infinite x there into NaN.
  auto run = [&](int buf, bool part) {
#pragma unroll
    for (int kh = (KG == 1 ? 0 : kg); kh < 2; kh += KG)
      if (!part || kh == part_half) compute(C0{}, C2{}, buf, kh, true);
  };

  // kStages LDS buffers.  While k-tile t is multiplied from buffer t % kStages,
  // everything k-tile t + kStages - 1 needs streams straight into its buffer; the
  // barrier at the end of a k-tile waits only for the direct loads of k-tile t + 1
  // (vmcnt may still count the DPW loads of each later k-tile, issued last), so each
  // load has kStages - 1 k-tiles of work to arrive.  Loads past the last k-tile re-read it (clamped) into a buffer no one reads
  // again, so the loop body has no data-dependent branches.  This workgroup's k-tiles:
  // [kt0, kt0 + KT) of the layer's; the layer's last k-tile is partial when K % 64 = 32.
  const int KT_all = (K + kBK - 1) / kBK;
  const int kt0 = blockIdx.y * kps;
  const int KT = min(KT_all, kt0 + kps) - kt0;
  auto kofs = [&](int t) { return (kt0 + min(t, KT - 1)) * kBK; };
  // LDS reads done and all but the last (kStages - 2) DPW vector-memory operations
  // (the direct loads of k-tiles t + 2 ...) complete, then the workgroup barrier.
  auto barrier_keep_last = [] {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kStages - 2) * DPW) : "memory");
  };
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) load_tile(t, kofs(t));
  // Bias of this lane's output column(s) for the unsplit epilogue, requested once the
  // first k-tiles' loads are out (the epilogue would otherwise wait a memory round trip
  // for it after the last k-tile).  Without a bias, or with split partials, the load
  // reads x and is unused.
  uint16_t braw[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const bool use = bias != nullptr && partial == nullptr;
    braw[j] = (use ? bias : x)[use ? min(n0 + (j == 0 ? c0 : c1), N - 1) : 0];
  }
  barrier_keep_last();
  if constexpr (KG == 2) {
    // Software-pipelined k loop: a wave's share of a k-tile is two k16 steps of one
    // 32-row half (kh = kg), with that half's group data.  The B operand of the next
    // step is dequantised while the MFMAs of the current one run, across the barrier
    // too: the barrier sits between the two steps, because a buffer only has to stay
    // intact until its fragments are in registers.  Per k-tile t:
    //   issue the direct loads of k-tile t + kStages - 1 (into the buffer of k-tile
    //     t - 1, whose fragments every wave read before the previous barrier);
    //   MFMAs of step 0 of t, interleaved with the dequant of step 1 of t;
    //   barrier (k-tile t + 1 has landed);
    //   read the fragments and group data of k-tile t + 1;
    //   MFMAs of step 1 of t, interleaved with the dequant of step 0 of t + 1.
    // After the last k-tile the reads of "k-tile KT" hit the clamped re-load of the
    // last one (valid data); what is dequantised from them is never multiplied.
    const int kh = kg;
    auto keep_of = [&](int t) { return !(kt0 + t == KT_all - 1 && K % kBK != 0) || kh == part_half; };
    auto read_a = [&](half8v(&a)[FM], int buf, int s) {
      const int k = 16 * s + 32 * kh + kq;
      const int pos = (k >> 3) ^ rx;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const half8v*>(&As[buf][(wm * 32 * FM + 32 * i + lc) * kBK + 8 * pos]);
    };
    auto read_w = [&](u32x4& wlo, u32x4& whi, int buf, int s) {
      const int k = 16 * s + 32 * kh + kq;
      const uint32_t* brow = &Bs[buf][k * BW + (((wloc >> 2) ^ swz(k)) << 2) + (wloc & 3)];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wlo[j] = brow[j * BW];
        whi[j] = brow[(4 + j) * BW];
      }
    };
    auto dequant = [&](const u32x4& wlo, const u32x4& whi, half8v(&bf)[2]) {
      const uint32_t w[8] = {wlo[0], wlo[1], wlo[2], wlo[3], whi[0], whi[1], whi[2], whi[3]};
      u32x4 b0w, b1w;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t pb = __builtin_amdgcn_perm(w[2 * pr + 1], w[2 * pr], sel);
        b0w[pr] = b_pair<BF16>((pb & mask) | uk.magic, mult, off0, sc0);
        if constexpr (FN == 2) b1w[pr] = b_pair<BF16>(((pb >> 8) & mask) | uk.magic, mult, off1, sc1);
      }
      bf[0] = __builtin_bit_cast(half8v, b0w);
      if constexpr (FN == 2) bf[1] = __builtin_bit_cast(half8v, b1w);
    };
    auto mfma_step = [&](const half8v(&a)[FM], const half8v(&bf)[2]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32<BF16>(a[i], bf[j], acc[i][j]);
      }
    };
    // One MFMA, then a few VALU instructions, FM * FN times: the dequant issues while
    // the matrix core works.
    auto interleave = [] {
#pragma unroll
      for (int i = 0; i < FM * FN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
      }
    };
    half8v a0[FM], a1[FM], b0[2], b1[2];
    u32x4 w0lo, w0hi, w1lo, w1hi;
    read_a(a0, 0, 0);
    read_w(w0lo, w0hi, 0, 0);
    read_w(w1lo, w1hi, 0, 1);
    apply_group(0, kh, keep_of(0));
    dequant(w0lo, w0hi, b0);
    // mul = false only on the last k-tile, for the k-group whose half of a partial last
    // k-tile holds no new rows: its MFMAs are skipped (zero weights would still turn an
    // infinite x there into NaN); it still takes part in the barrier.
    auto body = [&](int kt, bool mul) {
      const int buf = kt % kStages, nbuf = (kt + 1) % kStages;
      load_tile((kt + kStages - 1) % kStages, kofs(kt + kStages - 1));
      read_a(a1, buf, 1);
      if (mul) mfma_step(a0, b0);
      dequant(w1lo, w1hi, b1);
      interleave();
      barrier_keep_last();
      read_a(a0, nbuf, 0);
      read_w(w0lo, w0hi, nbuf, 0);
      read_w(w1lo, w1hi, nbuf, 1);
      apply_group(nbuf, kh, keep_of(kt + 1));
      if (mul) mfma_step(a1, b1);
      dequant(w0lo, w0hi, b0);
      interleave();
    };
    for (int kt = 0; kt < KT - 1; ++kt) body(kt, true);
    body(KT - 1, keep_of(KT - 1));
  } else if constexpr (FM == 1) {
    // 32-row tiles: a software-pipelined k loop of one k-group (four k16 steps per k-tile, both halves):
    // the B operand of step s + 1 is read and dequantised while the MFMAs of step s run,
    // and the barrier sits before the last step of a k-tile, whose MFMAs overlap the
    // dequant of the next k-tile's first step (the buffer a barrier releases only has to
    // stay intact until its fragments are in registers).  Steps of the unused half of a
    // partial last k-tile are read and dequantised but not multiplied; after the last
    // k-tile the reads of "k-tile KT" hit the clamped re-load of the last one (valid
    // data) and what is dequantised from them is never multiplied.
    auto part_of = [&](int t) { return kt0 + t == KT_all - 1 && K % kBK != 0; };
    auto mul_of = [&](int t, int st) { return !part_of(t) || (st >> 1) == part_half; };
    auto dequant1 = [&](const Frag& f, half8v(&bf)[2]) {
      const uint32_t w[8] = {f.wlo[0], f.wlo[1], f.wlo[2], f.wlo[3], f.whi[0], f.whi[1], f.whi[2], f.whi[3]};
      u32x4 b0w, b1w;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t pb = __builtin_amdgcn_perm(w[2 * pr + 1], w[2 * pr], sel);
        b0w[pr] = b_pair<BF16>((pb & mask) | uk.magic, mult, off0, sc0);
        if constexpr (FN == 2) b1w[pr] = b_pair<BF16>(((pb >> 8) & mask) | uk.magic, mult, off1, sc1);
      }
      bf[0] = __builtin_bit_cast(half8v, b0w);
      if constexpr (FN == 2) bf[1] = __builtin_bit_cast(half8v, b1w);
    };
    auto mfma1 = [&](const Frag& f, const half8v(&bf)[2]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma32<BF16>(f.a[i], bf[j], acc[i][j]);
      }
    };
    // One MFMA, then a share of the dequant's VALU instructions, FM * FN times.
    auto interleave1 = [] {
#pragma unroll
      for (int i = 0; i < FM * FN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 20 / (FM * FN), 0);  // VALU
      }
    };
    // Step st (0..3) of buffer buf: fragments f; half st / 2's group data.
    auto read_step = [&](Frag& f, int buf, int st) { read_frag(f, buf, st & 1, st >> 1); };
    Frag fa, fb;
    half8v ba[2], bb[2];
    read_step(fa, 0, 0);
    apply_group(0, 0, true);
    dequant1(fa, ba);
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt % kStages, nbuf = (kt + 1) % kStages;
      load_tile((kt + kStages - 1) % kStages, kofs(kt + kStages - 1));
      // step 0 (fa, ba) | dequant step 1 -> (fb, bb)
      read_step(fb, buf, 1);
      if (mul_of(kt, 0)) mfma1(fa, ba);
      dequant1(fb, bb);
      interleave1();
      // step 1 (fb, bb) | dequant step 2 -> (fa, ba), with half 1's group data
      read_step(fa, buf, 2);
      if (mul_of(kt, 1)) mfma1(fb, bb);
      apply_group(buf, 1, true);
      dequant1(fa, ba);
      interleave1();
      // step 2 (fa, ba) | dequant step 3 -> (fb, bb)
      read_step(fb, buf, 3);
      if (mul_of(kt, 2)) mfma1(fa, ba);
      dequant1(fb, bb);
      interleave1();
      barrier_keep_last();
      // step 3 (fb, bb) | dequant step 0 of k-tile kt + 1 -> (fa, ba)
      read_step(fa, nbuf, 0);
      if (mul_of(kt, 3)) mfma1(fb, bb);
      apply_group(nbuf, 0, true);
      dequant1(fa, ba);
      interleave1();
    }
  } else {
    // 64-row tiles (two workgroups per CU, whose waves overlap each other): step by step.
    for (int kt = 0; kt < KT; ++kt) {
      load_tile((kt + kStages - 1) % kStages, kofs(kt + kStages - 1));
      run(kt % kStages, kt0 + kt == KT_all - 1 && K % kBK != 0);
      barrier_keep_last();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped extra loads have landed too
  __syncthreads();  // every wave is done with the buffers

  // Two k-groups: group 1 hands its sums to group 0 through LDS (register order,
  // conflict-free), group 0 adds them and finishes the tile.
  if constexpr (KG == 2) {
    // In two rounds of half the accumulators each (the x buffers hold one half).
    float* red = reinterpret_cast<float*>(&As[0][0]) + w4 * (ACC / 2) * 64 + lane;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      if (kg == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int v = (i * FN + j) * 16 + r;
              if (v / (ACC / 2) == round) red[(v % (ACC / 2)) * 64] = acc[i][j][r];
            }
      }
      __syncthreads();
      if (kg == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int v = (i * FN + j) * 16 + r;
              if (v / (ACC / 2) == round) acc[i][j][r] += red[(v % (ACC / 2)) * 64];
            }
      }
      __syncthreads();
    }
  }
  const bool owner = KG == 1 || kg == 0;  // holds finished sums

  // Epilogue.  32x32 MFMA output: lane l, register r holds row 8(r/4) + 4(l/32) + r%4
  // of the block, MFMA column l % 32 -> tile column c0 / c1 (for FN = 2 the pair
  // c0, c0 + 1).
  if (partial != nullptr) {
    // Split K: this split's fp32 sums, no bias, to partial[split][M][N]; rows >= M
    // and columns >= N are not stored.  Written through past the XCD's L2 (agent-scope
    // stores, sc1): the split-sum kernel reads each partial once, from any XCD, so
    // keeping it dirty in this XCD's L2 buys nothing (measured: M = 512 on 11008 x 4096
    // g64 61.5 -> 60.2 and 63.1 -> 60.9 us per call on two boxes; M = 64 23.2 -> 22.2
    // on one, unchanged on the other).
    float* pout = partial + (int64_t)blockIdx.y * M * N;
    const int n = n0 + c0;
    if (owner && n < N) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 32 * FM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < M) {
            if (FN == 2)
              *reinterpret_cast<floatx2*>(&pout[(int64_t)row * N + n]) = floatx2{acc[i][0][r], acc[i][FN - 1][r]};
            else
              __hip_atomic_store(&pout[(int64_t)row * N + n], acc[i][0][r], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
    }
    return;
  }
  // The fp16 tile (bias added in fp32) is staged in LDS over the x buffers, then
  // written as whole 16-byte pieces of rows.
  _Float16* Ys = &As[0][0];
  __syncthreads();  // every wave is done reading As (and the k-group exchange)
  if (owner) {
    float bj[FN];
  #pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + (j == 0 ? c0 : c1);
      bj[j] = (bias != nullptr && n < N) ? act_to_float<BF16>(braw[j]) : 0.f;
    }
  #pragma unroll
    for (int i = 0; i < FM; ++i)
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 * FM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (FN == 2)
          *reinterpret_cast<uint32_t*>(&Ys[row * YLD + c0]) =
              pack_act2<BF16>(acc[i][0][r] + bj[0], acc[i][FN - 1][r] + bj[FN - 1]);
        else
          reinterpret_cast<uint16_t*>(Ys)[row * YLD + c0] = float_to_act<BF16>(acc[i][0][r] + bj[0]);
      }
  }
  __syncthreads();
  constexpr int PR = BN / 8;  // 16-byte pieces per row
#pragma unroll
  for (int q = tid; q < BM * PR; q += THREADS) {
    const int row = q / PR, p = q % PR;
    const int grow = m0 + row, gcol = n0 + 8 * p;
    if (grow < M && gcol < N) {
      const int64_t orow = GROUPED ? (int64_t)moe.sorted_slots[first + grow] : (int64_t)grow;  // scattered
      *reinterpret_cast<u32x4*>(&y[orow * N + gcol]) = *reinterpret_cast<const u32x4*>(&Ys[row * YLD + 8 * p]);
    }
  }
}

// y = round(sum over splits of partial[s] + bias) to fp16 or (BF16) bfloat16, 4
// columns per thread, splits summed in order (deterministic).
template <bool BF16, int B>
__global__ __launch_bounds__(256) void tile_reduce_kernel(const float* __restrict__ partial,
                                                          const uint16_t* __restrict__ bias, int64_t MN,
                                                          int N, int splits, uint16_t* __restrict__ y) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= MN) return;
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  // The four bias values (n % 4 == 0: N is a multiple of 32) are requested first, so that
  // they arrive with the partials: one memory round trip, not two.  Without a bias the
  // load reads the first partial and is not used.
  const int n = (int)(e % N);
  const uint16_t* bsrc = bias != nullptr ? bias + n : reinterpret_cast<const uint16_t*>(partial);
  const u32x2_t braw = *reinterpret_cast<const u32x2_t*>(bsrc);
  __builtin_amdgcn_sched_barrier(0);
  floatx4 a = sum_splits<B>(partial + e, MN, splits);
  if (bias != nullptr) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] += act_to_float<BF16>((uint16_t)(braw[j >> 1] >> (16 * (j & 1))));
  }
  *reinterpret_cast<u32x2_t*>(y + e) = u32x2_t{pack_act2<BF16>(a[0], a[1]), pack_act2<BF16>(a[2], a[3])};
}

template <bool BF16>
static hipError_t launch_tile_t(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                                const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                                const TilePlan& p, float* partial, uint16_t* y, hipStream_t stream) {
  const bool split = p.splits > 1;
  auto go = [&](auto kern, int bm, int bn, int threads) {
    const int m_tiles = (M + bm - 1) / bm;
    hipLaunchKernelGGL(kern, dim3((unsigned)tile_blocks(m_tiles, N, bn), (unsigned)p.splits), dim3(threads), 0,
                       stream, x, reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<const uint32_t*>(qzeros),
                       reinterpret_cast<const _Float16*>(scales), M, K, N, g, m_tiles, p.kps, bias,
                       split ? partial : nullptr, y, MoeTiles{});
  };
  switch (p.variant) {
    case 0: go(tile_kernel<8, 1, 1, 2, BF16>, 256, 128, 512); break;
    case 1: go(tile_kernel<2, 1, 1, 1, BF16>, 64, 128, 256); break;
    default: go(tile_kernel<1, 1, 1, 1, BF16>, 32, 128, 256); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const int64_t MN = (int64_t)M * N;
  const int64_t blocks = (MN / 4 + 255) / 256;
  auto red = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, partial, bias, MN, N, p.splits, y);
  };
  const int b = split_batch(p.splits);
  if (b == 4) red(tile_reduce_kernel<BF16, 4>);
  else if (b == 8) red(tile_reduce_kernel<BF16, 8>);
  else red(tile_reduce_kernel<BF16, 16>);
  return hipGetLastError();
}

hipError_t launch_tile_grouped(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                               const uint16_t* scales, int K, int N, int g, int variant, const MoeTiles& moe,
                               uint16_t* y, hipStream_t stream) {
  auto go = [&](auto kern, int bn, int threads, int sub = 1, int lo = 0, int hi = 1 << 30) {
    MoeTiles m = moe;
    m.sub = sub;
    m.lo = lo;
    m.hi = hi;
    hipLaunchKernelGGL(kern, dim3((unsigned)tile_blocks((int64_t)moe.tiles * sub, N, bn), 1u), dim3(threads), 0,
                       stream, x, reinterpret_cast<const uint32_t*>(qweight),
                       reinterpret_cast<const uint32_t*>(qzeros), reinterpret_cast<const _Float16*>(scales), 0, K,
                       N, g, 1, (K + kBK - 1) / kBK, nullptr, nullptr, y, m);
  };
  // 256-row tables: two launches over the same table, the 256 x 128 tile on the
  // entries of at least 128 rows, then the 64 x 128 tile on the smaller ones (an
  // expert's last few rows), each as two 64-row parts (a part past the rows exits).
  // A 256-row tile costs about one dequant pass of the expert's weights whatever its
  // rows, a 64-row part about two fifths of that.  The other variants take every entry in one
  // launch.
  switch (variant) {
    case 0:
      go(tile_kernel<8, 1, 1, 2, false, true>, 128, 512, 1, 128);
      go(tile_kernel<2, 1, 1, 1, false, true>, 128, 256, 2, 0, 128);
      break;
    case 1: go(tile_kernel<2, 1, 1, 1, false, true>, 128, 256); break;  // 64 x 128
    default: go(tile_kernel<1, 1, 1, 1, false, true>, 128, 256); break;  // 32 x 128
  }
  return hipGetLastError();
}

hipError_t launch_tile(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                       const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                       const TilePlan& p, bool bf16, float* partial, uint16_t* y, hipStream_t stream) {
  return bf16 ? launch_tile_t<true>(x, qweight, qzeros, scales, bias, M, K, N, g, p, partial, y, stream)
              : launch_tile_t<false>(x, qweight, qzeros, scales, bias, M, K, N, g, p, partial, y, stream);
}

}  // namespace awq
