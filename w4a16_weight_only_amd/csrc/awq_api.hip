// C ABI of the AWQ W4A16 library: argument checks, launch planning, workspace.
// The declarations and their contracts are in include/awq_w4a16.h.
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/awq_w4a16.h"
#include "awq_kernels.h"

using namespace awq;

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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

// Compute units for host-only plan queries: the current device's, or 256 (MI355X)
// when no device is visible.
int query_cus() {
  int count = 0;
  if (hipGetDeviceCount(&count) == hipSuccess && count > 0) return device_cus();
  (void)hipGetLastError();
  return 256;
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
      return "AWQ_ERR_UNSUPPORTED: needs K % 32 == 0, N % 32 == 0, group_size -1 or a multiple of 32, sizes <= 2^24, "
             "launches within the grid and offset limits (or a workspace the call may not allocate)";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP: the HIP runtime reported an error";
    default: return "AWQ: unknown status";
  }
}

int awq_validate_pack(int64_t K, int64_t N, int64_t group_size, int64_t qweight_rows,
                      int64_t qweight_cols, int64_t qzeros_rows, int64_t qzeros_cols,
                      int64_t scales_rows, int64_t scales_cols, int64_t bias_len) {
  return validate_pack(K, N, group_size, qweight_rows, qweight_cols, qzeros_rows, qzeros_cols, scales_rows,
                       scales_cols, bias_len);
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
  Plan p;
  return plan_gemm(M, K, N, group_size, query_cus(), false, p);
}

int awq_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t group_size, int* family, int* splits,
                  int* grid_x, int* grid_y, int* block, int64_t* workspace_bytes) {
  Plan p;
  const int st = plan_gemm(M, K, N, group_size, query_cus(), false, p);
  if (st != AWQ_OK) return st;
  if (family) *family = p.family;
  if (splits) *splits = p.family == 2 ? p.dp.splits : (p.family == 0 ? p.sk.splits : p.tp.splits);
  if (grid_x) *grid_x = (int)p.grid_x;
  if (grid_y) *grid_y = p.grid_y;
  if (block) *block = p.block;
  if (workspace_bytes) *workspace_bytes = p.workspace_bytes();
  return AWQ_OK;
}

int awq_gemm_plan_tail(int64_t M, int64_t K, int64_t N, int64_t group_size, int64_t* rows, int* splits,
                       int* grid_x, int* grid_y, int* block) {
  Plan p;
  const int st = plan_gemm(M, K, N, group_size, query_cus(), false, p);
  if (st != AWQ_OK) return st;
  const bool tail = p.family == 1 && p.rows1 < M;
  if (rows) *rows = tail ? M - p.rows1 : 0;
  if (splits) *splits = tail ? p.tail.tp.splits : 0;
  if (grid_x) *grid_x = tail ? (int)p.tail.grid_x : 0;
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
  RtnPlan p;
  int st = plan_rtn(K, N, group_size, sym, p);
  if (st != AWQ_OK) return st;
  const int g = eff_group(K, group_size);
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
  Plan p;
  const int pst = plan_gemm(M, K, N, group_size, device_cus(), bf16, p);
  if (pst != AWQ_OK) return pst;
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

int64_t awq_moe_tiles(int64_t S, int64_t E, int64_t block_rows) { return moe_tiles(S, E, block_rows); }

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
  MoePlan mp;
  int st = plan_moe(T, topk, E, K, N, group_size, 0, mp);  // sizes only
  if (st != AWQ_OK) return st;
  if (T == 0) return AWQ_OK;
  if (!x_f16 || !qweight || !qzeros || !scales_f16 || !expert_ids || !y_f16) return AWQ_ERR_NULL;
  if (!aligned16(x_f16) || !aligned16(qweight) || !aligned16(qzeros) || !aligned16(scales_f16) || !aligned16(y_f16))
    return AWQ_ERR_ALIGN;
  st = plan_moe(T, topk, E, K, N, group_size, device_cus(), mp);
  if (st != AWQ_OK) return st;
  const int64_t S = T * topk;
  const int g = eff_group(K, group_size);
  const int64_t G = K / g;
  const auto* x = static_cast<const uint16_t*>(x_f16);
  const auto* sc = static_cast<const uint16_t*>(scales_f16);
  auto* y = static_cast<uint16_t*>(y_f16);
  if (mp.skinny) {
    Plan p;
    p.accum_bytes = mp.accum_bytes;
    p.partial_bytes = mp.partial_bytes;
    uint64_t* accum = nullptr;
    float* partial = nullptr;
    if (mp.sk.splits > 1) {
      st = get_workspace(p, stream, &accum, &partial);
      if (st != AWQ_OK) return st;
      if (mp.sk.atomic) partial = reinterpret_cast<float*>(accum + skinny_accum_entries(mp.sk));
    }
    const SkinnyExperts ex{expert_ids, (int)topk, (int)mp.tiles_e, (int)mp.chunks, (int)E, K * (N / 8), G * (N / 8),
                           G * N};
    hipError_t e = launch_skinny_experts(x, qweight, qzeros, sc, (int)T, (int)K, (int)N, g, mp.sk, ex, accum, partial,
                                         y, stream);
    return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
  }
  // Scratch: tile table (16-byte entries), offsets, sorted slots; written by the
  // alignment kernel before the product reads it, on the same stream.
  void* scratch = nullptr;
  st = get_scratch(mp.scratch_bytes, stream, &scratch);
  if (st != AWQ_OK) return st;
  int32_t* table = static_cast<int32_t*>(scratch);
  int32_t* offsets = table + 4 * mp.tiles;
  int32_t* sorted = offsets + E + 1;
  hipError_t e = launch_moe_align(expert_ids, (int)S, (int)E, mp.block_rows, (int)mp.tiles, offsets, sorted, table,
                                  stream);
  if (e != hipSuccess) return AWQ_ERR_HIP;
  MoeTiles moe{sorted, table, (int)topk, (int)mp.tiles, K * (N / 8), G * (N / 8), G * N};
  e = launch_tile_grouped(x, qweight, qzeros, sc, (int)K, (int)N, g, mp.variant, moe, y, stream);
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
