// Routed experts: alignment of routed slots by expert, for the tile kernel's grouped
// mode (vLLM article, section 5.4: a routed-expert layer runs a 4-bit WNA16 MoE
// kernel over per-expert qweight / qzeros / scales).
//
// One workgroup counts the slots of each expert in LDS, scans the counts into
// offsets (and the per-expert tile counts into table positions), writes one table
// entry (expert, first sorted row, rows, 0) per tile of block_rows rows, and
// scatters every slot to its expert's segment through LDS cursors.  Within an
// expert the slot order depends on the atomics' order; every row of the grouped
// product depends only on its own slot, so the product does not.
#include "awq_device.h"
#include "awq_kernels.h"

namespace awq {

constexpr int kAlignThreads = 1024;
constexpr int kAlignMaxExperts = 1024;

__global__ __launch_bounds__(kAlignThreads) void moe_align_kernel(const int32_t* __restrict__ ids, int S, int E,
                                                                 int block_rows, int tiles,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ sorted_slots,
                                                                 int32_t* __restrict__ table) {
  __shared__ int cnt[kAlignMaxExperts];
  __shared__ int off[kAlignMaxExperts + 1];
  __shared__ int tstart[kAlignMaxExperts + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;
  __syncthreads();
  // Slots whose expert id is outside [0, E) are not routed anywhere.
  for (int s = tid; s < S; s += kAlignThreads) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, t = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = a;
      tstart[e] = t;
      a += cnt[e];
      t += (cnt[e] + block_rows - 1) / block_rows;
    }
    off[E] = a;
    tstart[E] = t;  // <= tiles: sum of ceil(c / b) <= S / b + E
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kAlignThreads) offsets[e] = off[e];
  // Table entry i belongs to the expert e with tstart[e] <= i < tstart[e + 1].
  for (int i = tid; i < tiles; i += kAlignThreads) {
    int4 ent = {-1, 0, 0, 0};
    if (i < tstart[E]) {
      int lo = 0, hi = E - 1;  // last e with tstart[e] <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tstart[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int j = i - tstart[lo];
      ent = int4{lo, off[lo] + j * block_rows, min(block_rows, cnt[lo] - j * block_rows), 0};
    }
    reinterpret_cast<int4*>(table)[i] = ent;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = off[e];  // cursors
  __syncthreads();
  for (int s = tid; s < S; s += kAlignThreads) {
    const int e = ids[s];
    if (e >= 0 && e < E) sorted_slots[atomicAdd(&cnt[e], 1)] = s;
  }
}

hipError_t launch_moe_align(const int32_t* expert_ids, int S, int E, int block_rows, int tiles,
                            int32_t* offsets, int32_t* sorted_slots, int32_t* table, hipStream_t stream) {
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(kAlignThreads), 0, stream, expert_ids, S, E, block_rows, tiles,
                     offsets, sorted_slots, table);
  return hipGetLastError();
}

}  // namespace awq
