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

// MFMA tile family geometry.
constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kTileK = 32;
constexpr int kTileThreads = 256;

hipError_t launch_dequant(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                          int K, int N, int g, float* out, hipStream_t stream);

// partial: [n_tiles][splits][mrows][256] fp32; counters: [n_tiles] uint32, zero on entry.
hipError_t launch_skinny(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                         const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                         int splits, float* partial, uint32_t* counters, uint16_t* y,
                         hipStream_t stream);

hipError_t launch_tile(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                       const uint16_t* scales, const uint16_t* bias, int M, int K, int N, int g,
                       uint16_t* y, hipStream_t stream);

}  // namespace awq
