// Internal interface between the C-ABI layer (qkvf_api.cpp) and the gfx950
// kernels (qkvf_kernels.hip).  Not installed; the public API is include/qkvf.h.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace qkvf {

constexpr int kHidden = 8192;       // K of the projection
constexpr int kHeadDim = 64;        // every head is 64 columns
constexpr int kQPerKv = 8;          // q heads (and gate heads) per KV head
constexpr int kPageSlots = 16;      // slots per cache page
constexpr int kSlotWidth = 128;     // K(64) | V(64) per slot
constexpr int kMaxRows = 16;        // tokens per call
constexpr int kTileRows = 16;       // W rows per MFMA tile
constexpr int kWaves = 8;           // waves per projection block
constexpr int kGrid = 256;          // projection blocks: one per CU
constexpr int kTilesPerBlock = 9;   // 16-row tiles each projection block owns

// Columns for nkv KV heads: [q | k | v | gate] = 2 * (8 + 1) * nkv heads.
constexpr int cols_for(int nkv) { return 2 * (kQPerKv + 1) * nkv * kHeadDim; }
// K split across blocks: 72*nkv row tiles * (32/nkv) splits = 2304 = 256 * 9
// tile-splits for every supported nkv.
constexpr int splits_for(int nkv) { return 32 / nkv; }

// Workspace layout (floats): fp32 partials [splits][M][N] (splits * N = 36864
// for every nkv, M <= 16), then the gathered cos|sin rows [16][64], then the
// slots as int64 [16].
constexpr size_t kPartialFloats = size_t(32) * 1152 * kMaxRows;
constexpr size_t kAuxRowsOffset = kPartialFloats;
constexpr size_t kAuxSlotsOffset = kAuxRowsOffset + size_t(kMaxRows) * kHeadDim;
constexpr size_t kWorkspaceFloats = kAuxSlotsOffset + size_t(kMaxRows) * 2;

// Enqueue the projection partials and the epilogue on `stream`.  Shapes were
// validated by the caller; ws holds kWorkspaceFloats floats on this device.
hipError_t launch_front(int nkv, int M, const void *x, const void *W,
                        const int64_t *positions, const int64_t *slots,
                        const float *cos_sin, void *y, void *kv_cache,
                        float *ws, hipStream_t stream);

}  // namespace qkvf
