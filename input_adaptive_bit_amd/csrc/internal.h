// Host-side interfaces between the C ABI (grinqh_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "grinqh.h"

namespace grinqh {

struct DeviceInfo {
    int device;
    int cu_count;
};

// Cached per-device query; false if no device is visible or the query failed.
bool current_device_info(DeviceInfo* out, hipError_t* err);

// Status code of a HIP error.
grinqh_status map_hip_error(hipError_t e);

// Host checks of grinqh_gemv's operands (all but the workspace): GRINQH_OK,
// or the status the call returns without touching the device.
grinqh_status check_gemv_operands(const grinqh_layout* L, const void* x, int x_dtype, const float* theta,
                                  const uint32_t* planes, const uint16_t* s, const uint16_t* z, const void* y,
                                  int y_dtype);

hipError_t launch_pack(const grinqh_layout& L, const uint8_t* q, uint32_t* planes,
                       hipStream_t stream);

hipError_t launch_assign_bits(const grinqh_layout& L, const void* x, int x_dtype,
                              const float* theta, uint8_t* bits, int32_t* active_idx,
                              int32_t* n_active, hipStream_t stream);

// Launch plan of the GEMV for a layout on a device (pure host arithmetic).
struct GemvPlan {
    int lane_groups;    // lane groups per wave (1, 2, 4 or 8)
    int tile_outputs;   // outputs per workgroup tile: (64 / lane_groups) * 64
    int n_tiles;        // ceil(padded d_out / tile_outputs)
    int chunk;          // input channels per slice (<= 256)
    int n_splits;       // ceil(d_in / chunk)
    size_t ws_acc;      // byte offset of the fp32 accumulators [n_tiles * tile_outputs]
    size_t ws_ctrl;     // byte offset of the per-tile control blocks (256 bytes each:
                        // arrival counter, then the sum of x over loaded channels)
    size_t ws_bytes;    // total workspace bytes
};

// One GEMV of a launch group (kernel argument, passed by value).
struct GemvDesc {
    const void* x;
    const float* theta;
    const uint32_t* planes;
    const uint16_t* s;
    const uint16_t* z;
    void* y;
    float* acc;
    unsigned* ctrl;
    int d_in, d_out, row_words, chunk, n_splits, n_tiles, wg_begin, x_dtype, y_dtype;
    // ceil(2^32 / n_splits): the tile of local item a is the high word of
    // a * split_magic (exact while a * n_splits < 2^32); 0 where that does not
    // hold for every item, or for one split (the kernel then divides)
    uint32_t split_magic;
};

constexpr int kMaxGroup = 8;
constexpr int kCtrlWords = 64;       // one 256-byte line per tile

struct GemvGroupArgs {
    GemvDesc g[kMaxGroup];
    int n;
};

// Launch shape shared by every GEMV of one launch: lane groups per wave
// (tile width: 1, 2, 4 or 8) and the slice length in input channels.
struct LaunchShape {
    int lane_groups;
    int chunk;
};

// Plan of one GEMV at a launch shape.
GemvPlan plan_gemv(const grinqh_layout& L, const LaunchShape& shape);
// Process-wide launch-shape overrides set through grinqh_debug_force_launch
// (0 = the library's own choice).
struct LaunchOverride {
    int lane_groups;    // 0, 1, 2, 4 or 8
    int chunk;          // 0 or 1 .. 256
    int prefill_tile;   // 0, 1 (128 x 128), 2 (256 x 128) or 3 (256 x 256)
};
LaunchOverride launch_override();

// Launch shape for one launch of these n GEMVs (a group, or n = 1): slices
// of up to 256 channels, 4 lane groups per wave (2 when that gives more than
// four workgroups per CU, 8 when it gives too few to reach most CUs), and
// the slices shortened until the workgroup count reaches a multiple of the
// CU count; then the overrides.  Cached per host thread.
LaunchShape choose_launch(const grinqh_layout* layouts, int n, const DeviceInfo& dev);

// Prefill GEMM: rows sums, then the MFMA kernel (prefill.hip).
size_t prefill_workspace_bytes(int M);
long prefill_tiles(const grinqh_layout& L, int M);
// Tile (tokens x outputs): 256 x 256, 256 x 128 or 128 x 128, whichever has
// the least estimated time on cu_count CUs (128 x 128 up to 128 tokens),
// unless an override is set.
hipError_t launch_prefill(const grinqh_layout& L, const uint16_t* x, int M, const uint32_t* planes,
                          const uint16_t* s, const uint16_t* z, void* y, int y_dtype, float* rowsum,
                          int cu_count, hipStream_t stream);

void fill_desc(GemvDesc* g, const grinqh_layout& L, const GemvPlan& plan, const void* x, int x_dtype,
               const float* theta, const uint32_t* planes, const uint16_t* s, const uint16_t* z,
               void* y, int y_dtype, void* workspace, int wg_begin);

hipError_t launch_gemv_group(int n_planes, int lane_groups, const GemvGroupArgs& args, int total_wg,
                             hipStream_t stream);

hipError_t launch_gemv(const grinqh_layout& L, const GemvPlan& plan, const void* x,
                       int x_dtype, const float* theta, const uint32_t* planes,
                       const uint16_t* s, const uint16_t* z, void* y, int y_dtype,
                       void* workspace, hipStream_t stream);

hipError_t launch_debug_codes(const grinqh_layout& L, const uint8_t* bits,
                              const uint32_t* planes, uint8_t* codes, hipStream_t stream);

}  // namespace grinqh
