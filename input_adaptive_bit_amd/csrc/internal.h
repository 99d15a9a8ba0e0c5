// Host-side interfaces between the C ABI (grinqh_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/grinqh.h"

namespace grinqh {

struct DeviceInfo {
    int device;
    int cu_count;
};

// Cached per-device query; false if no device is visible or the query failed.
bool current_device_info(DeviceInfo* out, hipError_t* err);

hipError_t launch_pack(const grinqh_layout& L, const uint8_t* q, uint32_t* planes,
                       hipStream_t stream);

hipError_t launch_assign_bits(const grinqh_layout& L, const void* x, int x_dtype,
                              const float* theta, uint8_t* bits, int32_t* active_idx,
                              int32_t* n_active, hipStream_t stream);

// Launch plan of the GEMV for a layout on a device (pure host arithmetic).
struct GemvPlan {
    int tile_outputs;   // outputs per workgroup tile
    int n_tiles;        // ceil(padded d_out / tile_outputs)
    int chunk;          // input channels per split
    int n_splits;       // ceil(d_in / chunk)
    size_t ws_partials; // byte offset of the fp32 partial sums
    size_t ws_counters; // byte offset of the per-tile arrival counters
    size_t ws_bytes;    // total workspace bytes
};

GemvPlan plan_gemv(const grinqh_layout& L, const DeviceInfo& dev);

hipError_t launch_gemv(const grinqh_layout& L, const GemvPlan& plan, const void* x,
                       int x_dtype, const float* theta, const uint32_t* planes,
                       const uint16_t* s, const uint16_t* z, void* y, int y_dtype,
                       void* workspace, hipStream_t stream);

hipError_t launch_debug_codes(const grinqh_layout& L, const uint8_t* bits,
                              const uint32_t* planes, uint8_t* codes, hipStream_t stream);

}  // namespace grinqh
