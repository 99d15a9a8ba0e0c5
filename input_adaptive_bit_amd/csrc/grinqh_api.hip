// C ABI of the GRINQH decode GEMV: argument checks, device query, dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call
// touches neither the device nor the stream.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace grinqh {
namespace {

constexpr int kMaxDim = 1 << 20;
constexpr int kMaxDevices = 64;

std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not queried yet
std::atomic<int> g_force_groups{0}, g_force_chunk{0}, g_force_prefill{0};

bool valid_layout(const grinqh_layout* L) {
    if (L == nullptr) return false;
    if (L->d_in < 1 || L->d_in > kMaxDim || L->d_out < 1 || L->d_out > kMaxDim) return false;
    if (L->b_max != 2 && L->b_max != 4 && L->b_max != 6 && L->b_max != 8) return false;
    if (L->n_planes != L->b_max / 2) return false;
    if (L->row_words != ((L->d_out + 63) / 64) * 4) return false;
    return true;
}

bool valid_dtype(int d) { return d == GRINQH_BF16 || d == GRINQH_F32; }

// The GEMV kernel addresses the planes with 32-bit byte offsets and marks
// entries past a list end with offsets from 2^31 up, so the planes of one
// GEMV must stay below 2 GiB.
constexpr size_t kMaxGemvPlaneBytes = 0x7FFFFF00u;

size_t packed_bytes(const grinqh_layout* L) {
    return static_cast<size_t>(L->d_in) * L->n_planes * L->row_words * 4u;
}

int dtype_bytes(int d) { return d == GRINQH_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

// The common tile width of a group: the narrowest any member would pick.
size_t group_ws_bytes(const grinqh_layout* layouts, int n, const LaunchShape& shape) {
    size_t total = 0;
    for (int k = 0; k < n; ++k) total += plan_gemv(layouts[k], shape).ws_bytes;
    return total;
}

grinqh_status map_error(hipError_t e) {
    if (e == hipSuccess) return GRINQH_OK;
    if (e == hipErrorNoDevice || e == hipErrorInvalidDevice) return GRINQH_ENODEV;
    return GRINQH_EDEVICE;
}

}  // namespace

grinqh_status map_hip_error(hipError_t e) { return map_error(e); }

grinqh_status check_gemv_operands(const grinqh_layout* L, const void* x, int x_dtype, const float* theta,
                                  const uint32_t* planes, const uint16_t* s, const uint16_t* z, const void* y,
                                  int y_dtype) {
    if (!valid_layout(L) || x == nullptr || theta == nullptr || planes == nullptr || s == nullptr ||
        z == nullptr || y == nullptr)
        return GRINQH_EINVAL;
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return GRINQH_EINVAL;
    if (packed_bytes(L) > kMaxGemvPlaneBytes) return GRINQH_EINVAL;
    if (!aligned(x, dtype_bytes(x_dtype)) || !aligned(y, dtype_bytes(y_dtype)) || !aligned(theta, 4) ||
        !aligned(planes, 16) || !aligned(s, 2) || !aligned(z, 2))
        return GRINQH_EALIGN;
    // x and y must not overlap
    if (overlap(x, static_cast<size_t>(L->d_in) * dtype_bytes(x_dtype), y,
                static_cast<size_t>(L->d_out) * dtype_bytes(y_dtype)))
        return GRINQH_EINVAL;
    return GRINQH_OK;
}

LaunchOverride launch_override() {
    return LaunchOverride{g_force_groups.load(std::memory_order_relaxed), g_force_chunk.load(std::memory_order_relaxed),
                          g_force_prefill.load(std::memory_order_relaxed)};
}

bool current_device_info(DeviceInfo* out, hipError_t* err) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
        *err = (e == hipSuccess) ? hipErrorNoDevice : e;
        return false;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return false;
    }
    int cu = (dev >= 0 && dev < kMaxDevices) ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
    if (cu == 0) {
        e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cu <= 0) {
            *err = (e == hipSuccess) ? hipErrorInvalidDevice : e;
            return false;
        }
        if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cu, std::memory_order_relaxed);
    }
    out->device = dev;
    out->cu_count = cu;
    *err = hipSuccess;
    return true;
}

}  // namespace grinqh

using namespace grinqh;

extern "C" {

int32_t grinqh_version(void) { return 100; }

const char* grinqh_status_string(grinqh_status status) {
    switch (status) {
        case GRINQH_OK: return "ok";
        case GRINQH_EINVAL: return "invalid argument";
        case GRINQH_EALIGN: return "misaligned pointer";
        case GRINQH_ENOSPACE: return "workspace too small";
        case GRINQH_ENODEV: return "no HIP device";
        case GRINQH_EDEVICE: return "HIP runtime error";
    }
    return "unknown status";
}

grinqh_status grinqh_layout_init(int32_t d_in, int32_t d_out, int32_t b_max, grinqh_layout* out) {
    if (out == nullptr) return GRINQH_EINVAL;
    if (d_in < 1 || d_in > kMaxDim || d_out < 1 || d_out > kMaxDim) return GRINQH_EINVAL;
    if (b_max != 2 && b_max != 4 && b_max != 6 && b_max != 8) return GRINQH_EINVAL;
    out->d_in = d_in;
    out->d_out = d_out;
    out->b_max = b_max;
    out->n_planes = b_max / 2;
    out->row_words = ((d_out + 63) / 64) * 4;
    return GRINQH_OK;
}

size_t grinqh_packed_bytes(const grinqh_layout* L) {
    if (!valid_layout(L)) return 0;
    return static_cast<size_t>(L->d_in) * L->n_planes * L->row_words * 4u;
}

size_t grinqh_gemv_workspace_bytes(const grinqh_layout* L) {
    if (!valid_layout(L)) return 0;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return 0;
    return plan_gemv(*L, choose_launch(L, 1, dev)).ws_bytes;
}

grinqh_status grinqh_pack(const grinqh_layout* L, const uint8_t* q, uint32_t* planes,
                          void* stream) {
    if (!valid_layout(L) || q == nullptr || planes == nullptr) return GRINQH_EINVAL;
    if (!aligned(planes, 16)) return GRINQH_EALIGN;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    return map_error(launch_pack(*L, q, planes, static_cast<hipStream_t>(stream)));
}

grinqh_status grinqh_assign_bits(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                                 const float* theta, uint8_t* bits, int32_t* active_idx,
                                 int32_t* n_active, void* stream) {
    if (!valid_layout(L) || x == nullptr || theta == nullptr || bits == nullptr)
        return GRINQH_EINVAL;
    if (!valid_dtype(x_dtype)) return GRINQH_EINVAL;
    if (!aligned(x, dtype_bytes(x_dtype)) || !aligned(theta, 4)) return GRINQH_EALIGN;
    if ((active_idx && !aligned(active_idx, 4)) || (n_active && !aligned(n_active, 4)))
        return GRINQH_EALIGN;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    return map_error(launch_assign_bits(*L, x, x_dtype, theta, bits, active_idx, n_active,
                                        static_cast<hipStream_t>(stream)));
}

grinqh_status grinqh_gemv(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                          const float* theta, const uint32_t* planes, const uint16_t* s,
                          const uint16_t* z, void* y, grinqh_dtype y_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const grinqh_status st = check_gemv_operands(L, x, x_dtype, theta, planes, s, z, y, y_dtype);
    if (st != GRINQH_OK) return st;
    if (workspace == nullptr) return GRINQH_EINVAL;
    if (!aligned(workspace, 256)) return GRINQH_EALIGN;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    GemvPlan plan = plan_gemv(*L, choose_launch(L, 1, dev));
    if (workspace_bytes < plan.ws_bytes) return GRINQH_ENOSPACE;
    return map_error(launch_gemv(*L, plan, x, x_dtype, theta, planes, s, z, y, y_dtype,
                                 workspace, static_cast<hipStream_t>(stream)));
}

size_t grinqh_gemv_group_workspace_bytes(const grinqh_layout* layouts, int32_t n) {
    if (layouts == nullptr || n < 1 || n > GRINQH_MAX_GROUP) return 0;
    for (int k = 0; k < n; ++k)
        if (!valid_layout(&layouts[k]) || layouts[k].b_max != layouts[0].b_max) return 0;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return 0;
    return group_ws_bytes(layouts, n, choose_launch(layouts, n, dev));
}

grinqh_status grinqh_gemv_group(const grinqh_layout* layouts, const grinqh_gemv_operands* ops,
                                int32_t n, grinqh_dtype x_dtype, grinqh_dtype y_dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (layouts == nullptr || ops == nullptr || workspace == nullptr) return GRINQH_EINVAL;
    if (n < 1 || n > GRINQH_MAX_GROUP) return GRINQH_EINVAL;
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return GRINQH_EINVAL;
    if (!aligned(workspace, 256)) return GRINQH_EALIGN;
    const size_t xb = dtype_bytes(x_dtype), yb = dtype_bytes(y_dtype);
    for (int k = 0; k < n; ++k) {
        const grinqh_layout* L = &layouts[k];
        const grinqh_gemv_operands& o = ops[k];
        if (!valid_layout(L) || L->b_max != layouts[0].b_max) return GRINQH_EINVAL;
        if (packed_bytes(L) > kMaxGemvPlaneBytes) return GRINQH_EINVAL;
        if (!o.x || !o.theta || !o.planes || !o.s || !o.z || !o.y) return GRINQH_EINVAL;
        if (!aligned(o.x, xb) || !aligned(o.y, yb) || !aligned(o.theta, 4) || !aligned(o.planes, 16) ||
            !aligned(o.s, 2) || !aligned(o.z, 2))
            return GRINQH_EALIGN;
    }
    for (int k = 0; k < n; ++k) {
        const size_t ny = static_cast<size_t>(layouts[k].d_out) * yb;
        for (int m = 0; m < n; ++m) {
            if (overlap(ops[k].y, ny, ops[m].x, static_cast<size_t>(layouts[m].d_in) * xb)) return GRINQH_EINVAL;
            if (m != k && overlap(ops[k].y, ny, ops[m].y, static_cast<size_t>(layouts[m].d_out) * yb))
                return GRINQH_EINVAL;
        }
    }
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    const LaunchShape shape = choose_launch(layouts, n, dev);
    if (workspace_bytes < group_ws_bytes(layouts, n, shape)) return GRINQH_ENOSPACE;
    GemvGroupArgs args{};
    args.n = n;
    char* ws = static_cast<char*>(workspace);
    int wg = 0;
    for (int k = 0; k < n; ++k) {
        const GemvPlan plan = plan_gemv(layouts[k], shape);
        fill_desc(&args.g[k], layouts[k], plan, ops[k].x, x_dtype, ops[k].theta, ops[k].planes, ops[k].s,
                  ops[k].z, ops[k].y, y_dtype, ws, wg);
        ws += plan.ws_bytes;
        wg += plan.n_tiles * plan.n_splits;
    }
    return map_error(launch_gemv_group(layouts[0].n_planes, shape.lane_groups, args, wg,
                                       static_cast<hipStream_t>(stream)));
}

size_t grinqh_prefill_workspace_bytes(int32_t M) {
    return (M < 1 || M > kMaxDim) ? 0 : prefill_workspace_bytes(M);
}

grinqh_status grinqh_prefill_gemm(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype, int32_t M,
                                  const uint32_t* planes, const uint16_t* s, const uint16_t* z, void* y,
                                  grinqh_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (!valid_layout(L) || x == nullptr || planes == nullptr || s == nullptr || z == nullptr ||
        y == nullptr || workspace == nullptr)
        return GRINQH_EINVAL;
    if (x_dtype != GRINQH_BF16 || !valid_dtype(y_dtype)) return GRINQH_EINVAL;
    if (M < 1 || M > kMaxDim || L->d_in % 8 != 0) return GRINQH_EINVAL;
    if (packed_bytes(L) > kMaxGemvPlaneBytes) return GRINQH_EINVAL;
    if (prefill_tiles(*L, M) > 0x7FFFFFFFL) return GRINQH_EINVAL;
    const size_t yb = dtype_bytes(y_dtype);
    if (!aligned(x, 16) || !aligned(planes, 16) || !aligned(s, 2) || !aligned(z, 2) || !aligned(y, yb) ||
        !aligned(workspace, 256))
        return GRINQH_EALIGN;
    if (workspace_bytes < prefill_workspace_bytes(M)) return GRINQH_ENOSPACE;
    if (overlap(x, static_cast<size_t>(M) * L->d_in * 2u, y, static_cast<size_t>(M) * L->d_out * yb))
        return GRINQH_EINVAL;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    return map_error(launch_prefill(*L, static_cast<const uint16_t*>(x), M, planes, s, z, y, y_dtype,
                                    static_cast<float*>(workspace), dev.cu_count, static_cast<hipStream_t>(stream)));
}

grinqh_status grinqh_debug_force_launch(int32_t lane_groups, int32_t chunk, int32_t prefill_tile) {
    if (lane_groups != 0 && lane_groups != 1 && lane_groups != 2 && lane_groups != 4 && lane_groups != 8)
        return GRINQH_EINVAL;
    if (chunk < 0 || chunk > 256 || prefill_tile < 0 || prefill_tile > 3) return GRINQH_EINVAL;
    g_force_groups.store(lane_groups, std::memory_order_relaxed);
    g_force_chunk.store(chunk, std::memory_order_relaxed);
    g_force_prefill.store(prefill_tile, std::memory_order_relaxed);
    return GRINQH_OK;
}

grinqh_status grinqh_debug_codes(const grinqh_layout* L, const uint8_t* bits,
                                 const uint32_t* planes, uint8_t* codes, void* stream) {
    if (!valid_layout(L) || bits == nullptr || planes == nullptr || codes == nullptr)
        return GRINQH_EINVAL;
    if (!aligned(planes, 16)) return GRINQH_EALIGN;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_error(e);
    return map_error(launch_debug_codes(*L, bits, planes, codes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
