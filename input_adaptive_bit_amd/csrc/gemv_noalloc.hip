// grinqh_gemv_noalloc: the decode GEMV with its workspace in a static device
// array instead of a caller buffer, for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation).  Same kernels and results as grinqh_gemv.
//
// The array ("scratch") is a file-scope __device__ array: each GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code the name `scratch` is only a host-side handle for the
// symbol, never a device address: the device address of the current GPU's
// copy comes from hipGetSymbolAddress, once per device, and only that address
// is handed to kernels.  The first call on a device clears the array with a
// fill kernel queued on that call's stream; every GEMV leaves its workspace
// zeroed again, so later calls need no clearing.
#include <mutex>

#include "internal.h"

namespace grinqh {
namespace {

constexpr size_t kScratchBytes = 1u << 20;     // GRINQH_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GRINQH_NOALLOC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];       // device address of each GPU's copy, once set up

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
    for (size_t i = blockIdx.x * 256u + threadIdx.x; i < n16; i += static_cast<size_t>(gridDim.x) * 256u)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address; the first call on a device looks it
// up and queues the clearing fill on `stream`.
hipError_t device_scratch(int device, hipStream_t stream, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        zero_fill_kernel<<<dim3(256), dim3(256), 0, stream>>>(static_cast<uint4*>(ptr), kScratchBytes / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace
}  // namespace grinqh

using namespace grinqh;

extern "C" grinqh_status grinqh_gemv_noalloc(const grinqh_layout* L, const void* x, grinqh_dtype x_dtype,
                                             const float* theta, const uint32_t* planes, const uint16_t* s,
                                             const uint16_t* z, void* y, grinqh_dtype y_dtype, void* stream) {
    const grinqh_status st = check_gemv_operands(L, x, x_dtype, theta, planes, s, z, y, y_dtype);
    if (st != GRINQH_OK) return st;
    DeviceInfo dev;
    hipError_t e;
    if (!current_device_info(&dev, &e)) return map_hip_error(e);
    if (dev.device < 0 || dev.device >= kMaxScratchDevices) return GRINQH_ENODEV;
    const GemvPlan plan = plan_gemv(*L, choose_launch(L, 1, dev));
    if (plan.ws_bytes > kScratchBytes) return GRINQH_ENOSPACE;
    void* ws = nullptr;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    e = device_scratch(dev.device, hs, &ws);
    if (e != hipSuccess) return map_hip_error(e);
    return map_hip_error(launch_gemv(*L, plan, x, x_dtype, theta, planes, s, z, y, y_dtype, ws, hs));
}
