// static_scratch.hip -- tra_execute for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation): the plan's scratch (the partials of a split
// aggregation, the range-check flags of the packed max / min-plus path) lives
// in one fixed array per device instead of a caller-provided workspace.
//
// The array's name is only a host-side stand-in for the device symbol: host
// code uses the address hipGetSymbolAddress returns for the current device,
// taken once per device and kept for the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "plan.h"
#include "tra.h"

// Largest scratch a plan may run with here: 16 MiB per device (a split
// aggregation of up to 4 M fp32 outputs over 1 partial, or of 512 K outputs
// split 8 ways, e.g. a 256 x 256 product split 8 ways takes 2 MiB).
#ifndef TRA_STATIC_SCRATCH_BYTES
#define TRA_STATIC_SCRATCH_BYTES (16u << 20)
#endif

namespace tra {

static int fail(int code, const std::string &msg)
{
    set_error(msg);
    return code;
}

constexpr size_t kStaticScratchBytes = TRA_STATIC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call on each device.
static int scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TRA_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(TRA_E_HIP, "device index out of range");
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TRA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return TRA_OK;
}

}  // namespace tra

extern "C" size_t tra_static_scratch_bytes(void) { return tra::kStaticScratchBytes; }

extern "C" int tra_execute_static(tra_plan_t plan, const void *x_rel, const void *y_rel, void *z_rel,
                                  void *hip_stream)
{
    if (!plan) return tra::fail(TRA_E_NULL, "plan is NULL");
    tra_plan_info_t info;
    int rc = tra_plan_info(plan, &info);
    if (rc) return rc;
    if (info.workspace_bytes > tra::kStaticScratchBytes)
        return tra::fail(TRA_E_WORKSPACE, "the plan needs " + std::to_string(info.workspace_bytes) +
                                              " bytes of scratch; tra_execute_static holds " +
                                              std::to_string(tra::kStaticScratchBytes) +
                                              " (use tra_execute with a workspace)");
    void *ws = nullptr;
    if (info.workspace_bytes > 0) {
        rc = tra::scratch_address(&ws);
        if (rc) return rc;
    }
    return tra_execute(plan, x_rel, y_rel, z_rel, ws, info.workspace_bytes ? tra::kStaticScratchBytes : 0,
                       hip_stream);
}
