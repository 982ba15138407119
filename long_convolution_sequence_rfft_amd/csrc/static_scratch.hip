// static_scratch.hip -- hyena_forward_noalloc: the forward chain with its
// workspace in a fixed device array of this library instead of a caller
// buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below exists once per GPU the library runs on and is
// held until the process ends.  In host code its name is only a host-side
// stand-in, so the host never passes it to a kernel: the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in g_scratch_ptr[device]; every launch, copy or record
// uses that pointer.  No call here allocates or frees memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "plan.h"

namespace {

constexpr size_t kScratchBytes = HYENA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The stream's device (the current device for the null stream).
hyena_status stream_device(void* stream, int& dev)
{
    hipError_t e;
    if (stream != nullptr) e = hipStreamGetDevice((hipStream_t)stream, &dev);
    else e = hipGetDevice(&dev);
    if (e != hipSuccess) return hy::fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return hy::fail(HYENA_ERR_DEVICE, "device index out of range");
    return HYENA_OK;
}

// Device address of this device's copy of `scratch`, looked up on first use
// with that device current.
hyena_status scratch_of(int dev, void*& ptr)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hy::fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return hy::fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr)
            return hy::fail(HYENA_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") +
                                                  hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
        hy::log_msg("static scratch of device %d at %p (%zu bytes)", dev, p, kScratchBytes);
    }
    ptr = g_scratch_ptr[dev];
    return HYENA_OK;
}

}  // namespace

extern "C" hyena_status hyena_forward_noalloc(hyena_plan_t plan, const void* u,
                                              const void* const* gates, const void* H,
                                              const float* D, void* y, void* stream)
{
    const hy::Plan* pp = hy::plan_of(plan);
    if (pp == nullptr) return hy::fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    const hy::Plan& p = *pp;
    if (p.workspace_bytes > kScratchBytes)
        return hy::fail(HYENA_ERR_UNSUPPORTED,
                        "hyena_forward_noalloc: the plan needs a " +
                            std::to_string(p.workspace_bytes) +
                            "-byte workspace, more than the static scratch's " +
                            std::to_string(kScratchBytes) + " bytes; use hyena_forward");
    int dev = 0;
    hyena_status st = stream_device(stream, dev);
    if (st != HYENA_OK) return st;
    void* ws = nullptr;
    st = scratch_of(dev, ws);
    if (st != HYENA_OK) return st;
    st = hy::check_forward_args(p, u, gates, H, D, y, ws);
    if (st != HYENA_OK) return st;
    // The scratch keeps whatever the last call on this device left in it.
    // The chain writes every intermediate it reads, so only the twiddle
    // tables must be this plan's: write them unless the record says they are
    // (which also drops other plans' records, since this call overwrites the
    // rest of the scratch).
    if (!hy::ws_record_use(ws, p.workspace_bytes, p.token)) {
        st = hy::launch_tw_init(p, ws, stream);
        if (st != HYENA_OK) return st;
        hy::ws_record_init(ws, p.workspace_bytes, p.token);
    }
    // one stream only: a chain of several chunks would otherwise create the
    // library's second stream on first use
    hy::SingleStreamScope one_stream;
    return hy::run_forward(p, u, gates, H, D, y, ws, stream);
}
