// dl_device.hip -- the device-side pieces of the host API (dl_api.hip), kept
// apart so that the API itself is plain host code: the per-slot phase
// kernel, and the static scratch of dl_decode_step_staged_noalloc.
#include <mutex>

#include <hip/hip_runtime.h>

#include "dl_internal.h"

namespace dl {

// Set the phase of one slot (or of all when slot < 0, skipping released
// slots when active_only).  A kernel rather than a memset so that calls stay
// capturable into HIP graphs.
__global__ void slot_phase_kernel(int *t0, int B, int slot, int value, int active_only)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B && (slot < 0 || b == slot) && !(active_only && t0[b] < 0))
        t0[b] = value;
}

hipError_t launch_slot_phase(int *t0, int B, int slot, int value, bool active_only, hipStream_t st)
{
    const int blocks = slot >= 0 ? 1 : (B + 255) / 256;
    const int first = slot >= 0 ? slot : 0;
    hipLaunchKernelGGL(slot_phase_kernel, dim3(blocks), dim3(slot >= 0 ? 1 : 256), 0, st,
                       t0 + first, slot >= 0 ? 1 : B, slot >= 0 ? 0 : -1, value, active_only ? 1 : 0);
    return hipGetLastError();
}

// Scratch of dl_decode_step_staged_noalloc: the per-step replay coefficient
// rows ([B*H][2M+2] floats) that ReplayPrep writes and AppendDecode reads,
// held in module memory so that the call allocates nothing.  Every GPU the
// library runs on has its own copy, kept until the process ends; each call
// on a GPU reuses that GPU's copy, so calls that overlap on one GPU race.
// Every coefficient the second stage reads is written by the first stage of
// the same call, so nothing here needs clearing between calls.
static __device__ __align__(256) float scratch[kScratchFloats];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.  In host code the array's name is only a
// host-side stand-in: kernels must be given this address.
constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static float *scratch_addr[kMaxDevices];

hipError_t scratch_on_current_device(float **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        scratch_addr[dev] = static_cast<float *>(p);
    }
    *out = scratch_addr[dev];
    return hipSuccess;
}

} // namespace dl
