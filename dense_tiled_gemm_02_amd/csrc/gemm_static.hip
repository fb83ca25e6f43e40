// gemm_run_static: gemm_run for callers that cannot allocate device memory.
// A plan that splits K across workgroups needs a workspace (arrival counters
// and fp32 partial tiles); here it is a fixed file-scope device array instead
// of a caller's buffer.  Declared in include/gemm.h.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to a kernel.

#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "../../include/gemm.h"
#include "api_internal.h"
#include "kernels.h"

namespace {

static_assert(GEMM_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");

// Each device the library runs on holds one copy until the process ends.
// The kernels leave its counter region at zero after every launch; it is
// zero-filled once per device before the first use.
static __device__ __align__(256) unsigned char scratch[GEMM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch`, per device; nullptr until looked up

// The device address of this device's scratch (set up on first use: looked
// up with `device` current, its counter region zero-filled on `stream`).
gemm_status scratch_of(int device, hipStream_t stream, void** out) {
    if (device < 0 || device >= kMaxDevices)
        return dtg::record_error(GEMM_ERR_UNSUPPORTED, "gemm_run_static: device index out of range");
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[device] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return dtg::record_error(GEMM_ERR_HIP, hipGetErrorString(e));
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
            return dtg::record_error(GEMM_ERR_HIP, hipGetErrorString(e));
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e == hipSuccess && ptr == nullptr) e = hipErrorInvalidSymbol;
        if (e == hipSuccess) e = dtg::zero_words(ptr, dtg::kCounterBytes / 4, stream);
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) {
            char msg[256];
            snprintf(msg, sizeof msg, "gemm_run_static: scratch set-up on device %d: %s", device,
                     hipGetErrorString(e));
            return dtg::record_error(GEMM_ERR_HIP, msg);
        }
        g_ptr[device] = ptr;
    }
    *out = g_ptr[device];
    return GEMM_OK;
}

}  // namespace

extern "C" gemm_status gemm_run_static(const gemm_plan* plan, const void* A, const void* B, const void* C,
                                       void* D, void* stream) {
    size_t need = 0;
    gemm_status st = gemm_workspace_size(plan, &need);
    if (st != GEMM_OK) return st;
    if (need == 0) return gemm_run(plan, A, B, C, D, nullptr, 0, stream);
    if (need > static_cast<size_t>(GEMM_STATIC_SCRATCH_BYTES)) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "gemm_run_static: the plan needs %zu bytes of workspace, the static scratch holds %zu "
                 "(use gemm_run with a workspace, or force fewer K slices)",
                 need, static_cast<size_t>(GEMM_STATIC_SCRATCH_BYTES));
        return dtg::record_error(GEMM_ERR_WORKSPACE, msg);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    int device = -1;
    hipError_t e = hipStreamGetDevice(s, &device);
    if (e != hipSuccess) return dtg::record_error(GEMM_ERR_HIP, hipGetErrorString(e));
    void* ws = nullptr;
    st = scratch_of(device, s, &ws);
    if (st != GEMM_OK) return st;
    return gemm_run(plan, A, B, C, D, ws, static_cast<size_t>(GEMM_STATIC_SCRATCH_BYTES), stream);
}
