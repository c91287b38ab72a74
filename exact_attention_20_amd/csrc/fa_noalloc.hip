// fa_bwd_noalloc (include/fa.h): fa_bwd in its deterministic mode with the
// workspace in a static device array instead of caller memory, for callers
// that cannot allocate.
//
// The backward's workspace holds two float32 row vectors (the LSE in base-2
// units and D = rowsum(dO * O)); the dQ kernel writes both for every query
// row before the key-side kernel reads them, so nothing in the array has to
// start at zero.  Each GPU the library runs on holds one copy of the array
// until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// The array's device address, per device.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address hipGetSymbolAddress
// returns (with that device current) may be handed to kernels.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

int scratch_of_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::call_once(g_once[dev], [dev]() {
        g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    });
    if (g_status[dev] != hipSuccess || !g_scratch[dev]) return FA_ERR_LAUNCH;
    *ptr = g_scratch[dev];
    return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, void* dq, void* dk, void* dv,
                              int B, int H, int Nq, int Nk, int d, float scale, int causal,
                              int dtype, void* stream) {
    // every argument is checked before the first HIP call
    bool work = false;
    const int chk = fa::bwd_check_args(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, dtype, &work);
    if (chk != FA_OK || !work) return chk;
    if (fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype, 1) > (size_t)FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_SCRATCH;
    void* ws = nullptr;
    const int st = scratch_of_current_device(&ws);
    if (st != FA_OK) return st;
    return fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype, 1, ws,
                  (size_t)FA_NOALLOC_SCRATCH_BYTES, stream);
}
