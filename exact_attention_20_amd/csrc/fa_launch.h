// Internal host-side launch interface between the C ABI (fa_api.cpp) and the
// kernels (fa_fwd.hip, fa_bwd.hip).  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // may be null
    int Nq;
    int Nk;
    int n_qtiles;      // ceil(Nq / BR) for the chosen kernel
    int total_wg;      // B * H * n_qtiles
    float scale_log2;  // scale * log2(e)
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dO;
    void* dq;
    void* dk;
    void* dv;
    float* lse2;       // [B,H,Nq] float32 workspace: LSE * log2(e), +inf for empty rows
    float* dvec;       // [B,H,Nq] float32 workspace: rowsum(dO * O)
    int Nq;
    int Nk;
    int BH;
    float scale;
    float scale_log2;
};

// Query rows per forward workgroup for a dtype (used to size the grid).
int fwd_rows_per_workgroup(int dtype, int d);

hipError_t launch_fwd(int dtype, int d, bool causal, int BH, FwdParams p, hipStream_t stream);
hipError_t launch_bwd(int d, bool causal, BwdParams p, hipStream_t stream);

}  // namespace fa
