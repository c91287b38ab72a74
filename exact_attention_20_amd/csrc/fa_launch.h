// Internal host-side launch interface between the C ABI (fa_api.cpp) and the
// kernels (fa_fwd.hip, fa_bwd.hip).  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Masks of the forward and backward kernels.
//   kMaskNone:   every key is visible;
//   kMaskCausal: key j is visible to query i iff j <= i + (Nk - Nq);
//   kMaskWindow: iff i + off - wl <= j <= i + off + wr, off = Nk - Nq, with
//                the reaches wl, wr >= 0 in the params; a side without a
//                bound holds kWindowUnbounded (large enough that every
//                sequence fits inside it, small enough that no offset sum
//                overflows: |off| <= FA_MAX_SEQ = 2^23).
enum { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };
constexpr int kWindowUnbounded = 1 << 28;

// A variable-length batch: B sequences packed along the token axis of
// head-major tensors (q, o, dO, dq: [H, total_q, d]; k, v, dk, dv:
// [H, total_k, d]; lse and the backward row vectors: [H, total_q]).
// Sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
// cu_k[b] .. cu_k[b+1]-1 of every head.  A workgroup finds its (batch,
// head) pair and tile with varlen_slot() and its sequence's lengths and
// first rows with seq_geometry() (fa_device.h).
struct VarlenParams {
    const int* cu_q;   // [B+1] device offsets of the query rows
    const int* cu_k;   // [B+1] device offsets of the key rows
    int B;             // sequences
    int H;             // heads
    int total_q;       // packed query rows per head
    int total_k;       // packed key rows per head
    int max_q;         // bound on every sequence's query count (sizes the grid)
    int max_k;         // bound on every sequence's key count
};

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;        // may be null
    int Nq;
    int Nk;
    int n_qtiles;      // ceil(Nq / BR) for the chosen kernel
    int n_slots;       // workgroups per (batch, head): n_qtiles, or ceil(n_qtiles / 2) when paired
    int paired;        // bf16 kernel: a workgroup runs query tiles n-1-j and j of one head
    int persist;       // bf16 causal d = 128: the persistent grid over the pairs (paired = 1)
    int soft_exp2;     // bf16, no window: one exponential in soft_exp2 (2, 4, 8) by exp2_poly; 0 = none
    int total_wg;      // B * H * n_slots (split-KV: B * H * n_qtiles * n_splits; persistent: the grid)
    float scale_log2;  // scale * log2(e)
    int wl, wr;        // window reaches (kMaskWindow only)
    int BH;               // B * H (split-KV and persistent modes)
    // split-KV mode only
    int n_splits;         // runs of key tiles per query tile
    int tiles_per_split;  // 64-key tiles per run
    float* o_part;        // [n_splits, B*H, Nq, d] fp32 partial outputs
    float* lse_part;      // [n_splits, B*H, Nq] fp32 partial LSE, log2 units
    VarlenParams vl;      // variable-length mode only
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
    float* dqacc;      // [B,H,Nq,d] float32 workspace of the atomic mode: dQ / scale
    int Nq;
    int Nk;
    int BH;
    int kv_slots;      // dK/dV workgroups per (batch, head): 128-key tiles, halved when paired
    int kv_paired;
    int q_slots;       // dQ workgroups per (batch, head): 128-query tiles, halved when paired
    int q_paired;
    float scale;
    float scale_log2;
    int wl, wr;        // window reaches (kMaskWindow only)
    VarlenParams vl;   // variable-length mode only
};

// Query rows per forward workgroup for a dtype (used to size the grid).
int fwd_rows_per_workgroup(int dtype, int d);

// Whether the bf16 forward pairs query tiles (n-1-j with j) in one workgroup:
// causal only, where it evens out the work, and only for grids large enough
// that halving the workgroup count still fills the GPU several times over.
bool fwd_pair_tiles(int dtype, int d, bool causal, long bh, int n_qtiles);
// The persistent grid size for a forward call, or 0 for the one-workgroup-
// per-item launch.
int fwd_persist_grid(int dtype, int d, bool causal, long bh, int n_qtiles);
// The same decision for the backward kernels' key and query tiles.
bool bwd_pair_tiles(bool causal, long bh, int n_tiles);

// fa_bwd's checks of everything but the workspace (status codes of fa.h);
// *work is false when the call has nothing to compute.  No HIP call.
int bwd_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, const void* dq, const void* dk, const void* dv, int B, int H,
                   int Nq, int Nk, int d, float scale, int dtype, bool* work);

hipError_t launch_fwd(int dtype, int d, int mask, FwdParams p, hipStream_t stream);
// bf16 forward over a variable-length batch (p.vl); grid B*H*n_slots.
hipError_t launch_fwd_varlen(int d, int mask, FwdParams p, hipStream_t stream);
// bf16 split-KV forward: partial kernel, then the combine kernel.
hipError_t launch_fwd_split(int d, bool causal, FwdParams p, hipStream_t stream);
// varlen: the kernels take each (batch, head)'s geometry from p.vl; the
// row-wise pre-pass covers all H * total_q packed rows.
hipError_t launch_bwd(int d, int mask, bool varlen, BwdParams p, hipStream_t stream);
// The atomic-dQ (non-deterministic) backward: a pre-pass over the `rows`
// query rows, one key-side kernel adding dQ into p.dqacc with atomics, and
// the dQ conversion.
hipError_t launch_bwd_atomic(int d, int mask, bool varlen, BwdParams p, long rows, hipStream_t stream);
// fp32 backward (fa_bwd_f32.hip): the dQ kernel (which also writes D and
// LSE2), then the dK/dV kernel; q_slots and kv_slots count 64-row tiles.
hipError_t launch_bwd_f32(int d, int mask, BwdParams p, hipStream_t stream);

}  // namespace fa
