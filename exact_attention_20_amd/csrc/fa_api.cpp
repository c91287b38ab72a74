// C ABI entry points declared in include/fa.h: argument validation, variant
// dispatch and launch on the caller's stream.  Validation runs before any HIP
// call, so a rejected call enqueues nothing and touches no output.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shared checks of sizes, head dim, dtype and scale.
int check_common(int B, int H, int Nq, int Nk, int d, float scale, int dtype) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
    if (Nq > FA_MAX_SEQ || Nk > FA_MAX_SEQ) return FA_ERR_SHAPE;
    // every element index must fit in int64 and the grid in 32 bits
    const long double elems = (long double)B * H * (long double)(Nq > Nk ? Nq : Nk) * 128.0L;
    if (elems > 4.0e18L) return FA_ERR_SHAPE;
    if ((long double)B * H * ((Nq + 63) / 64 + 1) > 2.0e9L) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// Kernel mask of a call: a causal flag, or the reaches of a local window
// (-1 = unbounded side).  A window unbounded on the left that reaches 0 keys
// to the right is the causal mask and takes the causal kernels; one unbounded
// on both sides takes the unmasked kernels.
struct Mask {
    int mode, wl, wr;
};

Mask causal_mask(int causal) { return Mask{causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0}; }

int window_mask(int window_left, int window_right, Mask* m) {
    if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
    if (window_left == -1 && window_right == -1) {
        *m = Mask{fa::kMaskNone, 0, 0};
    } else if (window_left == -1 && window_right == 0) {
        *m = Mask{fa::kMaskCausal, 0, 0};
    } else {
        // reaches beyond any sequence are unbounded; clamping keeps the
        // kernels' offset sums inside int
        auto reach = [](int w) { return w < 0 || w > fa::kWindowUnbounded ? fa::kWindowUnbounded : w; };
        *m = Mask{fa::kMaskWindow, reach(window_left), reach(window_right)};
    }
    return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nk, int d, float scale, Mask mask,
             int dtype, void* stream, int soft_exp2 = 0) {
    int st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    const long BH = (long)B * H;
    if (BH == 0 || Nq == 0) return FA_OK;
    if (!q || !o || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
    if (!aligned16(q) || !aligned16(o) || (Nk > 0 && (!aligned16(k) || !aligned16(v)))) return FA_ERR_ALIGN;
    if (lse && !aligned4(lse)) return FA_ERR_ALIGN;

    const int br = fa::fwd_rows_per_workgroup(dtype, d);
    const int n_qtiles = (Nq + br - 1) / br;
    fa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.Nq = Nq;
    p.Nk = Nk;
    p.n_qtiles = n_qtiles;
    const bool causal = mask.mode == fa::kMaskCausal;
    const int persist = fa::fwd_persist_grid(dtype, d, causal, BH, n_qtiles);
    p.paired = (persist > 0 || fa::fwd_pair_tiles(dtype, d, causal, BH, n_qtiles)) ? 1 : 0;
    p.persist = persist > 0 ? 1 : 0;
    p.n_slots = p.paired ? (n_qtiles + 1) / 2 : n_qtiles;
    p.total_wg = persist > 0 ? persist : (int)(BH * p.n_slots);
    p.BH = (int)BH;
    p.soft_exp2 = soft_exp2;
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.wl = mask.wl;
    p.wr = mask.wr;
    return hip_status(fa::launch_fwd(dtype, d, mask.mode, p, (hipStream_t)stream));
}

// Runs of 64-key tiles for the split-KV forward.  n_splits = 0 asks for
// enough workgroups to cover the GPU's 512 resident slots four times (at
// least 4 key tiles per run); the effective count is ceil(tiles / per_run).
struct SplitPlan {
    int n_qtiles, n_splits, tiles_per_split;
};

SplitPlan plan_split(long BH, int Nq, int Nk, int n_splits) {
    SplitPlan sp;
    sp.n_qtiles = (Nq + 127) / 128;
    const int n_kt = Nk > 0 ? (Nk + 63) / 64 : 1;
    int want = n_splits;
    if (want == 0) {
        const long units = BH * sp.n_qtiles;
        const long target = (2048 + units - 1) / units;
        const int cap = n_kt / 4 > 1 ? n_kt / 4 : 1;
        want = (int)(target < cap ? target : cap);
        if (want < 1) want = 1;
    }
    if (want > n_kt) want = n_kt;
    sp.tiles_per_split = (n_kt + want - 1) / want;
    sp.n_splits = (n_kt + sp.tiles_per_split - 1) / sp.tiles_per_split;
    return sp;
}

size_t split_part_bytes(long BH, int Nq, int d, int n_splits, size_t* lse_off) {
    const size_t rows = (size_t)n_splits * BH * Nq;
    const size_t obytes = (rows * d * sizeof(float) + 255) & ~(size_t)255;
    const size_t lbytes = (rows * sizeof(float) + 255) & ~(size_t)255;
    if (lse_off) *lse_off = obytes;
    return obytes + lbytes;
}

}  // namespace

extern "C" size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype, int n_splits) {
    if (check_common(B, H, Nq, Nk, d, 1.0f, dtype) != FA_OK) return 0;
    if (dtype != FA_BF16 || n_splits < 0 || n_splits > FA_MAX_SPLITS) return 0;
    const long BH = (long)B * H;
    if (BH == 0 || Nq == 0) return 0;
    const SplitPlan sp = plan_split(BH, Nq, Nk, n_splits);
    return split_part_bytes(BH, Nq, d, sp.n_splits, nullptr);
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, float scale, int causal,
                              int dtype, int n_splits, void* workspace, size_t workspace_bytes,
                              void* stream) {
    int st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (n_splits < 0 || n_splits > FA_MAX_SPLITS) return FA_ERR_SHAPE;
    const long BH = (long)B * H;
    if (BH == 0 || Nq == 0) return FA_OK;
    if (!q || !o || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
    if (!aligned16(q) || !aligned16(o) || (Nk > 0 && (!aligned16(k) || !aligned16(v)))) return FA_ERR_ALIGN;
    if (lse && !aligned4(lse)) return FA_ERR_ALIGN;
    const SplitPlan sp = plan_split(BH, Nq, Nk, n_splits);
    size_t lse_off = 0;
    const size_t need = split_part_bytes(BH, Nq, d, sp.n_splits, &lse_off);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    // one workgroup per (head, query tile, run), then one per output row
    if ((long double)BH * sp.n_qtiles * sp.n_splits > 2.0e9L || (long double)BH * Nq > 2.0e9L)
        return FA_ERR_SHAPE;

    fa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.Nq = Nq;
    p.Nk = Nk;
    p.n_qtiles = sp.n_qtiles;
    p.n_slots = sp.n_qtiles;
    p.paired = 0;
    p.total_wg = (int)(BH * sp.n_qtiles * sp.n_splits);
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.BH = (int)BH;
    p.n_splits = sp.n_splits;
    p.tiles_per_split = sp.tiles_per_split;
    p.o_part = (float*)workspace;
    p.lse_part = (float*)((char*)workspace + lse_off);
    return hip_status(fa::launch_fwd_split(d, causal != 0, p, (hipStream_t)stream));
}

int fa::bwd_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dO, const void* dq, const void* dk, const void* dv, int B, int H,
                       int Nq, int Nk, int d, float scale, int dtype, bool* work) {
    *work = false;
    const int st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    // the key-side grid (64- or 128-key tiles) must fit in 32 bits as well
    if ((long double)B * H * ((Nk + 63) / 64 + 1) > 2.0e9L) return FA_ERR_SHAPE;
    if ((long)B * H == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
    const bool has_q = Nq > 0, has_k = Nk > 0;
    if ((has_q && (!q || !o || !lse || !dO || !dq)) || (has_k && (!k || !v || !dk || !dv))) return FA_ERR_NULL;
    if (has_q && (!aligned16(q) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) || !aligned4(lse)))
        return FA_ERR_ALIGN;
    if (has_k && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))) return FA_ERR_ALIGN;
    *work = true;
    return FA_OK;
}

namespace {

// The backward workspace over `rows` query rows: LSE2 and D (float32 row
// vectors), and in the atomic mode the float32 dQ buffer [rows, d]; each part
// rounded up to 256 bytes.
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t bwd_ws_bytes(size_t rows, int d, int deterministic) {
    return 2 * round256(rows * sizeof(float)) + (deterministic ? 0 : round256(rows * d * sizeof(float)));
}

}  // namespace

extern "C" size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype, int deterministic) {
    if (check_common(B, H, Nq, Nk, d, 1.0f, dtype) != FA_OK) return 0;
    // fp32 has one (deterministic) algorithm whatever the argument says
    return bwd_ws_bytes((size_t)B * H * Nq, d, deterministic || dtype == FA_F32);
}

namespace {

int bwd_impl(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dO, void* dq, void* dk, void* dv,
             int B, int H, int Nq, int Nk, int d, float scale, Mask mask,
             int dtype, int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
    bool work = false;
    int st = fa::bwd_check_args(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, dtype, &work);
    if (st != FA_OK || !work) return st;
    const long BH = (long)B * H;
    const size_t need = fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype, deterministic);
    if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;

    const size_t rows = (size_t)BH * Nq;
    const size_t vec_bytes = round256(rows * sizeof(float));
    fa::BwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.dO = dO;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.lse2 = (float*)workspace;
    p.dvec = (float*)((char*)workspace + vec_bytes);
    p.dqacc = deterministic ? nullptr : (float*)((char*)workspace + 2 * vec_bytes);
    p.Nq = Nq;
    p.Nk = Nk;
    p.BH = (int)BH;
    p.scale = scale;
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.wl = mask.wl;
    p.wr = mask.wr;
    if (dtype == FA_F32) {
        p.dqacc = nullptr;
        p.q_slots = (Nq + 63) / 64;
        p.kv_slots = (Nk + 63) / 64;
        return hip_status(fa::launch_bwd_f32(d, mask.mode, p, (hipStream_t)stream));
    }
    const int n_kt = (Nk + 127) / 128, n_qt = (Nq + 127) / 128;
    const bool causal = mask.mode == fa::kMaskCausal;
    p.kv_paired = fa::bwd_pair_tiles(causal, BH, n_kt) ? 1 : 0;
    p.kv_slots = p.kv_paired ? (n_kt + 1) / 2 : n_kt;
    p.q_paired = fa::bwd_pair_tiles(causal, BH, n_qt) ? 1 : 0;
    p.q_slots = p.q_paired ? (n_qt + 1) / 2 : n_qt;
    if (deterministic) return hip_status(fa::launch_bwd(d, mask.mode, false, p, (hipStream_t)stream));
    return hip_status(fa::launch_bwd_atomic(d, mask.mode, false, p, (long)rows, (hipStream_t)stream));
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal_mask(causal), dtype, stream);
}

extern "C" int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, float scale,
                             int window_left, int window_right, int dtype, void* stream) {
    Mask m;
    const int st = window_mask(window_left, window_right, &m);
    if (st != FA_OK) return st;
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, m, dtype, stream);
}

extern "C" int fa_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Nq, int Nk, int d, float scale, int causal,
                                int dtype, int period, void* stream) {
    const int st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (period != 2 && period != 4 && period != 8) return FA_ERR_PERIOD;
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal_mask(causal), dtype, stream, period);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, void* dq, void* dk, void* dv,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, int deterministic, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal_mask(causal),
                    dtype, deterministic, workspace, workspace_bytes, stream);
}

extern "C" int fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             int B, int H, int Nq, int Nk, int d, float scale,
                             int window_left, int window_right, int dtype, int deterministic,
                             void* workspace, size_t workspace_bytes, void* stream) {
    Mask m;
    const int st = window_mask(window_left, window_right, &m);
    if (st != FA_OK) return st;
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, m, dtype, deterministic,
                    workspace, workspace_bytes, stream);
}

namespace {

// Checks of a variable-length call's sizes, head dim, dtype (bf16 only),
// scale and offset pointers.  Leaves *work = false when there is nothing
// to compute.
int check_varlen(const int* cu_q, const int* cu_k, int B, int H, int total_q, int total_k,
                 int max_q, int max_k, int d, float scale, int dtype, bool* work) {
    if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return FA_ERR_SHAPE;
    if (max_q > FA_MAX_SEQ || max_k > FA_MAX_SEQ) return FA_ERR_SHAPE;
    const long double elems = (long double)H * (total_q > total_k ? total_q : total_k) * 128.0L;
    if (elems > 4.0e18L) return FA_ERR_SHAPE;
    // grids: B*H workgroups per 64 rows of the longest sequence, and the
    // backward pre-pass over H*total_q rows
    if ((long double)B * H * ((max_q > max_k ? max_q : max_k) / 64 + 2) > 2.0e9L) return FA_ERR_SHAPE;
    if ((long double)H * total_q > 2.0e11L) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    *work = B > 0 && H > 0;
    if (*work && (!cu_q || !cu_k)) return FA_ERR_NULL;
    if (*work && (!aligned4(cu_q) || !aligned4(cu_k))) return FA_ERR_ALIGN;
    return FA_OK;
}

fa::VarlenParams varlen_params(const int* cu_q, const int* cu_k, int B, int H, int total_q,
                               int total_k, int max_q, int max_k) {
    fa::VarlenParams v;
    v.cu_q = cu_q;
    v.cu_k = cu_k;
    v.B = B;
    v.H = H;
    v.total_q = total_q;
    v.total_k = total_k;
    v.max_q = max_q;
    v.max_k = max_k;
    return v;
}

}  // namespace

extern "C" int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                             float scale, int window_left, int window_right, int dtype, void* stream) {
    Mask m;
    int st = window_mask(window_left, window_right, &m);
    if (st != FA_OK) return st;
    bool work = false;
    st = check_varlen(cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k,
                      d, scale, dtype, &work);
    if (st != FA_OK) return st;
    if (!work || total_q == 0 || max_seqlen_q == 0) return FA_OK;
    if (!q || !o || (total_k > 0 && (!k || !v))) return FA_ERR_NULL;
    if (!aligned16(q) || !aligned16(o) || (total_k > 0 && (!aligned16(k) || !aligned16(v)))) return FA_ERR_ALIGN;
    if (lse && !aligned4(lse)) return FA_ERR_ALIGN;

    fa::FwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.n_slots = (max_seqlen_q + 127) / 128;   // query tiles of the longest sequence
    p.n_qtiles = p.n_slots;
    p.paired = 0;
    p.total_wg = (int)((long)B * H * p.n_slots);
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.wl = m.wl;
    p.wr = m.wr;
    p.vl = varlen_params(cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k);
    return hip_status(fa::launch_fwd_varlen(d, m.mode, p, (hipStream_t)stream));
}

extern "C" size_t fa_bwd_varlen_workspace_bytes(int H, int total_q, int d, int dtype, int deterministic) {
    // fa_bwd's workspace over the H * total_q packed rows
    if (H < 0 || total_q < 0 || (d != 64 && d != 128) || dtype != FA_BF16) return 0;
    if ((long double)H * total_q > 2.0e11L) return 0;
    return bwd_ws_bytes((size_t)H * total_q, d, deterministic);
}

extern "C" int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dO, void* dq, void* dk, void* dv,
                             const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                             float scale, int window_left, int window_right, int dtype,
                             int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
    Mask m;
    int st = window_mask(window_left, window_right, &m);
    if (st != FA_OK) return st;
    bool work = false;
    st = check_varlen(cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k,
                      d, scale, dtype, &work);
    if (st != FA_OK) return st;
    if (!work || (total_q == 0 && total_k == 0)) return FA_OK;
    const bool has_q = total_q > 0, has_k = total_k > 0;
    if ((has_q && (!q || !o || !lse || !dO || !dq)) || (has_k && (!k || !v || !dk || !dv))) return FA_ERR_NULL;
    if (has_q && (!aligned16(q) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) || !aligned4(lse)))
        return FA_ERR_ALIGN;
    if (has_k && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))) return FA_ERR_ALIGN;
    const size_t need = fa_bwd_varlen_workspace_bytes(H, total_q, d, dtype, deterministic);
    if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;

    const size_t rows = (size_t)H * total_q;
    const size_t vec_bytes = round256(rows * sizeof(float));
    fa::BwdParams p = {};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.dO = dO;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.lse2 = (float*)workspace;
    p.dvec = (float*)((char*)workspace + vec_bytes);
    p.dqacc = deterministic ? nullptr : (float*)((char*)workspace + 2 * vec_bytes);
    p.BH = (int)((long)B * H);
    // workgroups per (batch, head): tiles of the longest sequence, unpaired
    p.kv_slots = (max_seqlen_k + 127) / 128;
    p.q_slots = (max_seqlen_q + 127) / 128;
    p.kv_paired = 0;
    p.q_paired = 0;
    p.scale = scale;
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.wl = m.wl;
    p.wr = m.wr;
    p.vl = varlen_params(cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k);
    if (deterministic) return hip_status(fa::launch_bwd(d, m.mode, true, p, (hipStream_t)stream));
    return hip_status(fa::launch_bwd_atomic(d, m.mode, true, p, (long)rows, (hipStream_t)stream));
}

extern "C" const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "negative size or sizes beyond the supported limits";
        case FA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
        case FA_ERR_DTYPE: return "unsupported dtype for this call";
        case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned (lse: 4-byte)";
        case FA_ERR_WORKSPACE: return "workspace is NULL or smaller than fa_bwd_workspace_bytes()";
        case FA_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_WINDOW: return "window reaches must be >= 0, or -1 for an unbounded side";
        case FA_ERR_SCRATCH: return "the call needs more than fa_bwd_noalloc's static buffer (FA_NOALLOC_SCRATCH_BYTES)";
        case FA_ERR_PERIOD: return "the software-exponential period must be 2, 4 or 8";
        default: return "unknown status";
    }
}
