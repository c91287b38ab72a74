// Attention backward by recomputation for gfx950 ("01 · IO-awareness、online
// softmax 与 tiling" §5; "让注意力计算留在片上" §04):
//
//   P = exp(scale*S - LSE) rebuilt tile by tile from the saved LSE,
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Two launches on the caller's stream, no atomics (deterministic):
//   1. dQ   : one workgroup per (batch*head, 128-query tile) walking the key
//             tiles it can see, like the forward pass.  Each wave owns 32
//             queries: Q and dO sit in registers, K / V tiles stream through
//             LDS, dQ accumulates in registers.  It first computes its rows'
//             D = rowsum(dO * O) and LSE in log2 units (+inf for a row with
//             no visible key, so its P is exactly 0) and writes both to the
//             workspace.
//   2. dK/dV: one workgroup per (batch*head, 128-key tile) walking the query
//             tiles that can see it (the loop order of §5), reading D and
//             LSE2 from the workspace.  Each wave owns 32 keys: K and V sit in
//             registers, Q / dO tiles stream through LDS, dK and dV
//             accumulate in registers for the whole walk.
// S and dP are computed in both (7 products instead of 5) in exchange for no
// dQ atomics and no dS round trip through memory.
//
// Register formulation (32x32x16 bf16 MFMA, fp32 accumulate).  In each main
// kernel the products over the head dimension (S, dP) take the streamed tile
// as the A operand (ds_read_b128 rows) and the resident operand from
// registers, so each lane ends up owning ONE row of the resident side (a key
// in dK/dV, a query in dQ) with 16 of its partners per 32-block -- exactly the B
// operand layout of the products over the streamed side (dV^T += dO^T P and
// dK^T += Q^T dS, dQ^T += K^T dS^T), whose A operands are
// transposed reads (ds_read_b64_tr_b16) of the same LDS tiles.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// Pack the P (or dS) values of a 32x32 accumulator into the bf16 B operands
// of two 16-wide k-steps: item i = 4g + e of the accumulator (partner
// 8g + 4*(lane/32) + e of the block) goes to k-step (g/2), slot 4(g%2) + e,
// which is the order tile_read_tr hands out the matching rows.
__device__ __forceinline__ void pack_pairs(const float (&x)[16], u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        lo[i >> 1] = pack_bf16x2(x[i], x[i + 1]);
        hi[i >> 1] = pack_bf16x2(x[8 + i], x[8 + i + 1]);
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  BKV = 128 keys per workgroup (4 waves x 32), BQ = 64 queries per
// step.  LDS per stage: Q tile, dO tile (swizzled [BQ][D] bf16) and the BQ
// values of LSE*log2e and D; two stages, the next one filled while the
// current one is used.
// ---------------------------------------------------------------------------
// PART: 0 computes dK and dV, 1 only dV (S and P^T dO), 2 only dK (S, dP,
// dS and dS^T Q).  At d = 128 both accumulators, K and V do not fit two
// waves per SIMD (about 440 registers), so the key side runs as a dV kernel
// and a dK kernel, recomputing S in each, at two waves per SIMD.
template <int D, int MASK, bool VARLEN = false, int PART = 0>
__global__ void __launch_bounds__(256, (D == 64 || PART != 0) ? 2 : 1) bwd_dkdv_kernel(BwdParams p) {
    constexpr bool kDV = PART != 2, kDK = PART != 1;
    constexpr int BKV = 128, BQ = 64;
    constexpr int NQB = BQ / 32;              // 32-query blocks per step
    constexpr int NQC = BQ / 16;              // 16-query k-steps
    constexpr int NKK = D / 16;               // 16-wide k-steps over d
    constexpr int NDB = D / 32;               // 32-row blocks of dK^T / dV^T
    constexpr int T_BYTES = BQ * D * 2;       // one Q or dO tile
    constexpr int V_OFF = 2 * T_BYTES;        // row vectors after the two tiles
    constexpr int STAGE = V_OFF + 2 * BQ * 4; // + LSE2[BQ] + D[BQ]
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hg = lane >> 5;
    // key tiles of this workgroup: j (ascending j = heavy causal tiles
    // first), then with pairing its mirror n-1-j (equal causal work per
    // workgroup)
    int bh, slot;
    if (VARLEN) varlen_slot(p.vl, p.kv_slots, blockIdx.x, bh, slot);
    else map_head_tile(blockIdx.x, p.BH * p.kv_slots, p.kv_slots, bh, slot);
    // the (batch, head) pair's lengths and first rows (variable-length
    // batches: its own sequence's; a workgroup past its key tiles exits)
    SeqGeometry sg;
    if constexpr (VARLEN) sg = seq_geometry(p.vl, bh);
    else sg = SeqGeometry{p.Nq, p.Nk, (size_t)bh * p.Nq, (size_t)bh * p.Nk};
    const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
    // query q sees key j iff j <= q + offr (causal, windows) and, for a
    // window, j >= q + offl (the mask family of the forward kernels)
    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    const int n_kt = (Nk + BKV - 1) / BKV;
    if (VARLEN && slot >= n_kt) return;
    const int n_items = (p.kv_paired && slot != n_kt - 1 - slot) ? 2 : 1;

    const bf16* Qh = (const bf16*)p.q + sg.q_row0 * D;
    const bf16* Kh = (const bf16*)p.k + sg.k_row0 * D;
    const bf16* Vh = (const bf16*)p.v + sg.k_row0 * D;
    const bf16* dOh = (const bf16*)p.dO + sg.q_row0 * D;

    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, (uint32_t)Nk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh, (uint32_t)Nk * D * 2);
    const TileCopy<D, BQ, 4> copier(wave, lane);
    const i32x4 rq_w = make_rsrc_words(Qh, (uint32_t)Nq * D * 2);
    const i32x4 rdo_w = make_rsrc_words(dOh, (uint32_t)Nq * D * 2);
    const uint32_t smem_lds = lds_address(smem);

    for (int it = 0; it < n_items; ++it) {
    const int kt = it == 0 ? slot : n_kt - 1 - slot;
    const int k0 = kt * BKV;
    const int kw = k0 + wave * 32;            // this wave's first key
    const int kj = kw + l32;                  // this lane's key

    // K^T and V^T as B operands: lane = key, 8 consecutive d per k-step
    // (rows past Nk read as zero; their dK / dV are never written).
    bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const uint32_t o = (uint32_t)kj * D * 2 + (16 * kk + 8 * hg) * 2;
        kreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rk, o, 0));
        if constexpr (kDK) vreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rv, o, 0));
    }

    // Query range: the walk starts at the first query tile that sees the
    // tile's first key (q >= j - offr) and, for a window, ends after the last
    // query that sees its last key (q <= j - offl).
    const int qstart = kRight ? max(0, k0 - offr) : 0;
    const int qt0 = qstart / BQ;
    const int qend = kLeft ? max(0, min(Nq, k0 + BKV - offl)) : Nq;
    const int n_qt = (qend + BQ - 1) / BQ;
    const int wq_first = kRight ? kw - offr : 0;        // first query that sees this wave's first key
    const int wq_last = kLeft ? kw + 31 - offl : Nq;    // last query that sees its last key

    auto load_step = [&](int qt, int stage) {
        const uint32_t base = smem_lds + stage * STAGE;
        copier.issue(rq_w, qt * BQ, base);
        copier.issue(rdo_w, qt * BQ, base + T_BYTES);
    };
    // The step's LSE2 and D values (one query per lane of wave 0) are loaded
    // one step ahead into registers and written to the stage's LDS slot just
    // before the end-of-step barrier.  Rows past Nq get LSE2 = +inf (P = 0).
    static_assert(BQ == 64, "one query per lane of wave 0");
    const float* L2h = p.lse2 + sg.q_row0;
    const float* Dh = p.dvec + sg.q_row0;
    float nl2 = INFINITY, ndd = 0.f;
    auto fetch_vec = [&](int qt) {
        const int q = qt * BQ + lane;
        nl2 = q < Nq ? L2h[q] : INFINITY;
        ndd = q < Nq ? Dh[q] : 0.f;
    };
    auto store_vec = [&](int stage) {
        float* v = (float*)(smem + stage * STAGE + V_OFF);
        v[lane] = nl2;
        v[BQ + lane] = ndd;
    };

    f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dkacc[db] = zero16();
        dvacc[db] = zero16();
    }

    if (qt0 < n_qt) {
        load_step(qt0, 0);
        if (wave == 0) {
            fetch_vec(qt0);
            store_vec(0);
        }
    }
    // vmcnt(0): K, V registers and the first stage.  The compiler is then
    // told the registers are loaded (mark_loaded), so it puts no waits for
    // them inside the walk, where the hardware counter also counts the next
    // stage's copies.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (qt0 < n_qt) tile_barrier();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        mark_loaded(kreg[kk]);
        if constexpr (kDK) mark_loaded(vreg[kk]);
    }

    for (int qt = qt0; qt < n_qt; ++qt) {
        const int st = (qt - qt0) & 1;
        const char* qs = smem + st * STAGE;
        const char* dos = qs + T_BYTES;
        const float* l2s = (const float*)(qs + V_OFF);
        const float* dds = l2s + BQ;
        const int q0 = qt * BQ;
        const bool has_next = qt + 1 < n_qt;
        if (has_next) {
            load_step(qt + 1, st ^ 1);
            if (wave == 0) fetch_vec(qt + 1);
        }

        if (q0 + BQ - 1 >= wq_first && (!kLeft || q0 <= wq_last)) {
            // ---- S = Q K^T and dP = dO V^T (lane = key, items = queries) ----
            f32x16 s[NQB], dp[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                s[qb] = zero16();
                dp[qb] = zero16();
            }
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    s[qb] = mfma_bf16(tile_read_row<D>(qs, qb * 32, kk, lane), kreg[kk], s[qb]);
                    if constexpr (kDK)
                        dp[qb] = mfma_bf16(tile_read_row<D>(dos, qb * 32, kk, lane), vreg[kk], dp[qb]);
                }
            // At d = 128 the operand reads run four ahead of the MFMAs here and
            // two per MFMA in the products below (+4.9% on the Llama-shaped
            // backward); at d = 64 the compiler's own order measured 1.8% faster.
            if constexpr (D == 128) {
                constexpr int nm = (kDK ? 2 : 1) * NKK * NQB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < nm - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            // ---- P = 2^(S*scale*log2e - LSE2), dS = P * (dP - D) ----
            // ---- mask: only steps that straddle a bound or the tail ----
            const bool need_mask = (q0 + BQ > Nq) || (kRight && q0 + offr < kw + 31) ||
                                   (kLeft && q0 + BQ - 1 + offl > kw);
            if (need_mask) {
                // item 4g+e of block qb is query q0 + 4*hg + o, o = qb*32 + g*8 + e:
                // visible iff lo <= o <= hi (q < Nq, kj <= q + offr, kj >= q + offl)
                const int qb0 = q0 + 4 * hg;
                const int lo = kRight ? kj - offr - qb0 : -(1 << 30);
                int hi = Nq - 1 - qb0;
                if (kLeft) hi = min(hi, kj - offl - qb0);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int o = qb * 32 + (i >> 2) * 8 + (i & 3);
                        if (o < lo || o > hi) s[qb][i] = -INFINITY;
                    }
            }
            u32x4 pw[NQC], dsw[NQC];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float pv[16], dsv[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ql = qb * 32 + g * 8 + 4 * hg;   // local query of item 4g
                    const f32x4 l2 = *(const f32x4*)(l2s + ql);
                    f32x4 dd = {};
                    if constexpr (kDK) dd = *(const f32x4*)(dds + ql);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sv = s[qb][4 * g + e];
                        const float pe = exp2_hw(fmaf(sv, p.scale_log2, -l2[e]));
                        pv[4 * g + e] = pe;
                        if constexpr (kDK) dsv[4 * g + e] = pe * (dp[qb][4 * g + e] - dd[e]);
                    }
                }
                if constexpr (kDV) pack_pairs(pv, pw[2 * qb], pw[2 * qb + 1]);
                if constexpr (kDK) pack_pairs(dsv, dsw[2 * qb], dsw[2 * qb + 1]);
            }
            // ---- dV^T += dO^T P ;  dK^T += Q^T dS ----
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    if constexpr (kDV)
                        dvacc[db] = mfma_bf16(tile_read_tr<D>(dos, qc * 16, db * 32, lane),
                                              __builtin_bit_cast(bf16x8, pw[qc]), dvacc[db]);
                    if constexpr (kDK)
                        dkacc[db] = mfma_bf16(tile_read_tr<D>(qs, qc * 16, db * 32, lane),
                                              __builtin_bit_cast(bf16x8, dsw[qc]), dkacc[db]);
                }
            }
            if constexpr (D == 128) {   // two transposed reads per MFMA
                constexpr int nm = ((kDV ? 1 : 0) + (kDK ? 1 : 0)) * NQC * NDB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
                for (int i = 0; i < nm; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    if (i < nm - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
            }
        }

        if (has_next) {
            if (wave == 0) store_vec(st ^ 1);
            vmem_wait_all();   // this wave's copies of the next stage landed
        }
        // the next step's LSE2 / D loads are complete on every path (see
        // mark_loaded), so the next fetch_vec adds no wait behind the copies
        mark_loaded(nl2);
        mark_loaded(ndd);
        tile_barrier();
    }

    // ---- dK = scale * dK^T, dV = dV^T (lane = key, items = d) ----
    if (kj < Nk) {
        bf16* dKr = (bf16*)p.dk + sg.k_row0 * D + (size_t)kj * D;
        bf16* dVr = (bf16*)p.dv + sg.k_row0 * D + (size_t)kj * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = db * 32 + g * 8 + 4 * hg;
                if constexpr (kDK) {
                    u32x2 wk;
                    wk[0] = pack_bf16x2(dkacc[db][4 * g] * p.scale, dkacc[db][4 * g + 1] * p.scale);
                    wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale);
                    *(u32x2*)(dKr + dcol) = wk;
                }
                if constexpr (kDV) {
                    u32x2 wv;
                    wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                    wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                    *(u32x2*)(dVr + dcol) = wv;
                }
            }
    }
    }   // items
}

// ---------------------------------------------------------------------------
// 3. dQ.  BQ = 128 queries per workgroup (4 waves x 32), BC = 64 keys per
// step; K and V tiles double-buffered in LDS exactly as in the forward pass.
// ---------------------------------------------------------------------------
template <int D, int MASK, bool VARLEN = false>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdParams p) {
    constexpr int BQ = 128, BC = 64;
    constexpr int NKK = D / 16;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int NKC = BC / 16;
    constexpr int T_BYTES = BC * D * 2;
    constexpr int BUF_BYTES = 2 * T_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hg = lane >> 5;
    // query tiles of this workgroup: n-1-j (heavy causal tiles first), then
    // with pairing its mirror j
    int bh, slot;
    if (VARLEN) varlen_slot(p.vl, p.q_slots, blockIdx.x, bh, slot);
    else map_head_tile(blockIdx.x, p.BH * p.q_slots, p.q_slots, bh, slot);
    SeqGeometry sg;
    if constexpr (VARLEN) sg = seq_geometry(p.vl, bh);
    else sg = SeqGeometry{p.Nq, p.Nk, (size_t)bh * p.Nq, (size_t)bh * p.Nk};
    const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    const int n_qt = (Nq + BQ - 1) / BQ;
    if (VARLEN && slot >= n_qt) return;
    const int n_items = (p.q_paired && slot != n_qt - 1 - slot) ? 2 : 1;

    const bf16* Qh = (const bf16*)p.q + sg.q_row0 * D;
    const bf16* Kh = (const bf16*)p.k + sg.k_row0 * D;
    const bf16* Vh = (const bf16*)p.v + sg.k_row0 * D;
    const bf16* dOh = (const bf16*)p.dO + sg.q_row0 * D;

    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh, (uint32_t)Nq * D * 2);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dOh, (uint32_t)Nq * D * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const bf16*)p.o + sg.q_row0 * D, (uint32_t)Nq * D * 2);
    const TileCopy<D, BC, 4> copier(wave, lane);
    const i32x4 rk_w = make_rsrc_words(Kh, (uint32_t)Nk * D * 2);
    const i32x4 rv_w = make_rsrc_words(Vh, (uint32_t)Nk * D * 2);
    const uint32_t smem_lds = lds_address(smem);

    for (int it = 0; it < n_items; ++it) {
    const int qt = it == 0 ? n_qt - 1 - slot : slot;
    const int q0 = qt * BQ;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    // key tiles [t_first, ntiles) of this query tile, as in the forward pass
    const int kend = kRight ? min(Nk, q0 + BQ + offr) : Nk;
    const int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;
    const int t_first = kLeft ? max(0, q0 + offl) / BC : 0;
    const int kend_w = kRight ? min(Nk, qw + 32 + offr) : Nk;
    const int kbeg_w = kLeft ? qw + offl : 0;

    // this lane's query: Q and dO as B operands, and the same columns of O
    // (for D = rowsum(dO * O)), its LSE
    bf16x8 qreg[NKK], doreg[NKK];
    u32x4 oreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const uint32_t o = (uint32_t)qi * D * 2 + (16 * kk + 8 * hg) * 2;
        qreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rq, o, 0));
        doreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rdo, o, 0));
        oreg[kk] = buf_load128(ro, o, 0);
    }
    const float lse_i = qi < Nq ? p.lse[sg.q_row0 + qi] : -INFINITY;

    auto load_tile = [&](int k0, int buf) {
        copier.issue(rk_w, k0, smem_lds + buf * BUF_BYTES);
        copier.issue(rv_w, k0, smem_lds + buf * BUF_BYTES + T_BYTES);
    };

    f32x16 dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] = zero16();

    if (ntiles > t_first) load_tile(t_first * BC, 0);
    // vmcnt(0): Q, dO, LSE2, D registers and the first tiles; then the same
    // mark_loaded as in the dK/dV kernel
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (ntiles > t_first) tile_barrier();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        mark_loaded(qreg[kk]);
        mark_loaded(doreg[kk]);
        mark_loaded(oreg[kk]);
    }
    mark_loaded(lse_i);
    // D = rowsum(dO * O) in fp32 (this lane's half of the columns, then the
    // partner lane's) and LSE * log2(e) (+inf for a row with no visible key,
    // so its P is exactly 0).  The dK/dV kernel, launched after this one,
    // reads both from the workspace.
    float dd = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 dw = __builtin_bit_cast(u32x4, doreg[kk]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dd += bf16_lo(dw[i]) * bf16_lo(oreg[kk][i]) + bf16_hi(dw[i]) * bf16_hi(oreg[kk][i]);
    }
    dd = xhalf_sum(dd);
    // rows past Nq: P = 0
    const float l2 = qi < Nq ? (lse_i == -INFINITY ? INFINITY : lse_i * kLog2e) : INFINITY;
    if (qi < Nq && hg == 0) {
        p.lse2[sg.q_row0 + qi] = l2;
        p.dvec[sg.q_row0 + qi] = dd;
    }
    // dP - D in the dP product itself: one more k-step whose A operand is 1
    // in columns 0 and 1 for every key and whose B operand holds -D split
    // into two bf16 parts (hi + lo = -D within 2^-16 relative), so the
    // accumulator ends at dP - D and dS = P * acc needs no subtraction
    u32x4 ones_w = zero_u32x4(), negd_w = zero_u32x4();
    if (hg == 0) {
        const float dh = bf16_lo(pack_bf16x2(-dd, 0.f));   // -D rounded to bf16
        ones_w[0] = pack_bf16x2(1.f, 1.f);
        negd_w[0] = pack_bf16x2(-dd, -dd - dh);
    }
    const bf16x8 ones_a = __builtin_bit_cast(bf16x8, ones_w), negd_b = __builtin_bit_cast(bf16x8, negd_w);

    for (int t = t_first; t < ntiles; ++t) {
        const int k0 = t * BC;
        const int buf = (t - t_first) & 1;
        const char* kbuf = smem + buf * BUF_BYTES;
        const char* vbuf = kbuf + T_BYTES;
        const bool has_next = t + 1 < ntiles;
        if (has_next) load_tile(k0 + BC, (t + 1 - t_first) & 1);

        if (k0 < kend_w && (!kLeft || k0 + BC > kbeg_w)) {
            // ---- S^T = K Q^T, dP^T = V dO^T (lane = query, items = keys) ----
            f32x16 s[NKB], dp[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s[kb] = zero16();
                dp[kb] = mfma_bf16(ones_a, negd_b, zero16());   // -D in every item
            }
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    s[kb] = mfma_bf16(tile_read_row<D>(kbuf, kb * 32, kk, lane), qreg[kk], s[kb]);
                    dp[kb] = mfma_bf16(tile_read_row<D>(vbuf, kb * 32, kk, lane), doreg[kk], dp[kb]);
                }
            // operand reads four ahead of the MFMAs at d = 128, as in dK/dV
            if constexpr (D == 128) {
                constexpr int nm = 2 * NKK * NKB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < nm - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            // ---- dS^T = P * (dP - D), P = 2^(S*scale*log2e - LSE2) ----
            // ---- mask: only tiles that straddle a bound or the tail ----
            const bool need_mask = (k0 + BC > Nk) || (kRight && k0 + BC - 1 > qw + offr) ||
                                   (kLeft && k0 < qw + 31 + offl);
            if (need_mask) {
                // item i of block kb is key k0 + 4*hg + o, o = kb*32 + (i/4)*8 + i%4:
                // visible iff lo <= o <= hi (key < Nk, key <= qi + offr, key >= qi + offl)
                const int kb0 = k0 + 4 * hg;
                int hi = Nk - 1 - kb0;
                if (kRight) hi = min(hi, qi + offr - kb0);
                const int lo = kLeft ? qi + offl - kb0 : -(1 << 30);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
                        if (o < lo || o > hi) s[kb][i] = -INFINITY;
                    }
            }
            u32x4 dsw[NKC];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float dsv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float sv = s[kb][i];
                    const float pe = exp2_hw(fmaf(sv, p.scale_log2, -l2));
                    dsv[i] = pe * dp[kb][i];   // dp holds dP - D
                }
                pack_pairs(dsv, dsw[2 * kb], dsw[2 * kb + 1]);
            }
            // ---- dQ^T += K^T dS^T ----
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 sb = __builtin_bit_cast(bf16x8, dsw[kc]);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dqacc[db] = mfma_bf16(tile_read_tr<D>(kbuf, kc * 16, db * 32, lane), sb, dqacc[db]);
            }
            if constexpr (D == 128) {   // two transposed reads per MFMA
                constexpr int nm = NKC * NDB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
                for (int i = 0; i < nm; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    if (i < nm - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
            }
        }

        if (has_next) vmem_wait_all();
        tile_barrier();
    }

    // ---- dQ = scale * dQ^T (lane = query, items = d) ----
    if (qi < Nq) {
        bf16* dQr = (bf16*)p.dq + sg.q_row0 * D + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(dqacc[db][4 * g] * p.scale, dqacc[db][4 * g + 1] * p.scale);
                w[1] = pack_bf16x2(dqacc[db][4 * g + 2] * p.scale, dqacc[db][4 * g + 3] * p.scale);
                *(u32x2*)(dQr + db * 32 + g * 8 + 4 * hg) = w;
            }
    }
    }   // items
}

// ---------------------------------------------------------------------------
// part: -1 the dQ kernel, 0/1/2 the key-side kernel's PART
template <int D, int MASK, bool VARLEN>
static const void* bwd_kernel_m(int part) {
    if (part < 0) return (const void*)bwd_dq_kernel<D, MASK, VARLEN>;
    if constexpr (D == 64) return (const void*)bwd_dkdv_kernel<D, MASK, VARLEN, 0>;
    else return part == 1 ? (const void*)bwd_dkdv_kernel<D, MASK, VARLEN, 1> : (const void*)bwd_dkdv_kernel<D, MASK, VARLEN, 2>;
}

template <int D, bool VARLEN>
static const void* bwd_kernel(int part, int mask) {
    if (mask == kMaskCausal) return bwd_kernel_m<D, kMaskCausal, VARLEN>(part);
    if (mask == kMaskWindow) return bwd_kernel_m<D, kMaskWindow, VARLEN>(part);
    return bwd_kernel_m<D, kMaskNone, VARLEN>(part);
}

template <int D>
static const void* bwd_kernel(int part, int mask, bool varlen) {
    return varlen ? bwd_kernel<D, true>(part, mask) : bwd_kernel<D, false>(part, mask);
}

template <int D>
static hipError_t launch_bwd_d(int mask, bool varlen, const BwdParams& p, hipStream_t s) {
    BwdParams pp = p;
    void* args[] = {&pp};
    // dQ first: it also writes every query row's D and LSE * log2(e) to the
    // workspace, which the dK/dV kernel reads (stream order)
    const long grid_q = (long)p.BH * p.q_slots;
    if (grid_q > 0) {   // with Nk == 0 every row is empty and dQ = 0 is written
        const void* fn = bwd_kernel<D>(-1, mask, varlen);
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid_q), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    const long grid_kv = (long)p.BH * p.kv_slots;
    // with Nq == 0 the walk is empty and dK = dV = 0 are written; d = 128:
    // the dV kernel, then the dK kernel
    for (int part = D == 64 ? 0 : 1; grid_kv > 0 && part <= (D == 64 ? 0 : 2); ++part) {
        const void* fn = bwd_kernel<D>(part, mask, varlen);
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid_kv), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Pair mirrored tiles in the dK/dV and dQ kernels on large causal grids of
// short sequences (every workgroup then does the same causal work; measured
// +11% at N=4096 d=64, +2% at d=128).
bool bwd_pair_tiles(bool causal, long bh, int n_tiles) {
    return causal && n_tiles >= 2 && n_tiles <= 64 && bh * n_tiles >= 4 * 512;
}

hipError_t launch_bwd(int d, int mask, bool varlen, BwdParams p, hipStream_t stream) {
    return d == 64 ? launch_bwd_d<64>(mask, varlen, p, stream) : launch_bwd_d<128>(mask, varlen, p, stream);
}

}  // namespace fa
