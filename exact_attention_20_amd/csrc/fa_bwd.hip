// Attention backward by recomputation for gfx950 ("01 · IO-awareness、online
// softmax 与 tiling" §5; "让注意力计算留在片上" §04):
//
//   P = exp(scale*S - LSE) rebuilt tile by tile from the saved LSE,
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Deterministic mode (the default): two launches on the caller's stream, no
// atomics:
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
//             registers (d = 64; at d = 128 two waves share a 32-key slice,
//             K and V sit in LDS, section 4), Q / dO tiles stream through
//             LDS, dK and dV accumulate in registers for the whole walk.
// S and dP are computed in both (7 products instead of 5) in exchange for no
// dQ atomics and no dS round trip through memory.  The atomic mode (section
// 4) computes all five in one key-side kernel.
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
// d = 64 only: at d = 128, K, V, dK and dV of a wave's 32 keys do not fit two
// waves per SIMD, and the key side is bwd_fused_kernel without its dQ part
// (eight waves, two per 32-key slice, each taking half of every step).
template <int D, int MASK, bool VARLEN = false>
__global__ void __launch_bounds__(256, 2) bwd_dkdv_kernel(BwdParams p) {
    static_assert(D == 64, "the d = 128 key side is bwd_fused_kernel<128, ..., false>");
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
    else map_head_tile(blockIdx.x, p.BH * p.kv_slots, p.kv_slots, bh, slot, MASK == kMaskCausal && !p.kv_paired);
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
        vreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rv, o, 0));
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
        mark_loaded(vreg[kk]);
    }

    // Operand reads are per-lane offsets formed once plus immediates (the
    // stage, Q or dO, the query block, the k-step's rows; a row's swizzle
    // depends on its index mod 16 only); the walk is unrolled by two so the
    // stage is a constant.
    uint32_t rowoff[NKK], trq[2 * NDB];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) rowoff[kk] = tile_offset<D>((uint32_t)l32, (uint32_t)(2 * kk + hg));
    {
        const uint32_t gi = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t row = 4 * hg + (gi >> 2) + 8 * h;
                const uint32_t col = db * 32 + (lane & 16) + 4 * (gi & 3);
                trq[2 * db + h] = tile_offset<D>(row, col >> 3) + (col & 4) * 2;
            }
    }

    auto walk_step = [&](const int qt, auto stage_c) {
        constexpr int st = decltype(stage_c)::value;
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
                    s[qb] = mfma_bf16(*(const bf16x8*)(qs + qb * 32 * D * 2 + rowoff[kk]), kreg[kk], s[qb]);
                    dp[qb] = mfma_bf16(*(const bf16x8*)(dos + qb * 32 * D * 2 + rowoff[kk]), vreg[kk], dp[qb]);
                }
            // (the compiler's own order of the operand reads: an explicit
            // four-ahead order measured 1.8% slower at d = 64)
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
                    dd = *(const f32x4*)(dds + ql);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sv = s[qb][4 * g + e];
                        const float pe = exp2_hw(fmaf(sv, p.scale_log2, -l2[e]));
                        pv[4 * g + e] = pe;
                        dsv[4 * g + e] = pe * (dp[qb][4 * g + e] - dd[e]);
                    }
                }
                pack_pairs(pv, pw[2 * qb], pw[2 * qb + 1]);
                pack_pairs(dsv, dsw[2 * qb], dsw[2 * qb + 1]);
            }
            // ---- dV^T += dO^T P ;  dK^T += Q^T dS ----
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const char* dr = dos + qc * 16 * D * 2;
                    const char* qr = qs + qc * 16 * D * 2;
                    const bf16x8 dot = concat8(lds_read_tr16(dr + trq[2 * db]), lds_read_tr16(dr + trq[2 * db + 1]));
                    const bf16x8 qto = concat8(lds_read_tr16(qr + trq[2 * db]), lds_read_tr16(qr + trq[2 * db + 1]));
                    dvacc[db] = mfma_bf16(dot, __builtin_bit_cast(bf16x8, pw[qc]), dvacc[db]);
                    dkacc[db] = mfma_bf16(qto, __builtin_bit_cast(bf16x8, dsw[qc]), dkacc[db]);
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
    };
    for (int qt = qt0; qt < n_qt; qt += 2) {
        walk_step(qt, std::integral_constant<int, 0>{});
        if (qt + 1 < n_qt) walk_step(qt + 1, std::integral_constant<int, 1>{});
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
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[db][4 * g] * p.scale, dkacc[db][4 * g + 1] * p.scale);
                wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale);
                *(u32x2*)(dKr + dcol) = wk;
                wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *(u32x2*)(dVr + dcol) = wv;
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
    else map_head_tile(blockIdx.x, p.BH * p.q_slots, p.q_slots, bh, slot, MASK == kMaskCausal && !p.q_paired);
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

    // Operand reads are per-lane offsets formed once plus immediates (the
    // buffer, K or V, the key block, the k-step's rows): the swizzle of a row
    // depends on its index mod 16 only, and every block starts on a multiple
    // of 16.  The tile loop is unrolled by two so the buffer is a constant.
    uint32_t rowoff[NKK], trk[2 * NDB];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) rowoff[kk] = tile_offset<D>((uint32_t)l32, (uint32_t)(2 * kk + hg));
    {
        const uint32_t gi = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t row = 4 * hg + (gi >> 2) + 8 * h;
                const uint32_t col = db * 32 + (lane & 16) + 4 * (gi & 3);
                trk[2 * db + h] = tile_offset<D>(row, col >> 3) + (col & 4) * 2;
            }
    }

    auto tile_step = [&](const int t, auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        const int k0 = t * BC;
        const char* kbuf = smem + buf * BUF_BYTES;
        const char* vbuf = kbuf + T_BYTES;
        const bool has_next = t + 1 < ntiles;
        if (has_next) load_tile(k0 + BC, buf ^ 1);

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
                    s[kb] = mfma_bf16(*(const bf16x8*)(kbuf + kb * 32 * D * 2 + rowoff[kk]), qreg[kk], s[kb]);
                    dp[kb] = mfma_bf16(*(const bf16x8*)(vbuf + kb * 32 * D * 2 + rowoff[kk]), doreg[kk], dp[kb]);
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
                for (int db = 0; db < NDB; ++db) {
                    const char* kr = kbuf + kc * 16 * D * 2;
                    const bf16x8 kt = concat8(lds_read_tr16(kr + trk[2 * db]), lds_read_tr16(kr + trk[2 * db + 1]));
                    dqacc[db] = mfma_bf16(kt, sb, dqacc[db]);
                }
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
    };
    for (int t = t_first; t < ntiles; t += 2) {
        tile_step(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>{});
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
// 4. Atomic mode: one key-side kernel for dV, dK and dQ.  The walk is that of
// bwd_dkdv_kernel (one workgroup per (batch*head, 128-key tile), 64-query
// steps); each step also forms the tile's share of dQ, dS K over its 128
// keys, and adds it to an fp32 dQ buffer with atomics, so every visible
// (query, key) pair costs the 5 products of the loop in §5: S, dP, dV, dK
// and dQ (the dQ "needs atomic adds or a separate reduction" remark there).
//
// QSPLIT waves share each 32-key slice: wave w owns keys 32*(w%4) .. +31 of
// the tile and queries (w/4)*WQ .. +WQ-1 of every step (WQ = 64 / QSPLIT).
// At d = 128 this keeps dK, dV, S, dP and the dQ block within 256 registers
// (two waves per SIMD, eight-wave workgroups); the slice's partial dK and dV
// are summed through LDS at the end of the walk.  At d = 64, QSPLIT = 1.
//
// Each step: S, dP, P, dS as in bwd_dkdv_kernel; dS (bf16) goes to an LDS
// tile [128 keys][64 queries]; dV^T += dO^T P and dK^T += Q^T dS; barrier;
// then wave w forms one 32x32 block of the step's dQ (query block w / NDB,
// head-dim block w % NDB) as dS K over the 128 keys -- A = dS read
// transposed from the dS tile, B = K read transposed from a K tile kept in
// LDS for the whole walk -- and adds its 16 values per lane to the fp32 dQ
// buffer with buffer atomics (rows past Nq fall outside the buffer range and
// are dropped by the hardware).
//
// The atomics are issued after the next stage's copies and are left in
// flight across the end-of-step barrier: vector memory operations of a wave
// complete in issue order, so waiting until no more than kAtomics are
// outstanding waits for the copies (and the previous steps' atomics) only.
//
// Cost: one float32 atomic add per (query row, head-dim column, 128-key
// tile), 64 x d per step, and MI355X retires about 3.2e11 such adds per
// second chip-wide (buffer atomics to distinct addresses, measured, 1.3 TB/s
// of payload).  That bounds this kernel well above the
// two deterministic kernels' time (0.87 vs 0.52 ms at B=4 H=16 N=4096 d=64
// causal), which is why the deterministic mode is the default.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void vmem_wait_n() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    // vmcnt bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) not waited on
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// DQ = false builds the same key-side walk without the dQ part (no dS tile,
// no mid-step barrier, no atomics): the deterministic mode's dK/dV kernel at
// d = 128, where the eight-wave split lets dK and dV share one walk at two
// waves per SIMD.
template <int D, int MASK, bool VARLEN = false, int QSPLIT = 1, bool DQ = true>
__global__ void __launch_bounds__(256 * QSPLIT, (D == 64 || QSPLIT == 2) ? 2 : 1) bwd_fused_kernel(BwdParams p) {
    constexpr int NW = 4 * QSPLIT;
    constexpr int BKV = 128, BQ = 64, WQ = BQ / QSPLIT;
    constexpr int NQB = WQ / 32;              // 32-query blocks per wave and step
    constexpr int NQC = WQ / 16;              // 16-query k-steps
    constexpr int NKK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int DQB = 2 * NDB / NW;         // 32x32 dQ blocks per wave (same query block)
    static_assert(DQB >= 1 && DQB * NW == 2 * NDB && NDB % DQB == 0, "dQ blocks split evenly");
    constexpr int T_BYTES = BQ * D * 2;
    constexpr int V_OFF = 2 * T_BYTES;
    constexpr int STAGE = V_OFF + 2 * BQ * 4;
    // d = 128: the B operands of S and dP (K and V of the wave's keys) are
    // read from K and V tiles kept in LDS for the walk instead of held in 64
    // registers (the kernel would spill otherwise)
    constexpr bool kKRegs = D == 64 || QSPLIT == 1;
    constexpr int K_OFF = 2 * STAGE;              // K tile [BKV][D] (dQ's B operand, and S's at d = 128)
    constexpr int VT_OFF = K_OFF + BKV * D * 2;   // V tile [BKV][D] (d = 128 only)
    constexpr int DS_OFF = VT_OFF + (kKRegs ? 0 : BKV * D * 2);   // dS^T tile [BKV][BQ]
    constexpr int SMEM = DQ ? DS_OFF + BKV * BQ * 2 : DS_OFF;
    static_assert(K_OFF % 1024 == 0 && VT_OFF % 1024 == 0 && DS_OFF % 1024 == 0, "tiles start on 1 KiB");
    static_assert(SMEM <= 160 * 1024, "LDS of one CU");
    static_assert(QSPLIT == 1 || 4 * NDB * 16 * 64 * 4 <= SMEM, "room for the partial dK / dV");
    constexpr int kAtomics = DQ ? 16 * DQB : 0;   // its fp32 dQ values per lane and step
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hg = lane >> 5;
    const int wk = wave & 3, wq = wave >> 2;  // key slice, query part
    const int qw0 = wq * WQ;                  // this wave's first query of a step
    const int dq_qb = wave * DQB / NDB, dq_db = wave * DQB % NDB;   // its first dQ block
    int bh, slot;
    if (VARLEN) varlen_slot(p.vl, p.kv_slots, blockIdx.x, bh, slot);
    else map_head_tile(blockIdx.x, p.BH * p.kv_slots, p.kv_slots, bh, slot, MASK == kMaskCausal && !p.kv_paired);
    SeqGeometry sg;
    if constexpr (VARLEN) sg = seq_geometry(p.vl, bh);
    else sg = SeqGeometry{p.Nq, p.Nk, (size_t)bh * p.Nq, (size_t)bh * p.Nk};
    const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
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
    float* dQa = DQ ? p.dqacc + sg.q_row0 * D : nullptr;

    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, (uint32_t)Nk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh, (uint32_t)Nk * D * 2);
    const TileCopy<D, BQ, NW> copier(wave, lane);
    const TileCopy<D, BKV, NW> kcopier(wave, lane);
    const i32x4 rq_w = make_rsrc_words(Qh, (uint32_t)Nq * D * 2);
    const i32x4 rdo_w = make_rsrc_words(dOh, (uint32_t)Nq * D * 2);
    const i32x4 rk_w = make_rsrc_words(Kh, (uint32_t)Nk * D * 2);
    const uint32_t smem_lds = lds_address(smem);
    const char* ktile = smem + K_OFF;
    const i32x4 rv_w = make_rsrc_words(Vh, (uint32_t)Nk * D * 2);
    char* dstile = smem + DS_OFF;

    // this lane's byte offsets of its dQ block items in a step's rows:
    // item 4g+e is query 32*dq_qb + 8g + 4hg + e, column 32*dq_db + l32
    const uint32_t dq_off0 = (uint32_t)(((dq_qb * 32 + 4 * hg) * D + dq_db * 32 + l32) * 4);

    // d = 128: every operand read is one of these per-lane offsets plus an
    // immediate (the stage, the tile, the k-step's rows).  The swizzle of a
    // row depends on its index mod 16 only, and every tile row block starts
    // on a multiple of 16, so a row read of rows r0 + l32 is r0 * 2D bytes
    // plus the offset of row l32, and likewise for the transposed reads.
    uint32_t qrow[NKK], kvrow[NKK], trq[2 * NDB];
    if constexpr (!kKRegs) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const uint32_t r = tile_offset<D>((uint32_t)l32, (uint32_t)(2 * kk + hg));
            qrow[kk] = (uint32_t)(qw0 * D * 2) + r;                 // rows qw0 + l32 of a stage tile
            kvrow[kk] = (uint32_t)(K_OFF + wk * 32 * D * 2) + r;    // rows wk*32 + l32 of the K tile
        }
        const uint32_t gi = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t row = 4 * hg + (gi >> 2) + 8 * h;
                const uint32_t col = db * 32 + (lane & 16) + 4 * (gi & 3);
                trq[2 * db + h] = (uint32_t)(qw0 * D * 2) + tile_offset<D>(row, col >> 3) + (col & 4) * 2;
            }
    }

    for (int it = 0; it < n_items; ++it) {
    const int kt = it == 0 ? slot : n_kt - 1 - slot;
    const int k0 = kt * BKV;
    const int kw = k0 + wk * 32;              // this wave's first key
    const int kj = kw + l32;                  // this lane's key

    // K^T and V^T as B operands (lane = key) in registers, or read from the
    // K and V tiles at d = 128
    bf16x8 kreg[kKRegs ? NKK : 1], vreg[kKRegs ? NKK : 1];
#pragma unroll
    for (int kk = 0; kk < (kKRegs ? NKK : 0); ++kk) {
        const uint32_t o = (uint32_t)kj * D * 2 + (16 * kk + 8 * hg) * 2;
        kreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rk, o, 0));
        vreg[kk] = __builtin_bit_cast(bf16x8, buf_load128(rv, o, 0));
    }

    const int qstart = kRight ? max(0, k0 - offr) : 0;
    const int qt0 = qstart / BQ;
    const int qend = kLeft ? max(0, min(Nq, k0 + BKV - offl)) : Nq;
    const int n_qt = (qend + BQ - 1) / BQ;
    const int wq_first = kRight ? kw - offr : 0;
    const int wq_last = kLeft ? kw + 31 - offl : Nq;

    auto load_step = [&](int qt, int stage) {
        const uint32_t base = smem_lds + stage * STAGE;
        copier.issue(rq_w, qt * BQ, base);
        copier.issue(rdo_w, qt * BQ, base + T_BYTES);
    };
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

    if (DQ || !kKRegs) kcopier.issue(rk_w, k0, smem_lds + K_OFF);
    if (!kKRegs) kcopier.issue(rv_w, k0, smem_lds + VT_OFF);
    if (qt0 < n_qt) {
        load_step(qt0, 0);
        if (wave == 0) {
            fetch_vec(qt0);
            store_vec(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    tile_barrier();
#pragma unroll
    for (int kk = 0; kk < (kKRegs ? NKK : 0); ++kk) {
        mark_loaded(kreg[kk]);
        mark_loaded(vreg[kk]);
    }

    // The walk, unrolled by two so that the stage buffer of a step is a
    // compile-time constant (its operand addresses then take it as an
    // immediate offset).
    auto walk_step = [&](const int qt, auto stage_c) {
        constexpr int st = decltype(stage_c)::value;
        const char* qs = smem + st * STAGE;
        const char* dos = qs + T_BYTES;
        const float* l2s = (const float*)(qs + V_OFF);
        const float* dds = l2s + BQ;
        const int q0 = qt * BQ;
        const int qa = q0 + qw0;              // this wave's first query
        const bool has_next = qt + 1 < n_qt;
        if (has_next) {
            load_step(qt + 1, st ^ 1);
            if (wave == 0) fetch_vec(qt + 1);
        }

        const bool active = kw < Nk && qa + WQ - 1 >= wq_first && (!kLeft || qa <= wq_last);
        const int ln = lane;
        const char* sb = smem + st * STAGE;   // this step's stage (an immediate)
        if (active) {
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
                    if constexpr (kKRegs) {
                        s[qb] = mfma_bf16(tile_read_row<D>(qs, qw0 + qb * 32, kk, ln), kreg[kk], s[qb]);
                        dp[qb] = mfma_bf16(tile_read_row<D>(dos, qw0 + qb * 32, kk, ln), vreg[kk], dp[qb]);
                    } else {   // NQB = 1
                        const bf16x8 kb = *(const bf16x8*)(smem + kvrow[kk]);
                        const bf16x8 vb = *(const bf16x8*)(smem + (VT_OFF - K_OFF) + kvrow[kk]);
                        s[qb] = mfma_bf16(*(const bf16x8*)(sb + qrow[kk]), kb, s[qb]);
                        dp[qb] = mfma_bf16(*(const bf16x8*)(sb + T_BYTES + qrow[kk]), vb, dp[qb]);
                    }
                }
            if constexpr (D == 128 && NQB == 1 && !kKRegs) {
                // the four operand reads of a k-step (Q, dO, K, V) two k-steps
                // ahead of its two MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    if (kk + 2 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                }
            }
            // ---- mask: steps that straddle a bound, the query tail or the
            // key tail (keys past Nk: P = 0, so dS stays finite) ----
            const bool need_mask = (qa + WQ > Nq) || (kw + 31 >= Nk) || (kRight && qa + offr < kw + 31) ||
                                   (kLeft && qa + WQ - 1 + offl > kw);
            if (need_mask) {
                const int qb0 = qa + 4 * hg;
                const int lo = kRight ? kj - offr - qb0 : -(1 << 30);
                int hi = kj < Nk ? Nq - 1 - qb0 : -(1 << 30);
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
                    const int ql = qw0 + qb * 32 + g * 8 + 4 * hg;
                    const f32x4 l2 = *(const f32x4*)(l2s + ql);
                    const f32x4 dd = *(const f32x4*)(dds + ql);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pe = exp2_hw(fmaf(s[qb][4 * g + e], p.scale_log2, -l2[e]));
                        pv[4 * g + e] = pe;
                        dsv[4 * g + e] = pe * (dp[qb][4 * g + e] - dd[e]);
                    }
                }
                pack_pairs(pv, pw[2 * qb], pw[2 * qb + 1]);
                pack_pairs(dsv, dsw[2 * qb], dsw[2 * qb + 1]);
            }
            // ---- dS^T into the dS tile: k-step qc holds queries
            // qc*16 + 4hg + {0..3} (words 0, 1) and qc*16 + 8 + 4hg + {0..3} ----
            const uint32_t krow = (uint32_t)(wk * 32 + l32);
#pragma unroll
            for (int qc = 0; qc < (DQ ? NQC : 0); ++qc) {
                const uint32_t ch = (uint32_t)(qw0 / 8 + 2 * qc);
                u32x2 a, b;
                a[0] = dsw[qc][0];
                a[1] = dsw[qc][1];
                b[0] = dsw[qc][2];
                b[1] = dsw[qc][3];
                *(u32x2*)(dstile + tile_offset<BQ>(krow, ch) + 8 * hg) = a;
                *(u32x2*)(dstile + tile_offset<BQ>(krow, ch + 1) + 8 * hg) = b;
            }
            // ---- dV^T += dO^T P ;  dK^T += Q^T dS ----
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    bf16x8 dot, qt_op;
                    if constexpr (kKRegs) {
                        dot = tile_read_tr<D>(dos, qw0 + qc * 16, db * 32, ln);
                        qt_op = tile_read_tr<D>(qs, qw0 + qc * 16, db * 32, ln);
                    } else {
                        const char* d0 = sb + T_BYTES + qc * 16 * D * 2;
                        const char* q0p = sb + qc * 16 * D * 2;
                        dot = concat8(lds_read_tr16(d0 + trq[2 * db]), lds_read_tr16(d0 + trq[2 * db + 1]));
                        qt_op = concat8(lds_read_tr16(q0p + trq[2 * db]), lds_read_tr16(q0p + trq[2 * db + 1]));
                    }
                    dvacc[db] = mfma_bf16(dot, __builtin_bit_cast(bf16x8, pw[qc]), dvacc[db]);
                    dkacc[db] = mfma_bf16(qt_op, __builtin_bit_cast(bf16x8, dsw[qc]), dkacc[db]);
                }
            if constexpr (D == 128) {   // two transposed reads per MFMA, four ahead
                constexpr int nm = 2 * NQC * NDB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
                for (int i = 0; i < nm; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    if (i < nm - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
            }
        } else if constexpr (DQ) {
            // no visible pair for this wave: its part of the dS tile is zero
            const uint32_t krow = (uint32_t)(wk * 32 + l32);
            u32x2 z;
            z[0] = z[1] = 0u;
#pragma unroll
            for (int qc = 0; qc < NQC; ++qc) {
                const uint32_t ch = (uint32_t)(qw0 / 8 + 2 * qc);
                *(u32x2*)(dstile + tile_offset<BQ>(krow, ch) + 8 * hg) = z;
                *(u32x2*)(dstile + tile_offset<BQ>(krow, ch + 1) + 8 * hg) = z;
            }
        }
        if constexpr (DQ) tile_barrier();   // the whole dS tile is written

        // ---- dQ block += dS K over the tile's 128 keys, added to the fp32
        // buffer (rows q0 .. q0+63; rows past Nq are outside the range) ----
        if constexpr (DQ) {
            f32x16 dq[DQB];
#pragma unroll
            for (int b = 0; b < DQB; ++b) dq[b] = zero16();
#pragma unroll
            for (int kc = 0; kc < BKV / 16; ++kc) {
                const bf16x8 a = tile_read_tr<BQ>(dstile, kc * 16, dq_qb * 32, ln);
#pragma unroll
                for (int b = 0; b < DQB; ++b)
                    dq[b] = mfma_bf16(a, tile_read_tr<D>(ktile, kc * 16, (dq_db + b) * 32, ln), dq[b]);
            }
            const __amdgpu_buffer_rsrc_t rdq =
                make_rsrc(dQa + (size_t)q0 * D, (uint32_t)(min(BQ, Nq - q0) * D * 4));
            // row group g of the block through the scalar offset, the rest
            // in the instruction's immediate: one offset register in all
#pragma unroll
            for (int b = 0; b < DQB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t o = dq_off0 + (uint32_t)(((i & 3) * D + 32 * b) * 4);
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[b][i], rdq, o, (i >> 2) * 8 * D * 4, 0);
                }
        }

        if (has_next) {
            if (wave == 0) store_vec(st ^ 1);
            vmem_wait_n<kAtomics>();   // the next stage's copies landed; atomics may still fly
        }
        mark_loaded(nl2);
        mark_loaded(ndd);
        tile_barrier();
    };
    for (int qt = qt0; qt < n_qt; qt += 2) {
        walk_step(qt, std::integral_constant<int, 0>{});
        if (qt + 1 < n_qt) walk_step(qt + 1, std::integral_constant<int, 1>{});
    }

    // ---- QSPLIT > 1: sum the slice's partial dK^T, dV^T through LDS (the
    // stages, K and dS tiles are free after the walk) ----
    if constexpr (QSPLIT > 1) {
        float* red = (float*)smem + wk * (NDB * 16 * 64);
        auto reduce = [&](f32x16 (&acc)[NDB]) {
            if (wq != 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) red[(db * 16 + i) * 64 + lane] = acc[db][i];
            }
            tile_barrier();
            if (wq == 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[db][i] += red[(db * 16 + i) * 64 + lane];
            }
            tile_barrier();
        };
        reduce(dkacc);
        reduce(dvacc);
    }

    // ---- dK = scale * dK^T, dV = dV^T (lane = key, items = d) ----
    if (wq == 0 && kj < Nk) {
        bf16* dKr = (bf16*)p.dk + sg.k_row0 * D + (size_t)kj * D;
        bf16* dVr = (bf16*)p.dv + sg.k_row0 * D + (size_t)kj * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = db * 32 + g * 8 + 4 * hg;
                u32x2 wk2, wv;
                wk2[0] = pack_bf16x2(dkacc[db][4 * g] * p.scale, dkacc[db][4 * g + 1] * p.scale);
                wk2[1] = pack_bf16x2(dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale);
                *(u32x2*)(dKr + dcol) = wk2;
                wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *(u32x2*)(dVr + dcol) = wv;
            }
    }
    }   // items
}

// Atomic mode, before the fused kernel: for every query row, D = rowsum(dO * O)
// and LSE * log2(e) (+inf for a row with no visible key) into the workspace,
// and the row of the fp32 dQ buffer set to zero.  D / 8 lanes per row, 16
// bytes each.
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p, long rows) {
    constexpr int TPR = D / 8, RPB = 256 / TPR;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    if (row >= rows) return;   // whole rows leave together
    const size_t e0 = (size_t)row * D + 8 * c;
    const u32x4 a = ldg128((const bf16*)p.dO + e0), b = ldg128((const bf16*)p.o + e0);
    float dd = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) dd += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) dd += __shfl_xor(dd, m, TPR);
    if (c == 0) {
        const float lse = p.lse[row];
        p.lse2[row] = lse == -INFINITY ? INFINITY : lse * kLog2e;
        p.dvec[row] = dd;
    }
    f32x4 z;
    z[0] = z[1] = z[2] = z[3] = 0.f;
    *(f32x4*)(p.dqacc + e0) = z;
    *(f32x4*)(p.dqacc + e0 + 4) = z;
}

// Atomic mode, after the fused kernel: dQ = scale * (fp32 buffer), rounded to
// bf16; 8 elements per lane.
__global__ void __launch_bounds__(256) bwd_dq_convert_kernel(const float* acc, bf16* dq, float scale,
                                                             size_t n8) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = *(const f32x4*)(acc + 8 * i), b = *(const f32x4*)(acc + 8 * i + 4);
    u32x4 w;
    w[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
    w[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
    w[2] = pack_bf16x2(b[0] * scale, b[1] * scale);
    w[3] = pack_bf16x2(b[2] * scale, b[3] * scale);
    *(u32x4*)(dq + 8 * i) = w;
}

// ---------------------------------------------------------------------------
// Deterministic mode.  keyside = false: the dQ kernel; true: the key-side
// kernel (bwd_dkdv_kernel at d = 64, bwd_fused_kernel without its dQ part
// at d = 128).
template <int D, int MASK, bool VARLEN>
static const void* bwd_kernel_m(bool keyside) {
    if (!keyside) return (const void*)bwd_dq_kernel<D, MASK, VARLEN>;
    if constexpr (D == 64) return (const void*)bwd_dkdv_kernel<D, MASK, VARLEN>;
    else return (const void*)bwd_fused_kernel<D, MASK, VARLEN, 2, false>;
}

template <int D, bool VARLEN>
static const void* bwd_kernel(bool keyside, int mask) {
    if (mask == kMaskCausal) return bwd_kernel_m<D, kMaskCausal, VARLEN>(keyside);
    if (mask == kMaskWindow) return bwd_kernel_m<D, kMaskWindow, VARLEN>(keyside);
    return bwd_kernel_m<D, kMaskNone, VARLEN>(keyside);
}

template <int D>
static const void* bwd_kernel(bool keyside, int mask, bool varlen) {
    return varlen ? bwd_kernel<D, true>(keyside, mask) : bwd_kernel<D, false>(keyside, mask);
}

template <int D>
static hipError_t launch_bwd_d(int mask, bool varlen, const BwdParams& p, hipStream_t s) {
    BwdParams pp = p;
    void* args[] = {&pp};
    // dQ first: it also writes every query row's D and LSE * log2(e) to the
    // workspace, which the key-side kernel reads (stream order)
    const long grid_q = (long)p.BH * p.q_slots;
    if (grid_q > 0) {   // with Nk == 0 every row is empty and dQ = 0 is written
        hipError_t e = hipLaunchKernel(bwd_kernel<D>(false, mask, varlen), dim3((unsigned)grid_q), dim3(256),
                                       args, 0, s);
        if (e != hipSuccess) return e;
    }
    // with Nq == 0 the walk is empty and dK = dV = 0 are written; d = 128:
    // eight waves per workgroup, two per 32-key slice
    const long grid_kv = (long)p.BH * p.kv_slots;
    if (grid_kv > 0) {
        hipError_t e = hipLaunchKernel(bwd_kernel<D>(true, mask, varlen), dim3((unsigned)grid_kv),
                                       dim3(D == 64 ? 256 : 512), args, 0, s);
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

template <int D, bool VARLEN>
static const void* bwd_fused(int mask) {
    constexpr int QS = D == 64 ? 1 : 2;
    if (mask == kMaskCausal) return (const void*)bwd_fused_kernel<D, kMaskCausal, VARLEN, QS>;
    if (mask == kMaskWindow) return (const void*)bwd_fused_kernel<D, kMaskWindow, VARLEN, QS>;
    return (const void*)bwd_fused_kernel<D, kMaskNone, VARLEN, QS>;
}

// Atomic mode: pre-pass (D, LSE2, dQ buffer = 0), the fused key-side
// kernel, then dQ = scale * buffer in bf16.
template <int D>
static hipError_t launch_bwd_atomic_d(int mask, bool varlen, const BwdParams& p, long rows, hipStream_t s) {
    BwdParams pp = p;
    if (rows > 0) {
        constexpr int RPB = 256 / (D / 8);
        long rr = rows;
        void* args[] = {&pp, &rr};
        hipError_t e = hipLaunchKernel((const void*)bwd_prep_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)),
                                       dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    const long grid_kv = (long)p.BH * p.kv_slots;
    if (grid_kv > 0) {
        void* args[] = {&pp};
        const void* fn = varlen ? bwd_fused<D, true>(mask) : bwd_fused<D, false>(mask);
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid_kv), dim3(D == 64 ? 256 : 512), args, 0, s);
        if (e != hipSuccess) return e;
    }
    if (rows > 0) {
        const float* acc = p.dqacc;
        bf16* dq = (bf16*)p.dq;
        float scale = p.scale;
        size_t n8 = (size_t)rows * D / 8;
        void* args[] = {&acc, &dq, &scale, &n8};
        hipError_t e = hipLaunchKernel((const void*)bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)),
                                       dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_bwd(int d, int mask, bool varlen, BwdParams p, hipStream_t stream) {
    return d == 64 ? launch_bwd_d<64>(mask, varlen, p, stream) : launch_bwd_d<128>(mask, varlen, p, stream);
}

hipError_t launch_bwd_atomic(int d, int mask, bool varlen, BwdParams p, long rows, hipStream_t stream) {
    return d == 64 ? launch_bwd_atomic_d<64>(mask, varlen, p, rows, stream)
                   : launch_bwd_atomic_d<128>(mask, varlen, p, rows, stream);
}

}  // namespace fa
