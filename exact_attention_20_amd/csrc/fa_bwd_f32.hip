// Attention backward for fp32 inputs and outputs on gfx950: true fp32
// products on the 32x32x2 fp32 MFMA and an fp32 recomputation of the
// softmax ("01 · IO-awareness、online softmax 与 tiling" §5: S and P are
// recomputed from Q, K and the saved LSE; dV = P^T dO, dP = dO V^T,
// D = rowsum(dO * O), dS = P * (dP - D), dQ = scale * dS K,
// dK = scale * dS^T Q).
//
// Two kernels and no atomics, so the result is bitwise repeatable:
//   bwd_f32_dq_kernel    one workgroup per (batch*head, 64-query tile), two
//                        waves of 32 queries.  It writes every query row's D
//                        and LSE * log2(e) to the workspace, then walks the
//                        key tiles accumulating dQ^T = K^T dS^T.
//   bwd_f32_dkdv_kernel  one workgroup per (batch*head, 64-key tile), two
//                        waves of 32 keys, launched after the first on the
//                        same stream; it walks the query tiles accumulating
//                        dV^T = dO^T P and dK^T = Q^T dS.
//
// 32x32x2 fp32 MFMA lanes: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32] and receives D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
// in its register r.  The dQ kernel forms S^T = K Q^T (each lane owns one
// query, the column), the dK/dV kernel S = Q K^T (each lane owns one key), so
// the row-wise LSE and D, and the mask, are per-lane values or per-register
// LDS broadcasts, and P or dS go from the accumulator straight into the
// B operand of the next product.  The operand rows staged in LDS are padded
// to d + 1 floats: the 32 rows a half-wave reads then fall in distinct banks.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int MASK>
__global__ void __launch_bounds__(128) bwd_f32_dq_kernel(BwdParams p) {
    constexpr int BQ = 64, BC = D == 128 ? 32 : 64;   // K + V tiles within 33 KiB
    constexpr int NKB = BC / 32, NDB = D / 32;
    constexpr int KS = D + 1;
    __shared__ float ks[BC * KS];
    __shared__ float vs[BC * KS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hg = lane >> 5;
    int bh, qt;
    map_head_tile(blockIdx.x, p.BH * p.q_slots, p.q_slots, bh, qt, MASK == kMaskCausal);
    qt = p.q_slots - 1 - qt;   // the heaviest causal tiles first
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    const int q0 = qt * BQ;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    const bool live = qi < Nq;
    const size_t row = (size_t)bh * Nq + qi;
    const float* Kh = (const float*)p.k + (size_t)bh * Nk * D;
    const float* Vh = (const float*)p.v + (size_t)bh * Nk * D;

    // this lane's query: columns 2kk + hg of Q and dO (the B operands), and
    // D = rowsum(dO * O) over the same columns, then the partner lane's half
    float qreg[D / 2], doreg[D / 2];
    float dd = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
        const size_t e = row * D + 2 * kk + hg;
        qreg[kk] = live ? ((const float*)p.q)[e] : 0.f;
        doreg[kk] = live ? ((const float*)p.dO)[e] : 0.f;
        dd = fmaf(doreg[kk], live ? ((const float*)p.o)[e] : 0.f, dd);
    }
    dd += __shfl_xor(dd, 32);
    // LSE * log2(e); +inf for a row with no visible key and for rows past
    // Nq, so their P is exactly 0
    const float lse_i = live ? p.lse[row] : -INFINITY;
    const float l2 = lse_i == -INFINITY ? INFINITY : lse_i * kLog2e;
    if (live && hg == 0) {
        p.lse2[row] = l2;
        p.dvec[row] = dd;
    }

    // key tiles [t_first, ntiles) this query tile can see
    const int kend = kRight ? min(Nk, q0 + BQ + offr) : Nk;
    const int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;
    const int t_first = kLeft ? max(0, q0 + offl) / BC : 0;
    const int kend_w = kRight ? min(Nk, qw + 32 + offr) : Nk;
    const int kbeg_w = kLeft ? qw + offl : 0;

    f32x16 dqacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqacc[db] = zero16();

    for (int t = t_first; t < ntiles; ++t) {
        const int k0 = t * BC;
        __syncthreads();   // the previous tile's reads are done
        for (int c = tid; c < BC * D / 4; c += 128) {
            const int r = c / (D / 4), cc = c % (D / 4);
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = kv;
            if (k0 + r < Nk) {
                kv = *(const f32x4*)(Kh + (size_t)(k0 + r) * D + cc * 4);
                vv = *(const f32x4*)(Vh + (size_t)(k0 + r) * D + cc * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[r * KS + cc * 4 + e] = kv[e];
                vs[r * KS + cc * 4 + e] = vv[e];
            }
        }
        __syncthreads();
        if (k0 >= kend_w || (kLeft && k0 + BC <= kbeg_w)) continue;   // no key of the tile visible to this wave

        // S^T = K Q^T and dP^T = V dO^T
        f32x16 s[NKB], dp[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = zero16();
            dp[kb] = zero16();
        }
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int a = (kb * 32 + l32) * KS + 2 * kk + hg;
                s[kb] = mfma_f32(ks[a], qreg[kk], s[kb]);
                dp[kb] = mfma_f32(vs[a], doreg[kk], dp[kb]);
            }

        // P = 2^(S * scale * log2(e) - LSE * log2(e)), 0 where masked;
        // dS^T = P * (dP - D) replaces S^T
        const bool need_mask = (k0 + BC > Nk) || (kRight && k0 + BC - 1 > qw + offr) ||
                               (kLeft && k0 < qw + 31 + offl);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float pv = exp2_hw(fmaf(s[kb][i], p.scale_log2, -l2));
                if (need_mask) {
                    const int key = k0 + kb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
                    const bool vis = key < Nk && (!kRight || key <= qi + offr) && (!kLeft || key >= qi + offl);
                    if (!vis) pv = 0.f;
                }
                s[kb][i] = pv * (dp[kb][i] - dd);
            }

        // dQ^T += K^T dS^T: two keys (one per 32-lane half) per MFMA
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dqacc[db] = mfma_f32(ks[key * KS + db * 32 + l32], s[kb][i], dqacc[db]);
            }
    }

    // dQ = scale * dQ^T transposed back: this lane's query row, 4 columns a store
    if (live) {
        float* dQr = (float*)p.dq + row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = dqacc[db][4 * g + e] * p.scale;
                *(f32x4*)(dQr + db * 32 + g * 8 + 4 * hg) = w;
            }
    }
}

template <int D, int MASK>
__global__ void __launch_bounds__(128) bwd_f32_dkdv_kernel(BwdParams p) {
    constexpr int BK = 64, BQ = D == 128 ? 32 : 64;   // Q + dO tiles within 33 KiB
    constexpr int NQB = BQ / 32, NDB = D / 32;
    constexpr int QS = D + 1;
    __shared__ float qs[BQ * QS];
    __shared__ float dos[BQ * QS];
    __shared__ float l2s[BQ];
    __shared__ float dds[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hg = lane >> 5;
    int bh, kt;
    map_head_tile(blockIdx.x, p.BH * p.kv_slots, p.kv_slots, bh, kt, MASK == kMaskCausal);   // first key tiles see the most queries
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    const int k0 = kt * BK;
    const int kw = k0 + wave * 32;
    const int kj = kw + l32;
    const bool live = kj < Nk;
    const size_t krow = (size_t)bh * Nk + kj;
    const float* Qh = (const float*)p.q + (size_t)bh * Nq * D;
    const float* dOh = (const float*)p.dO + (size_t)bh * Nq * D;
    const float* L2h = p.lse2 + (size_t)bh * Nq;
    const float* Dh = p.dvec + (size_t)bh * Nq;

    // this lane's key: columns 2kk + hg of K and V (the B operands)
    float kreg[D / 2], vreg[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
        const size_t e = krow * D + 2 * kk + hg;
        kreg[kk] = live ? ((const float*)p.k)[e] : 0.f;
        vreg[kk] = live ? ((const float*)p.v)[e] : 0.f;
    }

    // query q sees key j iff j <= q + offr and (windows) j >= q + offl: the
    // query tiles [t_first, t_end) reach this workgroup's keys
    const int qbeg = kRight ? max(0, k0 - offr) : 0;
    const int qend = kLeft ? min(Nq, k0 + BK - offl) : Nq;   // exclusive
    const int t_first = qbeg / BQ;
    const int t_end = qend > 0 ? (qend + BQ - 1) / BQ : 0;

    f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dkacc[db] = zero16();
        dvacc[db] = zero16();
    }

    for (int t = t_first; t < t_end; ++t) {
        const int q0 = t * BQ;
        __syncthreads();   // the previous tile's reads are done
        for (int c = tid; c < BQ * D / 4; c += 128) {
            const int r = c / (D / 4), cc = c % (D / 4);
            f32x4 qv = {0.f, 0.f, 0.f, 0.f}, ov = qv;
            if (q0 + r < Nq) {
                qv = *(const f32x4*)(Qh + (size_t)(q0 + r) * D + cc * 4);
                ov = *(const f32x4*)(dOh + (size_t)(q0 + r) * D + cc * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qs[r * QS + cc * 4 + e] = qv[e];
                dos[r * QS + cc * 4 + e] = ov[e];
            }
        }
        // rows past Nq: P = 0 (LSE2 = +inf) and D = 0
        for (int r = tid; r < BQ; r += 128) {
            const bool in = q0 + r < Nq;
            l2s[r] = in ? L2h[q0 + r] : INFINITY;
            dds[r] = in ? Dh[q0 + r] : 0.f;
        }
        __syncthreads();
        // no query of the tile sees a key of this wave
        if ((kRight && q0 + BQ - 1 + offr < kw) || (kLeft && q0 + offl > kw + 31)) continue;

        // S = Q K^T and dP = dO V^T
        f32x16 s[NQB], dp[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            s[qb] = zero16();
            dp[qb] = zero16();
        }
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int a = (qb * 32 + l32) * QS + 2 * kk + hg;
                s[qb] = mfma_f32(qs[a], kreg[kk], s[qb]);
                dp[qb] = mfma_f32(dos[a], vreg[kk], dp[qb]);
            }

        // P replaces S, dS = P * (dP - D) replaces dP; 0 where masked
        const bool need_mask = (kRight && kw + 31 > q0 + offr) || (kLeft && kw < q0 + BQ - 1 + offl);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = qb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
                float pv = exp2_hw(fmaf(s[qb][i], p.scale_log2, -l2s[r]));
                if (need_mask) {
                    const int q = q0 + r;
                    const bool vis = (!kRight || kj <= q + offr) && (!kLeft || kj >= q + offl);
                    if (!vis) pv = 0.f;
                }
                s[qb][i] = pv;
                dp[qb][i] = pv * (dp[qb][i] - dds[r]);
            }

        // dV^T += dO^T P and dK^T += Q^T dS: two queries (one per 32-lane
        // half) per MFMA
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = qb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dvacc[db] = mfma_f32(dos[r * QS + db * 32 + l32], s[qb][i], dvacc[db]);
                    dkacc[db] = mfma_f32(qs[r * QS + db * 32 + l32], dp[qb][i], dkacc[db]);
                }
            }
    }

    // this lane's key row of dK = scale * dK^T and dV = dV^T, 4 columns a store
    if (live) {
        float* dKr = (float*)p.dk + krow * D;
        float* dVr = (float*)p.dv + krow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 wk, wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = dkacc[db][4 * g + e] * p.scale;
                    wv[e] = dvacc[db][4 * g + e];
                }
                *(f32x4*)(dKr + db * 32 + g * 8 + 4 * hg) = wk;
                *(f32x4*)(dVr + db * 32 + g * 8 + 4 * hg) = wv;
            }
    }
}

template <int D, int MASK>
static hipError_t launch_bwd_f32_m(const BwdParams& p, hipStream_t s) {
    BwdParams pp = p;
    void* args[] = {&pp};
    // the dQ kernel first: it writes D and LSE2, which the dK/dV kernel reads
    const long grid_q = (long)p.BH * p.q_slots;
    if (grid_q > 0) {
        hipError_t e = hipLaunchKernel((const void*)bwd_f32_dq_kernel<D, MASK>, dim3((unsigned)grid_q), dim3(128),
                                       args, 0, s);
        if (e != hipSuccess) return e;
    }
    const long grid_kv = (long)p.BH * p.kv_slots;
    if (grid_kv > 0) {
        hipError_t e = hipLaunchKernel((const void*)bwd_f32_dkdv_kernel<D, MASK>, dim3((unsigned)grid_kv),
                                       dim3(128), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_f32_d(int mask, const BwdParams& p, hipStream_t s) {
    if (mask == kMaskCausal) return launch_bwd_f32_m<D, kMaskCausal>(p, s);
    if (mask == kMaskWindow) return launch_bwd_f32_m<D, kMaskWindow>(p, s);
    return launch_bwd_f32_m<D, kMaskNone>(p, s);
}

hipError_t launch_bwd_f32(int d, int mask, BwdParams p, hipStream_t stream) {
    return d == 64 ? launch_bwd_f32_d<64>(mask, p, stream) : launch_bwd_f32_d<128>(mask, p, stream);
}

}  // namespace fa
