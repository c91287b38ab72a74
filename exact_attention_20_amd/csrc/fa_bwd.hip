// Attention backward by recomputation for gfx950 ("01 · IO-awareness、online
// softmax 与 tiling" §5; "让注意力计算留在片上" §04):
//
//   P = exp(scale*S - LSE) rebuilt tile by tile from the saved LSE,
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three launches on the caller's stream:
//   1. prep   : D = rowsum(dO * O) in fp32, and zero the fp32 dQ accumulator.
//   2. main   : one workgroup per (batch*head, 128-key tile), the loop order of
//               §5 (fix a key tile, walk the query tiles that can see it).
//               dK and dV stay in registers for the whole walk; each query
//               tile's dQ contribution is added into the fp32 accumulator
//               with float atomics.
//   3. convert: dq = dQ accumulator * scale, rounded to the output dtype.
//
// Register formulation (32x32x16 bf16 MFMA, fp32 accumulate), per wave of 32
// keys: S = Q K^T and dP = dO V^T come out with lane = key and 16 queries
// per lane, which is exactly the B-operand shape of the two products that
// contract over queries (dV^T = dO^T P, dK^T = Q^T dS); the A operands are
// q-permuted transposed copies of the Q and dO tiles in LDS.  dQ contracts
// over keys, so dS goes through LDS once per query tile.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// 1. D_i = sum_d dO_i * O_i; zero the dQ accumulator row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                       float* __restrict__ dvec, float* __restrict__ dq_acc,
                                                       long rows) {
    constexpr int TPR = D / 8;      // threads per row, 8 bf16 each
    constexpr int RPB = 256 / TPR;  // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = ldg128(O + row * D + c * 8);
        const u32x4 b = ldg128(dO + row * D + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
        f32x4 z;
        z[0] = z[1] = z[2] = z[3] = 0.f;
        *(f32x4*)(dq_acc + row * D + c * 8) = z;
        *(f32x4*)(dq_acc + row * D + c * 8 + 4) = z;
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (row < rows && c == 0) dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. main backward kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) bwd_main_kernel(BwdParams p) {
    constexpr int BKV = 128;                 // keys per workgroup: 4 waves x 32
    constexpr int BQ = D == 64 ? 64 : 32;    // queries per step
    constexpr int NQB = BQ / 32;             // 32-query blocks per step
    constexpr int NQC = BQ / 16;             // 16-query k-steps (products over q)
    constexpr int NKK = D / 16;              // 16-wide k-steps over d
    constexpr int NDB = D / 32;              // 32-row blocks over d
    constexpr int QROW = D * 2;              // bytes of a row-major [*, D] tile row
    constexpr int TROW = BQ * 2;             // bytes of a transposed [D, BQ] tile row
    constexpr int SROW = BKV * 2;            // bytes of a dS / K^T row
    constexpr int UN = (BQ / 4) * (D / 8);   // 4-row x 8-col units per staged tile
    static_assert(NQB * NDB == 4, "one 32x32 dQ block per wave");
    static_assert(2 * UN <= 256, "one staging unit per thread");

    __shared__ __attribute__((aligned(16))) char qs[BQ * QROW];
    __shared__ __attribute__((aligned(16))) char dos[BQ * QROW];
    __shared__ __attribute__((aligned(16))) char qts[D * TROW];
    __shared__ __attribute__((aligned(16))) char dots[D * TROW];
    __shared__ __attribute__((aligned(16))) char dss[BQ * SROW];
    __shared__ __attribute__((aligned(16))) char kts[D * SROW];
    __shared__ __attribute__((aligned(16))) float lse2s[BQ];
    __shared__ __attribute__((aligned(16))) float dvs[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hg = lane >> 5;
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int n_kt = (Nk + BKV - 1) / BKV;
    const int bh = blockIdx.x / n_kt;
    const int kt = blockIdx.x - bh * n_kt;
    const int k0 = kt * BKV;
    const int kj = k0 + wave * 32 + l32;     // this lane's key

    const bf16* Qh = (const bf16*)p.q + (size_t)bh * Nq * D;
    const bf16* Kh = (const bf16*)p.k + (size_t)bh * Nk * D;
    const bf16* Vh = (const bf16*)p.v + (size_t)bh * Nk * D;
    const bf16* dOh = (const bf16*)p.dO + (size_t)bh * Nq * D;
    const float* LSEh = p.lse + (size_t)bh * Nq;
    const float* Dh = p.dvec + (size_t)bh * Nq;
    float* dQh = p.dq_acc + (size_t)bh * Nq * D;

    // K^T and V^T as B operands (lane = key, 8 d-values per k-step)
    bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        u32x4 a = zero_u32x4(), b = zero_u32x4();
        if (kj < Nk) {
            a = ldg128(Kh + (size_t)kj * D + 16 * kk + 8 * hg);
            b = ldg128(Vh + (size_t)kj * D + 16 * kk + 8 * hg);
        }
        kreg[kk] = __builtin_bit_cast(bf16x8, a);
        vreg[kk] = __builtin_bit_cast(bf16x8, b);
    }
    // K^T of the whole key tile into LDS, natural key order (B operand of dQ)
    for (int u = tid; u < (BKV / 4) * (D / 8); u += 256) {
        const int kg = u / (D / 8), dc = u % (D / 8);
        u32x4 r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * kg + j;
            r[j] = key < Nk ? ldg128(Kh + (size_t)key * D + dc * 8) : zero_u32x4();
        }
        u32x2 cols[8];
        transpose4x8(r, cols);
        const uint32_t pos = 4 * kg;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(u32x2*)(kts + swz<SROW>(dc * 8 + e, pos >> 3) + (pos & 4u) * 2) = cols[e];
    }

    f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dvacc[db] = zero16();
        dkacc[db] = zero16();
    }

    const int qstart = CAUSAL ? max(0, k0 - off) : 0;   // first query that sees key k0
    const int n_qt = (Nq + BQ - 1) / BQ;
    const int wq = wave / NDB, wd = wave % NDB;          // this wave's dQ block

    for (int qt = qstart / BQ; qt < n_qt; ++qt) {
        const int q0 = qt * BQ;
        __syncthreads();   // the previous step's LDS reads are finished
        // ---- stage Q and dO, row-major and transposed (q-permuted) ----
        if (tid < 2 * UN) {
            const int which = tid / UN, u = tid % UN;
            const bf16* src = which ? dOh : Qh;
            char* rm = which ? dos : qs;
            char* tr = which ? dots : qts;
            const int rg = u / (D / 8), dc = u % (D / 8);
            u32x4 r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = q0 + 4 * rg + j;
                r[j] = q < Nq ? ldg128(src + (size_t)q * D + dc * 8) : zero_u32x4();
                *(u32x4*)(rm + swz<QROW>(4 * rg + j, dc)) = r[j];
            }
            u32x2 cols[8];
            transpose4x8(r, cols);
            const uint32_t pos = (rg >> 2) * 16 + kperm((rg & 3) * 4);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *(u32x2*)(tr + swz<TROW>(dc * 8 + e, pos >> 3) + (pos & 4u) * 2) = cols[e];
        }
        if (tid < BQ) {
            const int q = q0 + tid;
            float l2 = INFINITY, dd = 0.f;   // +inf: P = 0 for rows beyond Nq or without keys
            if (q < Nq) {
                const float L = LSEh[q];
                if (L != -INFINITY) l2 = L * kLog2e;
                dd = Dh[q];
            }
            lse2s[tid] = l2;
            dvs[tid] = dd;
        }
        __syncthreads();

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
                const bf16x8 a = *(const bf16x8*)(qs + swz<QROW>(qb * 32 + l32, 2 * kk + hg));
                s[qb] = mfma_bf16(a, kreg[kk], s[qb]);
                const bf16x8 b = *(const bf16x8*)(dos + swz<QROW>(qb * 32 + l32, 2 * kk + hg));
                dp[qb] = mfma_bf16(b, vreg[kk], dp[qb]);
            }

        // ---- P = exp2(S*scale*log2e - LSE*log2e), dS = P * (dP - D) ----
        u32x4 pw[NQC], dsw[NQC];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ql = qb * 32 + g * 8 + 4 * hg;   // local query of item 4g
                const f32x4 l2 = *(const f32x4*)(lse2s + ql);
                const f32x4 dd = *(const f32x4*)(dvs + ql);
                float pv[4], dsv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * g + e;
                    const int q = q0 + ql + e;
                    const bool vis = kj < Nk && (!CAUSAL || kj <= q + off);
                    const float pe = vis ? exp2_hw(fmaf(s[qb][i], p.scale_log2, -l2[e])) : 0.f;
                    pv[e] = pe;
                    dsv[e] = pe * (dp[qb][i] - dd[e]);
                    // write dS (bf16) for the dQ product: row = local query, col = local key
                    const int kl = wave * 32 + l32;
                    *(bf16*)(dss + swz<SROW>(ql + e, kl >> 3) + (kl & 7) * 2) = (bf16)dsv[e];
                }
                const int qc = qb * 2 + (g >> 1);
                pw[qc][(g & 1) * 2 + 0] = pack_bf16x2(pv[0], pv[1]);
                pw[qc][(g & 1) * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
                dsw[qc][(g & 1) * 2 + 0] = pack_bf16x2(dsv[0], dsv[1]);
                dsw[qc][(g & 1) * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
            }

        // ---- dV^T += dO^T P ;  dK^T += Q^T dS ----
#pragma unroll
        for (int qc = 0; qc < NQC; ++qc) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[qc]);
            const bf16x8 sb = __builtin_bit_cast(bf16x8, dsw[qc]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 a = *(const bf16x8*)(dots + swz<TROW>(db * 32 + l32, 2 * qc + hg));
                dvacc[db] = mfma_bf16(a, pb, dvacc[db]);
                const bf16x8 b = *(const bf16x8*)(qts + swz<TROW>(db * 32 + l32, 2 * qc + hg));
                dkacc[db] = mfma_bf16(b, sb, dkacc[db]);
            }
        }
        __syncthreads();   // dS of all four waves is in LDS

        // ---- dQ[q][d] += sum over this tile's keys of dS[q][key] K[key][d] ----
        {
            f32x16 acc = zero16();
#pragma unroll
            for (int kc = 0; kc < BKV / 16; ++kc) {
                const bf16x8 a = *(const bf16x8*)(dss + swz<SROW>(wq * 32 + l32, 2 * kc + hg));
                const bf16x8 b = *(const bf16x8*)(kts + swz<SROW>(wd * 32 + l32, 2 * kc + hg));
                acc = mfma_bf16(a, b, acc);
            }
            const int dcol = wd * 32 + l32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = q0 + wq * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
                if (q < Nq) unsafeAtomicAdd(dQh + (size_t)q * D + dcol, acc[i]);
            }
        }
    }

    // ---- dK = scale * dK^T acc, dV = dV^T acc (lane = key, items = d) ----
    if (kj < Nk) {
        bf16* dKr = (bf16*)p.dk + (size_t)bh * Nk * D + (size_t)kj * D;
        bf16* dVr = (bf16*)p.dv + (size_t)bh * Nk * D + (size_t)kj * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = db * 32 + g * 8 + 4 * hg;
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[db][4 * g] * p.scale, dkacc[db][4 * g + 1] * p.scale);
                wk[1] = pack_bf16x2(dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale);
                wv[0] = pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]);
                wv[1] = pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *(u32x2*)(dKr + dcol) = wk;
                *(u32x2*)(dVr + dcol) = wv;
            }
    }
}

// ---------------------------------------------------------------------------
// 3. dq = scale * dQ accumulator, rounded to bf16.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                            long n8, float scale) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = *(const f32x4*)(acc + i * 8);
    const f32x4 b = *(const f32x4*)(acc + i * 8 + 4);
    u32x4 w;
    w[0] = pack_bf16x2(a[0] * scale, a[1] * scale);
    w[1] = pack_bf16x2(a[2] * scale, a[3] * scale);
    w[2] = pack_bf16x2(b[0] * scale, b[1] * scale);
    w[3] = pack_bf16x2(b[2] * scale, b[3] * scale);
    *(u32x4*)(dq + i * 8) = w;
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t launch_bwd_d(bool causal, const BwdParams& p, hipStream_t s) {
    const long rows = (long)p.BH * p.Nq;
    if (rows > 0) {
        constexpr int RPB = 256 / (D / 8);
        const long grid = (rows + RPB - 1) / RPB;
        const bf16* o = (const bf16*)p.o;
        const bf16* dO = (const bf16*)p.dO;
        float* dvec = p.dvec;
        float* acc = p.dq_acc;
        long r = rows;
        void* args[] = {&o, &dO, &dvec, &acc, &r};
        hipError_t e = hipLaunchKernel((const void*)bwd_prep_kernel<D>, dim3((unsigned)grid), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    const int n_kt = (p.Nk + 127) / 128;
    const long grid_main = (long)p.BH * n_kt;
    if (grid_main > 0) {   // with Nq == 0 the walk is empty and dK = dV = 0 are written
        BwdParams pp = p;
        void* args[] = {&pp};
        const void* fn = causal ? (const void*)bwd_main_kernel<D, true> : (const void*)bwd_main_kernel<D, false>;
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid_main), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    if (rows > 0) {
        const long n8 = rows * D / 8;
        const float* acc = p.dq_acc;
        bf16* dq = (bf16*)p.dq;
        long n = n8;
        float sc = p.scale;
        void* args[] = {&acc, &dq, &n, &sc};
        hipError_t e = hipLaunchKernel((const void*)bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)),
                                       dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_bwd(int d, bool causal, BwdParams p, hipStream_t stream) {
    return d == 64 ? launch_bwd_d<64>(causal, p, stream) : launch_bwd_d<128>(causal, p, stream);
}

}  // namespace fa
