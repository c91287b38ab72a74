// Fused attention forward for gfx950 (MI355X): the FA2-order tiled forward
// ("01 · IO-awareness、online softmax 与 tiling" §2-§4; "FlashAttention 1～4
// 全解汇总", FlashAttention-2 algorithm) written for CDNA4 wave64 + MFMA.
//
// One workgroup owns one (batch*head, query tile).  Each wave owns 32 query
// rows of the tile (split over queries, so no cross-wave reduction).  Key /
// value tiles stream through LDS, double-buffered; S and P never leave the
// chip.
//
// Register-level formulation (bf16 path, 32x32x16 MFMA):
//   S^T[key][q] = K Q^T    : A = K rows from LDS, B = this wave's Q held in
//                            VGPRs, so each lane ends up owning ONE query
//                            (column l%32) and 16 of its keys per 32-key block.
//   row max / row sum      : lane-local over the 16*NKB values, then one
//                            exchange with the other 32-lane half.
//   O^T[dv][q] += V^T P^T  : B = P^T straight from the S^T accumulator (no
//                            LDS round trip), A = V^T, read from the
//                            untransposed V tile in LDS with the transposing
//                            ds_read_b64_tr_b16, keys in the order the
//                            accumulator hands them out.
//   The rescale by alpha = 2^(m_old - m_new) is a per-lane scalar because a
//   lane's O^T items all belong to its one query.
// exp is computed as exp2 with scale*log2(e) folded into one FMA (§4 of the
// IO-awareness page); LSE is converted back to natural-log units at the end.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// Workgroup id -> (batch*head, query tile): XCD-grouped heads (see
// map_head_tile); within a head the heaviest (last, for causal) query tile is
// issued first so the short tiles fill the tail.
__device__ __forceinline__ void map_workgroup(int w, int total, int n_qtiles, int& bh, int& qt, bool causal) {
    map_head_tile(w, total, n_qtiles, bh, qt, causal);
    qt = n_qtiles - 1 - qt;
}

// ---------------------------------------------------------------------------
// bf16 inputs, bf16 output, fp32 accumulation.  BR = 128 (4 waves x 32 rows),
// BC = 64 keys per tile.
//
// K and V tiles go from HBM straight into LDS (buffer_load ... lds: no VGPR
// staging), row-major with 16-byte chunks permuted by tile_swizzle.  Operands:
//   K  (A of S^T = K Q^T)   : ds_read_b128, 8 consecutive d of one key row.
//   V^T(A of O^T += V^T P^T): two ds_read_b64_tr_b16 per MFMA.  Within each
//       16-lane group that read hands lane i element e of the 8 bytes read by
//       lane 4e + i/4 (element i%4), so if those lanes read 4 key rows x 16
//       dv columns, lane i receives 4 consecutive keys of dv column i -- the
//       key-contiguous V^T operand, with V itself stored untransposed.
// ---------------------------------------------------------------------------

// Slack (log2 units) the scaling base may lag the true row maximum before O
// and l are rescaled: P values stay <= 2^8, far inside bf16 and fp32 range.
constexpr float kRescaleSlack = 8.0f;

// Fast path of the online softmax: once every row of a wave has a scaling
// base (set by the wave's first key tile with the row maximum), later tiles
// keep that base and skip the row maximum.  Any base gives the same O / l
// and m + log l in exact arithmetic; in floating point P, l and O~ keep their
// relative precision whatever the base, so the only hazard of a base below
// the true maximum is overflow, of l or of O~ = sum P V (which can overflow
// with l in range when |V| is beyond about 2^64).  A row whose lane-local
// running sum ends the query tile outside [0, kFastSumLimit], or whose O~
// accumulators are not all finite (overflow, or NaN inputs), marks the wave,
// and the workgroup then recomputes the query tile with the per-tile maximum
// and the conditional rescale above.
constexpr float kFastSumLimit = 0x1p64f;

// SPLIT: split-KV mode.  The key tiles of each query tile are divided into
// p.n_splits runs of p.tiles_per_split tiles, one workgroup per (batch*head,
// query tile, run); each writes its normalised partial O (fp32) and partial
// LSE (log2 units) to p.o_part / p.lse_part, and fwd_combine_kernel merges
// them.  Without SPLIT the workgroup owns whole query tiles.
// Waves per SIMD the register budget must allow: 2 at d = 128 (LDS holds
// two workgroups per CU), 3 at d = 64 (32 KiB of LDS per workgroup; 2, 3
// and 4 measured the same without the output staging, and 3 leaves the
// staging its registers).
template <int D>
constexpr int fwd_waves_per_simd() { return D == 64 ? 3 : 2; }

// MASK: kMaskNone, kMaskCausal (key j visible to query i iff j <= i + off,
// off = Nk - Nq) or kMaskWindow (iff i + off - wl <= j <= i + off + wr, the
// reaches p.wl, p.wr; an unbounded side holds kWindowUnbounded).
// VARLEN: the (batch, head) pair's lengths and rows come from the packed
// variable-length batch in p.vl; n_slots then counts the query tiles of the
// longest sequence, and a workgroup past its own sequence's tiles exits.
// PERSIST: a persistent grid (p.total_wg workgroups, a multiple of 8, about
// as many as fit on the device at once) over mirrored pairs of query tiles
// (p.paired, an even p.n_qtiles; p.n_slots = n_qtiles / 2 pairs per head).
// The T = BH * n_slots pairs, in head-major order, are cut into eight equal
// runs, one per XCD: workgroup w is on XCD x = w mod 8 (the hardware deals
// workgroup ids to the eight XCDs in turn) and takes pairs l, l + G, l + 2G,
// ... of run x (l = w / 8, G = p.total_wg / 8), so each XCD's workgroups
// share the K/V of a few consecutive heads at a time, and every XCD gets the
// same number of pairs whatever the head count.  Every pair holds the same
// causal work, so the workgroups stay balanced, and a workgroup prefetches
// its next item's first key tile even when the item belongs to another head;
// no workgroup waits to be dispatched after the first.
// SWEXP: 0, or 2, 4 or 8 for the opt-in software exponential (f3): one
// exponential of P in SWEXP is computed by exp2_poly on the FMA pipe instead
// of v_exp_f32 (chosen at compile time by its position in the tile).
template <int D, int MASK, bool SPLIT, bool VARLEN = false, bool PERSIST = false, int SWEXP = 0>
__global__ void __launch_bounds__(256, fwd_waves_per_simd<D>()) fwd_bf16_kernel(FwdParams p) {
    static_assert(SWEXP == 0 || SWEXP == 2 || SWEXP == 4 || SWEXP == 8, "one exponential in 2, 4 or 8");
    static_assert(!PERSIST || (!SPLIT && !VARLEN), "the persistent schedule is for whole fixed-length query tiles");
    static_assert(!PERSIST || D == 128, "the persistent Q warm-up covers 128 rows of 256 bytes");
    constexpr int BR = 128, BC = 64;
    constexpr int NKK = D / 16;        // k-steps over d for S^T
    constexpr int NKB = BC / 32;       // 32-key blocks per tile
    constexpr int NDB = D / 32;        // 32-row blocks of O^T
    constexpr int NKC = BC / 16;       // 16-key k-steps for O^T += V^T P^T
    // d = 128 uses the linear-offset tiles (lin_offset: every operand read
    // is one base register plus an immediate), d = 64 the swizzled ones
    constexpr bool kLin = D == 128;
    constexpr uint32_t PK = kLinPieceK, PV = kLinPieceV;
    constexpr int K_BYTES = kLin ? lin_tile_bytes<BC, PK>() : BC * D * 2;   // one K tile
    constexpr int V_BYTES = kLin ? lin_tile_bytes<BC, PV>() : BC * D * 2;   // one V tile
    constexpr int BUF_BYTES = K_BYTES + V_BYTES;                            // K tile + V tile
    using KCopy = std::conditional_t<kLin, LinTileCopy<BC, 4, PK>, TileCopy<D, BC, 4>>;
    using VCopy = std::conditional_t<kLin, LinTileCopy<BC, 4, PV>, TileCopy<D, BC, 4>>;
    using QCopy = std::conditional_t<kLin, LinTileCopy<BR, 4, PK>, TileCopy<D, BR, 4>>;

    __shared__ __attribute__((aligned(1024))) char smem[2 * BUF_BYTES];
    __shared__ int redo_flag[4];   // per wave: a row left the fast path's range
    __shared__ __attribute__((aligned(16))) int l2_sink[64];   // destination of l2_touch (never read)

    // wave index through readfirstlane: everything derived from it (LDS
    // addresses, the per-wave causal limits) stays in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hg = lane >> 5;
    // The workgroup's query tiles: tile n-1-j, then with pairing its mirror
    // j of the same head (causal: the two tiles together see n+1 rows of key
    // tiles whatever j is, so every workgroup gets the same work).
    int bh, slot, split = 0;
    if (SPLIT) {
        int r;
        map_head_tile(blockIdx.x, p.total_wg, p.n_qtiles * p.n_splits, bh, r);
        slot = p.n_qtiles - 1 - r / p.n_splits;   // so that tile n-1-slot is tile r / n_splits
        split = r % p.n_splits;
    } else if (VARLEN) {
        varlen_slot(p.vl, p.n_slots, blockIdx.x, bh, slot);
    } else if (PERSIST) {
        bh = 0;   // set per item below
        slot = 0;
    } else {
        map_head_tile(blockIdx.x, p.total_wg, p.n_slots, bh, slot, MASK == kMaskCausal && !p.paired);
    }
    // the (batch, head) pair's lengths and first rows in the [rows, D] views
    SeqGeometry sg;
    if constexpr (VARLEN) sg = seq_geometry(p.vl, bh);
    else sg = SeqGeometry{p.Nq, p.Nk, (size_t)bh * p.Nq, (size_t)bh * p.Nk};
    const int Nq = sg.Nq, Nk = sg.Nk, off = Nk - Nq;
    const int nqt = VARLEN ? (Nq + BR - 1) / BR : p.n_qtiles;
    if (VARLEN && slot >= nqt) return;   // past the sequence's last query tile
    // persistent schedule: this workgroup's XCD x, its index l there, G
    // workgroups per XCD, and its pairs u0 + l, u0 + l + G, ... of the XCD's
    // run [u0, u0 + U) of the T = BH * n_slots pairs (T < 2^31: fa_fwd
    // bounds B * H * (ceil(Nq / 64) + 1) by 2e9)
    const int px = blockIdx.x & 7, pl = blockIdx.x >> 3, pG = p.total_wg >> 3;
    int n_items = (!SPLIT && p.paired && slot != nqt - 1 - slot) ? 2 : 1;
    int pu0 = 0;
    if constexpr (PERSIST) {
        const long long T = (long long)p.BH * p.n_slots;
        pu0 = (int)(T * px / 8);
        const int U = (int)(T * (px + 1) / 8) - pu0;
        n_items = pl < U ? 2 * ((U - pl + pG - 1) / pG) : 0;
    }
    // right bound: key <= query + offr; left bound (windows): key >= query + offl
    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    // the fast softmax path (kFastSumLimit); split-KV runs, bound by HBM,
    // keep the per-tile maximum
    constexpr bool kFast = !SPLIT;
    const bf16* Qh = (const bf16*)p.q + sg.q_row0 * D;
    const bf16* Kh = (const bf16*)p.k + sg.k_row0 * D;
    const bf16* Vh = (const bf16*)p.v + sg.k_row0 * D;
    const uint32_t q_bytes = (uint32_t)Nq * D * 2, k_bytes = (uint32_t)Nk * D * 2;

    // Buffer resources over this head's Q, K and V: rows past Nq / Nk read as
    // zero, so ragged tails need no branches.
    // The copies go through async_load_lds16 (invisible to the compiler's
    // wait analysis): with the builtin form the compiler waits for the copy
    // of tile t+1 before the first V read of tile t, which puts a full HBM /
    // L2 round trip inside every tile.  Completion is awaited explicitly at
    // the end-of-tile barrier instead.
    const KCopy kcopier(wave, lane);
    const VCopy vcopier(wave, lane);
    // (set per item under the persistent schedule; nk_w, nv_w, nq_w are the
    // next item's, which the last key tile and the epilogue prefetch)
    i32x4 rk_w = make_rsrc_words(Kh, k_bytes);
    i32x4 rv_w = make_rsrc_words(Vh, k_bytes);
    i32x4 nk_w = rk_w, nv_w = rv_w;
    const uint32_t smem_lds = lds_address(smem);
    auto load_tile_r = [&](const i32x4& rk, const i32x4& rv, int k0, int buf) {
        kcopier.issue(rk, k0, smem_lds + buf * BUF_BYTES);
        vcopier.issue(rv, k0, smem_lds + buf * BUF_BYTES + K_BYTES);
    };
    auto load_tile = [&](int k0, int buf) { load_tile_r(rk_w, rv_w, k0, buf); };

    // Q takes the same route: the BR x D query tile (exactly one K + V
    // buffer) is copied into whichever buffer is idle at the start of an
    // item, then each wave reads its 32 rows into registers.  The kernel thus
    // has no register loads from memory at all, so the compiler's wait
    // analysis never sees a load in flight inside the key loop; there the
    // hardware counter also counts the copies of the next key tile, and any
    // wait it placed would stall every tile on them.
    static_assert((kLin ? lin_tile_bytes<BR, PK>() : BR * D * 2) <= BUF_BYTES, "a query tile fits one K + V buffer");
    const QCopy qcopier(wave, lane);
    // per-lane bases of the immediate-offset operand reads
    const uint32_t kbase = kLin ? lin_row_base<BC, PK>(lane) : 0u;
    const uint32_t qbase = kLin ? lin_row_base<BR, PK>(lane) : 0u;
    const uint32_t trbase = kLin ? lin_tr_base<PV>(lane) : 0u;
    i32x4 rq_w = make_rsrc_words(Qh, q_bytes);
    i32x4 nq_w = rq_w;
    auto load_q_r = [&](const i32x4& rq, int q0_, int buf) { qcopier.issue(rq, q0_, smem_lds + buf * BUF_BYTES); };
    auto load_q = [&](int q0_, int buf) { load_q_r(rq_w, q0_, buf); };
    bf16x8 qreg[NKK];
    // Key tiles a query tile needs: causal stops after the last key its last
    // query can see; tiles beyond are skipped entirely.
    auto tiles_of = [&](int qt_) {
        const int kend_ = kRight ? min(Nk, qt_ * BR + BR + offr) : Nk;
        return kend_ > 0 ? (kend_ + BC - 1) / BC : 0;
    };
    // first key tile a query tile needs (a window's left bound skips the rest)
    auto first_tile_of = [&](int qt_) { return kLeft ? max(0, qt_ * BR + offl) / BC : 0; };

    int b0 = 0;               // LDS buffer of the current item's first key tile
    bool prefetched = false;  // its Q and first key tile were issued by the previous item
    bool careful = false;     // recomputation of an item: row maximum on every tile
    for (int it = 0; it < n_items; ++it) {
    // this item's query tile, and the next item's (-1: none)
    int qt, nxt_qt = -1;
    if constexpr (PERSIST) {
        // item it: pair u0 + l + (it / 2) G, its tile n-1-s, then s
        const int u = pu0 + pl + (it >> 1) * pG, hh = u / p.n_slots, s_ = u - hh * p.n_slots;
        bh = hh;
        qt = (it & 1) ? s_ : nqt - 1 - s_;
        sg.q_row0 = (size_t)bh * Nq;
        sg.k_row0 = (size_t)bh * Nk;
        Qh = (const bf16*)p.q + sg.q_row0 * D;
        rq_w = make_rsrc_words(Qh, q_bytes);
        rk_w = make_rsrc_words((const bf16*)p.k + sg.k_row0 * D, k_bytes);
        rv_w = make_rsrc_words((const bf16*)p.v + sg.k_row0 * D, k_bytes);
        if (it + 1 < n_items) {
            if (!(it & 1)) {   // the mirror tile of the same head
                nxt_qt = s_;
                nq_w = rq_w;
                nk_w = rk_w;
                nv_w = rv_w;
            } else {           // the next pair: another head, probably
                const int u2 = u + pG, hh2 = u2 / p.n_slots, s2 = u2 - hh2 * p.n_slots;
                const size_t bh2 = (size_t)hh2;
                nxt_qt = nqt - 1 - s2;
                nq_w = make_rsrc_words((const bf16*)p.q + bh2 * Nq * D, q_bytes);
                nk_w = make_rsrc_words((const bf16*)p.k + bh2 * Nk * D, k_bytes);
                nv_w = make_rsrc_words((const bf16*)p.v + bh2 * Nk * D, k_bytes);
            }
        }
    } else {
        qt = it == 0 ? nqt - 1 - slot : slot;
        if (it + 1 < n_items) nxt_qt = slot;
    }
    const int q0 = qt * BR;
    const int qw = q0 + wave * 32;     // this wave's first query
    const int qi = qw + l32;           // this lane's query
    // key tiles [t_lo, t_hi) of this item (a run of them in split-KV mode)
    const int t_lo = SPLIT ? split * p.tiles_per_split : first_tile_of(qt);
    const int t_hi = SPLIT ? min(tiles_of(qt), t_lo + p.tiles_per_split) : tiles_of(qt);
    const int ntiles = t_hi > t_lo ? t_hi - t_lo : 0;
    // last key + 1 this wave sees; a wave whose rows all lie past Nq skips the math
    const int kend_w = qw >= Nq ? 0 : kRight ? min(Nk, qw + 32 + offr) : Nk;
    const int kbeg_w = kLeft ? qw + offl : 0;   // first key the wave's first row sees
    const bool more = nxt_qt >= 0;
    const int next_ntiles = more ? tiles_of(nxt_qt) - first_tile_of(nxt_qt) : 0;
    // Under the persistent schedule the second item of a pair walks its key
    // tiles downwards, from the diagonal: the 16 or so workgroups on a head
    // start their second items at staggered times, and walking down they all
    // read the same key tile at the same time (item s of length 2s + 2 begins
    // when the first, of length 64 - 2s, ends), so the head's K/V stays in
    // L2 instead of being read at as many offsets as there are workgroups.
    // The online softmax does not depend on the order of the tiles.
    const bool rev = PERSIST && (it & 1);
    const int t_first = rev ? t_hi - 1 : t_lo;   // the item's first key tile
    const int nxt_first = !more ? 0 : (PERSIST && !(it & 1)) ? tiles_of(nxt_qt) - 1 : first_tile_of(nxt_qt);

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
    float m_run = -INFINITY;   // running max of scale*log2e*S for this lane's query
    float l_run = 0.f;         // partial running sum over this lane's keys
    float nbase = 0.f;         // -m_run, or 0 while the row has seen no key (every term is then 0)
    bool have_base = false;    // every row of the wave has a base (wave-uniform)

    // Q into the idle buffer b0^1 (issued after the previous item's loop
    // when that item prefetched this one's first key tile into b0)
    if (!prefetched) {
        load_q(q0, b0 ^ 1);
        if (ntiles > 0) load_tile(t_first * BC, b0);
    }
    vmem_wait_all();
    tile_barrier();
    {
        const char* qbuf = smem + (b0 ^ 1) * BUF_BYTES;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qreg[kk] = kLin ? lin_read_row<BR>(qbuf + qbase, wave * 32, kk) : tile_read_row<D>(qbuf, wave * 32, kk, lane);
    }
    tile_barrier();   // every wave holds its Q rows before b0^1 takes the next key tile

    for (int i_t = 0; i_t < ntiles; ++i_t) {
        const int t = rev ? t_first - i_t : t_lo + i_t;
        const int k0 = t * BC;
        const int buf = (b0 + i_t) & 1;
        const char* kbuf = smem + buf * BUF_BYTES;
        const char* vbuf = kbuf + K_BYTES;
        const char* kread = kbuf + kbase;    // d = 128 tiles: operand = base + immediate
        const char* vread = vbuf + trbase;
        // the other buffer takes the next key tile, or the next item's first
        const bool has_next = i_t + 1 < ntiles || next_ntiles > 0;
        if (i_t + 1 < ntiles) load_tile(rev ? k0 - BC : k0 + BC, buf ^ 1);
        else if (has_next) load_tile_r(nk_w, nv_w, nxt_first * BC, buf ^ 1);
        // Persistent schedule: the next item's Q tile is copied in only after
        // this item's epilogue (its LDS buffer is the one this last tile
        // reads, then the output staging), so its lines are brought into the
        // L2 now, one line per lane (the 128 x 256-byte tile is 256 lines, 64
        // per wave), while this tile computes; the end-of-tile wait below
        // awaits these loads too (or, if the next item has no key tile, its
        // prologue's wait does), and the copy then hits the L2.  (A timing
        // probe that skipped the later items' Q copies bounds the gain at
        // 2.1% on the Llama-shaped workload; this measured +1.3% to +1.9%.)
        if (PERSIST && i_t + 1 == ntiles && more)
            l2_touch(nq_w, lds_address(l2_sink), (uint32_t)lane * 128 + (uint32_t)wave * 8192,
                     (uint32_t)nxt_qt * BR * D * 2);

        if (k0 < kend_w && (!kLeft || k0 + BC > kbeg_w)) {
            // ---- S^T = K Q^T (fp32 accumulators) ----
            f32x16 s[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    s[kb] = mfma_bf16(kLin ? lin_read_row<BC>(kread, kb * 32, kk) : tile_read_row<D>(kbuf, kb * 32, kk, lane),
                                      qreg[kk], s[kb]);
                }
            }
            // K-operand reads run 4 ahead of the MFMAs: 4 reads, then alternate
            // MFMA / read.  Deeper bursts measured slower (8 ahead -1%, 12-16
            // ahead -3%): a wave's burst of LDS reads delays the operand reads
            // of the other wave on the SIMD.
            constexpr int kAhead = NKK * NKB < 4 ? NKK * NKB : 4;
            __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
            for (int i = 0; i < NKK * NKB - kAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            // ---- mask: only tiles that straddle the diagonal or the tail ----
            const bool need_mask = (k0 + BC > Nk) || (kRight && k0 + BC - 1 > qw + offr) ||
                                   (kLeft && k0 < qw + 31 + offl);
            if (need_mask) {
                // item i of block kb is key k0 + kb*32 + (i/4)*8 + 4*hg + i%4: it is
                // visible iff its offset within the tile, past 4*hg, is <= lim
                // (key < Nk and key <= qi + offr): one compare per item, and for
                // a window also >= lo (key >= qi + offl)
                int lim = Nk - 1 - k0 - 4 * hg;
                if (kRight) lim = min(lim, qi + offr - k0 - 4 * hg);
                const int lo = kLeft ? qi + offl - k0 - 4 * hg : 0;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int o = kb * 32 + (i >> 2) * 8 + (i & 3);
                        if (o > lim || (kLeft && o < lo)) s[kb][i] = -INFINITY;
                    }
            }
            // ---- online softmax update (base-2, scale folded) ----
            // m_run is the scaling base.  It moves (and O, l are rescaled by
            // alpha) only when some row's new maximum exceeds it by more than
            // kRescaleSlack; otherwise P = 2^(s - m_run) <= 2^kRescaleSlack and
            // nothing is rescaled.  Exact after the final O / l ("FlashAttention
            // 1～4 全解汇总", FlashAttention-4 conditional softmax rescaling).
            if (!kFast || careful || !have_base) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = xhalf_max(mx) * p.scale_log2;
            // The decision is per row (a row that keeps its base multiplies by
            // exactly 1), so every row's result depends on that row alone; the
            // branch only skips the work when no row of the wave needs it.
            const bool grow = mx > m_run + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = grow ? mx : m_run;
                // alpha = 0 on a row's first visible tile (m_run = -inf)
                const float alpha = grow ? exp2_hw(m_run - m_new) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
                m_run = m_new;
                nbase = (m_run == -INFINITY) ? 0.f : -m_run;
            }
            // a row with no visible key so far keeps the maximum path
            have_base = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0;
            }
            // ---- P and O^T += V^T P^T, one 16-key block at a time ----
            // A block's P is packed right before its P.V MFMAs, so the
            // exponentials of the next block run while they execute.  Wave
            // priority is raised while this wave feeds the matrix cores, so
            // the other wave of the SIMD takes the issue slots they leave.
            __builtin_amdgcn_s_setprio(1);
            // fp32 row sums in four chains, each started with its first value
            // (P >= +0, so this equals adding it to 0, which the compiler
            // cannot fold away because of signed zeros)
            float rs[4];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int kb = kc >> 1, i0 = (kc & 1) * 8;
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = exp2_hw(fmaf(s[kb][i0 + 2 * j], p.scale_log2, nbase));
                    const float x1 = fmaf(s[kb][i0 + 2 * j + 1], p.scale_log2, nbase);
                    // the tile's exponential number kc*8 + 2j + 1 of 32
                    const bool soft = SWEXP > 0 && (kc * 8 + 2 * j + 1) % (SWEXP > 0 ? SWEXP : 1) == SWEXP - 1;
                    const float p1 = soft ? exp2_poly(x1) : exp2_hw(x1);
                    if (kc == 0 && j < 2) {
                        rs[2 * j] = p0;
                        rs[2 * j + 1] = p1;
                    } else {
                        rs[(2 * j) & 3] += p0;
                        rs[(2 * j + 1) & 3] += p1;
                    }
                    w[j] = pack_bf16x2(p0, p1);
                }
                const bf16x8 pb = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] = mfma_bf16(kLin ? lin_read_tr<PV>(vread, kc * 16, db * 32) : tile_read_tr<D>(vbuf, kc * 16, db * 32, lane),
                                         pb, oacc[db]);
            }
            l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
            // Issue order: the first block's 24 VALU instructions (8 FMA, 8
            // exp, 4 adds, 4 packs) and two V^T operands (four transposed
            // reads), then per MFMA two transposed reads and 7*4/NDB of the
            // next block's VALU instructions.  Measured against the compiler's
            // own order (all exponentials, then P.V in bursts of eight reads):
            // +2.3% on the Llama-shaped causal workload, +4% on the
            // training-step forward, -1.3% at N = 32768.
            {
                constexpr int vAhead = 2;
                // software exponentials add 8 VALU instructions each, 8 / SWEXP per block
                constexpr int kExtraV = SWEXP > 0 ? 8 * (8 / (SWEXP > 0 ? SWEXP : 1)) : 0;
                __builtin_amdgcn_sched_group_barrier(0x002, 24 + kExtraV, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * vAhead, 1);
#pragma unroll
                for (int i = 0; i < NKC * NDB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    if (i < NKC * NDB - vAhead) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                    if (i < (NKC - 1) * NDB) __builtin_amdgcn_sched_group_barrier(0x002, (7 * 4 + kExtraV) / NDB, 1);
                }
            }
        }

        __builtin_amdgcn_s_setprio(0);
        if (has_next) vmem_wait_all();   // this wave's copies of the next tile landed
        tile_barrier();
    }
    if (kFast && !careful && ntiles > 0) {
        // did any wave of the workgroup leave the fast path's range?  Then
        // run this item again, from its Q tile, with the per-tile maximum;
        // both LDS buffers are reloaded (the recomputation's last tile
        // fetches the next item's first tile again).
        // l_run only grows (a sum of terms >= 0; inf and NaN persist), so its
        // final value is checked once, after the last tile; the O~
        // accumulators by their sum (inf and NaN propagate through it; a
        // finite sum that overflows only costs a recomputation)
        float osum = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) osum += oacc[db][i];
        const bool bad = __builtin_amdgcn_ballot_w64(!(l_run <= kFastSumLimit) || !(fabsf(osum) <= 0x1.fffffep127f)) != 0;
        if (lane == 0) redo_flag[wave] = bad ? 1 : 0;
        tile_barrier();
        if ((redo_flag[0] | redo_flag[1] | redo_flag[2] | redo_flag[3]) != 0) {
            careful = true;
            prefetched = false;
            --it;
            continue;
        }
    }
    careful = false;

    // The next item's first key tile is already in LDS (buffer b0 below);
    // the other buffer is idle since the loop's last barrier.  The epilogue
    // stages O there first, except in the causal d = 64 kernel (the one whose
    // launches pair query tiles): there the buffer takes the next item's Q
    // tile right away, while this item's epilogue runs.
    prefetched = next_ntiles > 0 && ntiles > 0;
    b0 = (b0 + ntiles) & 1;
    constexpr bool kStageO = D == 128 || MASK != kMaskCausal;
    if (!kStageO && prefetched) load_q_r(nq_w, nxt_qt * BR, b0 ^ 1);

    // ---- epilogue: O = O~ / l, LSE = ln2 * (m + log2 l) ----
    const float l_tot = xhalf_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (SPLIT) {
        // partial result of this run of key tiles: O_s = O~ / l (fp32) and
        // LSE_s = m + log2 l (log2 units; -inf when the run saw no key)
        if (qi < Nq) {
            const size_t row = ((size_t)split * p.BH + bh) * Nq + qi;
            float* Op = p.o_part + row * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * g + e] * inv;
                    *(f32x4*)(Op + db * 32 + g * 8 + 4 * hg) = w;
                }
            if (hg == 0) p.lse_part[row] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
        }
        continue;
    }
    // O goes through LDS so that HBM sees whole rows: a lane holds one
    // query's d values in 8-byte pieces, so direct stores write scattered
    // 16-byte pieces per instruction and stall on their data registers.
    // Each wave writes its 32 rows into its own part of the idle buffer
    // (swizzled like the K/V tiles), reads them back row-contiguous and
    // stores 16 bytes per lane; no other wave touches those rows.  (Measured
    // +1.5% at d = 128 and +3.7% on the non-causal d = 64 GPT-2 shape; on
    // paired causal d = 64 launches direct stores, which let the next item's
    // Q tile load during the epilogue, measured 2.9% faster.  Choosing per
    // item at run time cost 11% there, so the choice is per kernel.)
    if constexpr (kStageO && kLin) {
        // the query-sized region in the query tile's layout: the wave's row
        // r (of 32) is row 32*wave + r, i.e. piece r at offset 256*wave; read
        // back four rows per pass (16 lanes a row), stored as whole rows
        char* obuf = smem + (b0 ^ 1) * BUF_BYTES;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                *(u32x2*)(obuf + lin_offset<BR, PK>(wave * 32 + l32, db * 4 + g) + hg * 8) = w;
            }
        bf16* Ow = (bf16*)p.o + sg.q_row0 * D + (size_t)qw * D;
        const int rr = lane >> 4, cc = lane & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + rr;
            const u32x4 x = *(const u32x4*)(obuf + lin_offset<BR, PK>(wave * 32 + r, cc));
            if (qw + r < Nq) *(u32x4*)(Ow + (size_t)r * D + cc * 8) = x;
        }
    } else if constexpr (kStageO) {
        char* ost = smem + (b0 ^ 1) * BUF_BYTES + wave * 32 * (D * 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                *(u32x2*)(ost + tile_offset<D>(l32, db * 4 + g) + hg * 8) = w;
            }
        constexpr int CPR = D / 8;          // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;       // rows per 64-lane pass
        bf16* Ow = (bf16*)p.o + sg.q_row0 * D + (size_t)qw * D;
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += RPI) {
            const int r = r0 + lane / CPR, c = lane % CPR;
            const u32x4 x = *(const u32x4*)(ost + tile_offset<D>(r, c));
            if (qw + r < Nq) *(u32x4*)(Ow + (size_t)r * D + c * 8) = x;
        }
    } else if (qi < Nq) {
        bf16* Oh = (bf16*)p.o + sg.q_row0 * D + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                *(u32x2*)(Oh + db * 32 + g * 8 + 4 * hg) = w;
            }
    }
    if (qi < Nq && hg == 0 && p.lse)
        p.lse[sg.q_row0 + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (kStageO && more) {
        // every wave has read its staged rows before the buffer takes the
        // next item's Q tile (or, unprefetched, that item's own copies)
        tile_barrier();
        if (prefetched) load_q_r(nq_w, nxt_qt * BR, b0 ^ 1);
    }
    }   // items
}
// ---------------------------------------------------------------------------
// Split-KV combine: the partial results (O_s, L_s) of a row over disjoint key
// runs merge by the online-softmax rescale ("01 · IO-awareness、online
// softmax 与 tiling" §2: the update is order-insensitive):
//   M = max_s L_s,  w_s = 2^(L_s - M),  O = sum_s w_s O_s / sum_s w_s,
//   LSE = ln2 * (M + log2 sum_s w_s).
// A row no run saw (every L_s = -inf) gets O = 0, LSE = -inf.
// One workgroup of 256 threads per row: thread t owns 8 output columns
// (chunk t % (D/8)) of the runs s = t / (D/8), + 256 / (D/8), ...; it loads
// four of its runs at a time and merges them with the same rescale against
// its own running maximum, so a thread waits for memory once per four runs
// (one round trip at the decode shape).  The threads' partial sums are then
// rescaled to the block's maximum and added across the run lanes through
// LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) fwd_combine_kernel(FwdParams p) {
    constexpr int TPR = D / 8;          // 8-column chunks per row
    constexpr int J = 256 / TPR;        // run lanes
    constexpr int U = 4;                // runs a thread loads at once
    __shared__ float red[J][D + 4];
    __shared__ float wred[4];
    const long rows = (long)p.BH * p.Nq;
    const long row = blockIdx.x;
    const int t = threadIdx.x, c = t % TPR, j = t / TPR;
    const int ns = p.n_splits;
    // Each thread merges its runs s = j, j + J, ... U at a time (all loads of
    // a group in flight together) with the online rescale, keeping its own
    // maximum Mt; the threads' results are then rescaled to the block's M.
    float Mt = -INFINITY, wsum = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s0 = j; s0 < ns; s0 += U * J) {
        float L[U];
        f32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * J;
            const bool ok = s < ns;
            const size_t r = (size_t)(ok ? s : 0) * rows + row;
            L[u] = ok ? p.lse_part[r] : -INFINITY;
            const float* Op = p.o_part + r * D + c * 8;
            a[u] = *(const f32x4*)Op;          // run 0's values when !ok: weight 0 below
            b[u] = *(const f32x4*)(Op + 4);
        }
        float mc = Mt;
#pragma unroll
        for (int u = 0; u < U; ++u) mc = fmaxf(mc, L[u]);
        if (mc == -INFINITY) continue;          // no run of this group (or before) saw a key
        const float alpha = exp2_hw(Mt - mc);   // 0 while Mt = -inf
        wsum *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        Mt = mc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = L[u] == -INFINITY ? 0.f : exp2_hw(L[u] - Mt);
            wsum += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] = fmaf(w, a[u][e], acc[e]);
                acc[4 + e] = fmaf(w, b[u][e], acc[4 + e]);
            }
        }
    }
    // M = max over the threads' maxima
    float M = Mt;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if ((t & 63) == 0) wred[t >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    const float scale = Mt == -INFINITY ? 0.f : exp2_hw(Mt - M);
#pragma unroll
    for (int e = 0; e < 8; ++e) red[j][c * 8 + e] = acc[e] * scale;
    if (c == 0) red[j][D] = wsum * scale;
    __syncthreads();
    if (t < D) {
        float o = 0.f, ws = 0.f;
        for (int jj = 0; jj < J; ++jj) {
            o += red[jj][t];
            ws += red[jj][D];
        }
        ((bf16*)p.o)[row * D + t] = (bf16)(ws > 0.f ? o / ws : 0.f);
        if (t == 0 && p.lse) p.lse[row] = ws > 0.f ? (M + __log2f(ws)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs and output: true fp32 products on the 32x32x2 fp32 MFMA.
// BR = BC = 64 (2 waves x 32 rows); single-buffered LDS.
// ---------------------------------------------------------------------------
template <int D, int MASK>
__global__ void __launch_bounds__(128) fwd_f32_kernel(FwdParams p) {
    constexpr int BR = 64, BC = D == 128 ? 32 : 64;   // LDS: K (padded) + V within 64 KiB
    constexpr int NKB = BC / 32, NDB = D / 32;
    constexpr int KS = D + 1;          // padded K row: lanes on 32 rows hit 32 banks
    __shared__ float ks[BC * KS];
    __shared__ __attribute__((aligned(16))) float vs[BC * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hg = lane >> 5;
    int bh, qt;
    map_workgroup(blockIdx.x, p.total_wg, p.n_qtiles, bh, qt, MASK == kMaskCausal);
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int q0 = qt * BR;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    const float* Qh = (const float*)p.q + (size_t)bh * Nq * D;
    const float* Kh = (const float*)p.k + (size_t)bh * Nk * D;
    const float* Vh = (const float*)p.v + (size_t)bh * Nk * D;

    constexpr bool kRight = MASK != kMaskNone, kLeft = MASK == kMaskWindow;
    const int offr = off + (MASK == kMaskWindow ? p.wr : 0);
    const int offl = off - (MASK == kMaskWindow ? p.wl : 0);
    const int kend = kRight ? min(Nk, q0 + BR + offr) : Nk;
    const int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;
    const int t_first = kLeft ? max(0, q0 + offl) / BC : 0;
    const int kend_w = kRight ? min(Nk, qw + 32 + offr) : Nk;
    const int kbeg_w = kLeft ? qw + offl : 0;

    float qreg[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qreg[kk] = qi < Nq ? Qh[(size_t)qi * D + 2 * kk + hg] : 0.f;

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
    float m_run = -INFINITY, l_run = 0.f;

    for (int t = t_first; t < ntiles; ++t) {
        const int k0 = t * BC;
        __syncthreads();
        for (int c = tid; c < BC * D / 4; c += 128) {
            const int r = c / (D / 4), cc = c % (D / 4);
            f32x4 kv, vv;
            if (k0 + r < Nk) {
                kv = *(const f32x4*)(Kh + (size_t)(k0 + r) * D + cc * 4);
                vv = *(const f32x4*)(Vh + (size_t)(k0 + r) * D + cc * 4);
            } else {
                kv[0] = kv[1] = kv[2] = kv[3] = 0.f;
                vv = kv;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ks[r * KS + cc * 4 + e] = kv[e];
            *(f32x4*)(vs + r * D + cc * 4) = vv;
        }
        __syncthreads();
        if (k0 >= kend_w || (kLeft && k0 + BC <= kbeg_w)) continue;

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                s[kb] = mfma_f32(ks[(kb * 32 + l32) * KS + 2 * kk + hg], qreg[kk], s[kb]);

        const bool need_mask = (k0 + BC > Nk) || (kRight && k0 + BC - 1 > qw + offr) ||
                               (kLeft && k0 < qw + 31 + offl);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + kb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
                    const bool vis = key < Nk && (!kRight || key <= qi + offr) && (!kLeft || key >= qi + offl);
                    if (!vis) s[kb][i] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * p.scale_log2);
        const float base = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_hw(m_run - base);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[kb][i] = exp2_hw(fmaf(s[kb][i], p.scale_log2, -base));
                rs += s[kb][i];
            }
        l_run = alpha * l_run + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        // O^T += V^T P^T, two keys (one per 32-lane half) per MFMA
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + (i >> 2) * 8 + 4 * hg + (i & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] = mfma_f32(vs[key * D + db * 32 + l32], s[kb][i], oacc[db]);
            }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qi < Nq) {
        float* Oh = (float*)p.o + (size_t)bh * Nq * D + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * g + e] * inv;
                *(f32x4*)(Oh + db * 32 + g * 8 + 4 * hg) = w;
            }
        if (hg == 0 && p.lse)
            p.lse[(size_t)bh * Nq + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
int fwd_rows_per_workgroup(int dtype, int d) {
    (void)d;
    return dtype == 0 ? 64 : 128;
}

// 256 CUs x 2 resident workgroups = 512 slots; pair when the unpaired grid
// covers them at least four times and a workgroup's start-up (Q and first key
// tile from HBM) and epilogue are a noticeable share of its work: short
// sequences with d = 64 (measured +10% at N=4096).  At d = 128 pairing on its
// own gained nothing at N=4096 and cost L2 locality (twice the heads in flight
// per XCD: 1.4x the L2 miss traffic), and at N=32768 it lost 1.6%; there the
// pairs run on the persistent grid below (+1% to +1.6% at N = 4096: no
// workgroup waits for dispatch after the first).
bool fwd_pair_tiles(int dtype, int d, bool causal, long bh, int n_qtiles) {
    return dtype == 1 && d == 64 && causal && n_qtiles >= 2 && n_qtiles <= 64 && bh * n_qtiles >= 4 * 512;
}

// The persistent causal d = 128 grid: one workgroup per resident slot (512),
// when the heads' mirrored pairs of query tiles give every workgroup at
// least two of them and close to the same number.  The busiest workgroups
// take ceil(T / 512) of the T pairs; when T / (512 ceil(T / 512)) falls
// below 0.8 (a last round of pairs that few workgroups share), the
// one-workgroup-per-tile grid, balanced tile by tile, is faster.  (Measured:
// 2.06 and 2.25 pairs per workgroup ran 6-13% faster on that grid at 16 to
// 704 query tiles per head; 2.5 ran 0.5-7% faster persistent, except -0.9%
// at 512 query tiles.)
int fwd_persist_grid(int dtype, int d, bool causal, long bh, int n_qtiles) {
    constexpr int kSlots = 512;
    if (!(dtype == 1 && d == 128 && causal && n_qtiles >= 2 && n_qtiles % 2 == 0)) return 0;
    const long T = bh * (n_qtiles / 2);
    const long per_wg = (T + kSlots - 1) / kSlots;
    const bool ok = T >= 2L * kSlots && 10 * T >= 8 * kSlots * per_wg;
    return ok ? kSlots : 0;
}

template <typename KernelT>
static hipError_t launch(KernelT kernel, int grid, int block, const FwdParams& p, hipStream_t s) {
    FwdParams pp = p;
    void* args[] = {&pp};
    return hipLaunchKernel((const void*)kernel, dim3(grid), dim3(block), args, 0, s);
}

// the software-exponential forward (bf16, no window): period p.soft_exp2
template <int D, int MASK, bool PERSIST>
static hipError_t launch_soft_exp2(const FwdParams& p, hipStream_t s) {
    if (p.soft_exp2 == 2) return launch(fwd_bf16_kernel<D, MASK, false, false, PERSIST, 2>, p.total_wg, 256, p, s);
    if (p.soft_exp2 == 4) return launch(fwd_bf16_kernel<D, MASK, false, false, PERSIST, 4>, p.total_wg, 256, p, s);
    return launch(fwd_bf16_kernel<D, MASK, false, false, PERSIST, 8>, p.total_wg, 256, p, s);
}

template <int MASK>
static hipError_t launch_fwd_mask(int dtype, int d, const FwdParams& p, hipStream_t stream) {
    const int grid = p.total_wg;
    if constexpr (MASK != kMaskWindow) {
        if (p.soft_exp2 && dtype == 1) {
            if (d == 64) return launch_soft_exp2<64, MASK, false>(p, stream);
            if constexpr (MASK == kMaskCausal)
                if (p.persist) return launch_soft_exp2<128, MASK, true>(p, stream);
            return launch_soft_exp2<128, MASK, false>(p, stream);
        }
    }
    if constexpr (MASK == kMaskCausal)
        if (p.persist) return launch(fwd_bf16_kernel<128, kMaskCausal, false, false, true>, grid, 256, p, stream);
    if (dtype == 1)
        return d == 64 ? launch(fwd_bf16_kernel<64, MASK, false>, grid, 256, p, stream)
                       : launch(fwd_bf16_kernel<128, MASK, false>, grid, 256, p, stream);
    return d == 64 ? launch(fwd_f32_kernel<64, MASK>, grid, 128, p, stream)
                   : launch(fwd_f32_kernel<128, MASK>, grid, 128, p, stream);
}

hipError_t launch_fwd(int dtype, int d, int mask, FwdParams p, hipStream_t stream) {
    if (p.total_wg == 0) return hipSuccess;
    if (mask == kMaskCausal) return launch_fwd_mask<kMaskCausal>(dtype, d, p, stream);
    if (mask == kMaskWindow) return launch_fwd_mask<kMaskWindow>(dtype, d, p, stream);
    return launch_fwd_mask<kMaskNone>(dtype, d, p, stream);
}

hipError_t launch_fwd_varlen(int d, int mask, FwdParams p, hipStream_t stream) {
    if (p.total_wg == 0) return hipSuccess;
    const int g = p.total_wg;
    if (d == 64) {
        if (mask == kMaskCausal) return launch(fwd_bf16_kernel<64, kMaskCausal, false, true>, g, 256, p, stream);
        if (mask == kMaskWindow) return launch(fwd_bf16_kernel<64, kMaskWindow, false, true>, g, 256, p, stream);
        return launch(fwd_bf16_kernel<64, kMaskNone, false, true>, g, 256, p, stream);
    }
    if (mask == kMaskCausal) return launch(fwd_bf16_kernel<128, kMaskCausal, false, true>, g, 256, p, stream);
    if (mask == kMaskWindow) return launch(fwd_bf16_kernel<128, kMaskWindow, false, true>, g, 256, p, stream);
    return launch(fwd_bf16_kernel<128, kMaskNone, false, true>, g, 256, p, stream);
}

hipError_t launch_fwd_split(int d, bool causal, FwdParams p, hipStream_t stream) {
    if (p.total_wg == 0) return hipSuccess;
    hipError_t e;
    if (d == 64)
        e = causal ? launch(fwd_bf16_kernel<64, kMaskCausal, true>, p.total_wg, 256, p, stream)
                   : launch(fwd_bf16_kernel<64, kMaskNone, true>, p.total_wg, 256, p, stream);
    else
        e = causal ? launch(fwd_bf16_kernel<128, kMaskCausal, true>, p.total_wg, 256, p, stream)
                   : launch(fwd_bf16_kernel<128, kMaskNone, true>, p.total_wg, 256, p, stream);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((long)p.BH * p.Nq);
    return d == 64 ? launch(fwd_combine_kernel<64>, grid, 256, p, stream)
                   : launch(fwd_combine_kernel<128>, grid, 256, p, stream);
}

}  // namespace fa
