/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * Exact scaled-dot-product attention, computed tile by tile with the online
 * softmax so that the Nq x Nk score matrix S and probability matrix P never
 * reach device memory:
 *
 *     S = scale * Q K^T,   P = row-softmax(S),   O = P V,
 *     LSE_i = m_i + ln(l_i)  (row max m, row sum l = sum_j exp(S_ij - m_i)).
 *
 * Pages defining the operations (cited by title and section):
 *   "01 · IO-awareness、online softmax 与 tiling": §1 (the three-step
 *       definition), §2 (online softmax state m, l, O and its rescale),
 *       §3 (tiled forward: one kernel instance per query tile, loop over key
 *       tiles, deferred normalisation, LSE saved), §5 (backward by
 *       recomputation from LSE and its gradient formulas).
 *   "FlashAttention 1～4 全解汇总": FlashAttention-2 algorithm (parallel over
 *       query row blocks, O_i = O~_i / l_i, L_i = m_i + log l_i).
 *   "让注意力计算留在片上：分块 Softmax 的计算与访存分析": §02 (the m, l, u
 *       recurrence), §04 (recompute P from the saved L in backward).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout   q, o, dO, dq: [B, H, Nq, d];  k, v, dk, dv: [B, H, Nk, d];
 *          lse: [B, H, Nq].  All contiguous, row-major, d innermost.
 * dtype    q, k, v, o, dO, dq, dk, dv share `dtype` (FA_F32 or FA_BF16);
 *          lse is always float32; all accumulation is float32; bf16 results
 *          are rounded to nearest even.
 * d        64 or 128.
 * scale    multiplies the logits (S = scale * Q K^T); must be finite and > 0.
 *          Usually 1/sqrt(d).
 * causal   nonzero: key j is visible to query i iff j <= i + (Nk - Nq)
 *          (bottom-right alignment; j <= i when Nq == Nk).  A query row with
 *          no visible key gets O = 0 and LSE = -inf and contributes nothing
 *          to the gradients.
 * Memory   the caller owns all device memory.  The library allocates nothing,
 *          frees nothing and keeps no pointer after returning (the one
 *          exception: fa_bwd_noalloc's static per-device array).  Pointers to
 *          tensors must be 16-byte aligned device pointers; lse 4-byte aligned.
 * Streams  `stream` is a hipStream_t (NULL = the null stream).  Work is
 *          enqueued asynchronously; no host synchronisation happens.  Faults
 *          inside a kernel surface at the caller's next synchronisation.
 * Errors   0 on success, a negative fa_status_t otherwise.  Arguments are
 *          validated before any HIP call; on a validation error nothing is
 *          enqueued and outputs are untouched.  The entry points are
 *          stateless and may be called from several host threads.
 * Empty    B, H or Nq equal to 0 is a no-op that returns FA_OK (pointers may
 *          then be NULL).  Nk == 0 is valid: every row is empty.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_F32 = 0,
    FA_BF16 = 1
} fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,       /* a required pointer is NULL                    */
    FA_ERR_SHAPE = -2,      /* negative size, or sizes beyond the limits     */
    FA_ERR_HEAD_DIM = -3,   /* d is not 64 or 128                            */
    FA_ERR_DTYPE = -4,      /* unknown dtype, or one this call does not take */
    FA_ERR_ALIGN = -5,      /* a tensor pointer is not 16-byte aligned       */
    FA_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than required       */
    FA_ERR_LAUNCH = -7,     /* the HIP runtime refused a kernel launch       */
    FA_ERR_SCALE = -8,      /* scale is not finite or not > 0                */
    FA_ERR_WINDOW = -9,     /* a window reach below -1                       */
    FA_ERR_SCRATCH = -10,   /* beyond fa_bwd_noalloc's static buffer         */
    FA_ERR_PERIOD = -11     /* fa_fwd_soft_exp2's period is not 2, 4 or 8    */
} fa_status_t;

/* Largest Nq or Nk accepted (keeps every in-head byte offset within 32 bits). */
#define FA_MAX_SEQ (1 << 23)

/*
 * Forward pass ("01 · IO-awareness、online softmax 与 tiling" §3;
 * "FlashAttention 1～4 全解汇总", FlashAttention-2 algorithm).
 *
 *   in : q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,d]          (dtype)
 *   out: o [B,H,Nq,d] (dtype), lse [B,H,Nq] (float32, natural log)
 *
 * lse may be NULL, in which case it is not written.  o must not alias q, k
 * or v.  Deterministic: the same inputs give bitwise the same outputs.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           int dtype, void* stream);

/*
 * fa_fwd with part of the softmax's exponentials computed in software on the
 * FMA pipe ("FlashAttention 1～4 全解汇总", FlashAttention-4, software-
 * emulated exponential; the exponent in base 2 as in "01 · IO-awareness、
 * online softmax 与 tiling" §4): one of every `period` (2, 4 or 8)
 * exponentials of P is 2^floor(x) * p(x - floor(x)) with p a degree-3
 * polynomial (Remez minimax fit, relative error <= 7.5e-5), the rest are the
 * hardware's v_exp_f32.  Arguments, layouts and errors are those of fa_fwd;
 * bf16 only (FA_ERR_DTYPE otherwise); a period other than 2, 4 or 8 returns
 * FA_ERR_PERIOD.  Results meet fa_fwd's tolerance but differ from it in the
 * last bits.
 *
 * On MI355X this is slower than fa_fwd: v_exp_f32 issues on the same pipe
 * as the FMAs (about 2 FMA slots per exponential), while the polynomial takes
 * 9 VALU instructions, so moving exponentials to it adds VALU work instead of
 * relieving a separate unit.  It is kept for that measurement.
 */
int fa_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, float scale, int causal,
                     int dtype, int period, void* stream);

/*
 * Split-KV forward ("01 · IO-awareness、online softmax 与 tiling" §2: the
 * online update is order-insensitive, so partial results over disjoint key
 * ranges merge exactly by rescaling).  Same inputs, outputs and semantics as
 * fa_fwd, for grids too small to fill the GPU -- decoding, where Nq is a few
 * rows and Nk is long.  The 64-key tiles each 128-row query tile sees are
 * divided into runs, one workgroup per (batch, head, query tile, run); each
 * writes its normalised partial O (fp32) and partial LSE into the workspace,
 * and a second kernel merges them:
 *     M = max_s L_s,  w_s = 2^(L_s - M),  O = sum w_s O_s / sum w_s,
 *     LSE = ln2 * (M + log2 sum w_s).
 *
 *   n_splits  runs per query tile, 1..FA_MAX_SPLITS, or 0 to let the library
 *             choose (enough workgroups to cover the GPU about four times over,
 *             at least 4 key tiles per run).  The effective count is
 *             ceil(T / ceil(T / n_splits)) for T = ceil(Nk / 64) key tiles.
 *   workspace device memory of at least fa_fwd_splitkv_workspace_bytes() for
 *             the same arguments; contents on entry ignored, on exit
 *             unspecified.  Calls that share a workspace must not overlap.
 *
 * Only FA_BF16 (FA_ERR_DTYPE otherwise).  Deterministic.  Rounding differs
 * from fa_fwd (the partials are merged in fp32), within the same tolerance.
 */
#define FA_MAX_SPLITS 1024

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype, int n_splits);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, int n_splits, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes and mode: two
 * float32 row vectors [B,H,Nq] (the LSE in base-2 units and D = rowsum(dO *
 * O)) and, for FA_BF16 unless `deterministic`, a float32 dQ buffer
 * [B,H,Nq,d]; each part rounded up to 256 bytes.  Returns 0 for invalid sizes
 * or dtype.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype, int deterministic);

/*
 * Backward pass by recomputation ("01 · IO-awareness、online softmax 与
 * tiling" §5; "让注意力计算留在片上" §04):
 *
 *   P = exp(scale * Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,
 *   D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 *   in : q, k, v, o (the forward output), lse (the forward LSE), dO
 *   out: dq [B,H,Nq,d], dk [B,H,Nk,d], dv [B,H,Nk,d]           (dtype)
 *   workspace: device memory of at least fa_bwd_workspace_bytes() for the
 *   same sizes and mode; its contents on entry are ignored and on exit are
 *   unspecified.
 *
 * The loop of §5 fixes a key block and walks the query blocks that see it,
 * so dK and dV of a block are finished in one place while dQ is summed over
 * key blocks, which takes atomic adds or a separate reduction; whether that
 * sum is reproducible is the `deterministic` choice (the same section):
 *   deterministic != 0 dQ is accumulated in registers by a second kernel per
 *                      query tile, which computes S and dP again (7 products
 *                      per visible (query, key) pair at d = 64, 8 at
 *                      d = 128); every output is bitwise repeatable.  The
 *                      faster mode on MI355X, and the one to use.
 *   deterministic = 0  one kernel per key tile computes S, dP, dS, dV, dK and
 *                      dS K (5 products per pair) and adds dS K into the
 *                      float32 dQ buffer with atomics.  dK and dV are bitwise
 *                      repeatable; dQ's float32 sum runs in whatever order
 *                      the atomics land, so its bf16 rounding can differ
 *                      between calls.  Its 64 x d atomic adds per 64-query x
 *                      128-key step bound it by the chip's float32 atomic
 *                      rate (about 3.2e11 adds/s on MI355X): at B=4 H=16
 *                      N=4096 d=64 causal that is 2.8e8 adds, >= 0.86 ms,
 *                      where the deterministic mode takes about 0.52 ms.
 * Both modes meet the same tolerance against the exact gradients.  D is
 * formed once per row in float32 from the bf16 dO and O; the key-side
 * products use it as float32, while the deterministic dQ kernel folds -D into
 * its dP product as a pair of bf16 values whose sum is -D within 2^-16
 * relative (one more MFMA k-step instead of a subtraction per score), so
 * dQ and dK see D to within that rounding.
 *
 * FA_F32: every product in true float32 (the 32x32x2 fp32 MFMA) with float32
 * D and LSE; one algorithm, the deterministic one (a query-side kernel for dQ,
 * a key-side kernel for dK and dV), whatever `deterministic` says, so every
 * output is bitwise repeatable and the workspace is the two row vectors.
 *
 * Calls that share a workspace must not overlap.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           int dtype, int deterministic, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * arguments and results as fa_bwd with deterministic = 1 (bitwise the same
 * outputs), without the workspace: its two row vectors live in a static
 * device array of
 * FA_NOALLOC_SCRATCH_BYTES held by each GPU the library runs on until the
 * process ends.  The call allocates and frees nothing.
 *
 * Limit: fa_bwd_workspace_bytes(..., 1) of the call must not exceed
 * FA_NOALLOC_SCRATCH_BYTES, i.e. B * H * Nq <= 1,048,576 query rows (e.g.
 * B=8 H=32 N=4096, or B=1 H=32 N=32768); beyond it the call returns
 * FA_ERR_SCRATCH and enqueues nothing.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress, with the device
 * current).  Every call on one GPU shares its array, so calls that overlap on
 * one GPU (other streams, other host threads) race and must be ordered by the
 * caller; nothing in the array needs clearing between calls.
 */
#define FA_NOALLOC_SCRATCH_BYTES (8u << 20)

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, void* stream);

/*
 * Local (sliding-window) attention.  The tiled forward of "01 · IO-awareness、
 * online softmax 与 tiling" §3 applies a mask to each score block before the
 * online update and names sliding windows among its masks; the pages fix no
 * formula for one.  The reading taken here extends the causal rule above:
 * with off = Nk - Nq, key j is visible to query i iff
 *
 *     i + off - window_left  <=  j  <=  i + off + window_right,
 *
 * each reach >= 0, or -1 for a side with no bound (FA_ERR_WINDOW below -1).
 * (-1, 0) is exactly the causal mask and (-1, -1) no mask: those calls run
 * the causal / unmasked kernels and give bitwise the results of fa_fwd /
 * fa_bwd with causal = 1 / 0.  A sliding window of W keys ending at the
 * diagonal is (W - 1, 0).  Key tiles wholly outside a query tile's window
 * are skipped, so the work scales with the visible pairs.  A row with no
 * visible key gets O = 0 and LSE = -inf, as under the causal mask.
 *
 * Arguments, layouts, ownership, dtypes, modes and errors are those of
 * fa_fwd and fa_bwd, with (window_left, window_right) in place of causal.
 * fa_bwd_window must be given the window its forward pass used.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale,
                  int window_left, int window_right, int dtype, void* stream);

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dO, void* dq, void* dk, void* dv,
                  int B, int H, int Nq, int Nk, int d, float scale,
                  int window_left, int window_right, int dtype, int deterministic,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Variable-length (packed) batches.  The tiled forward of "01 · IO-awareness、
 * online softmax 与 tiling" §3 lists variable-length batches among the masks
 * it applies to each score block; the pages fix no layout.  Here B sequences
 * of different lengths are packed along the token axis of head-major tensors:
 *
 *   q, o, dO, dq: [H, total_q, d];  k, v, dk, dv: [H, total_k, d];
 *   lse: [H, total_q] (float32, natural log);
 *   cu_seqlens_q, cu_seqlens_k: int32 [B+1] device arrays; sequence b owns
 *   query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 *   cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of every head.
 *
 * Every sequence attends only within itself, with the mask taken over its
 * own lengths (off = Lk_b - Lq_b in the rules above).  The mask is a window
 * pair as in fa_fwd_window: (-1, -1) none, (-1, 0) causal, else a local
 * window.  max_seqlen_q and max_seqlen_k (<= FA_MAX_SEQ) must bound every
 * sequence's lengths; they size the grids.  The offsets must start at 0,
 * never decrease and end at most at total_q / total_k; the kernels clamp
 * offsets into [0, total] and lengths to the maxima, so inconsistent offsets
 * cannot cause an access outside the tensors, but the results of such
 * sequences are unspecified.  Rows outside every sequence (past
 * cu_seqlens[B]) are not written.  Since the host never reads the offsets,
 * they may be produced on the stream just before the call.
 *
 * Only FA_BF16 (FA_ERR_DTYPE otherwise).  The forward is deterministic;
 * fa_bwd_varlen has fa_bwd's two modes.  B, H or total_q equal to 0 is a
 * no-op that returns FA_OK.  fa_bwd_varlen's workspace: at least
 * fa_bwd_varlen_workspace_bytes(H, total_q, d, dtype, deterministic) bytes
 * (fa_bwd's workspace over the H * total_q packed rows); the same mask and
 * offsets as the forward call must be given.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                  float scale, int window_left, int window_right, int dtype, void* stream);

size_t fa_bwd_varlen_workspace_bytes(int H, int total_q, int d, int dtype, int deterministic);

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dO, void* dq, void* dk, void* dv,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                  int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                  float scale, int window_left, int window_right, int dtype,
                  int deterministic, void* workspace, size_t workspace_bytes, void* stream);

/* A static, human-readable description of a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
