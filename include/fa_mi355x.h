/*
 * fa_mi355x.h -- C ABI of the fused attention forward library for AMD
 * Instinct MI355X (gfx950).  Library: libfa_mi355x.so.
 *
 * Operation.  For every batch b and head h, with Q, K, V the [N, d] slices:
 *
 *     S   = scale * Q K^T                 (fp32 accumulation)
 *     S_ij = -inf  where causal and j > i  (key j is kept iff j <= query i)
 *     O   = softmax_rows(S) V             (stored as fp16)
 *     LSE_i = ln sum_j exp(S_ij)          (fp32, natural log)
 *
 * computed as a fused pass that tiles the queries, streams K/V blocks through
 * on-chip memory and keeps a running row max and row sum, so the N x N score
 * matrix never reaches device memory.  The method is the one described in
 * "TCA 51%，MFU 不足 8%——GPU 的隐藏性能损耗" (section "FA2 TCA 虚高归因":
 * online softmax accumulates softmax@V block by block without materialising
 * the [B, L, L] map) and in "第 17 章 TMA + Warp Specialization 把 FA2 写到
 * SOTA" §17.5 (per K/V tile: S = Q K^T, running max/sum update, rescale of
 * the O accumulator, O += P V, final division by the row sum).  The tensor
 * layout [B, H, N, d] with d contiguous is the one of §17.3 of the same
 * chapter.  The causal mask, the scale and the LSE output are not on those
 * pages; they are defined as above.
 *
 * Conventions shared by every entry point:
 *   - q, k, v, o, lse and the descale arrays are DEVICE pointers owned by the
 *     caller; the library allocates, frees and retains none of them and may
 *     be called from several host threads at once.  Its only state is a
 *     per-device cache of the current device's compute-unit and XCD counts
 *     (read from the runtime on first use after a call's arguments have been
 *     validated), which choose launch shapes and never change results
 *     beyond rounding.
 *   - q, k, v: [B, H, N, d] contiguous, element type given by the dtype.
 *     o: [B, H, N, d] contiguous IEEE fp16 for every input dtype.
 *     lse: [B, H, N] contiguous fp32; required (never NULL when B*H*N > 0).
 *     q, k, v, o must be 16-byte aligned, lse 4-byte aligned.
 *   - d must be 64 or 128.  N >= 1 may be any length (ragged tails are
 *     masked).  B, H >= 1.  If B*H*N == 0 the call does nothing and returns
 *     FA_OK without reading any pointer.
 *   - scale must be finite and > 0 (1/sqrt(d) is the usual choice).
 *   - stream: a hipStream_t (NULL = the null stream).  The call only enqueues
 *     work and returns; results are ready when the stream reaches that point.
 *   - Errors: invalid arguments return a negative fa_status synchronously,
 *     before any HIP runtime call, and nothing is launched.  A failed kernel
 *     launch returns FA_ERR_LAUNCH.  Faults during execution surface at the
 *     caller's next synchronisation with the stream, as usual for HIP.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

typedef enum {
  FA_DTYPE_FP16 = 0,      /* IEEE binary16 */
  FA_DTYPE_BF16 = 1,      /* bfloat16 */
  FA_DTYPE_FP8_E4M3 = 2   /* OCP 8-bit E4M3 ("e4m3fn": no inf, max 448) */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,       /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,      /* B, H or N negative, or the problem is too large */
  FA_ERR_HEAD_DIM = -3,   /* d not in {64, 128} */
  FA_ERR_DTYPE = -4,      /* unknown dtype */
  FA_ERR_ALIGN = -5,      /* a pointer is not aligned as required */
  FA_ERR_LAUNCH = -6,     /* the HIP runtime refused the kernel launch */
  FA_ERR_SCALE = -7,      /* scale not finite and positive */
  FA_ERR_CAUSAL = -8,     /* causal not 0 or 1 */
  FA_ERR_LAYOUT = -9,     /* unknown tensor layout */
  FA_ERR_MIN_KEYS = -10,  /* fa_fwd_fp8_pv: min_keys negative */
  FA_ERR_WORKSPACE = -11, /* fa_fwd_kvsplit: workspace_bytes too small or negative */
  FA_ERR_SCRATCH = -12    /* fa_fwd_kvsplit_noalloc: split needs more than the static scratch */
} fa_status;

/* Memory layout of q, k, v and o (lse is always [B, H, N]). */
typedef enum {
  FA_LAYOUT_BHND = 0,     /* [B, H, N, d]: the rows of one head are adjacent */
  FA_LAYOUT_BNHD = 1      /* [B, N, H, d]: row n of every head, then row n+1 */
} fa_layout;

/*
 * fa_fwd -- attention forward for fp16, bf16 or fp8 inputs.
 * With dtype FA_DTYPE_FP8_E4M3 every head uses unit dequantization scales
 * (the fp8 codes are the values); use fa_fwd_fp8 to pass per-head scales.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
           int dtype, void* stream);

/*
 * fa_fwd_fp8 -- attention forward for OCP e4m3 inputs with per-head
 * dequantization scales.  The value of an input element is its e4m3 code
 * value times the float32 scale of its (b, h) head: descale_q[b*H + h] for Q,
 * and likewise for K and V.  descale_q, descale_k, descale_v are device
 * arrays of B*H floats, each finite and > 0 (other values give unspecified
 * results; they are not read on the host).  O and LSE are those of the
 * dequantized problem.  QK^T runs on fp8 matrix instructions with fp32
 * accumulation; P V runs in fp16 (the e4m3 values of V are exact in fp16).
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v,
               const float* descale_q, const float* descale_k,
               const float* descale_v, void* o, float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d, float scale,
               int causal, void* stream);

/*
 * fa_fwd_ex -- the same operation for either tensor layout and any dtype.
 * layout FA_LAYOUT_BHND gives exactly fa_fwd (or fa_fwd_fp8); with
 * FA_LAYOUT_BNHD, q, k, v and o are [B, N, H, d] contiguous (element (b, n,
 * h, i) at ((b*N + n)*H + h)*d + i), the layout the kernels of "Flash
 * Attention CUDA Kernel 优化: 从 56 到 986 TFLOPS on B300" take (section
 * V14, 坑二) -- while lse stays [B, H, N].  The
 * descale arrays are read for fp8 only: all three NULL means unit scales,
 * otherwise all three must be given (FA_ERR_NULL) as for fa_fwd_fp8.  For
 * [B, N, H, d] one head's rows span N*H*d elements, which must stay within
 * 2^30 bytes (FA_ERR_SHAPE).  An unknown layout returns FA_ERR_LAYOUT.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v,
              const float* descale_q, const float* descale_k,
              const float* descale_v, void* o, float* lse,
              int64_t B, int64_t H, int64_t N, int64_t d, float scale,
              int causal, int dtype, int layout, void* stream);

/*
 * fa_fwd_fp8_pv -- fa_fwd_ex for fp8 inputs with P V on the fp8 matrix
 * instructions as well, the fp8 scheme of "第 17 章 TMA + Warp Specialization
 * 把 FA2 写到 SOTA" (section 17.7: softmax output converted to fp8 before
 * the P V product, scales per block).  Here each query row's probabilities
 * of one 64-key block are multiplied by a power of two 2^k that brings the
 * largest into (128, 256], rounded to e4m3 (round to nearest even), and the
 * matrix instruction scales them back by 2^-k; the row sum is taken before
 * the rounding.  e4m3 keeps 3 fraction bits, so a row that sees few keys
 * loses accuracy: query tiles (128 rows) whose first row sees fewer than
 * min_keys keys (causal: row i sees i + 1; otherwise every row sees N) run
 * P V in fp16 exactly as fa_fwd_ex does.  min_keys = 0 puts every tile on
 * fp8 P V; min_keys > N gives fa_fwd_ex's result bit for bit.  512 keeps
 * max |O error| within 3e-2 on N(0, 1) inputs quantized per head (measured
 * 1.2e-2 at rows 512-1023, below 4e-3 past row 4096).  Other arguments as for
 * fa_fwd_ex with dtype FA_DTYPE_FP8_E4M3 (descales: all three or none);
 * min_keys < 0 returns FA_ERR_MIN_KEYS.  One or two kernels are enqueued
 * (disjoint query tiles).  Returns FA_OK or a negative fa_status.
 */
int fa_fwd_fp8_pv(const void* q, const void* k, const void* v,
                  const float* descale_q, const float* descale_k,
                  const float* descale_v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                  int causal, int layout, int64_t min_keys, void* stream);

/*
 * fa_fwd_fp8_kvtile -- attention forward for OCP e4m3 inputs whose K and V
 * carry one dequantization scale per tile of 64 consecutive key rows, the
 * per-block scale of "第 17 章 TMA + Warp Specialization 把 FA2 写到 SOTA"
 * (section 17.7, item 1: every K tile brings its own scale, so that one
 * scale for the whole tensor does not cost precision), applied to V's rows
 * in the same way.  Q keeps one scale per head.  With nt = ceil(N / 64):
 *   q element (b, h, n, i) = e4m3 code * descale_q[b*H + h]
 *   k element (b, h, n, i) = e4m3 code * descale_k[(b*H + h)*nt + n/64]
 *   v element (b, h, n, i) = e4m3 code * descale_v[(b*H + h)*nt + n/64]
 * descale_q: B*H floats; descale_k, descale_v: B*H*nt floats; all device
 * arrays, required (FA_ERR_NULL), 4-byte aligned (FA_ERR_ALIGN), each a
 * positive normal float (others give unspecified results; they are not
 * read on the host); |V| must stay within the fp16 range.  O and LSE are
 * those of the dequantized problem.  QK^T runs on the fp8 matrix
 * instructions, each key tile's scale folded into that block's scores.
 * pv_min_keys < 0: P V in fp16 (V's codes times the power-of-two part of
 * its tile scale are exact in fp16; the rest of the scale multiplies the
 * block's probabilities); pv_min_keys >= 0: P V on the fp8 matrix
 * instructions for the query tiles fa_fwd_fp8_pv would put there (the tile
 * scale's power of two travels in the instruction's block scale).  Other
 * arguments as for fa_fwd_ex with dtype FA_DTYPE_FP8_E4M3.  One or two
 * kernels are enqueued.  Returns FA_OK or a negative fa_status.
 */
int fa_fwd_fp8_kvtile(const void* q, const void* k, const void* v,
                      const float* descale_q, const float* descale_k,
                      const float* descale_v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                      int causal, int layout, int64_t pv_min_keys, void* stream);

/*
 * fa_fwd_kvsplit_workspace -- bytes of device workspace fa_fwd_kvsplit needs
 * for this problem: 0 when it would not split (then it runs fa_fwd_ex's
 * kernels and needs none), otherwise the size of the per-chunk partial
 * results (O rounded to fp16, LSE in fp32).  Arguments as for fa_fwd_ex (the
 * layout does not matter);
 * invalid ones return the negative fa_status fa_fwd_ex would.
 */
int64_t fa_fwd_kvsplit_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                 int causal, int dtype);

/*
 * fa_fwd_kvsplit -- fa_fwd_ex for grids too small or too unequal to fill the
 * GPU: few heads, or causal, where the longest query tiles would run alone
 * at the end (the under-filled launch measured in "TCA 51%，MFU 不足 8%",
 * section "基于 NCU 进行校验": a 256-block grid on 320 block slots leaves
 * part of the machine at half load).  The key range of long query tiles is cut into
 * chunks that separate workgroups process; a second kernel merges them with
 * LSE = ln sum_c exp(LSE_c) and O = sum_c exp(LSE_c - LSE) O_c, the identity
 * the LSE output exists for.  Chunks start at or before their tile's first
 * row, so every row has keys in every chunk.  The library chooses the chunk
 * size (or no split, when it estimates no gain; then it is fa_fwd_ex); the
 * result matches fa_fwd_ex within rounding (each chunk's O is rounded to
 * fp16 once before the merge, which then adds a few fp32 operations per
 * element).  workspace: device memory of at least
 * fa_fwd_kvsplit_workspace() bytes, 256-byte aligned (FA_ERR_ALIGN), owned
 * by the caller, contents irrelevant before and after; it may be NULL when
 * that size is 0 (FA_ERR_NULL otherwise).  workspace_bytes below the
 * requirement or negative returns FA_ERR_WORKSPACE.  Two kernels are
 * enqueued when splitting.  Other arguments and errors as for fa_fwd_ex.
 */
int fa_fwd_kvsplit(const void* q, const void* k, const void* v,
                   const float* descale_q, const float* descale_k,
                   const float* descale_v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                   int causal, int dtype, int layout, void* workspace,
                   int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_kvsplit_noalloc -- fa_fwd_kvsplit for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and split, with the
 * split workspace in a static device array of the library instead of a
 * caller buffer.  Arguments as for fa_fwd_kvsplit without workspace and
 * workspace_bytes; the caller still passes every input and output.  The
 * array holds fa_fwd_kvsplit_noalloc_max_bytes() bytes (64 MiB) on every
 * GPU the library runs on, from the first call on that GPU until the
 * process ends; a problem whose split needs more (fa_fwd_kvsplit_workspace)
 * returns FA_ERR_SCRATCH before any launch, and one that is not split needs
 * none.  The call itself allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.  Its first call on each device looks up that
 * device's array address (hipGetSymbolAddress); if the runtime refuses, it
 * returns FA_ERR_LAUNCH.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's partial results (each call writes every part
 * it reads, so nothing needs clearing): calls that overlap in time on one
 * GPU -- concurrent streams, or several host threads -- race and give
 * undefined results; serialize them.  Errors as for fa_fwd_kvsplit.
 */
int fa_fwd_kvsplit_noalloc(const void* q, const void* k, const void* v,
                           const float* descale_q, const float* descale_k,
                           const float* descale_v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                           int causal, int dtype, int layout, void* stream);

/* Bytes of the static split workspace of fa_fwd_kvsplit_noalloc. */
int64_t fa_fwd_kvsplit_noalloc_max_bytes(void);

/*
 * fa_fwd_fp8_pv_kvsplit -- fa_fwd_fp8_pv with the key-range split of
 * fa_fwd_kvsplit: query tiles whose first row sees fewer than min_keys keys
 * (short ones) run unsplit with P V in fp16, the others are split into chunks
 * with P V on the fp8 matrix instructions, and the chunks are merged through
 * their LSE.  Accuracy as fa_fwd_fp8_pv, plus the fp16 rounding of each
 * chunk's O before the merge.
 * workspace: at least fa_fwd_kvsplit_workspace(B, H, N, d, causal,
 * FA_DTYPE_FP8_E4M3) bytes, 256-byte aligned, or NULL when that is 0 (then
 * this is fa_fwd_fp8_pv).  Errors as for fa_fwd_fp8_pv and fa_fwd_kvsplit.
 */
int fa_fwd_fp8_pv_kvsplit(const void* q, const void* k, const void* v,
                          const float* descale_q, const float* descale_k,
                          const float* descale_v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                          int causal, int layout, int64_t min_keys, void* workspace,
                          int64_t workspace_bytes, void* stream);

/*
 * fa_bwd -- gradients of the attention forward pass (fp16 or bf16 inputs,
 * [B, H, N, d] layout).  Given dout = dL/dO for some loss L, it writes
 *
 *     dq = dL/dQ,  dk = dL/dK,  dv = dL/dV      (fp32 [B, H, N, d])
 *     delta_i = sum_c dout_ic * o_ic              (fp32 [B, H, N])
 *
 * by the chain rule through O = P V, P = softmax(scale Q K^T [+ causal
 * mask]): dV = P^T dO, dP = dO V^T, dS = P * (dP - delta), dQ = scale dS K,
 * dK = scale dS^T Q.  P is recomputed block by block from lse, so the N x N
 * matrices never reach device memory (the recomputation "TCA 51%，MFU 不足 8%"
 * counts for the backward pass; the pages give no further detail of it).
 * q, k, v, dout: the forward's inputs and the incoming gradient, element type
 * dtype; o (fp16) and lse (fp32 [B, H, N]): the forward's outputs for the
 * same q, k, v, scale and causal (fa_fwd's, or any consistent pair).  All
 * pointers are device pointers, 16-byte aligned, none NULL when B*H*N > 0;
 * the library allocates nothing (delta is the caller's workspace and an
 * output).  dtype FP8 returns FA_ERR_DTYPE.  Two kernels are enqueued on
 * the stream: dQ with delta, then dK and dV together.  P and dS enter the
 * products dV, dQ, dK rounded to dtype (dK's dS formed from that rounded P);
 * everything else accumulates in fp32.  Returns FA_OK or a negative fa_status.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, float* dq, float* dk, float* dv,
           float* delta, int64_t B, int64_t H, int64_t N, int64_t d,
           float scale, int causal, int dtype, void* stream);

/* Short English description of a status code (never NULL, static storage). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
