/*
 * exattn - tiled exact softmax attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the shared library libexattn.so. Plain pointers and sizes only.
 *
 * The operation (forward): for every batch entry (or packed sequence) b, query head h and
 * query row i, with g = h / (heads_q / heads_kv) the KV head of h:
 *   s_ij  = scale * q_i . k_j  (+ a_ij for an additive mask)
 *   key j is hidden when j >= the sequence's key count, when causal and j > i
 *   (top-left alignment), when a bool mask holds 0, or when an additive mask holds -inf;
 *   out_i = sum_j softmax_j(s_ij) v_j over visible keys,
 *   lse_i = ln sum_j exp(s_ij) over visible keys (natural log, fp32).
 * A row with no visible key gets out = 0 and lse = -inf.
 * Sources: the forward keeps a running row max and row sum and emits a log-sum-exp
 * (FlyDSL PR #1033 "[Bugfix][Kernel] Fix NaN from the lazy rescale on a wide score range",
 * sections "Root cause", "The fix"); masks hide keys as in OpenWAM PR #64 (cuDNN SDPA
 * backward padding fix), section "Fix"; grouped KV heads and causal masking as in
 * flash-dmattn PR #122 "Fix NaN/Inf values in dV gradients during backward pass",
 * section "Problem".
 *
 * The operation (backward), given dout = dL/dout: P is recomputed from the stored lse as
 * exp(s - lse) (OpenWAM PR #64, "Summary"); dv = P^T dout and dk = scale * dS^T q
 * (flash-dmattn PR #122, "Solution", item 2), with dS = P * (dout v^T - rowsum(dout * out))
 * and dq = scale * dS k. dk and dv of a KV head sum over the query heads that share it.
 * Keys that no query can see receive exactly zero dk and dv.
 *
 * Ownership and ordering (NVIDIA cudnn-frontend PR #429 "Fix stream-ordering and
 * input-validation holes in the SM100 DSA backward interface", first commit message):
 *   - The caller owns every buffer. The library allocates no device memory and never
 *     synchronises; all work is enqueued in order on the caller's `stream`
 *     (a hipStream_t passed as void*, NULL = the null stream).
 *   - Outputs are write-only: out, lse, dq, dk, dv are fully written, including rows of
 *     packed tensors past cu_seqlens[num_seqs] (PFCCLab cudnn-frontend PR #9 "DSA: fix dK
 *     SMEM handoff race and two latent NaN sources in the dense indexer", item 2), so no
 *     result depends on their previous contents (flash-dmattn PR #122, "Root Cause" 1).
 *   - The backward workspace is cleared by the library on `stream` before use.
 *
 * Errors: every argument is validated on the host before anything is enqueued. On a
 * non-OK status nothing was enqueued and no output was touched, except EXATTN_ERR_HIP,
 * which reports a failed kernel launch. exattn_last_error() gives a per-thread message.
 * Rejected instead of run (cudnn-frontend PR #429, second and third commit messages;
 * cudnn-frontend PR #9, item 4): a dtype other than bf16 or fp16, a head_dim other than 64 or 128,
 * heads_q not a multiple of heads_kv, unaligned pointers or strides, a mask together with
 * cu_seqlens, a non-finite scale.
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXATTN_ABI_VERSION 2

typedef enum exattn_status {
  EXATTN_OK = 0,
  EXATTN_ERR_NULL = 1,       /* a required pointer is NULL */
  EXATTN_ERR_DTYPE = 2,      /* dtype not accepted by the call (bf16/fp16; fp8 e4m3 for fp8) */
  EXATTN_ERR_HEAD_DIM = 3,   /* head_dim not in {64, 128} */
  EXATTN_ERR_SHAPE = 4,      /* negative sizes, heads_q % heads_kv != 0, size overflow, an
                                unknown variant or a non-zero reserved field */
  EXATTN_ERR_STRIDE = 5,     /* a stride is negative, not a multiple of 8 elements, or too
                                large for the kernels' 32-bit tile offsets (see below) */
  EXATTN_ERR_ALIGN = 6,      /* a q/k/v/out/dout/dq/dk/dv pointer is not 16-byte aligned */
  EXATTN_ERR_MASK = 7,       /* bad mask kind, NULL mask, negative mask stride, mask + varlen */
  EXATTN_ERR_VARLEN = 8,     /* num_seqs < 1, max_seqlen < 0, or one cu_seqlens pointer NULL */
  EXATTN_ERR_WORKSPACE = 9,  /* workspace NULL, too small or not 256-byte aligned */
  EXATTN_ERR_SCALE = 10,     /* scale (or an fp8 descale) is NaN or infinite */
  EXATTN_ERR_HIP = 11        /* a HIP launch failed; see exattn_last_error() */
} exattn_status;

/* Element type of q, k, v, out, dout, dq, dk, dv (all the same). fp16 is threaded through
 * every kernel instead of being rejected (cudnn-frontend PR #429, the fp16 follow-up
 * commit: the element type reaches the kernel rather than being hard-coded). Additive
 * masks are bf16 for either type. EXATTN_DTYPE_FP8_E4M3 (OCP e4m3: 4 exponent bits, bias
 * 7, 3 mantissa bits, largest finite 448) is the input type of exattn_fwd_fp8 only; its
 * output is bf16. */
typedef enum exattn_dtype {
  EXATTN_DTYPE_BF16 = 0,
  EXATTN_DTYPE_FP16 = 1,
  EXATTN_DTYPE_FP8_E4M3 = 2
} exattn_dtype;

typedef enum exattn_mask_kind {
  EXATTN_MASK_NONE = 0,
  EXATTN_MASK_BOOL_U8 = 1,   /* uint8, nonzero = attend, 0 = hidden */
  EXATTN_MASK_ADD_BF16 = 2   /* bf16 added to the scaled score; -inf hides */
} exattn_mask_kind;

/*
 * Problem description (host memory; read during the call only).
 *
 * Dense layout (cu_seqlens_q == NULL): q, dout, out are [batch, seqlen_q, heads_q, head_dim]
 * and k, v are [batch, seqlen_k, heads_kv, head_dim], addressed through element strides
 * x_stride = {batch, token, head}; the head_dim stride is 1. lse is a contiguous fp32
 * [batch, heads_q, seqlen_q] array.
 *
 * Packed layout (cu_seqlens_q != NULL): q/dout/out are [seqlen_q, heads_q, head_dim] and k/v
 * are [seqlen_k, heads_kv, head_dim] where seqlen_q/seqlen_k are the packed row counts
 * (total_q, total_k); x_stride[0] is ignored. Sequence s owns query rows
 * [cu_seqlens_q[s], cu_seqlens_q[s+1]) and key rows [cu_seqlens_k[s], cu_seqlens_k[s+1]);
 * both arrays are int32 device memory with num_seqs + 1 non-decreasing entries starting at
 * 0 and ending at most at seqlen_q / seqlen_k; max_seqlen_q/k bound every sequence length.
 * lse is a contiguous fp32 [heads_q, seqlen_q] array. Causal alignment is per sequence.
 *
 * Gradient outputs dq, dk, dv are contiguous in the layout of q, k, v above.
 *
 * The mask (dense only) is indexed by element strides mask_stride = {b, h, i, j}; a stride
 * of 0 broadcasts that axis (key-broadcast and per-batch masks); mask_stride[3] must be 1.
 *
 * Size limits of the 16-bit (bf16/fp16) path: the kernels address a tile of up to 128 rows
 * through 32-bit byte offsets, so every token stride (x_stride[1] of q, k, v, out, dout)
 * and heads_q * head_dim and heads_kv * head_dim must be below 2^23 elements
 * (EXATTN_ERR_STRIDE / EXATTN_ERR_SHAPE otherwise). The fp8 forward needs its token
 * strides below 2^24 elements.
 *
 * Packed sequences with device offsets (the library never reads device memory on the
 * host, so it cannot check them): the kernels clamp every offset into [0, seqlen_q] (or
 * [0, seqlen_k]) and take sequence s as rows [c_s, max(c_s, c_{s+1})) of the clamped values,
 * so no offset array makes a kernel read or write outside the tensors. A sequence longer
 * than max_seqlen_q (max_seqlen_k) is truncated to its first max_seqlen_q query rows
 * (max_seqlen_k key rows): attention is computed over the truncated sequence, and the rows
 * and keys past the truncation are written like rows past cu_seqlens[num_seqs] (out 0,
 * lse -inf, dq 0, dk 0, dv 0). Callers that want every row computed pass max_seqlen at
 * least the longest sequence; the Python binding checks this whenever the offsets are on
 * the host.
 */
typedef struct exattn_problem {
  int32_t dtype;         /* exattn_dtype */
  int32_t batch;         /* dense: batch size; packed: ignored */
  int32_t seqlen_q;      /* dense: query length; packed: total query rows */
  int32_t seqlen_k;      /* dense: key length; packed: total key rows */
  int32_t heads_q;
  int32_t heads_kv;
  int32_t head_dim;      /* 64 or 128 */
  int32_t causal;        /* 0 or 1 */
  float scale;           /* multiplies q.k; finite (0 gives uniform attention) */
  int32_t mask_kind;     /* exattn_mask_kind */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];   /* out as read by the backward; the forward writes it contiguous */
  int64_t do_stride[3];  /* dout (backward only) */
  int64_t mask_stride[4];
  const void* mask;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t num_seqs;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t fwd_variant;   /* forward tiling for this call, 0 = default (see below) */
  int32_t bwd_variant;   /* backward kernels for this call, 0 = default (see below) */
  int32_t reserved;      /* must be 0 */
} exattn_problem;

/*
 * Tilings (fwd_variant, bwd_variant), selected per call so that concurrent calls from
 * different threads never see each other's choice. Every variant computes the same
 * function up to fp32 rounding; they exist to compare designs.
 *   fwd_variant 0 (default): 8 waves x 32 query rows per workgroup with the lazy rescale
 *     (threshold 8 in log2 units; FlyDSL PR #1033, "The fix"); 1: the same tiling with an
 *     eager rescale whenever a row max grows; 2: 4 waves x 64 rows, lazy, one wave per SIMD
 *     (bf16, head_dim 128, no mask, dense; other problems run variant 0).
 *   bwd_variant 0 (default): a dK/dV kernel (one workgroup per block of keys, the wave
 *     computing dS and dK one query tile behind the wave computing P and dV) and a separate
 *     dQ kernel (one workgroup per block of query rows, recomputing P and dP), no atomics,
 *     bitwise reproducible; 1: one fused kernel that adds dQ partial products into an fp32
 *     workspace accumulator with atomics, then a conversion pass (bf16 only, larger
 *     workspace; fp16 problems run variant 0); 2: as 0 with a dK/dV kernel whose two waves
 *     per key group work on the same query tile, two barriers per tile; 3: as 0, but the
 *     dK/dV kernel also stores every dS tile it forms (rounded to the input format, as for
 *     its dK product) in the workspace, and dQ = dS K is formed from it without recomputing
 *     S and dP; bitwise reproducible. Dense layouts whose dS takes at most 64 GiB
 *     (batch * heads_q * ceil(seqlen_q / 64) * ceil(seqlen_k / 128) * 16 KiB); other
 *     problems run variant 0.
 * Other values are rejected with EXATTN_ERR_SHAPE.
 */

/* ABI version of the loaded library (EXATTN_ABI_VERSION at build time). */
int exattn_abi_version(void);

/* Metadata-only support check: validates the description without touching device
 * memory (cudnn-frontend PR #429: a support gate must reject what the kernels cannot
 * run). Pointers to tensors are not checked here. */
exattn_status exattn_check(const exattn_problem* p);

/*
 * Forward. q, k, v: device pointers of the problem's dtype laid out as described above.
 * out: device pointer of that dtype, written contiguous ([batch, seqlen_q, heads_q,
 * head_dim] or packed [seqlen_q, heads_q, head_dim]); its o_stride entry is ignored.
 * lse: fp32 device pointer (layout above). Every element of out and lse is written.
 */
exattn_status exattn_fwd(const exattn_problem* p, const void* q, const void* k,
                         const void* v, void* out, float* lse, void* stream);

/*
 * fp8 forward (FlyDSL PR #1033, "[Bugfix][Kernel] Fix NaN from the lazy rescale on a wide
 * score range", section "The fp8 helper, second commit"). q, k, v: device e4m3 bytes in the
 * dense layout above (p->dtype = EXATTN_DTYPE_FP8_E4M3, head_dim 128, no mask, no
 * cu_seqlens; strides multiples of 16 elements), each with one float descale: the
 * represented values are q * q_descale and so on. The softmax sees the scores
 * s_ij = q_i . k_j * scale * q_descale * k_descale. Key tiles of 64 are walked in order
 * with a running base per query row: when, in a group of 32 consecutive rows (one
 * 64-wide wave), some row's tile max exceeds its base by more than 8 (log2 units), every
 * row of the group is rebased onto its own tile max, but never more than 16 (log2 units)
 * below the row's running max; exponentials against the base (at most 2^8) are rounded to
 * e4m3 for the product with v, the row sum takes them unrounded. out (bf16, written
 * contiguous [batch, seqlen_q, heads_q, 128]) is (rounded P) v * v_descale / row sum, so it
 * differs from exact attention of the represented values by the e4m3 rounding of P; lse
 * (fp32 [batch, heads_q, seqlen_q], natural log) is the exact log-sum-exp up to fp32
 * rounding. Rows with no visible key get out = 0, lse = -inf. Descales must be finite
 * (EXATTN_ERR_SCALE otherwise); errors as for exattn_fwd.
 */
exattn_status exattn_fwd_fp8(const exattn_problem* p, const void* q, const void* k,
                             const void* v, float q_descale, float k_descale, float v_descale,
                             void* out, float* lse, void* stream);

/* Bytes of device workspace exattn_bwd needs for this problem (its bwd_variant included):
 * fp32 [lse * log2(e) | rowsum(dout * out)] per (row, head), an int32 ranking of the
 * packed sequences, for bwd_variant 1 the fp32 dQ accumulator, and for bwd_variant 3 the
 * stored dS (B * heads_q * ceil(seqlen_q / 64) * ceil(seqlen_k / 128) * 16 KiB, 8.6 GB at
 * B2 S8192 H32). The workspace is the
 * caller's memory, as every buffer is (NVIDIA cudnn-frontend PR #429, first commit
 * message: the caller owns the scratch the backward needs and its zero-fill is enqueued on
 * the launch stream). Returns 0 on invalid input. */
size_t exattn_bwd_workspace_size(const exattn_problem* p);

/*
 * Backward. q, k, v, out, dout: device inputs of the problem's dtype (strides in p); lse:
 * fp32 device input as written by exattn_fwd for the same problem (read only). dq, dk, dv:
 * device outputs of that dtype, contiguous, every element written. The fused variant
 * (bwd_variant 1) applies to bf16 only; fp16 problems always take the default split
 * backward. workspace: device memory of at least
 * exattn_bwd_workspace_size(p) bytes, 256-byte aligned, owned by the caller; its contents
 * on entry do not matter and on exit are unspecified. Concurrent calls must not share a
 * workspace. With the default backward variant every output (dq included) is bitwise
 * reproducible: each dq row is summed over keys in a fixed order by one workgroup. The
 * fused variant accumulates dq with fp32 atomics instead, so there dq may differ between
 * runs by re-association of fp32 sums, within the bound that PFCCLab cudnn-frontend PR #9
 * states in "How it was verified" (an fp32 atomic accumulation is not bitwise stable
 * against itself: cudnn-frontend PR #429, "API and compatibility impact").
 */
exattn_status exattn_bwd(const exattn_problem* p, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse, void* dq,
                         void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Backward without any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments and results as exattn_bwd, except that the workspace is a library-owned
 * device array of EXATTN_NOALLOC_MAX_WORKSPACE bytes per GPU (resolved on the first call
 * on each device, held until the process ends). The caller still passes every input and
 * output. Problems whose exattn_bwd_workspace_size exceeds that maximum are rejected with
 * EXATTN_ERR_WORKSPACE before anything is enqueued. Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams or threads) race on it
 * and must not be issued; consecutive calls on one stream are safe (each call rewrites
 * what it reads). The kernel timing of exattn_timing_enable does not cover this call.
 * The current device must be the stream's device.
 */
#define EXATTN_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
exattn_status exattn_bwd_noalloc(const exattn_problem* p, const void* q, const void* k,
                                 const void* v, const void* out, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, void* stream);

/* Static description of a status code. Rejections are reported as statuses instead of
 * being run or silently accepted (cudnn-frontend PR #429, "Validate the input contract":
 * an unsupported input fails loudly with a message). */
const char* exattn_status_string(exattn_status s);

/* Message of the last non-OK status returned on the calling thread ("" if none): which
 * argument was rejected and why (cudnn-frontend PR #429, "Validate the input contract"). */
const char* exattn_last_error(void);

/*
 * Kernel timing. While enabled, every kernel the library launches is bracketed by a pair
 * of HIP events recorded on the launch stream (at most 4096 pairs between reads).
 * exattn_timing_read waits for the recorded events, writes for up to `max` kernel names
 * the summed milliseconds and launch counts, clears the record and returns the number of
 * names written (or -1 on a HIP error). names[i] points to static strings.
 */
exattn_status exattn_timing_enable(int enable);
int exattn_timing_read(const char** names, double* total_ms, int* launches, int max);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
