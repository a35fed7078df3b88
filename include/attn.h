/*
 * dense_attention_amd — fused dense attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ or framework types cross it.
 *
 * Operation (the plain definition of softmax attention; "B200 Attention Kernel
 * from Scratch to Near-SOTA in 60 Diagrams", Chapter 1, "ii. Work
 * Parallelization" gives the Q·Kᵀ -> online softmax -> P·V loop and the final
 * division by the row sum; "Attention for sm90, Line by Line", "Why does the
 * kernel use exp2 rather than exp?" gives the natural-log residual):
 *
 *     o[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:]·k[b,h,j,:]) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(scale * q[b,h,i,:]·k[b,h,j,:])
 *
 * attn_fwd: no mask or bias, the same sequence length S for queries and keys.
 * attn_fwd_ex adds an optional causal mask (then the sums above run over the
 * keys a row may see), attn_fwd_strided other layouts and key lengths, and
 * attn_fwd_partial / attn_merge / attn_fwd_split key ranges.  Computed tile by
 * tile with an online softmax so the S×S score matrix never reaches device
 * memory; fp32 accumulation; O is rounded to the input dtype with
 * round-to-nearest-even, LSE is stored in fp32.
 *
 * Layout (attn_fwd, attn_fwd_ex, attn_fwd_split): q, k, v, o are contiguous
 * row-major [B, H, S, D] arrays of the same dtype (D fastest, then S, then H,
 * then B).  lse is a contiguous [B, H, S] fp32 array.  All pointers are DEVICE
 * pointers on the current HIP device.
 *
 * Ownership: the caller owns every buffer (the split-KV workspace included)
 * and the stream.  The library never allocates, frees or synchronises, and
 * keeps no pointer past the call.  Work is enqueued asynchronously on `stream`
 * (a hipStream_t; NULL means the default stream).
 *
 * Errors: every entry point returns ATTN_OK (0) or a negative attn_status.
 * Arguments are validated before anything is launched; on an error nothing is
 * enqueued.  Device faults during execution surface at the caller's next
 * synchronisation of the stream, not here.  Entry points are thread-safe.
 */
#ifndef DENSE_ATTENTION_AMD_ATTN_H
#define DENSE_ATTENTION_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
enum attn_dtype {
  ATTN_F16 = 0,  /* IEEE binary16 */
  ATTN_BF16 = 1, /* bfloat16 */
  ATTN_F32 = 2   /* IEEE binary32: only as the output type of attn_merge */
};

/* Return codes. */
enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,    /* q, k, v or o is NULL for a non-empty problem */
  ATTN_ERR_DTYPE = -2,   /* dtype is not an attn_dtype */
  ATTN_ERR_SHAPE = -3,   /* negative size, unsupported D, or a size whose offsets overflow */
  ATTN_ERR_ALIGN = -4,   /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_ERR_SCALE = -5,   /* scale is NaN or infinite */
  ATTN_ERR_DEVICE = -6,  /* no current HIP device, or it is not a gfx950 GPU */
  ATTN_ERR_LAUNCH = -7,  /* the kernel launch failed (attn_last_error() has the HIP text) */
  ATTN_ERR_ARG = -8,     /* an option is out of range */
  ATTN_ERR_SCRATCH = -9  /* attn_fwd_split_noalloc: the partials exceed the static scratch */
};

/*
 * attn_fwd — O = softmax(scale·Q·Kᵀ)·V and LSE over [B, H, S, D].
 *
 *   q, k, v  device pointers to B·H·S·D elements of `dtype`, read only.
 *   o        device pointer to B·H·S·D elements of `dtype`, written.  May not
 *            alias q, k or v.
 *   lse      device pointer to B·H·S floats, written; NULL skips the LSE.
 *   B, H, S  batch, heads, sequence length, each >= 0.  Any S >= 1 is
 *            accepted (no tile-multiple requirement).  B·H·S == 0 is an empty
 *            problem: ATTN_OK, nothing is launched, pointers may be NULL.
 *   D        head dimension: 64 or 128.
 *   scale    finite multiplier of the scores (commonly 1/sqrt(D)); 0 gives
 *            uniform attention, negative values are allowed.
 *   dtype    ATTN_F16 or ATTN_BF16.
 *   stream   hipStream_t to enqueue on (NULL = default stream).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, float scale, int dtype, void* stream);

/* Tuning and testing knobs for attn_fwd_ex.  Zero-initialise, then set fields. */
typedef struct attn_fwd_options {
  /* Lazy O-rescale threshold in log2 units: a row's running maximum is moved
   * only when a tile's maximum exceeds it by more than this, otherwise the
   * exponent absorbs the difference (P <= 2^threshold).  0 rescales whenever
   * the maximum grows (the textbook update).  Negative selects the default, 8.
   * Must be <= 64 for ATTN_BF16 and <= 15 for ATTN_F16, else ATTN_ERR_ARG: P
   * is rounded to the input type before P·V, and a kept maximum lets p reach
   * 2^threshold, which must stay finite in that type (fp16 ends at 65504 <
   * 2^16; bf16 and the fp32 sums hold 2^64 times any row's length).  ("B200
   * Attention Kernel from Scratch to Near-SOTA in 60 Diagrams", Chapter 11 -
   * Skip O rescale: skipping is allowed while no intermediate value
   * overflows; "Attention for sm90, Line by Line", "What is rescale_threshold
   * and when does it help?") */
  float rescale_threshold;
  /* Kernel tile variant, 0 = the library's choice; otherwise an id listed by
   * attn_variant_info().  A variant must support D and dtype. */
  int variant;
  /* Persistent grid size in workgroups, 0 = the library's choice (all CUs at
   * full occupancy, capped at the number of work items; with a causal mask,
   * one workgroup per work item, the longest first). */
  int grid;
  /* Causal mask.  0: none.  1: query row i (0-based) attends to keys
   * j <= i + (Skv - Sq), i.e. the last query row sees every key (equal
   * lengths: j <= i).  2: query row i attends to keys j <= i + causal_offset
   * (for a shard of keys or queries cut out of a longer sequence).  A query
   * row that sees no key gets O = 0 and LSE = -inf.  ("Attention for sm90,
   * Line by Line", "What does the persistent flag do in the sm90 attention
   * config?": the mask makes the work per query tile vary widely, which a
   * static persistent schedule balances badly.) */
  int causal;
  int causal_offset;  /* used when causal == 2 */
  int reserved[2];    /* must be zero */
} attn_fwd_options_t;

/* attn_fwd with options; opts == NULL behaves exactly like attn_fwd. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, float scale, int dtype, void* stream,
                const attn_fwd_options_t* opts);

/* Launch configuration the library would use (for reporting and benchmarks). */
typedef struct attn_config {
  int variant;            /* tile variant id (see attn_variant_info) */
  int block_m;            /* query rows per work item */
  int block_n;            /* keys per K/V tile */
  int waves;              /* 64-lane waves per workgroup */
  int stages;             /* K/V ring depth in LDS */
  int lds_bytes;          /* LDS per workgroup */
  int work_items;         /* B·H·ceil(S/block_m) */
  int grid;               /* workgroups launched (persistent) */
  int workgroups_per_cu;  /* occupancy the grid was sized for */
  int num_cus;            /* compute units on the device */
} attn_config_t;

/* Fills *out for the current device; opts as in attn_fwd_ex (may be NULL).
 * Performs the same validation as attn_fwd_ex except for the data pointers. */
int attn_get_config(int B, int H, int S, int D, int dtype,
                    const attn_fwd_options_t* opts, attn_config_t* out);

/* Describes tile variant `index` (0-based, in [0, attn_variant_count())):
 * writes its id, head dim, dtype, block_m, block_n, waves, stages,
 * key_split (1: the workgroup's two groups of waves hold the same block_m
 * query rows and each streams half of the keys, merging at the end; 0: every
 * wave holds its own rows of one shared key stream) and soft_exp (0: every
 * exponential on the transcendental unit; k > 0: one score in k takes 2^x
 * from a cubic polynomial on the vector ALU, the selective software exp2 of
 * "B200 Attention Kernel from Scratch to Near-SOTA in 60 Diagrams",
 * Chapter 9; such variants are never the library's default).  Any output
 * pointer may be NULL.  Host-only; touches no device. */
int attn_variant_count(void);
int attn_variant_info(int index, int* id, int* head_dim, int* dtype, int* block_m,
                      int* block_n, int* waves, int* stages, int* key_split, int* soft_exp);

/* ---- general layouts, KV ranges and split-KV --------------------------------- */

/* Element strides of a [B, H, S, D] view whose head dimension is contiguous
 * (stride 1).  Contiguous BHSD is {H·S·D, S·D, D}; contiguous BSHD (tokens
 * outermost, heads interleaved per token) is {S·H·D, D, H·D}.  A slice of keys
 * [a, b) of a BHSD tensor is the same strides with the base pointer advanced by
 * a·D.  Every stride must be >= 0 and a multiple of 8 elements (16 bytes), and
 * seq_stride < 2^24. */
typedef struct attn_layout {
  int64_t batch_stride;
  int64_t head_stride;
  int64_t seq_stride;
} attn_layout_t;

/*
 * attn_fwd_strided — attn_fwd over arbitrary strided views and separate query
 * and key lengths: o[b,h,i,:] = Σ_j softmax_j(scale·q_i·k_j)·v_j over the Skv
 * keys of head (b, h), for each of its Sq queries (B200 page, Appendix,
 * "Benchmark Calibration": a variant that consumes and produces contiguous
 * BSHD directly, with no layout-conversion copies).
 *
 *   q_layout, k_layout, v_layout, o_layout  strides of each tensor; NULL means
 *            contiguous [B, H, S, D] for that tensor (S = Sq for q and o, Skv
 *            for k and v).  o must not overlap itself or the inputs.
 *   lse      contiguous [B, H, Sq] fp32, or NULL.
 *   Sq, Skv  >= 0; Sq·Skv == 0 with B·H > 0 and Sq > 0 is rejected (a query
 *            with no keys has no softmax); B·H·Sq == 0 is an empty problem.
 * Other arguments and errors as attn_fwd_ex.
 */
int attn_fwd_strided(const void* q, const attn_layout_t* q_layout,
                     const void* k, const attn_layout_t* k_layout,
                     const void* v, const attn_layout_t* v_layout,
                     void* o, const attn_layout_t* o_layout, float* lse,
                     int B, int H, int Sq, int Skv, int D, float scale, int dtype, void* stream,
                     const attn_fwd_options_t* opts);

/*
 * attn_fwd_partial — attention of Sq queries over one range of Skv keys (for
 * example one device's shard of the sequence), as the carrier the ranges
 * merge with ("Learning FlashAttention the Hard Way - Part 2", "Wrap-Up": the
 * running (max, sum, output) triple is associative, which is what licenses
 * streaming or splitting the KV axis; its references name split-KV):
 *
 *   o_part[b,h,i,:]  = Σ_{j in range} e^{s_ij - lse_part[b,h,i]} v_j   (fp32)
 *   lse_part[b,h,i]  = ln Σ_{j in range} e^{s_ij},   s_ij = scale·q_i·k_j
 *
 *   o_part    device pointer, contiguous [B, H, Sq, D] fp32, 16-byte aligned.
 *   lse_part  device pointer, contiguous [B, H, Sq] fp32; required.
 * Inputs, layouts and errors as attn_fwd_strided; Skv >= 1.
 */
int attn_fwd_partial(const void* q, const attn_layout_t* q_layout,
                     const void* k, const attn_layout_t* k_layout,
                     const void* v, const attn_layout_t* v_layout,
                     float* o_part, float* lse_part,
                     int B, int H, int Sq, int Skv, int D, float scale, int dtype, void* stream,
                     const attn_fwd_options_t* opts);

/*
 * attn_merge — combines n_parts partials of disjoint key ranges of the same
 * queries into the attention over their union:
 *
 *   lse = ln Σ_g e^{lse_g},   o = Σ_g e^{lse_g - lse} · o_g
 *
 * (the combine step of the same page's "The Move Stack": partial reductions
 * of separate workgroups joined by a separate kernel).
 *
 *   o_parts    n_parts consecutive contiguous [B, H, S, D] fp32 arrays.
 *   lse_parts  n_parts consecutive contiguous [B, H, S] fp32 arrays.  A
 *              partial with lse = -inf (no keys) has weight 0; a row whose
 *              partials are all -inf gets o = 0 and lse = -inf.
 *   o          output of `dtype` (ATTN_F16, ATTN_BF16, or ATTN_F32 for an
 *              fp32 result that can itself be merged again), strides o_layout
 *              (NULL = contiguous), 16-byte aligned.
 *   lse        contiguous [B, H, S] fp32, or NULL.
 *   n_parts    >= 1.
 */
int attn_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o,
               const attn_layout_t* o_layout, float* lse, int B, int H, int S, int D, int dtype,
               void* stream);

/*
 * attn_fwd_split — attn_fwd with the keys of every (b, h, query tile) split
 * into `kv_splits` ranges processed by separate workgroups, then merged: more
 * independent work items when B·H·ceil(S/block_m) would leave compute units
 * idle.  One launch computes all partials into `workspace`, a second merges
 * them into o and lse.  ("Learning FlashAttention the Hard Way - Part 2",
 * "Wrap-Up": the running (max, sum, output) carrier of a key range is
 * associative, which is what licenses splitting the key axis across
 * workgroups; its References name split-KV as the split-K of that carrier.)
 *
 *   kv_splits        >= 1, or 0 for the library's choice: no split unless the
 *                    items would fill at most half of the compute units,
 *                    then up to one item per compute unit with ranges of at
 *                    least 1024 keys (4096 where more than a quarter of the
 *                    units would already be busy).
 *   workspace        device memory of at least
 *                    attn_fwd_split_workspace_size(B, H, S, D, kv_splits)
 *                    bytes, 256-byte aligned, owned by the caller; its
 *                    contents on entry do not matter and on return are
 *                    unspecified.  Calls that share a workspace must be
 *                    ordered on one stream.
 * Other arguments as attn_fwd_ex.
 */
size_t attn_fwd_split_workspace_size(int B, int H, int S, int D, int kv_splits);
int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int S, int D, float scale, int dtype, void* stream, int kv_splits,
                   void* workspace, size_t workspace_bytes, const attn_fwd_options_t* opts);

/*
 * attn_fwd_split_noalloc — attn_fwd_split for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The fp32 partials of the
 * key ranges go to a static device array of ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends; the call
 * itself allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine).
 *
 *   kv_splits  as attn_fwd_split.  A problem whose partials,
 *              attn_fwd_split_workspace_size(B, H, S, D, n) bytes for the n
 *              ranges used, exceed ATTN_NOALLOC_SCRATCH_BYTES is refused with
 *              ATTN_ERR_SCRATCH and nothing is launched (with kv_splits > 0
 *              before any device query).  With a single range no scratch is
 *              used.
 *
 * Every call on one device shares that device's scratch: calls that may
 * overlap on a device (different streams, threads) race and must be ordered
 * by the caller, e.g. on one stream.  The scratch holds the last call's
 * partials afterwards; nothing in it has to be cleared between calls.  Other
 * arguments and errors as attn_fwd_split.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int S, int D, float scale, int dtype, void* stream,
                           int kv_splits, const attn_fwd_options_t* opts);

/* Static description of a status code.  Never NULL. */
const char* attn_strerror(int status);

/* Detail of the last error returned on the calling thread (e.g. the HIP error
 * string of a failed launch); "" when there is none.  Never NULL. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_ATTENTION_AMD_ATTN_H */
