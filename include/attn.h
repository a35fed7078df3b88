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
 * non-causal, no mask or bias, the same sequence length S for queries and keys.
 * Computed tile by tile with an online softmax so the S×S score matrix never
 * reaches device memory; fp32 accumulation; O is rounded to the input dtype
 * with round-to-nearest-even, LSE is stored in fp32.
 *
 * Layout: q, k, v, o are contiguous row-major [B, H, S, D] arrays of the same
 * dtype (D fastest, then S, then H, then B).  lse is a contiguous [B, H, S]
 * fp32 array.  All pointers are DEVICE pointers on the current HIP device.
 *
 * Ownership: the caller owns every buffer and the stream.  The library never
 * allocates, frees or synchronises, and keeps no pointer past the call.  Work
 * is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 * default stream).
 *
 * Errors: every entry point returns ATTN_OK (0) or a negative attn_status.
 * Arguments are validated before anything is launched; on an error nothing is
 * enqueued.  Device faults during execution surface at the caller's next
 * synchronisation of the stream, not here.  Entry points are thread-safe.
 */
#ifndef DENSE_ATTENTION_AMD_ATTN_H
#define DENSE_ATTENTION_AMD_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
enum attn_dtype {
  ATTN_F16 = 0,  /* IEEE binary16 */
  ATTN_BF16 = 1  /* bfloat16 */
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
  ATTN_ERR_ARG = -8      /* an option is out of range */
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
   * Must be <= 64.  ("B200 Attention Kernel from Scratch to Near-SOTA in 60
   * Diagrams", Chapter 11 - Skip O rescale; "Attention for sm90, Line by Line",
   * "What is rescale_threshold and when does it help?") */
  float rescale_threshold;
  /* Kernel tile variant, 0 = the library's choice; otherwise an id listed by
   * attn_variant_info().  A variant must support D and dtype. */
  int variant;
  /* Persistent grid size in workgroups, 0 = the library's choice (all CUs at
   * full occupancy, capped at the number of work items). */
  int grid;
  int reserved[4];  /* must be zero */
} attn_fwd_options_t;

/* attn_fwd with options; opts == NULL behaves exactly like attn_fwd. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, float scale, int dtype, void* stream,
                const attn_fwd_options_t* opts);

/* Launch configuration the library would use (for reporting and benchmarks). */
typedef struct attn_config {
  int variant;            /* tile variant id */
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
 * writes its id, head dim, dtype, block_m, block_n, waves and stages.
 * Host-only; touches no device. */
int attn_variant_count(void);
int attn_variant_info(int index, int* id, int* head_dim, int* dtype, int* block_m,
                      int* block_n, int* waves, int* stages);

/* Static description of a status code.  Never NULL. */
const char* attn_strerror(int status);

/* Detail of the last error returned on the calling thread (e.g. the HIP error
 * string of a failed launch); "" when there is none.  Never NULL. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_ATTENTION_AMD_ATTN_H */
