/*
 * fd_decode.h -- C ABI of the split-KV decode-attention library (gfx950).
 *
 * The operation (slavadubrov.com, "What is Flash-Decoding, and when does it
 * speed up LLMs?", sections "What is Flash-Decoding" and "Why decode needs a
 * different schedule"): at each decode step a sequence adds a single query
 * position, and that query attends over every key / value the sequence has
 * cached so far. Flash-Decoding cuts the cached history into pieces that
 * separate workgroups process in parallel; every piece produces its own
 * partial result together with the log-sum-exp of its scores, and a final
 * reduction merges the pieces, renormalising them, so that the result is
 * exactly unsplit attention over the whole history. The
 * aiexpertsdirectory.org summary of the method (operational constraints)
 * notes that this reduction is a small extra cost that matters only for
 * very short histories, which the planner below accounts for.
 *
 * Per sequence b and query head h (kv head h / (Hq/Hkv)):
 *   s_i   = scale * <q[b,h,:], k_i>                  for i < seq_lens[b]
 *   out   = sum_i e^{s_i} v_i / sum_i e^{s_i}         (fp32)
 *   lse   = ln sum_i e^{s_i}                          (natural log, fp32)
 *   seq_lens[b] == 0 gives out = 0, lse = -inf.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is caller-owned. Device pointers are HIP device
 *     memory of the current device; host pointers are marked "host". The
 *     library allocates nothing and keeps no mutable global state; calls are
 *     reentrant and thread-safe.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream). Nothing is synchronised.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     failed check the call returns a negative fd_status, launches nothing
 *     and writes nothing. A launch failure reported by HIP returns
 *     FD_ERR_HIP.
 *   - Caller's contract, not checked: 0 <= seq_lens[b] <= max_seq_len;
 *     every block id a sequence reaches is in [0, num_blocks); outputs do
 *     not alias inputs. (Out-of-range lengths are clamped into
 *     [0, max_seq_len] and block ids into [0, num_blocks) on the device so a
 *     broken call cannot read outside the buffers, but its result is
 *     meaningless.)
 *   - Determinism: for fixed inputs, num_splits and device the result is
 *     bitwise reproducible (no atomics; every reduction runs in a fixed
 *     order). Only fd_decode_attn on 2 to 64 sequences consults the device:
 *     it sizes its length-aware pieces from the device's compute-unit
 *     count, so two devices with different counts may round differently.
 */
#ifndef FD_DECODE_H
#define FD_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
  FD_OK = 0,
  FD_ERR_INVALID_ARG = -1,  /* null pointer, bad shape, bad alignment */
  FD_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head_dim, dtype) */
  FD_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  FD_ERR_HIP = -4           /* HIP reported an error at launch */
} fd_status;

typedef enum fd_dtype {
  FD_DTYPE_F32 = 0,         /* q, k, v are IEEE float32 */
  FD_DTYPE_BF16 = 1,        /* q, k, v are bfloat16; math in fp32 */
  FD_DTYPE_FP8_E4M3 = 2,    /* q bfloat16; k, v 8-bit E4M3 codes (OCP 8-bit
                               float: sign, 4-bit exponent with bias 7,
                               3-bit mantissa, no infinities) with one fp32
                               scale per kv head for K and one for V; only
                               the *_fp8 entry points take it */
  FD_DTYPE_INT8 = 3         /* q bfloat16; k, v 8-bit two's-complement
                               integers with one fp32 scale per (position,
                               kv head) for K and one for V; only the *_int8
                               entry points take it */
} fd_dtype;

/*
 * Shape of one decode-attention call.
 *
 *   q            [batch, num_q_heads, head_dim]              (dtype)
 *   contiguous   k, v [batch, num_kv_heads, max_seq_len, head_dim]
 *   paged        k, v pools [num_blocks, num_kv_heads, block_size, head_dim];
 *                block_table int32 [batch, max_blocks_per_seq]; position i of
 *                sequence b is slot i % block_size of block
 *                block_table[b, i / block_size] (PagedAttention's block
 *                table, listed by title among the sources of the "Faster Than
 *                Flash" page). Entries past a sequence's last block are
 *                never read.
 *   out          fp32 [batch, num_q_heads, head_dim]; lse fp32 [batch, Hq]
 *
 * num_q_heads must be a multiple of num_kv_heads; query head h reads kv head
 * h / (num_q_heads / num_kv_heads) (grouped-query attention).
 */
typedef struct fd_shape {
  int32_t batch;               /* >= 1 */
  int32_t num_q_heads;         /* >= 1 */
  int32_t num_kv_heads;        /* >= 1, divides num_q_heads */
  int32_t head_dim;            /* 64 or 128 */
  int32_t max_seq_len;         /* L >= 0: bound on seq_lens[]; sets split size */
  int32_t block_size;          /* 0 = contiguous; else a multiple of 16, <= 4096 */
  int32_t max_blocks_per_seq;  /* paged: block_table row stride, >= ceil(L/bs) */
  int32_t num_blocks;          /* paged: blocks in each of the k and v pools */
  int32_t dtype;               /* fd_dtype */
  float scale;                 /* logit scale; <= 0 selects 1/sqrt(head_dim) */
} fd_shape;

/* Split sizing used by every call below: with S = num_splits and
 * L = max_seq_len, split s covers positions [s*P, (s+1)*P) of each sequence,
 * P = ceil(ceil(L / S) / g) * g where g = max(16, block_size). A sequence
 * shorter than s*P leaves split s empty; its partial is o = 0, lse = -inf. */

/*
 * Choose the number of splits for a call (host only, no device access).
 *
 * The pages give the regimes, not a rule: splitting helps when a small batch
 * offers too few independent blocks for a long history, while for a short
 * history or a batch that already fills the GPU the extra partials and the
 * reduction may cost more than they save (slavadubrov.com, "Why decode needs
 * a different schedule"; aiexpertsdirectory.org, operational constraints).
 * The rule here: with units = batch * num_kv_heads (times the groups of up
 * to 16 query heads), return 1 if units already cover num_cus, if L is
 * short, or if L is under 1024 and units cover half of num_cus (for an
 * 8-bit cache, 8 units); otherwise size splits so that the attended tokens
 * spread over about num_cus workgroups (twice that for an int8 cache with
 * 2 to 64 sequences, and for splits over 1024 tokens when sum_seq_len
 * shows a ragged batch), no split shorter than a minimum length.
 *
 *   shape        host pointer, validated as for fd_decode_attn
 *   num_cus      compute units of the device (hipDeviceProp_t
 *                multiProcessorCount), >= 1
 *   sum_seq_len  sum of seq_lens[] if the caller knows it, else -1 (then
 *                every sequence is taken to be max_seq_len long)
 *   num_splits   host out: the chosen S >= 1
 */
int fd_plan_splits(const fd_shape* shape, int num_cus, int64_t sum_seq_len,
                   int* num_splits);

/*
 * Bytes of device workspace fd_decode_attn needs for num_splits splits:
 * 0 when num_splits == 1, else room for the fp32 partials
 * o_part [batch, Hq, S, head_dim] and lse_part [batch, Hq, S] (natural log),
 * 256-byte aligned. These are the per-piece partial outputs and their
 * log-sum-exp values that the final reduction merges (slavadubrov.com,
 * "What is Flash-Decoding, and when does it speed up LLMs?", section "Why
 * decode needs a different schedule"). shape and bytes are host pointers;
 * shape is validated as for fd_decode_attn and num_splits must be in
 * [1, 65535] (FD_ERR_INVALID_ARG otherwise).
 */
int fd_workspace_size(const fd_shape* shape, int num_splits, size_t* bytes);

/*
 * Full decode attention, the operation of slavadubrov.com, "What is
 * Flash-Decoding, and when does it speed up LLMs?" (sections "What is
 * Flash-Decoding" and "Why decode needs a different schedule"): the split
 * kernel computes every split's partial output and log-sum-exp in
 * parallel, then (if num_splits > 1) the log-sum-exp combine kernel merges
 * them into exact attention over the whole history, both on `stream`. For 2
 * to 64 sequences and num_splits > 1 the split kernel cuts each sequence
 * into up to num_splits equal pieces sized by its own length instead of the
 * uniform splits above (an internal choice: the result is the same
 * attention; see Determinism above).
 *
 *   q, k_cache, v_cache  device, dtype per shape, 16-byte aligned
 *   block_table          device int32, non-NULL iff shape->block_size > 0
 *   seq_lens             device int32 [batch]
 *   num_splits           S >= 1 (e.g. from fd_plan_splits); S == 1 writes
 *                        `out` directly and needs no workspace
 *   workspace            device, >= fd_workspace_size bytes, 16-byte aligned
 *                        (ignored, may be NULL, when S == 1). Scratch only:
 *                        its contents on entry do not matter.
 *   out                  device fp32 [batch, Hq, head_dim], 16-byte aligned
 *   lse_out              device fp32 [batch, Hq] natural log, or NULL
 */
int fd_decode_attn(const fd_shape* shape, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_table,
                   const int32_t* seq_lens, int num_splits, void* workspace,
                   size_t workspace_bytes, float* out, float* lse_out,
                   void* stream);
/* (shape->dtype FD_DTYPE_FP8_E4M3 or FD_DTYPE_INT8 is rejected here with
 * FD_ERR_INVALID_ARG: such a cache needs its scales, fd_decode_attn_fp8 or
 * fd_decode_attn_int8.) */

/*
 * fd_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the partials go to a 4 MiB
 * array the library keeps on each device it runs on (from the first such
 * call on that device until the process ends). The call allocates nothing.
 *
 * Arguments, outputs and errors as for fd_decode_attn, plus
 * FD_ERR_WORKSPACE (nothing launched) when the call's workspace
 * (fd_workspace_size) would exceed 4 MiB (4194304 bytes), and FD_ERR_HIP if
 * the array's device address cannot be obtained. Every call on a device
 * shares that device's array: calls that overlap on one device (other
 * streams, other threads) race and give wrong results; serialise them.
 */
int fd_decode_attn_noalloc(const fd_shape* shape, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table,
                           const int32_t* seq_lens, int num_splits,
                           float* out, float* lse_out, void* stream);

/*
 * The split step alone: per split s, the partial output of attention over
 * that split's positions, normalised by its own softmax sum, and its
 * log-sum-exp (the per-piece result of slavadubrov.com, "Why decode needs a
 * different schedule"). Empty splits get o = 0, lse = -inf. These partials can be
 * combined with fd_combine_partials, also after gathering partials computed
 * over different shards of a history.
 *
 *   o_part    device fp32 [batch, Hq, num_splits, head_dim], 16-byte aligned
 *   lse_part  device fp32 [batch, Hq, num_splits], natural log
 * Other arguments as for fd_decode_attn.
 */
int fd_decode_partials(const fd_shape* shape, const void* q,
                       const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int num_splits, float* o_part, float* lse_part,
                       void* stream);

/*
 * Decode attention over an 8-bit float cache (shape->dtype must be
 * FD_DTYPE_FP8_E4M3): every key of kv head g is decode(code) * k_scale[g]
 * and every value decode(code) * v_scale[g], and the result is the
 * attention above over those dequantized values, in fp32 (the comparison
 * the slavadubrov.com page asks for holds the cache precision fixed,
 * section "Interpret the reported result"; the "Faster Than Flash" page's
 * abstract reads its cache in low-bit form). Half the bytes of a bf16 cache
 * per token, so about half the time on this memory-bound path.
 *
 *   q                 device bf16 [batch, Hq, head_dim], 16-byte aligned
 *   k_cache, v_cache  device uint8 codes, layouts as for fd_decode_attn
 *                     (one byte per element), 16-byte aligned
 *   k_scale, v_scale  device fp32 [num_kv_heads], 4-byte aligned
 * Other arguments, outputs and errors as for fd_decode_attn.
 */
int fd_decode_attn_fp8(const fd_shape* shape, const void* q,
                       const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int num_splits, void* workspace,
                       size_t workspace_bytes, float* out, float* lse_out,
                       void* stream);

/* The split step alone over an 8-bit float cache: as fd_decode_partials,
 * with the cache and scales of fd_decode_attn_fp8. */
int fd_decode_partials_fp8(const fd_shape* shape, const void* q,
                           const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table,
                           const int32_t* seq_lens, int num_splits,
                           float* o_part, float* lse_part, void* stream);

/*
 * Decode attention over an 8-bit integer cache (shape->dtype must be
 * FD_DTYPE_INT8) with one scale per cached position and kv head: the key
 * at position i of sequence b, kv head g is code * k_scale[.., i], the
 * value code * v_scale[.., i], and the result is the attention above over
 * those dequantized values, in fp32. As for fd_decode_attn_fp8, the cache
 * precision is an input that the comparison holds fixed (slavadubrov.com,
 * "What is Flash-Decoding", section "Interpret the reported result"), and
 * the cache is read in a low-bit form (the "Faster Than Flash" page,
 * abstract); here the scale is per position. Per position this reads
 * 2 * head_dim code bytes and 8 scale bytes per kv head.
 *
 *   q                 device bf16 [batch, Hq, head_dim], 16-byte aligned
 *   k_cache, v_cache  device int8 codes (two's complement), layouts as for
 *                     fd_decode_attn (one byte per element), 16-byte
 *                     aligned
 *   k_scale, v_scale  device fp32, 16-byte aligned, one row of scales per
 *                     (sequence or block, kv head) in whole 16-position
 *                     groups: contiguous [batch, Hkv, Lp] with
 *                     Lp = ceil(max_seq_len / 16) * 16 (position i of
 *                     sequence b at [b, g, i]); paged [num_blocks, Hkv,
 *                     block_size] (position i at [block_table[b, i / bs],
 *                     g, i % bs]). Only the scales of attended positions
 *                     are used; the others (the row padding included) may
 *                     hold anything, NaN included, but must be allocated.
 * Other arguments, outputs and errors as for fd_decode_attn.
 */
int fd_decode_attn_int8(const fd_shape* shape, const void* q,
                        const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int num_splits, void* workspace,
                        size_t workspace_bytes, float* out, float* lse_out,
                        void* stream);

/* The split step alone over an 8-bit integer cache: as fd_decode_partials,
 * with the cache and scales of fd_decode_attn_int8. */
int fd_decode_partials_int8(const fd_shape* shape, const void* q,
                            const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table,
                            const int32_t* seq_lens, int num_splits,
                            float* o_part, float* lse_part, void* stream);

/*
 * Block-sparse decode ("Faster Than Flash: Exploiting Attention Sparsity
 * for Efficient Long-Context Decoding", abstract): a 4-bit copy of the keys
 * is scanned to estimate each 16-token block's best logit, a top-delta rule
 * keeps the blocks that matter, and exact attention runs over those only.
 * The page defines neither the quantizer nor the rule; the readings here:
 *
 * Key summary (fd_build_key_summary), per 16-token block and kv head, over
 * the block's attended rows: amax = max |k| (all dims); inv = 7 / amax and
 * scale = amax / 7, each one correctly rounded fp32 operation (0 when
 * amax = 0); code = rint(k * inv) (fp32 product, ties to even), in [-7, 7],
 * stored as 4-bit two's complement, dim 2m in the low nibble of byte m of
 * the row's head_dim / 2 bytes. Rows past a sequence's length get code 0.
 * Each block's 16 rows form one record of 8 * head_dim bytes in which row n's
 * piece p (its bytes p * head_dim/8 .. (p+1) * head_dim/8 - 1, p = 0..3)
 * sits at byte offset head_dim/8 * (n + 16 p): the order in which the scan
 * reads them, one contiguous request per wave.
 *
 *   codes   device uint8 records, one per (16-token block, kv head):
 *           contiguous [batch, Hkv, ceil(max_seq_len/16), 8 * head_dim],
 *           paged [num_blocks, Hkv, block_size/16, 8 * head_dim] (the same
 *           bytes as a [.., block_size, head_dim/2] pool); 16-byte aligned
 *   scales  device fp32: contiguous [batch, Hkv, ceil(max_seq_len/16)];
 *           paged [num_blocks, Hkv, block_size/16]; 4-byte aligned
 * Only blocks holding at least one attended token are written. bf16 keys
 * only (shape->dtype FD_DTYPE_BF16); k_cache / block_table / seq_lens as
 * for fd_decode_attn.
 */
int fd_build_key_summary(const fd_shape* shape, const void* k_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         void* codes, float* scales, void* stream);

/*
 * Sparse decode over the summary: in split s of sequence b and kv head g,
 * with est[j, h] = scale_attn * scales[j] * max over block j's attended
 * tokens of <q[b,h], codes>, block j is kept when
 * est[j, h] >= max_j' est[j', h] - delta for some query head h of g (the
 * maximum taken over the split's blocks only: no workgroup waits on
 * another). The result is exact attention over every kept block's tokens;
 * delta = +INFINITY keeps every block (the dense result up to rounding).
 *
 *   delta      >= 0, natural-log units (not NaN)
 *   num_splits as for fd_decode_attn, with at most 8192 tokens per split
 *              and tokens per split x max(16, Hq / Hkv) <= 131072 (the
 *              block estimates of a split live in on-chip memory);
 *              FD_ERR_UNSUPPORTED otherwise
 *   kept_out   device uint8 [batch, Hkv, ceil(max_seq_len/16)] receiving
 *              1 (kept) / 0 for every block holding an attended token
 *              (other entries untouched), or NULL
 * Supported: bf16 (shape->dtype FD_DTYPE_BF16), head_dim 64 / 128, at most
 * 128 query heads per kv head. Other arguments as for fd_decode_attn.
 */
int fd_decode_attn_sparse(const fd_shape* shape, const void* q,
                          const void* k_cache, const void* v_cache,
                          const void* codes, const float* scales,
                          const int32_t* block_table,
                          const int32_t* seq_lens, float delta,
                          int num_splits, void* workspace,
                          size_t workspace_bytes, float* out, float* lse_out,
                          uint8_t* kept_out, void* stream);

/*
 * The same two block-sparse calls over an 8-bit float cache
 * (shape->dtype FD_DTYPE_FP8_E4M3, codes and scales as for
 * fd_decode_attn_fp8): the summary quantizes every attended key element as
 * the fp32 product decode(code) * k_scale[g] (one rounding; g its kv head),
 * otherwise exactly as fd_build_key_summary; the estimates, the top-delta
 * rule and the result are those of fd_decode_attn_sparse, with exact
 * attention over the dequantized cache (keys decode(code) * k_scale[g],
 * values decode(code) * v_scale[g]). The "Faster Than Flash" abstract
 * scans a low-bit copy of the keys; here the cache itself is low-bit too,
 * its precision held fixed as slavadubrov.com, "Interpret the reported
 * result", asks of comparisons.
 *
 *   k_scale, v_scale  device fp32 [Hkv], 4-byte aligned
 * Other arguments, limits and layouts as for the bf16 calls. A shape of
 * another dtype, or a missing or misaligned scale, is FD_ERR_INVALID_ARG
 * (and an E4M3 shape passed to the bf16 calls is FD_ERR_UNSUPPORTED).
 */
int fd_build_key_summary_fp8(const fd_shape* shape, const void* k_cache,
                             const float* k_scale, const int32_t* block_table,
                             const int32_t* seq_lens, void* codes,
                             float* scales, void* stream);
int fd_decode_attn_sparse_fp8(const fd_shape* shape, const void* q,
                              const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const void* codes, const float* scales,
                              const int32_t* block_table,
                              const int32_t* seq_lens, float delta,
                              int num_splits, void* workspace,
                              size_t workspace_bytes, float* out,
                              float* lse_out, uint8_t* kept_out,
                              void* stream);

/*
 * The same two block-sparse calls over an int8 cache with one fp32 scale
 * per (position, kv head) (shape->dtype FD_DTYPE_INT8; codes and scales
 * laid out as for fd_decode_attn_int8): the summary quantizes every
 * attended key element as the fp32 product code * k_scale[position] (one
 * rounding), and the result is exact attention over the dequantized cache
 * (keys code * k_scale, values code * v_scale, per position), otherwise as
 * fd_decode_attn_sparse.
 *
 *   k_scale, v_scale  device fp32, contiguous [batch, Hkv, Lp] with
 *                     Lp = ceil(max_seq_len / 16) * 16, paged
 *                     [num_blocks, Hkv, block_size]; 16-byte aligned for
 *                     the sparse call, 4-byte for the summary
 * Other arguments, limits and layouts as for the bf16 calls; errors as for
 * the E4M3 calls.
 */
int fd_build_key_summary_int8(const fd_shape* shape, const void* k_cache,
                              const float* k_scale,
                              const int32_t* block_table,
                              const int32_t* seq_lens, void* codes,
                              float* scales, void* stream);
int fd_decode_attn_sparse_int8(const fd_shape* shape, const void* q,
                               const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const void* codes, const float* scales,
                               const int32_t* block_table,
                               const int32_t* seq_lens, float delta,
                               int num_splits, void* workspace,
                               size_t workspace_bytes, float* out,
                               float* lse_out, uint8_t* kept_out,
                               void* stream);

/*
 * The reduction step alone: for each (b, h), with M = max_s lse_part[b,h,s],
 *   out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M},
 *   lse = M + ln sum_s e^{lse_s - M};
 * splits with lse = -inf contribute nothing; if all are -inf, out = 0 and
 * lse = -inf. (The merging step of slavadubrov.com, same section: it
 * turns the pieces back into the full-history result.)
 *
 *   batch, num_q_heads, head_dim (64 or 128), num_splits >= 1
 *   o_part, lse_part  device fp32, layouts as for fd_decode_partials
 *   out               device fp32 [batch, Hq, head_dim], 16-byte aligned
 *   lse_out           device fp32 [batch, Hq], or NULL
 */
int fd_combine_partials(int batch, int num_q_heads, int head_dim,
                        int num_splits, const float* o_part,
                        const float* lse_part, float* out, float* lse_out,
                        void* stream);

/* Static description of an fd_status value (never NULL). */
const char* fd_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_DECODE_H */
