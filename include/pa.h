/*
 * pa.h: C ABI of the paged-KV-cache hot path for AMD Instinct MI355X (gfx950).
 *
 * The library computes two things. First, attention over a KV cache stored in
 * fixed-size, non-contiguous physical blocks, addressed through a per-request
 * block table. Second, the reshape_and_cache write that scatters new K/V rows
 * into those blocks through slot_mapping.
 *
 * Sources, cited by page title and section:
 *   [MEM]    "deep dive into vLLM 05: KV cache memory core" (arganzheng.life)
 *   [LAYOUT] "vLLM KV Cache Layout 可视化" (riverclouds.net)
 *   [MGMT]   "KV Cache 与推理服务内存管理" (pinghaoyang.com.cn)
 *   [INSIDE] "vLLM 技术内幕——像操作系统管理内存一样管理 KV 缓存" (openeuler.csdn.net)
 *
 * Conventions shared by every entry point:
 *   - Ownership: every pointer argument is caller-owned memory. "Device" means
 *     memory the GPU can read (hipMalloc / torch CUDA tensors); descriptors are
 *     host memory. The library allocates nothing and may be called from several
 *     host threads. Between calls it keeps, per device, only the CU count (read
 *     once) and the address of pa_decode_no_alloc's scratch, a static device
 *     array of the library.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream). Work is enqueued asynchronously; no call synchronises or reads
 *     device memory on the host.
 *   - Errors: arguments the host can check (null pointers, sizes, formats,
 *     alignment, view extents against the stated allocation size, workspace
 *     size) are validated before anything is enqueued. A failed check returns
 *     a non-zero pa_status and enqueues nothing. A failed launch returns
 *     PA_ERR_HIP; pa_last_hip_error() gives the HIP error code.
 *   - Device-side values (slots, block ids, context lengths) cannot be checked
 *     on the host. The kernels bound them instead, so that a bad value never
 *     leads to an access outside the cache:
 *       * a slot outside [0, num_blocks*block_size) is skipped;
 *       * a block-table entry outside [0, num_blocks) contributes no tokens;
 *       * a context length is clamped to
 *         [0, min(max_context_len, bt_stride*block_size)].
 *     Results for such inputs are unspecified but memory-safe.
 *   - Byte order is little-endian throughout.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 4

/* Size of the static device scratch array behind pa_decode_no_alloc (bytes, per GPU). */
#define PA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
    PA_ERR_INVALID_ARGUMENT = 2,  /* negative count, inconsistent sizes, reserved field not 0 */
    PA_ERR_UNSUPPORTED = 3,       /* format, head size, head ratio or block size not implemented */
    PA_ERR_MISALIGNED = 4,        /* a pointer, stride or row width breaks the stated alignment */
    PA_ERR_VIEW_OUT_OF_RANGE = 5, /* a cache view's rows reach past the stated allocation size */
    PA_ERR_WORKSPACE = 6,         /* workspace NULL or smaller than the *_workspace_bytes query */
    PA_ERR_HIP = 7,               /* a HIP launch failed; see pa_last_hip_error() */
    PA_ERR_SCRATCH_LIMIT = 8      /* pa_decode_no_alloc: the call needs more than
                                     PA_STATIC_SCRATCH_BYTES of scratch */
} pa_status;

/* KV storage formats.
 *   PA_KV_F16, PA_KV_BF16: dense rows. One token's row holds num_kv_heads
 *     heads of head_dim 16-bit values, head-major ([num_kv_heads, head_dim]),
 *     so a per-layer cache has the [num_blocks, block_size, num_kv_heads,
 *     head_dim] shape given in [MEM] §1.2. Queries and outputs use the same
 *     16-bit type.
 *   PA_KV_MLA656_E4M3: the 656-byte MLA row of [LAYOUT] (section on two caches
 *     sharing one block table). Bytes [0,512) hold 512 OCP e4m3 latent values.
 *     Bytes [512,528) hold 4 float32 scales; scale k multiplies latent values
 *     [128k, 128k+128). Bytes [528,656) hold 64 bf16 RoPE values. Queries are
 *     bf16 [.., num_q_heads, 576] (512 latent dims, then 64 RoPE dims).
 *     Outputs are bf16 [.., num_q_heads, 512]: the softmax-weighted
 *     dequantized latent ([MEM] §3.3: attention stays in latent space).
 *   PA_KV_FP8_E4M3: dense rows as for PA_KV_BF16, one OCP e4m3 byte per value
 *     ([MEM] §3.4: quantize on write, dequantize on read, FP8 the safest
 *     format). Every K value is its code times pa_attn_desc.k_scale and every V
 *     value its code times v_scale (one float32 scale per cache). Queries and
 *     outputs are bf16. Written by pa_quantize_and_cache.
 */
typedef enum pa_kv_format {
    PA_KV_F16 = 0,
    PA_KV_BF16 = 1,
    PA_KV_MLA656_E4M3 = 2,
    PA_KV_FP8_E4M3 = 3
} pa_kv_format;

/* One view over a flat cache allocation: the KVCacheTensor parameters of
 * [LAYOUT] (section "block ID 只是个编号") plus the row width. The row of
 * (layer, block b, position pos) starts at
 *     base + offset + layer*layer_stride + b*block_stride + pos*row_bytes.
 * Layer-outer layouts have block_stride = page and
 * layer_stride = page*num_blocks. Block-outer layouts have
 * layer_stride = page and block_stride = the bytes of a whole block
 * ([LAYOUT], layout section). All fields are byte counts >= 0. */
typedef struct pa_cache_view {
    int64_t offset;
    int64_t layer_stride;
    int64_t block_stride;
    int32_t row_bytes;
    int32_t reserved;             /* must be 0 */
} pa_cache_view;

/* Static description of an attention call's cache and heads (host memory). */
typedef struct pa_attn_desc {
    int32_t kv_format;            /* pa_kv_format */
    int32_t num_q_heads;          /* query heads */
    int32_t num_kv_heads;         /* K/V heads; num_q_heads % num_kv_heads == 0. Query head h reads
                                     K/V head h / (num_q_heads/num_kv_heads) ([MEM] §3.2). Dense:
                                     group size 1..16 at head_dim 128, else 1, 2, 4 or 8. MLA: 1 */
    int32_t qk_dim;               /* dense: head_dim (64, 128 or 256). MLA: 576 */
    int32_t v_dim;                /* dense: == qk_dim. MLA: 512 */
    int32_t block_size;           /* tokens per block: a power of two from 16 to 256 */
    int32_t layer;                /* layer index applied to the views' layer_stride */
    int32_t partition_size;       /* decode only: tokens per split-context partition, a positive
                                     multiple of block_size (at most 64 blocks are used); 0 lets the
                                     library choose from the item count estimate
                                     num_kv_heads*num_seqs*ceil(max_context_len/P): 1024 tokens if
                                     it reaches 8192, else the largest of 768, 512 reaching 2048,
                                     else 256 (whole blocks). For the MLA format: tokens per
                                     work-group range, a multiple of 32 */
    int64_t num_blocks;           /* physical blocks addressable through the views */
    pa_cache_view k_view;         /* K rows (MLA: the 656-byte rows) */
    pa_cache_view v_view;         /* V rows (dense only; ignored for MLA) */
    int64_t k_cache_bytes;        /* size of the allocation at k_cache, for the extent check */
    int64_t v_cache_bytes;        /* size of the allocation at v_cache (dense only) */
    float k_scale;                /* PA_KV_FP8_E4M3 only: K value = code * k_scale (finite, > 0) */
    float v_scale;                /* PA_KV_FP8_E4M3 only: V value = code * v_scale (finite, > 0) */
} pa_attn_desc;

/* ABI version of the loaded library (PA_ABI_VERSION). */
int32_t pa_abi_version(void);

/* Static, human-readable name of a status code. */
const char* pa_status_string(int32_t status);

/* HIP error code (hipError_t) of the last PA_ERR_HIP on the calling host thread, else 0. */
int32_t pa_last_hip_error(void);

/* reshape_and_cache: scatter new rows into one or two cache views through one slot_mapping.
 *
 * Defined by [LAYOUT], section "kernel 那一侧": each token's slot is split into
 * block = slot / block_size and position = slot % block_size. The row is
 * written at base + offset + layer*layer_stride + block*block_stride +
 * position*row_bytes, using that view's own strides. [INSIDE] §2.1 names the
 * fused operator; [MGMT] shows a decode step writing the new token's K/V at
 * (physical block, offset in block).
 *
 *   k, v           device; row t of each source starts at k + t*k_pitch (v + t*v_pitch) and holds
 *                  k_view.row_bytes (v_view.row_bytes) bytes, copied bit-exactly. v may be NULL to
 *                  write only the k view. For dense caches the source rows are [num_kv_heads,
 *                  head_dim] values. For the DSA dual cache of [LAYOUT], k carries packed MLA rows
 *                  and v packed indexer rows.
 *   slot_mapping   device int64 [num_tokens]: physical block*block_size + in-block position. A
 *                  negative slot marks padding and is skipped. Two tokens with the same slot in one
 *                  call race (caller error).
 *   k_cache, v_cache  device allocation bases; *_cache_bytes give their sizes.
 *   layer          layer index into the views' layer_stride.
 *   block_size, num_blocks  the pool geometry (slot < num_blocks*block_size).
 * Alignment: every address involved must be 4-byte aligned (row_bytes, pitches, strides, offsets,
 * bases). 16-byte alignment of all of them selects the 16-byte copy path.
 * num_tokens == 0 is a no-op. */
int32_t pa_reshape_and_cache(const void* k, int64_t k_pitch, const void* v, int64_t v_pitch,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             void* k_cache, int64_t k_cache_bytes, pa_cache_view k_view,
                             void* v_cache, int64_t v_cache_bytes, pa_cache_view v_view,
                             int32_t layer, int32_t block_size, int64_t num_blocks, void* stream);

/* pa_quantize_and_cache_mla: quantize-on-write of the DSA dual cache through one slot_mapping.
 *
 * [MEM] §3.4: the cache may be stored at low precision by quantizing as it is written (FP8 being the
 * safest format) and dequantizing as it is read; finer scale groups are more accurate. [LAYOUT]
 * (two caches sharing one block table) fixes the rows: an MLA row is 512 B of FP8 latent, 16 B of
 * scale and 128 B of BF16 RoPE (656 B); an indexer row is 128 B of FP8 key and a 4 B FP32 scale
 * (132 B). Per group of 128 values (latent values [128k, 128k+128) share scale k; the indexer key has
 * one group): scale = amax / 448 in float32, and each value x is stored as the OCP E4M3 code (bias 7,
 * max 448) nearest to x / scale (float32 division), ties to the even mantissa, with the quotient's
 * sign, saturating at 448. A group of zeros stores scale 0 and zero codes. The rows are then
 * written exactly as pa_reshape_and_cache writes them, and pa_decode reads the MLA view.
 *
 *   latent         device bf16 [num_tokens, 512]; row t at latent + t*latent_pitch (bytes).
 *   rope           device bf16 [num_tokens, 64], copied unchanged into bytes [528, 656) of the row.
 *   index_key      device bf16 [num_tokens, 128], or NULL to write only the MLA view.
 *   slot_mapping   device int64 [num_tokens]; negative slots are skipped, as in pa_reshape_and_cache.
 *   mla_cache, index_cache  device allocation bases (may be the same allocation, as in [LAYOUT]'s
 *                  dual cache); *_cache_bytes give their sizes for the extent check.
 *   mla_view       row_bytes must be 656; index_view row_bytes must be 132.
 * Inputs must be finite (otherwise the rows are unspecified). Alignment: latent, rope, index_key
 * and their pitches 16 bytes; mla_cache and the MLA view 16 bytes; index_cache and the index view
 * 4 bytes. num_tokens == 0 is a no-op. */
int32_t pa_quantize_and_cache_mla(const void* latent, int64_t latent_pitch, const void* rope, int64_t rope_pitch,
                                  const void* index_key, int64_t index_pitch, const int64_t* slot_mapping,
                                  int32_t num_tokens, void* mla_cache, int64_t mla_cache_bytes,
                                  pa_cache_view mla_view, void* index_cache, int64_t index_cache_bytes,
                                  pa_cache_view index_view, int32_t layer, int32_t block_size,
                                  int64_t num_blocks, void* stream);

/* pa_quantize_and_cache: quantize-on-write of dense K/V rows into a PA_KV_FP8_E4M3 cache.
 *
 * [MEM] §3.4: the cache may be stored at low precision by quantizing as it is written. Every value
 * x of a source row (num_kv_heads * head_dim values of src_format, PA_KV_F16 or PA_KV_BF16) is
 * stored as the OCP e4m3 code nearest to x / k_scale (x / v_scale for V), the quotient taken in
 * float32, ties to the even mantissa, saturating at 448. The rows then land exactly where
 * pa_reshape_and_cache puts them (view row_bytes = num_kv_heads * head_dim, one byte per value).
 *   k, v           device rows; row t at k + t*k_pitch (bytes), 2*row_bytes bytes each. v may be NULL.
 *   k_scale, v_scale  finite, > 0; the same values go into the pa_attn_desc of the decode.
 *   Other arguments as for pa_reshape_and_cache.
 * Inputs must be finite (otherwise the codes are unspecified). Alignment: sources and pitches 16
 * bytes; cache bases, view offsets, strides and row_bytes 8 bytes. num_tokens == 0 is a no-op. */
int32_t pa_quantize_and_cache(const void* k, int64_t k_pitch, const void* v, int64_t v_pitch, int32_t src_format,
                              float k_scale, float v_scale, const int64_t* slot_mapping, int32_t num_tokens,
                              void* k_cache, int64_t k_cache_bytes, pa_cache_view k_view, void* v_cache,
                              int64_t v_cache_bytes, pa_cache_view v_view, int32_t layer, int32_t block_size,
                              int64_t num_blocks, void* stream);

/* pa_copy_blocks: the data movement of copy-on-write (and of any block move inside a pool).
 *
 * [INSIDE] §2.2: physical blocks carry a reference count; a sequence about to write into a block
 * shared with others (count above 1) gets a new physical block, the contents are copied, and the old
 * block's count drops by one. The counting and allocation are the caller's; this call does the
 * copy: for each pair (src, dst) and each layer l < num_layers, the page of dst (block_size rows
 * starting at offset + l*layer_stride + dst*block_stride) takes the bytes of src's page, in the K
 * view and, if v_cache is not NULL, the V view.
 *
 *   block_pairs    device int64 [num_pairs, 2]: (src, dst) physical block ids. A pair with an id
 *                  outside [0, num_blocks) is skipped. No block may be the dst of two pairs or both a
 *                  src and a dst in one call (caller error: the result is then unspecified).
 *   k_cache, v_cache, *_bytes, *_view  as for pa_reshape_and_cache; every layer < num_layers of
 *                  each view must lie inside its allocation.
 * Alignment: bases, view offsets and strides 4 bytes (16 bytes selects 16-byte copies).
 * num_pairs == 0 or num_layers == 0 is a no-op. */
int32_t pa_copy_blocks(void* k_cache, int64_t k_cache_bytes, pa_cache_view k_view, void* v_cache,
                       int64_t v_cache_bytes, pa_cache_view v_view, const int64_t* block_pairs, int32_t num_pairs,
                       int32_t num_layers, int32_t block_size, int64_t num_blocks, void* stream);

/* Workspace bytes pa_decode needs for this shape (0 when no split-context partials are needed). */
size_t pa_decode_workspace_bytes(const pa_attn_desc* desc, int32_t num_seqs, int32_t max_context_len);

/* pa_decode: one query token per sequence attends to its whole paged context.
 *
 * out[b, h] = softmax_t(scale * q[b, h] . K_t) applied to V_t, for tokens t in [0, context_lens[b]).
 * Token t of sequence b is read from physical block block_tables[b*bt_stride + t/block_size] at
 * position t % block_size ([MEM] §2 read path; [MGMT] paged_attention; [INSIDE] §2.1: the kernel
 * knows only the block table and reads block by block). The softmax runs online over blocks and over
 * split-context partitions merged by log-sum-exp; both are exact rearrangements, computed in fp32.
 *
 *   out            device [num_seqs, num_q_heads, v_dim] in the query type (dense: the KV type;
 *                  MLA: bf16). Rounded to nearest even.
 *   q              device [num_seqs, num_q_heads, qk_dim], contiguous.
 *   k_cache, v_cache  device allocation bases of the K and V views (v_cache unused and may be NULL
 *                  for MLA).
 *   block_tables   device int32 [num_seqs, bt_stride]; entries past ceil(ctx/block_size) are not read.
 *   context_lens   device int32 [num_seqs]: tokens to attend, the current one included (the caller
 *                  writes it first). 0 gives an output of 0.
 *   max_context_len  host upper bound of context_lens; sizes the grid.
 *   scale          softmax scale, finite and >= 0 (e.g. 1/sqrt(qk_dim)).
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...) bytes (may be NULL when
 *                  that is 0). Its contents on entry do not matter.
 * Alignment: q, out, cache bases, view offsets, strides and row_bytes: 16 bytes.
 * num_seqs == 0 is a no-op. */
int32_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                  int32_t num_seqs, int32_t max_context_len, float scale, const pa_attn_desc* desc,
                  void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode_no_alloc: pa_decode without a workspace argument and without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Computes exactly what pa_decode computes, with the same
 * kernels and bitwise the same results. The split-context partials go to a static device array of
 * PA_STATIC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds until the process ends.
 * Its address is looked up once per device, on the first call that needs it. The call calls no
 * allocator (no hipMalloc, no hipFree).
 *
 *   Arguments as for pa_decode, without workspace and workspace_bytes.
 *   Returns PA_ERR_SCRATCH_LIMIT, enqueueing nothing, when
 *   pa_decode_workspace_bytes(desc, num_seqs, max_context_len) > PA_STATIC_SCRATCH_BYTES.
 *   Every other error is pa_decode's.
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (on different
 * streams, or from several host threads without ordering) race and give undefined results. Calls
 * ordered on one stream are safe. The array keeps the last call's contents; nothing in it needs to
 * start at zero, because each call writes every partial it reads. */
int32_t pa_decode_no_alloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                           int32_t num_seqs, int32_t max_context_len, float scale, const pa_attn_desc* desc,
                           void* stream);

/* Workspace bytes pa_prefill_chunk needs. */
size_t pa_prefill_workspace_bytes(const pa_attn_desc* desc, int32_t num_seqs, int32_t total_q,
                                  int32_t max_query_len, int32_t max_seq_len);

/* pa_prefill_chunk: causal query chunks attending to already-cached paged context (varlen).
 *
 * [INSIDE] §3.2: a long prompt is processed in chunks under a per-step token budget. Each chunk
 * attends causally to the context already in the cache, and decodes run in the same step. Sequence
 * b owns query rows [query_start_loc[b], query_start_loc[b+1]). Its seq_lens[b] tokens, this chunk's
 * included, are in the cache (written first, as for decode). Query row i of sequence b sits at
 * absolute position a = seq_lens[b] - qlen_b + i and attends to tokens [0, a]. A decode is a chunk of
 * length 1.
 *
 *   out            device [total_q, num_q_heads, v_dim] in the query type.
 *   q              device [total_q, num_q_heads, qk_dim].
 *   seq_lens       device int32 [num_seqs]; query_start_loc device int32 [num_seqs+1], with
 *                  query_start_loc[0] == 0 and query_start_loc[num_seqs] == total_q; qlen_b <= seq_lens[b].
 *   max_query_len, max_seq_len  host upper bounds of qlen_b and seq_lens[b]; size the grid.
 *   Other arguments as for pa_decode. Dense formats only. */
int32_t pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                         int32_t max_query_len, int32_t max_seq_len, float scale,
                         const pa_attn_desc* desc, void* workspace, size_t workspace_bytes,
                         void* stream);

/* pa_indexer_topk: lightning-indexer scores over the indexer view of the DSA dual cache, then each
 * sequence's top-k token selection.
 *
 * [LAYOUT] (two caches sharing one block table): the lightning indexer stores per token a 132-byte
 * row (128 OCP e4m3 key values, then one float32 scale) used to select a sparse top-k set of tokens;
 * the indexer and MLA views share one block table. The pages give no scoring formula; this call
 * computes the published lightning indexer's. For decode token b with index queries q[b, j]
 * (j < num_index_heads, 128 bf16 values each) and head weights w[b, j] (float32), the score of
 * context position t is
 *     I[b, t] = sum_j w[b, j] * max(q[b, j] . k_t, 0),   k_t = codes_t * scale_t,
 * read through the block table as pa_decode reads K. It is computed as
 * scale_t * sum_j w[b, j] * max(q[b, j] . codes_t, 0) in float32 (equal for scale_t >= 0, which is
 * what pa_quantize_and_cache_mla stores). The top_k positions of highest score are selected; equal
 * scores are taken from the earliest position first, and when the context has at most top_k tokens
 * every one is selected.
 *
 *   topk_positions device int32 [num_seqs, top_k]: the selected positions in ascending order; -1
 *                  past topk_lens[b].
 *   topk_slots     device int32 [num_seqs, top_k]: slot of each selected position
 *                  (block_tables[b][t / block_size] * block_size + t % block_size), -1 past
 *                  topk_lens[b] and for an invalid block id. These feed pa_mla_sparse_decode.
 *   topk_lens      device int32 [num_seqs]: min(top_k, context length).
 *   scores         device float32 [num_seqs, score_stride], score_stride >= max_context_len:
 *                  written with I[b, t] for t < context length (-inf for positions in an invalid
 *                  block); the other entries are untouched.
 *   q_index        device bf16 [num_seqs, num_index_heads, 128]; head_weights device float32
 *                  [num_seqs, num_index_heads]. num_index_heads: 16, 32, 48 or 64.
 *   index_cache, index_cache_bytes, index_view, layer  the indexer view (row_bytes 132).
 *   block_tables, bt_stride, context_lens, max_context_len, block_size, num_blocks  as for pa_decode.
 * num_blocks * block_size must fit in int32. Scores are unspecified for non-finite inputs or a
 * negative scale (memory-safe). Alignment: q_index, index_cache, the view's offset, block_stride
 * and layer * layer_stride 16 bytes; everything else 4 bytes.
 * num_seqs == 0 is a no-op. */
int32_t pa_indexer_topk(int32_t* topk_positions, int32_t* topk_slots, int32_t* topk_lens, int32_t top_k,
                        float* scores, int64_t score_stride, const void* q_index, const float* head_weights,
                        int32_t num_index_heads, const void* index_cache, int64_t index_cache_bytes,
                        pa_cache_view index_view, int32_t layer, const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                        int32_t block_size, int64_t num_blocks, void* stream);

/* pa_mla_sparse_decode: MLA decode over a selected set of cache rows (DSA sparse attention).
 *
 * The MLA decode of pa_decode ([MEM] §3.3, row format PA_KV_MLA656_E4M3), except that sequence b
 * attends only to the rows at slots[b * slot_stride + i], i < slot_counts[b] (one softmax over
 * them), each at block = slot / block_size, position = slot % block_size of the desc's view
 * ([LAYOUT], section "kernel 那一侧"). A slot outside [0, num_blocks * block_size) contributes no
 * token; no valid slot gives an output of 0. [LAYOUT] (two caches sharing one block table) has the
 * indexer pick these tokens: pa_indexer_topk writes slots and counts in this form.
 *
 *   out, q         as for an MLA pa_decode: bf16 [num_seqs, num_q_heads, 512] and [.., 576].
 *   kv_cache       allocation base of desc->k_view (desc->kv_format must be PA_KV_MLA656_E4M3).
 *   slots          device int32 [num_seqs, slot_stride]; slot_counts device int32 [num_seqs], each
 *                  clamped to [0, min(max_count, slot_stride)].
 *   workspace      at least pa_decode_workspace_bytes(desc, num_seqs, max_count) bytes.
 * num_blocks * block_size must fit in int32. Alignment: out, q, kv_cache and the view 16 bytes;
 * slots and slot_counts 4 bytes. num_seqs == 0 is a no-op. */
int32_t pa_mla_sparse_decode(void* out, const void* q, const void* kv_cache, const int32_t* slots,
                             int32_t slot_stride, const int32_t* slot_counts, int32_t num_seqs, int32_t max_count,
                             float scale, const pa_attn_desc* desc, void* workspace, size_t workspace_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
