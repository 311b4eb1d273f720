// Internal launch parameters shared by the host API (api.hip) and the kernel files.
// Not part of the public ABI; include/pa.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

// ---------------------------------------------------------------------------
// reshape_and_cache
// ---------------------------------------------------------------------------
struct CacheWriteParams {
    const char* src[2];        // source rows of view 0 (k) and view 1 (v)
    int64_t pitch[2];          // bytes between source rows
    char* dst[2];              // cache base + view offset + layer * layer_stride
    int64_t block_stride[2];
    int32_t row_bytes[2];
    int32_t vec16[2];          // 1: every address of the view is 16-byte aligned
    const int64_t* slots;      // [num_tokens]
    int32_t num_tokens;
    int32_t num_views;         // 1 or 2
    int32_t block_size;
    int32_t pad_;
    int64_t num_slots;         // num_blocks * block_size
};
hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream);

// Quantize-on-write of the DSA dual cache: bf16 latent [T, 512] + RoPE [T, 64] -> 656-byte MLA rows,
// optional bf16 indexer key [T, 128] -> 132-byte indexer rows, through one slot_mapping.
struct QuantWriteParams {
    const char* latent;        // row t at latent + t * latent_pitch: 512 bf16
    const char* rope;          // 64 bf16
    const char* index_key;     // 128 bf16, or null (MLA view only)
    int64_t latent_pitch, rope_pitch, index_pitch;
    const int64_t* slots;      // [num_tokens]
    char* mla_dst;             // cache base + view offset + layer * layer_stride
    char* idx_dst;
    int64_t mla_block_stride, idx_block_stride;
    int64_t num_slots;         // num_blocks * block_size
    int32_t num_tokens;
    int32_t block_size;
};
hipError_t launch_quant_cache_write(const QuantWriteParams& p, hipStream_t stream);

// Quantize-on-write of dense 16-bit K/V rows into E4M3 rows with one float32 scale per cache.
struct QuantDenseParams {
    const char* src[2];        // row t at src + t * pitch
    int64_t pitch[2];
    char* dst[2];              // cache base + view offset + layer * layer_stride
    int64_t block_stride[2];
    float scale[2];            // value = code * scale
    float inv_scale[2];        // 1 / scale, correctly rounded
    const int64_t* slots;
    int64_t num_slots;
    int32_t row_values;        // values per row (= bytes per cache row)
    int32_t num_tokens, num_views, block_size;
    int32_t src_f16;           // 1: fp16 sources, 0: bf16
};
hipError_t launch_quant_dense_write(const QuantDenseParams& p, hipStream_t stream);

// Copy-on-write's data movement: for each (src, dst) block pair and each layer, copy the page
// (block_size contiguous rows) of every view.
struct BlockCopyParams {
    char* base[2];             // cache base + view offset (layer 0)
    int64_t layer_stride[2], block_stride[2];
    int64_t page_bytes[2];     // block_size * row_bytes
    int32_t vec16[2];          // 1: every address of the view is 16-byte aligned
    const int64_t* pairs;      // [num_pairs, 2]: src block, dst block
    int64_t num_blocks;
    int32_t num_pairs, num_layers, num_views;
};
hipError_t launch_block_copy(const BlockCopyParams& p, hipStream_t stream);

// ---------------------------------------------------------------------------
// Dense paged decode (fp16 / bf16 rows, head_dim 64 / 128 / 256; group 1, 2, 4, 8, or 2..16 at head_dim 128)
// ---------------------------------------------------------------------------
struct DenseDecodeParams {
    void* out;                 // [num_seqs, Hq, D]
    const void* q;             // [num_seqs, Hq, D]
    const char* k;             // cache base + view offset + layer * layer_stride
    const char* v;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start_loc;  // null for pa_decode. Otherwise sequence s's query is row
                                     // query_start_loc[s], and only sequences with exactly one query
                                     // row take part (the decode rows of a mixed prefill call).
    float* part_ml;            // [num_seqs, Hq, max_parts, 2]: running max (log2 domain), sum
    float* part_acc;           // [num_seqs, Hq, max_parts, D]: unnormalised accumulator
    int64_t k_block_stride, v_block_stride;
    int64_t num_blocks;
    int32_t k_row_bytes, v_row_bytes;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_q_heads, num_kv_heads;
    int32_t block_size;
    int32_t tiles_per_block_log2;  // log2(block_size / 16)
    int32_t partition_tokens;  // multiple of block_size, <= 64 * block_size
    int32_t max_parts;         // ceil(max_context_len / partition_tokens)
    int32_t max_context_len;   // clamp for context_lens
    float scale_log2;          // softmax scale * log2(e)
    int32_t is_bf16;
    int32_t head_dim;
    int32_t group;             // query heads per wave item (Hq / Hkv, or 4 when kv_shift is 1)
    int32_t kv_shift;          // item K/V head >> kv_shift = stored K/V head (1: two waves of four
                               // query heads share each stored head; num_kv_heads counts the items)
    int32_t kv_fp8;            // 1: E4M3 rows (one byte per value), bf16 queries and outputs
    float v_scale;             // FP8 rows: V value = code * v_scale (K's scale is folded into scale_log2)
};
hipError_t launch_decode_dense(const DenseDecodeParams& p, hipStream_t stream);   // picks the kernel below
hipError_t launch_decode_fp8(const DenseDecodeParams& p, hipStream_t stream);     // FP8 rows (decode_fp8.hip)
hipError_t launch_decode_mfma(const DenseDecodeParams& p, hipStream_t stream);    // head_dim 128, group 2..16
hipError_t launch_decode_reduce(const DenseDecodeParams& p, hipStream_t stream);  // partition merge

// ---------------------------------------------------------------------------
// MLA latent decode over 656-byte rows (one latent K/V head, num_q_heads query heads)
// ---------------------------------------------------------------------------
// Work is counted in units of 32 consecutive tokens of one sequence. The units of all sequences,
// in sequence order, form one stream; work-group w takes units [w * per, (w + 1) * per) of it
// (per = units_per_wg, or ceil(total / num_wgs) when units_per_wg is 0) for heads
// [blockIdx.y * heads_per_wg, +heads_per_wg). A run of units of one sequence inside one range is a
// segment. A segment that is the whole sequence writes out directly; otherwise it writes a partial
// to slot s + w, and the merge kernel combines the slots of each sequence. (s + w grows by at least
// one from each segment to the next, so slots are distinct and below num_seqs + num_wgs.)
struct MlaDecodeParams {
    void* out;                 // bf16 [num_seqs, Hq, 512]
    const void* q;             // bf16 [num_seqs, Hq, 576]
    const char* kv;            // cache base + view offset + layer * layer_stride
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* part_ml;            // [slots, Hq, 2]: reference max (log2 domain), sum
    uint16_t* part_acc;        // [slots, Hq, 512]: the partial's output O / l, bf16
    int32_t* seq_meta;         // [num_seqs, 2]: first and last work-group of the sequence
    int64_t block_stride;
    int64_t num_blocks;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t heads_per_wg;      // 128, 96, 64, 32 or 16, dividing num_q_heads
    int32_t block_size;
    int32_t block_size_log2;
    int32_t max_context_len;   // clamp for context_lens
    int32_t num_wgs;           // work-groups along x
    int32_t units_per_wg;      // 0: balanced over num_wgs
    float scale_log2;          // softmax scale * log2(e)
    // Sparse form: token i of sequence s is the row at slot slots[s * slot_stride + i] (block =
    // slot >> block_size_log2, position = slot & (block_size - 1)); context_lens holds the number of
    // slots and block_tables is unused. A slot outside [0, num_slots) contributes no token.
    const int32_t* slots;      // nullptr: the dense form, through block_tables
    int64_t slot_stride;
    int64_t num_slots;
};
hipError_t launch_decode_mla(const MlaDecodeParams& p, hipStream_t stream);

// ---------------------------------------------------------------------------
// DSA indexer: scores of every context token from the indexer rows, then each sequence's top-k
// ---------------------------------------------------------------------------
struct IndexerParams {
    const char* idx;           // cache base + view offset + layer * layer_stride (132-byte rows)
    const uint16_t* q;         // bf16 [num_seqs, num_heads, 128]
    const float* w;            // [num_seqs, num_heads]
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* scores;             // [num_seqs, score_stride]
    int32_t* topk_pos;         // [num_seqs, top_k]
    int32_t* topk_slots;       // [num_seqs, top_k]
    int32_t* topk_lens;        // [num_seqs]
    int64_t score_stride;
    int64_t block_stride;
    int64_t num_blocks;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_heads;         // 16, 32, 48 or 64
    int32_t block_size;
    int32_t block_size_log2;
    int32_t max_context_len;   // clamp for context_lens
    int32_t top_k;
};
hipError_t launch_indexer_topk(const IndexerParams& p, hipStream_t stream);

// ---------------------------------------------------------------------------
// Causal chunks over paged context (query length >= 2), head_dim 128, group 1..16
// ---------------------------------------------------------------------------
struct PrefillParams {
    void* out;                 // [total_q, Hq, 128]
    const void* q;             // [total_q, Hq, 128]
    const char* k;             // cache base + view offset + layer * layer_stride
    const char* v;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* query_start_loc;  // [num_seqs + 1]
    int64_t k_block_stride, v_block_stride;
    int64_t num_blocks;
    int32_t k_row_bytes, v_row_bytes;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_q_heads, num_kv_heads;
    int32_t block_size;
    int32_t tiles_per_block_log2;
    int32_t max_seq_len;       // clamp for seq_lens
    int32_t max_query_len;     // clamp for query lengths
    float scale_log2;
    int32_t is_bf16;
    int32_t group;             // Hq / Hkv
    int32_t rows_per_item;     // query rows (position x head) per wave
    int32_t total_q;           // query rows of the call (bounds the grid)
};
hipError_t launch_prefill_chunk(const PrefillParams& p, hipStream_t stream);
// Chunk rows and the decode rows of the same call in one launch (decode rows on the grouped-query
// matrix-core decode: head_dim 128, group 2..16), then the decode rows' partition merge.
hipError_t launch_mixed_chunk(const PrefillParams& pp, const DenseDecodeParams& dp, hipStream_t stream);

}  // namespace pa
