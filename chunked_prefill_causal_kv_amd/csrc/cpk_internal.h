// Internal declarations shared by the HIP kernels and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpk {

// One attention launch: a chunk of query rows of one sequence (scalar mode)
// or of every sequence of a packed step (varlen mode), over keys read from a
// [batch][kv_heads][cap][D] cache.
//
// Query row i of a sequence sits at causal position causal_base + i and sees
// key j iff  key_lo <= j <= causal_base + i  and  j < n_keys.  Optionally an
// additive mask [rows][mask_ld] (same dtype as q) is added to the scaled
// scores instead (rolling cache form).
struct AttnArgs {
    const void *q;      // token-major [*, Hq, D]; the sequence's rows start at q_row0
    const void *k;      // cache [batch][Hkv][cap][D]
    const void *v;
    void *out;          // token-major [*, Hq, D]; rows start at out_row0
    const void *mask;   // optional additive mask [rows][mask_ld]
    int Hq, Hkv, D;
    int cap;            // positions per (slot, head) in k / v
    int mask_ld;
    float scale;        // softmax scale
    float scale_log2;   // scale * log2(e)

    // scalar mode (varlen == 0)
    int slot;           // cache batch index
    int q_row0, out_row0;
    int rows;           // issued rows (padded width)
    int q_src_rows;     // rows present in q: pad rows repeat row q_src_rows - 1
    int out_rows;       // rows written to out
    int n_keys;         // keys [0, n_keys) exist for this call
    int key_lo;         // keys below key_lo are invisible
    int causal_base;    // row i sees keys <= causal_base + i

    // varlen mode: per-sequence device arrays (rows of sequence s are
    // cu_rows[s] .. cu_rows[s+1], its cache slot slots[s], its cached length
    // past_lens[s]); sequences with fewer than min_rows rows are skipped.
    int varlen;
    const int32_t *cu_rows;
    const int32_t *past_lens;
    const int32_t *slots;
    int n_seqs;
    int min_rows;

    // key-range split (scalar mode, bf16/fp16 only): grid.y = n_parts and
    // part p covers the absolute key tiles [p * part_tiles, (p + 1) *
    // part_tiles).  With n_parts > 1 each workgroup writes fp32 partial
    // records [M, den, pad, pad, O[D]] (running maximum in the exp2 domain,
    // sum and unnormalised output) per (row, query head) to
    // part_ws[p][row][head] instead of the output; launch_attention_combine
    // merges them in part order.
    int n_parts;        // 1: no split
    int part_tiles;
    float *part_ws;

    // fused append (scalar mode, bf16/fp16): with k_new set, keys at or
    // past new_base are read from k_new / v_new (token-major
    // [new_rows][Hkv][D]; key new_base + i is row min(i, new_rows - 1), so a
    // padded tail repeats the last real row) instead of the cache, and the
    // part-0 workgroup of a row block writes the cache rows new_base + (its
    // rows) of its KV head from them (physical rows (ring_start + position)
    // mod cap in a ring buffer); with seqlens set, one workgroup sets
    // seqlens[slot] = len_after.
    const void *k_new;
    const void *v_new;
    int new_base;
    int new_rows;
    int32_t *seqlens;
    int len_after;

    // rolling ring buffer (64-column kernel): logical key s of the rolling
    // view sits at physical row (ring_start + s) mod cap; 0 = no ring
    int ring_start;

    // paged cache (varlen mode): with block_size > 0, k / v are pools
    // [n_blocks][Hkv][block_size][D] and position p of the sequence in slot
    // s lives in block block_table[s * max_blocks + p / block_size] (ids
    // clamped into [0, n_blocks)); block_size is a multiple of 256
    const int32_t *block_table;
    int max_blocks, block_size, n_blocks;

    // carried merge (scalar mode, key split; the 64-column kernel's
    // scheduled form): with prev_ws set, the launch also merges the parts
    // that an earlier split launch of the same shapes left in prev_ws
    // (part_ws's layout: n_parts records per (row, query head) of out_rows
    // rows) into prev_out [out_rows][Hq][D] with the combine's arithmetic,
    // the (row, head) pairs spread over the grid's workgroups
    const float *prev_ws;
    void *prev_out;
};

// Row of position `pos` (head g) in a paged pool, as an element offset; the
// block id is clamped into the pool so a bad table cannot address outside.
__device__ __forceinline__ int64_t paged_row(const int32_t *table, int max_blocks, int bs,
                                             int n_blocks, int Hkv, int slot, int g, int pos)
{
    int b = table[(int64_t)slot * max_blocks + pos / bs];
    b = b < 0 ? 0 : (b >= n_blocks ? n_blocks - 1 : b);
    return ((int64_t)b * Hkv + g) * bs + pos % bs;
}

// Split-KV decode: one query row per sequence.
struct DecodeArgs {
    const void *q;      // token-major [*, Hq, D]
    void *k;            // cache (written only by the fused append)
    void *v;
    void *out;
    float *ws;          // partials [n_seqs][Hq][max_segs][D + 4] (m, l, pad, pad, acc[D])
    int Hq, Hkv, D, cap;
    float scale_log2;
    int max_segs;       // segments allocated per (seq, head) in ws
    // varlen arrays (a sequence takes part iff it has exactly one row)
    const int32_t *cu_rows;
    const int32_t *past_lens;
    const int32_t *slots;
    int n_seqs;
    // paged cache, as in AttnArgs (block_size 0: contiguous [batch][Hkv][cap][D])
    const int32_t *block_table;
    int max_blocks, block_size, n_blocks;
    // fused append (k_new non-null): the workgroup whose segment holds a
    // sequence's new key writes that row of k_new/v_new (token-major
    // [*, Hkv, D], row cu_rows[s]) into the cache before reading it, and
    // sets seqlens_k[slot] to past_len + 1
    const void *k_new;
    const void *v_new;
    int32_t *seqlens_k;
};

constexpr int kDecodeSeg = 256;   // keys per decode work item (4 waves x 64)

// Launchers (return hipError_t of the launch).
hipError_t launch_kv_append(const void *k_new, const void *v_new, void *ck, void *cv,
                            int32_t *seqlens, int Hkv, int cap, int row_bytes, int slot,
                            int past, int rows, int src_rows, int len_after, hipStream_t st);
// paged (block_size > 0): ck / cv are pools, as in AttnArgs
hipError_t launch_kv_append_varlen(const void *k_new, const void *v_new, void *ck, void *cv,
                                   int32_t *seqlens, int Hkv, int cap, int row_bytes,
                                   const int32_t *cu_rows, const int32_t *past_lens,
                                   const int32_t *slots, int n_seqs, int total_rows,
                                   const int32_t *block_table, int max_blocks, int block_size,
                                   int n_blocks, bool skip_single, hipStream_t st);
hipError_t launch_set_len(int32_t *seqlens, int b, int len, hipStream_t st);
// rows [0, len) of slot src copied to slot dst (every KV head); seqlens[dst] = len
hipError_t launch_kv_copy_prefix(const void *k, const void *v, int32_t *seqlens, int Hkv,
                                 int cap, int row_bytes, int src, int dst, int len,
                                 hipStream_t st);
hipError_t launch_roll_append(const void *k_old, const void *v_old, const void *k_chunk,
                              const void *v_chunk, void *k_new, void *v_new, int B, int H,
                              int C, int c, int row_bytes, hipStream_t st);
// ring buffer: chunk row t of (b, h) -> physical slot (start + t) mod C
hipError_t launch_ring_append(const void *k_chunk, const void *v_chunk, void *k_ring,
                              void *v_ring, int B, int H, int C, int c, int row_bytes, int start,
                              hipStream_t st);
// logical view: out slot s <- physical slot (start + s) mod C
hipError_t launch_ring_view(const void *k_ring, const void *v_ring, void *k_out, void *v_out,
                            int B, int H, int C, int row_bytes, int start, hipStream_t st);

// Attention: grid.x = row blocks x KV heads (KV head fastest), grid.z = sequences.
// `wide` selects the 128-column bf16/fp16 kernel (chunk and varlen
// attention only: the rolling form keeps the 64-column kernel, which also
// takes the explicit additive mask, so both of its forms stay bit-equal).
constexpr int kWideMinGroups = 256;   // auto choice: wide once its grid fills the CUs ...
// ... and the launch holds at least this many visible (row, key) pairs per
// query head (rows x (past + rows / 2)): below it the 64-column kernel's
// smaller per-workgroup fixed cost outweighs the 128-column kernel's cheaper
// tiles (measured on the 32/8-head, D = 128 shapes)
constexpr int64_t kWideMinPairs = (int64_t)24 << 20;
int attn_rows_per_block(int dtype, int group, bool wide);
// bf16/fp16 kernel of a launch: the 64-column kernel (its latency-scheduled
// form wherever the launch reads a contiguous cache, its general form over
// a paged pool), the 128-column kernel, or the 64-column kernel's general
// form everywhere (diagnostics)
enum AttnKernel { kAttnNarrow = 0, kAttnWide = 1, kAttnNarrowGeneral = 2 };
hipError_t launch_attention(const AttnArgs &a, int dtype, int row_blocks, int n_seq_grid,
                            int kernel, hipStream_t st);

hipError_t launch_decode(const DecodeArgs &a, int dtype, int max_segs, hipStream_t st);

// Key tile of the bf16/fp16 attention kernel, and the merge of split parts
// (a.n_parts > 1) into a.out.
constexpr int kAttnTileKeys = 128;
// most block-table entries per sequence in a paged attention call (the
// attention kernels stage a workgroup's entries in LDS)
constexpr int kMaxTableBlocks = 512;
hipError_t launch_attention_combine(const AttnArgs &a, int dtype, hipStream_t st);
bool decode_supported(int dtype, int D, int group, int capacity);

// Sets the calling thread's error message (cpk_last_error) and returns code.
int fail_status(int code, const char *msg);

}  // namespace cpk
