/*
 * cpk.h -- C ABI of the chunked-prefill causal-attention library for AMD
 * MI355X (gfx950).
 *
 * A chunk of `rows` query rows at absolute positions [past_len,
 * past_len + rows) attends causally over every cached key/value in
 * [0, past_len + rows); its own K/V are appended to a cache bound at
 * physical capacity first.  Chunked prefill is exact: its visible set per
 * query equals one-shot prefill's (ONNX GenAI Wiki "Chunked Prefill",
 * section 1: 1.1 append-only cache, 1.2 causal mask, 1.3 capacity kept
 * apart from length).
 *
 * Conventions shared by every call:
 *  - Return value: CPK_OK (0) or a negative CPK_E* status.  No exception or
 *    abort crosses the ABI.  cpk_last_error() gives a message for the last
 *    failing call on the calling thread.
 *  - Validation runs on the host before anything is launched; on error no
 *    device memory is written.
 *  - Ownership: the caller owns every device buffer (cache, seqlens_k,
 *    inputs, outputs, workspace).  The library allocates no device memory.
 *  - Streams: every device call is asynchronous on the caller's stream
 *    (`stream` is a hipStream_t passed as void*; NULL is the default
 *    stream).  No call synchronises the host.
 *  - Layouts: token-major q / out / new K/V rows are [rows, heads, D]
 *    contiguous; caches are [batch, kv_heads, capacity, D] contiguous.
 *    Device pointers must be 16-byte aligned.
 *  - Dtypes: CPK_F32, CPK_F16, CPK_BF16; q, K/V, masks and outputs of one
 *    call share one dtype.  Accumulation is fp32.
 *  - Head dims: 64 or 128.  q_heads must be a multiple of kv_heads
 *    (grouped-query attention with contiguous groups: query head h reads
 *    KV head h / (q_heads / kv_heads)), with q_heads / kv_heads <= 64.
 */
#ifndef CPK_H
#define CPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum cpk_status {
    CPK_OK = 0,
    CPK_EINVAL = -1,      /* bad size, index, flag or NULL pointer          */
    CPK_EDTYPE = -2,      /* unsupported dtype / head-dim combination      */
    CPK_ECAPACITY = -3,   /* positions past the cache's physical capacity  */
    CPK_EALIGN = -4,      /* device pointer not 16-byte aligned            */
    CPK_EWORKSPACE = -5,  /* workspace missing or too small                */
    CPK_EHIP = -6,        /* the HIP runtime reported an error             */
};

enum cpk_dtype { CPK_F32 = 0, CPK_F16 = 1, CPK_BF16 = 2 };

/* phases of a packed mixed step (cpk_varlen_step_phases) */
enum cpk_varlen_phase {
    CPK_PHASE_APPEND = 1,    /* every sequence's new rows into the cache      */
    CPK_PHASE_DECODE = 2,    /* one-row sequences: split-KV decode + combine  */
    CPK_PHASE_PREFILL = 4,   /* sequences of two or more rows: chunk attention */
    CPK_PHASE_ALL = 7,
};

/* bf16/fp16 attention kernel choice (cpk_set_attention_kernel) */
enum cpk_attention_kernel {
    CPK_ATTN_AUTO = 0,     /* by grid size and work (the default)           */
    CPK_ATTN_NARROW = 1,   /* 64 query columns per workgroup, 8 waves       */
    CPK_ATTN_WIDE = 2,     /* 128 query columns per workgroup, 4 waves      */
    CPK_ATTN_NARROW_GENERAL = 3, /* the 64-column kernel's general form even
                                    where its latency-scheduled form applies */
};

/*
 * A KV cache bound at physical capacity, with the true number of valid
 * positions per sequence carried beside it in seqlens_k (ONNX GenAI Wiki
 * "Chunked Prefill", section 1.3).
 *   k, v       device, [batch][kv_heads][capacity][head_dim] of dtype
 *   seqlens_k  device, int32[batch]: valid positions (a count, not count-1)
 */
typedef struct cpk_kv_cache {
    void *k;
    void *v;
    int32_t *seqlens_k;
    int32_t batch;
    int32_t kv_heads;
    int32_t capacity;
    int32_t head_dim;
    int32_t dtype;
} cpk_kv_cache;

/* ------------------------------------------------------------ host logic */

/*
 * Query-axis padding ladder (ONNX GenAI Wiki "Chunked Prefill", sections 4
 * and 6): three equally spaced widths at or below the chunk width W, the
 * step rounded up so that the top rung is W itself -- {171, 342, 512} for
 * W = 512.  Writes the distinct rungs in increasing order to out[0..*n).
 * out must hold 3 ints.  CPK_EINVAL if W < 1 or a pointer is NULL.
 */
int cpk_ladder_rungs(int W, int *out, int *n);

/*
 * Smallest rung of the ladder of W that holds `rows` real rows; rows equal
 * to a rung are not padded.  CPK_EINVAL if W < 1, rows < 1 or rows > W.
 */
int cpk_ladder_width(int W, int rows, int *width);

/*
 * Split an L-token prompt into W-row chunks, the last one taking the
 * remainder (same page, sections 2 and 3): chunk i starts at past[i] and
 * holds rows[i] rows.  max is the capacity of past/rows; *n receives the
 * chunk count.  CPK_EINVAL if L < 0, W < 1 or max is too small.
 */
int cpk_split_chunks(int L, int W, int32_t *past, int32_t *rows, int max, int *n);

/*
 * Token-budget step rule (Ultralytics glossary "Chunked Prefill", section
 * on how chunked prefill works): every running decode gets one row first,
 * the waiting prompt fills what is left:
 *   *prompt_rows = max(0, min(budget - n_decode, prompt_remaining)).
 * CPK_EINVAL if an argument is negative or n_decode > budget.
 */
int cpk_plan_step(int budget, int n_decode, int prompt_remaining, int *prompt_rows);

/* -------------------------------------------------------- device calls */

/*
 * Append `rows` positions to sequence b at [past_len, past_len + rows) from
 * the token-major rows k_new/v_new [real_rows][kv_heads][head_dim], then set
 * seqlens_k[b] = past_len + rows.  Positions past real_rows repeat the last
 * real row (query-axis padding, ONNX GenAI Wiki "Chunked Prefill", section
 * 4); real_rows == rows is a plain append.  Earlier positions are never
 * touched (same page, section 1.1).  A byte copy.
 * CPK_ECAPACITY if past_len + rows > capacity (a cache with no room left
 * can be read but not written); CPK_EINVAL if real_rows < 1,
 * real_rows > rows or b is out of range.
 */
int cpk_kv_append(const cpk_kv_cache *cache, int b, const void *k_new,
                  const void *v_new, int past_len, int rows, int real_rows,
                  void *stream);

/*
 * Causal attention of one chunk over sequence b's cache, which must already
 * hold the chunk's own K/V (append first).
 *   q    [real_rows][q_heads][head_dim].  `rows` rows are computed: row i
 *        sits at absolute position past_len + i and sees keys
 *        [0, past_len + i]; rows past real_rows repeat q's last row (the
 *        padded rows of ONNX GenAI Wiki "Chunked Prefill", section 4).
 *   out  [real_rows][q_heads][head_dim]: only the real rows are written
 *        (truncation, same section); padded rows are discarded.
 *   scale <= 0 selects 1/sqrt(head_dim).
 * CPK_EINVAL if real_rows > rows, real_rows < 1 or q_heads is not a
 * multiple of kv_heads; CPK_ECAPACITY if past_len + rows > capacity.
 */
int cpk_chunk_attention(const void *q, const cpk_kv_cache *cache, int b,
                        int q_heads, int past_len, int rows, int real_rows,
                        float scale, void *out, void *stream);

/*
 * Roll sequence b's logical length back to new_len (ONNX GenAI Wiki
 * "Chunked Prefill", section 4): seqlens_k[b] = new_len.  Bytes past it
 * are not cleared; the next append overwrites them.  cur_len is the
 * caller's host copy of the current length.  CPK_EINVAL if new_len < 0 or
 * new_len > cur_len.
 */
int cpk_rewind(const cpk_kv_cache *cache, int b, int new_len, int cur_len,
               void *stream);

/*
 * Prompt-prefix reuse (the prompt caching the Ultralytics glossary "Chunked
 * Prefill" lists among related serving techniques): copy positions
 * [0, len) of every KV head from slot src_slot to slot dst_slot of the same
 * cache and set seqlens_k[dst_slot] = len; a chunked prefill of the rest of
 * the prompt then starts at past_len = len and never recomputes the prefix.
 * (A paged cache shares prefix blocks between block tables instead.)
 * CPK_EINVAL if a slot is out of range, src == dst, or len is outside
 * [0, capacity].
 */
int cpk_kv_copy_prefix(const cpk_kv_cache *cache, int src_slot, int dst_slot, int len,
                       void *stream);

/*
 * One padded prefill forward in a single call (ONNX GenAI Wiki "Chunked
 * Prefill", section 4): round real_rows up the ladder of W (pad != 0) or
 * not (pad == 0, the page's switch that turns padding off); widen q, k and
 * v by repeating their last real row; append every padded row; attend
 * every padded row; write the real rows to out; rewind the cache to
 * past_len + real_rows.  q [real_rows][q_heads][D], k/v
 * [real_rows][kv_heads][D], out [real_rows][q_heads][D].  Same result
 * (output bits, cache bytes, seqlens_k) as cpk_kv_append(rows = width) +
 * cpk_chunk_attention(rows = width) + cpk_rewind(past_len + real_rows).
 * bf16/fp16 run as one launch: the attention kernel reads the chunk's own
 * keys from k/v and writes them to the cache itself (fused append); fp32
 * runs as an append launch that records the true length plus an attention
 * launch.  The padding is an index clamp inside the kernels, so no scratch
 * memory is used.  k and v must not overlap the cache.
 * *issued_rows (may be NULL) receives the padded width.
 * CPK_EINVAL if real_rows < 1 or real_rows > W; CPK_ECAPACITY if the
 * padded rows do not fit.
 */
int cpk_prefill_chunk(const void *q, const void *k, const void *v,
                      const cpk_kv_cache *cache, int b, int q_heads,
                      int past_len, int real_rows, int W, int pad, float scale,
                      void *out, int *issued_rows, void *stream);

/*
 * Device workspace bytes cpk_varlen_step needs for a step of n_seqs
 * sequences whose longest decode context (keys a one-row sequence reads)
 * is max_ctx: n_seqs * q_heads * ceil(max_ctx / 256) * (head_dim + 4) * 4,
 * one fp32 record (running max, sum, partial output) per query head and
 * 256-key slice of a decode row's context.
 */
size_t cpk_varlen_workspace_size(int n_seqs, int q_heads, int max_ctx,
                                 int head_dim);

/*
 * One packed mixed step under a token budget (Ultralytics glossary
 * "Chunked Prefill", section on how chunked prefill works): sequence s owns
 * packed rows [cu_rows[s], cu_rows[s+1]) of q [total_rows][q_heads][D] and
 * k_new/v_new [total_rows][kv_heads][D], sits in cache slot slots[s] and
 * has past_lens[s] positions cached.  Every sequence appends its rows and
 * attends them causally; a one-row sequence (a decode row) is computed by
 * the split-KV decode path.  out is [total_rows][q_heads][D].
 *   slots, cu_rows, past_lens   device int32 arrays (drive the kernels)
 *   h_cu_rows, h_past_lens      host copies (validation, launch geometry)
 *   ws / ws_bytes               device workspace, at least
 *                               cpk_varlen_workspace_size(...) bytes
 * Slots must be distinct.  CPK_ECAPACITY if a sequence's rows do not fit;
 * CPK_EWORKSPACE if the workspace is too small.
 */
int cpk_varlen_step(const void *q, const void *k_new, const void *v_new,
                    const cpk_kv_cache *cache, const int32_t *slots,
                    const int32_t *cu_rows, const int32_t *past_lens,
                    const int32_t *h_slots, const int32_t *h_cu_rows,
                    const int32_t *h_past_lens, int n_seqs, int total_rows,
                    int q_heads, float scale, void *out, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step as cpk_varlen_step, with the same arguments, validation and results
 * bit for bit, but the decode partials go to a static device array of
 * CPK_NOALLOC_SCRATCH_BYTES (96 MiB) that the library holds on every GPU it
 * runs on until the process ends, instead of a caller workspace.  The call
 * allocates nothing.  CPK_EWORKSPACE if the step's decode partials
 * (cpk_varlen_workspace_size) exceed that size; CPK_EHIP if the array's
 * address cannot be taken on the current device.  Every call on one GPU
 * shares its array, so calls that overlap on one GPU (two streams or two
 * threads) race; serialize them.
 */
#define CPK_NOALLOC_SCRATCH_BYTES (96ull << 20)
int cpk_varlen_step_noalloc(const void *q, const void *k_new, const void *v_new,
                            const cpk_kv_cache *cache, const int32_t *slots,
                            const int32_t *cu_rows, const int32_t *past_lens,
                            const int32_t *h_slots, const int32_t *h_cu_rows,
                            const int32_t *h_past_lens, int n_seqs, int total_rows,
                            int q_heads, float scale, void *out, void *stream);

/*
 * cpk_varlen_step restricted to the given phases (a nonzero subset of
 * CPK_PHASE_ALL), with the same arguments, validation and errors.  The
 * decode and prefill phases read the cache after the append and write
 * disjoint output rows (decode also the workspace), so a caller may run
 * APPEND | DECODE on one stream and PREFILL on a second stream that waits
 * for the first's append; cpk_varlen_step is all three on one stream.  The
 * outputs are bit-identical either way.
 */
int cpk_varlen_step_phases(const void *q, const void *k_new, const void *v_new,
                           const cpk_kv_cache *cache, const int32_t *slots,
                           const int32_t *cu_rows, const int32_t *past_lens,
                           const int32_t *h_slots, const int32_t *h_cu_rows,
                           const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                           float scale, void *out, void *ws, size_t ws_bytes, int phases,
                           void *stream);

/*
 * Rolling fixed-capacity cache step (Horizon developer blog "Chunk
 * Prefill", section 3): new = cat(old, chunk)[c:] along positions, for K
 * and V.  Out of place: k_new/v_new must not overlap k_old/v_old (the
 * caller swaps buffers between chunks).
 *   k_old, v_old, k_new, v_new   [B][H][C][D]
 *   k_chunk, v_chunk             [B][c][H][D] token-major
 * CPK_EINVAL if c < 1, c > C or the buffers overlap.
 */
int cpk_roll_append(const void *k_old, const void *v_old, const void *k_chunk,
                    const void *v_chunk, void *k_new, void *v_new, int B,
                    int H, int C, int c, int D, int dtype, void *stream);

/*
 * Attention of one chunk over a right-aligned rolling cache (Horizon
 * developer blog "Chunk Prefill", section 4).  k, v [Hkv][C][D] hold
 * absolute positions [abs_end - C, abs_end) right-aligned (slot s holds
 * position abs_end - C + s); q [c][Hq][D] holds positions
 * [abs_end - c, abs_end).  Slot s is visible to query row i iff its
 * position a satisfies n_leftpad <= a <= abs_end - c + i.
 *   mask  NULL: the rule above is evaluated in the kernel (masked slots
 *         are skipped); or a (c, C) additive mask of the call's dtype
 *         (0 visible, -32768 masked) added to the scaled scores.  For
 *         every row that sees at least one slot both forms give the same
 *         bits.
 *   out   [c][Hq][D]
 *   ws    NULL, or device workspace of at least
 *         cpk_roll_workspace_size(...) bytes (owned by the caller, 16-byte
 *         aligned, no initial contents needed).  With a workspace the key
 *         range is split across workgroups (a chunk of c rows over C slots
 *         otherwise occupies only (c / rows per block) x Hkv workgroups) and
 *         the parts are merged in a fixed order by a second launch; the
 *         result then differs from the unsplit one only by rounding.  Both
 *         mask forms of one call split identically.
 * CPK_EINVAL if c > C, abs_end < c or the sizes are inconsistent;
 * CPK_EWORKSPACE if ws is too small.
 */
int cpk_roll_attention(const void *q, const void *k, const void *v,
                       const void *mask, int abs_end, int n_leftpad, int Hq,
                       int Hkv, int C, int c, int D, int dtype, float scale,
                       void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * A paged KV cache for the packed mixed step: K and V pools of fixed-size
 * blocks, and per sequence slot a table of block ids (paged attention, one
 * of the serving techniques the Ultralytics glossary "Chunked Prefill" lists
 * beside chunked prefill: a prompt prefilled over several steps grows its
 * cache block by block instead of reserving its whole length up front; and
 * shared prefix blocks give the prompt-prefix reuse listed there too).
 * Position p of slot s lives in block block_table[s * max_blocks +
 * p / block_size] at row p % block_size.  Blocks may be shared between
 * slots (a common prefix is then stored once); appends write only the
 * blocks of the positions they append.
 *   k, v        device pools [n_blocks][kv_heads][block_size][head_dim]
 *   block_table device int32 [batch][max_blocks]; entries for the positions
 *               a call touches must name blocks in [0, n_blocks) (the
 *               kernels clamp out-of-range ids, so a bad table gives wrong
 *               values, never an access outside the pools)
 *   seqlens_k   device int32 [batch]
 *   block_size  a positive multiple of 256 (a key tile or decode segment
 *               never crosses a block)
 * A slot's capacity is max_blocks * block_size; max_blocks is at most 512
 * (the attention kernels stage a workgroup's table entries on chip).  bf16
 * and fp16 only.
 */
typedef struct cpk_paged_cache {
    void *k;
    void *v;
    int32_t *block_table;
    int32_t *seqlens_k;
    int32_t batch;
    int32_t kv_heads;
    int32_t block_size;
    int32_t n_blocks;
    int32_t max_blocks;
    int32_t head_dim;
    int32_t dtype;
} cpk_paged_cache;

/*
 * cpk_varlen_step_phases over a paged cache: same arguments, phases,
 * workspace and results (bit for bit, given the same contents at the same
 * positions) as over a contiguous cache.  CPK_EINVAL for a NULL table,
 * block_size not a positive multiple of 256, non-positive counts or
 * max_blocks above 512; CPK_EDTYPE for fp32.
 */
int cpk_paged_varlen_step(const void *q, const void *k_new, const void *v_new,
                          const cpk_paged_cache *cache, const int32_t *slots,
                          const int32_t *cu_rows, const int32_t *past_lens,
                          const int32_t *h_slots, const int32_t *h_cu_rows,
                          const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                          float scale, void *out, void *ws, size_t ws_bytes, int phases,
                          void *stream);

/*
 * Rolling cache as a ring buffer (the rolling cache of the Horizon developer
 * blog "Chunk Prefill", sections 3 and 4, without the O(C) shift per chunk).
 * A ring of C physical slots per (batch, head), [B][H][C][D], and a start
 * index: logical slot s (0 = oldest, C-1 = newest) of the literal shifted
 * cache cat(old, chunk)[c:] is physical slot (start + s) mod C.  The caller
 * keeps start; a ring that starts zeroed with start = 0 matches a literal
 * cache that starts zeroed.
 *
 * cpk_ring_append writes the c chunk rows ([B][c][H][D]) over the c oldest
 * slots, physical (start + t) mod C for row t; the caller then sets
 * start = (start + c) mod C, after which the logical view equals the
 * literal shift byte for byte.  O(c) bytes moved instead of O(C).
 * CPK_EINVAL if c > C, start outside [0, C), or a chunk overlaps a ring.
 */
int cpk_ring_append(const void *k_chunk, const void *v_chunk, void *k_ring, void *v_ring,
                    int B, int H, int C, int c, int D, int dtype, int start, void *stream);

/*
 * cpk_roll_attention over a ring (batch 1: k_ring / v_ring [Hkv][C][D]) whose
 * logical slot 0 is physical slot `start` (the value after the chunk's
 * append).  Keys are visited in logical order, so the result is bit-identical
 * to cpk_roll_attention over the literal shifted cache; mask, workspace and
 * errors as there, plus CPK_EINVAL if start is outside [0, C).
 */
int cpk_ring_attention(const void *q, const void *k_ring, const void *v_ring,
                       const void *mask, int abs_end, int n_leftpad, int Hq, int Hkv,
                       int C, int c, int D, int dtype, float scale, int start, void *out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * One rolling chunk over a ring in one launch (batch 1): the result of
 * cpk_ring_append(k_chunk, v_chunk, k_ring, v_ring, 1, Hkv, C, c, D, dtype,
 * start) followed by cpk_ring_attention(..., start = (start + c) mod C),
 * bit for bit in the output and in both rings.  The chunk's rows
 * (token-major [c][Hkv][D]) are the keys of the last c logical slots: the
 * attention kernel reads them from the chunk and writes them over the c
 * oldest ring slots, which no query of this chunk sees, so the write and
 * the reads never meet.  The caller advances start by c afterwards.  fp32
 * runs the append and the attention as two launches.  The rolling cache
 * step and its attention: Horizon developer blog "Chunk Prefill", sections
 * 3 and 4.  Errors: those of both calls, all checked before anything is
 * launched (CPK_EINVAL if a chunk overlaps a ring or the rings overlap).
 */
int cpk_ring_step(const void *q, const void *k_chunk, const void *v_chunk, void *k_ring,
                  void *v_ring, const void *mask, int abs_end, int n_leftpad, int Hq, int Hkv,
                  int C, int c, int D, int dtype, float scale, int start, void *out, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * cpk_ring_step with the merge of its key-range parts carried into the
 * next chunk's launch (the same rolling step, Horizon developer blog
 * "Chunk Prefill", sections 3 and 4, run as a pipeline over the chunks):
 * the launch appends the chunk and leaves this chunk's parts unmerged in
 * ws (out is not written yet), and, with prev_ws set, merges the parts an
 * earlier deferred call of the same shapes left in prev_ws into that
 * call's out, passed here as prev_out.  The chunk's output is complete
 * once the next deferred call (or cpk_roll_flush(ws, out)) has run on the
 * same stream; it is bit-identical to cpk_ring_step's.  A chain of calls
 * alternates two workspaces (each cpk_roll_workspace_size bytes): call j
 * writes ws_j and merges ws_(j-1).  Only shapes that split the key range
 * (bf16/fp16, cpk_roll_workspace_size > 0) are deferred.  Errors: those of
 * cpk_ring_step, all checked before anything is launched; CPK_EINVAL if
 * the shapes do not split or ws is NULL, if prev_ws is set without
 * prev_out, if prev_ws overlaps ws, or if prev_out overlaps q, a chunk, a
 * ring, the mask, ws or prev_ws; CPK_EALIGN if prev_ws or prev_out is not
 * 16-byte aligned.  The caller keeps prev_ws's shapes equal to this call's.
 */
int cpk_ring_step_deferred(const void *q, const void *k_chunk, const void *v_chunk,
                           void *k_ring, void *v_ring, const void *mask, int abs_end,
                           int n_leftpad, int Hq, int Hkv, int C, int c, int D, int dtype,
                           float scale, int start, void *out, void *ws, size_t ws_bytes,
                           const void *prev_ws, void *prev_out, void *stream);

/*
 * cpk_roll_attention over the literal shifted cache with the same carried
 * merge as cpk_ring_step_deferred (Horizon developer blog "Chunk Prefill",
 * section 4, run as a pipeline over the chunks): this chunk's parts stay in
 * ws, and the parts a previous deferred call of the same shapes left in
 * prev_ws are merged into prev_out by this launch; bit-identical to
 * cpk_roll_attention once merged.  Errors: those of cpk_roll_attention,
 * all checked before anything is launched; CPK_EINVAL if the shapes do not
 * split or ws is NULL, if prev_ws is set without prev_out, if prev_ws
 * overlaps ws, or if prev_out overlaps q, k, v, the mask, ws or prev_ws;
 * CPK_EALIGN if prev_ws or prev_out is not 16-byte aligned.
 */
int cpk_roll_attention_deferred(const void *q, const void *k, const void *v, const void *mask,
                                int abs_end, int n_leftpad, int Hq, int Hkv, int C, int c, int D,
                                int dtype, float scale, void *out, void *ws, size_t ws_bytes,
                                const void *prev_ws, void *prev_out, void *stream);

/*
 * The merge a deferred rolling call (cpk_ring_step_deferred or
 * cpk_roll_attention_deferred) left pending: the parts in ws, written with
 * these shapes, merged into out [c][Hq][D] (one combine launch).
 * CPK_EINVAL if the shapes do not split, a buffer is NULL or out overlaps
 * ws; CPK_EWORKSPACE if ws_bytes is below cpk_roll_workspace_size;
 * CPK_EALIGN if ws or out is not 16-byte aligned.
 */
int cpk_roll_flush(const void *ws, size_t ws_bytes, void *out, int Hq, int Hkv, int C, int c,
                   int D, int dtype, void *stream);

/*
 * The logical view of a ring as a contiguous cache: out slot s = physical
 * slot (start + s) mod C, for K and V, [B][H][C][D] each (interoperation
 * and checks; not on the per-chunk path).  CPK_EINVAL if start is outside
 * [0, C) or an output overlaps an input.
 */
int cpk_ring_view(const void *k_ring, const void *v_ring, void *k_out, void *v_out, int B,
                  int H, int C, int D, int dtype, int start, void *stream);

/*
 * Workspace bytes cpk_roll_attention uses for a split key range with these
 * shapes: parts x c x Hq x (head_dim + 4) x 4 (one fp32 record per part,
 * row and query head: running maximum, sum, two pad words, the partial
 * output).  0 when the shapes are not split (fp32, or enough workgroups
 * without splitting); a call may then pass ws = NULL.
 */
size_t cpk_roll_workspace_size(int Hq, int Hkv, int C, int c, int head_dim,
                               int dtype);

/* ------------------------------------------------------------ diagnostics */

/* Message for the last failing call on this thread ("" if none). */
const char *cpk_last_error(void);

/* Library ABI version (major * 100 + minor). */
int cpk_version(void);

/*
 * Which bf16/fp16 kernel serves chunk attention (cpk_chunk_attention,
 * cpk_prefill_chunk) and the prompt rows of cpk_varlen_step; fp32 is
 * unaffected, and the rolling forms (cpk_roll_attention, cpk_ring_*)
 * always take the narrow kernel (only CPK_ATTN_NARROW_GENERAL applies to
 * them).  Both kernels compute the same attention to within rounding; each
 * alone is deterministic and gives a row the same bits whether its prompt
 * runs in one pass or in chunks.  CPK_ATTN_AUTO takes the wide kernel when
 * its launch has at least as many workgroups as the GPU has compute units
 * (256) and at least 24 x 2^20 visible (row, key) pairs per query head
 * (rows x past + rows x (rows + 1) / 2, summed over a varlen launch's
 * prompt sequences), else the narrow one.  The narrow kernel runs in a latency-scheduled
 * form wherever the launch reads a contiguous cache (causal, computed or
 * explicit-mask visibility, ring buffer, key split) and in its general form
 * over a paged pool; the two forms give identical bits, and
 * CPK_ATTN_NARROW_GENERAL forces the general form.  The setting is
 * process-wide and meant for diagnostics and tests; it returns the previous
 * setting, or CPK_EINVAL for an unknown kind.
 */
int cpk_set_attention_kernel(int kind);

/*
 * Name and compute-unit count of the current HIP device.  name receives at
 * most name_len bytes including the terminator.  CPK_EHIP if no device.
 */
int cpk_device_info(char *name, int name_len, int *compute_units);

#ifdef __cplusplus
}
#endif

#endif /* CPK_H */
