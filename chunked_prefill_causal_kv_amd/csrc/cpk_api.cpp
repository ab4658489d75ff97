// C-ABI entry points: argument validation, host logic (ladder, chunk split,
// step planner) and kernel dispatch.  Every check runs before any launch, so
// a call that fails writes no device memory.
#include "../../include/cpk.h"
#include "cpk_internal.h"

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return CPK_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(CPK_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

// status and message for the other translation units' entry points
int cpk::fail_status(int code, const char *msg) { return fail(code, "%s", msg); }

namespace {

int elem_size(int dtype)
{
    return dtype == CPK_F32 ? 4 : (dtype == CPK_F16 || dtype == CPK_BF16) ? 2 : 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_dtype_dim(int dtype, int D)
{
    if (elem_size(dtype) == 0) return fail(CPK_EDTYPE, "unknown dtype %d", dtype);
    if (D != 64 && D != 128) return fail(CPK_EDTYPE, "head_dim %d not supported (64 or 128)", D);
    return CPK_OK;
}

int check_cache(const cpk_kv_cache *c)
{
    if (!c) return fail(CPK_EINVAL, "cache is NULL");
    if (!c->k || !c->v || !c->seqlens_k) return fail(CPK_EINVAL, "cache pointers must be set");
    if (c->batch < 1 || c->kv_heads < 1 || c->capacity < 1)
        return fail(CPK_EINVAL, "cache sizes must be positive");
    int r = check_dtype_dim(c->dtype, c->head_dim);
    if (r) return r;
    if (!aligned16(c->k) || !aligned16(c->v)) return fail(CPK_EALIGN, "cache k/v not 16-byte aligned");
    if (((uintptr_t)c->seqlens_k & 3u) != 0) return fail(CPK_EALIGN, "seqlens_k not 4-byte aligned");
    return CPK_OK;
}

int check_heads(int Hq, int Hkv)
{
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(CPK_EINVAL, "q_heads %d must be a positive multiple of kv_heads %d", Hq, Hkv);
    if (Hq / Hkv > 64) return fail(CPK_EINVAL, "group size %d above 64", Hq / Hkv);
    return CPK_OK;
}

float resolve_scale(float scale, int D)
{
    return scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
}

void fill_scale(cpk::AttnArgs &a, float scale)
{
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
}

int ladder_width_impl(int W, int rows)
{
    const int step = (W + 2) / 3;
    for (int i = 1; i <= 3; ++i) {
        const int r = i * step < W ? i * step : W;
        if (r >= rows) return r;
    }
    return W;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

std::atomic<int> g_attn_kernel{CPK_ATTN_AUTO};

// The kernel serving a bf16/fp16 chunk or varlen attention launch of `rows`
// rows (the longest sequence's, in varlen) and `pairs` visible (row, key)
// pairs per query head (summed over the launch's sequences): the 128-column
// kernel once its grid fills the CUs and the launch is long enough to
// amortise its per-workgroup fixed cost, else the 64-column one (unless
// overridden).
int pick_kernel(int dtype, int group, int kv_heads, int rows, int64_t pairs)
{
    if (dtype == CPK_F32) return cpk::kAttnNarrow;
    const int k = g_attn_kernel.load(std::memory_order_relaxed);
    if (k == CPK_ATTN_WIDE) return cpk::kAttnWide;
    if (k == CPK_ATTN_NARROW) return cpk::kAttnNarrow;
    if (k == CPK_ATTN_NARROW_GENERAL) return cpk::kAttnNarrowGeneral;
    const int br = cpk::attn_rows_per_block(dtype, group, true);
    const bool fills = (int64_t)((rows + br - 1) / br) * kv_heads >= cpk::kWideMinGroups;
    return fills && pairs >= cpk::kWideMinPairs ? cpk::kAttnWide : cpk::kAttnNarrow;
}

// Visible (row, key) pairs per query head of `rows` causal rows after `past` keys.
int64_t causal_pairs(int past, int rows)
{
    return (int64_t)rows * past + (int64_t)rows * (rows + 1) / 2;
}

}  // namespace

extern "C" {

int cpk_version(void) { return 103; }

int cpk_set_attention_kernel(int kind)
{
    if (kind != CPK_ATTN_AUTO && kind != CPK_ATTN_NARROW && kind != CPK_ATTN_WIDE &&
        kind != CPK_ATTN_NARROW_GENERAL)
        return fail(CPK_EINVAL, "set_attention_kernel: unknown kind %d", kind);
    return g_attn_kernel.exchange(kind);
}

const char *cpk_last_error(void) { return g_err.c_str(); }

int cpk_device_info(char *name, int name_len, int *compute_units)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    if (name && name_len > 0) snprintf(name, (size_t)name_len, "%s", prop.gcnArchName);
    if (compute_units) *compute_units = prop.multiProcessorCount;
    return ok();
}

int cpk_ladder_rungs(int W, int *out, int *n)
{
    if (W < 1 || !out || !n) return fail(CPK_EINVAL, "ladder: W=%d must be >= 1", W);
    const int step = (W + 2) / 3;
    int cnt = 0;
    for (int i = 1; i <= 3; ++i) {
        const int r = i * step < W ? i * step : W;
        if (cnt == 0 || out[cnt - 1] != r) out[cnt++] = r;
    }
    *n = cnt;
    return ok();
}

int cpk_ladder_width(int W, int rows, int *width)
{
    if (!width) return fail(CPK_EINVAL, "width is NULL");
    if (W < 1 || rows < 1 || rows > W)
        return fail(CPK_EINVAL, "ladder: rows=%d outside [1, W=%d]", rows, W);
    *width = ladder_width_impl(W, rows);
    return ok();
}

int cpk_split_chunks(int L, int W, int32_t *past, int32_t *rows, int max, int *n)
{
    if (L < 0 || W < 1 || !n) return fail(CPK_EINVAL, "split: L=%d W=%d", L, W);
    const int need = (L + W - 1) / W;
    *n = need;
    if (need > max || (need > 0 && (!past || !rows)))
        return fail(CPK_EINVAL, "split: %d chunks do not fit max=%d", need, max);
    for (int i = 0; i < need; ++i) {
        past[i] = i * W;
        rows[i] = (L - i * W) < W ? (L - i * W) : W;
    }
    return ok();
}

int cpk_plan_step(int budget, int n_decode, int prompt_remaining, int *prompt_rows)
{
    if (!prompt_rows || budget < 0 || n_decode < 0 || prompt_remaining < 0 || n_decode > budget)
        return fail(CPK_EINVAL, "plan: budget=%d n_decode=%d remaining=%d", budget, n_decode,
                    prompt_remaining);
    const int room = budget - n_decode;
    *prompt_rows = room < prompt_remaining ? room : prompt_remaining;
    return ok();
}

int cpk_kv_append(const cpk_kv_cache *cache, int b, const void *k_new, const void *v_new,
                  int past_len, int rows, int real_rows, void *stream)
{
    int r = check_cache(cache);
    if (r) return r;
    if (b < 0 || b >= cache->batch) return fail(CPK_EINVAL, "append: b=%d out of range", b);
    if (!k_new || !v_new) return fail(CPK_EINVAL, "append: NULL input");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(CPK_EALIGN, "append: input not aligned");
    if (past_len < 0 || rows < 1 || real_rows < 1 || real_rows > rows)
        return fail(CPK_EINVAL, "append: past_len=%d rows=%d real_rows=%d", past_len, rows,
                    real_rows);
    if ((int64_t)past_len + rows > cache->capacity)
        return fail(CPK_ECAPACITY, "append: %d + %d rows exceed capacity %d", past_len, rows,
                    cache->capacity);
    const int rb = cache->head_dim * elem_size(cache->dtype);
    return hip_status(cpk::launch_kv_append(k_new, v_new, cache->k, cache->v, cache->seqlens_k,
                                            cache->kv_heads, cache->capacity, rb, b, past_len,
                                            rows, real_rows, past_len + rows, (hipStream_t)stream),
                      "kv_append launch");
}

// Chunk attention; with k_new / v_new set (bf16/fp16 only) the kernel also
// performs the chunk's append (fused): it reads the chunk's own keys from
// the new rows, writes them to the cache (padded rows repeat the last real
// row) and sets seqlens_k[b] = past_len + real_rows.
static int attention_common(const void *q, const cpk_kv_cache *cache, int b, int q_heads,
                            int past_len, int rows, int real_rows, float scale, void *out,
                            hipStream_t st, const void *k_new = nullptr,
                            const void *v_new = nullptr)
{
    int r = check_cache(cache);
    if (r) return r;
    if ((r = check_heads(q_heads, cache->kv_heads))) return r;
    if (b < 0 || b >= cache->batch) return fail(CPK_EINVAL, "attention: b=%d out of range", b);
    if (!q || !out) return fail(CPK_EINVAL, "attention: NULL q/out");
    if (!aligned16(q) || !aligned16(out)) return fail(CPK_EALIGN, "attention: q/out not aligned");
    if (rows < 1 || real_rows < 1 || real_rows > rows || past_len < 0)
        return fail(CPK_EINVAL, "attention: rows=%d real_rows=%d past_len=%d", rows, real_rows,
                    past_len);
    if ((int64_t)past_len + rows > cache->capacity)
        return fail(CPK_ECAPACITY, "attention: %d + %d rows exceed capacity %d", past_len, rows,
                    cache->capacity);
    cpk::AttnArgs a = {};
    a.q = q; a.k = cache->k; a.v = cache->v; a.out = out; a.mask = nullptr;
    a.Hq = q_heads; a.Hkv = cache->kv_heads; a.D = cache->head_dim; a.cap = cache->capacity;
    fill_scale(a, resolve_scale(scale, a.D));
    a.slot = b; a.q_row0 = 0; a.out_row0 = 0; a.rows = rows; a.q_src_rows = real_rows;
    a.out_rows = real_rows; a.n_keys = past_len + rows; a.key_lo = 0; a.causal_base = past_len;
    if (k_new) {
        a.k_new = k_new; a.v_new = v_new; a.new_base = past_len; a.new_rows = real_rows;
        a.seqlens = cache->seqlens_k; a.len_after = past_len + real_rows;
    }
    const int kern = pick_kernel(cache->dtype, q_heads / cache->kv_heads, cache->kv_heads, rows,
                                 causal_pairs(past_len, rows));
    const int br = cpk::attn_rows_per_block(cache->dtype, q_heads / cache->kv_heads,
                                            kern == cpk::kAttnWide);
    return hip_status(cpk::launch_attention(a, cache->dtype, (rows + br - 1) / br, 1, kern, st),
                      "attention launch");
}

int cpk_chunk_attention(const void *q, const cpk_kv_cache *cache, int b, int q_heads,
                        int past_len, int rows, int real_rows, float scale, void *out,
                        void *stream)
{
    return attention_common(q, cache, b, q_heads, past_len, rows, real_rows, scale, out,
                            (hipStream_t)stream);
}

int cpk_kv_copy_prefix(const cpk_kv_cache *cache, int src_slot, int dst_slot, int len,
                       void *stream)
{
    int r = check_cache(cache);
    if (r) return r;
    if (src_slot < 0 || src_slot >= cache->batch || dst_slot < 0 || dst_slot >= cache->batch ||
        src_slot == dst_slot)
        return fail(CPK_EINVAL, "copy_prefix: slots %d -> %d (batch %d)", src_slot, dst_slot,
                    cache->batch);
    if (len < 0 || len > cache->capacity)
        return fail(CPK_EINVAL, "copy_prefix: len=%d outside [0, capacity %d]", len,
                    cache->capacity);
    return hip_status(cpk::launch_kv_copy_prefix(cache->k, cache->v, cache->seqlens_k,
                                                 cache->kv_heads, cache->capacity,
                                                 cache->head_dim * elem_size(cache->dtype),
                                                 src_slot, dst_slot, len, (hipStream_t)stream),
                      "copy_prefix launch");
}

int cpk_rewind(const cpk_kv_cache *cache, int b, int new_len, int cur_len, void *stream)
{
    int r = check_cache(cache);
    if (r) return r;
    if (b < 0 || b >= cache->batch) return fail(CPK_EINVAL, "rewind: b=%d out of range", b);
    if (new_len < 0 || new_len > cur_len || cur_len > cache->capacity)
        return fail(CPK_EINVAL, "rewind: new_len=%d cur_len=%d", new_len, cur_len);
    return hip_status(cpk::launch_set_len(cache->seqlens_k, b, new_len, (hipStream_t)stream),
                      "rewind launch");
}

int cpk_prefill_chunk(const void *q, const void *k, const void *v, const cpk_kv_cache *cache,
                      int b, int q_heads, int past_len, int real_rows, int W, int pad,
                      float scale, void *out, int *issued_rows, void *stream)
{
    int r = check_cache(cache);
    if (r) return r;
    if (W < 1 || real_rows < 1 || real_rows > W)
        return fail(CPK_EINVAL, "prefill_chunk: real_rows=%d outside [1, W=%d]", real_rows, W);
    if (!k || !v) return fail(CPK_EINVAL, "prefill_chunk: NULL k/v");
    if (!aligned16(k) || !aligned16(v)) return fail(CPK_EALIGN, "prefill_chunk: k/v not aligned");
    const int width = pad ? ladder_width_impl(W, real_rows) : real_rows;
    // validate everything the three launches need before the first one
    if ((r = check_heads(q_heads, cache->kv_heads))) return r;
    if (b < 0 || b >= cache->batch) return fail(CPK_EINVAL, "prefill_chunk: b=%d out of range", b);
    if (!q || !out) return fail(CPK_EINVAL, "prefill_chunk: NULL q/out");
    if (!aligned16(q) || !aligned16(out)) return fail(CPK_EALIGN, "prefill_chunk: q/out not aligned");
    if (past_len < 0) return fail(CPK_EINVAL, "prefill_chunk: past_len=%d", past_len);
    if ((int64_t)past_len + width > cache->capacity)
        return fail(CPK_ECAPACITY, "prefill_chunk: %d + %d padded rows exceed capacity %d",
                    past_len, width, cache->capacity);
    hipStream_t st = (hipStream_t)stream;
    if (cache->dtype != CPK_F32) {
        // one launch: the attention kernel appends the chunk itself (it
        // reads the chunk's keys from k/v, writes the padded rows to the
        // cache and records the true length past_len + real_rows)
        r = attention_common(q, cache, b, q_heads, past_len, width, real_rows, scale, out, st,
                             k, v);
        if (r) return r;
        if (issued_rows) *issued_rows = width;
        return ok();
    }
    const int rb = cache->head_dim * elem_size(cache->dtype);
    // the append writes the padded rows but records the true length
    // past_len + real_rows (the rewind of the padding, folded into the copy;
    // attention takes its key range from its arguments, not from seqlens_k)
    r = hip_status(cpk::launch_kv_append(k, v, cache->k, cache->v, cache->seqlens_k,
                                         cache->kv_heads, cache->capacity, rb, b, past_len, width,
                                         real_rows, past_len + real_rows, st),
                   "prefill_chunk append");
    if (r) return r;
    r = attention_common(q, cache, b, q_heads, past_len, width, real_rows, scale, out, st);
    if (r) return r;
    if (issued_rows) *issued_rows = width;
    return ok();
}

size_t cpk_varlen_workspace_size(int n_seqs, int q_heads, int max_ctx, int head_dim)
{
    if (n_seqs < 1 || q_heads < 1 || head_dim < 1) return 0;
    const int segs = max_ctx < 1 ? 1 : (max_ctx + cpk::kDecodeSeg - 1) / cpk::kDecodeSeg;
    return (size_t)n_seqs * (size_t)q_heads * (size_t)segs * (size_t)(head_dim + 4) * sizeof(float);
}

int cpk_varlen_step(const void *q, const void *k_new, const void *v_new,
                    const cpk_kv_cache *cache, const int32_t *slots, const int32_t *cu_rows,
                    const int32_t *past_lens, const int32_t *h_slots, const int32_t *h_cu_rows,
                    const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                    float scale, void *out, void *ws, size_t ws_bytes, void *stream)
{
    return cpk_varlen_step_phases(q, k_new, v_new, cache, slots, cu_rows, past_lens, h_slots,
                                  h_cu_rows, h_past_lens, n_seqs, total_rows, q_heads, scale,
                                  out, ws, ws_bytes, CPK_PHASE_ALL, stream);
}

}  // extern "C"

// Block-table addressing of a paged pool (nullptr: contiguous cache).
struct Paging {
    const int32_t *table;
    int max_blocks, block_size, n_blocks;
};

static int varlen_impl(const void *q, const void *k_new, const void *v_new,
                       const cpk_kv_cache *cache, const Paging *pg, const int32_t *slots,
                       const int32_t *cu_rows, const int32_t *past_lens,
                       const int32_t *h_slots, const int32_t *h_cu_rows,
                       const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                       float scale, void *out, void *ws, size_t ws_bytes, int phases,
                       void *stream);

extern "C" {

int cpk_varlen_step_phases(const void *q, const void *k_new, const void *v_new,
                           const cpk_kv_cache *cache, const int32_t *slots,
                           const int32_t *cu_rows, const int32_t *past_lens,
                           const int32_t *h_slots, const int32_t *h_cu_rows,
                           const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                           float scale, void *out, void *ws, size_t ws_bytes, int phases,
                           void *stream)
{
    return varlen_impl(q, k_new, v_new, cache, nullptr, slots, cu_rows, past_lens, h_slots,
                       h_cu_rows, h_past_lens, n_seqs, total_rows, q_heads, scale, out, ws,
                       ws_bytes, phases, stream);
}

int cpk_paged_varlen_step(const void *q, const void *k_new, const void *v_new,
                          const cpk_paged_cache *pc, const int32_t *slots,
                          const int32_t *cu_rows, const int32_t *past_lens,
                          const int32_t *h_slots, const int32_t *h_cu_rows,
                          const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                          float scale, void *out, void *ws, size_t ws_bytes, int phases,
                          void *stream)
{
    if (!pc) return fail(CPK_EINVAL, "paged: cache is NULL");
    if (!pc->block_table) return fail(CPK_EINVAL, "paged: block_table is NULL");
    if (pc->block_size < 256 || pc->block_size % 256 != 0)
        return fail(CPK_EINVAL, "paged: block_size %d must be a positive multiple of 256",
                    pc->block_size);
    if (pc->n_blocks < 1 || pc->max_blocks < 1 || pc->max_blocks > cpk::kMaxTableBlocks)
        return fail(CPK_EINVAL, "paged: n_blocks=%d max_blocks=%d (at most %d blocks per sequence)",
                    pc->n_blocks, pc->max_blocks, cpk::kMaxTableBlocks);
    if ((int64_t)pc->max_blocks * pc->block_size > INT32_MAX / 2)
        return fail(CPK_EINVAL, "paged: max_blocks x block_size too large");
    if (pc->dtype == CPK_F32) return fail(CPK_EDTYPE, "paged: bf16 or fp16 only");
    if (((uintptr_t)pc->block_table & 3u) != 0)
        return fail(CPK_EALIGN, "paged: block_table not 4-byte aligned");
    cpk_kv_cache view = {};
    view.k = pc->k; view.v = pc->v; view.seqlens_k = pc->seqlens_k;
    view.batch = pc->batch; view.kv_heads = pc->kv_heads; view.head_dim = pc->head_dim;
    view.dtype = pc->dtype; view.capacity = pc->max_blocks * pc->block_size;
    const Paging pg = {pc->block_table, pc->max_blocks, pc->block_size, pc->n_blocks};
    return varlen_impl(q, k_new, v_new, &view, &pg, slots, cu_rows, past_lens, h_slots,
                       h_cu_rows, h_past_lens, n_seqs, total_rows, q_heads, scale, out, ws,
                       ws_bytes, phases, stream);
}

}  // extern "C"

static int varlen_impl(const void *q, const void *k_new, const void *v_new,
                       const cpk_kv_cache *cache, const Paging *pg, const int32_t *slots,
                       const int32_t *cu_rows, const int32_t *past_lens,
                       const int32_t *h_slots, const int32_t *h_cu_rows,
                       const int32_t *h_past_lens, int n_seqs, int total_rows, int q_heads,
                       float scale, void *out, void *ws, size_t ws_bytes, int phases,
                       void *stream)
{
    if (phases < 1 || (phases & ~CPK_PHASE_ALL))
        return fail(CPK_EINVAL, "varlen: phases=%d", phases);
    int r = check_cache(cache);
    if (r) return r;
    if ((r = check_heads(q_heads, cache->kv_heads))) return r;
    if (n_seqs < 1 || total_rows < 1) return fail(CPK_EINVAL, "varlen: n_seqs=%d total_rows=%d", n_seqs, total_rows);
    if (!q || !k_new || !v_new || !out || !slots || !cu_rows || !past_lens || !h_slots ||
        !h_cu_rows || !h_past_lens)
        return fail(CPK_EINVAL, "varlen: NULL argument");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return fail(CPK_EALIGN, "varlen: q/k/v/out not aligned");
    if (h_cu_rows[0] != 0 || h_cu_rows[n_seqs] != total_rows)
        return fail(CPK_EINVAL, "varlen: cu_rows must run from 0 to total_rows");
    std::vector<char> used((size_t)cache->batch, 0);
    int max_ctx = 0, max_rows = 0, n_dec = 0, n_pre = 0;
    int64_t pre_pairs = 0;   // visible pairs per head of the prompt rows
    int pre_lo = n_seqs, pre_hi = 0;   // range of the sequences with prompt rows
    const int G = q_heads / cache->kv_heads;
    const bool dec_ok = cpk::decode_supported(cache->dtype, cache->head_dim, G, cache->capacity);
    for (int s = 0; s < n_seqs; ++s) {
        const int rows = h_cu_rows[s + 1] - h_cu_rows[s];
        if (rows < 1) return fail(CPK_EINVAL, "varlen: sequence %d has %d rows", s, rows);
        const int slot = h_slots[s];
        if (slot < 0 || slot >= cache->batch) return fail(CPK_EINVAL, "varlen: slot %d out of range", slot);
        if (used[(size_t)slot]) return fail(CPK_EINVAL, "varlen: slot %d used twice", slot);
        used[(size_t)slot] = 1;
        const int past = h_past_lens[s];
        if (past < 0) return fail(CPK_EINVAL, "varlen: past_len %d", past);
        if ((int64_t)past + rows > cache->capacity)
            return fail(CPK_ECAPACITY, "varlen: sequence %d needs %d positions, capacity %d", s,
                        past + rows, cache->capacity);
        if (rows == 1 && dec_ok) {
            ++n_dec;
            if (past + 1 > max_ctx) max_ctx = past + 1;
        } else {
            ++n_pre;
            pre_pairs += causal_pairs(past, rows);
            if (rows > max_rows) max_rows = rows;
            if (s < pre_lo) pre_lo = s;
            pre_hi = s + 1;
        }
    }
    const int max_segs = (max_ctx + cpk::kDecodeSeg - 1) / cpk::kDecodeSeg;
    if (n_dec > 0 && (phases & CPK_PHASE_DECODE)) {
        const size_t need = cpk_varlen_workspace_size(n_seqs, q_heads, max_ctx, cache->head_dim);
        if (!ws || ws_bytes < need)
            return fail(CPK_EWORKSPACE, "varlen: workspace %zu bytes, need %zu", ws_bytes, need);
        if (!aligned16(ws)) return fail(CPK_EALIGN, "varlen: workspace not aligned");
    }
    hipStream_t st = (hipStream_t)stream;
    const int rb = cache->head_dim * elem_size(cache->dtype);
    // a call that both appends and decodes leaves the decode rows' append to
    // the decode kernel (fused); the copy kernel then moves only prompt rows
    const bool fuse_dec = n_dec > 0 && (phases & CPK_PHASE_APPEND) && (phases & CPK_PHASE_DECODE);
    if ((phases & CPK_PHASE_APPEND) && (n_pre > 0 || !fuse_dec)) {
        r = hip_status(cpk::launch_kv_append_varlen(
                           k_new, v_new, cache->k, cache->v, cache->seqlens_k, cache->kv_heads,
                           cache->capacity, rb, cu_rows, past_lens, slots, n_seqs, total_rows,
                           pg ? pg->table : nullptr, pg ? pg->max_blocks : 0,
                           pg ? pg->block_size : 0, pg ? pg->n_blocks : 0, fuse_dec, st),
                       "varlen append");
        if (r) return r;
    }
    const float sc = resolve_scale(scale, cache->head_dim);
    if (n_dec > 0 && (phases & CPK_PHASE_DECODE)) {
        cpk::DecodeArgs d = {};
        d.q = q; d.k = cache->k; d.v = cache->v; d.out = out; d.ws = (float *)ws;
        d.Hq = q_heads; d.Hkv = cache->kv_heads; d.D = cache->head_dim; d.cap = cache->capacity;
        d.scale_log2 = (float)((double)sc * 1.4426950408889634);
        d.max_segs = max_segs;
        d.cu_rows = cu_rows; d.past_lens = past_lens; d.slots = slots; d.n_seqs = n_seqs;
        if (fuse_dec) {
            d.k_new = k_new; d.v_new = v_new; d.seqlens_k = cache->seqlens_k;
        }
        if (pg) {
            d.block_table = pg->table; d.max_blocks = pg->max_blocks;
            d.block_size = pg->block_size; d.n_blocks = pg->n_blocks;
        }
        r = hip_status(cpk::launch_decode(d, cache->dtype, max_segs, st), "varlen decode");
        if (r) return r;
    }
    if (n_pre > 0 && (phases & CPK_PHASE_PREFILL)) {
        cpk::AttnArgs a = {};
        a.q = q; a.k = cache->k; a.v = cache->v; a.out = out; a.mask = nullptr;
        a.Hq = q_heads; a.Hkv = cache->kv_heads; a.D = cache->head_dim; a.cap = cache->capacity;
        fill_scale(a, sc);
        // the launch covers only the range of sequences with prompt rows
        // (row offsets stay absolute); a decode row inside the range is
        // skipped by its workgroups
        a.varlen = 1; a.cu_rows = cu_rows + pre_lo; a.past_lens = past_lens + pre_lo;
        a.slots = slots + pre_lo; a.n_seqs = pre_hi - pre_lo; a.min_rows = dec_ok ? 2 : 1;
        if (pg) {
            a.block_table = pg->table; a.max_blocks = pg->max_blocks;
            a.block_size = pg->block_size; a.n_blocks = pg->n_blocks;
        }
        const int kern = pick_kernel(cache->dtype, G, cache->kv_heads, max_rows, pre_pairs);
        const int br = cpk::attn_rows_per_block(cache->dtype, G, kern == cpk::kAttnWide);
        r = hip_status(cpk::launch_attention(a, cache->dtype, (max_rows + br - 1) / br,
                                             pre_hi - pre_lo, kern, st),
                       "varlen prefill");
        if (r) return r;
    }
    return ok();
}

extern "C" {

int cpk_roll_append(const void *k_old, const void *v_old, const void *k_chunk,
                    const void *v_chunk, void *k_new, void *v_new, int B, int H, int C, int c,
                    int D, int dtype, void *stream)
{
    int r = check_dtype_dim(dtype, D);
    if (r) return r;
    if (B < 1 || H < 1 || C < 1 || c < 1 || c > C)
        return fail(CPK_EINVAL, "roll_append: B=%d H=%d C=%d c=%d", B, H, C, c);
    if (!k_old || !v_old || !k_chunk || !v_chunk || !k_new || !v_new)
        return fail(CPK_EINVAL, "roll_append: NULL buffer");
    if (!aligned16(k_old) || !aligned16(v_old) || !aligned16(k_chunk) || !aligned16(v_chunk) ||
        !aligned16(k_new) || !aligned16(v_new))
        return fail(CPK_EALIGN, "roll_append: buffer not aligned");
    const size_t cache_bytes = (size_t)B * H * C * D * elem_size(dtype);
    const size_t chunk_bytes = (size_t)B * H * c * D * elem_size(dtype);
    const void *srcs[4] = {k_old, v_old, k_chunk, v_chunk};
    const size_t sz[4] = {cache_bytes, cache_bytes, chunk_bytes, chunk_bytes};
    for (int i = 0; i < 4; ++i)
        if (overlaps(srcs[i], sz[i], k_new, cache_bytes) || overlaps(srcs[i], sz[i], v_new, cache_bytes))
            return fail(CPK_EINVAL, "roll_append: output overlaps an input");
    if (overlaps(k_new, cache_bytes, v_new, cache_bytes))
        return fail(CPK_EINVAL, "roll_append: k_new and v_new overlap");
    return hip_status(cpk::launch_roll_append(k_old, v_old, k_chunk, v_chunk, k_new, v_new, B, H,
                                              C, c, D * elem_size(dtype), (hipStream_t)stream),
                      "roll_append launch");
}

// Key-range split of a rolling attention: parts of whole key tiles so that
// (row blocks x KV heads x parts) reaches about kSplitTarget workgroups.  A
// function of the shapes only, so the explicit-mask and computed-visibility
// forms of one call split identically.
static const int kSplitTarget = 256;

static void roll_split(int Hq, int Hkv, int C, int c, int dtype, int *n_parts, int *part_tiles)
{
    *n_parts = 1;
    *part_tiles = 0;
    if (dtype == CPK_F32 || Hkv < 1 || Hq < Hkv || Hq % Hkv) return;
    const int br = cpk::attn_rows_per_block(dtype, Hq / Hkv, false);
    const int base = ((c + br - 1) / br) * Hkv;
    const int tiles = (C + cpk::kAttnTileKeys - 1) / cpk::kAttnTileKeys;
    int s = kSplitTarget / (base > 0 ? base : 1);
    if (s > tiles) s = tiles;
    if (s <= 1) return;
    const int pt = (tiles + s - 1) / s;
    *part_tiles = pt;
    *n_parts = (tiles + pt - 1) / pt;
}

size_t cpk_roll_workspace_size(int Hq, int Hkv, int C, int c, int head_dim, int dtype)
{
    if (Hq < 1 || Hkv < 1 || C < 1 || c < 1 || head_dim < 1) return 0;
    int parts, pt;
    roll_split(Hq, Hkv, C, c, dtype, &parts, &pt);
    if (parts <= 1) return 0;
    return (size_t)parts * (size_t)c * (size_t)Hq * (size_t)(head_dim + 4) * sizeof(float);
}

// Every check of a rolling attention call, before anything is launched.
static int roll_check(const void *q, const void *k, const void *v, const void *mask, int abs_end,
                      int n_leftpad, int Hq, int Hkv, int C, int c, int D, int dtype, void *out,
                      void *ws, size_t ws_bytes)
{
    int r = check_dtype_dim(dtype, D);
    if (r) return r;
    if ((r = check_heads(Hq, Hkv))) return r;
    if (C < 1 || c < 1 || c > C || abs_end < c || n_leftpad < 0)
        return fail(CPK_EINVAL, "roll_attention: C=%d c=%d abs_end=%d n_leftpad=%d", C, c, abs_end,
                    n_leftpad);
    if (!q || !k || !v || !out) return fail(CPK_EINVAL, "roll_attention: NULL buffer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(CPK_EALIGN, "roll_attention: buffer not aligned");
    if (mask && ((uintptr_t)mask & 3u)) return fail(CPK_EALIGN, "roll_attention: mask not aligned");
    if (ws) {
        const size_t need = cpk_roll_workspace_size(Hq, Hkv, C, c, D, dtype);
        if (ws_bytes < need)
            return fail(CPK_EWORKSPACE, "roll_attention: workspace %zu bytes, need %zu", ws_bytes,
                        need);
        if (!aligned16(ws)) return fail(CPK_EALIGN, "roll_attention: workspace not aligned");
    }
    return ok();
}

// Rolling attention over k/v (a literal shifted cache, or a ring whose
// logical slot 0 is ring_start).  With k_chunk / v_chunk set (bf16/fp16),
// the kernel also appends the chunk: its rows are the keys of the last c
// slots, read from the chunk and written to their ring slots.
// Deferred (defer, bf16/fp16 with a split): the parts stay in ws for a later
// merge instead of a combine launch, and the parts an earlier deferred call
// left in prev_ws (same shapes) are merged into prev_out by this launch.
static int roll_attention_impl(const void *q, const void *k, const void *v, const void *mask,
                               int abs_end, int n_leftpad, int Hq, int Hkv, int C, int c, int D,
                               int dtype, float scale, int ring_start, void *out, void *ws,
                               size_t ws_bytes, void *stream, const void *k_chunk = nullptr,
                               const void *v_chunk = nullptr, bool defer = false,
                               const void *prev_ws = nullptr, void *prev_out = nullptr)
{
    int r = roll_check(q, k, v, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, out, ws,
                       ws_bytes);
    if (r) return r;
    cpk::AttnArgs a = {};
    a.q = q; a.k = k; a.v = v; a.out = out; a.mask = mask;
    a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.cap = C; a.mask_ld = C;
    fill_scale(a, resolve_scale(scale, D));
    a.slot = 0; a.q_row0 = 0; a.out_row0 = 0; a.rows = c; a.q_src_rows = c; a.out_rows = c;
    a.n_keys = C;
    if (mask) {
        // the additive mask decides visibility over every slot
        a.key_lo = 0;
        a.causal_base = C - 1;
    } else {
        // slot s holds position abs_end - C + s; visible iff
        // n_leftpad <= position <= abs_end - c + i
        const int64_t lo = (int64_t)n_leftpad - ((int64_t)abs_end - C);
        a.key_lo = lo < 0 ? 0 : (lo > C ? C : (int)lo);
        a.causal_base = C - c;
    }
    int parts = 1, pt = 0;
    if (ws) roll_split(Hq, Hkv, C, c, dtype, &parts, &pt);
    a.n_parts = parts;
    a.part_tiles = pt;
    a.part_ws = (float *)ws;
    a.ring_start = ring_start;
    if (k_chunk) {
        a.k_new = k_chunk; a.v_new = v_chunk; a.new_base = C - c; a.new_rows = c;
        a.seqlens = nullptr;
    }
    const int br = cpk::attn_rows_per_block(dtype, Hq / Hkv, false);
    // the narrow kernel (its general form when that is forced)
    const int kern = g_attn_kernel.load(std::memory_order_relaxed) == CPK_ATTN_NARROW_GENERAL
                         ? cpk::kAttnNarrowGeneral
                         : cpk::kAttnNarrow;
    if (prev_ws) {
        if (kern == cpk::kAttnNarrow) {
            // the scheduled form merges them beside its first tile's loads
            a.prev_ws = (const float *)prev_ws;
            a.prev_out = prev_out;
        } else {
            // the general form has no carried merge: a combine launch first
            cpk::AttnArgs m = a;
            m.part_ws = (float *)prev_ws;
            m.out = prev_out;
            r = hip_status(cpk::launch_attention_combine(m, dtype, (hipStream_t)stream),
                           "deferred merge");
            if (r) return r;
        }
    }
    r = hip_status(cpk::launch_attention(a, dtype, (c + br - 1) / br, 1, kern, (hipStream_t)stream),
                   "roll_attention launch");
    if (r || parts <= 1 || defer) return r;
    return hip_status(cpk::launch_attention_combine(a, dtype, (hipStream_t)stream),
                      "roll_attention combine");
}

int cpk_roll_attention(const void *q, const void *k, const void *v, const void *mask,
                       int abs_end, int n_leftpad, int Hq, int Hkv, int C, int c, int D,
                       int dtype, float scale, void *out, void *ws, size_t ws_bytes,
                       void *stream)
{
    return roll_attention_impl(q, k, v, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, scale,
                               0, out, ws, ws_bytes, stream);
}

int cpk_ring_attention(const void *q, const void *k_ring, const void *v_ring, const void *mask,
                       int abs_end, int n_leftpad, int Hq, int Hkv, int C, int c, int D,
                       int dtype, float scale, int start, void *out, void *ws, size_t ws_bytes,
                       void *stream)
{
    if (C < 1 || start < 0 || start >= C)
        return fail(CPK_EINVAL, "ring_attention: start=%d outside [0, C=%d)", start, C);
    return roll_attention_impl(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D,
                               dtype, scale, start, out, ws, ws_bytes, stream);
}

int cpk_ring_append(const void *k_chunk, const void *v_chunk, void *k_ring, void *v_ring, int B,
                    int H, int C, int c, int D, int dtype, int start, void *stream)
{
    int r = check_dtype_dim(dtype, D);
    if (r) return r;
    if (B < 1 || H < 1 || C < 1 || c < 1 || c > C || start < 0 || start >= C)
        return fail(CPK_EINVAL, "ring_append: B=%d H=%d C=%d c=%d start=%d", B, H, C, c, start);
    if (!k_chunk || !v_chunk || !k_ring || !v_ring)
        return fail(CPK_EINVAL, "ring_append: NULL buffer");
    if (!aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(k_ring) || !aligned16(v_ring))
        return fail(CPK_EALIGN, "ring_append: buffer not aligned");
    const size_t ring_bytes = (size_t)B * H * C * D * elem_size(dtype);
    const size_t chunk_bytes = (size_t)B * H * c * D * elem_size(dtype);
    const void *srcs[2] = {k_chunk, v_chunk};
    for (int i = 0; i < 2; ++i)
        if (overlaps(srcs[i], chunk_bytes, k_ring, ring_bytes) ||
            overlaps(srcs[i], chunk_bytes, v_ring, ring_bytes))
            return fail(CPK_EINVAL, "ring_append: a chunk overlaps a ring");
    if (overlaps(k_ring, ring_bytes, v_ring, ring_bytes))
        return fail(CPK_EINVAL, "ring_append: k_ring and v_ring overlap");
    return hip_status(cpk::launch_ring_append(k_chunk, v_chunk, k_ring, v_ring, B, H, C, c,
                                              D * elem_size(dtype), start, (hipStream_t)stream),
                      "ring_append launch");
}

// Checks of a ring step's chunk, rings and start (after roll_check).
static int ring_step_check(const void *k_chunk, const void *v_chunk, const void *k_ring,
                           const void *v_ring, int Hkv, int C, int c, int D, int dtype, int start)
{
    if (start < 0 || start >= C)
        return fail(CPK_EINVAL, "ring_step: start=%d outside [0, C=%d)", start, C);
    if (!k_chunk || !v_chunk) return fail(CPK_EINVAL, "ring_step: NULL chunk");
    if (!aligned16(k_chunk) || !aligned16(v_chunk))
        return fail(CPK_EALIGN, "ring_step: chunk not aligned");
    const size_t ring_bytes = (size_t)Hkv * C * D * elem_size(dtype);
    const size_t chunk_bytes = (size_t)c * Hkv * D * elem_size(dtype);
    const void *srcs[2] = {k_chunk, v_chunk};
    for (int i = 0; i < 2; ++i)
        if (overlaps(srcs[i], chunk_bytes, k_ring, ring_bytes) ||
            overlaps(srcs[i], chunk_bytes, v_ring, ring_bytes))
            return fail(CPK_EINVAL, "ring_step: a chunk overlaps a ring");
    if (overlaps(k_ring, ring_bytes, v_ring, ring_bytes))
        return fail(CPK_EINVAL, "ring_step: k_ring and v_ring overlap");
    return ok();
}

int cpk_ring_step(const void *q, const void *k_chunk, const void *v_chunk, void *k_ring,
                  void *v_ring, const void *mask, int abs_end, int n_leftpad, int Hq, int Hkv,
                  int C, int c, int D, int dtype, float scale, int start, void *out, void *ws,
                  size_t ws_bytes, void *stream)
{
    int r = roll_check(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, out,
                       ws, ws_bytes);
    if (r) return r;
    if ((r = ring_step_check(k_chunk, v_chunk, k_ring, v_ring, Hkv, C, c, D, dtype, start)))
        return r;
    const int next = (start + c) % C;
    if (dtype == CPK_F32) {
        // fp32 has no fused form: the append, then the attention
        r = hip_status(cpk::launch_ring_append(k_chunk, v_chunk, k_ring, v_ring, 1, Hkv, C, c,
                                               D * elem_size(dtype), start, (hipStream_t)stream),
                       "ring_step append");
        if (r) return r;
        return roll_attention_impl(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D,
                                   dtype, scale, next, out, ws, ws_bytes, stream);
    }
    return roll_attention_impl(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D,
                               dtype, scale, next, out, ws, ws_bytes, stream, k_chunk, v_chunk);
}

// Checks of a deferred rolling call (after roll_check): the shapes split
// the key range, ws is set, and a carried merge's buffers are aligned and
// overlap nothing this launch reads or writes.  k / v are the cache or the
// rings; k_extra / v_extra the chunk rows of a ring step (or NULL).
static int deferred_check(const char *who, const void *q, const void *k, const void *v,
                          const void *mask, int Hq, int Hkv, int C, int c, int D, int dtype,
                          const void *ws, const void *prev_ws, const void *prev_out,
                          const void *k_extra, const void *v_extra, size_t extra_bytes)
{
    const size_t need = cpk_roll_workspace_size(Hq, Hkv, C, c, D, dtype);
    if (need == 0 || !ws)
        return fail(CPK_EINVAL, "%s: these shapes do not split the key range", who);
    if (!prev_ws) return ok();
    if (!prev_out) return fail(CPK_EINVAL, "%s: prev_ws without prev_out", who);
    if (!aligned16(prev_ws) || !aligned16(prev_out))
        return fail(CPK_EALIGN, "%s: prev_ws / prev_out not aligned", who);
    if (overlaps(prev_ws, need, ws, need)) return fail(CPK_EINVAL, "%s: prev_ws overlaps ws", who);
    const size_t out_bytes = (size_t)c * Hq * D * elem_size(dtype);
    const size_t kv_bytes = (size_t)Hkv * C * D * elem_size(dtype);
    const size_t mask_bytes = (size_t)c * C * elem_size(dtype);
    const void *read[8] = {q, k, v, prev_ws, mask, k_extra, v_extra, ws};
    const size_t len[8] = {out_bytes, kv_bytes, kv_bytes, need, mask_bytes, extra_bytes,
                           extra_bytes, need};
    for (int i = 0; i < 8; ++i)
        if (read[i] && overlaps(prev_out, out_bytes, read[i], len[i]))
            return fail(CPK_EINVAL, "%s: prev_out overlaps another buffer of the call", who);
    return ok();
}

int cpk_roll_attention_deferred(const void *q, const void *k, const void *v, const void *mask,
                                int abs_end, int n_leftpad, int Hq, int Hkv, int C, int c, int D,
                                int dtype, float scale, void *out, void *ws, size_t ws_bytes,
                                const void *prev_ws, void *prev_out, void *stream)
{
    int r = roll_check(q, k, v, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, out, ws,
                       ws_bytes);
    if (r) return r;
    if ((r = deferred_check("roll_attention_deferred", q, k, v, mask, Hq, Hkv, C, c, D, dtype,
                            ws, prev_ws, prev_out, nullptr, nullptr, 0)))
        return r;
    return roll_attention_impl(q, k, v, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, scale,
                               0, out, ws, ws_bytes, stream, nullptr, nullptr, true, prev_ws,
                               prev_out);
}

int cpk_ring_step_deferred(const void *q, const void *k_chunk, const void *v_chunk,
                           void *k_ring, void *v_ring, const void *mask, int abs_end,
                           int n_leftpad, int Hq, int Hkv, int C, int c, int D, int dtype,
                           float scale, int start, void *out, void *ws, size_t ws_bytes,
                           const void *prev_ws, void *prev_out, void *stream)
{
    int r = roll_check(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D, dtype, out,
                       ws, ws_bytes);
    if (r) return r;
    if ((r = ring_step_check(k_chunk, v_chunk, k_ring, v_ring, Hkv, C, c, D, dtype, start)))
        return r;
    const size_t chunk_bytes = (size_t)c * Hkv * D * elem_size(dtype);
    if ((r = deferred_check("ring_step_deferred", q, k_ring, v_ring, mask, Hq, Hkv, C, c, D,
                            dtype, ws, prev_ws, prev_out, k_chunk, v_chunk, chunk_bytes)))
        return r;
    return roll_attention_impl(q, k_ring, v_ring, mask, abs_end, n_leftpad, Hq, Hkv, C, c, D,
                               dtype, scale, (start + c) % C, out, ws, ws_bytes, stream, k_chunk,
                               v_chunk, true, prev_ws, prev_out);
}

int cpk_roll_flush(const void *ws, size_t ws_bytes, void *out, int Hq, int Hkv, int C, int c,
                   int D, int dtype, void *stream)
{
    int r = check_dtype_dim(dtype, D);
    if (r) return r;
    if ((r = check_heads(Hq, Hkv))) return r;
    if (C < 1 || c < 1 || c > C) return fail(CPK_EINVAL, "roll_flush: C=%d c=%d", C, c);
    const size_t need = cpk_roll_workspace_size(Hq, Hkv, C, c, D, dtype);
    if (need == 0)
        return fail(CPK_EINVAL, "roll_flush: these shapes do not split the key range");
    if (!ws || !out) return fail(CPK_EINVAL, "roll_flush: NULL buffer");
    if (ws_bytes < need)
        return fail(CPK_EWORKSPACE, "roll_flush: workspace %zu bytes, need %zu", ws_bytes, need);
    if (!aligned16(ws) || !aligned16(out)) return fail(CPK_EALIGN, "roll_flush: not aligned");
    if (overlaps(out, (size_t)c * Hq * D * elem_size(dtype), ws, need))
        return fail(CPK_EINVAL, "roll_flush: out overlaps ws");
    int parts, pt;
    roll_split(Hq, Hkv, C, c, dtype, &parts, &pt);
    cpk::AttnArgs a = {};
    a.out = out; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
    a.out_row0 = 0; a.out_rows = c;
    a.n_parts = parts; a.part_tiles = pt; a.part_ws = (float *)ws;
    return hip_status(cpk::launch_attention_combine(a, dtype, (hipStream_t)stream),
                      "roll_flush combine");
}

int cpk_ring_view(const void *k_ring, const void *v_ring, void *k_out, void *v_out, int B, int H,
                  int C, int D, int dtype, int start, void *stream)
{
    int r = check_dtype_dim(dtype, D);
    if (r) return r;
    if (B < 1 || H < 1 || C < 1 || start < 0 || start >= C)
        return fail(CPK_EINVAL, "ring_view: B=%d H=%d C=%d start=%d", B, H, C, start);
    if (!k_ring || !v_ring || !k_out || !v_out) return fail(CPK_EINVAL, "ring_view: NULL buffer");
    if (!aligned16(k_ring) || !aligned16(v_ring) || !aligned16(k_out) || !aligned16(v_out))
        return fail(CPK_EALIGN, "ring_view: buffer not aligned");
    const size_t bytes = (size_t)B * H * C * D * elem_size(dtype);
    const void *ins[2] = {k_ring, v_ring};
    for (int i = 0; i < 2; ++i)
        if (overlaps(ins[i], bytes, k_out, bytes) || overlaps(ins[i], bytes, v_out, bytes))
            return fail(CPK_EINVAL, "ring_view: output overlaps a ring");
    if (overlaps(k_out, bytes, v_out, bytes)) return fail(CPK_EINVAL, "ring_view: outputs overlap");
    return hip_status(cpk::launch_ring_view(k_ring, v_ring, k_out, v_out, B, H, C,
                                            D * elem_size(dtype), start, (hipStream_t)stream),
                      "ring_view launch");
}

}  // extern "C"
