// Cache writes: append-only KV append (single sequence and packed varlen),
// the rolling cache shift, and the stream-ordered length update.
//
// All of them are byte copies in 16-byte vectors: consecutive threads move
// consecutive 16-byte pieces of one head's D-vector, so both the token-major
// source rows and the head-major cache rows are read and written in
// contiguous runs.  HBM-bound; no arithmetic touches the data.
#include "cpk_internal.h"

namespace cpk {
namespace {

typedef uint4 vec16;  // 16 bytes

// cache[slot][h][past + r][:] = new[min(r, src_rows - 1)][h][:], then
// seqlens[slot] = len_after.  Rows past src_rows repeat the last real row:
// the query-axis padding of the ONNX GenAI Wiki "Chunked Prefill", section
// 4, done as an index clamp.
__global__ void kv_append_kernel(const vec16 *__restrict__ kn, const vec16 *__restrict__ vn,
                                 vec16 *__restrict__ ck, vec16 *__restrict__ cv,
                                 int32_t *__restrict__ seqlens, int Hkv, int cap, int vpr,
                                 int slot, int past, int rows, int src_rows, int len_after)
{
    const int64_t total = (int64_t)rows * Hkv * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int c = (int)(i % vpr);
        const int64_t rh = i / vpr;
        const int h = (int)(rh % Hkv);
        const int r = (int)(rh / Hkv);
        const int sr = r < src_rows ? r : src_rows - 1;
        const int64_t src = ((int64_t)sr * Hkv + h) * vpr + c;
        const int64_t dst = (((int64_t)slot * Hkv + h) * cap + past + r) * vpr + c;
        ck[dst] = kn[src];
        cv[dst] = vn[src];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && seqlens) seqlens[slot] = len_after;
}

// Packed step: row t of the packed k_new/v_new belongs to the sequence s with
// cu_rows[s] <= t < cu_rows[s+1]; it lands at position past_lens[s] + (t -
// cu_rows[s]) of cache slot slots[s].  With skip_single, the rows of
// one-row sequences are left out (the decode kernel appends those itself).
__global__ void kv_append_varlen_kernel(const vec16 *__restrict__ kn, const vec16 *__restrict__ vn,
                                        vec16 *__restrict__ ck, vec16 *__restrict__ cv,
                                        int32_t *__restrict__ seqlens, int Hkv, int cap, int vpr,
                                        const int32_t *__restrict__ cu_rows,
                                        const int32_t *__restrict__ past_lens,
                                        const int32_t *__restrict__ slots, int n_seqs,
                                        int total_rows, const int32_t *__restrict__ table,
                                        int max_blocks, int bs, int n_blocks, int skip_single)
{
    const int64_t total = (int64_t)total_rows * Hkv * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int c = (int)(i % vpr);
        const int64_t rh = i / vpr;
        const int h = (int)(rh % Hkv);
        const int t = (int)(rh / Hkv);
        // binary search: largest s with cu_rows[s] <= t
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_rows[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int s = lo;
        if (skip_single && cu_rows[s + 1] - cu_rows[s] == 1) continue;
        const int r = t - cu_rows[s];
        const int pos = past_lens[s] + r;
        const int64_t row = bs ? paged_row(table, max_blocks, bs, n_blocks, Hkv, slots[s], h, pos)
                               : ((int64_t)slots[s] * Hkv + h) * cap + pos;
        const int64_t dst = row * vpr + c;
        const int64_t src = ((int64_t)t * Hkv + h) * vpr + c;
        ck[dst] = kn[src];
        cv[dst] = vn[src];
        if (h == 0 && c == 0 && t == cu_rows[s + 1] - 1)
            seqlens[slots[s]] = past_lens[s] + r + 1;
    }
}

__global__ void set_len_kernel(int32_t *seqlens, int b, int len)
{
    if (threadIdx.x == 0) seqlens[b] = len;
}

// Rolling cache (Horizon developer blog "Chunk Prefill", section 3):
// new = cat(old, chunk)[c:] along positions.  Slot s < C - c takes old slot
// s + c; the last c slots take the chunk's rows.  Out of place.
__global__ void roll_append_kernel(const vec16 *__restrict__ ko, const vec16 *__restrict__ vo,
                                   const vec16 *__restrict__ kc, const vec16 *__restrict__ vc,
                                   vec16 *__restrict__ kn, vec16 *__restrict__ vn, int B, int H,
                                   int C, int c, int vpr)
{
    const int64_t total = (int64_t)B * H * C * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = (int)(i % vpr);
        const int64_t r1 = i / vpr;
        const int s = (int)(r1 % C);
        const int64_t bh = r1 / C;
        const int h = (int)(bh % H);
        const int b = (int)(bh / H);
        if (s < C - c) {
            const int64_t src = (bh * C + s + c) * vpr + e;
            kn[i] = ko[src];
            vn[i] = vo[src];
        } else {
            const int t = s - (C - c);
            const int64_t src = (((int64_t)b * c + t) * H + h) * vpr + e;
            kn[i] = kc[src];
            vn[i] = vc[src];
        }
    }
}

int grid_for(int64_t items)
{
    int64_t blocks = (items + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;   // grid-stride beyond ~32 waves per CU
    return (int)blocks;
}

// Ring-buffer append: the c new rows overwrite the c oldest physical slots.
__global__ void ring_append_kernel(const vec16 *__restrict__ kc, const vec16 *__restrict__ vc,
                                   vec16 *__restrict__ kr, vec16 *__restrict__ vr, int B, int H,
                                   int C, int c, int vpr, int start)
{
    const int64_t total = (int64_t)B * c * H * vpr;   // chunk order [B][c][H][vpr]
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = (int)(i % vpr);
        const int64_t r1 = i / vpr;
        const int h = (int)(r1 % H);
        const int64_t r2 = r1 / H;
        const int t = (int)(r2 % c);
        const int b = (int)(r2 / c);
        int slot = start + t;
        if (slot >= C) slot -= C;
        const int64_t dst = (((int64_t)b * H + h) * C + slot) * vpr + e;
        kr[dst] = kc[i];
        vr[dst] = vc[i];
    }
}

// Logical view of a ring: slot s of the output is physical slot (start + s) mod C.
__global__ void ring_view_kernel(const vec16 *__restrict__ kr, const vec16 *__restrict__ vr,
                                 vec16 *__restrict__ ko, vec16 *__restrict__ vo, int B, int H,
                                 int C, int vpr, int start)
{
    const int64_t total = (int64_t)B * H * C * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = (int)(i % vpr);
        const int64_t r1 = i / vpr;
        const int s = (int)(r1 % C);
        const int64_t bh = r1 / C;
        int slot = start + s;
        if (slot >= C) slot -= C;
        const int64_t src = (bh * C + slot) * vpr + e;
        ko[i] = kr[src];
        vo[i] = vr[src];
    }
}

// Prefix copy between two slots of one cache: rows [0, len) of every KV head.
__global__ void kv_copy_prefix_kernel(const vec16 *__restrict__ ck, const vec16 *__restrict__ cv,
                                      vec16 *__restrict__ dk, vec16 *__restrict__ dv,
                                      int32_t *seqlens, int Hkv, int cap, int vpr, int src,
                                      int dst, int len)
{
    const int64_t total = (int64_t)Hkv * len * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int e = (int)(i % vpr);
        const int64_t r1 = i / vpr;
        const int pos = (int)(r1 % len);
        const int h = (int)(r1 / len);
        const int64_t so = (((int64_t)src * Hkv + h) * cap + pos) * vpr + e;
        const int64_t d = (((int64_t)dst * Hkv + h) * cap + pos) * vpr + e;
        dk[d] = ck[so];
        dv[d] = cv[so];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) seqlens[dst] = len;
}

}  // namespace

hipError_t launch_kv_copy_prefix(const void *k, const void *v, int32_t *seqlens, int Hkv,
                                 int cap, int row_bytes, int src, int dst, int len,
                                 hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)Hkv * len * vpr;
    hipLaunchKernelGGL(kv_copy_prefix_kernel, dim3(grid_for(items > 0 ? items : 1)), dim3(256),
                       0, st, (const vec16 *)k, (const vec16 *)v, (vec16 *)k, (vec16 *)v,
                       seqlens, Hkv, cap, vpr, src, dst, len);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void *k_new, const void *v_new, void *ck, void *cv,
                            int32_t *seqlens, int Hkv, int cap, int row_bytes, int slot,
                            int past, int rows, int src_rows, int len_after, hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)rows * Hkv * vpr;
    hipLaunchKernelGGL(kv_append_kernel, dim3(grid_for(items)), dim3(256), 0, st,
                       (const vec16 *)k_new, (const vec16 *)v_new, (vec16 *)ck, (vec16 *)cv,
                       seqlens, Hkv, cap, vpr, slot, past, rows, src_rows, len_after);
    return hipGetLastError();
}

hipError_t launch_kv_append_varlen(const void *k_new, const void *v_new, void *ck, void *cv,
                                   int32_t *seqlens, int Hkv, int cap, int row_bytes,
                                   const int32_t *cu_rows, const int32_t *past_lens,
                                   const int32_t *slots, int n_seqs, int total_rows,
                                   const int32_t *block_table, int max_blocks, int block_size,
                                   int n_blocks, bool skip_single, hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)total_rows * Hkv * vpr;
    hipLaunchKernelGGL(kv_append_varlen_kernel, dim3(grid_for(items)), dim3(256), 0, st,
                       (const vec16 *)k_new, (const vec16 *)v_new, (vec16 *)ck, (vec16 *)cv,
                       seqlens, Hkv, cap, vpr, cu_rows, past_lens, slots, n_seqs, total_rows,
                       block_table, max_blocks, block_size, n_blocks, skip_single ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_set_len(int32_t *seqlens, int b, int len, hipStream_t st)
{
    hipLaunchKernelGGL(set_len_kernel, dim3(1), dim3(64), 0, st, seqlens, b, len);
    return hipGetLastError();
}

hipError_t launch_roll_append(const void *k_old, const void *v_old, const void *k_chunk,
                              const void *v_chunk, void *k_new, void *v_new, int B, int H,
                              int C, int c, int row_bytes, hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)B * H * C * vpr;
    hipLaunchKernelGGL(roll_append_kernel, dim3(grid_for(items)), dim3(256), 0, st,
                       (const vec16 *)k_old, (const vec16 *)v_old, (const vec16 *)k_chunk,
                       (const vec16 *)v_chunk, (vec16 *)k_new, (vec16 *)v_new, B, H, C, c, vpr);
    return hipGetLastError();
}

hipError_t launch_ring_append(const void *k_chunk, const void *v_chunk, void *k_ring,
                              void *v_ring, int B, int H, int C, int c, int row_bytes, int start,
                              hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)B * c * H * vpr;
    hipLaunchKernelGGL(ring_append_kernel, dim3(grid_for(items)), dim3(256), 0, st,
                       (const vec16 *)k_chunk, (const vec16 *)v_chunk, (vec16 *)k_ring,
                       (vec16 *)v_ring, B, H, C, c, vpr, start);
    return hipGetLastError();
}

hipError_t launch_ring_view(const void *k_ring, const void *v_ring, void *k_out, void *v_out,
                            int B, int H, int C, int row_bytes, int start, hipStream_t st)
{
    const int vpr = row_bytes / 16;
    const int64_t items = (int64_t)B * H * C * vpr;
    hipLaunchKernelGGL(ring_view_kernel, dim3(grid_for(items)), dim3(256), 0, st,
                       (const vec16 *)k_ring, (const vec16 *)v_ring, (vec16 *)k_out,
                       (vec16 *)v_out, B, H, C, vpr, start);
    return hipGetLastError();
}

}  // namespace cpk
