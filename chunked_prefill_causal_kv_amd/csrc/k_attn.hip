// Chunk attention over a KV cache: flash-style tiled attention with online
// softmax for gfx950.
//
// What is computed (per query row at causal position p, query head h, KV
// head g = h / G): softmax(scale * q k_j) over the visible keys j, times v_j.
// Visibility is the causal rule over absolute positions (ONNX GenAI Wiki
// "Chunked Prefill", section 1.2), so a chunk sees exactly what one-shot
// prefill sees; the rolling-cache form adds a lower bound or an additive
// mask (Horizon developer blog "Chunk Prefill", section 4).
//
// bf16 / fp16 kernel (attn_mfma_kernel)
// -------------------------------------
// * Work item: 64 "query columns" = G query heads x (64/G) rows that share
//   one KV head, so every K/V tile staged in LDS serves the whole GQA group.
//   Workgroups are numbered KV head fastest, so with 8 KV heads each XCD
//   (and its L2) serves a single KV head.
// * K/V tiles of 128 keys, double-buffered in LDS and filled by direct
//   global->LDS 16-byte loads (no register staging).  Both tiles stay
//   row-major [key][d]; the 16-byte chunks of each row are XOR-swizzled
//   (by choosing which global chunk each lane fetches) so that the MFMA
//   fragment reads below are free of bank conflicts.  Tiles are aligned to
//   absolute key 0, so a query row visits the same tile sequence whether its
//   prompt runs in one pass or in chunks.
// * 8 waves: 2 groups of 32 query columns x 4 slices of 32 keys of every
//   tile.  Each wave keeps its own online-softmax state for its 32 columns;
//   the 4 key slices are merged once at the end through LDS (an
//   in-workgroup split of the key range).  Two waves per SIMD let one
//   wave's softmax (VALU) overlap the other's matrix work.
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_{bf16,f16}: a lane then holds one query column and
//   16 keys, so the row max is 15 in-lane max operations plus one
//   cross-half exchange, and the probabilities are already in the B-operand
//   layout of O^T = V^T P^T.  V^T fragments come straight from the
//   row-major V tile through the LDS transpose read (ds_read_b64_tr_b16).
// * Online softmax in the exp2 domain (scale * log2 e folded into one FMA).
//   The running maximum is only raised when a tile's maximum exceeds it by
//   more than 2^8; otherwise the stale maximum is kept (probabilities up to
//   256, exact after the final normalisation).  This removes almost every
//   rescale of the 128 accumulator registers.  The row sum accumulates the
//   rounded probabilities with packed dot products, so numerator and
//   denominator use the same weights.
// * Key indices at or past n_keys are clamped to the last valid key for the
//   load and masked out of the softmax, so bytes beyond the valid length
//   (stale pads, poison) are never read.
//
// fp32 kernel (attn_f32_kernel): one query column per lane, VALU FMAs in
// fp32 with an exact per-tile rescale.  Full precision, no reduced-precision
// step; used where fp32 storage is requested.
#include "cpk_internal.h"

#include <hip/hip_bf16.h>
#include <limits.h>
#include <math.h>

namespace cpk {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct Bf16 {
    typedef bf16x8_t vec8;
    static constexpr uint32_t kOnes = 0x3f803f80u;   // (1.0, 1.0)
    static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(vec8, a),
                                                       __builtin_bit_cast(vec8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    }
    static __device__ __forceinline__ float to_f32(uint32_t bits16)
    {
        return __uint_as_float(bits16 << 16);
    }
    static __device__ __forceinline__ uint32_t from_f32(float x)
    {
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi)
    {
        const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
};

struct F16 {
    typedef f16x8_t vec8;
    static constexpr uint32_t kOnes = 0x3c003c00u;   // (1.0, 1.0)
    static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(vec8, a),
                                                      __builtin_bit_cast(vec8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
    }
    static __device__ __forceinline__ float to_f32(uint32_t bits16)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    }
    static __device__ __forceinline__ uint32_t from_f32(float x)
    {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi)
    {
        const f16x2_t v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
};

constexpr int kQC = 64;         // query columns per workgroup (2 groups of 32)
constexpr int kBK = 128;        // keys per LDS tile (4 slices of 32)
constexpr int kThreads = 512;   // 8 waves = 2 column groups x 4 key slices
static_assert(kBK == kAttnTileKeys, "split parts are counted in key tiles");
constexpr float kLazyLog2 = 8.0f;

// The two 32-lane halves of a wave hold the same query column (different
// keys).  Exchange through ds_bpermute (__shfl_xor across 32 lanes); max and
// + are commutative, so both halves obtain bit-identical results.
__device__ __forceinline__ float pair_max(float x)
{
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float pair_sum(float x)
{
    return x + __shfl_xor(x, 32);
}

template <int D>
struct Tile {
    static constexpr int NCH = D / 8;                 // 16-byte chunks per key row
    static constexpr int STAGE = 2 * kBK * D;         // one buffer: K then V, uint16 elements
    static constexpr int LOADS = kBK * NCH / kThreads;   // 16-byte loads per thread per tensor
    static constexpr int WAVES = kThreads / 64;
    static constexpr int D4 = D / 4;                  // float4 columns of an epilogue row
    // chunk swizzles: stored position = chunk ^ swizzle(row)
    static __device__ __forceinline__ int swz_k(int row) { return row % NCH; }
    static __device__ __forceinline__ int swz_v(int row) { return (row % (NCH / 4)) << 2; }
    // epilogue rows (one query column of one key slice, D floats) are
    // float4-swizzled by the column index instead of padded
    static __device__ __forceinline__ int swz_o(int col) { return col & (D4 - 1); }
};

// One field from each 64-byte line of the argument block, read at kernel
// entry: the four scalar-cache misses are then in flight together, and the
// kernel's later argument reads (each behind a data-dependent branch) hit
// the scalar cache instead of waiting on one miss after another.
__device__ __forceinline__ void prefetch_args(const AttnArgs &a)
{
    static_assert(sizeof(AttnArgs) <= 256, "four lines");
    const void *f0 = a.q;
    const int f1 = a.varlen, f2 = a.n_parts, f3 = a.ring_start;
    asm volatile("" ::"s"(f0), "s"(f1), "s"(f2), "s"(f3));
}

struct SeqView {
    int slot, q_row0, out_row0, rows, q_src_rows, out_rows, n_keys, key_lo, causal_base;
};

__device__ __forceinline__ bool resolve_seq(const AttnArgs &a, int z, SeqView &s)
{
    if (!a.varlen) {
        s.slot = a.slot; s.q_row0 = a.q_row0; s.out_row0 = a.out_row0; s.rows = a.rows;
        s.q_src_rows = a.q_src_rows; s.out_rows = a.out_rows; s.n_keys = a.n_keys;
        s.key_lo = a.key_lo; s.causal_base = a.causal_base;
        return true;
    }
    const int r0 = a.cu_rows[z], r1 = a.cu_rows[z + 1];
    const int rows = r1 - r0;
    if (rows < a.min_rows || rows <= 0) return false;
    const int past = a.past_lens[z];
    s.slot = a.slots[z]; s.q_row0 = r0; s.out_row0 = r0; s.rows = rows; s.q_src_rows = rows;
    s.out_rows = rows; s.n_keys = past + rows; s.key_lo = 0; s.causal_base = past;
    return true;
}

// Fused append: the cache rows of one row block and KV head, copied from
// the new rows in 16-byte pieces (by part 0 alone when the key range is
// split).  append_load reads this workgroup's pieces into registers and
// append_store writes them, so a kernel can put the loads in flight beside
// its first tile loads and issue the stores after its first full wait.  No
// workgroup reads the cache rows being written (keys at or past new_base
// come from the new rows), so the stores may land at any time.  The pieces
// live in registers: a local ext_vector array indexed by unrolled constants.
template <int D, int THREADS, int MAXROWS>
constexpr int append_pieces()
{
    return (MAXROWS * (D / 8) * 2 + THREADS - 1) / THREADS;
}

template <int D, int THREADS, int JB, int JE>
__device__ __forceinline__ void append_load(const AttnArgs &a, int g, int r0, int n_rows, int tid,
                                            u32x4_t (&val)[JE - JB])
{
    constexpr int NCH = D / 8;
    const int n = n_rows * NCH;   // pieces per tensor; n_rows >= 1
#pragma unroll
    for (int j = JB; j < JE; ++j) {
        // a piece index past the end re-reads the last piece, so the load
        // needs no branch and the value no merge at a join (which would make
        // the compiler wait for it at once); only the store is conditional
        if (j == 0 || j * THREADS < 2 * n) {   // uniform
            const int c = min(tid + j * THREADS, 2 * n - 1);
            const bool isv = c >= n;
            const int cc = isv ? c - n : c;
            const int src = min(r0 + cc / NCH, a.new_rows - 1);
            const uint16_t *sp = (const uint16_t *)(isv ? a.v_new : a.k_new) +
                                 ((int64_t)src * a.Hkv + g) * D + (cc % NCH) * 8;
            val[j - JB] = *(const __attribute__((address_space(1))) u32x4_t *)sp;
        }
    }
}

template <int D, int THREADS, int JB, int JE>
__device__ __forceinline__ void append_store(const AttnArgs &a, int g, int r0, int n_rows, int tid,
                                             const u32x4_t (&val)[JE - JB], bool set_len)
{
    constexpr int NCH = D / 8;
    const int n = n_rows * NCH;
    uint16_t *ck = (uint16_t *)a.k + ((int64_t)a.slot * a.Hkv + g) * a.cap * D;
    uint16_t *cv = (uint16_t *)a.v + ((int64_t)a.slot * a.Hkv + g) * a.cap * D;
#pragma unroll
    for (int j = JB; j < JE; ++j) {
        const int c = tid + j * THREADS;
        if (c < 2 * n) {
            const bool isv = c >= n;
            const int cc = isv ? c - n : c;
            // physical row of logical position new_base + r0 + cc/NCH (a
            // ring buffer starts at ring_start; the identity otherwise)
            int row = a.new_base + r0 + cc / NCH + a.ring_start;
            if (row >= a.cap) row -= a.cap;
            uint16_t *dp = (isv ? cv : ck) + (int64_t)row * D + (cc % NCH) * 8;
            *(u32x4_t *)dp = val[j - JB];
        }
    }
    if (set_len && a.seqlens && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0)
        a.seqlens[a.slot] = a.len_after;
}

// Pieces [JB, JE) loaded and stored back to back.  Callers that count
// their waits on tile loads call this before any tile load: loads complete
// in order, and older outstanding stores only make a wait stricter.
template <int D, int THREADS, int JB, int JE>
__device__ __forceinline__ void fused_append(const AttnArgs &a, int g, int r0, int n_rows, int tid,
                                             bool set_len)
{
    if constexpr (JE > JB) {
        if (JB * THREADS < 2 * n_rows * (D / 8)) {   // uniform: any piece from JB on
            u32x4_t val[JE - JB];
            append_load<D, THREADS, JB, JE>(a, g, r0, n_rows, tid, val);
            append_store<D, THREADS, JB, JE>(a, g, r0, n_rows, tid, val, set_len);
        }
    }
}

// Source of one 16-byte piece of a K or V tile: the cache row of logical
// key `key` of this KV head (physical row (ring_start + key) mod cap), or
// (fused append, key >= new_base) the matching new row.
__device__ __forceinline__ const char *kv_src(const uint16_t *cache_head, const void *new_rows,
                                              const AttnArgs &a, int g, int D, int key,
                                              int chunk_elem)
{
    if (key >= a.new_base && new_rows) {
        const int i = min(key - a.new_base, a.new_rows - 1);
        return (const char *)((const uint16_t *)new_rows + ((int64_t)i * a.Hkv + g) * D +
                              chunk_elem);
    }
    int phys = key + a.ring_start;
    if (phys >= a.cap) phys -= a.cap;
    return (const char *)(cache_head + (int64_t)phys * D + chunk_elem);
}

// Merge of the split parts of a key range: for each (row, query head), in
// part order, M = max_p M_p, f_p = 2^(M_p - M), out = sum_p f_p O_p /
// sum_p f_p den_p.  One unit is 8 consecutive outputs of one (row, head)
// (unit / (D / 8) is the pair row * Hq + head): two 16-byte record loads
// per part and one 16-byte store.  The records of up to kCombineBatch parts
// are loaded at once (one memory round trip); more parts are merged batch
// by batch, rescaling the running sums when a later batch raises the
// maximum (for at most kCombineBatch parts, exactly the two-pass formula
// above).  The combine launch and the carried merge of the scheduled
// 64-column kernel both run this, so their outputs are identical.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 4;

template <typename TR, int D>
__device__ __forceinline__ void combine_unit(const float *part_ws, int n_parts, int out_rows,
                                             int Hq, void *out, int out_row0, int unit)
{
    constexpr int TPP = D / 8;                       // units per (row, head)
    const int pair = unit / TPP;
    const int row = pair / Hq;
    const int head = pair % Hq;
    const int d0 = (unit % TPP) * 8;
    const int64_t stride = (int64_t)out_rows * Hq * (D + 4);
    const float *rec = part_ws + (int64_t)pair * (D + 4);
    float M = -INFINITY;
    float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int p0 = 0; p0 < n_parts; p0 += kCombineBatch) {
        float2 md[kCombineBatch];
        float4 x0[kCombineBatch], x1[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            // past the last part: re-read a valid record, weighted 0 below
            const float *r = rec + (int64_t)min(p0 + i, n_parts - 1) * stride;
            md[i] = *(const float2 *)r;
            x0[i] = *(const float4 *)(r + 4 + d0);
            x1[i] = *(const float4 *)(r + 8 + d0);
        }
        float bm = M;
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i)
            if (p0 + i < n_parts) bm = fmaxf(bm, md[i].x);
        if (bm != M) {   // M == -inf: nothing merged yet, the sums are 0
            const float alpha = M == -INFINITY ? 0.f : exp2f(M - bm);
#pragma unroll
            for (int e = 0; e < 8; ++e) num[e] *= alpha;
            den *= alpha;
            M = bm;
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const float f = (p0 + i >= n_parts || md[i].x == -INFINITY) ? 0.f : exp2f(md[i].x - M);
            num[0] = __builtin_fmaf(f, x0[i].x, num[0]);
            num[1] = __builtin_fmaf(f, x0[i].y, num[1]);
            num[2] = __builtin_fmaf(f, x0[i].z, num[2]);
            num[3] = __builtin_fmaf(f, x0[i].w, num[3]);
            num[4] = __builtin_fmaf(f, x1[i].x, num[4]);
            num[5] = __builtin_fmaf(f, x1[i].y, num[5]);
            num[6] = __builtin_fmaf(f, x1[i].z, num[6]);
            num[7] = __builtin_fmaf(f, x1[i].w, num[7]);
            den = __builtin_fmaf(f, md[i].y, den);
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float o0 = den > 0.f ? num[2 * i] / den : 0.f;
        const float o1 = den > 0.f ? num[2 * i + 1] / den : 0.f;
        w[i] = TR::pack(o0, o1);
    }
    uint16_t *op = (uint16_t *)out + ((int64_t)(out_row0 + row) * Hq + head) * D + d0;
    *(uint4 *)op = make_uint4(w[0], w[1], w[2], w[3]);
}

// Block rows of a paged pool for one workgroup's key tiles.  At the start
// the workgroup stages the block ids of its key range (clamped into the
// pool) in LDS; a tile's lookup is then an LDS read, so no extra global
// load sits among the tile loads, whose waits count them.  A barrier must
// separate stage() from the first row().
struct PagedTiles {
    int b0 = 0;      // first block of the range
    int nb = 0;      // staged entries - 1
    const int *tab = nullptr;
    __device__ __forceinline__ void stage(const AttnArgs &a, int slot, int key_first,
                                          int key_last, int *lds, int tid, int nthreads)
    {
        const int last = a.max_blocks - 1;
        b0 = min(max(key_first / a.block_size, 0), last);
        const int b1 = min(max(key_last / a.block_size, b0), last);
        nb = min(b1 - b0, kMaxTableBlocks - 1);
        tab = lds;
        for (int i = tid; i <= nb; i += nthreads) {
            const int b = a.block_table[(int64_t)slot * a.max_blocks + b0 + i];
            lds[i] = b < 0 ? 0 : (b >= a.n_blocks ? a.n_blocks - 1 : b);
        }
    }
    // element offset of tile kt's first row (head g); the tile lies in one block
    __device__ __forceinline__ int64_t row(const AttnArgs &a, int g, int kt, int tile_keys) const
    {
        const int key0 = kt * tile_keys;
        const int i = min(max(key0 / a.block_size - b0, 0), nb);
        return ((int64_t)tab[i] * a.Hkv + g) * a.block_size + key0 % a.block_size;
    }
};

template <typename TR, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_mfma_kernel(AttnArgs a)
{
    using TL = Tile<D>;
    constexpr int NCH = TL::NCH;
    constexpr int NS = D / 16;      // k-steps of the QK^T contraction
    constexpr int NDB = D / 32;     // 32-wide d blocks of O^T

    // Two separately declared tile buffers (K then V in each): the compiler
    // can then tell that reading one while the other is being filled by
    // direct loads needs no wait for those loads.
    __shared__ __attribute__((aligned(16))) uint16_t buf0[TL::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t buf1[TL::STAGE];
    __shared__ float ml[2 * 4 * kQC];
    __shared__ int ptab[PAGED ? kMaxTableBlocks : 1];

    prefetch_args(a);
    SeqView sv;
    if (!resolve_seq(a, blockIdx.z, sv)) return;
    const int G = a.Hq / a.Hkv;
    const int BR = kQC / G;                 // rows per workgroup
    // blockIdx.x = row_block * Hkv + kv_head: consecutive workgroups go to
    // consecutive XCDs, so with 8 KV heads each XCD serves one KV head and
    // its L2 holds that head's K/V for all of the XCD's row blocks.
    const int g = blockIdx.x % a.Hkv;
    const int r0 = (blockIdx.x / a.Hkv) * BR;
    if (r0 >= sv.rows) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int lane = tid & 63;
    const int c32 = lane & 31;
    const int hi = lane >> 5;
    const int qg = wave >> 2;               // query-column group: columns 32*qg .. +32
    const int ks = wave & 3;                // key slice: keys 32*ks .. +32 of each tile
    const int qc = qg * 32 + c32;           // this lane's query column

    const uint16_t *kc = (const uint16_t *)a.k + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const uint16_t *vc = (const uint16_t *)a.v + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const bool fused = a.k_new != nullptr;
    // keys at or past new_lo come from the new rows (never from the cache)
    const int new_lo = fused ? a.new_base : INT_MAX;
    // fused append: the first piece of every thread (the whole append once
    // G >= 4) is loaded now, beside the query and first tile loads, and
    // stored after the first tile's wait (one round trip less before the
    // first tile); further pieces (G < 4) are copied at once
    const bool app_on = fused && blockIdx.y == 0;
    const int app_rows = min(r0 + BR, sv.rows) - r0;
    u32x4_t app[1];
    if (app_on) {
        append_load<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app);
        fused_append<D, kThreads, 1, append_pieces<D, kThreads, kQC>()>(a, g, r0, app_rows, tid,
                                                                        false);
    }

    // ---- query fragment (B operand of S^T = K Q^T): column qc
    uint4 qf[NS];
    int lim, qrow;
    {
        const int row = r0 + qc / G;
        const bool ok = (qc < BR * G) && (row < sv.rows);
        const int rr = ok ? row : r0;
        const int srow = rr < sv.q_src_rows ? rr : sv.q_src_rows - 1;
        const int head = g * G + (ok ? qc % G : 0);
        qrow = rr;
        lim = sv.causal_base + rr;
        const uint16_t *qp =
            (const uint16_t *)a.q + ((int64_t)(sv.q_row0 + srow) * a.Hq + head) * D + 8 * hi;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *(const uint4 *)(qp + 16 * s);
    }

    // ---- key range of this workgroup
    const int last_row = min(r0 + BR, sv.rows) - 1;
    const int key_end = min(sv.n_keys, sv.causal_base + last_row + 1);   // exclusive
    int t_first = sv.key_lo / kBK;
    int t_last = (key_end - 1) / kBK;
    if (a.n_parts > 1) {
        // this workgroup's part of the key range (absolute tiles), possibly empty
        t_first = max(t_first, (int)blockIdx.y * a.part_tiles);
        t_last = min(t_last, ((int)blockIdx.y + 1) * a.part_tiles - 1);
    }

    // ---- direct global->LDS tile loads: load i of this wave fills LDS
    // chunks [(i*WAVES + wave)*64, +64) of the tile, one 16-byte chunk per
    // lane.  The per-lane element offsets inside a tile are loop invariant;
    // each tile adds one uniform base, and only a tile that runs past the
    // last valid key clamps its rows (to re-read the last valid key).
    uint32_t koff[TL::LOADS], voff[TL::LOADS];   // byte offsets inside a tile
    int lrow[TL::LOADS];
#pragma unroll
    for (int i = 0; i < TL::LOADS; ++i) {
        const int t = (i * TL::WAVES + wave) * 64 + lane;
        const int row = t / NCH;
        const int pos = t % NCH;
        lrow[i] = row;
        koff[i] = (uint32_t)(row * D + (pos ^ TL::swz_k(row)) * 8) * 2u;
        voff[i] = (uint32_t)(row * D + (pos ^ TL::swz_v(row)) * 8) * 2u;
    }
    auto load16 = [](const char *src, uint16_t *dst) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    };
    PagedTiles ptiles;
    auto issue_tile = [&](int kt, uint16_t *Kb) {
        uint16_t *Vb = Kb + kBK * D;
        const int key0 = kt * kBK;
        // physical row of the tile's first key (rolling ring buffer; the
        // identity otherwise), and whether the tile's rows stay contiguous
        int phys0 = key0 + a.ring_start;
        if (phys0 >= a.cap) phys0 -= a.cap;
        const bool nowrap = phys0 + kBK <= a.cap;
        const char *kt_base, *vt_base;
        if constexpr (PAGED) {
            // paged pool: the tile lies inside one block
            const int64_t row = ptiles.row(a, g, kt, kBK);
            kt_base = (const char *)((const uint16_t *)a.k + row * D);
            vt_base = (const char *)((const uint16_t *)a.v + row * D);
        } else {
            kt_base = (const char *)(kc + (int64_t)phys0 * D);
            vt_base = (const char *)(vc + (int64_t)phys0 * D);
        }
        if (key0 + kBK <= sv.n_keys && key0 + kBK <= new_lo && nowrap) {
#pragma unroll
            for (int i = 0; i < TL::LOADS; ++i) {
                const int blk = i * TL::WAVES + wave;
                load16(kt_base + koff[i], Kb + blk * 64 * 8);
                load16(vt_base + voff[i], Vb + blk * 64 * 8);
            }
        } else if (!fused && nowrap) {
            // the tile runs past the last valid key: those rows re-read it
#pragma unroll
            for (int i = 0; i < TL::LOADS; ++i) {
                const int blk = i * TL::WAVES + wave;
                const uint32_t back =
                    (uint32_t)max(0, key0 + lrow[i] - (sv.n_keys - 1)) * (uint32_t)(D * 2);
                load16(kt_base + (koff[i] - back), Kb + blk * 64 * 8);
                load16(vt_base + (voff[i] - back), Vb + blk * 64 * 8);
            }
        } else {
            // per-row sources: fused append (rows at or past new_base come
            // from the new rows) or a ring tile that wraps around
#pragma unroll
            for (int i = 0; i < TL::LOADS; ++i) {
                const int blk = i * TL::WAVES + wave;
                const int key = min(key0 + lrow[i], sv.n_keys - 1);
                const int kch = (int)(koff[i] / 2u) - lrow[i] * D;   // swizzled chunk element
                const int vch = (int)(voff[i] / 2u) - lrow[i] * D;
                load16(kv_src(kc, a.k_new, a, g, D, key, kch), Kb + blk * 64 * 8);
                load16(kv_src(vc, a.v_new, a, g, D, key, vch), Vb + blk * 64 * 8);
            }
        }
    };

    // ---- accumulators
    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = a.scale_log2;
    const float inv_scale = 1.0f / a.scale;
    const uint16_t *maskp = (const uint16_t *)a.mask;

    // V^T fragment addressing for the LDS transpose read: in each 16-lane
    // group, lane s supplies 4 elements of row (s/4); lane i receives
    // element i of the 4 rows.  Row j of half-read j2 is key
    // 16*s2 + 8*j2 + 4*hi + j of this wave's 32 keys, columns
    // d = 32*db + 16*g16 .. +16, so the lane receives V[key][d] for the same
    // keys, in the same order, as its probabilities for that k-step.
    const int g16 = (lane >> 4) & 1;
    const int si = lane & 15;
    const int vrow_off = ks * 32 + 4 * hi + (si >> 2);   // + 16*s2 + 8*j2
    const int vcol = 16 * g16 + 4 * (si & 3);            // + 32*db
    const int krow = ks * 32 + c32;

    // one tile: wait for its loads, start the next tile's loads into the
    // other buffer, then compute on this one
    // Explicit additive mask.  With an 8-byte aligned mask whose row length
    // is a multiple of 4, the lane's 16 keys of a tile are 4 runs of 4
    // consecutive keys: one 8-byte load per run (a run starting at or past
    // the row's end is re-read from the row's last run; those keys are
    // masked out whatever the values).  Those words are loaded one tile
    // ahead, behind the next tile's loads, so the wait at the start of a
    // tile covers them.
    const uint16_t *mrow = maskp ? maskp + (int64_t)qrow * a.mask_ld : nullptr;
    const bool mfast = maskp && (a.mask_ld & 3) == 0 && ((uintptr_t)maskp & 7u) == 0;
    uint2 mnext[4];
    auto load_mask = [&](int kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key0 = min(kt * kBK + ks * 32 + 8 * r + 4 * hi, a.mask_ld - 4);
            mnext[r] = *(const uint2 *)(mrow + key0);
        }
    };
    if (mfast && t_last >= t_first) load_mask(t_first);

    auto tile_step = [&](int kt, const uint16_t *Kb, uint16_t *next) {
        __builtin_amdgcn_s_waitcnt(0);     // this wave's loads of tile kt have landed
        __syncthreads();                   // ... and every wave's; `next` is free again
        // the append's loads have landed with the first tile's
        if (kt == t_first && app_on)
            append_store<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app, true);
        const int kbase = kt * kBK + ks * 32;
        float mvals[16];
        if (mfast) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mvals[4 * r + 0] = TR::to_f32(mnext[r].x & 0xffffu);
                mvals[4 * r + 1] = TR::to_f32(mnext[r].x >> 16);
                mvals[4 * r + 2] = TR::to_f32(mnext[r].y & 0xffffu);
                mvals[4 * r + 3] = TR::to_f32(mnext[r].y >> 16);
            }
        } else if (maskp) {
            // other layouts: element loads of this tile (issued before the
            // next tile's loads, so waiting for them does not wait for those)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kbase + 8 * (j >> 2) + 4 * hi + (j & 3);
                mvals[j] = TR::to_f32(mrow[key < sv.n_keys ? key : sv.n_keys - 1]);
            }
        }
        if (kt < t_last) {
            issue_tile(kt + 1, next);
            if (mfast) load_mask(kt + 1);
        }
        const uint16_t *Vb = Kb + kBK * D;

        // S^T[32 keys x 32 cols] for this wave's key slice and column group.
        // Matrix sections run at raised wave priority: the wave that reaches
        // them first keeps the matrix pipe while its SIMD partner does vector
        // work, which de-phases the two waves of a SIMD.
        __builtin_amdgcn_s_setprio(1);
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
        {
            const uint16_t *kr = Kb + krow * D;
            const int sk = TL::swz_k(krow);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 ka = *(const uint4 *)(kr + ((2 * s + hi) ^ sk) * 8);
                sacc = TR::mfma(ka, qf[s], sacc);
            }
        }
        __builtin_amdgcn_s_setprio(0);

        // Accumulator register j of lane (c32, hi) holds key
        // kbase + 8*(j/4) + 4*hi + (j%4) for query column qc.
        const bool full = (kt * kBK >= sv.key_lo) && ((kt + 1) * kBK <= sv.n_keys) &&
                          ((kt + 1) * kBK - 1 <= sv.causal_base + r0);
        if (maskp) {
            // additive mask; entries at or below the fill value (-32768)
            // exclude the slot (their weight underflows to exactly 0
            // whenever the row sees any slot)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kbase + 8 * (j >> 2) + 4 * hi + (j & 3);
                const bool vis = key >= sv.key_lo && key < sv.n_keys && mvals[j] > -32768.0f;
                sacc[j] = vis ? sacc[j] + mvals[j] * inv_scale : -INFINITY;
            }
        } else if (!full) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kbase + 8 * (j >> 2) + 4 * hi + (j & 3);
                const bool vis = key >= sv.key_lo && key <= lim && key < sv.n_keys;
                sacc[j] = vis ? sacc[j] : -INFINITY;
            }
        }

        // online softmax (exp2 domain), lazy maximum
        float mx = sacc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
        mx = pair_max(mx);
        const float mt = mx * c;
        const bool need = mt > m_run + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float alpha = need ? exp2f(m_run - mt) : 1.0f;
            m_run = need ? mt : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
        const float mu = m_run == -INFINITY ? 0.f : m_run;
        uint4 pb[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * s2 + 2 * i], c, -mu));
                const float p1 =
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * s2 + 2 * i + 1], c, -mu));
                w[i] = TR::pack(p0, p1);
                l_run = TR::dot2(w[i], TR::kOnes, l_run);
            }
            pb[s2] = make_uint4(w[0], w[1], w[2], w[3]);
        }

        // O^T[d x cols] += V^T[d x 32 keys] P^T[32 keys x cols]
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint2 half[2];
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const int vrow = vrow_off + 16 * s2 + 8 * j2;
                    const int dd = 32 * db + vcol;
                    const uint16_t *vp =
                        Vb + vrow * D + (((dd >> 3) ^ TL::swz_v(vrow)) << 3) + (dd & 7);
                    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
                    half[j2] = __builtin_bit_cast(uint2, r);
                }
                const uint4 va = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
                oacc[db] = TR::mfma(va, pb[s2], oacc[db]);
            }
        __builtin_amdgcn_s_setprio(0);
    };

    if constexpr (PAGED) {
        ptiles.stage(a, sv.slot, t_first * kBK, (t_last + 1) * kBK - 1, ptab, tid, kThreads);
        __syncthreads();
    }
    if (t_last >= t_first) {
        issue_tile(t_first, buf0);
        for (int kt = t_first; kt <= t_last; kt += 2) {
            tile_step(kt, buf0, buf1);
            if (kt + 1 <= t_last) tile_step(kt + 1, buf1, buf0);
        }
    } else if (app_on) {
        append_store<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app, true);
    }
    __syncthreads();   // all waves are done with the tiles: reuse LDS below

    // ---- merge the four key slices' partial states, normalise, write rows
    // (slices 0-1 stage their rows in buf0, slices 2-3 in buf1)
    float *Ms = ml;
    float *Ls = ml + 4 * kQC;
    auto orow = [&](int slice, int col) -> float * {
        float *base = (float *)(slice < 2 ? buf0 : buf1);
        return base + ((slice & 1) * kQC + col) * D;
    };
    {
        const float lt = pair_sum(l_run);
        if (hi == 0) {
            Ms[ks * kQC + qc] = m_run;
            Ls[ks * kQC + qc] = lt;
        }
    }
    __syncthreads();
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, Ms[w * kQC + qc]);
        float den = 0.f, mine = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = Ms[w * kQC + qc];
            const float e = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            den += e * Ls[w * kQC + qc];
            if (w == ks) mine = e;
        }
        // split parts keep the slices' sum unnormalised (the combine
        // normalises over all parts); otherwise normalise here
        const float f = a.n_parts > 1 ? mine : (den > 0.f ? mine / den : 0.f);
        float *dst = orow(ks, qc);
        const int sw = TL::swz_o(qc);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d4 = db * 8 + 2 * j4 + hi;     // float4 column of d = 4*d4
                float4 v4 = make_float4(oacc[db][4 * j4] * f, oacc[db][4 * j4 + 1] * f,
                                        oacc[db][4 * j4 + 2] * f, oacc[db][4 * j4 + 3] * f);
                *(float4 *)(dst + 4 * (d4 ^ sw)) = v4;
            }
    }
    __syncthreads();
    {
        constexpr int PARTS = kThreads / kQC;    // threads per query column
        constexpr int DP = D / PARTS;            // output elements per thread
        const int oc = tid / PARTS;
        const int part = tid % PARTS;
        const int row = r0 + oc / G;
        if (oc < BR * G && row < sv.out_rows && a.n_parts > 1) {
            // partial record of this part: [M, den, 0, 0, O[D]]
            const int head = g * G + oc % G;
            float *rec =
                a.part_ws + (((int64_t)blockIdx.y * sv.out_rows + row) * a.Hq + head) * (D + 4);
            if (part == 0) {
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < 4; ++w) M = fmaxf(M, Ms[w * kQC + oc]);
                float den = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float mw = Ms[w * kQC + oc];
                    den += ((mw == -INFINITY) ? 0.f : exp2f(mw - M)) * Ls[w * kQC + oc];
                }
                *(float4 *)rec = make_float4(M, den, 0.f, 0.f);
            }
            const int sw = TL::swz_o(oc);
#pragma unroll
            for (int d4 = 0; d4 < DP; d4 += 4) {
                const int d = part * DP + d4;
                const int off = 4 * ((d >> 2) ^ sw);
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    const float4 y = *(const float4 *)(orow(w4, oc) + off);
                    x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
                }
                *(float4 *)(rec + 4 + d) = x;
            }
        } else if (oc < BR * G && row < sv.out_rows) {
            const int head = g * G + oc % G;
            uint16_t *op = (uint16_t *)a.out + ((int64_t)(sv.out_row0 + row) * a.Hq + head) * D +
                           part * DP;
            const int sw = TL::swz_o(oc);
#pragma unroll
            for (int d8 = 0; d8 < DP; d8 += 8) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x0 = 0.f, x1 = 0.f;
                    const int d = part * DP + d8 + 2 * i;
                    const int off = 4 * ((d >> 2) ^ sw) + (d & 3);
#pragma unroll
                    for (int w4 = 0; w4 < 4; ++w4) {
                        const float *src = orow(w4, oc);
                        x0 += src[off];
                        x1 += src[off + 1];
                    }
                    w[i] = TR::pack(x0, x1);
                }
                *(uint4 *)(op + d8) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

// ------------------------------------------------------------ wide kernel
//
// attn_wide_kernel: 128 query columns per workgroup, 4 waves (one per SIMD)
// and 64-key tiles.  Wave w takes column group w / 2 (64 columns = two
// 32-column MFMA blocks) and key half w % 2 (32 of the 64 keys of every
// tile).  Every K or V fragment a wave reads from LDS feeds two MFMAs and
// every staged tile serves 128 columns: half the LDS reads and L2->LDS fill
// per flop of attn_mfma_kernel.
//
// With a single wave per SIMD nothing hides latency but the wave's own
// instruction stream, so the loop is software-pipelined across tiles: while
// the matrix unit computes the scores of tile t+1 the vector unit turns
// the scores of tile t into probabilities, and while it accumulates P V of
// tile t the vector unit masks and reduces the scores of tile t+1.  K and V
// tiles live in separate two-stage rings, K one tile ahead of V, so one
// barrier per tile suffices.  Fragment layouts, swizzles, the lazy maximum
// and the split records are those of attn_mfma_kernel; the two key halves
// are merged once at the end through LDS.

constexpr int kWQC = 128;        // query columns per workgroup
constexpr int kWThreads = 256;   // 4 waves = 2 column groups x 2 key halves
constexpr int kWBK = 64;         // keys per tile
constexpr int kWStages = 4;      // ring slots: tiles are loaded three ahead

// Exchange between the two 32-lane halves without LDS: permlane32_swap of a
// value with itself yields the low half's value in every lane (first
// result) and the high half's (second); both halves then combine the same
// operands in the same order, so their results are bit-identical.
__device__ __forceinline__ float half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keep a value in accumulation registers: the matrix instructions read
// their A/B operands from them directly, which leaves the vector registers
// to the softmax.  (An empty asm with an "a" constraint; no instruction.)
__device__ __forceinline__ uint4 in_agprs(uint4 x)
{
    u32x4_t t = {x.x, x.y, x.z, x.w};
    asm volatile("" : "+a"(t));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Mark a value as produced here: an empty asm that takes and returns it in
// vector registers, so that its computation is not moved past a later
// branch (it is then scheduled among the independent matrix instructions
// before that branch).  No instruction is emitted.
__device__ __forceinline__ uint4 here(uint4 x)
{
    u32x4_t t = {x.x, x.y, x.z, x.w};
    asm volatile("" : "+v"(t));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// One work item of the 128-column kernel: row block and KV head bx, split
// part by, sequence bz.
template <typename TR, int D, bool PAGED>
__device__ __forceinline__ void attn_wide_item(const AttnArgs &a, int bx, int by, int bz)
{
    using TL = Tile<D>;
    constexpr int NCH = TL::NCH;
    constexpr int NS = D / 16;      // k-steps of the QK^T contraction
    constexpr int NDB = D / 32;     // 32-wide d blocks of O^T
    constexpr int WAVES = kWThreads / 64;
    constexpr int TILE = kWBK * D;                  // uint16 elements of one K or V tile
    constexpr int LOADS = kWBK * NCH / kWThreads;   // 16-byte loads per thread per tensor
    static_assert(kWBK * NCH % kWThreads == 0, "tile loads split evenly");
    static_assert(kAttnTileKeys % kWBK == 0, "split parts are whole tiles");
    // s_waitcnt immediates (gfx9 encoding): vector memory count <= the
    // loads of one or two later tiles (2 * LOADS per tile per wave), the
    // other counters unconstrained
    constexpr int kTileLoads = 2 * LOADS;
    static_assert(2 * kTileLoads < 64, "vmcnt field is 6 bits");
    constexpr int kWaitOne =
        (kTileLoads & 15) | (7 << 4) | (15 << 8) | ((kTileLoads >> 4) << 14);
    constexpr int kWaitTwo =
        ((2 * kTileLoads) & 15) | (7 << 4) | (15 << 8) | ((2 * kTileLoads) >> 4 << 14);

    // Four ring slots, each a K tile then a V tile, declared as separate
    // arrays so that the compiler can tell that reading one slot while
    // others are being filled by direct loads needs no wait for those loads.
    // After the loop, slot 2*kh + (column / 64) stages the fp32 partial sums
    // of 64 columns of key half kh.
    static_assert(kWStages == 4, "four statically named ring slots");
    static_assert(64 * D * 4 <= 2 * TILE * 2, "a slot holds 64 fp32 partial rows");
    __shared__ __attribute__((aligned(16))) uint16_t ring0[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t ring1[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t ring2[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t ring3[2 * TILE];
    __shared__ float ml[2 * 2 * kWQC];
    __shared__ int ptab[PAGED ? kMaxTableBlocks : 1];

    SeqView sv;
    if (!resolve_seq(a, bz, sv)) return;
    const int G = a.Hq / a.Hkv;
    const int BR = kWQC / G;                // rows per workgroup
    const int g = bx % a.Hkv;       // KV head fastest: one KV head per XCD
    const int r0 = (bx / a.Hkv) * BR;
    if (r0 >= sv.rows) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c32 = lane & 31;
    const int hi = lane >> 5;
    const int cg = wave >> 1;               // columns 64*cg .. +64
    const int kh = wave & 1;                // keys 32*kh .. +32 of every tile

    const uint16_t *kc = (const uint16_t *)a.k + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const uint16_t *vc = (const uint16_t *)a.v + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const bool fused = a.k_new != nullptr;

    // ---- query fragments (B operand of S^T = K Q^T) of the two column
    // blocks, loaded before the fused append's copy so that the two round
    // trips overlap, and moved to accumulation registers after it
    uint4 qf[2][NS];
    int lim[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int qc = cg * 64 + cb * 32 + c32;
        const int row = r0 + qc / G;
        const bool ok = (qc < BR * G) && (row < sv.rows);
        const int rr = ok ? row : r0;
        const int srow = rr < sv.q_src_rows ? rr : sv.q_src_rows - 1;
        const int head = g * G + (ok ? qc % G : 0);
        lim[cb] = sv.causal_base + rr;
        const uint16_t *qp =
            (const uint16_t *)a.q + ((int64_t)(sv.q_row0 + srow) * a.Hq + head) * D + 8 * hi;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[cb][s] = *(const uint4 *)(qp + 16 * s);
    }
    if (fused && by == 0) {
        fused_append<D, kWThreads, 0, append_pieces<D, kWThreads, kWQC>()>(
            a, g, r0, min(r0 + BR, sv.rows) - r0, tid, true);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[cb][s] = in_agprs(qf[cb][s]);

    // ---- key range of this workgroup (and of its split part), in tiles
    const int last_row = min(r0 + BR, sv.rows) - 1;
    const int key_end = min(sv.n_keys, sv.causal_base + last_row + 1);   // exclusive
    int t_first = sv.key_lo / kWBK;
    int t_last = (key_end - 1) / kWBK;
    if (a.n_parts > 1) {
        constexpr int R = kAttnTileKeys / kWBK;
        t_first = max(t_first, by * a.part_tiles * R);
        t_last = min(t_last, (by + 1) * a.part_tiles * R - 1);
    }

    // ---- direct global->LDS tile loads: load i of this wave fills LDS
    // chunks [(i*WAVES + wave)*64, +64) of the tile, one 16-byte chunk per
    // lane, holding global chunk (pos ^ swizzle(row)) of its row; rows past
    // the last valid key re-read that key
    auto load16 = [](const char *src, uint16_t *dst) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    };
    PagedTiles ptiles;
    int64_t prow = 0;   // paged: first row of the tile being issued (set by refill)
    auto issue = [&](const uint16_t *base, int kt, uint16_t *dst, bool is_v) {
        const int key0 = kt * kWBK;
        const char *tb = (const char *)(base + (int64_t)key0 * D);
        if constexpr (PAGED) {
            // paged pool: the tile lies inside one block
            tb = (const char *)((const uint16_t *)(is_v ? a.v : a.k) + prow * D);
        }
        const int clamp = sv.n_keys - 1 - key0;
        if (!fused || key0 + kWBK <= a.new_base) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int blk = i * WAVES + wave;
                const int t = blk * 64 + lane;
                const int row = t / NCH;
                const int pos = t % NCH;
                const int sw = is_v ? TL::swz_v(row) : TL::swz_k(row);
                const uint32_t off = (uint32_t)(min(row, clamp) * D + (pos ^ sw) * 8) * 2u;
                load16(tb + off, dst + blk * 64 * 8);
            }
        } else {
            // fused append: rows at or past new_base come from the new rows
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int blk = i * WAVES + wave;
                const int t = blk * 64 + lane;
                const int row = t / NCH;
                const int pos = t % NCH;
                const int sw = is_v ? TL::swz_v(row) : TL::swz_k(row);
                load16(kv_src(base, is_v ? a.v_new : a.k_new, a, g, D, key0 + min(row, clamp),
                              (pos ^ sw) * 8),
                       dst + blk * 64 * 8);
            }
        }
    };

    // ---- accumulators and per-column softmax state
    f32x16_t oacc[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][cb][j] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    const float c = a.scale_log2;

    const int g16 = (lane >> 4) & 1;
    const int si = lane & 15;
    const int vrow_off = kh * 32 + 4 * hi + (si >> 2);   // + 16*s2 + 8*j2
    const int vcol = 16 * g16 + 4 * (si & 3);            // + 32*db
    const int krow = kh * 32 + c32;

    // ---- the pieces of one tile's work for this wave
    // S^T[32 keys x 64 cols] from the K tile at Kb (each K fragment read
    // once, all reads issued up front, each feeding both column blocks)
    auto scores = [&](const uint16_t *Kb, f32x16_t (&sa)[2]) {
        const uint16_t *kr = Kb + krow * D;
        const int sk = TL::swz_k(krow);
        uint4 kf[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) kf[s] = *(const uint4 *)(kr + ((2 * s + hi) ^ sk) * 8);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int j = 0; j < 16; ++j) sa[cb][j] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sa[0] = TR::mfma(kf[s], qf[0][s], sa[0]);
            sa[1] = TR::mfma(kf[s], qf[1][s], sa[1]);
        }
    };
    // register j of sa[cb] in lane (c32, hi): key
    // 64*kt + 32*kh + 8*(j/4) + 4*hi + (j%4) of column 64*cg + 32*cb + c32
    auto mask_scores = [&](int kt, f32x16_t (&sa)[2]) {
        const bool full = (kt * kWBK >= sv.key_lo) && ((kt + 1) * kWBK <= sv.n_keys) &&
                          ((kt + 1) * kWBK - 1 <= sv.causal_base + r0);
        if (!full) {
            const int kbase = kt * kWBK + kh * 32 + 4 * hi;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const int lo = sv.key_lo - kbase;
                const int hi_ = min(lim[cb], sv.n_keys - 1) - kbase;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int o = 8 * (j >> 2) + (j & 3);
                    sa[cb][j] = (o >= lo && o <= hi_) ? sa[cb][j] : -INFINITY;
                }
            }
        }
    };
    auto tile_max = [&](const f32x16_t (&sa)[2], float (&mt)[2]) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float mx = sa[cb][0];
#pragma unroll
            for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sa[cb][j]);
            mt[cb] = half_max(mx) * c;
        }
    };
    // online softmax (exp2 domain), lazy maximum: raise the running maximum
    // only where a tile's exceeds it by more than 2^8 (rare after the first
    // tile)
    auto rescale = [&](const float (&mt)[2]) {
        const bool n0 = mt[0] > m_run[0] + kLazyLog2;
        const bool n1 = mt[1] > m_run[1] + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(n0 || n1) != 0) {
            const float al0 = n0 ? exp2f(m_run[0] - mt[0]) : 1.0f;
            const float al1 = n1 ? exp2f(m_run[1] - mt[1]) : 1.0f;
            m_run[0] = n0 ? mt[0] : m_run[0];
            m_run[1] = n1 ? mt[1] : m_run[1];
            l_run[0] *= al0;
            l_run[1] *= al1;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    oacc[db][0][j] *= al0;
                    oacc[db][1][j] *= al1;
                }
        }
    };
    // probabilities as B operands (k-step s2 holds registers 8*s2 .. +7)
    auto probs = [&](const f32x16_t (&sa)[2], uint4 (&pb)[2][2]) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const float mu = m_run[cb] == -INFINITY ? 0.f : m_run[cb];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(sa[cb][8 * s2 + 2 * i], c, -mu));
                    const float p1 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(sa[cb][8 * s2 + 2 * i + 1], c, -mu));
                    w[i] = TR::pack(p0, p1);
                }
                pb[cb][s2] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    // V^T fragments of this wave's 32 keys of the V tile at Vb (k-step s2,
    // d block db), and O^T[d x 64 cols] += V^T[d x 32 keys] P^T[32 keys x
    // 64 cols] (each fragment feeding both column blocks), then the row
    // sums of P
    auto vfrags = [&](const uint16_t *Vb, uint4 (&vf)[NDB][2]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint2 half[2];
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const int vrow = vrow_off + 16 * s2 + 8 * j2;
                    const int dd = 32 * db + vcol;
                    const uint16_t *vp =
                        Vb + vrow * D + (((dd >> 3) ^ TL::swz_v(vrow)) << 3) + (dd & 7);
                    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
                    half[j2] = __builtin_bit_cast(uint2, r);
                }
                vf[db][s2] = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
            }
    };
    auto accumulate = [&](const uint4 (&vf)[NDB][2], const uint4 (&pb)[2][2]) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                oacc[db][0] = TR::mfma(vf[db][s2], pb[0][s2], oacc[db][0]);
                oacc[db][1] = TR::mfma(vf[db][s2], pb[1][s2], oacc[db][1]);
            }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                l_run[cb] = TR::dot2(pb[cb][s2].x, TR::kOnes, l_run[cb]);
                l_run[cb] = TR::dot2(pb[cb][s2].y, TR::kOnes, l_run[cb]);
                l_run[cb] = TR::dot2(pb[cb][s2].z, TR::kOnes, l_run[cb]);
                l_run[cb] = TR::dot2(pb[cb][s2].w, TR::kOnes, l_run[cb]);
            }
    };

    // ---- software-pipelined tile loop over four ring slots: tile
    // t_first + i sits in slot i % 4 and is loaded three steps ahead.  The
    // step for tile t (t < t_last) computes the scores of tile t+1 on the
    // matrix unit while the vector unit turns the scores of tile t into
    // probabilities, then accumulates P V of tile t while the vector unit
    // masks and reduces the scores of tile t+1; the running-maximum check
    // for tile t+1 closes the step.  It needs K(t+1) and V(t): it waits for
    // its loads with at most those of tile t+2 pending, passes a barrier
    // (after which the slot of tile t-1, whose K and V were last read by
    // the two previous steps, is free) and refills that slot with tile t+3.
    // The barrier carries no memory fence, which would wait for every load
    // in flight; empty asm statements with a memory clobber keep the
    // compiler from moving LDS accesses across it.
    auto sync = [&](bool one_pending) {
        if (one_pending)
            __builtin_amdgcn_s_waitcnt(kWaitOne);
        else
            __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto refill = [&](int t, uint16_t *slot) {
        if (t <= t_last) {
            if constexpr (PAGED) prow = ptiles.row(a, g, t, kWBK);
            issue(kc, t, slot, false);
            issue(vc, t, slot + TILE, true);
        }
    };
    auto step = [&](int t, const uint16_t *cur, const uint16_t *nxt, uint16_t *free_slot,
                    f32x16_t (&scur)[2], f32x16_t (&snxt)[2]) {
        // V(t) is complete and visible since the previous step's barrier
        uint4 vf[NDB][2];
        vfrags(cur + TILE, vf);
        sync(t + 2 <= t_last);
        refill(t + 3, free_slot);
        uint4 pb[2][2];
        float mt[2];
        scores(nxt, snxt);
        probs(scur, pb);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) pb[cb][s2] = here(pb[cb][s2]);
        mask_scores(t + 1, snxt);
        accumulate(vf, pb);
        tile_max(snxt, mt);
        rescale(mt);
    };
    auto drain = [&](const uint16_t *cur, const f32x16_t (&scur)[2]) {
        sync(false);
        uint4 vf[NDB][2];
        vfrags(cur + TILE, vf);
        uint4 pb[2][2];
        probs(scur, pb);
        accumulate(vf, pb);
    };
    if constexpr (PAGED) {
        ptiles.stage(a, sv.slot, t_first * kWBK, (t_last + 1) * kWBK - 1, ptab, tid, kWThreads);
        __syncthreads();
    }
    if (t_last >= t_first) {
        f32x16_t s0[2], s1[2];
        refill(t_first, ring0);
        refill(t_first + 1, ring1);
        refill(t_first + 2, ring2);
        {
            // tile t_first: its loads are the oldest of up to three tiles
            if (t_first + 2 <= t_last)
                __builtin_amdgcn_s_waitcnt(kWaitTwo);
            else
                __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            float mt[2];
            scores(ring0, s0);
            mask_scores(t_first, s0);
            tile_max(s0, mt);
            rescale(mt);
        }
        // whole rounds of four steps, then up to three, then the last tile
        int t = t_first;
        for (; t + 4 <= t_last; t += 4) {
            step(t, ring0, ring1, ring3, s0, s1);
            step(t + 1, ring1, ring2, ring0, s1, s0);
            step(t + 2, ring2, ring3, ring1, s0, s1);
            step(t + 3, ring3, ring0, ring2, s1, s0);
        }
        if (t < t_last) step(t++, ring0, ring1, ring3, s0, s1);
        if (t < t_last) step(t++, ring1, ring2, ring0, s1, s0);
        if (t < t_last) step(t++, ring2, ring3, ring1, s0, s1);
        const int last = (t_last - t_first) & 3;   // slot of the last tile
        const uint16_t *cur = last == 0 ? ring0 : last == 1 ? ring1 : last == 2 ? ring2 : ring3;
        if (last & 1)
            drain(cur, s1);
        else
            drain(cur, s0);
    }
    __syncthreads();   // all waves are done with the tiles: reuse LDS below

    // ---- merge the two key halves: half kh stages its scaled partial sums
    // (fp32 [column][D], float4-swizzled by column) at float offset kh*128*D
    float *Ms = ml;
    float *Ls = ml + 2 * kWQC;
    // fp32 partial row of key half h, column col
    auto stage_row = [&](int h, int col) -> float * {
        uint16_t *slot = h == 0 ? (col < 64 ? ring0 : ring1) : (col < 64 ? ring2 : ring3);
        return (float *)slot + (col & 63) * D;
    };
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const float lt = half_sum(l_run[cb]);
        if (hi == 0) {
            Ms[kh * kWQC + cg * 64 + cb * 32 + c32] = m_run[cb];
            Ls[kh * kWQC + cg * 64 + cb * 32 + c32] = lt;
        }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int col = cg * 64 + cb * 32 + c32;
        const float m0 = Ms[col], m1 = Ms[kWQC + col];
        const float M = fmaxf(m0, m1);
        const float e0 = (m0 == -INFINITY) ? 0.f : exp2f(m0 - M);
        const float e1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - M);
        const float den = e0 * Ls[col] + e1 * Ls[kWQC + col];
        const float mine = kh ? e1 : e0;
        // split parts keep the sum unnormalised (the combine normalises)
        const float f = a.n_parts > 1 ? mine : (den > 0.f ? mine / den : 0.f);
        float *dst = stage_row(kh, col);
        const int sw = TL::swz_o(col);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d4 = db * 8 + 2 * j4 + hi;     // float4 column of d = 4*d4
                const float4 v4 =
                    make_float4(oacc[db][cb][4 * j4] * f, oacc[db][cb][4 * j4 + 1] * f,
                                oacc[db][cb][4 * j4 + 2] * f, oacc[db][cb][4 * j4 + 3] * f);
                *(float4 *)(dst + 4 * (d4 ^ sw)) = v4;
            }
    }
    __syncthreads();
    {
        constexpr int PARTS = kWThreads / kWQC;   // threads per query column
        constexpr int DP = D / PARTS;             // output elements per thread
        const int oc = tid / PARTS;
        const int part = tid % PARTS;
        const int row = r0 + oc / G;
        const float *s0 = stage_row(0, oc);
        const float *s1 = stage_row(1, oc);
        const int sw = TL::swz_o(oc);
        if (oc < BR * G && row < sv.out_rows && a.n_parts > 1) {
            const int head = g * G + oc % G;
            float *rec =
                a.part_ws + (((int64_t)by * sv.out_rows + row) * a.Hq + head) * (D + 4);
            if (part == 0) {
                const float m0 = Ms[oc], m1 = Ms[kWQC + oc];
                const float M = fmaxf(m0, m1);
                const float den = ((m0 == -INFINITY) ? 0.f : exp2f(m0 - M)) * Ls[oc] +
                                  ((m1 == -INFINITY) ? 0.f : exp2f(m1 - M)) * Ls[kWQC + oc];
                *(float4 *)rec = make_float4(M, den, 0.f, 0.f);
            }
#pragma unroll
            for (int d4 = 0; d4 < DP; d4 += 4) {
                const int d = part * DP + d4;
                const int off = 4 * ((d >> 2) ^ sw);
                const float4 x = *(const float4 *)(s0 + off);
                const float4 y = *(const float4 *)(s1 + off);
                *(float4 *)(rec + 4 + d) = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
            }
        } else if (oc < BR * G && row < sv.out_rows) {
            const int head = g * G + oc % G;
            uint16_t *op = (uint16_t *)a.out + ((int64_t)(sv.out_row0 + row) * a.Hq + head) * D +
                           part * DP;
#pragma unroll
            for (int d8 = 0; d8 < DP; d8 += 8) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int d = part * DP + d8 + 4 * i;
                    const int off = 4 * ((d >> 2) ^ sw);
                    const float4 x = *(const float4 *)(s0 + off);
                    const float4 y = *(const float4 *)(s1 + off);
                    w[2 * i] = TR::pack(x.x + y.x, x.y + y.y);
                    w[2 * i + 1] = TR::pack(x.z + y.z, x.w + y.w);
                }
                *(uint4 *)(op + d8) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

// The 128-column kernel: one work item per workgroup.
template <typename TR, int D, bool PAGED>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_wide_kernel(AttnArgs a)
{
    prefetch_args(a);
    attn_wide_item<TR, D, PAGED>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ------------------------------------------------------- scheduled kernel
//
// attn_sched_kernel: the 64-column kernel's work split (8 waves = 2 column
// groups x 4 key slices of 128-key tiles, tiles double-buffered in LDS) for
// launches over a contiguous cache (causal, computed or explicit additive
// mask visibility, a ring buffer, a key-range split into parts; a paged
// pool takes attn_mfma_kernel), scheduled for latency:
// * all eight K fragment reads of a tile are issued before its first
//   matrix instruction, so the QK^T chain is not broken by LDS round trips;
// * the V^T fragments of the tile are read right after the QK^T
//   instructions, so those reads complete while the vector unit runs the
//   softmax (whose cross-half exchange is a register permute, not an LDS
//   operation that would have to wait for them);
// * P V accumulates into four independent register blocks per k-step, so
//   consecutive matrix instructions do not depend on each other;
// * tiles that lie entirely inside the chunk's new rows (fused append) are
//   loaded with per-lane offsets precomputed for the new rows' stride,
//   without per-row source selection;
// * the next tile's direct-to-LDS loads are issued by column group 0
//   alone, so group 1's waves never stall on the address unit;
// * the workgroup's query rows are read from global memory once, into LDS
//   by column group 1 beside the first tile's loads (the four key-slice
//   waves of a column group need the same query fragments), and each wave
//   takes its fragments from LDS after the first tile's barrier;
// * with prev_ws set (a deferred ring step), column group 1 also merges its
//   workgroup's share of the previous split launch's parts (combine_unit)
//   while the first tile is in flight.
// Arithmetic, fragment layouts, swizzles, the lazy maximum, the epilogue
// merge and the fused append are those of attn_mfma_kernel, so results are
// bit-identical to it.
template <typename TR, int D, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_sched_kernel(AttnArgs a)
{
    using TL = Tile<D>;
    constexpr int NCH = TL::NCH;
    constexpr int NS = D / 16;      // k-steps of the QK^T contraction
    constexpr int NDB = D / 32;     // 32-wide d blocks of O^T

    __shared__ __attribute__((aligned(16))) uint16_t buf0[TL::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t buf1[TL::STAGE];
    __shared__ float ml[2 * 4 * kQC];
    __shared__ __attribute__((aligned(16))) uint16_t qbuf[kQC * D];   // the workgroup's query rows

    prefetch_args(a);
    SeqView sv;
    if (!resolve_seq(a, blockIdx.z, sv)) return;
    const int G = a.Hq / a.Hkv;
    const int BR = kQC / G;                 // rows per workgroup
    const int g = blockIdx.x % a.Hkv;       // KV head fastest: one KV head per XCD
    const int r0 = (blockIdx.x / a.Hkv) * BR;
    if (r0 >= sv.rows) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c32 = lane & 31;
    const int hi = lane >> 5;
    const int qg = wave >> 2;               // query-column group
    const int ks = wave & 3;                // key slice of every tile
    const int qc = qg * 32 + c32;

    const uint16_t *kc = (const uint16_t *)a.k + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const uint16_t *vc = (const uint16_t *)a.v + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const bool fused = a.k_new != nullptr;
    const int new_lo = fused ? a.new_base : INT_MAX;
    // new rows usable without clamping: keys [new_base, new_hi)
    const int new_hi = fused ? min(sv.n_keys, a.new_base + a.new_rows) : INT_MIN;
    const bool app_on = fused && blockIdx.y == 0;
    const int app_rows = min(r0 + BR, sv.rows) - r0;
    u32x4_t app[1];
    if (app_on) {
        append_load<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app);
        fused_append<D, kThreads, 1, append_pieces<D, kThreads, kQC>()>(a, g, r0, app_rows, tid,
                                                                        false);
    }

    // ---- query fragment (B operand of S^T = K Q^T): column qc.  The
    // 64 columns' query rows are read once per workgroup into LDS by column
    // group 1 (chunk p of column c stored at p ^ (c mod NCH)), and every wave
    // takes its fragments from there after the first tile's barrier.
    uint4 qf[NS];
    int lim, qrow;
    {
        const int row = r0 + qc / G;
        const bool ok = (qc < BR * G) && (row < sv.rows);
        const int rr = ok ? row : r0;
        lim = min(sv.causal_base + rr, sv.n_keys - 1);
        qrow = rr;
    }
    if (qg == 1) {
        constexpr int QLD = kQC * NCH / (4 * 64);   // 1 KB loads per group-1 wave
#pragma unroll
        for (int i = 0; i < QLD; ++i) {
            const int blk = i * 4 + (wave - 4);
            const int t = blk * 64 + lane;          // destination chunk
            const int col = t / NCH;
            const int pch = (t % NCH) ^ (col % NCH);  // source chunk
            const int row = r0 + col / G;
            const bool ok = (col < BR * G) && (row < sv.rows);
            const int rr = ok ? row : r0;
            const int srow = rr < sv.q_src_rows ? rr : sv.q_src_rows - 1;
            const int head = g * G + (ok ? col % G : 0);
            const uint16_t *src =
                (const uint16_t *)a.q + ((int64_t)(sv.q_row0 + srow) * a.Hq + head) * D + pch * 8;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(qbuf + blk * 64 * 8), 16, 0, 0);
        }
        // carried merge of an earlier split launch's parts: this
        // workgroup's share of the merge units, taken by column group 1
        // while the first tile is in flight (every workgroup of a scalar
        // launch has rows, so all of them get here)
        if (__builtin_expect(a.prev_ws != nullptr, 0)) {   // laid out off the hot path
            constexpr int kMT = kThreads / 2;
            const int units = a.out_rows * a.Hq * (D / 8);
            const int n_wg = gridDim.x * gridDim.y;
            const int per = (units + n_wg - 1) / n_wg;
            const int u0 = (blockIdx.y * gridDim.x + blockIdx.x) * per;
            const int u1 = min(units, u0 + per);
            for (int u = u0 + (tid - kMT); u < u1; u += kMT)
                combine_unit<TR, D>(a.prev_ws, a.n_parts, a.out_rows, a.Hq, a.prev_out, 0, u);
        }
    }
    auto read_q = [&]() __attribute__((always_inline)) {
        const uint16_t *qr = qbuf + qc * D;
        const int sq = qc % NCH;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *(const uint4 *)(qr + ((2 * s + hi) ^ sq) * 8);
    };

    const int last_row = min(r0 + BR, sv.rows) - 1;
    const int key_end = min(sv.n_keys, sv.causal_base + last_row + 1);   // exclusive
    int t_first = sv.key_lo / kBK;
    int t_last = (key_end - 1) / kBK;
    if (a.n_parts > 1) {
        // this workgroup's part of the key range (absolute tiles), possibly empty
        t_first = max(t_first, (int)blockIdx.y * a.part_tiles);
        t_last = min(t_last, ((int)blockIdx.y + 1) * a.part_tiles - 1);
    }

    // ---- tile loads, issued by column group 0 alone (waves 0-3, one per
    // SIMD): a wave stalls while the address unit works through its loads,
    // and group 0 reaches the tile barrier early, so it absorbs that stall
    // while group 1's waves keep their matrix work going.  Load i of loader
    // wave lw fills LDS chunks [(i*LW + lw)*64, +64), one 16-byte chunk per
    // lane: tile row i*RSTEP + row0 (RSTEP = LW*64/NCH rows apart), chunk
    // pos.  The swizzles depend on the row modulo NCH, which RSTEP leaves
    // unchanged, so one per-lane offset serves every load of the tile and
    // load i adds a uniform i*RSTEP rows to the (scalar) base: byte offsets
    // for cache rows (stride D) and for the new rows (stride Hkv*D).
    constexpr int LW = TL::WAVES / 2;
    const int lw = qg == 0 ? wave : -1;
    constexpr int RSTEP = LW * 64 / NCH;
    constexpr int NLD = kBK / RSTEP;
    static_assert(RSTEP % NCH == 0, "row step keeps the swizzle");
    const int row0 = ((lw < 0 ? 0 : lw) * 64 + lane) / NCH;
    const int pos0 = lane % NCH;
    const uint32_t kch = (uint32_t)((pos0 ^ TL::swz_k(row0)) * 8);
    const uint32_t vch = (uint32_t)((pos0 ^ TL::swz_v(row0)) * 8);
    const uint32_t koff = ((uint32_t)row0 * D + kch) * 2u;
    const uint32_t voff = ((uint32_t)row0 * D + vch) * 2u;
    const uint32_t nkoff = ((uint32_t)row0 * a.Hkv * D + kch) * 2u;
    const uint32_t nvoff = ((uint32_t)row0 * a.Hkv * D + vch) * 2u;
    auto load16 = [](const char *src, uint16_t *dst) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    };
    auto issue_tile = [&](int kt, uint16_t *Kb) __attribute__((always_inline)) {
        if (lw < 0) return;   // wave-uniform: group 1 issues no loads
        uint16_t *Vb = Kb + kBK * D;
        const int key0 = kt * kBK;
        // physical row of the tile's first key (rolling ring buffer; the
        // identity otherwise), and whether the tile's rows stay contiguous
        int phys0 = key0 + a.ring_start;
        if (phys0 >= a.cap) phys0 -= a.cap;
        const bool nowrap = phys0 + kBK <= a.cap;
        if (key0 + kBK <= sv.n_keys && key0 + kBK <= new_lo && nowrap) {
            // cache rows
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int blk = i * LW + lw;
                const int64_t e = (int64_t)(phys0 + i * RSTEP) * D;
                load16((const char *)(kc + e) + koff, Kb + blk * 64 * 8);
                load16((const char *)(vc + e) + voff, Vb + blk * 64 * 8);
            }
        } else if (key0 >= new_lo && key0 + kBK <= new_hi) {
            // new rows of the chunk (fused append), no clamping needed
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int blk = i * LW + lw;
                const int64_t e = ((int64_t)(key0 - a.new_base + i * RSTEP) * a.Hkv + g) * D;
                load16((const char *)((const uint16_t *)a.k_new + e) + nkoff, Kb + blk * 64 * 8);
                load16((const char *)((const uint16_t *)a.v_new + e) + nvoff, Vb + blk * 64 * 8);
            }
        } else {
            // per-row sources: rows past the last valid key re-read it;
            // keys at or past new_base come from the new rows (fused); a
            // ring tile that wraps maps each row on its own
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int blk = i * LW + lw;
                const int key = min(key0 + i * RSTEP + row0, sv.n_keys - 1);
                load16(kv_src(kc, fused ? a.k_new : nullptr, a, g, D, key, (int)kch),
                       Kb + blk * 64 * 8);
                load16(kv_src(vc, fused ? a.v_new : nullptr, a, g, D, key, (int)vch),
                       Vb + blk * 64 * 8);
            }
        }
    };

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = a.scale_log2;
    const float inv_scale = 1.0f / a.scale;

    // Explicit additive mask (rolling form).  With an 8-byte aligned mask
    // whose row length is a multiple of 4, the lane's 16 keys of a tile are
    // 4 runs of 4 consecutive keys: one 8-byte load per run (a run starting
    // at or past the row's end is re-read from the row's last run; those
    // keys are masked out whatever the values), loaded one tile ahead behind
    // the next tile's loads, so the wait at the start of a tile covers them.
    // (a compile-time choice: MASK instances serve launches with a mask)
    const uint16_t *maskp = MASK ? (const uint16_t *)a.mask : nullptr;
    const uint16_t *mrow = MASK ? maskp + (int64_t)qrow * a.mask_ld : nullptr;
    const bool mfast = MASK && (a.mask_ld & 3) == 0 && ((uintptr_t)maskp & 7u) == 0;
    uint2 mnext[4];
    auto load_mask = [&](int kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key0 = min(kt * kBK + ks * 32 + 8 * r + 4 * hi, a.mask_ld - 4);
            mnext[r] = *(const uint2 *)(mrow + key0);
        }
    };
    if (MASK && mfast && t_last >= t_first) load_mask(t_first);

    const int g16 = (lane >> 4) & 1;
    const int si = lane & 15;
    const int vrow_off = ks * 32 + 4 * hi + (si >> 2);   // + 16*s2 + 8*j2
    const int vcol = 16 * g16 + 4 * (si & 3);            // + 32*db
    const int krow = ks * 32 + c32;

    auto tile_step = [&](int kt, const uint16_t *Kb, uint16_t *next) {
        __builtin_amdgcn_s_waitcnt(0);     // this wave's loads of tile kt have landed
        __syncthreads();                   // ... and every wave's; `next` is free again
        if (kt == t_first) read_q();       // the query rows have landed too
        if (kt == t_first && app_on)
            append_store<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app, true);
        float mvals[16];
        if constexpr (!MASK) {
        } else if (mfast) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mvals[4 * r + 0] = TR::to_f32(mnext[r].x & 0xffffu);
                mvals[4 * r + 1] = TR::to_f32(mnext[r].x >> 16);
                mvals[4 * r + 2] = TR::to_f32(mnext[r].y & 0xffffu);
                mvals[4 * r + 3] = TR::to_f32(mnext[r].y >> 16);
            }
        } else {
            // other layouts: element loads of this tile, issued before the
            // next tile's loads so that waiting for them does not wait for those
            const int kb0 = kt * kBK + ks * 32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kb0 + 8 * (j >> 2) + 4 * hi + (j & 3);
                mvals[j] = TR::to_f32(mrow[key < sv.n_keys ? key : sv.n_keys - 1]);
            }
        }
        if (kt < t_last) {
            issue_tile(kt + 1, next);
            if (MASK && mfast) load_mask(kt + 1);
        }
        const uint16_t *Vb = Kb + kBK * D;

        // S^T[32 keys x 32 cols]: every K fragment read, then the chain
        __builtin_amdgcn_s_setprio(1);
        uint4 kf[NS];
        {
            const uint16_t *kr = Kb + krow * D;
            const int sk = TL::swz_k(krow);
#pragma unroll
            for (int s = 0; s < NS; ++s) kf[s] = *(const uint4 *)(kr + ((2 * s + hi) ^ sk) * 8);
        }
        __builtin_amdgcn_sched_barrier(0);   // every K read is issued before the first MFMA
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) sacc = TR::mfma(kf[s], qf[s], sacc);
        // V^T fragments of this wave's 32 keys, in flight during the softmax
        uint4 vf[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint2 half[2];
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const int vrow = vrow_off + 16 * s2 + 8 * j2;
                    const int dd = 32 * db + vcol;
                    const uint16_t *vp =
                        Vb + vrow * D + (((dd >> 3) ^ TL::swz_v(vrow)) << 3) + (dd & 7);
                    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)vp);
                    half[j2] = __builtin_bit_cast(uint2, r);
                }
                vf[db][s2] = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
            }
        // issue order: each matrix instruction followed by two of the V^T
        // fragment reads
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * NDB / NS, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);

        // register j of lane (c32, hi): key kbase + 8*(j/4) + 4*hi + (j%4)
        const int kbase = kt * kBK + ks * 32;
        const bool full = (kt * kBK >= sv.key_lo) && ((kt + 1) * kBK <= sv.n_keys) &&
                          ((kt + 1) * kBK - 1 <= sv.causal_base + r0);
        if constexpr (MASK) {
            // additive mask; entries at or below the fill value (-32768)
            // exclude the slot (their weight underflows to exactly 0
            // whenever the row sees any slot)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kbase + 8 * (j >> 2) + 4 * hi + (j & 3);
                const bool vis = key >= sv.key_lo && key < sv.n_keys && mvals[j] > -32768.0f;
                sacc[j] = vis ? sacc[j] + mvals[j] * inv_scale : -INFINITY;
            }
        } else if (!full) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = kbase + 8 * (j >> 2) + 4 * hi + (j & 3);
                sacc[j] = (key >= sv.key_lo && key <= lim) ? sacc[j] : -INFINITY;
            }
        }
        float mx = sacc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
        mx = half_max(mx);
        const float mt = mx * c;
        const bool need = mt > m_run + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float alpha = need ? exp2f(m_run - mt) : 1.0f;
            m_run = need ? mt : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
        const float mu = m_run == -INFINITY ? 0.f : m_run;
        uint4 pb[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * s2 + 2 * i], c, -mu));
                const float p1 =
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * s2 + 2 * i + 1], c, -mu));
                w[i] = TR::pack(p0, p1);
                l_run = TR::dot2(w[i], TR::kOnes, l_run);
            }
            pb[s2] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // O^T[d x cols] += V^T[d x 32 keys] P^T[32 keys x cols]
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] = TR::mfma(vf[db][s2], pb[s2], oacc[db]);
        __builtin_amdgcn_s_setprio(0);
    };

    if (t_last >= t_first) {
        issue_tile(t_first, buf0);
        for (int kt = t_first; kt <= t_last; kt += 2) {
            tile_step(kt, buf0, buf1);
            if (kt + 1 <= t_last) tile_step(kt + 1, buf1, buf0);
        }
    } else if (app_on) {
        append_store<D, kThreads, 0, 1>(a, g, r0, app_rows, tid, app, true);
    }
    __syncthreads();   // all waves are done with the tiles: reuse LDS below

    // ---- merge the four key slices' partial states, normalise, write rows
    float *Ms = ml;
    float *Ls = ml + 4 * kQC;
    auto orow = [&](int slice, int col) -> float * {
        float *base = (float *)(slice < 2 ? buf0 : buf1);
        return base + ((slice & 1) * kQC + col) * D;
    };
    {
        const float lt = half_sum(l_run);
        if (hi == 0) {
            Ms[ks * kQC + qc] = m_run;
            Ls[ks * kQC + qc] = lt;
        }
    }
    __syncthreads();
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, Ms[w * kQC + qc]);
        float den = 0.f, mine = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = Ms[w * kQC + qc];
            const float e = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            den += e * Ls[w * kQC + qc];
            if (w == ks) mine = e;
        }
        // split parts keep the slices' sum unnormalised (the combine
        // normalises over all parts); otherwise normalise here
        const float f = a.n_parts > 1 ? mine : (den > 0.f ? mine / den : 0.f);
        float *dst = orow(ks, qc);
        const int sw = TL::swz_o(qc);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d4 = db * 8 + 2 * j4 + hi;
                float4 v4 = make_float4(oacc[db][4 * j4] * f, oacc[db][4 * j4 + 1] * f,
                                        oacc[db][4 * j4 + 2] * f, oacc[db][4 * j4 + 3] * f);
                *(float4 *)(dst + 4 * (d4 ^ sw)) = v4;
            }
    }
    __syncthreads();
    {
        constexpr int PARTS = kThreads / kQC;
        constexpr int DP = D / PARTS;
        const int oc = tid / PARTS;
        const int part = tid % PARTS;
        const int row = r0 + oc / G;
        if (oc < BR * G && row < sv.out_rows && a.n_parts > 1) {
            // partial record of this part: [M, den, 0, 0, O[D]]
            const int head = g * G + oc % G;
            float *rec =
                a.part_ws + (((int64_t)blockIdx.y * sv.out_rows + row) * a.Hq + head) * (D + 4);
            if (part == 0) {
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < 4; ++w) M = fmaxf(M, Ms[w * kQC + oc]);
                float den = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float mw = Ms[w * kQC + oc];
                    den += ((mw == -INFINITY) ? 0.f : exp2f(mw - M)) * Ls[w * kQC + oc];
                }
                *(float4 *)rec = make_float4(M, den, 0.f, 0.f);
            }
            const int sw = TL::swz_o(oc);
#pragma unroll
            for (int d4 = 0; d4 < DP; d4 += 4) {
                const int d = part * DP + d4;
                const int off = 4 * ((d >> 2) ^ sw);
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    const float4 y = *(const float4 *)(orow(w4, oc) + off);
                    x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
                }
                *(float4 *)(rec + 4 + d) = x;
            }
        } else if (oc < BR * G && row < sv.out_rows) {
            const int head = g * G + oc % G;
            uint16_t *op = (uint16_t *)a.out + ((int64_t)(sv.out_row0 + row) * a.Hq + head) * D +
                           part * DP;
            const int sw = TL::swz_o(oc);
#pragma unroll
            for (int d8 = 0; d8 < DP; d8 += 8) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x0 = 0.f, x1 = 0.f;
                    const int d = part * DP + d8 + 2 * i;
                    const int off = 4 * ((d >> 2) ^ sw) + (d & 3);
#pragma unroll
                    for (int w4 = 0; w4 < 4; ++w4) {
                        const float *src = orow(w4, oc);
                        x0 += src[off];
                        x1 += src[off + 1];
                    }
                    w[i] = TR::pack(x0, x1);
                }
                *(uint4 *)(op + d8) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

// Merge of the split parts of a key range (combine_unit above), one
// thread per 8 consecutive outputs of a (row, head).
template <typename TR, int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a)
{
    const int unit = blockIdx.x * kCombineThreads + threadIdx.x;
    if (unit < a.out_rows * a.Hq * (D / 8))
        combine_unit<TR, D>(a.part_ws, a.n_parts, a.out_rows, a.Hq, a.out, a.out_row0, unit);
}

// ------------------------------------------------------------------ fp32

constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a)
{
    __shared__ float Ks[kF32Keys][D];
    __shared__ float Vs[kF32Keys][D];
    __shared__ float Qs[kQC][D + 1];

    SeqView sv;
    if (!resolve_seq(a, blockIdx.z, sv)) return;
    const int G = a.Hq / a.Hkv;
    const int BR = kQC / G;
    const int g = blockIdx.x % a.Hkv;
    const int r0 = (blockIdx.x / a.Hkv) * BR;
    if (r0 >= sv.rows) return;
    const int t = threadIdx.x;

    const int row = r0 + t / G;
    const bool ok = (t < BR * G) && (row < sv.rows);
    const int rr = ok ? row : r0;
    const int srow = rr < sv.q_src_rows ? rr : sv.q_src_rows - 1;
    const int head = g * G + (ok ? t % G : 0);
    const int lim = sv.causal_base + rr;
    const float *qp = (const float *)a.q + ((int64_t)(sv.q_row0 + srow) * a.Hq + head) * D;
    for (int d = 0; d < D; ++d) Qs[t][d] = qp[d];

    const float *kc = (const float *)a.k + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const float *vc = (const float *)a.v + ((int64_t)sv.slot * a.Hkv + g) * a.cap * D;
    const float *maskp = (const float *)a.mask;

    const int last_row = min(r0 + BR, sv.rows) - 1;
    const int key_end = min(sv.n_keys, sv.causal_base + last_row + 1);
    const int t_first = sv.key_lo / kF32Keys;
    const int t_last = (key_end - 1) / kF32Keys;

    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    float m = -INFINITY, l = 0.f;

    for (int kt = t_first; kt <= t_last; ++kt) {
        __syncthreads();
        for (int i = t; i < kF32Keys * D / 4; i += 64) {
            const int kk = i / (D / 4), d4 = i % (D / 4);
            const int key = kt * kF32Keys + kk;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (key < sv.n_keys) {
                kv = *(const float4 *)(kc + (int64_t)key * D + 4 * d4);
                vv = *(const float4 *)(vc + (int64_t)key * D + 4 * d4);
            }
            *(float4 *)&Ks[kk][4 * d4] = kv;
            *(float4 *)&Vs[kk][4 * d4] = vv;
        }
        __syncthreads();
        float s[kF32Keys];
        float tmax = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < kF32Keys; ++kk) {
            const int key = kt * kF32Keys + kk;
            bool vis = key >= sv.key_lo && key < sv.n_keys && (maskp || key <= lim);
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(Qs[t][d], Ks[kk][d], dot);
            float sc = dot * a.scale;
            if (maskp && vis) sc += maskp[(int64_t)rr * a.mask_ld + key];
            s[kk] = vis ? sc : -INFINITY;
            tmax = fmaxf(tmax, s[kk]);
        }
        const float mn = fmaxf(m, tmax);
        if (mn != -INFINITY) {
            const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
            if (alpha != 1.f) {
                l *= alpha;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] *= alpha;
            }
            m = mn;
#pragma unroll
            for (int kk = 0; kk < kF32Keys; ++kk) {
                const float p = (s[kk] == -INFINITY) ? 0.f : expf(s[kk] - m);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vs[kk][d], acc[d]);
            }
        }
    }
    if (ok && row < sv.out_rows) {
        float *op = (float *)a.out + ((int64_t)(sv.out_row0 + row) * a.Hq + head) * D;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 4)
            *(float4 *)(op + d) =
                make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
    }
}

}  // namespace

int attn_rows_per_block(int dtype, int group, bool wide)
{
    (void)dtype;
    return (wide ? kWQC : kQC) / group;
}

// Launch one instance of a bf16/fp16 kernel template for the dtype, head
// dim and paging of the call.
#define CPK_LAUNCH_MFMA(KERNEL, THREADS)                                                      \
    do {                                                                                    \
        const bool pg = a.block_size != 0;                                                 \
        if (dtype == 1) {                                                                  \
            if (a.D == 64) {                                                               \
                if (pg) hipLaunchKernelGGL((KERNEL<F16, 64, true>), grid, dim3(THREADS), 0, st, a);   \
                else hipLaunchKernelGGL((KERNEL<F16, 64, false>), grid, dim3(THREADS), 0, st, a);   \
            } else {                                                                       \
                if (pg) hipLaunchKernelGGL((KERNEL<F16, 128, true>), grid, dim3(THREADS), 0, st, a);  \
                else hipLaunchKernelGGL((KERNEL<F16, 128, false>), grid, dim3(THREADS), 0, st, a);  \
            }                                                                              \
        } else {                                                                           \
            if (a.D == 64) {                                                               \
                if (pg) hipLaunchKernelGGL((KERNEL<Bf16, 64, true>), grid, dim3(THREADS), 0, st, a);  \
                else hipLaunchKernelGGL((KERNEL<Bf16, 64, false>), grid, dim3(THREADS), 0, st, a);  \
            } else {                                                                       \
                if (pg) hipLaunchKernelGGL((KERNEL<Bf16, 128, true>), grid, dim3(THREADS), 0, st, a); \
                else hipLaunchKernelGGL((KERNEL<Bf16, 128, false>), grid, dim3(THREADS), 0, st, a); \
            }                                                                              \
        }                                                                                  \
    } while (0)

hipError_t launch_attention(const AttnArgs &a, int dtype, int row_blocks, int n_seq_grid,
                            int kernel, hipStream_t st)
{
    const dim3 grid(row_blocks * a.Hkv, a.n_parts > 1 ? a.n_parts : 1, n_seq_grid);
    // the scheduled form covers every launch over a contiguous cache
    // (causal, computed or explicit-mask visibility, ring buffer, key split)
    const bool plain = a.block_size == 0;
    if (kernel == kAttnWide && dtype != 0) {
        CPK_LAUNCH_MFMA(attn_wide_kernel, kWThreads);
    } else if (dtype == 0) {
        if (a.D == 64)
            hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, st, a);
    } else if (kernel == kAttnNarrow && plain) {
        const dim3 blk(kThreads);
        if (dtype == 1) {
            if (a.D == 64) {
                if (a.mask) hipLaunchKernelGGL((attn_sched_kernel<F16, 64, true>), grid, blk, 0, st, a);
                else hipLaunchKernelGGL((attn_sched_kernel<F16, 64, false>), grid, blk, 0, st, a);
            } else {
                if (a.mask) hipLaunchKernelGGL((attn_sched_kernel<F16, 128, true>), grid, blk, 0, st, a);
                else hipLaunchKernelGGL((attn_sched_kernel<F16, 128, false>), grid, blk, 0, st, a);
            }
        } else {
            if (a.D == 64) {
                if (a.mask) hipLaunchKernelGGL((attn_sched_kernel<Bf16, 64, true>), grid, blk, 0, st, a);
                else hipLaunchKernelGGL((attn_sched_kernel<Bf16, 64, false>), grid, blk, 0, st, a);
            } else {
                if (a.mask) hipLaunchKernelGGL((attn_sched_kernel<Bf16, 128, true>), grid, blk, 0, st, a);
                else hipLaunchKernelGGL((attn_sched_kernel<Bf16, 128, false>), grid, blk, 0, st, a);
            }
        }
    } else {
        CPK_LAUNCH_MFMA(attn_mfma_kernel, kThreads);
    }
    return hipGetLastError();
}

hipError_t launch_attention_combine(const AttnArgs &a, int dtype, hipStream_t st)
{
    const int per_block = kCombineThreads / (a.D / 8);
    const int pairs = a.out_rows * a.Hq;
    const dim3 grid((pairs + per_block - 1) / per_block);
    const dim3 block(kCombineThreads);
    if (dtype == 1) {
        if (a.D == 64) hipLaunchKernelGGL((attn_combine_kernel<F16, 64>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_combine_kernel<F16, 128>), grid, block, 0, st, a);
    } else {
        if (a.D == 64) hipLaunchKernelGGL((attn_combine_kernel<Bf16, 64>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_combine_kernel<Bf16, 128>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace cpk
