// Decode rows: one query row per sequence over that sequence's whole cache.
//
// Decode reads the entire cache for a handful of flops per byte, so it is
// bound by HBM bandwidth (Ultralytics glossary "Chunked Prefill", section
// on prefill, decode and generation stalls).  The kernel is built for
// streaming:
//
// * Split-KV: a work item is (sequence, KV head, 256-key segment), so a
//   batch of sequences with contexts from hundreds to tens of thousands of
//   keys turns into thousands of short, equal-sized items; the dispatcher's
//   tail at the end of the grid is then a small part of the step.
// * GQA packing: the G query heads of one KV head are computed together,
//   so each K/V byte is read from HBM once per KV head, not once per query
//   head.
// * A key row is spread over D/8 lanes, 16 bytes (8 elements) per lane, and
//   the lane groups of a wave take consecutive keys, so each load
//   instruction reads one contiguous 1 KB span of rows (measured 0.7%
//   faster than lane groups each taking 4 consecutive keys).  Each of the 4
//   waves streams 64 keys in steps of 4 keys per lane group, with the next
//   step's K/V loads in flight while the current step computes (double
//   buffering in registers, non-temporal loads).
// * QK^T: packed 2-element dot products (v_dot2_f32_{bf16,f16}) in fp32,
//   summed over the lane group with DPP butterflies that leave identical
//   bits in every lane.  Softmax is online per query head with a lazy
//   running maximum.  P is rounded to the storage type in pairs of keys, so
//   PV is again packed dot products, over two keys at a time, accumulated
//   in fp32; the running sum adds the same rounded P.
// * Keys at or past the sequence's length are never loaded.
//
// * Fused append: in a step that also appends, the workgroup whose segment
//   holds a sequence's new key writes that K/V row into the cache itself.
// * Epilogue: the 16 lane groups' (m, l, acc) meet in LDS; one thread per
//   head forms the weights exp2(m - M) and the merged l, then every thread
//   folds two adjacent columns over the lane groups in lane-group order.
//   The segment record goes out with non-temporal stores: measured on a
//   2.33 GB step of 64 sequences, the kernel gains 10 us and the combine,
//   whose reads of the records then come from memory rather than L2,
//   loses 2 us.
//
// decode_combine merges the per-segment (max, sum, acc) partials of every
// (sequence, query head) in a fixed order (deterministic, no atomics).
#include "cpk_internal.h"

#include <math.h>

namespace cpk {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;

struct DBf16 {
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
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
    static constexpr uint32_t kOnes = 0x3F803F80u;   // (1.0, 1.0)
};

struct DF16 {
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
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
    static constexpr uint32_t kOnes = 0x3C003C00u;   // (1.0, 1.0)
};

constexpr int kThreadsDec = 256;                               // 4 waves
constexpr int kKeysPerWave = kDecodeSeg / (kThreadsDec / 64);   // 64
constexpr int kKK = 4;              // keys per lane group per streaming step
constexpr float kLazyLog2Dec = 8.0f;

__device__ __forceinline__ uint32_t dw(const uint4 &v, int j)
{
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Sum over the LPK lanes (8 or 16) of an aligned lane group, returned in all
// of them with identical bits: xor-1 and xor-2 exchanges (quad permutes), a
// half-row mirror (lane i <-> 7 - i) and, for 16 lanes, a row mirror
// (lane i <-> 15 - i).  Each step adds two operands in both orders, so all
// lanes of the group end with the same value.  All are DPP register moves.
template <int LPK>
__device__ __forceinline__ float group_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x141, 0xF, 0xF, false));
    if constexpr (LPK == 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   0x140, 0xF, 0xF, false));
    return x;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache rows are read once per decode step: non-temporal loads keep them from
// displacing reusable lines in the caches.
__device__ __forceinline__ uint4 load_stream(const char *base, uint32_t off)
{
    const u32x4 t = __builtin_nontemporal_load((const u32x4 *)(base + off));
    return make_uint4(t.x, t.y, t.z, t.w);
}

struct KVStep {
    uint4 k[kKK];
    uint4 v[kKK];
};

// waves per SIMD the register budget is held to (G = 8 keeps 2: its
// accumulators alone need 64 VGPRs)
template <int G>
constexpr int decode_waves() { return G <= 4 ? 3 : 2; }

template <typename TR, int D, int G>
__global__ __launch_bounds__(kThreadsDec)
__attribute__((amdgpu_waves_per_eu(decode_waves<G>())))
void decode_kernel(DecodeArgs a)
{
    constexpr int LPK = D / 8;                 // lanes per key row, 16 bytes each
    constexpr int GPW = 64 / LPK;              // lane groups per wave
    constexpr int NG = GPW * (kThreadsDec / 64);   // lane groups per workgroup
    constexpr int STEP = GPW * kKK;            // keys per wave per step
    constexpr int WS = D + 4;                  // workspace record: m, l, pad, pad, acc[D]
    __shared__ float Mg[NG][G];
    __shared__ float Lg[NG][G];
    __shared__ float Eg[NG][G];   // per (lane group, head) merge weights
    __shared__ float Mh[G];       // per head maximum over the lane groups
    __shared__ float Lh[G];       // per head weighted sum of l
    __shared__ __attribute__((aligned(16))) float Ag[NG][G][D];

    const int z = blockIdx.z;
    const int row0 = a.cu_rows[z];
    if (a.cu_rows[z + 1] - row0 != 1) return;
    const int n_keys = a.past_lens[z] + 1;
    const int seg = blockIdx.x;
    const int sb = seg * kDecodeSeg;
    if (sb >= n_keys) return;
    const int g = blockIdx.y;
    const int slot = a.slots[z];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int gq = lane / LPK;                 // lane group inside the wave
    const int gi = wave * GPW + gq;            // lane group inside the workgroup
    const int j = lane % LPK;                  // this lane's 8 elements: [8j, 8j + 8)

    // uniform bases (of this slot and KV head, or of the block holding this
    // 256-key segment in a paged pool; key_org is the key at the base);
    // per-lane 32-bit byte offsets
    const int key_org = a.block_size ? sb : 0;
    const int64_t head_off =
        (a.block_size ? paged_row(a.block_table, a.max_blocks, a.block_size, a.n_blocks, a.Hkv,
                                  slot, g, sb)
                      : ((int64_t)slot * a.Hkv + g) * a.cap) * D * 2;
    const char *kbase = (const char *)a.k + head_off;
    const char *vbase = (const char *)a.v + head_off;

    // fused append: the segment holding the new key (position n_keys - 1)
    // writes this KV head's new K/V row into the cache first; the stores
    // complete before the barrier, so the workgroup then reads the row back
    // with the rest of its keys
    if (a.k_new && sb + kDecodeSeg >= n_keys) {
        constexpr int V16 = D * 2 / 16;   // 16-byte pieces per row
        if (tid < 2 * V16) {
            const int part = tid / V16, c = tid % V16;
            const uint4 *src = (const uint4 *)(part ? a.v_new : a.k_new) +
                               ((int64_t)row0 * a.Hkv + g) * V16 + c;
            char *dst = (char *)(part ? a.v : a.k) + head_off +
                        (uint32_t)(n_keys - 1 - key_org) * (D * 2) + 16u * c;
            *(uint4 *)dst = *src;
        }
        if (g == 0 && tid == 0) a.seqlens_k[slot] = n_keys;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    uint4 qv[G];
    const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)row0 * a.Hq + g * G) * D + 8 * j;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *(const uint4 *)(qp + (int64_t)h * D);

    // the wave streams keys [wbase, wlast]; in step st, lane group gq takes
    // keys wbase + st*STEP + kk*GPW + gq (kk = 0 .. kKK-1), so each load
    // instruction (one kk) reads GPW consecutive keys: one contiguous
    // 64 x 16-byte span per wave.  Keys are clamped to
    // wlast, so a step past the end re-reads only that row.
    const int wbase = sb + wave * kKeysPerWave;
    const int wlast = min(n_keys, wbase + kKeysPerWave) - 1;
    auto load_step = [&](int st, KVStep &b) __attribute__((always_inline)) {
        const int key0 = wbase + st * STEP + gq;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
            const uint32_t off =
                (uint32_t)(min(key0 + kk * GPW, wlast) - key_org) * (D * 2) + 16u * j;
            b.k[kk] = load_stream(kbase, off);
            b.v[kk] = load_stream(vbase, off);
        }
    };

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    const float c = a.scale_log2;   // > 0: the maximum of raw scores is the maximum of scaled ones
    auto compute_step = [&](int st, const KVStep &b) __attribute__((always_inline)) {
        const int key0 = wbase + st * STEP + gq;
        float s[kKK][G];
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) acc = TR::dot2(dw(qv[h], w), dw(b.k[kk], w), acc);
                s[kk][h] = group_sum<LPK>(acc);
            }
        if (wbase + (st + 1) * STEP - 1 > wlast) {   // wave-uniform: the step has keys past wlast
#pragma unroll
            for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (key0 + kk * GPW > wlast) s[kk][h] = -INFINITY;
        }
        // online softmax per head with a lazy maximum: the reference m (log2
        // domain) is raised only when a step's maximum exceeds it by more
        // than 2^8.  p is rounded to the storage type in pairs of keys, and l
        // sums the rounded values, so the normalisation matches what PV uses.
        uint32_t pp[kKK / 2][G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int kk = 1; kk < kKK; ++kk) mx = fmaxf(mx, s[kk][h]);
            mx *= c;
            if (mx > m[h] + kLazyLog2Dec) {
                const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
                m[h] = mx;
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
            }
            const float mu = m[h] == -INFINITY ? 0.f : m[h];
#pragma unroll
            for (int t = 0; t < kKK / 2; ++t) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * t][h], c, -mu));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * t + 1][h], c, -mu));
                pp[t][h] = TR::pack(p0, p1);
                l[h] = TR::dot2(pp[t][h], TR::kOnes, l[h]);
            }
        }
        // PV over key pairs: (v_k0[d], v_k1[d]) . (p_k0, p_k1) with packed dots
#pragma unroll
        for (int t = 0; t < kKK / 2; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x0 = dw(b.v[2 * t], w), x1 = dw(b.v[2 * t + 1], w);
                const uint32_t ev = __builtin_amdgcn_perm(x1, x0, 0x05040100u);   // element 2w
                const uint32_t od = __builtin_amdgcn_perm(x1, x0, 0x07060302u);   // element 2w+1
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h][2 * w] = TR::dot2(pp[t][h], ev, o[h][2 * w]);
                    o[h][2 * w + 1] = TR::dot2(pp[t][h], od, o[h][2 * w + 1]);
                }
            }
    };

    // stream the wave's keys: step st + 1 is in flight while step st
    // computes.  The step loop is unrolled in full (its length is fixed) so
    // that no buffer is carried around a loop back edge: the compiler then
    // keeps each prefetch in place and its wait counts exact.  The step count
    // is rounded up to even: a step past wlast scores all its keys -inf
    // (weight 0), and the prefetch after the last pair is a clamped re-read.
    constexpr int kSteps = kKeysPerWave / STEP;
    const int steps = wlast >= wbase ? (wlast - wbase + STEP) / STEP : 0;
    if (steps > 0) {
        KVStep b0, b1;
        load_step(0, b0);
#pragma unroll
        for (int st = 0; st < kSteps; st += 2) {
            if (st >= steps) break;   // wave-uniform
            load_step(st + 1, b1);
            __builtin_amdgcn_sched_barrier(0);   // issue the prefetch before any wait
            compute_step(st, b0);
            if (st + 2 < kSteps) load_step(st + 2, b0);
            __builtin_amdgcn_sched_barrier(0);
            compute_step(st + 1, b1);
        }
    }

    // merge the lane groups of this work item
    if (j == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            Mg[gi][h] = m[h];
            Lg[gi][h] = l[h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float *dst = &Ag[gi][h][8 * j];
        *(float4 *)dst = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
        *(float4 *)(dst + 4) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
    }
    __syncthreads();

    // each head's maximum over the lane groups, the lane groups' weights
    // exp2(m - M) and the weighted sum of l, once per head
    if (tid < G) {
        const int h = tid;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < NG; ++q) M = fmaxf(M, Mg[q][h]);
        float lsum = 0.f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const float mq = Mg[q][h];
            const float e = (mq == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq - M);
            Eg[q][h] = e;
            lsum = __builtin_fmaf(e, Lg[q][h], lsum);
        }
        Mh[h] = M;
        Lh[h] = lsum;
    }
    __syncthreads();

    // two adjacent columns per thread
    static_assert((G * D / 2) % kThreadsDec == 0 || G * D / 2 < kThreadsDec, "column pairs");
    for (int idx = tid; idx < G * D / 2; idx += kThreadsDec) {
        const int h = (2 * idx) / D;
        const int d = (2 * idx) % D;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const float e = Eg[q][h];
            const float2 x = *(const float2 *)&Ag[q][h][d];
            acc0 = __builtin_fmaf(e, x.x, acc0);
            acc1 = __builtin_fmaf(e, x.y, acc1);
        }
        float *rec = a.ws + (((int64_t)z * a.Hq + g * G + h) * a.max_segs + seg) * WS;
        typedef float f2v __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(f2v{acc0, acc1}, (f2v *)(rec + 4 + d));
        if (d == 0) {
            __builtin_nontemporal_store(Mh[h], rec);
            __builtin_nontemporal_store(Lh[h], rec + 1);
        }
    }
}

// Merge the segment partials of one (sequence, query head).  Four waves:
// wave w takes segments w, w + 4, w + 8, ... and each lane D/64 columns.  A
// wave loads kCombBatch of its segments' records at once (all loads in
// flight, so the merge costs about one memory round trip, not one per
// segment), folds them in increasing segment order into its running (max,
// sum, acc), and the four waves' results are then merged in wave order
// through LDS.  Fixed order throughout: deterministic, no atomics.
constexpr int kCombThreads = 256;
constexpr int kCombBatch = 16;

template <typename TR, int D>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(DecodeArgs a)
{
    constexpr int WS = D + 4;
    constexpr int CPL = D / 64;   // columns per lane
    constexpr int NWV = kCombThreads / 64;
    __shared__ float wm[NWV], wl[NWV];
    __shared__ __attribute__((aligned(16))) float wacc[NWV][D];
    const int z = blockIdx.y;
    const int row0 = a.cu_rows[z];
    if (a.cu_rows[z + 1] - row0 != 1) return;
    const int n_keys = a.past_lens[z] + 1;
    const int n_segs = (n_keys + kDecodeSeg - 1) / kDecodeSeg;
    const int head = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const float *rec = a.ws + ((int64_t)z * a.Hq + head) * a.max_segs * WS;

    float M = -INFINITY, L = 0.f, acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s0 = wave; s0 < n_segs; s0 += NWV * kCombBatch) {
        float ms[kCombBatch], ls[kCombBatch], xs[kCombBatch][CPL];
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            // past the last segment: re-read a valid record, weighted 0 below
            const float *r = rec + (int64_t)min(s0 + NWV * i, n_segs - 1) * WS;
            ms[i] = r[0];
            ls[i] = r[1];
#pragma unroll
            for (int c = 0; c < CPL; ++c) xs[i][c] = r[4 + CPL * lane + c];
        }
        float bm = M;
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i)
            if (s0 + NWV * i < n_segs) bm = fmaxf(bm, ms[i]);
        if (bm != M) {   // M == -inf: nothing merged yet, L and acc are 0
            const float alpha = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - bm);
            L *= alpha;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] *= alpha;
            M = bm;
        }
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            const float e = (s0 + NWV * i < n_segs && ms[i] != -INFINITY)
                                ? __builtin_amdgcn_exp2f(ms[i] - M) : 0.f;
            L = __builtin_fmaf(e, ls[i], L);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(e, xs[i][c], acc[c]);
        }
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = L;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) wacc[wave][CPL * lane + c] = acc[c];
    __syncthreads();
    if (wave != 0) return;
    float Mt = wm[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) Mt = fmaxf(Mt, wm[w]);
    float Lt = 0.f, at[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) at[c] = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const float e = wm[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[w] - Mt);
        Lt = __builtin_fmaf(e, wl[w], Lt);
#pragma unroll
        for (int c = 0; c < CPL; ++c) at[c] = __builtin_fmaf(e, wacc[w][CPL * lane + c], at[c]);
    }
    uint16_t *op = (uint16_t *)a.out + ((int64_t)row0 * a.Hq + head) * D + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) op[c] = (uint16_t)TR::from_f32(Lt > 0.f ? at[c] / Lt : 0.f);
}

template <typename TR, int D>
hipError_t launch_decode_t(const DecodeArgs &a, int G, int max_segs, hipStream_t st)
{
    const dim3 grid(max_segs, a.Hkv, a.n_seqs);
    switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<TR, D, 1>), grid, dim3(kThreadsDec), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<TR, D, 2>), grid, dim3(kThreadsDec), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<TR, D, 4>), grid, dim3(kThreadsDec), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_kernel<TR, D, 8>), grid, dim3(kThreadsDec), 0, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<TR, D>), dim3(a.Hq, a.n_seqs), dim3(kCombThreads), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int dtype, int D, int group, int capacity)
{
    // key rows are addressed with 32-bit byte offsets inside one (slot, head)
    return (dtype == 1 || dtype == 2) && (D == 64 || D == 128) &&
           (group == 1 || group == 2 || group == 4 || group == 8) &&
           (int64_t)capacity * D * 2 <= (int64_t)UINT32_MAX;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int max_segs, hipStream_t st)
{
    const int G = a.Hq / a.Hkv;
    if (dtype == 2)
        return a.D == 64 ? launch_decode_t<DBf16, 64>(a, G, max_segs, st)
                         : launch_decode_t<DBf16, 128>(a, G, max_segs, st);
    return a.D == 64 ? launch_decode_t<DF16, 64>(a, G, max_segs, st)
                     : launch_decode_t<DF16, 128>(a, G, max_segs, st);
}

}  // namespace cpk
