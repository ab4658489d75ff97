// Decode rows: one query row per sequence over that sequence's whole cache.
//
// Decode reads the entire cache for a handful of flops per byte, so it is
// bound by HBM bandwidth (Ultralytics glossary "Chunked Prefill", section
// on prefill, decode and generation stalls).  The kernel is built for
// streaming:
//
// * Split-KV: a work item is (sequence, KV head, 256-key segment), so a
//   batch of sequences with contexts from hundreds to tens of thousands of
//   keys turns into thousands of equal-sized items that fill all CUs.
// * GQA packing: the G query heads of one KV head are computed together,
//   so each K/V byte is read from HBM once per KV head, not once per query
//   head.
// * Each key row is read by 8 lanes; lane j reads bytes [16j, 16j+16) and
//   [128+16j, 128+16j+16) of the row, so every load instruction of a wave
//   covers whole 128-byte lines of 8 consecutive keys.  QK^T uses packed
//   2-element dot products (v_dot2_f32_{bf16,f16}) in fp32, reduced across
//   the 8 lanes with butterflies; PV accumulates in fp32.
// * Keys at or past the sequence's length are never loaded.
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
    static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
    static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
    static __device__ __forceinline__ uint32_t from_f32(float x)
    {
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    }
};

struct DF16 {
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), c, false);
    }
    static __device__ __forceinline__ float lo(uint32_t x)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t x)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
    }
    static __device__ __forceinline__ uint32_t from_f32(float x)
    {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
    }
};

constexpr int kThreadsDec = 256;
constexpr int kGroups = kThreadsDec / 8;            // 32 key lanes-groups per item
constexpr int kKeysPerGroup = kDecodeSeg / kGroups; // 8

__device__ __forceinline__ uint32_t dw(const uint4 &v, int j)
{
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

template <typename TR, int D, int G>
__global__ __launch_bounds__(kThreadsDec) void decode_kernel(DecodeArgs a)
{
    constexpr int NCH = D / 64;              // 16-byte chunks per lane per row
    constexpr int WS = D + 4;                // workspace record: m, l, pad, pad, acc[D]
    __shared__ float Mg[kGroups][G];
    __shared__ float Lg[kGroups][G];
    __shared__ __attribute__((aligned(16))) float Ag[kGroups][G][D];

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
    const int gi = tid >> 3;
    const int j = tid & 7;

    const uint16_t *kc = (const uint16_t *)a.k + ((int64_t)slot * a.Hkv + g) * a.cap * D;
    const uint16_t *vc = (const uint16_t *)a.v + ((int64_t)slot * a.Hkv + g) * a.cap * D;

    // query slices of the G heads of this KV head
    uint4 qv[G][NCH];
    const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)row0 * a.Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
            qv[h][ch] = *(const uint4 *)(qp + (int64_t)h * D + ch * 64 + 8 * j);

    uint4 kr[kKeysPerGroup][NCH], vr[kKeysPerGroup][NCH];
#pragma unroll
    for (int it = 0; it < kKeysPerGroup; ++it) {
        const int key = sb + gi + kGroups * it;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            if (key < n_keys) {
                kr[it][ch] = *(const uint4 *)(kc + (int64_t)key * D + ch * 64 + 8 * j);
                vr[it][ch] = *(const uint4 *)(vc + (int64_t)key * D + ch * 64 + 8 * j);
            } else {
                kr[it][ch] = make_uint4(0, 0, 0, 0);
                vr[it][ch] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    // scores in the exp2 domain
    float s[kKeysPerGroup][G];
#pragma unroll
    for (int it = 0; it < kKeysPerGroup; ++it) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float acc = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int w = 0; w < 4; ++w) acc = TR::dot2(dw(qv[h][ch], w), dw(kr[it][ch], w), acc);
            acc += __shfl_xor(acc, 1, 8);
            acc += __shfl_xor(acc, 2, 8);
            acc += __shfl_xor(acc, 4, 8);
            const int key = sb + gi + kGroups * it;
            s[it][h] = key < n_keys ? acc * a.scale_log2 : -INFINITY;
        }
    }

    // per-group softmax over its keys, then P V
    float m[G], l[G], o[G][NCH * 8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = s[0][h];
#pragma unroll
        for (int it = 1; it < kKeysPerGroup; ++it) m[h] = fmaxf(m[h], s[it][h]);
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < NCH * 8; ++e) o[h][e] = 0.f;
    }
#pragma unroll
    for (int it = 0; it < kKeysPerGroup; ++it) {
        float p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            p[h] = (m[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[it][h] - m[h]);
            l[h] += p[h];
        }
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x = dw(vr[it][ch], w);
                const float v0 = TR::lo(x), v1 = TR::hi(x);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h][ch * 8 + 2 * w] = __builtin_fmaf(p[h], v0, o[h][ch * 8 + 2 * w]);
                    o[h][ch * 8 + 2 * w + 1] = __builtin_fmaf(p[h], v1, o[h][ch * 8 + 2 * w + 1]);
                }
            }
    }

    // merge the 32 groups of this item
    if (j == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            Mg[gi][h] = m[h];
            Lg[gi][h] = l[h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            float *dst = &Ag[gi][h][ch * 64 + 8 * j];
            *(float4 *)dst = make_float4(o[h][ch * 8], o[h][ch * 8 + 1], o[h][ch * 8 + 2],
                                         o[h][ch * 8 + 3]);
            *(float4 *)(dst + 4) = make_float4(o[h][ch * 8 + 4], o[h][ch * 8 + 5],
                                               o[h][ch * 8 + 6], o[h][ch * 8 + 7]);
        }
    __syncthreads();

    for (int idx = tid; idx < G * D; idx += kThreadsDec) {
        const int h = idx / D;
        const int d = idx % D;
        float M = -INFINITY;
        for (int q = 0; q < kGroups; ++q) M = fmaxf(M, Mg[q][h]);
        float acc = 0.f, lsum = 0.f;
        for (int q = 0; q < kGroups; ++q) {
            const float mq = Mg[q][h];
            const float e = (mq == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq - M);
            acc = __builtin_fmaf(e, Ag[q][h][d], acc);
            lsum = __builtin_fmaf(e, Lg[q][h], lsum);
        }
        float *rec = a.ws + (((int64_t)z * a.Hq + g * G + h) * a.max_segs + seg) * WS;
        rec[4 + d] = acc;
        if (d == 0) {
            rec[0] = M;
            rec[1] = lsum;
        }
    }
}

template <typename TR, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a)
{
    constexpr int WS = D + 4;
    const int z = blockIdx.y;
    const int row0 = a.cu_rows[z];
    if (a.cu_rows[z + 1] - row0 != 1) return;
    const int n_keys = a.past_lens[z] + 1;
    const int n_segs = (n_keys + kDecodeSeg - 1) / kDecodeSeg;
    const int head = blockIdx.x;
    const int d = threadIdx.x;
    const float *rec = a.ws + ((int64_t)z * a.Hq + head) * a.max_segs * WS;
    float M = -INFINITY;
    for (int s = 0; s < n_segs; ++s) M = fmaxf(M, rec[s * WS]);
    float acc = 0.f, lsum = 0.f;
    for (int s = 0; s < n_segs; ++s) {
        const float ms = rec[s * WS];
        const float e = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
        acc = __builtin_fmaf(e, rec[s * WS + 4 + d], acc);
        lsum = __builtin_fmaf(e, rec[s * WS + 1], lsum);
    }
    const float r = lsum > 0.f ? acc / lsum : 0.f;
    uint16_t *op = (uint16_t *)a.out + ((int64_t)row0 * a.Hq + head) * D;
    op[d] = (uint16_t)TR::from_f32(r);
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
    hipLaunchKernelGGL((decode_combine_kernel<TR, D>), dim3(a.Hq, a.n_seqs), dim3(D), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int dtype, int D, int group)
{
    return (dtype == 1 || dtype == 2) && (D == 64 || D == 128) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
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
