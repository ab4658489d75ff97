// The packed mixed step for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the split-KV decode partials live in a static device array
// instead of a caller workspace.
//
// The array's name is only a host-side stand-in for its device address, so
// host code never passes it to a kernel: the address is taken once per
// device with hipGetSymbolAddress, with that device current, and kept.
// Every call on a GPU shares that GPU's array; calls that overlap on one GPU
// (two streams, or two host threads) race on it.  Nothing in it needs to
// start at zero: the decode kernel writes every partial record its combine
// reads.
#include "cpk_internal.h"
#include "cpk.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = (size_t)CPK_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];

// the current device's address of the scratch array (nullptr and a nonzero
// status on failure)
int scratch_ptr(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CPK_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CPK_EHIP;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return CPK_OK;
}

}  // namespace

extern "C" int cpk_varlen_step_noalloc(const void *q, const void *k_new, const void *v_new,
                                       const cpk_kv_cache *cache, const int32_t *slots,
                                       const int32_t *cu_rows, const int32_t *past_lens,
                                       const int32_t *h_slots, const int32_t *h_cu_rows,
                                       const int32_t *h_past_lens, int n_seqs, int total_rows,
                                       int q_heads, float scale, void *out, void *stream)
{
    void *ws = nullptr;
    const int r = scratch_ptr(&ws);
    if (r != CPK_OK) return cpk::fail_status(r, "varlen_noalloc: no scratch address on this device");
    // the workspace check inside reports a step whose decode partials exceed
    // the scratch size (CPK_EWORKSPACE)
    return cpk_varlen_step(q, k_new, v_new, cache, slots, cu_rows, past_lens, h_slots,
                           h_cu_rows, h_past_lens, n_seqs, total_rows, q_heads, scale, out, ws,
                           kScratchBytes, stream);
}
