// nsa_decode_step_noalloc: the decode step with its workspace in a static
// device array, for callers that cannot allocate (code under graph capture,
// serving loops that forbid allocation).
//
// `scratch` below is a file-scope device array.  In host code its name is a
// host-side stand-in, not a device address, so the address each device holds
// it at is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed on.  Every call on a device shares
// the device's array and leaves its last contents there; the decode step
// needs nothing in it to start at zero (it writes every workspace byte it
// reads).  Calls that overlap on one device -- on two streams, or from two
// host threads -- race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nsa.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices];   // the array's device address, per device (null until looked up)

nsa_status scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NSA_ERR_HIP;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NSA_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return NSA_OK;
}

}  // namespace

extern "C" {

nsa_status nsa_decode_step_noalloc(const nsa_config *cfg, const int32_t *seq_lens, const void *q,
                                   const void *k_cache, const void *v_cache, const void *cmp_k, const void *cmp_v,
                                   const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                                   int32_t *idx_out, void *stream)
{
    const size_t need = nsa_workspace_bytes(cfg, NSA_OP_DECODE);
    if (need == 0)   // an invalid configuration: the decode step's own checks report which
        return nsa_decode_step(cfg, seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out,
                               nullptr, 0, stream);
    // the decode step's pointer checks, before any HIP call
    if (!seq_lens || !q || !k_cache || !v_cache || !cmp_k || !cmp_v || !w_g || !b_g || !o) return NSA_ERR_NULL;
    const void *ptrs[] = {seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out};
    for (const void *p : ptrs)
        if ((uintptr_t)p & 15u) return NSA_ERR_ALIGN;
    if (need > kScratchBytes) return NSA_ERR_WORKSPACE;
    void *ws = nullptr;
    const nsa_status st = scratch_ptr(&ws);
    if (st != NSA_OK) return st;
    return nsa_decode_step(cfg, seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out, ws,
                           kScratchBytes, stream);
}

}  // extern "C"
