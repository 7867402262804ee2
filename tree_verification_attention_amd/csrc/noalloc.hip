// Allocation-free variant of tree_attn_forward, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// tree_attn_forward keeps the split partials -- fp32 O and LSE of every prefix part and of the
// masked tree part, plus one part count per sequence -- in a workspace the caller allocates.
// Here that workspace is one file-scope device array, `scratch`, of TA_NOALLOC_SCRATCH_BYTES.
// Every GPU the library runs on holds its own copy of the array from the moment the library's
// code object is loaded on it until the process ends. Host code never passes the array's name
// to a kernel or a copy (on the host it only stands in for the symbol): the device address of
// each GPU's copy is looked up once per device, with that device current, and kept.
//
// Nothing in the array has to start at zero: every slot the combine reads is written by the
// same call's prefix launch first (the part counts included). All calls on one GPU share the
// array and it keeps the last call's contents, so calls that overlap on one GPU (other streams,
// other host threads) race; the caller serialises them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "treeattn.h"

namespace {

static __device__ __align__(256) char scratch[TA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of each GPU's copy, once looked up

// This GPU's copy of the scratch array: looked up on the first call on the device (with that
// device current), kept afterwards.
int scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TA_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TA_EHIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return TA_OK;
}

}  // namespace

extern "C" int tree_attn_forward_noalloc(const ta_problem *p, void *o, float *lse,
                                         int32_t *err_flag, hipStream_t stream) {
    size_t need = 0;
    int rc = tree_attn_workspace_size(p, &need);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if (need > (size_t)TA_NOALLOC_SCRATCH_BYTES) return TA_ESCRATCH;
    void *ws = nullptr;
    if ((rc = scratch_of_current_device(&ws))) return rc;
    return tree_attn_forward(p, o, lse, ws, (size_t)TA_NOALLOC_SCRATCH_BYTES, err_flag, stream);
}
