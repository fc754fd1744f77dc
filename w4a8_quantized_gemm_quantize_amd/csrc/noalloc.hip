// noalloc.hip -- the fused W4A8 entry point for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the workspace of w4a8_gemm_bf16act (activation codes and
// scales, split-K partials) lives in a static device array instead of caller
// memory.
//
// The array is file-scope device memory that the runtime places once per
// device when it loads the library's code there, and keeps until the process
// ends.  In host code its name is only a stand-in, not a device address: its
// address on the current device comes from hipGetSymbolAddress, taken once
// per device on the first call made with that device current and cached.
// Every call on a GPU shares that GPU's array and leaves its contents behind,
// so calls that overlap on one GPU (two streams, two host threads) race.  No
// kernel here needs the array cleared: each call writes every byte it later
// reads (the codes and scales of its rows, every partial-sum slot of its
// slices).
#include <atomic>

#include "w4a8.h"
#include "launch.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[W4A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The array's device address on the current device (null on failure).
void *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

w4a8_status w4a8_gemm_bf16act_noalloc(const uint16_t *a, const uint8_t *w_packed,
                                      const uint8_t *grp_scale, const float *ch_scale,
                                      int64_t m, int64_t n, int64_t k, int32_t group, void *out,
                                      w4a8_dtype out_dtype, hipStream_t stream) {
    // Shape, pointer and alignment rules of w4a8_gemm_bf16act: the checks run
    // through its validation with the scratch as the workspace of exactly the
    // size the call needs, so this entry point cannot accept anything that one
    // rejects.  First the size limit, before the device is touched.
    if (k <= 0 || m < 0 || n < 0) return W4A8_ERR_SHAPE;
    if (m == 0 || n == 0) return W4A8_OK;
    const size_t base = w4a8_gemm_bf16act_workspace_bytes(m, k);
    if (base == 0 || base > (size_t)W4A8_NOALLOC_SCRATCH_BYTES) return W4A8_ERR_UNSUPPORTED;
    // the split-K partials only when they fit beside the codes; otherwise the
    // one-pass kernels, whose result is the same bit for bit
    size_t need = base + w4a8_gemm_workspace_bytes(m, n, k);
    if (need > (size_t)W4A8_NOALLOC_SCRATCH_BYTES) need = base;
    if (!a || !w_packed || !grp_scale || !ch_scale || !out) return W4A8_ERR_NULL;
    if (!aligned16(a) || !aligned16(w_packed) || !aligned16(grp_scale) || !aligned16(ch_scale) ||
        !aligned16(out))
        return W4A8_ERR_MISALIGNED;
    void *ws = scratch_on_current_device();
    if (!ws) return W4A8_ERR_HIP;
    return w4a8_gemm_bf16act(a, w_packed, grp_scale, ch_scale, m, n, k, group, out, out_dtype,
                             ws, need, stream);
}

}  // extern "C"
