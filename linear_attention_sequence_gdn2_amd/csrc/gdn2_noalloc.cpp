// gdn2_noalloc.cpp -- gdn2_chunk_fwd_noalloc: the forward of gdn2_chunk_fwd for callers that
// cannot allocate (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The chunk records that gdn2_chunk_fwd keeps in its caller-given workspace live
// here in a file-scope device array instead, one copy per GPU, held until the process ends.
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "gdn2.h"

namespace {

constexpr size_t kScratchBytes = (size_t)256 << 20;
constexpr int kMaxDevices = 64;

// The records of one call (see gdn2_chunk_fwd_workspace_size).  In host code this name is only
// a stand-in for the symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// This device's copy of the scratch array (nullptr if the runtime cannot give its address).
void *scratch_ptr(int dev) {
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    return g_ptr[dev];
}

size_t elem(int dtype) { return dtype == GDN2_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

size_t gdn2_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int gdn2_chunk_fwd_noalloc(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *b, const void *w, const float *S0, float *o,
                           float *S_final, void *stream) {
    // the shape checks of gdn2_chunk_fwd, and the records of one batch element must fit
    if (gdn2_chunk_fwd_workspace_size(shape) == (size_t)-1) return GDN2_ERR_UNSUPPORTED;
    gdn2_shape one = *shape;
    one.B = 1;
    if (gdn2_chunk_fwd_workspace_size(&one) > kScratchBytes) return GDN2_ERR_SCRATCH;
    if (!q || !k || !v || !log_alpha || !b || !w || !o) return GDN2_ERR_INVALID_ARG;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN2_ERR_HIP;
    void *ws = scratch_ptr(dev);
    if (!ws) return GDN2_ERR_HIP;
    // batch elements are independent: run them in the largest groups whose records fit
    gdn2_shape grp = *shape;
    int bg = shape->B;
    for (;;) {
        grp.B = bg;
        if (gdn2_chunk_fwd_workspace_size(&grp) <= kScratchBytes) break;
        bg = (bg + 1) / 2;
    }
    const size_t tok = (size_t)shape->T * shape->H;   // (token, head) rows per batch element
    const size_t qk = tok * shape->dk * elem(shape->qkv_dtype), vv = tok * shape->dv * elem(shape->qkv_dtype);
    const size_t ge = shape->gate_dtype == GDN2_GATES_BF16_LOGITS ? 2 : 4;
    const size_t la_b = tok * ((shape->gate_scalar & GDN2_SCALAR_DECAY) ? 1 : shape->dk) * ge;
    const size_t b_b = tok * ((shape->gate_scalar & GDN2_SCALAR_ERASE) ? 1 : shape->dk) * ge;
    const size_t w_b = tok * ((shape->gate_scalar & GDN2_SCALAR_WRITE) ? 1 : shape->dv) * ge;
    const size_t st = (size_t)shape->H * shape->dk * shape->dv;   // floats of one batch element's state
    auto at = [](const void *p, size_t bytes) {
        return p ? static_cast<const void *>(static_cast<const char *>(p) + bytes) : nullptr;
    };
    for (int b0 = 0; b0 < shape->B; b0 += bg) {
        grp.B = shape->B - b0 < bg ? shape->B - b0 : bg;
        const size_t n = (size_t)b0;
        const int rc = gdn2_chunk_fwd(&grp, at(q, n * qk), at(k, n * qk), at(v, n * vv), at(log_alpha, n * la_b),
                                      at(b, n * b_b), at(w, n * w_b), S0 ? S0 + n * st : nullptr,
                                      o + n * tok * shape->dv, S_final ? S_final + n * st : nullptr, ws,
                                      kScratchBytes, stream);
        if (rc != GDN2_OK) return rc;
    }
    return GDN2_OK;
}

}  // extern "C"
