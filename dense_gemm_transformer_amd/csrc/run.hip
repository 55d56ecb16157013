// gemm_run: argument checks, then one launch (two for split-K TILED plans)
// on the caller's stream.  No allocation, no synchronisation.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels/common.h"
#include "tlgemm_internal.h"

namespace tlg {

int launch_generic(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                   hipStream_t stream);
template <int I>
int launch_stream_in(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                     hipStream_t stream);
template <int I>
int launch_tiled_in(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                    hipStream_t stream);

static int launch_stream(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                         hipStream_t s) {
    if (p.in_dt == TLG_F32) return launch_stream_in<TLG_F32>(p, X, W, bias, Y, ws, s);
    if (p.in_dt == TLG_F16) return launch_stream_in<TLG_F16>(p, X, W, bias, Y, ws, s);
    return launch_stream_in<TLG_BF16>(p, X, W, bias, Y, ws, s);
}

static int launch_tiled(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                        hipStream_t s) {
    if (p.in_dt == TLG_F32) return launch_tiled_in<TLG_F32>(p, X, W, bias, Y, ws, s);
    if (p.in_dt == TLG_F16) return launch_tiled_in<TLG_F16>(p, X, W, bias, Y, ws, s);
    return launch_tiled_in<TLG_BF16>(p, X, W, bias, Y, ws, s);
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s launch failed: %s", what, hipGetErrorString(e));
        return TLG_ERR_LAUNCH;
    }
    return TLG_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace tlg

using namespace tlg;

// ---- the library's own scratch, for callers that cannot allocate ----------------------
// One array per device the library runs on, held until the process ends.  Host
// code never uses its name as an address: the name is a host-side stand-in; the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The counter block must start at zero; completed runs leave it zero.  A
// kernel, not a memset, so the first call may sit inside a captured graph.
__global__ __launch_bounds__(256) void zero_counters_kernel(u32x4* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = u32x4{0u, 0u, 0u, 0u};
}
}  // namespace

// Device address of this device's scratch; its counter block is cleared
// (on `stream`) the first time a device is seen.
static int scratch_for_device(void** out, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("gemm_run_no_alloc: no current device below %d", kMaxDevices);
        return TLG_ERR_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error("gemm_run_no_alloc: hipGetSymbolAddress failed on device %d: %s", dev, hipGetErrorString(e));
            return TLG_ERR_LAUNCH;
        }
        constexpr int n = (int)(kWsCounterBytes / 16);
        hipLaunchKernelGGL(zero_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<u32x4*>(ptr),
                           n);
        const int rc = check_launch("zero_counters_kernel");
        if (rc != TLG_OK) return rc;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TLG_OK;
}

extern "C" int gemm_run_no_alloc(tlg_plan_t p, const void* X, const void* W, const void* bias, void* Y, void* stream) {
    if (!p) {
        set_error("gemm_run_no_alloc: NULL plan");
        return TLG_ERR_INVALID_ARG;
    }
    if (p->ws_bytes > kScratchBytes) {
        set_error("gemm_run_no_alloc: the plan needs %zu bytes of scratch, the library holds %zu per device",
                  p->ws_bytes, (size_t)kScratchBytes);
        return TLG_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    if (p->ws_bytes) {
        const int rc = scratch_for_device(&ws, static_cast<hipStream_t>(stream));
        if (rc != TLG_OK) return rc;
    }
    return gemm_run(p, X, W, bias, Y, ws, p->ws_bytes, stream);
}

extern "C" int gemm_run(tlg_plan_t p, const void* X, const void* W, const void* bias, void* Y,
                        void* workspace, size_t ws_bytes, void* stream) {
    if (!p) {
        set_error("gemm_run: NULL plan");
        return TLG_ERR_INVALID_ARG;
    }
    if (!X || !W || !Y) {
        set_error("gemm_run: X, W and Y must be non-NULL");
        return TLG_ERR_INVALID_ARG;
    }
    const bool want_bias = (p->epi & TLG_EPI_BIAS) != 0;
    if (want_bias != (bias != nullptr)) {
        set_error(want_bias ? "gemm_run: plan has TLG_EPI_BIAS but bias is NULL"
                            : "gemm_run: bias given but the plan has no TLG_EPI_BIAS");
        return TLG_ERR_INVALID_ARG;
    }
    const uintptr_t align = (uintptr_t)X | (uintptr_t)W | (uintptr_t)Y | (uintptr_t)bias |
                            (uintptr_t)workspace;
    if (align & 15u) {
        set_error("gemm_run: every pointer must be 16-byte aligned");
        return TLG_ERR_MISALIGNED;
    }
    const size_t isz = dtype_size(p->in_dt), osz = dtype_size(p->out_dt);
    const size_t ybytes = (size_t)p->M * p->N * osz;
    if (overlaps(Y, ybytes, X, (size_t)p->M * p->K * isz) || overlaps(Y, ybytes, W, (size_t)p->N * p->K * isz) ||
        (bias && overlaps(Y, ybytes, bias, (size_t)p->N * isz))) {
        set_error("gemm_run: Y overlaps an input");
        return TLG_ERR_INVALID_ARG;
    }
    if (p->ws_bytes) {
        if (!workspace || ws_bytes < p->ws_bytes) {
            set_error("gemm_run: workspace of %zu bytes needed, %zu given", p->ws_bytes,
                      workspace ? ws_bytes : (size_t)0);
            return TLG_ERR_WORKSPACE;
        }
        if (overlaps(workspace, p->ws_bytes, Y, ybytes)) {
            set_error("gemm_run: workspace overlaps Y");
            return TLG_ERR_INVALID_ARG;
        }
        // partials written there while the inputs are still being read
        if (overlaps(workspace, p->ws_bytes, X, (size_t)p->M * p->K * isz) ||
            overlaps(workspace, p->ws_bytes, W, (size_t)p->N * p->K * isz) ||
            (bias && overlaps(workspace, p->ws_bytes, bias, (size_t)p->N * isz))) {
            set_error("gemm_run: workspace overlaps an input");
            return TLG_ERR_INVALID_ARG;
        }
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (p->variant) {
    case TLG_VARIANT_GENERIC: return launch_generic(*p, X, W, bias, Y, s);
    case TLG_VARIANT_STREAM: return launch_stream(*p, X, W, bias, Y, workspace, s);
    case TLG_VARIANT_TILED: return launch_tiled(*p, X, W, bias, Y, workspace, s);
    default: set_error("gemm_run: corrupt plan"); return TLG_ERR_INVALID_ARG;
    }
}
