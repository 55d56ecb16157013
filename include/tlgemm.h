/*
 * tlgemm — transformer linear-layer GEMM for one MI355X (gfx950).
 *
 *   Y[m][n] = act( sum_k X[m][k] * w(n,k)  (+ bias[n]) )
 *
 * The operation is the PyTorch linear layer of "One multiply, one RTX 5090,
 * eight kernels", section "The multiply": X holds one input vector per row,
 * the weight W is stored out×in ([N][K], so w(n,k) = W[n][k]) and every
 * output is the dot product of a row of X with a row of W.  The second
 * layout is the square row-major product C = A·B of "Writing a CUDA matmul
 * that catches cuBLAS", sections "The nine kernels" and "Kernel 1 → 2", with
 * B stored [K][N] (w(n,k) = B[k][n]).  The optional epilogue — bias add, then
 * tanh-GELU — is fused into the store as the pages do for their linear layers
 * ("Optimizing a GPT-2-class transformer on a GPU", Act II; "Writing a CUDA
 * matmul that catches cuBLAS", sections "The bias add did not need to exist"
 * and "The residual and GELU go the same way").  The planner picks one of
 * several kernels per shape, the routing-table idea of the first page's
 * Act II and of the second page's section "One kernel was never going to be
 * enough".
 *
 * The two transposed-input layouts complete the four transpose cases of
 * "Writing a CUDA matmul that catches cuBLAS" (section "Putting it in the
 * model, where it behaves differently") and with them the backward pass of
 * the same layer (section "Then: a language model on top of it"): with the
 * first operand stored [K][M], the weight gradient dW = dYᵀ·X is one call
 * (A = dY stored [tokens][out], B = X stored [tokens][in]), and dX = dY·W is
 * the TLG_KN layout.  The residual flag adds the layer's output onto what Y
 * already holds, the fused residual of that page's section "The residual and
 * GELU go the same way, and cost three detours".
 *
 * Conventions for every entry point:
 *  - Every tensor is dense and row-major with no padding: X [M][K] (or
 *    [K][M] for the TLG_AT_* layouts), W [N][K] (TLG_NK, TLG_AT_NK) or
 *    [K][N] (TLG_KN, TLG_AT_KN), bias [N], Y [M][N].
 *  - X, W and bias use the input element type; Y uses the output type.
 *    Products accumulate in fp32.  Half-precision outputs are rounded to
 *    nearest-even once, after the epilogue.
 *  - Device pointers are raw HIP device addresses (for example a torch
 *    tensor's data_ptr()).  The caller owns all memory; the library never
 *    allocates device memory and never frees caller buffers.
 *  - Status codes: 0 on success, a negative TLG_ERR_* value otherwise.  No
 *    C++ exception crosses this interface.  gemm_last_error() returns a
 *    thread-local message for the most recent failure on the calling thread.
 */
#ifndef TLGEMM_H
#define TLGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (the arithmetic is always fp32-accumulate). */
typedef enum { TLG_F32 = 0, TLG_F16 = 1, TLG_BF16 = 2 } tlg_dtype;

/* Operand layouts.  TLG_NK: W[N][K], Y = X·Wᵀ (PyTorch out×in).
 * TLG_KN: B[K][N], Y = X·B (row-major square GEMM).
 * TLG_AT_NK, TLG_AT_KN: as TLG_NK and TLG_KN with the first operand stored
 * transposed, A[K][M], so x(m,k) = A[k][m] (Y = Aᵀ·Wᵀ and Y = Aᵀ·B).  These
 * two take no bias or GELU (TLG_ERR_UNSUPPORTED); TLG_EPI_RESIDUAL is allowed,
 * for accumulating gradients. */
typedef enum { TLG_NK = 0, TLG_KN = 1, TLG_AT_NK = 2, TLG_AT_KN = 3 } tlg_layout;

/* Epilogue flags, applied in this order: bias, then GELU, then the residual.
 * TLG_EPI_RESIDUAL: Y is an input as well as the output; the result is
 * act(X·Wᵀ + bias) + Y, each element of Y read once before it is written
 * (summed in fp32, then rounded to the output type). */
enum { TLG_EPI_BIAS = 1u, TLG_EPI_GELU_TANH = 2u, TLG_EPI_RESIDUAL = 4u };

/* Status codes. */
enum {
    TLG_OK = 0,
    TLG_ERR_INVALID_ARG = -1, /* bad shape, enum, flag, NULL pointer or aliasing */
    TLG_ERR_UNSUPPORTED = -2, /* valid request this library does not implement */
    TLG_ERR_MISALIGNED = -3,  /* a pointer is not 16-byte aligned */
    TLG_ERR_WORKSPACE = -4,   /* workspace missing or smaller than gemm_workspace_size */
    TLG_ERR_NOMEM = -5,       /* host allocation failed */
    TLG_ERR_LAUNCH = -6       /* the HIP runtime refused a launch */
};

/* Kernel families the planner chooses between. */
typedef enum {
    TLG_VARIANT_AUTO = -1,
    TLG_VARIANT_GENERIC = 0, /* predicated LDS-tiled fp32-FMA kernel: any shape, any alignment */
    TLG_VARIANT_STREAM = 1,  /* narrow M: weights streamed HBM->registers, MFMA, one-launch split-K */
    TLG_VARIANT_TILED = 2    /* LDS-tiled MFMA kernel, optional split-K across workgroups */
} tlg_variant;

typedef struct tlg_plan* tlg_plan_t;

/* Planner overrides (tests and tuning). Zero / TLG_VARIANT_AUTO means "planner's choice". */
typedef struct {
    int variant; /* tlg_variant */
    int split_k; /* split of K across workgroups; 0 = planner */
    int tile;    /* index into the variant's tile list; 0 = planner, k>0 selects entry k-1 */
} tlg_plan_opts;

/* What the planner chose (for reports and tests). */
typedef struct {
    int variant;            /* tlg_variant */
    int tile_m, tile_n, tile_k;
    int split_k;            /* K ranges summed per output (1 = no split) */
    int threads;            /* threads per workgroup */
    int64_t workgroups;     /* total workgroups over all launches of one run */
    int launches;           /* kernel launches per gemm_run */
    size_t workspace_bytes; /* == gemm_workspace_size */
} tlg_plan_info;

/*
 * gemm_plan — choose a kernel, tile and split for one linear-layer shape.
 * Host-only and pure: no device call, no allocation on the device.
 * Supported (in_dt, out_dt): (F32,F32), (F16,F16), (F16,F32), (BF16,BF16),
 * (BF16,F32).  M, N, K must be >= 1; epi_flags only TLG_EPI_* bits.
 * On success *out holds a new plan (free with gemm_destroy); on error *out
 * is set to NULL and a TLG_ERR_* code is returned.
 */
int gemm_plan(tlg_plan_t* out, int64_t M, int64_t N, int64_t K, tlg_dtype in_dt, tlg_dtype out_dt,
              tlg_layout layout, uint32_t epi_flags);

/* gemm_plan with overrides; opts may be NULL.  A forced variant that cannot
 * run the shape (for example STREAM with M > 64) returns TLG_ERR_UNSUPPORTED. */
int gemm_plan_ex(tlg_plan_t* out, int64_t M, int64_t N, int64_t K, tlg_dtype in_dt,
                 tlg_dtype out_dt, tlg_layout layout, uint32_t epi_flags, const tlg_plan_opts* opts);

/* Bytes of device workspace gemm_run needs (0 when the plan needs none, or p is NULL). */
size_t gemm_workspace_size(tlg_plan_t p);

/* Fill *info with the plan's choices. */
int gemm_plan_info(tlg_plan_t p, tlg_plan_info* info);

/*
 * gemm_run — enqueue Y = act(X·Wᵀ + bias) (+ Y with TLG_EPI_RESIDUAL) on
 * `stream` (a hipStream_t; NULL means the default stream) and return after
 * the launch; errors inside a kernel surface at the next synchronisation.
 * X, W, Y (and bias if TLG_EPI_BIAS) must be non-NULL device pointers, 16-byte aligned; bias must
 * be NULL when TLG_EPI_BIAS is not set.  Y must not overlap X, W or bias.
 * workspace: device memory of at least gemm_workspace_size(p) bytes when
 * that is non-zero, overlapping none of X, W, bias and Y (TLG_ERR_INVALID_ARG
 * otherwise); it may be NULL when the size is 0.  Its first 64 KiB
 * hold arrival counters and the rest fp32 split partials.  It must be
 * zero-filled before its first use; after that every completed run of any
 * plan leaves the counters zero (split stream plans reset the counter of
 * each output tile in their last workgroup, tiled split plans write only
 * past the counters), so one workspace serves any sequence of plans whose
 * sizes it covers.  Runs in flight at the same time need distinct
 * workspaces.  A plan is immutable: concurrent runs of one plan are safe
 * when each has its own workspace.
 */
int gemm_run(tlg_plan_t p, const void* X, const void* W, const void* bias, void* Y,
             void* workspace, size_t ws_bytes, void* stream);

/*
 * gemm_run_no_alloc — gemm_run for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, checks and result as gemm_run, without the
 * workspace: split plans use a scratch array the library keeps in device
 * memory, 32 MiB per device, held from the first call on a device until the
 * process ends.  A plan whose gemm_workspace_size exceeds 32 MiB is refused
 * with TLG_ERR_WORKSPACE before any launch.  Nothing is allocated or freed:
 * the first call on a device looks up that device's array and clears its
 * counter block with a kernel on `stream`; every completed run leaves the
 * counters zero again.  All calls on one device share its array, so calls
 * that can overlap on one device (other streams, or work not yet finished on
 * another stream) race and must be serialised by the caller; calls on one
 * stream are ordered by the stream.
 */
int gemm_run_no_alloc(tlg_plan_t p, const void* X, const void* W, const void* bias, void* Y, void* stream);

/* Free a plan.  NULL is a no-op. */
int gemm_destroy(tlg_plan_t p);

/* Human-readable summary of the plan's choices, NUL-terminated and truncated
 * to n bytes.  Returns the length the full text needs (excluding the NUL). */
int gemm_plan_describe(tlg_plan_t p, char* buf, size_t n);

/* Static text for a status code. */
const char* gemm_status_string(int status);

/* Thread-local text of the most recent error on this thread ("" if none). */
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TLGEMM_H */
