// Generic predicated kernel: any M, N, K, any row alignment, every dtype
// pair, all four operand layouts, fused epilogue and residual.  It is the correctness fallback
// the planner uses when rows are not 16-byte aligned.
//
// Shared-memory block tiling and register tiling as on "Writing a CUDA
// matmul that catches cuBLAS" ("Kernels 3–5: reuse, at three levels"): a
// 64×64 output tile per workgroup, K in slices of 16 staged through LDS,
// 4×4 outputs per thread, fp32 FMA.  Every global access is bounds-checked;
// out-of-range K contributes exact zeros.

#include "common.h"

namespace tlg {

template <int IN, int OUT, int LAYOUT, uint32_t EPI>
__global__ __launch_bounds__(256) void generic_kernel(const void* __restrict__ X, const void* __restrict__ W,
                                                     const void* __restrict__ bias, void* __restrict__ Y,
                                                     int M, int N, int K, int resid) {
    constexpr int BM = kGenericBM, BN = kGenericBN, BK = kGenericBK;
    __shared__ float As[BK][BM + 1];  // [k][m]
    __shared__ float Bs[BK][BN + 1];  // [k][n]
    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    float acc[4][4] = {};

    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < (BM * BK) / 256; ++i) {
            const int e = t + 256 * i;
            const int r = e / BK, kk = e % BK;
            const int m = m0 + r, k = k0 + kk;
            const int64_t xi = layout_a_transposed(LAYOUT) ? (int64_t)k * M + m : (int64_t)m * K + k;
            As[kk][r] = (m < M && k < K) ? load_elem<IN>(X, xi) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < (BN * BK) / 256; ++i) {
            const int e = t + 256 * i;
            if constexpr (!layout_b_kn(LAYOUT)) {
                const int c = e / BK, kk = e % BK;
                const int n = n0 + c, k = k0 + kk;
                Bs[kk][c] = (n < N && k < K) ? load_elem<IN>(W, (int64_t)n * K + k) : 0.0f;
            } else {
                const int kk = e / BN, c = e % BN;
                const int n = n0 + c, k = k0 + kk;
                Bs[kk][c] = (n < N && k < K) ? load_elem<IN>(W, (int64_t)k * N + n) : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            float b = 0.0f;
            if constexpr ((EPI & TLG_EPI_BIAS) != 0) b = load_elem<IN>(bias, n);
            float v = epilogue<EPI>(acc[i][j], b);
            if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
            store_out<OUT>(Y, (int64_t)m * N + n, v);
        }
    }
}

int launch_generic(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                   hipStream_t stream) {
    const dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y, 1);
    return with_types(p.in_dt, p.out_dt, [&](auto in, auto out) {
        return with_layout(p.layout, [&](auto lay) {
            constexpr int L = decltype(lay)::value;
            auto go = [&](auto epi) {
                hipLaunchKernelGGL((generic_kernel<decltype(in)::value, decltype(out)::value, L,
                                                   (uint32_t)decltype(epi)::value>),
                                   grid, dim3(256), 0, stream, X, W, bias, Y, (int)p.M, (int)p.N, (int)p.K,
                                   (int)((p.epi & TLG_EPI_RESIDUAL) != 0));
                return check_launch("generic_kernel");
            };
            // the planner admits no bias or GELU with a transposed first operand
            if constexpr (layout_a_transposed(L)) return go(ic<0>{});
            else return with_epi(p.epi, go);
        });
    });
}

}  // namespace tlg
