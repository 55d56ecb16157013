// Stream kernel for narrow M (M <= 64, weight out×in).
//
// "One multiply, one RTX 5090, eight kernels" ("The multiply", "Filling the
// chip", "Where the time goes"): with 16 input rows each weight value takes
// part in only 16 products, so the multiply is a stream of W from memory and
// its time is the time to read W.  The design for gfx950:
//
//  * One workgroup owns 16 rows of W (16 output columns) over all of K.  Its
//    waves split K into contiguous ranges (the split-K of "Filling the
//    chip"), so a 4096-row weight gives 256 workgroups, one per CU, and every
//    CU streams its own 128 KiB slab of W.
//  * W never touches LDS: each lane issues 16-byte loads straight into
//    registers, all of a chunk's loads before any use, so one wave keeps
//    LOADS×1 KiB of W in flight.  The 4 lanes of a W row read 64
//    consecutive bytes per load and consecutive loads continue the row.
//  * Products run on MFMA: 16×16×32 for fp16/bf16 (one 16-row block of X is
//    one MFMA row block) and 16×16×4 for fp32.  For fp32 one 16-byte load
//    feeds four MFMAs: the k order inside a chunk is permuted identically
//    for X and W, which leaves the dot products unchanged.
//  * The wave partials are summed through LDS in a fixed order (wave 0, 1,
//    ...), so results are bitwise reproducible run to run, then the fused
//    epilogue (bias, GELU, rounding) writes Y.  No workspace, one launch.
//
// Rows of X past M and rows of W past N are clamped to valid rows (their
// outputs are never stored); K past each wave's range loads as zero.

#pragma once
#include "common.h"

namespace tlg {

template <int IN, int OUT, uint32_t EPI, int WAVES, int LOADS, int ROWB, bool EVENK>
__global__ __launch_bounds__(64 * WAVES) void stream_kernel(const void* __restrict__ Xv,
                                                           const void* __restrict__ Wv,
                                                           const void* __restrict__ bias,
                                                           void* __restrict__ Y, int M, int N, int K,
                                                           int kper) {
    using S = typename Elem<IN>::storage;
    constexpr bool F32 = IN == TLG_F32;
    constexpr int EPV = Elem<IN>::per16;   // elements per 16-byte load
    constexpr int KSTEP = 4 * EPV;         // k covered by one load across the 4 lane groups
    constexpr int CK = LOADS * KSTEP;      // k per chunk
    const S* __restrict__ X = static_cast<const S*>(Xv);
    const S* __restrict__ W = static_cast<const S*>(Wv);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const S* Wrow = W + (int64_t)min(n0 + r, N - 1) * K;
    const int kbeg = w * kper;
    const int kend = min(kbeg + kper, K);

    f32x4 acc[ROWB];
#pragma unroll
    for (int rb = 0; rb < ROWB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = kbeg; kc < kend; kc += CK) {
        u32x4 wv[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int k = kc + j * KSTEP + g * EPV;
            if (EVENK || k < kend)
                wv[j] = ldg16(Wrow + k);
            else
                wv[j] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb) {
            const S* Xrow = X + (int64_t)min(rb * 16 + r, M - 1) * K;
            u32x4 xv[LOADS];
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const int k = kc + j * KSTEP + g * EPV;
                if (EVENK || k < kend)
                    xv[j] = ldg16(Xrow + k);
                else
                    xv[j] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                if constexpr (F32) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[rb] = mfma16_f32(__uint_as_float(xv[j][i]), __uint_as_float(wv[j][i]), acc[rb]);
                } else {
                    acc[rb] = mfma16_16bit<IN>(xv[j], wv[j], acc[rb]);
                }
            }
        }
    }

    // Fixed-order reduction of the wave partials.  A 16×16 MFMA accumulator
    // holds column (lane % 16), rows 4*(lane / 16) + v.
    __shared__ float red[WAVES][ROWB][4][64];
#pragma unroll
    for (int rb = 0; rb < ROWB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][rb][v][lane] = acc[rb][v];
    __syncthreads();

    for (int o = threadIdx.x; o < ROWB * 256; o += 64 * WAVES) {
        const int rb = o >> 8, ml = (o >> 4) & 15, c = o & 15;
        const int src = (ml >> 2) * 16 + c, v = ml & 3;
        float s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) s += red[ww][rb][v][src];
        const int m = rb * 16 + ml, n = n0 + c;
        if (m < M && n < N) {
            float b = 0.0f;
            if constexpr ((EPI & TLG_EPI_BIAS) != 0) b = load_elem<IN>(bias, n);
            store_out<OUT>(Y, (int64_t)m * N + n, epilogue<EPI>(s, b));
        }
    }
}

template <int I, int WAVES, int LOADS>
static int launch_stream_cfg(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                             hipStream_t stream) {
    constexpr int epv = Elem<I>::per16;
    constexpr int ck = LOADS * 4 * epv;
    int kper = (int)ceil_div(ceil_div(p.K, WAVES), epv) * epv;
    const bool evenk = (p.K % ((int64_t)WAVES * ck)) == 0;
    if (evenk) kper = (int)(p.K / WAVES);
    const dim3 grid((unsigned)p.grid_x), block(64 * WAVES);
    auto with_out = [&](auto f) {
        if constexpr (I == TLG_F32) return f(ic<TLG_F32>{});
        else if (p.out_dt == TLG_F32) return f(ic<TLG_F32>{});
        else return f(ic<I>{});
    };
    return with_out([&](auto out) {
        return with_epi(p.epi, [&](auto epi) {
            constexpr int O = decltype(out)::value;
            constexpr uint32_t E = (uint32_t)decltype(epi)::value;
            auto go = [&](auto rowb, auto even) {
                hipLaunchKernelGGL((stream_kernel<I, O, E, WAVES, LOADS, decltype(rowb)::value,
                                                  decltype(even)::value>),
                                   grid, block, 0, stream, X, W, bias, Y, (int)p.M, (int)p.N, (int)p.K, kper);
                return check_launch("stream_kernel");
            };
            auto by_rowb = [&](auto even) {
                if (p.rowb == 1) return go(ic<1>{}, even);
                if (p.rowb == 2) return go(ic<2>{}, even);
                return go(ic<4>{}, even);
            };
            return evenk ? by_rowb(std::true_type{}) : by_rowb(std::false_type{});
        });
    });
}

// All stream launches for one input dtype; explicitly instantiated once per
// dtype in its own translation unit.
template <int I>
int launch_stream_in(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                     hipStream_t stream) {
    static_assert(kNumStream == 3, "stream configurations changed");
    switch (p.tile) {
    case 0: return launch_stream_cfg<I, kStream[0].waves, kStream[0].loads>(p, X, W, bias, Y, stream);
    case 1: return launch_stream_cfg<I, kStream[1].waves, kStream[1].loads>(p, X, W, bias, Y, stream);
    default: return launch_stream_cfg<I, kStream[2].waves, kStream[2].loads>(p, X, W, bias, Y, stream);
    }
}

}  // namespace tlg
