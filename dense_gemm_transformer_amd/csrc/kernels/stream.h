// Stream kernel for narrow M (weight out×in): 16 to 64 rows per workgroup.
//
// "One multiply, one RTX 5090, eight kernels" ("The multiply", "Tiles, blocks
// and SMs", "Filling the chip", "Where the time goes"): with 16 input rows
// each weight value takes part in only 16 products, so the multiply is a
// stream of W from memory.  The design for gfx950:
//
//  * A workgroup has NB × KW waves.  It owns BN = 16·NB rows of W (each wave
//    16 rows: one MFMA column block) and one K range of the grid's split.
//    Inside the workgroup the KW waves of a column block split the K range
//    again, so a 16-row tile over all of K is 8 waves that never talk to
//    another workgroup (NB = 1, KW = 8: 256 workgroups for 4096 rows).
//  * W never passes through LDS: each lane issues 16-byte loads straight into
//    registers, all of a chunk's loads before the first product, so a wave
//    keeps LOADS KiB of W in flight.
//  * The X slice of the workgroup's K range is read with fully coalesced
//    loads (consecutive threads, consecutive 16 bytes of one row) into LDS
//    and every wave takes its MFMA operands from there.
//  * Products run on MFMA: 16×16×32 for fp16/bf16 (a 16-row block of X is
//    one MFMA row block) and 16×16×4 for fp32.  For fp32 one 16-byte load
//    feeds four MFMAs: the k order inside a chunk is permuted identically
//    for X and W, which leaves every dot product unchanged.
//  * The KW wave partials of a column block are summed through LDS in wave
//    order.  With a grid split (S > 1, the split-K of "Filling the chip")
//    each workgroup then publishes its partial tile, takes a ticket for the
//    tile, and the last to arrive sums the S partials in split order.  Both
//    sums run in a fixed order, so results are bitwise reproducible (the
//    rule of "Optimizing a GPT-2-class transformer on a GPU", Act I).  One
//    launch, no atomics on data.
//
// Rows of X past M and rows of W past N are clamped to valid rows (their
// outputs are never stored); K past the split's range loads as zero.
#pragma once
#include "common.h"

namespace tlg {

template <int IN, int NB, int KW, int LOADS, int ROWB>
struct StreamGeom {
    static constexpr int EPV = Elem<IN>::per16;  // elements per 16-byte load
    static constexpr int KSTEP = 4 * EPV;        // k covered by one load across the 4 lane groups
    static constexpr int CK = LOADS * KSTEP;     // k per wave per chunk
    static constexpr int WCK = KW * CK;          // k per workgroup per chunk
    static constexpr int XROWS = 16 * ROWB;
    static constexpr int LDX = WCK + EPV;        // padded LDS row of the X chunk (elements)
    static constexpr int X_BYTES = XROWS * LDX * (int)sizeof(typename Elem<IN>::storage);
    static constexpr int RED_BYTES = KW > 1 ? NB * KW * ROWB * 4 * 64 * 4 : 0;
    static constexpr int LDS_BYTES = X_BYTES + RED_BYTES;
    static constexpr bool FITS = LDS_BYTES <= 160 * 1024;
};

template <int IN, int OUT, uint32_t EPI, int NB, int KW, int LOADS, int ROWB, bool EVEN, bool SPLIT>
__global__ __launch_bounds__(64 * NB * KW) void stream_kernel(const void* __restrict__ Xv,
                                                             const void* __restrict__ Wv,
                                                             const void* __restrict__ bias,
                                                             void* __restrict__ Yv, float* __restrict__ ws,
                                                             unsigned* __restrict__ tickets, int M, int N,
                                                             int K, int kper, int resid) {
    using S = typename Elem<IN>::storage;
    using G = StreamGeom<IN, NB, KW, LOADS, ROWB>;
    constexpr bool F32 = IN == TLG_F32;
    constexpr int THREADS = 64 * NB * KW;
    constexpr int EPV = G::EPV, KSTEP = G::KSTEP, CK = G::CK, WCK = G::WCK, LDX = G::LDX;
    constexpr int XVPR = WCK / EPV;              // 16-byte vectors per X chunk row
    constexpr int XVEC = G::XROWS * XVPR;
    constexpr int XPT = (XVEC + THREADS - 1) / THREADS;
    constexpr int BN = 16 * NB;
    const S* __restrict__ X = static_cast<const S*>(Xv);
    const S* __restrict__ W = static_cast<const S*>(Wv);
    void* __restrict__ Y = Yv;

    __shared__ __attribute__((aligned(16))) char lds[G::LDS_BYTES];
    S* xs = reinterpret_cast<S*>(lds);

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nb = wave / KW, kw = wave % KW;
    const int r = lane & 15, g = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int n0 = tile * BN;
    // Grid z walks blocks of 16·ROWB rows of X (more than one only when M
    // exceeds them, as for the 128-row layers); W is re-read per row block.
    const int mb = blockIdx.z * G::XROWS;
    X += (int64_t)mb * K;
    Y = static_cast<char*>(Y) + (int64_t)mb * N * (OUT == TLG_F32 ? 4 : 2);
    M = min(M - mb, G::XROWS);
    const S* Wrow = W + (int64_t)min(n0 + nb * 16 + r, N - 1) * K;
    const int kbeg = split * kper;
    const int kend = min(kbeg + kper, K);

    f32x4 acc[ROWB];
#pragma unroll
    for (int rb = 0; rb < ROWB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = kbeg; kc < kend; kc += WCK) {
        // X chunk first (cache-resident, coalesced), then this wave's W
        // stream; the scheduling barrier keeps every load ahead of the first use.
        u32x4 xr[XPT];
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int v = t + THREADS * i;
            const int row = v / XVPR, k = kc + (v % XVPR) * EPV;
            if ((XVEC % THREADS == 0 || v < XVEC) && (EVEN || k < kend))
                xr[i] = ldg16(X + (int64_t)min(row, M - 1) * K + k);
            else
                xr[i] = u32x4{0u, 0u, 0u, 0u};
        }
        const int kw0 = kc + kw * CK;
        u32x4 wv[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int k = kw0 + j * KSTEP + g * EPV;
            if (EVEN || k < kend)
                wv[j] = ldg16(Wrow + k);
            else
                wv[j] = u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int v = t + THREADS * i;
            if (XVEC % THREADS == 0 || v < XVEC)
                *reinterpret_cast<u32x4*>(xs + (v / XVPR) * LDX + (v % XVPR) * EPV) = xr[i];
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb) {
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const u32x4 xv =
                    *reinterpret_cast<const u32x4*>(xs + (rb * 16 + r) * LDX + kw * CK + j * KSTEP + g * EPV);
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[rb] = mfma16_f32(__uint_as_float(xv[e]), __uint_as_float(wv[j][e]), acc[rb]);
                } else {
                    acc[rb] = mfma16_16bit<IN>(xv, wv[j], acc[rb]);
                }
            }
        }
        if (kc + WCK < kend) __syncthreads();  // the next chunk overwrites xs
    }

    // In-workgroup K reduction: wave kw = 0 of each column block sums the KW
    // partials in wave order.  A 16×16 MFMA accumulator holds column
    // (lane % 16) and rows 4*(lane / 16) + e.
    if constexpr (KW > 1) {
        float* red = reinterpret_cast<float*>(lds + G::X_BYTES);  // [nb][kw][rb][e][lane]
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(((nb * KW + kw) * ROWB + rb) * 4 + e) * 64 + lane] = acc[rb][e];
        __syncthreads();
        if (kw == 0) {
#pragma unroll
            for (int rb = 0; rb < ROWB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float s = red[(((nb * KW) * ROWB + rb) * 4 + e) * 64 + lane];
#pragma unroll
                    for (int q = 1; q < KW; ++q) s += red[(((nb * KW + q) * ROWB + rb) * 4 + e) * 64 + lane];
                    acc[rb][e] = s;
                }
        }
    }

    const int n = n0 + nb * 16 + r;
    if constexpr (!SPLIT) {
        if (kw != 0) return;
        float b = 0.0f;
        if constexpr ((EPI & TLG_EPI_BIAS) != 0)
            if (n < N) b = load_elem<IN>(bias, n);
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = rb * 16 + 4 * g + e;
                if (m < M && n < N) {
                    float v = epilogue<EPI>(acc[rb][e], b);
                    if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
                    store_out<OUT>(Y, (int64_t)m * N + n, v);
                }
            }
    } else {
        // Partials in fragment order [split][tile][nb][rb][lane] (one
        // 16-byte store per lane); the reducing workgroup reads the same order.
        f32x4* frag = reinterpret_cast<f32x4*>(ws);
        const int64_t tiles = (int64_t)gridDim.x * gridDim.z;
        const int64_t tid = (int64_t)blockIdx.z * gridDim.x + tile;  // ticket of this (row block, tile)
        const int64_t per_split = tiles * NB * ROWB * 64;
        const int64_t base = ((tid * NB + nb) * ROWB) * 64 + lane;
        if (kw == 0)
#pragma unroll
            for (int rb = 0; rb < ROWB; ++rb) frag[split * per_split + base + rb * 64] = acc[rb];
        // Release this workgroup's partials at device scope (one fence after
        // the workgroup barrier covers every wave), then take the tile's ticket.
        __syncthreads();
        __shared__ unsigned last;
        if (t == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            last = atomicAdd(&tickets[tid], 1u) == gridDim.y - 1;
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (!last || kw != 0) return;
        const int splits = gridDim.y;
        float b = 0.0f;
        if constexpr ((EPI & TLG_EPI_BIAS) != 0)
            if (n < N) b = load_elem<IN>(bias, n);
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb) {
            f32x4 part[kStreamMaxSplit];  // every split's fragment in flight, then the ordered sum
#pragma unroll
            for (int z = 0; z < kStreamMaxSplit; ++z)
                part[z] = z < splits ? frag[z * per_split + base + rb * 64] : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 s4 = part[0];
#pragma unroll
            for (int z = 1; z < kStreamMaxSplit; ++z)
                if (z < splits) s4 += part[z];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = rb * 16 + 4 * g + e;
                if (m < M && n < N) {
                    float v = epilogue<EPI>(s4[e], b);
                    if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
                    store_out<OUT>(Y, (int64_t)m * N + n, v);
                }
            }
        }
        if (t == 0) __hip_atomic_store(&tickets[tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Narrow 16-bit layers (M <= 16, K a multiple of 512 up to 4096): the 16
// weight rows of a tile live in LDS for the whole K range.  Timed on the
// 16×4096×4096 layer with cold weights, this beats streaming the weight into
// registers by 0.3-0.8 µs of ~9 (probe kernels, rocprofv3 medians on several
// boxes), for two reasons:
//  * each direct load (global_load_lds) reads one contiguous KiB of a weight
//    row, where an MFMA-operand load spreads 64 bytes over each of 16 rows;
//    the weight is never in registers, so it needs no staging;
//  * X goes straight to registers in the MFMA operand layout, each wave its
//    own K range, X and weight loads interleaved: X needs no LDS store and no
//    barrier of its own, and never waits behind the whole weight stream.
// Wave w fetches weight rows 2w and 2w+1; instruction (row R, KiB h) lands
// at LDS row R, bytes [1 KiB·h, 1 KiB·(h+1)), lane l at 16·l.  The lanes
// fetch the 16-byte chunks of that KiB permuted, chunk c at c ^ (R % 16), so
// the operand reads of 16 rows at one k hit 16 distinct 4-bank groups.  Wave
// w then multiplies K range [w·K/8, (w+1)·K/8) and the 8 partials are summed
// through LDS in wave order, as in the register-streaming kernel.
// PR: KiB-instructions per weight row (K = 512·PR); a wave issues 2·PR
// direct loads and 2·PR X loads and runs 2·PR MFMA steps of 32 k, all
// unrolled with no condition, so every load is issued before the first wait.
template <int IN, int OUT, uint32_t EPI, int PR>
__global__ __launch_bounds__(512) void stream_dl_kernel(const void* __restrict__ Xv, const void* __restrict__ Wv,
                                                       const void* __restrict__ bias, void* __restrict__ Y, int M,
                                                       int N, int resid) {
    static_assert(IN != TLG_F32 && PR >= 1 && PR * kStreamDlKStep <= kStreamDlMaxK, "16-bit operands, K in LDS");
    using S = uint16_t;
    constexpr int KW = 8, K = PR * kStreamDlKStep, STEPS = 2 * PR, KPW = K / KW;
    __shared__ __attribute__((aligned(16))) S wl[16 * K];
    __shared__ float red[KW * 4 * 64];
    const S* __restrict__ X = static_cast<const S*>(Xv);
    const S* __restrict__ W = static_cast<const S*>(Wv);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const S* xrow = X + (int64_t)min(r, M - 1) * K + w * KPW + 8 * g;  // rows past M repeat row M-1, never stored
    u32x4 xr[STEPS];
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
        xr[j] = ldg16(xrow + 32 * j);
        const int R = 2 * w + j / PR, h = j % PR;
        const int c = ((h << 6) + lane) ^ (R & 15);
        const S* src = W + (int64_t)min(n0 + R, N - 1) * K + 8 * c;  // rows past N repeat row N-1, never stored
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (__attribute__((address_space(3))) void*)(wl + R * K + h * 512), 16, 0,
                                         2 /* nt: streamed once */);
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): this wave's X and direct loads have landed
    __syncthreads();                                   // and every other wave's weight rows
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
        const int c = (w * KPW + 32 * j) / 8 + g;  // 16-byte chunk of weight row r
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wl + r * K + 8 * (c ^ r));
        acc = mfma16_16bit<IN>(xr[j], wv, acc);
    }
    // wave partials summed in wave order; a 16×16 accumulator holds column
    // (lane % 16) and rows 4·(lane / 16) + e
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(w * 4 + e) * 64 + lane] = acc[e];
    __syncthreads();
    if (w != 0) return;
    const int n = n0 + r;
    float b = 0.0f;
    if constexpr ((EPI & TLG_EPI_BIAS) != 0)
        if (n < N) b = load_elem<IN>(bias, n);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float sum = red[e * 64 + lane];
#pragma unroll
        for (int q = 1; q < KW; ++q) sum += red[(q * 4 + e) * 64 + lane];
        const int m = 4 * g + e;
        if (m < M && n < N) {
            float v = epilogue<EPI>(sum, b);
            if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
            store_out<OUT>(Y, (int64_t)m * N + n, v);
        }
    }
}

template <int I, int NB, int KW, int LOADS>
static int launch_stream_cfg(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                             hipStream_t stream) {
    const int S = p.split;
    const int kper = (int)p.kper;
    const bool even = (int64_t)kper * S == p.K && kper % (KW * LOADS * 4 * Elem<I>::per16) == 0;
    const dim3 grid((unsigned)p.grid_x, (unsigned)S, (unsigned)p.grid_z), block(64 * NB * KW);
    unsigned* tickets = static_cast<unsigned*>(ws);
    float* part = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + kWsCounterBytes) : nullptr;
    auto with_out = [&](auto f) {
        if constexpr (I == TLG_F32) return f(ic<TLG_F32>{});
        else if (p.out_dt == TLG_F32) return f(ic<TLG_F32>{});
        else return f(ic<I>{});
    };
    return with_out([&](auto out) {
        return with_epi(p.epi, [&](auto epi) {
            constexpr int O = decltype(out)::value;
            constexpr uint32_t E = (uint32_t)decltype(epi)::value;
            auto go = [&](auto rowb, auto ev, auto sp) -> int {
                constexpr int RB = decltype(rowb)::value;
                if constexpr (!StreamGeom<I, NB, KW, LOADS, RB>::FITS) {
                    set_error("stream configuration does not fit in LDS for M=%lld", (long long)p.M);
                    return TLG_ERR_UNSUPPORTED;
                } else {
                    hipLaunchKernelGGL((stream_kernel<I, O, E, NB, KW, LOADS, RB, decltype(ev)::value,
                                                      decltype(sp)::value>),
                                       grid, block, 0, stream, X, W, bias, Y, part, tickets, (int)p.M, (int)p.N,
                                       (int)p.K, kper, (int)((p.epi & TLG_EPI_RESIDUAL) != 0));
                    return check_launch("stream_kernel");
                }
            };
            auto by_split = [&](auto rowb, auto ev) {
                return S > 1 ? go(rowb, ev, std::true_type{}) : go(rowb, ev, std::false_type{});
            };
            auto by_even = [&](auto rowb) {
                return even ? by_split(rowb, std::true_type{}) : by_split(rowb, std::false_type{});
            };
            if (p.rowb == 1) return by_even(ic<1>{});
            if (p.rowb == 2) return by_even(ic<2>{});
            return by_even(ic<4>{});
        });
    });
}

template <int I>
static int launch_stream_dl(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                            hipStream_t stream) {
    if constexpr (I == TLG_F32) {
        set_error("the direct-load stream tile takes 16-bit inputs");
        return (int)TLG_ERR_UNSUPPORTED;
    } else {
        // the planner's conditions, checked again before the launch
        if (p.M > 16 || p.K % kStreamDlKStep != 0 || p.K > kStreamDlMaxK || p.split != 1 || p.grid_z != 1) {
            set_error("direct-load stream tile: shape outside its limits");
            return (int)TLG_ERR_INVALID_ARG;
        }
        auto with_out = [&](auto f) {
            if (p.out_dt == TLG_F32) return f(ic<TLG_F32>{});
            return f(ic<I>{});
        };
        return with_out([&](auto out) {
            return with_epi(p.epi, [&](auto epi) {
                constexpr int O = decltype(out)::value;
                constexpr uint32_t E = (uint32_t)decltype(epi)::value;
                const int resid = (p.epi & TLG_EPI_RESIDUAL) != 0;
                auto go = [&](auto pr) {
                    hipLaunchKernelGGL((stream_dl_kernel<I, O, E, decltype(pr)::value>), dim3((unsigned)p.grid_x),
                                       dim3(512), 0, stream, X, W, bias, Y, (int)p.M, (int)p.N, resid);
                    return check_launch("stream_dl_kernel");
                };
                static_assert(kStreamDlMaxK == 8 * kStreamDlKStep, "one instantiation per K");
                switch (p.K / kStreamDlKStep) {
                case 1: return go(ic<1>{});
                case 2: return go(ic<2>{});
                case 3: return go(ic<3>{});
                case 4: return go(ic<4>{});
                case 5: return go(ic<5>{});
                case 6: return go(ic<6>{});
                case 7: return go(ic<7>{});
                default: return go(ic<8>{});
                }
            });
        });
    }
}

// All stream launches for one input dtype; explicitly instantiated once per
// dtype in its own translation unit.
template <int I>
int launch_stream_in(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                     hipStream_t stream) {
    static_assert(kNumStream == 10 && kStream[5].dl, "stream configurations changed");
#define TLG_STREAM_CASE(i) \
    case i: return launch_stream_cfg<I, kStream[i].nb, kStream[i].kw, kStream[i].loads>(p, X, W, bias, Y, ws, stream);
    switch (p.tile) {
        TLG_STREAM_CASE(0)
        TLG_STREAM_CASE(1)
        TLG_STREAM_CASE(2)
        TLG_STREAM_CASE(3)
        TLG_STREAM_CASE(4)
    case 5: return launch_stream_dl<I>(p, X, W, bias, Y, stream);
        TLG_STREAM_CASE(6)
        TLG_STREAM_CASE(7)
        TLG_STREAM_CASE(8)
        TLG_STREAM_CASE(9)
    default: set_error("bad stream tile"); return (int)TLG_ERR_INVALID_ARG;
    }
#undef TLG_STREAM_CASE
}

}  // namespace tlg
