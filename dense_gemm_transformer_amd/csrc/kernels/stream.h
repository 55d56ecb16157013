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
//    keeps LOADS KiB of W in flight.  Pipelined options go one chunk further:
//    chunk c + 1's loads are issued before chunk c's products, into a second
//    register set and a second X buffer, so that the products hide the loads.
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
//    launch, no atomics on data.  The partials cross XCDs, whose L2s are not
//    kept coherent with one another; they are written and read with
//    device-scope accesses (written through the writer's L2, read past the
//    reader's), and the writer waits for its stores to complete before it
//    takes the ticket.  A device-scope release and acquire would write back
//    and invalidate whole L2s instead: measured on a 16-row probe, 13-17 µs
//    against 10.2 µs for this form and 8.2 µs with no reduction at all.
//
// Rows of X past M and rows of W past N are clamped to valid rows (their
// outputs are never stored); K past the split's range loads as zero.
#pragma once
#include "common.h"

namespace tlg {

template <int IN, int NB, int KW, int LOADS, int ROWB, bool PIPE = false>
struct StreamGeom {
    static constexpr int EPV = Elem<IN>::per16;  // elements per 16-byte load
    static constexpr int KSTEP = 4 * EPV;        // k covered by one load across the 4 lane groups
    static constexpr int CK = LOADS * KSTEP;     // k per wave per chunk
    static constexpr int WCK = KW * CK;          // k per workgroup per chunk
    static constexpr int XROWS = 16 * ROWB;
    static constexpr int LDX = WCK + EPV;        // padded LDS row of the X chunk (elements)
    static constexpr int X_BUF = XROWS * LDX;  // elements of one staged X chunk
    static constexpr int X_BYTES = (PIPE ? 2 : 1) * X_BUF * (int)sizeof(typename Elem<IN>::storage);
    static constexpr int RED_BYTES = KW > 1 ? NB * KW * ROWB * 4 * 64 * 4 : 0;
    static constexpr int LDS_BYTES = X_BYTES + RED_BYTES;
    static constexpr bool FITS = LDS_BYTES <= 160 * 1024;
};

template <int IN, int OUT, uint32_t EPI, int NB, int KW, int LOADS, int ROWB, bool EVEN, bool SPLIT, bool PIPE>
__global__ __launch_bounds__(64 * NB * KW) void stream_kernel(const void* __restrict__ Xv,
                                                             const void* __restrict__ Wv,
                                                             const void* __restrict__ bias,
                                                             void* __restrict__ Yv, float* __restrict__ ws,
                                                             unsigned* __restrict__ tickets, int M, int N,
                                                             int K, int kper, int resid) {
    using S = typename Elem<IN>::storage;
    using G = StreamGeom<IN, NB, KW, LOADS, ROWB, PIPE>;
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

    // X chunk first (cache-resident, coalesced), then this wave's W stream.
    auto load_chunk = [&](int kc, u32x4 (&xr)[XPT], u32x4 (&wv)[LOADS]) {
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
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int k = kw0 + j * KSTEP + g * EPV;
            if (EVEN || k < kend)
                wv[j] = ldg16(Wrow + k);
            else
                wv[j] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stage_x = [&](S* xb, const u32x4 (&xr)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int v = t + THREADS * i;
            if (XVEC % THREADS == 0 || v < XVEC)
                *reinterpret_cast<u32x4*>(xb + (v / XVPR) * LDX + (v % XVPR) * EPV) = xr[i];
        }
    };
    auto multiply = [&](const S* xb, const u32x4 (&wv)[LOADS]) {
#pragma unroll
        for (int rb = 0; rb < ROWB; ++rb) {
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const u32x4 xv =
                    *reinterpret_cast<const u32x4*>(xb + (rb * 16 + r) * LDX + kw * CK + j * KSTEP + g * EPV);
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[rb] = mfma16_f32(__uint_as_float(xv[e]), __uint_as_float(wv[j][e]), acc[rb]);
                } else {
                    acc[rb] = mfma16_16bit<IN>(xv, wv[j], acc[rb]);
                }
            }
        }
    };
    if constexpr (!PIPE) {
        // Every load of a chunk ahead of its first product (the scheduling
        // barrier), then one X buffer: a barrier before the next chunk's staging.
        for (int kc = kbeg; kc < kend; kc += WCK) {
            u32x4 xr[XPT], wv[LOADS];
            load_chunk(kc, xr, wv);
            __builtin_amdgcn_sched_barrier(0);
            stage_x(xs, xr);
            __syncthreads();
            multiply(xs, wv);
            if (kc + WCK < kend) __syncthreads();  // the next chunk overwrites xs
        }
    } else {
        // Pipelined chunks: chunk c + 1's X and weight loads go out before
        // chunk c's products, so they land while the MFMAs run.  Two register
        // sets and two X buffers alternate (set and buffer A for even chunks, B
        // for odd), so no prefetched register is copied: a copy would wait for
        // the prefetch before the loop goes on.  The one barrier per chunk also
        // orders the staging of chunk c + 2 into a buffer after every wave's
        // products from it.  The last chunk leaves the loop before issuing a
        // prefetch, so the wait before each chunk's products covers only that
        // chunk's loads.
        u32x4 xa[XPT], wa[LOADS], xb_[XPT], wb[LOADS];
        S* const bufa = xs;
        S* const bufb = xs + G::X_BUF;
        load_chunk(kbeg, xa, wa);
        for (int kc = kbeg; kc < kend;) {  // an empty range (none is planned) skips the loop
            stage_x(bufa, xa);
            __syncthreads();
            if (kc + WCK >= kend) {
                multiply(bufa, wa);
                break;
            }
            load_chunk(kc + WCK, xb_, wb);
            __builtin_amdgcn_sched_barrier(0);
            multiply(bufa, wa);
            kc += WCK;
            stage_x(bufb, xb_);
            __syncthreads();
            if (kc + WCK >= kend) {
                multiply(bufb, wb);
                break;
            }
            load_chunk(kc + WCK, xa, wa);
            __builtin_amdgcn_sched_barrier(0);
            multiply(bufb, wb);
            kc += WCK;
        }
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
        // The host keeps the partial region below 2^31 bytes (one buffer
        // descriptor covers it).
        const int64_t tiles = (int64_t)gridDim.x * gridDim.z;
        const int64_t tid = (int64_t)blockIdx.z * gridDim.x + tile;  // ticket of this (row block, tile)
        const int64_t per_split = tiles * NB * ROWB * 64;
        const int64_t base = ((tid * NB + nb) * ROWB) * 64 + lane;
        const i32x4 prs = buffer_rsrc(ws, (int64_t)gridDim.y * per_split * 16);
        if (kw == 0)
#pragma unroll
            for (int rb = 0; rb < ROWB; ++rb)
                buffer_store16(__builtin_bit_cast(u32x4, acc[rb]), prs,
                               (uint32_t)((split * per_split + base + rb * 64) * 16), 0, kAuxDevice);
        // Every store of this wave has completed (written through its L2)
        // before the workgroup barrier, and so before the ticket is taken.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ unsigned last;
        if (t == 0)
            last = __hip_atomic_fetch_add(&tickets[tid], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   gridDim.y - 1;
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
                part[z] = z < splits ? __builtin_bit_cast(f32x4, buffer_load16(prs, (uint32_t)((z * per_split + base +
                                                                                              rb * 64) * 16), 0,
                                                                               kAuxDevice))
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
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

// Wait until at most N vector-memory operations of this wave are in flight
// (direct loads to LDS included).  The scheduling barriers keep the LDS reads
// of the phase this wait covers below it.
template <int N> __device__ inline void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Narrow 16-bit layers (M <= 16, K a multiple of 512 up to 4096): wave w
// owns K range [w·K/8, (w+1)·K/8) and fetches exactly the weights it
// multiplies, all 16 rows of the tile over that range, into an LDS region of
// its own by direct loads (global_load_lds); X goes straight to registers in
// the MFMA operand layout.  Timed on the 16×4096×4096 layer with cold
// weights (probe kernels, rocprofv3 medians), against the alternatives:
//  * streaming the weight into registers costs 1.5-2 µs more of ~9: an
//    MFMA-operand load spreads 64 bytes over each of 16 rows, where a direct
//    load here reads 128-byte runs of 8 rows;
//  * fetching whole rows per wave and multiplying after one workgroup
//    barrier (no product starts before the last weight byte of the tile has
//    landed) measured 8.6-8.8 against 8.2 µs at K = 4096, and 0.2-0.7 µs
//    more at every K from 512 to 3584 but one: at K = 2048 it was 0.5 µs
//    faster (6.1 against 6.7 µs), a case no tuned workload has.
// The wave's range is fetched in PR phases of 64 columns.  A phase is two X
// loads and two direct loads of 8 rows × 128 bytes (lane l: row 8i + l/8,
// 16-byte chunk l%8), and each phase has an LDS array of its own, so the wait
// before a phase's reads covers that phase's loads only (with one array for
// all of them the compiler waits for every load of the wave).  Products start
// as soon as the first phase has landed, with no barrier.  Chunk c of row R
// sits at position c ^ ((R/2) % 8) of its 128-byte slot, so the 16 lanes
// reading one k of 16 rows (two rows per 256 bytes) hit 16 distinct 4-bank
// groups.  The 8 wave partials are summed through LDS in wave order; waves
// 0-3 each finish one of the four accumulator rows.
// PR: 512-column steps of K (K = 512·PR); a wave issues 4·PR loads up front
// and runs 2·PR MFMA steps of 32 k, all unrolled.
template <int IN, int OUT, uint32_t EPI, int PR>
__global__ __launch_bounds__(512) void stream_dl_kernel(const void* __restrict__ Xv, const void* __restrict__ Wv,
                                                       const void* __restrict__ bias, void* __restrict__ Y, int M,
                                                       int N, int resid) {
    static_assert(IN != TLG_F32 && PR >= 1 && PR * kStreamDlKStep <= kStreamDlMaxK, "16-bit operands, K in LDS");
    static_assert(kStreamDlMaxK / kStreamDlKStep <= 8, "one LDS array per phase, at most 8");
    using S = uint16_t;
    constexpr int KW = 8, K = PR * kStreamDlKStep, KPW = K / KW;  // KPW = 64·PR: PR phases of 64 columns
    constexpr int PH = KW * 16 * 64;                             // one phase of every wave
    __shared__ __attribute__((aligned(16))) S ph0[PH];
    __shared__ __attribute__((aligned(16))) S ph1[PR > 1 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph2[PR > 2 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph3[PR > 3 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph4[PR > 4 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph5[PR > 5 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph6[PR > 6 ? PH : 8];
    __shared__ __attribute__((aligned(16))) S ph7[PR > 7 ? PH : 8];
    __shared__ float red[KW * 4 * 64];
    const S* __restrict__ X = static_cast<const S*>(Xv);
    const S* __restrict__ W = static_cast<const S*>(Wv);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    // this wave's part of phase p: two 1 KiB blocks of 8 rows × 64 columns
    auto region = [&](auto pc) -> S* {
        constexpr int p = decltype(pc)::value;
        S* a = p == 0 ? ph0 : p == 1 ? ph1 : p == 2 ? ph2 : p == 3 ? ph3 : p == 4 ? ph4 : p == 5 ? ph5 : p == 6 ? ph6 : ph7;
        return a + w * (16 * 64);
    };
    const S* xrow = X + (int64_t)min(r, M - 1) * K + w * KPW + 8 * g;  // rows past M repeat row M-1, never stored
    const int lr = lane >> 3, lc = lane & 7;
    u32x4 xr[2 * PR];
    auto issue = [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        S* dst = region(pc);
        xr[2 * p] = ldg16(xrow + 64 * p);
        xr[2 * p + 1] = ldg16(xrow + 64 * p + 32);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int R = 8 * i + lr;
            const S* src = W + (int64_t)min(n0 + R, N - 1) * K + w * KPW + 64 * p + 8 * (lc ^ ((R >> 1) & 7));
            __builtin_amdgcn_global_load_lds((const void*)src,  // rows past N repeat row N-1, never stored
                                             (__attribute__((address_space(3))) void*)(dst + 512 * i), 16, 0,
                                             2 /* nt: streamed once */);
        }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int rd = 512 * (r >> 3) + 64 * (r & 7), sw = (r >> 1) & 7;
    auto multiply = [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        wait_vmem<4 * (PR - p - 1)>();  // this phase's X and weight loads have landed
        const S* src = region(pc) + rd;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 wv = *reinterpret_cast<const u32x4*>(src + 8 * ((4 * i + g) ^ sw));
            acc = mfma16_16bit<IN>(xr[2 * p + i], wv, acc);
        }
    };
    using std::integral_constant;
    issue(integral_constant<int, 0>{});
    if constexpr (PR > 1) issue(integral_constant<int, 1>{});
    if constexpr (PR > 2) issue(integral_constant<int, 2>{});
    if constexpr (PR > 3) issue(integral_constant<int, 3>{});
    if constexpr (PR > 4) issue(integral_constant<int, 4>{});
    if constexpr (PR > 5) issue(integral_constant<int, 5>{});
    if constexpr (PR > 6) issue(integral_constant<int, 6>{});
    if constexpr (PR > 7) issue(integral_constant<int, 7>{});
    multiply(integral_constant<int, 0>{});
    if constexpr (PR > 1) multiply(integral_constant<int, 1>{});
    if constexpr (PR > 2) multiply(integral_constant<int, 2>{});
    if constexpr (PR > 3) multiply(integral_constant<int, 3>{});
    if constexpr (PR > 4) multiply(integral_constant<int, 4>{});
    if constexpr (PR > 5) multiply(integral_constant<int, 5>{});
    if constexpr (PR > 6) multiply(integral_constant<int, 6>{});
    if constexpr (PR > 7) multiply(integral_constant<int, 7>{});
    // wave partials summed in wave order; a 16×16 accumulator holds column
    // (lane % 16) and rows 4·(lane / 16) + e
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(w * 4 + e) * 64 + lane] = acc[e];
    __syncthreads();
    if (w >= 4) return;
    float sum = red[w * 64 + lane];  // wave w < 4 finishes accumulator row e = w
#pragma unroll
    for (int q = 1; q < KW; ++q) sum += red[(q * 4 + w) * 64 + lane];
    const int m = 4 * g + w, n = n0 + r;
    if (m < M && n < N) {
        float b = 0.0f;
        if constexpr ((EPI & TLG_EPI_BIAS) != 0) b = load_elem<IN>(bias, n);
        float v = epilogue<EPI>(sum, b);
        if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
        store_out<OUT>(Y, (int64_t)m * N + n, v);
    }
}

template <int I, int NB, int KW, int LOADS, bool PIPE, int RBF>
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
                if constexpr (!StreamGeom<I, NB, KW, LOADS, RB, PIPE>::FITS) {
                    set_error("stream configuration does not fit in LDS for M=%lld", (long long)p.M);
                    return TLG_ERR_UNSUPPORTED;
                } else {
                    hipLaunchKernelGGL((stream_kernel<I, O, E, NB, KW, LOADS, RB, decltype(ev)::value,
                                                      decltype(sp)::value, PIPE>),
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
            if constexpr (RBF != 0) {  // the option fixes the row blocks: one instantiation
                if (p.rowb != RBF) {
                    set_error("stream configuration takes %d-row blocks of X, the plan has %d", 16 * RBF, 16 * p.rowb);
                    return (int)TLG_ERR_INVALID_ARG;
                }
                return by_even(ic<RBF>{});
            } else {
                if (p.rowb == 1) return by_even(ic<1>{});
                if (p.rowb == 2) return by_even(ic<2>{});
                return by_even(ic<4>{});
            }
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
    static_assert(kNumStream == 15 && kStream[5].dl, "stream configurations changed");
#define TLG_STREAM_CASE(i)                                                                                     \
    case i:                                                                                                     \
        return launch_stream_cfg<I, kStream[i].nb, kStream[i].kw, kStream[i].loads, kStream[i].pipe != 0,      \
                                 kStream[i].rb>(p, X, W, bias, Y, ws, stream);
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
        TLG_STREAM_CASE(10)
        TLG_STREAM_CASE(11)
        TLG_STREAM_CASE(12)
        TLG_STREAM_CASE(13)
        TLG_STREAM_CASE(14)
    default: set_error("bad stream tile"); return (int)TLG_ERR_INVALID_ARG;
    }
#undef TLG_STREAM_CASE
}

}  // namespace tlg
