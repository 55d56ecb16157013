// LDS-tiled MFMA kernel for the compute-bound shapes (square GEMM, the
// batched GPT-2 stack) and, with split-K, the 128-row GPT-2 layers.
//
// The ladder of "Writing a CUDA matmul that catches cuBLAS" (block tiling,
// register/warp tiling, double buffering in "Kernel 8: the loop was shaped
// wrong", matrix-core fragments in "Kernel 9"/"Kernel 10") rebuilt for gfx950:
//
//  * A workgroup computes a BM×BN tile with WM×WN waves; each wave owns a
//    (BM/WM)×(BN/WN) block of 32×32 MFMA accumulators (fp32:
//    v_mfma_f32_32x32x2_f32; fp16/bf16: v_mfma_f32_32x32x16_*).
//  * K advances in slices of BK (64 to 256 bytes of each operand row),
//    fetched with 16-byte loads into registers two slices ahead of the one
//    being multiplied from LDS; two LDS buffers, one barrier per slice.
//    With one wave per SIMD nothing else hides the issue time of those
//    loads and of the LDS stores, so both are spread between the MFMAs of
//    the current slice (scheduling group barriers), and exact-fit tiles load
//    through buffer descriptors: one lane offset per operand instead of a
//    64-bit address per load, which keeps the loop free of register spills.
//  * Tiles that list a stage count (16-bit [M][K]·[N][K] operands, exact
//    fit) skip the registers: global_load_lds_dwordx4 writes each slice
//    straight into one of that many LDS buffers, unpadded and swizzled, with
//    no LDS stores and no staging registers; waits on the vector-memory
//    counter and one barrier per slice order the buffers.
//  * Tiles marked persistent run one workgroup per resident slot, each
//    walking tiles b, b + grid, ...; the last phases of a tile load the next
//    tile's first slices, so its start overlaps this tile's end.
//  * LDS rows are k-contiguous with a 16-byte pad (stride 80 B), so the
//    16-byte operand reads of 16 consecutive rows hit 64 distinct banks.
//    A [K][N] weight or [K][M] first operand is stored to LDS as it lies in
//    memory, n- or m-contiguous.  fp32 fragments are then gathered with
//    scalar reads (stride BN+8 floats, so the two half-waves read disjoint
//    bank halves); 16-bit fragments with two LDS transpose reads of four k
//    rows each (stride BN+32 elements, 16 dwords mod 64 banks, so the four
//    rows of one read fall in disjoint banks).
//  * For fp32 one 16-byte read feeds four MFMAs; the k order inside a slice
//    is permuted identically for both operands, which leaves each dot
//    product unchanged.
//  * Workgroup ids are remapped so that tiles sharing operand panels run on
//    one XCD (ids are dealt to the 8 XCDs round-robin, each with its own L2),
//    then grouped 8 tile-rows at a time.
//  * Split-K ("Optimizing a GPT-2-class transformer on a GPU", Act I): grid
//    dimension y splits K; each split writes fp32 partials to the workspace
//    and a second kernel sums them in split order (fixed order, so results
//    are reproducible) and applies the epilogue.

#pragma once
#include "common.h"

namespace tlg {

// Waves per SIMD the register allocation must allow: a wave tile of up to
// 64×64 (64 accumulator registers) leaves room for two waves, up to 32×32 for
// four, so LDS rather than registers limits how many workgroups share a CU.
template <int BM, int BN, int WM, int WN>
constexpr int tiled_occupancy() {
    constexpr int acc = (BM / WM) * (BN / WN) / 64;
    return acc <= 16 ? 4 : acc <= 64 ? 2 : 1;
}

// Static LDS of one workgroup: two buffers of each operand tile (the arrays
// the kernel declares; the padded row lengths are the kernel's), or ST
// unpadded, swizzled buffers when the operands are loaded straight into LDS.
template <int IN, int LAYOUT, int BM, int BN, int BK, int ST = 0>
constexpr int tiled_lds_bytes() {
    constexpr bool f32 = IN == TLG_F32;
    constexpr int es = f32 ? 4 : 2, epv = 16 / es;
    if constexpr (ST > 0) return ST * (BM + BN) * BK * es;
    constexpr int a = layout_a_transposed(LAYOUT) ? BK * (BM + (f32 ? 8 : 32)) : BM * (BK + epv);
    constexpr int b = layout_b_kn(LAYOUT) ? BK * (BN + (f32 ? 8 : 32)) : BN * (BK + epv);
    return 2 * (a + b) * es;
}

// Workgroups per CU the launch bound asks the register allocation to allow:
// the register rule above, raised to two for direct-load tiles whose LDS
// leaves room for a second workgroup (128×192×64: 80 KiB).  Without the bound
// the compiler may take more than half the register file for such a tile, and
// the second workgroup the LDS admits would not fit (bf16 8192-row qkv and fc
// measured 0.8–1.2 % faster with it).
template <int IN, int LAYOUT, int BM, int BN, int BK, int WM, int WN, int ST>
constexpr int tiled_min_groups() {
    constexpr int regs = tiled_occupancy<BM, BN, WM, WN>();
    constexpr bool two = ST > 0 && 2 * tiled_lds_bytes<IN, LAYOUT, BM, BN, BK, ST>() <= 160 * 1024;
    return two && regs < 2 ? 2 : regs;
}

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maxima, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int IN, int OUT, int LAYOUT, uint32_t EPI, int BM, int BN, int BK, int WM, int WN, bool EVEN,
          bool SPLIT, int ST, bool PERS>
__global__ __launch_bounds__(64 * WM * WN, (tiled_min_groups<IN, LAYOUT, BM, BN, BK, WM, WN, ST>())) void tiled_kernel(const void* __restrict__ Xv,
                                                            const void* __restrict__ Wv,
                                                            const void* __restrict__ bias,
                                                            void* __restrict__ Y, float* __restrict__ ws,
                                                            int M, int N, int K, int kper, int resid) {
    using S = typename Elem<IN>::storage;
    constexpr bool F32 = IN == TLG_F32;
    constexpr int THREADS = 64 * WM * WN;
    constexpr int EPV = Elem<IN>::per16;  // elements per 16 bytes
    constexpr int VPR = BK / EPV;         // 16-byte vectors per tile row
    static_assert(BK * (int)sizeof(S) % 64 == 0, "a slice is a multiple of 64 bytes of each operand row");
    constexpr int LDA = BK + EPV;         // padded LDS row (elements)
    constexpr bool KNB = layout_b_kn(LAYOUT);         // weight stored [K][N]
    constexpr bool AT = layout_a_transposed(LAYOUT);  // first operand stored [K][M]
    constexpr bool B_NMAJOR = KNB;                    // [K][N] stays n-contiguous in LDS
    constexpr int LDBN = BN + (F32 ? 8 : 32);         // its padded row (elements)
    constexpr bool A_MMAJOR = AT;                     // [K][M] stays m-contiguous in LDS
    constexpr int LDAM = BM + (F32 ? 8 : 32);         // its padded row (elements)
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is a multiple of 32×32");
    constexpr int MV = BM / EPV, NV = BN / EPV;  // 16-byte vectors per [K][M] / [K][N] row of the tile
    constexpr int AV = A_MMAJOR ? BK * MV / THREADS : BM * VPR / THREADS;
    constexpr int BV = !KNB ? BN * VPR / THREADS : BK * NV / THREADS;
    static_assert(AV >= 1 && BV >= 1, "every thread loads");
    static_assert(AV * THREADS == (A_MMAJOR ? BK * MV : BM * VPR), "A loads divide evenly");
    static_assert(BV * THREADS == (KNB ? BK * NV : BN * VPR), "weight loads divide evenly");
    // ST > 0: operands go from memory straight into LDS (global_load_lds,
    // no staging registers, no LDS stores) through ST buffers.
    constexpr bool DL = ST > 0;
    static_assert(!DL || (!F32 && !AT && !KNB && EVEN && ST >= 2 && ST <= 4),
                  "direct loads: 16-bit, exact fit, both operands k-contiguous");
    constexpr int A_ELEMS = DL ? BM * BK : A_MMAJOR ? BK * LDAM : BM * LDA;
    constexpr int B_ELEMS = DL ? BN * BK : B_NMAJOR ? BK * LDBN : BN * LDA;
    static_assert((DL ? ST : 2) * (A_ELEMS + B_ELEMS) * (int)sizeof(S) ==
                      tiled_lds_bytes<IN, LAYOUT, BM, BN, BK, ST>(),
                  "the launcher's LDS figure matches the arrays");

    // One LDS array per operand and buffer: separate objects, so the compiler
    // sees that stores (or direct loads) into one buffer never alias operand
    // reads from another, and every access lies within 64 KiB of its
    // operand's base (the reach of the DS offset field).
    __shared__ __attribute__((aligned(16))) S lds_a0[A_ELEMS];
    __shared__ __attribute__((aligned(16))) S lds_a1[A_ELEMS];
    __shared__ __attribute__((aligned(16))) S lds_b0[B_ELEMS];
    __shared__ __attribute__((aligned(16))) S lds_b1[B_ELEMS];
    __shared__ __attribute__((aligned(16))) S lds_a2[ST > 2 ? A_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S lds_b2[ST > 2 ? B_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S lds_a3[ST > 3 ? A_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) S lds_b3[ST > 3 ? B_ELEMS : 8];
    auto abuf = [&](int b) -> S* { return b == 0 ? lds_a0 : b == 1 ? lds_a1 : b == 2 ? lds_a2 : lds_a3; };
    auto bbuf = [&](int b) -> S* { return b == 0 ? lds_b0 : b == 1 ? lds_b1 : b == 2 ? lds_b2 : lds_b3; };

    const S* __restrict__ X = static_cast<const S*>(Xv);
    const S* __restrict__ W = static_cast<const S*>(Wv);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int r = lane & 31, g = lane >> 5;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    // ---- tile coordinates: XCD-aware remap, then groups of 8 tile-rows ----
    const int gx = (N + BN - 1) / BN, gy = (M + BM - 1) / BM;
    const int total = gx * gy;
    constexpr int GROUP = 8;
    auto tile_origin = [&](int id, int& tm0, int& tn0) {
        int lin = id;
        if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
        const int group_tiles = GROUP * gx;
        const int first = (lin / group_tiles) * GROUP;
        const int rows_in_group = min(gy - first, GROUP);
        const int within = lin % group_tiles;
        tm0 = (first + within % rows_in_group) * BM;
        tn0 = (within / rows_in_group) * BN;
    };
    int m0, n0;  // this tile's origin (a persistent workgroup moves on to further tiles)
    tile_origin(blockIdx.x, m0, n0);

    const int z = blockIdx.y;
    const int kbeg = z * kper;
    const int kend = min(kbeg + kper, K);
    const int nslices = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    // EVEN (exact-fit tiles, every operand region below 2 GiB, checked by the
    // host) loads through buffer descriptors: a uniform base per operand tile
    // plus one 32-bit lane offset, the per-load offsets uniform.
    constexpr int ES = (int)sizeof(S);
    static_assert(THREADS % VPR == 0 && (!B_NMAJOR || THREADS % NV == 0) && (!A_MMAJOR || THREADS % MV == 0),
                  "each thread's loads share one lane offset");
    const uint32_t a_lane = A_MMAJOR ? (uint32_t)(((t / MV) * M + (t % MV) * EPV) * ES)
                                     : (uint32_t)(((t / VPR) * K + (t % VPR) * EPV) * ES);
    const uint32_t b_lane = !KNB ? (uint32_t)(((t / VPR) * K + (t % VPR) * EPV) * ES)
                                 : (uint32_t)(((t / NV) * N + (t % NV) * EPV) * ES);
    i32x4 rsrc_a = {0, 0, 0, 0}, rsrc_b = {0, 0, 0, 0};
    auto make_rsrc = [&](int tm0, int tn0, i32x4& qa, i32x4& qb) {
        qa = AT ? buffer_rsrc(X + tm0, ((int64_t)K * M - tm0) * ES) : buffer_rsrc(X + (int64_t)tm0 * K, (int64_t)BM * K * ES);
        qb = KNB ? buffer_rsrc(W + tn0, ((int64_t)K * N - tn0) * ES) : buffer_rsrc(W + (int64_t)tn0 * K, (int64_t)BN * K * ES);
    };
    if constexpr (EVEN) make_rsrc(m0, n0, rsrc_a, rsrc_b);
    // The next tile's descriptors (persistent loop): slice index s >= nslices
    // loads slice s - nslices of that tile.
    i32x4 nrsrc_a = rsrc_a, nrsrc_b = rsrc_b;
    auto gload = [&](int s, u32x4 (&ra)[AV], u32x4 (&rbv)[BV]) {
        if constexpr (EVEN) {
            i32x4 qa = rsrc_a, qb = rsrc_b;
            if constexpr (PERS) {
                if (s >= nslices) {
                    s -= nslices;
                    qa = nrsrc_a;
                    qb = nrsrc_b;
                }
            }
            const int k0 = kbeg + s * BK;
#pragma unroll
            for (int i = 0; i < AV; ++i) {
                if constexpr (A_MMAJOR)
                    ra[i] = buffer_load16(qa, a_lane, (k0 + i * (THREADS / MV)) * M * ES, 0);
                else
                    ra[i] = buffer_load16(qa, a_lane, (k0 + i * (THREADS / VPR) * K) * ES, 0);
            }
#pragma unroll
            for (int i = 0; i < BV; ++i) {
                if constexpr (!KNB)
                    rbv[i] = buffer_load16(qb, b_lane, (k0 + i * (THREADS / VPR) * K) * ES, 0);
                else
                    rbv[i] = buffer_load16(qb, b_lane, (k0 + i * (THREADS / NV)) * N * ES, 0);
            }
            return;
        }
        const int k0 = kbeg + s * BK;
        // Ragged tiles: out-of-range rows and columns are clamped to valid
        // ones (their outputs are never stored), K past the range loads zeros.
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int v = t + THREADS * i;
            if constexpr (A_MMAJOR) {
                const int kr = v / MV, mv = v % MV;
                const int k = k0 + kr;
                const int m = min(m0 + mv * EPV, M - EPV);
                if (k < kend)
                    ra[i] = ldg16(X + (int64_t)k * M + m);
                else
                    ra[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                const int row = v / VPR, k = k0 + (v % VPR) * EPV;
                const int m = min(m0 + row, M - 1);
                if (k < kend)
                    ra[i] = ldg16(X + (int64_t)m * K + k);
                else
                    ra[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int v = t + THREADS * i;
            if constexpr (!KNB) {
                const int row = v / VPR, k = k0 + (v % VPR) * EPV;
                const int n = EVEN ? n0 + row : min(n0 + row, N - 1);
                if (EVEN || k < kend)
                    rbv[i] = ldg16(W + (int64_t)n * K + k);
                else
                    rbv[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                const int kr = v / NV, nv = v % NV;
                const int k = k0 + kr;
                const int n = EVEN ? n0 + nv * EPV : min(n0 + nv * EPV, N - EPV);
                if (EVEN || k < kend)
                    rbv[i] = ldg16(W + (int64_t)k * N + n);
                else
                    rbv[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto lstore = [&](int buf, const u32x4 (&ra)[AV], const u32x4 (&rbv)[BV]) {
        S* As = buf ? lds_a1 : lds_a0;
        S* Bs = buf ? lds_b1 : lds_b0;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int v = t + THREADS * i;
            if constexpr (A_MMAJOR) {
                *reinterpret_cast<u32x4*>(As + (v / MV) * LDAM + (v % MV) * EPV) = ra[i];
            } else {
                *reinterpret_cast<u32x4*>(As + (v / VPR) * LDA + (v % VPR) * EPV) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int v = t + THREADS * i;
            if constexpr (!KNB) {
                *reinterpret_cast<u32x4*>(Bs + (v / VPR) * LDA + (v % VPR) * EPV) = rbv[i];
            } else {
                *reinterpret_cast<u32x4*>(Bs + (v / NV) * LDBN + (v % NV) * EPV) = rbv[i];
            }
        }
    };

    // ---- direct loads into swizzled, unpadded LDS tiles ----
    // One global_load_lds_dwordx4 of a wave fills 1 KiB of LDS: lane l lands
    // at base + 16·l, the base being the same for all lanes, so the layout is
    // set by which memory each lane fetches.  A k-contiguous tile (rows of
    // VPR 16-byte chunks) keeps logical chunk c of row R at chunk position
    // c ^ ((R / RPB) % VPR), RPB = 16 / VPR rows per 256 bytes: the operand
    // reads of 16 consecutive rows at one chunk then hit 64 distinct banks, as
    // the padded rows of the staged path do.  Instruction q of an operand
    // fills its bytes [1 KiB·q, 1 KiB·(q+1)); wave w issues q = w, w + WAVES,
    // ...  The swizzle repeats every 4·WAVES·RPB rows, so each lane's fetch
    // offset is the same in all of its instructions up to a uniform row step
    // and is computed once.  (The transposed fragment reads of a [K][N]
    // weight are library intrinsics without alias information, before which
    // the compiler waits for every outstanding direct load; such tiles keep
    // the staged path.)
    constexpr int WAVES = WM * WN;
    constexpr int RPB = VPR <= 16 ? 16 / VPR : 1;
    uint32_t dl_off = 0;  // element offset of this lane's first fetch within either operand tile
    if constexpr (DL) {
        static_assert(VPR <= 16 && (4 * WAVES) % VPR == 0 && 64 % VPR == 0, "k-contiguous swizzle repeats per wave");
        static_assert((BM * VPR) % (64 * WAVES) == 0 && (BN * VPR) % (64 * WAVES) == 0, "whole instructions per wave");
        const int R = (64 / VPR) * wave + lane / VPR;
        dl_off = (uint32_t)(R * K + EPV * ((lane % VPR) ^ ((R / RPB) % VPR)));
    }
    constexpr int AQ = BM * VPR / (64 * WAVES);  // direct loads per wave per slice: first operand
    constexpr int BQ = BN * VPR / (64 * WAVES);  // and the weight
    int nm0 = 0, nn0 = 0;  // the next tile's origin (persistent loop)
    auto dload = [&](int s, int buf) {
        int tm0 = m0, tn0 = n0;
        if constexpr (PERS) {
            if (s >= nslices) {  // slice s - nslices of the next tile
                s -= nslices;
                tm0 = nm0;
                tn0 = nn0;
            }
        }
        const int k0 = kbeg + s * BK;
        const S* xa = X + (int64_t)tm0 * K + k0 + dl_off;
        const S* wb = W + (int64_t)tn0 * K + k0 + dl_off;
        S* As = abuf(buf);
        S* Bs = bbuf(buf);
        constexpr int64_t step = (int64_t)(64 / VPR) * WAVES;  // rows between a wave's instructions
#pragma unroll
        for (int i = 0; i < AQ; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xa + i * step * K),
                                             (__attribute__((address_space(3))) void*)(As + (wave + WAVES * i) * 512),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < BQ; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(wb + i * step * K),
                                             (__attribute__((address_space(3))) void*)(Bs + (wave + WAVES * i) * 512),
                                             16, 0, 0);
    };

    using Acc = f32x16;
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto compute = [&](int buf, auto mid) {
        const S* As = abuf(buf);
        const S* Bs = bbuf(buf);
        if constexpr (F32) {
#pragma unroll
            for (int kq = 0; kq < BK / 8; ++kq) {
                f32x4 a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if constexpr (A_MMAJOR) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            a[i][e] = As[(kq * 8 + 4 * g + e) * LDAM + wm0 + i * 32 + r];
                    } else {
                        a[i] = *reinterpret_cast<const f32x4*>(As + (wm0 + i * 32 + r) * LDA + kq * 8 + 4 * g);
                    }
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (B_NMAJOR) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            b[j][e] = Bs[(kq * 8 + 4 * g + e) * LDBN + wn0 + j * 32 + r];
                    } else {
                        b[j] = *reinterpret_cast<const f32x4*>(Bs + (wn0 + j * 32 + r) * LDA + kq * 8 + 4 * g);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32_f32(a[i][e], b[j][e], acc[i][j]);
                if (kq == (BK / 8) / 2 - 1) mid();
            }
        } else {
            // Operand fragments for k-step kq+1 are read from LDS while the
            // MFMAs of k-step kq issue, so LDS latency overlaps the math.  A
            // fragment of an m- or n-contiguous tile (lane: row r, k = 8g..8g+7)
            // is two transpose reads: lane L names row 8g + (L%16)/4 (+4 for
            // the second read) and column 16·((L/16)%2) + 4·(L%4) of the
            // 32-wide block, and receives column r of k rows 8g..8g+3 (+4).
            constexpr int KQ = BK / 16;
            u32x4 a[2][TM], b[2][TN];
            const int tr_row = 8 * g + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            auto tr_frag = [&](const S* p, int ld) {
                const u32x2 lo = lds_read_tr16(p + tr_row * ld + tr_col);
                const u32x2 hi = lds_read_tr16(p + (tr_row + 4) * ld + tr_col);
                return u32x4{lo[0], lo[1], hi[0], hi[1]};
            };
            // Swizzled tiles (direct loads): this lane's chunk permutation.  Its
            // rows wm0 + 32i + r and wn0 + 32j + r all share r's swizzle.
            const int sw = (r / RPB) % VPR;
            auto frag = [&](int kq, u32x4(&fa)[TM], u32x4(&fb)[TN]) {
                if constexpr (DL) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        fa[i] = *reinterpret_cast<const u32x4*>(As + (wm0 + i * 32 + r) * BK + EPV * ((2 * kq + g) ^ sw));
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        fb[j] = *reinterpret_cast<const u32x4*>(Bs + (wn0 + j * 32 + r) * BK + EPV * ((2 * kq + g) ^ sw));
                    return;
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if constexpr (A_MMAJOR)
                        fa[i] = tr_frag(As + kq * 16 * LDAM + wm0 + i * 32, LDAM);
                    else
                        fa[i] = *reinterpret_cast<const u32x4*>(As + (wm0 + i * 32 + r) * LDA + kq * 16 + 8 * g);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (B_NMAJOR)
                        fb[j] = tr_frag(Bs + kq * 16 * LDBN + wn0 + j * 32, LDBN);
                    else
                        fb[j] = *reinterpret_cast<const u32x4*>(Bs + (wn0 + j * 32 + r) * LDA + kq * 16 + 8 * g);
                }
            };
            frag(0, a[0], b[0]);
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                if (kq + 1 < KQ) frag(kq + 1, a[(kq + 1) & 1], b[(kq + 1) & 1]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma32_16bit<IN>(a[kq & 1][i], b[kq & 1][j], acc[i][j]);
                if (kq == KQ / 2 - 1) mid();
            }
        }
    };

    // Issue order of one phase (one slice multiplied from LDS while the next
    // is stored to the other buffer and the one after is loaded): the first
    // k-step's operand reads, then every MFMA followed by its share of the
    // other work — the global loads over the first half of the MFMAs, the next
    // k-step's operand reads inside each k-step, and the LDS stores over the
    // second half.  Whole phase as one scheduling region for 16-bit inputs; fp32
    // splits it at the middle k-step (measured: 2803 vs 3809 cycles per
    // 256×256×64 bf16 slice, 8481 vs 8564 per 256×256×16 fp32 slice).
    constexpr int NKQ = F32 ? BK / 8 : BK / 16;
    constexpr int FR = (A_MMAJOR ? (F32 ? 4 : 2) : 1) * TM + (B_NMAJOR ? (F32 ? 4 : 2) : 1) * TN;
    constexpr int NMF = F32 ? NKQ * 4 * TM * TN : NKQ * TM * TN;
    constexpr int MPK = NMF / NKQ, HALF = NMF / 2;
    constexpr int NVM = AV + BV, NDW = AV + BV;
    constexpr int SV = HALF / NVM > 0 ? HALF / NVM : 1;
    constexpr int SR = MPK / FR > 0 ? MPK / FR : 1;
    constexpr int SW = HALF / NDW > 0 ? HALF / NDW : 1;
    // 16-bit tiles whose last k-step has an MFMA for every LDS store keep the
    // stores out of the earlier k-steps: LDS operations complete in order, so
    // a fragment read issued after a store cannot be waited for without the
    // store, and stores mixed into the k-steps that still read fragments
    // stall their MFMAs.  (Square bf16 256×256×64: 2-3 % faster.)  Other
    // tiles spread the stores over the second half of the MFMAs.
    constexpr bool LATE_ST = !F32 && NDW <= MPK;
    constexpr int ST0 = LATE_ST ? (NKQ - 1) * MPK : HALF, SW0 = LATE_ST ? MPK / NDW : SW;
    auto slot = [&](int m, bool loads, bool stores) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (loads && m % SV == 0 && m / SV < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (m / MPK < NKQ - 1 && (m % MPK) % SR == 0 && (m % MPK) / SR < FR)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next k-step's operand read
        if (stores && m >= ST0 && (m - ST0) % SW0 == 0 && (m - ST0) / SW0 < NDW)
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS stores: A's first, then the weight's
    };
    auto whole_phase = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
#pragma unroll
        for (int m = 0; m < NMF; ++m) slot(m, true, true);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto first_half = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
#pragma unroll
        for (int m = 0; m < HALF; ++m) slot(m, true, false);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto second_half = [&]() {
#pragma unroll
        for (int m = HALF; m < NMF; ++m) slot(m, false, true);
        __builtin_amdgcn_sched_barrier(0);
    };
    // Direct-load phase: no LDS stores; the next slices' loads over the first
    // half of the MFMAs.
    auto dl_phase = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
#pragma unroll
        for (int m = 0; m < NMF; ++m) slot(m, true, false);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto nothing = [] {};
    // One steady-state phase: multiply buffer cb, store `st` into the other
    // buffer, load slice ls into `ld`.
    auto phase = [&](int cb, int ls, u32x4 (&lda)[AV], u32x4 (&ldb)[BV], const u32x4 (&sta)[AV],
                     const u32x4 (&stb)[BV]) {
        gload(ls, lda, ldb);
        if constexpr (F32) {
            compute(cb, first_half);
            lstore(cb ^ 1, sta, stb);
            second_half();
        } else {
            compute(cb, nothing);
            lstore(cb ^ 1, sta, stb);
            whole_phase();
        }
    };

    // ---- epilogue: a 32×32 accumulator holds column (lane % 32) and rows
    // 8*(e/4) + 4*(lane/32) + e%4 for register e.
    // Exact-fit tiles leave through LDS: each wave stages 16 rows × WTN of its
    // tile (fp32, row stride WTN+8 floats, so the two half-waves' writes land
    // on disjoint banks), then every lane takes whole 16-byte runs of one row,
    // applies bias, GELU and the residual, converts and stores them: full-line
    // writes and one store per 16 bytes instead of one per element.  The
    // operand buffers are free once every wave is past its last multiply:
    // each wave takes a strip of its own from them; where the four arrays
    // hold fewer strips than there are waves, the per-element path below.
    constexpr int SROW = WTN + 8;  // staged row stride (floats)
    constexpr int STG = 16 * SROW;
    // Strips of STG floats that fit in each operand array; wave w takes strip
    // w of a0, a1, b0, b1 in turn.
    constexpr int SA = A_ELEMS * (int)sizeof(S) / (STG * 4), SB = B_ELEMS * (int)sizeof(S) / (STG * 4);
    constexpr bool STAGED = 2 * SA + 2 * SB >= WM * WN;
    constexpr int OB = SPLIT ? 4 : (OUT == TLG_F32 ? 4 : 2);  // bytes per written element
    constexpr int EPC = 16 / OB;                               // elements per 16-byte store
    constexpr int CPR = WTN / EPC;                             // 16-byte runs per staged row
    // Stage the accumulators through this wave's strip stg, then apply bias,
    // GELU and the residual and store (generic, so that it is instantiated
    // only where it is used).  A half-strip holds 16·CPR runs.  Where CPR
    // divides 64 a lane keeps one column set for all its runs (bias loaded
    // once); otherwise (wave tiles 96 or 192 columns wide) the lanes take
    // runs 64 apart with a guard on the last round, and each run's columns
    // and bias are its own.
    constexpr bool EVEN_RUNS = 64 % CPR == 0 && (16 * CPR) % 64 == 0;
    constexpr int NRUN = (16 * CPR + 63) / 64;
    auto store_staged = [&](auto* stg) {
        // Opaque copy of the lane index: everything the epilogue derives from
        // it is computed here, after the loop, instead of being hoisted in
        // front of it and held in registers through it (which spilled the
        // 256×256 bf16 loop once the residual read was added).
        int el = lane;
        asm volatile("" : "+v"(el));
        const int col = (el % CPR) * EPC;  // the same columns for every run of this lane
        // Bias of each of this lane's runs, one vector load per run: a lane's
        // runs sit at the same columns in every 16-row half-strip.
        constexpr int NB = EVEN_RUNS ? 1 : NRUN;
        float bq[NB][EPC];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            if constexpr (!SPLIT && (EPI & TLG_EPI_BIAS) != 0)
                load_bias_run<IN, EPC>(bias, n0 + wn0 + (EVEN_RUNS ? col : ((el + 64 * q) % CPR) * EPC), bq[q]);
            else
#pragma unroll
                for (int u = 0; u < EPC; ++u) bq[q][u] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 8 * h; e < 8 * h + 8; ++e)
                        stg[(8 * ((e >> 2) & 1) + 4 * g + (e & 3)) * SROW + j * 32 + r] = acc[i][j][e];
                // LDS operations of one wave complete in order: the reads
                // below see these writes, and the next half's writes follow them.
#pragma unroll
                for (int q = 0; q < NRUN; ++q) {
                    const int run = el + 64 * q;
                    if (!EVEN_RUNS && run >= 16 * CPR) break;
                    const int row = run / CPR;
                    const int rcol = EVEN_RUNS ? col : (run % CPR) * EPC;  // this run's first column in the strip
                    const int nrun = n0 + wn0 + rcol;
                    const float* brun = bq[EVEN_RUNS ? 0 : q];
                    const float* src = stg + row * SROW + rcol;
                    float v[EPC];
#pragma unroll
                    for (int u = 0; u < EPC; u += 4) {
                        const f32x4 x = *reinterpret_cast<const f32x4*>(src + u);
                        v[u] = x[0], v[u + 1] = x[1], v[u + 2] = x[2], v[u + 3] = x[3];
                    }
                    const int64_t m = m0 + wm0 + i * 32 + 16 * h + row;
                    u32x4 out;
                    if constexpr (SPLIT) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) out[u] = __float_as_uint(v[u]);
                        *reinterpret_cast<u32x4*>(ws + ((int64_t)z * M + m) * N + nrun) = out;
                    } else {
#pragma unroll
                        for (int u = 0; u < EPC; ++u) v[u] = epilogue<EPI>(v[u], brun[u]);
                        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(Y) + (m * N + nrun) * OB);
                        if (resid) {
                            float rv[EPC];
                            unpack16<OUT>(*dst, rv);
#pragma unroll
                            for (int u = 0; u < EPC; ++u) v[u] += rv[u];
                        }
                        out = pack16<OUT>(v);
                        *dst = out;
                    }
                }
            }
        }
    };

    // Per-element epilogue: ragged tiles, and persistent tiles whose free LDS
    // buffer holds fewer staging strips than there are waves.
    auto store_direct = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn0 + j * 32 + r;
                float b = 0.0f;
                if constexpr (!SPLIT && (EPI & TLG_EPI_BIAS) != 0)
                    if (n < N) b = load_elem<IN>(bias, n);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + wm0 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    if (m >= M || n >= N) continue;
                    if constexpr (SPLIT) {
                        ws[((int64_t)z * M + m) * N + n] = acc[i][j][e];
                    } else {
                        float v = epilogue<EPI>(acc[i][j][e], b);
                        if (resid) v += load_elem<OUT>(Y, (int64_t)m * N + n);
                        store_out<OUT>(Y, (int64_t)m * N + n, v);
                    }
                }
            }
        }
    };

    if constexpr (PERS) {
        // Persistent workgroup: tiles blockIdx.x, blockIdx.x + gridDim.x, ...
        // (the host sizes the grid to the workgroups resident at once).  The
        // slice pipeline runs on across tiles: the last phases of a tile load
        // the next tile's first two slices, and the finished tile leaves
        // through the LDS buffer its last slice was read from while the next
        // tile's first slice waits in the other.  The host guarantees an even
        // slice count, so a tile always ends after the second phase of a pair.
        static_assert(EVEN && !SPLIT && (ST == 0 || ST == 2), "persistent tiles: exact fit, no split, two buffers");
        const int last = nslices - 1;
        u32x4 ra0[AV], rb0[BV], ra1[AV], rb1[BV];
        if constexpr (DL) {
            dload(0, 0);
        } else {
            gload(0, ra0, rb0);
            gload(1, ra1, rb1);
            lstore(0, ra0, rb0);
            __syncthreads();
        }
        for (int tile = blockIdx.x;;) {
            const int next = tile + (int)gridDim.x;
            const bool more = next < total;
            nm0 = m0;
            nn0 = n0;
            if (more) {
                tile_origin(next, nm0, nn0);
                if constexpr (!DL) make_rsrc(nm0, nn0, nrsrc_a, nrsrc_b);
            }
            // slice j <= last of this tile; past it slice j - nslices of the next
            // tile, or this tile's last slice again when there is none
            auto src = [&](int j) { return j <= last || more ? j : last; };
            if constexpr (DL) {
                // buffer 0 holds (or is receiving) slice s, as in the direct-load loop below
                for (int s = 0; s < nslices; s += 2) {
                    wait_vmcnt<0>();
                    __syncthreads();
                    dload(src(s + 1), 1);
                    compute(0, nothing);
                    dl_phase();
                    wait_vmcnt<0>();
                    __syncthreads();
                    dload(src(s + 2), 0);
                    compute(1, nothing);
                    dl_phase();
                }
                __syncthreads();  // every wave is past its reads of buffer 1
            } else {
                for (int s = 0; s < nslices; s += 2) {
                    phase(0, src(s + 2), ra0, rb0, ra1, rb1);
                    __syncthreads();
                    phase(1, src(s + 3), ra1, rb1, ra0, rb0);
                    __syncthreads();
                }
            }
            if constexpr (SA + SB >= WM * WN)  // every wave's strip in the buffer the last slice freed
                store_staged(wave < SA ? reinterpret_cast<float*>(lds_a1) + wave * STG
                                       : reinterpret_cast<float*>(lds_b1) + (wave - SA) * STG);
            else
                store_direct();
            __syncthreads();  // staging read back before the next tile's slice 1 is stored to buffer 1
            if (!more) {
                if constexpr (DL) wait_vmcnt<0>();  // the last re-read has landed before the workgroup ends
                break;
            }
            tile = next;
            m0 = nm0;
            n0 = nn0;
            rsrc_a = nrsrc_a;
            rsrc_b = nrsrc_b;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        }
        return;
    }

    // Two slices of loads in flight: while slice s is multiplied from one LDS
    // buffer, slice s+1 waits in registers for the other buffer and slice s+2
    // is being fetched.  The loop is unrolled by two so each register set is
    // named statically.  Buffer b is rewritten only after the barrier that
    // follows its last read.
    // Every compute and load in the loop is unconditional, which keeps the
    // accumulators in place across iterations and lets each wait cover only
    // the slice about to be stored.  The loop runs over every pair of slices;
    // prefetches past the last slice re-read the last one (an L2 hit; the
    // copy lands in a buffer nothing reads), so no tail code with its own
    // register allocation follows the loop: an odd count leaves one multiply.
    if constexpr (DL) {
        // ST-1 slices in flight ahead of the one being multiplied; buffer
        // s % ST holds slice s.  Unrolled by ST so that every buffer is named
        // statically (the host guarantees a slice count that is a positive
        // multiple of ST).  Before slice s is read, this wave waits for its
        // own loads of it, and the barrier that follows covers every wave's
        // loads and frees the buffer read one step earlier, which the next
        // load then refills.  Prefetches past the last slice re-read it into
        // a buffer nothing reads again.
        constexpr int LPW = AQ + BQ;
        if (nslices > 0) {
            const int last = nslices - 1;
#pragma unroll
            for (int q = 0; q < ST - 1; ++q) dload(min(q, last), q);
            for (int s = 0; s < nslices; s += ST) {
#pragma unroll
                for (int u = 0; u < ST; ++u) {
                    wait_vmcnt<(ST - 2) * LPW>();
                    __syncthreads();
                    dload(min(s + u + ST - 1, last), (u + ST - 1) % ST);
                    compute(u, nothing);
                    dl_phase();
                }
            }
            wait_vmcnt<0>();  // the re-reads have landed before the LDS is reused below
        }
    } else if (nslices > 0) {
        u32x4 ra0[AV], rb0[BV], ra1[AV], rb1[BV];
        const int last = nslices - 1;
        gload(0, ra0, rb0);
        gload(min(1, last), ra1, rb1);
        lstore(0, ra0, rb0);
        __syncthreads();
        // At the top of each pair: buffer 0 holds slice s, ra1 slice s+1.
        int s = 0;
        for (; s + 1 < nslices; s += 2) {
            phase(0, min(s + 2, last), ra0, rb0, ra1, rb1);  // multiply s, store s+1, load s+2
            __syncthreads();
            phase(1, min(s + 3, last), ra1, rb1, ra0, rb0);  // multiply s+1, store s+2, load s+3
            __syncthreads();
        }
        if (s < nslices) compute(0, nothing);  // odd count: the last slice is in buffer 0
    }

    if constexpr (EVEN && STAGED) {
        __syncthreads();
        float* stg = wave < SA           ? reinterpret_cast<float*>(lds_a0) + wave * STG
                     : wave < 2 * SA       ? reinterpret_cast<float*>(lds_a1) + (wave - SA) * STG
                     : wave < 2 * SA + SB  ? reinterpret_cast<float*>(lds_b0) + (wave - 2 * SA) * STG
                                           : reinterpret_cast<float*>(lds_b1) + (wave - 2 * SA - SB) * STG;
        store_staged(stg);
        return;
    }
    // ---- per-element epilogue (ragged tiles) ----
    store_direct();
}

// Sum the split partials in split order, then the epilogue.  Four outputs per thread.
template <int IN, int OUT, uint32_t EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits,
                                                           const void* __restrict__ bias,
                                                           void* __restrict__ Y, int64_t MN, int N, int resid) {
    const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (base >= MN) return;
    // Every split's values in flight at once (in groups of 8), then the sum in split order.
    float v[4][8];
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < splits; z0 += 8) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e][q] = (z0 + q < splits && base + e < MN) ? ws[(int64_t)(z0 + q) * MN + base + e] : 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (z0 + q < splits) s[e] += v[e][q];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t idx = base + e;
        if (idx >= MN) return;
        float b = 0.0f;
        if constexpr ((EPI & TLG_EPI_BIAS) != 0) b = load_elem<IN>(bias, idx % N);
        float y = epilogue<EPI>(s[e], b);
        if (resid) y += load_elem<OUT>(Y, idx);
        store_out<OUT>(Y, idx, y);
    }
}

// A workgroups-per-CU cap is enforced by asking for unused dynamic LDS:
// just past 1/(CAP+1) of the CU's 160 KiB per workgroup.
template <int CAP, int STATIC_LDS>
constexpr int tiled_dyn_lds() {
    constexpr int kLdsPerCu = 160 * 1024, st = STATIC_LDS;
    constexpr int dyn = CAP > 0 && st < kLdsPerCu / (CAP + 1) + 1024 ? kLdsPerCu / (CAP + 1) + 1024 - st : 0;
    static_assert(CAP == 0 || (st + dyn) * CAP <= kLdsPerCu, "the cap still fits CAP workgroups");
    return dyn;
}

// Workgroups of `kernel` resident on the whole device at once (a multiple of
// eight, so that persistent workgroup b keeps XCD b % 8 for all its tiles),
// at most `total`.
static int resident_grid(const void* kernel, int threads, int dyn, int total) {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] <= 0 && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = 0;
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, dyn) != hipSuccess) per = 0;
    int g = (cus[dev] > 0 ? cus[dev] : 1) * (per > 0 ? per : 1);
    if (g >= 8) g &= ~7;
    return g < total ? g : total;
}

template <int I, int O, int L, uint32_t E, int BM, int BN, int BK, int WM, int WN, int CAP, int DLS, int PRS>
static int launch_tiled_cfg(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                            float* ws, hipStream_t stream) {
    constexpr int dyn = tiled_dyn_lds<CAP, tiled_lds_bytes<I, L, BM, BN, BK>()>();
    // Direct loads into LDS where the tile takes them: 16-bit operands, both
    // k-contiguous, exact-fit tiles and a slice count per split that is a
    // multiple of the stage count.
    constexpr int ST = DLS > 0 && I != TLG_F32 && !layout_a_transposed(L) && !layout_b_kn(L) ? DLS : 0;
    constexpr int dyn_dl = ST > 0 ? tiled_dyn_lds<CAP, tiled_lds_bytes<I, L, BM, BN, BK, ST>()>() : 0;
    const int S = p.split;
    const int kper = (int)(ceil_div(ceil_div(p.K, S), BK) * BK);
    const int64_t es = I == TLG_F32 ? 4 : 2;
    // exact-fit tiles address each operand through a 32-bit buffer range
    const bool fits32 = (layout_a_transposed(L) ? p.K * p.M * es : (int64_t)BM * p.K * es) < INT32_MAX &&
                        (layout_b_kn(L) ? p.K * p.N * es : (int64_t)BN * p.K * es) < INT32_MAX;
    const int resid = (p.epi & TLG_EPI_RESIDUAL) != 0;
    const bool even = p.M % BM == 0 && p.N % BN == 0 && (int64_t)kper * S == p.K && fits32;
    // The plan decides (its stage count); the conditions are checked again here.
    const bool direct = p.stages > 0;
    if (direct && (p.stages != ST || !even || (kper / BK) % (ST > 0 ? ST : 1) != 0)) {
        set_error("tiled kernel: plan asks for direct loads the tile cannot take");
        return (int)TLG_ERR_INVALID_ARG;
    }
    const dim3 grid((unsigned)(p.grid_x * p.grid_y), (unsigned)S), block(64 * WM * WN);
    // stc: the direct-load stage count (0: staged loads)
    auto go = [&](auto ev, auto sp, auto stc) {
        constexpr int st = decltype(stc)::value;
        hipLaunchKernelGGL((tiled_kernel<I, O, L, E, BM, BN, BK, WM, WN, decltype(ev)::value, decltype(sp)::value, st,
                                         false>),
                           grid, block, st > 0 ? dyn_dl : dyn, stream, X, W, bias, Y, ws, (int)p.M, (int)p.N, (int)p.K,
                           kper, resid);
        return check_launch("tiled_kernel");
    };
    auto go_split = [&](auto ev, auto stc) {
        constexpr int st = decltype(stc)::value;
        hipLaunchKernelGGL((tiled_kernel<I, TLG_F32, L, 0u, BM, BN, BK, WM, WN, decltype(ev)::value, true, st, false>), grid,
                           block, st > 0 ? dyn_dl : dyn, stream, X, W, nullptr, nullptr, ws, (int)p.M, (int)p.N,
                           (int)p.K, kper, 0);
        return check_launch("tiled_kernel");
    };
    if (p.persist) {
        if constexpr (PRS > 0) {
            if (!even || S != 1 || (kper / BK) % 2 != 0 || kper < 2 * BK || (direct && ST != 2)) {
                set_error("tiled kernel: plan asks for persistent workgroups the shape cannot take");
                return (int)TLG_ERR_INVALID_ARG;
            }
            auto go_persistent = [&](auto stc) {
                constexpr int st = decltype(stc)::value;
                const int d = st > 0 ? dyn_dl : dyn;
                const int G = resident_grid(
                    reinterpret_cast<const void*>(&tiled_kernel<I, O, L, E, BM, BN, BK, WM, WN, true, false, st, true>),
                    64 * WM * WN, d, (int)(p.grid_x * p.grid_y));
                hipLaunchKernelGGL((tiled_kernel<I, O, L, E, BM, BN, BK, WM, WN, true, false, st, true>),
                                   dim3((unsigned)G), block, d, stream, X, W, bias, Y, ws, (int)p.M, (int)p.N, (int)p.K,
                                   kper, resid);
                return check_launch("tiled_kernel");
            };
            if constexpr (ST == 2) {
                if (direct) return go_persistent(ic<2>{});
            }
            return go_persistent(ic<0>{});
        }
        set_error("tiled kernel: persistent workgroups on a tile without them");
        return (int)TLG_ERR_INVALID_ARG;
    }
    int rc;
    if (direct) {
        if constexpr (ST > 0)
            rc = S > 1 ? go_split(std::true_type{}, ic<ST>{}) : go(std::true_type{}, std::false_type{}, ic<ST>{});
        else
            rc = (int)TLG_ERR_UNSUPPORTED;  // not reached: direct implies ST > 0
    } else if (S > 1) {  // partials carry no epilogue: the reducer applies it
        rc = even ? go_split(std::true_type{}, ic<0>{}) : go_split(std::false_type{}, ic<0>{});
    } else {
        rc = even ? go(std::true_type{}, std::false_type{}, ic<0>{}) : go(std::false_type{}, std::false_type{}, ic<0>{});
    }
    if (rc != TLG_OK || S == 1) return rc;
    const int64_t MN = p.M * p.N;
    hipLaunchKernelGGL((splitk_reduce_kernel<I, O, E>), dim3((unsigned)ceil_div(MN, 1024)), dim3(256), 0, stream,
                       (const float*)ws, S, bias, Y, MN, (int)p.N, resid);
    return check_launch("splitk_reduce_kernel");
}


// All launches for one input dtype; explicitly instantiated once per dtype
// in its own translation unit (tiled_f32.hip, tiled_f16.hip, tiled_bf16.hip).
template <int I>
int launch_tiled_in(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y, void* ws,
                    hipStream_t stream) {
    // split partials follow the workspace's counter block, which tiled plans leave untouched
    float* wsf = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + kWsCounterBytes) : nullptr;
    auto with_out = [&](auto f) {
        if constexpr (I == TLG_F32) return f(ic<TLG_F32>{});
        else if (p.out_dt == TLG_F32) return f(ic<TLG_F32>{});
        else return f(ic<I>{});
    };
    return with_out([&](auto out) {
        return with_layout(p.layout, [&](auto lay) {
            auto by_epi = [&](auto epi) {
                constexpr int O = decltype(out)::value, L = decltype(lay)::value;
                constexpr uint32_t E = (uint32_t)decltype(epi)::value;
                constexpr const TileCfg* T = I == TLG_F32 ? kTiledF32 : kTiled16;
                constexpr int count = I == TLG_F32 ? kNumTiledF32 : kNumTiled16;
                static_assert(kNumTiledF32 == 10 && kNumTiled16 == 13, "tile lists changed");
#define TLG_TILED_CASE(i)                                                                                     \
    case i:                                                                                                   \
        if constexpr (i < count) {                                                                            \
            constexpr TileCfg c = T[i];                                                                       \
            if constexpr (tile_fits_layout(c, I, L))                                                          \
                return launch_tiled_cfg<I, O, L, E, c.bm, c.bn, c.bk, c.wm, c.wn, c.cap, c.dl, c.pers>(       \
                    p, X, W, bias, Y, wsf, stream);                                                           \
        }                                                                                                     \
        break;
                switch (p.tile) {
                    TLG_TILED_CASE(0)
                    TLG_TILED_CASE(1)
                    TLG_TILED_CASE(2)
                    TLG_TILED_CASE(3)
                    TLG_TILED_CASE(4)
                    TLG_TILED_CASE(5)
                    TLG_TILED_CASE(6)
                    TLG_TILED_CASE(7)
                    TLG_TILED_CASE(8)
                    TLG_TILED_CASE(9)
                    TLG_TILED_CASE(10)
                    TLG_TILED_CASE(11)
                    TLG_TILED_CASE(12)
                default: break;
                }
                set_error("bad tiled tile");
                return (int)TLG_ERR_INVALID_ARG;
#undef TLG_TILED_CASE
            };
            // the planner admits no bias or GELU with a transposed first operand
            if constexpr (layout_a_transposed(decltype(lay)::value)) return by_epi(ic<0>{});
            else return with_epi(p.epi, by_epi);
        });
    });
}

}  // namespace tlg
