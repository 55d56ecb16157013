// The operations around the linear layers of a GPT-2 block: layer
// normalisation and fused causal attention (C ABI in include/tlglayer.h).
//
// Both are HBM-bound at GPT-2 sizes (the layer normalisation reads and writes
// each row once; attention reads q, k, v once and writes its output once), so
// they are built for coalesced 16-byte traffic and for keeping what is reused
// on chip, not for MFMA rate.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels/common.h"
#include "tlglayer.h"
#include "tlgemm_internal.h"

namespace tlg {
namespace {

// ---- vector loads and stores of VE consecutive elements ---------------------------
template <int BYTES> struct Raw;
template <> struct Raw<2> { using T = uint16_t; };
template <> struct Raw<4> { using T = uint32_t; };
template <> struct Raw<8> { using T = u32x2; };
template <> struct Raw<16> { using T = u32x4; };

template <int DT, int VE> __device__ inline void load_vec(const void* p, int64_t idx, float* v) {
    using S = typename Elem<DT>::storage;
    using R = typename Raw<VE * (int)sizeof(S)>::T;
    struct Pack { S e[VE]; };
    const Pack pk = __builtin_bit_cast(Pack, *reinterpret_cast<const R*>(static_cast<const S*>(p) + idx));
#pragma unroll
    for (int u = 0; u < VE; ++u) v[u] = Elem<DT>::to_f32(pk.e[u]);
}

template <int DT> __device__ inline typename Elem<DT>::storage to_storage(float v) {
    if constexpr (DT == TLG_F32) return v;
    else if constexpr (DT == TLG_F16) return __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
    else return f32_to_bf16_rne(v);
}

template <int DT, int VE> __device__ inline void store_vec(void* p, int64_t idx, const float* v) {
    using S = typename Elem<DT>::storage;
    using R = typename Raw<VE * (int)sizeof(S)>::T;
    if constexpr (DT != TLG_F32 && VE % 2 == 0) {  // pairs through one packed conversion each
        struct Words { uint32_t w[VE / 2]; };
        Words wd;
#pragma unroll
        for (int u = 0; u < VE / 2; ++u) wd.w[u] = pack2<DT>(v[2 * u], v[2 * u + 1]);
        *reinterpret_cast<R*>(static_cast<S*>(p) + idx) = __builtin_bit_cast(R, wd);
    } else {
        struct Pack { S e[VE]; };
        Pack pk;
#pragma unroll
        for (int u = 0; u < VE; ++u) pk.e[u] = to_storage<DT>(v[u]);
        *reinterpret_cast<R*>(static_cast<S*>(p) + idx) = __builtin_bit_cast(R, pk);
    }
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// ---- layer normalisation ------------------------------------------------------------
// The pages split a row over two warps so that enough threads are resident to
// keep loads in flight.  On gfx950 the measure is bytes in flight per CU, so a
// wave owns whole rows instead, and R (two) rows at a time: a lane holds vectors
// lane, lane+64, ... of each of its rows (every load instruction of the wave
// covers 64 consecutive vectors) and issues all of them before the first
// reduction.  Mean and squared deviations come from registers (two passes
// over the values, one read of the row); no LDS, no barrier.
constexpr int kLnMaxPerLane = 64;  // values a lane holds: C <= 64 * 64

// NVMAX: VE-wide vectors a lane holds per row, the smallest of the
// instantiated counts that covers C (the host picks it), so that the row and
// the gamma and beta vectors stay in registers at full occupancy.
template <int DT, int VE, int R, int NVMAX>
__global__ __launch_bounds__(256) void layernorm_kernel(const void* __restrict__ X, const void* __restrict__ gamma,
                                                        const void* __restrict__ beta, void* __restrict__ Y,
                                                        float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                        int64_t rows, int C, float eps) {
    static_assert(NVMAX * VE * R <= kLnMaxPerLane, "values a lane holds");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * R;
    float v[R][NVMAX][VE];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NVMAX; ++j) {
            const int e = (lane + 64 * j) * VE;
            if (row0 + r < rows && e < C) load_vec<DT, VE>(X, (row0 + r) * C + e, v[r][j]);
        }
    // gamma and beta do not depend on the row: their loads go out with the
    // rows', not after the statistics (a second memory round trip)
    float gv[NVMAX][VE], bv[NVMAX][VE];
#pragma unroll
    for (int j = 0; j < NVMAX; ++j) {
        const int e = (lane + 64 * j) * VE;
        if (e < C) {
            load_vec<DT, VE>(gamma, e, gv[j]);
            load_vec<DT, VE>(beta, e, bv[j]);
        }
    }
    const float inv_c = 1.0f / (float)C;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        if (row >= rows) break;  // wave-uniform
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NVMAX; ++j)
            if ((lane + 64 * j) * VE < C)
#pragma unroll
                for (int u = 0; u < VE; ++u) s += v[r][j][u];
        const float mu = wave_sum(s) * inv_c;
        float q = 0.0f;
#pragma unroll
        for (int j = 0; j < NVMAX; ++j)
            if ((lane + 64 * j) * VE < C)
#pragma unroll
                for (int u = 0; u < VE; ++u) {
                    const float d = v[r][j][u] - mu;
                    q += d * d;
                }
        const float rs = 1.0f / sqrtf(wave_sum(q) * inv_c + eps);
#pragma unroll
        for (int j = 0; j < NVMAX; ++j) {
            const int e = (lane + 64 * j) * VE;
            if (e < C) {
                float y[VE];
#pragma unroll
                for (int u = 0; u < VE; ++u) y[u] = (v[r][j][u] - mu) * rs * gv[j][u] + bv[j][u];
                store_vec<DT, VE>(Y, row * C + e, y);
            }
        }
        if (lane == 0) {
            if (mean_out) mean_out[row] = mu;
            if (rstd_out) rstd_out[row] = rs;
        }
    }
}

// ---- fused causal attention ------------------------------------------------------------
// One workgroup per (batch, head) with four waves.  Queries come in blocks of
// 16 rows; with causality block q needs q + 1 key blocks of 16, so wave w
// takes blocks w and 7 - w of every group of eight: 9 key blocks per wave at
// T = 128, the same on every wave (and on every SIMD).  The head's keys and
// values pass through LDS in chunks of 64 keys (values transposed,
// [dimension][key]); each wave keeps the running state of both its query
// blocks in registers across the chunks.  The chunk keeps a workgroup's LDS
// at 37 KiB whatever T is, so three workgroups share a CU and the 768 heads
// of B 64 × 12 run in one round (with the head's whole K and V resident, 69
// KiB, two fitted and they took one and a half).  For each key block up to
// the query block (causality as a loop bound), in key order:
//  * S = Q Kᵀ on v_mfma_f32_16x16x4_f32: lane group kk holds dimensions
//    16kk .. 16kk+15 of its query row (in registers, pre-scaled by
//    log2(e)/sqrt(64)) and of its key row (four 16-byte LDS reads); the same
//    permutation of the dimensions on both sides leaves each dot product
//    unchanged.  Two accumulators take alternate steps, summed at the end;
//  * S passes through the wave's 16×16 LDS tile into the A-operand layout of
//    P V, where lane (row i, group kk) holds keys 4kk .. 4kk+3 of row i:
//    masking, the row maximum (four local values and two exchanges), the
//    rescaling factor exp2(m_old - m_new), P = exp2(S - m_new) and the lane's
//    part of the row sum are per-lane work;
//  * the four output tiles (dimensions in blocks of 16, accumulator layout:
//    lane (dimension d, group g) holds rows 4g..4g+3) are rescaled with the
//    factors of their rows, fetched by lane exchange, then O += P V with the
//    values read four keys at a time from the transposed copy.
// The row sums meet at the end the same way.
//
// LDS layouts, XOR-swizzled so that the reads are conflict-free: key row j
// of a chunk holds its sixteen 16-byte chunks at chunk ^ (j % 16); transposed
// value row d holds its four-key chunks at chunk ^ (d % 16); the score tile
// has a row stride of 20 floats.  Keys and values past T are loaded as zero,
// so masked keys (p = 0) multiply finite values.
constexpr int kHeadSize = 64, kKeyBlock = 32, kKeyChunk = 64;

// 16-byte loads each thread keeps in flight while filling the key and value tiles.
constexpr int kLoadGroup = 8;

__device__ inline int k_at(int j, int chunk) { return j * kHeadSize + ((chunk ^ (j & 15)) << 2); }
__device__ inline int p_at(int m, int n) { return m * 32 + (n ^ ((m & 7) << 2)); }
template <int TMAX> __device__ inline int vt_at(int d, int key) {
    return d * TMAX + ((((key >> 2) ^ (d & 15)) << 2) | (key & 3));
}
constexpr int kTile16 = 20;  // row stride of the 16×16 score tile (floats)

// The running state of one 16-row query block (its query rows are re-read
// from memory, an L2 hit, for each chunk: holding both blocks' would spill).
struct QBlock {
    f32x4 o[4];   // output tiles, dimensions 16dt .. 16dt+15
    float m, lp;  // running maximum and this lane's part of the row sum
    int q0, myrow;
    bool on;      // the block exists (wave-uniform)
};

template <int DT, bool CAUSAL, int TMAX>
__global__ __launch_bounds__(256, TMAX <= 128 ? 3 : 1) void attention_kernel(const void* __restrict__ qkv,
                                                                            void* __restrict__ out,
                                                                            float* __restrict__ lse, int T, int NH) {
    // Up to 128 keys, chunks of 64 (three workgroups per CU); beyond, the
    // whole head stays resident: with few heads per CU there is no occupancy
    // to win, and chunks there measured slower (B 16, T 256: 50.9 vs 43.6 µs).
    constexpr int HS = kHeadSize, KC = TMAX <= 128 ? kKeyChunk : TMAX;
    constexpr int EPV = Elem<DT>::per16;  // elements per 16-byte vector
    static_assert(EPV == 4, "the fp32 kernel");
    static_assert(TMAX % KC == 0, "whole chunks");
    constexpr int VPR = HS / EPV;  // 16-byte vectors per row
    static_assert((2 * KC * VPR) % (256 * kLoadGroup) == 0, "whole rounds of loads fill a chunk");
    __shared__ __attribute__((aligned(16))) float Ks[KC * HS];
    __shared__ __attribute__((aligned(16))) float Vt[HS * KC];
    __shared__ __attribute__((aligned(16))) float Ps[4 * 16 * kTile16];
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int64_t C = (int64_t)NH * HS, C3 = 3 * C;
    const int64_t head = (int64_t)b * T * C3 + (int64_t)h * HS;  // q of row 0 of this head
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15, kk = lane >> 4;
    float* P = Ps + wave * 16 * kTile16;
    const float qscale = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
    const int nqb = (T + 15) / 16;

    // One key block of 16 (keys j0 .. j0+15, the chunk starting at key c0) into a query block's state.
    auto step = [&](QBlock& st, const float* q, int j0, int c0) {
        // S: key row j0 + c16 (rows past T are zero; their scores are masked below)
        const int kl = j0 - c0 + c16;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f32x4 kv = *reinterpret_cast<const f32x4*>(Ks + k_at(kl, 4 * kk + t));
            s0 = mfma16_f32(q[4 * t], kv[0], s0);
            s1 = mfma16_f32(q[4 * t + 1], kv[1], s1);
            s0 = mfma16_f32(q[4 * t + 2], kv[2], s0);
            s1 = mfma16_f32(q[4 * t + 3], kv[3], s1);
        }
        // accumulator layout (key c16, rows 4kk + e) -> operand layout (row c16, keys 4kk ..
        // 4kk+3).  LDS operations of one wave complete in issue order; the empty asm
        // statements keep the compiler from reordering these accesses across each other.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < 4; ++e) P[(4 * kk + e) * kTile16 + c16] = s0[e] + s1[e];
        const f32x4 sv = *reinterpret_cast<const f32x4*>(P + c16 * kTile16 + 4 * kk);
        asm volatile("" ::: "memory");
        float p[4] = {sv[0], sv[1], sv[2], sv[3]};
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int key = j0 + 4 * kk + u;
            const bool keep = key < T && st.myrow < T && (!CAUSAL || key <= st.myrow);
            p[u] = keep ? p[u] : -INFINITY;
            bm = fmaxf(bm, p[u]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 16, 64));  // the row's other key groups
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float mn = fmaxf(st.m, bm);
        const float ms = mn == -INFINITY ? 0.0f : mn;  // a row with nothing visible yet stays at zero
        const float corr = __builtin_amdgcn_exp2f(st.m - ms);
        st.m = mn;
        float ps = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            p[u] = __builtin_amdgcn_exp2f(p[u] - ms);
            ps += p[u];
        }
        st.lp = st.lp * corr + ps;
        // rescaling factors of the accumulator rows 4kk + e (held by lanes 4kk + e of group 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ce = __shfl(corr, 4 * kk + e, 64);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) st.o[dt][e] *= ce;
        }
        // O += P V: keys j0 + 4kk + u, dimensions 16dt + c16 of the value tile
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const f32x4 vv = *reinterpret_cast<const f32x4*>(Vt + vt_at<KC>(16 * dt + c16, j0 - c0 + 4 * kk));
#pragma unroll
            for (int u = 0; u < 4; ++u) st.o[dt] = mfma16_f32(p[u], vv[u], st.o[dt]);
        }
    };

    QBlock blk[2];
    int resident = -1;  // first key of the chunk in LDS
    for (int group = 0; group < nqb; group += 8) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            QBlock& st = blk[half];
            const int qblk = group + (half ? 7 - wave : wave);
            st.on = qblk < nqb;
            st.q0 = qblk * 16;
            st.myrow = st.q0 + c16;  // this lane's row in the operand layout
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            st.m = -INFINITY;
            st.lp = 0.0f;
        }
        // keys the group needs (workgroup-uniform, so every wave meets every barrier)
        const int gend = CAUSAL ? min(T, (group + 8) * 16) : T;
        for (int c0 = 0; c0 < gend; c0 += KC) {
            if (c0 != resident) {  // workgroup-uniform: a chunk that holds all of T is loaded once
                __syncthreads();  // the previous chunk's reads are done
                for (int base = threadIdx.x; base < 2 * KC * VPR; base += 256 * kLoadGroup) {
                    // keys c0 .. c0+KC-1 and their values, 16-byte vectors: each thread has its kLoadGroup
                    // loads in flight before it stores any of them
                    float f[kLoadGroup][EPV];
#pragma unroll
                    for (int i = 0; i < kLoadGroup; ++i) {
                        const int idx = base + 256 * i;
                        const bool isv = idx >= KC * VPR;
                        const int rem = isv ? idx - KC * VPR : idx, j = rem / VPR, c = (rem % VPR) * EPV;
#pragma unroll
                        for (int u = 0; u < EPV; ++u) f[i][u] = 0.0f;
                        if (c0 + j < T)
                            load_vec<DT, EPV>(qkv, head + (int64_t)(c0 + j) * C3 + (isv ? 2 : 1) * C + c, f[i]);
                    }
#pragma unroll
                    for (int i = 0; i < kLoadGroup; ++i) {
                        const int idx = base + 256 * i;
                        const bool isv = idx >= KC * VPR;
                        const int rem = isv ? idx - KC * VPR : idx, j = rem / VPR, c = (rem % VPR) * EPV;
                        if (isv) {
#pragma unroll
                            for (int u = 0; u < EPV; ++u) Vt[vt_at<KC>(c + u, j)] = f[i][u];
                        } else {
                            *reinterpret_cast<f32x4*>(Ks + k_at(j, c >> 2)) = f32x4{f[i][0], f[i][1], f[i][2], f[i][3]};
                        }
                    }
                }
                __syncthreads();
                resident = c0;
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                QBlock& st = blk[half];
                if (!st.on) continue;  // wave-uniform
                const int kend = min(CAUSAL ? min(T, st.q0 + 16) : T, c0 + KC);
                if (c0 >= kend) continue;
                float q[16];  // dimensions 16kk .. 16kk+15 of row myrow, pre-scaled
#pragma unroll
                for (int c = 0; c < 16; c += EPV)
                    load_vec<DT, EPV>(qkv, head + (int64_t)min(st.myrow, T - 1) * C3 + 16 * kk + c, q + c);
#pragma unroll
                for (int c = 0; c < 16; ++c) q[c] *= qscale;
                for (int j0 = c0; j0 < kend; j0 += 16) step(st, q, j0, c0);
            }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            QBlock& st = blk[half];
            if (!st.on) continue;
            float l = st.lp + __shfl_xor(st.lp, 16, 64);
            l += __shfl_xor(l, 32, 64);
            if (kk == 0 && lse && st.myrow < T)
                lse[((int64_t)b * NH + h) * T + st.myrow] = (st.m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
            const float inv = 1.0f / l;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ie = __shfl(inv, 4 * kk + e, 64);
                const int row = st.q0 + 4 * kk + e;
                if (row < T) {
                    const int64_t orow = ((int64_t)b * T + row) * C + (int64_t)h * HS;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const float y = st.o[dt][e] * ie;
                        store_vec<DT, 1>(out, orow + 16 * dt + c16, &y);
                    }
                }
            }
        }
    }
}

// 16-bit inputs: the same algorithm on v_mfma_f32_32x32x16_{bf16,f16}.  Keys
// and values stay 16-bit in LDS.  A key row's eight 16-byte chunks sit at
// chunk ^ ((j/2) % 8) (two 128-byte rows share the 64 banks, so sixteen rows
// read one chunk each without conflict).  Value rows are padded to 80
// elements; the B operand of P V (eight consecutive keys of one dimension)
// comes from two LDS transpose reads, and rows past T are zero so that masked
// keys (p = 0) multiply finite values.  A lane's 16 keys of a row are
// 8g..8g+7 and 16+8g..16+8g+7, the two 8-key halves of the P operand.
constexpr int kVStride16 = 80;

__device__ inline int k16_at(int j, int chunk) { return j * kHeadSize + ((chunk ^ ((j >> 1) & 7)) << 3); }

// Up to 128 keys the LDS of three workgroups fits a CU (52 KiB each); the
// register bound that lets three share it (at most 168 per lane) is asked
// for explicitly: at the compiler's own choice of 188 registers only two
// fitted, and 768 heads took one and a half rounds instead of one (B 64,
// T 128, 12 heads, bf16: 23.3 -> 16.1 µs, bitwise the same result).
template <int DT, bool CAUSAL, int TMAX>
__global__ __launch_bounds__(256, TMAX <= 128 ? 3 : 1) void attention16_kernel(const void* __restrict__ qkv, void* __restrict__ out,
                                                          float* __restrict__ lse, int T, int NH) {
    using S = typename Elem<DT>::storage;
    constexpr int HS = kHeadSize, VST = kVStride16;
    constexpr int TPAD = (TMAX + 31) / 32 * 32;
    __shared__ __attribute__((aligned(16))) S Ks[TMAX * HS];
    __shared__ __attribute__((aligned(16))) S Vs[TPAD * VST];
    __shared__ __attribute__((aligned(16))) float Ps[4 * 32 * 32];
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int64_t C = (int64_t)NH * HS, C3 = 3 * C;
    const int64_t head = (int64_t)b * T * C3 + (int64_t)h * HS;  // q of row 0 of this head
    const S* X = static_cast<const S*>(qkv);

    // keys and values: 16-byte vectors of 8 elements, copied as they are, with
    // kLoadGroup loads of each thread in flight before it stores any of them
    const int tz = (T + 31) / 32 * 32;  // value rows up to the last key block, zero past T
    const int nvec = (T + tz) * 8;
    for (int base = threadIdx.x; base < nvec; base += 256 * kLoadGroup) {
        u32x4 v[kLoadGroup];
#pragma unroll
        for (int i = 0; i < kLoadGroup; ++i) {
            const int idx = base + 256 * i;
            const bool isv = idx >= T * 8;
            const int i2 = isv ? idx - T * 8 : idx, j = i2 >> 3, ch = i2 & 7;
            v[i] = u32x4{0u, 0u, 0u, 0u};
            if (idx < nvec && (!isv || j < T))
                v[i] = *reinterpret_cast<const u32x4*>(X + head + (int64_t)j * C3 + (isv ? 2 * C : C) + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < kLoadGroup; ++i) {
            const int idx = base + 256 * i;
            const bool isv = idx >= T * 8;
            const int i2 = isv ? idx - T * 8 : idx, j = i2 >> 3, ch = i2 & 7;
            if (idx < nvec) *reinterpret_cast<u32x4*>(isv ? Vs + j * VST + ch * 8 : Ks + k16_at(j, ch)) = v[i];
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 31, g = lane >> 5;
    float* P = Ps + wave * 1024;
    const float sscale = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64), applied to the fp32 scores
    const int tr_row = 8 * g + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto gather_rows = [&](float (&dst)[16]) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(P + p_at(0, 8 * qd + 4 * g));
            dst[4 * qd] = x[0], dst[4 * qd + 1] = x[1], dst[4 * qd + 2] = x[2], dst[4 * qd + 3] = x[3];
        }
    };
    for (int qb = 0; qb < T; qb += 128) {
        const int row0 = qb + wave * 32;
        if (row0 >= T) break;  // wave-uniform
        const int myrow = row0 + r;
        // A operand of S, chunk c: row myrow, head dimensions 16c + 8g .. +7
        u32x4 q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            q[c] = *reinterpret_cast<const u32x4*>(X + head + (int64_t)min(myrow, T - 1) * C3 + 16 * c + 8 * g);
        f32x16 o0, o1;
#pragma unroll
        for (int e = 0; e < 16; ++e) o0[e] = o1[e] = 0.0f;
        float m = -INFINITY, lp = 0.0f;
        const int kend = CAUSAL ? min(T, row0 + 32) : T;
        for (int j0 = 0; j0 < kend; j0 += kKeyBlock) {
            const int kr = min(j0 + r, T - 1);
            f32x16 sacc;
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                sacc = mfma32_16bit<DT>(q[c], *reinterpret_cast<const u32x4*>(Ks + k16_at(kr, 2 * c + g)), sacc);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int e = 0; e < 16; ++e) P[p_at(8 * (e >> 2) + 4 * g + (e & 3), r)] = sacc[e] * sscale;
            float p[16];  // keys 8g+c (c < 8) and 16+8g+c-8 (c >= 8) of this block
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int n = (k4 < 2 ? 8 * g : 16 + 8 * g) + 4 * (k4 & 1);
                const f32x4 x = *reinterpret_cast<const f32x4*>(P + p_at(r, n));
                p[4 * k4] = x[0], p[4 * k4 + 1] = x[1], p[4 * k4 + 2] = x[2], p[4 * k4 + 3] = x[3];
            }
            float bm = -INFINITY;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int key = j0 + (c < 8 ? 8 * g + c : 16 + 8 * g + c - 8);
                const bool keep = key < T && myrow < T && (!CAUSAL || key <= myrow);
                p[c] = keep ? p[c] : -INFINITY;
                bm = fmaxf(bm, p[c]);
            }
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mn = fmaxf(m, bm);
            const float ms = mn == -INFINITY ? 0.0f : mn;
            const float corr = __builtin_amdgcn_exp2f(m - ms);
            m = mn;
            float ps = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                p[c] = __builtin_amdgcn_exp2f(p[c] - ms);
                ps += p[c];
            }
            lp = lp * corr + ps;
            asm volatile("" ::: "memory");
            if (g == 0) P[p_at(0, r)] = corr;
            asm volatile("" ::: "memory");
            float cr[16];
            gather_rows(cr);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                o0[e] *= cr[e];
                o1[e] *= cr[e];
            }
            // O += P V over the block's two 16-key halves
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const u32x4 a = pack16<DT>(p + 8 * kc);
                const S* vb = Vs + (j0 + 16 * kc) * VST;
                const u32x2 b0l = lds_read_tr16(vb + tr_row * VST + tr_col);
                const u32x2 b0h = lds_read_tr16(vb + (tr_row + 4) * VST + tr_col);
                const u32x2 b1l = lds_read_tr16(vb + tr_row * VST + 32 + tr_col);
                const u32x2 b1h = lds_read_tr16(vb + (tr_row + 4) * VST + 32 + tr_col);
                o0 = mfma32_16bit<DT>(a, u32x4{b0l[0], b0l[1], b0h[0], b0h[1]}, o0);
                o1 = mfma32_16bit<DT>(a, u32x4{b1l[0], b1l[1], b1h[0], b1h[1]}, o1);
            }
        }
        const float l = lp + __shfl_xor(lp, 32, 64);
        if (g == 0 && lse && myrow < T)
            lse[((int64_t)b * NH + h) * T + myrow] = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
        asm volatile("" ::: "memory");
        if (g == 0) P[p_at(0, r)] = 1.0f / l;
        asm volatile("" ::: "memory");
        float inv[16];
        gather_rows(inv);
        // The output leaves through the wave's score tile: each 32-dimension half
        // of the block's 32 rows is written there in the accumulator layout and
        // read back as 16 consecutive dimensions of one row per lane, for two
        // 16-byte stores per half instead of sixteen 2-byte ones.
        const int srow = lane >> 1, sd = 16 * (lane & 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int e = 0; e < 16; ++e)
                P[p_at(8 * (e >> 2) + 4 * g + (e & 3), r)] = (half ? o1[e] : o0[e]) * inv[e];
            asm volatile("" ::: "memory");
            float y[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(P + p_at(srow, sd + 4 * q));
                y[4 * q] = x[0], y[4 * q + 1] = x[1], y[4 * q + 2] = x[2], y[4 * q + 3] = x[3];
            }
            asm volatile("" ::: "memory");
            if (row0 + srow < T) {
                const int64_t o = ((int64_t)b * T + row0 + srow) * C + (int64_t)h * HS + 32 * half + sd;
                store_vec<DT, 8>(out, o, y);
                store_vec<DT, 8>(out, o + 8, y + 8);
            }
        }
    }
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int DT, int VE, int R, int NV>
int launch_layernorm(const void* X, const void* g, const void* b, void* Y, float* mean, float* rstd, int64_t rows,
                     int C, float eps, hipStream_t s) {
    const int64_t grid = (rows + 4 * R - 1) / (4 * R);
    hipLaunchKernelGGL((layernorm_kernel<DT, VE, R, NV>), dim3((unsigned)grid), dim3(256), 0, s, X, g, b, Y, mean,
                       rstd, rows, C, eps);
    return check_launch("layernorm_kernel");
}

// Rows per wave: two where the values a lane holds allow it.  Measured at
// 8192 x 768: one row per wave 10.2 / 9.4 us (fp32 / bf16), two 9.8 / 8.6 us,
// four 11.1 / 10.7 us (more loads in flight per wave, but half the waves).
// Vectors per lane per row: the smallest of 1, 2, 3, 4, 8, 16, 32, 64 that
// covers the row.
template <int DT, int VE>
int layernorm_ve(const void* X, const void* g, const void* b, void* Y, float* mean, float* rstd, int64_t rows, int C,
                 float eps, hipStream_t s) {
    const int need = (C + 64 * VE - 1) / (64 * VE);  // vectors per lane per row
    auto go = [&](auto nvc) -> int {
        constexpr int NV = decltype(nvc)::value;
        if constexpr (NV * VE > kLnMaxPerLane) {
            return (int)TLG_ERR_UNSUPPORTED;  // not reached: C <= 64 * kLnMaxPerLane is checked by the caller
        } else {
            if constexpr (2 * NV * VE <= kLnMaxPerLane)
                return launch_layernorm<DT, VE, 2, NV>(X, g, b, Y, mean, rstd, rows, C, eps, s);
            else
                return launch_layernorm<DT, VE, 1, NV>(X, g, b, Y, mean, rstd, rows, C, eps, s);
        }
    };
    if (need <= 1) return go(std::integral_constant<int, 1>{});
    if (need <= 2) return go(std::integral_constant<int, 2>{});
    if (need <= 3) return go(std::integral_constant<int, 3>{});
    if (need <= 4) return go(std::integral_constant<int, 4>{});
    if (need <= 8) return go(std::integral_constant<int, 8>{});
    if (need <= 16) return go(std::integral_constant<int, 16>{});
    if (need <= 32) return go(std::integral_constant<int, 32>{});
    return go(std::integral_constant<int, 64>{});
}

template <int DT>
int layernorm_dt(const void* X, const void* g, const void* b, void* Y, float* mean, float* rstd, int64_t rows,
                 int C, float eps, hipStream_t s) {
    constexpr int es = (int)sizeof(typename Elem<DT>::storage);
    // the widest vector that divides the row and keeps every access aligned
    auto fits = [&](int ve) {
        const size_t a = (size_t)ve * es;
        return C % ve == 0 && aligned(X, a) && aligned(Y, a) && aligned(g, a) && aligned(b, a);
    };
    if constexpr (es == 2)
        if (fits(8)) return layernorm_ve<DT, 8>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    if (fits(4)) return layernorm_ve<DT, 4>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    if (fits(2)) return layernorm_ve<DT, 2>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    return layernorm_ve<DT, 1>(X, g, b, Y, mean, rstd, rows, C, eps, s);
}

template <int DT, bool CAUSAL>
int attention_dt(const void* qkv, void* out, float* lse, int64_t B, int T, int NH, hipStream_t s) {
    const dim3 grid((unsigned)(B * NH));
    if constexpr (DT == TLG_F32) {
        if (T <= 128) hipLaunchKernelGGL((attention_kernel<DT, CAUSAL, 128>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
        else hipLaunchKernelGGL((attention_kernel<DT, CAUSAL, 256>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
    } else {
        if (T <= 128)
            hipLaunchKernelGGL((attention16_kernel<DT, CAUSAL, 128>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
        else
            hipLaunchKernelGGL((attention16_kernel<DT, CAUSAL, 256>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
    }
    return check_launch("attention_kernel");
}

}  // namespace
}  // namespace tlg

using namespace tlg;

extern "C" {

int tlg_layernorm(const void* X, const void* gamma, const void* beta, void* Y, float* mean, float* rstd,
                  int64_t rows, int64_t C, float eps, tlg_dtype dt, void* stream) {
    if (!X || !gamma || !beta || !Y || rows < 1 || C < 1 || !(eps >= 0.0f) ||
        ((int)dt != TLG_F32 && (int)dt != TLG_F16 && (int)dt != TLG_BF16)) {
        set_error("tlg_layernorm: NULL pointer, rows or C < 1, eps < 0 or unknown dtype");
        return TLG_ERR_INVALID_ARG;
    }
    if (C > 64 * kLnMaxPerLane || rows >= (int64_t(1) << 32)) {
        set_error("tlg_layernorm: C = %lld exceeds %d (or too many rows)", (long long)C, 64 * kLnMaxPerLane);
        return TLG_ERR_UNSUPPORTED;
    }
    const size_t es = dt == TLG_F32 ? 4 : 2;
    if (!aligned(X, es) || !aligned(Y, es) || !aligned(gamma, es) || !aligned(beta, es) ||
        (mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4))) {
        set_error("tlg_layernorm: pointers must be aligned to their element size");
        return TLG_ERR_MISALIGNED;
    }
    const size_t bytes = (size_t)rows * (size_t)C * es, sb = (size_t)rows * 4;
    if (overlaps(Y, bytes, X, bytes) || overlaps(Y, bytes, gamma, C * es) || overlaps(Y, bytes, beta, C * es)) {
        set_error("tlg_layernorm: Y overlaps an input");
        return TLG_ERR_INVALID_ARG;
    }
    for (const float* st : {mean, rstd}) {
        if (st && (overlaps(st, sb, X, bytes) || overlaps(st, sb, Y, bytes) || overlaps(st, sb, gamma, C * es) ||
                   overlaps(st, sb, beta, C * es))) {
            set_error("tlg_layernorm: mean or rstd overlaps X, Y, gamma or beta");
            return TLG_ERR_INVALID_ARG;
        }
    }
    if (mean && rstd && overlaps(mean, sb, rstd, sb)) {
        set_error("tlg_layernorm: mean overlaps rstd");
        return TLG_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dt == TLG_F32) return layernorm_dt<TLG_F32>(X, gamma, beta, Y, mean, rstd, rows, (int)C, eps, s);
    if (dt == TLG_F16) return layernorm_dt<TLG_F16>(X, gamma, beta, Y, mean, rstd, rows, (int)C, eps, s);
    return layernorm_dt<TLG_BF16>(X, gamma, beta, Y, mean, rstd, rows, (int)C, eps, s);
}

int tlg_attention(const void* qkv, void* out, float* lse, int64_t B, int64_t T, int64_t n_head, int64_t head_size,
                  tlg_dtype dt, int causal, void* stream) {
    if (!qkv || !out || B < 1 || T < 1 || n_head < 1 || head_size < 1 ||
        ((int)dt != TLG_F32 && (int)dt != TLG_F16 && (int)dt != TLG_BF16)) {
        set_error("tlg_attention: NULL pointer, a size < 1 or unknown dtype");
        return TLG_ERR_INVALID_ARG;
    }
    if (head_size != kHeadSize || T > 256 || B * n_head >= (int64_t(1) << 31) || n_head * head_size >= (1 << 24)) {
        set_error("tlg_attention: supported are head_size 64 and T <= 256 (got %lld, %lld)", (long long)head_size,
                  (long long)T);
        return TLG_ERR_UNSUPPORTED;
    }
    if (!aligned(qkv, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4))) {
        set_error("tlg_attention: qkv and out must be 16-byte aligned");
        return TLG_ERR_MISALIGNED;
    }
    const size_t es = dt == TLG_F32 ? 4 : 2;
    const size_t C = (size_t)n_head * head_size;
    const size_t ob = (size_t)B * T * C * es, qb = (size_t)B * T * 3 * C * es, lb = (size_t)B * n_head * T * 4;
    if (overlaps(out, ob, qkv, qb) || (lse && (overlaps(lse, lb, out, ob) || overlaps(lse, lb, qkv, qb)))) {
        set_error("tlg_attention: out overlaps qkv, or lse overlaps out or qkv");
        return TLG_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int t = (int)T, nh = (int)n_head;
    auto go = [&](auto c) {
        constexpr bool CA = decltype(c)::value != 0;
        if (dt == TLG_F32) return attention_dt<TLG_F32, CA>(qkv, out, lse, B, t, nh, s);
        if (dt == TLG_F16) return attention_dt<TLG_F16, CA>(qkv, out, lse, B, t, nh, s);
        return attention_dt<TLG_BF16, CA>(qkv, out, lse, B, t, nh, s);
    };
    return causal ? go(ic<1>{}) : go(ic<0>{});
}

}  // extern "C"
