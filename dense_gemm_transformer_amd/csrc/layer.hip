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
    struct Pack { S e[VE]; };
    Pack pk;
#pragma unroll
    for (int u = 0; u < VE; ++u) pk.e[u] = to_storage<DT>(v[u]);
    *reinterpret_cast<R*>(static_cast<S*>(p) + idx) = __builtin_bit_cast(R, pk);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// ---- layer normalisation ------------------------------------------------------------
// 256 threads = 4 waves = 2 rows; waves 2r and 2r+1 hold the two halves of
// row r.  A lane holds vectors lane, lane+64, ... of its half, so every load
// instruction of a wave covers 64 consecutive vectors.  Each wave reduces its
// half's mean and squared deviations from registers; the halves are combined
// once through LDS with the pairwise update of means and squared deviations
// (Chan, Golub and LeVeque), which needs no second read of the row.
constexpr int kLnMaxPerLane = 64;  // values a lane holds: C <= 2 * 64 * 64

template <int DT, int VE>
__global__ __launch_bounds__(256) void layernorm_kernel(const void* __restrict__ X, const void* __restrict__ gamma,
                                                        const void* __restrict__ beta, void* __restrict__ Y,
                                                        float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                        int64_t rows, int C, float eps) {
    constexpr int NVMAX = kLnMaxPerLane / VE;
    __shared__ float part[2][2][2];  // [row in workgroup][half][mean, squared deviations]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rw = wave >> 1, half = wave & 1;
    const int64_t row = (int64_t)blockIdx.x * 2 + rw;
    const bool live = row < rows;
    const int h0 = (C + 1) / 2;  // the first half's length; VE > 1 needs C % (2 VE) == 0
    const int hstart = half ? h0 : 0, hlen = half ? C - h0 : h0;
    const int64_t base = row * C + hstart;

    float v[NVMAX][VE];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NVMAX; ++j) {
        const int e = (lane + 64 * j) * VE;
        if (live && e < hlen) {
            load_vec<DT, VE>(X, base + e, v[j]);
#pragma unroll
            for (int u = 0; u < VE; ++u) s += v[j][u];
        }
    }
    const float nw = (float)hlen;
    const float mw = hlen > 0 ? wave_sum(s) / nw : 0.0f;
    float q = 0.0f;
#pragma unroll
    for (int j = 0; j < NVMAX; ++j) {
        const int e = (lane + 64 * j) * VE;
        if (live && e < hlen) {
#pragma unroll
            for (int u = 0; u < VE; ++u) {
                const float d = v[j][u] - mw;
                q += d * d;
            }
        }
    }
    const float m2w = wave_sum(q);
    if (lane == 0) {
        part[rw][half][0] = mw;
        part[rw][half][1] = m2w;
    }
    __syncthreads();
    // Both waves combine the halves in the same order, so they agree exactly.
    const float n0 = (float)h0, n1 = (float)(C - h0), n = (float)C;
    const float mu0 = part[rw][0][0], mu1 = part[rw][1][0];
    const float delta = mu1 - mu0;
    const float mu = mu0 + delta * (n1 / n);
    const float m2 = part[rw][0][1] + part[rw][1][1] + delta * delta * (n0 * n1 / n);
    const float rs = 1.0f / sqrtf(m2 / n + eps);
    if (!live) return;
#pragma unroll
    for (int j = 0; j < NVMAX; ++j) {
        const int e = (lane + 64 * j) * VE;
        if (e < hlen) {
            float g[VE], b[VE], y[VE];
            load_vec<DT, VE>(gamma, hstart + e, g);
            load_vec<DT, VE>(beta, hstart + e, b);
#pragma unroll
            for (int u = 0; u < VE; ++u) y[u] = (v[j][u] - mu) * rs * g[u] + b[u];
            store_vec<DT, VE>(Y, base + e, y);
        }
    }
    if (half == 0 && lane == 0) {
        if (mean_out) mean_out[row] = mu;
        if (rstd_out) rstd_out[row] = rs;
    }
}

// ---- fused causal attention ------------------------------------------------------------
// One workgroup per (batch, head).  The head's keys and values are converted
// to fp32 into LDS once; 256 threads take 128 query rows at a time, two lanes
// per row, each lane holding 32 of the 64 dimensions of q and of the output.
// Keys are visited in blocks of 8 up to the last row of the wave (causality
// as a loop bound); lanes mask keys past their own row.  The softmax runs
// online in base 2: q is pre-scaled by log2(e)/sqrt(64), each block raises
// the running maximum and rescales the running sum and output by
// exp2(m_old - m_new), and the output is divided by the sum once at the end.
constexpr int kHeadSize = 64, kKeyBlock = 8;

template <int DT, bool CAUSAL, int TMAX>
__global__ __launch_bounds__(256) void attention_kernel(const void* __restrict__ qkv, void* __restrict__ out,
                                                        float* __restrict__ lse, int T, int NH) {
    constexpr int HS = kHeadSize, HH = HS / 2;
    constexpr int EPV = Elem<DT>::per16;  // elements per 16-byte vector
    __shared__ __attribute__((aligned(16))) float kv[2 * TMAX * HS];
    float* Ks = kv;
    float* Vs = kv + TMAX * HS;
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int64_t C = (int64_t)NH * HS, C3 = 3 * C;
    const int64_t head = (int64_t)b * T * C3 + (int64_t)h * HS;  // q of row 0 of this head

    // keys and values: T rows of HS elements each, 16-byte vectors
    constexpr int VPR = HS / EPV;
    for (int idx = threadIdx.x; idx < 2 * T * VPR; idx += 256) {
        const int which = idx / (T * VPR), rem = idx % (T * VPR), j = rem / VPR, c = (rem % VPR) * EPV;
        float f[EPV];
        load_vec<DT, EPV>(qkv, head + (int64_t)j * C3 + (which + 1) * C + c, f);
        float* dst = (which ? Vs : Ks) + j * HS + c;
#pragma unroll
        for (int u = 0; u < EPV; u += 4) *reinterpret_cast<f32x4*>(dst + u) = f32x4{f[u], f[u + 1], f[u + 2], f[u + 3]};
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int half = threadIdx.x & 1;
    const float qscale = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
    for (int qb = 0; qb < T; qb += 128) {
        const int i = qb + (threadIdx.x >> 1);
        const bool live = i < T;
        const int row_last = min(T - 1, qb + wave * 32 + 31);  // the wave's last query row
        if (qb + wave * 32 >= T) break;
        float q[HH], o[HH];
        if (live) {
#pragma unroll
            for (int c = 0; c < HH; c += EPV) load_vec<DT, EPV>(qkv, head + (int64_t)i * C3 + half * HH + c, q + c);
        } else {
#pragma unroll
            for (int c = 0; c < HH; ++c) q[c] = 0.0f;
        }
#pragma unroll
        for (int c = 0; c < HH; ++c) {
            q[c] *= qscale;
            o[c] = 0.0f;
        }
        float m = -INFINITY, l = 0.0f;
        const int jend = CAUSAL ? row_last + 1 : T;
        for (int j0 = 0; j0 < jend; j0 += kKeyBlock) {
            float s[kKeyBlock];
            float bm = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < kKeyBlock; ++kk) {
                const int j = j0 + kk;
                const float* kr = Ks + min(j, T - 1) * HS + half * HH;
                float part = 0.0f;
#pragma unroll
                for (int c = 0; c < HH; c += 4) {
                    const f32x4 kv4 = *reinterpret_cast<const f32x4*>(kr + c);
                    part = fmaf(q[c], kv4[0], part);
                    part = fmaf(q[c + 1], kv4[1], part);
                    part = fmaf(q[c + 2], kv4[2], part);
                    part = fmaf(q[c + 3], kv4[3], part);
                }
                const float full = part + __shfl_xor(part, 1, 64);
                const bool keep = live && j < T && (!CAUSAL || j <= i);
                s[kk] = keep ? full : -INFINITY;
                bm = fmaxf(bm, s[kk]);
            }
            const float mn = fmaxf(m, bm);
            if (mn == -INFINITY) continue;  // nothing visible yet in this row
            const float corr = __builtin_amdgcn_exp2f(m - mn);  // 0 while m is still -inf
            l *= corr;
#pragma unroll
            for (int c = 0; c < HH; ++c) o[c] *= corr;
#pragma unroll
            for (int kk = 0; kk < kKeyBlock; ++kk) {
                const float p = __builtin_amdgcn_exp2f(s[kk] - mn);  // 0 for masked keys
                l += p;
                const float* vr = Vs + min(j0 + kk, T - 1) * HS + half * HH;
#pragma unroll
                for (int c = 0; c < HH; c += 4) {
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(vr + c);
                    o[c] = fmaf(p, vv[0], o[c]);
                    o[c + 1] = fmaf(p, vv[1], o[c + 1]);
                    o[c + 2] = fmaf(p, vv[2], o[c + 2]);
                    o[c + 3] = fmaf(p, vv[3], o[c + 3]);
                }
            }
            m = mn;
        }
        if (live) {
            const float inv = 1.0f / l;
#pragma unroll
            for (int c = 0; c < HH; ++c) o[c] *= inv;
            const int64_t orow = ((int64_t)b * T + i) * C + (int64_t)h * HS + half * HH;
#pragma unroll
            for (int c = 0; c < HH; c += EPV) store_vec<DT, EPV>(out, orow + c, o + c);
            // log-sum-exp in natural units: (m + log2 l) * ln 2
            if (lse && half == 0) lse[((int64_t)b * NH + h) * T + i] = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
        }
    }
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int DT, int VE>
int launch_layernorm(const void* X, const void* g, const void* b, void* Y, float* mean, float* rstd, int64_t rows,
                     int C, float eps, hipStream_t s) {
    const int64_t grid = (rows + 1) / 2;
    hipLaunchKernelGGL((layernorm_kernel<DT, VE>), dim3((unsigned)grid), dim3(256), 0, s, X, g, b, Y, mean, rstd,
                       rows, C, eps);
    return check_launch("layernorm_kernel");
}

template <int DT>
int layernorm_dt(const void* X, const void* g, const void* b, void* Y, float* mean, float* rstd, int64_t rows,
                 int C, float eps, hipStream_t s) {
    constexpr int es = (int)sizeof(typename Elem<DT>::storage);
    // the widest vector that divides both halves and keeps every access aligned
    auto fits = [&](int ve) {
        const size_t a = (size_t)ve * es;
        return C % (2 * ve) == 0 && aligned(X, a) && aligned(Y, a) && aligned(g, a) && aligned(b, a);
    };
    if constexpr (es == 2)
        if (fits(8)) return launch_layernorm<DT, 8>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    if (fits(4)) return launch_layernorm<DT, 4>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    if (fits(2)) return launch_layernorm<DT, 2>(X, g, b, Y, mean, rstd, rows, C, eps, s);
    return launch_layernorm<DT, 1>(X, g, b, Y, mean, rstd, rows, C, eps, s);
}

template <int DT, bool CAUSAL>
int attention_dt(const void* qkv, void* out, float* lse, int64_t B, int T, int NH, hipStream_t s) {
    const dim3 grid((unsigned)(B * NH));
    if (T <= 128) hipLaunchKernelGGL((attention_kernel<DT, CAUSAL, 128>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
    else hipLaunchKernelGGL((attention_kernel<DT, CAUSAL, 256>), grid, dim3(256), 0, s, qkv, out, lse, T, NH);
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
    if (C > 2 * 64 * kLnMaxPerLane || rows >= (int64_t(1) << 32)) {
        set_error("tlg_layernorm: C = %lld exceeds %d (or too many rows)", (long long)C, 2 * 64 * kLnMaxPerLane);
        return TLG_ERR_UNSUPPORTED;
    }
    const size_t es = dt == TLG_F32 ? 4 : 2;
    if (!aligned(X, es) || !aligned(Y, es) || !aligned(gamma, es) || !aligned(beta, es) ||
        (mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4))) {
        set_error("tlg_layernorm: pointers must be aligned to their element size");
        return TLG_ERR_MISALIGNED;
    }
    const size_t bytes = (size_t)rows * (size_t)C * es;
    if (overlaps(Y, bytes, X, bytes) || overlaps(Y, bytes, gamma, C * es) || overlaps(Y, bytes, beta, C * es)) {
        set_error("tlg_layernorm: Y overlaps an input");
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
    if (overlaps(out, (size_t)B * T * C * es, qkv, (size_t)B * T * 3 * C * es) ||
        (lse && overlaps(lse, (size_t)B * n_head * T * 4, out, (size_t)B * T * C * es))) {
        set_error("tlg_attention: out overlaps qkv (or lse overlaps out)");
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
