// Hardware ceilings measured beside the datasheet peaks, for the benchmark's
// reports: the launch floor (an empty kernel), the rate of a plain read of a
// buffer, and the MFMA issue rate with no memory traffic.  These kernels are
// measurement probes: no GEMM path calls them.  They sit in their own shared
// library (libtlgceil.so) with a C ABI of plain pointers and sizes.
//
// "Optimizing a GPT-2-class transformer on a GPU" (Act V) and "One multiply,
// one RTX 5090, eight kernels" ("Where the time goes", "What was not
// measured") time an empty kernel and loads-only / math-only variants to
// locate where a kernel's time goes; these are the gfx950 counterparts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tlgceil.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ void empty_kernel(int* flag) {
    if (threadIdx.x == 0x7fffffff) flag[0] = 1;  // never true: keeps the kernel non-trivial to the compiler
}

// Each workgroup of 8 waves reads one 128 KiB block: every load instruction
// of a wave covers 1 KiB of consecutive bytes, all 16 loads of a lane are in
// flight before the first is used.  The xor of the data is stored only if it
// equals a value it never takes, so the loads cannot be dropped.
constexpr int kReadLoads = 16, kReadWaves = 8;
constexpr size_t kReadBlock = (size_t)kReadWaves * kReadLoads * 1024;

// On-chip read rate: 256 workgroups of 8 waves, workgroup b re-reading its
// own 96 KiB block (3 MiB per XCD, within its 4 MB L2) `reps` times.  Every
// pass a lane issues 12 loads of 16 bytes, 6 into each half of the block,
// before it uses the first (each load instruction of a wave covers 1 KiB of
// consecutive bytes): 96 KiB per workgroup in flight, more than the CU's L1
// holds, so the data comes from L2.  Each half takes its offset through an empty asm
// statement of its own every pass, so the compiler cannot keep one pass's
// data for the next, and the data is summed.
constexpr size_t kL2Block = 96 * 1024;
constexpr int kL2Grid = 256;
__global__ __launch_bounds__(64 * kReadWaves) void read_l2_kernel(const char* __restrict__ base, int reps,
                                                                  float* __restrict__ sink) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    constexpr int kLoads = 12, kPerHalf = kLoads / 2;
    constexpr size_t kHalf = kL2Block / 2, kWave = kHalf / kReadWaves;  // 6 KiB per wave and half
    static_assert(kWave == kPerHalf * 1024, "a wave's loads tile its part of each half");
    const uint32_t off = (uint32_t)(blockIdx.x * kL2Block + (size_t)w * kWave + lane * 16);
    uint32_t x = 0;
    for (int r = 0; r < reps; ++r) {
        uint32_t o[2] = {off, (uint32_t)(off + kHalf)};
        asm volatile("" : "+v"(o[0]));
        asm volatile("" : "+v"(o[1]));
        u32x4 v[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            v[j] = *reinterpret_cast<const u32x4*>(base + o[j / kPerHalf] + (j % kPerHalf) * 1024);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) x += v[j][0] + v[j][1] + v[j][2] + v[j][3];
    }
    if (x == 0x9e3779b9u) sink[threadIdx.x] = 1.0f;
}

__global__ __launch_bounds__(64 * kReadWaves) void read_kernel(const char* __restrict__ base, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const char* p = base + (size_t)blockIdx.x * kReadBlock;
    u32x4 v[kReadLoads];
#pragma unroll
    for (int j = 0; j < kReadLoads; ++j)
        v[j] = *reinterpret_cast<const u32x4*>(p + ((size_t)w * kReadLoads + j) * 1024 + lane * 16);
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kReadLoads; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    if (x == 0x9e3779b9u) sink[threadIdx.x] = 1.0f;
}

// Sixteen independent 32x32 accumulators per wave, so consecutive MFMAs never
// wait on each other; the operands stay in registers.  One wave per SIMD
// (256 threads per workgroup, one workgroup per CU when the grid is the CU count).
// With `stamps`, thread 0 of each workgroup records the shader-clock counter
// (s_memtime) and the constant-rate counter (s_memrealtime) before and after
// the MFMA loop: their ratio is the core clock the loop ran at.
template <bool BF16>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink,
                                                   unsigned long long* __restrict__ stamps) {
    unsigned long long c0 = 0, r0 = 0;
    if (stamps && threadIdx.x == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    f32x16 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    const float a = 1.0f + threadIdx.x * 1e-7f, b = 1.0f - threadIdx.x * 1e-7f;
    u32x4 ra, rb;
    for (int e = 0; e < 4; ++e) {
        ra[e] = 0x3f803f80u + threadIdx.x;
        rb[e] = 0x3f803f80u - threadIdx.x;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (BF16)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra),
                                                                 __builtin_bit_cast(bf16x8, rb), acc[i], 0, 0, 0);
            else
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (stamps && threadIdx.x == 0) {
        const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        unsigned long long* o = stamps + 4 * (size_t)blockIdx.x;
        o[0] = c0;
        o[1] = c1;
        o[2] = r0;
        o[3] = r1;
    }
    if (s == 1234.5f) sink[threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Empty kernel over `grid` workgroups of 64 threads.
int tlg_ceil_empty(int grid, int* flag, void* stream) {
    if (grid <= 0 || !flag) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream, flag);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Read `bytes` bytes from `p` (16-byte aligned, a multiple of 128 KiB).
// `sink` must hold 512 floats.
int tlg_ceil_read(const void* p, size_t bytes, float* sink, void* stream) {
    if (!p || !sink || bytes == 0 || bytes % kReadBlock != 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return -1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)(bytes / kReadBlock)), dim3(64 * kReadWaves), 0,
                       (hipStream_t)stream, static_cast<const char*>(p), sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Re-read a 24 MiB buffer's 96 KiB blocks `reps` times (one workgroup per block).
int tlg_ceil_read_l2(const void* p, int reps, float* sink, void* stream) {
    if (!p || !sink || reps <= 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return -1;
    hipLaunchKernelGGL(read_l2_kernel, dim3(kL2Grid), dim3(64 * kReadWaves), 0, (hipStream_t)stream,
                       static_cast<const char*>(p), reps, sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// MFMA issue probe: `grid` workgroups of 4 waves, each wave issuing
// 16·iters MFMAs (bf16 != 0: 32x32x16 bf16, 32768 flop each; else 32x32x2
// fp32, 4096 flop each).  `sink` must hold 256 floats.
int tlg_ceil_mfma(int bf16, int grid, int iters, float* sink, void* stream) {
    return tlg_ceil_mfma_clock(bf16, grid, iters, sink, nullptr, stream);
}

// The same probe; `stamps` (NULL or 4·grid counters) receives per workgroup
// the shader-clock counter before and after the loop, then the constant-rate
// counter before and after.
int tlg_ceil_mfma_clock(int bf16, int grid, int iters, float* sink, unsigned long long* stamps, void* stream) {
    if (grid <= 0 || iters <= 0 || !sink) return -1;
    if (bf16)
        hipLaunchKernelGGL(mfma_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, sink, stamps);
    else
        hipLaunchKernelGGL(mfma_kernel<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, sink, stamps);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Rate of the constant-rate counter (s_memrealtime) of the current device, in kHz.
int tlg_ceil_wall_clock_khz(int* khz) {
    if (!khz) return -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -6;
    return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : -6;
}

}  // extern "C"
