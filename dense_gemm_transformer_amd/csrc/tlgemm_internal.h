// Internal declarations shared by the planner (host C++) and the launch glue
// (HIP).  Nothing here is part of the public C ABI in include/tlgemm.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tlgemm.h"

namespace tlg {

// MI355X: 256 compute units in 8 XCDs of 32.
constexpr int kNumCUs = 256;
constexpr int kNumXCDs = 8;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int dtype_size(int dt) { return dt == TLG_F32 ? 4 : 2; }

// One entry of a variant's tile list.
struct TileCfg {
    int bm, bn, bk;  // workgroup tile (rows of Y, columns of Y, K per pipeline stage)
    int wm, wn;      // waves along M and N
};

// Tiles of the LDS-tiled MFMA kernel, per input class.  The index is what
// tlg_plan_opts::tile selects (entry k-1).
// fp32 operands: v_mfma_f32_32x32x2_f32, wave tile (bm/wm)×(bn/wn).
constexpr TileCfg kTiledF32[] = {
    {128, 128, 16, 2, 2},  // 0: square and wide shapes
    {64, 64, 16, 2, 2},    // 1: narrow grids (M = 128 layers), pairs with split-K
    {256, 128, 16, 4, 2},  // 2: large M
};
// 16-bit operands: v_mfma_f32_32x32x16_{f16,bf16}.
constexpr TileCfg kTiled16[] = {
    {128, 128, 32, 2, 2},
    {64, 64, 32, 2, 2},
    {256, 128, 32, 4, 2},
};
constexpr int kNumTiledF32 = sizeof(kTiledF32) / sizeof(kTiledF32[0]);
constexpr int kNumTiled16 = sizeof(kTiled16) / sizeof(kTiled16[0]);

// Stream kernel: one workgroup owns 16 output columns (16 rows of W), its
// waves split K, and each wave keeps `loads` 16-byte weight loads per lane in
// flight per chunk.
struct StreamCfg {
    int waves;  // waves per workgroup = in-workgroup K split
    int loads;  // 16-byte loads per lane per chunk
};
constexpr StreamCfg kStream[] = {
    {8, 16},  // 0: 512-wide fp16 chunks per wave (256 fp32)
    {4, 16},  // 1
    {8, 8},   // 2
};
constexpr int kNumStream = sizeof(kStream) / sizeof(kStream[0]);
constexpr int kStreamMaxM = 64;  // 4 row blocks of 16

// Generic kernel: 64×64 tile, 256 threads, 4×4 outputs per thread.
constexpr int kGenericBM = 64, kGenericBN = 64, kGenericBK = 16;

}  // namespace tlg

struct tlg_plan {
    int64_t M, N, K;
    int in_dt, out_dt, layout;
    uint32_t epi;
    int variant;
    int tile;      // index into the variant's list
    int split;     // K split (TILED: across workgroups; STREAM: waves)
    int rowb;      // STREAM: 16-row blocks covering M
    int threads;
    int64_t grid_x, grid_y, grid_z;
    int launches;
    size_t ws_bytes;
    int bm, bn, bk;
};

namespace tlg {
void set_error(const char* fmt, ...);
int launch_plan(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                void* ws, void* stream);
}  // namespace tlg
