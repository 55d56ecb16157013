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

// Layout bits: the weight is [K][N] (TLG_KN, TLG_AT_KN); the first operand is
// stored transposed, [K][M] (TLG_AT_NK, TLG_AT_KN).
constexpr bool layout_b_kn(int layout) { return (layout & 1) != 0; }
constexpr bool layout_a_transposed(int layout) { return layout >= TLG_AT_NK; }

// Epilogue flags that select a kernel at compile time; TLG_EPI_RESIDUAL is a
// run-time argument of the same kernels (one read of Y per output element).
constexpr uint32_t kEpiKernel = TLG_EPI_BIAS | TLG_EPI_GELU_TANH;

// One entry of a variant's tile list.
struct TileCfg {
    int bm, bn, bk;  // workgroup tile (rows of Y, columns of Y, K per pipeline stage)
    int wm, wn;      // waves along M and N
    int cap = 0;     // workgroups per CU at most (enforced with unused LDS); 0: as registers and LDS allow
    int dl = 0;      // 16-bit [M][K]·[N][K] exact fit: LDS stages filled by direct loads (0: staged in registers)
    int pers = 0;    // exact fit, no split, even slice count: one workgroup per resident slot loops over tiles
};

// Tiles of the LDS-tiled MFMA kernel, per input class.  The index is what
// tlg_plan_opts::tile selects (entry k-1).
// fp32 operands: v_mfma_f32_32x32x2_f32, wave tile (bm/wm)×(bn/wn).
constexpr TileCfg kTiledF32[] = {
    {128, 128, 16, 2, 2, 2},  // 0: square and wide shapes; two per CU (a third leaves a one-per-CU tail)
    {64, 64, 16, 2, 2},    // 1: narrow grids, pairs with split-K
    {256, 128, 16, 2, 2},  // 2: 128×64 wave tiles
    {128, 128, 32, 2, 2},  // 3: deeper K slice
    {256, 256, 16, 2, 2},  // 4: 128×128 wave tiles
    {256, 256, 16, 2, 4},  // 5: eight waves, two per SIMD, 128×64 wave tiles
    {128, 128, 16, 2, 2, 2, 0, 1},  // 6: entry 0 with persistent workgroups
    {64, 64, 16, 2, 2, 0, 0, 1},    // 7: entry 1 with persistent workgroups
    // 128×192 (64×96 per wave): whole rounds at the GPT-2 widths (768 → 256
    // tiles at 8192 rows, so proj needs no K split), as for 16-bit inputs.
    {128, 192, 16, 2, 2},           // 8
    {128, 192, 32, 2, 2, 0, 0, 1},  // 9: persistent (32-deep slices leave a staging strip for every wave)
};
// 16-bit operands: v_mfma_f32_32x32x16_{f16,bf16}.  A slice of 32 elements
// is only 256 MFMA cycles per wave, too short to hide one slice of load
// latency, so the default slice is 64 or 128 elements deep.  Entries 6-8
// fill their LDS stages with direct loads (dl stages) where the operands
// allow it ([M][K]·[N][K], exact fit) and otherwise run as the staged tile of
// the same shape.  Measured against staging on the GPT-2 linears at 8192
// rows: faster for some shapes (attention output, proj), slower for others
// (qkv), so they are separate entries for the table search to choose from.
// Entry 9 is the staged 128x128x64 tile with persistent workgroups (faster
// for qkv and fc, whose grids span two to three rounds of resident slots).
constexpr TileCfg kTiled16[] = {
    {128, 128, 64, 2, 2},         // 0
    {64, 64, 64, 2, 2},           // 1: narrow grids, pairs with split-K
    {256, 128, 64, 2, 2},         // 2
    {256, 128, 32, 2, 2},         // 3: short slices; two workgroups per CU fit in LDS (the 64-deep 256x128 tile fits one)
    {256, 256, 64, 2, 2},         // 4
    {256, 256, 64, 2, 4},         // 5: eight waves, two per SIMD: one's stalls are the other's MFMA time
    {128, 128, 64, 2, 2, 0, 2},   // 6: direct loads, two stages
    {256, 128, 64, 2, 2, 0, 2},   // 7: direct loads, two stages
    {128, 128, 32, 2, 2, 0, 4},   // 8: direct loads, four 32-deep stages (three slices in flight)
    {128, 128, 64, 2, 2, 0, 0, 1},  // 9: persistent, the next tile's first slices loaded during this one's end
    {128, 128, 64, 2, 2, 0, 2, 1},  // 10: persistent with direct loads (warm-fast, slower in a cold pass of GPT-2 layers)
    // 128×192 tiles (64×96 per wave): at 8192 rows the GPT-2 widths 768 and 2304
    // make 256 or 768 of them, whole rounds of the 256 CUs where 128×128 makes
    // 1.5 or 4.5.  Warm probe, bf16 with bias: proj 8192×768×3072 54.3 → 42.9 µs
    // (11), qkv 8192×2304×768 39.8 → 38.1 µs (12, against entry 10).
    {128, 192, 64, 2, 2, 0, 0, 1},  // 11: persistent, staged
    {128, 192, 64, 2, 2, 0, 2, 1},  // 12: persistent with direct loads (80 KiB: two per CU)
};
// Whether a tile's operand loads divide evenly over its threads for a
// layout: every thread issues the same whole number of 16-byte loads of each
// operand, and a thread's loads of an [K][N] or [K][M] operand (stored
// n- or m-contiguous in LDS) share one lane offset, so the row width in
// 16-byte vectors divides the thread count.  The tiled kernel asserts the same
// at compile time; the planner refuses the rest (the 128×192 tiles take no
// [K][N] weight: 24 vectors per row against 256 threads).
constexpr bool tile_fits_layout(const TileCfg& c, int in_dt, int layout) {
    const int threads = 64 * c.wm * c.wn, epv = in_dt == TLG_F32 ? 4 : 8;
    const int vpr = c.bk / epv, mv = c.bm / epv, nv = c.bn / epv;
    const bool at = layout_a_transposed(layout), kn = layout_b_kn(layout);
    const int a_vec = at ? c.bk * mv : c.bm * vpr, b_vec = kn ? c.bk * nv : c.bn * vpr;
    return threads % vpr == 0 && (!kn || threads % nv == 0) && (!at || threads % mv == 0) &&
           a_vec >= threads && a_vec % threads == 0 && b_vec >= threads && b_vec % threads == 0;
}

constexpr int kNumTiledF32 = sizeof(kTiledF32) / sizeof(kTiledF32[0]);
constexpr int kNumTiled16 = sizeof(kTiled16) / sizeof(kTiled16[0]);

// Stream kernel: a workgroup has nb × kw waves; it owns 16·nb rows of W
// (16 per wave) and one K range of the grid split, which its kw waves split
// again.  Each wave keeps `loads` 16-byte weight loads per lane in flight per
// chunk (a chunk is loads·32 fp16/bf16 or loads·16 fp32 elements of K).
struct StreamCfg {
    int nb;      // 16-row column blocks per workgroup
    int kw;      // waves splitting the workgroup's K range
    int loads;   // 16-byte loads per lane per chunk
    int dl = 0;  // the weight tile goes to LDS by direct loads, X to registers (16-bit, M <= 16, no split)
    int rb = 0;  // 16-row blocks of X per workgroup (0: all of M up to 64 rows, else 32-row blocks)
    int pipe = 0;  // chunk c + 1's loads go out before chunk c's products; two X buffers in LDS
};
constexpr StreamCfg kStream[] = {
    {1, 8, 16},  // 0: 16-row tiles over all of K by 8 waves; no inter-workgroup traffic (M <= 16)
    {1, 8, 4},   // 1: same with 128-wide fp16 chunks (room in LDS for X up to 32 rows)
    {8, 1, 16},  // 2: 128-row tiles, K split across workgroups
    {4, 1, 32},  // 3: 64-row tiles, 1024-wide fp16 chunks, K split across workgroups
    {2, 4, 4},   // 4: 32-row tiles, 4-way in-workgroup split
    {1, 8, 16, 1},  // 5: 16-row tiles, all of the tile's weight rows in LDS (K a multiple of 512, at most 4096)
    // One chunk per workgroup for the fp32 layers at K = 768 (4·12·16 or
    // 8·6·16): no second round of X staging, barrier and loads.  Measured on
    // the 128-row GPT-2 linears against the two-chunk tiles: attention output
    // 5.9 vs 7.4 µs, qkv 12.3 vs 14.0 µs.
    {2, 4, 12, 0, 1},  // 6: 32-column tiles, 16-row blocks of X walked by grid z
    {1, 4, 12, 0, 1},  // 7: 16-column tiles, 16-row blocks
    {1, 8, 6},         // 8: 16-column tiles, 8 waves over K
    // 48 columns × 32 rows per workgroup: the widest one-chunk tile whose X chunk
    // and weight rows still fit one workgroup per CU; it reads the least X per
    // output of the tiles here (fc at 128 rows: 256 workgroups, 11.5 vs 13.4 µs
    // for the 32×32 three-chunk tile in a probe; qkv 11.0 vs 12.3 µs).
    {3, 4, 12, 0, 2},  // 9
    // The one-chunk tiles load all of K before the first product: on qkv at
    // 128 rows (stage timestamps, one box) the loads take 4.2 µs and the
    // products 3-4 µs after them, never overlapping.  These split K = 768 into
    // chunks whose loads are issued a chunk ahead of the products.
    {3, 4, 6, 0, 2, 1},  // 10: 48 columns × 32 rows, two chunks of 384 (fp32)
    {3, 4, 3, 0, 2, 1},  // 11: 48 columns × 32 rows, four chunks of 192
    {2, 4, 6, 0, 1, 1},  // 12: 32 columns × 16 rows, two chunks
    {1, 4, 6, 0, 1, 1},  // 13: 16 columns × 16 rows, two chunks
    {2, 4, 3, 0, 1, 1},  // 14: 32 columns × 16 rows, four chunks
};
// Direct-load stream tile: 16 weight rows of K 16-bit elements resident in LDS.
constexpr int kStreamDlMaxK = 4096, kStreamDlKStep = 512;
constexpr int kNumStream = sizeof(kStream) / sizeof(kStream[0]);
constexpr int kStreamMaxM = 64;      // rows of X one stream workgroup covers (4 blocks of 16)
constexpr int kStreamMaxRows = 256;  // beyond this the tiled kernel always wins (W re-read per row block)
constexpr int kStreamMaxSplit = 16;  // K splits summed by the last workgroup of a tile
constexpr int kLdsBytes = 160 * 1024;

// LDS of one stream workgroup: the X chunk (16·rowb rows, padded by 16
// bytes) plus the in-workgroup reduction buffer.  rowb is 1, 2 or 4.
inline int64_t stream_lds_bytes(const StreamCfg& c, int in_dt, int rowb) {
    if (c.dl) return 16 * kStreamDlMaxK * 2 + 8 * 4 * 64 * 4;  // weight rows, wave partials
    const int64_t esize = in_dt == 0 ? 4 : 2, epv = 16 / esize;
    const int64_t wck = (int64_t)c.kw * c.loads * 4 * epv;
    const int64_t x = (c.pipe ? 2 : 1) * 16 * rowb * (wck + epv) * esize;
    const int64_t red = c.kw > 1 ? (int64_t)c.nb * c.kw * rowb * 4 * 64 * 4 : 0;
    return x + red;
}

// Generic kernel: 64×64 tile, 256 threads, 4×4 outputs per thread.
constexpr int kGenericBM = 64, kGenericBN = 64, kGenericBK = 16;

}  // namespace tlg

struct tlg_plan {
    int64_t M, N, K;
    int in_dt, out_dt, layout;
    uint32_t epi;
    int variant;
    int tile;      // index into the variant's list
    int split;     // K split across workgroups (TILED, STREAM)
    int64_t kper;  // K range per split (STREAM)
    int rowb;      // STREAM: 16-row blocks covering M
    int threads;
    int64_t grid_x, grid_y, grid_z;
    int launches;
    size_t ws_bytes;
    int bm, bn, bk;
    int stages;  // TILED: LDS stages filled by direct loads (0: loads staged through registers)
    int persist;  // TILED: workgroups loop over tiles (grid sized at launch to the resident workgroups)
};

namespace tlg {
void set_error(const char* fmt, ...);
int launch_plan(const tlg_plan& p, const void* X, const void* W, const void* bias, void* Y,
                void* ws, void* stream);
// Workspace of every split plan: a fixed block of arrival counters first,
// then the fp32 partials.  Split stream plans keep one counter per
// (row block, tile) there and their last workgroup per tile resets it;
// tiled split plans never touch the block.  So every completed run of any
// plan leaves the counters zero, and one workspace, zeroed once, serves any
// sequence of plans.
constexpr size_t kWsCounterBytes = 64 * 1024;
constexpr int64_t kWsMaxTickets = (int64_t)(kWsCounterBytes / 4);
// The library-held scratch of gemm_run_no_alloc (per device), laid out as a
// workspace: counter block, then partials.
constexpr size_t kScratchBytes = 32u << 20;
constexpr int kMaxDevices = 64;
}  // namespace tlg
