// Planner for the transformer linear layer: shape -> kernel, tile, split.
//
// Host-only and pure (no HIP call), so it is exercised by CPU tests.
// The routing idea is the per-shape dispatch table of "Optimizing a
// GPT-2-class transformer on a GPU" (Act II: no single kernel wins every
// shape, so each shape goes to its measured winner) and the tile/split
// choice of "Writing a CUDA matmul that catches cuBLAS" ("One kernel was
// never going to be enough"; "A stale constant, and two wrong explanations
// for it").  Exact shapes that were measured live in dispatch_table.inc;
// other shapes fall back to the fill rule below.

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "tlgemm_internal.h"

namespace tlg {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
}

struct TableRow {
    int64_t M, N, K;
    int in_dt, out_dt, layout;
    uint32_t epi;
    int variant, tile, split;
};

static const TableRow kTable[] = {
#include "dispatch_table.inc"
};

static const TableRow* table_lookup(int64_t M, int64_t N, int64_t K, int in_dt, int out_dt, int layout,
                                    uint32_t epi) {
    for (const TableRow& r : kTable) {
        if (r.M == M && r.N == N && r.K == K && r.in_dt == in_dt && r.out_dt == out_dt &&
            r.layout == layout && r.epi == epi)
            return &r;
    }
    return nullptr;
}

static bool valid_pair(int in_dt, int out_dt) {
    if (in_dt == TLG_F32) return out_dt == TLG_F32;
    if (in_dt == TLG_F16) return out_dt == TLG_F16 || out_dt == TLG_F32;
    if (in_dt == TLG_BF16) return out_dt == TLG_BF16 || out_dt == TLG_F32;
    return false;
}

// Rows of X and of the weight must start on 16-byte boundaries for the
// vectorised kernels (every row start is then aligned when the base is).
// X rows hold K elements, or M for the transposed-A layouts; weight rows K
// (out×in) or N ([K][N]).
static bool rows_aligned16(const tlg_plan& p) {
    const int64_t isz = dtype_size(p.in_dt);
    if (((layout_a_transposed(p.layout) ? p.M : p.K) * isz) % 16) return false;
    if (((layout_b_kn(p.layout) ? p.N : p.K) * isz) % 16) return false;
    return true;
}

static const TileCfg& tiled_cfg(int in_dt, int idx) {
    return in_dt == TLG_F32 ? kTiledF32[idx] : kTiled16[idx];
}
static int tiled_count(int in_dt) { return in_dt == TLG_F32 ? kNumTiledF32 : kNumTiled16; }

static int fill_generic(tlg_plan& p) {
    p.variant = TLG_VARIANT_GENERIC;
    p.tile = 0;
    p.split = 1;
    p.bm = kGenericBM;
    p.bn = kGenericBN;
    p.bk = kGenericBK;
    p.threads = 256;
    p.grid_x = ceil_div(p.N, kGenericBN);
    p.grid_y = ceil_div(p.M, kGenericBM);
    if (p.grid_y > 65535) {
        set_error("generic kernel: M=%lld needs more than 65535 row tiles", (long long)p.M);
        return TLG_ERR_UNSUPPORTED;
    }
    p.grid_z = 1;
    p.launches = 1;
    p.ws_bytes = 0;
    return TLG_OK;
}

// 16-row blocks of X per stream workgroup: all of M when it is at most 64,
// otherwise 32-row blocks walked by grid z.
static int stream_rowb(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= kStreamMaxM ? 4 : 2; }

static int fill_stream(tlg_plan& p, int tile, int split) {
    if (p.M > kStreamMaxRows) {
        set_error("stream kernel handles M <= %d (got M=%lld)", kStreamMaxRows, (long long)p.M);
        return TLG_ERR_UNSUPPORTED;
    }
    if (p.layout != TLG_NK) {
        set_error("stream kernel needs the out×in (NK) weight layout");
        return TLG_ERR_UNSUPPORTED;
    }
    if (!rows_aligned16(p)) {
        set_error("stream kernel needs K*elem_size to be a multiple of 16 bytes");
        return TLG_ERR_UNSUPPORTED;
    }
    if (tile < 0 || tile >= kNumStream) {
        set_error("stream tile index %d out of range", tile);
        return TLG_ERR_INVALID_ARG;
    }
    const StreamCfg& c = kStream[tile];
    if (c.dl && (p.in_dt == TLG_F32 || p.M > 16 || p.K % kStreamDlKStep != 0 || p.K > kStreamDlMaxK || split > 1)) {
        set_error("stream configuration %d needs 16-bit inputs, M <= 16, K a multiple of %d up to %d and no split",
                  tile, kStreamDlKStep, kStreamDlMaxK);
        return TLG_ERR_UNSUPPORTED;
    }
    const int rowb = c.rb ? c.rb : stream_rowb(p.M);
    if (stream_lds_bytes(c, p.in_dt, rowb) > kLdsBytes) {
        set_error("stream configuration %d does not fit in LDS for M=%lld", tile, (long long)p.M);
        return TLG_ERR_UNSUPPORTED;
    }
    const int64_t bn = 16 * c.nb;
    const int64_t wck = (int64_t)c.kw * c.loads * (p.in_dt == TLG_F32 ? 16 : 32);  // K per workgroup chunk
    const int64_t tiles = ceil_div(p.N, bn);
    const int64_t chunks = ceil_div(p.K, wck);
    int64_t S = split;
    if (S == 0) {  // fill rule: one workgroup per CU, each split at least one full chunk
        S = std::min<int64_t>(std::min<int64_t>(ceil_div(kNumCUs, tiles), chunks), kStreamMaxSplit);
    }
    if (S < 1 || S > kStreamMaxSplit || S > chunks) {
        set_error("stream split_k=%lld must be in 1..%lld", (long long)S,
                  (long long)std::min<int64_t>(chunks, kStreamMaxSplit));
        return TLG_ERR_UNSUPPORTED;
    }
    // Each split covers whole chunks; drop splits that would be empty.
    p.kper = ceil_div(ceil_div(p.K, S), wck) * wck;
    S = ceil_div(p.K, p.kper);
    p.variant = TLG_VARIANT_STREAM;
    p.tile = tile;
    p.split = (int)S;
    p.rowb = rowb;
    p.bm = 16 * rowb;
    p.bn = (int)bn;
    p.bk = c.dl ? (int)p.K : (int)wck;
    p.threads = 64 * c.nb * c.kw;
    p.grid_x = tiles;
    p.grid_y = S;
    p.grid_z = ceil_div(p.M, 16 * rowb);
    p.launches = 1;
    const int64_t slots = tiles * p.grid_z;  // (row block, tile) pairs, one ticket each
    if (S > 1 && slots > kWsMaxTickets) {
        set_error("stream split-K: %lld output tiles exceed the %lld arrival counters of a workspace",
                  (long long)slots, (long long)kWsMaxTickets);
        return TLG_ERR_UNSUPPORTED;
    }
    const int64_t part_bytes = S > 1 ? (int64_t)S * slots * bn * 16 * rowb * (int64_t)sizeof(float) : 0;
    if (part_bytes >= INT32_MAX) {  // the kernel addresses its partials through one buffer descriptor
        set_error("stream split-K: %lld bytes of partials exceed 2 GiB", (long long)part_bytes);
        return TLG_ERR_UNSUPPORTED;
    }
    p.ws_bytes = S > 1 ? kWsCounterBytes + (size_t)part_bytes : 0;
    return TLG_OK;
}

// Narrow-M choice: with enough 16-row tiles to fill the chip the whole K
// range of a tile stays inside one workgroup (no inter-workgroup traffic,
// whose device-scope fences cost several microseconds on a multi-XCD part);
// otherwise 128-row tiles split K across workgroups.
static int auto_stream(tlg_plan& p) {
    const int rowb = stream_rowb(p.M);
    if (ceil_div(p.N, 16) * ceil_div(p.M, 16 * rowb) >= kNumCUs / 2) {
        if (p.in_dt != TLG_F32 && p.M <= 16 && p.K % kStreamDlKStep == 0 && p.K <= kStreamDlMaxK)
            return fill_stream(p, 5, 1);
        for (int cfg : {0, 1, 4})
            if (stream_lds_bytes(kStream[cfg], p.in_dt, rowb) <= kLdsBytes) return fill_stream(p, cfg, 1);
    }
    return fill_stream(p, 2, 0);
}

static int fill_tiled(tlg_plan& p, int tile, int split) {
    if (!rows_aligned16(p)) {
        set_error("tiled kernel needs 16-byte aligned rows (%s and %s times elem_size a multiple of 16)",
                  layout_a_transposed(p.layout) ? "M" : "K", layout_b_kn(p.layout) ? "N" : "K");
        return TLG_ERR_UNSUPPORTED;
    }
    if (tile < 0 || tile >= tiled_count(p.in_dt)) {
        set_error("tiled tile index %d out of range", tile);
        return TLG_ERR_INVALID_ARG;
    }
    const TileCfg& c = tiled_cfg(p.in_dt, tile);
    if (!tile_fits_layout(c, p.in_dt, p.layout)) {
        set_error("tiled tile %dx%d does not take layout %d (its loads do not divide over its threads)", c.bm, c.bn,
                  p.layout);
        return TLG_ERR_UNSUPPORTED;
    }
    const int64_t ksteps = ceil_div(p.K, c.bk);
    if (split < 0 || split > ksteps) {
        set_error("split_k=%d must be in 1..%lld for K=%lld", split, (long long)ksteps, (long long)p.K);
        return TLG_ERR_UNSUPPORTED;
    }
    p.variant = TLG_VARIANT_TILED;
    p.tile = tile;
    p.split = split < 1 ? 1 : split;
    p.bm = c.bm;
    p.bn = c.bn;
    p.bk = c.bk;
    p.threads = 64 * c.wm * c.wn;
    p.grid_x = ceil_div(p.N, c.bn);
    p.grid_y = ceil_div(p.M, c.bm);
    p.grid_z = p.split;
    if (p.grid_x * p.grid_y >= (int64_t(1) << 31) || p.split > 65535 ||
        (p.split > 1 && p.M * p.N >= (int64_t(1) << 40))) {
        set_error("tiled kernel: grid too large for M=%lld N=%lld split=%d", (long long)p.M, (long long)p.N,
                  p.split);
        return TLG_ERR_UNSUPPORTED;
    }
    p.launches = p.split > 1 ? 2 : 1;
    p.ws_bytes = p.split > 1 ? kWsCounterBytes + (size_t)p.split * (size_t)p.M * (size_t)p.N * sizeof(float) : 0;
    // Direct loads into LDS: 16-bit [M][K]·[N][K] operands, exact-fit tiles,
    // each split a whole number of stage rounds, operand panels in 32-bit range.
    const int64_t kper = ceil_div(ceil_div(p.K, p.split), c.bk) * c.bk;
    const int64_t es = dtype_size(p.in_dt);
    const bool at = layout_a_transposed(p.layout), kn = layout_b_kn(p.layout);
    const bool exact = p.M % c.bm == 0 && p.N % c.bn == 0 && kper * p.split == p.K &&
                       (at ? p.K * p.M * es : (int64_t)c.bm * p.K * es) < INT32_MAX &&
                       (kn ? p.K * p.N * es : (int64_t)c.bn * p.K * es) < INT32_MAX;
    p.stages = 0;
    if (c.dl > 0 && p.in_dt != TLG_F32 && p.layout == TLG_NK && exact && (kper / c.bk) % c.dl == 0)
        p.stages = c.dl;
    // Persistent workgroups: exact fit, no split, an even number of slices.
    p.persist = c.pers && (p.stages == 0 || p.stages == 2) && exact && p.split == 1 && (kper / c.bk) % 2 == 0 &&
                kper >= 2 * c.bk;
    return TLG_OK;
}

// Fill rule for shapes the table does not list: keep at least one
// workgroup per CU busy, splitting K when the output tiles alone cannot
// (small M·N against a long K, as in the narrow GPT-2 layers).
static int auto_plan(tlg_plan& p) {
    if (!rows_aligned16(p)) return fill_generic(p);
    if (p.layout == TLG_NK && p.M <= kStreamMaxM) return auto_stream(p);
    // Up to a few hundred rows with few output columns the stream kernel's
    // grid (16-column tiles × 32-row blocks) still fits one workgroup per CU:
    // latency-bound shapes with no LDS pipeline to fill.  Wider outputs make
    // every tile re-read X, and the tiled kernel with split-K wins.
    if (p.layout == TLG_NK && p.M <= kStreamMaxRows && ceil_div(p.N, 16) * ceil_div(p.M, 32) <= kNumCUs)
        return auto_stream(p);
    // Outputs that fill every CU with 256×256 tiles take them: half the
    // operand bytes per flop of 128×128 (square 4096 bf16 → bf16 on MI355X:
    // 145 µs with 128×128, ~111 µs with 256×256).
    const int huge = p.in_dt == TLG_F32 ? 5 : 4;
    const TileCfg& ch = tiled_cfg(p.in_dt, huge);
    if (p.M % ch.bm == 0 && p.N % ch.bn == 0 && ceil_div(p.M, ch.bm) * ceil_div(p.N, ch.bn) >= kNumCUs &&
        fill_tiled(p, huge, 1) == TLG_OK)
        return TLG_OK;
    const int big = 0, small = 1;
    const TileCfg& cb = tiled_cfg(p.in_dt, big);
    const int64_t tiles_big = ceil_div(p.M, cb.bm) * ceil_div(p.N, cb.bn);
    if (tiles_big >= kNumCUs) return fill_tiled(p, big, 1);
    const TileCfg& cs = tiled_cfg(p.in_dt, small);
    const int64_t tiles_small = ceil_div(p.M, cs.bm) * ceil_div(p.N, cs.bn);
    const int64_t ksteps = ceil_div(p.K, cs.bk);
    int split = 1;
    while (tiles_small * split < kNumCUs && ksteps / (2 * split) >= 4) split *= 2;
    return fill_tiled(p, small, split);
}

}  // namespace tlg

using namespace tlg;

extern "C" {

int gemm_plan_ex(tlg_plan_t* out, int64_t M, int64_t N, int64_t K, tlg_dtype in_dt, tlg_dtype out_dt,
                 tlg_layout layout, uint32_t epi_flags, const tlg_plan_opts* opts) {
    if (!out) {
        set_error("gemm_plan: out is NULL");
        return TLG_ERR_INVALID_ARG;
    }
    *out = nullptr;
    if (M < 1 || N < 1 || K < 1) {
        set_error("gemm_plan: M, N, K must be >= 1 (got %lld, %lld, %lld)", (long long)M, (long long)N,
                  (long long)K);
        return TLG_ERR_INVALID_ARG;
    }
    if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) {
        set_error("gemm_plan: dimensions of 2^31 or more are not supported");
        return TLG_ERR_UNSUPPORTED;
    }
    if ((int)in_dt < TLG_F32 || (int)in_dt > TLG_BF16 || (int)out_dt < TLG_F32 || (int)out_dt > TLG_BF16) {
        set_error("gemm_plan: unknown dtype (%d, %d)", (int)in_dt, (int)out_dt);
        return TLG_ERR_INVALID_ARG;
    }
    if ((int)layout < TLG_NK || (int)layout > TLG_AT_KN) {
        set_error("gemm_plan: unknown layout %d", (int)layout);
        return TLG_ERR_INVALID_ARG;
    }
    if (epi_flags & ~(uint32_t)(TLG_EPI_BIAS | TLG_EPI_GELU_TANH | TLG_EPI_RESIDUAL)) {
        set_error("gemm_plan: unknown epilogue flags 0x%x", epi_flags);
        return TLG_ERR_INVALID_ARG;
    }
    if (layout_a_transposed(layout) && (epi_flags & (TLG_EPI_BIAS | TLG_EPI_GELU_TANH))) {
        set_error("gemm_plan: the transposed-A layouts take no bias or GELU (only TLG_EPI_RESIDUAL)");
        return TLG_ERR_UNSUPPORTED;
    }
    if (!valid_pair(in_dt, out_dt)) {
        set_error("gemm_plan: unsupported (in, out) dtype pair (%d, %d)", (int)in_dt, (int)out_dt);
        return TLG_ERR_UNSUPPORTED;
    }
    tlg_plan p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.in_dt = in_dt;
    p.out_dt = out_dt;
    p.layout = layout;
    p.epi = epi_flags;
    p.rowb = 0;

    const int variant = opts ? opts->variant : TLG_VARIANT_AUTO;
    const int split = opts ? opts->split_k : 0;
    const int tile_sel = opts ? opts->tile : 0;
    if (split < 0 || tile_sel < 0) {
        set_error("gemm_plan: negative split_k or tile");
        return TLG_ERR_INVALID_ARG;
    }
    int rc;
    if (variant == TLG_VARIANT_AUTO) {
        const TableRow* row = (split == 0 && tile_sel == 0)
                                  ? table_lookup(M, N, K, in_dt, out_dt, layout, epi_flags & kEpiKernel)
                                  : nullptr;
        if (row) {
            rc = row->variant == TLG_VARIANT_STREAM  ? fill_stream(p, row->tile, row->split)
                 : row->variant == TLG_VARIANT_TILED ? fill_tiled(p, row->tile, row->split)
                                                     : fill_generic(p);
        } else if (split != 0 || tile_sel != 0) {
            set_error("gemm_plan: split_k/tile overrides need an explicit variant");
            return TLG_ERR_INVALID_ARG;
        } else {
            rc = auto_plan(p);
        }
    } else if (variant == TLG_VARIANT_GENERIC) {
        if (split > 1 || tile_sel > 1) {
            set_error("generic kernel has one tile and no split");
            return TLG_ERR_UNSUPPORTED;
        }
        rc = fill_generic(p);
    } else if (variant == TLG_VARIANT_STREAM) {
        if (tile_sel == 0 && split == 0)
            rc = p.M <= kStreamMaxRows && p.layout == TLG_NK && rows_aligned16(p) ? auto_stream(p)
                                                                                : fill_stream(p, 0, 0);
        else
            rc = fill_stream(p, tile_sel ? tile_sel - 1 : 2, split);
    } else if (variant == TLG_VARIANT_TILED) {
        rc = fill_tiled(p, tile_sel ? tile_sel - 1 : 0, split);
    } else {
        set_error("gemm_plan: unknown variant %d", variant);
        return TLG_ERR_INVALID_ARG;
    }
    if (rc != TLG_OK) return rc;
    tlg_plan* h = new (std::nothrow) tlg_plan(p);
    if (!h) {
        set_error("gemm_plan: out of host memory");
        return TLG_ERR_NOMEM;
    }
    *out = h;
    return TLG_OK;
}

int gemm_plan(tlg_plan_t* out, int64_t M, int64_t N, int64_t K, tlg_dtype in_dt, tlg_dtype out_dt,
              tlg_layout layout, uint32_t epi_flags) {
    return gemm_plan_ex(out, M, N, K, in_dt, out_dt, layout, epi_flags, nullptr);
}

size_t gemm_workspace_size(tlg_plan_t p) { return p ? p->ws_bytes : 0; }

int gemm_plan_info(tlg_plan_t p, tlg_plan_info* info) {
    if (!p || !info) {
        set_error("gemm_plan_info: NULL argument");
        return TLG_ERR_INVALID_ARG;
    }
    info->variant = p->variant;
    info->tile_m = p->bm;
    info->tile_n = p->bn;
    info->tile_k = p->bk;
    info->split_k = p->split;
    info->threads = p->threads;
    info->workgroups = p->grid_x * p->grid_y * p->grid_z +
                       (p->launches > 1 ? ceil_div(p->M * p->N, 256 * 4) : 0);  // + split-K reducer
    info->launches = p->launches;
    info->workspace_bytes = p->ws_bytes;
    return TLG_OK;
}

int gemm_destroy(tlg_plan_t p) {
    delete p;
    return TLG_OK;
}

int gemm_plan_describe(tlg_plan_t p, char* buf, size_t n) {
    if (!p) {
        set_error("gemm_plan_describe: NULL plan");
        return TLG_ERR_INVALID_ARG;
    }
    static const char* vname[] = {"generic", "stream", "tiled"};
    static const char* dname[] = {"f32", "f16", "bf16"};
    static const char* lname[] = {"NK", "KN", "AT_NK", "AT_KN"};
    char tmp[320];
    int len = snprintf(tmp, sizeof tmp,
                       "variant=%s M=%lld N=%lld K=%lld in=%s out=%s layout=%s epi=%s%s%s tile=%dx%dx%d "
                       "split=%d threads=%d grid=%lldx%lldx%lld launches=%d ws=%zu%s%s%s",
                       vname[p->variant], (long long)p->M, (long long)p->N, (long long)p->K,
                       dname[p->in_dt], dname[p->out_dt], lname[p->layout],
                       (p->epi & TLG_EPI_BIAS) ? "bias" : "none", (p->epi & TLG_EPI_GELU_TANH) ? "+gelu" : "",
                       (p->epi & TLG_EPI_RESIDUAL) ? "+res" : "", p->bm, p->bn, p->bk, p->split,
                       p->threads, (long long)p->grid_x, (long long)p->grid_y, (long long)p->grid_z,
                       p->launches, p->ws_bytes,
                       (p->variant == TLG_VARIANT_TILED && p->stages) || (p->variant == TLG_VARIANT_STREAM && kStream[p->tile].dl)
                           ? " load=direct"
                           : "",
                       p->variant == TLG_VARIANT_TILED && p->persist ? " persistent" : "",
                       p->variant == TLG_VARIANT_STREAM && kStream[p->tile].pipe ? " pipelined" : "");
    if (buf && n) {
        size_t c = (size_t)len < n - 1 ? (size_t)len : n - 1;
        memcpy(buf, tmp, c);
        buf[c] = '\0';
    }
    return len;
}

const char* gemm_status_string(int status) {
    switch (status) {
    case TLG_OK: return "ok";
    case TLG_ERR_INVALID_ARG: return "invalid argument";
    case TLG_ERR_UNSUPPORTED: return "unsupported";
    case TLG_ERR_MISALIGNED: return "misaligned pointer";
    case TLG_ERR_WORKSPACE: return "workspace missing or too small";
    case TLG_ERR_NOMEM: return "out of host memory";
    case TLG_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char* gemm_last_error(void) { return g_last_error; }

}  // extern "C"
