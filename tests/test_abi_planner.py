"""C-ABI and planner checks that need no GPU (the planner is host-only)."""

import ctypes
import os
import re

import pytest

from dense_gemm_transformer_amd import tlgemm as t

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tlgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(t.EXPORTS)
    lib = ctypes.CDLL(t.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_ceiling_probe_library_exports_its_header():
    """The benchmark's probe library loads without a GPU and exports what include/tlgceil.h declares."""
    hdr = os.path.join(os.path.dirname(HEADER), "tlgceil.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tlg_ceil_\w+)\s*\(", text)))
    assert names == ["tlg_ceil_empty", "tlg_ceil_mfma", "tlg_ceil_mfma_clock", "tlg_ceil_read",
                     "tlg_ceil_read_l2", "tlg_ceil_wall_clock_khz"]
    lib = ctypes.CDLL(os.path.join(os.path.dirname(t.LIB_PATH), "libtlgceil.so"))
    for name in names:
        assert hasattr(lib, name), name


def _plan(*a, **k):
    return t.Plan.create(*a, **k)


def test_narrow_fp16_goes_to_stream():
    p = _plan(16, 4096, 4096, "f16", "f16")
    i = p.info
    assert i.variant == t.VARIANT_STREAM and i.workgroups == 256 and i.threads == 512
    # 16-row tiles, 8 waves split all of K inside the workgroup: no split across workgroups
    assert (i.tile_n, i.tile_k, i.split_k, i.launches, i.workspace_bytes) == (16, 4096, 1, 1, 0)


def test_stream_split_rules():
    # narrow N: 128-row tiles with K split across workgroups
    i = _plan(16, 768, 3072, "f16").info
    assert (i.variant, i.tile_n, i.split_k) == (t.VARIANT_STREAM, 128, 6)
    assert i.workspace_bytes == 65536 + 6 * 6 * 128 * 16 * 4  # the counter block, then fragment-order partials
    i = _plan(5, 1000, 1000, "f32").info  # fp32 chunk of 256: 4 chunks over 8 tiles
    assert (i.variant, i.split_k) == (t.VARIANT_STREAM, 4)
    i = _plan(16, 4096, 4096, "f16", variant=t.VARIANT_STREAM, tile=3, split_k=1).info
    assert (i.split_k, i.workspace_bytes, i.workgroups) == (1, 0, 32)
    with pytest.raises(t.TlgError):
        _plan(16, 4096, 4096, "f16", variant=t.VARIANT_STREAM, tile=3, split_k=17)
    i = _plan(16, 4096, 4096, "f16", variant=t.VARIANT_STREAM, tile=3, split_k=3).info  # 8 chunks over 3 splits
    assert i.split_k == 3
    # X for 64 rows over a 4096-wide chunk does not fit in LDS
    with pytest.raises(t.TlgError) as e:
        _plan(64, 4096, 4096, "f16", variant=t.VARIANT_STREAM, tile=1)
    assert e.value.status == t.ERR_UNSUPPORTED
    assert _plan(64, 4096, 4096, "f16").info.variant == t.VARIANT_STREAM
    assert _plan(33, 4096, 4096, "bf16").info.tile_m == 64


def _table_rows():
    """Rows of the measured dispatch table: (M, N, K, in, out, layout, epi, variant, tile, split)."""
    path = os.path.join(os.path.dirname(t.__file__), "csrc", "dispatch_table.inc")
    rows = []
    for line in open(path):
        m = re.match(r"\{(\d+), (\d+), (\d+), (\d), (\d), (\d), (\d)u, (\d), (\d+), (\d+)\},", line.strip())
        if m and int(m.group(1)) > 0:
            rows.append(tuple(int(x) for x in m.groups()))
    return rows


def test_dispatch_table_rows_drive_the_planner():
    """Every measured row is what the default plan of its exact shape becomes."""
    rows = _table_rows()
    assert len(rows) == 31  # 15 forward shapes, 16 backward (dX and dW of four linears, fp32 and bf16)
    assert sum(r[5] == 3 for r in rows) == 8  # the weight gradients: transposed first operand
    dt, lay = {0: "f32", 1: "f16", 2: "bf16"}, {0: "NK", 1: "KN", 2: "AT_NK", 3: "AT_KN"}
    for M, N, K, i, o, l, epi, variant, tile, split in rows:
        args = (M, N, K, dt[i], dt[o], lay[l], bool(epi & 1), bool(epi & 2))
        want = _plan(*args, variant=variant, tile=tile + 1, split_k=split).describe()
        assert _plan(*args).describe() == want


def test_square_fp32_goes_to_tiled():
    p = _plan(4096, 4096, 4096, "f32", "f32", "KN")
    i = p.info
    assert i.variant == t.VARIANT_TILED and i.split_k == 1 and i.workspace_bytes == 0  # measured table row
    # an unlisted square shape falls back to the fill rule's 128×128 tiles
    i = _plan(2048, 2048, 2048, "f32", "f32", "KN").info
    assert (i.tile_m, i.tile_n, i.workgroups) == (128, 128, 256)
    # outputs that 256×256 tiles alone spread over every CU take them
    i = _plan(4096, 4096, 4096, "bf16", "bf16", "KN").info  # no table row for bf16 output
    assert (i.tile_m, i.tile_n, i.workgroups, i.split_k) == (256, 256, 256, 1)
    i = _plan(8192, 4096, 1024, "f32", "f32", "NK").info
    assert (i.tile_m, i.tile_n, i.workgroups, i.threads) == (256, 256, 512, 512)
    i = _plan(4096, 4096 + 128, 4096, "bf16", "bf16", "KN").info  # ragged: the fill rule
    assert (i.tile_m, i.tile_n) == (128, 128)


def test_dispatch_table_rows_are_exact_shape_matches():
    # the table lists the 128x768x768 fp32 layer with bias; without bias the fill rule applies
    with_bias = _plan(128, 768, 768, "f32", bias=True).describe()
    assert "variant=stream" in with_bias
    assert _plan(128, 2304, 768, "f32", bias=True).info.variant == t.VARIANT_STREAM  # measured row
    assert _plan(128, 2304, 768, "f32").info.variant == t.VARIANT_TILED  # no table row without bias


@pytest.mark.parametrize("N,K", [(2304, 768), (768, 768), (3072, 768), (768, 3072)])
def test_gpt2_layer_shapes_m128(N, K):
    """Without a table row (no bias): 768 outputs fit one stream grid (16-column
    tiles × 32-row blocks, all of K per workgroup); wider layers take the tiled
    kernel with split-K.  With bias the measured rows apply (checked against the
    table itself above); each is a single-pass stream plan or a split-K plan."""
    i = _plan(128, N, K, "f32").info
    if N == 768:
        assert i.variant == t.VARIANT_STREAM and (i.tile_m, i.tile_n) == (32, 16)
        assert i.workgroups == (N // 16) * 4 and i.split_k == 1 and i.workspace_bytes == 0
    else:
        assert i.variant == t.VARIANT_TILED and i.split_k > 1
        tiles = -(-128 // i.tile_m) * -(-N // i.tile_n)
        assert tiles * i.split_k >= 256 or K // (i.tile_k * i.split_k) < 8
        assert i.workspace_bytes == 65536 + i.split_k * 128 * N * 4  # counter block (left alone), partials
    j = _plan(128, N, K, "f32", bias=True, gelu=(N == 3072)).info
    assert (j.variant == t.VARIANT_STREAM and j.workspace_bytes == 0) or j.split_k > 1


def test_large_m_goes_to_tiled():
    for N, K in [(2304, 768), (768, 768), (3072, 768), (768, 3072)]:
        i = _plan(8192, N, K, "bf16", bias=True).info
        assert i.variant == t.VARIANT_TILED and i.split_k == 1


def test_misaligned_rows_go_to_generic():
    assert _plan(8, 10, 7, "f32").info.variant == t.VARIANT_GENERIC          # K*4 not a multiple of 16
    assert _plan(8, 10, 12, "f16").info.variant == t.VARIANT_GENERIC         # K*2 = 24
    assert _plan(200, 10, 16, "f32", layout="KN").info.variant == t.VARIANT_GENERIC  # N*4 = 40


def test_forced_variants_and_errors():
    p = _plan(100, 64, 64, "bf16", variant=t.VARIANT_GENERIC)
    assert p.info.variant == t.VARIANT_GENERIC
    with pytest.raises(t.TlgError) as e:
        _plan(300, 64, 64, "bf16", variant=t.VARIANT_STREAM)  # more rows than the stream kernel walks
    assert e.value.status == t.ERR_UNSUPPORTED
    assert _plan(100, 64, 64, "bf16", variant=t.VARIANT_STREAM).info.variant == t.VARIANT_STREAM
    with pytest.raises(t.TlgError) as e:
        _plan(10, 64, 64, "f32", layout="KN", variant=t.VARIANT_STREAM)
    assert e.value.status == t.ERR_UNSUPPORTED
    p = _plan(100, 64, 64, "f32", variant=t.VARIANT_TILED, split_k=3, tile=2)
    i = p.info
    assert (i.split_k, i.tile_m, i.launches, i.workspace_bytes) == (3, 64, 2, 65536 + 3 * 100 * 64 * 4)
    with pytest.raises(t.TlgError) as e:
        _plan(100, 64, 64, "f32", variant=t.VARIANT_TILED, split_k=5)  # 4 slices of 16
    assert e.value.status == t.ERR_UNSUPPORTED
    with pytest.raises(t.TlgError) as e:
        _plan(100, 64, 64, "f32", split_k=2)  # override without a variant
    assert e.value.status == t.ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((0, 1, 1, "f32"), t.ERR_INVALID_ARG),
    ((1, -3, 1, "f32"), t.ERR_INVALID_ARG),
    ((1, 1, 0, "f32"), t.ERR_INVALID_ARG),
    ((1, 1, 1, 7), t.ERR_INVALID_ARG),
])
def test_bad_shapes_and_dtypes(args, status):
    with pytest.raises(t.TlgError) as e:
        t.gemm_plan(*args)
    assert e.value.status == status


def test_unsupported_pairs_and_flags():
    with pytest.raises(t.TlgError) as e:
        t.gemm_plan(4, 4, 4, "f32", "f16")
    assert e.value.status == t.ERR_UNSUPPORTED
    with pytest.raises(t.TlgError) as e:
        t.gemm_plan(4, 4, 4, "f16", "bf16")
    assert e.value.status == t.ERR_UNSUPPORTED
    with pytest.raises(t.TlgError) as e:  # flags 1, 2, 4 are defined; 8 is not
        t.gemm_plan(4, 4, 4, "f32", "f32", "NK", 8)
    assert e.value.status == t.ERR_INVALID_ARG
    with pytest.raises(t.TlgError) as e:  # layouts 0..3 are defined
        t.gemm_plan(4, 4, 4, "f32", "f32", 4, 0)
    assert e.value.status == t.ERR_INVALID_ARG


def test_null_handling_and_describe():
    lib = t.lib()
    assert lib.gemm_plan(None, 1, 1, 1, 0, 0, 0, 0) == t.ERR_INVALID_ARG
    h = ctypes.c_void_p(1234)
    assert lib.gemm_plan(ctypes.byref(h), 0, 1, 1, 0, 0, 0, 0) == t.ERR_INVALID_ARG
    assert h.value is None  # *out is cleared on error
    assert lib.gemm_destroy(None) == t.OK
    assert lib.gemm_workspace_size(None) == 0
    assert lib.gemm_plan_info(None, None) == t.ERR_INVALID_ARG
    p = _plan(16, 4096, 4096, "f16")
    full = p.describe()
    assert "variant=stream" in full and "M=16" in full
    buf = ctypes.create_string_buffer(10)
    n = lib.gemm_plan_describe(p.handle, buf, 10)
    assert n == len(full) and buf.value.decode() == full[:9]
    assert t.gemm_status_string(t.ERR_MISALIGNED) == "misaligned pointer"
    assert t.gemm_status_string(42) == "unknown status"


def test_run_argument_errors_without_launch():
    """gemm_run rejects bad arguments before touching the device."""
    p = _plan(16, 64, 64, "f32", bias=True)
    lib = t.lib()
    good = 1 << 20
    assert lib.gemm_run(None, good, good, good, good, None, 0, None) == t.ERR_INVALID_ARG
    assert lib.gemm_run(p.handle, None, good, good, good * 4, None, 0, None) == t.ERR_INVALID_ARG
    assert lib.gemm_run(p.handle, good, 2 * good, None, 3 * good, None, 0, None) == t.ERR_INVALID_ARG  # bias missing
    assert lib.gemm_run(p.handle, good + 4, 2 * good, 4 * good, 3 * good, None, 0, None) == t.ERR_MISALIGNED
    assert lib.gemm_run(p.handle, good, 2 * good, 4 * good, good + 64, None, 0, None) == t.ERR_INVALID_ARG  # Y aliases X
    q = _plan(128, 768, 768, "f32", variant=t.VARIANT_TILED, split_k=4, tile=2)
    big = 1 << 24
    assert lib.gemm_run(q.handle, big, 2 * big, None, 3 * big, None, 0, None) == t.ERR_WORKSPACE
    assert lib.gemm_run(q.handle, big, 2 * big, None, 3 * big, 8 * big, 16, None) == t.ERR_WORKSPACE
    assert "workspace" in t.gemm_last_error()
    ws = q.workspace_size
    for clash in (big, 2 * big):  # the workspace over X, then over W: the partials would overwrite inputs
        assert lib.gemm_run(q.handle, big, 2 * big, None, 3 * big, clash, ws, None) == t.ERR_INVALID_ARG
        assert "overlaps an input" in t.gemm_last_error()


# --- transposed first operand and the residual -------------------------------------

def test_transposed_first_operand_layouts_plan():
    for layout in ("AT_NK", "AT_KN"):
        i = _plan(768, 3072, 8192, "bf16", "bf16", layout).info  # dW-shaped: M, N = out, in; K = tokens
        assert i.variant == t.VARIANT_TILED
        assert f"layout={layout} " in _plan(768, 3072, 8192, "f32", "f32", layout).describe()
        # rows of the [K][M] operand must be 16-byte aligned for the tiled kernel
        assert _plan(100, 64, 64, "f32", "f32", layout).info.variant == t.VARIANT_TILED
        assert _plan(99, 64, 64, "f32", "f32", layout).info.variant == t.VARIANT_GENERIC
        with pytest.raises(t.TlgError) as e:
            _plan(16, 4096, 4096, "f16", "f16", layout, variant=t.VARIANT_STREAM)
        assert e.value.status == t.ERR_UNSUPPORTED


def test_transposed_first_operand_takes_no_bias_or_gelu():
    for bias, gelu in ((True, False), (False, True), (True, True)):
        with pytest.raises(t.TlgError) as e:
            _plan(64, 64, 64, "f32", "f32", "AT_NK", bias, gelu)
        assert e.value.status == t.ERR_UNSUPPORTED
    assert "+res" in _plan(64, 64, 64, "f32", "f32", "AT_KN", residual=True).describe()


def test_residual_flag_plans_like_its_base_epilogue():
    # the residual is a run-time argument of the same kernels: the measured rows still apply
    for args in ((16, 4096, 4096, "f16", "f16"), (8192, 3072, 768, "bf16", "bf16", "NK", True, True)):
        base = _plan(*args).describe()
        res = _plan(*args, residual=True).describe()
        assert res.replace("+res", "") == base


def test_bad_layout_and_flags_rejected():
    h = ctypes.c_void_p()
    lib = ctypes.CDLL(t.LIB_PATH)
    assert lib.gemm_plan(ctypes.byref(h), 8, 8, 8, 0, 0, 4, 0) == t.ERR_INVALID_ARG
    assert lib.gemm_plan(ctypes.byref(h), 8, 8, 8, 0, 0, 0, 8) == t.ERR_INVALID_ARG
    assert lib.gemm_plan(ctypes.byref(h), 8, 8, 8, 0, 0, 2, 4) == t.OK
    lib.gemm_destroy(h)


def test_stream_split_counter_block_limit():
    """Split stream plans keep one arrival counter per (row block, tile) in the workspace's fixed
    64 KiB counter block; a forced split with more tiles than counters is refused, not overrun."""
    i = _plan(16, 16384 * 16, 8192, "f16", variant=t.VARIANT_STREAM, tile=1, split_k=2).info  # 16384 tiles: fits
    assert i.split_k == 2 and i.workspace_bytes == 65536 + 2 * 16384 * 16 * 16 * 4
    with pytest.raises(t.TlgError) as e:
        _plan(16, 16385 * 16, 8192, "f16", variant=t.VARIANT_STREAM, tile=1, split_k=2)
    assert e.value.status == t.ERR_UNSUPPORTED and "counters" in str(e.value)
    i = _plan(16, 16385 * 16, 8192, "f16", variant=t.VARIANT_STREAM, tile=1, split_k=1).info  # no split: no counters
    assert i.workspace_bytes == 0


def test_stream_weight_rows_in_lds_planning():
    """The LDS-resident stream tile (option 6): 16-bit, M <= 16, K a multiple of 512 up to 4096, no split;
    the planner takes it for such narrow layers with enough 16-row tiles to fill the chip."""
    i = _plan(16, 4096, 2048, "bf16").info
    assert (i.variant, i.tile_n, i.tile_k, i.split_k, i.workgroups, i.threads) == (t.VARIANT_STREAM, 16, 2048, 1, 256, 512)
    assert "tile=16x16x2048 " in _plan(16, 4096, 2048, "bf16").describe()
    assert _plan(16, 4096, 2048, "bf16").describe().endswith(" load=direct")
    assert "load=direct" not in _plan(16, 4096, 2048, "bf16", variant=t.VARIANT_STREAM, tile=1).describe()
    for args in [(16, 64, 512, "f32"), (17, 64, 512, "f16"), (16, 64, 520, "f16"), (16, 64, 4608, "bf16")]:
        with pytest.raises(t.TlgError) as e:
            _plan(*args, variant=t.VARIANT_STREAM, tile=6)
        assert e.value.status == t.ERR_UNSUPPORTED
    with pytest.raises(t.TlgError):
        _plan(16, 64, 1024, "f16", variant=t.VARIANT_STREAM, tile=6, split_k=2)
    assert _plan(16, 4096, 4608, "f16").info.tile_k != 4608  # too long for LDS: the register-streaming tile


def test_search_walks_every_tile_option():
    """The option counts the measured search walks match the planner's tile lists: the last option of each
    list plans, the one past it is refused (16-bit tiled list; fp32's is shorter)."""
    from dense_gemm_transformer_amd import tune

    p = t.Plan.create(16, 4096, 4096, "f16", "f16", "NK", variant=t.VARIANT_STREAM, tile=tune.STREAM_OPTIONS)
    p.close()
    with pytest.raises(t.TlgError):
        t.Plan.create(16, 4096, 4096, "f16", "f16", "NK", variant=t.VARIANT_STREAM, tile=tune.STREAM_OPTIONS + 1)
    p = t.Plan.create(512, 576, 768, "bf16", "bf16", "NK", variant=t.VARIANT_TILED, tile=tune.TILED_OPTIONS)
    p.close()
    with pytest.raises(t.TlgError):
        t.Plan.create(512, 576, 768, "bf16", "bf16", "NK", variant=t.VARIANT_TILED, tile=tune.TILED_OPTIONS + 1)
    p = t.Plan.create(512, 576, 768, "f32", "f32", "NK", variant=t.VARIANT_TILED, tile=10)  # fp32's last entry
    p.close()
    with pytest.raises(t.TlgError):
        t.Plan.create(512, 576, 768, "f32", "f32", "NK", variant=t.VARIANT_TILED, tile=11)


def test_wide_128x192_tiles_plan():
    """Tiled options 12 and 13 (128×192, persistent; staged and direct-load): exact fits at the GPT-2 widths
    plan persistent, the direct-load entry fills LDS by direct loads where the operands allow it."""
    p = t.Plan.create(8192, 768, 3072, "bf16", "bf16", "NK", bias=True, variant=t.VARIANT_TILED, tile=12)
    i = p.info
    assert (i.tile_m, i.tile_n, i.tile_k, i.threads) == (128, 192, 64, 256)
    assert "persistent" in p.describe() and "load=direct" not in p.describe()
    p.close()
    p = t.Plan.create(8192, 2304, 768, "bf16", "bf16", "NK", bias=True, variant=t.VARIANT_TILED, tile=13)
    assert "persistent" in p.describe() and "load=direct" in p.describe(), p.describe()
    p.close()
    # a transposed first operand keeps staged loads; [K][N] weights are refused (24 vectors per row of the
    # tile against 256 threads); a split or a ragged N is not persistent
    p = t.Plan.create(2048, 768, 768, "bf16", "bf16", "AT_NK", variant=t.VARIANT_TILED, tile=13)
    assert "persistent" in p.describe() and "load=direct" not in p.describe(), p.describe()
    p.close()
    for layout in ("KN", "AT_KN"):
        with pytest.raises(t.TlgError) as e:
            t.Plan.create(2048, 768, 768, "bf16", "bf16", layout, variant=t.VARIANT_TILED, tile=12)
        assert e.value.status == t.ERR_UNSUPPORTED
    for (M, N, K), split in [((512, 576, 1536), 2), ((512, 500, 768), 1)]:
        p = t.Plan.create(M, N, K, "bf16", "bf16", "NK", variant=t.VARIANT_TILED, tile=12, split_k=split)
        assert "persistent" not in p.describe(), p.describe()
        p.close()


def test_stream_pipelined_options_planning():
    """Pipelined stream options (entries 10-14): the description says so, the row blocks are the option's own
    whatever M is, the automatic split spreads the column tiles over the 256 CUs in whole chunks (here one or
    two chunks per split, little left to overlap), and a forced split keeps several chunks per workgroup.  Their two X buffers fit LDS for fp32 and 16-bit inputs."""
    for tile, (bn, bm, bk32) in {11: (48, 32, 384), 12: (48, 32, 192), 13: (32, 16, 384), 14: (16, 16, 384),
                                 15: (32, 16, 192)}.items():
        for M in (1, 16, 40, 128, 256):
            p = _plan(M, 768, 768, "f32", variant=t.VARIANT_STREAM, tile=tile, split_k=1)
            i = p.info
            assert p.describe().endswith(" pipelined"), p.describe()
            assert (i.tile_m, i.tile_n, i.tile_k, i.split_k) == (bm, bn, bk32, 1)
            assert i.workgroups == -(-768 // bn) * -(-M // bm) and i.workspace_bytes == 0  # grid z walks row blocks
        auto = _plan(128, 768, 3072, "f32", variant=t.VARIANT_STREAM, tile=tile).info
        s0 = min(-(-256 // (768 // bn)), 3072 // bk32, 16)  # the fill rule: 256 CUs over the column tiles
        kper = -(-(-(-3072 // s0)) // bk32) * bk32            # whole chunks per split
        assert auto.split_k == -(-3072 // kper)
        forced = _plan(128, 768, 3072, "f32", variant=t.VARIANT_STREAM, tile=tile, split_k=4).info
        assert forced.split_k == 4 and 3072 // 4 // forced.tile_k == 768 // bk32
        h = _plan(16, 4096, 4096, "bf16", variant=t.VARIANT_STREAM, tile=tile, split_k=1)
        assert h.info.tile_k == 2 * bk32 and h.describe().endswith(" pipelined")  # 16-byte loads: twice the k
    assert not _plan(128, 768, 768, "f32", variant=t.VARIANT_STREAM, tile=10, split_k=1).describe().endswith(
        " pipelined")
