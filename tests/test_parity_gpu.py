"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: max|Y - ref| / max|ref| <= 1e-5 for fp32 inputs and <= 1e-2 for
fp16/bf16 inputs (fp32 accumulation), the matmul error measure of "Writing a
CUDA matmul that catches cuBLAS" ("The measurement was nearly wrong").
Exact cases (identity and permutation weights, replicated rows, repeat
runs) must match bitwise.
"""

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs, tlgemm
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import TOL, device_case, normalized_error, run_case, to_device, to_f64  # noqa: E402

PAIRS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]
EPIS = [(False, False), (True, False), (False, True), (True, True)]


def _check(case, **force):
    Y, desc = run_case(case, **force)
    ref = oracle.linear_case(case)
    err = normalized_error(to_f64(Y), ref)
    assert err <= TOL[case.in_dtype], f"{desc}: err {err:.3e}"
    return Y, desc


def _case(seed, M, N, K, pair, layout="NK", epi=(False, False)):
    return inputs.random_case(seed, M, N, K, pair[0], pair[1], layout, bias=epi[0], gelu=epi[1])


# --- every variant, dtype pair, layout and epilogue at ragged sizes ---------------------

@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("layout", ["NK", "KN"])
@pytest.mark.parametrize("epi", EPIS, ids=["none", "bias", "gelu", "bias+gelu"])
def test_generic(pair, layout, epi):
    for shape in [(1, 1, 1), (37, 70, 29), (130, 65, 100)]:
        c = _case(1, *shape, pair, layout, epi)
        _, desc = _check(c, variant=tlgemm.VARIANT_GENERIC)
        assert "variant=generic" in desc


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("epi", EPIS, ids=["none", "bias", "gelu", "bias+gelu"])
@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 13, 14, 15])
def test_stream(pair, epi, tile):
    ran = 0
    for M, N, K in [(1, 16, 8), (16, 48, 512), (5, 50, 520), (17, 36, 1032), (40, 100, 264), (64, 16, 4096),
                    (3, 300, 3000), (100, 40, 264), (130, 36, 520)]:
        c = _case(2, M, N, K, pair, "NK", epi)
        try:
            _, desc = _check(c, variant=tlgemm.VARIANT_STREAM, tile=tile)
        except tlgemm.TlgError as e:  # configurations whose X chunk does not fit in LDS for this M
            assert e.status == tlgemm.ERR_UNSUPPORTED and "LDS" in str(e), str(e)
            continue
        assert "variant=stream" in desc
        ran += 1
    assert ran >= 2


@pytest.mark.parametrize("pair", PAIRS[1:], ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("epi", EPIS, ids=["none", "bias", "gelu", "bias+gelu"])
def test_stream_weight_rows_in_lds(pair, epi):
    """Stream option 6: the 16 weight rows of a tile in LDS by direct loads, X in registers (M <= 16,
    K a multiple of 512 up to 4096), ragged N and M, with and without the residual."""
    for (M, N, K), res in [((1, 16, 512), False), ((16, 48, 512), True), ((5, 50, 1024), False),
                           ((16, 4096, 4096), False), ((13, 100, 3584), True), ((16, 264, 2048), False)]:
        c = inputs.random_case(23, M, N, K, pair[0], pair[1], "NK", bias=epi[0], gelu=epi[1], residual=res)
        _, desc = _check(c, variant=tlgemm.VARIANT_STREAM, tile=6)
        assert "variant=stream" in desc and f"tile=16x16x{K} " in desc, desc


@pytest.mark.parametrize("tile", [11, 12, 13, 14, 15])
def test_stream_pipelined(tile):
    """Pipelined stream options (chunk c + 1's loads ahead of chunk c's products, two X buffers and two
    register sets alternating): every linear of the 128-row GPT-2 layer and the 128×768×768 linear with
    one split (2 to 16 chunks per workgroup), all outputs against the oracle; then ragged M, N and K,
    16-bit inputs and a grid split on top (the automatic split gives one chunk per split)."""
    for c in [inputs.workload_fp32_linear_128x768()] + inputs.workload_gpt2_layer(M=128, dtype="f32"):
        _, desc = _check(c, variant=tlgemm.VARIANT_STREAM, tile=tile, split_k=1)
        assert desc.endswith(" pipelined") and " split=1 " in desc, desc
    for (M, N, K), pair, split, epi in [((37, 70, 1000), ("f32", "f32"), 1, (True, True)),
                                        ((100, 130, 2056), ("f32", "f32"), 2, (True, False)),
                                        ((16, 200, 3000), ("f16", "f16"), 1, (False, True)),
                                        ((33, 96, 4104), ("bf16", "f32"), 2, (True, True))]:
        c = _case(24, M, N, K, pair, "NK", epi)
        _, desc = _check(c, variant=tlgemm.VARIANT_STREAM, tile=tile, split_k=split)
        assert desc.endswith(" pipelined"), desc


def test_stream_weight_rows_in_lds_limits():
    """Shapes outside the LDS-resident tile are refused, not run."""
    for args in [(16, 64, 512, "f32"), (17, 64, 512, "f16"), (16, 64, 520, "f16"), (16, 64, 4608, "bf16")]:
        with pytest.raises(tlgemm.TlgError) as e:
            tlgemm.Plan.create(*args, variant=tlgemm.VARIANT_STREAM, tile=6)
        assert e.value.status == tlgemm.ERR_UNSUPPORTED
    with pytest.raises(tlgemm.TlgError) as e:
        tlgemm.Plan.create(16, 64, 1024, "f16", variant=tlgemm.VARIANT_STREAM, tile=6, split_k=2)
    assert e.value.status == tlgemm.ERR_UNSUPPORTED


@pytest.mark.parametrize("pair", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32")], ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_stream_forced_split(pair, split):
    """Cross-workgroup split-K with the last-arriving reduction, ragged K and N tails."""
    for M, N, K in [(16, 260, 3000), (33, 520, 2048), (64, 132, 4104), (130, 100, 2056)]:
        c = _case(5, M, N, K, pair, "NK", (True, True))
        ck = 512 if pair[0] != "f32" else 256
        if split > -(-K // ck):  # more splits than K chunks: refused by the planner
            with pytest.raises(tlgemm.TlgError) as e:
                run_case(c, variant=tlgemm.VARIANT_STREAM, tile=3, split_k=split)
            assert e.value.status == tlgemm.ERR_UNSUPPORTED
            continue
        _, desc = _check(c, variant=tlgemm.VARIANT_STREAM, tile=3, split_k=split)
        # each split covers whole chunks, so a split that would be empty is dropped
        kper = -(-(-(-K // split)) // ck) * ck
        assert f"split={-(-K // kper)} " in desc


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("layout", ["NK", "KN"])
@pytest.mark.parametrize("epi", EPIS, ids=["none", "bias", "gelu", "bias+gelu"])
def test_tiled(pair, layout, epi):
    for tile in range(1, 11 if pair[0] == "f32" else 14):
        if layout == "KN" and tile >= (9 if pair[0] == "f32" else 12):  # 128×192 takes no [K][N] weight
            with pytest.raises(tlgemm.TlgError):
                tlgemm.Plan.create(256, 384, 64, pair[0], pair[1], layout, variant=tlgemm.VARIANT_TILED, tile=tile)
            continue
        for (M, N, K), split in [((130, 136, 72), 1), ((256, 256, 256), 1), ((64, 64, 32), 1),
                                 ((200, 264, 400), 3), ((33, 520, 1024), 4)]:
            c = _case(3, M, N, K, pair, layout, epi)
            _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
            assert "variant=tiled" in desc


@pytest.mark.parametrize("tile", [7, 8, 9])
def test_tiled_direct_loads(tile):
    """Exact-fit 16-bit [M][K]·[N][K] tiles whose operands go straight into swizzled LDS stages.

    Long K (many stage rounds), split-K partials, every epilogue and both
    output widths; the plan must report the direct-load path.  K per split is
    a multiple of 768, a whole number of stage rounds.
    """
    for (M, N, K), split, epi, pair in [((512, 512, 1536), 1, (True, True), ("bf16", "bf16")),
                                        ((256, 512, 1536), 2, (True, False), ("f16", "f32")),
                                        ((512, 256, 768), 1, (False, False), ("f16", "f16")),
                                        ((256, 256, 3072), 4, (False, True), ("bf16", "f32"))]:
        c = _case(13, M, N, K, pair, "NK", epi)
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
        assert "load=direct" in desc, desc


def test_tiled_direct_loads_residual():
    for tile in (7, 9):
        c = inputs.random_case(14, 512, 512, 1536, "bf16", "bf16", "NK", bias=True, residual=True)
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile)
        assert "load=direct" in desc and "+res" in desc, desc


def test_tiled_staged_when_direct_loads_do_not_fit():
    """Ragged tiles, an odd slice count per split, [K][N] weights and tiles without direct loads
    keep the register-staged path."""
    for (M, N, K), split, layout, tile in [((500, 512, 1024), 1, "NK", 7), ((512, 512, 192), 1, "NK", 7),
                                           ((512, 512, 1024), 1, "KN", 7), ((512, 512, 1056), 1, "NK", 9),
                                           ((512, 512, 1024), 1, "NK", 1)]:
        c = _case(16, M, N, K, ("bf16", "bf16"), layout, (True, False))
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
        assert "load=direct" not in desc, desc


# --- the workloads at their full sizes ---------------------------------------------------

def test_fp32_linear_128x768():
    c = inputs.workload_fp32_linear_128x768()
    _check(c)


def test_fp16_narrow_16x4096x4096():
    c = inputs.workload_fp16_narrow()
    _, desc = _check(c)
    assert "variant=stream" in desc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpt2_layer_m128(dtype):
    for c in inputs.workload_gpt2_layer(M=128, dtype=dtype):
        _check(c)


def test_tiled_persistent():
    """Persistent workgroups (tile option 10, 128x128x64): a workgroup per resident slot loops over tiles, loading
    the next tile's first slices while the current one finishes.  1024 or 512 tiles: several per workgroup.
    Every output is compared, so a tile the loop skips or stores twice cannot go unseen."""
    for (M, N, K), pair, layout, epi, res in [((4096, 4096, 256), ("bf16", "bf16"), "NK", (True, True), False),
                                              ((4096, 2048, 512), ("f16", "f32"), "NK", (True, False), False),
                                              ((2048, 4096, 128), ("bf16", "f32"), "KN", (False, False), False),
                                              ((4096, 4096, 128), ("bf16", "bf16"), "NK", (True, False), True)]:
        c = inputs.random_case(17, M, N, K, pair[0], pair[1], layout, bias=epi[0], gelu=epi[1], residual=res)
        for tile in (10, 11):  # staged; direct loads where the operands allow them
            _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile)
            assert "persistent" in desc, desc
            assert ("load=direct" in desc) == (tile == 11 and layout == "NK"), desc


def test_tiled_128x192():
    """Tiled options 12 and 13 (128×192, 64×96 per wave): the staged epilogue's rows hold 12 (16-bit out) or
    24 (fp32 out) 16-byte runs, which the lanes take 64 apart with a guard.  Persistent grids of several
    rounds (staged, and direct loads at two per CU), a transposed first operand, the residual, split partials
    through the same epilogue, and an odd slice count (no persistence).  Every output is compared with the oracle."""
    for (M, N, K), pair, layout, epi, res, tile, split, want in [
            ((4096, 3072, 256), ("bf16", "bf16"), "NK", (True, True), False, 12, 1, "persistent"),
            ((4096, 4608, 128), ("bf16", "bf16"), "NK", (True, False), False, 13, 1, "load=direct persistent"),
            ((2048, 1536, 256), ("f16", "f32"), "AT_NK", (False, False), True, 12, 1, "persistent"),
            ((4096, 2304, 128), ("bf16", "bf16"), "NK", (False, False), True, 13, 1, "persistent"),
            ((512, 576, 1536), ("f16", "f32"), "NK", (True, True), False, 12, 2, "split=2"),
            ((512, 576, 1536), ("bf16", "bf16"), "NK", (False, True), True, 13, 2, "split=2"),
            ((256, 384, 192), ("bf16", "bf16"), "NK", (True, True), False, 12, 1, "tile=128x192x64")]:
        c = inputs.random_case(21, M, N, K, pair[0], pair[1], layout, bias=epi[0], gelu=epi[1], residual=res)
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
        assert want in desc, desc
        assert "tile=128x192x64" in desc, desc
        if split > 1 or K // 64 % 2:
            assert "persistent" not in desc, desc
    # fp32 options 9 and 10 (128×192×16, and ×32 persistent): 24 runs per staged row
    for (M, N, K), epi, res, tile, split in [((512, 576, 384), (True, True), False, 9, 1),
                                             ((512, 576, 768), (True, False), True, 9, 2),
                                             ((2048, 1536, 256), (True, True), False, 10, 1)]:
        c = inputs.random_case(22, M, N, K, "f32", "f32", "NK", bias=epi[0], gelu=epi[1], residual=res)
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
        assert "tile=128x192x" in desc and (("persistent" in desc) == (tile == 10)), desc


def test_tiled_persistent_f32():
    """fp32 persistent entries (options 7 and 8: 128x128x16 capped at two per CU, 64x64x16; option 10:
    128x192x32, whose staged epilogue rows hold 24 16-byte runs)."""
    for tile, (M, N, K) in [(7, (4096, 4096, 64)), (8, (2048, 2048, 96)), (10, (4096, 3072, 128))]:
        c = inputs.random_case(20, M, N, K, "f32", "f32", "KN" if tile == 7 else "NK", bias=tile == 8, gelu=tile == 8)
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile)
        assert "persistent" in desc, desc


def test_tiled_persistent_small_and_fallbacks():
    """Fewer tiles than resident workgroups (one tile each), and shapes the persistent loop does not take."""
    c = _case(18, 512, 512, 512, ("bf16", "bf16"), "NK", (True, True))
    _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=10)
    assert "persistent" in desc, desc
    for (M, N, K), split in [((512, 512, 192), 1), ((512, 512, 1024), 2), ((500, 512, 512), 1)]:
        c = _case(19, M, N, K, ("bf16", "bf16"), "NK", (True, False))
        _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=10, split_k=split)
        assert "persistent" not in desc, desc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_square_4096(dtype):
    """All 16.7 M outputs of the square workload against the oracle (the plan the bench times)."""
    c = inputs.workload_square(dtype=dtype)
    _, desc = _check(c)
    assert "variant=tiled" in desc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("which", range(4), ids=["qkv", "attn_out", "fc", "proj"])
def test_gpt2_stack_m8192_first_layer(dtype, which):
    """Every output of each linear of the stack's first layer (8192 rows) against the oracle."""
    c = inputs.workload_gpt2_stack(layers=1, dtype=dtype)[which]
    _check(c)


# --- exact properties ------------------------------------------------------------------

@pytest.mark.parametrize("variant,tile,split", [(tlgemm.VARIANT_GENERIC, 0, 0), (tlgemm.VARIANT_STREAM, 0, 0),
                                                 (tlgemm.VARIANT_STREAM, 3, 4), (tlgemm.VARIANT_STREAM, 5, 0),
                                                 (tlgemm.VARIANT_TILED, 1, 1), (tlgemm.VARIANT_TILED, 2, 4)])
def test_identity_and_permutation_bitwise(variant, tile, split):
    M, K = 48, 1024
    X = inputs.normal(5, (M, K), 1.0, "f32")
    perm = np.random.default_rng(1).permutation(K)
    for Wnp, want in [(np.eye(K, dtype=np.float32), X), (np.eye(K, dtype=np.float32)[perm], X[:, perm])]:
        c = inputs.LinearCase("perm", M, K, K, "f32", "f32", "NK", False, False, X, Wnp, None)
        Y, _ = run_case(c, variant=variant, tile=tile, split_k=split)
        assert np.array_equal(Y.cpu().numpy(), want)


def test_repeat_runs_bitwise():
    for c, kw in [(inputs.workload_fp16_narrow(), {}),
                  (inputs.random_case(9, 16, 768, 3072, "f16"), dict(variant=tlgemm.VARIANT_STREAM, tile=3, split_k=6)),
                  (inputs.random_case(9, 128, 768, 3072, "f32", bias=True), {}),
                  (inputs.random_case(9, 100, 264, 512, "bf16", bias=True, gelu=True),
                   dict(variant=tlgemm.VARIANT_TILED, split_k=5, tile=2))]:
        dev = device_case(c)
        first, _ = run_case(c, dev=dev, **kw)
        for _ in range(5):
            again, _ = run_case(c, dev=dev, **kw)
            assert torch.equal(first, again)


def test_replicated_rows_bitwise():
    K = 4096
    row = inputs.uniform(3, (1, K), -0.05, 0.05, "f16")
    c = inputs.workload_fp16_narrow()
    c.X = np.repeat(row, 16, axis=0)
    Y, _ = run_case(c)
    assert all(torch.equal(Y[0], Y[i]) for i in range(16))


def test_misaligned_pointer_rejected():
    c = inputs.random_case(4, 16, 64, 64, "f32")
    X, W, _ = device_case(c)
    Y = torch.empty((16, 65), device="cuda:0", dtype=torch.float32)
    p = tlgemm.Plan.create(16, 64, 64, "f32")
    with pytest.raises(tlgemm.TlgError) as e:
        p.run_ptrs(X.data_ptr() + 4, W.data_ptr(), 0, Y.data_ptr())
    assert e.value.status == tlgemm.ERR_MISALIGNED


def test_stream_argument_and_workspace_reuse():
    """Two plans sharing one workspace on a side stream give the oracle's results."""
    s = torch.cuda.Stream()
    cases = [inputs.random_case(11 + i, 128, 768, 768, "f32", bias=True) for i in range(2)]
    plans = [tlgemm.Plan.create(128, 768, 768, "f32", bias=True, variant=tlgemm.VARIANT_TILED, split_k=4, tile=2)
             for _ in cases]
    ws = torch.empty(max(p.workspace_size for p in plans), dtype=torch.uint8, device="cuda:0")
    outs = []
    with torch.cuda.stream(s):
        for c, p in zip(cases, plans):
            X, W, b = device_case(c)
            outs.append(tlgemm.run(p, X, W, b, workspace=ws, stream=s))
    s.synchronize()
    for c, y in zip(cases, outs):
        assert normalized_error(to_f64(y), oracle.linear_case(c)) <= 1e-5


def test_workspace_shared_between_plan_kinds():
    """One workspace, zeroed once, serves a tiled split plan (fp32 partials), then a split stream plan
    (arrival counters), then the tiled plan again: the partials never land on the counters."""
    tiled_case = inputs.random_case(21, 128, 768, 3072, "f32", bias=True)
    stream_case = inputs.random_case(22, 16, 768, 3072, "f16", bias=True, gelu=True)
    tiled = tlgemm.Plan.create(128, 768, 3072, "f32", bias=True, variant=tlgemm.VARIANT_TILED, split_k=8, tile=2)
    stream = tlgemm.Plan.create(16, 768, 3072, "f16", bias=True, gelu=True, variant=tlgemm.VARIANT_STREAM,
                                tile=3, split_k=6)
    try:
        assert "split=8" in tiled.describe() and "split=6" in stream.describe()
        ws = torch.zeros(max(tiled.workspace_size, stream.workspace_size), dtype=torch.uint8, device="cuda:0")
        for c, p in [(tiled_case, tiled), (stream_case, stream), (tiled_case, tiled), (stream_case, stream)]:
            X, W, b = device_case(c)
            Y = tlgemm.run(p, X, W, b, workspace=ws)
            torch.cuda.synchronize()
            assert normalized_error(to_f64(Y), oracle.linear_case(c)) <= TOL[c.in_dtype], p.describe()
        assert not torch.any(ws[:65536]), "a completed run left a counter set"
    finally:
        tiled.close()
        stream.close()


def test_subnormal_fp16_inputs_not_flushed():
    """Subnormal fp16 weights (|w| < 2^-14) must contribute, not flush to zero."""
    M, N, K = 16, 32, 4096
    X = inputs.store(np.ones((M, K)), "f16")
    W = inputs.store(np.full((N, K), 2.0 ** -20), "f16")  # subnormal in fp16
    c = inputs.LinearCase("sub", M, N, K, "f16", "f32", "NK", False, False, X, W, None)
    Y, _ = run_case(c)
    assert np.allclose(Y.cpu().numpy(), K * 2.0 ** -20, rtol=1e-6)
