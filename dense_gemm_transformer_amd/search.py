"""Cost model, candidate choice and keep/revert rule of the dispatch-table search.

The search loop of "Optimizing a GPT-2-class transformer on a GPU" (Act V):
propose only candidates that satisfy hard constraints, predict their cost
with a roofline model with penalties, correct that prior with a regression
on physical features that learns only its errors, spend measurements on the
predicted best plus the candidates the model is least sure of, score by
distance from the physical floor, and replace an incumbent only when a
paired measurement in the same window says so.  The regression's
coefficients are the residual report: a feature with a large coefficient
names a cost the prior misprices.

Pure host code (numpy only), so every rule here is tested without a GPU;
``tune.py`` runs the measurements.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# MI355X figures the prior starts from: datasheet peaks, the CU count, and
# the derating the ceiling probes measure (MFMA issue ~93 % of peak, a plain
# cold read ~61 % of HBM, an empty launch ~2 µs of stream time).
PEAK_MFMA = {"f32": 157.3e12, "f16": 2516.6e12, "bf16": 2516.6e12}
PEAK_HBM = 8.0e12
L2_BW = 24.0e12          # aggregate L2 -> CU bandwidth assumed by the prior (8 XCDs)
NUM_CUS = 256
MFMA_DERATE = 0.93
HBM_DERATE = 0.61
LAUNCH_S = 2.0e-6
ROUND_S = 1.5e-6         # pipeline fill and epilogue per round of workgroups
ELEM = {"f32": 4, "f16": 2, "bf16": 2}
VARIANT_STREAM, VARIANT_TILED = 1, 2


@dataclass
class Shape:
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    residual: bool = False

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: each operand read once, Y written once (and read once with a residual)."""
        ei, eo = ELEM[self.in_dtype], ELEM[self.out_dtype]
        return ei * (self.M * self.K + self.N * self.K) + eo * self.M * self.N * (2 if self.residual else 1)

    def floor_s(self) -> float:
        """The physical floor: the larger of the MFMA and HBM roofline times at the datasheet peaks."""
        return max(self.flops / PEAK_MFMA[self.in_dtype], self.bytes / PEAK_HBM)


@dataclass
class Config:
    """What a plan does, as the planner reports it (tlg_plan_info)."""
    variant: int
    tile_m: int
    tile_n: int
    tile_k: int
    split: int
    threads: int
    workgroups: int
    launches: int
    key: str = ""


def occupancy(shape: Shape, c: Config) -> int:
    """Workgroups per CU the kernel can hold: the register bound of the tiled kernel (accumulators per wave)
    and its LDS (two buffers of both operand tiles); the stream kernel runs one large workgroup per CU."""
    if c.variant != VARIANT_TILED:
        return 1
    waves = max(c.threads // 64, 1)
    acc = c.tile_m * c.tile_n // waves // 64
    reg = 4 if acc <= 16 else 2 if acc <= 64 else 1
    lds = 2 * (c.tile_m + c.tile_n) * (c.tile_k + 16 // ELEM[shape.in_dtype]) * ELEM[shape.in_dtype]
    return max(1, min(reg, (160 * 1024) // max(lds, 1)))


@dataclass
class Features:
    occ: int
    rounds: int
    fill: float
    split: int
    launches: int
    l2_bytes: float
    extra_bytes: float
    half: bool = False       # 16-bit operands
    slices: float = 1.0      # K slices each workgroup multiplies (pipeline length)
    tile_area: int = 4096    # outputs per workgroup

    def vector(self) -> np.ndarray:
        """Regression inputs; the intercept is the first entry."""
        return np.array([1.0, math.log2(self.occ), float(self.rounds - 1), 1.0 - self.fill,
                         math.log2(self.split), float(self.launches - 1), float(self.half),
                         math.log2(max(self.slices, 1.0)), math.log2(self.tile_area / 4096)])


FEATURE_NAMES = ("bias", "log2 occupancy", "extra rounds", "idle fraction of the last round", "log2 split",
                 "extra launches", "16-bit operands", "log2 K slices per workgroup", "log2 tile area / 64x64")


def main_workgroups(shape: Shape, c: Config) -> int:
    """Workgroups of the GEMM kernel itself (the planner's count includes a split reducer's 1024 outputs each)."""
    if c.launches > 1:
        return c.workgroups - math.ceil(shape.M * shape.N / 1024)
    return c.workgroups


def features(shape: Shape, c: Config) -> Features:
    occ = occupancy(shape, c)
    wg = max(main_workgroups(shape, c), 1)
    waves = wg / (NUM_CUS * occ)  # rounds of workgroups if every slot on every CU were busy
    rounds = max(1, math.ceil(waves - 1e-9))
    fill = waves / rounds
    kper = shape.K / max(c.split, 1)
    l2 = wg * (c.tile_m + c.tile_n) * kper * ELEM[shape.in_dtype]
    extra = 2.0 * 4 * shape.M * shape.N * c.split if c.split > 1 else 0.0  # fp32 partials written, read back
    return Features(occ, rounds, fill, c.split, c.launches, l2, extra, shape.in_dtype != "f32",
                    kper / max(c.tile_k, 1), c.tile_m * c.tile_n)


def prior_s(shape: Shape, f: Features) -> float:
    """Roofline with penalties: the slowest of MFMA time (derated, stretched by the idle slots of the last
    round of workgroups), HBM time (derated, with split partials) and L2 time, plus launch and per-round
    latency."""
    t_math = shape.flops / (PEAK_MFMA[shape.in_dtype] * MFMA_DERATE) / f.fill
    t_mem = (shape.bytes + f.extra_bytes) / (PEAK_HBM * HBM_DERATE)
    t_l2 = f.l2_bytes / L2_BW
    return max(t_math, t_mem, t_l2) + LAUNCH_S * f.launches + ROUND_S * f.rounds


class ResidualModel:
    """Ridge regression of log(measured / prior) on the physical features.

    The prior stays the default prediction; the regression learns only its
    errors, and its coefficients say which cost the prior misprices.
    """

    def __init__(self, ridge: float = 0.1):
        self.ridge = ridge
        self.X: list[np.ndarray] = []
        self.y: list[float] = []
        self.beta: np.ndarray | None = None
        self.cov: np.ndarray | None = None
        self.sigma2 = 0.0

    def add(self, f: Features, prior: float, measured: float) -> None:
        self.X.append(f.vector())
        self.y.append(math.log(measured / prior))

    def fit(self) -> None:
        if len(self.y) < 2:
            return
        X = np.array(self.X)
        y = np.array(self.y)
        A = X.T @ X + self.ridge * np.eye(X.shape[1])
        Ainv = np.linalg.inv(A)
        self.beta = Ainv @ X.T @ y
        r = y - X @ self.beta
        dof = max(len(y) - X.shape[1], 1)
        self.sigma2 = float(r @ r) / dof
        self.cov = Ainv

    def correction(self, f: Features) -> float:
        """Predicted log(measured / prior) for these features (0 before the first fit)."""
        return 0.0 if self.beta is None else float(f.vector() @ self.beta)

    def std(self, f: Features) -> float:
        """Standard deviation of that prediction (the model's uncertainty); large before any fit."""
        if self.cov is None:
            return 1.0
        x = f.vector()
        return math.sqrt(max(self.sigma2, 1e-4) * (1.0 + float(x @ self.cov @ x)))

    def predict_s(self, f: Features, prior: float) -> float:
        return prior * math.exp(self.correction(f))

    def report(self) -> list[tuple[str, float, str]]:
        """(feature, coefficient, verdict) sorted by size; positive: the prior underprices it."""
        if self.beta is None:
            return []
        out = []
        for name, b in zip(FEATURE_NAMES, self.beta):
            out.append((name, float(b), "model UNDERprices" if b > 0 else "model OVERprices"))
        return sorted(out, key=lambda t: -abs(t[1]))


def constrained(shape: Shape, cands: list[Config], min_slices: int = 2) -> list[Config]:
    """Port 1 — what may be proposed: the planner has already applied the hard limits (LDS, grid, split ≤
    K steps); drop splits that leave fewer than ``min_slices`` K slices per split, and candidates whose
    grid reaches less than a quarter of the CUs when another candidate of the same variant fills them."""
    out = []
    for c in cands:
        if c.variant == VARIANT_TILED and c.split > 1 and shape.K / c.split < min_slices * c.tile_k:
            continue
        out.append(c)
    fills = {}
    for c in out:
        fills[c.variant] = max(fills.get(c.variant, 0), c.workgroups)
    return [c for c in out if not (c.workgroups < NUM_CUS // 4 and fills[c.variant] >= NUM_CUS)]


def choose(shape: Shape, cands: list[Config], model: ResidualModel, budget: int, explore: int,
           incumbent_key: str) -> list[Config]:
    """Port 4 — which experiments to run: the ``budget`` candidates with the lowest corrected prediction,
    then the ``explore`` remaining ones the model is least sure about, plus the incumbent."""
    scored = []
    for c in cands:
        f = features(shape, c)
        p = prior_s(shape, f)
        scored.append((model.predict_s(f, p), model.std(f), c))
    scored.sort(key=lambda t: t[0])
    picked = [t[2] for t in scored[:budget]]
    rest = sorted(scored[budget:], key=lambda t: -t[1])
    picked += [t[2] for t in rest[:explore]]
    if incumbent_key and all(c.key != incumbent_key for c in picked):
        picked += [c for c in cands if c.key == incumbent_key]
    return picked


@dataclass
class Decision:
    keep_incumbent: bool
    ratio: float          # median over rounds of challenger / incumbent time (paired)
    wins: int             # rounds the challenger was faster
    rounds: int
    reason: str = field(default="")


def decide(incumbent: list[float], challenger: list[float], margin: float = 0.01) -> Decision:
    """Port 2 — selection, paired: per-round times of incumbent and challenger from the same window.  The
    challenger replaces the incumbent only if its median paired ratio is below 1 - margin and it is faster
    in at least two thirds of the rounds; otherwise the incumbent stays (a stale number from another window
    is never compared)."""
    assert len(incumbent) == len(challenger) and incumbent, "paired rounds"
    ratios = sorted(c / i for c, i in zip(challenger, incumbent))
    n = len(ratios)
    med = ratios[n // 2] if n % 2 else 0.5 * (ratios[n // 2 - 1] + ratios[n // 2])
    wins = sum(c < i for c, i in zip(challenger, incumbent))
    if med < 1.0 - margin and 3 * wins >= 2 * n:
        return Decision(False, med, wins, n, f"challenger faster by {100 * (1 - med):.1f} % in {wins}/{n} rounds")
    return Decision(True, med, wins, n, f"within margin or not consistent ({100 * (1 - med):+.1f} %, {wins}/{n})")


def efficiency(shape: Shape, measured_s: float) -> float:
    """Port 2 — the score: the physical floor over the measured time (1.0 means at the roofline)."""
    return shape.floor_s() / measured_s
