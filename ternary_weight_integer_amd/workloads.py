"""Seeded synthetic inputs for the I2_S ternary-weight x int8-activation matmul.

This module only draws random numbers.  It holds none of the method's
arithmetic (no packing, no quantization, no dot products), so that both the
GPU path and the CPU oracle can be fed the very same bytes from it without
sharing any of the computation.

Shapes follow the Qwen2-1.5B decoder geometry given in "VibeASR in audio.cpp"
(Architecture / Decoder): hidden 1536, intermediate 8960, 12 query heads and
2 KV heads of width 128, so the seven ternary projections are
q/o 1536x1536, k/v 256x1536, gate/up 8960x1536 and down 1536x8960
(stored [out][K], K contiguous).

Recipe (every workload): ``numpy.random.default_rng(seed)`` with seed 0,
weights drawn before activations.  Ternary weights are i.i.d. over
{-1, 0, +1} with probabilities 0.3 / 0.4 / 0.3.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TERNARY_P = (0.3, 0.4, 0.3)

# Qwen2-1.5B projection shapes, (out, K).
QWEN2_1P5B_PROJ = {
    "q": (1536, 1536),
    "k": (256, 1536),
    "v": (256, 1536),
    "o": (1536, 1536),
    "gate": (8960, 1536),
    "up": (8960, 1536),
    "down": (1536, 8960),
}


@dataclass
class Case:
    """One matmul case: ternary weight w[out][K] (int8 in {-1,0,1}), weight
    scale ws, and F32 activations x[N][K]."""

    name: str
    w: np.ndarray
    ws: float
    x: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.w.shape[0])

    @property
    def K(self) -> int:
        return int(self.w.shape[1])

    @property
    def N(self) -> int:
        return int(self.x.shape[0])


def ternary(rng: np.random.Generator, rows: int, K: int, p=TERNARY_P) -> np.ndarray:
    """i.i.d. ternary matrix [rows][K] over {-1, 0, +1} with probabilities p."""
    return rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(rows, K), p=list(p)).astype(np.int8)


def normal(rng: np.random.Generator, N: int, K: int, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal((N, K)) * std).astype(np.float32)


def with_outliers(rng: np.random.Generator, x: np.ndarray, frac: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """Scale round(frac*K) positions per row (drawn without replacement) by factor."""
    x = x.copy()
    N, K = x.shape
    cnt = int(round(frac * K))
    for n in range(N):
        idx = rng.choice(K, size=cnt, replace=False)
        x[n, idx] = (x[n, idx] * np.float32(factor)).astype(np.float32)
    return x


def relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, np.float32(0)).astype(np.float32)


def random_case(seed: int, rows: int, K: int, N: int, ws: float = 0.015, std: float = 1.0, name: str | None = None) -> Case:
    rng = np.random.default_rng(seed)
    w = ternary(rng, rows, K)
    x = normal(rng, N, K, std)
    return Case(name or f"rand_s{seed}_{rows}x{K}_N{N}", w, ws, x)


# --- the five workloads ----------------------------------------------------

def small_case(seed: int = 0) -> Case:
    """Single matmul: w[64][256], ws 0.02, x[4][256] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, 64, 256)
    x = normal(rng, 4, 256)
    return Case("small_64x256_N4", w, 0.02, x)


def decode_up_case(seed: int = 0) -> Case:
    """Decode GEMV: FFN up w[8960][1536], ws 0.015, one row x[1][1536] ~ N(0,1)
    with 1% of its entries (15 positions) scaled by 20."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, 8960, 1536)
    x = with_outliers(rng, normal(rng, 1, 1536))
    return Case("decode_up_8960x1536_N1", w, 0.015, x)


def down_small_batch_case(seed: int = 0) -> Case:
    """Down projection: w[1536][8960], ws 0.015, x[8][8960] = ReLU(N(0, 0.5))."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, 1536, 8960)
    x = relu(normal(rng, 8, 8960, 0.5))
    return Case("down_1536x8960_N8", w, 0.015, x)


def prefill_gate_case(seed: int = 0, N: int = 512) -> Case:
    """Prefill GEMM: gate w[8960][1536], ws 0.015, x[512][1536] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, 8960, 1536)
    x = normal(rng, N, 1536)
    return Case(f"prefill_gate_8960x1536_N{N}", w, 0.015, x)


def layer_sweep_cases(seed: int = 0, Ns=(1, 64)) -> list[Case]:
    """All seven Qwen2-1.5B projections at each N, ws 0.015, x ~ N(0,1)."""
    out = []
    for proj, (rows, K) in QWEN2_1P5B_PROJ.items():
        rng = np.random.default_rng(seed)
        w = ternary(rng, rows, K)
        for N in Ns:
            x = normal(rng, N, K)
            out.append(Case(f"layer_{proj}_{rows}x{K}_N{N}", w, 0.015, x, {"proj": proj}))
    return out


def headroom_case(N: int = 1) -> Case:
    """int32 headroom: w[1536][8960] all +1 (every code 2), x == 127.0."""
    w = np.ones((1536, 8960), dtype=np.int8)
    x = np.full((N, 8960), 127.0, dtype=np.float32)
    return Case(f"headroom_1536x8960_N{N}", w, 0.015, x)


def zero_row_case(N: int = 1, zero_row: int = 0, seed: int = 0) -> Case:
    """Gate shape w[8960][1536] with activation row `zero_row` all zero."""
    rng = np.random.default_rng(seed)
    w = ternary(rng, 8960, 1536)
    x = normal(rng, N, 1536)
    x[zero_row, :] = 0.0
    return Case(f"zero_row_8960x1536_N{N}_r{zero_row}", w, 0.015, x)


@dataclass
class LayerCase:
    """One decoder layer's seven ternary projections at decode time: weights
    (int8 ternary, [out][K]), the q/k/v F32 biases, and the three activation
    rows they read (the normed hidden state for q/k/v, the attention output
    for o and gate/up's input, the FFN hidden state for down)."""
    name: str
    w: dict
    ws: float
    bias: dict
    x_hidden: np.ndarray
    x_attn: np.ndarray
    x_ffn: np.ndarray
    meta: dict = field(default_factory=dict)


def decode_layer_case(seed: int = 0, N: int = 1) -> LayerCase:
    """Qwen2-1.5B-shaped decoder layer, N activation rows: weights in the
    order q, k, v, o, gate, up, down, then biases ~ N(0, 0.1) for q, k, v,
    then x_hidden, x_attn ~ N(0, 1) and x_ffn = ReLU(N(0, 0.5))."""
    rng = np.random.default_rng(seed)
    w = {n: ternary(rng, *QWEN2_1P5B_PROJ[n]) for n in ("q", "k", "v", "o", "gate", "up", "down")}
    bias = {n: (0.1 * rng.standard_normal(QWEN2_1P5B_PROJ[n][0])).astype(np.float32) for n in ("q", "k", "v")}
    x_hidden = normal(rng, N, 1536)
    x_attn = normal(rng, N, 1536)
    x_ffn = relu(normal(rng, N, 8960, std=0.5))
    return LayerCase(f"decode_layer_qwen2_1p5b_N{N}", w, 0.015, bias, x_hidden, x_attn, x_ffn,
                     {"layers": 28, "N": N})


# ---------------------------------------------------------------------------
# I8_S encoder block MLP ("VibeASR in audio.cpp", Architecture / Encoder):
# seven stages with strides 1, 2, 2, 4, 5, 5, 8 (3200 samples per frame at
# 24 kHz) and widths 32 .. 2048; each ConvNeXt-style block ends in
# FC1 -> ReLU -> FC2.  The FC1 expansion is not given on the pages; the
# ConvNeXt design's 4x is taken.  Stage s sees samples / (s1 * ... * s_s)
# positions of a 4-second clip.

ENCODER_CHANNELS = (32, 64, 128, 256, 512, 1024, 2048)
ENCODER_STRIDES = (1, 2, 2, 4, 5, 5, 8)
ENCODER_MLP_RATIO = 4


@dataclass
class EncoderMlpCase:
    name: str
    stage: int
    C: int
    N: int
    w1: np.ndarray      # int8 [4C][C]  (FC1, output channel = row)
    w1_scale: float
    b1: np.ndarray      # f32 [4C]
    w2: np.ndarray      # int8 [C][4C]  (FC2)
    w2_scale: float
    b2: np.ndarray      # f32 [C]
    x: np.ndarray       # int8 [N][C]   (the block's normed input, already I8_S)
    x_scale: float


def _int8_bell(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """Bell-shaped int8 values (a normal draw rounded and clipped to +-127)."""
    return np.clip(np.rint(rng.normal(0.0, std, size=shape)), -127, 127).astype(np.int8)


def encoder_positions(stage: int, seconds: float = 4.0, sample_rate: int = 24000) -> int:
    n = int(round(seconds * sample_rate))
    for s in ENCODER_STRIDES[: stage + 1]:
        n //= s
    return n


def encoder_mlp_case(stage: int = 3, seed: int = 0, seconds: float = 4.0) -> EncoderMlpCase:
    """One block MLP of encoder stage `stage` (default 3: C = 256, 6000
    positions): int8 weights with std 24 (scales 0.004 / 0.003), biases
    ~ N(0, 0.1), the input int8 with std 40 plus 0.1% of entries at +-127
    (scale 0.03); weights drawn before activations."""
    rng = np.random.default_rng(seed)
    C = ENCODER_CHANNELS[stage]
    H = ENCODER_MLP_RATIO * C
    N = encoder_positions(stage, seconds)
    w1 = _int8_bell(rng, (H, C), 24.0)
    b1 = rng.normal(0.0, 0.1, size=H).astype(np.float32)
    w2 = _int8_bell(rng, (C, H), 24.0)
    b2 = rng.normal(0.0, 0.1, size=C).astype(np.float32)
    x = _int8_bell(rng, (N, C), 40.0)
    k = max(1, x.size // 1000)
    idx = rng.choice(x.size, size=k, replace=False)
    x.flat[idx] = np.where(rng.random(k) < 0.5, -127, 127).astype(np.int8)
    return EncoderMlpCase(name=f"encoder_mlp_stage{stage}_C{C}_N{N}", stage=stage, C=C, N=N,
                          w1=w1, w1_scale=0.004, b1=b1, w2=w2, w2_scale=0.003, b2=b2, x=x, x_scale=0.03)


# ---------------------------------------------------------------------------
# Per-channel W8A8 ("Experiment - int8 W8A8 path (the practical default)"):
# the same Qwen2-1.5B projection shapes with F32 weights ~ N(0, 0.02) (to be
# quantized per channel) and the I2_S workloads' activations.


@dataclass
class W8A8Case:
    name: str
    OC: int
    K: int
    M: int
    w: np.ndarray   # f32 [OC][K]
    x: np.ndarray   # f32 [M][K]


def w8a8_case(which: str = "prefill", seed: int = 0) -> W8A8Case:
    """'prefill': gate projection 8960 x 1536 against 512 rows ~ N(0,1);
    'decode': the same weight against one row ~ N(0,1) with 1% of entries
    scaled by 20.  Weights drawn before activations."""
    rng = np.random.default_rng(seed)
    OC, K = QWEN2_1P5B_PROJ["gate"]
    w = rng.normal(0.0, 0.02, size=(OC, K)).astype(np.float32)
    if which == "prefill":
        M = 512
        x = normal(rng, M, K)
    elif which == "decode":
        M = 1
        x = with_outliers(rng, normal(rng, M, K))
    else:
        raise ValueError(which)
    return W8A8Case(name=f"w8a8_{which}_gate_{OC}x{K}_M{M}", OC=OC, K=K, M=M, w=w, x=x)
