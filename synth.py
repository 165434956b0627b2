"""Seeded synthetic inputs for the MosaicQuant fused W4A4 + sparse-residual GEMM.

This module only draws inputs. It holds none of the method's arithmetic (no
quantizer, no score, no packing, no matmul), so the oracle under ``oracle/``
and the HIP library under ``dense_sparse_bit_amd/`` can both be fed from it
without sharing any computation.

Workloads stand in for the linear layers the MosaicQuant summary evaluates
(LLaMA3 3B/8B and Qwen3 4B-32B, batch 4-32; "Risultati Sperimentali"). No
trained weights or calibration text exist here, so the weights and activations
are random with the shapes and outlier structure listed in ``CONFIGS``:

* weights ``W[N][K]`` (out x in) are N(0, 0.02) in fp32, optionally with a
  fraction of entries (positions drawn without replacement) scaled by 10;
* activations ``X[M][K]`` are N(0, 1) or Student-t(3)/sqrt(3) (unit variance),
  with a fraction of input channels scaled by a factor, optionally a first row
  ("BOS-like" token) scaled by 100, then rounded to bf16 (round to nearest
  even) where the workload says bf16;
* each workload draws W and X from two independent child streams of
  ``numpy.random.SeedSequence(seed)``.

Counts are ``floor(fraction * population)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    M: int
    K: int
    N: int
    x_dist: str            # "normal" or "t3"
    x_bf16: bool
    x_channel_frac: float  # fraction of input channels that are outliers
    x_channel_scale: float
    x_bos_scale: float     # 0 = no BOS-like row, else row 0 is scaled by this
    w_outlier_frac: float  # fraction of weight entries scaled by 10
    bn: int                # residual block rows (output features)
    bk: int                # residual block cols (input features)
    budgets: tuple         # residual budgets in percent of blocks
    group: int = 128

    @property
    def nb(self) -> int:
        return (self.N // self.bn) * (self.K // self.bk)

    def k_blocks(self, pct: int) -> int:
        """Number of residual blocks for a budget in percent (floor)."""
        return (pct * self.nb) // 100

    @property
    def default_budget(self) -> int:
        return 10 if 10 in self.budgets else self.budgets[-1]


def _llama(name, M, K, N, budgets):
    return Config(name, M, K, N, "normal", True, 0.01, 50.0, 0.0, 0.005, 64, 64, budgets)


def _qwen(name, M, K, N):
    return Config(name, M, K, N, "t3", True, 0.02, 40.0, 0.0, 0.005, 64, 64, (10,))


CONFIGS = {
    c.name: c
    for c in [
        # the small case: fp32 activations, 4 outlier channels x30, plain N(0, 0.02) weights
        Config("tiny", 4, 512, 512, "normal", False, 4 / 512, 30.0, 0.0, 0.0, 64, 64, (10,)),
        _llama("llama3_8b_qo", 16, 4096, 4096, (10,)),
        _llama("llama3_8b_up_m4", 4, 4096, 14336, (0, 5, 10, 20)),
        _llama("llama3_8b_up_m32", 32, 4096, 14336, (0, 5, 10, 20)),
        _llama("llama3_8b_down_m4", 4, 14336, 4096, (0, 5, 10, 20)),
        _llama("llama3_8b_down_m32", 32, 14336, 4096, (0, 5, 10, 20)),
        _qwen("qwen3_32b_up", 32, 5120, 25600),
        _qwen("qwen3_32b_down", 32, 25600, 5120),
        Config("qwen3_14b_prefill", 2048, 5120, 17408, "normal", True, 0.01, 50.0, 100.0,
               0.005, 128, 64, (0, 10)),
    ]
}

# The workload the benchmark line is quoted on.
BENCH_CONFIG = "qwen3_14b_prefill"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    cfg: Config
    W: np.ndarray          # fp32 [N][K]
    X: np.ndarray          # fp32 [M][K] (exact widening of the bf16 values when x_bf16)
    X_bits: np.ndarray | None  # uint16 bf16 bits [M][K] when x_bf16, else None

    @property
    def x_dtype(self) -> str:
        return "bf16" if self.X_bits is not None else "f32"

    def x_raw(self) -> np.ndarray:
        """The activation array as it is handed to the library (bf16 bits or fp32)."""
        return self.X_bits if self.X_bits is not None else self.X


def draw_weights(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    W = rng.standard_normal((cfg.N, cfg.K), dtype=np.float32)
    W *= np.float32(0.02)
    n_out = math.floor(cfg.w_outlier_frac * cfg.N * cfg.K)
    if n_out:
        idx = rng.choice(cfg.N * cfg.K, size=n_out, replace=False)
        W.reshape(-1)[idx] *= np.float32(10.0)
    return W


def draw_activations(cfg: Config, rng: np.random.Generator, M: int | None = None) -> np.ndarray:
    M = cfg.M if M is None else M
    if cfg.x_dist == "normal":
        X = rng.standard_normal((M, cfg.K), dtype=np.float32)
    elif cfg.x_dist == "t3":
        X = (rng.standard_t(3, size=(M, cfg.K)) / math.sqrt(3.0)).astype(np.float32)
    else:
        raise ValueError(cfg.x_dist)
    n_ch = math.floor(cfg.x_channel_frac * cfg.K)
    if n_ch:
        ch = rng.choice(cfg.K, size=n_ch, replace=False)
        X[:, ch] *= np.float32(cfg.x_channel_scale)
    if cfg.x_bos_scale:
        X[0] *= np.float32(cfg.x_bos_scale)
    return X


def make_inputs(name_or_cfg, seed: int = 0) -> Inputs:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    s_w, s_x = np.random.SeedSequence(seed).spawn(2)
    W = draw_weights(cfg, np.random.default_rng(s_w))
    X = draw_activations(cfg, np.random.default_rng(s_x))
    bits = None
    if cfg.x_bf16:
        bits = f32_to_bf16_bits(X)
        X = bf16_bits_to_f32(bits)
    return Inputs(cfg, W, X, bits)


def custom_config(name="custom", *, M, K, N, bn=64, bk=64, x_bf16=True, x_dist="normal",
                  x_channel_frac=0.01, x_channel_scale=50.0, x_bos_scale=0.0,
                  w_outlier_frac=0.005, budgets=(10,)) -> Config:
    """A workload of the same family at another shape (parity and edge-case tests)."""
    return Config(name, M, K, N, x_dist, x_bf16, x_channel_frac, x_channel_scale, x_bos_scale,
                  w_outlier_frac, bn, bk, tuple(budgets))


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
