"""Seeded synthetic inputs for the RFQ W4A4 linear layer.

This module holds no quantization or GEMM arithmetic: it only draws random
activations and weights and rounds them to bfloat16, so that the CPU oracle
and the HIP library can be fed the same bytes.

The value structure follows what the pages describe for the layers RFQ is
applied to: heavy-tailed activations with a few large outlier channels
("Activation Outliers Matter: Robust Recovery for Quantized Multimodal LLMs",
§1; the outlier example in "大模型量化中的双线性尾部问题与QuaRot正交旋转解决方案",
§2.1), and for the down-projection the product of a gated pair, SiLU(a)*b
(same blog page, §2.2, the SwiGLU form). They stand in for real Wan2.2 and
Qwen3-VL activations, which are not available; the shapes are those of the
named layers.

Streams: config i uses numpy SeedSequence(26081 + i). Its children are
keyed by spawn_key: (0,) outlier channels and their gains, (1, j) rows
[256 j, 256 j + 256) of X, (2, j) rows of W. So any row range can be
regenerated on its own, bit for bit.
"""

from dataclasses import dataclass

import numpy as np

ROW_CHUNK = 256
BASE_SEED = 26081


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    M: int
    K: int
    N: int
    x_dist: str          # "normal", "student_t3", "laplace", "silu_product"
    n_outliers: int      # outlier channels of X
    gain_lo: float       # outlier gain range [lo, hi]
    gain_hi: float
    w_sigma: float
    y_dtype: str         # "fp32" or "bf16"
    description: str

    @property
    def seed(self):
        return BASE_SEED + self.index


CONFIGS = {
    c.name: c
    for c in [
        Config(1, "tiny", 64, 256, 128, "normal", 2, 50.0, 50.0, 0.02, "fp32",
               "tiny RFQ linear: X N(0,1) with 2 outlier channels x50; W N(0,0.02^2); Y fp32"),
        Config(2, "qwen3vl_attn_proj", 2048, 4096, 4096, "student_t3", 20, 30.0, 100.0, 0.02, "bf16",
               "Qwen3-VL-8B-style attention projection: X Student-t(3), 0.5% of channels x U[30,100]"),
        Config(3, "qwen3vl_ffn_up", 4096, 4096, 12288, "student_t3", 20, 30.0, 100.0, 0.02, "bf16",
               "Qwen3-VL-8B-style FFN up/gate projection: X as the attention projection"),
        Config(4, "wan22_ffn", 4096, 5120, 13824, "laplace", 8, 80.0, 80.0, 0.015, "bf16",
               "Wan2.2-DiT-style FFN: X Laplace(0,1) plus 8 fixed outlier channels x80"),
        Config(5, "dit_ffn_down", 32768, 13824, 5120, "silu_product", 0, 1.0, 1.0, 0.015, "bf16",
               "long-sequence DiT FFN down-projection: X = SiLU(a)*b, a, b ~ N(0,1)"),
    ]
}


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite by construction."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg, *key):
    return np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=key))


def outliers(cfg):
    """(channel indices, gains) of the outlier channels of X, drawn without
    replacement from the config's own stream."""
    if cfg.n_outliers == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.float32)
    g = _rng(cfg, 0)
    ch = np.sort(g.choice(cfg.K, size=cfg.n_outliers, replace=False)).astype(np.int64)
    gains = g.uniform(cfg.gain_lo, cfg.gain_hi, size=cfg.n_outliers).astype(np.float32)
    return ch, gains


def _x_chunk_f32(cfg, j, ch, gains):
    g = _rng(cfg, 1, j)
    rows = min(ROW_CHUNK, cfg.M - j * ROW_CHUNK)
    shape = (rows, cfg.K)
    if cfg.x_dist == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
    elif cfg.x_dist == "student_t3":
        x = g.standard_t(3.0, size=shape).astype(np.float32)
    elif cfg.x_dist == "laplace":
        x = g.laplace(0.0, 1.0, size=shape).astype(np.float32)
    elif cfg.x_dist == "silu_product":
        a = g.standard_normal(shape, dtype=np.float32)
        b = g.standard_normal(shape, dtype=np.float32)
        x = (a / (np.float32(1.0) + np.exp(-a))) * b
    else:
        raise ValueError(cfg.x_dist)
    if ch.size:
        x[:, ch] *= gains[None, :]
    return x


def x_bf16(cfg, row_start=0, row_stop=None):
    """Rows [row_start, row_stop) of X as bfloat16 bits, uint16 [rows, K]."""
    row_stop = cfg.M if row_stop is None else row_stop
    ch, gains = outliers(cfg)
    out = np.empty((row_stop - row_start, cfg.K), dtype=np.uint16)
    j0, j1 = row_start // ROW_CHUNK, (row_stop + ROW_CHUNK - 1) // ROW_CHUNK
    for j in range(j0, j1):
        lo = j * ROW_CHUNK
        xb = f32_to_bf16_bits(_x_chunk_f32(cfg, j, ch, gains))
        a, b = max(lo, row_start), min(lo + xb.shape[0], row_stop)
        out[a - row_start:b - row_start] = xb[a - lo:b - lo]
    return out


def x_rows_bf16(cfg, rows):
    """Selected rows of X (any order) as bfloat16 bits."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, cfg.K), dtype=np.uint16)
    ch, gains = outliers(cfg)
    for j in np.unique(rows // ROW_CHUNK):
        xb = f32_to_bf16_bits(_x_chunk_f32(cfg, int(j), ch, gains))
        sel = np.nonzero(rows // ROW_CHUNK == j)[0]
        out[sel] = xb[rows[sel] - j * ROW_CHUNK]
    return out


def w_bf16(cfg):
    """W [N, K] as bfloat16 bits, N(0, w_sigma^2)."""
    out = np.empty((cfg.N, cfg.K), dtype=np.uint16)
    for j in range((cfg.N + ROW_CHUNK - 1) // ROW_CHUNK):
        g = _rng(cfg, 2, j)
        rows = min(ROW_CHUNK, cfg.N - j * ROW_CHUNK)
        w = g.standard_normal((rows, cfg.K), dtype=np.float32) * np.float32(cfg.w_sigma)
        out[j * ROW_CHUNK:j * ROW_CHUNK + rows] = f32_to_bf16_bits(w)
    return out


def sample_rows(cfg, n_random=254, seed_key=3):
    """Deterministic row sample for full-size checks: 0, M-1 and n_random seeded rows."""
    g = _rng(cfg, seed_key)
    n_random = min(n_random, max(cfg.M - 2, 0))
    mid = g.choice(np.arange(1, cfg.M - 1), size=n_random, replace=False) if n_random else []
    return np.unique(np.concatenate([[0, cfg.M - 1], mid]).astype(np.int64))
