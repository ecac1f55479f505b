"""Seeded synthetic GEMM operands for the IM-Unpack integer GEMM path.

This module holds none of the method's arithmetic.  It only draws random
numbers, applies the outlier ("heavy hitter") masks that the workload
recipes describe, and rounds float32 to bfloat16 for storage.  The CPU
oracle and the HIP path both consume the arrays it returns, so neither
side generates inputs for the other.

The recipes stand in for the matrices the IM-Unpack summary page measures
on (IM-Unpack page, "Key results" and "Measured effects" table: LLaMA-7B
linear-layer and attention-output GEMMs; ViT/RoBERTa/T5 training GEMMs).
Those weights and datasets are not available, so every operand is a seeded
draw with the shape and outlier structure given below.

Storage conventions
-------------------
* ``Operand.stored`` is what lives in memory: float32 values (dtype "f32")
  or bfloat16 bit patterns held in ``uint16`` (dtype "bf16"), shaped
  ``(batch, srows, scols)`` row-major.
* ``layout == "normal"``: the logical matrix is the stored one.
  ``layout == "transposed"``: the logical matrix is the transpose of the
  stored one (a weight ``W`` of shape N x K used as ``B = W^T``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

STRATEGIES = ("row", "col", "mix")


@dataclass
class Operand:
    name: str
    stored: np.ndarray  # (batch, srows, scols), float32 or uint16 (bf16 bits)
    dtype: str  # "f32" | "bf16"
    layout: str  # "normal" | "transposed"

    @property
    def batch(self) -> int:
        return int(self.stored.shape[0])

    @property
    def rows(self) -> int:  # logical rows
        return int(self.stored.shape[1] if self.layout == "normal" else self.stored.shape[2])

    @property
    def cols(self) -> int:  # logical cols
        return int(self.stored.shape[2] if self.layout == "normal" else self.stored.shape[1])

    def logical_bits(self, b: int = 0) -> np.ndarray:
        """Stored array of batch entry ``b`` viewed in logical orientation (a view, no arithmetic)."""
        s = self.stored[b]
        return s if self.layout == "normal" else s.T

    def transposed_view(self, name: str) -> "Operand":
        """The same stored bytes used as the logical transpose."""
        return Operand(name, self.stored, self.dtype,
                       "transposed" if self.layout == "normal" else "normal")


@dataclass
class Problem:
    """One GEMM C = A @ B with the quantization / unpacking parameters."""
    name: str
    a: Operand
    b: Operand
    beta: int
    bits: int
    p_num: int = 95
    p_den: int = 100
    strat_a: str = "mix"
    strat_b: str = "mix"
    gamma: int = 2
    extra: dict = field(default_factory=dict)
    clip: bool = False  # the clipping quantizer of the ablation rows

    @property
    def mnk(self):
        return self.a.rows, self.a.cols, self.b.cols

    def with_strategies(self, sa: str, sb: str) -> "Problem":
        return Problem(f"{self.name}[{sa}/{sb}]", self.a, self.b, self.beta, self.bits,
                       self.p_num, self.p_den, sa, sb, self.gamma, dict(self.extra), self.clip)


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Only finite inputs are produced by the recipes here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# value models
# ----------------------------------------------------------------------------

def activations(rng: np.random.Generator, rows: int, cols: int,
                n_channels: int = 6, channel_scale: float = 50.0,
                spike_p: float = 0.001, spike_scale: float = 20.0) -> np.ndarray:
    """N(0,1) activations with a few fixed outlier channels and random spikes.

    ``n_channels`` distinct seeded columns are multiplied by ``channel_scale``;
    an i.i.d. Bernoulli(``spike_p``) mask multiplies entries by ``spike_scale``.
    """
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    nch = min(n_channels, cols)
    ch = rng.choice(cols, size=nch, replace=False)
    x[:, ch] *= np.float32(channel_scale)
    spikes = rng.random((rows, cols), dtype=np.float32) < spike_p
    x[spikes] *= np.float32(spike_scale)
    return x


def weights(rng: np.random.Generator, rows: int, cols: int, std: float = 0.02,
            spike_p: float = 0.0005, spike_scale: float = 15.0) -> np.ndarray:
    """N(0, std^2) weights with an i.i.d. Bernoulli(``spike_p``) mask scaled by ``spike_scale``."""
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    spikes = rng.random((rows, cols), dtype=np.float32) < spike_p
    w[spikes] *= np.float32(spike_scale)
    return w


def gradients(rng: np.random.Generator, rows: int, cols: int, nu: float = 3.0,
              scale: float = 1e-3) -> np.ndarray:
    """Heavy-tailed output gradients: i.i.d. Student-t(nu) times ``scale``."""
    return (rng.standard_t(nu, size=(rows, cols)) * scale).astype(np.float32)


def attention_logits(rng: np.random.Generator, seq: int, kv: int, logit_std: float = 3.0) -> np.ndarray:
    """One head's N(0, logit_std^2) attention logits, float32 (seq x kv)."""
    return rng.standard_normal((seq, kv), dtype=np.float32) * np.float32(logit_std)


def attention_probs(rng: np.random.Generator, heads: int, seq: int, kv: Optional[int] = None,
                    logit_std: float = 3.0) -> np.ndarray:
    """Row softmax of N(0, logit_std^2) logits, computed in float32; (heads, seq, kv)."""
    kv = seq if kv is None else kv
    out = np.empty((heads, seq, kv), dtype=np.float32)
    for h in range(heads):
        z = attention_logits(rng, seq, kv, logit_std)
        z -= z.max(axis=1, keepdims=True)
        np.exp(z, out=z)
        z /= z.sum(axis=1, keepdims=True)
        out[h] = z
    return out


def attn_values(rng: np.random.Generator, heads: int, seq: int, dim: int,
                n_dims: int = 2, dim_scale: float = 40.0) -> np.ndarray:
    """N(0,1) values with ``n_dims`` seeded outlier head dimensions scaled by ``dim_scale``."""
    v = rng.standard_normal((heads, seq, dim), dtype=np.float32)
    for h in range(heads):
        d = rng.choice(dim, size=min(n_dims, dim), replace=False)
        v[h][:, d] *= np.float32(dim_scale)
    return v


def _store(name: str, x: np.ndarray, dtype: str, layout: str) -> Operand:
    if x.ndim == 2:
        x = x[None]
    if dtype == "bf16":
        return Operand(name, f32_to_bf16_bits(x), "bf16", layout)
    return Operand(name, np.ascontiguousarray(x, dtype=np.float32), "f32", layout)


# ----------------------------------------------------------------------------
# workload recipes
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("tiny", "llama_linear", "mlp_up", "attn_out", "training")


def tiny(seed: int = 1000, m: int = 64, k: int = 128, n: int = 64) -> Problem:
    """Tiny fp32 GEMM: N(0,1) entries, Bernoulli(0.01) heavy hitters x30; beta=15, b=5, Mix."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(r, c):
        x = rng.standard_normal((r, c), dtype=np.float32)
        x[rng.random((r, c), dtype=np.float32) < 0.01] *= np.float32(30.0)
        return x

    a = _store("A", draw(m, k), "f32", "normal")
    b = _store("B", draw(k, n), "f32", "normal")
    return Problem("tiny", a, b, beta=15, bits=5)


def llama_linear(seed: int = 1001, m: int = 2048, k: int = 4096, n: int = 4096,
                 beta: int = 15, bits: int = 5, name: str = "llama_linear") -> Problem:
    """LLaMA-7B-shaped linear layer: X (m x k) activations times W^T, W stored n x k."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = activations(rng, m, k)
    w = weights(rng, n, k)
    return Problem(name, _store("X", x, "bf16", "normal"),
                   _store("W^T", w, "bf16", "transposed"), beta=beta, bits=bits)


def mlp_up(seed: int = 1002, m: int = 2048, k: int = 4096, n: int = 11008) -> Problem:
    """MLP up-projection: X (m x k) times W^T with W stored n x k; beta=31, b=4, Mix."""
    return llama_linear(seed, m, k, n, beta=31, bits=4, name="mlp_up")


def attn_out(seed: int = 1003, heads: int = 32, seq: int = 2048, dim: int = 128) -> Problem:
    """Batched attention output: per head P (seq x seq softmax) times V (seq x dim)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = attention_probs(rng, heads, seq)
    v = attn_values(rng, heads, seq, dim)
    return Problem("attn_out", _store("P", p, "bf16", "normal"),
                   _store("V", v, "bf16", "normal"), beta=15, bits=5)


def attn_logits(seed: int = 1003, heads: int = 32, seq: int = 2048) -> np.ndarray:
    """The logits the attention-output problem's P is the softmax of (the same
    draws as ``attn_out`` with the same seed): (heads, seq, seq) float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([attention_logits(rng, seq, seq) for _ in range(heads)])


def training(seed: int = 1004, tokens: int = 8192, d_in: int = 768, d_out: int = 3072) -> List[Problem]:
    """Forward, dgrad and wgrad GEMMs of a d_in -> d_out linear layer; beta=31, b=4, Mix.

    fwd:   X (tokens x d_in)  @ W^T   (W stored d_out x d_in)
    dgrad: dY (tokens x d_out) @ W
    wgrad: dY^T (d_out x tokens) @ X  (dY used through its transpose)
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _store("X", activations(rng, tokens, d_in), "bf16", "normal")
    w = _store("W^T", weights(rng, d_out, d_in), "bf16", "transposed")
    dy = _store("dY", gradients(rng, tokens, d_out), "bf16", "normal")
    w_n = Operand("W", w.stored, "bf16", "normal")
    dy_t = dy.transposed_view("dY^T")
    return [Problem("train_fwd", x, w, beta=31, bits=4),
            Problem("train_dgrad", dy, w_n, beta=31, bits=4),
            Problem("train_wgrad", dy_t, x, beta=31, bits=4)]


def config(idx: int, **shape) -> List[Problem]:
    """The five workload recipes by index (0 tiny ... 4 training), seed 1000 + index."""
    seed = 1000 + idx
    if idx == 0:
        return [tiny(seed, **shape)]
    if idx == 1:
        return [llama_linear(seed, **shape)]
    if idx == 2:
        return [mlp_up(seed, **shape)]
    if idx == 3:
        return [attn_out(seed, **shape)]
    if idx == 4:
        return training(seed, **shape)
    raise ValueError(f"no workload recipe {idx}")


def random_problem(seed: int, m: int, k: int, n: int, *, dtype: str = "bf16",
                   layout_a: str = "normal", layout_b: str = "normal", batch: int = 1,
                   beta: int = 15, bits: int = 5, strat_a: str = "mix", strat_b: str = "mix",
                   kind: str = "linear", p=(95, 100), clip: bool = False) -> Problem:
    """A small problem of any shape with one of the recipe value models.

    kind "linear": activations x weights (config-1 models); "grad": Student-t
    operands; "attn": softmax probabilities x values; "gauss": N(0,1) with
    1% x30 heavy hitters (the tiny recipe).
    """
    rng = np.random.Generator(np.random.PCG64(seed))

    def logical_to_stored(x, layout):
        return np.ascontiguousarray(np.swapaxes(x, -1, -2)) if layout == "transposed" else x

    av = np.empty((batch, m, k), np.float32)
    bv = np.empty((batch, k, n), np.float32)
    for h in range(batch):
        if kind == "linear":
            av[h] = activations(rng, m, k)
            bv[h] = weights(rng, k, n)
        elif kind == "grad":
            av[h] = gradients(rng, m, k)
            bv[h] = gradients(rng, k, n)
        elif kind == "attn":
            av[h] = attention_probs(rng, 1, m, k)[0]
            bv[h] = attn_values(rng, 1, k, n)[0]
        elif kind == "gauss":
            a = rng.standard_normal((m, k), dtype=np.float32)
            a[rng.random((m, k), dtype=np.float32) < 0.01] *= np.float32(30.0)
            b = rng.standard_normal((k, n), dtype=np.float32)
            b[rng.random((k, n), dtype=np.float32) < 0.01] *= np.float32(30.0)
            av[h], bv[h] = a, b
        else:
            raise ValueError(kind)
    a = _store("A", logical_to_stored(av, layout_a), dtype, layout_a)
    b = _store("B", logical_to_stored(bv, layout_b), dtype, layout_b)
    return Problem(f"rand{seed}_{m}x{k}x{n}", a, b, beta=beta, bits=bits, p_num=p[0], p_den=p[1],
                   strat_a=strat_a, strat_b=strat_b, clip=clip)
