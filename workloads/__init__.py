"""Seeded synthetic inputs for the optimizer update, shared by tests and bench.

This module holds no optimizer arithmetic: it only draws random numbers and
casts them to the storage dtypes (with torch's CPU casts, round to nearest
even).  Both the oracle and the HIP path consume exactly the arrays it
returns.

Storage arrays are numpy: fp32 as ``float32``, fp16 and bf16 as ``uint16``
bit patterns.  ``to_torch`` views them as torch tensors of the storage dtype.

Workload shapes follow the subject page "Investigate a 256-thread SM103 path
for small 32-bit optimizer tensors" (bitsandbytes fork, issue 8): the tensor
sizes of its coverage matrix (section "Correctness oracle"), the direct-op
benchmark sizes and the bias/norm/LoRA-like collections of section "B300
benchmark and acceptance".  The page does not print the collection shapes,
so ``model_collection`` is a stand-in of that kind.
"""
from __future__ import annotations

import numpy as np
import torch

STORAGE_NP = {"fp32": np.float32, "fp16": np.uint16, "bf16": np.uint16}
STORAGE_TORCH = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
STORAGE_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}

# Tensor sizes of the coverage matrix plus the boundary controls.
SWEEP_N = (1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512, 513,
           1023, 1024, 1025, 4095, 4096, 4097)
# Direct-op benchmark cells plus boundary controls.
DIRECT_N = (1, 32, 64, 128, 256, 512, 768, 1023, 1024, 1025, 2048, 4096)
GRAD_PATTERNS = ("zero", "normal", "mixed")
SNAPSHOT_STEPS = (1, 2, 10, 1000)

N_256M = 1 << 28
N_1G = 1 << 30


def rng(*key: int) -> np.random.Generator:
    """Counter-keyed generator: the same key always gives the same stream."""
    return np.random.default_rng([int(k) for k in key])


def cast_storage(x32: np.ndarray, storage: str) -> np.ndarray:
    """fp32 numpy -> storage array (float32, or uint16 bits), RNE via torch."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if storage == "fp32":
        return x32
    t = torch.from_numpy(x32).to(STORAGE_TORCH[storage])
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_torch(a: np.ndarray, storage: str, device=None) -> torch.Tensor:
    """Storage array -> torch tensor of the storage dtype (copied to ``device``)."""
    if storage == "fp32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(STORAGE_TORCH[storage])
    return t.to(device) if device is not None else t.clone()


def from_torch(t: torch.Tensor) -> np.ndarray:
    """Torch tensor (any device) -> storage numpy array (float32 or uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def params(n: int, storage: str, g: np.random.Generator) -> np.ndarray:
    """Parameters ~ U(-1, 1), cast to storage."""
    return cast_storage(g.uniform(-1.0, 1.0, n).astype(np.float32), storage)


def grads(n: int, pattern: str, storage: str, g: np.random.Generator,
          sigma: float = 1.0) -> np.ndarray:
    """Gradients of one pattern, cast to storage (see ``grads_f32``)."""
    return cast_storage(grads_f32(n, pattern, g, sigma), storage)


def grads_f32(n: int, pattern: str, g: np.random.Generator, sigma: float = 1.0) -> np.ndarray:
    """Gradients of one pattern in fp32.

    zero   : all +0
    normal : N(0, sigma^2)  (sigma is the standard deviation)
    mixed  : random sign, |g| = 10^U(-8, 3) (log-uniform over 11 decades);
             fp16 storage rounds the smallest to zero, which exercises
             skip_zeros.
    """
    if pattern == "zero":
        x = np.zeros(n, np.float32)
    elif pattern == "normal":
        x = (g.standard_normal(n) * sigma).astype(np.float32)
    elif pattern == "mixed":
        sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
        x = (sign * 10.0 ** g.uniform(-8.0, 3.0, n)).astype(np.float32)
    else:
        raise ValueError(pattern)
    return x


def zero_states(n: int, kind: str) -> tuple[np.ndarray, np.ndarray]:
    """Zero-initialised fp32 states: state1 has n floats (Adam) or 2n (AdEMAMix)."""
    k = 2 if kind == "ademamix" else 1
    return np.zeros(k * n, np.float32), np.zeros(n, np.float32)


def model_collection(layers: int = 24) -> list[tuple[str, tuple[int, ...]]]:
    """Model-like parameter collection: per layer 4 norm vectors (1024),
    5 biases (4 x 1024 + 1 x 4096), 8 rank-16 LoRA factors (4 x 16x1024 and
    4 x 1024x16), 2 weights 1024x4096 and 2 weights 1024x1024; then one
    32000x1024 embedding.  505 tensors, 287,866,880 elements for 24 layers."""
    out: list[tuple[str, tuple[int, ...]]] = []
    for layer in range(layers):
        for j in range(4):
            out.append((f"l{layer}.norm{j}", (1024,)))
        for j in range(4):
            out.append((f"l{layer}.bias{j}", (1024,)))
        out.append((f"l{layer}.bias_ffn", (4096,)))
        for j in range(4):
            out.append((f"l{layer}.lora_a{j}", (16, 1024)))
        for j in range(4):
            out.append((f"l{layer}.lora_b{j}", (1024, 16)))
        for j in range(2):
            out.append((f"l{layer}.w_ffn{j}", (1024, 4096)))
        for j in range(2):
            out.append((f"l{layer}.w_attn{j}", (1024, 1024)))
    out.append(("embedding", (32000, 1024)))
    return out


def numel(shape: tuple[int, ...]) -> int:
    r = 1
    for s in shape:
        r *= s
    return r


# fp32 state planes per element: Adam m, v; AdEMAMix m, v, m2; one-state kinds m.
STATE_PLANES = {"adam": 2, "ademamix": 3, "momentum": 1, "rmsprop": 1, "adagrad": 1, "lion": 1}


def bytes_per_element_8bit(kind: str, storage: str) -> float:
    """Algorithmic HBM bytes per element and step of the 8-bit block-wise
    path: read p, g, one code per moment; write p and the codes; plus one
    fp32 absmax per moment and 256-element block, read and written."""
    s = STORAGE_BYTES[storage]
    k = STATE_PLANES[kind]            # moments: Adam 2, AdEMAMix 3
    return (2 * s + k) + (s + k) + 2 * 4 * k / 256


def bytes_per_element(kind: str, storage: str) -> int:
    """Algorithmic HBM bytes per element and step: read p, g, the fp32 states;
    write p and the fp32 states (the gradient is only read)."""
    s = STORAGE_BYTES[storage]
    k = STATE_PLANES[kind]
    return (2 * s + 4 * k) + (s + 4 * k)
