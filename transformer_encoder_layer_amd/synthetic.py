"""Seeded synthetic inputs for the encoder-layer workloads.

This module holds no arithmetic of the layer itself: it only draws random
numbers (numpy PCG64 keyed by (config seed, tensor id)) in fp64 and lists the
workload shapes.  The tests feed the same drawn buffers, rounded to the
storage dtype, to both the GPU library and the CPU oracle; the benchmark
uses them as its input data.

Tensor ids: 0 = layer input x, 1 = upstream gradient dy, 2 = sequence
lengths, 100 + 16*layer + k = k-th parameter of a layer (order below).

The pages' workloads (BERT-Large pretraining at sequence 128, BERT-Base
fine-tuning shapes, a long-sequence layer, the memory-saving stack with
progressive layer dropping) run on real text; no dataset or trained weights
are used here.  N(0,1) hidden states and N(0, 0.02^2) weights of the same
shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

PARAM_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
               "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    pre_ln: bool
    dtype: str              # "f32" | "f16" | "bf16"
    attn_p: float
    hidden_p: float
    seed: int
    lengths: Optional[Tuple[int, int]] = None   # inclusive range, None = no padding
    layers: int = 1
    gelu_checkpoint: bool = False
    attn_dropout_checkpoint: bool = False
    normalize_invertible: bool = False
    pld: Optional[Tuple[float, float, int]] = None   # (theta_bar, gamma, step)
    notes: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 16, 64, 4, 256, True, "f32", 0.0, 0.0, 1234, lengths=(8, 16)),
    "bert_large": Workload("bert_large", 64, 128, 1024, 16, 4096, True, "f16", 0.1, 0.1, 1234, layers=24),
    "bert_base_postln": Workload("bert_base_postln", 32, 512, 768, 12, 3072, False, "bf16", 0.1, 0.1, 42,
                                 lengths=(64, 512)),
    "long_seq": Workload("long_seq", 8, 2048, 1024, 16, 4096, True, "bf16", 0.1, 0.0, 1234),
    "memsave_stack": Workload("memsave_stack", 128, 128, 1024, 16, 4096, True, "f16", 0.1, 0.1, 7, layers=24,
                              gelu_checkpoint=True, attn_dropout_checkpoint=True, normalize_invertible=True,
                              pld=(0.5, 0.001, 5000)),
}


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def normal(seed: int, tensor_id: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    return mean + std * rng(seed, tensor_id).standard_normal(size=shape, dtype=np.float64)


def param_shapes(w: Workload):
    H, F = w.hidden, w.ffn
    return {"w_qkv": (3 * H, H), "b_qkv": (3 * H,), "w_o": (H, H), "b_o": (H,), "ln1_g": (H,), "ln1_b": (H,),
            "w_1": (F, H), "b_1": (F,), "w_2": (H, F), "b_2": (H,), "ln2_g": (H,), "ln2_b": (H,)}


def layer_params(w: Workload, layer: int = 0, random_affine: bool = False) -> dict:
    """Weights ~N(0, 0.02^2); biases 0, gamma 1, beta 0.  With random_affine
    the biases are ~N(0, 0.02^2), gamma ~1 + N(0, 0.1^2) and beta ~N(0, 0.02^2)
    so that every bias and affine code path carries non-trivial values."""
    out = {}
    for k, name in enumerate(PARAM_NAMES):
        shape = param_shapes(w)[name]
        tid = 100 + 16 * layer + k
        if name.startswith("w_"):
            out[name] = normal(w.seed, tid, shape, 0.02)
        elif name.endswith("_g"):
            out[name] = normal(w.seed, tid, shape, 0.1, 1.0) if random_affine else np.ones(shape)
        else:
            out[name] = normal(w.seed, tid, shape, 0.02) if random_affine else np.zeros(shape)
    return out


def layer_input(w: Workload) -> np.ndarray:
    return normal(w.seed, 0, (w.tokens, w.hidden))


def upstream_grad(w: Workload) -> np.ndarray:
    return normal(w.seed, 1, (w.tokens, w.hidden))


def seq_lengths(w: Workload) -> np.ndarray:
    if w.lengths is None:
        return np.full(w.batch, w.seq, dtype=np.int32)
    lo, hi = w.lengths
    return rng(w.seed, 2).integers(lo, hi + 1, size=w.batch).astype(np.int32)


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_storage(a: np.ndarray, dtype: str):
    """fp64 numpy array -> CPU torch tensor of the storage dtype (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dtype(dtype))
