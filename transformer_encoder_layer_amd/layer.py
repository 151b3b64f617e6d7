"""torch.nn front end of the fused encoder layer.

``EncoderLayer`` holds the twelve parameters (nn.Linear layout) and calls the
C ABI through ``binding``: forward and backward each run entirely in the HIP
library on the current torch stream.  torch provides device memory (the
per-forward ``saved`` buffer, a ``scratch`` buffer shared by all layers on a
device) and the stream; nothing of the layer is computed in torch.

``EncoderStack`` stacks layers with distinct layer ids (as the DeepSpeed
guide's deepcopy of one layer spec does) and implements progressive layer
dropping: at step t every layer is kept with probability
theta(t) = (1 - theta_bar) exp(-gamma t) + theta_bar (PLD page, "core
mechanism"); the keep decision is the counter-based gate of tel_pld_keep, so
every process derives the same gates without communication.  A dropped layer
is the identity in forward and backward.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B

_DTYPES = {torch.float32: B.TEL_F32, torch.float16: B.TEL_F16, torch.bfloat16: B.TEL_BF16}


@dataclass
class LayerConfig:
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int = 0
    attn_dropout: float = 0.1
    hidden_dropout: float = 0.1
    pre_ln: bool = True
    seed: int = 1234
    layer_id: int = 0
    dtype: torch.dtype = torch.float16
    ln_eps: float = 1e-12
    attn_dropout_checkpoint: bool = False
    normalize_invertible: bool = False
    gelu_checkpoint: bool = False
    pack_tokens: bool = False
    stochastic_mode: bool = False

    def to_c(self) -> B.tel_config:
        return B.tel_config(self.batch, self.seq, self.hidden, self.heads, self.ffn, self.attn_dropout,
                            self.hidden_dropout, int(self.pre_ln), self.seed, self.layer_id,
                            _DTYPES[self.dtype], self.ln_eps, int(self.attn_dropout_checkpoint),
                            int(self.normalize_invertible), int(self.gelu_checkpoint),
                            int(self.pack_tokens), int(self.stochastic_mode))


_scratch = {}


def scratch_buffer(device: torch.device, nbytes: int) -> torch.Tensor:
    """A uint8 device buffer of at least nbytes, shared by every layer on the device."""
    key = (device.type, device.index)
    buf = _scratch.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _scratch[key] = buf
    return buf


def _round256(n: int) -> int:
    return (n + 255) // 256 * 256


class _Chain:
    """One forward's hand-down of site-2 masked gradients through a Pre-LN
    stack (tel_layer_backward_chain): the backward of a layer writes the
    masked dx of the run layer below it, which that layer's backward takes
    as its drop2(dy) only while its dy is still that same, unmodified dx
    tensor (same storage and version counter); otherwise it masks dy
    itself.  The results are the same bits either way."""

    def __init__(self):
        self.pending = None  # (layer it is for, dx, dx._version, masked dx)


class _LayerFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, lengths, step, valid, layer, chain, below, *params):
        dev = x.device
        if valid is not None:
            B.tel_layer_set_valid_tokens(layer.handle, valid)
        # grad mode is off inside Function.forward; whether autograd will call
        # backward is what needs_input_grad says
        need_grad = any(ctx.needs_input_grad)
        x = x.contiguous()
        y = torch.empty_like(x)
        saved = torch.empty(layer.saved_bytes, dtype=torch.uint8, device=dev) if need_grad else None
        scratch = scratch_buffer(dev, layer.scratch_bytes if need_grad
                                 else _round256(layer.scratch_bytes) + layer.saved_bytes)
        P = B.make_params(dict(zip(B.PARAM_NAMES, params)))
        training = int(layer.training)
        B.tel_layer_forward(layer.handle, P, x, lengths, training, step, y, saved, scratch)
        ctx.layer = layer
        ctx.step = step
        ctx.training_flag = training
        ctx.saved_buf = saved
        ctx.save_for_backward(x, *params)
        ctx.lengths = lengths
        ctx.valid = valid
        ctx.chain, ctx.below = chain, below
        return y

    @staticmethod
    def backward(ctx, dy):
        layer = ctx.layer
        x, *params = ctx.saved_tensors
        dy = dy.contiguous()
        dx = torch.empty_like(x)
        grads = [torch.empty_like(p) for p in params]
        scratch = scratch_buffer(x.device, layer.scratch_bytes)
        if ctx.valid is not None:
            B.tel_layer_set_valid_tokens(layer.handle, ctx.valid)
        P = B.make_params(dict(zip(B.PARAM_NAMES, params)))
        G = B.make_grads(dict(zip(B.PARAM_NAMES, grads)))
        chain, below = ctx.chain, ctx.below
        dyd = None
        if chain is not None:
            pend, chain.pending = chain.pending, None
            if (pend is not None and pend[0] is layer and pend[1].data_ptr() == dy.data_ptr()
                    and pend[1].shape == dy.shape and pend[1].stride() == dy.stride() and dy._version == pend[2]):
                dyd = pend[3]
        if dyd is not None or below is not None:
            dxd = torch.empty_like(x) if below is not None else None
            B.tel_layer_backward_chain(layer.handle, P, x, ctx.lengths, ctx.training_flag, ctx.step, dy, dyd,
                                       ctx.saved_buf, scratch, dx, below.handle if below is not None else None,
                                       dxd, G)
            if below is not None:
                chain.pending = (below, dx, dx._version, dxd)
        else:
            B.tel_layer_backward(layer.handle, P, x, ctx.lengths, ctx.training_flag, ctx.step, dy, ctx.saved_buf,
                                 scratch, dx, G)
        ctx.saved_buf = None
        ctx.chain = ctx.below = None
        return (dx, None, None, None, None, None, None, *grads)


class EncoderLayer(torch.nn.Module):
    def __init__(self, cfg: LayerConfig, device="cuda"):
        super().__init__()
        self.cfg = cfg
        H = cfg.hidden
        F = cfg.ffn if cfg.ffn > 0 else 4 * H
        self.ffn = F
        self.handle = B.tel_layer_create(cfg.to_c())
        self.saved_bytes, self.scratch_bytes = B.tel_layer_workspace_bytes(self.handle)
        shapes = {"w_qkv": (3 * H, H), "b_qkv": (3 * H,), "w_o": (H, H), "b_o": (H,), "ln1_g": (H,),
                  "ln1_b": (H,), "w_1": (F, H), "b_1": (F,), "w_2": (H, F), "b_2": (H,), "ln2_g": (H,),
                  "ln2_b": (H,)}
        for n in B.PARAM_NAMES:
            init = torch.ones if n.endswith("_g") else torch.zeros
            self.register_parameter(n, torch.nn.Parameter(init(shapes[n], dtype=cfg.dtype, device=device)))

    def params(self):
        return [getattr(self, n) for n in B.PARAM_NAMES]

    def forward(self, x: torch.Tensor, key_lengths: Optional[torch.Tensor] = None, step: int = 0,
                valid_tokens: Optional[int] = None, _chain: Optional[_Chain] = None,
                _below: Optional["EncoderLayer"] = None):
        """valid_tokens: sum of key_lengths (token packing); computed on the
        host from key_lengths when packing is on and it is not given.
        _chain, _below: set by EncoderStack (the stack's hand-down of masked
        gradients and the run layer below this one)."""
        valid = None
        if self.cfg.pack_tokens and key_lengths is not None:
            valid = int(key_lengths.sum().item()) if valid_tokens is None else int(valid_tokens)
        return _LayerFn.apply(x, key_lengths, int(step), valid, self, _chain, _below, *self.params())

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                B.tel_layer_destroy(h)
            except Exception:
                pass
            self.handle = None


def pld_theta(step: int, theta_bar: float = 0.5, gamma: float = 0.001) -> float:
    return B.tel_pld_theta(step, theta_bar, gamma)


def pld_gates(seed: int, layers: int, step: int, theta_bar: float, gamma: float):
    """Keep decision of each of `layers` layers at this step (PLD page, "core
    mechanism"): every layer is kept with probability theta(step), decided by
    the counter-based gate of tel_pld_keep keyed by (seed, layer id, step)."""
    theta = pld_theta(step, theta_bar, gamma)
    return [B.tel_pld_keep(seed, i, step, theta) for i in range(layers)]


class EncoderStack(torch.nn.Module):
    def __init__(self, cfg: LayerConfig, layers: int, device="cuda", pld: Optional[tuple] = None,
                 params: Optional[list] = None, layer_ids: Optional[list] = None):
        """pld: (theta_bar, gamma) or None.  params: optional list (one per
        layer) of dicts name -> tensor giving each layer's initial values.
        layer_ids: the id of each layer (its dropout and PLD key; default
        0 .. layers-1), e.g. for a stack that holds part of a model."""
        super().__init__()
        self.layer_ids = list(range(layers)) if layer_ids is None else [int(i) for i in layer_ids]
        assert len(self.layer_ids) == layers
        self.layers = torch.nn.ModuleList(
            [EncoderLayer(LayerConfig(**{**cfg.__dict__, "layer_id": i}), device) for i in self.layer_ids])
        if params is not None:
            with torch.no_grad():
                for layer, vals in zip(self.layers, params):
                    for n in B.PARAM_NAMES:
                        getattr(layer, n).copy_(vals[n])
        self.pld = pld
        self.seed = cfg.seed

    def gates(self, step: int):
        if self.pld is None or not self.training:
            return [True] * len(self.layers)
        theta = pld_theta(step, *self.pld)
        return [B.tel_pld_keep(self.seed, i, step, theta) for i in self.layer_ids]

    def forward(self, x, key_lengths=None, step: int = 0, taps: Optional[list] = None):
        """A dropped layer is the identity: its input passes on unchanged, in
        the forward and (through autograd) in the backward.  taps: optional
        list that receives (layer index, input tensor) of every layer run."""
        run = [(i, layer) for i, (layer, keep) in enumerate(zip(self.layers, self.gates(step))) if keep]
        # Pre-LN, unpacked: each layer's backward masks the gradient of the
        # run layer below it (tel_layer_backward_chain)
        chain = _Chain() if (self.layers[0].cfg.pre_ln and not self.layers[0].cfg.pack_tokens
                             and torch.is_grad_enabled()) else None
        for j, (i, layer) in enumerate(run):
            if taps is not None:
                taps.append((i, x))
            below = run[j - 1][1] if chain is not None and j > 0 else None
            if below is not None and below.training != layer.training:
                below = None
            x = layer(x, key_lengths, step, _chain=chain, _below=below)
        return x
