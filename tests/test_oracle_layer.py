"""Pins of the whole-layer oracle.

* dropout 0: torch.nn.TransformerEncoderLayer in float64 on the CPU (a
  library special case of the same definition), forward and autograd
  backward, Pre-LN and Post-LN, with key padding;
* dropout > 0: central finite differences of sum(y * dy) for every
  parameter and the input (the masks are a fixed function of the seed);
* hidden-dropout structure: each residual branch element is either dropped
  or scaled by 1/(1-p), exactly where the site's mask says.
"""
import numpy as np
import pytest
import torch

import oracle
from transformer_encoder_layer_amd import synthetic as syn

NAMES = syn.PARAM_NAMES


def _torch_layer(w, p):
    layer = torch.nn.TransformerEncoderLayer(
        d_model=w.hidden, nhead=w.heads, dim_feedforward=w.ffn, dropout=0.0, activation="gelu",
        layer_norm_eps=1e-12, batch_first=True, norm_first=w.pre_ln, dtype=torch.float64)
    sd = {
        "self_attn.in_proj_weight": p["w_qkv"], "self_attn.in_proj_bias": p["b_qkv"],
        "self_attn.out_proj.weight": p["w_o"], "self_attn.out_proj.bias": p["b_o"],
        "linear1.weight": p["w_1"], "linear1.bias": p["b_1"],
        "linear2.weight": p["w_2"], "linear2.bias": p["b_2"],
        "norm1.weight": p["ln1_g"], "norm1.bias": p["ln1_b"],
        "norm2.weight": p["ln2_g"], "norm2.bias": p["ln2_b"],
    }
    layer.load_state_dict({k: torch.from_numpy(np.array(v)) for k, v in sd.items()})
    layer.train()
    return layer


TORCH_MAP = {"w_qkv": "self_attn.in_proj_weight", "b_qkv": "self_attn.in_proj_bias",
             "w_o": "self_attn.out_proj.weight", "b_o": "self_attn.out_proj.bias",
             "w_1": "linear1.weight", "b_1": "linear1.bias", "w_2": "linear2.weight", "b_2": "linear2.bias",
             "ln1_g": "norm1.weight", "ln1_b": "norm1.bias", "ln2_g": "norm2.weight", "ln2_b": "norm2.bias"}


@pytest.mark.parametrize("pre_ln", [True, False])
@pytest.mark.parametrize("shape", ["tiny", "wide"])
def test_layer_matches_torch_fp64(pre_ln, shape):
    w = syn.WORKLOADS["tiny"].with_(pre_ln=pre_ln)
    if shape == "wide":
        w = w.with_(batch=3, seq=24, hidden=96, heads=3, ffn=160, lengths=(1, 24), seed=77)
    p = syn.layer_params(w, random_affine=True)
    # larger weights so that the softmax is far from uniform
    for k in ("w_qkv", "w_o", "w_1", "w_2"):
        p[k] = p[k] * 8.0
    x = syn.layer_input(w)
    dy = syn.upstream_grad(w)
    lengths = syn.seq_lengths(w)
    if shape == "wide":
        lengths[0] = 1  # a sequence with a single valid key
    cfg = oracle.LayerCfg(w.batch, w.seq, w.hidden, w.heads, w.ffn, pre_ln=pre_ln, training=True)
    y, _ = oracle.layer_forward(cfg, p, x, lengths)
    dx, grads = oracle.layer_backward(cfg, p, x, lengths, dy)

    layer = _torch_layer(w, p)
    xt = torch.from_numpy(x.reshape(w.batch, w.seq, w.hidden)).clone().requires_grad_(True)
    pad = torch.arange(w.seq)[None, :] >= torch.from_numpy(lengths.astype(np.int64))[:, None]
    yt = layer(xt, src_key_padding_mask=pad)
    yt.backward(torch.from_numpy(dy.reshape(w.batch, w.seq, w.hidden)))
    assert np.abs(y - yt.detach().numpy().reshape(-1, w.hidden)).max() < 1e-10
    assert np.abs(dx - xt.grad.numpy().reshape(-1, w.hidden)).max() < 1e-10
    named = dict(layer.named_parameters())
    for n in NAMES:
        g_t = named[TORCH_MAP[n]].grad.numpy()
        assert np.abs(grads[n] - g_t).max() < 1e-10 * max(1.0, np.abs(g_t).max()), n


def _loss(cfg, p, x, lengths, dy):
    y, _ = oracle.layer_forward(cfg, p, x, lengths)
    return float((y * dy).sum())


def _fd_check(cfg, p, x, lengths, dy, n_samples=None, seed=0):
    dx, grads = oracle.layer_backward(cfg, p, x, lengths, dy)
    h = 1e-6
    r = np.random.default_rng(seed)
    targets = [("x", x, dx)] + [(n, p[n], grads[n]) for n in NAMES]
    for name, arr, grad in targets:
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        idx = np.arange(flat.size) if n_samples is None else r.choice(flat.size, min(n_samples, flat.size),
                                                                      replace=False)
        fd = np.empty(len(idx))
        for k, i in enumerate(idx):
            old = flat[i]
            flat[i] = old + h
            fp = _loss(cfg, p, x, lengths, dy)
            flat[i] = old - h
            fm = _loss(cfg, p, x, lengths, dy)
            flat[i] = old
            fd[k] = (fp - fm) / (2 * h)
        an = gflat[idx]
        scale = max(np.abs(an).max(), 1e-3)
        assert np.abs(fd - an).max() <= 1e-6 * scale, name


@pytest.mark.parametrize("pre_ln", [True, False])
def test_layer_backward_fd_with_dropout_small(pre_ln):
    w = syn.Workload("fd", 1, 4, 8, 2, 16, pre_ln, "f32", 0.1, 0.1, 31, lengths=None)
    p = syn.layer_params(w, random_affine=True)
    for k in ("w_qkv", "w_o", "w_1", "w_2"):
        p[k] = p[k] * 20.0
    x = syn.layer_input(w)
    dy = syn.upstream_grad(w)
    lengths = np.array([3], dtype=np.int32)
    pf = float(np.float32(0.3))
    cfg = oracle.LayerCfg(1, 4, 8, 2, 16, pre_ln=pre_ln, training=True, attn_p=pf, hidden_p=pf,
                          seed=31, step=2, layer_id=1)
    # the chosen seed must actually drop something at both sites
    assert (oracle.dropout_mask(31, 1, 0, 2, pf, 0, 16 * 2) == 0).any()
    assert (oracle.dropout_mask(31, 1, 1, 2, pf, 0, 32) == 0).any()
    _fd_check(cfg, p, x, lengths, dy)


@pytest.mark.parametrize("pre_ln", [True, False])
def test_layer_backward_fd_tiny_sampled(pre_ln):
    w = syn.WORKLOADS["tiny"].with_(pre_ln=pre_ln)
    p = syn.layer_params(w, random_affine=True)
    for k in ("w_qkv", "w_o", "w_1", "w_2"):
        p[k] = p[k] * 8.0
    x = syn.layer_input(w)
    dy = syn.upstream_grad(w)
    lengths = syn.seq_lengths(w)
    pf = float(np.float32(0.1))
    cfg = oracle.LayerCfg(w.batch, w.seq, w.hidden, w.heads, w.ffn, pre_ln=pre_ln, training=True,
                          attn_p=pf, hidden_p=pf, seed=1234, step=0, layer_id=0)
    _fd_check(cfg, p, x, lengths, dy, n_samples=12, seed=1)


@pytest.mark.parametrize("pre_ln", [True, False])
def test_hidden_dropout_structure(pre_ln):
    w = syn.WORKLOADS["tiny"].with_(pre_ln=pre_ln)
    p = syn.layer_params(w, random_affine=True)
    x = syn.layer_input(w)
    lengths = syn.seq_lengths(w)
    pf = float(np.float32(0.25))
    cfg = oracle.LayerCfg(w.batch, w.seq, w.hidden, w.heads, w.ffn, pre_ln=pre_ln, training=True,
                          attn_p=0.0, hidden_p=pf, seed=5, step=9, layer_id=2, batch_offset=4)
    y, a = oracle.layer_forward(cfg, p, x, lengths, want_acts=True)
    T, H = w.tokens, w.hidden
    e0 = 4 * w.seq * H  # element index t_global*H + c with t_global offset by batch_offset*S
    m1 = oracle.dropout_mask(5, 2, 1, 9, pf, e0, T * H).reshape(T, H)
    m2 = oracle.dropout_mask(5, 2, 2, 9, pf, e0, T * H).reshape(T, H)
    res1 = x if pre_ln else x
    branch1 = (a["ln2_in"] if pre_ln else a["ln1_in"]) - res1
    assert np.abs(branch1 - a["attn_proj"] * m1 / (1 - pf)).max() < 1e-12
    res2 = a["ln2_in"] if pre_ln else a["ln1_out"]
    out2 = y if pre_ln else a["ln2_in"]
    assert np.abs(out2 - res2 - a["ffn_out"] * m2 / (1 - pf)).max() < 1e-12
    assert 0.15 < (1 - m1).mean() < 0.35


def test_invertible_backward_matches_standard():
    w = syn.WORKLOADS["tiny"]
    p = syn.layer_params(w, random_affine=True)
    x = syn.layer_input(w)
    dy = syn.upstream_grad(w)
    lengths = syn.seq_lengths(w)
    for pre_ln in (True, False):
        cfg = oracle.LayerCfg(w.batch, w.seq, w.hidden, w.heads, w.ffn, pre_ln=pre_ln, training=True,
                              attn_p=0.1, hidden_p=0.1, seed=3)
        a = oracle.layer_backward(cfg, p, x, lengths, dy, ln_invertible=False)
        b = oracle.layer_backward(cfg, p, x, lengths, dy, ln_invertible=True)
        assert np.abs(a[0] - b[0]).max() < 1e-10
        for n in NAMES:
            assert np.abs(a[1][n] - b[1][n]).max() < 1e-10 * max(1, np.abs(a[1][n]).max()), n
