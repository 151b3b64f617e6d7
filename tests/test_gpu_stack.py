"""Stacks of layers through the torch front end (layer.EncoderStack and its
autograd function), checked layer by layer against the fp64 oracle with
teacher forcing: the oracle gets the GPU's own input to layer l and the
gradient the GPU passed down to layer l's output, so each comparison covers
exactly one layer at its full shape -- every sequence, every element of y,
dx and all twelve parameter gradients.

Progressive layer dropping (PLD page, "core mechanism"): the stack's gates
must equal the oracle's, a dropped layer must be the identity in forward and
backward (the stack equals one built from the kept layers alone), and a
dropped layer's parameters receive no gradient."""
import numpy as np
import pytest

import oracle
from _harness import NAMES, compare_full, oracle_full
from transformer_encoder_layer_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def _stack(w, n_layers, pld=None, layer_ids=None):
    from transformer_encoder_layer_amd.layer import EncoderStack, LayerConfig
    cfg = LayerConfig(w.batch, w.seq, w.hidden, w.heads, w.ffn, float(np.float32(w.attn_p)),
                      float(np.float32(w.hidden_p)), w.pre_ln, w.seed, 0, syn.torch_dtype(w.dtype), 1e-12,
                      w.attn_dropout_checkpoint, w.normalize_invertible, w.gelu_checkpoint)
    ids = list(range(n_layers)) if layer_ids is None else list(layer_ids)
    params = []
    for l in ids:
        p64 = syn.layer_params(w, l)
        params.append({n: syn.to_storage(p64[n], w.dtype).cuda() for n in NAMES})
    st = EncoderStack(cfg, len(ids), pld=pld, params=params, layer_ids=ids)
    st.train()
    return st


def _run_stack(st, w, step, lengths=None):
    """Forward + backward of the whole stack; returns (taps, y, dy_top): taps
    are (layer index, input) with .grad filled by the backward."""
    import torch
    x = syn.to_storage(syn.layer_input(w), w.dtype).cuda().requires_grad_(True)
    dy = syn.to_storage(syn.upstream_grad(w), w.dtype).cuda()
    lens = None if lengths is None else torch.from_numpy(np.asarray(lengths, dtype=np.int32)).cuda()
    taps = []
    y = st(x, lens, step, taps=taps)
    for _, t in taps[1:]:
        t.retain_grad()
    y.backward(dy)
    torch.cuda.synchronize()
    return taps, y, dy


def _teacher_forced(w, st, taps, y, dy, pos, step, lengths):
    """Layer at tap position pos against the oracle fed the GPU's own input
    and upstream gradient."""
    idx, x_in = taps[pos]
    out = taps[pos + 1][1] if pos + 1 < len(taps) else y
    g_out = taps[pos + 1][1].grad if pos + 1 < len(taps) else dy
    p64 = syn.layer_params(w, idx)
    params_r = {n: syn.to_storage(p64[n], w.dtype).double().numpy() for n in NAMES}
    o_y, o_dx, o_g = oracle_full(w, params_r, x_in.detach().double().cpu().numpy(),
                                 g_out.double().cpu().numpy(), lengths, step=step, layer_id=idx,
                                 invertible=w.normalize_invertible)
    layer = st.layers[idx]
    grads = {n: getattr(layer, n).grad.double().cpu().numpy() for n in NAMES}
    compare_full(w, out.detach().double().cpu().numpy(), x_in.grad.double().cpu().numpy(), grads, o_y, o_dx, o_g,
                 tag=f"{w.name} layer {idx}")


@pytest.mark.timeout(900)
def test_bert_large_stack_teacher_forced():
    # the 24-layer BERT-Large stack (B64 S128, fp16, dropout 0.1/0.1, distinct
    # layer ids); layers 0, 11 and 23 in full
    w = syn.WORKLOADS["bert_large"]
    st = _stack(w, w.layers)
    taps, y, dy = _run_stack(st, w, step=0)
    assert [i for i, _ in taps] == list(range(24))
    lengths = syn.seq_lengths(w)
    for pos in (0, 11, 23):
        _teacher_forced(w, st, taps, y, dy, pos, 0, lengths)


@pytest.mark.timeout(900)
def test_memsave_pld_stack_teacher_forced():
    # the memory-saving stack (B128 S128 fp16, GELU / attention-dropout
    # checkpointing, invertible LayerNorm) with PLD at t = 5000
    # (theta = 0.50337, seed 7): gates as the oracle's, skipped layers get no
    # gradient, first and last kept layers in full
    w = syn.WORKLOADS["memsave_stack"]
    theta_bar, gamma, t = w.pld
    st = _stack(w, w.layers, pld=(theta_bar, gamma))
    theta = oracle.pld_theta(t, theta_bar, gamma)
    want = [oracle.pld_keep(w.seed, l, t, theta) for l in range(w.layers)]
    assert st.gates(t) == want and 0 < sum(want) < w.layers
    taps, y, dy = _run_stack(st, w, step=t)
    assert [i for i, _ in taps] == [l for l in range(w.layers) if want[l]]
    for l in range(w.layers):
        if not want[l]:
            assert all(getattr(st.layers[l], n).grad is None for n in NAMES), l
    lengths = syn.seq_lengths(w)
    for pos in (0, len(taps) - 1):
        _teacher_forced(w, st, taps, y, dy, pos, t, lengths)


def test_pld_stack_small_identity_and_parity():
    # 8 small layers (B2 S128 H256, fp16, padded lengths) with PLD gates at
    # step 7000, seed 11 (theta = 0.5005): layers 1, 2 and 5 dropped.
    import torch
    w = syn.Workload("pld_small", 2, 128, 256, 4, 1024, True, "f16", 0.1, 0.1, 11, lengths=(40, 128), layers=8)
    t, pld = 7000, (0.5, 0.001)
    st = _stack(w, w.layers, pld=pld)
    gates = st.gates(t)
    theta = oracle.pld_theta(t, *pld)
    assert gates == [oracle.pld_keep(w.seed, l, t, theta) for l in range(w.layers)]
    kept = [l for l in range(w.layers) if gates[l]]
    assert kept == [0, 3, 4, 6, 7]
    lengths = syn.seq_lengths(w)
    taps, y, dy = _run_stack(st, w, step=t, lengths=lengths)
    assert [i for i, _ in taps] == kept
    # a dropped layer is the identity: the same computation as a stack built
    # from the kept layers alone, bit for bit, in forward and backward
    ref = _stack(w, len(kept), layer_ids=kept)
    taps2, y2, _ = _run_stack(ref, w, step=t, lengths=lengths)
    assert torch.equal(y.detach(), y2.detach())
    assert torch.equal(taps[0][1].grad, taps2[0][1].grad)
    for a, b in zip([st.layers[l] for l in kept], ref.layers):
        for n in NAMES:
            assert torch.equal(getattr(a, n).grad, getattr(b, n).grad), n
    for l in range(w.layers):
        if not gates[l]:
            assert all(getattr(st.layers[l], n).grad is None for n in NAMES)
    # every kept layer against the oracle, teacher-forced
    for pos in range(len(kept)):
        _teacher_forced(w, st, taps, y, dy, pos, t, lengths)
