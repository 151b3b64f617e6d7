"""Chained backward through Pre-LN stacks (tel_layer_backward_chain): each
layer's LayerNorm-1 backward also applies the next layer's hidden-dropout
mask (site 2, DS guide hidden_dropout_ratio; AI-infra blog section 5.1) to
the gradient it passes down, in place of a separate pass over dy in that
layer.  Every output of every layer must keep the bits of the plain
tel_layer_backward path, and the torch front end (EncoderStack) must take the
chained path."""
import numpy as np
import pytest

from _harness import NAMES
from transformer_encoder_layer_amd import synthetic as syn

pytestmark = pytest.mark.gpu

SMALL = dict(batch=4, seq=128, hidden=256, heads=4, ffn=1024)


def _layers(w, n):
    import torch
    from transformer_encoder_layer_amd import binding as B
    from transformer_encoder_layer_amd.layer import LayerConfig
    hs, Ps, saved = [], [], []
    for l in range(n):
        cfg = LayerConfig(w.batch, w.seq, w.hidden, w.heads, w.ffn, float(np.float32(w.attn_p)),
                          float(np.float32(w.hidden_p)), True, w.seed, l, syn.torch_dtype(w.dtype), 1e-12,
                          w.attn_dropout_checkpoint, w.normalize_invertible, w.gelu_checkpoint)
        h = B.tel_layer_create(cfg.to_c())
        p64 = syn.layer_params(w, l)
        hs.append(h)
        Ps.append({n_: syn.to_storage(p64[n_], w.dtype).cuda() for n_ in NAMES})
        saved.append(torch.empty(B.tel_layer_workspace_bytes(h)[0], dtype=torch.uint8, device="cuda"))
    scratch = torch.empty(max(B.tel_layer_workspace_bytes(h)[1] for h in hs), dtype=torch.uint8, device="cuda")
    return hs, Ps, saved, scratch


def _run(w, hs, Ps, saved, scratch, chained, training, lengths, step=5):
    """Forward through the stack, then backward, plain or chained; returns
    every layer's dx and gradients (as host arrays)."""
    import torch
    from transformer_encoder_layer_amd import binding as B
    x0 = syn.to_storage(syn.layer_input(w), w.dtype).cuda()
    dy = syn.to_storage(syn.upstream_grad(w), w.dtype).cuda()
    lens = None if lengths is None else torch.from_numpy(np.asarray(lengths, dtype=np.int32)).cuda()
    xs = [x0]
    for l, h in enumerate(hs):
        y = torch.empty_like(x0)
        B.tel_layer_forward(h, B.make_params(Ps[l]), xs[-1], lens, training, step, y, saved[l], scratch)
        xs.append(y)
    out = {}
    g, gd = dy, None
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    for i, l in enumerate(reversed(range(len(hs)))):
        dx = torch.empty_like(x0)
        G = {n: torch.empty_like(Ps[l][n]) for n in NAMES}
        if chained:
            below = hs[l - 1] if l > 0 else None
            od = bufs[i % 2] if below is not None else None
            B.tel_layer_backward_chain(hs[l], B.make_params(Ps[l]), xs[l], lens, training, step, g, gd, saved[l],
                                       scratch, dx, below, od, B.make_grads(G))
            gd = od
        else:
            B.tel_layer_backward(hs[l], B.make_params(Ps[l]), xs[l], lens, training, step, g, saved[l], scratch, dx,
                                 B.make_grads(G))
        torch.cuda.synchronize()
        out[f"dx{l}"] = dx.cpu()
        out.update({f"{n}{l}": G[n].cpu() for n in NAMES})
        g = dx
    return out


@pytest.mark.parametrize("dtype,shape,n,training,lengths", [
    ("f16", "small", 3, 1, (70, 128, 128, 100)),
    ("bf16", "small", 3, 1, None),     # fp32 residual gradient: the other LayerNorm-1 form
    ("f16", "small", 2, 0, None),      # no dropout: the handed-down gradient is dx itself
    ("f16", "bert_large", 2, 1, None),
])
def test_chain_equals_unchained(dtype, shape, n, training, lengths):
    from transformer_encoder_layer_amd import binding as B
    if shape == "small":
        w = syn.Workload("chain", **SMALL, pre_ln=True, dtype=dtype, attn_p=0.1, hidden_p=0.1, seed=11,
                         lengths=lengths)
    else:
        w = syn.WORKLOADS["bert_large"]
    print("case", dtype, shape, n, training, lengths, flush=True)
    hs, Ps, saved, scratch = _layers(w, n)
    try:
        a = _run(w, hs, Ps, saved, scratch, False, training, lengths)
        b = _run(w, hs, Ps, saved, scratch, True, training, lengths)
        for k in a:
            assert np.array_equal(a[k].double().numpy(), b[k].double().numpy()), k
    finally:
        for h in hs:
            B.tel_layer_destroy(h)


def test_encoder_stack_takes_the_chain(monkeypatch):
    import torch
    from transformer_encoder_layer_amd import binding as B
    from test_gpu_stack import _stack
    w = syn.Workload("chain", **SMALL, pre_ln=True, dtype="f16", attn_p=0.1, hidden_p=0.1, seed=12)
    calls = {"chain": 0, "plain": 0}
    chain_fn, plain_fn = B.tel_layer_backward_chain, B.tel_layer_backward

    def chain(*a, **k):
        calls["chain"] += 1
        return chain_fn(*a, **k)

    def plain(*a, **k):
        calls["plain"] += 1
        return plain_fn(*a, **k)

    monkeypatch.setattr(B, "tel_layer_backward_chain", chain)
    monkeypatch.setattr(B, "tel_layer_backward", plain)
    st = _stack(w, 3)
    x = syn.to_storage(syn.layer_input(w), w.dtype).cuda().requires_grad_(True)
    dy = syn.to_storage(syn.upstream_grad(w), w.dtype).cuda()
    y = st(x, None, 5)
    y.backward(dy)
    torch.cuda.synchronize()
    assert calls == {"chain": 3, "plain": 0}, calls
    # the same layers called one by one through the plain backward
    hs = [layer.handle for layer in st.layers]
    Ps = [{n: getattr(layer, n).detach() for n in NAMES} for layer in st.layers]
    saved = [torch.empty(layer.saved_bytes, dtype=torch.uint8, device="cuda") for layer in st.layers]
    scratch = torch.empty(max(layer.scratch_bytes for layer in st.layers), dtype=torch.uint8, device="cuda")
    ref = _run(w, hs, Ps, saved, scratch, False, 1, None)
    assert np.array_equal(x.grad.cpu().double().numpy(), ref["dx0"].double().numpy())
    for l, layer in enumerate(st.layers):
        for n in NAMES:
            assert np.array_equal(getattr(layer, n).grad.cpu().double().numpy(), ref[f"{n}{l}"].double().numpy()), \
                (l, n)
