"""GPU parity of the fused layer (through the C ABI) against the fp64 oracle.

Tolerances: fp32 max-abs 1e-5 on y, dx and every gradient; fp16/bf16
max-abs 2e-2 on y and relative-norm 5e-2 on dx and each gradient; dropout
masks bit-exact (test_gpu_masks.py).  Small cases run every sequence
through the oracle.  The Post-LN BERT-Base and long-sequence workloads are
compared in full (whole batch, full upstream gradient); the BERT-Large and
memory-saving stacks in full, layer by layer, in test_gpu_stack.py.  The
remaining full-size cases here compare sampled sequences (dy is zero on the
others, so every weight gradient is exactly the sum over the sampled
sequences, which the oracle computes)."""
import numpy as np
import pytest

import oracle
from _harness import (NAMES, compare, compare_full, compare_packed, gpu_layer, oracle_full, oracle_layer, prepare,
                      rel_norm, zero_padding_grad)
from transformer_encoder_layer_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def _run(w, batches=None, dy_rows=None, step=0, layer_id=0, switches=None, random_affine=True,
         weight_scale=1.0, invertible=None):
    data = prepare(w, layer=layer_id, random_affine=random_affine, weight_scale=weight_scale)
    g = gpu_layer(w, data, step=step, layer_id=layer_id, dy_rows=dy_rows, switches=switches)
    inv = w.normalize_invertible if invertible is None else invertible
    o = oracle_layer(w, data, step=step, layer_id=layer_id, batches=batches, dy_rows=dy_rows, invertible=inv)
    bs = list(range(w.batch)) if batches is None else batches
    rep = compare(w, g, o, bs)
    print(w.name, {k: f"{v:.3g}" for k, v in rep.items()})
    return g, o


# ------------------------------------------------------------------ tiny fp32
@pytest.mark.parametrize("pre_ln", [True, False])
def test_tiny_fp32(pre_ln):
    w = syn.WORKLOADS["tiny"].with_(pre_ln=pre_ln)
    _run(w, weight_scale=4.0)


@pytest.mark.parametrize("pre_ln", [True, False])
def test_tiny_fp32_dropout(pre_ln):
    w = syn.WORKLOADS["tiny"].with_(pre_ln=pre_ln, attn_p=0.1, hidden_p=0.1)
    _run(w, step=3, layer_id=2, weight_scale=4.0)


# ------------------------------------------------------------------ MFMA paths, small shapes
SMALL = dict(batch=4, seq=128, hidden=256, heads=4, ffn=1024)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pre_ln", [True, False])
def test_small_lowp(dtype, pre_ln):
    w = syn.Workload("small", **SMALL, pre_ln=pre_ln, dtype=dtype, attn_p=0.1, hidden_p=0.1, seed=11,
                     lengths=(1, 128))
    _run(w, step=7, layer_id=1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_lowp_ragged_seq(dtype):
    # S = 192: attention has a partial 128-query block; lengths hit block edges
    w = syn.Workload("ragged", 2, 192, 128, 2, 512, True, dtype, 0.1, 0.1, 5, lengths=(63, 65))
    _run(w)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_lowp_seq64(dtype):
    # S = 64: the single-workgroup attention backward with half its waves idle
    w = syn.Workload("s64", 3, 64, 256, 4, 1024, True, dtype, 0.1, 0.1, 13, lengths=(1, 64))
    _run(w, step=4)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_lowp_d32_simt_attention(dtype):
    # head width 32 takes the generic attention kernel
    w = syn.Workload("d32", 2, 64, 128, 4, 512, False, dtype, 0.1, 0.1, 9, lengths=(5, 64))
    _run(w)


def test_max_hidden_head128():
    # the largest hidden width the layer accepts (2048: eight 256-column
    # groups per LayerNorm lane) with 128-wide heads (generic attention
    # kernel at its largest head width).  fp16: in bf16 the output error at
    # this width is bf16's rounding (8x fp16's, 3 fewer mantissa bits) and
    # reaches the 2e-2 output bound itself.
    w = syn.Workload("h2048", 2, 64, 2048, 16, 4096, True, "f16", 0.1, 0.1, 17, lengths=(20, 64))
    _run(w, step=2)


def test_hidden1536_postln():
    # hidden 1536: six 256-column groups per LayerNorm lane; 24 heads of 64
    w = syn.Workload("h1536", 2, 128, 1536, 24, 2048, False, "bf16", 0.1, 0.1, 19, lengths=(40, 128))
    _run(w)


# ------------------------------------------------------------------ masks
@pytest.mark.parametrize("site", [0, 1, 2])
def test_dropout_masks_bitexact(site):
    import torch
    from transformer_encoder_layer_amd import binding as B
    from transformer_encoder_layer_amd.layer import LayerConfig
    cfg = LayerConfig(3, 64, 128, 2, 512, 0.1, 0.25, True, 99, 5, torch.float16)
    h = B.tel_layer_create(cfg.to_c())
    try:
        n = 3 * 2 * 64 * 64 if site == 0 else 3 * 64 * 128
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
        B.tel_debug_dropout_mask(h, site, 77, out)
        got = out.cpu().numpy()
    finally:
        B.tel_layer_destroy(h)
    p = float(np.float32(0.1 if site == 0 else 0.25))
    want = oracle.dropout_mask(99, 5, site, 77, p, 0, n)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ memory switches
@pytest.mark.parametrize("pre_ln", [True, False])
def test_checkpoint_switches_bitwise(pre_ln):
    w = syn.Workload("sw", **SMALL, pre_ln=pre_ln, dtype="f16", attn_p=0.1, hidden_p=0.1, seed=3,
                     lengths=(30, 128))
    data = prepare(w, random_affine=True)
    base = gpu_layer(w, data, step=1)
    for sw in (dict(gelu_checkpoint=True), dict(attn_dropout_checkpoint=True),
               dict(gelu_checkpoint=True, attn_dropout_checkpoint=True)):
        other = gpu_layer(w, data, step=1, switches=sw)
        for k in base:
            assert np.array_equal(base[k], other[k]), (sw, k)


@pytest.mark.parametrize("pre_ln", [True, False])
def test_invertible_layernorm(pre_ln):
    w = syn.Workload("inv", **SMALL, pre_ln=pre_ln, dtype="f16", attn_p=0.1, hidden_p=0.1, seed=4,
                     lengths=(30, 128), normalize_invertible=True)
    _run(w, step=2)


def test_run_to_run_deterministic():
    w = syn.Workload("det", **SMALL, pre_ln=True, dtype="bf16", attn_p=0.1, hidden_p=0.1, seed=8)
    data = prepare(w, random_affine=True)
    a = gpu_layer(w, data, step=4)
    b = gpu_layer(w, data, step=4)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_run_to_run_deterministic_bert_large():
    # BERT-Large shapes: both weight-gradient pairs split k (2 and 4 ways) and
    # the last-arriving split reduces each tile; whichever split arrives last,
    # the partials are summed in split order, so every output keeps its bits
    w = syn.WORKLOADS["bert_large"]
    data = prepare(w, random_affine=True)
    a = gpu_layer(w, data, step=1, layer_id=4)
    for _ in range(2):
        b = gpu_layer(w, data, step=1, layer_id=4)
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_stochastic_mode_bert_large():
    # Relaxed determinism (stochastic_mode): the grouped weight-gradient
    # launches add their k-splits (2 for W_2 + W_1, 4 for W_o + W_qkv at these
    # shapes) into the zeroed gradients with packed fp16 atomics.  Only those
    # eight gradients change, by about one fp16 rounding per split, and the
    # whole layer stays within the oracle's tolerances over the full batch.
    w = syn.WORKLOADS["bert_large"]
    data = prepare(w, layer=4, random_affine=True)
    det = gpu_layer(w, data, step=1, layer_id=4)
    sto = gpu_layer(w, data, step=1, layer_id=4, switches=dict(stochastic_mode=True))
    pair = {"g_w_o", "g_b_o", "g_w_qkv", "g_b_qkv", "g_w_1", "g_b_1", "g_w_2", "g_b_2"}
    for k in det:
        if k in pair:
            assert rel_norm(sto[k], det[k]) < 2e-3, k
        else:
            assert np.array_equal(sto[k], det[k]), k
    o_y, o_dx, o_g = oracle_full(w, data["params_r"], data["x_r"], data["dy_r"], data["lengths"], step=1,
                                 layer_id=4)
    compare_full(w, sto["y"], sto["dx"], {n: sto["g_" + n] for n in NAMES}, o_y, o_dx, o_g, tag="stochastic")


def test_inference_forward_no_saved():
    import torch
    from transformer_encoder_layer_amd import binding as B
    from transformer_encoder_layer_amd.layer import LayerConfig
    w = syn.Workload("inf", **SMALL, pre_ln=True, dtype="f16", attn_p=0.1, hidden_p=0.1, seed=6)
    data = prepare(w, random_affine=True)
    ref = gpu_layer(w, data, training=False, backward=False)
    o = oracle_layer(w, data, training=False, backward=False)
    compare(w, ref, o, list(range(w.batch)), check_grads=False)
    cfg = LayerConfig(w.batch, w.seq, w.hidden, w.heads, w.ffn, 0.1, 0.1, True, 6, 0, torch.float16)
    h = B.tel_layer_create(cfg.to_c())
    try:
        sv, sc = B.tel_layer_workspace_bytes(h)
        P = {n: data["params_t"][n].cuda() for n in NAMES}
        x = data["x_t"].cuda()
        y = torch.empty_like(x)
        scratch = torch.empty((sc + 255) // 256 * 256 + sv, dtype=torch.uint8, device="cuda")
        B.tel_layer_forward(h, B.make_params(P), x, None, 0, 0, y, None, scratch)
        torch.cuda.synchronize()
        assert np.array_equal(y.double().cpu().numpy(), ref["y"])
        with pytest.raises(B.TelError):
            B.tel_layer_backward(h, B.make_params(P), x, None, 0, 0, x, scratch, scratch, y,
                                 B.make_grads(P))
    finally:
        B.tel_layer_destroy(h)


# ------------------------------------------------------------------ token packing
def _run_packed(w, batches=None, dy_rows=None, step=0, layer_id=0, random_affine=True):
    data = prepare(w, layer=layer_id, random_affine=random_affine)
    zero_padding_grad(w, data)
    valid = int(np.asarray(data["lengths"]).sum())
    assert (valid + 255) // 256 * 256 < w.batch * w.seq, "case must leave padding for packing to remove"
    g = gpu_layer(w, data, step=step, layer_id=layer_id, dy_rows=dy_rows, pack=True)
    o = oracle_layer(w, data, step=step, layer_id=layer_id, batches=batches, dy_rows=dy_rows)
    bs = list(range(w.batch)) if batches is None else batches
    rep = compare_packed(w, g, o, bs)
    print(w.name, "packed", {k: f"{v:.3g}" for k, v in rep.items()})


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pre_ln", [True, False])
def test_packed_tokens_short_seq(dtype, pre_ln):
    # S = 128 (whole-sequence attention kernels); sum of lengths leaves >= 256 rows to skip
    w = syn.Workload("packed128", 8, 128, 256, 4, 1024, pre_ln, dtype, 0.1, 0.1, 21, lengths=(9, 100))
    _run_packed(w, step=4, layer_id=3)


@pytest.mark.parametrize("pre_ln", [True, False])
def test_packed_tokens_streaming(pre_ln):
    # S = 256 (streaming attention kernels, partial key blocks)
    w = syn.Workload("packed256", 4, 256, 256, 4, 1024, pre_ln, "bf16", 0.1, 0.1, 23, lengths=(30, 150))
    _run_packed(w, step=2, layer_id=1)


def test_packed_tokens_bert_base_postln():
    # the padded Post-LN workload at full size, two sequences checked
    w = syn.WORKLOADS["bert_base_postln"]
    rows = np.zeros(w.batch, dtype=bool)
    rows[[0, 31]] = True
    _run_packed(w, batches=[0, 31], dy_rows=rows, random_affine=False)


def test_packed_tokens_bert_large_shape():
    # BERT-Large shapes with padding: the packed rows (valid tokens rounded up
    # to 256) are the k of the weight gradients, which still run as grouped
    # pairs, the last one also summing the LayerNorm gamma/beta partials
    w = syn.WORKLOADS["bert_large"].with_(lengths=(64, 128))
    rows = np.zeros(w.batch, dtype=bool)
    rows[[3, 50]] = True
    _run_packed(w, batches=[3, 50], dy_rows=rows, step=1, layer_id=2)


# ------------------------------------------------------------------ full-size workloads, sampled
def _sampled(name, batches, **over):
    w = syn.WORKLOADS[name].with_(**over)
    rows = np.zeros(w.batch, dtype=bool)
    rows[batches] = True
    return _run(w, batches=batches, dy_rows=rows, random_affine=False)


def test_full_bert_large_layer():
    _sampled("bert_large", [0, 63])


def test_full_bert_large_shape_postln():
    # Post-LN at the BERT-Large shapes, where the last weight-gradient pair
    # runs grouped and both LayerNorm gamma/beta sums (LN2's from the first
    # backward kernel on) ride with its reduction
    w = syn.WORKLOADS["bert_large"].with_(pre_ln=False)
    rows = np.zeros(w.batch, dtype=bool)
    rows[[9, 40]] = True
    _run(w, batches=[9, 40], dy_rows=rows, layer_id=5, step=3, random_affine=True)


def test_full_bert_large_layer23():
    w = syn.WORKLOADS["bert_large"]
    rows = np.zeros(w.batch, dtype=bool)
    rows[[17]] = True
    _run(w, batches=[17], dy_rows=rows, layer_id=23, step=5, random_affine=False)


def test_profiling_hook_keeps_results():
    # On the BERT-Large shapes the W_o and W_qkv weight gradients run as one
    # grouped launch whose split-K reduction also sums the LayerNorm gamma/beta
    # partial rows.  Profiling the W_o kernel splits the pair into two
    # launches and the LayerNorm sums into launches of their own: every output
    # keeps its bits (one fixed summation order either way) except those two
    # weight gradients and their bias gradients, whose k-split may change.
    from transformer_encoder_layer_amd import binding as B
    w = syn.WORKLOADS["bert_large"]
    data = prepare(w, random_affine=True)
    a = gpu_layer(w, data, step=2, layer_id=3)
    b = gpu_layer(w, data, step=2, layer_id=3, prof_kernel=B.KERNELS["out_wgrad"])
    split = {"g_w_o", "g_b_o", "g_w_qkv", "g_b_qkv"}
    for k in a:
        if k in split:
            assert rel_norm(b[k], a[k]) < 1e-3, k
        else:
            assert np.array_equal(a[k], b[k]), k


def test_profiling_pair_and_reduce_ids():
    # The grouped weight-gradient ids time the GEMM kernel of the pair and the
    # launch after it (its split-K reduction) without changing the launches:
    # every output keeps its bits, and each event pair spans a positive time.
    from transformer_encoder_layer_amd import binding as B
    w = syn.WORKLOADS["bert_large"]
    data = prepare(w, random_affine=True)
    a = gpu_layer(w, data, step=1, layer_id=2)
    for site in ("ffn_wgrad_pair", "ffn_wgrad_reduce", "attn_wgrad_pair", "attn_wgrad_reduce"):
        b = gpu_layer(w, data, step=1, layer_id=2, prof_kernel=B.KERNELS[site])
        assert float(b.pop("prof_ms")[0]) > 0.0, site
        for k in a:
            assert np.array_equal(a[k], b[k]), (site, k)


def _full(name, layer_id=0, step=0, random_affine=False):
    # the whole batch with the full upstream gradient: every element of y,
    # dx and the twelve parameter gradients against the oracle
    w = syn.WORKLOADS[name]
    data = prepare(w, layer=layer_id, random_affine=random_affine)
    g = gpu_layer(w, data, step=step, layer_id=layer_id)
    o_y, o_dx, o_g = oracle_full(w, data["params_r"], data["x_r"], data["dy_r"], data["lengths"], step=step,
                                 layer_id=layer_id, invertible=w.normalize_invertible)
    compare_full(w, g["y"], g["dx"], {n: g["g_" + n] for n in NAMES}, o_y, o_dx, o_g, tag=name)


@pytest.mark.timeout(600)
def test_full_bert_base_postln():
    _full("bert_base_postln", layer_id=2, step=1)


@pytest.mark.timeout(600)
def test_full_long_seq():
    _full("long_seq", step=3)


def test_full_memsave_layer():
    _sampled("memsave_stack", [0, 127])


def test_debug_build_checks_key_lengths():
    # libtel_debug.so reads the device key lengths back before launching
    # anything: valid lengths give the release library's results bit for
    # bit; a length outside [1, S] is refused on the host, before any kernel
    import ctypes
    import torch
    from transformer_encoder_layer_amd import binding as B
    from transformer_encoder_layer_amd.layer import LayerConfig
    D = B.lib(B.DEBUG_LIB_PATH)
    assert B.tel_debug_checks_enabled(D)
    w = syn.Workload("dbg", 3, 64, 256, 4, 1024, True, "f16", 0.1, 0.1, 31, lengths=(5, 64))
    data = prepare(w, random_affine=True)
    ref = gpu_layer(w, data, step=2)
    cfg = LayerConfig(w.batch, w.seq, w.hidden, w.heads, w.ffn, float(np.float32(0.1)), float(np.float32(0.1)),
                      True, w.seed, 0, torch.float16).to_c()
    h = ctypes.c_void_p()
    assert D.tel_layer_create(ctypes.byref(cfg), ctypes.byref(h)) == 0
    try:
        sv, sc = ctypes.c_size_t(), ctypes.c_size_t()
        assert D.tel_layer_workspace_bytes(h, ctypes.byref(sv), ctypes.byref(sc)) == 0
        P = {n: data["params_t"][n].cuda() for n in NAMES}
        x = data["x_t"].cuda()
        y = torch.empty_like(x)
        dx = torch.empty_like(x)
        G = {n: torch.empty_like(P[n]) for n in NAMES}
        saved = torch.empty(sv.value, dtype=torch.uint8, device="cuda")
        scratch = torch.empty(sc.value, dtype=torch.uint8, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        good = torch.from_numpy(data["lengths"]).cuda()
        params = B.make_params(P)
        assert D.tel_layer_forward(h, ctypes.byref(params), x.data_ptr(), good.data_ptr(), 1, 2, y.data_ptr(),
                                   saved.data_ptr(), scratch.data_ptr(), st) == 0
        grads = B.make_grads(G)
        assert D.tel_layer_backward(h, ctypes.byref(params), x.data_ptr(), good.data_ptr(), 1, 2,
                                    data["dy_t"].cuda().data_ptr(), saved.data_ptr(), scratch.data_ptr(),
                                    dx.data_ptr(), ctypes.byref(grads), st) == 0
        torch.cuda.synchronize()
        assert np.array_equal(y.double().cpu().numpy(), ref["y"])
        assert np.array_equal(dx.double().cpu().numpy(), ref["dx"])
        for bad in ([0, 10, 20], [64, 65, 3]):
            lens = torch.tensor(bad, dtype=torch.int32, device="cuda")
            rc = D.tel_layer_forward(h, ctypes.byref(params), x.data_ptr(), lens.data_ptr(), 1, 2, y.data_ptr(),
                                     saved.data_ptr(), scratch.data_ptr(), st)
            assert rc == B.TEL_ERR_INVALID_ARG and b"key_lengths" in D.tel_last_error()
    finally:
        D.tel_layer_destroy(h)
