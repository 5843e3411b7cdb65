"""GPU parity of tree_lmhead_nll (output layer fused with the weighted NLL)
against the float64 oracle (oracle/lmhead.py).

Inputs are bf16, rounded once on the host; the oracle sees the rounded values.
Bars: loss to 1e-4 relative, LSE to 1e-3 absolute (fp32 accumulation of exact
bf16 products).  dh and dW are sums over the vocabulary / the tokens of
dlogits rounded to bf16 (relative error 2^-9 per term) times bf16 operands,
accumulated in fp32 and stored in bf16 (2^-9 of the result): elementwise
|gpu - ref| <= 1e-2 |ref| + 4e-3 M, where M is the sum of the magnitudes of
the element's terms (|dlogits| |W| for dh, |dlogits|^T |h| for dW), the
quantity that bounds the rounding error of a sum."""
import numpy as np
import pytest
import torch

import prefix_shared_masked_amd as pkg
from oracle.lmhead import lmhead_vocab_rows, lmhead_weighted_nll
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def inputs(N, V, Dm, seed, p_ignore=0.2):
    rng = np.random.default_rng(seed)
    h = torch.from_numpy(rng.standard_normal((N, Dm), dtype=np.float32)).bfloat16()
    Wt = torch.from_numpy((rng.standard_normal((V, Dm), dtype=np.float32) / np.sqrt(Dm)).astype(np.float32)).bfloat16()
    labels = rng.integers(0, V, N).astype(np.int32)
    labels[rng.random(N) < p_ignore] = -100
    w = rng.random(N).astype(np.float32)
    return h, Wt, labels, w


def grad_close(name, got, ref, mag):
    got = got.float().cpu().double().numpy()
    err = np.abs(got - ref)
    bar = 1e-2 * np.abs(ref) + 4e-3 * mag
    bad = err > bar
    assert not bad.any(), f"{name}: {int(bad.sum())} of {bad.size} outside, max err {err.max():.3e}"


def run(N, V, Dm, seed, vocab_chunk=0, grads=True):
    print(f"[lmhead] N={N} V={V} Dm={Dm} chunk={vocab_chunk}", flush=True)
    h, Wt, labels, w = inputs(N, V, Dm, seed)
    loss, lse, dh, dW, err = pkg.tree_lmhead_nll(h.to(DEV), Wt.to(DEV), torch.from_numpy(labels).to(DEV),
                                                 torch.from_numpy(w).to(DEV), need_grad=grads,
                                                 vocab_chunk=vocab_chunk)
    torch.cuda.synchronize()
    ref = lmhead_weighted_nll(h.double().numpy(), Wt.double().numpy(), labels, w)
    assert int(err.item()) == 0
    assert loss.item() == pytest.approx(ref["loss"], rel=1e-4)
    np.testing.assert_allclose(lse.cpu().numpy(), ref["lse"], rtol=0, atol=1e-3)
    if grads:
        absdl = np.abs(ref["dlogits"])
        grad_close("dh", dh, ref["dh"], absdl @ np.abs(Wt.double().numpy()))
        grad_close("dW", dW, ref["dW"], absdl.T @ np.abs(h.double().numpy()))
    return loss, dh, dW


def test_small_ragged_tiles():
    run(300, 1000, 64, 0)                        # 2 token tiles (one ragged), 4 vocab tiles (one ragged)


@pytest.mark.parametrize("chunk", [256, 512, 768])
def test_backward_chunks(chunk):
    run(290, 1000, 96, 1, vocab_chunk=chunk)     # several recompute chunks, a ragged last one


def test_forward_only_and_single_token():
    run(1, 300, 32, 2, grads=False)
    run(1, 300, 32, 2)


def test_mid_size():
    run(1500, 12000, 256, 3)


def test_bad_label_flag_and_ignore():
    h, Wt, labels, w = inputs(40, 257, 32, 4, p_ignore=0.0)
    labels[3] = 257          # out of range: contributes 0 and raises the flag
    labels[5] = -100
    loss, lse, dh, dW, err = pkg.tree_lmhead_nll(h.to(DEV), Wt.to(DEV), torch.from_numpy(labels).to(DEV),
                                                 torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    ok = labels.copy()
    ok[3] = -100
    ref = lmhead_weighted_nll(h.double().numpy(), Wt.double().numpy(), ok, w)
    assert loss.item() == pytest.approx(ref["loss"], rel=1e-4)
    absdl = np.abs(ref["dlogits"])
    grad_close("dh", dh, ref["dh"], absdl @ np.abs(Wt.double().numpy()))
    grad_close("dW", dW, ref["dW"], absdl.T @ np.abs(h.double().numpy()))


@pytest.mark.timeout(900)
def test_full_output_layer_sampled():
    """The Qwen3-0.6B output-layer shape (V = 151,936, Dm = 1,024) over the
    spine tree's 16,352 tokens with g/K weights: LSE, token loss and dh of
    sampled tokens against the oracle row by row; dW on 64 sampled
    vocabulary rows (labels among them) element by element against the
    full-vocabulary oracle; <dW, W> == <dh, h> (both equal
    sum_t,v dlogits_tv logits_tv); bitwise repeatable."""
    tree = W.spine_tree()
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    N, V, Dm = plan.n_tokens, 151936, 1024
    g = torch.Generator().manual_seed(7)
    h = torch.randn(N, Dm, generator=g).bfloat16()
    Wt = (torch.randn(V, Dm, generator=g) / 32.0).bfloat16()
    labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int32)
    labels[torch.rand(N, generator=g) < 0.1] = -100
    w = torch.from_numpy((plan.view()["g"] / plan.n_leaves).astype(np.float32))
    args = (h.to(DEV), Wt.to(DEV), labels.to(DEV), w.to(DEV))
    loss, lse, dh, dW, err = pkg.tree_lmhead_nll(*args)
    loss2, lse2, dh2, dW2, _ = pkg.tree_lmhead_nll(*args)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(loss, loss2) and torch.equal(lse, lse2) and torch.equal(dh, dh2) and torch.equal(dW, dW2)
    rows = np.unique(np.concatenate([np.random.default_rng(0).integers(0, N, 40), [0, N - 1]]))
    W64 = Wt.double().numpy()
    h64 = h.double().numpy()
    lab = labels.numpy()
    for t in rows:
        x = W64 @ h64[t]
        m = x.max()
        lse_t = m + np.log(np.exp(x - m).sum())
        assert abs(lse[t].item() - lse_t) <= 1e-3, t
        if lab[t] != -100:
            p = np.exp(x - lse_t)
            p[lab[t]] -= 1.0
            ref_dh = w[t].item() * (p @ W64)
            mag = w[t].item() * (np.abs(p) @ np.abs(W64))
            got = dh[t].float().cpu().double().numpy()
            assert (np.abs(got - ref_dh) <= 1e-2 * np.abs(ref_dh) + 4e-3 * mag).all(), t
    rng = np.random.default_rng(1)
    vrows = np.unique(np.concatenate([rng.choice(V, 56, replace=False), lab[lab >= 0][:6], [0, V - 1]]))
    print(f"[lmhead] full-size dW on {len(vrows)} vocabulary rows", flush=True)
    rv = lmhead_vocab_rows(h64, W64, lab, w.numpy(), vrows)
    assert np.abs(lse.cpu().numpy() - rv["lse"]).max() <= 1e-3
    grad_close("dW(sampled rows)", dW[torch.from_numpy(vrows).to(DEV)], rv["dW"], rv["dW_abs"])
    a = float((dW.double() * Wt.to(DEV).double()).sum())
    b = float((dh.double() * h.to(DEV).double()).sum())
    assert a == pytest.approx(b, rel=2e-2)
