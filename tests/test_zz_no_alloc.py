"""The allocation-free split-KV decode entry point (tree_decode_splitkv_noalloc),
through the C ABI, against the workspace entry point it mirrors: outputs
bitwise equal on two calls in a row, the second with a smaller input (the
fixed scratch keeps the first call's contents), and within the decode bar of
the float64 oracle; a request whose partials exceed the fixed scratch is
refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
import prefix_shared_masked_amd as pkg

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(lens, Hq, Hkv, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    B, d = len(lens), 128
    total = int(sum(lens)) + 64
    q = torch.randn(B, Hq, d, generator=g, device=DEV).bfloat16()
    k = torch.randn(total, Hkv, d, generator=g, device=DEV).bfloat16()
    v = torch.randn(total, Hkv, d, generator=g, device=DEV).bfloat16()
    starts = np.concatenate([[7], 7 + np.cumsum(lens)[:-1]]).astype(np.int32)
    span_ptr = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    spans = torch.from_numpy(np.stack([starts, np.asarray(lens, np.int32)], 1)).to(DEV)
    return q, k, v, span_ptr, spans


@pytest.mark.parametrize("first,second", [((8, 32, 8, [4096, 1000, 70000, 33, 2048, 65536, 1, 5000]),
                                           (3, 8, 2, [300, 20, 900]))])
def test_noalloc_decode_matches_workspace_call(first, second):
    for call, (B, Hq, Hkv, lens) in enumerate((first, second)):
        print(f"[noalloc] call {call}: B={B} Hq={Hq} Hkv={Hkv} max_len={max(lens)}", flush=True)
        q, k, v, span_ptr, spans = _inputs(lens, Hq, Hkv, 40 + call)
        need, S = pkg.decode_ws_bytes(B, Hq, 128, max(lens))
        assert need <= pkg.DECODE_SCRATCH_BYTES
        o_ref, l_ref = pkg.tree_decode_splitkv(q, k, v, span_ptr, spans, max(lens))
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(l_ref)
        pkg.tree_decode_splitkv_noalloc(q, k, v, span_ptr, spans, max(lens), o=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        ro, rl = oracle.decode_attention(*(t.float().cpu().double().numpy() for t in (q, k, v)),
                                         span_ptr.cpu().numpy(), spans.cpu().numpy())
        err = np.abs(o.float().cpu().numpy() - ro)
        assert (err <= 2e-2 + 1e-2 * np.abs(ro)).all(), float(err.max())
        assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


def test_noalloc_decode_refuses_partials_beyond_the_scratch():
    B, Hq, Hkv = 16, 64, 8
    need, _ = pkg.decode_ws_bytes(B, Hq, 128, 1 << 18)
    assert need > pkg.DECODE_SCRATCH_BYTES
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(64, Hkv, 128, dtype=torch.bfloat16, device=DEV)
    span_ptr = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    spans = torch.zeros(1, 2, dtype=torch.int32, device=DEV)
    o, lse = torch.empty_like(q), torch.empty(B, Hq, device=DEV)
    with pytest.raises(ValueError, match="scratch"):
        pkg.tree_decode_splitkv_noalloc(q, k, k, span_ptr, spans, 1 << 18, o=o, lse=lse)
    # the C call itself refuses it too (status 4, nothing launched)
    L = pkg.load_library()
    st = L.tree_decode_splitkv_noalloc(1, pkg._ptr(q), pkg._ptr(k), pkg._ptr(k), pkg._ptr(span_ptr), pkg._ptr(spans),
                                       B, Hq, Hkv, 128, 1 << 18, 0.0, 0, pkg._ptr(o), pkg._ptr(lse), pkg._stream(q))
    assert st == 4
