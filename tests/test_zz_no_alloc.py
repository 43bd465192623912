"""recsa_decode_multi_noalloc (the multi-sequence decode for callers that cannot
allocate: its sequence table lives in a fixed device table inside the library)
against recsa_decode_multi with a caller workspace, through the C ABI, on two
calls in a row, the second with fewer sequences (the table keeps the first call's
longer contents).  Both take the same kernel, so outputs and debug records must be
identical; one sequence of each call is also checked against the oracle."""
import numpy as np
import pytest
import torch

import long_context_recsa_amd as R
import synth
from long_context_recsa_amd.layer import decode_multi
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _sequences(base, lengths, cap):
    out = []
    for i, L in enumerate(lengths):
        w = synth.scaled(base, L, prefill_n=0, cfg_id=5000 + i, needles=0)
        K, V = synth.gen_kv(w, 0, L)
        W = synth.pool_w(w)
        layer = P.make_layer(w, capacity=cap)
        P.load_cache(layer, K, V, W, L, w.dtype)
        layer.build(L)
        out.append((w, K, V, W, layer))
    return out


@pytest.mark.parametrize("name", ["tiny_f32_4k", "qwen3_4b_131k"])
def test_noalloc_matches_workspace_call(name):
    base = synth.WORKLOADS[name]
    if name == "tiny_f32_4k":
        base = synth.scaled(base, 4096, n_kv=2, n_q=4)
        lengths_all = [int(x) for x in np.random.default_rng(3).integers(20, 4097, size=40)]
        cap = 4096
    else:
        base = synth.scaled(base, 8192, n_kv=2, n_q=8)
        lengths_all = [int(x) for x in np.random.default_rng(4).integers(300, 6001, size=40)]
        cap = 6000
    seqs = _sequences(base, lengths_all, cap)
    rng = np.random.default_rng(7)
    Q = synth.to_storage(rng.standard_normal((40, base.n_q, base.d)).astype(np.float32), base.dtype)
    G = base.n_q // base.n_kv
    for n in (40, 34):        # both past the 32 sequences whose table travels with the launch
        _say(f"case noalloc {name} n_seq={n}")
        layers = [s[4] for s in seqs[:n]]
        q = P.to_device(Q[:n], base.dtype)
        ref = torch.empty((n, base.n_q, base.d), dtype=torch.float32, device=layers[0].device)
        got = torch.full_like(ref, 9.0)
        ref, dref = decode_multi(layers, q, debug=True, out=ref)
        got, dgot = decode_multi(layers, q, debug=True, out=got, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"n_seq={n}: no-alloc output differs from the workspace call"
        for k in ("selected", "kth_gap", "n_keys"):
            assert torch.equal(dgot[k].nan_to_num(-1.0) if k == "kth_gap" else dgot[k],
                               dref[k].nan_to_num(-1.0) if k == "kth_gap" else dref[k]), k
        i = n - 1
        w, K, V, W, _ = seqs[i]
        tree = P.head_tree(K, V, W, 0, w, w.L)
        sub = {k: v[i * w.n_q:(i + 1) * w.n_q] for k, v in dgot.items()}
        rows = [(0, h) for h in range(G)]
        rep = P.check_rows(tree, Q[i:i + 1].astype(np.float64), rows, lambda j: w.L, w.k, w.rope_base,
                           w.softmax_scale, got[i:i + 1], sub, G, w.dtype, head_of=lambda h: 0)
        _say(f"n_seq={n}: identical to the workspace call; sequence {i} vs oracle", rep)


def test_noalloc_refuses_past_its_table():
    base = synth.scaled(synth.WORKLOADS["tiny_f32_4k"], 64)
    seqs = _sequences(base, [64], 64)
    layer = seqs[0][4]
    descs = (R.recsa_tree_desc * 4097)(*([layer.desc] * 4097))
    q = torch.zeros((4097, base.n_q, base.d), dtype=torch.float32, device=layer.device)
    out = torch.empty_like(q)
    with pytest.raises(R.RecsaError) as e:
        R.recsa_decode_multi_noalloc(layer.p, descs, 4097, ctypes_ptr(q), ctypes_ptr(out))
    assert e.value.status == R.RECSA_ERR_INVALID_ARG


def ctypes_ptr(t):
    import ctypes
    return ctypes.c_void_p(t.data_ptr())
