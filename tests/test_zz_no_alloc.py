"""dsw_walk_static, the allocation-free entry point, against dsw_walk: the
same plan and kernels on the same inputs give the same tokens and logits bit
for bit.  Each case makes two calls in a row on the shared static workspace,
the second with a smaller input, then checks the rejections of sizes beyond
the static array and of flags it does not serve."""
import numpy as np
import pytest

import gpu_helpers as gh
import parity
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dsw():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import serial_draft_head_amd as m
    m.lib()
    return m


# (V, B, gamma, temps) of the first and the second (smaller) call, and the
# flags: the one-request MFMA kernel, the all-to-all kernel with a 4-request
# tile (forced), and the batched kernel (whose sampled logits go to the static
# array when no logits are asked for) with four tiles per epilogue and with
# more requests
PAIRS = [
    ((151_936, 1, 7, "greedy"), (32_000, 1, 5, "cycle"), 0),
    ((100_003, 3, 7, "mixed"), (4_097, 2, 4, "mixed"), 8),
    ((100_003, 3, 7, "mixed"), (4_097, 2, 4, "mixed"), 0),
    ((129_280, 40, 5, "mixed"), (60_000, 6, 3, "mixed"), 0),
]


def _inputs(V, B, gamma, temps, rnd):
    W1, W2 = workloads.weights(2, V=V)
    inp = workloads.round_inputs(2, 7000 + rnd, B=B, gamma=gamma, V=V, temps=temps)
    return W1, W2, inp


@pytest.mark.parametrize("first,second,flags", PAIRS)
def test_static_entry_matches_dsw_walk(dsw, first, second, flags):
    for i, (V, B, gamma, temps) in enumerate((first, second)):
        gh.say(f"static entry, call {i + 1}: V={V} B={B} gamma={gamma} {temps} flags={flags}")
        W1, W2, inp = _inputs(V, B, gamma, temps, i)
        W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
        base, anchor, T, uni = gh.round_dev(torch, inp)
        # with and without the logits output (the batched kernel then keeps the
        # sampled logits in the static array)
        ts, ls = dsw.walk_static(W1d, W2d, base, anchor, T, uni, want_logits=True, flags=flags)
        ts2, _ = dsw.walk_static(W1d, W2d, base, anchor, T, uni, flags=flags)
        torch.cuda.synchronize()
        assert dsw.static_status(0) == 0
        walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags)
        th, lh = walker.walk(W1d, W2d, base, anchor, T, uni, want_logits=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        walker.close()
        assert torch.equal(ts, th) and torch.equal(ts2, th)
        assert torch.equal(ls.view(torch.int16), lh.view(torch.int16))
        rep = parity.check_round(parity.Weights(W1, W2), inp["base"], inp["anchor"], inp["T"], inp["uniforms"],
                                 ts.cpu().numpy(), gh.logits_host(torch, ls))
        gh.say(rep)


def test_static_entry_rejects_what_it_cannot_serve(dsw):
    V, B, gamma = 151_936, 120, 1
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    inp = workloads.round_inputs(0, 1, B=B, gamma=gamma, V=V, temps="mixed")
    base, anchor, T, uni = gh.round_dev(torch, inp)
    # the batched kernel's sampled logits would need B * V * 2 = 36.5 MB > 32 MiB of the array
    with pytest.raises(dsw.DswError) as e:
        dsw.walk_static(W1d, W2d, base, anchor, T, uni)
    assert e.value.code == -12
    # with the caller's logits the kernel keeps them there: served
    ts, ls = dsw.walk_static(W1d, W2d, base, anchor, T, uni, want_logits=True)
    torch.cuda.synchronize()
    assert dsw.static_status(0) == 0
    rep = parity.check_round(parity.Weights(W1, W2), inp["base"], inp["anchor"], inp["T"], inp["uniforms"],
                             ts.cpu().numpy(), gh.logits_host(torch, ls), requests=[0, B - 1])
    gh.say(rep)
    L = dsw.lib()
    nul = [None] * 9
    assert L.dsw_walk_static(0, V, 0, 0, *nul, 1, 257, None) == -3            # gamma above 256
    assert L.dsw_walk_static(0, V, 0, 0, *nul, 257, 1, None) == -2            # more than 256 requests
    assert L.dsw_walk_static(0, V, 0, dsw.FLAG_GUMBEL, *nul, 1, 1, None) == -11
    assert L.dsw_walk_static(0, V, 0, dsw.FLAG_GRU, *nul, 1, 1, None) == -11
    assert L.dsw_walk_static(0, V, 0, 0, *nul, 1, 1, None) == -1             # null tensors
    assert L.dsw_walk_static(0, V, 0, 0, *nul, 0, 1, None) == 0              # nothing to do
