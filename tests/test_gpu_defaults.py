"""GPU parity at the measured workloads' own sizes, on the kernels the planner
picks by default (no engine flags): the paths bench.py times.  Every request
and every step is checked against the oracle (teacher forced), with the rules
of tests/parity.py.

Coverage per workload (requests x steps x rounds):
  V = 151,936, gamma = 7, one greedy request:        1 x 7 x 100 rounds
  V = 151,936, gamma = 16, mixed T, 1 request:        1 x 16 x 3 rounds (T cycles 0, 0.6, 1)
                                    4 requests:        4 x 16 x 2 rounds
                                   16 requests:       16 x 16 x 2 rounds
  V = 248,320, gamma = 16, one greedy request, bf16:  1 x 16 x 2 rounds
                                              int8:   1 x 16 x 2 rounds (T cycles)
  V = 129,280, gamma = 5, mixed T, 64 / 128 / 253 requests: B x 5 x 1 round
"""
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


def _kernel_name(dsw, pl):
    if pl.batch_tile == 256:
        return "batched"
    return ("valu" if pl.engine == dsw.ENGINE_VALU else "mfma") + f"_b{pl.batch_tile}"


def _merge(tot, rep):
    for k, v in rep.items():
        tot[k] = tot.get(k, 0) + v
    return tot


def test_headline_100_rounds(dsw):
    """V = 151,936, gamma = 7, one greedy request: 100 seeded rounds back to
    back on one handle, every step of every round against the oracle."""
    index, n_rounds = 1, 100
    wl = workloads.WORKLOADS[index]
    gh.say(f"{wl.name}: {n_rounds} rounds, default plan")
    W1, W2 = workloads.weights(index)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=1)
    pl = walker.query_plan(1)
    gh.say("plan", pl.as_dict())
    rounds = [workloads.round_inputs(index, r, B=1) for r in range(n_rounds)]
    outs = []
    for inp in rounds:
        base, anchor, T, uni = gh.round_dev(torch, inp)
        outs.append(walker.walk(W1d, W2d, base, anchor, T, uni, want_logits=True))
    torch.cuda.synchronize()
    assert walker.status() == 0
    tot = {}
    for r, (inp, (t, l)) in enumerate(zip(rounds, outs)):
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], t.cpu().numpy(),
                                 gh.logits_host(torch, l))
        _merge(tot, rep)
    gh.say("total", tot)
    assert tot["steps"] == n_rounds * wl.gamma
    gh.report({"test": "headline_100_rounds", "workload": wl.name, "kernel": _kernel_name(dsw, pl), "B": 1,
               "rounds": n_rounds, "requests_checked": "all", "steps_checked": "all", **tot})
    walker.close()


# (workload, requests, rounds, W2 storage)
DEFAULT_CASES = [(2, 1, 3, "bf16"), (2, 4, 2, "bf16"), (2, 16, 2, "bf16"), (3, 1, 2, "bf16"), (3, 1, 2, "int8"),
                 (4, 64, 1, "bf16"), (4, 64, 1, "int8"), (4, 128, 1, "bf16"), (4, 253, 1, "bf16")]


@pytest.mark.parametrize("index,B,n_rounds,dt", DEFAULT_CASES)
def test_default_plan_every_request_every_step(dsw, index, B, n_rounds, dt):
    wl = workloads.WORKLOADS[index]
    gh.say(f"{wl.name} B={B} {dt}: {n_rounds} rounds, default plan, every request and step")
    W1, W2 = workloads.weights(index)
    W1d = gh.bf16_dev(torch, W1)
    if dt == "int8":
        Q, sc = workloads.quantize_int8(W2)
        w = parity.Weights(W1, Q=Q, scale=sc)
        W2d, sd = gh.int8_dev(torch, Q, sc)
    else:
        w = parity.Weights(W1, W2)
        W2d, sd = gh.bf16_dev(torch, W2), None
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=B, w2_dtype=dsw.INT8 if dt == "int8" else dsw.BF16)
    pl = walker.query_plan(B)
    gh.say("plan", pl.as_dict())
    temps = "cycle" if (index == 3 and dt == "int8") else None
    tot = {}
    for rnd in range(n_rounds):
        inp = workloads.round_inputs(index, rnd, B=B, temps=temps)
        toks, lg = gh.run(torch, walker, W1d, W2d, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        gh.say("round", rnd, rep)
        _merge(tot, rep)
    assert tot["steps"] == n_rounds * B * wl.gamma
    gh.report({"test": "default_plan", "workload": wl.name, "kernel": _kernel_name(dsw, pl), "B": B, "w2": dt,
               "rounds": n_rounds, "requests_checked": "all", "steps_checked": "all", **tot})
    walker.close()
