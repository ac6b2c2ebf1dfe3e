"""GPU parity of the persistent walk against the CPU oracle, through the C ABI.

Every case prints what it runs before it runs it, so a failure names itself.
"""
import os
import sys

import numpy as np
import pytest

import parity
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dsw():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import serial_draft_head_amd as m
    m.lib()
    return m


DEV = "cuda:0"


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def round_dev(inp):
    return (bf16_dev(inp["base"]), torch.from_numpy(inp["anchor"]).to(DEV),
            torch.from_numpy(inp["T"]).to(DEV), torch.from_numpy(inp["uniforms"]).to(DEV))


def run(walker, W1d, W2d, inp, want_logits=True, scale=None):
    base, anchor, T, uni = round_dev(inp)
    tokens, logits = walker.walk(W1d, W2d, base, anchor, T, uni, w2_scale=scale,
                                 want_logits=want_logits)
    torch.cuda.synchronize()
    st = walker.status()
    assert st == 0, f"device status {st}"
    lg = None if logits is None else logits.view(torch.int16).cpu().numpy().view(np.uint16)
    return tokens.cpu().numpy(), lg


SHAPES = [  # (V, B, gamma, temps)
    (1, 2, 2, "greedy"),
    (12, 1, 3, "greedy"),
    (257, 3, 4, "mixed"),
    (1000, 1, 7, "greedy"),
    (4097, 4, 5, "mixed"),
    (32_000, 1, 7, "greedy"),
    (65_537, 16, 3, "mixed"),
    (100_003, 5, 16, "mixed"),
]


ENGINES = {"mfma": 8, "valu": 4}


@pytest.mark.parametrize("engine", list(ENGINES))
@pytest.mark.parametrize("V,B,gamma,temps", SHAPES)
def test_parity_small_and_ragged(dsw, V, B, gamma, temps, engine):
    say(f"parity V={V} B={B} gamma={gamma} temps={temps} engine={engine}")
    W1, W2 = workloads.weights(0, V=V)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(V, gamma_max=16, B_max=16, flags=ENGINES[engine])
    say("plan", walker.query_plan(B).as_dict())
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for rnd in range(2):
        inp = workloads.round_inputs(2, rnd, B=B, gamma=gamma, V=V, temps=temps)
        toks, lg = run(walker, W1d, W2d, inp)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        say("round", rnd, rep)
    walker.close()


def test_toy_workload_many_rounds(dsw):
    """1,000 rounds back to back on one handle (V = 32,000, gamma = 7, T cycling
    0, 0.6, 1): the parity state alternates with no memset; each chunk of 100
    rounds is launched without a host synchronisation, then every round is
    checked against the oracle."""
    wl = workloads.WORKLOADS[0]
    say("toy workload, 1,000 rounds back to back")
    W1, W2 = workloads.weights(0)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=1)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for chunk in range(10):
        rounds = [workloads.round_inputs(0, 100 * chunk + r, B=1, temps="cycle") for r in range(100)]
        outs = []
        for inp in rounds:
            base, anchor, T, uni = round_dev(inp)
            outs.append(walker.walk(W1d, W2d, base, anchor, T, uni, want_logits=True))
        torch.cuda.synchronize()
        assert walker.status() == 0
        for r, (inp, (t, l)) in enumerate(zip(rounds, outs)):
            lg = l.view(torch.int16).cpu().numpy().view(np.uint16)
            rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"],
                                     t.cpu().numpy(), lg)
        say("rounds", 100 * chunk, "..", 100 * chunk + 99, rep)
    walker.close()


def test_no_state_pollution_between_greedy_and_sampled(dsw):
    V = 32_000
    say("greedy -> sampled -> greedy on one handle")
    W1, W2 = workloads.weights(0, V=V)
    walker = dsw.Walker(V, gamma_max=7, B_max=4)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    g = workloads.round_inputs(0, 5, B=4, gamma=7, V=V, temps="greedy")
    s = workloads.round_inputs(2, 6, B=4, gamma=7, V=V, temps="mixed")
    s["T"][:] = 1.0
    t1, l1 = run(walker, W1d, W2d, g)
    run(walker, W1d, W2d, s)
    t2, l2 = run(walker, W1d, W2d, g)
    assert np.array_equal(t1, t2) and np.array_equal(l1, l2)


def test_logits_optional_and_tokens_identical(dsw):
    V = 40_000
    say("tokens without the logits output")
    W1, W2 = workloads.weights(0, V=V)
    walker = dsw.Walker(V, gamma_max=7, B_max=4)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(2, 9, B=4, gamma=7, V=V, temps="mixed")
    t1, _ = run(walker, W1d, W2d, inp, want_logits=True)
    t2, l2 = run(walker, W1d, W2d, inp, want_logits=False)
    assert l2 is None and np.array_equal(t1, t2)


@pytest.mark.parametrize("engine", list(ENGINES))
def test_force_stream_is_bit_identical_to_resident(dsw, engine):
    V = 60_000
    say(f"streamed plan vs resident plan, engine={engine}")
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    res = dsw.Walker(V, gamma_max=7, B_max=4, flags=ENGINES[engine])
    st = dsw.Walker(V, gamma_max=7, B_max=4, flags=dsw.FLAG_FORCE_STREAM | ENGINES[engine])
    assert st.query_plan(4).stream_rows == st.query_plan(4).rows_per_wg
    inp = workloads.round_inputs(2, 11, B=4, gamma=7, V=V, temps="mixed")
    a = run(res, W1d, W2d, inp)
    b = run(st, W1d, W2d, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("V", [60_000, 151_936, 248_320])
def test_streamed_prefetch_one_request(dsw, V):
    """One request with nothing on chip: the first streamed tiles of every
    wave are loaded into LDS one step ahead, the rest streamed in the step.
    Tokens and logits are the resident walk's, bit for bit, greedy and
    sampled, and the oracle's."""
    say(f"one request, W2 streamed with the cross-step prefetch, V={V}")
    W1, W2 = workloads.weights(1, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    res = dsw.Walker(V, gamma_max=7, B_max=1)
    st = dsw.Walker(V, gamma_max=7, B_max=1, flags=dsw.FLAG_FORCE_STREAM)
    plan = st.query_plan(1)
    say("plan", plan.as_dict())
    assert plan.stream_rows == plan.rows_per_wg and 0 < plan.prefetch_tiles <= plan.tiles_per_wave
    w = parity.Weights(W1, W2)
    for r, temps in enumerate(("greedy", "cycle", "cycle")):
        inp = workloads.round_inputs(1, 60 + r, B=1, gamma=7, V=V, temps=temps)
        a = run(res, W1d, W2d, inp, want_logits=True)
        b = run(st, W1d, W2d, inp, want_logits=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], b[0], b[1])
        say(rep)
    res.close()
    st.close()


def test_outputs_outside_the_request_untouched(dsw):
    V, B, gamma = 9_999, 3, 5
    say("sentinels around tokens and logits")
    W1, W2 = workloads.weights(0, V=V)
    walker = dsw.Walker(V, gamma_max=8, B_max=8)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(2, 2, B=B, gamma=gamma, V=V, temps="mixed")
    base, anchor, T, uni = round_dev(inp)
    n = B * gamma * V
    big_l = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=DEV)
    big_t = torch.full((B * gamma + 64,), -5, dtype=torch.int32, device=DEV)
    lg = big_l[:n].view(B, gamma, V)
    tk = big_t[:B * gamma].view(B, gamma)
    walker.walk(W1d, W2d, base, anchor, T, uni, tokens=tk, logits=lg)
    torch.cuda.synchronize()
    assert walker.status() == 0
    assert torch.all(big_l[n:] == 7.0).item() and torch.all(big_t[B * gamma:] == -5).item()


def test_device_checks_latch_status_and_recover(dsw):
    V = 5_000
    say("anchor out of range and missing uniforms latch a status; the next call is clean")
    W1, W2 = workloads.weights(0, V=V)
    walker = dsw.Walker(V, gamma_max=4, B_max=2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(0, 1, B=2, gamma=4, V=V)
    base, anchor, T, uni = round_dev(inp)
    bad = torch.tensor([3, V + 7], dtype=torch.int32, device=DEV)
    walker.walk(W1d, W2d, base, bad, T, uni)
    assert walker.status() == -21
    Ts = torch.tensor([0.0, 1.0], dtype=torch.float32, device=DEV)
    walker.walk(W1d, W2d, base, anchor, Ts, None)
    assert walker.status() == -22
    toks, lg = run(walker, W1d, W2d, inp)
    parity.check_round(parity.Weights(W1, W2), inp["base"], inp["anchor"], inp["T"],
                       inp["uniforms"], toks, lg)


def test_host_argument_errors(dsw):
    V = 1_000
    walker = dsw.Walker(V, gamma_max=4, B_max=2)
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(0, 1, B=3, gamma=4, V=V)
    base, anchor, T, uni = round_dev(inp)
    with pytest.raises(dsw.DswError) as e:
        walker.walk(W1d, W2d, base, anchor, T, uni)
    assert e.value.code == -2
    with pytest.raises(ValueError):
        walker.walk(W1d, W2d.float(), base, anchor, T, uni)


@pytest.mark.parametrize("engine", list(ENGINES))
@pytest.mark.parametrize("index,B", [(1, 1), (2, 1), (2, 4), (2, 16), (3, 1)])
def test_full_size_workloads(dsw, index, B, engine):
    wl = workloads.WORKLOADS[index]
    say(f"full size {wl.name} B={B} engine={engine}")
    W1, W2 = workloads.weights(index)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=B, flags=ENGINES[engine])
    say("plan", walker.query_plan(B).as_dict())
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for rnd in range(2 if B <= 4 else 1):
        inp = workloads.round_inputs(index, rnd, B=B)
        toks, lg = run(walker, W1d, W2d, inp)
        steps = None if B * wl.gamma <= 32 else [0, wl.gamma - 1]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 steps=steps)
        say("round", rnd, rep)


def test_cooperative_launch_is_bit_identical(dsw):
    V = 50_000
    say("cooperative launch vs the default launch")
    W1, W2 = workloads.weights(0, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    plain = dsw.Walker(V, gamma_max=7, B_max=4)
    coop = dsw.Walker(V, gamma_max=7, B_max=4, flags=dsw.FLAG_COOPERATIVE)
    for rnd in range(3):
        inp = workloads.round_inputs(2, 20 + rnd, B=4, gamma=7, V=V, temps="mixed")
        a = run(plain, W1d, W2d, inp)
        b = run(coop, W1d, W2d, inp)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# One vocabulary size per compiled MFMA shape (register tiles, tiles per wave):
# the planner picks the shape from ceil(ceil(V / 256) / 16 / 4) tiles per wave.
SHAPE_VOCABS = [(32_000, (2, 2)), (60_000, (4, 4)), (129_280, (8, 8)), (151_936, (8, 10)),
                (200_000, (8, 16))]


@pytest.mark.parametrize("B", [3, 13])
@pytest.mark.parametrize("V,shape", SHAPE_VOCABS)
def test_every_mfma_shape(dsw, V, shape, B):
    say(f"mfma shape {shape} V={V} B={B}")
    W1, W2 = workloads.weights(0, V=V)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(V, gamma_max=4, B_max=16, flags=dsw.FLAG_MFMA_GEMV)
    pl = walker.query_plan(B)
    assert (pl.reg_tiles, pl.max_tiles) == shape and pl.batch_tile == (4 if B <= 4 else 16)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for temps in ("greedy", "mixed"):
        inp = workloads.round_inputs(2, 7, B=B, gamma=3, V=V, temps=temps)
        toks, lg = run(walker, W1d, W2d, inp)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        say(temps, rep)


# single rounding (logit = bf16(base + fp32 dot)) on every kernel and engine
SINGLE_CASES = [  # (V, B, gamma, temps, flags, w2 dtype)
    (32_000, 1, 5, "greedy", 0, "bf16"),         # MFMA, one request
    (100_003, 1, 4, "cycle", 4, "bf16"),         # VALU
    (60_000, 3, 4, "mixed", 8, "bf16"),          # MFMA, 4-request tile
    (129_280, 20, 3, "mixed", 0, "bf16"),        # batched
    (60_000, 1, 4, "cycle", 0, "int8"),          # VALU int8
    (60_000, 3, 3, "mixed", 8, "int8"),          # MFMA int8
]


@pytest.mark.parametrize("V,B,gamma,temps,flags,dt", SINGLE_CASES)
def test_single_rounding(dsw, V, B, gamma, temps, flags, dt):
    say(f"single rounding V={V} B={B} gamma={gamma} temps={temps} flags={flags} {dt}")
    W1, W2 = workloads.weights(4, V=V)
    W1d = bf16_dev(W1)
    if dt == "int8":
        Q, sc = workloads.quantize_int8(W2)
        w = parity.Weights(W1, Q=Q, scale=sc)
        W2d, sd = int8_dev(Q, sc)
    else:
        w = parity.Weights(W1, W2)
        W2d, sd = bf16_dev(W2), None
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags | dsw.FLAG_SINGLE_ROUND,
                        w2_dtype=dsw.INT8 if dt == "int8" else dsw.BF16)
    say("plan", walker.query_plan(B).as_dict())
    for rnd in range(3):
        inp = workloads.round_inputs(4, 70 + rnd, B=B, gamma=gamma, V=V, temps=temps)
        toks, lg = run(walker, W1d, W2d, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 single_round=True)
        say(rnd, rep)
    walker.close()


# uniforms drawn on the device (Philox keyed by seed, request, step and the
# handle's round counter), checked against the oracle's own Philox
@pytest.mark.parametrize("V,B,gamma,flags", [(32_000, 1, 6, 0), (60_000, 1, 3, 4), (60_000, 3, 4, 8),
                                             (129_280, 20, 3, 0)])
def test_device_uniforms(dsw, V, B, gamma, flags):
    import oracle
    say(f"device uniforms V={V} B={B} gamma={gamma} flags={flags}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags)
    seed = 0x5EED_0000_0000 + V
    walker.set_seed(seed)
    seen = []
    for rnd in range(3):
        inp = workloads.round_inputs(2, 80 + rnd, B=B, gamma=gamma, V=V, temps="cycle" if B == 1 else "mixed")
        if B == 1:
            inp["T"][:] = 1.0
        ctr = walker.round_counter()
        base, anchor, T, _ = round_dev(inp)
        tokens, logits = walker.walk(W1d, W2d, base, anchor, T, None, want_logits=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        uni = oracle.device_uniforms(seed, ctr, B, gamma)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], uni, toks, lg)
        say(rnd, "round counter", ctr, rep)
        assert walker.round_counter() == ctr + 1
        seen.append(ctr)
    assert len(set(seen)) == 3
    # without a seed, a sampled request with no uniforms is a latched device error
    walker.set_seed(seed, enable=False)
    inp = workloads.round_inputs(2, 90, B=B, gamma=gamma, V=V, temps="cycle")
    inp["T"][:] = 1.0
    base, anchor, T, _ = round_dev(inp)
    walker.walk(W1d, W2d, base, anchor, T, None)
    torch.cuda.synchronize()
    assert walker.status() == -22
    walker.close()


# Gumbel-max sampling (DSW_FLAG_GUMBEL): every kernel family, ragged and full
# sizes; the oracle draws the same Philox noise from (seed, round counter)
GUMBEL_CASES = [  # (V, B, gamma, flags, w2 dtype)
    (32_000, 1, 6, 0, "bf16"),        # one-request MFMA engine
    (60_001, 1, 3, 0, "bf16"),        # short walk: VALU engine, ragged vocabulary
    (4_097, 3, 5, 8, "bf16"),         # MFMA, batch tile 4, ragged
    (151_936, 1, 7, 0, "bf16"),       # the headline shape
    (248_320, 1, 4, 0, "bf16"),       # 12 register + 4 LDS tiles per wave
    (151_936, 16, 3, 8, "bf16"),      # MFMA, batch tile 16
    (60_000, 4, 4, 4, "bf16"),        # VALU, batch tile 4
    (129_280, 1, 4, 0, "int8"),       # int8 rows, VALU
    (60_000, 4, 3, 0, "int8"),        # int8 rows, MFMA
    # the batched kernel: four tiles per epilogue up to 4 requests, ragged
    # and empty shards, LDS and streamed tiles, full groups and many groups
    (4_097, 4, 5, 0, "bf16"),
    (151_936, 2, 3, 16, "bf16"),
    (151_936, 16, 3, 0, "bf16"),
    (60_000, 20, 4, 1, "bf16"),
    (129_280, 64, 3, 0, "bf16"),
    (32_000, 253, 2, 0, "bf16"),
]


@pytest.mark.parametrize("V,B,gamma,flags,dt", GUMBEL_CASES)
def test_gumbel_max(dsw, V, B, gamma, flags, dt):
    say(f"gumbel-max V={V} B={B} gamma={gamma} flags={flags} {dt}")
    W1, W2 = workloads.weights(2, V=V)
    W1d = bf16_dev(W1)
    if dt == "int8":
        Q, sc = workloads.quantize_int8(W2)
        w = parity.Weights(W1, Q=Q, scale=sc)
        W2d, sd = int8_dev(Q, sc)
    else:
        w = parity.Weights(W1, W2)
        W2d, sd = bf16_dev(W2), None
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags | dsw.FLAG_GUMBEL,
                        w2_dtype=dsw.INT8 if dt == "int8" else dsw.BF16)
    say("plan", walker.query_plan(B).as_dict())
    seed = 0x6A6B_0000_0000 + V + B
    walker.set_seed(seed)
    checked = 0
    for rnd in range(2):
        inp = workloads.round_inputs(2, 40 + rnd, B=B, gamma=gamma, V=V, temps="mixed")
        if B == 1:
            inp["T"][:] = (1.0, 0.6)[rnd]
        ctr = walker.round_counter()
        base, anchor, T, uni = round_dev(inp)
        # the uniforms argument is not used by Gumbel-max
        tokens, logits = walker.walk(W1d, W2d, base, anchor, T, uni if rnd else None, w2_scale=sd,
                                     want_logits=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], None, toks, lg,
                                 gumbel=(seed, ctr))
        say(rnd, "round counter", ctr, rep)
        checked += rep["sampled_exact_checked"]
        assert walker.round_counter() == ctr + 1
        # the same round without logits out draws the same noise: same tokens
        walker.set_round_counter(ctr)
        tokens2, _ = walker.walk(W1d, W2d, base, anchor, T, None, w2_scale=sd)
        torch.cuda.synchronize()
        assert walker.status() == 0
        assert np.array_equal(tokens2.cpu().numpy(), toks)
    assert checked > 0
    walker.close()


def test_gumbel_max_needs_a_seed_and_a_small_batch(dsw):
    V = 4_096
    W1, W2 = workloads.weights(2, V=V)
    walker = dsw.Walker(V, gamma_max=3, B_max=2, flags=dsw.FLAG_GUMBEL)
    inp = workloads.round_inputs(2, 1, B=2, gamma=3, V=V, temps="mixed")
    base, anchor, T, _ = round_dev(inp)
    with pytest.raises(dsw.DswError) as e:   # no seed yet
        walker.walk(bf16_dev(W1), bf16_dev(W2), base, anchor, T, None)
    assert e.value.code == -11
    walker.close()
    # beyond 16 requests only the batched kernel serves, and it has Gumbel-max
    # for bf16 rows with double rounding only
    with pytest.raises(dsw.DswError) as e:
        dsw.Walker(V, gamma_max=3, B_max=17, flags=dsw.FLAG_GUMBEL, w2_dtype=dsw.INT8)
    assert e.value.code == -11
    with pytest.raises(dsw.DswError) as e:
        dsw.Walker(V, gamma_max=3, B_max=17, flags=dsw.FLAG_GUMBEL | dsw.FLAG_SINGLE_ROUND)
    assert e.value.code == -11
    dsw.Walker(V, gamma_max=3, B_max=17, flags=dsw.FLAG_GUMBEL).close()


# HIP graph replays: nothing is cleared between replays (epochs come from the
# device round counter) and device-drawn noise is keyed by that counter, so
# each replay must be a correct walk with fresh noise.  Eager copies and
# synchronisations run between the replays.
@pytest.mark.parametrize("B,flags,temps,replays", [(1, 0, "cycle", 100), (3, 64, "mixed", 8), (4, 0, "mixed", 8),
                                                   (20, 0, "mixed", 8)])
def test_graph_replays_are_fresh_walks(dsw, B, flags, temps, replays):
    import oracle
    say(f"graph replays B={B} flags={flags} {temps}")
    V, gamma = 32_000, 4
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags)
    seed = 0xC0FFEE + B
    walker.set_seed(seed)
    inp = workloads.round_inputs(2, 300, B=B, gamma=gamma, V=V, temps=temps)
    base, anchor, T, _ = round_dev(inp)  # the graph's static inputs
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=DEV)
    logits = torch.empty((B, gamma, V), dtype=torch.bfloat16, device=DEV)
    walker.walk(W1d, W2d, base, anchor, T, None, tokens=tokens, logits=logits)  # eager warm-up
    torch.cuda.synchronize()
    assert walker.status() == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        walker.walk(W1d, W2d, base, anchor, T, None, tokens=tokens, logits=logits)
    torch.cuda.synchronize()
    seen = []
    for r in range(replays):
        inp = workloads.round_inputs(2, 301 + r, B=B, gamma=gamma, V=V, temps=temps)
        nb, na, nt, _ = round_dev(inp)
        base.copy_(nb)
        anchor.copy_(na)
        T.copy_(nt)
        torch.cuda.synchronize()
        ctr = walker.round_counter()
        g.replay()
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        if flags & dsw.FLAG_GUMBEL:
            rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], None, toks, lg,
                                     gumbel=(seed, ctr))
        else:
            uni = oracle.device_uniforms(seed, ctr, B, gamma)
            rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], uni, toks, lg)
        if r % 10 == 0:
            say(r, "round counter", ctr, rep)
        assert walker.round_counter() == ctr + 1
        seen.append(ctr)
    assert len(set(seen)) == replays
    del g
    walker.close()


# The GRU serial head: the state after every step against the oracle's cell
# on the GPU's previous state, and the logits / tokens of every step against
# the oracle's step on the GPU's operand bf16(h) (both teacher forced).
GRU_CASES = [  # (V, gamma, temps)
    (4_097, 5, "greedy"), (32_000, 7, "cycle"), (151_936, 16, "greedy"), (151_936, 8, "hot"),
    (248_320, 4, "greedy")]


@pytest.mark.parametrize("V,gamma,temps", GRU_CASES)
def test_gru_head(dsw, V, gamma, temps):
    import oracle
    say(f"gru head V={V} gamma={gamma} {temps}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    cell = workloads.gru_cell_weights(1)
    celld = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
             torch.from_numpy(cell[3]).to(DEV))
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GRU)
    say("plan", walker.query_plan(1).as_dict())
    for rnd in range(2):
        inp = workloads.round_inputs(2, 500 + rnd, B=1, gamma=gamma, V=V,
                                     temps="cycle" if temps == "hot" else temps)
        if temps == "hot":
            inp["T"][:] = 1.0
        h0 = workloads.gru_h0(1, rnd, 1)
        base, anchor, T, uni = round_dev(inp)
        tokens, logits, states = walker.walk_gru(W1d, W2d, celld, torch.from_numpy(h0[0]).to(DEV), base,
                                                 anchor, T, uni, want_logits=True, want_states=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        st = states.cpu().numpy()
        n, worst, ratio = parity.check_gru_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
        ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 latents=ub)
        say(rnd, f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
        # the same walk without the optional outputs gives the same tokens
        t2, _, _ = walker.walk_gru(W1d, W2d, celld, torch.from_numpy(h0[0]).to(DEV), base, anchor, T, uni)
        torch.cuda.synchronize()
        assert walker.status() == 0 and np.array_equal(t2.cpu().numpy(), toks)
    walker.close()


RNN_CASES = [(4_097, 5, "greedy"), (32_000, 7, "cycle"), (151_936, 16, "greedy")]


@pytest.mark.parametrize("V,gamma,temps", RNN_CASES)
def test_rnn_head(dsw, V, gamma, temps):
    import oracle
    say(f"rnn head V={V} gamma={gamma} {temps}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    cell = workloads.rnn_cell_weights(1)
    celld = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
             torch.from_numpy(cell[3]).to(DEV))
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_RNN)
    for rnd in range(2):
        inp = workloads.round_inputs(2, 600 + rnd, B=1, gamma=gamma, V=V, temps=temps)
        h0 = workloads.gru_h0(2, rnd, 1)
        base, anchor, T, uni = round_dev(inp)
        tokens, logits, states = walker.walk_rnn(W1d, W2d, celld, torch.from_numpy(h0[0]).to(DEV), base,
                                                 anchor, T, uni, want_logits=True, want_states=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        st = states.cpu().numpy()
        n, worst, ratio = parity.check_rnn_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
        ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 latents=ub)
        say(rnd, f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
    # a GRU handle refuses the RNN call
    g = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GRU)
    with pytest.raises(dsw.DswError) as e:
        g.walk_rnn(W1d, W2d, celld, torch.zeros(256, device=DEV), base, anchor, T, uni)
    assert e.value.code == -11
    g.close()
    walker.close()


GATED_CASES = [(4_097, 5, "greedy"), (32_000, 7, "cycle"), (151_936, 16, "greedy"), (248_320, 16, "cycle")]


@pytest.mark.parametrize("V,gamma,temps", GATED_CASES)
def test_gated_head(dsw, V, gamma, temps):
    import oracle
    say(f"gated head V={V} gamma={gamma} {temps}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    gate = workloads.gated_weights(1)
    gated = (torch.from_numpy(gate[0]).to(DEV), torch.from_numpy(gate[1]).to(DEV),
             torch.from_numpy(gate[2]).to(DEV))
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GATED)
    say("plan", walker.query_plan(1).as_dict())
    for rnd in range(2):
        inp = workloads.round_inputs(2, 700 + rnd, B=1, gamma=gamma, V=V, temps=temps)
        h0 = workloads.gru_h0(2, rnd, 1)
        base, anchor, T, uni = round_dev(inp)
        tokens, logits, states = walker.walk_gated(W1d, W2d, gated, torch.from_numpy(h0[0]).to(DEV), base,
                                                   anchor, T, uni, want_logits=True, want_states=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        st = states.cpu().numpy()
        n, worst, ratio = parity.check_gated_states(W1, gate, h0[0], toks[0], inp["anchor"][0], st)
        ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 latents=ub)
        say(rnd, f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
    walker.close()


def test_gated_head_closed_gate_is_the_markov_walk(dsw):
    # gate bias -1e4: g = 1 / (1 + inf) = 0 exactly, so h = x = W1[prev] and the
    # operand bf16(h) is the Markov walk's; tokens and logits agree bit for bit
    V, gamma = 32_000, 7
    say(f"gated head, closed gate, V={V} gamma={gamma}")
    W1, W2 = workloads.weights(2, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    Gq, gs, _ = workloads.gated_weights(1)
    gated = (torch.from_numpy(Gq).to(DEV), torch.from_numpy(gs).to(DEV),
             torch.full((256,), -1e4, dtype=torch.float32, device=DEV))
    wg = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GATED)
    wm = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_MFMA_GEMV)
    for rnd in range(3):
        inp = workloads.round_inputs(2, 800 + rnd, B=1, gamma=gamma, V=V, temps="cycle")
        base, anchor, T, uni = round_dev(inp)
        h0 = torch.from_numpy(workloads.gru_h0(2, rnd, 1)[0]).to(DEV)
        tg, lgg, st = wg.walk_gated(W1d, W2d, gated, h0, base, anchor, T, uni, want_logits=True, want_states=True)
        tm, lgm = wm.walk(W1d, W2d, base, anchor, T, uni, want_logits=True)
        torch.cuda.synchronize()
        assert wg.status() == 0 and wm.status() == 0
        assert torch.equal(tg, tm) and torch.equal(lgg.view(torch.int16), lgm.view(torch.int16))
        prevs = [int(inp["anchor"][0])] + tg[0, :-1].cpu().tolist()
        want = torch.from_numpy(oracle_rows_f32(W1, prevs)).to(DEV)
        assert torch.equal(st, want)
    wg.close()
    wm.close()


def oracle_rows_f32(W1_bits, rows):
    """W1 rows as exact f32 values (bf16 bits shifted into the high half)."""
    return (np.asarray(W1_bits[rows], np.uint32) << 16).view(np.float32)


def test_gated_head_argument_errors(dsw):
    V, gamma = 4_096, 3
    W1, W2 = workloads.weights(2, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(2, 1, B=1, gamma=gamma, V=V)
    base, anchor, T, uni = round_dev(inp)
    Gq, gs, gb = workloads.gated_weights(1)
    Gqd, gsd, gbd = torch.from_numpy(Gq).to(DEV), torch.from_numpy(gs).to(DEV), torch.from_numpy(gb).to(DEV)
    h0 = torch.zeros(256, device=DEV)
    g = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GATED)
    # a matrix that is not 16-byte aligned
    buf = torch.zeros(256 * 256 + 16, dtype=torch.int8, device=DEV)
    bad = buf[1:1 + 256 * 256].view(256, 256)
    with pytest.raises(dsw.DswError) as e:
        g.walk_gated(W1d, W2d, (bad, gsd, gbd), h0, base, anchor, T, uni)
    assert e.value.code == -11
    # the Markov, GRU and RNN calls refuse a gated handle; the gated call refuses a GRU handle
    with pytest.raises(dsw.DswError) as e:
        g.walk(W1d, W2d, base, anchor, T, uni)
    assert e.value.code == -11
    r = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_GRU)
    with pytest.raises(dsw.DswError) as e:
        r.walk_gated(W1d, W2d, (Gqd, gsd, gbd), h0, base, anchor, T, uni)
    assert e.value.code == -11
    r.close()
    # the handle still walks after the refused calls
    tokens, _, _ = g.walk_gated(W1d, W2d, (Gqd, gsd, gbd), h0, base, anchor, T, uni)
    torch.cuda.synchronize()
    assert g.status() == 0 and tokens.shape == (1, gamma)
    g.close()


DOMINO_CASES = [(4_097, 5, "greedy", 2560), (32_000, 15, "cycle", 2560), (151_936, 16, "greedy", 4096),
                (151_936, 7, "greedy", 8)]


@pytest.mark.parametrize("V,gamma,temps,d", DOMINO_CASES)
def test_domino_head(dsw, V, gamma, temps, d):
    import oracle
    say(f"domino head V={V} gamma={gamma} {temps} d={d}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    cell = workloads.domino_cell_weights(1, d=d)
    celld = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
             torch.from_numpy(cell[3]).to(DEV))
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_DOMINO)
    for rnd in range(2):
        inp = workloads.round_inputs(2, 900 + rnd, B=1, gamma=gamma, V=V, temps=temps)
        h0 = workloads.gru_h0(2, rnd, 1)
        H = workloads.domino_hidden(2, rnd, 1, gamma, d=d)
        base, anchor, T, uni = round_dev(inp)
        tokens, logits, states = walker.walk_domino(W1d, W2d, celld, bf16_dev(H[0]), torch.from_numpy(h0[0]).to(DEV),
                                                    base, anchor, T, uni, want_logits=True, want_states=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        st = states.cpu().numpy()
        n, worst, ratio = parity.check_gru_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st, hidden=H[0])
        ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 latents=ub)
        say(rnd, f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
    walker.close()


def test_domino_head_argument_errors(dsw):
    V, gamma, d = 4_096, 3, 64
    W1, W2 = workloads.weights(2, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(2, 1, B=1, gamma=gamma, V=V)
    base, anchor, T, uni = round_dev(inp)
    cell = workloads.domino_cell_weights(1, d=d)
    celld = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
             torch.from_numpy(cell[3]).to(DEV))
    H = bf16_dev(workloads.domino_hidden(2, 1, 1, gamma, d=d)[0])
    h0 = torch.zeros(256, device=DEV)
    g = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=dsw.FLAG_DOMINO)
    # hidden width not a multiple of 8, and misaligned hidden states
    c12 = workloads.domino_cell_weights(1, d=12)
    c12d = (bf16_dev(c12[0]), celld[1], celld[2], celld[3])
    with pytest.raises(dsw.DswError) as e:
        g.walk_domino(W1d, W2d, c12d, bf16_dev(workloads.domino_hidden(2, 1, 1, gamma, d=12)[0]), h0, base,
                      anchor, T, uni)
    assert e.value.code == -11
    buf = torch.zeros(gamma * d + 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dsw.DswError) as e:
        g.walk_domino(W1d, W2d, celld, buf[1:1 + gamma * d].view(gamma, d), h0, base, anchor, T, uni)
    assert e.value.code == -11
    # the other heads' calls refuse the handle; more than 16 steps are refused at creation
    with pytest.raises(dsw.DswError) as e:
        g.walk(W1d, W2d, base, anchor, T, uni)
    assert e.value.code == -11
    with pytest.raises(dsw.DswError) as e:
        dsw.Walker(V, gamma_max=17, B_max=1, flags=dsw.FLAG_DOMINO)
    assert e.value.code == -3
    tokens, _, _ = g.walk_domino(W1d, W2d, celld, H, h0, base, anchor, T, uni)
    torch.cuda.synchronize()
    assert g.status() == 0 and tokens.shape == (1, gamma)
    g.close()


@pytest.mark.parametrize("head", ["gru", "rnn", "gated", "domino"])
def test_recurrent_heads_single_rounding_and_device_uniforms(dsw, head):
    # every recurrent head with DSW_FLAG_SINGLE_ROUND and sampled steps whose
    # uniforms the device draws from the seed (T = 1 at every step)
    import oracle
    V, gamma, d = 32_000, 9, 256
    say(f"{head} head, single rounding, device uniforms, V={V} gamma={gamma}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    flag = {"gru": dsw.FLAG_GRU, "rnn": dsw.FLAG_RNN, "gated": dsw.FLAG_GATED, "domino": dsw.FLAG_DOMINO}[head]
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=flag | dsw.FLAG_SINGLE_ROUND)
    seed = 0x5EED_1234 + flag
    walker.set_seed(seed)
    if head in ("gru", "rnn"):
        cell = workloads.gru_cell_weights(3, gates=3 if head == "gru" else 1)
    elif head == "domino":
        cell = workloads.domino_cell_weights(3, d=d)
    else:
        cell = workloads.gated_weights(3)
    if head == "gated":
        dev_cell = tuple(torch.from_numpy(a).to(DEV) for a in cell)
    else:
        dev_cell = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
                    torch.from_numpy(cell[3]).to(DEV))
    for rnd in range(2):
        inp = workloads.round_inputs(2, 950 + rnd, B=1, gamma=gamma, V=V, temps="cycle")
        inp["T"][:] = 1.0
        h0 = workloads.gru_h0(3, rnd, 1)
        h0d = torch.from_numpy(h0[0]).to(DEV)
        base, anchor, T, _ = round_dev(inp)
        ctr = walker.round_counter()
        kw = dict(want_logits=True, want_states=True)
        if head == "gru":
            tokens, logits, states = walker.walk_gru(W1d, W2d, dev_cell, h0d, base, anchor, T, None, **kw)
        elif head == "rnn":
            tokens, logits, states = walker.walk_rnn(W1d, W2d, dev_cell, h0d, base, anchor, T, None, **kw)
        elif head == "gated":
            tokens, logits, states = walker.walk_gated(W1d, W2d, dev_cell, h0d, base, anchor, T, None, **kw)
        else:
            H = workloads.domino_hidden(3, rnd, 1, gamma, d=d)
            tokens, logits, states = walker.walk_domino(W1d, W2d, dev_cell, bf16_dev(H[0]), h0d, base, anchor, T,
                                                        None, **kw)
        torch.cuda.synchronize()
        assert walker.status() == 0 and walker.round_counter() == ctr + 1
        toks = tokens.cpu().numpy()
        lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        st = states.cpu().numpy()
        if head == "gru":
            n, worst, ratio = parity.check_gru_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
        elif head == "rnn":
            n, worst, ratio = parity.check_rnn_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
        elif head == "gated":
            n, worst, ratio = parity.check_gated_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
        else:
            n, worst, ratio = parity.check_gru_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st, hidden=H[0])
        ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
        uni = oracle.device_uniforms(seed, ctr, 1, gamma)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], uni, toks, lg, latents=ub,
                                 single_round=True)
        assert rep["sampled"] == gamma
        say(rnd, f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
    walker.close()


def _random_configs(n, seed=2026):
    """Seeded random walks over the planner's paths: ragged vocabularies, any
    batch, 1..16 steps, bf16 or int8 rows, engine, streaming, rounding and
    sampler flags (combinations the planner refuses are drawn again)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        V = int(rng.integers(1_000, 160_000))
        B = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 40]))
        gamma = int(rng.integers(1, 17))
        gamma = max(1, min(gamma, 3_000_000 // (V * B)))  # the oracle's share stays small
        dt = "int8" if rng.random() < 0.25 else "bf16"
        opts = [0, 8, 4, 8 | 1, 64] if B <= 16 else [0, 16]
        flags = int(rng.choice(opts)) | (32 if rng.random() < 0.3 else 0)
        if dt == "int8" and (flags & 4) and B > 1:
            continue  # int8 rows on the VALU engine: one request
        temps = "greedy" if rng.random() < 0.3 else "mixed"
        out.append((V, B, gamma, dt, flags, temps))
    return out


@pytest.mark.parametrize("V,B,gamma,dt,flags,temps", _random_configs(12))
def test_random_walks(dsw, V, B, gamma, dt, flags, temps):
    import oracle  # noqa: F401  (parity loads it)
    say(f"random walk V={V} B={B} gamma={gamma} {dt} flags={flags} {temps}")
    W1, W2 = workloads.weights(2, V=V)
    W1d = bf16_dev(W1)
    if dt == "int8":
        Q, sc = workloads.quantize_int8(W2)
        w = parity.Weights(W1, Q=Q, scale=sc)
        W2d, sd = int8_dev(Q, sc)
    else:
        w = parity.Weights(W1, W2)
        W2d, sd = bf16_dev(W2), None
    walker = dsw.Walker(V, gamma_max=gamma, B_max=B, flags=flags,
                        w2_dtype=dsw.INT8 if dt == "int8" else dsw.BF16)
    seed = 0xABCD_0000 + V
    if flags & 64:
        walker.set_seed(seed)
    say("plan", walker.query_plan(B).as_dict())
    for rnd in range(2):
        inp = workloads.round_inputs(2, 1000 + rnd, B=B, gamma=gamma, V=V, temps=temps)
        ctr = walker.round_counter()
        toks, lg = run(walker, W1d, W2d, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 single_round=bool(flags & 32), gumbel=(seed, ctr) if flags & 64 else None)
        say(rnd, rep)
    walker.close()


def _random_head_configs(n, seed=2027):
    rng = np.random.default_rng(seed)
    heads = ["gru", "rnn", "gated", "domino"]
    return [(heads[i % 4], int(rng.integers(1_000, 200_000)), int(rng.integers(1, 17)),
             "greedy" if rng.random() < 0.4 else "cycle", bool(rng.random() < 0.4), 8 * int(rng.integers(1, 513)))
            for i in range(n)]


@pytest.mark.parametrize("head,V,gamma,temps,single,d", _random_head_configs(8))
def test_random_recurrent_walks(dsw, head, V, gamma, temps, single, d):
    import oracle
    say(f"random {head} walk V={V} gamma={gamma} {temps} single={single} d={d}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    flag = {"gru": dsw.FLAG_GRU, "rnn": dsw.FLAG_RNN, "gated": dsw.FLAG_GATED, "domino": dsw.FLAG_DOMINO}[head]
    walker = dsw.Walker(V, gamma_max=gamma, B_max=1, flags=flag | (dsw.FLAG_SINGLE_ROUND if single else 0))
    if head == "gated":
        cell = workloads.gated_weights(V % 7)
        dev_cell = tuple(torch.from_numpy(a).to(DEV) for a in cell)
    else:
        cell = (workloads.domino_cell_weights(V % 7, d=d) if head == "domino"
                else workloads.gru_cell_weights(V % 7, gates=3 if head == "gru" else 1))
        dev_cell = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
                    torch.from_numpy(cell[3]).to(DEV))
    inp = workloads.round_inputs(2, 1100 + gamma, B=1, gamma=gamma, V=V, temps=temps)
    h0 = workloads.gru_h0(V % 5, gamma, 1)
    h0d = torch.from_numpy(h0[0]).to(DEV)
    base, anchor, T, uni = round_dev(inp)
    kw = dict(want_logits=True, want_states=True)
    H = None
    if head == "domino":
        H = workloads.domino_hidden(V % 5, gamma, 1, gamma, d=d)
        tokens, logits, states = walker.walk_domino(W1d, W2d, dev_cell, bf16_dev(H[0]), h0d, base, anchor, T, uni,
                                                    **kw)
    else:
        fn = {"gru": walker.walk_gru, "rnn": walker.walk_rnn, "gated": walker.walk_gated}[head]
        tokens, logits, states = fn(W1d, W2d, dev_cell, h0d, base, anchor, T, uni, **kw)
    torch.cuda.synchronize()
    assert walker.status() == 0
    toks = tokens.cpu().numpy()
    lg = logits.view(torch.int16).cpu().numpy().view(np.uint16)
    st = states.cpu().numpy()
    if head == "rnn":
        n, worst, ratio = parity.check_rnn_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
    elif head == "gated":
        n, worst, ratio = parity.check_gated_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st)
    else:
        n, worst, ratio = parity.check_gru_states(W1, cell, h0[0], toks[0], inp["anchor"][0], st,
                                                  hidden=None if H is None else H[0])
    ub = oracle.rne_bf16(st.astype(np.float64))[1][None]
    rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg, latents=ub,
                             single_round=single)
    say(f"states: {n} steps, largest error {worst:.3g} ({ratio:.3f} of its bound)", rep)
    walker.close()


def test_gru_head_argument_errors(dsw):
    V = 4_096
    W1, W2 = workloads.weights(2, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(2, 1, B=1, gamma=3, V=V)
    base, anchor, T, uni = round_dev(inp)
    g = dsw.Walker(V, gamma_max=3, B_max=1, flags=dsw.FLAG_GRU)
    with pytest.raises(dsw.DswError) as e:   # a GRU handle takes dsw_walk_gru only
        g.walk(W1d, W2d, base, anchor, T, uni)
    assert e.value.code == -11
    g.close()
    m = dsw.Walker(V, gamma_max=3, B_max=1)
    cell = workloads.gru_cell_weights(1)
    celld = (bf16_dev(cell[0]), bf16_dev(cell[1]), torch.from_numpy(cell[2]).to(DEV),
             torch.from_numpy(cell[3]).to(DEV))
    with pytest.raises(dsw.DswError) as e:   # and a Markov handle refuses it
        m.walk_gru(W1d, W2d, celld, torch.zeros(256, device=DEV), base, anchor, T, uni)
    assert e.value.code == -11
    m.close()
    with pytest.raises(dsw.DswError) as e:
        dsw.Walker(V, gamma_max=3, B_max=2, flags=dsw.FLAG_GRU)
    assert e.value.code == -11


# int8 rows + fp32 row scales: one vocabulary per compiled int8 shape, plus
# ragged sizes; the harness quantizes once and both sides consume (q, scale).
I8_VOCABS = [(257, (4, 4)), (4097, (4, 4)), (60_000, (4, 4)), (129_280, (8, 8)),
             (248_320, (16, 16))]
I8_ONE_SHAPES = {257: (2, 2), 4097: (2, 2), 60_000: (4, 4), 129_280: (8, 8), 248_320: (12, 16)}


def int8_dev(Q, scale):
    return torch.from_numpy(np.ascontiguousarray(Q)).to(DEV), torch.from_numpy(scale).to(DEV)


@pytest.mark.parametrize("B", [1, 3, 13])
@pytest.mark.parametrize("V,shape", I8_VOCABS)
def test_int8_rows(dsw, V, shape, B):
    say(f"int8 shape {shape} V={V} B={B}")
    W1, W2 = workloads.weights(3, V=V)
    Q, sc = workloads.quantize_int8(W2)
    w = parity.Weights(W1, Q=Q, scale=sc)
    walker = dsw.Walker(V, gamma_max=4, B_max=16, w2_dtype=dsw.INT8, flags=dsw.FLAG_MFMA_GEMV)
    pl = walker.query_plan(B)
    if B == 1:  # one request: rows widened to bf16 on chip, the bf16 one-request shapes
        shape = I8_ONE_SHAPES[V]
    assert (pl.engine, pl.reg_tiles, pl.max_tiles, pl.stream_rows) == (1, *shape, 0)
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    for temps in ("greedy", "mixed"):
        inp = workloads.round_inputs(3, 11, B=B, gamma=3, V=V, temps=temps)
        toks, lg = run(walker, W1d, Qd, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        say(temps, rep)
    walker.close()


# one request: int8 rows widened to bf16 on chip (VALU engine), including the
# vocabulary whose shard overflows registers and LDS (int8 rows streamed)
@pytest.mark.parametrize("V", [257, 4097, 60_000, 129_280, 248_320])
def test_int8_rows_valu(dsw, V):
    say(f"int8 valu V={V}")
    W1, W2 = workloads.weights(3, V=V)
    Q, sc = workloads.quantize_int8(W2)
    w = parity.Weights(W1, Q=Q, scale=sc)
    walker = dsw.Walker(V, gamma_max=4, B_max=1, w2_dtype=dsw.INT8, flags=dsw.FLAG_VALU_GEMV)
    pl = walker.query_plan(1)
    say("plan", pl.as_dict())
    assert pl.engine == 0 and pl.reg_slots <= 2
    assert (pl.stream_rows > 0) == (V == 248_320)
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    for rnd, temps in enumerate(("greedy", "cycle", "cycle", "cycle")):
        inp = workloads.round_inputs(3, 40 + rnd, B=1, gamma=4, V=V, temps=temps)
        toks, lg = run(walker, W1d, Qd, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        say(temps, inp["T"], rep)
    walker.close()


def test_int8_valu_force_stream_is_bit_identical(dsw):
    V = 100_003
    say(f"int8 valu streamed vs resident V={V}")
    W1, W2 = workloads.weights(3, V=V)
    Q, sc = workloads.quantize_int8(W2)
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    res = dsw.Walker(V, gamma_max=5, B_max=1, w2_dtype=dsw.INT8, flags=dsw.FLAG_VALU_GEMV)
    stm = dsw.Walker(V, gamma_max=5, B_max=1, w2_dtype=dsw.INT8,
                     flags=dsw.FLAG_VALU_GEMV | dsw.FLAG_FORCE_STREAM)
    assert stm.query_plan(1).stream_rows == stm.query_plan(1).rows_per_wg
    for rnd in range(3):
        inp = workloads.round_inputs(3, 50 + rnd, B=1, gamma=5, V=V, temps="cycle")
        a = run(res, W1d, Qd, inp, scale=sd)
        b = run(stm, W1d, Qd, inp, scale=sd)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_int8_force_stream_is_bit_identical(dsw):
    V = 100_003
    say(f"int8 streamed vs resident V={V}")
    W1, W2 = workloads.weights(3, V=V)
    Q, sc = workloads.quantize_int8(W2)
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    res = dsw.Walker(V, gamma_max=5, B_max=5, w2_dtype=dsw.INT8)
    stm = dsw.Walker(V, gamma_max=5, B_max=5, w2_dtype=dsw.INT8, flags=dsw.FLAG_FORCE_STREAM)
    assert stm.query_plan(5).stream_rows == stm.query_plan(5).rows_per_wg
    for rnd in range(2):
        inp = workloads.round_inputs(3, 30 + rnd, B=5, gamma=5, V=V, temps="mixed")
        a = run(res, W1d, Qd, inp, scale=sd)
        b = run(stm, W1d, Qd, inp, scale=sd)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("B", [1, 4])
def test_int8_full_size_large_vocab(dsw, B):
    wl = workloads.WORKLOADS[3]
    say(f"int8 full size {wl.name} B={B}")
    W1, W2 = workloads.weights(3)
    Q, sc = workloads.quantize_int8(W2)
    w = parity.Weights(W1, Q=Q, scale=sc)
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=B, w2_dtype=dsw.INT8)
    say("plan", walker.query_plan(B).as_dict())
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    for rnd in range(2):
        inp = workloads.round_inputs(3, rnd, B=B, temps="cycle" if B == 1 else "mixed")
        toks, lg = run(walker, W1d, Qd, inp, scale=sd)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg,
                                 steps=[0, 1, wl.gamma - 1])
        say("round", rnd, rep)
    walker.close()


# ---- the batched kernel (more than 16 requests, or FLAG_BATCHED) -----------

def check_subset(w, inp, toks, lg, idx, steps=None):
    """Parity of the requests `idx` only (requests are independent)."""
    sub = lambda a: np.ascontiguousarray(a[idx])  # noqa: E731
    return parity.check_round(w, sub(inp["base"]), sub(inp["anchor"]), sub(inp["T"]),
                              sub(inp["uniforms"]), sub(toks), sub(lg), steps=steps)


# aligned (V % 8 == 0: base rows stream straight into LDS) and unaligned vocabularies
# V = 151,936 keeps two tiles per wave in LDS beside the ring
BATCHED_CASES = [(257, 17), (4_096, 40), (32_000, 64), (65_537, 33), (129_280, 24), (140_000, 19),
                 (151_936, 20), (190_000, 18)]
# plans with LDS tiles (9 tiles per wave: 8 register tiles and one in LDS; 12:
# 10 register tiles and two in LDS) and with ten register tiles
LDS_TILE_VOCABS = (140_000, 190_000)
TEN_TILE_VOCABS = (151_936, 190_000)


@pytest.mark.parametrize("temps", ["greedy", "mixed"])
@pytest.mark.parametrize("V,B", BATCHED_CASES)
def test_batched_parity(dsw, V, B, temps):
    say(f"batched V={V} B={B} {temps}")
    W1, W2 = workloads.weights(4, V=V)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(V, gamma_max=4, B_max=B)
    pl = walker.query_plan(B)
    say("plan", pl.as_dict())
    assert pl.batch_tile == 256
    assert (pl.lds_tiles > 0) == (V in LDS_TILE_VOCABS)
    assert (pl.reg_tiles == 10) == (V in TEN_TILE_VOCABS)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(4, 3, B=B, gamma=3, V=V, temps=temps)
    toks, lg = run(walker, W1d, W2d, inp)
    idx = np.unique(np.r_[0, B - 1, np.arange(0, B, 5)])
    rep = check_subset(w, inp, toks, lg, idx)
    say(rep)
    walker.close()


@pytest.mark.parametrize("B", [3, 16])
def test_batched_kernel_at_small_batches(dsw, B):
    V = 100_000
    say(f"batched kernel forced at B={B}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(V, gamma_max=5, B_max=B, flags=dsw.FLAG_BATCHED)
    assert walker.query_plan(B).batch_tile == 256
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for rnd in range(2):
        inp = workloads.round_inputs(2, 40 + rnd, B=B, gamma=5, V=V, temps="mixed")
        toks, lg = run(walker, W1d, W2d, inp)
        say(parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg))
    walker.close()


# Up to 4 requests on the batched kernel: four tiles share one epilogue.
# Vocabularies with dead register tiles (V = 4,099: shards of 17 rows; V =
# 100,003: 7 tiles per wave on the 8-tile shape), ten register tiles (V =
# 151,936: the last group of four holds two), ten register tiles and two LDS
# tiles in that group (V = 190,000), streamed tiles (FORCE_STREAM), an
# unaligned vocabulary, logits out or not.
@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("V,stream", [(4_099, False), (100_003, False), (151_936, False), (190_000, False),
                                      (60_000, True)])
def test_batched_four_tile_epilogue(dsw, V, stream, B):
    say(f"batched four-tile epilogue V={V} B={B} stream={stream}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    flags = dsw.FLAG_BATCHED | (dsw.FLAG_FORCE_STREAM if stream else 0)
    walker = dsw.Walker(V, gamma_max=5, B_max=B, flags=flags)
    pl = walker.query_plan(B)
    say("plan", pl.as_dict())
    assert pl.batch_tile == 256
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    for rnd in range(2):
        inp = workloads.round_inputs(2, 80 + rnd, B=B, gamma=5, V=V, temps="mixed")
        toks, lg = run(walker, W1d, W2d, inp)
        say(parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg))
        toks2, _ = run(walker, W1d, W2d, inp, want_logits=False)
        assert np.array_equal(toks, toks2)
    walker.close()


def test_batched_stream_logits_and_state(dsw):
    V, B = 40_000, 37
    say(f"batched streamed vs resident, logits optional, V={V} B={B}")
    W1, W2 = workloads.weights(4, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    res = dsw.Walker(V, gamma_max=4, B_max=B)
    stm = dsw.Walker(V, gamma_max=4, B_max=B, flags=dsw.FLAG_FORCE_STREAM)
    assert stm.query_plan(B).stream_rows == stm.query_plan(B).rows_per_wg
    for rnd in range(3):
        inp = workloads.round_inputs(4, 50 + rnd, B=B, gamma=4, V=V, temps="mixed")
        a = run(res, W1d, W2d, inp)
        b = run(stm, W1d, W2d, inp)
        c = run(res, W1d, W2d, inp, want_logits=False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.array_equal(a[0], c[0])


def test_batched_device_checks(dsw):
    V, B = 20_000, 20
    say("batched device status latch")
    W1, W2 = workloads.weights(4, V=V)
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    walker = dsw.Walker(V, gamma_max=3, B_max=B)
    inp = workloads.round_inputs(4, 60, B=B, gamma=3, V=V, temps="mixed")
    base, anchor, T, uni = round_dev(inp)
    bad = anchor.clone()
    bad[5] = V + 3
    walker.walk(W1d, W2d, base, bad, T, uni)
    assert walker.status() == -21
    walker.walk(W1d, W2d, base, anchor, torch.ones_like(T), None)
    assert walker.status() == -22
    toks, lg = run(walker, W1d, W2d, inp)   # the next call is clean
    parity.check_round(parity.Weights(W1, W2), inp["base"], inp["anchor"], inp["T"], inp["uniforms"],
                       toks, lg)


def test_batched_int8(dsw):
    V, B = 129_280, 40
    say(f"batched int8 V={V} B={B}")
    W1, W2 = workloads.weights(4, V=V)
    Q, sc = workloads.quantize_int8(W2)
    w = parity.Weights(W1, Q=Q, scale=sc)
    walker = dsw.Walker(V, gamma_max=3, B_max=B, w2_dtype=dsw.INT8)
    assert walker.query_plan(B).batch_tile == 256
    W1d = bf16_dev(W1)
    Qd, sd = int8_dev(Q, sc)
    inp = workloads.round_inputs(4, 70, B=B, gamma=3, V=V, temps="mixed")
    toks, lg = run(walker, W1d, Qd, inp, scale=sd)
    say(check_subset(w, inp, toks, lg, np.unique(np.r_[0, B - 1, np.arange(0, B, 4)])))
    walker.close()


@pytest.mark.parametrize("B", [64, 128, 253])
def test_batched_full_size(dsw, B):
    wl = workloads.WORKLOADS[4]
    say(f"batched full size {wl.name} B={B}")
    W1, W2 = workloads.weights(4)
    w = parity.Weights(W1, W2)
    walker = dsw.Walker(wl.V, gamma_max=wl.gamma, B_max=B)
    say("plan", walker.query_plan(B).as_dict())
    W1d, W2d = bf16_dev(W1), bf16_dev(W2)
    inp = workloads.round_inputs(4, 0, B=B)
    toks, lg = run(walker, W1d, W2d, inp)
    rng = np.random.default_rng(B)
    idx = np.unique(np.r_[0, B - 1, rng.choice(B, size=10, replace=False)])
    say(check_subset(w, inp, toks, lg, idx, steps=[0, wl.gamma - 1]))
    walker.close()
