"""The cross-workgroup exchange under stress, on every kernel family:

* step epochs across the 32-bit wrap of the step sequence number and of the
  launch counter (the counters set just below the wrap with the test hook);
* bounded waits: with a spin limit of one poll the waits give up, the device
  latches DSW_ERR_DEV_TIMEOUT, every workgroup exits, a walk launched while
  the error is latched leaves its outputs untouched, and after dsw_status the
  next walk is correct again;
* scrambled arrival order: every workgroup sleeps a pseudo-random time
  before it posts, and the walk must give the same bits as without;
* fewer workgroups than CUs (larger shards, fewer in each rendezvous);
* the Gumbel-max variate the kernels compute, against binary64 for every
  uniform their noise can take (the basis of the Gumbel-max tolerance).

The pages' resident walk posts every CTA's key and polls until every CTA has
arrived, with a round parity instead of a memset ("Keeping the Draft Walk on
Chip", section "The idea: make the walk resident").
"""
import numpy as np
import pytest

import gpu_helpers as gh
import parity
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

V = 65_537


@pytest.fixture(scope="module")
def dsw():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import serial_draft_head_amd as m
    m.lib()
    return m


# (name, requests, flags, gamma_max): one-request MFMA, VALU, the all-to-all
# MFMA kernel with a 4-request tile, the batched kernel with more requests
# than one MFMA column block and with fewer, and the GRU head (whose state
# gather is one more exchange per step)
FAMILIES = [("mfma_b1", 1, 0, 16), ("valu_b1", 1, 4, 7), ("mfma_b4", 3, 8, 7), ("batched", 20, 0, 16),
            ("batched_small", 12, 16, 16), ("gru", 1, 128, 5)]


def _setup(dsw, B, flags, gamma_max):
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker = dsw.Walker(V, gamma_max=gamma_max, B_max=B, flags=flags)
    gh.say("plan", walker.query_plan(B).as_dict())
    return w, W1, W1d, W2d, walker


def _gru_args(dsw):
    cell = workloads.gru_cell_weights(1)
    celld = (gh.bf16_dev(torch, cell[0]), gh.bf16_dev(torch, cell[1]), torch.from_numpy(cell[2]).to(gh.DEV),
             torch.from_numpy(cell[3]).to(gh.DEV))
    h0 = workloads.gru_h0(1, 0, 1)[0]
    return cell, celld, h0


def _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp, tokens=None):
    """One walk and its parity check; returns (tokens, logits)."""
    base, anchor, T, uni = gh.round_dev(torch, inp)
    if name == "gru":
        cell, celld, h0 = _gru_args(dsw)
        t, l, st = walker.walk_gru(W1d, W2d, celld, torch.from_numpy(h0).to(gh.DEV), base, anchor, T, uni,
                                   want_logits=True, want_states=True)
        torch.cuda.synchronize()
        assert walker.status() == 0
        toks, lg, sts = t.cpu().numpy(), gh.logits_host(torch, l), st.cpu().numpy()
        parity.check_gru_states(W1, cell, h0, toks[0], inp["anchor"][0], sts)
        import oracle
        ub = oracle.rne_bf16(sts.astype(np.float64))[1][None]
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg, latents=ub)
    else:
        toks, lg = gh.run(torch, walker, W1d, W2d, inp)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
    gh.say(rep)
    return toks, lg


@pytest.mark.parametrize("name,B,flags,gamma_max", FAMILIES)
@pytest.mark.parametrize("start", ["seq_wrap", "counter_wrap"])
def test_epochs_across_the_wrap(dsw, name, B, flags, gamma_max, start):
    # seq_wrap: the launch counter n just below 2^32 / gamma_max, so that
    # n * gamma_max + k wraps within the three launches; counter_wrap: n itself
    # wraps from 2^32 - 1 to 0
    n0 = (2 ** 32) // gamma_max - 1 if start == "seq_wrap" else 2 ** 32 - 2
    gh.say(f"{name} B={B} gamma_max={gamma_max}: counters from {n0}")
    w, W1, W1d, W2d, walker = _setup(dsw, B, flags, gamma_max)
    gamma = gamma_max
    _walk_and_check(dsw, name, walker, w, W1, W1d, W2d,
                    workloads.round_inputs(2, 5000, B=B, gamma=gamma, V=V, temps="mixed"))
    walker.set_round_counter(n0)
    for r in range(3):
        assert walker.round_counter() == (n0 + r) % 2 ** 32
        gh.say("round", r, "seq", ((n0 + r) % 2 ** 32) * gamma_max % 2 ** 32)
        inp = workloads.round_inputs(2, 5001 + r, B=B, gamma=gamma, V=V, temps="mixed" if r else "greedy")
        _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)
    assert walker.round_counter() == (n0 + 3) % 2 ** 32
    walker.close()


@pytest.mark.parametrize("name,B,flags,gamma_max", FAMILIES)
def test_bounded_waits_give_up(dsw, name, B, flags, gamma_max):
    gh.say(f"{name} B={B}: spin limit 1")
    w, W1, W1d, W2d, walker = _setup(dsw, B, flags, gamma_max)
    gamma = min(gamma_max, 5)
    inp = workloads.round_inputs(2, 5100, B=B, gamma=gamma, V=V, temps="mixed")
    _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)   # a clean walk first
    ctr0 = walker.round_counter()
    base, anchor, T, uni = gh.round_dev(torch, inp)
    gru = _gru_args(dsw) if name == "gru" else None

    def launch(tokens):
        if gru is not None:
            walker.walk_gru(W1d, W2d, gru[1], torch.from_numpy(gru[2]).to(gh.DEV), base, anchor, T, uni,
                            tokens=tokens)
        else:
            walker.walk(W1d, W2d, base, anchor, T, uni, tokens=tokens)

    walker.set_debug(spin_limit=1)
    launch(torch.empty((B, gamma), dtype=torch.int32, device=gh.DEV))
    # launched while that error is latched: returns at once, outputs untouched
    walker.set_debug(spin_limit=0)
    sentinel = torch.full((B, gamma), -7, dtype=torch.int32, device=gh.DEV)
    launch(sentinel)
    torch.cuda.synchronize()
    ctr1 = walker.round_counter()
    st = walker.status()
    gh.say("status", st, "round counter", ctr0, "->", ctr1)
    assert st == -20, f"want DSW_ERR_DEV_TIMEOUT, got {st}"
    assert torch.all(sentinel == -7).item(), "a walk ran while a device error was latched"
    # the counter advances only if workgroup 0 finished every step of the failed walk
    assert ctr1 in (ctr0, ctr0 + 1)
    assert walker.round_counter() == 0   # dsw_status re-zeroed the workspace
    _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)
    walker.close()


@pytest.mark.parametrize("name,B,flags,gamma_max", FAMILIES)
def test_scrambled_arrival_order_gives_the_same_bits(dsw, name, B, flags, gamma_max):
    gh.say(f"{name} B={B}: skewed posts")
    w, W1, W1d, W2d, walker = _setup(dsw, B, flags, gamma_max)
    gamma = min(gamma_max, 6)
    for r in range(2):
        inp = workloads.round_inputs(2, 5200 + r, B=B, gamma=gamma, V=V, temps="mixed")
        walker.set_debug(skew=0)
        t0, l0 = _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)
        walker.set_debug(skew=1)
        t1, l1 = _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)
        assert np.array_equal(t0, t1) and np.array_equal(l0, l1)
    walker.close()


@pytest.mark.parametrize("name,B,flags,gamma_max", [f for f in FAMILIES if f[0] != "gru"])
@pytest.mark.parametrize("grid", [8, 37, 255])
def test_fewer_workgroups(dsw, name, B, flags, gamma_max, grid):
    """dsw_set_grid: the walk over fewer workgroups than CUs, so that each
    owns a larger shard (V = 6,007: 751 rows each over 8) and fewer take
    part in every rendezvous, against the oracle."""
    Vg = 6_007
    gh.say(f"{name} B={B}: grid {grid}")
    W1, W2 = workloads.weights(2, V=Vg)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker = dsw.Walker(Vg, gamma_max=gamma_max, B_max=B, flags=flags)
    walker.set_grid(grid)
    plan = walker.query_plan(B).as_dict()
    gh.say("plan", plan)
    assert plan["grid"] == grid
    for r in range(2):
        inp = workloads.round_inputs(2, 5300 + r, B=B, gamma=min(gamma_max, 7), V=Vg, temps="mixed")
        _walk_and_check(dsw, name, walker, w, W1, W1d, W2d, inp)
    walker.close()


def test_gumbel_variate_error(dsw):
    """The kernels' G = -ln(-ln U) for every U = (2 i + 1) 2^-24, i < 2^23,
    against binary64: within 2e-6 (the bound the Gumbel-max tolerance of
    tests/parity.py counts on)."""
    out = torch.empty(1 << 23, dtype=torch.float32, device=gh.DEV)
    dsw.debug_gumbel_table(out)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    U = (2.0 * np.arange(1 << 23, dtype=np.float64) + 1.0) * 2.0 ** -24
    ref = -np.log(-np.log(U))
    err = np.abs(g - ref)
    i = int(np.argmax(err))
    gh.say(f"largest |G - G64| {err[i]:.3g} at U = {U[i]!r} (G = {ref[i]:.6f})")
    assert np.all(np.isfinite(g))
    assert err.max() <= 2e-6
