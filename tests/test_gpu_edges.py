"""Constructed edge cases on every kernel family, against the oracle and
against closed forms:

* a zero vocabulary table (W2 = 0): every logit equals its base logit bit for
  bit, so a greedy token is the first argmax of the base row (a special case
  that reduces to numpy.argmax);
* equal maxima planted in rows owned by different workgroups -- the last row
  of one shard and the first of the next, rows of three shards, the last row
  V - 1 -- where the smallest id must win ("Keeping the Draft Walk on Chip",
  section "The idea: make the walk resident": ties go to the smallest id);
* -0 and +0 base logits tied at the maximum (compared as numbers: -0 = +0);
* sampled steps at the ends of the uniform's range, u = 0 and u = 1 - 2^-24,
  where the inverse CDF meets its first row and its last-positive-weight
  fallback (vLLM PR #64442, "Details"), and a tiny temperature (T = 1e-3)
  under which most shards carry no mass in fp32.
"""
import numpy as np
import pytest

import gpu_helpers as gh
import parity
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

V = 100_003      # ragged: the last shard is short
GAMMA = 5


@pytest.fixture(scope="module")
def dsw():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import serial_draft_head_amd as m
    m.lib()
    return m


# (name, requests, flags): the one-request MFMA and VALU engines, the MFMA
# all-to-all kernel with 4- and 16-request tiles (forced: by default 2 and
# more requests take the batched kernel), and the batched kernel
FAMILIES = [("mfma_b1", 1, 0), ("valu_b1", 1, 4), ("mfma_b4", 3, 8), ("mfma_b16", 8, 8), ("batched_b3", 3, 0),
            ("batched_b20", 20, 0)]


def _walker(dsw, B, flags):
    w = dsw.Walker(V, gamma_max=GAMMA, B_max=B, flags=flags)
    pl = w.query_plan(B)
    gh.say("plan", pl.as_dict())
    return w, pl


def _noise_base(rng, B, lo=-7.9, hi=7.9):
    return np.clip(2.0 * rng.standard_normal((B, GAMMA, V)), lo, hi).astype(np.float32)


@pytest.mark.parametrize("name,B,flags", FAMILIES)
def test_zero_table_logits_are_the_base(dsw, name, B, flags):
    gh.say(f"zero W2, {name} B={B}")
    W1, _ = workloads.weights(0, V=V)
    W2 = np.zeros((V, 256), np.uint16)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker, _ = _walker(dsw, B, flags)
    for rnd in range(3):
        inp = workloads.round_inputs(2, 4000 + rnd, B=B, gamma=GAMMA, V=V, temps="mixed")
        toks, lg = gh.run(torch, walker, W1d, W2d, inp)
        assert np.array_equal(lg, inp["base"]), "logits differ from the base logits with W2 = 0"
        for b in range(B):
            if inp["T"][b] == 0:
                base_f = (inp["base"][b].astype(np.uint32) << 16).view(np.float32)
                assert np.array_equal(toks[b], np.argmax(base_f, axis=1)), f"request {b}"
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        gh.say(rnd, rep)
    walker.close()


def _planted_sets(R, grid, b):
    """Rows tied at the maximum for each step of request b, across shards."""
    last = (V - 1) // R                     # the shard holding row V - 1
    c = 1 + (37 * b) % (last - 1)           # a shard boundary inside the vocabulary
    sets = [
        [R * c - 1, R * c],                 # last row of shard c - 1, first row of shard c
        [V - 1],                            # the very last row alone
        [V - 1, R * (last - 1) + R // 2, 0],  # three shards, the first row wins
        [R * 5 + 7, R * 9, V - 2],          # three shards
        sorted({R * last, V - 1}),          # first and last row of the short last shard
    ]
    return sets


@pytest.mark.parametrize("name,B,flags", FAMILIES)
def test_planted_ties_across_workgroups(dsw, name, B, flags):
    gh.say(f"planted ties, {name} B={B}")
    W1, _ = workloads.weights(0, V=V)
    W2 = np.zeros((V, 256), np.uint16)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker, pl = _walker(dsw, B, flags)
    R, grid = pl.rows_per_wg, pl.grid
    rng = np.random.default_rng(11 + B)
    base = _noise_base(rng, B)
    want = np.zeros((B, GAMMA), np.int32)
    for b in range(B):
        for k, rows in enumerate(_planted_sets(R, grid, b)):
            base[b, k, rows] = 16.0
            want[b, k] = min(rows)
    inp = {"base": workloads.to_bf16_bits(base), "anchor": rng.integers(0, V, B).astype(np.int32),
           "T": np.zeros(B, np.float32), "uniforms": rng.random((B, GAMMA), dtype=np.float32)}
    toks, lg = gh.run(torch, walker, W1d, W2d, inp)
    assert np.array_equal(toks, want), f"tokens {toks} want {want}"
    rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
    gh.say(rep)
    walker.close()


@pytest.mark.parametrize("name,B,flags", FAMILIES)
def test_signed_zeros_tied_at_the_maximum(dsw, name, B, flags):
    gh.say(f"-0 and +0 at the maximum, {name} B={B}")
    W1, _ = workloads.weights(0, V=V)
    W2 = np.zeros((V, 256), np.uint16)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker, pl = _walker(dsw, B, flags)
    R = pl.rows_per_wg
    rng = np.random.default_rng(5 + B)
    bits = workloads.to_bf16_bits(-(np.abs(2.0 * rng.standard_normal((B, GAMMA, V))) + 1.0))
    want = np.zeros((B, GAMMA), np.int32)
    for b in range(B):
        for k in range(GAMMA):
            i, j = R * (1 + (b + k) % 50) + 3, R * (60 + k) + 1   # different workgroups, i < j
            bits[b, k, i] = 0x8000   # -0
            bits[b, k, j] = 0x0000   # +0
            want[b, k] = i
    inp = {"base": bits, "anchor": rng.integers(0, V, B).astype(np.int32), "T": np.zeros(B, np.float32),
           "uniforms": rng.random((B, GAMMA), dtype=np.float32)}
    toks, lg = gh.run(torch, walker, W1d, W2d, inp)
    assert np.array_equal(toks, want), f"tokens {toks} want {want}"
    rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
    gh.say(rep)
    walker.close()


U_EDGES = np.array([0.0, 1.0 - 2.0 ** -24, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -23], np.float32)


@pytest.mark.parametrize("temp", [1.0, 1e-3])
@pytest.mark.parametrize("name,B,flags", FAMILIES)
def test_sampler_edges(dsw, name, B, flags, temp):
    gh.say(f"sampler edges T={temp}, {name} B={B}")
    W1, W2 = workloads.weights(2, V=V)
    w = parity.Weights(W1, W2)
    W1d, W2d = gh.bf16_dev(torch, W1), gh.bf16_dev(torch, W2)
    walker, _ = _walker(dsw, B, flags)
    for rnd in range(2):
        inp = workloads.round_inputs(2, 4100 + rnd, B=B, gamma=GAMMA, V=V, temps="mixed")
        inp["T"][:] = temp
        inp["uniforms"] = np.stack([np.roll(U_EDGES, b + rnd) for b in range(B)]).astype(np.float32)
        toks, lg = gh.run(torch, walker, W1d, W2d, inp)
        rep = parity.check_round(w, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], toks, lg)
        gh.say(rnd, rep)
        assert rep["sampled"] == B * GAMMA
    walker.close()
