"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-worked
fixtures, exact rational brute force, a bit-pattern search for rounding,
library routines (numpy argmax, torch's float32->bf16 cast, numpy matmul) on
special cases, and closed-form sampler probabilities.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import brute_force as bf
import workloads
from exact_bf16 import rne_bits, value

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32_to_bf16_bits_torch(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_of(values):
    """Exact bf16 values (python floats) -> bit patterns, via the exact search."""
    return np.array([rne_bits(Fraction(v)) for v in values], dtype=np.uint16)


# --------------------------------------------------------------------------- RNE
class TestRounding:
    def test_random_against_exact_search(self, oracle_mod):
        rng = np.random.default_rng(1)
        x = np.concatenate([
            rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
            rng.standard_normal(1000),
        ])
        _, bits = oracle_mod.rne_bf16(x)
        for xi, bi in zip(x, bits):
            assert int(bi) == rne_bits(Fraction(float(xi))), xi

    def test_every_halfway_point_in_several_binades(self, oracle_mod):
        mids, want = [], []
        for hi in (0x3F, 0x40, 0x41, 0x00, 0x80 | 0x3F, 0x7F):
            for lo in range(0, 0x100):
                p = (hi << 8) | lo
                if (p & 0x7F80) == 0x7F80:
                    continue
                q = p + 1
                if (q & 0x7F80) == 0x7F80:
                    continue
                m = (value(p) + value(q)) / 2
                mids.append(float(m))          # exact in binary64
                want.append(rne_bits(m))
        _, bits = oracle_mod.rne_bf16(np.array(mids))
        assert [int(b) for b in bits] == want
        # the tie goes to the even pattern in every case
        assert all(w % 2 == 0 for w in want)

    def test_matches_torch_cast_where_f64_equals_f32(self, oracle_mod):
        rng = np.random.default_rng(2)
        x32 = (rng.standard_normal(200_000) * 3).astype(np.float32)
        x32 = np.concatenate([x32, x32 * np.float32(1e-30), x32 * np.float32(1e30)])
        _, bits = oracle_mod.rne_bf16(x32.astype(np.float64))
        assert np.array_equal(bits, f32_to_bf16_bits_torch(x32))

    def test_edges(self, oracle_mod):
        cases = [
            (0.0, 0x0000), (-0.0, 0x8000),
            (2.0 ** -133, 0x0001),                    # smallest subnormal
            (3 * 2.0 ** -134, 0x0002),                # tie between 1 and 2 ulps -> even (2)
            (2.0 ** -134, 0x0000),                    # tie between 0 and 1 ulp -> even (0)
            (-(2.0 ** -135), 0x8000),                 # tiny negative rounds to -0
            (float(value(0x7F7F)), 0x7F7F),           # largest finite
            (2.0 ** 128 - 2.0 ** 119, 0x7F80),        # tie between max (2^128 - 2^120) and 2^128 -> inf
            (2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100, 0x7F7F),
            (-(2.0 ** 129), 0xFF80),
        ]
        xs = np.array([c[0] for c in cases])
        _, bits = oracle_mod.rne_bf16(xs)
        for (x, want), b in zip(cases, bits):
            assert int(b) == want, (x, hex(int(b)))


# ------------------------------------------------------------------ hand fixtures
def test_hand_worked_walk(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_walk_v4_r2.json")) as f:
        g = json.load(f)
    W1 = bits_of(np.ravel(g["W1"])).reshape(g["V"], g["r"])
    W2 = bits_of(np.ravel(g["W2"])).reshape(g["V"], g["r"])
    base = bits_of(np.ravel(g["base"])).reshape(1, g["gamma"], g["V"])
    toks, logits = oracle_mod.walk(W1, base, [g["anchor"]], [g["T"]], W2_bits=W2)
    assert toks[0].tolist() == g["expected_tokens"]
    want = [[int(x, 16) for x in row] for row in g["expected_logits_bits"]]
    assert logits[0].tolist() == want


def test_hand_worked_walk_single_rounding(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_walk_v4_r2_single.json")) as f:
        g = json.load(f)
    W1 = bits_of(np.ravel(g["W1"])).reshape(g["V"], g["r"])
    W2 = bits_of(np.ravel(g["W2"])).reshape(g["V"], g["r"])
    base = bits_of(np.ravel(g["base"])).reshape(1, g["gamma"], g["V"])
    toks, logits = oracle_mod.walk(W1, base, [g["anchor"]], [g["T"]], W2_bits=W2, single_round=True)
    assert toks[0].tolist() == g["expected_tokens"]
    want = [[int(x, 16) for x in row] for row in g["expected_logits_bits"]]
    assert logits[0].tolist() == want


def test_philox_known_answers(oracle_mod):
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        g = json.load(f)
    for v in g["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        assert [int(x) for x in oracle_mod.philox4x32_10(ctr, key)] == [int(x, 16) for x in v["out"]]


def test_device_uniforms_follow_their_definition(oracle_mod):
    # u(b, k) = top 24 bits of word 0 of Philox(counter (k, b, round, tag), key = seed) / 2^24
    seed, rnd, B, gamma = 0x0123456789ABCDEF, 77, 5, 9
    u = oracle_mod.device_uniforms(seed, rnd, B, gamma)
    for b in range(B):
        for k in range(gamma):
            w = int(oracle_mod.philox4x32_10([k, b, rnd, 0x44535721], [seed & 0xFFFFFFFF, seed >> 32])[0])
            assert u[b, k] == np.float32((w >> 8) / 2.0 ** 24)
    big = oracle_mod.device_uniforms(7, 3, 256, 64).ravel()
    assert big.min() >= 0.0 and big.max() < 1.0
    # 16 equal bins over 16,384 draws: each within 5 sigma of 1,024
    counts = np.bincount((big * 16).astype(int), minlength=16)
    assert np.all(np.abs(counts - 1024) < 5 * math.sqrt(1024 * 15 / 16))
    # a new round or seed gives new uniforms
    assert not np.array_equal(oracle_mod.device_uniforms(7, 4, 256, 64).ravel(), big)
    assert not np.array_equal(oracle_mod.device_uniforms(8, 3, 256, 64).ravel(), big)


def test_hand_worked_gumbel(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_gumbel.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert oracle_mod.gumbel_from_uniforms(c["logits"], c["T"], c["U"]) == c["token"], c


def test_gumbel_uniforms_follow_their_definition(oracle_mod):
    # U(b, k, v) = (2 (w >> 9) + 1) / 2^24, w = word v % 4 of
    # Philox(counter (v / 4, 256 k + b, round, tag), key = seed)
    seed, rnd = 0xFEDCBA9876543210, 1234
    rng = np.random.default_rng(5)
    for _ in range(300):
        b, k, v = int(rng.integers(0, 256)), int(rng.integers(0, 64)), int(rng.integers(0, 1 << 20))
        w = oracle_mod.philox4x32_10([v >> 2, (k << 8) | b, rnd, 0x47554D42],
                                     [seed & 0xFFFFFFFF, seed >> 32])
        want = bf.gumbel_uniform(w, v)
        got = oracle_mod.gumbel_uniform(seed, rnd, b, k, v)
        assert Fraction(got) == want
        assert 0.0 < got < 1.0
        assert float(np.float32(got)) == got  # exact in binary32
    # neighbouring rows, requests, steps and rounds draw different noise
    u0 = oracle_mod.gumbel_uniform(seed, rnd, 3, 2, 100)
    for args in ((seed, rnd, 3, 2, 101), (seed, rnd, 4, 2, 100), (seed, rnd, 3, 3, 100),
                 (seed, rnd + 1, 3, 2, 100), (seed + 1, rnd, 3, 2, 100)):
        assert oracle_mod.gumbel_uniform(*args) != u0


def test_gumbel_max_draws_follow_softmax(oracle_mod):
    # the argmax of logit / T + G is a draw from softmax(logit / T): frequencies
    # over 40,000 rounds of noise within 5 sigma of the softmax probabilities
    logits = [0.0, 1.0, -0.5, 2.0, 0.25]
    lb = bits_of(logits)
    for T in (0.7, 1.6):
        N = 40000
        counts = np.zeros(len(logits))
        for rnd in range(N):
            counts[int(np.argmax(oracle_mod.gumbel_scores(lb, T, 99, rnd, 1, 2)))] += 1
        p = np.exp(np.array(logits) / T)
        p /= p.sum()
        sigma = np.sqrt(N * p * (1 - p))
        assert np.all(np.abs(counts - N * p) < 5 * sigma), (T, counts, N * p)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_gumbel(oracle_mod, seed):
    V, gamma, B = 12, 3, 3
    d = workloads.toy(seed + 700, V=V, r=4, B=B, gamma=gamma, base_std=1.5)
    key, rnd = 1000 + seed, 17 * seed + 3
    for T in (0.6, 1.0, 2.5):
        Tv = np.full(B, T, np.float32)
        toks, logits = oracle_mod.walk(d["W1"], d["base"], d["anchor"], Tv, W2_bits=d["W2"],
                                       gumbel=True, seed=key, round_counter=rnd)
        for b in range(B):
            prev = int(d["anchor"][b])
            for k in range(gamma):
                u = [value(d["W1"][prev, j]) for j in range(4)]
                lb = bf.step_logits(d["W2"], u, d["base"][b, k])
                assert logits[b, k].tolist() == lb
                U = [bf.gumbel_uniform(oracle_mod.philox4x32_10(
                    [v >> 2, (k << 8) | b, rnd, 0x47554D42], [key & 0xFFFFFFFF, key >> 32]), v)
                    for v in range(V)]
                tok, gap = bf.gumbel_exact(lb, T, U)
                if gap > 1e-12:
                    assert toks[b, k] == tok
                prev = int(toks[b, k])


def test_gumbel_walk_small_temperature_is_greedy(oracle_mod):
    V = 2000
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(0, 5, B=2, gamma=6, V=V)
    t0, lg0 = oracle_mod.walk(W1, inp["base"], inp["anchor"], [0.0, 0.0], W2_bits=W2)
    t1, lg1 = oracle_mod.walk(W1, inp["base"], inp["anchor"], [1e-4, 1e-4], W2_bits=W2, forced=t0,
                              gumbel=True, seed=3, round_counter=9)
    assert np.array_equal(lg0, lg1)
    # G lies in [-ln(-ln 2^-25), -ln(-ln(1 - 2^-25))] = [-2.9, 17.3]: a logit gap
    # above 0.01 is worth 100 at T = 1e-4, more than any difference of noise
    for b in range(2):
        for k in range(6):
            lv = np.sort(oracle_mod.bf16_bits_to_f64(lg1[b, k]))
            if lv[-1] - lv[-2] > 0.01:
                assert t1[b, k] == t0[b, k]


def test_gumbel_walk_uses_its_own_request_step_and_round(oracle_mod):
    # the walk's token at (b, k) is the argmax of the scores of (b, k, round) on
    # its own logits; greedy requests in the same batch are unaffected
    V = 1500
    W1, W2 = workloads.weights(2, V=V)
    inp = workloads.round_inputs(3, 0, B=3, gamma=5, V=V)
    T = np.array([0.8, 0.0, 1.2], np.float32)
    toks, lg = oracle_mod.walk(W1, inp["base"], inp["anchor"], T, W2_bits=W2, gumbel=True, seed=11,
                               round_counter=40)
    for b in (0, 2):
        for k in range(5):
            sc = oracle_mod.gumbel_scores(lg[b, k], T[b], 11, 40, b, k)
            assert toks[b, k] == int(np.argmax(sc))
    tg, _ = oracle_mod.walk(W1, inp["base"][1:2], inp["anchor"][1:2], [0.0], W2_bits=W2)
    assert np.array_equal(toks[1], tg[0])
    # another round counter draws other tokens somewhere
    t2, _ = oracle_mod.walk(W1, inp["base"], inp["anchor"], T, W2_bits=W2, gumbel=True, seed=11,
                            round_counter=41)
    assert not np.array_equal(t2[[0, 2]], toks[[0, 2]])


# ------------------------------------------------------------ GRU serial head
def test_hand_worked_gru(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_gru_r1.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        r = c["r"]
        Wih = bits_of(np.asarray(c["Wih"], dtype=np.float64).ravel()).reshape(3 * r, r)
        Whh = bits_of(np.asarray(c["Whh"], dtype=np.float64).ravel()).reshape(3 * r, r)
        out = oracle_mod.gru_cell(c["x"], c["h"], Wih, Whh, c["bih"], c["bhh"])
        assert np.allclose(out, c["out"], rtol=0, atol=1e-14), (c, out)


def _torch_gru(r, x, h, Wih, Whh, bih, bhh):
    import torch
    cell = torch.nn.GRUCell(r, r).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(value_f64(Wih)))
        cell.weight_hh.copy_(torch.from_numpy(value_f64(Whh)))
        cell.bias_ih.copy_(torch.from_numpy(np.asarray(bih, np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(np.asarray(bhh, np.float64)))
        return cell(torch.from_numpy(np.asarray(x, np.float64))[None],
                    torch.from_numpy(np.asarray(h, np.float64))[None])[0].numpy()


def value_f64(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("r", [1, 8, 256])
def test_gru_cell_matches_torch_grucell(oracle_mod, r):
    # torch.nn.GRUCell in float64 is an independent implementation of the same cell
    Wih, Whh, bih, bhh = workloads.gru_cell_weights(r, r=r)
    rng = np.random.default_rng(r)
    for _ in range(5):
        x = value_f64(workloads.to_bf16_bits(rng.standard_normal(r)))
        h = np.tanh(rng.standard_normal(r))
        want = _torch_gru(r, x, h, Wih, Whh, bih, bhh)
        got = oracle_mod.gru_cell(x, h, Wih, Whh, bih, bhh)
        assert np.allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_gru_walk_brute_force(oracle_mod, seed):
    # V = 12, r = 4: states from torch's GRUCell, the operand bf16(h) by the exact
    # bit-pattern search, the logits as exact rationals
    V, r, gamma, B = 12, 4, 3, 3
    d = workloads.toy(seed + 800, V=V, r=r, B=B, gamma=gamma, w2_std=0.5, base_std=0.5)
    cell = workloads.gru_cell_weights(seed, r=r)
    h0 = workloads.gru_h0(seed, 0, B, r=r)
    T = np.zeros(B, np.float32)
    toks, logits, states = oracle_mod.walk_gru(d["W1"], d["base"], d["anchor"], T, cell, h0, W2_bits=d["W2"])
    for b in range(B):
        prev, h = int(d["anchor"][b]), h0[b].astype(np.float64)
        for k in range(gamma):
            x = value_f64(d["W1"][prev])
            h = _torch_gru(r, x, h, *cell)
            assert np.allclose(states[b, k], h, rtol=0, atol=1e-13)
            u = [value(rne_bits(Fraction(float(v)))) for v in states[b, k]]
            lb = bf.step_logits(d["W2"], u, d["base"][b, k])
            assert logits[b, k].tolist() == lb
            assert toks[b, k] == bf.argmax_lowest(lb)
            prev = int(toks[b, k])


def test_hand_worked_rnn(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_rnn_r1.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        r = c["r"]
        Wih = bits_of(np.asarray(c["Wih"], dtype=np.float64).ravel()).reshape(r, r)
        Whh = bits_of(np.asarray(c["Whh"], dtype=np.float64).ravel()).reshape(r, r)
        out = oracle_mod.rnn_cell(c["x"], c["h"], Wih, Whh, c["bih"], c["bhh"])
        assert np.allclose(out, c["out"], rtol=0, atol=1e-14), (c, out)


def _torch_rnn(r, x, h, Wih, Whh, bih, bhh):
    import torch
    cell = torch.nn.RNNCell(r, r, nonlinearity="tanh").double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(value_f64(Wih)))
        cell.weight_hh.copy_(torch.from_numpy(value_f64(Whh)))
        cell.bias_ih.copy_(torch.from_numpy(np.asarray(bih, np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(np.asarray(bhh, np.float64)))
        return cell(torch.from_numpy(np.asarray(x, np.float64))[None],
                    torch.from_numpy(np.asarray(h, np.float64))[None])[0].numpy()


@pytest.mark.parametrize("r", [1, 8, 256])
def test_rnn_cell_matches_torch_rnncell(oracle_mod, r):
    Wih, Whh, bih, bhh = workloads.rnn_cell_weights(r, r=r)
    rng = np.random.default_rng(100 + r)
    for _ in range(5):
        x = value_f64(workloads.to_bf16_bits(rng.standard_normal(r)))
        h = np.tanh(rng.standard_normal(r))
        want = _torch_rnn(r, x, h, Wih, Whh, bih, bhh)
        got = oracle_mod.rnn_cell(x, h, Wih, Whh, bih, bhh)
        assert np.allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_rnn_walk_brute_force(oracle_mod, seed):
    V, r, gamma, B = 12, 4, 3, 3
    d = workloads.toy(seed + 900, V=V, r=r, B=B, gamma=gamma, w2_std=0.5, base_std=0.5)
    cell = workloads.rnn_cell_weights(seed, r=r)
    h0 = workloads.gru_h0(seed, 1, B, r=r)
    toks, logits, states = oracle_mod.walk_rnn(d["W1"], d["base"], d["anchor"], np.zeros(B, np.float32), cell,
                                               h0, W2_bits=d["W2"])
    for b in range(B):
        prev, h = int(d["anchor"][b]), h0[b].astype(np.float64)
        for k in range(gamma):
            h = _torch_rnn(r, value_f64(d["W1"][prev]), h, *cell)
            assert np.allclose(states[b, k], h, rtol=0, atol=1e-13)
            u = [value(rne_bits(Fraction(float(v)))) for v in states[b, k]]
            lb = bf.step_logits(d["W2"], u, d["base"][b, k])
            assert logits[b, k].tolist() == lb
            assert toks[b, k] == bf.argmax_lowest(lb)
            prev = int(toks[b, k])


# ---------------------------------------------------------------- gated head
def test_hand_worked_gated(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_gated.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        r = c["r"]
        out = oracle_mod.gated_cell(c["x"], c["h"], np.asarray(c["Gq"], np.int8).reshape(r, r),
                                    np.asarray(c["gs"], np.float32), np.asarray(c["gb"], np.float32))
        # s and b are f32: ln 3 rounds to f32 (relative error <= 2^-24), which moves h' by < 1e-7
        assert np.allclose(out, c["out"], rtol=0, atol=1e-6), (c, out)


def _mp_gated(x, h, Gq, gs, gb):
    """The gated update in 50-digit arithmetic (mpmath), element by element."""
    import mpmath
    mpmath.mp.dps = 50
    out = []
    for j in range(len(x)):
        acc = mpmath.fsum(mpmath.mpf(int(Gq[j, i])) * mpmath.mpf(float(h[i])) for i in range(len(x)))
        g = 1 / (1 + mpmath.exp(-(mpmath.mpf(float(gs[j])) * acc + mpmath.mpf(float(gb[j])))))
        out.append(float(g * mpmath.mpf(float(h[j])) + (1 - g) * mpmath.mpf(float(x[j]))))
    return np.asarray(out)


@pytest.mark.parametrize("seed", range(3))
def test_gated_walk_brute_force(oracle_mod, seed):
    V, r, gamma, B = 12, 4, 3, 3
    d = workloads.toy(seed + 950, V=V, r=r, B=B, gamma=gamma, w2_std=0.5, base_std=0.5)
    gate = workloads.gated_weights(seed, r=r)
    h0 = workloads.gru_h0(seed, 2, B, r=r)
    toks, logits, states = oracle_mod.walk_gated(d["W1"], d["base"], d["anchor"], np.zeros(B, np.float32), gate,
                                                 h0, W2_bits=d["W2"])
    for b in range(B):
        prev, h = int(d["anchor"][b]), h0[b].astype(np.float64)
        for k in range(gamma):
            h = _mp_gated(value_f64(d["W1"][prev]), h, *gate)
            assert np.allclose(states[b, k], h, rtol=0, atol=1e-13)
            u = [value(rne_bits(Fraction(float(v)))) for v in states[b, k]]
            lb = bf.step_logits(d["W2"], u, d["base"][b, k])
            assert logits[b, k].tolist() == lb
            assert toks[b, k] == bf.argmax_lowest(lb)
            prev = int(toks[b, k])


def test_gated_walk_limits_and_invariants(oracle_mod):
    V, r, B, gamma = 2000, 256, 2, 5
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(1, 4, B=B, gamma=gamma, V=V, temps="mixed")
    Gq, gs, gb = workloads.gated_weights(0)
    h0 = workloads.gru_h0(0, 4, B)
    args = (W1, inp["base"], inp["anchor"], inp["T"])
    # a closed gate (g = 0 exactly: exp(1e4) overflows) is the Markov walk
    t0, l0, s0 = oracle_mod.walk_gated(*args, (Gq, gs, np.full(r, -1e4, np.float32)), h0,
                                       uniforms=inp["uniforms"], W2_bits=W2)
    tm, lm = oracle_mod.walk(*args, uniforms=inp["uniforms"], W2_bits=W2)
    assert np.array_equal(t0, tm) and np.array_equal(l0, lm)
    for b in range(B):
        prev = int(inp["anchor"][b])
        for k in range(gamma):
            assert np.array_equal(s0[b, k], value_f64(W1[prev]))
            prev = int(t0[b, k])
    # an open gate (g = 1 exactly) keeps h0: every step is the plain step on bf16(h0)
    t1, l1, s1 = oracle_mod.walk_gated(*args, (Gq, gs, np.full(r, 1e4, np.float32)), h0,
                                       uniforms=inp["uniforms"], W2_bits=W2)
    for b in range(B):
        ub = oracle_mod.rne_bf16(h0[b].astype(np.float64))[1]
        for k in range(gamma):
            assert np.array_equal(s1[b, k], h0[b].astype(np.float64))
            tok, lg = oracle_mod.step(ub, inp["base"][b, k], inp["T"][b], inp["uniforms"][b, k], W2_bits=W2)
            assert np.array_equal(lg, l1[b, k]) and tok == t1[b, k]
    # the synthetic gate: each new state lies between the old state and x (a
    # convex blend), the gate is not saturated, and (-Gq, -s) is the same gate
    t2, l2, s2 = oracle_mod.walk_gated(*args, (Gq, gs, gb), h0, uniforms=inp["uniforms"], W2_bits=W2)
    t3, l3, s3 = oracle_mod.walk_gated(*args, (-Gq, -gs, gb), h0, uniforms=inp["uniforms"], W2_bits=W2)
    assert np.array_equal(t2, t3) and np.array_equal(l2, l3) and np.array_equal(s2, s3)
    for b in range(B):
        prev, h = int(inp["anchor"][b]), h0[b].astype(np.float64)
        for k in range(gamma):
            x = value_f64(W1[prev])
            lo, hi = np.minimum(h, x), np.maximum(h, x)
            assert np.all(s2[b, k] >= lo - 1e-15) and np.all(s2[b, k] <= hi + 1e-15)
            w = np.where(np.abs(x - h) > 1e-3, (s2[b, k] - x) / np.where(np.abs(x - h) > 1e-3, h - x, 1.0), 0.5)
            assert 0.02 < np.median(w) < 0.98 and np.ptp(w) > 0.3  # gates spread over (0, 1)
            h, prev = s2[b, k], int(t2[b, k])
    # the gate reads the state: moving h0 alone changes the gates of step 0
    _, _, s4 = oracle_mod.walk_gated(*args, (Gq, gs, gb), -h0, uniforms=inp["uniforms"], W2_bits=W2)
    x0 = value_f64(W1[int(inp["anchor"][0])])
    ok = (np.abs(h0[0] - x0) > 0.05) & (np.abs(-h0[0] - x0) > 0.05)
    g_a = (s2[0, 0] - x0)[ok] / (h0[0] - x0)[ok]
    g_b = (s4[0, 0] - x0)[ok] / (-h0[0] - x0)[ok]
    assert ok.sum() > 100 and np.median(np.abs(g_a - g_b)) > 0.05


# ---------------------------------------------------------------- Domino's head
def test_hand_worked_domino(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_domino.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        r, d = c["r"], c["d"]
        Wih = bits_of(np.asarray(c["Wih"], dtype=np.float64).ravel()).reshape(3 * r, r + d)
        Whh = bits_of(np.asarray(c["Whh"], dtype=np.float64).ravel()).reshape(3 * r, r)
        out = oracle_mod.gru_cell_in(c["x"] + c["H"], c["h"], Wih, Whh, c["bih"], c["bhh"])
        assert np.allclose(out, c["out"], rtol=0, atol=1e-14), (c, out)


def _torch_gru_in(r, n_in, x, h, Wih, Whh, bih, bhh):
    import torch
    cell = torch.nn.GRUCell(n_in, r).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(value_f64(Wih)))
        cell.weight_hh.copy_(torch.from_numpy(value_f64(Whh)))
        cell.bias_ih.copy_(torch.from_numpy(np.asarray(bih, np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(np.asarray(bhh, np.float64)))
        return cell(torch.from_numpy(np.asarray(x, np.float64))[None],
                    torch.from_numpy(np.asarray(h, np.float64))[None])[0].numpy()


@pytest.mark.parametrize("r,d", [(1, 1), (8, 5), (256, 2560)])
def test_domino_cell_matches_torch_grucell(oracle_mod, r, d):
    Wih, Whh, bih, bhh = workloads.domino_cell_weights(r + d, d=d, r=r)
    rng = np.random.default_rng(300 + r)
    for _ in range(3):
        x = value_f64(workloads.to_bf16_bits(rng.standard_normal(r + d)))
        h = np.tanh(rng.standard_normal(r))
        want = _torch_gru_in(r, r + d, x, h, Wih, Whh, bih, bhh)
        got = oracle_mod.gru_cell_in(x, h, Wih, Whh, bih, bhh)
        assert np.allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_domino_walk_brute_force(oracle_mod, seed):
    V, r, d, gamma, B = 12, 4, 3, 3, 3
    dd = workloads.toy(seed + 970, V=V, r=r, B=B, gamma=gamma, w2_std=0.5, base_std=0.5)
    cell = workloads.domino_cell_weights(seed, d=d, r=r)
    H = workloads.domino_hidden(seed, 0, B, gamma, d=d)
    h0 = workloads.gru_h0(seed, 3, B, r=r)
    toks, logits, states = oracle_mod.walk_domino(dd["W1"], dd["base"], dd["anchor"], np.zeros(B, np.float32),
                                                  cell, H, h0, W2_bits=dd["W2"])
    for b in range(B):
        prev, h = int(dd["anchor"][b]), h0[b].astype(np.float64)
        for k in range(gamma):
            x = np.concatenate([value_f64(dd["W1"][prev]), value_f64(H[b, k])])
            h = _torch_gru_in(r, r + d, x, h, *cell)
            assert np.allclose(states[b, k], h, rtol=0, atol=1e-13)
            u = [value(rne_bits(Fraction(float(v)))) for v in states[b, k]]
            lb = bf.step_logits(dd["W2"], u, dd["base"][b, k])
            assert logits[b, k].tolist() == lb
            assert toks[b, k] == bf.argmax_lowest(lb)
            prev = int(toks[b, k])


def test_domino_walk_reduces_to_the_gru_walk(oracle_mod):
    # zero hidden states (or zero hidden columns of Wih) leave the GRU walk on Wih[:, :r]
    V, r, d, B, gamma = 2000, 256, 64, 2, 5
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(1, 5, B=B, gamma=gamma, V=V, temps="mixed")
    Wih, Whh, bih, bhh = workloads.domino_cell_weights(1, d=d)
    h0 = workloads.gru_h0(0, 5, B)
    args = (W1, inp["base"], inp["anchor"], inp["T"])
    tg, lg, sg = oracle_mod.walk_gru(*args, (np.ascontiguousarray(Wih[:, :r]), Whh, bih, bhh), h0,
                                     uniforms=inp["uniforms"], W2_bits=W2)
    zH = np.zeros((B, gamma, d), np.uint16)
    t0, l0, s0 = oracle_mod.walk_domino(*args, (Wih, Whh, bih, bhh), zH, h0, uniforms=inp["uniforms"], W2_bits=W2)
    assert np.array_equal(t0, tg) and np.array_equal(l0, lg) and np.array_equal(s0, sg)
    H = workloads.domino_hidden(1, 5, B, gamma, d=d)
    Wz = Wih.copy()
    Wz[:, r:] = 0
    t1, l1, s1 = oracle_mod.walk_domino(*args, (Wz, Whh, bih, bhh), H, h0, uniforms=inp["uniforms"], W2_bits=W2)
    assert np.array_equal(t1, tg) and np.array_equal(s1, sg)
    # and the hidden states do move the walk
    t2, _, s2 = oracle_mod.walk_domino(*args, (Wih, Whh, bih, bhh), H, h0, uniforms=inp["uniforms"], W2_bits=W2)
    assert np.abs(s2[:, 0] - sg[:, 0]).max() > 0.05


def test_gru_walk_teacher_forcing_and_zero_cell(oracle_mod):
    V, r = 2000, 256
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(1, 4, B=2, gamma=5, V=V, temps="mixed")
    cell = workloads.gru_cell_weights(0)
    h0 = workloads.gru_h0(0, 4, 2)
    t0, l0, s0 = oracle_mod.walk_gru(W1, inp["base"], inp["anchor"], inp["T"], cell, h0,
                                     uniforms=inp["uniforms"], W2_bits=W2)
    # forcing the oracle's own tokens and (f32-exact) states reproduces the walk
    s32 = s0.astype(np.float32)
    t1, l1, s1 = oracle_mod.walk_gru(W1, inp["base"], inp["anchor"], inp["T"], cell, h0,
                                     uniforms=inp["uniforms"], W2_bits=W2, forced=t0, forced_h=s32)
    assert np.array_equal(t0[:, 0], t1[:, 0]) and np.array_equal(l0[:, 0], l1[:, 0])
    # each step is the plain walk's step with the operand bf16(h_k)
    for b in range(2):
        for k in range(5):
            ub = oracle_mod.rne_bf16(s0[b, k])[1]
            tok, lg = oracle_mod.step(ub, inp["base"][b, k], inp["T"][b], inp["uniforms"][b, k], W2_bits=W2)
            assert np.array_equal(lg, l0[b, k]) and tok == t0[b, k]
    # a zero cell halves the state every step: h_k = h0 / 2^(k+1)
    z = (np.zeros((3 * r, r), np.uint16), np.zeros((3 * r, r), np.uint16), np.zeros(3 * r, np.float32),
         np.zeros(3 * r, np.float32))
    _, _, sz = oracle_mod.walk_gru(W1, inp["base"], inp["anchor"], [0.0, 0.0], z, h0, W2_bits=W2)
    for k in range(5):
        assert np.array_equal(sz[:, k], h0.astype(np.float64) / 2.0 ** (k + 1))


def test_hand_worked_sampler(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_sampler.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        lb = bits_of(c["logits"])
        assert oracle_mod.sample(lb, c["T"], c["u"]) == c["token"], c
    # the closed-form boundary e/(e+1)
    p0 = math.e / (math.e + 1.0)
    lb = bits_of([1.0, 0.0])
    assert oracle_mod.sample(lb, 1.0, np.nextafter(np.float32(p0), np.float32(0))) == 0
    assert oracle_mod.sample(lb, 1.0, np.nextafter(np.float32(p0), np.float32(1))) == 1


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(50))
def test_brute_force_v12_r4_all_anchors(oracle_mod, seed):
    d = workloads.toy(seed, V=12, r=4, B=12, gamma=3, w2_std=0.5, base_std=1.0)
    anchors = np.arange(12, dtype=np.int32)
    base = d["base"]
    T = np.zeros(12, dtype=np.float32)
    toks, logits = oracle_mod.walk(d["W1"], base, anchors, T, W2_bits=d["W2"])
    for b in range(12):
        bt, bl, _ = bf.walk(d["W1"], d["W2"], base[b], anchors[b])
        assert toks[b].tolist() == bt
        assert logits[b].tolist() == bl


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_int8_variant(oracle_mod, seed):
    d = workloads.toy(seed + 100, V=12, r=4, B=12, gamma=3, w2_std=0.5, base_std=0.2)
    Q, scale = workloads.quantize_int8(d["W2"])
    anchors = np.arange(12, dtype=np.int32)
    T = np.zeros(12, dtype=np.float32)
    toks, logits = oracle_mod.walk(d["W1"], d["base"], anchors, T, Q=Q, scale=scale)
    for b in range(12):
        bt, bl, _ = bf.walk(d["W1"], None, d["base"][b], anchors[b], Q=Q, scale=scale)
        assert toks[b].tolist() == bt
        assert logits[b].tolist() == bl


@pytest.mark.parametrize("seed", range(5))
def test_bigram_route(oracle_mod, seed):
    """logit_k = bf16(base_k + bf16((W2 W1^T)[:, prev])), through the exact V x V bigram matrix."""
    V, r = 12, 4
    d = workloads.toy(seed + 200, V=V, r=r, B=1, gamma=3)
    W1 = [[value(x) for x in row] for row in d["W1"]]
    W2 = [[value(x) for x in row] for row in d["W2"]]
    bigram = [[sum(W2[v][j] * W1[p][j] for j in range(r)) for p in range(V)] for v in range(V)]
    toks, logits = oracle_mod.walk(d["W1"], d["base"], d["anchor"], [0.0], W2_bits=d["W2"])
    prev = int(d["anchor"][0])
    for k in range(3):
        want = [rne_bits(value(d["base"][0, k, v]) + value(rne_bits(bigram[v][prev]))) for v in range(V)]
        assert logits[0, k].tolist() == want
        prev = int(toks[0, k])


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_sampled(oracle_mod, seed):
    V = 12
    d = workloads.toy(seed + 300, V=V, r=4, B=1, gamma=3, base_std=1.5)
    for T in (0.6, 1.0, 2.5):
        toks, logits = oracle_mod.walk(d["W1"], d["base"], d["anchor"], [T],
                                       uniforms=d["uniforms"], W2_bits=d["W2"])
        bt, bl, margin = bf.walk(d["W1"], d["W2"], d["base"][0], d["anchor"][0], T=T,
                                 uniforms=d["uniforms"][0])
        assert logits[0].tolist() == bl
        if margin > 1e-12:
            assert toks[0].tolist() == bt


@pytest.mark.parametrize("seed", range(25))
def test_brute_force_single_rounding(oracle_mod, seed):
    d = workloads.toy(seed + 400, V=12, r=4, B=12, gamma=3, w2_std=0.5, base_std=1.0)
    anchors = np.arange(12, dtype=np.int32)
    T = np.zeros(12, dtype=np.float32)
    toks, logits = oracle_mod.walk(d["W1"], d["base"], anchors, T, W2_bits=d["W2"], single_round=True)
    for b in range(12):
        bt, bl, _ = bf.walk(d["W1"], d["W2"], d["base"][b], anchors[b], single=True)
        assert toks[b].tolist() == bt
        assert logits[b].tolist() == bl


@pytest.mark.parametrize("seed", range(5))
def test_brute_force_single_rounding_int8_and_sampled(oracle_mod, seed):
    d = workloads.toy(seed + 500, V=12, r=4, B=12, gamma=3, w2_std=0.5, base_std=0.2)
    Q, scale = workloads.quantize_int8(d["W2"])
    anchors = np.arange(12, dtype=np.int32)
    toks, logits = oracle_mod.walk(d["W1"], d["base"], anchors, np.zeros(12, np.float32), Q=Q,
                                   scale=scale, single_round=True)
    for b in range(12):
        bt, bl, _ = bf.walk(d["W1"], None, d["base"][b], anchors[b], Q=Q, scale=scale, single=True)
        assert toks[b].tolist() == bt and logits[b].tolist() == bl
    e = workloads.toy(seed + 600, V=12, r=4, B=1, gamma=3, base_std=1.5)
    for T in (0.6, 1.0):
        toks, logits = oracle_mod.walk(e["W1"], e["base"], e["anchor"], [T], uniforms=e["uniforms"],
                                       W2_bits=e["W2"], single_round=True)
        bt, bl, margin = bf.walk(e["W1"], e["W2"], e["base"][0], e["anchor"][0], T=T,
                                 uniforms=e["uniforms"][0], single=True)
        assert logits[0].tolist() == bl
        if margin > 1e-12:
            assert toks[0].tolist() == bt


def test_single_rounding_special_cases(oracle_mod):
    # base = 0: both modes round the dot product once, so they agree (and equal
    # the rounding of a numpy matmul); W2 = 0: both give the base logits
    V, r = 500, 256
    W1, W2 = workloads.weights(0, V=V, r=r)
    base0 = np.zeros((1, 5, V), dtype=np.uint16)
    t1, l1 = oracle_mod.walk(W1, base0, [3], [0.0], W2_bits=W2)
    t2, l2 = oracle_mod.walk(W1, base0, [3], [0.0], W2_bits=W2, single_round=True)
    assert np.array_equal(l1, l2) and np.array_equal(t1, t2)
    d = workloads.toy(9, V=V, r=r, B=4, gamma=3)
    Wz = np.zeros((V, r), dtype=np.uint16)
    for sr in (False, True):
        toks, logits = oracle_mod.walk(d["W1"], d["base"], d["anchor"], np.zeros(4, np.float32),
                                       W2_bits=Wz, single_round=sr)
        assert np.array_equal(logits, d["base"])
    # the two modes differ somewhere on ordinary inputs (the flag is not a no-op)
    e = workloads.toy(11, V=V, r=r, B=1, gamma=4, base_std=2.0)
    _, la = oracle_mod.walk(e["W1"], e["base"], e["anchor"], [0.0], W2_bits=e["W2"])
    _, lb = oracle_mod.walk(e["W1"], e["base"], e["anchor"], [0.0], W2_bits=e["W2"], single_round=True)
    assert not np.array_equal(la, lb)


# ------------------------------------------------------------- special cases
def test_zero_w2_gives_argmax_of_base(oracle_mod):
    V, r, gamma = 300, 256, 4
    d = workloads.toy(7, V=V, r=r, B=V, gamma=gamma)
    W2 = np.zeros((V, r), dtype=np.uint16)
    anchors = np.arange(V, dtype=np.int32)
    toks, logits = oracle_mod.walk(d["W1"], d["base"], anchors, np.zeros(V, np.float32), W2_bits=W2)
    assert np.array_equal(logits, d["base"])
    basef = oracle_mod.bf16_bits_to_f64(d["base"])
    assert np.array_equal(toks, np.argmax(basef, axis=2))


def test_zero_base_is_single_rounding_of_numpy_matmul(oracle_mod):
    V, r = 1000, 256
    W1, W2 = workloads.weights(0, V=V, r=r)
    base = np.zeros((1, 7, V), dtype=np.uint16)
    toks, logits = oracle_mod.walk(W1, base, [5], [0.0], W2_bits=W2)
    W1f, W2f = oracle_mod.bf16_bits_to_f64(W1), oracle_mod.bf16_bits_to_f64(W2)
    prev = 5
    for k in range(7):
        acc = W2f @ W1f[prev]                          # numpy / BLAS route
        want = [rne_bits(Fraction(float(a))) for a in acc]
        assert logits[0, k].tolist() == want
        wv = [value(w) for w in want]
        assert int(toks[0, k]) == wv.index(max(wv))    # first maximum of the emitted logits
        prev = int(toks[0, k])


def test_medium_vocab_against_numpy_and_exact_rounding(oracle_mod):
    V, r, gamma = 1000, 256, 7
    W1, W2 = workloads.weights(0, V=V, r=r)
    inp = workloads.round_inputs(0, 0, B=1, gamma=gamma, V=V)
    toks, logits = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], W2_bits=W2)
    W1f, W2f = oracle_mod.bf16_bits_to_f64(W1), oracle_mod.bf16_bits_to_f64(W2)
    prev = int(inp["anchor"][0])
    for k in range(gamma):
        acc = W2f @ W1f[prev]
        bias = [rne_bits(Fraction(float(a))) for a in acc]
        want = [rne_bits(value(inp["base"][0, k, v]) + value(bias[v])) for v in range(V)]
        assert logits[0, k].tolist() == want
        lv = oracle_mod.bf16_bits_to_f64(logits[0, k])
        assert toks[0, k] == int(np.argmax(lv))        # numpy: first occurrence
        prev = int(toks[0, k])


def test_vocab_of_one():
    import oracle
    W1 = workloads.to_bf16_bits(np.ones((1, 8)))
    W2 = workloads.to_bf16_bits(np.full((1, 8), 0.5))
    base = workloads.to_bf16_bits(np.zeros((2, 5, 1)))
    toks, _ = oracle.walk(W1, base, [0, 0], [0.0, 1.0], uniforms=np.full((2, 5), 0.99, np.float32),
                          W2_bits=W2)
    assert toks.tolist() == [[0] * 5, [0] * 5]


def test_constructed_exact_ties_pick_lowest_index(oracle_mod):
    V, r = 64, 256
    W1 = workloads.to_bf16_bits(np.ones((V, r)))
    W2 = np.zeros((V, r), dtype=np.uint16)
    base = np.zeros((1, 3, V), dtype=np.float32)
    base[0, 0, [17, 40, 63]] = 2.5                   # three-way tie at the top
    base[0, 1, :] = 1.0                              # all equal
    base[0, 2, [63, 5]] = -0.0                       # -0 and +0 compare equal
    base[0, 2, :5] = -1.0
    toks, _ = oracle_mod.walk(W1, workloads.to_bf16_bits(base), [0], [0.0], W2_bits=W2)
    assert toks[0].tolist() == [17, 0, 5]


# ------------------------------------------------------------------- sampler
def test_sampler_grid_matches_closed_form(oracle_mod):
    rng = np.random.default_rng(5)
    logits_bits = workloads.to_bf16_bits(rng.standard_normal(40) * 2)
    vals = list(oracle_mod.bf16_bits_to_f64(logits_bits))
    for T in (0.6, 1.0):
        import mpmath
        M = max(vals)
        w = [mpmath.e ** ((mpmath.mpf(l) - M) / mpmath.mpf(float(np.float32(T)))) for l in vals]
        Z = sum(w)
        p = [float(x / Z) for x in w]
        N = 20000
        counts = np.zeros(len(vals), dtype=int)
        for i in range(N):
            u = np.float32((i + 0.5) / N)
            counts[oracle_mod.sample(logits_bits, T, u)] += 1
        assert np.all(np.abs(counts - N * np.asarray(p)) <= 1.0 + 1e-9), (counts, N * np.asarray(p))


def test_sampler_monotone_and_endpoints(oracle_mod):
    rng = np.random.default_rng(6)
    logits_bits = workloads.to_bf16_bits(rng.standard_normal(500) * 3)
    us = np.sort(rng.random(400).astype(np.float32))
    toks = [oracle_mod.sample(logits_bits, 1.0, u) for u in us]
    assert all(a <= b for a, b in zip(toks, toks[1:]))
    assert oracle_mod.sample(logits_bits, 1.0, 0.0) == 0
    # weights that underflow to zero are never drawn; u = 0 takes the first positive weight
    lb = bits_of([-3.0e38, -3.0e38, 5.0, 1.0, -3.0e38])
    assert oracle_mod.sample(lb, 0.6, 0.0) == 2
    assert oracle_mod.sample(lb, 0.6, np.float32(0.9999999)) == 3


def test_small_temperature_is_argmax_and_zero_temperature_is_argmax(oracle_mod):
    V = 2000
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(0, 3, B=1, gamma=7, V=V)
    t0, lg0 = oracle_mod.walk(W1, inp["base"], inp["anchor"], [0.0], W2_bits=W2)
    # T = 0 is the lowest-index argmax of the emitted logits
    for k in range(7):
        assert t0[0, k] == int(np.argmax(oracle_mod.bf16_bits_to_f64(lg0[0, k])))
    # T -> 0+ with a clear gap reduces to the argmax
    t1, lg1 = oracle_mod.walk(W1, inp["base"], inp["anchor"], [1e-4],
                              uniforms=np.full((1, 7), 0.5, np.float32), forced=t0, W2_bits=W2)
    for k in range(7):
        lv = np.sort(oracle_mod.bf16_bits_to_f64(lg1[0, k]))
        if lv[-1] - lv[-2] > 0.01:
            assert t1[0, k] == t0[0, k]


def test_teacher_forcing_with_own_tokens_is_free_running(oracle_mod):
    V = 3000
    W1, W2 = workloads.weights(1, V=V)
    inp = workloads.round_inputs(2, 1, B=3, gamma=6, V=V, temps="mixed")
    t0, l0 = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2)
    t1, l1 = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2,
                             forced=t0)
    assert np.array_equal(t0, t1) and np.array_equal(l0, l1)
    # forcing a different history changes later steps only
    f = t0.copy()
    f[:, 2] = (f[:, 2] + 1) % V
    t2, l2 = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2,
                             forced=f)
    assert np.array_equal(l2[:, :3], l0[:, :3])
    assert not np.array_equal(l2[:, 3], l0[:, 3])


def test_thread_count_does_not_change_results(oracle_mod):
    V = 5000
    W1, W2 = workloads.weights(0, V=V)
    inp = workloads.round_inputs(2, 4, B=2, gamma=5, V=V, temps="mixed")
    oracle_mod.set_threads(1)
    a = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2)
    oracle_mod.set_threads(8)
    b = oracle_mod.walk(W1, inp["base"], inp["anchor"], inp["T"], inp["uniforms"], W2_bits=W2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_int8_quantizer_recipe():
    # row max 127 * 2^-7 gives the exact scale 2^-7; -63.5 * 2^-7 / 2^-7 is a tie -> even -64
    W2 = workloads.to_bf16_bits(np.array([[0.0, 0.0], [127 / 128, -63.5 / 128], [0.02, -0.0201]]))
    Q, s = workloads.quantize_int8(W2)
    assert s[0] == 0 and Q[0].tolist() == [0, 0]
    assert s[1] == np.float32(2.0 ** -7) and Q[1].tolist() == [127, -64]
    assert int(Q[2, 1]) == -127 and s[2] == np.float32(abs(float(value(int(W2[2, 1])))) / 127)
