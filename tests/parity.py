"""Teacher-forced parity of a GPU round against the CPU oracle.

Rules (the walk is exact by definition; the GPU only sums in fp32 in another
order):
  * logits: each GPU logit lies in [bf16(base + bf16(acc - E)), bf16(base + bf16(acc + E))]
    where acc is the exact dot product and E = g_r * sum_j |w_j u_j| bounds
    any fp32 summation of r = 256 terms (g_r = r 2^-24 / (1 - r 2^-24)), plus
    2^-24 (|acc| + E) for int8 rows, whose fp32 sum is then scaled in fp32; and it
    is within one bf16 ulp of the oracle's logit (the ulp taken at the largest
    of |oracle logit|, |GPU logit| and |bias|, so that cancellation in
    base + bias cannot fake a miss), except where that fp32 interval itself
    reaches two ulps: when the fp32 sum straddles a midpoint of the first
    rounding and the second rounding then meets a tie, double rounding turns
    one bias ulp into two logit ulps.  There 2 ulps are allowed and counted;
  * greedy tokens: the GPU token is always the lowest-index argmax of the
    GPU's own logits; it equals the oracle's token wherever the oracle's
    top-two gap exceeds 2 ulps, and elsewhere its oracle logit is within
    2 ulps of the oracle's maximum;
  * sampled tokens: from the GPU's own logits in binary64, C_{t-1} - d <= u Z < C_t + d
    with d = 1e-5 Z, and the token equals the oracle's draw on those logits
    wherever u Z is farther than d from every boundary.
  * Gumbel-max tokens (flag DSW_FLAG_GUMBEL): with the binary64 scores
    S_v = l_v / T - ln(-ln U_v) of the GPU's own logits and the oracle's noise,
    S_tok >= max S - d with d = 1e-4, and the token equals the oracle's
    argmax wherever the top two scores are more than 2 d apart.  d covers the
    GPU's fp32 score l * fp32(1/T) + G: the product (two roundings of a value
    below 2^6: under 3e-6), the variate G, which the kernels compute within
    2e-6 of binary64 for every U their noise can take (test_gumbel_variate_error
    evaluates the kernels' own function on all 2^23 of them), and the final
    fp32 sum (half an ulp below 2^6: under 4e-6); together under 1e-5 = d / 10.
Step k uses prev = the GPU's token k-1 (teacher forcing), so every step is
judged on its own.

Single-rounding mode (logit = bf16(base + fp32 dot)): the interval becomes
[bf16(base + acc - E'), bf16(base + acc + E')] with E' = E + 2^-24 (|base + acc| + E),
the fp32 addition rounding once more before the one rounding to bf16.
"""
from __future__ import annotations

import numpy as np

import oracle

R = 256
GAMMA_R = R * 2.0 ** -24 / (1 - R * 2.0 ** -24)
SAMPLE_TOL = 1e-5
GUMBEL_TOL = 1e-4


def bf16_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


class Weights:
    """f64 views of the bf16 (or int8) tables, computed once per test."""

    def __init__(self, W1_bits, W2_bits=None, Q=None, scale=None):
        self.W1_bits, self.W2_bits, self.Q, self.scale = W1_bits, W2_bits, Q, scale
        self.W1 = oracle.bf16_bits_to_f64(W1_bits)
        if W2_bits is not None:
            self.W2 = oracle.bf16_bits_to_f64(W2_bits)
        else:
            self.W2 = Q.astype(np.float64) * scale.astype(np.float64)[:, None]
        self.W2abs = np.abs(self.W2)


def _gap_top2(o):
    """Index of the oracle's first maximum, the maximum and the gap to the runner-up."""
    top = int(np.argmax(o))
    omax = o[top]
    if o.size == 1:
        return top, omax, np.inf
    rest = o.copy()
    rest[top] = -np.inf
    return top, omax, omax - rest.max()


def check_round(w: Weights, base, anchor, T, uniforms, gpu_tokens, gpu_logits, steps=None,
                single_round=False, gumbel=None, latents=None, requests=None):
    """Assert the parity rules for one round; return a small report dict.
    gumbel: (seed, round counter) of a Gumbel-max walk, else None.
    latents: [B, gamma, r] bf16 bits of the GEMV operand of every step (the GRU
    head's bf16(h)), else None (the Markov head's W1[prev]).
    steps / requests: the steps and requests checked (default: all).

    The GPU logits are first compared bit for bit with the oracle's; the
    fp32-accumulation interval, the ulp rule and the two-ulp count are then
    evaluated on the differing elements only (an element equal to the
    oracle's lies in the interval, whose ends are roundings of values on
    either side of the exact sum)."""
    B, gamma, V = base.shape
    g_seed, g_round = gumbel if gumbel is not None else (0, 0)
    steps = list(range(gamma)) if steps is None else list(steps)
    requests = list(range(B)) if requests is None else list(requests)
    if latents is None:
        or_tok, or_lg = oracle.walk(w.W1_bits, base, anchor, T, uniforms, W2_bits=w.W2_bits, Q=w.Q,
                                    scale=w.scale, forced=gpu_tokens, single_round=single_round,
                                    gumbel=gumbel is not None, seed=g_seed, round_counter=g_round)
    else:  # one oracle step per (request, step) on the given operand
        assert gumbel is None
        or_tok = np.empty((B, gamma), np.int32)
        or_lg = np.empty((B, gamma, V), np.uint16)
        for b in requests:
            for k in steps:
                uk = 0.0 if uniforms is None else uniforms[b, k]
                or_tok[b, k], or_lg[b, k] = oracle.step(latents[b, k], base[b, k], T[b], uk,
                                                        W2_bits=w.W2_bits, Q=w.Q, scale=w.scale,
                                                        single_round=single_round)
    rep = {"steps": 0, "exact_logits": 0, "logits": 0, "near_ties": 0, "token_match": 0,
           "sampled": 0, "sampled_exact_checked": 0, "two_ulp_double_rounding": 0}
    for b in requests:
        for k in steps:
            gb, ob = gpu_logits[b, k], or_lg[b, k]
            g = oracle.bf16_bits_to_f64(gb)
            o = oracle.bf16_bits_to_f64(ob)
            idx = np.nonzero(gb != ob)[0]
            if idx.size:
                prev = int(anchor[b]) if k == 0 else int(gpu_tokens[b, k - 1])
                u = w.W1[prev] if latents is None else oracle.bf16_bits_to_f64(latents[b, k])
                W = w.W2[idx]
                acc = W @ u
                E = GAMMA_R * (w.W2abs[idx] @ np.abs(u))
                if w.Q is not None:  # the fp32 product scale * sum rounds once more
                    E = E + 2.0 ** -24 * (np.abs(acc) + E)
                bias = oracle.rne_bf16(acc)[0]
                bse = oracle.bf16_bits_to_f64(base[b, k][idx])
                if single_round:
                    E1 = E + 2.0 ** -24 * (np.abs(bse + acc) + E)
                    Llo = oracle.rne_bf16(bse + acc - E1)[0]
                    Lhi = oracle.rne_bf16(bse + acc + E1)[0]
                else:
                    Llo = oracle.rne_bf16(bse + oracle.rne_bf16(acc - E)[0])[0]
                    Lhi = oracle.rne_bf16(bse + oracle.rne_bf16(acc + E)[0])[0]
                gi, oi = g[idx], o[idx]
                bad = np.nonzero((gi < Llo) | (gi > Lhi))[0]
                assert bad.size == 0, f"b={b} k={k}: logits outside the fp32 bound at {idx[bad[:5]]} " \
                                      f"gpu={gi[bad[:5]]} oracle={oi[bad[:5]]}"
                ulp = bf16_ulp(np.maximum.reduce([np.abs(oi), np.abs(gi), np.abs(bias)]))
                diff = np.abs(gi - oi)
                reach = np.maximum(Lhi - oi, oi - Llo)          # what fp32 accumulation can reach
                far = np.nonzero((diff > ulp) & ~((reach > ulp) & (diff <= 2 * ulp)))[0]
                assert far.size == 0, f"b={b} k={k}: logits beyond 1 ulp at {idx[far[:5]]} " \
                                      f"gpu={gi[far[:5]]} oracle={oi[far[:5]]}"
                rep["two_ulp_double_rounding"] += int(np.count_nonzero(diff > ulp))
                rep["exact_logits"] += V - int(np.count_nonzero(diff))
            else:
                rep["exact_logits"] += V
            rep["steps"] += 1
            rep["logits"] += V
            tok = int(gpu_tokens[b, k])
            assert 0 <= tok < V
            if T[b] == 0:
                assert tok == int(np.argmax(g)), f"b={b} k={k}: token {tok} is not the first argmax of the GPU's own logits"
                top, omax, gap = _gap_top2(o)
                if gap > 2 * bf16_ulp(omax):
                    assert tok == int(or_tok[b, k]), f"b={b} k={k}: token {tok} vs oracle {or_tok[b, k]}"
                    rep["token_match"] += 1
                else:
                    rep["near_ties"] += 1
                    assert o[tok] >= omax - 2 * bf16_ulp(omax)
                    rep["token_match"] += int(tok == int(or_tok[b, k]))
            elif gumbel is not None:
                rep["sampled"] += 1
                S = oracle.gumbel_scores(gb, T[b], g_seed, g_round, b, k)
                top = int(np.argmax(S))
                assert S[tok] >= S[top] - GUMBEL_TOL, \
                    f"b={b} k={k}: Gumbel-max token {tok} scores {S[tok]}, best {top} scores {S[top]}"
                second = np.delete(S, top).max() if V > 1 else -np.inf
                if S[top] - second > 2 * GUMBEL_TOL:
                    assert tok == top, f"b={b} k={k}: Gumbel-max token {tok} vs oracle {top}"
                    rep["sampled_exact_checked"] += 1
            else:
                rep["sampled"] += 1
                Tb = float(np.float32(T[b]))
                M = g.max()
                wts = np.exp((g - M) / Tb)
                C = np.cumsum(wts)
                Z = C[-1]
                t = float(np.float32(uniforms[b, k])) * Z
                d = SAMPLE_TOL * Z
                cprev = C[tok - 1] if tok > 0 else 0.0
                assert cprev - d <= t < C[tok] + d, f"b={b} k={k}: sampled token {tok} does not hold u*Z"
                margin = np.min(np.abs(C - t))
                if margin > d:
                    want = oracle.sample(gb, T[b], uniforms[b, k])
                    assert tok == want, f"b={b} k={k}: sampled {tok} vs oracle {want}"
                    rep["sampled_exact_checked"] += 1
    return rep


# ---------------------------------------------------------------- GRU head
F32_EPS = 2.0 ** -24


def check_gru_states(W1_bits, cell, h0, gpu_tokens, anchor, gpu_states, hidden=None):
    """The GPU's state after every step against the oracle's binary64 GRU cell
    applied to the GPU's previous state (teacher forcing), within a bound of
    the fp32 evaluation: each of the six dot products (r bf16 x bf16 or bf16 x
    fp32 terms, fma) and its bias adds err <= g_(r+4) (sum |w v| + |b|) with
    g_n = n 2^-24 / (1 - n 2^-24); sigmoid' <= 1/4, tanh' <= 1; each fp32
    exp/divide/tanh adds 4 ulps of its result, the final blend 3 ulps.
    hidden: [gamma, d] bf16 bits of Domino's head, appended to every step's
    input (Wih is then [3r, r + d] and the dot products have r + d terms).
    Returns (steps checked, largest error, largest error / bound)."""
    Wih, Whh, bih, bhh = cell
    Wi, Wh = oracle.bf16_bits_to_f64(Wih), oracle.bf16_bits_to_f64(Whh)
    r = Wh.shape[1]
    n_in = Wi.shape[1]
    gam = (n_in + 4) * F32_EPS / (1 - (n_in + 4) * F32_EPS)
    gamma = gpu_states.shape[0]
    worst, worst_ratio = 0.0, 0.0
    for k in range(gamma):
        prev = int(anchor) if k == 0 else int(gpu_tokens[k - 1])
        x = oracle.bf16_bits_to_f64(W1_bits[prev])
        if hidden is not None:
            x = np.concatenate([x, oracle.bf16_bits_to_f64(hidden[k])])
        h = h0.astype(np.float64) if k == 0 else gpu_states[k - 1].astype(np.float64)
        want = oracle.gru_cell_in(x, h, Wih, Whh, bih, bhh)
        gi = Wi @ x + bih
        gh = Wh @ h + bhh
        Ei = gam * (np.abs(Wi) @ np.abs(x) + np.abs(bih))
        Eh = gam * (np.abs(Wh) @ np.abs(h) + np.abs(bhh))
        gi, gh, Ei, Eh = (a.reshape(3, r) for a in (gi, gh, Ei, Eh))
        rg = 1 / (1 + np.exp(-(gi[0] + gh[0])))
        zg = 1 / (1 + np.exp(-(gi[1] + gh[1])))
        ng = np.tanh(gi[2] + rg * gh[2])
        e_r = 0.25 * (Ei[0] + Eh[0]) + 4 * F32_EPS * rg
        e_z = 0.25 * (Ei[1] + Eh[1]) + 4 * F32_EPS * zg
        e_n = Ei[2] + rg * Eh[2] + e_r * np.abs(gh[2]) + 4 * F32_EPS * (np.abs(ng) + np.abs(gi[2] + rg * gh[2]))
        bound = e_z * np.abs(ng - h) + (1 - zg) * e_n + 3 * F32_EPS * (np.abs(ng) + np.abs(h))
        bound = 2 * bound + 1e-9
        err = np.abs(gpu_states[k].astype(np.float64) - want)
        assert np.all(err <= bound), f"k={k}: state error {err.max()} above its bound at {np.argmax(err - bound)}"
        worst = max(worst, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / bound).max()))
    return gamma, worst, worst_ratio


def check_gated_states(W1_bits, gate, h0, gpu_tokens, anchor, gpu_states):
    """As check_gru_states for the gated head, g = sigmoid(s (Gq h) + b),
    h' = g h + (1 - g) x: the fp32 pre-activation errs by at most
    g_(r+4) (|s| sum |q h| + |b|) (exact int8 x fp32 products, fp32 sums, the
    scale and the bias), which passes through sigmoid' <= 1/4; exp, add and
    divide add 4 ulps of g; the blend errs by |dg| |h - x| plus 3 ulps of
    |h| + |x|.  Returns (steps checked, largest error, largest error / bound)."""
    Gq, gs, gb = gate
    Q = np.asarray(Gq, np.float64)
    s = np.asarray(gs, np.float64)
    b = np.asarray(gb, np.float64)
    r = Q.shape[1]
    gam = (r + 4) * F32_EPS / (1 - (r + 4) * F32_EPS)
    worst, worst_ratio = 0.0, 0.0
    for k in range(gpu_states.shape[0]):
        prev = int(anchor) if k == 0 else int(gpu_tokens[k - 1])
        x = oracle.bf16_bits_to_f64(W1_bits[prev])
        h = h0.astype(np.float64) if k == 0 else gpu_states[k - 1].astype(np.float64)
        want = oracle.gated_cell(x, h, Gq, gs, gb)
        g = 1 / (1 + np.exp(-(s * (Q @ h) + b)))
        e_g = 0.25 * gam * (np.abs(s) * (np.abs(Q) @ np.abs(h)) + np.abs(b)) + 4 * F32_EPS * g
        bound = 2 * (e_g * np.abs(h - x) + 3 * F32_EPS * (np.abs(h) + np.abs(x))) + 1e-9
        err = np.abs(gpu_states[k].astype(np.float64) - want)
        assert np.all(err <= bound), f"k={k}: state error {err.max()} above its bound at {np.argmax(err - bound)}"
        worst = max(worst, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / bound).max()))
    return gpu_states.shape[0], worst, worst_ratio


def check_rnn_states(W1_bits, cell, h0, gpu_tokens, anchor, gpu_states):
    """As check_gru_states for the tanh RNN cell: the error of the fp32
    pre-activation (two dot products and biases, g_(r+4) sum |w v|) passes
    through tanh' <= 1; tanh and the adds add 4 ulps of the result and 2 of the
    pre-activation.  Returns (steps checked, largest error, largest error / bound)."""
    Wih, Whh, bih, bhh = cell
    Wi, Wh = oracle.bf16_bits_to_f64(Wih), oracle.bf16_bits_to_f64(Whh)
    r = Wi.shape[1]
    gam = (r + 4) * F32_EPS / (1 - (r + 4) * F32_EPS)
    worst, worst_ratio = 0.0, 0.0
    for k in range(gpu_states.shape[0]):
        prev = int(anchor) if k == 0 else int(gpu_tokens[k - 1])
        x = oracle.bf16_bits_to_f64(W1_bits[prev])
        h = h0.astype(np.float64) if k == 0 else gpu_states[k - 1].astype(np.float64)
        want = oracle.rnn_cell(x, h, Wih, Whh, bih, bhh)
        pre = Wi @ x + bih + Wh @ h + bhh
        E = gam * (np.abs(Wi) @ np.abs(x) + np.abs(bih) + np.abs(Wh) @ np.abs(h) + np.abs(bhh))
        bound = 2 * (E + 4 * F32_EPS * np.abs(want) + 2 * F32_EPS * np.abs(pre)) + 1e-9
        err = np.abs(gpu_states[k].astype(np.float64) - want)
        assert np.all(err <= bound), f"k={k}: state error {err.max()} above its bound at {np.argmax(err - bound)}"
        worst = max(worst, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / bound).max()))
    return gpu_states.shape[0], worst, worst_ratio
