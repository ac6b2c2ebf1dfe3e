"""Brute-force walk with exact rationals (Fraction) and high-precision exp (mpmath).

A pin for the oracle on tiny walks (the size of the pages' Fig 2 toy, V = 12,
r = 4, three steps).  It shares no code with the oracle: dot products are exact
rationals, rounding is the bit-pattern search of exact_bf16.
"""
from fractions import Fraction

import mpmath

from exact_bf16 import rne_bits, value

mpmath.mp.dps = 60


def bias_exact(W2, u, v, Q=None, scale=None):
    if Q is None:
        return sum(value(W2[v, j]) * u[j] for j in range(len(u)))
    dot = sum(Fraction(int(Q[v, j])) * u[j] for j in range(len(u)))
    return Fraction(float(scale[v])) * dot


def step_logits(W2, u, base_row, Q=None, scale=None, single=False):
    """bf16 logit bits of one step: bf16(base + bf16(dot)), or bf16(base + dot)
    rounded once when `single`."""
    V = len(base_row)
    out = []
    for v in range(V):
        dot = bias_exact(W2, u, v, Q, scale)
        if single:
            out.append(rne_bits(value(base_row[v]) + dot))
        else:
            out.append(rne_bits(value(base_row[v]) + value(rne_bits(dot))))
    return out


def argmax_lowest(logit_bits):
    vals = [value(x) for x in logit_bits]
    best = 0
    for v in range(1, len(vals)):
        if vals[v] > vals[best]:
            best = v
    return best


def sample_exact(logit_bits, T, uniform):
    """Inverse CDF at 60 digits: (token, distance of u*Z to the nearest boundary / Z)."""
    vals = [mpmath.mpf(value(x).numerator) / value(x).denominator for x in logit_bits]
    M = max(vals)
    w = [mpmath.e ** ((l - M) / mpmath.mpf(float(T))) for l in vals]
    C = []
    run = mpmath.mpf(0)
    for x in w:
        run += x
        C.append(run)
    Z = C[-1]
    t = mpmath.mpf(float(uniform)) * Z
    tok = next(v for v in range(len(C)) if C[v] > t)
    margin = min(abs(C[v] - t) for v in range(len(C))) / Z
    return tok, float(margin)


def walk(W1, W2, base, anchor, T=0.0, uniforms=None, Q=None, scale=None, single=False):
    """Greedy or sampled walk of one request.  Returns (tokens, logits bits, min sampling margin)."""
    gamma = base.shape[0]
    prev = int(anchor)
    toks, logits, margin = [], [], 1.0
    for k in range(gamma):
        u = [value(W1[prev, j]) for j in range(W1.shape[1])]
        lb = step_logits(W2, u, base[k], Q, scale, single)
        if T == 0.0:
            tok = argmax_lowest(lb)
        else:
            tok, m = sample_exact(lb, T, uniforms[k])
            margin = min(margin, m)
        toks.append(tok)
        logits.append(lb)
        prev = tok
    return toks, logits, margin


def gumbel_uniform(philox_words, v):
    """U of vocabulary row v from the four Philox words of its group of four rows:
    the odd multiple (2 (w >> 9) + 1) 2^-24 of 2^-24, as an exact rational."""
    w = int(philox_words[v % 4])
    return Fraction(2 * (w >> 9) + 1, 2 ** 24)


def gumbel_exact(logit_bits, T, U):
    """Gumbel-max at 60 digits: (token, gap between the two largest scores)."""
    sc = []
    for x, u in zip(logit_bits, U):
        l = mpmath.mpf(value(x).numerator) / value(x).denominator
        uu = mpmath.mpf(u.numerator) / u.denominator
        sc.append(l / mpmath.mpf(float(T)) - mpmath.log(-mpmath.log(uu)))
    best = 0
    for v in range(1, len(sc)):
        if sc[v] > sc[best]:
            best = v
    rest = [s for v, s in enumerate(sc) if v != best]
    gap = float(sc[best] - max(rest)) if rest else 1.0
    return best, gap
