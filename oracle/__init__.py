"""CPU oracle for DSpark's serial Markov draft walk -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``serial_draft_head_amd``) never imports it and shares no code with it.

The arithmetic lives in ``walk_oracle.c`` (plain C, binary64, OpenMP over
vocabulary rows).  This module only compiles it with gcc, loads it with
ctypes and converts numpy arrays.  bf16 tensors are passed as ``uint16`` bit
patterns.

What it computes (see the header of walk_oracle.c for the passages followed):
"Keeping the Draft Walk on Chip" (tie-pilot-qxw.github.io), section
"The serial part of a parallel drafter": ``u = W1[prev]``,
``logit = bf16(base + bf16(W2 @ u))``, argmax or a sample of
``softmax(logit / T)``, ``prev = tok``; the sampler is the inverse CDF of
vLLM PR #64442, section "Details", or (the ``gumbel`` mode) Gumbel-max from
counter-based noise, the pages' small-batch sampler (section "The idea: make
the walk resident").  ``walk_gru`` is the GRU serial head (section "Beyond
DSpark: other serial heads"): the state goes through a standard GRU cell fed
with ``W1[prev]`` and the vocabulary matrix reads ``bf16(h)``; ``walk_rnn``
the tanh RNN head and ``walk_gated`` DSpark's gated head (read as a convex gate
between the state and ``W1[prev]``, the gate computed from the state by one
int8 matrix).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "walk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile walk_oracle.c into liboracle.so with gcc (IEEE binary64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i, f = ctypes.c_int, ctypes.c_float
    lib.oracle_rne_bf16.restype = ctypes.c_double
    lib.oracle_rne_bf16.argtypes = [ctypes.c_double]
    lib.oracle_rne_bf16_array.restype = None
    lib.oracle_rne_bf16_array.argtypes = [P, P, P, ctypes.c_long]
    lib.oracle_step.restype = i
    lib.oracle_step.argtypes = [i, i, P, P, P, P, P, f, f, P, i]
    lib.oracle_sample.restype = i
    lib.oracle_sample.argtypes = [i, P, f, f]
    lib.oracle_walk.restype = i
    lib.oracle_walk.argtypes = [i, i, i, i, P, P, P, P, P, P, P, P, P, P, P, i]
    lib.oracle_walk_ex.restype = i
    lib.oracle_walk_ex.argtypes = [i, i, i, i, P, P, P, P, P, P, P, P, P, P, P, i,
                                   ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_gumbel_uniform.restype = ctypes.c_double
    lib.oracle_gumbel_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i, i, i]
    lib.oracle_gumbel_scores.restype = i
    lib.oracle_gumbel_scores.argtypes = [i, P, f, ctypes.c_uint64, ctypes.c_uint32, i, i, P]
    lib.oracle_gumbel_from_uniforms.restype = i
    lib.oracle_gumbel_from_uniforms.argtypes = [i, P, ctypes.c_double, P]
    lib.oracle_gru_cell.restype = None
    lib.oracle_gru_cell.argtypes = [i, P, P, P, P, P, P, P]
    lib.oracle_walk_gru.restype = i
    lib.oracle_walk_gru.argtypes = [i, i, i, i] + [P] * 18 + [i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_rnn_cell.restype = None
    lib.oracle_rnn_cell.argtypes = [i, P, P, P, P, P, P, P]
    lib.oracle_walk_rnn.restype = i
    lib.oracle_walk_rnn.argtypes = [i, i, i, i] + [P] * 18 + [i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_gated_cell.restype = None
    lib.oracle_gated_cell.argtypes = [i, P, P, P, P, P, P]
    lib.oracle_walk_gated.restype = i
    lib.oracle_gru_cell_in.restype = None
    lib.oracle_gru_cell_in.argtypes = [i, i, P, P, P, P, P, P, P]
    lib.oracle_walk_domino.restype = i
    lib.oracle_walk_domino.argtypes = [i, i, i, i, i] + [P] * 19 + [i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_walk_gated.argtypes = [i, i, i, i] + [P] * 17 + [i, ctypes.c_uint64, ctypes.c_uint32]
    lib.oracle_threads.restype = i
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_device_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i, i, P]
    lib.oracle_device_uniforms.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [i]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def rne_bf16(x):
    """Round float64 values to bf16, ties to even.  Returns (values f64, bits u16)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    bits = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_rne_bf16_array(_ptr(x), _ptr(y), _ptr(bits), x.size)
    return y, bits


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns (a plain reinterpretation)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


SINGLE_ROUND = 1  # mode bit: logit = bf16(base + dot), rounded once
GUMBEL = 2        # mode bit: sampled requests draw by Gumbel-max from counter-based noise


def step(u_bits, base_bits, T, uniform, W2_bits=None, Q=None, scale=None, single_round=False):
    """One step for one request.  Returns (token, logits_bits[V]).  single_round:
    the sum base + dot is rounded to bf16 once (default: the dot first, then the sum)."""
    u_bits = _c(u_bits, np.uint16)
    base_bits = _c(base_bits, np.uint16)
    W2_bits, Q, scale = _c(W2_bits, np.uint16), _c(Q, np.int8), _c(scale, np.float32)
    V = base_bits.shape[0]
    r = u_bits.shape[0]
    out = np.empty(V, dtype=np.uint16)
    tok = _load().oracle_step(V, r, _ptr(u_bits), _ptr(W2_bits), _ptr(Q), _ptr(scale),
                              _ptr(base_bits), float(T), float(uniform), _ptr(out),
                              SINGLE_ROUND if single_round else 0)
    if tok < 0:
        raise RuntimeError(f"oracle_step failed with {tok}")
    return tok, out


def sample(logits_bits, T, uniform) -> int:
    """Inverse-CDF draw over softmax(logits / T) for given bf16 logits."""
    lb = _c(logits_bits, np.uint16)
    tok = _load().oracle_sample(lb.shape[0], _ptr(lb), float(T), float(uniform))
    if tok < 0:
        raise RuntimeError(f"oracle_sample failed with {tok}")
    return tok


def walk(W1_bits, base_bits, anchor, T, uniforms=None, W2_bits=None, Q=None, scale=None,
         forced=None, want_logits=True, single_round=False, gumbel=False, seed=0, round_counter=0):
    """The whole walk.  Shapes: W1 [V,r] u16, W2 [V,r] u16 (or Q [V,r] i8 + scale [V] f32),
    base [B,gamma,V] u16, anchor [B] i32, T [B] f32, uniforms [B,gamma] f32 or None,
    forced [B,gamma] i32 or None (teacher forcing: step k>0 uses forced[:,k-1] as prev).
    gumbel: sampled requests draw by Gumbel-max from the noise of `seed` and the
    device round counter `round_counter` (uniforms are then not used).

    Returns (tokens [B,gamma] i32, logits [B,gamma,V] u16 or None)."""
    W1_bits = _c(W1_bits, np.uint16)
    W2_bits, Q, scale = _c(W2_bits, np.uint16), _c(Q, np.int8), _c(scale, np.float32)
    base_bits = _c(base_bits, np.uint16)
    anchor = _c(anchor, np.int32)
    T = _c(T, np.float32)
    uniforms = _c(uniforms, np.float32)
    forced = _c(forced, np.int32)
    V, r = W1_bits.shape
    B, gamma = base_bits.shape[0], base_bits.shape[1]
    assert base_bits.shape[2] == V
    tokens = np.empty((B, gamma), dtype=np.int32)
    logits = np.empty((B, gamma, V), dtype=np.uint16) if want_logits else None
    mode = (SINGLE_ROUND if single_round else 0) | (GUMBEL if gumbel else 0)
    rc = _load().oracle_walk_ex(V, r, B, gamma, _ptr(W1_bits), _ptr(W2_bits), _ptr(Q), _ptr(scale),
                                _ptr(base_bits), _ptr(anchor), _ptr(T), _ptr(uniforms),
                                _ptr(forced), _ptr(tokens), _ptr(logits), mode,
                                int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF)
    if rc != 0:
        raise RuntimeError(f"oracle_walk failed with {rc}")
    return tokens, logits


def philox4x32_10(ctr, key):
    """Philox-4x32-10 of a 4-word counter and a 2-word key (4 output words)."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def device_uniforms(seed: int, round_counter: int, B: int, gamma: int):
    """[B, gamma] f32: the uniforms a walk draws on the device from `seed`
    when the handle's round counter is `round_counter`."""
    out = np.empty((B, gamma), dtype=np.float32)
    _load().oracle_device_uniforms(int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF,
                                   int(B), int(gamma), _ptr(out))
    return out


def gumbel_uniform(seed: int, round_counter: int, b: int, k: int, v: int) -> float:
    """The Gumbel-max noise uniform U in (0, 1) of vocabulary row v, request b, step k."""
    return _load().oracle_gumbel_uniform(int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF,
                                         int(b), int(k), int(v))


def gumbel_scores(logits_bits, T, seed: int, round_counter: int, b: int, k: int):
    """f64 perturbed scores logit / T - ln(-ln U) of one request and step, for given bf16 logits."""
    lb = _c(logits_bits, np.uint16)
    out = np.empty(lb.shape[0], dtype=np.float64)
    rc = _load().oracle_gumbel_scores(lb.shape[0], _ptr(lb), float(T), int(seed) & (2 ** 64 - 1),
                                      int(round_counter) & 0xFFFFFFFF, int(b), int(k), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_gumbel_scores failed with {rc}")
    return out


def gumbel_from_uniforms(logits, T, U) -> int:
    """Gumbel-max draw over f64 logits with given uniforms U in (0, 1)."""
    lg = _c(logits, np.float64)
    u = _c(U, np.float64)
    tok = _load().oracle_gumbel_from_uniforms(lg.shape[0], _ptr(lg), float(T), _ptr(u))
    if tok < 0:
        raise RuntimeError(f"oracle_gumbel_from_uniforms failed with {tok}")
    return tok


def gru_cell(x, h, Wih_bits, Whh_bits, bih, bhh):
    """One GRU cell in binary64: x, h [r] -> h' [r]; Wih, Whh [3r, r] bf16 bits
    (gates r, z, n), bih, bhh [3r] f32."""
    x = _c(x, np.float64)
    h = _c(h, np.float64)
    r = x.shape[0]
    Wih_bits, Whh_bits = _c(Wih_bits, np.uint16), _c(Whh_bits, np.uint16)
    bih, bhh = _c(bih, np.float32), _c(bhh, np.float32)
    assert Wih_bits.shape == (3 * r, r) and Whh_bits.shape == (3 * r, r) and h.shape == (r,)
    out = np.empty(r, dtype=np.float64)
    _load().oracle_gru_cell(r, _ptr(x), _ptr(h), _ptr(Wih_bits), _ptr(Whh_bits), _ptr(bih), _ptr(bhh),
                            _ptr(out))
    return out


def rnn_cell(x, h, Wih_bits, Whh_bits, bih, bhh):
    """One tanh RNN cell in binary64: x, h [r] -> tanh(Wih x + bih + Whh h + bhh) [r];
    Wih, Whh [r, r] bf16 bits, bih, bhh [r] f32."""
    x = _c(x, np.float64)
    h = _c(h, np.float64)
    r = x.shape[0]
    Wih_bits, Whh_bits = _c(Wih_bits, np.uint16), _c(Whh_bits, np.uint16)
    bih, bhh = _c(bih, np.float32), _c(bhh, np.float32)
    assert Wih_bits.shape == (r, r) and Whh_bits.shape == (r, r) and h.shape == (r,)
    out = np.empty(r, dtype=np.float64)
    _load().oracle_rnn_cell(r, _ptr(x), _ptr(h), _ptr(Wih_bits), _ptr(Whh_bits), _ptr(bih), _ptr(bhh),
                            _ptr(out))
    return out


def gated_cell(x, h, Gq, gs, gb):
    """One step of the gated head in binary64: x, h [r] -> g h + (1 - g) x with
    g = sigmoid(gs * (Gq @ h) + gb); Gq [r, r] int8 codes, gs, gb [r] f32."""
    x = _c(x, np.float64)
    h = _c(h, np.float64)
    r = x.shape[0]
    Gq, gs, gb = _c(Gq, np.int8), _c(gs, np.float32), _c(gb, np.float32)
    assert Gq.shape == (r, r) and gs.shape == (r,) and gb.shape == (r,) and h.shape == (r,)
    out = np.empty(r, dtype=np.float64)
    _load().oracle_gated_cell(r, _ptr(x), _ptr(h), _ptr(Gq), _ptr(gs), _ptr(gb), _ptr(out))
    return out


def walk_gated(W1_bits, base_bits, anchor, T, gate, h0, uniforms=None, W2_bits=None, Q=None, scale=None,
               forced=None, forced_h=None, want_logits=True, single_round=False, gumbel=False, seed=0,
               round_counter=0):
    """The gated head's walk.  gate = (Gq [r,r] int8, gs [r] f32, gb [r] f32); the
    other arguments and the result as walk_gru."""
    W1_bits = _c(W1_bits, np.uint16)
    W2_bits, Q, scale = _c(W2_bits, np.uint16), _c(Q, np.int8), _c(scale, np.float32)
    Gq, gs, gb = _c(gate[0], np.int8), _c(gate[1], np.float32), _c(gate[2], np.float32)
    h0 = _c(h0, np.float32)
    base_bits = _c(base_bits, np.uint16)
    anchor, T = _c(anchor, np.int32), _c(T, np.float32)
    uniforms, forced, forced_h = _c(uniforms, np.float32), _c(forced, np.int32), _c(forced_h, np.float32)
    V, r = W1_bits.shape
    B, gamma = base_bits.shape[0], base_bits.shape[1]
    assert base_bits.shape[2] == V and h0.shape == (B, r) and Gq.shape == (r, r)
    tokens = np.empty((B, gamma), dtype=np.int32)
    logits = np.empty((B, gamma, V), dtype=np.uint16) if want_logits else None
    states = np.empty((B, gamma, r), dtype=np.float64)
    mode = (SINGLE_ROUND if single_round else 0) | (GUMBEL if gumbel else 0)
    rc = _load().oracle_walk_gated(V, r, B, gamma, _ptr(W1_bits), _ptr(W2_bits), _ptr(Q), _ptr(scale),
                                   _ptr(Gq), _ptr(gs), _ptr(gb), _ptr(h0), _ptr(base_bits),
                                   _ptr(anchor), _ptr(T), _ptr(uniforms), _ptr(forced), _ptr(forced_h),
                                   _ptr(tokens), _ptr(logits), _ptr(states), mode,
                                   int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF)
    if rc != 0:
        raise RuntimeError(f"oracle_walk_gated failed with {rc}")
    return tokens, logits, states


def gru_cell_in(x, h, Wih_bits, Whh_bits, bih, bhh):
    """The GRU cell with an input wider than the state: x [in], h [r];
    Wih [3r, in], Whh [3r, r] bf16 bits, bih, bhh [3r] f32."""
    x = _c(x, np.float64)
    h = _c(h, np.float64)
    r, n_in = h.shape[0], x.shape[0]
    Wih_bits, Whh_bits = _c(Wih_bits, np.uint16), _c(Whh_bits, np.uint16)
    bih, bhh = _c(bih, np.float32), _c(bhh, np.float32)
    assert Wih_bits.shape == (3 * r, n_in) and Whh_bits.shape == (3 * r, r)
    out = np.empty(r, dtype=np.float64)
    _load().oracle_gru_cell_in(r, n_in, _ptr(x), _ptr(h), _ptr(Wih_bits), _ptr(Whh_bits), _ptr(bih), _ptr(bhh),
                               _ptr(out))
    return out


def walk_domino(W1_bits, base_bits, anchor, T, cell, H_bits, h0, uniforms=None, W2_bits=None, Q=None,
                scale=None, forced=None, forced_h=None, want_logits=True, single_round=False, gumbel=False,
                seed=0, round_counter=0):
    """Domino's head: the GRU walk with the drafter's hidden states appended to
    every step's input.  cell = (Wih [3r, r+d] u16, Whh [3r, r] u16, bih, bhh
    [3r] f32); H_bits [B, gamma, d] bf16 bits; otherwise as walk_gru."""
    W1_bits = _c(W1_bits, np.uint16)
    W2_bits, Q, scale = _c(W2_bits, np.uint16), _c(Q, np.int8), _c(scale, np.float32)
    Wih, Whh, bih, bhh = _c(cell[0], np.uint16), _c(cell[1], np.uint16), _c(cell[2], np.float32), \
        _c(cell[3], np.float32)
    H_bits = _c(H_bits, np.uint16)
    h0 = _c(h0, np.float32)
    base_bits = _c(base_bits, np.uint16)
    anchor, T = _c(anchor, np.int32), _c(T, np.float32)
    uniforms, forced, forced_h = _c(uniforms, np.float32), _c(forced, np.int32), _c(forced_h, np.float32)
    V, r = W1_bits.shape
    B, gamma = base_bits.shape[0], base_bits.shape[1]
    d = H_bits.shape[2]
    assert base_bits.shape[2] == V and h0.shape == (B, r) and H_bits.shape[:2] == (B, gamma)
    assert Wih.shape == (3 * r, r + d)
    tokens = np.empty((B, gamma), dtype=np.int32)
    logits = np.empty((B, gamma, V), dtype=np.uint16) if want_logits else None
    states = np.empty((B, gamma, r), dtype=np.float64)
    mode = (SINGLE_ROUND if single_round else 0) | (GUMBEL if gumbel else 0)
    rc = _load().oracle_walk_domino(V, r, d, B, gamma, _ptr(W1_bits), _ptr(W2_bits), _ptr(Q), _ptr(scale),
                                    _ptr(Wih), _ptr(Whh), _ptr(bih), _ptr(bhh), _ptr(H_bits), _ptr(h0),
                                    _ptr(base_bits), _ptr(anchor), _ptr(T), _ptr(uniforms), _ptr(forced),
                                    _ptr(forced_h), _ptr(tokens), _ptr(logits), _ptr(states), mode,
                                    int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF)
    if rc != 0:
        raise RuntimeError(f"oracle_walk_domino failed with {rc}")
    return tokens, logits, states


def walk_rnn(W1_bits, base_bits, anchor, T, cell, h0, **kw):
    """The RNN head's walk: as walk_gru with cell = (Wih [r,r] u16, Whh [r,r] u16, bih [r], bhh [r])."""
    return walk_gru(W1_bits, base_bits, anchor, T, cell, h0, _fn="oracle_walk_rnn", **kw)


def walk_gru(W1_bits, base_bits, anchor, T, cell, h0, uniforms=None, W2_bits=None, Q=None, scale=None,
             forced=None, forced_h=None, want_logits=True, single_round=False, gumbel=False, seed=0,
             round_counter=0, _fn="oracle_walk_gru"):
    """The GRU head's walk.  cell = (Wih [3r,r] u16, Whh [3r,r] u16, bih [3r] f32, bhh [3r] f32);
    h0 [B,r] f32; forced_h [B,gamma,r] f32 or None (teacher forcing of the state).
    Returns (tokens [B,gamma] i32, logits [B,gamma,V] u16 or None, states [B,gamma,r] f64)."""
    W1_bits = _c(W1_bits, np.uint16)
    W2_bits, Q, scale = _c(W2_bits, np.uint16), _c(Q, np.int8), _c(scale, np.float32)
    Wih, Whh, bih, bhh = _c(cell[0], np.uint16), _c(cell[1], np.uint16), _c(cell[2], np.float32), \
        _c(cell[3], np.float32)
    h0 = _c(h0, np.float32)
    base_bits = _c(base_bits, np.uint16)
    anchor, T = _c(anchor, np.int32), _c(T, np.float32)
    uniforms, forced, forced_h = _c(uniforms, np.float32), _c(forced, np.int32), _c(forced_h, np.float32)
    V, r = W1_bits.shape
    B, gamma = base_bits.shape[0], base_bits.shape[1]
    assert base_bits.shape[2] == V and h0.shape == (B, r)
    tokens = np.empty((B, gamma), dtype=np.int32)
    logits = np.empty((B, gamma, V), dtype=np.uint16) if want_logits else None
    states = np.empty((B, gamma, r), dtype=np.float64)
    mode = (SINGLE_ROUND if single_round else 0) | (GUMBEL if gumbel else 0)
    rc = getattr(_load(), _fn)(V, r, B, gamma, _ptr(W1_bits), _ptr(W2_bits), _ptr(Q), _ptr(scale),
                                 _ptr(Wih), _ptr(Whh), _ptr(bih), _ptr(bhh), _ptr(h0), _ptr(base_bits),
                                 _ptr(anchor), _ptr(T), _ptr(uniforms), _ptr(forced), _ptr(forced_h),
                                 _ptr(tokens), _ptr(logits), _ptr(states), mode,
                                 int(seed) & (2 ** 64 - 1), int(round_counter) & 0xFFFFFFFF)
    if rc != 0:
        raise RuntimeError(f"{_fn} failed with {rc}")
    return tokens, logits, states
