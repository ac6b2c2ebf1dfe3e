"""MI355X-native serial Markov draft walk (DSpark's head): Python binding.

This module only marshals arguments into the C ABI of ``include/dsw.h``
(``libdsw.so``, built in-tree by ``serial_draft_head_amd.build``).  Every step
of the walk runs in the library's HIP kernels; PyTorch supplies device memory
and the stream.  Importing works without a GPU (the planner and the error
strings are host code); calling ``walk`` needs the built library and a GPU,
and raises if either is missing -- there is no fallback.

The walk (from "Keeping the Draft Walk on Chip", tie-pilot-qxw.github.io,
section "The serial part of a parallel drafter"): for k < gamma,
``u = W1[prev]``, ``logit = bf16(base[:, k] + bf16(W2 @ u))``, then the
lowest-index argmax (T == 0) or an inverse-CDF sample of ``softmax(logit / T)``
driven by ``uniforms[:, k]``, and ``prev = tok``.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import threading
import weakref

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsw.so")

OK = 0
ERR = {
    -1: "DSW_ERR_NULL", -2: "DSW_ERR_BATCH", -3: "DSW_ERR_GAMMA", -4: "DSW_ERR_RANK",
    -5: "DSW_ERR_DTYPE", -6: "DSW_ERR_VOCAB", -7: "DSW_ERR_LAUNCH", -8: "DSW_ERR_HIP",
    -9: "DSW_ERR_DEVICE", -10: "DSW_ERR_PLAN", -11: "DSW_ERR_ARG", -12: "DSW_ERR_SCRATCH",
    -20: "DSW_ERR_DEV_TIMEOUT", -21: "DSW_ERR_DEV_TOKEN", -22: "DSW_ERR_DEV_UNIFORMS",
}
BF16, INT8 = 0, 1
PATH_RESIDENT, PATH_PARTIAL = 0, 1
FLAG_FORCE_STREAM = 1
FLAG_COOPERATIVE = 2
FLAG_VALU_GEMV = 4
FLAG_MFMA_GEMV = 8
FLAG_BATCHED = 16
FLAG_SINGLE_ROUND = 32
FLAG_GUMBEL = 64
FLAG_GRU = 128
FLAG_RNN = 256
FLAG_GATED = 512
FLAG_DOMINO = 1024
ENGINE_VALU, ENGINE_MFMA = 0, 1
RANK = 256


class DswError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERR.get(code, code)} ({strerror(code)})")


class DevInfo(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_int), ("simds_per_cu", ctypes.c_int),
                ("wave_size", ctypes.c_int), ("vgprs_per_simd_lane", ctypes.c_int),
                ("lds_bytes_per_cu", ctypes.c_int), ("max_lds_per_block", ctypes.c_int),
                ("xcd_count", ctypes.c_int), ("clock_khz", ctypes.c_int),
                ("l2_bytes", ctypes.c_longlong), ("hbm_bytes", ctypes.c_longlong),
                ("cooperative", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("grid", ctypes.c_int), ("block", ctypes.c_int),
                ("rows_per_wg", ctypes.c_int), ("reg_slots", ctypes.c_int),
                ("reg_rows", ctypes.c_int), ("lds_rows", ctypes.c_int),
                ("stream_rows", ctypes.c_int), ("batch_tile", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("onchip_bytes", ctypes.c_longlong),
                ("stream_bytes", ctypes.c_longlong), ("workspace_bytes", ctypes.c_longlong),
                ("engine", ctypes.c_int), ("tiles_per_wave", ctypes.c_int),
                ("reg_tiles", ctypes.c_int), ("lds_tiles", ctypes.c_int),
                ("max_tiles", ctypes.c_int), ("static_lds_bytes", ctypes.c_int),
                ("w2_dtype", ctypes.c_int), ("ring_slots", ctypes.c_int),
                ("rows_pad", ctypes.c_int), ("prefetch_tiles", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded libdsw.so.  Raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
        L.dsw_device_info.argtypes = [I, ctypes.POINTER(DevInfo)]
        L.dsw_plan_compute.argtypes = [ctypes.POINTER(DevInfo), I, I, I, I, I, U,
                                       ctypes.POINTER(PlanInfo)]
        L.dsw_create.argtypes = [ctypes.POINTER(P), I, I, I, I, I, I, U]
        L.dsw_walk.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, P]
        L.dsw_walk_gru.argtypes = [P] * 15 + [I, I, P]
        L.dsw_walk_rnn.argtypes = [P] * 15 + [I, I, P]
        L.dsw_walk_gated.argtypes = [P] * 14 + [I, I, P]
        L.dsw_walk_domino.argtypes = [P] * 9 + [I] + [P] * 7 + [I, I, P]
        L.dsw_status.argtypes = [P]
        L.dsw_query_plan.argtypes = [P, I, ctypes.POINTER(PlanInfo)]
        L.dsw_destroy.argtypes = [P]
        L.dsw_strerror.argtypes = [I]
        L.dsw_strerror.restype = ctypes.c_char_p
        L.dsw_set_seed.argtypes = [P, ctypes.c_ulonglong, I]
        L.dsw_round_counter.argtypes = [P, ctypes.POINTER(ctypes.c_uint)]
        L.dsw_set_trace.argtypes = [P, P, ctypes.c_longlong]
        L.dsw_set_debug.argtypes = [P, U, U]
        L.dsw_set_round_counter.argtypes = [P, U]
        L.dsw_set_grid.argtypes = [P, I]
        L.dsw_debug_epoch.argtypes = [U]
        L.dsw_debug_epoch.restype = U
        L.dsw_debug_gumbel_table.argtypes = [P, P]
        L.dsw_walk_static.argtypes = [I, I, I, U] + [P] * 9 + [I, I, P]
        L.dsw_static_init.argtypes = [I]
        L.dsw_static_status.argtypes = [I]
        for f in ("dsw_device_info", "dsw_plan_compute", "dsw_create", "dsw_walk", "dsw_walk_gru", "dsw_walk_rnn",
                  "dsw_walk_gated", "dsw_walk_domino", "dsw_status", "dsw_query_plan", "dsw_destroy", "dsw_set_seed",
                  "dsw_round_counter", "dsw_set_trace", "dsw_set_debug", "dsw_set_round_counter", "dsw_set_grid",
                  "dsw_debug_gumbel_table", "dsw_walk_static", "dsw_static_init", "dsw_static_status"):
            getattr(L, f).restype = I
        _lib = L
        return L


def strerror(code: int) -> str:
    return lib().dsw_strerror(int(code)).decode()


def _check(code: int, where: str):
    if code != OK:
        raise DswError(code, where)


def device_info(device: int = 0) -> DevInfo:
    d = DevInfo()
    _check(lib().dsw_device_info(int(device), ctypes.byref(d)), "dsw_device_info")
    return d


def plan(dev: DevInfo, V: int, gamma: int, B: int, w2_dtype: int = BF16, flags: int = 0,
         r: int = RANK) -> PlanInfo:
    """The planner's decision for an (invented or real) device.  Host only."""
    out = PlanInfo()
    _check(lib().dsw_plan_compute(ctypes.byref(dev), int(V), int(r), int(gamma), int(B),
                                  int(w2_dtype), int(flags), ctypes.byref(out)),
           "dsw_plan_compute")
    return out


def _stream_handle(torch, device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def debug_epoch(seq: int) -> int:
    """The epoch a mailbox word carries at step sequence number seq (host only)."""
    return int(lib().dsw_debug_epoch(ctypes.c_uint(int(seq) & 0xFFFFFFFF)))


def debug_gumbel_table(out, stream=None) -> None:
    """out: float32 device tensor of 2^23 elements; fills it with the kernels'
    Gumbel variate -ln(-ln U) for U = (2 i + 1) 2^-24 (dsw_debug_gumbel_table)."""
    import torch
    if out.dtype != torch.float32 or out.numel() != 1 << 23 or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out: want a contiguous float32 device tensor of 2^23 elements")
    _check(lib().dsw_debug_gumbel_table(ctypes.c_void_p(out.data_ptr()),
                                        _stream_handle(torch, out.device, stream)), "dsw_debug_gumbel_table")


# Handles still open when the interpreter exits are destroyed by an atexit
# hook, which runs before the HIP runtime (and any profiler attached to the
# process) is torn down; finalizers that run later, during interpreter
# shutdown, do nothing.
_open_walkers = weakref.WeakSet()


def _close_all():
    for w in list(_open_walkers):
        try:
            w.close()
        except Exception:
            pass
    _walkers.clear()


atexit.register(_close_all)


class Walker:
    """A handle of the library: workspace for walks of vocabulary V with at
    most gamma_max steps and B_max requests on one device."""

    def __init__(self, V: int, gamma_max: int, B_max: int, w2_dtype: int = BF16,
                 device: int = 0, flags: int = 0, r: int = RANK):
        self.V, self.gamma_max, self.B_max = int(V), int(gamma_max), int(B_max)
        self.w2_dtype, self.device, self.flags, self.r = int(w2_dtype), int(device), int(flags), r
        h = ctypes.c_void_p()
        _check(lib().dsw_create(ctypes.byref(h), self.device, self.V, int(r), self.gamma_max,
                                self.B_max, self.w2_dtype, int(flags)), "dsw_create")
        self._h = h
        _open_walkers.add(self)

    def close(self):
        """Destroy the handle (waits for its device).  Idempotent."""
        if getattr(self, "_h", None):
            h, self._h = self._h, None
            lib().dsw_destroy(h)
        _open_walkers.discard(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self, _finalizing=sys.is_finalizing):
        # during interpreter shutdown the atexit hook has already closed every
        # handle; never call into the runtime from a late finalizer (the
        # default argument keeps the check usable after module globals are
        # cleared)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def set_debug(self, spin_limit: int = 0, skew: int = 0) -> None:
        """Diagnostics (dsw_set_debug): polls before a device wait gives up (0 =
        the default), and pseudo-random delays before every post (0 = none)."""
        _check(lib().dsw_set_debug(self._h, ctypes.c_uint(int(spin_limit)), ctypes.c_uint(int(skew))),
               "dsw_set_debug")

    def set_grid(self, grid: int) -> None:
        """dsw_set_grid: later walks use `grid` workgroups (0 = one per CU)."""
        _check(lib().dsw_set_grid(self._h, int(grid)), "dsw_set_grid")

    def set_round_counter(self, value: int) -> None:
        """Test hook (dsw_set_round_counter): waits for the device, then sets the
        round counter and the launch counters of both kernel families."""
        _check(lib().dsw_set_round_counter(self._h, ctypes.c_uint(int(value) & 0xFFFFFFFF)),
               "dsw_set_round_counter")

    def query_plan(self, B: int) -> PlanInfo:
        out = PlanInfo()
        _check(lib().dsw_query_plan(self._h, int(B), ctypes.byref(out)), "dsw_query_plan")
        return out

    def set_seed(self, seed: int, enable: bool = True) -> None:
        """Walks with uniforms=None draw their uniforms on the device (dsw_set_seed)."""
        _check(lib().dsw_set_seed(self._h, ctypes.c_ulonglong(int(seed) & (2 ** 64 - 1)), int(bool(enable))),
               "dsw_set_seed")

    def round_counter(self) -> int:
        """The device round counter (waits for the device)."""
        out = ctypes.c_uint(0)
        _check(lib().dsw_round_counter(self._h, ctypes.byref(out)), "dsw_round_counter")
        return int(out.value)

    def status(self) -> int:
        """Wait for the device; return (and clear) the latched device status code."""
        return lib().dsw_status(self._h)

    def walk(self, W1, W2, base, anchor, T, uniforms=None, w2_scale=None, tokens=None,
             logits=None, want_logits=False, stream=None):
        """One round.  Tensors live on this handle's device:
        W1 bf16 [V,256]; W2 bf16 [V,256] (or int8 + w2_scale f32 [V]);
        base bf16 [B,gamma,V]; anchor int32 [B]; T float32 [B] (0 = greedy);
        uniforms float32 [B,gamma], or None when every T is 0 or after set_seed (drawn on the device).
        Returns (tokens int32 [B,gamma], logits bf16 [B,gamma,V] or None)."""
        import torch
        dev = torch.device("cuda", self.device)
        B, gamma, V = (int(x) for x in base.shape)
        need = [(W1, torch.bfloat16, (self.V, self.r), "W1"),
                (base, torch.bfloat16, (B, gamma, self.V), "base"),
                (anchor, torch.int32, (B,), "anchor"), (T, torch.float32, (B,), "T")]
        if self.w2_dtype == BF16:
            need.append((W2, torch.bfloat16, (self.V, self.r), "W2"))
        else:
            need.append((W2, torch.int8, (self.V, self.r), "W2"))
            need.append((w2_scale, torch.float32, (self.V,), "w2_scale"))
        if uniforms is not None:
            need.append((uniforms, torch.float32, (B, gamma), "uniforms"))
        if tokens is None:
            tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        need.append((tokens, torch.int32, (B, gamma), "tokens"))
        if logits is None and want_logits:
            logits = torch.empty((B, gamma, self.V), dtype=torch.bfloat16, device=dev)
        if logits is not None:
            need.append((logits, torch.bfloat16, (B, gamma, self.V), "logits"))
        for t, dt, shape, name in need:
            if t is None:
                raise ValueError(f"{name} is required")
            if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"{name}: want {dt} {shape} contiguous on {dev}, got "
                                 f"{t.dtype} {tuple(t.shape)} on {t.device}")
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        rc = lib().dsw_walk(self._h, ptr(W1), ptr(W2), ptr(w2_scale), ptr(base), ptr(anchor),
                            ptr(T), ptr(uniforms), ptr(tokens), ptr(logits), B, gamma,
                            _stream_handle(torch, dev, stream))
        _check(rc, "dsw_walk")
        return tokens, logits

    def walk_gru(self, W1, W2, cell, h0, base, anchor, T, uniforms=None, tokens=None, logits=None,
                 states=None, want_logits=False, want_states=False, stream=None):
        """One round of the GRU serial head (handle made with FLAG_GRU; one request).
        cell = (Wih bf16 [3r,r], Whh bf16 [3r,r], bih f32 [3r], bhh f32 [3r]); h0 f32 [r];
        other tensors as walk().  Returns (tokens [B,gamma], logits or None,
        states f32 [gamma, r] or None)."""
        return self._walk_cell(self._cell_spec(cell, 3), "dsw_walk_gru", W1, W2, cell, h0, base, anchor, T,
                               uniforms, tokens, logits, states, want_logits, want_states, stream)

    def walk_rnn(self, W1, W2, cell, h0, base, anchor, T, uniforms=None, tokens=None, logits=None,
                 states=None, want_logits=False, want_states=False, stream=None):
        """One round of the RNN serial head (handle made with FLAG_RNN; one request).
        cell = (Wih bf16 [r,r], Whh bf16 [r,r], bih f32 [r], bhh f32 [r]); as walk_gru otherwise."""
        return self._walk_cell(self._cell_spec(cell, 1), "dsw_walk_rnn", W1, W2, cell, h0, base, anchor, T,
                               uniforms, tokens, logits, states, want_logits, want_states, stream)

    def walk_gated(self, W1, W2, gate, h0, base, anchor, T, uniforms=None, tokens=None, logits=None,
                   states=None, want_logits=False, want_states=False, stream=None):
        """One round of DSpark's gated serial head (handle made with FLAG_GATED; one
        request).  gate = (Gq int8 [r,r], gate_scale f32 [r], gate_bias f32 [r]):
        g = sigmoid(gate_scale * (Gq h) + gate_bias), h = g h + (1 - g) W1[prev];
        as walk_gru otherwise."""
        import torch
        r = self.r
        spec = [(gate[0], torch.int8, (r, r), "Gq"), (gate[1], torch.float32, (r,), "gate_scale"),
                (gate[2], torch.float32, (r,), "gate_bias")]
        return self._walk_cell(spec, "dsw_walk_gated", W1, W2, gate, h0, base, anchor, T, uniforms, tokens,
                               logits, states, want_logits, want_states, stream)

    def walk_domino(self, W1, W2, cell, H, h0, base, anchor, T, uniforms=None, tokens=None, logits=None,
                    states=None, want_logits=False, want_states=False, stream=None):
        """One round of Domino's serial head (handle made with FLAG_DOMINO; one
        request): the GRU head whose input at step k is [W1[prev]; H[k]].
        cell = (Wih bf16 [3r, r+d], Whh bf16 [3r, r], bih f32 [3r], bhh f32 [3r]);
        H bf16 [gamma, d]; as walk_gru otherwise."""
        import torch
        r = self.r
        gamma, d = int(base.shape[1]), int(H.shape[-1])
        spec = [(cell[0], torch.bfloat16, (3 * r, r + d), "Wih"), (cell[1], torch.bfloat16, (3 * r, r), "Whh"),
                (cell[2], torch.float32, (3 * r,), "bih"), (cell[3], torch.float32, (3 * r,), "bhh")]
        return self._walk_cell(spec, "dsw_walk_domino", W1, W2, cell, h0, base, anchor, T, uniforms, tokens,
                               logits, states, want_logits, want_states, stream,
                               after_h0=[(H, torch.bfloat16, (gamma, d), "H")], after_h0_ints=[d])

    def _cell_spec(self, cell, gates):
        import torch
        r = self.r
        return [(cell[0], torch.bfloat16, (gates * r, r), "Wih"), (cell[1], torch.bfloat16, (gates * r, r), "Whh"),
                (cell[2], torch.float32, (gates * r,), "bih"), (cell[3], torch.float32, (gates * r,), "bhh")]

    def _walk_cell(self, spec, fname, W1, W2, cell, h0, base, anchor, T, uniforms, tokens, logits,
                   states, want_logits, want_states, stream, after_h0=(), after_h0_ints=()):
        import torch
        dev = torch.device("cuda", self.device)
        B, gamma, V = (int(x) for x in base.shape)
        r = self.r
        need = [(W1, torch.bfloat16, (self.V, r), "W1"), (W2, torch.bfloat16, (self.V, r), "W2")] + spec + [
                (h0, torch.float32, (r,), "h0")] + list(after_h0) + [
                (base, torch.bfloat16, (B, gamma, self.V), "base"),
                (anchor, torch.int32, (B,), "anchor"), (T, torch.float32, (B,), "T")]
        if uniforms is not None:
            need.append((uniforms, torch.float32, (B, gamma), "uniforms"))
        if tokens is None:
            tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        need.append((tokens, torch.int32, (B, gamma), "tokens"))
        if logits is None and want_logits:
            logits = torch.empty((B, gamma, self.V), dtype=torch.bfloat16, device=dev)
        if logits is not None:
            need.append((logits, torch.bfloat16, (B, gamma, self.V), "logits"))
        if states is None and want_states:
            states = torch.empty((gamma, r), dtype=torch.float32, device=dev)
        if states is not None:
            need.append((states, torch.float32, (gamma, r), "states"))
        for t, dt, shape, name in need:
            if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"{name}: want {dt} {shape} contiguous on {dev}, got "
                                 f"{t.dtype} {tuple(t.shape)} on {t.device}")
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        rc = getattr(lib(), fname)(self._h, ptr(W1), ptr(W2), *[ptr(t[0]) for t in spec], ptr(h0),
                                   *[ptr(t[0]) for t in after_h0], *after_h0_ints, ptr(base), ptr(anchor), ptr(T), ptr(uniforms), ptr(tokens), ptr(logits),
                                   ptr(states), B, gamma, _stream_handle(torch, dev, stream))
        _check(rc, fname)
        return tokens, logits, states


_walkers = {}


def walk_static(W1, W2, base, anchor, T, uniforms=None, w2_scale=None, tokens=None, logits=None,
                want_logits=False, flags=0, stream=None):
    """One round through dsw_walk_static: no handle, no allocation in the
    library (its workspace is a static device array; outputs that are None
    are allocated here, by torch).  Tensors and results as Walker.walk; the
    device is W1's.  Calls on one GPU must not overlap."""
    import torch
    dev = W1.device
    B, gamma, V = (int(x) for x in base.shape)
    dtype = INT8 if W2.dtype == torch.int8 else BF16
    need = [(W1, torch.bfloat16, (V, RANK), "W1"), (base, torch.bfloat16, (B, gamma, V), "base"),
            (anchor, torch.int32, (B,), "anchor"), (T, torch.float32, (B,), "T")]
    if dtype == BF16:
        need.append((W2, torch.bfloat16, (V, RANK), "W2"))
    else:
        need.append((W2, torch.int8, (V, RANK), "W2"))
        need.append((w2_scale, torch.float32, (V,), "w2_scale"))
    if uniforms is not None:
        need.append((uniforms, torch.float32, (B, gamma), "uniforms"))
    if tokens is None:
        tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    need.append((tokens, torch.int32, (B, gamma), "tokens"))
    if logits is None and want_logits:
        logits = torch.empty((B, gamma, V), dtype=torch.bfloat16, device=dev)
    if logits is not None:
        need.append((logits, torch.bfloat16, (B, gamma, V), "logits"))
    for t, dt, shape, name in need:
        if t is None:
            raise ValueError(f"{name} is required")
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name}: want {dt} {shape} contiguous on {dev}, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device}")
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib().dsw_walk_static(int(dev.index or 0), V, dtype, int(flags), ptr(W1), ptr(W2), ptr(w2_scale),
                               ptr(base), ptr(anchor), ptr(T), ptr(uniforms), ptr(tokens), ptr(logits), B, gamma,
                               _stream_handle(torch, dev, stream))
    _check(rc, "dsw_walk_static")
    return tokens, logits


def static_init(device: int = 0) -> None:
    """dsw_static_init: set up dsw_walk_static on `device` (outside graph capture)."""
    _check(lib().dsw_static_init(int(device)), "dsw_static_init")


def static_status(device: int = 0) -> int:
    """dsw_static_status: wait, then return and clear the latched device status of dsw_walk_static."""
    return lib().dsw_static_status(int(device))


def walk(W1, W2, base, anchor, T, uniforms=None, w2_scale=None, want_logits=False, stream=None):
    """Functional form: one round with a cached handle per (device, V, dtype,
    stream).  A handle serves one stream at a time (its workspace and counters
    are not shared between concurrent walks), so walks on different streams
    get different handles."""
    import torch
    B, gamma, V = (int(x) for x in base.shape)
    device = W1.device.index if W1.device.index is not None else torch.cuda.current_device()
    dtype = INT8 if W2.dtype == torch.int8 else BF16
    sid = int((stream if stream is not None else torch.cuda.current_stream(device)).cuda_stream)
    key = (device, V, dtype, sid)
    w = _walkers.get(key)
    if w is None or w.gamma_max < gamma or w.B_max < B:
        if w is not None:
            w.close()
        w = Walker(V, max(gamma, 16), max(B, 16), dtype, device)
        _walkers[key] = w
    return w.walk(W1, W2, base, anchor, T, uniforms, w2_scale, want_logits=want_logits,
                  stream=stream)
