"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/dsw.h declares, and the planner behaves on invented
devices.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsw.h")


@pytest.fixture(scope="module")
def dsw():
    import serial_draft_head_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libdsw.so is not built (run __graft_entry__.build())")
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsw_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("dsw_create", "dsw_walk", "dsw_status", "dsw_query_plan", "dsw_destroy",
                 "dsw_strerror", "dsw_plan_compute", "dsw_device_info"):
        assert want in names


def test_library_exports_every_declared_function(dsw):
    lib = ctypes.CDLL(dsw.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_error_strings(dsw):
    for code in list(dsw.ERR) + [0]:
        s = dsw.strerror(code)
        assert s and s != "unknown error", code
    assert dsw.strerror(12345) == "unknown error"


def test_null_and_argument_errors_without_a_device(dsw):
    L = dsw.lib()
    assert L.dsw_walk(None, None, None, None, None, None, None, None, None, None, 1, 1, None) == -1
    assert L.dsw_status(None) == -1
    assert L.dsw_query_plan(None, 1, None) == -1
    assert L.dsw_destroy(None) == 0
    h = ctypes.c_void_p()
    assert L.dsw_create(None, 0, 100, 256, 7, 1, 0, 0) == -1
    assert L.dsw_create(ctypes.byref(h), 0, 100, 128, 7, 1, 0, 0) == -4      # rank
    assert L.dsw_create(ctypes.byref(h), 0, 100, 256, 7, 1, 7, 0) == -5      # dtype
    assert L.dsw_create(ctypes.byref(h), 0, 0, 256, 7, 1, 0, 0) == -6        # vocab
    assert L.dsw_create(ctypes.byref(h), 0, 100, 256, 0, 1, 0, 0) == -3      # gamma
    assert L.dsw_create(ctypes.byref(h), 0, 100, 256, 7, 0, 0, 0) == -2      # batch
    assert L.dsw_walk_gru(None, *([None] * 14), 1, 1, None) == -1
    assert L.dsw_walk_rnn(None, *([None] * 14), 1, 1, None) == -1
    assert L.dsw_walk_gated(None, *([None] * 13), 1, 1, None) == -1
    assert L.dsw_walk_domino(None, *([None] * 8), 64, *([None] * 7), 1, 1, None) == -1


def test_debug_and_test_hooks_without_a_handle(dsw):
    L = dsw.lib()
    assert L.dsw_set_debug(None, 1, 0) == -1
    assert L.dsw_set_round_counter(None, 5) == -1
    assert L.dsw_debug_gumbel_table(None, None) == -1
    h = ctypes.c_void_p()
    assert L.dsw_create(ctypes.byref(h), 0, 100, 256, 4097, 1, 0, 0) == -3  # gamma_max above 4096


EPOCH_PERIOD = 1 << 27


def test_epoch_range_and_period(dsw):
    """Epochs lie in [1, 2^27] (never the 0 of a cleared word) and repeat with
    period 2^27 in the step sequence number, which divides 2^32: the same
    sequence number mod 2^27 gives the same epoch, also across the 32-bit wrap."""
    rng = __import__("numpy").random.default_rng(7)
    seqs = [0, 1, EPOCH_PERIOD - 1, EPOCH_PERIOD, 2 ** 32 - 1, 2 ** 32 - 16, 2 ** 31] + \
        [int(x) for x in rng.integers(0, 2 ** 32, 200)]
    for s in seqs:
        e = dsw.debug_epoch(s)
        assert 1 <= e <= EPOCH_PERIOD, (s, e)
        assert e == (s % EPOCH_PERIOD) + 1
        assert dsw.debug_epoch((s + EPOCH_PERIOD) % 2 ** 32) == e
        assert dsw.debug_epoch((s + 1) % 2 ** 32) != e


@pytest.mark.parametrize("gamma_max", [1, 7, 16, 5, 4096])
def test_epochs_distinct_across_the_wrap(dsw, gamma_max):
    """Steps of consecutive launches around the 32-bit wrap of the sequence
    number s = n * gamma_max + k, and around the wrap of the counter n itself,
    carry pairwise distinct epochs (the reads of one launch only ever meet
    words of that launch or of the one before)."""
    for n0 in ((2 ** 32) // gamma_max - 2, 2 ** 32 - 2, 2 ** 28 - 2, 0):
        epochs = []
        for n in range(n0, n0 + 4):
            for k in range(gamma_max if gamma_max <= 64 else 64):
                epochs.append(dsw.debug_epoch(((n % 2 ** 32) * gamma_max + k) % 2 ** 32))
        # consecutive launches: 2 gamma_max steps never share an epoch
        for i in range(len(epochs)):
            window = epochs[i:i + 2 * min(gamma_max, 64)]
            assert len(set(window)) == len(window), (gamma_max, n0, i)


def fake_device(dsw, cus=256, lds_cu=160 * 1024, lds_blk=160 * 1024):
    d = dsw.DevInfo()
    d.cu_count, d.simds_per_cu, d.wave_size, d.vgprs_per_simd_lane = cus, 4, 64, 512
    d.lds_bytes_per_cu, d.max_lds_per_block, d.xcd_count = lds_cu, lds_blk, 8
    d.clock_khz, d.l2_bytes, d.hbm_bytes, d.cooperative = 2_400_000, 4 << 20, 288 << 30, 1
    return d


def shards_cover(V, grid, R):
    covered = 0
    for c in range(grid):
        lo, hi = c * R, min(V, c * R + R)
        if hi > lo:
            assert lo == covered
            covered = hi
    return covered == V


def test_planner_follows_a_reduced_grid(dsw):
    """dsw_set_grid hands the planner a device with fewer CUs: shards grow to
    ceil(V / grid) rows, up to what one workgroup holds."""
    for G in (8, 37, 255):
        for B, flags, gamma in ((1, 0, 16), (1, 4, 7), (3, 0, 7), (20, 0, 16)):
            p = dsw.plan(fake_device(dsw, cus=G), 6_007, gamma, B, flags=flags).as_dict()
            assert p["grid"] == G and p["rows_per_wg"] >= -(-6_007 // G)
    with pytest.raises(dsw.DswError):   # 1,025 rows: more than a workgroup takes
        dsw.plan(fake_device(dsw, cus=8), 8_193, 7, 1)


def test_planner_prefetches_streamed_tiles_only_where_lds_is_left(dsw):
    """The cross-step prefetch of streamed tiles: one bf16 request with
    nothing resident gets LDS slots for the first streamed tiles of each
    wave; resident shards, several requests and int8 rows get none."""
    dev = fake_device(dsw)
    for V in (60_000, 151_936, 248_320):
        p = dsw.plan(dev, V, 7, 1, flags=1).as_dict()  # DSW_FLAG_FORCE_STREAM
        assert p["reg_tiles"] == 0 and p["lds_tiles"] == 0 and p["stream_rows"] == p["rows_per_wg"]
        assert 0 < p["prefetch_tiles"] <= p["tiles_per_wave"]
        assert 4 * p["prefetch_tiles"] * 8192 <= p["lds_bytes"] <= dev.max_lds_per_block - p["static_lds_bytes"]
        assert dsw.plan(dev, V, 7, 1).as_dict()["prefetch_tiles"] == 0            # resident
        assert dsw.plan(dev, V, 7, 4, flags=1).as_dict()["prefetch_tiles"] == 0   # four requests
        assert dsw.plan(dev, V, 7, 1, w2_dtype=1, flags=1).as_dict()["prefetch_tiles"] == 0  # int8


ENGINES = {"mfma": 8, "valu": 4, "batched": 16}   # flags forcing each kernel / engine


@pytest.mark.parametrize("engine", list(ENGINES))
@pytest.mark.parametrize("cus", [8, 80, 256])
@pytest.mark.parametrize("V", [1, 12, 1000, 32_000, 65_537, 151_936, 248_320])
@pytest.mark.parametrize("B", [1, 4, 16])
def test_planner_partitions_rows_and_respects_capacity(dsw, engine, cus, V, B):
    d = fake_device(dsw, cus=cus)
    flags = ENGINES[engine]
    rows = -(-V // min(cus, 256))
    if engine == "batched":
        rows = -(-rows // 16) * 16   # shards of whole 16-row tiles
    cap = {"valu": 4 * 256, "mfma": 4 * 16 * 16, "batched": 4 * 12 * 16}[engine]
    if rows > cap:
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, V, 7, B, flags=flags)
        assert e.value.code == -6
        return
    p = dsw.plan(d, V, 7, B, flags=flags)
    assert p.engine == (0 if engine == "valu" else 1)
    assert p.grid == min(cus, 256) and p.block == 256
    assert p.rows_per_wg == rows
    assert shards_cover(V, p.grid, p.rows_per_wg)
    assert p.reg_rows + p.lds_rows + p.stream_rows == p.rows_per_wg
    assert p.batch_tile >= B
    assert p.lds_bytes >= p.lds_rows * 512
    assert p.lds_bytes + p.static_lds_bytes <= d.max_lds_per_block
    assert p.lds_bytes + p.static_lds_bytes > d.lds_bytes_per_cu // 2   # one workgroup per CU
    assert p.onchip_bytes + p.stream_bytes == V * 512
    assert p.path == (1 if p.stream_rows > 0 else 0)
    if engine == "batched":
        assert p.batch_tile == 256 and 2 <= p.ring_slots <= 4
        assert p.rows_pad % 128 == 0 and p.rows_pad >= rows
        assert p.lds_bytes >= 4 * p.lds_tiles * 8192 + p.ring_slots * (8192 + 32 * p.rows_pad)
    if engine != "valu":
        assert p.tiles_per_wave * 4 * 16 >= rows
        # one request keeps up to 4 more tiles per wave in VGPRs, the batched
        # kernel (bf16) 2 more
        assert p.reg_tiles <= {1: 12, 256: 10}.get(p.batch_tile, 8) and p.tiles_per_wave <= p.max_tiles
        assert p.reg_tiles + p.lds_tiles <= max(p.tiles_per_wave, p.reg_tiles)
        assert p.lds_bytes >= p.lds_rows * 512
    else:
        assert p.reg_rows <= p.reg_slots * 256
        assert p.reg_slots <= {1: 3, 4: 2, 16: 1}[p.batch_tile]


def test_planner_choices_on_mi355x_shapes(dsw):
    d = fake_device(dsw)
    pick = lambda p: (p.rows_per_wg, p.tiles_per_wave, p.reg_tiles, p.lds_tiles, p.stream_rows)
    # by default one request takes the MFMA engine with batch tile 1, bf16 or
    # int8 rows (widened on chip)
    assert dsw.plan(d, 151_936, 7, 1).engine == 1 and dsw.plan(d, 151_936, 7, 1).batch_tile == 1
    assert dsw.plan(d, 151_936, 7, 2).engine == 1
    i1 = dsw.plan(d, 151_936, 7, 1, w2_dtype=dsw.INT8)
    assert (i1.engine, i1.batch_tile, i1.reg_tiles, i1.max_tiles) == (1, 1, 10, 10)
    # short walks of one bf16 request take the VALU engine (its shard load is shorter)
    assert dsw.plan(d, 151_936, 3, 1).engine == 0 and dsw.plan(d, 151_936, 4, 1).engine == 1
    assert pick(dsw.plan(d, 32_000, 7, 1, flags=8)) == (125, 2, 2, 0, 0)
    # one request on the MFMA engine: 10 tiles per wave all in registers (8 AGPR + 2 VGPR)
    c1 = dsw.plan(d, 151_936, 7, 1, flags=8)
    assert pick(c1) == (594, 10, 10, 0, 0) and c1.path == 0 and c1.onchip_bytes == 151_936 * 512
    assert c1.batch_tile == 1
    # V = 248,320: 12 register tiles and 4 LDS tiles per wave, nothing streamed
    c3 = dsw.plan(d, 248_320, 16, 1, flags=8)
    assert pick(c3) == (970, 16, 12, 4, 0) and c3.batch_tile == 1
    # two requests: the 4-request tile with 8 AGPR tiles and 2 LDS tiles
    assert pick(dsw.plan(d, 151_936, 7, 2, flags=8)) == (594, 10, 8, 2, 0)
    c2 = dsw.plan(d, 151_936, 16, 16, flags=8)
    assert pick(c2) == (594, 10, 8, 2, 0) and c2.batch_tile == 16
    # by default 2 and more requests take the batched kernel; where it has no
    # shape (beyond 12 tiles per wave) the all-to-all MFMA kernel
    assert [dsw.plan(d, 151_936, 16, b).batch_tile for b in (1, 2, 3, 4, 16)] == [1, 256, 256, 256, 256]
    assert [dsw.plan(d, 248_320, 16, b).batch_tile for b in (2, 3, 4, 16)] == [4, 4, 4, 16]
    # 4 requests at V = 248,320: 8 AGPR tiles per wave, LDS for some, the rest streamed
    c3 = dsw.plan(d, 248_320, 16, 4, flags=8)
    assert c3.rows_per_wg == 970 and c3.tiles_per_wave == 16 and c3.path == 1 and c3.stream_rows > 0
    c4 = dsw.plan(d, 129_280, 5, 16, flags=8)
    assert pick(c4) == (505, 8, 8, 0, 0)
    # the VALU engine keeps whole 256-row groups per lane
    v1 = dsw.plan(d, 151_936, 7, 1, flags=4)
    assert (v1.engine, v1.reg_slots, v1.reg_rows, v1.lds_rows, v1.stream_rows) == (0, 3, 594, 0, 0)
    v3 = dsw.plan(d, 248_320, 16, 1, flags=4)
    assert (v3.reg_slots, v3.lds_rows, v3.stream_rows) == (3, 202, 0)


def test_planner_batched_kernel(dsw):
    d = fake_device(dsw)
    # beyond 16 requests the batched kernel takes over, with 16-row aligned shards
    c4 = dsw.plan(d, 129_280, 5, 253)
    assert (c4.batch_tile, c4.rows_per_wg, c4.rows_pad, c4.tiles_per_wave, c4.reg_tiles) == (256, 512, 512, 8, 8)
    assert c4.lds_tiles == 0 and c4.stream_rows == 0 and c4.ring_slots == 4
    assert c4.onchip_bytes == 129_280 * 512
    assert dsw.plan(d, 129_280, 5, 16, flags=dsw.FLAG_MFMA_GEMV).batch_tile == 16
    assert dsw.plan(d, 129_280, 5, 3, flags=dsw.FLAG_BATCHED).batch_tile == 256
    # int8 rows beyond the batched shapes fall back to the all-to-all kernel
    assert dsw.plan(d, 248_320, 16, 8, w2_dtype=dsw.INT8).batch_tile == 16
    # V = 151,936 with 64 requests: ten register tiles per wave (two in VGPRs)
    c2 = dsw.plan(d, 151_936, 16, 64)
    assert (c2.rows_per_wg, c2.tiles_per_wave, c2.reg_tiles, c2.lds_tiles, c2.stream_rows) == (608, 10, 10, 0, 0)
    assert c2.ring_slots >= 2
    # Gumbel-max beyond 4 requests keeps 8 register tiles and two LDS tiles
    g2 = dsw.plan(d, 151_936, 16, 64, flags=dsw.FLAG_GUMBEL)
    assert (g2.reg_tiles, g2.lds_tiles) == (8, 2)
    assert dsw.plan(d, 151_936, 16, 4, flags=dsw.FLAG_GUMBEL | dsw.FLAG_BATCHED).reg_tiles == 10
    # 9 tiles per wave: 8 register tiles and one LDS tile
    c9 = dsw.plan(d, 140_000, 16, 64)
    assert (c9.tiles_per_wave, c9.reg_tiles, c9.lds_tiles) == (9, 8, 1)
    i8 = dsw.plan(d, 129_280, 5, 64, w2_dtype=dsw.INT8)
    assert (i8.reg_tiles, i8.max_tiles, i8.w2_dtype, i8.onchip_bytes) == (8, 8, dsw.INT8, 129_280 * 256)
    with pytest.raises(dsw.DswError) as e:   # no VALU engine for the batched kernel
        dsw.plan(d, 129_280, 5, 64, flags=dsw.FLAG_VALU_GEMV)
    assert e.value.code == -11


def test_planner_gumbel_max_kernels(dsw):
    d = fake_device(dsw)
    G = dsw.FLAG_GUMBEL
    # bf16 rows, double rounding: the same kernels as the inverse CDF (the
    # batched kernel from 2 requests); the shard layout is the same plan as
    # without the flag, and up to 4 requests on the all-to-all kernels keep one
    # step's noise per row in LDS
    for B, tile in ((1, 1), (2, 256), (3, 256), (4, 256), (8, 256), (16, 256), (17, 256), (253, 256)):
        assert dsw.plan(d, 129_280, 5, B, flags=G).batch_tile == tile
    for B in (4, 16, 253):
        a, b = dsw.plan(d, 129_280, 5, B, flags=G), dsw.plan(d, 129_280, 5, B)
        assert a.as_dict() == b.as_dict()
    assert dsw.plan(d, 129_280, 5, 4, flags=G | dsw.FLAG_BATCHED).batch_tile == 256
    a, b = dsw.plan(d, 151_936, 7, 1, flags=G), dsw.plan(d, 151_936, 7, 1)
    keys = ("engine", "rows_per_wg", "tiles_per_wave", "reg_tiles", "lds_tiles", "stream_rows", "batch_tile")
    assert [a.as_dict()[k] for k in keys] == [b.as_dict()[k] for k in keys]
    assert a.static_lds_bytes == b.static_lds_bytes + 4 * 640
    a16, b16 = dsw.plan(d, 151_936, 7, 16, flags=G | dsw.FLAG_MFMA_GEMV), dsw.plan(d, 151_936, 7, 16,
                                                                                   flags=dsw.FLAG_MFMA_GEMV)
    assert a16.static_lds_bytes == b16.static_lds_bytes
    # int8 rows or single rounding: the all-to-all kernels, up to 16 requests
    assert dsw.plan(d, 248_320, 16, 2, w2_dtype=dsw.INT8, flags=G).batch_tile == 4
    assert dsw.plan(d, 129_280, 5, 8, w2_dtype=dsw.INT8, flags=G).batch_tile == 16
    assert dsw.plan(d, 129_280, 5, 8, flags=G | dsw.FLAG_SINGLE_ROUND).batch_tile == 16
    for B, flags, dt in ((17, G, dsw.INT8), (253, G | dsw.FLAG_SINGLE_ROUND, dsw.BF16),
                         (4, G | dsw.FLAG_BATCHED, dsw.INT8)):
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, 129_280, 5, B, w2_dtype=dt, flags=flags)
        assert e.value.code == -11


def test_planner_gru_head(dsw):
    d = fake_device(dsw)
    R = dsw.FLAG_GRU
    # one bf16 request on the one-request MFMA engine, also for short walks
    for gamma in (1, 3, 16):
        p = dsw.plan(d, 151_936, gamma, 1, flags=R)
        assert (p.engine, p.batch_tile, p.reg_tiles, p.max_tiles) == (1, 1, 10, 10)
        q = dsw.plan(d, 151_936, 16, 1)
        # the state, the cell rows and the recurrent pre-activations take LDS
        assert p.static_lds_bytes == q.static_lds_bytes + 256 * 4 + 4 * 6 * (512 + 4) + 4 * 3 * 4
    assert dsw.plan(d, 248_320, 16, 1, flags=R).max_tiles == 16
    for B, flags, dt, code in ((2, R, dsw.BF16, -11), (1, R | dsw.FLAG_GUMBEL, dsw.BF16, -11),
                               (1, R | dsw.FLAG_BATCHED, dsw.BF16, -11), (1, R | dsw.FLAG_VALU_GEMV, dsw.BF16, -11),
                               (1, R, dsw.INT8, -5)):
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, 151_936, 7, B, w2_dtype=dt, flags=flags)
        assert e.value.code == code
    # the RNN head: the same plan, one gate instead of three in LDS
    n = dsw.plan(d, 151_936, 7, 1, flags=dsw.FLAG_RNN)
    assert (n.engine, n.batch_tile, n.reg_tiles) == (1, 1, 10)
    assert n.static_lds_bytes == dsw.plan(d, 151_936, 16, 1).static_lds_bytes + 256 * 4 + 4 * 2 * (512 + 4) + 4 * 4
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(d, 151_936, 7, 1, flags=R | dsw.FLAG_RNN)
    assert e.value.code == -11
    # the state is spread over at most 4 elements per workgroup: 64 CUs at least
    assert dsw.plan(fake_device(dsw, cus=64), 32_000, 7, 1, flags=R).grid == 64
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(fake_device(dsw, cus=63), 32_000, 7, 1, flags=R)
    assert e.value.code == -10


def test_planner_gated_head(dsw):
    d = fake_device(dsw)
    Q = dsw.FLAG_GATED
    # the one-request MFMA engine; the whole gate matrix (widened to bf16), its
    # scales and biases, the state, its low pieces and the gates take 133 KiB of LDS
    p = dsw.plan(d, 151_936, 7, 1, flags=Q)
    q = dsw.plan(d, 151_936, 16, 1)
    assert (p.engine, p.batch_tile, p.reg_tiles, p.max_tiles, p.stream_rows) == (1, 1, 10, 10, 0)
    assert p.static_lds_bytes == q.static_lds_bytes + 256 * 256 * 2 + 4 * 256 * 4 + 2 * 256 * 2
    # V = 248,320: the matrix displaces LDS tiles of the shard, which then streams part of its rows
    full, gated = dsw.plan(d, 248_320, 16, 1), dsw.plan(d, 248_320, 16, 1, flags=Q)
    assert full.stream_rows == 0 and gated.stream_rows > 0 and gated.lds_tiles < full.lds_tiles
    assert gated.static_lds_bytes + gated.lds_bytes <= 160 * 1024
    # no state exchange, so no lower bound on the grid
    assert dsw.plan(fake_device(dsw, cus=32), 32_000, 7, 1, flags=Q).grid == 32
    for B, flags, dt, code in ((2, Q, dsw.BF16, -11), (1, Q | dsw.FLAG_GUMBEL, dsw.BF16, -11),
                               (1, Q | dsw.FLAG_BATCHED, dsw.BF16, -11), (1, Q | dsw.FLAG_VALU_GEMV, dsw.BF16, -11),
                               (1, Q | dsw.FLAG_GRU, dsw.BF16, -11), (1, Q | dsw.FLAG_RNN, dsw.BF16, -11),
                               (1, Q, dsw.INT8, -5)):
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, 151_936, 7, B, w2_dtype=dt, flags=flags)
        assert e.value.code == code


def test_planner_domino_head(dsw):
    d = fake_device(dsw)
    D = dsw.FLAG_DOMINO
    p, g = dsw.plan(d, 151_936, 16, 1, flags=D), dsw.plan(d, 151_936, 16, 1, flags=dsw.FLAG_GRU)
    assert (p.engine, p.batch_tile, p.reg_tiles) == (1, 1, 10)
    # the GRU head's LDS and the hidden states' pre-activations of 16 steps with their partial sums
    assert p.static_lds_bytes == g.static_lds_bytes + 5 * 16 * 3 * 4
    for B, flags, dt, code in ((2, D, dsw.BF16, -11), (1, D | dsw.FLAG_GRU, dsw.BF16, -11),
                               (1, D | dsw.FLAG_GATED, dsw.BF16, -11), (1, D, dsw.INT8, -5)):
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, 151_936, 7, B, w2_dtype=dt, flags=flags)
        assert e.value.code == code
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(d, 151_936, 17, 1, flags=D)
    assert e.value.code == -3
    # one state element per workgroup: r workgroups
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(fake_device(dsw, cus=128), 32_000, 7, 1, flags=D)
    assert e.value.code == -10


def test_planner_int8_rows(dsw):
    d = fake_device(dsw)
    pick = lambda p: (p.engine, p.tiles_per_wave, p.reg_tiles, p.lds_tiles, p.stream_rows)  # noqa: E731
    # with more than one request int8 codes take half the registers: V = 248,320
    # is fully resident at 16 tiles per wave
    c3 = dsw.plan(d, 248_320, 16, 2, w2_dtype=dsw.INT8, flags=dsw.FLAG_MFMA_GEMV)
    assert pick(c3) == (1, 16, 16, 0, 0) and c3.path == 0 and c3.w2_dtype == dsw.INT8
    assert c3.onchip_bytes == 248_320 * 256 and c3.stream_bytes == 0
    assert pick(dsw.plan(d, 248_320, 16, 16, w2_dtype=dsw.INT8)) == (1, 16, 16, 0, 0)
    # one request takes the one-request MFMA engine: rows widened to bf16 on
    # chip, 12 register and 4 LDS tiles per wave as in bf16, nothing streamed
    one = dsw.plan(d, 248_320, 16, 1, w2_dtype=dsw.INT8)
    assert pick(one) == (1, 16, 12, 4, 0) and one.batch_tile == 1 and one.path == 0
    assert one.onchip_bytes == 248_320 * 256 and one.stream_bytes == 0
    # forced onto the VALU engine: two widened register groups, LDS rows (bf16,
    # 512 bytes each) and the rest streamed as int8 every step
    v = dsw.plan(d, 248_320, 16, 1, w2_dtype=dsw.INT8, flags=dsw.FLAG_VALU_GEMV)
    assert (v.engine, v.reg_slots, v.reg_rows) == (0, 2, 512) and v.path == 1
    assert v.lds_rows == (v.lds_bytes // 512) and v.lds_rows + v.stream_rows == 970 - 512
    assert v.stream_bytes == 256 * v.stream_rows * 256 and v.onchip_bytes + v.stream_bytes == 248_320 * 256
    # small vocabularies fit in the two register groups
    assert dsw.plan(d, 100_000, 7, 1, w2_dtype=dsw.INT8, flags=dsw.FLAG_VALU_GEMV).path == 0
    # short walks of one int8 request take the VALU engine, like bf16
    assert dsw.plan(d, 100_000, 3, 1, w2_dtype=dsw.INT8).engine == 0
    # smaller vocabularies take the smaller compiled shapes of the all-to-all
    # kernel; by default 3 requests take the batched one
    M = dsw.FLAG_MFMA_GEMV
    assert dsw.plan(d, 60_000, 7, 3, w2_dtype=dsw.INT8, flags=M).reg_tiles == 4
    assert dsw.plan(d, 129_280, 7, 3, w2_dtype=dsw.INT8, flags=M).reg_tiles == 8
    assert dsw.plan(d, 129_280, 7, 3, w2_dtype=dsw.INT8).batch_tile == 256
    # streaming everything works for int8 too
    s = dsw.plan(d, 248_320, 16, 1, w2_dtype=dsw.INT8, flags=1)
    assert (s.reg_rows, s.lds_rows, s.stream_rows, s.stream_bytes) == (0, 0, 970, 248_320 * 256)
    # the VALU engine takes int8 rows for one request only
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(d, 248_320, 16, 2, w2_dtype=dsw.INT8, flags=4)
    assert e.value.code == -5
    assert dsw.plan(d, 248_320, 16, 1).w2_dtype == dsw.BF16


def test_planner_stream_fallback_on_small_devices(dsw):
    # 32 KiB of LDS beside the 4-request kernel's staging leaves no room for
    # the two LDS tiles per wave that V = 151,936 needs: those rows stream
    d = fake_device(dsw, cus=256, lds_cu=32 * 1024, lds_blk=32 * 1024)
    p = dsw.plan(d, 151_936, 7, 4)
    assert (p.engine, p.reg_tiles, p.lds_tiles) == (1, 8, 0)
    assert p.stream_rows == 96 and p.path == 1
    # the same walk on the full device stays on chip
    assert dsw.plan(fake_device(dsw), 151_936, 7, 4).stream_rows == 0
    # and the 16-request kernel does not fit 64 KiB at all
    with pytest.raises(dsw.DswError) as e:
        dsw.plan(fake_device(dsw, lds_cu=64 * 1024, lds_blk=64 * 1024), 151_936, 7, 16)
    assert e.value.code == -10


def test_planner_force_stream_keeps_nothing_on_chip(dsw):
    d = fake_device(dsw)
    for flags in (1, 1 | 4):
        p = dsw.plan(d, 151_936, 7, 1, flags=flags)
        assert p.reg_rows == 0 and p.lds_rows == 0 and p.stream_rows == 594 and p.onchip_bytes == 0


def test_planner_rejects_bad_arguments(dsw):
    d = fake_device(dsw)
    for kw, code in [(dict(r=128), -4), (dict(w2_dtype=9), -5), (dict(V=0), -6),
                     (dict(B=257), -2), (dict(gamma=-1), -3)]:
        args = dict(V=1000, gamma=7, B=1)
        args.update(kw)
        r = args.pop("r", 256)
        with pytest.raises(dsw.DswError) as e:
            dsw.plan(d, r=r, **args)
        assert e.value.code == code
