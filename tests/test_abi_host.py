"""Host-side checks of the C-ABI library (no kernel launches, no GPU needed).

Every call here fails argument validation, which the library performs on the host before
any HIP call, so nothing reaches the device.
"""
import ctypes
import os

import pytest

import int4_weight_only_gemm_amd as w4


def test_library_exports_every_declared_symbol():
    names = w4.header_functions()
    assert set(names) >= {"w4a16_gemm", "w4_pack", "w4a16_plan", "w4_status_string", "w4_last_error",
                          "w8a16_gemm", "w8_pack", "w8a16_plan", "w4_quantize", "w4_read_probe",
                          "w4a4_gemm", "w4a4_plan", "a4_quantize"}
    lib = w4.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/w4a16.h but not exported"


def test_status_strings():
    for code in range(8):
        s = w4.status_string(code)
        assert s and s != "unknown status"
    assert w4.status_string(99) == "unknown status"


A16, W16, S8, Z4, C16 = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000  # never dereferenced


def _gemm(*args):
    return w4.lib().w4a16_gemm(*args)


GEMMS = {"w4a16": lambda *a: w4.lib().w4a16_gemm(*a), "w8a16": lambda *a: w4.lib().w8a16_gemm(*a)}


@pytest.mark.parametrize("which", sorted(GEMMS))
@pytest.mark.parametrize("ptrs", [
    (None, W16, S8, Z4, C16), (A16, None, S8, Z4, C16), (A16, W16, None, Z4, C16),
    (A16, W16, S8, None, C16), (A16, W16, S8, Z4, None)])
def test_null_pointers(ptrs, which):
    assert GEMMS[which](*ptrs, 5, 128, 64, None) == 1
    assert w4.lib().w4_last_error()


@pytest.mark.parametrize("which", sorted(GEMMS))
@pytest.mark.parametrize("mkn", [(0, 128, 64), (5, 0, 64), (5, 64, 64), (5, 129, 64), (5, 200, 64),
                                 (5, 128, 0), (-1, 128, 8), (5, -128, 8), (1 << 31, 1 << 20, 1 << 20)])
def test_bad_shapes(mkn, which):
    assert GEMMS[which](A16, W16, S8, Z4, C16, *mkn, None) == 2


def test_packed_weight_limit_follows_code_width():
    # packed codes must stay below 2 GiB: K*N/2 bytes for 4-bit codes, K*N bytes for 8-bit
    K, N = 1 << 16, 1 << 15          # 2^31 weights: 1 GiB packed at 4 bits, 2 GiB at 8 bits
    assert w4.plan(1, K, N)["splits"] >= 1
    with pytest.raises(w4.W4Error):
        w4.plan(1, K, N, bits=8)
    assert w4.plan(1, K, N // 2, bits=8)["splits"] >= 1


@pytest.mark.parametrize("which", sorted(GEMMS))
@pytest.mark.parametrize("ptrs", [
    (A16 + 2, W16, S8, Z4, C16), (A16, W16 + 4, S8, Z4, C16), (A16, W16, S8, Z4, C16 + 8),
    (A16, W16, S8 + 1, Z4, C16)])
def test_misaligned(ptrs, which):
    assert GEMMS[which](*ptrs, 5, 128, 64, None) == 3


AS4 = 0x60000  # activation scales (never dereferenced)


@pytest.mark.parametrize("ptrs", [
    (None, AS4, W16, S8, Z4, C16), (A16, None, W16, S8, Z4, C16), (A16, AS4, None, S8, Z4, C16),
    (A16, AS4, W16, None, Z4, C16), (A16, AS4, W16, S8, None, C16), (A16, AS4, W16, S8, Z4, None)])
def test_w4a4_null_pointers(ptrs):
    assert w4.lib().w4a4_gemm(*ptrs, 5, 128, 64, None) == 1


@pytest.mark.parametrize("mkn", [(0, 128, 64), (5, 64, 64), (5, 129, 64), (5, 128, 0), (1 << 31, 1 << 20, 1 << 20)])
def test_w4a4_bad_shapes(mkn):
    assert w4.lib().w4a4_gemm(A16, AS4, W16, S8, Z4, C16, *mkn, None) == 2


@pytest.mark.parametrize("ptrs", [
    (A16 + 2, AS4, W16, S8, Z4, C16), (A16, AS4 + 2, W16, S8, Z4, C16), (A16, AS4, W16 + 4, S8, Z4, C16),
    (A16, AS4, W16, S8, Z4, C16 + 8), (A16, AS4, W16, S8 + 1, Z4, C16)])
def test_w4a4_misaligned(ptrs):
    assert w4.lib().w4a4_gemm(*ptrs, 5, 128, 64, None) == 3


def test_a4_quantize_validation():
    q = w4.lib().a4_quantize
    assert q(None, W16, AS4, 2, 128, None) == 1
    assert q(A16, None, AS4, 2, 128, None) == 1
    assert q(A16, W16, None, 2, 128, None) == 1
    assert q(A16, W16, AS4, 0, 128, None) == 2
    assert q(A16, W16, AS4, 2, 64, None) == 2
    assert q(A16, W16, AS4, 2, 200, None) == 2
    assert q(A16 + 8, W16, AS4, 2, 128, None) == 3
    assert q(A16, W16 + 2, AS4, 2, 128, None) == 3
    assert q(A16, W16, AS4 + 1, 2, 128, None) == 3


def test_pack8_validation():
    lib = w4.lib()
    assert lib.w8_pack(None, W16, 4, 4, None) == 1
    assert lib.w8_pack(A16, None, 4, 4, None) == 1
    assert lib.w8_pack(A16, W16, 6, 4, None) == 2
    assert lib.w8_pack(A16, W16, 0, 4, None) == 2
    assert lib.w8_pack(A16, W16, 4, 0, None) == 2
    assert lib.w8_pack(A16, W16 + 2, 4, 4, None) == 3


def test_pack_validation():
    lib = w4.lib()
    assert lib.w4_pack(None, W16, 8, 4, None) == 1
    assert lib.w4_pack(A16, None, 8, 4, None) == 1
    assert lib.w4_pack(A16, W16, 12, 4, None) == 2
    assert lib.w4_pack(A16, W16, 0, 4, None) == 2
    assert lib.w4_pack(A16, W16, 8, 0, None) == 2
    assert lib.w4_pack(A16, W16 + 2, 8, 4, None) == 3


def test_read_probe_validation():
    lib = w4.lib()
    probe = lib.w4_read_probe
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert probe(None, 64, W16, 4, None) == 1
    assert probe(A16, 64, None, 4, None) == 1
    assert probe(A16, 40, W16, 4, None) == 2   # not a multiple of 16
    assert probe(A16, 0, W16, 4, None) == 2
    assert probe(A16, 64, W16, 0, None) == 2
    assert probe(A16, 1 << 31, W16, 4, None) == 2
    assert probe(A16, 64, W16, 65536, None) == 2
    assert probe(A16 + 8, 64, W16, 4, None) == 3
    assert probe(A16, 64, W16 + 2, 4, None) == 3


def test_kernel_choice_by_shape():
    # bf16 kernel from M = 64; from M = 17 only for large GEMMs (K*N >= 2^25)
    assert w4.plan(63, 128, 64)["kernel"] in (1, 2)
    assert w4.plan(64, 128, 64)["kernel"] == 3
    assert w4.plan(16, 4096, 8192)["kernel"] in (1, 2)
    assert w4.plan(17, 4096, 8192)["kernel"] == 3
    assert w4.plan(32, 4096, 8192)["kernel"] == 3
    assert w4.plan(33, 4096, 8192)["kernel"] == 3
    assert w4.plan(40, 4096, 8191)["kernel"] in (1, 2)
    assert w4.plan(40, 3584, 4608)["kernel"] in (1, 2)
    assert w4.plan(40, 3584, 37888)["kernel"] == 3
    assert w4.plan(63, 18944, 3584)["kernel"] == 3


def test_quantize_validation():
    lib = w4.lib()
    qz = lib.w4_quantize
    qz.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    assert qz(None, W16, S8, Z4, 128, 4, None) == 1
    assert qz(A16, W16, None, Z4, 128, 4, None) == 1
    assert qz(A16, W16, S8, Z4, 100, 4, None) == 2   # K not a multiple of 128
    assert qz(A16, W16, S8, Z4, 128, 0, None) == 2
    assert qz(A16, W16, S8, Z4, 128 * 65536, 1, None) == 2  # too many groups for the grid
    assert qz(A16 + 1, W16, S8, Z4, 128, 4, None) == 3
    assert qz(A16, W16 + 2, S8, Z4, 128, 4, None) == 3
    assert qz(A16, W16, S8 + 1, Z4, 128, 4, None) == 3


def test_plan_covers_shapes():
    # every shape of the synthetic workloads has a valid plan that tiles N and K exactly;
    # a balanced wide plan runs whole rounds of 256 tiles unsplit and splits the rest.  The
    # kernels rely on these identities: they derive their tile and row-block counts from N
    # and M, and their count of split-part workgroups from the tile, row-block and split
    # counts, instead of receiving them
    import synth
    seen = set()
    shapes = [(g.M, g.K, g.N, g.bits, g.act4) for wl in synth.WORKLOADS.values() for g in wl.gemms]
    shapes += [(M, K, N, bits, a4) for M in (1, 5, 16, 17, 40, 64, 160) for K, N in ((3584, 4608), (18944, 3584), (128, 3))
               for bits, a4 in ((8, False), (4, True))]
    # the large-M search at every row count 17..200 on shapes where its 4-group floor, the
    # 32-row blocks up to 64 rows and the half-chip guard each decide some plans
    shapes += [(M, K, N, 4, False) for M in range(17, 201) for K, N in ((4096, 4096), (8960, 1536), (2048, 8192),
                                                                         (1536, 2048), (2048, 2048), (11008, 4096))]
    for key in shapes:
        if key in seen:
            continue
        seen.add(key)
        M, K, N, bits, a4 = key
        p = w4.plan(M, K, N, bits=bits, a4=a4)
        groups = K // 128
        # the narrow-tile kernel (either code width): rows in one 16-row block, at most 64
        # groups, staged activations within 64 KiB, at most one round of 256 tiles
        G = K // 128
        stage = max(G * M * 272 + 16 + G * 64, 8 * M * 16 * 4)
        narrow = M <= 16 and G <= 64 and stage <= 65536 and (N + 15) // 16 <= 256
        if a4:  # every row count runs on the 4-bit-activation small-M kernel
            assert p["kernel"] in (6, 7)
        elif bits == 8:  # the narrow-tile kernel where it applies, else the 8-bit small-M kernel
            assert p["kernel"] in (4, 5, 8)
            assert (p["kernel"] == 8) == narrow, (M, K, N, p)
        else:
            assert (p["kernel"] == 3) == (M >= 64 or (M >= 17 and K * N >= 1 << 25))
            assert (p["kernel"] == 8) == narrow, (M, K, N, p)
        if True:
            if p["kernel"] == 3:
                assert p["tile_n"] == 256 and p["tile_m"] <= 160
            elif p["kernel"] == 8:
                assert (p["tile_m"], p["tile_n"], p["splits"], p["m_blocks"]) == (16, 16, 1, 1)
            else:  # 16-row blocks, or (4-bit activations) one 32-row block at 17..32 rows
                assert (p["tile_m"], p["tile_n"]) == ((32 if a4 and 16 < M <= 32 else 16), 64)
            assert p["n_tiles"] * p["tile_n"] >= N > (p["n_tiles"] - 1) * p["tile_n"]
            assert p["m_blocks"] * p["tile_m"] >= M > (p["m_blocks"] - 1) * p["tile_m"]
            tiles = p["n_tiles"] * p["m_blocks"]
            full = p["full_tiles"]
            assert full % 256 == 0 and 0 <= full < tiles
            assert full == 0 or (p["kernel"] in (1, 4, 6) and p["splits"] > 1)
            assert (p["workspace_bytes"] > 0) == (p["splits"] > 1)
            gps, stride = p["groups_per_split"], p["group_stride"]
            if p["kernel"] == 3 and stride == groups and groups % gps:
                # steps shared out evenly: walk every workgroup's range and count the
                # workgroups each tile receives
                assert 1 <= gps < groups and p["tile_m"] <= 64  # blocks of up to two row tiles
                assert p["workgroups"] == -(-tiles * groups // gps)
                per_tile = [0] * tiles
                for w in range(p["workgroups"]):
                    u, end = w * gps, min(w * gps + gps, tiles * groups)
                    for t in range(u // groups, (end - 1) // groups + 1):
                        per_tile[t] += 1
                assert p["splits"] == max(per_tile) and min(per_tile) >= 2
            else:  # each tile split alike into `splits` workgroups (kernel 3: stride = their span)
                assert stride == (p["splits"] * gps if p["kernel"] == 3 else 0)
                assert p["splits"] * gps >= groups
                assert (p["splits"] - 1) * gps < groups
                assert p["workgroups"] == full + (tiles - full) * p["splits"]
            if p["kernel"] not in (3, 8):  # every workgroup resident at once
                per_cu = (2 if p["tile_m"] == 32 else 3) if p["kernel"] in (1, 4, 6) else 1
                assert p["workgroups"] <= 256 * per_cu or p["splits"] == 1
            if p["kernel"] == 8:
                assert p["workgroups"] == p["n_tiles"] <= 256
    with pytest.raises(w4.W4Error):
        w4.plan(5, 100, 64)


def test_every_plan_has_a_kernel_instance():
    # the plan entry points run the same instance check as the GEMM entry points (which
    # return W4_ERR_PLAN before launching anything): every plan the planners emit, for every
    # row count up to the bf16 kernel's range and beyond, names a compiled kernel
    for M in list(range(1, 80)) + [96, 128, 160, 161, 200, 320]:
        for K, N in ((128, 3), (1536, 1536), (3584, 4608), (3584, 37888), (18944, 3584), (4096, 22016)):
            for bits, a4 in ((4, False), (8, False), (4, True)):
                p = w4.plan(M, K, N, bits=bits, a4=a4)  # raises W4Error(W4_ERR_PLAN) otherwise
                if p["kernel"] != 3:
                    rows = min(M, p["tile_m"])
                    assert p["tile_m"] == 16 or (p["tile_m"] == 32 and a4 and 5 <= (rows + 3) // 4 <= 8)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_no_device_is_reported():
    # valid arguments on a host with no GPU: the device check fails before any launch
    assert _gemm(A16, W16, S8, Z4, C16, 5, 128, 64, None) == 4


def test_measured_plan_choices():
    # plan decisions backed by measured launches (graph replays, HBM-resident weights):
    # qkv and o at M=5 take the wide shape at 3 splits (a tall workgroup would leave waves
    # idle), down keeps the tall shape at 4 splits, and 8-bit down at M=1 spreads over 96 CUs
    # with the wide shape (8-bit near-ties at M <= 4: 9.41 us tall, 8.60 wide)
    p = w4.plan(5, 3584, 4608)
    assert (p["kernel"], p["splits"]) == (1, 3), p
    # o at M=5 (224 sixteen-column tiles, one round of CUs) runs on the narrow-tile kernel
    # without a K split: 7.20 -> 5.48 us measured (graph replays, weights from HBM); qkv
    # (288 tiles, a second partial round) measured 7.46 small-M against 8.52 narrow
    p = w4.plan(5, 3584, 3584)
    assert (p["kernel"], p["splits"], p["workgroups"]) == (8, 1, 224), p
    p = w4.plan(5, 18944, 3584)
    assert (p["kernel"], p["splits"]) == (2, 4), p
    p = w4.plan(1, 8960, 1536, bits=8)
    assert (p["kernel"], p["splits"], p["workgroups"]) == (4, 4, 96), p
    # gate_up at M=5: two whole rounds unsplit, the remaining 80 tiles split three ways
    p = w4.plan(5, 3584, 37888)
    assert (p["kernel"], p["full_tiles"], p["splits"], p["workgroups"]) == (1, 512, 3, 752), p
    # bf16 kernel at M = 64..96: splits of at least 4 groups, with two row blocks (qkv and o
    # at M=64: 1 x 14 splits measured 20.6 and 18.6 us, 2 x 7 measured 16.8 and 15.3 us);
    # the M=160 plans are the model's (within 3% of the fastest forced plan per shape)
    for M, K, N, want in ((64, 3584, 4608, (2, 32, 7)), (64, 3584, 3584, (2, 32, 7)), (96, 3584, 3584, (2, 48, 7)),
                          (64, 4096, 4096, (2, 32, 8)), (160, 4096, 12288, (1, 160, 5)),
                          (160, 4096, 4096, (2, 80, 8)), (160, 4096, 22016, (1, 160, 2)),
                          (160, 11008, 4096, (1, 160, 15))):
        p = w4.plan(M, K, N)
        assert p["kernel"] == 3 and (p["m_blocks"], p["tile_m"], p["splits"]) == want, (M, K, N, p)
    # bf16 kernel at M = 17..64 on wide outputs: the (tile, group) steps shared out evenly,
    # one round of workgroups instead of 2-3 rounds of whole-tile splits (Qwen2.5-7B gate_up
    # at M=40: 5 splits in 3 rounds 45.8 us, 17 shared steps 38.3 us; M=24 36.9 -> 32.4;
    # Llama-2-7B gate_up at M=24: 31.2 -> 25.0)
    for M, K, N, want in ((40, 3584, 37888, (17, 244, 3)), (24, 3584, 37888, (17, 244, 3)),
                          (24, 4096, 22016, (11, 251, 4))):
        p = w4.plan(M, K, N)
        assert p["kernel"] == 3 and p["group_stride"] == K // 128, (M, K, N, p)
        assert (p["groups_per_split"], p["workgroups"], p["splits"]) == want, (M, K, N, p)
    # a single 16-row block hands a tall plan at one group per wave to the wide shape (M=1
    # draft: qkv 4.52 -> 4.49, o 4.70 -> 4.57, down 7.36 -> 7.16 us; 8-bit qkv 5.69 -> 5.36 us);
    # more rows per workgroup keep the tall shape (W4A4 at M=32: 9.21 tall, 10.30 wide)
    # the M=1 draft's qkv and o run narrow (4.56 -> 3.52 and 4.55 -> 3.48 us); its down
    # (70 groups, more than a wave's eight at once) keeps the small-M split plan
    for K, N, want in ((1536, 2048, (8, 1)), (1536, 1536, (8, 1)), (8960, 1536, (1, 6))):
        p = w4.plan(1, K, N)
        assert (p["kernel"], p["splits"]) == want, (K, N, p)
    # with 8-bit codes too (qkv 4.98 -> 3.91, o 4.99 -> 3.88 us against the small-M kernel)
    for K, N in ((1536, 2048), (1536, 1536)):
        assert w4.plan(1, K, N, bits=8)["kernel"] == 8
    assert w4.plan(24, 1536, 2048)["kernel"] == 2
    p = w4.plan(32, 4096, 4096, a4=True)
    assert (p["kernel"], p["tile_m"], p["splits"]) == (7, 32, 4), p
    # where splits of 4 groups would leave most CUs idle, the model's plan stands
    p = w4.plan(64, 2048, 2048)
    assert (p["m_blocks"], p["splits"], p["groups_per_split"]) == (1, 16, 1), p
