"""Host-only checks of the measuring tools.  The ceiling library (the
benchmark's streams, csrc/ceilings.hip) loads, exports its entry points and
rejects bad arguments before anything touches the GPU (placeholder pointers are
never dereferenced on these paths); the clock-stamp tool's patch still applies
to the prefill source."""
import ctypes

import pytest

from sparse_attention_layerrouter_amd import ceilings

P = ctypes.c_void_p(0x1000)
NULL = ctypes.c_void_p(0)


def test_library_exports_its_entry_points():
    L = ceilings.lib()
    for name in ceilings.EXPORTS:
        assert hasattr(L, name), name


@pytest.mark.parametrize("buf,nbytes,chunk,sink,why", [
    (NULL, 1 << 20, 1 << 15, P, "null"),
    (P, 1 << 20, 1 << 15, NULL, "null"),
    (ctypes.c_void_p(0x1004), 1 << 20, 1 << 15, P, "aligned"),
    (P, 1 << 20, 0, P, "32 KiB"),
    (P, 1 << 20, 3 << 14, P, "32 KiB"),     # 48 KiB: not a multiple of 32 KiB
    (P, 0, 1 << 15, P, "divide"),
    (P, 3 << 15, 1 << 16, P, "divide"),     # 96 KiB in 64 KiB chunks
])
def test_read_validation(buf, nbytes, chunk, sink, why):
    L = ceilings.lib()
    assert L.fa_ceiling_read(buf, nbytes, chunk, sink, NULL) == 1
    assert why in L.fa_ceiling_last_error().decode()


@pytest.mark.parametrize("rd,sm,shape,nwg,iters,seed,out,why", [
    (3, 0, 0, 1, 2, P, P, "reads_per_8"),
    (10, 1, 0, 1, 2, P, P, "reads_per_8"),
    (8, 2, 0, 1, 2, P, P, "softmax"),
    (8, 1, 2, 1, 2, P, P, "shape"),
    (8, 1, -1, 1, 2, P, P, "shape"),
    (8, 1, 0, 0, 2, P, P, "n_workgroups"),
    (8, 1, 1, 1, 0, P, P, "iterations"),
    (8, 1, 0, 1, 2, NULL, P, "null"),
    (8, 1, 1, 1, 2, P, NULL, "null"),
])
def test_mix_validation(rd, sm, shape, nwg, iters, seed, out, why):
    L = ceilings.lib()
    assert L.fa_ceiling_mix(rd, sm, shape, nwg, iters, seed, out, NULL) == 1
    assert why in L.fa_ceiling_last_error().decode()


def test_mix_flop_count():
    # 2 workgroups x 8 waves x 3 iterations x 8 products x (32 x 32 x 16 x 2)
    assert ceilings.mix_flop(2, 3) == 2 * 8 * 3 * 8 * 32768
    assert ceilings.mix_flop(2, 3, shape=1) == 2 * 8 * 3 * 8 * 16384


@pytest.mark.parametrize("kind,nwg,threads,iters,out,cyc,why", [
    (3, 1, 256, 1, P, P, "kind"),
    (-1, 1, 256, 1, P, P, "kind"),
    (0, 0, 256, 1, P, P, "n_workgroups"),
    (0, 1, 96, 1, P, P, "threads"),
    (0, 1, 2048, 1, P, P, "threads"),
    (0, 1, 0, 1, P, P, "threads"),
    (1, 1, 256, 0, P, P, "iterations"),
    (2, 1, 256, 1, NULL, P, "null"),
    (2, 1, 256, 1, P, NULL, "null"),
])
def test_valu_validation(kind, nwg, threads, iters, out, cyc, why):
    L = ceilings.lib()
    assert L.fa_ceiling_valu(kind, nwg, threads, iters, out, cyc, NULL) == 1
    assert why in L.fa_ceiling_last_error().decode()


def test_phase_stamp_patch_applies_to_the_prefill_source():
    # the stamping tool patches the prefill kernel by anchors; they must still be there
    import os

    from sparse_attention_layerrouter_amd import phase_stamps

    path = os.path.join(os.path.dirname(phase_stamps.__file__), "csrc", "prefill.hip")
    with open(path) as f:
        src = f.read()
    out = phase_stamps._instrument(src)
    assert "fa_stamps_read" in out and out.count("__builtin_amdgcn_s_memtime()") == 1
    assert out.count("g_wg + (size_t)blockIdx.x * 8") == 1
