"""The ceiling streams on the GPU: the read stream reads every 32-bit word of
its buffer exactly once (the XOR of its per-thread results equals the XOR of
the buffer, computed on the host), and the product stream runs every
(shape, read rate, softmax mix) variant with finite, repeatable output, and the
VALU issue stream runs each kind with finite, repeatable output and every wave's
cycle count written."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,chunk", [(1 << 15, 1 << 15), (3 << 20, 1 << 20),
                                          (64 << 20, 1 << 15), (64 << 20, 4 << 20)])
def test_read_stream_reads_every_word_once(nbytes, chunk):
    import torch

    from sparse_attention_layerrouter_amd import ceilings

    rng = np.random.default_rng(nbytes + chunk)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((nbytes // chunk * 256,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ceilings.fa_ceiling_read(buf, chunk, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # a dropped or repeated 16-byte load per thread changes the per-thread XORs
    per_thread = host.reshape(nbytes // chunk, chunk // 4096, 256, 4)
    expect = np.bitwise_xor.reduce(np.bitwise_xor.reduce(per_thread, axis=3), axis=1).reshape(-1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), expect)


def test_product_stream_variants_run_and_repeat():
    import torch

    from sparse_attention_layerrouter_amd import ceilings

    rng = np.random.default_rng(3)
    bits = ((rng.integers(0, 2, 4096) << 15) | (123 << 7) | rng.integers(0, 128, 4096)).astype(
        np.uint16)
    seed = torch.from_numpy(bits.view(np.int16)).cuda()
    n_wg = 8
    for shape in (0, 1):
        for rd in (0, 2, 4, 6, 8):
            for sm in (False, True):
                a = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
                b = torch.empty_like(a)
                ceilings.fa_ceiling_mix(rd, sm, n_wg, 6, seed, a, shape=shape)
                ceilings.fa_ceiling_mix(rd, sm, n_wg, 6, seed, b, shape=shape)
                torch.cuda.synchronize()
                assert torch.isfinite(a).all(), (shape, rd, sm)
                assert torch.equal(a, b), (shape, rd, sm)


def test_valu_stream_kinds_run_and_repeat():
    import torch

    from sparse_attention_layerrouter_amd import ceilings

    for n_wg, threads in ((4, 1024), (3, 256)):
        for kind in (0, 1, 2):
            a = torch.empty(n_wg * threads, dtype=torch.float32, device="cuda")
            b = torch.empty_like(a)
            cyc = torch.zeros(n_wg * threads // 32, dtype=torch.int64, device="cuda")
            ceilings.fa_ceiling_valu(kind, n_wg, threads, 50, a, cyc)
            ceilings.fa_ceiling_valu(kind, n_wg, threads, 50, b, cyc)
            torch.cuda.synchronize()
            assert torch.isfinite(a).all(), kind
            assert torch.equal(a, b), kind
            assert (cyc.view(-1, 2)[:, 0] > 0).all(), kind  # every wave wrote its ticks
