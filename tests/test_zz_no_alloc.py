"""The no-allocation decode entry point (fa_attn_decode_noalloc) against
fa_attn_decode: the same kernels over the same inputs, with the split partials in
the library's static device scratch instead of a caller workspace, so outputs
and lse must be bit-identical.  Two calls in a row, the second with a smaller
input (fewer sequences, shorter caches, a different layer kind mix), and a
route-host (per-kind kernel) call; the fused KV append writes the same cache
rows."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_layerrouter_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_decode_matches_workspace_decode(dtype):
    hq, hkv, d = 32, 8, 128
    scale = 1 / math.sqrt(d)
    cases = [  # (batch, max_cache, lengths, route rows, layer, use host route)
        (8, 40000, [40000, 39000, 123, 1, 20000, 64, 65, 33333], [[1, 0]] * 4 + [[0, 1]] * 4, 0,
         False),
        (3, 5000, [5000, 1, 4097], [[0, 0], [0, 0], [0, 0]], 1, True),
    ]
    for i, (B, n_max, lens, r, layer, host) in enumerate(cases):
        kc = synth.device_normal((B, hkv, n_max, d), seed=40 + i, dtype_name=dtype)
        vc = synth.device_normal((B, hkv, n_max, d), seed=50 + i, dtype_name=dtype)
        kc2, vc2 = kc.clone(), vc.clone()
        q = synth.device_normal((B, hq, d), seed=60 + i, dtype_name=dtype)
        kn = synth.device_normal((B, hkv, d), seed=70 + i, dtype_name=dtype)
        vn = synth.device_normal((B, hkv, d), seed=80 + i, dtype_name=dtype)
        cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        r_np = np.array(r, np.uint8)
        rd = torch.from_numpy(r_np).to(DEV)
        rh = r_np if host else None
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        l1 = torch.empty((B, hq), dtype=torch.float32, device=DEV)
        l2 = torch.empty_like(l1)
        _lib.fa_attn_decode(q, o1, kc, vc, cl, rd, layer, 128, 2048, 64, scale, k_new=kn,
                            v_new=vn, lse=l1, route_host=rh)
        _lib.fa_attn_decode_noalloc(q, o2, kc2, vc2, cl, rd, layer, 128, 2048, 64, scale,
                                    k_new=kn, v_new=vn, lse=l2, route_host=rh)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o1), bits(o2)), f"case {i}: outputs differ"
        assert torch.equal(l1, l2), f"case {i}: lse differs"
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2), f"case {i}: caches differ"
        for b, n in enumerate(lens):  # the appended token landed at position n - 1
            assert torch.equal(kc2[b, :, n - 1], kn[b])


def test_noalloc_rejects_partials_above_the_scratch():
    """Host-side size check: batch 512 with 32 heads and 32 splits (a 4096-token
    cache) needs more than the 64 MiB scratch; nothing is launched."""
    q = torch.empty((512, 32, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.empty((512, 8, 4096, 128), dtype=torch.bfloat16, device=DEV)
    cl = torch.full((512,), 4096, dtype=torch.int32, device=DEV)
    rd = torch.ones((512, 1), dtype=torch.uint8, device=DEV)
    with pytest.raises(_lib.FluxAttnError) as e:
        _lib.fa_attn_decode_noalloc(q, torch.empty_like(q), kc, kc, cl, rd, 0, 128, 2048, 64, 0.1)
    assert e.value.status == _lib.FA_ERR_WORKSPACE
