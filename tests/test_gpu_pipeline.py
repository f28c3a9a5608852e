"""Page-pipelined encode to host memory (lynx_encode_to_host): the host copies of the anchor and
residual segments are byte-identical to a plain device encode, for group sizes of one page, a
ragged split, the whole request and more than the request, on one stream and on two."""
import numpy as np
import pytest
import torch

from decode_attention_lynx_amd import lynx, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group_pages", [1, 3, 10, 16])
@pytest.mark.parametrize("two_streams", [False, True])
def test_encode_to_host_matches_device_encode(gpu, group_pages, two_streams):
    P, C, alpha, Hkv, n_pages = 256, 64, 255.0, 2, 10
    print(f"[pipeline] group_pages={group_pages} two_streams={two_streams}", flush=True)
    kv = synth.make_kv_torch(n_pages * P, Hkv, 128, seed=7)
    anc_dev, res_dev = lynx.encode(kv, P, C, alpha)
    cs = torch.cuda.current_stream()
    xs = torch.cuda.Stream() if two_streams else None
    anc_h, res_h = lynx.encode_to_host(kv, P, C, alpha, group_pages, compute_stream=cs, copy_stream=xs)
    (xs or cs).synchronize()
    torch.cuda.synchronize()
    assert anc_h.is_pinned() and res_h.is_pinned()
    assert torch.equal(anc_h, anc_dev.cpu())
    assert torch.equal(res_h, res_dev.cpu())


def test_encode_to_host_reuses_buffers(gpu):
    """Two requests through the same staging buffer and host tensors: the second overwrites the first."""
    P, C, alpha, Hkv, n_pages = 256, 32, 63.0, 1, 6
    xs = torch.cuda.Stream()
    kv1 = synth.make_kv_torch(n_pages * P, Hkv, 128, seed=1)
    kv2 = synth.make_kv_torch(n_pages * P, Hkv, 128, seed=2)
    need = lynx.lib().lynx_encode_to_host_staging_bytes(4, P, Hkv, 128, C)
    staging = torch.empty(need, dtype=torch.uint8, device="cuda")
    a1, r1 = lynx.encode_to_host(kv1, P, C, alpha, 4, staging=staging, copy_stream=xs)
    xs.synchronize()
    first = a1.clone()
    a2, r2 = lynx.encode_to_host(kv2, P, C, alpha, 4, anchor_host=a1, residual_host=r1, staging=staging,
                                 copy_stream=xs)
    xs.synchronize()
    torch.cuda.synchronize()
    ad, rd = lynx.encode(kv2, P, C, alpha)
    assert torch.equal(a2, ad.cpu()) and torch.equal(r2, rd.cpu())
    assert not torch.equal(first, a2)
