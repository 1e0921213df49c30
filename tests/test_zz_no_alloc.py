"""fdk_attention_noalloc (the entry point for callers that cannot allocate)
against fdk_attention, which allocates its own buffers: the same kernels on
the same inputs, so the outputs must agree bit for bit.  Two calls in a row
on the shared per-GPU scratch, the second with a smaller input (the first
call's contents are still in the scratch), then the oversize refusal.
"""
import math

import numpy as np
import pytest

import transformer_latent_pixel_amd as fd
import workloads as W
from gpu_util import bf16_bits, dev, say, torch_cuda

pytestmark = pytest.mark.gpu


def _inputs(seed, heads, kv, n, hd, nf):
    fold = math.log2(math.e) / math.sqrt(hd)
    q = W.standard_normal(seed, 1, heads * n * hd).reshape(heads, n, hd) * 1.5
    k = W.standard_normal(seed, 2, nf * kv * n * hd).reshape(nf, kv, n, hd) * 1.5
    v = W.standard_normal(seed, 3, nf * kv * n * hd).reshape(nf, kv, n, hd)
    return [dev(bf16_bits(x).view(np.int16)) for x in (q * fold, k, v)]


def _both(heads, kv, n, hd, nf, first, splits, seed):
    torch = torch_cuda()
    q, k, v = _inputs(seed, heads, kv, n, hd, nf)
    ref = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    got = torch.full((n, heads * hd), 0x7FC0, dtype=torch.int16, device="cuda")
    fd.fdk_attention(q, k, v, nf, first, heads, n, hd, ref, kv_heads=kv, splits=splits)
    stream = torch.cuda.current_stream()
    fd.fdk_attention_noalloc(q, k, v, nf, first, heads, n, hd, got, stream=stream,
                             kv_heads=kv, splits=splits)
    torch.cuda.synchronize()
    a, b = got.cpu().numpy(), ref.cpu().numpy()
    say(f"noalloc heads={heads} kv={kv} n={n} hd={hd} frames={nf} splits={splits}: "
        f"{int((a != b).sum())} of {a.size} differ")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cases", [
    # first call, then a smaller one on the same scratch
    [(16, 16, 1560, 64, 2, 1, 0), (4, 4, 300, 64, 2, 0, 0)],      # 4 key splits each
    [(8, 2, 1000, 64, 3, 2, 2), (2, 1, 37, 64, 1, 0, 1)],         # GQA, then one split
    [(4, 4, 300, 16, 2, 1, 0), (3, 3, 5, 16, 2, 0, 0)],           # head_dim 16 kernel
])
def test_noalloc_matches_allocating_entry_point_on_consecutive_calls(cases):
    for i, c in enumerate(cases):
        _both(*c, seed=40 + i)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    torch = torch_cuda()
    heads, n, hd, nf = 64, 8160, 64, 2          # ring alone ~268 MB > 48 MiB
    z = torch.zeros(16, dtype=torch.int16, device="cuda")
    lib = fd.load_library()
    st = lib.fdk_attention_noalloc(z.data_ptr(), z.data_ptr(), z.data_ptr(), nf, 0, heads,
                                   heads, n, hd, 0, z.data_ptr(), None)
    assert st == fd.FD_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not z.cpu().numpy().any()            # nothing was enqueued
