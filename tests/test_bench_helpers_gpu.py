"""The measurement helpers behind bench.py's ceilings, through the C ABI: the
chunk-order stream writes, for each 64-token chunk, output unit j = the xor of the
three inputs' unit j mod 1024 (16-byte units), and rejects shapes it cannot walk."""
import numpy as np
import pytest
import torch

import chunked_linear_attention_gla_amd as gla

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("BH,T,segments", [(1, 64, 1), (3, 256, 2), (2, 512, 8)])
def test_chunk_stream_output(BH, T, segments):
    r = np.random.default_rng(7 + BH + T + segments)
    nb = BH * T * 256
    ins = [r.integers(0, 2 ** 32, size=nb // 4, dtype=np.uint32) for _ in range(3)]
    q, k, v = (torch.from_numpy(a.view(np.int32)).cuda() for a in ins)
    o = torch.full((2 * nb // 4,), -1, dtype=torch.int32, device="cuda")
    gla.bench_chunk_stream(q, k, v, o, BH, T, segments)
    torch.cuda.synchronize()
    x = (ins[0] ^ ins[1] ^ ins[2]).reshape(BH * T // 64, 1024, 4)   # chunk, unit, word
    want = np.concatenate([x, x], axis=1).reshape(-1)                # units 0..2047 of each chunk
    assert np.array_equal(o.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("T,segments", [(100, 1), (256, 3), (128, 0)])
def test_chunk_stream_rejects_shapes(T, segments):
    nb = max(T, 64) * 256
    q, k, v = (torch.zeros(nb, dtype=torch.uint8, device="cuda") for _ in range(3))
    o = torch.zeros(2 * nb, dtype=torch.uint8, device="cuda")
    with pytest.raises(gla.GLAError):
        gla.bench_chunk_stream(q, k, v, o, 1, T, segments)
