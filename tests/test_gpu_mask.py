"""GPU parity of the boolean -> additive mask conversion
(``sdpa_mask_convert``) against the oracle ``oracle.mask.mask_convert``:
bit-exact, every element, for sizes that leave every remainder of the 16-byte
chunks and span the grid-stride loop several times."""
import sys

import numpy as np
import pytest
import torch

import attention_flash_sdpa_amd as sdpa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sdpa.load()
    return torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


SHAPES = [(1,), (15,), (16,), (17,), (1000003,), (2, 4, 333, 517), (3, 8192, 1024)]


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_mask_convert_bit_exact(dev, shape, dt):
    from oracle import mask as om

    print(f"mask_convert {shape} {dt}", flush=True)
    sys.stdout.flush()
    g = torch.Generator().manual_seed(sum(shape))
    m = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
    m[torch.rand(shape, generator=g) < 0.5] = 0
    out = torch.full(shape, 1.0, dtype=dt, device=dev)
    sdpa.mask_convert(m.to(dev), out=out)
    torch.cuda.synchronize()
    want = om.mask_convert(m.numpy(), "bf16" if dt == torch.bfloat16 else "f16")
    assert np.array_equal(_bits(out), want.view(np.uint16))


def test_mask_convert_bool_input_and_empty(dev):
    from oracle import mask as om

    m = torch.rand(5, 77, 130) < 0.3
    out = sdpa.mask_convert(m.to(dev), out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), om.mask_convert(m.numpy().astype(np.uint8), "f16").view(np.uint16))
    e = sdpa.mask_convert(torch.zeros(0, dtype=torch.bool, device=dev))
    assert e.numel() == 0


def test_hbm_read_probe_reads_without_writing(dev):
    # the probe's only store is guarded by a fold value random data does not
    # produce: the sink keeps its fill, and the stream stays usable
    print("hbm_read_probe 64 MiB", flush=True)
    g = torch.Generator().manual_seed(3)
    data = torch.randint(-2**31, 2**31 - 1, (16 * 1024 * 1024,), generator=g, dtype=torch.int32).to(dev)
    sink = torch.full((2048,), 7, dtype=torch.int32, device=dev)
    sdpa.hbm_read_probe(data, sink=sink)
    sdpa.hbm_read_probe(data[:4], sink=sink)                # 16 bytes: one partial workgroup
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
