"""The library's plain copy kernel (sms_copy_reference, the bandwidth
reference bench.py times the softmax kernels against): byte-exact copies of
sizes around its 1 KB workgroups, nothing written past the end."""

import sys

import pytest
import torch

from attention_softmax_amd import sms_copy_reference

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("nbytes", [16, 1008, 1024, 1040, 3 * 1024 * 1024 + 48])
def test_copy_is_exact(nbytes):
    say(f"copy reference {nbytes} B")
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    guard = 4096
    dst = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    sms_copy_reference(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all()), "bytes written past the end"


def test_copy_binding_checks():
    a = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        sms_copy_reference(a, torch.zeros(48, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        sms_copy_reference(a, torch.zeros(64, dtype=torch.uint8, device="cpu"))
    with pytest.raises(Exception):
        sms_copy_reference(a[:24], torch.zeros(24, dtype=torch.uint8, device=DEV))  # not 16 B
