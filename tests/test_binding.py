"""The Python binding's argument checks, on the CPU: nothing that would hand
the library a host pointer, a strided view or buffers of unequal size or
dtype gets past marshalling, and raw addresses need an explicit count and
dtype.  Stand-in objects play device tensors where a real one would need a
GPU; the binding only reads these attributes from a tensor.
"""
import pytest
import torch

import allreduce_reduction_amd as hc


class FakeDev:
    """Attributes the binding reads from a device tensor."""

    def __init__(self, addr, n=64, dtype=torch.float32, contiguous=True, cuda=True):
        self.addr, self.n, self.dtype, self.contig, self.is_cuda = addr, n, dtype, contiguous, cuda

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def is_contiguous(self):
        return self.contig


def fakes(P=4, **kw):
    return [FakeDev(0x100000 * (r + 1), **kw) for r in range(P)]


def test_well_formed_device_tensors_marshal():
    arr, n, dt = hc._ptrs(fakes(4, n=100, dtype=torch.bfloat16))
    assert n == 100 and dt == "bf16"
    assert [arr[r] for r in range(4)] == [0x100000 * (r + 1) for r in range(4)]


@pytest.mark.parametrize("bad", ["host", "strided", "size", "dtype"])
def test_rejected_buffers(bad):
    bufs = fakes(4)
    if bad == "host":
        bufs[2].is_cuda = False
    elif bad == "strided":
        bufs[1].contig = False
    elif bad == "size":
        bufs[3].n = 63
    else:
        bufs[3].dtype = torch.float16
    with pytest.raises(ValueError):
        hc._ptrs(bufs)


def test_unsupported_dtype_and_mixed_lists():
    with pytest.raises(TypeError):
        hc._ptrs(fakes(2, dtype=torch.float64))
    with pytest.raises(TypeError):
        hc._ptrs([fakes(1)[0], 0x200000])


def test_host_tensors_never_reach_the_library():
    with hc.Comm(4, "ring") as c:
        with pytest.raises(ValueError):
            c.allreduce([torch.ones(16) for _ in range(4)])


def test_raw_addresses_need_count_and_dtype():
    with hc.Comm(2, "ring") as c:
        with pytest.raises(ValueError):
            c.allreduce([0x100000, 0x200000])
        with pytest.raises(ValueError):
            c.allreduce([0x100000, 0x200000], "fp32")
        with pytest.raises(ValueError):
            c.out_of_place("allreduce", [0x100000, 0x200000], [0x300000, 0x400000])
