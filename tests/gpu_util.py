"""Helpers for the GPU parity tests: device copies, guard-banded outputs."""
import numpy as np
import torch

CANARY = 0xA5
PAD = 4096            # guard-band bytes before and after every output


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


class Guarded:
    """An output buffer with canary bytes on both sides; `view` is the
    tensor handed to the library, `check()` asserts the bands are intact."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = n
        self.raw = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device=dev())
        self.view = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def check(self):
        r = self.raw.cpu().numpy()
        assert np.all(r[:PAD] == CANARY), "write before the output buffer"
        assert np.all(r[PAD + self.nbytes:] == CANARY), "write past the output buffer"

    def numpy(self):
        return self.view.cpu().numpy()


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def assert_same_bytes(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(got != want)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s: got %s want %s"
                             % (what, len(bad), idx, hex(int(got[idx])), hex(int(want[idx]))))
