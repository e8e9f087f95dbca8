"""Helpers for GPU parity tests: host arrays -> device tensors and bitwise comparison."""
import sys

import numpy as np
import pytest

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    torch = None
    HAVE_GPU = False

requires_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")


def say(*a):
    """Progress line naming the case, flushed before the GPU step runs."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def match_rate(a, b):
    a, b = bits(a), bits(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.mean(a == b)) if a.size else 1.0


def assert_bitwise(got, want, what=""):
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d/%d words differ; first at %s: got %r want %r" %
                             (what, len(bad), g.size, i, np.asarray(got)[i], np.asarray(want)[i]))
