"""The benchmark's MFMA ceiling probe (bench_probe/librfqprobe.so) without a
GPU: it builds apart from librfq.so, exports its two calls, and rejects bad
arguments on the host before anything is launched."""
import pytest

import bench_probe
from mxfp4_activation_gemm_amd import _lib

FAKE = 0x10000000          # a well-aligned non-null address; never dereferenced here

pytestmark = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                reason="fake-pointer validation checks run on hosts without a GPU")


@pytest.fixture(scope="module")
def lib():
    return bench_probe.load()


def test_probe_is_not_part_of_the_layer_library():
    layer = _lib.load()
    for name in bench_probe.SIGNATURES:
        assert not hasattr(layer, name), name


@pytest.mark.parametrize("name", sorted(bench_probe.SIGNATURES))
def test_probe_validation(lib, name):
    def pr(a=FAKE, an=4096, b=FAKE, bn=4096, wg=4, it=10, st=FAKE, sink=FAKE):
        return getattr(lib, name)(a, an, b, bn, wg, it, st, sink, None)
    for bad in (dict(a=None), dict(sink=None), dict(a=FAKE + 8), dict(an=8), dict(bn=4100), dict(wg=0),
                dict(it=0)):
        assert pr(**bad) == 1, bad
