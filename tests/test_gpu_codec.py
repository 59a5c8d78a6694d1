"""GPU check of the device fp32 -> OCP e4m3fn conversion every quantizing
kernel uses, against the oracle's encoder (which is itself pinned to the
format's definition by the CPU tests).

The conversion is exercised through the library's diagnostic entry point
rra_e4m3fn_encode, on:
- every rounding midpoint between adjacent finite e4m3fn values (ties must go
  to the even code) and the four fp32 neighbours on each side of it;
- a strided sweep over every fp32 binade that maps to a normal or subnormal
  code, and the binades below the smallest subnormal;
- saturation: values between 448 and fp32's largest finite value, and +-inf;
- signed zeros.
Codes must agree bit-exactly, except that +0 and -0 are not told apart for
inputs that round to zero (the pages fix no sign for a zero code)."""
import numpy as np
import pytest

from gpu_util import dev, host_u8, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def _midpoints(oracle) -> np.ndarray:
    vals = oracle.e4m3fn_decode_array(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    mids = np.concatenate([mids, np.float32([464.0])])  # half-way to the next binade's 480
    # each midpoint and its fp32 neighbours 1..4 ulps away on either side
    out = [mids]
    up = mids.copy()
    dn = mids.copy()
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up, dn]
    return np.concatenate(out)


def _binade_sweep() -> np.ndarray:
    # exponents 2^-30 .. 2^9, every 2^7-th fp32 mantissa (65536 per binade)
    mant = np.arange(0, 1 << 23, 1 << 7, dtype=np.uint32)
    parts = []
    for e in range(-30, 10):
        bits = (np.uint32(e + 127) << np.uint32(23)) | mant
        parts.append(bits.view(np.float32))
    return np.concatenate(parts)


def _saturation() -> np.ndarray:
    big = np.geomspace(448.0, 3.0e38, 4096).astype(np.float32)
    return np.concatenate([big, np.float32([448.0, 449.0, 463.99997, 464.0, 464.00003, 480.0,
                                            np.inf, np.finfo(np.float32).max])])


def test_device_e4m3fn_matches_oracle(rra, oracle):
    say("[codec] device e4m3fn vs oracle")
    pos = np.concatenate([_midpoints(oracle), _binade_sweep(), _saturation(),
                          np.float32([0.0, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10])])
    x = np.concatenate([pos, -pos]).astype(np.float32)
    # a ragged tail that is not a multiple of the kernel's 4-wide vectors
    x = np.concatenate([x, np.float32([0.3, -7.5, 300.0])])
    gpu = host_u8(rra.e4m3fn_encode(dev(x)))
    ref = oracle.e4m3fn_encode_f32(x)
    same = (gpu == ref) | (((gpu & 0x7F) == 0) & ((ref & 0x7F) == 0))
    bad = np.flatnonzero(~same)
    assert bad.size == 0, [(float(x[i]), hex(gpu[i]), hex(ref[i])) for i in bad[:10]]
    print(dict(values=x.size, mismatches=int(bad.size)), flush=True)


def test_signed_zero_and_extremes(rra, oracle):
    say("[codec] spot values")
    x = np.float32([0.0, -0.0, 448.0, -448.0, 464.0, 1e30, -np.inf, 2.0 ** -6, 2.0 ** -9])
    gpu = host_u8(rra.e4m3fn_encode(dev(x)))
    assert list(gpu[2:]) == [0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x08, 0x01]
    assert gpu[0] & 0x7F == 0 and gpu[1] & 0x7F == 0
