"""Pins of the oracle's FP8 E4M3 dequantisation (the KV-page reading of the
pages' reduced-precision cache), against closed forms and against torch's
independent float8_e4m3fn conversion."""
import numpy as np
import torch


def _deq(codes, scale=1.0):
    import oracle
    c = np.asarray(codes, np.uint8).reshape(1, 1, -1)
    return oracle.dequant_e4m3(c, np.full((1, 1), scale, np.float32))[0, 0]


def test_closed_form_codes(orc):
    codes = [0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x40, 0x7E, 0xFE, 0xB8, 0x81]
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 2.0, 448.0, -448.0,
            -1.0, -(2.0 ** -9)]
    got = _deq(codes)
    assert np.array_equal(got, np.array(want, np.float32))
    assert np.signbit(got[1]) and not np.signbit(got[0])
    assert np.all(np.isnan(_deq([0x7F, 0xFF])))


def test_all_codes_against_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = _deq(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # the positive codes are strictly increasing up to the largest finite one
    assert np.all(np.diff(got[:0x7F]) > 0)


def test_scale_products_rounded_once(orc):
    u = 2.0 ** -23
    # exact products
    assert _deq([0x7E], 3.0)[0] == 1344.0
    assert _deq([0x01], 0.5)[0] == 2.0 ** -10
    # 1.875 * (1 + u) = 1.875 + 1.875 ulp -> rounds up to 2 ulp
    assert _deq([0x3F], 1 + u)[0] == np.float32(1.875 + 2 * u)
    # 1.125 * (1 + u) = 1.125 + 1.125 ulp -> rounds down to 1 ulp
    assert _deq([0x39], 1 + u)[0] == np.float32(1.125 + u)
    # 1.5 * (1 + u) = 1.5 + 1.5 ulp: a tie, to even -> 1.5 + 2 ulp
    assert _deq([0x3C], 1 + u)[0] == np.float32(1.5 + 2 * u)
    # per (page, KV head) scales
    import oracle
    c = np.full((2, 3, 4), 0x38, np.uint8)
    s = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    out = oracle.dequant_e4m3(c, s)
    assert np.array_equal(out, np.broadcast_to(s[:, :, None], (2, 3, 4)))
