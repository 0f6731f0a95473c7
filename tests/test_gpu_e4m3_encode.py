"""GPU parity of pca_e4m3_encode, the E4M3 encoder behind every fp8 result
(KV pages, fused KV epilogue, fp8 GEMM operands).

The kernels use gfx950's conversion instruction on inputs clamped to +-448;
these tests fix it against (a) the oracle's table-based encoder on every
rounding boundary of the format (each midpoint between neighbouring codes,
its neighbours in binary32, the saturation edge, the subnormal range) plus a
million log-uniform values, and (b) torch's own float8_e4m3fn cast on every
finite binary32 value.  Saturating round-to-nearest-even equals
round-to-nearest-even of the value clamped to +-448 (nothing in (448, 464)
rounds past 448, and from 464 up saturation gives 448), which is how (b)
states the expected codes with a cast that would otherwise produce NaN above
464.
"""
import numpy as np
import pytest
import torch

import prefill_causal_attention_amd as pca
from oracle import fp8

from _gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def _boundary_values() -> np.ndarray:
    t = fp8.decode_table()[:0x7F].astype(np.float32)        # 0 .. 448, every positive code
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)   # exact in binary32
    vals = [t, mids]
    for k in (1, 2, 3):
        for base in (t, mids):
            up = base.copy()
            dn = base.copy()
            for _ in range(k):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            vals += [up, dn]
    tiny = np.float32(2.0 ** -10)                             # half the smallest subnormal: a tie to 0
    vals.append(np.array([0.0, tiny, np.nextafter(tiny, np.float32(1)), 3 * tiny, 5 * tiny,
                          np.float32(2.0 ** -126), np.float32(1e-45), 448.0, 463.99997, 464.0,
                          np.nextafter(np.float32(464), np.float32(1e9)), 480.0, 1e6,
                          np.finfo(np.float32).max], dtype=np.float32))
    v = np.concatenate([np.abs(a) for a in vals]).astype(np.float32)
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_oracle_on_rounding_boundaries():
    require_gpu()
    rng = np.random.default_rng(9001)
    rand = (rng.choice([-1.0, 1.0], 1 << 20) * 2.0 ** rng.uniform(-12, 10, 1 << 20)).astype(np.float32)
    x = np.concatenate([_boundary_values(), rand])
    x = x[: len(x) - (len(x) % 4) - 1]                         # odd length: the scalar tail runs too
    n = len(x)
    say(f"e4m3_encode boundaries+random n={n} seed=9001")
    xd = torch.from_numpy(x).cuda()
    out = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    pca.e4m3_encode(xd, out[:n])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = fp8.encode(x.astype(np.float64))
    bad = np.nonzero(got[:n] != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]
    assert np.all(got[n:] == 0xA5)                              # nothing written past n


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 8])
def test_e4m3_encode_short_lengths(n):
    require_gpu()
    x = np.array([0.3, -448.0, 1e5, -0.0, 2.0 ** -9, 3 * 2.0 ** -10, -17.5, 240.0][:n], dtype=np.float32)
    say(f"e4m3_encode n={n}")
    out = torch.full((16,), 0xA5, dtype=torch.uint8, device="cuda")
    pca.e4m3_encode(torch.from_numpy(x).cuda(), out[:n])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:n], fp8.encode(x.astype(np.float64)))
    assert np.all(got[n:] == 0xA5)


def test_e4m3_encode_every_finite_fp32_matches_torch_cast():
    require_gpu()
    chunk = 1 << 28
    end = 0x7F800000                                            # +inf's bit pattern: all finite below
    mism = 0
    for sign in (0, -(1 << 31)):
        for start in range(0, end, chunk):
            say(f"e4m3_encode exhaustive sign={'-' if sign else '+'} bits [{start:#x}, {min(start + chunk, end):#x})")
            b = torch.arange(start, min(start + chunk, end), dtype=torch.int32, device="cuda")
            if sign:
                b |= sign
            x = b.view(torch.float32)
            got = torch.empty(x.numel(), dtype=torch.uint8, device="cuda")
            pca.e4m3_encode(x, got)
            want = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            ne = got != want
            cnt = int(ne.sum())
            if cnt:
                i = int(torch.nonzero(ne)[0])
                say(f"first mismatch bits={int(b[i]) & 0xFFFFFFFF:#010x} got={int(got[i]):#x} want={int(want[i]):#x}")
            mism += cnt
            del b, x, got, want, ne
    torch.cuda.synchronize()
    assert mism == 0
