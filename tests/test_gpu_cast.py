"""The P-cast conversion on the GPU, bit for bit against the oracle's E4M3 rounding.

pcast_cast_e4m3 runs the conversion device code of the attention kernels on a
caller array.  The P-cast summary ("Ottimizzazione 2", point 1) says that scaling
by a power of two is exact in fp32, so for S = 2^k the code must be that of the
exact product S*p rounded to nearest even onto the E4M3 grid (3 mantissa bits,
subnormal step 2^-9, values at or below 2^-10 to zero; section 1).  Checked here
for every fp32 probability p whose product S*p has an exponent in [-12, 9] (and
p <= 1), i.e. every binade where a code can be non-zero, for S = 2^0 .. 2^9, with
p = 0 and p = 1 besides.  For S = 3 and 448 the kernel rounds the product to fp32
first (the product is not exact there, as the summary notes for 448), so the codes
must equal the RNE of fl32(S*p).  S = 512 saturates: the codes of min(512 p, 448).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import core, e4m3

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MANT = 1 << 23
# value of every non-negative finite code 0x00 .. 0x7E, from the field definition
_TABLE = np.array([e4m3.decode_code(c) for c in range(256)])


@pytest.fixture(scope="module")
def sna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_numerics_amd
    softmax_numerics_amd.load_library()
    return softmax_numerics_amd


def _oracle_rne(x):
    """oracle E4M3 RNE (C core) of a float64 array, on 8 threads."""
    parts = np.array_split(x, 8)
    with ThreadPoolExecutor(8) as ex:
        return np.concatenate(list(ex.map(core.e4m3_rne, parts)))


def _gpu_codes(sna, p_dev, S):
    codes = torch.empty(p_dev.numel(), dtype=torch.uint8, device=p_dev.device)
    rc = sna.cast_e4m3(p_dev.data_ptr(), codes.data_ptr(), p_dev.numel(), S,
                       torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sna.strerror(rc)
    torch.cuda.synchronize()
    return codes.cpu().numpy()


def _binades(S):
    """Exponents e of the binades [2^e, 2^(e+1)) of p to cover: S*p from 2^-12 (S*p below
    2^-12 < 2^-10 is zero anyway) up to p < 1."""
    lo = int(np.floor(np.log2(2.0 ** -12 / S)))
    return list(range(lo, 0))


def _expected(p, S):
    if float(S).is_integer() and S == 2.0 ** round(np.log2(S)) and S <= 448:
        y = p.astype(np.float64) * S                       # exact: a power-of-two scale
    elif S > 448:
        y = np.minimum(p.astype(np.float64) * S, 448.0)    # saturating
    else:
        y = (p * np.float32(S)).astype(np.float64)         # fl32(S*p), then RNE
    return _oracle_rne(y)


@pytest.mark.parametrize("S", [float(2 ** k) for k in range(10)] + [3.0, 448.0, 512.0])
def test_cast_every_fp32_probability(sna, S):
    print(f"\n[case] cast S={S}: binades {_binades(S)[0]}..-1 of p, plus 0 and 1", flush=True)
    dev = torch.device("cuda:0")
    ramp = torch.arange(MANT, dtype=torch.int32, device=dev)
    ramp_np = np.arange(MANT, dtype=np.uint32)
    checked = 0
    for e in _binades(S):
        base = (e + 127) << 23
        p_dev = (ramp + base).view(torch.float32)
        got = _gpu_codes(sna, p_dev, S)
        assert got.max() <= 0x7E, f"binade 2^{e}: code above 0x7E"
        p = (ramp_np + np.uint32(base)).view(np.float32)
        want = _expected(p, S)
        bad = _TABLE[got] != want
        assert not bad.any(), (f"S={S}, binade 2^{e}: {int(bad.sum())} codes differ; first p = "
                               f"{float(p[bad][0])!r}: got {_TABLE[got][bad][0]!r}, want {want[bad][0]!r}")
        checked += MANT
    ends = torch.tensor([0.0, 0.0, 1.0, 1.0], dtype=torch.float32, device=dev)
    got = _gpu_codes(sna, ends, S)
    want = _expected(np.array([0.0, 0.0, 1.0, 1.0], dtype=np.float32), S)
    assert np.array_equal(_TABLE[got], want) and got[0] == 0
    print(f"[case] cast S={S}: {checked} values bit-identical", flush=True)


def test_cast_rejects_bad_arguments(sna):
    p = torch.zeros(8, dtype=torch.float32, device="cuda")
    c = torch.zeros(8, dtype=torch.uint8, device="cuda")
    assert sna.cast_e4m3(p.data_ptr(), c.data_ptr(), 6, 256.0, 0) == sna.PCAST_EINVAL
    assert sna.cast_e4m3(p.data_ptr(), c.data_ptr(), 8, 0.0, 0) == sna.PCAST_EINVAL
