"""CPU-side checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before touching a device."""
import os
import re

import pytest

import softmax_numerics_amd as sna

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # an aligned non-null address; never dereferenced by the checks below


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sna.LIB_PATH):
        from softmax_numerics_amd import build
        build.build()
    return sna.load_library()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pcast_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decl = r"^(?:const\s+)?(?:unsigned\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s+\*?([a-z_0-9]+)\("
    return set(re.findall(decl, text, flags=re.M))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == set(sna.EXPORTS)
    for name in declared:
        assert hasattr(lib, name)


def test_version_and_sizes(lib):
    assert lib.pcast_abi_version() == 10
    assert sna.stats_words(4, 32, 8192) == 4 * 32 * 128 * 2
    assert sna.stats_words(1, 1, 100) == 4
    assert sna.workspace_bytes(4, 32, 8192, 128, 256.0) == 4 * 32 * 8192 * 128
    assert sna.workspace_bytes(4, 32, 8192, 128, 0.0) == 2 * 4 * 32 * 8192 * 128


def test_sizes_for_any_sequence_length(lib):
    # the V copy and the counters take whole 64-key blocks
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for N in (1, 63, 65, 100, 4097):
        nb = (N + 63) // 64
        assert sna.workspace_bytes(2, 3, N, 128, 256.0) == 2 * 3 * nb * 64 * 128
        assert sna.workspace_bytes(2, 3, N, 64, 0.0) == 2 * 2 * 3 * nb * 64 * 64
        assert sna.stats_words(2, 5, N) == 2 * 5 * nb * 2
        # rotated FP8 logits: K codes in whole blocks, Q codes and exponents per row
        nkv, nq = 2 * 3 * nb * 64 * 128, 2 * 6 * N * 128
        base = up(up(up(nkv) + nkv) + 4 * 2 * 3 * nb)
        assert sna.workspace_bytes_qk8_rot(2, 6, 3, N, 128) == up(up(base + nq) + 4 * 2 * 6 * N)


def _call(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1, S=256.0,
             order=1, out=FAKE, stats=0, stream=0)
    a.update(kw)
    return sna.attn_fwd_pcast(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(out=0), sna.PCAST_EINVAL),
    (dict(B=0), sna.PCAST_EINVAL),
    (dict(Hq=3, Hkv=2), sna.PCAST_EINVAL),
    (dict(causal=2), sna.PCAST_EINVAL),
    (dict(order=2), sna.PCAST_EINVAL),
    (dict(S=-1.0), sna.PCAST_EINVAL),
    (dict(S=float("nan")), sna.PCAST_EINVAL),
    (dict(S=float("inf")), sna.PCAST_EINVAL),
    (dict(Q=FAKE + 8), sna.PCAST_EINVAL),
    (dict(stats=FAKE + 4), sna.PCAST_EINVAL),
    (dict(d=96), sna.PCAST_ENOTSUP),
])
def test_argument_errors(lib, kw, code):
    assert _call(**kw) == code
    assert sna.strerror(code) != "success"


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(workspace=FAKE + 4), sna.PCAST_EINVAL),
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(order=5), sna.PCAST_EINVAL),
])
def test_prepared_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, workspace=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1,
             S=256.0, order=1, out=FAKE, stats=0, stream=0)
    a.update(kw)
    assert sna.attn_fwd_pcast_prepared(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(V=0), sna.PCAST_EINVAL),
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(S=-2.0), sna.PCAST_EINVAL),
    (dict(d=32), sna.PCAST_ENOTSUP),
])
def test_prepare_argument_errors(lib, kw, code):
    a = dict(V=FAKE, B=1, Hkv=1, N=128, d=128, S=256.0, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.prepare_v(**a) == code


def test_qk8_workspace_layout(lib):
    # V codes, K codes, one int32 exponent per key block, each 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hkv, N, d in ((4, 32, 8192, 128), (1, 1, 64, 64), (2, 3, 192, 128), (2, 3, 100, 64)):
        nb = -(-N // 64)  # whole key blocks: the codes and the V copy of a partial block are padded
        nkv = B * Hkv * nb * 64 * d
        assert sna.workspace_bytes_qk8(B, Hkv, N, d) == up(up(up(nkv) + nkv) + 4 * B * Hkv * nb)
    assert sna.workspace_bytes_qk8(0, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(V=0), sna.PCAST_EINVAL),
    (dict(V=FAKE + 2), sna.PCAST_EINVAL),
    (dict(out=0), sna.PCAST_EINVAL),
    (dict(causal=3), sna.PCAST_EINVAL),
    (dict(S=float("nan")), sna.PCAST_EINVAL),
    (dict(Hq=3, Hkv=2), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_ENOTSUP),
    (dict(d=96), sna.PCAST_ENOTSUP),
])
def test_qk8_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1, S=256.0,
             order=1, out=FAKE, stats=0, stream=0)
    a.update(kw)
    assert sna.attn_fwd_pcast_qk8(**a) == code
    p = dict(Q=FAKE, workspace=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1, S=256.0, order=1,
             out=FAKE, stats=0, stream=0)
    if set(kw) <= set(p):
        p.update(kw)
        assert sna.attn_fwd_pcast_qk8_prepared(**p) == code


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), sna.PCAST_EINVAL),
    (dict(V=FAKE + 8), sna.PCAST_EINVAL),
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(B=0), sna.PCAST_EINVAL),
    (dict(d=32), sna.PCAST_ENOTSUP),
])
def test_prepare_qk8_argument_errors(lib, kw, code):
    a = dict(K=FAKE, V=FAKE, B=1, Hkv=1, N=128, d=128, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.prepare_qk8(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(lse=FAKE + 2), sna.PCAST_EINVAL),
    (dict(lost=FAKE + 1), sna.PCAST_EINVAL),
    (dict(order=3), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_ENOTSUP),
    (dict(d=32), sna.PCAST_ENOTSUP),
])
def test_rows_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, workspace=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1,
             S=256.0, order=1, out=FAKE, stats=0, lse=FAKE, lost=FAKE, stream=0)
    a.update(kw)
    assert sna.attn_fwd_pcast_rows(**a) == code


def test_decode_workspace_layout(lib):
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hkv, Nk, d, split in ((16, 8, 16384, 128, 1024), (1, 1, 64, 64, 64), (2, 3, 1000 * 64, 128, 4096)):
        n = -(-Nk // split)
        slots = B * Hkv * n * 32
        want = up(up(up(slots * d * 4) + slots * 8) + slots * 8)
        assert sna.decode_workspace_bytes(B, Hkv, Nk, d, split) == want
    assert sna.decode_workspace_bytes(1, 1, 64, 64, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(vop=0), sna.PCAST_EINVAL),
    (dict(workspace=FAKE + 8), sna.PCAST_EINVAL),
    (dict(Nq=0), sna.PCAST_EINVAL),
    (dict(Nq=4, Nk=3), sna.PCAST_EINVAL),  # more rows than cached keys
    (dict(split_keys=100), sna.PCAST_EINVAL),
    (dict(split_keys=0), sna.PCAST_EINVAL),
    (dict(order=2), sna.PCAST_EINVAL),
    (dict(Hq=3, Hkv=2), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_ENOTSUP),
    (dict(Hq=32, Hkv=8, Nq=9), sna.PCAST_ENOTSUP),
    (dict(d=80), sna.PCAST_ENOTSUP),
])
def test_decode_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, vop=FAKE, bias=0, B=1, Hq=8, Hkv=2, Nq=1, Nk=1024, d=128, S=256.0, order=1,
             split_keys=256, out=FAKE, stats=0, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.attn_decode_pcast(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(qk8_workspace=0), sna.PCAST_EINVAL),
    (dict(qk8_workspace=FAKE + 8), sna.PCAST_EINVAL),
    (dict(out=FAKE + 4), sna.PCAST_EINVAL),
    (dict(split_keys=100), sna.PCAST_EINVAL),
    (dict(order=3), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_ENOTSUP),
    (dict(Hq=32, Hkv=8, Nq=9), sna.PCAST_ENOTSUP),
    (dict(d=80), sna.PCAST_ENOTSUP),
])
def test_decode_qk8_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, qk8_workspace=FAKE, bias=0, B=1, Hq=8, Hkv=2, Nq=1, Nk=1024, d=128, S=256.0, order=1,
             split_keys=256, out=FAKE, stats=0, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.attn_decode_pcast_qk8(**a) == code


def test_bwd_workspace_layout(lib):
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hq, Hkv, N, d in ((4, 32, 32, 8192, 128), (1, 3, 1, 64, 64)):
        want = 2 * up(4 * B * Hq * N)  # -D and -lse * sqrt(d) per row, fp32
        assert sna.bwd_workspace_bytes(B, Hq, Hkv, N, d) == want
    # N not a multiple of 64: the row workspace of Np = whole blocks, then the padded copies of
    # Q, K, V (bf16), O (fp32), dO (bf16), lse, the bias (Np floats) and dQ, dK, dV (fp32)
    for B, Hq, Hkv, N, d in ((2, 4, 2, 100, 64), (1, 8, 1, 1000, 128)):
        Np = -(-N // 64) * 64
        nq, nk = B * Hq * Np * d, B * Hkv * Np * d
        off = 2 * up(4 * B * Hq * Np)
        for size in (2 * nq, 2 * nk, 2 * nk, 4 * nq, 2 * nq, 4 * B * Hq * Np, 4 * Np, 4 * nq, 4 * nk, 4 * nk):
            off = up(off) + size
        assert sna.bwd_workspace_bytes(B, Hq, Hkv, N, d) == up(off)


@pytest.mark.parametrize("kw,code", [
    (dict(O=0), sna.PCAST_EINVAL),
    (dict(dO=FAKE + 2), sna.PCAST_EINVAL),
    (dict(lse=FAKE + 1), sna.PCAST_EINVAL),
    (dict(dV=0), sna.PCAST_EINVAL),
    (dict(causal=5), sna.PCAST_EINVAL),
    (dict(Hq=3, Hkv=2), sna.PCAST_EINVAL),
    (dict(d=96), sna.PCAST_ENOTSUP),
    (dict(N=1 << 23), sna.PCAST_ENOTSUP),  # one head's rows reach 2 GiB
    (dict(N=(1 << 23) - 5), sna.PCAST_ENOTSUP),  # the same with the rows padded to whole blocks
])
def test_bwd_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, lse=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128,
             causal=1, dQ=FAKE, dK=FAKE, dV=FAKE, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.attn_bwd_pcast(**a) == code


def test_qk8_rot_workspace_layout(lib):
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for B, Hq, Hkv, N, d in ((4, 32, 32, 8192, 128), (1, 3, 1, 64, 64)):
        nkv, nq = B * Hkv * N * d, B * Hq * N * d
        base = up(up(up(nkv) + nkv) + 4 * B * Hkv * (N // 64))
        assert sna.workspace_bytes_qk8_rot(B, Hq, Hkv, N, d) == up(up(base + nq) + 4 * B * Hq * N)


@pytest.mark.parametrize("kw,code", [
    (dict(signs=0), sna.PCAST_EINVAL),
    (dict(signs=FAKE + 8), sna.PCAST_EINVAL),
    (dict(Q=FAKE + 4), sna.PCAST_EINVAL),
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(d=96), sna.PCAST_ENOTSUP),
])
def test_prepare_qk8_rot_argument_errors(lib, kw, code):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, signs=FAKE, B=1, Hq=2, Hkv=1, N=128, d=128, workspace=FAKE, stream=0)
    a.update(kw)
    assert sna.prepare_qk8_rot(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=0), sna.PCAST_EINVAL),
    (dict(out=0), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_ENOTSUP),
])
def test_qk8_rot_prepared_argument_errors(lib, kw, code):
    a = dict(workspace=FAKE, bias=0, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1, S=256.0, order=1, out=FAKE,
             stats=0, stream=0)
    a.update(kw)
    assert sna.attn_fwd_pcast_qk8_rot_prepared(**a) == code


def test_strerror_texts(lib):
    assert sna.strerror(0) == "success"
    _call(d=96)
    assert "d = 96" in sna.strerror(sna.PCAST_ENOTSUP)


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "softmax_numerics_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), f
                assert "pcast_oracle" not in text, f


def test_forward_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sna.forward(q, q, q)


@pytest.mark.parametrize("kw,code", [
    (dict(P=0), sna.PCAST_EINVAL),
    (dict(codes=0), sna.PCAST_EINVAL),
    (dict(P=FAKE + 4), sna.PCAST_EINVAL),
    (dict(codes=FAKE + 2), sna.PCAST_EINVAL),
    (dict(n=6), sna.PCAST_EINVAL),
    (dict(n=-4), sna.PCAST_EINVAL),
    (dict(S=0.0), sna.PCAST_EINVAL),
    (dict(S=-256.0), sna.PCAST_EINVAL),
    (dict(S=float("inf")), sna.PCAST_EINVAL),
])
def test_cast_argument_errors(lib, kw, code):
    a = dict(P=FAKE, codes=FAKE, n=1024, S=256.0, stream=0)
    a.update(kw)
    assert sna.cast_e4m3(**a) == code


def test_noalloc_rejects_inputs_above_its_scratch(lib):
    # 1 x 8 kv heads x 131072 keys x d 128 of E4M3 V = 2^27 bytes, twice the scratch: refused on the host
    rc = sna.attn_fwd_pcast_noalloc(FAKE, FAKE, FAKE, 0, 1, 8, 8, 131072, 128, 1, 256.0, 1, FAKE, 0, 0)
    assert rc == sna.PCAST_ENOTSUP and "scratch" in sna.strerror(rc)
    # S = 0 keeps a bf16 copy: twice the bytes, so half the keys fit
    assert sna.attn_fwd_pcast_noalloc(FAKE, FAKE, FAKE, 0, 1, 4, 4, 131072, 128, 1, 0.0, 1, FAKE, 0, 0) == sna.PCAST_ENOTSUP
    assert sna.attn_fwd_pcast_noalloc(0, FAKE, FAKE, 0, 1, 1, 1, 64, 64, 1, 256.0, 1, FAKE, 0, 0) == sna.PCAST_EINVAL


def _multi(**kw):
    a = dict(Q=FAKE, K=FAKE, workspace=FAKE, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1, biases=[0, 0],
             Ss=[256.0, 1.0], orders=[1, 0], outs=[FAKE, FAKE], stats=None, stream=0)
    a.update(kw)
    return sna.attn_fwd_pcast_multi(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), sna.PCAST_EINVAL),
    (dict(workspace=FAKE + 4), sna.PCAST_EINVAL),
    (dict(causal=2), sna.PCAST_EINVAL),
    (dict(outs=[FAKE, 0]), sna.PCAST_EINVAL),
    (dict(outs=[FAKE, FAKE + 4]), sna.PCAST_EINVAL),
    (dict(orders=[1, 3]), sna.PCAST_EINVAL),
    (dict(Ss=[256.0, float("nan")]), sna.PCAST_EINVAL),
    (dict(Ss=[256.0, -1.0]), sna.PCAST_EINVAL),
    (dict(stats=[FAKE, 0]), sna.PCAST_EINVAL),
    (dict(biases=[FAKE + 2, 0]), sna.PCAST_EINVAL),
    (dict(Ss=[256.0, 0.0]), sna.PCAST_ENOTSUP),
    (dict(d=96), sna.PCAST_ENOTSUP),
    (dict(Hq=3, Hkv=2), sna.PCAST_EINVAL),
])
def test_multi_argument_errors(lib, kw, code):
    assert _multi(**kw) == code


def test_multi_needs_a_configuration(lib):
    a = dict(Q=FAKE, K=FAKE, workspace=FAKE, B=1, Hq=2, Hkv=1, N=128, d=128, causal=1)
    assert sna.load_library().attn_fwd_pcast_multi(a["Q"], a["K"], a["workspace"], 1, 2, 1, 128, 128, 1, 0,
                                                   None, None, None, None, None, None) == sna.PCAST_EINVAL
