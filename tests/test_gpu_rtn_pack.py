"""GPU parity: grid fit, round-to-nearest and packing are bit-exact with the oracle."""
import numpy as np
import pytest

import qz_synth
from conftest import golden
from gpu_util import qz, to_dev, to_host
from oracle import grid, pack

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", golden("rtn_cases.json")["cases"])
def test_rtn_golden(case):
    q = qz()
    v = np.array(case["v"], np.float32)
    codes, s, z = q.qz_rtn(to_dev(v), case["bits"], case["group"])
    np.testing.assert_array_equal(to_host(s), np.array(case["scale_f32"], np.float32))
    np.testing.assert_array_equal(to_host(z), np.array(case["zero"], np.uint8))
    np.testing.assert_array_equal(to_host(codes), np.array(case["codes"], np.uint8))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape,group", [((64, 128), 128), ((70, 200), 8), ((5, 96), 1),
                                         ((33, 384), 128), ((1, 4096), 4096)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rtn_bit_exact(bits, shape, group, dtype):
    q = qz()
    d_o, d_i = shape
    if dtype == "bf16":
        wb = qz_synth.weights_bf16(11 + bits, d_o, d_i)
        wf = qz_synth.bf16_bits_to_f32(wb)
        W = to_dev(wb)
    else:
        wf = (np.random.default_rng(bits).standard_normal((d_o, d_i)) * 0.02).astype(np.float32)
        wf[0, :min(d_i, group)] = 0.0       # an all-zero group when it fits
        W = to_dev(wf)
    codes, s, z = q.qz_rtn(W, bits, group)
    s_ref, z_ref = grid.fit_grid_f32(wf, bits, group)
    np.testing.assert_array_equal(to_host(s), s_ref)
    np.testing.assert_array_equal(to_host(z), z_ref)
    np.testing.assert_array_equal(to_host(codes), grid.rtn_f32(wf, s_ref, z_ref, bits, group))


def test_rtn_caller_grid_clamps():
    q = qz()
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    s = np.full((8, 4), 0.01, np.float32)
    z = np.full((8, 4), 3, np.uint8)
    codes, _, _ = q.qz_rtn(to_dev(w), 3, 16, scales=to_dev(s), zeros=to_dev(z))
    np.testing.assert_array_equal(to_host(codes), grid.rtn_f32(w, s, z, 3, 16))


def test_rtn_rejects_nonfinite():
    q = qz()
    w = np.zeros((4, 32), np.float32)
    w[2, 5] = np.nan
    with pytest.raises(q.QzError) as e:
        q.qz_rtn(to_dev(w), 3, 16)
    assert e.value.status == -3


@pytest.mark.parametrize("bits", list(range(1, 9)))
@pytest.mark.parametrize("cols", [1, 11, 32, 128, 131, 4096])
def test_pack_bit_exact(bits, cols):
    q = qz()
    codes = np.random.default_rng(bits * 100 + cols).integers(0, 1 << bits, (9, cols)).astype(np.uint8)
    words = q.qz_pack(to_dev(codes), bits)
    w_ref = pack.pack(codes, bits)
    np.testing.assert_array_equal(to_host(words).view(np.uint32), w_ref)
    back = q.qz_unpack(words, cols, bits)
    np.testing.assert_array_equal(to_host(back), codes)


@pytest.mark.parametrize("case", golden("pack_cases.json")["cases"])
def test_pack_golden(case):
    q = qz()
    codes = np.array(case["codes"], np.uint8)
    words = q.qz_pack(to_dev(codes), case["bits"])
    np.testing.assert_array_equal(to_host(words).view(np.uint32),
                                  np.array(case["words"], np.uint64).astype(np.uint32))


@pytest.mark.parametrize("offset", [1, 16])
@pytest.mark.parametrize("bits", [3, 5, 8])
def test_pack_code_alignment(offset, bits):
    # rows of 64 codes starting 1 byte (the per-word kernel) or 16 bytes (the 32-code
    # unit kernel) into an allocation: the same words either way
    q = qz()
    import torch
    rows, cols = 7, 64
    codes = np.random.default_rng(offset * 10 + bits).integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    buf = torch.zeros(offset + rows * cols, dtype=torch.uint8, device="cuda")
    view = buf[offset:].view(rows, cols)
    view.copy_(torch.from_numpy(codes).cuda())
    words = q.qz_pack(view, bits)
    np.testing.assert_array_equal(to_host(words).view(np.uint32), pack.pack(codes, bits))


def test_pack_full_size_roundtrip():
    # 4096 x 12288 3-bit codes: round trip exact, sampled rows against the oracle
    q = qz()
    import torch
    codes = torch.randint(0, 8, (12288, 4096), dtype=torch.uint8, device="cuda")
    words = q.qz_pack(codes, 3)
    assert words.shape == (12288, 384)
    back = q.qz_unpack(words, 4096, 3)
    assert torch.equal(back, codes)
    rows = [0, 7, 5000, 12287]
    c_h = to_host(codes[rows])
    np.testing.assert_array_equal(to_host(words[rows]).view(np.uint32), pack.pack(c_h, 3))


def test_empty_inputs():
    q = qz()
    import torch
    codes = torch.empty((0, 16), dtype=torch.uint8, device="cuda")
    assert q.qz_pack(codes, 3).shape == (0, 2)
    c, s, z = q.qz_rtn(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 3, 8)
    assert c.shape == (0, 16)


def test_rtn_concurrent_streams_keep_their_own_status():
    """Each call's status word lives in its own workspace: a non-finite weight on one
    stream is reported there only, while clean calls on another stream, running at the
    same time from another host thread, keep reporting success."""
    import threading

    import torch
    q = qz()
    good = to_dev(qz_synth.weights_bf16(31, 256, 512))
    badh = qz_synth.bf16_bits_to_f32(qz_synth.weights_bf16(32, 256, 512))
    badh[100, 7] = np.nan
    bad = to_dev(badh)
    ref, _, _ = q.qz_rtn(good, 3, 128)
    ref = to_host(ref)
    errors = {"good": [], "bad": []}

    def run(W, key, n):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(n):
                try:
                    c, _, _ = q.qz_rtn(W, 3, 128)
                    if key == "good" and not np.array_equal(to_host(c), ref):
                        errors[key].append("codes")
                    if key == "bad":
                        errors[key].append("no error")
                except q.QzError as e:
                    if key == "good" or e.status != -3:
                        errors[key].append(str(e))

    th = [threading.Thread(target=run, args=(good, "good", 30)),
          threading.Thread(target=run, args=(bad, "bad", 30))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert errors == {"good": [], "bad": []}
