"""Pins for Philox4x32-10, the 16-point RHT, stochastic rounding and the NVFP4
two-level quantizer (oracle side, no GPU)."""
import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import hadamard as H
from oracle import nvfp4 as Q
from oracle import philox as P
import synth

HERE = os.path.dirname(__file__)
GOLD = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "philox_ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "philox_ref", "rocrand_philox_ref.cpp"),
                    "-o", exe], check=True, capture_output=True)
    def run(seed, subseq, n):
        out = subprocess.run([exe, str(seed), str(subseq), str(n)], check=True,
                             capture_output=True, text=True).stdout.split()
        return np.array([int(v) for v in out], dtype=np.uint32)
    return run


@pytest.mark.parametrize("seed,subseq", [(0, 0), (0x123456789ABCDEF, 0), (42, 1), (7, 0)])
def test_philox_vs_rocrand(rocrand_ref, seed, subseq):
    n = 4096
    ref = rocrand_ref(seed, subseq, n)
    got = P.stream_words(seed, np.arange(n), subsequence=subseq)
    assert np.array_equal(got, ref)


def test_philox_uniformity():
    from scipy import stats
    w = P.stream_words(99, np.arange(1 << 18))
    counts = np.bincount((w >> np.uint32(24)).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_sylvester_and_orthogonality():
    h = H.sylvester16()
    assert np.array_equal(h @ h, 16 * np.eye(16))
    s = H.sign_vector(5)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    ht = h * s[None, :] / 4.0
    assert np.allclose(ht @ ht.T, np.eye(16), atol=0)


def test_rht_matches_dense_and_inverts():
    x = synth.normal_f32(8, (64, 128)).astype(np.float64)
    s = H.sign_vector(123)
    z = H.rht16(x, s)
    zd = H.rht16_dense(x, s)
    assert np.all(np.abs(z - zd) <= 4 * 2.0 ** -24 * np.abs(x).reshape(-1, 16).sum(1).repeat(16).reshape(x.shape))
    # inverse of H16 diag(s)/4 is diag(s) H16 / 4
    h = H.sylvester16()
    back = ((z.reshape(-1, 16) @ h.T) / 4.0 * s[None, :]).reshape(x.shape)
    assert np.max(np.abs(back - x)) < 1e-5


def test_rht_gemm_invariance():
    a = synth.normal_f32(1, (32, 64)).astype(np.float64)
    b = synth.normal_f32(2, (48, 64)).astype(np.float64)
    s = H.sign_vector(9)
    c, bound = G.reference(a, b.T)
    c2, _ = G.reference(H.rht16(a, s), H.rht16(b, s).T)
    assert np.all(np.abs(c - c2) <= 1e-5 * bound)


def test_sr_page_example():
    """3.6 rounds to 3 or 4 with P(4) = 0.6 (gist.science lay summary)."""
    ex = GOLD["sr_example"]
    y = np.full(1 << 20, float(F.f32(ex["value"])))
    w = P.stream_words(2024, np.arange(y.size)).astype(np.float64)
    u = np.floor(w / 256.0) * 2.0 ** -24
    q = Q._sr_e2m1(y, u)
    assert set(np.unique(q)) == set(float(v) for v in ex["neighbours"])
    p = float(F.f32(ex["value"])) - 3.0
    freq = np.mean(q == 4.0)
    sigma = np.sqrt(p * (1 - p) / y.size)
    assert abs(freq - p) < 5 * sigma


def test_sr_unbiased_and_on_grid():
    y = F.f32(np.random.default_rng(0).uniform(-6, 6, 2000))
    reps = 512
    yy = np.repeat(y, reps)
    w = P.stream_words(7, np.arange(yy.size)).astype(np.float64)
    u = np.floor(w / 256.0) * 2.0 ** -24
    q = Q._sr_e2m1(yy, u).reshape(-1, reps)
    lo = np.array([Q.E2M1_MAG[np.searchsorted(Q.E2M1_MAG, abs(v), side="right") - 1] for v in y])
    hi = np.array([Q.E2M1_MAG[min(np.searchsorted(Q.E2M1_MAG, abs(v), side="right"), 7)] for v in y])
    aq = np.abs(q)
    assert np.all((aq == lo[:, None]) | (aq == hi[:, None]))
    err = q.mean(1) - y
    se = (hi - lo) / 2 / np.sqrt(reps) + 1e-12
    assert np.mean(np.abs(err) < 5 * se) > 0.999


def test_two_level_scale_reaches_top_codes():
    """The element carrying the tensor amax gets block scale 448 and code 6."""
    x = synth.normal_f32(3, (32, 64)).astype(np.float64)
    x[5, 17] = 50.0
    q, s, enc = Q.quantize(x)
    assert enc == float(F.f32(2688.0 / 50.0))
    assert F.decode(s[5, 1], F.E4M3) == 448.0
    codes = Q.unpack(q)
    assert codes[5, 17] == 0x7          # +6
    x[5, 17] = -50.0
    q, s, enc = Q.quantize(x)
    assert Q.unpack(q)[5, 17] == 0xF    # -6


def test_decode_to_bf16_is_exact():
    """Every E2M1 value times every finite E4M3 scale is a BF16 value."""
    e2 = F.decode(np.arange(16), F.E2M1)
    e4 = F.decode(np.arange(256), F.E4M3)
    e4 = e4[np.isfinite(e4)]
    prod = (e2[:, None] * e4[None, :]).ravel()
    assert np.array_equal(F.round_to(prod, F.BF16), prod)


def test_quantize_2d_blocks_and_roundtrip_error():
    x = synth.normal_f32(4, (64, 96)).astype(np.float64)
    q, s, enc = Q.quantize(x, block2d=True)
    assert s.shape == (4, 6)
    b = np.abs(x).reshape(4, 16, 6, 16).max(axis=(1, 3))
    assert np.array_equal(s, F.encode(F.f32(F.f32(b / 6.0) * enc), F.E4M3))
    xd = Q.dequantize(q, s, enc, block2d=True)
    # E2M1 relative step is at most 1/3 of the block scale unit; loose bound
    Sel = np.repeat(np.repeat(F.decode(s, F.E4M3), 16, 0), 16, 1) / enc
    assert np.all(np.abs(xd - x) <= 1.01 * Sel)
    # transposed weight: the 2D quantization of W^T is the transpose of W's
    qt, st, enct = Q.quantize(x, transpose=True, block2d=True)
    assert enct == enc and np.array_equal(st, s.T)
    assert np.array_equal(Q.unpack(qt), Q.unpack(q).T)


def test_quantize_transpose_rht_sr_shapes():
    x = synth.normal_f32(6, (64, 48)).astype(np.float64)
    q, s, enc = Q.quantize(x, transpose=True, rht=True, rht_seed=3, sr=True, sr_seed=11)
    assert q.shape == (48, 32) and s.shape == (48, 4)
    xd = Q.dequantize(q, s, enc)
    z = H.rht16(x.T, H.sign_vector(3))
    Sel = np.repeat(F.decode(s, F.E4M3), 16, 1) / enc
    assert np.all(np.abs(xd - z) <= 2.01 * Sel)


def test_zero_block_and_specials():
    x = np.zeros((16, 32))
    x[0, 16:] = 1.0
    q, s, enc = Q.quantize(x)
    assert s[0, 0] == 0 and np.all(Q.unpack(q)[:, :16] == 0)
    q, s, enc = Q.quantize(np.zeros((16, 16)))
    assert enc == 1.0 and np.all(q == 0)


@pytest.mark.parametrize("sr", [False, True])
def test_row_slice_with_tensor_amax_equals_whole_operand_rows(sr):
    """Quantizing some rows of an operand with the whole operand's amax and
    the rows' global indices gives exactly those rows of the whole
    quantization (codes, block scales, tensor scale) -- the tensor scale is
    the whole tensor's and the stochastic-rounding index is global."""
    x = synth.outlier_bf16_codes(12, (96, 80))
    xv = F.decode(x, F.BF16)
    q, s, enc = Q.quantize(xv, transpose=True, rht=True, rht_seed=5, sr=sr, sr_seed=21)
    A = float(np.max(np.abs(H.rht16(xv.T, H.sign_vector(5)))))
    rows = np.array([3, 17, 40, 79])
    q2, s2, enc2 = Q.quantize(xv[:, rows], transpose=True, rht=True, rht_seed=5, sr=sr,
                              sr_seed=21, tensor_amax=A, row_ids=rows)
    assert enc2 == enc
    assert np.array_equal(q2, q[rows]) and np.array_equal(s2, s[rows])
    # the slice's own amax differs from the tensor's, so without it the codes move
    q3, _, enc3 = Q.quantize(xv[:, rows], transpose=True, rht=True, rht_seed=5, sr=sr,
                             sr_seed=21, row_ids=rows)
    assert enc3 != enc
