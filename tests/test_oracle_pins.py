"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test fixes one step of the oracle against a closed form, an invariant, a
library routine, a brute-force loop or a hand-worked example, so that a
dropped term, a wrong sign or index, a transposed operand or a swapped step
order fails at least one of them.  Steps follow the FlashMemory DS-V4
Retriever README, sections "compressed_k format", "Architecture", "Joint
checkpoint + ensemble", "Usage" and the "Inference flow" figure.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
from oracle import OracleConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- fp8 decode

def test_e4m3fn_spot_values_from_spec():
    with open(os.path.join(GOLDEN, "e4m3fn_spot_values.json")) as f:
        g = json.load(f)
    for code, val in g["codes"].items():
        got = oracle.e4m3fn_value(int(code, 16))
        assert got == val, code
        assert math.copysign(1.0, got) == math.copysign(1.0, val), code
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3fn_value(int(code, 16)))


def test_e4m3fn_all_codes_match_torch_cast():
    # library routine: torch's float8_e4m3fn -> float64 view, all 256 codes
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3fn_table()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))


def test_e4m3fn_structure():
    tab = oracle.e4m3fn_table()
    pos = tab[:127]  # 0x00..0x7e
    assert np.all(np.diff(pos) > 0)                     # strictly increasing magnitudes
    assert np.array_equal(tab[128:255], -tab[:127])     # sign bit negates
    assert pos.max() == 448.0                           # largest finite value (not fnuz's 240)
    # subnormal spacing 2^-9, and the first normal continues it
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9, rtol=0, atol=0)


def test_decode_records_little_endian_scale():
    rec = np.zeros((3, 132), np.uint8)
    rec[0, :128] = 0x38                              # 1.0
    rec[0, 128:] = [0x00, 0x00, 0x00, 0x40]          # 2.0 little-endian
    rec[1, :128] = 0xB8                              # -1.0
    rec[1, 128:] = [0x00, 0x00, 0x80, 0x3F]          # 1.0 little-endian
    rec[2, 0] = 0x7E                                 # 448 at dim 0, zeros elsewhere
    rec[2, 128:] = np.frombuffer(np.float32(0.25).tobytes(), np.uint8)
    k = oracle.decode_records(rec)
    assert k.shape == (3, 128)
    assert np.all(k[0] == 2.0)
    assert np.all(k[1] == -1.0)
    assert k[2, 0] == 112.0 and np.all(k[2, 1:] == 0.0)


def test_decode_records_matches_torch_views():
    rng = np.random.default_rng(5)
    rec = rng.integers(0, 256, size=(64, 132), dtype=np.uint8)
    rec[:, :128][rec[:, :128] & 0x7F == 0x7F] = 0x00       # no NaN codes
    rec[:, 128:] = np.frombuffer(rng.uniform(-3, 3, 64).astype("<f4").tobytes(), np.uint8).reshape(64, 4)
    t = torch.from_numpy(rec[:, :128].copy()).view(torch.float8_e4m3fn).double()
    s = torch.from_numpy(rec[:, 128:].copy()).view(torch.float32).double()
    assert np.array_equal(oracle.decode_records(rec), (t * s).numpy())


# --------------------------------------------------------------------------- linear maps

def test_linear_is_out_by_in_without_bias():
    w = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])     # [out=2][in=3]
    x = np.array([1.0, -1.0, 2.0])
    assert np.array_equal(oracle.linear(w, x), [1 - 2 + 6, 4 - 5 + 12])
    rng = np.random.default_rng(0)
    w = rng.standard_normal((5, 7))
    x = rng.standard_normal(7)
    brute = [sum(w[o, i] * x[i] for i in range(7)) for o in range(5)]
    assert np.allclose(oracle.linear(w, x), brute, rtol=1e-14, atol=1e-14)
    assert np.allclose(oracle.linear(np.zeros((4, 3)), np.ones(3)), 0.0)


# --------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_form():
    a = np.array([3.0, 4.0])                 # mean square 12.5
    g = np.array([1.0, 2.0])
    eps = 1e-6
    exp = np.array([3.0, 8.0]) / math.sqrt(12.5 + eps)
    assert np.allclose(oracle.rmsnorm(a, g, eps), exp, rtol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1024) * 1e-3
    y = oracle.rmsnorm(x, np.ones(1024), eps)
    ms = np.mean(x * x)
    assert math.isclose(math.sqrt(np.mean(y * y)), math.sqrt(ms / (ms + eps)), rel_tol=1e-12)
    # scale invariance up to eps
    z = rng.standard_normal(1024)
    assert np.allclose(oracle.rmsnorm(7.0 * z, np.ones(1024), 0.0), oracle.rmsnorm(z, np.ones(1024), 0.0), rtol=1e-13)


# --------------------------------------------------------------------------- Hadamard

def test_hadamard_matches_scipy_and_is_orthonormal():
    for n in (1, 2, 4, 8, 128):
        h = oracle.hadamard_matrix(n)
        assert np.array_equal(h, scipy.linalg.hadamard(n).astype(np.float64))
    hn = oracle.hadamard_matrix(128) / math.sqrt(128)
    assert np.allclose(hn @ hn.T, np.eye(128), atol=1e-14)
    assert np.array_equal(hn, hn.T)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((64, 128))
    t = oracle.hadamard_transform(q)
    assert np.allclose(oracle.hadamard_transform(t), q, atol=1e-13)   # self-inverse
    assert np.allclose(np.linalg.norm(t, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)


def test_hadamard_hand_example():
    # H4 = [[1,1,1,1],[1,-1,1,-1],[1,1,-1,-1],[1,-1,-1,1]];  H4 [1,2,3,4] / 2 = [10,-2,-4,0] / 2
    assert np.allclose(oracle.hadamard_transform(np.array([1.0, 2.0, 3.0, 4.0])), [5.0, -1.0, -2.0, 0.0], atol=1e-15)
    e0 = np.zeros(128)
    e0[0] = 1.0
    assert np.allclose(oracle.hadamard_transform(e0), np.full(128, 1 / math.sqrt(128)), atol=1e-16)


# --------------------------------------------------------------------------- RoPE / YaRN

def test_rope_frequencies_plain():
    cfg = OracleConfig()
    th = oracle.rope_frequencies(cfg)
    assert th.shape == (32,)
    assert th[0] == 1.0
    assert math.isclose(th[16], 1.0 / 400.0, rel_tol=1e-14)   # 160000^(-1/2) = 1/400
    assert math.isclose(th[8], 160000.0 ** -0.25, rel_tol=1e-14)
    assert np.all(np.diff(th) < 0)


def test_yarn_bounds_and_blend_factor4():
    cfg = OracleConfig(yarn_factor=4.0, yarn_orig_ctx=65536, yarn_beta_fast=32.0, yarn_beta_slow=1.0)
    # by hand: 64 ln(65536/(2 pi 32)) / (2 ln 160000) = 15.45 -> floor 15;
    #          64 ln(65536/(2 pi))    / (2 ln 160000) = 24.71 -> ceil 25
    assert oracle.yarn_correction_range(cfg) == (15.0, 25.0)
    plain = oracle.rope_frequencies(OracleConfig())
    th = oracle.rope_frequencies(cfg)
    assert np.array_equal(th[:16], plain[:16])               # j <= 15: untouched
    assert np.allclose(th[25:], plain[25:] / 4.0, rtol=1e-15)  # j >= 25: interpolated by s
    assert math.isclose(th[20], plain[20] * (0.5 + 0.5 / 4.0), rel_tol=1e-14)   # ramp 1/2
    assert np.array_equal(oracle.rope_frequencies(OracleConfig(yarn_factor=1.0)), plain)


def _complex_rope(vec, pos, freqs, rope_dim):
    # independent formulation: adjacent pairs as complex numbers times e^{i pos theta}
    v = np.array(vec, dtype=np.float64)
    off = v.shape[-1] - rope_dim
    z = v[off::2] + 1j * v[off + 1::2]
    z = z * np.exp(1j * pos * np.asarray(freqs))
    out = v.copy()
    out[off::2] = z.real
    out[off + 1::2] = z.imag
    return out


def test_rope_matches_complex_rotation_and_invariants():
    cfg = OracleConfig()
    fr = oracle.rope_frequencies(cfg)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 128))
    for pos in (0, 1, 16384, 1048576, 1234567):
        r = oracle.apply_rope(q, pos, fr, 64)
        for h in range(4):
            assert np.allclose(r[h], _complex_rope(q[h], pos, fr, 64), atol=1e-12)
        assert np.array_equal(r[:, :64], q[:, :64])           # first 64 dims untouched
        pr = r[:, 64:].reshape(4, 32, 2)
        pq = q[:, 64:].reshape(4, 32, 2)
        assert np.allclose(np.linalg.norm(pr, axis=2), np.linalg.norm(pq, axis=2), rtol=1e-13)
    assert np.array_equal(oracle.apply_rope(q, 0, fr, 64), q)
    # relative position: <R(m) x, R(n) y> = <R(m - n) x, y>
    x, y = rng.standard_normal(128), rng.standard_normal(128)
    lhs = oracle.apply_rope(x[None], 700, fr, 64)[0] @ oracle.apply_rope(y[None], 300, fr, 64)[0]
    rhs = oracle.apply_rope(x[None], 400, fr, 64)[0] @ y
    assert math.isclose(lhs, rhs, rel_tol=1e-11, abs_tol=1e-11)


def test_rope_direction_and_pairing_hand_example():
    # only dim 64 set: pair j = 0 has theta = 1, so position p turns (1, 0) into (cos p, sin p)
    q = np.zeros((1, 128))
    q[0, 64] = 1.0
    r = oracle.apply_rope(q, 2, oracle.rope_frequencies(OracleConfig()), 64)
    exp = np.zeros(128)
    exp[64], exp[65] = math.cos(2.0), math.sin(2.0)
    assert np.allclose(r[0], exp, atol=1e-16)


# --------------------------------------------------------------------------- query branch, hand example

def test_prepare_query_layer_hand_example():
    """Tiny layer worked by hand: hidden 2, Q_LORA_RANK 2, 1 head of dim 4,
    RoPE on the last 2 dims (pair j = 0, theta = 1), position 1, eps 0.

    a = I [1, 1] = [1, 1]; mean square 1 so a_hat = gain = [1, 2];
    q_lin = wq_b a_hat = [1, 2, 3, -1]; RoPE turns (3, -1) by 1 rad:
    (3 cos 1 + sin 1, 3 sin 1 - cos 1); Hadamard: H4 v / 2.
    w = ([3, 4] . [1, 1]) * 4^-0.5 * 1^-0.5 = 3.5.
    Swapping RoPE and Hadamard, rotating the first dims, the opposite sign,
    a transposed wq_b or a missing 1/2 all change the result.
    """
    cfg = OracleConfig(hidden=2, q_lora_rank=2, n_heads=1, head_dim=4, rope_dim=2, rms_eps=0.0)
    lw = {
        "wq_a": np.eye(2),
        "q_norm": np.array([1.0, 2.0]),
        "wq_b": np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [1.0, -1.0]]),
        "w_proj": np.array([[3.0, 4.0]]),
    }
    out = oracle.prepare_query_layer(lw, np.array([1.0, 1.0]), 1, cfg)
    c, s = math.cos(1.0), math.sin(1.0)
    v = np.array([1.0, 2.0, 3 * c + s, 3 * s - c])
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64)
    assert np.allclose(out["a_hat"], [1.0, 2.0], atol=1e-15)
    assert np.allclose(out["q_lin"][0], [1.0, 2.0, 3.0, -1.0], atol=1e-15)
    assert np.allclose(out["q"][0], h4 @ v / 2.0, atol=1e-14)
    assert np.allclose(out["w"], [3.5], atol=1e-15)


def test_prepare_query_reshape_is_head_major():
    # 2 heads x dim 2, no RoPE dims: q[h][d] = (wq_b a_hat)[2 h + d], then a 2-point Hadamard
    cfg = OracleConfig(hidden=1, q_lora_rank=1, n_heads=2, head_dim=2, rope_dim=0, rms_eps=0.0)
    lw = {"wq_a": np.array([[1.0]]), "q_norm": np.array([1.0]),
          "wq_b": np.array([[1.0], [2.0], [3.0], [5.0]]), "w_proj": np.array([[1.0], [2.0]])}
    out = oracle.prepare_query_layer(lw, np.array([1.0]), 9, cfg)
    r = 1 / math.sqrt(2)
    assert np.allclose(out["q"], [[3 * r, -1 * r], [8 * r, -2 * r]], atol=1e-15)
    assert np.allclose(out["w"], np.array([1.0, 2.0]) * 0.5, atol=1e-16)   # 2^-1/2 * 2^-1/2


def test_prepare_query_gemv_against_loops():
    # full-size layer, projections checked against explicit loops on a few outputs
    cfg = OracleConfig()
    rng = np.random.default_rng(4)
    lw = {"wq_a": rng.standard_normal((1024, 4096)) / 64, "q_norm": 1 + 0.1 * rng.standard_normal(1024),
          "wq_b": rng.standard_normal((8192, 1024)) / 32, "w_proj": rng.standard_normal((64, 4096)) / 64}
    x = rng.standard_normal(4096)
    out = oracle.prepare_query_layer(lw, x, 0, cfg)   # position 0: RoPE is the identity
    for o in (0, 511, 1023):
        assert math.isclose(out["a"][o], math.fsum(lw["wq_a"][o, i] * x[i] for i in range(4096)), rel_tol=1e-10, abs_tol=1e-12)
    ms = math.fsum(v * v for v in out["a"]) / 1024
    for o in (3, 1000):
        assert math.isclose(out["a_hat"][o], out["a"][o] / math.sqrt(ms + 1e-6) * lw["q_norm"][o], rel_tol=1e-12)
    for h, d in ((0, 0), (5, 77), (63, 127)):
        row = 128 * h + d
        assert math.isclose(out["q_lin"][h, d], math.fsum(lw["wq_b"][row, i] * out["a_hat"][i] for i in range(1024)), rel_tol=1e-10, abs_tol=1e-12)
    assert np.allclose(out["q"], oracle.hadamard_transform(out["q_lin"]), atol=1e-12)
    for h in (0, 63):
        ref = math.fsum(lw["w_proj"][h, i] * x[i] for i in range(4096)) / math.sqrt(128 * 64)
        assert math.isclose(out["w"][h], ref, rel_tol=1e-10, abs_tol=1e-13)


# --------------------------------------------------------------------------- score

def test_sigmoid_library_and_symmetry():
    x = np.array([-800.0, -30.0, -1.0, 0.0, 0.5, 30.0, 800.0])
    assert np.allclose(oracle.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=0)
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    y = np.linspace(-20, 20, 81)
    assert np.allclose(oracle.sigmoid(-y), 1 - oracle.sigmoid(y), atol=1e-15)


def test_score_half_when_no_positive_dot():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((64, 128))
    w = rng.standard_normal(64)
    assert np.all(oracle.score_layer(np.zeros((5, 128)), q, w) == 0.5)          # k = 0
    assert np.all(oracle.score_layer(rng.standard_normal((5, 128)), q, np.zeros(64)) == 0.5)   # w = 0
    # every head dot product negative: k = -q_0 and all heads = q_0 scaled positive
    qq = np.abs(rng.standard_normal(64))[:, None] * q[0][None, :]
    assert np.all(oracle.score_layer(-q[0][None, :], qq, w) == 0.5)


def test_score_single_head_and_relu_per_head():
    k = np.array([[1.0, 2.0, 0.0, 0.0]])
    q = np.array([[0.5, 0.25, 0.0, 0.0]])   # k.q = 1
    assert math.isclose(oracle.score_layer(k, q, np.array([2.0]))[0], 1 / (1 + math.exp(-2.0)), rel_tol=1e-15)
    # two heads, dots +1 and -1: relu before weighting gives sigmoid(1), not sigmoid(0)
    q2 = np.array([[0.5, 0.25, 0, 0], [-0.5, -0.25, 0, 0]])
    assert math.isclose(oracle.score_layer(k, q2, np.array([1.0, 1.0]))[0], 1 / (1 + math.exp(-1.0)), rel_tol=1e-15)
    # negative weight on a positive dot lowers the score below 1/2
    assert oracle.score_layer(k, q2, np.array([-1.0, 5.0]))[0] < 0.5


def test_score_brute_force_loops_and_range():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((6, 8))
    q = rng.standard_normal((3, 8))
    w = rng.standard_normal(3)
    got = oracle.score_layer(k, q, w)
    for n in range(6):
        logit = 0.0
        for h in range(3):
            dot = sum(k[n, d] * q[h, d] for d in range(8))
            logit += max(dot, 0.0) * w[h]
        assert math.isclose(got[n], 1.0 / (1.0 + math.exp(-logit)), rel_tol=1e-13)
    big = oracle.score_layer(rng.standard_normal((1000, 128)) * 50, rng.standard_normal((64, 128)), rng.standard_normal(64) * 10)
    assert np.all((big >= 0) & (big <= 1))


def test_score_row_tail_and_ensemble():
    rng = np.random.default_rng(8)
    rec = np.zeros((10, 132), np.uint8)
    rec[:, :128] = rng.integers(0, 0x7E, size=(10, 128), dtype=np.uint8)
    rec[:, 128:] = np.frombuffer(np.full(10, 0.01, "<f4").tobytes(), np.uint8).reshape(10, 4)
    rec[7:] = 0xFF
    q = rng.standard_normal((3, 64, 128))
    w = rng.standard_normal((3, 64)) * 0.01
    per, ens = oracle.score_row(rec, q, w, valid_n=7, mode="max")
    assert np.all(np.isneginf(per[:, 7:])) and np.all(np.isneginf(ens[7:]))
    k = oracle.decode_records(rec[:7])
    for li in range(3):
        assert np.allclose(per[li, :7], oracle.score_layer(k, q[li], w[li]), rtol=1e-15)
    assert np.array_equal(ens[:7], per[:, :7].max(axis=0))
    _, mean = oracle.score_row(rec, q, w, valid_n=7, mode="mean")
    assert np.all(mean[:7] <= ens[:7] + 1e-15)
    assert np.allclose(mean[:7], (per[0, :7] + per[1, :7] + per[2, :7]) / 3, rtol=1e-15)


def test_ensemble_identities():
    s = np.array([0.1, 0.7, 0.5])
    assert np.array_equal(oracle.ensemble([s, s, s], "max"), s)
    assert np.allclose(oracle.ensemble([s, s, s], "mean"), s, rtol=1e-15)
    a, b, c = np.array([0.2, 0.9]), np.array([0.4, 0.1]), np.array([0.3, 0.2])
    assert np.array_equal(oracle.ensemble([a, b, c], "max"), [0.4, 0.9])
    assert np.allclose(oracle.ensemble([a, b, c], "mean"), [0.3, 0.4], rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.ensemble([a], "sum")


# --------------------------------------------------------------------------- selection

def _brute_topk(s, valid_n, k):
    order = sorted(range(valid_n), key=lambda i: (-s[i], i))
    m = [0] * len(s)
    for i in order[:k]:
        m[i] = 1
    return m


def test_select_topk_brute_force_every_k():
    rng = np.random.default_rng(9)
    for n in (1, 5, 17, 64):
        s = np.round(rng.uniform(0, 1, n), 1)           # many ties
        for vn in (0, n // 2, n):
            for k in range(0, n + 2):
                got = oracle.select_topk(s, vn, k)
                assert list(got) == _brute_topk(s, vn, k)
                assert got.sum() == min(k, vn)
                assert got[vn:].sum() == 0


def test_select_topk_ties_lowest_index():
    s = np.array([0.5, 0.9, 0.5, 0.5, 0.9])
    assert list(oracle.select_topk(s, 5, 3)) == [1, 1, 0, 0, 1]
    assert list(oracle.select_topk(s, 5, 4)) == [1, 1, 1, 0, 1]


def test_select_threshold_strict():
    s = np.array([0.5, 0.5000001, 0.4999, 0.9, 0.2])
    assert list(oracle.select_threshold(s, 5, 0.5)) == [0, 1, 0, 1, 0]
    assert list(oracle.select_threshold(s, 4, 0.0)) == [1, 1, 1, 1, 0]
    assert oracle.select_threshold(s, 0, 0.0).sum() == 0


def test_run_row_modes_exclusive():
    cfg = OracleConfig(hidden=2, q_lora_rank=2, n_heads=1, head_dim=4, rope_dim=2)
    lw = {"wq_a": np.eye(2), "q_norm": np.ones(2), "wq_b": np.ones((4, 2)), "w_proj": np.ones((1, 2))}
    rec = np.zeros((3, 8), np.uint8)
    with pytest.raises(ValueError):
        oracle.run_row([lw], np.ones(2), 0, rec, cfg, top_k=1, threshold=0.5)
    r = oracle.run_row([lw], np.ones(2), 0, rec, cfg, top_k=2)
    assert list(r["mask"]) == [1, 1, 0]          # all scores 0.5: ties to the lowest indices


# --------------------------------------------------------------------------- assemblers: prepare_query, run_row

def _assembler_cfg():
    # README "Architecture" on tiny sizes: 2 hidden dims, rank 2, 2 heads of
    # 4 dims, RoPE over all 4 dims (pairs (0, 1) and (2, 3)), eps 0 so that
    # the RMS divisions come out exact.  theta_j = base^(-2j/4): theta_0 = 1
    # and, with base = 4 / pi^2, theta_1 = pi / 2, so position 1 turns pair
    # (2, 3) by a quarter turn and position 2 by a half turn.  The weights
    # keep pair (0, 1) at zero, where any angle leaves it unchanged.
    return OracleConfig(hidden=2, q_lora_rank=2, n_heads=2, head_dim=4, rope_dim=4, rms_eps=0.0,
                        rope_base=4.0 / math.pi ** 2, n_layers=2)


def _assembler_weights():
    z = [0.0, 0.0]
    l0 = {"wq_a": np.eye(2), "q_norm": np.array([1.0, 1.0]),
          # head 0 dims 2, 3 <- (a0, a1); head 1 dims 2, 3 <- (a1, a0)
          "wq_b": np.array([z, z, [1.0, 0.0], [0.0, 1.0], z, z, [0.0, 1.0], [1.0, 0.0]]),
          "w_proj": np.eye(2)}
    l1 = {"wq_a": 2.0 * np.eye(2), "q_norm": np.array([2.0, 1.0]),
          # head 0 dims 2, 3 <- (a0 + a1, a0 - a1); head 1 dim 3 <- a0
          "wq_b": np.array([z, z, [1.0, 1.0], [1.0, -1.0], z, z, z, [1.0, 0.0]]),
          "w_proj": np.array([[0.0, 1.0], [1.0, 0.0]])}
    return [l0, l1]


def test_prepare_query_hand_worked_layers_rows_positions():
    """Two layers x two rows at distinct positions, worked by hand.

    Row 0: h = (1, 7) at position 1; row 1: h = (-7, 1) at position 2.
    Per head the (2, 3) pair (x, y) is turned counter-clockwise ((-y, x) at a
    quarter turn, (-x, -y) at a half turn), then the normalized 4-point
    Hadamard maps (0, 0, x', y') to (x'+y', x'-y', -x'-y', -x'+y') / 2.
    w = W_p h * (4 * 2)^-1/2.

    layer 0, row 0: a = (1, 7), mean a^2 = 25, a_hat = (0.2, 1.4)
      head 0: (0.2, 1.4) -> (-1.4, 0.2) -> (-0.6, -0.8, 0.6, 0.8)
      head 1: (1.4, 0.2) -> (-0.2, 1.4) -> (0.6, -0.8, -0.6, 0.8)
    layer 0, row 1: a = (-7, 1), a_hat = (-1.4, 0.2)
      head 0: (-1.4, 0.2) -> (1.4, -0.2) -> (0.6, 0.8, -0.6, -0.8)
      head 1: (0.2, -1.4) -> (-0.2, 1.4) -> (0.6, -0.8, -0.6, 0.8)
    layer 1, row 0: a = (2, 14), mean a^2 = 100, a_hat = (0.2, 1.4) * (2, 1) = (0.4, 1.4)
      head 0: (1.8, -1.0) -> (1.0, 1.8) -> (1.4, -0.4, -1.4, 0.4)
      head 1: (0.0, 0.4) -> (-0.4, 0.0) -> (-0.2, -0.2, 0.2, 0.2)
    layer 1, row 1: a = (-14, 2), a_hat = (-2.8, 0.2)
      head 0: (-2.6, -3.0) -> (2.6, 3.0) -> (2.8, -0.2, -2.8, 0.2)
      head 1: (0.0, -2.8) -> (0.0, 2.8) -> (1.4, -1.4, -1.4, 1.4)
    w: layer 0 rows (1, 7) and (-7, 1); layer 1 (swapped W_p) rows (7, 1) and (1, -7), each / sqrt(8).
    """
    cfg = _assembler_cfg()
    hidden = np.array([[1.0, 7.0], [-7.0, 1.0]])
    positions = np.array([1, 2], dtype=np.int64)
    q, w = oracle.prepare_query(_assembler_weights(), hidden, positions, cfg)
    want_q = np.array([
        [[[-0.6, -0.8, 0.6, 0.8], [0.6, -0.8, -0.6, 0.8]],
         [[0.6, 0.8, -0.6, -0.8], [0.6, -0.8, -0.6, 0.8]]],
        [[[1.4, -0.4, -1.4, 0.4], [-0.2, -0.2, 0.2, 0.2]],
         [[2.8, -0.2, -2.8, 0.2], [1.4, -1.4, -1.4, 1.4]]],
    ])
    want_w = np.array([[[1.0, 7.0], [-7.0, 1.0]], [[7.0, 1.0], [1.0, -7.0]]]) / math.sqrt(8.0)
    assert q.shape == (2, 2, 2, 4) and w.shape == (2, 2, 2)
    np.testing.assert_allclose(q, want_q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w, want_w, rtol=0, atol=1e-15)
    # the positions belong to their rows: swapped, row 0 head 0 turns by a half turn
    q_sw, _ = oracle.prepare_query(_assembler_weights(), hidden, positions[::-1].copy(), cfg)
    np.testing.assert_allclose(q_sw[0, 0, 0], [-0.8, 0.6, 0.8, -0.6], rtol=0, atol=1e-12)


def _run_row_case():
    """Two one-head layers whose prepared queries are unit vectors.

    h = (1, 1), wq_a = I, eps 0: a_hat = (1, 1).  Layer 0's wq_b rows are all
    (1/4, 1/4), so q_lin = (1, 1, 1, 1) / 2 and, at position 0 (no turn), the
    normalized Hadamard gives q = (1, 0, 0, 0); layer 1's rows carry signs
    (+, -, +, -), giving q = (0, 1, 0, 0).  W_p = (ln 3, ln 3) and the scale
    (4 * 1)^-1/2 give w = ln 3 in both layers.  Keys (scale 0.5, codes 2 k):
      chunk 0: k = (2, 0, 0, 0)   layer logits (2 ln 3, 0)  -> scores (0.9, 0.5)
      chunk 1: k = (1, 1, 0, 0)   (ln 3, ln 3)              -> (0.75, 0.75)
      chunk 2: k = (-1, -1, 0, 0) (0, 0)                    -> (0.5, 0.5)
      chunk 3: k = (0, 2, 0, 0)   (0, 2 ln 3)               -> (0.5, 0.9)
      chunk 4: k = (1, 0, 0, 0)   (ln 3, 0)                 -> (0.75, 0.5)
    since sigmoid(ln 3) = 3/4 and sigmoid(2 ln 3) = 9/10.
    """
    cfg = OracleConfig(hidden=2, q_lora_rank=2, n_heads=1, head_dim=4, rope_dim=4, rms_eps=0.0, n_layers=2)
    ln3 = math.log(3.0)
    quarter = np.full((4, 2), 0.25)
    signs = np.array([[1.0], [-1.0], [1.0], [-1.0]])
    layers = [{"wq_a": np.eye(2), "q_norm": np.ones(2), "wq_b": quarter, "w_proj": np.array([[ln3, ln3]])},
              {"wq_a": np.eye(2), "q_norm": np.ones(2), "wq_b": quarter * signs, "w_proj": np.array([[ln3, ln3]])}]
    codes = {0.0: 0x00, 2.0: 0x40, 4.0: 0x48, -2.0: 0xC0}  # e4m3fn: 2 = 0.1000.000, 4 = 0.1001.000
    keys = [(2, 0), (1, 1), (-1, -1), (0, 2), (1, 0)]
    rec = np.zeros((5, 8), np.uint8)
    for n, (k0, k1) in enumerate(keys):
        rec[n, 0] = codes[2.0 * k0]
        rec[n, 1] = codes[2.0 * k1]
        rec[n, 4:8] = np.frombuffer(np.array([0.5], "<f4").tobytes(), np.uint8)
    return cfg, layers, np.ones(2), rec


def test_run_row_hand_worked_max_and_mean():
    cfg, layers, h, rec = _run_row_case()
    per_layer = np.array([[0.9, 0.75, 0.5, 0.5, 0.75], [0.5, 0.75, 0.5, 0.9, 0.5]])
    r = oracle.run_row(layers, h, 0, rec, cfg, mode="max", top_k=1)
    np.testing.assert_allclose(r["q"], [[[1, 0, 0, 0]], [[0, 1, 0, 0]]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["w"], [[math.log(3.0)]] * 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["per_layer"], per_layer, rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["scores"], [0.9, 0.75, 0.5, 0.9, 0.75], rtol=0, atol=1e-15)
    assert list(r["mask"]) == [1, 0, 0, 0, 0]                     # 0.9 ties: chunk 0 before chunk 3
    r = oracle.run_row(layers, h, 0, rec, cfg, mode="mean", top_k=1)
    np.testing.assert_allclose(r["scores"], [0.7, 0.75, 0.5, 0.7, 0.625], rtol=0, atol=1e-15)
    assert list(r["mask"]) == [0, 1, 0, 0, 0]                     # the mean ranks chunk 1 first
    r = oracle.run_row(layers, h, 0, rec, cfg, mode="max", top_k=3)
    assert list(r["mask"]) == [1, 1, 0, 1, 0]                     # 0.75 ties: chunk 1 before chunk 4
    r = oracle.run_row(layers, h, 0, rec, cfg, mode="max", threshold=0.72)
    assert list(r["mask"]) == [1, 1, 0, 1, 1]
    r = oracle.run_row(layers, h, 0, rec, cfg, mode="mean", threshold=0.72)
    assert list(r["mask"]) == [0, 1, 0, 0, 0]


def test_run_row_hand_worked_valid_n():
    cfg, layers, h, rec = _run_row_case()
    r = oracle.run_row(layers, h, 0, rec, cfg, valid_n=3, mode="max", threshold=0.72)
    np.testing.assert_allclose(r["scores"][:3], [0.9, 0.75, 0.5], rtol=0, atol=1e-15)
    assert np.all(np.isneginf(r["scores"][3:])) and np.all(np.isneginf(r["per_layer"][:, 3:]))
    assert list(r["mask"]) == [1, 1, 0, 0, 0]                     # chunks 3 and 4 lie past valid_n
    r = oracle.run_row(layers, h, 0, rec, cfg, valid_n=3, mode="mean", top_k=2)
    assert list(r["mask"]) == [1, 1, 0, 0, 0]
    r = oracle.run_row(layers, h, 0, rec, cfg, valid_n=3, mode="max", top_k=5)
    assert list(r["mask"]) == [1, 1, 1, 0, 0]                     # K above valid_n keeps every valid chunk
    r = oracle.run_row(layers, h, 0, rec, cfg, valid_n=0, mode="max", top_k=2)
    assert r["mask"].sum() == 0 and np.all(np.isneginf(r["scores"]))


# --------------------------------------------------------------------------- resident set and recall delta

def _delta_by_sets(mask, prev):
    """Brute force with Python sets and an explicit loop."""
    cur_set = {n for n in range(len(mask)) if mask[n]}
    prev_set = set() if prev is None else {n for n in range(len(prev)) if prev[n]}
    return sorted(cur_set), sorted(cur_set - prev_set), sorted(prev_set - cur_set)


def test_resident_delta_brute_force_tiny():
    rng = np.random.default_rng(40)
    for n in (0, 1, 2, 7, 33):
        for _ in range(20):
            cur = (rng.uniform(size=n) < rng.uniform()).astype(np.uint8)
            prev = (rng.uniform(size=n) < rng.uniform()).astype(np.uint8)
            for p in (None, prev):
                got = oracle.resident_delta(cur, p)
                want = _delta_by_sets(cur, p)
                for g, w in zip(got, want):
                    assert list(g) == w


def test_resident_delta_identities():
    rng = np.random.default_rng(41)
    cur = (rng.uniform(size=5000) < 0.1).astype(np.uint8)
    prev = (rng.uniform(size=5000) < 0.1).astype(np.uint8)
    res, ent, lea = oracle.resident_delta(cur, prev)
    prev_res, _, _ = oracle.resident_delta(prev)
    # the new resident set is the previous one plus entering minus leaving
    assert sorted((set(prev_res) | set(ent)) - set(lea)) == list(res)
    assert len(res) == len(prev_res) + len(ent) - len(lea)
    assert not set(ent) & set(prev_res) and set(lea) <= set(prev_res)
    assert all(np.all(np.diff(x) > 0) for x in (res, ent, lea) if len(x) > 1)
    # same mask twice: nothing moves; no previous mask: everything enters
    r2, e2, l2 = oracle.resident_delta(cur, cur)
    assert len(e2) == 0 and len(l2) == 0 and list(r2) == list(res)
    r3, e3, l3 = oracle.resident_delta(cur)
    assert list(e3) == list(res) and len(l3) == 0


def test_resident_delta_counts_nonzero_bytes():
    cur = np.array([0, 1, 2, 255, 0], np.uint8)
    prev = np.array([7, 0, 1, 0, 0], np.uint8)
    res, ent, lea = oracle.resident_delta(cur, prev)
    assert list(res) == [1, 2, 3] and list(ent) == [1, 3] and list(lea) == [0]


# --------------------------------------------------------------------------- per-step top-K within the resident set

def _subset_topk_by_exchange(scores, subset, k):
    """Brute force: among all k-sets of valid list positions, the one set S
    where every chosen entry beats every left-out one (higher score, or the
    same score at an earlier position).  Returned in list order."""
    n = len(scores)
    valid = [p for p in range(len(subset)) if 0 <= subset[p] < n]
    k = min(k, len(valid))
    found = []
    for S in itertools.combinations(valid, k):
        rest = [u for u in valid if u not in S]
        if all(scores[subset[s]] > scores[subset[u]] or (scores[subset[s]] == scores[subset[u]] and s < u)
               for s in S for u in rest):
            found.append([subset[p] for p in S])
    assert len(found) == 1  # the rule makes the choice unique
    return found[0]


def test_subset_topk_brute_force_tiny():
    rng = np.random.default_rng(50)
    for _ in range(60):
        n = int(rng.integers(1, 12))
        scores = rng.integers(0, 4, n).astype(np.float64) / 4  # many ties
        scores[rng.uniform(size=n) < 0.1] = -np.inf
        m = int(rng.integers(0, 9))
        subset = rng.integers(-2, n + 2, m)                    # some entries out of range
        subset = np.array([x for i, x in enumerate(subset) if x < 0 or x >= n or x not in subset[:i]], np.int64)
        for k in (0, 1, 2, 5, 20):
            got = list(oracle.select_topk_subset(scores, subset, k))
            assert got == _subset_topk_by_exchange(scores, subset, k)


def test_subset_topk_over_all_chunks_is_the_row_top_k():
    rng = np.random.default_rng(51)
    scores = np.round(rng.uniform(size=3000), 2)                # ties
    for k in (0, 1, 512, 2999, 3000, 4000):
        mask = oracle.select_topk(scores, 3000, k)
        assert np.array_equal(oracle.select_topk_subset(scores, np.arange(3000), k), np.flatnonzero(mask))


def test_subset_topk_order_and_range():
    scores = np.array([0.1, 0.9, 0.5, 0.9, 0.3])
    # list order is kept (not score order); out-of-range entries are skipped
    assert list(oracle.select_topk_subset(scores, np.array([4, 3, 7, 1, -1, 0]), 3)) == [4, 3, 1]
    # tie at 0.9 between positions 1 and 3 of the list: the earlier one wins
    assert list(oracle.select_topk_subset(scores, np.array([0, 3, 2, 1]), 1)) == [3]
    assert list(oracle.select_topk_subset(scores, np.array([5, 6]), 2)) == []
    assert list(oracle.select_topk_subset(scores, np.array([2, 0]), 9)) == [2, 0]


# --------------------------------------------------------------------------- attention-logit masking

def test_mask_logits_loop_and_softmax():
    rng = np.random.default_rng(60)
    logits = rng.normal(size=(3, 40))
    mask = (rng.uniform(size=40) < 0.3).astype(np.uint8)
    mask[[0, 7]] = [2, 255]                                   # any non-zero byte keeps
    got = oracle.mask_logits(logits, mask)
    for r in range(3):
        for n in range(40):
            assert got[r, n] == (logits[r, n] if mask[n] else -np.inf)
    # a masked chunk gets zero attention weight; the kept ones share all of it
    kept = mask != 0
    p = scipy.special.softmax(got, axis=1)
    assert np.all(p[:, ~kept] == 0)
    assert np.allclose(p[:, kept], scipy.special.softmax(logits[:, kept], axis=1), rtol=1e-12, atol=0)
    assert np.array_equal(oracle.mask_logits(logits, np.ones(40)), logits)
    assert np.all(np.isneginf(oracle.mask_logits(logits, np.zeros(40))))
    assert not np.any(np.isneginf(logits))  # the input is not modified
