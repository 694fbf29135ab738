"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin is chosen so that a plausible slip in the oracle fails it:
  * bf16 rounding vs exact rational rounding (double rounding, tie handling);
  * RoPE vs the textbook complex-multiplication form (pairing, sign, angle);
  * RoPE relative-position invariance for any frequency table (q/k consistency);
  * YaRN special cases from its published definition;
  * one frame with an empty state vs causal scaled-dot-product attention (mask,
    scale, GQA head map);
  * a stream with B >= N*T vs full causal attention over all N*T tokens
    (virtual positions nT + i, frame indexing, state carry-over);
  * scores are a probability distribution over the pool (denominator Hq*T);
  * selection with ties keeps the older token;
  * the text phase after an evicting stream vs the last rows of one causal
    attention over every frame token and the text (D keeps what C evicted;
    positions continue at N*T; chunking does not matter).
Brute-force comparisons on tiny inputs live in test_oracle_bruteforce.py.
"""
from fractions import Fraction
import math
import random

import numpy as np
import pytest
import torch

from oracle import (CompressedState, LayerConfig, OracleStream, decode_step, frame_step,
                    round_f64_to_bf16, rope_cos_sin, rope_inv_freq, rope_rotate,
                    select_top_b, yarn_inv_freq, yarn_logit_scale)


# ---------------------------------------------------------------- rounding --

def _exact_bf16(x: float) -> float:
    """Nearest bf16 (8 significant bits, ties to even) by exact rationals."""
    if x == 0.0:
        return 0.0
    fx = Fraction(x)
    sign = -1 if fx < 0 else 1
    ax = abs(fx)
    e = math.floor(math.log2(ax))
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    q = Fraction(2) ** (e - 7)
    m = ax / q
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(sign * n * q)


def test_bf16_rounding_matches_exact_rationals():
    rnd = random.Random(7)
    vals = [rnd.gauss(0.0, 3.0) for _ in range(3000)]
    # Exact bf16 midpoints and values a hair above / below them: a double
    # rounding through fp32 gets the "hair above" cases wrong.
    for _ in range(300):
        b = _exact_bf16(rnd.uniform(0.5, 8.0))
        ulp = 2.0 ** (math.floor(math.log2(b)) - 7)
        mid = b + ulp / 2
        vals += [mid, -mid, mid + ulp * 2.0 ** -30, mid - ulp * 2.0 ** -30]
    got = round_f64_to_bf16(np.array(vals))
    want = np.array([_exact_bf16(v) for v in vals])
    assert np.array_equal(got, want)


# -------------------------------------------------------------------- RoPE --

def _textbook_rope(x, positions, theta):
    """x: [T][H][d]; pairs (k, k+d/2) as complex numbers times e^{i p theta_k}."""
    half = x.shape[-1] // 2
    z = x[..., :half] + 1j * x[..., half:]
    ang = np.outer(np.asarray(positions, dtype=np.float64), theta)     # [T][d/2]
    z = z * np.exp(1j * ang)[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_alpha_one_is_textbook_rope():
    rng = np.random.default_rng(1)
    T, H, d = 9, 3, 64
    x = rng.standard_normal((T, H, d)).astype(np.float32).astype(np.float64)
    positions = 4096 + np.arange(T) * 37
    theta_plain = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    assert np.allclose(rope_inv_freq(d, 10000.0), theta_plain, rtol=1e-15, atol=0)
    assert np.array_equal(yarn_inv_freq(d, 10000.0, 1.0, 32768), rope_inv_freq(d, 10000.0))
    c, s = rope_cos_sin(positions, rope_inv_freq(d, 10000.0))
    got = rope_rotate(x, c, s, "f32")
    want = _textbook_rope(x, positions, theta_plain)
    # cos/sin are fp32 and the output is fp32: agreement to a few fp32 ulps.
    assert np.max(np.abs(got - want)) < 4e-6 * np.max(np.abs(want))


@pytest.mark.parametrize("alpha", [1.0, 4.0, 8.0])
def test_rope_relative_position_invariance(alpha):
    rng = np.random.default_rng(2)
    d = 128
    theta = yarn_inv_freq(d, 1e6, alpha, 32768)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for p, pk, shift in [(300, 12, 1000), (5000, 4999, 70000), (7, 7, 123456)]:
        def dot(a, b):
            ca, sa = rope_cos_sin([a], theta)
            cb, sb = rope_cos_sin([b], theta)
            qa = rope_rotate(q, ca, sa, "f32")
            kb = rope_rotate(k, cb, sb, "f32")
            return float(np.sum(qa * kb))
        base = dot(p, pk)
        moved = dot(p + shift, pk + shift)
        assert abs(base - moved) < 1e-4 * math.sqrt(d)


def test_yarn_special_cases():
    d, base, L = 128, 1e6, 32768
    theta = rope_inv_freq(d, base)
    for alpha in (2.0, 4.0, 8.0):
        th = yarn_inv_freq(d, base, alpha, L)
        r = L * theta / (2 * math.pi)
        hi = r > 32.0           # many rotations in the original window: kept
        lo = r < 1.0            # less than one rotation: interpolated by 1/alpha
        assert hi.any() and lo.any()
        assert np.array_equal(th[hi], theta[hi])
        assert np.allclose(th[lo], theta[lo] / alpha, rtol=1e-15)
        mid = ~(hi | lo)        # ramp: strictly between the two
        assert np.all(th[mid] <= theta[mid]) and np.all(th[mid] >= theta[mid] / alpha)
    assert yarn_logit_scale(64, 1.0) == 1.0 / 8.0
    assert math.isclose(yarn_logit_scale(128, 4.0),
                        (0.1 * math.log(4.0) + 1.0) ** 2 / math.sqrt(128), rel_tol=1e-15)


# --------------------------------------------------------------- attention --

def _sdpa_causal(q_rot, k_rot, v, n_q, n_kv):
    """torch fp64 causal SDPA over [L][H][d] inputs with the GQA head map h -> h // G."""
    G = n_q // n_kv
    q = torch.from_numpy(q_rot).permute(1, 0, 2)                    # [Hq][L][d]
    k = torch.from_numpy(k_rot).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, is_causal=True)
    return o.permute(1, 0, 2).numpy()


def _rand_frame(rng, T, Hq, Hkv, d):
    f = lambda *s: rng.standard_normal(s).astype(np.float32).astype(np.float64)
    return f(T, Hq, d), f(T, Hkv, d), f(T, Hkv, d)


def test_single_frame_empty_state_is_causal_sdpa():
    cfg = LayerConfig(n_q_heads=6, n_kv_heads=2, head_dim=32, tokens_per_frame=11,
                      budget=8, dtype="f32", rope_base=1e4)
    rng = np.random.default_rng(3)
    Q, K, V = _rand_frame(rng, 11, 6, 2, 32)
    res = frame_step(cfg, CompressedState.empty(cfg), Q, K, V, n=0)
    want = _sdpa_causal(res.Q_rot, res.K_rot, V, 6, 2)
    assert np.max(np.abs(res.O_exact - want)) < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_eviction_stream_is_full_causal_attention(dtype):
    """With B >= N*T nothing is evicted and every frame's output equals its rows
    of one causal attention over all N*T tokens at positions 0..N*T-1."""
    T, N, Hq, Hkv, d = 7, 5, 4, 2, 32
    cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                      budget=N * T, dtype=dtype, rope_base=1e4)
    rng = np.random.default_rng(4)
    frames = [_rand_frame(rng, T, Hq, Hkv, d) for _ in range(N)]
    stream = OracleStream(cfg)
    outs = [stream.step(*f).O_exact for f in frames]
    Q = np.concatenate([f[0] for f in frames])
    K = np.concatenate([f[1] for f in frames])
    V = np.concatenate([f[2] for f in frames])
    theta = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    q_rot = _textbook_rope(Q, np.arange(N * T), theta)
    k_rot = _textbook_rope(K, np.arange(N * T), theta)
    if dtype == "bf16":
        q_rot, k_rot = round_f64_to_bf16(q_rot), round_f64_to_bf16(k_rot)
    else:
        q_rot = q_rot.astype(np.float32).astype(np.float64)
        k_rot = k_rot.astype(np.float32).astype(np.float64)
    want = _sdpa_causal(q_rot, k_rot, V, Hq, Hkv)
    got = np.concatenate(outs)
    # Differences come only from fp32 cos/sin in the oracle (and, for bf16,
    # the rare rotated element that rounds to the neighbouring bf16).
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.max(np.abs(got - want)) < tol
    assert stream.state.count == N * T


def _sdpa_masked(q_rot, k_rot, v, n_q, n_kv, visible):
    """torch fp64 SDPA over [L][H][d] inputs with a boolean [L][L] visibility mask."""
    G = n_q // n_kv
    q = torch.from_numpy(q_rot).permute(1, 0, 2)
    k = torch.from_numpy(k_rot).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=torch.from_numpy(visible))
    return o.permute(1, 0, 2).numpy()


def test_recent_window_stream_is_banded_causal_attention():
    """Recency policy (the ReKV-style window): the state before frame n holds the
    last min(B, nT) tokens, so a query at position p of frame n sees exactly the
    keys p' with max(0, nT - B) <= p' <= p: one banded causal attention."""
    T, N, B, Hq, Hkv, d = 7, 6, 16, 4, 2, 32
    cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                      budget=B, dtype="f32", rope_base=1e4, policy="recent")
    rng = np.random.default_rng(14)
    frames = [_rand_frame(rng, T, Hq, Hkv, d) for _ in range(N)]
    stream = OracleStream(cfg)
    outs = []
    for n, f in enumerate(frames):
        outs.append(stream.step(*f).O_exact)
        lo = max(0, (n + 1) * T - B)
        assert stream.state.pos.tolist() == list(range(lo, (n + 1) * T))
    L = N * T
    Q = np.concatenate([f[0] for f in frames])
    K = np.concatenate([f[1] for f in frames])
    V = np.concatenate([f[2] for f in frames])
    theta = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    q_rot = _textbook_rope(Q, np.arange(L), theta).astype(np.float32).astype(np.float64)
    k_rot = _textbook_rope(K, np.arange(L), theta).astype(np.float32).astype(np.float64)
    p = np.arange(L)
    lo = np.maximum(0, (p // T) * T - B)
    visible = (p[None, :] <= p[:, None]) & (p[None, :] >= lo[:, None])
    want = _sdpa_masked(q_rot, k_rot, V, Hq, Hkv, visible)
    assert np.max(np.abs(np.concatenate(outs) - want)) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_text_phase_is_the_tail_of_full_causal_attention(dtype):
    """After N frames with eviction (B < N*T), text tokens decoded in chunks of
    3, 1 and 2 equal the last 6 rows of one causal attention over all N*T frame
    tokens followed by the 6 text tokens, at positions 0..N*T+5: the text sees
    the detailed cache, not the compressed state."""
    T, N, B, Hq, Hkv, d = 7, 5, 9, 6, 2, 32
    cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                      budget=B, dtype=dtype, rope_base=1e4)
    rng = np.random.default_rng(21)
    frames = [_rand_frame(rng, T, Hq, Hkv, d) for _ in range(N)]
    text = _rand_frame(rng, 6, Hq, Hkv, d)
    if dtype == "bf16":
        frames = [tuple(round_f64_to_bf16(x) for x in f) for f in frames]
        text = tuple(round_f64_to_bf16(x) for x in text)
    stream = OracleStream(cfg)
    for f in frames:
        stream.step(*f)
    assert stream.state.count == B                     # C evicted; D holds everything
    outs = []
    for lo, hi in [(0, 3), (3, 4), (4, 6)]:
        res = stream.decode(*(x[lo:hi] for x in text))
        assert res.positions.tolist() == list(range(N * T + lo, N * T + hi))
        outs.append(res.O_exact)
    L = N * T + 6
    Q = np.concatenate([f[0] for f in frames] + [text[0]])
    K = np.concatenate([f[1] for f in frames] + [text[1]])
    V = np.concatenate([f[2] for f in frames] + [text[2]])
    theta = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    q_rot = _textbook_rope(Q, np.arange(L), theta)
    k_rot = _textbook_rope(K, np.arange(L), theta)
    if dtype == "bf16":
        q_rot, k_rot = round_f64_to_bf16(q_rot), round_f64_to_bf16(k_rot)
    else:
        q_rot = q_rot.astype(np.float32).astype(np.float64)
        k_rot = k_rot.astype(np.float32).astype(np.float64)
    want = _sdpa_causal(q_rot, k_rot, V, Hq, Hkv)[N * T:]
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.max(np.abs(np.concatenate(outs) - want)) < tol
    D_K, _ = stream.detailed()
    assert D_K.shape[0] == L


def test_text_phase_chunking_is_invisible():
    """Decoding t tokens at once equals decoding them one by one (causal mask
    inside the chunk, positions advancing by one)."""
    cfg = LayerConfig(n_q_heads=4, n_kv_heads=1, head_dim=64, tokens_per_frame=5,
                      budget=4, dtype="f32", rope_base=1e6, alpha=4.0)
    rng = np.random.default_rng(22)
    DK = rng.standard_normal((23, 1, 64)).astype(np.float32).astype(np.float64)
    DV = rng.standard_normal((23, 1, 64)).astype(np.float32).astype(np.float64)
    Q, K, V = _rand_frame(rng, 4, 4, 1, 64)
    whole = decode_step(cfg, DK, DV, Q, K, V)
    dk, dv, rows = DK, DV, []
    for i in range(4):
        r = decode_step(cfg, dk, dv, Q[i:i + 1], K[i:i + 1], V[i:i + 1])
        dk = np.concatenate([dk, r.K_rot])
        dv = np.concatenate([dv, r.V])
        rows.append(r.O_exact)
    assert np.array_equal(whole.K_rot, np.concatenate([dk[23:]]))
    assert np.max(np.abs(np.concatenate(rows) - whole.O_exact)) < 1e-12


def test_scores_are_a_distribution_over_the_pool():
    cfg = LayerConfig(n_q_heads=4, n_kv_heads=1, head_dim=64, tokens_per_frame=16,
                      budget=24, dtype="bf16", rope_base=1e6, alpha=4.0)
    rng = np.random.default_rng(5)
    stream = OracleStream(cfg)
    for n in range(4):
        res = stream.step(*_rand_frame(rng, 16, 4, 1, 64))
        assert res.scores.size == min(24, n * 16) + 16
        assert np.all(res.scores >= 0)
        assert abs(res.scores.sum() - 1.0) < 1e-12
        # The last frame token is visible only to the last query: its score is
        # exactly (1/(Hq*T)) * sum over heads of that query's weight on it.
        assert res.scores[-1] <= 1.0 / 16 + 1e-15


def test_select_ties_keep_the_older_token():
    scores = np.array([0.5, 0.1, 0.1, 0.3, 0.1], dtype=np.float64)
    pos = np.array([2, 9, 11, 40, 41])
    assert list(select_top_b(scores, pos, 3)) == [0, 1, 3]
    assert list(select_top_b(scores, pos, 4)) == [0, 1, 2, 3]
    assert list(select_top_b(scores, pos, 9)) == [0, 1, 2, 3, 4]


def test_exact_ties_keep_the_oldest_tokens():
    """With all-zero queries attention is uniform over the visible keys: every
    state key and the frame's first key (visible to every query) get
    bit-identical scores, and when only some of them fit the oldest are kept."""
    T, Hq, Hkv, d, B = 8, 2, 1, 32, 16
    cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                      budget=B, dtype="f32", rope_base=1e4)
    rng = np.random.default_rng(6)
    stream = OracleStream(cfg)
    for _ in range(2):
        stream.step(*_rand_frame(rng, T, Hq, Hkv, d))
    st = stream.state
    assert st.count == B
    _, K, V = _rand_frame(rng, T, Hq, Hkv, d)
    Q = np.zeros((T, Hq, d))
    tied = list(range(B + 1))           # B state keys and frame key 0
    for keep_n in (B - 3, B, B + 1):
        cfg2 = LayerConfig(**{**cfg.__dict__, "budget": keep_n})
        res = frame_step(cfg2, st, Q, K, V, n=2)
        assert len(set(res.scores32[tied].tolist())) == 1
        assert np.all(res.scores32[B + 1:] < res.scores32[0])
        assert res.keep.tolist() == tied[:keep_n]


def test_stream_state_invariants():
    T, Hq, Hkv, d, B = 16, 4, 2, 64, 40
    cfg = LayerConfig(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=T,
                      budget=B, dtype="bf16", rope_base=1e6)
    rng = np.random.default_rng(8)
    stream = OracleStream(cfg)
    prev = set()
    for n in range(7):
        res = stream.step(*_rand_frame(rng, T, Hq, Hkv, d))
        st = stream.state
        # Capacity: min(B, (n+1)T) tokens; the pool is the old state plus T.
        assert st.count == min(B, (n + 1) * T)
        assert res.pool_pos.size == min(B, n * T) + T
        new = set(st.pos.tolist())
        assert new <= prev | set(range(n * T, n * T + T))
        assert np.all(np.diff(st.pos) > 0)
        # The state is a subset of D: row r equals D at position pos[r].
        DK, DV = stream.detailed()
        assert np.array_equal(st.K, DK[st.pos].transpose(1, 0, 2))
        assert np.array_equal(st.V, DV[st.pos].transpose(1, 0, 2))
        prev = new
