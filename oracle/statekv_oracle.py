"""Plain CPU oracle of the StateKV streaming-prefill frame step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

Source: paper note "Linear Scaling Video VLMs for Long Video Understanding"
(papernotes.org, ECCV 2026), section "方法详解":
  * 整体框架 (overall framework): per layer, a compressed state C of capacity B
    and a detailed state D that accumulates every processed token; frame n
    attends only to C_{n-1} and to itself; per-frame cost O(T^2 + BT).
  * 关键设计 1 (dual state): the frame's queries attend over [Kbar_{n-1}; K_n].
  * 关键设计 2 (attention-driven temporal sinks): the candidate pool is the old
    state plus the frame's T tokens; each candidate's score is the average
    attention the frame's queries pay to it; TopK keeps B of them.
  * 关键设计 3 (virtual length and global RoPE scaling): RoPE angles use the
    logical stream position L_n = nT; one scaling factor alpha (YaRN-like) is
    fixed before prefill.
The attention and score equations are missing from the extracted text; the
readings used here (standard softmax attention, causal inside the frame, mean
over all T queries and all query heads) are listed in the design notes.

Arithmetic is float64 throughout.  Values are rounded only where the step
stores them: the rotated Q and K and the output O are rounded once, to nearest
even, to the storage dtype ("bf16" or "f32").  Scores are fp64 sums, rounded
to fp32 only for the Top-B decision (the precision the GPU takes it in).
Matrix products use numpy's float64 matmul as a library primitive.

The text phase (decode_step) attends text tokens over the whole detailed cache
D, continuing the virtual positions.

Parity: RoPE (alpha = 1), attention, scores, selection, the state update and
the text phase are pinned by tests (textbook complex-form RoPE,
relative-position invariance, reduction to causal scaled-dot-product attention
for frames and for the text after an evicting stream, score sum = 1, brute
force on tiny inputs, tie and subset invariants).  The YaRN frequency ramp and
logit temperature used for alpha > 1 are not on the pages: parity unpinned
beyond the invariance checks.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------

def round_f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), exactly once.

    Method: round to fp32 with round-to-odd (truncate toward zero, then set the
    last bit if anything was discarded), then round that fp32 to bf16 with
    ties-to-even.  Because fp32 keeps 16 more bits than bf16, the result equals
    a single correct rounding of the float64 input.  Returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    away = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(away, np.nextafter(f, np.float32(0.0)), f)
    inexact = (f.astype(np.float64) != x).astype(np.uint32)
    bits = (np.ascontiguousarray(f).view(np.uint32) | inexact).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def round_storage(x, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage dtype; returns float64."""
    if dtype == "bf16":
        return round_f64_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# RoPE with one global scaling factor (关键设计 3)
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/d) for k in [0, d/2), float64."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.array([base ** (-2.0 * kk / head_dim) for kk in k], dtype=np.float64)


def yarn_inv_freq(head_dim: int, base: float, alpha: float, orig_ctx: int) -> np.ndarray:
    """Frequencies under a fixed YaRN scaling factor alpha (alpha = 1: plain RoPE).

    YaRN (Peng et al., 2023): with r_k = L_orig * theta_k / (2 pi) rotations over
    the original window and ramp gamma(r) = clamp((r - 1) / (32 - 1), 0, 1),
    theta'_k = (1 - gamma) * theta_k / alpha + gamma * theta_k.
    """
    theta = rope_inv_freq(head_dim, base)
    if alpha == 1.0:
        return theta
    out = np.empty_like(theta)
    for k, th in enumerate(theta):
        r = orig_ctx * th / (2.0 * math.pi)
        gamma = min(max((r - 1.0) / (32.0 - 1.0), 0.0), 1.0)
        out[k] = (1.0 - gamma) * th / alpha + gamma * th
    return out


def yarn_logit_scale(head_dim: int, alpha: float) -> float:
    """Softmax scale sigma = mscale^2 / sqrt(d), mscale = 0.1 ln(alpha) + 1."""
    mscale = 1.0 if alpha <= 1.0 else 0.1 * math.log(alpha) + 1.0
    return mscale * mscale / math.sqrt(head_dim)


def rope_cos_sin(positions, inv_freq: np.ndarray):
    """fp32-rounded cos and sin of (p * theta_k), angles and trig in float64.

    Returns two float64 arrays of shape [len(positions)][d/2] holding fp32 values.
    """
    positions = np.asarray(positions, dtype=np.int64)
    cos = np.empty((positions.size, inv_freq.size), dtype=np.float64)
    sin = np.empty_like(cos)
    for a, p in enumerate(positions):
        for k, th in enumerate(inv_freq):
            ang = float(p) * float(th)
            cos[a, k] = math.cos(ang)
            sin[a, k] = math.sin(ang)
    return (cos.astype(np.float32).astype(np.float64),
            sin.astype(np.float32).astype(np.float64))


def rope_rotate(x, cos, sin, dtype: str) -> np.ndarray:
    """Rotate-half RoPE: pairs (k, k + d/2) rotated by the angle of frequency k.

    x: [T][H][d] storage values; cos, sin: [T][d/2].  The rotation is computed
    in float64 and rounded once to the storage dtype.
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    y = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return round_storage(y, dtype)


# --------------------------------------------------------------------------
# The frame step
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LayerConfig:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tokens_per_frame: int
    budget: int
    dtype: str
    rope_base: float
    alpha: float = 1.0
    rope_orig_ctx: int = 32768
    # "statekv": keep the B best-scoring candidates (关键设计 2).  "recent": keep
    # the B most recent tokens, a sliding window over the stream (the ReKV
    # baseline's compute-matched window, 实验关键数据).
    policy: str = "statekv"

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclasses.dataclass
class CompressedState:
    """Kbar, Vbar: [Hkv][k][d] float64 storage values; pos: [k] absolute positions."""

    K: np.ndarray
    V: np.ndarray
    pos: np.ndarray

    @staticmethod
    def empty(cfg: LayerConfig) -> "CompressedState":
        z = np.zeros((cfg.n_kv_heads, 0, cfg.head_dim), dtype=np.float64)
        return CompressedState(z, z.copy(), np.zeros((0,), dtype=np.int64))

    @property
    def count(self) -> int:
        return int(self.pos.size)


@dataclasses.dataclass
class StepResult:
    Q_rot: np.ndarray        # [T][Hq][d] storage values
    K_rot: np.ndarray        # [T][Hkv][d] storage values (appended to D)
    V: np.ndarray            # [T][Hkv][d] (appended to D)
    O_exact: np.ndarray      # [T][Hq][d] float64 attention output
    O: np.ndarray            # [T][Hq][d] rounded to the storage dtype
    pool_pos: np.ndarray     # [P] positions of the candidate pool
    scores: np.ndarray       # [P] float64 mean attention per candidate
    scores32: np.ndarray     # [P] the same rounded to fp32
    keep: np.ndarray         # indices into the pool, ascending position
    state: CompressedState   # the next compressed state


def select_top_b(scores32: np.ndarray, pool_pos: np.ndarray, budget: int) -> np.ndarray:
    """Top-B by (score descending, position ascending); returned in pool order.

    The tie rule keeps the older token.  With fewer than B candidates all are kept.
    """
    n = scores32.size
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    order = sorted(range(n), key=lambda j: (-float(scores32[j]), int(pool_pos[j])))
    kept = np.array(sorted(order[:budget], key=lambda j: int(pool_pos[j])), dtype=np.int64)
    return kept


def select_recent(pool_pos: np.ndarray, budget: int) -> np.ndarray:
    """The B most recent candidates (largest positions), returned in pool order."""
    n = pool_pos.size
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    order = sorted(range(n), key=lambda j: -int(pool_pos[j]))
    return np.array(sorted(order[:budget], key=lambda j: int(pool_pos[j])), dtype=np.int64)


def frame_step(cfg: LayerConfig, state: CompressedState, Q, K, V, n: int) -> StepResult:
    """One layer's StateKV step for frame n (0-based) of the stream.

    Q: [T][Hq][d], K and V: [T][Hkv][d], holding storage-precision values.
    """
    T, Hq, Hkv, d = cfg.tokens_per_frame, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = cfg.group
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    assert Q.shape == (T, Hq, d) and K.shape == (T, Hkv, d) and V.shape == (T, Hkv, d)

    # 1. RoPE at the virtual positions nT + i with the fixed scaled table.
    frame_pos = n * T + np.arange(T, dtype=np.int64)
    inv_freq = yarn_inv_freq(d, cfg.rope_base, cfg.alpha, cfg.rope_orig_ctx)
    cos, sin = rope_cos_sin(frame_pos, inv_freq)
    Q_rot = rope_rotate(Q, cos, sin, cfg.dtype)
    K_rot = rope_rotate(K, cos, sin, cfg.dtype)

    # 2. Candidate pool: old compressed state followed by the frame's tokens.
    K_pool = np.concatenate([state.K, K_rot.transpose(1, 0, 2)], axis=1)  # [Hkv][P][d]
    V_pool = np.concatenate([state.V, V.transpose(1, 0, 2)], axis=1)
    pool_pos = np.concatenate([state.pos, frame_pos])
    P = pool_pos.size

    # 3. Attention of every query head over the pool.  A key is visible to
    #    query token i iff its position is <= nT + i: all state keys, and the
    #    frame's keys causally.
    sigma = yarn_logit_scale(d, cfg.alpha)
    visible = pool_pos[None, :] <= frame_pos[:, None]                   # [T][P]
    O_exact = np.zeros((T, Hq, d), dtype=np.float64)
    col_sum = np.zeros(P, dtype=np.float64)
    for h in range(Hq):
        g = h // G
        logits = sigma * (Q_rot[:, h, :] @ K_pool[g].T)                  # [T][P]
        logits = np.where(visible, logits, -np.inf)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        probs = w / w.sum(axis=1, keepdims=True)
        O_exact[:, h, :] = probs @ V_pool[g]
        col_sum += probs.sum(axis=0)

    # 4. Importance score: attention to key j averaged over the frame's T
    #    queries and the layer's Hq query heads (masked pairs count as 0).
    scores = col_sum / float(Hq * T)
    scores32 = scores.astype(np.float32).astype(np.float64)

    # 5. Top-B selection (or the recency window) and the next compressed
    #    state, kept in position order.
    if cfg.policy == "recent":
        keep = select_recent(pool_pos, cfg.budget)
    else:
        keep = select_top_b(scores32, pool_pos, cfg.budget)
    new_state = CompressedState(K_pool[:, keep, :].copy(), V_pool[:, keep, :].copy(),
                                pool_pos[keep].copy())

    return StepResult(Q_rot=Q_rot, K_rot=K_rot, V=V.copy(), O_exact=O_exact,
                      O=round_storage(O_exact, cfg.dtype), pool_pos=pool_pos,
                      scores=scores, scores32=scores32, keep=keep, state=new_state)


# --------------------------------------------------------------------------
# The text phase over the detailed cache (整体框架, 关键设计 1 and 3)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeResult:
    Q_rot: np.ndarray        # [t][Hq][d] storage values
    K_rot: np.ndarray        # [t][Hkv][d] storage values (appended to D)
    V: np.ndarray            # [t][Hkv][d] (appended to D)
    positions: np.ndarray    # [t] stream positions of the text tokens
    O_exact: np.ndarray      # [t][Hq][d] float64 attention output
    O: np.ndarray            # [t][Hq][d] rounded to the storage dtype


def decode_step(cfg: LayerConfig, D_K, D_V, Q, K, V) -> DecodeResult:
    """t text tokens attend over the whole detailed cache D and over themselves.

    Once the frames are processed, generation mounts the full detailed state D
    as its KV cache (整体框架; 关键设计 1).  The text continues the virtual
    length: with P0 rows in D (every frame token, then earlier text), text
    token i sits at position P0 + i and is rotated with the same fixed table
    (关键设计 3).  It sees every D row and the text tokens up to itself.
    D_K, D_V: [P0][Hkv][d] storage values in stream order (row = position);
    Q: [t][Hq][d], K and V: [t][Hkv][d].
    """
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = cfg.group
    D_K = np.asarray(D_K, dtype=np.float64).reshape(-1, Hkv, d)
    D_V = np.asarray(D_V, dtype=np.float64).reshape(-1, Hkv, d)
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    t = Q.shape[0]
    assert Q.shape == (t, Hq, d) and K.shape == (t, Hkv, d) and V.shape == (t, Hkv, d)
    P0 = D_K.shape[0]
    positions = P0 + np.arange(t, dtype=np.int64)
    inv_freq = yarn_inv_freq(d, cfg.rope_base, cfg.alpha, cfg.rope_orig_ctx)
    cos, sin = rope_cos_sin(positions, inv_freq)
    Q_rot = rope_rotate(Q, cos, sin, cfg.dtype)
    K_rot = rope_rotate(K, cos, sin, cfg.dtype)
    keys = np.concatenate([D_K, K_rot], axis=0)          # [P0+t][Hkv][d], row = position
    vals = np.concatenate([D_V, V], axis=0)
    key_pos = np.arange(P0 + t, dtype=np.int64)
    visible = key_pos[None, :] <= positions[:, None]      # [t][P0+t]
    sigma = yarn_logit_scale(d, cfg.alpha)
    O_exact = np.zeros((t, Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        logits = sigma * (Q_rot[:, h, :] @ keys[:, g, :].T)
        logits = np.where(visible, logits, -np.inf)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        O_exact[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ vals[:, g, :]
    return DecodeResult(Q_rot=Q_rot, K_rot=K_rot, V=V.copy(), positions=positions,
                        O_exact=O_exact, O=round_storage(O_exact, cfg.dtype))


class OracleStream:
    """Runs the oracle over consecutive frames, then text tokens, and keeps the
    detailed cache D."""

    def __init__(self, cfg: LayerConfig):
        self.cfg = cfg
        self.state = CompressedState.empty(cfg)
        self.frames_done = 0
        self.text_done = 0
        self.D_K = []
        self.D_V = []

    def step(self, Q, K, V) -> StepResult:
        assert self.text_done == 0, "frames come before the text"
        res = frame_step(self.cfg, self.state, Q, K, V, self.frames_done)
        self.state = res.state
        self.D_K.append(res.K_rot)   # detailed state: every frame's rotated keys
        self.D_V.append(res.V)       # and values, appended in stream order
        self.frames_done += 1
        return res

    def decode(self, Q, K, V) -> DecodeResult:
        """Text tokens after everything so far, attending over the whole of D."""
        D_K, D_V = self.detailed()
        res = decode_step(self.cfg, D_K, D_V, Q, K, V)
        self.D_K.append(res.K_rot)
        self.D_V.append(res.V)
        self.text_done += res.positions.size
        return res

    def detailed(self):
        """D as ([rows][Hkv][d], [rows][Hkv][d]), rows = n*T + text tokens."""
        if not self.D_K:
            z = np.zeros((0, self.cfg.n_kv_heads, self.cfg.head_dim), dtype=np.float64)
            return z, z.copy()
        return np.concatenate(self.D_K, axis=0), np.concatenate(self.D_V, axis=0)
