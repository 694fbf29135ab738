"""Seeded synthetic frame streams for the StateKV frame step.

This module only draws inputs.  It holds none of the method's arithmetic
(no RoPE, attention, scoring or selection), so both the HIP path and the CPU
oracle can consume the same values without sharing any computation.

Workload shapes follow the paper note "Linear Scaling Video VLMs for Long
Video Understanding" (papernotes.org, ECCV 2026), section "主实验": video is
sampled at 1 FPS for up to 512 frames and the compressed-state budget is
B = 4096; a sliding window of 16 frames matched to that budget implies
T = 256 visual tokens per frame.  The temporal-sink structure (few keys that
attract cross-frame attention and drift slowly over time) follows the note's
"研究背景与动机" paragraph and "关键设计 2".  The datasets the note evaluates
on are not used; these Gaussian streams stand in for them.

Layout of one frame (token-major, as a projection produces it):
  Q [T][Hq][d], K [T][Hkv][d], V [T][Hkv][d]

Every value is drawn from numpy's PCG64 seeded by
SeedSequence([20261202, config_id, layer, frame_slot, stream_tag]) where
frame_slot = n + 1 for frame n and 0 for per-layer initial draws.
bf16 configurations round the fp32 draws to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ROOT_SEED = 20261202

TAG_Q, TAG_K, TAG_V, TAG_SINK, TAG_BURST, TAG_TEXT = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class StreamConfig:
    """One synthetic workload: a layer shape plus the stream generator."""

    name: str
    config_id: int
    dtype: str              # "f32" or "bf16": storage and input precision
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tokens_per_frame: int   # T
    budget: int             # B
    n_frames: int           # N
    n_layers: int
    rope_base: float
    alpha: float            # global RoPE scaling factor, fixed for the stream
    rope_orig_ctx: int = 32768
    n_sinks: int = 0        # drifting sink keys per frame (tokens 0..n_sinks-1)
    sink_norm: float = 3.0
    sink_drift: float = 0.05
    burst_frac: float = 0.0  # fraction of frames with a burst of novel keys
    burst_keys: int = 0
    burst_norm: float = 2.5
    first_key_scale: float = 1.0  # scale of key token 0 of frame 0 (tiny sink)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "StreamConfig":
        return dataclasses.replace(self, **kw)


def _yarn_alpha(n_tokens: int, orig_ctx: int) -> float:
    """Smallest integer scaling factor whose extended window holds the stream."""
    return float(max(1, math.ceil(n_tokens / orig_ctx)))


CONFIGS = {
    "tiny": StreamConfig(
        name="tiny", config_id=1, dtype="f32", n_q_heads=2, n_kv_heads=1,
        head_dim=64, tokens_per_frame=16, budget=32, n_frames=8, n_layers=1,
        rope_base=1e4, alpha=1.0, first_key_scale=4.0),
    "ivl3_1b": StreamConfig(
        name="ivl3_1b", config_id=2, dtype="bf16", n_q_heads=14, n_kv_heads=2,
        head_dim=64, tokens_per_frame=256, budget=4096, n_frames=64, n_layers=1,
        rope_base=1e6, alpha=_yarn_alpha(64 * 256, 32768), n_sinks=4),
    "ivl3_2b": StreamConfig(
        name="ivl3_2b", config_id=3, dtype="bf16", n_q_heads=12, n_kv_heads=2,
        head_dim=128, tokens_per_frame=256, budget=4096, n_frames=512, n_layers=28,
        rope_base=1e6, alpha=4.0, n_sinks=4),
    "qwen3vl_2b": StreamConfig(
        name="qwen3vl_2b", config_id=4, dtype="bf16", n_q_heads=16, n_kv_heads=8,
        head_dim=128, tokens_per_frame=1024, budget=4096, n_frames=256, n_layers=28,
        rope_base=1e6, alpha=_yarn_alpha(256 * 1024, 32768), n_sinks=8,
        burst_frac=0.1, burst_keys=32),
    "stress": StreamConfig(
        name="stress", config_id=5, dtype="bf16", n_q_heads=32, n_kv_heads=8,
        head_dim=128, tokens_per_frame=256, budget=16384, n_frames=512, n_layers=1,
        rope_base=1e6, alpha=_yarn_alpha(512 * 256, 32768), n_sinks=4),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16 value, returned as fp32 (low 16 bits zero)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (bits >> 16).astype(np.uint16)


def _rng(cfg: StreamConfig, layer: int, frame_slot: int, tag: int) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, cfg.config_id, layer, frame_slot, tag])
    return np.random.Generator(np.random.PCG64(ss))


class FrameStream:
    """Frames of one (config, layer) stream; sequential access is O(1) per frame."""

    def __init__(self, cfg: StreamConfig, layer: int = 0):
        self.cfg = cfg
        self.layer = layer
        self._sink_n = -1
        self._sink = None
        self._burst_frames = None
        if cfg.burst_keys > 0 and cfg.burst_frac > 0:
            n_burst = int(round(cfg.burst_frac * cfg.n_frames))
            rng = _rng(cfg, layer, 0, TAG_BURST)
            self._burst_frames = frozenset(
                int(f) for f in rng.choice(cfg.n_frames, size=n_burst, replace=False))

    def is_burst_frame(self, n: int) -> bool:
        return self._burst_frames is not None and n in self._burst_frames

    def _sinks_at(self, n: int) -> np.ndarray:
        """Sink keys of frame n: [n_sinks][Hkv][d] fp32 (before bf16 rounding)."""
        cfg = self.cfg
        shape = (cfg.n_sinks, cfg.n_kv_heads, cfg.head_dim)
        if self._sink is None or n < self._sink_n:
            z0 = _rng(cfg, self.layer, 0, TAG_SINK).standard_normal(shape, dtype=np.float32)
            self._sink = (cfg.sink_norm * z0).astype(np.float32)
            self._sink_n = 0
        while self._sink_n < n:
            m = self._sink_n + 1
            z = _rng(cfg, self.layer, m + 1, TAG_SINK).standard_normal(shape, dtype=np.float32)
            self._sink = (self._sink + np.float32(cfg.sink_drift) * z).astype(np.float32)
            self._sink_n = m
        return self._sink

    def frame(self, n: int):
        """(Q, K, V) of frame n as fp32 arrays holding storage-precision values."""
        cfg = self.cfg
        if not 0 <= n:
            raise ValueError("frame index must be >= 0")
        T, Hq, Hkv, d = cfg.tokens_per_frame, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        slot = n + 1
        q = _rng(cfg, self.layer, slot, TAG_Q).standard_normal((T, Hq, d), dtype=np.float32)
        k = _rng(cfg, self.layer, slot, TAG_K).standard_normal((T, Hkv, d), dtype=np.float32)
        v = _rng(cfg, self.layer, slot, TAG_V).standard_normal((T, Hkv, d), dtype=np.float32)
        if n == 0 and cfg.first_key_scale != 1.0:
            k[0] *= np.float32(cfg.first_key_scale)
        if cfg.n_sinks > 0:
            k[: cfg.n_sinks] = self._sinks_at(n)
        if self.is_burst_frame(n):
            rng = _rng(cfg, self.layer, slot, TAG_BURST)
            where = cfg.n_sinks + rng.choice(T - cfg.n_sinks, size=cfg.burst_keys, replace=False)
            z = rng.standard_normal((cfg.burst_keys, Hkv, d), dtype=np.float32)
            k[np.sort(where)] = np.float32(cfg.burst_norm) * z
        if cfg.dtype == "bf16":
            q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
        return q, k, v


def text_tokens(cfg: StreamConfig, first_pos: int, t: int, layer: int = 0):
    """(Q, K, V) of t text tokens starting at stream position first_pos (the
    text phase after the frames): N(0, 1) draws, [t][H][d] fp32 arrays holding
    storage values, seeded by (config, layer, first_pos + 1, text tag)."""
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    rng = _rng(cfg, layer, first_pos + 1, TAG_TEXT)
    q = rng.standard_normal((t, Hq, d), dtype=np.float32)
    k = rng.standard_normal((t, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((t, Hkv, d), dtype=np.float32)
    if cfg.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def stream_tokens(cfg: StreamConfig, n_frames: int, layer: int = 0):
    """Q, K, V of frames 0 .. n_frames-1 of one layer's stream, concatenated
    along tokens: [n_frames*T][H][d] fp32 arrays holding storage values.  The
    input of one-shot full causal attention over the same tokens."""
    T, Hq, Hkv, d = cfg.tokens_per_frame, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    L = n_frames * T
    Q = np.empty((L, Hq, d), dtype=np.float32)
    K = np.empty((L, Hkv, d), dtype=np.float32)
    V = np.empty((L, Hkv, d), dtype=np.float32)
    fs = FrameStream(cfg, layer)
    for n in range(n_frames):
        Q[n * T:(n + 1) * T], K[n * T:(n + 1) * T], V[n * T:(n + 1) * T] = fs.frame(n)
    return Q, K, V


def to_storage_bytes(x: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage of a frame tensor: uint16 bf16 bits or fp32."""
    if dtype == "bf16":
        return bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)
