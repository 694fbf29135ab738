"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on the
same seeded frames and compare them to the stated bars."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import FrameStream, StreamConfig
from oracle import CompressedState, LayerConfig, frame_step

# Output tolerance: max over (token, head) of ||O - O_ref||_inf / ||O_ref||_inf.
OUT_TOL = {"bf16": 2e-2, "f32": 1e-5}
# Selections must agree except for candidates within this relative distance of
# the B-th score.
BAND = 1e-6
# Scores: relative error of every candidate's fp32 score against the oracle's
# fp64 mean attention.  bf16 inputs: products are exact in fp32, so a weight's
# error comes from the fp32 sums and the exponent argument; measured below
# 7e-7.  fp32 inputs (the tiny and MHA test streams): every product of the
# logit is rounded too, and a weight 2^a of a low-scoring key carries about
# ln2 * |a| * 2^-24 from its fp32 argument (|a| up to ~20 in these streams);
# measured up to 1.9e-6, so the bar is 3e-6.
SCORE_TOL = {"bf16": 1e-6, "f32": 3e-6}


def oracle_cfg(wl: StreamConfig) -> LayerConfig:
    return LayerConfig(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                       tokens_per_frame=wl.tokens_per_frame, budget=wl.budget, dtype=wl.dtype,
                       rope_base=wl.rope_base, alpha=wl.alpha, rope_orig_ctx=wl.rope_orig_ctx)


def make_state(wl: StreamConfig, max_frames: int | None = None, max_text: int = 0,
               layers: int = 1) -> skv.StateKV:
    return skv.StateKV(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                       tokens_per_frame=wl.tokens_per_frame,
                       max_frames=max_frames or wl.n_frames, budget=wl.budget, alpha=wl.alpha,
                       dtype=wl.dtype, rope_base=wl.rope_base, rope_orig_ctx=wl.rope_orig_ctx,
                       max_text=max_text, n_layers=layers)


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)   # values are already bf16-representable: exact
    return t.cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_state_as_oracle(st: skv.StateKV, layer: int = 0) -> CompressedState:
    k, v, pos = st.compressed_view(layer)
    return CompressedState(to_f64(k), to_f64(v), pos.cpu().numpy().astype(np.int64))


def output_error(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    num = np.abs(o_gpu - o_ref).max(axis=-1)
    den = np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def selection_violations(res, keep_pos_gpu: np.ndarray, budget: int, policy: str = "statekv"):
    """Candidates kept by one side only whose oracle score lies outside the band
    (the recency window has no band: its set must be identical)."""
    kept_o = set(res.state.pos.tolist())
    kept_g = set(int(p) for p in keep_pos_gpu)
    if res.pool_pos.size <= budget or policy == "recent":
        return sorted(kept_o ^ kept_g)
    s = res.scores32
    order = sorted(range(s.size), key=lambda j: (-s[j], res.pool_pos[j]))
    s_b = s[order[budget - 1]]
    by_pos = {int(p): float(s[j]) for j, p in enumerate(res.pool_pos)}
    return sorted(p for p in kept_o ^ kept_g if abs(by_pos.get(p, np.inf) - s_b) > BAND * s_b)


class StepCheck:
    """Runs one stream on the GPU; frames in `check` are compared with the oracle
    started from the GPU's own state before that frame (teacher forcing).

    layers > 1 runs a stack: layer l of the stack takes the seeded stream of
    layer `layer + l`, and the layers in check_layers (default: all) are each
    compared with the oracle; step() then returns a list of reports."""

    def __init__(self, wl: StreamConfig, layer: int = 0, flags: int = 0, max_frames=None,
                 max_text: int = 0, layers: int = 1, check_layers=None):
        self.wl = wl
        self.cfg = oracle_cfg(wl)
        if flags & skv.FLAG_RECENT_WINDOW:
            self.cfg = dataclasses.replace(self.cfg, policy="recent")
        self.L = layers
        self.check_layers = list(range(layers)) if check_layers is None else list(check_layers)
        self.st = make_state(wl, max_frames, max_text, layers)
        if flags:
            self.st.set_flags(flags)
        self.streams = [FrameStream(wl, layer + l) for l in range(layers)]
        self.frames = self.streams[0]
        self.n = 0
        self.report = []

    def _inputs(self, frames):
        dt = self.wl.dtype
        if self.L == 1:
            return [to_device(x, dt) for x in frames[0]]
        return [to_device(np.stack([f[i] for f in frames]), dt) for i in range(3)]

    def step(self, check: bool):
        wl, n = self.wl, self.n
        frames = [fs.frame(n) for fs in self.streams]
        befores = {l: gpu_state_as_oracle(self.st, l) for l in self.check_layers} if check else None
        O = self.st.prefill_frame(*self._inputs(frames), n)
        self.n += 1
        if not check:
            return None
        torch.cuda.synchronize()
        reps = []
        for l in self.check_layers:
            o = O if self.L == 1 else O[l]
            reps.append(self._compare(l, befores[l], frames[l], o, n))
        return reps[0] if self.L == 1 else reps

    def _compare(self, layer, before, frame, O, n):
        wl = self.wl
        Q, K, V = frame
        res = frame_step(self.cfg, before, Q, K, V, n)
        rep = {"frame": n, "layer": layer, "out_err": output_error(to_f64(O), res.O_exact)}
        # Detailed cache rows of this frame: bit-exact rotated K and V.
        dk, dv = self.st.detailed_view(layer)
        T = wl.tokens_per_frame
        rep["d_k_exact"] = bool(np.array_equal(to_f64(dk[n * T:(n + 1) * T]), res.K_rot))
        rep["d_v_exact"] = bool(np.array_equal(to_f64(dv[n * T:(n + 1) * T]), res.V))
        # New compressed state: positions and rows.
        k_new, v_new, pos_new = self.st.compressed_view(layer)
        pos_new = pos_new.cpu().numpy().astype(np.int64)
        rep["state_size"] = (int(pos_new.size), int(res.state.count))
        rep["violations"] = selection_violations(res, pos_new, wl.budget, self.cfg.policy)
        # The state is a set of slots: positions are unique (slot order is free).
        rep["unique"] = bool(np.unique(pos_new).size == pos_new.size)
        # Every kept row equals the pool row at its position (bit-exact).
        K_pool = np.concatenate([before.K, res.K_rot.transpose(1, 0, 2)], axis=1)
        V_pool = np.concatenate([before.V, res.V.transpose(1, 0, 2)], axis=1)
        idx = {int(p): j for j, p in enumerate(res.pool_pos)}
        sel = [idx.get(int(p), -1) for p in pos_new]
        rep["rows_exact"] = (min(sel) >= 0
                             and bool(np.array_equal(to_f64(k_new), K_pool[:, sel]))
                             and bool(np.array_equal(to_f64(v_new), V_pool[:, sel])))
        # Independent of teacher forcing: every state row is the detailed-cache
        # row of its token, so moves done in earlier (unchecked) frames are
        # verified too.
        pos_t = torch.from_numpy(pos_new).to(dk.device)
        rep["state_matches_D"] = (bool(torch.equal(k_new, dk[pos_t].transpose(0, 1)))
                                  and bool(torch.equal(v_new, dv[pos_t].transpose(0, 1))))
        sc = self.st.scores(layer)
        if sc is not None and sc["frame"] == n:
            s_gpu = sc["scores"].cpu().numpy().astype(np.float64)
            rel = np.abs(s_gpu - res.scores) / np.maximum(res.scores, 1e-300)
            rep["score_rel_max"] = float(rel.max())
            rep["score_rel_p99"] = float(np.quantile(rel, 0.99))
            rep["score_rel_p50"] = float(np.quantile(rel, 0.5))
            rep["score_sum"] = float(s_gpu.sum())
            rep["pool_pos_exact"] = bool(np.array_equal(sc["pool_pos"].cpu().numpy(), res.pool_pos))
            kept = sc["pool_pos"].cpu().numpy()[sc["keep_flag"].cpu().numpy() == 1]
            rep["keep_flag_matches_state"] = sorted(kept.tolist()) == sorted(pos_new.tolist())
        self.report.append(rep)
        return rep


def assert_step_ok(rep, dtype: str, score_tol: float | None = None):
    score_tol = SCORE_TOL[dtype] if score_tol is None else score_tol
    assert rep["out_err"] <= OUT_TOL[dtype], rep
    assert rep["d_k_exact"] and rep["d_v_exact"], rep
    assert rep["state_size"][0] == rep["state_size"][1], rep
    assert rep["unique"] and rep["rows_exact"] and rep["state_matches_D"], rep
    assert not rep["violations"], rep
    if "score_rel_max" in rep:
        assert rep["score_rel_max"] <= score_tol, rep
        assert abs(rep["score_sum"] - 1.0) < 1e-4, rep
        assert rep["pool_pos_exact"] and rep["keep_flag_matches_state"], rep
