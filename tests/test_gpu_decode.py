"""Text phase over the detailed cache D: HIP path vs the CPU oracle (needs an MI355X).

After a stream of frames (with eviction, so the compressed state no longer
holds every token), text tokens are appended in chunks and attend causally
over the whole of D.  Bars:
  * O: max over (token, head) of ||O - O_ref||_inf / ||O_ref||_inf below 2e-2
    (bf16) or 1e-5 (fp32), the oracle computing from the GPU's D (whose frame
    rows are first checked bit-exactly against the oracle's RoPE);
  * the text rows appended to D (rotated K, V): bit-exact.
Chunk sizes cover one token (decode proper), a whole frame's worth (a prompt
chunk: many 32-row tiles, ragged tail) and both the one-split (direct output)
and the many-split (merge kernel) launch shapes.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream, text_tokens
from gpu_helpers import (OUT_TOL, StepCheck, assert_step_ok, make_state, oracle_cfg, output_error,
                         to_device, to_f64)
from oracle import decode_step, rope_cos_sin, rope_rotate, yarn_inv_freq
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _frame_rows_exact(cfg, dk, dv, frames, fs, T):
    """D rows of the given frames equal the oracle's RoPE of the frame's K (and V)."""
    inv = yarn_inv_freq(cfg.head_dim, cfg.rope_base, cfg.alpha, cfg.rope_orig_ctx)
    for n in frames:
        _, K, V = fs.frame(n)
        cos, sin = rope_cos_sin(n * T + np.arange(T), inv)
        if not np.array_equal(to_f64(dk[n * T:(n + 1) * T]), rope_rotate(K, cos, sin, cfg.dtype)):
            return False
        if not np.array_equal(to_f64(dv[n * T:(n + 1) * T]), V.astype(np.float64)):
            return False
    return True


def _run(wl, n_frames, chunks, check_frames=None, frame_cycle=None, env=None):
    """Prefill n_frames (frame n uses seeded frame n % frame_cycle), then decode
    the chunks; every chunk is checked against the oracle."""
    T = wl.tokens_per_frame
    cfg = oracle_cfg(wl)
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update(env or {})
    try:
        st = make_state(wl, max_frames=max(n_frames, 1), max_text=sum(chunks))
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    fs = FrameStream(wl)
    for n in range(n_frames):
        Q, K, V = fs.frame(n if frame_cycle is None else n % frame_cycle)
        st.prefill_frame(to_device(Q, wl.dtype), to_device(K, wl.dtype), to_device(V, wl.dtype), n)
    dk, dv = st.detailed_view()
    assert dk.shape[0] == n_frames * T
    if frame_cycle is None:
        frames = range(n_frames) if check_frames is None else check_frames
        assert _frame_rows_exact(cfg, dk, dv, frames, fs, T)
    D_K, D_V = to_f64(dk), to_f64(dv)
    worst = 0.0
    pos = n_frames * T
    for t in chunks:
        Q, K, V = text_tokens(wl, pos, t)
        O = st.decode(to_device(Q, wl.dtype), to_device(K, wl.dtype), to_device(V, wl.dtype))
        torch.cuda.synchronize()
        res = decode_step(cfg, D_K, D_V, Q, K, V)
        err = output_error(to_f64(O), res.O_exact)
        print(wl.name, "frames", n_frames, "chunk", t, "at", pos, "out_err", err, flush=True)
        assert err <= OUT_TOL[wl.dtype], (t, pos, err)
        dk, dv = st.detailed_view()
        assert dk.shape[0] == pos + t
        assert np.array_equal(to_f64(dk[pos:pos + t]), res.K_rot)
        assert np.array_equal(to_f64(dv[pos:pos + t]), res.V)
        D_K = np.concatenate([D_K, res.K_rot])
        D_V = np.concatenate([D_V, res.V])
        pos += t
        worst = max(worst, err)
    print("worst", wl.name, worst, flush=True)
    return st


SMALL_CASES = [
    # (config, frames, chunks)
    ("tiny", 8, [1, 16, 3, 1]),
    ("ragged_bf16_d64", 6, [1, 3, 200, 37, 1]),
    ("ragged_bf16_d128_yarn", 7, [1, 96, 5, 1]),
    ("f32_d128_mha", 5, [1, 33, 2]),
    ("bf16_g16_b_lt_t", 4, [1, 130, 2]),
    ("bf16_t1_b1", 6, [1, 1, 1]),
]


@pytest.mark.parametrize("name,frames,chunks", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_text_phase(name, frames, chunks):
    _run(SMALL[name], frames, chunks)


@pytest.mark.parametrize("env", [{"STATEKV_DECODE_WGS": "1"}, {"STATEKV_DECODE_WGS": "100000"}],
                         ids=["one_split", "one_block_per_split"])
def test_launch_shapes(env):
    """The result does not depend on the split geometry: one split (each
    work-group walks all keys and writes O) or one block per split."""
    _run(SMALL["ragged_bf16_d128_yarn"], 7, [1, 96, 3], env=env)


def test_text_without_frames():
    """No frame processed: the text attends over itself only (positions 0..)."""
    _run(SMALL["ragged_bf16_d64"], 0, [1, 5, 200])


FULL = [
    # (config, frames, chunks, frame_cycle): the stream's full length
    ("ivl3_1b", 64, [1, 1, 64, 1], None),
    ("ivl3_2b", 512, [1, 48, 1], None),
    ("stress", 512, [1, 1], None),
    # 262144 frame tokens; the frames cycle through 8 seeded frames (positions,
    # hence rotated keys, still differ) to keep host generation short
    ("qwen3vl_2b", 256, [1, 17, 1], 8),
]


@pytest.mark.parametrize("name,frames,chunks,cycle", FULL, ids=[c[0] for c in FULL])
def test_full_size_text_phase(name, frames, chunks, cycle):
    wl = CONFIGS[name]
    T = wl.tokens_per_frame
    check = sorted({0, frames // 2, frames - 1})
    _run(wl, frames, chunks, check_frames=check, frame_cycle=cycle)


@pytest.mark.parametrize("name,frames,check", [("ragged_bf16_d128_yarn", 7, None),
                                               ("ivl3_1b", 20, [15, 16, 19])],
                         ids=["small", "ivl3_1b"])
def test_frames_with_text_capacity(name, frames, check):
    """A state with text capacity lays out the frame step's split partials with
    a wider stride: the frames must still match the oracle, and the text
    that follows must too."""
    wl = (SMALL.get(name) or CONFIGS[name]).replace(n_frames=frames)
    chk = StepCheck(wl, flags=skv.FLAG_ALWAYS_SCORE, max_text=8)
    for n in range(frames):
        rep = chk.step(check=check is None or n in check)
        if rep is not None:
            print(name, rep, flush=True)
            assert_step_ok(rep, wl.dtype)
    dk, dv = chk.st.detailed_view()
    Q, K, V = text_tokens(wl, frames * wl.tokens_per_frame, 8)
    O = chk.st.decode(to_device(Q, wl.dtype), to_device(K, wl.dtype), to_device(V, wl.dtype))
    res = decode_step(oracle_cfg(wl), to_f64(dk), to_f64(dv), Q, K, V)
    assert output_error(to_f64(O), res.O_exact) <= OUT_TOL[wl.dtype]


def test_order_and_capacity_errors():
    wl = SMALL["ragged_bf16_d64"]
    st = make_state(wl, max_frames=2, max_text=5)
    fs = FrameStream(wl)
    f0 = [to_device(x, wl.dtype) for x in fs.frame(0)]
    st.prefill_frame(*f0, n=0)
    q, k, v = [to_device(x, wl.dtype) for x in text_tokens(wl, 200, 4)]
    st.decode(q, k, v)
    # frames after the text phase has begun: EORDER, state unchanged
    with pytest.raises(skv.StateKVError) as e:
        st.prefill_frame(*[to_device(x, wl.dtype) for x in fs.frame(1)], n=1)
    assert e.value.code == skv.STATEKV_EORDER
    # beyond max_text: ECAPACITY
    with pytest.raises(skv.StateKVError) as e:
        st.decode(q[:2], k[:2], v[:2])
    assert e.value.code == skv.STATEKV_ECAPACITY
    st.decode(q[:1], k[:1], v[:1])
    dk, _ = st.detailed_view()
    assert dk.shape[0] == 205
    # a state created without text capacity rejects decode
    st2 = make_state(wl, max_frames=1)
    with pytest.raises(skv.StateKVError) as e:
        st2.decode(q[:1], k[:1], v[:1])
    assert e.value.code == skv.STATEKV_ECAPACITY


def test_chunk_longer_than_a_frame_is_rejected():
    wl = SMALL["tiny"]
    st = make_state(wl, max_text=64)
    q, k, v = [to_device(x, wl.dtype) for x in text_tokens(wl, 0, 17)]
    with pytest.raises(skv.StateKVError) as e:
        st.decode(q, k, v)
    assert e.value.code == skv.STATEKV_EINVAL


@pytest.mark.parametrize("t,field", [(1, "k"), (1, "q"), (50, "v")], ids=["fused_k", "fused_q", "rope_v"])
def test_nonfinite_text_is_reported(t, field):
    """A NaN in the text inputs is reported by the next view, whether the
    attention kernel rotates the tokens itself (one row tile) or not."""
    wl = SMALL["ragged_bf16_d64"]
    st = make_state(wl, max_frames=1, max_text=64)
    st.prefill_frame(*[to_device(x, wl.dtype) for x in FrameStream(wl).frame(0)], n=0)
    q, k, v = (x.copy() for x in text_tokens(wl, 200, t))
    {"q": q, "k": k, "v": v}[field][t - 1, 0, 3] = np.nan
    st.decode(*[to_device(x, wl.dtype) for x in (q, k, v)])
    with pytest.raises(skv.StateKVError) as e:
        st.detailed_view()
    assert e.value.code == skv.STATEKV_ENONFINITE
