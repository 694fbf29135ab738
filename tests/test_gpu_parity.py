"""HIP path vs the CPU oracle on the same seeded frames (needs an MI355X).

Every checked frame is teacher-forced: the oracle starts from the GPU's own
compressed state before that frame.  Bars:
  * O: max over (token, head) of ||O - O_ref||_inf / ||O_ref||_inf below 2e-2
    (bf16) or 1e-5 (fp32);
  * rotated K and V appended to D, and every kept state row: bit-exact;
  * kept index sets: identical except candidates whose oracle score is within
    1e-6 relative of the B-th score;
  * scores (when computed): relative error below 1e-6 (bf16; 3e-6 for fp32
    inputs, whose logits carry fp32 rounding), summing to 1.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream, StreamConfig
from gpu_helpers import (StepCheck, assert_step_ok, gpu_state_as_oracle, make_state,
                         oracle_cfg, output_error, selection_violations, to_device, to_f64)
from oracle import OracleStream, frame_step

pytestmark = pytest.mark.gpu


def _small(name, cid, **kw):
    base = dict(name=name, config_id=cid, dtype="bf16", n_q_heads=8, n_kv_heads=2,
                head_dim=64, tokens_per_frame=200, budget=700, n_frames=6, n_layers=1,
                rope_base=1e6, alpha=1.0, n_sinks=4)
    base.update(kw)
    return StreamConfig(**base)


SMALL = {
    "tiny": CONFIGS["tiny"],
    # rows 800 = 3 full 256-row tiles + 32, pool 900 = 14 key blocks + 4
    "ragged_bf16_d64": _small("ragged_bf16_d64", 101),
    "ragged_bf16_d128_yarn": _small("ragged_bf16_d128_yarn", 102, n_q_heads=12, n_kv_heads=4,
                                    head_dim=128, tokens_per_frame=96, budget=333, n_frames=7,
                                    alpha=4.0, n_sinks=2),
    "f32_d128_mha": _small("f32_d128_mha", 103, dtype="f32", n_q_heads=3, n_kv_heads=3,
                           head_dim=128, tokens_per_frame=33, budget=50, n_frames=5,
                           rope_base=1e4, alpha=2.0, n_sinks=1),
    "bf16_t1_b1": _small("bf16_t1_b1", 104, n_q_heads=2, n_kv_heads=1, tokens_per_frame=1,
                         budget=1, n_frames=6, n_sinks=0),
    "bf16_g16_b_lt_t": _small("bf16_g16_b_lt_t", 105, n_q_heads=16, n_kv_heads=1,
                              tokens_per_frame=130, budget=97, n_frames=4, n_sinks=3),
    # G*T = 99 rows per KV head (not a multiple of 32) with several key splits
    "bf16_rows99_splits": _small("bf16_rows99_splits", 107, n_q_heads=6, n_kv_heads=2,
                                 tokens_per_frame=33, budget=700, n_frames=24, n_sinks=2),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_stream_every_frame(name):
    wl = SMALL[name]
    chk = StepCheck(wl, flags=skv.FLAG_ALWAYS_SCORE)
    for _ in range(wl.n_frames):
        rep = chk.step(check=True)
        print(rep, flush=True)
        assert_step_ok(rep, wl.dtype)


# Launch-shape overrides read at state creation change the split geometry
# (hence the rounding order of the split merges), never the method: every frame
# still matches the oracle.
SHAPES = [
    ("ragged_bf16_d64", {"STATEKV_ATTN_SPLITS": "1"}),
    ("ragged_bf16_d64", {"STATEKV_ATTN_SPLITS": "3", "STATEKV_SCORE_RSPLITS": "1"}),
    ("ragged_bf16_d128_yarn", {"STATEKV_SCORE_SLOTS": "8", "STATEKV_SCORE_RSPLITS": "64"}),
    # one split of up to 7 key blocks at d=128: the long-split loop, its
    # prefetch groups ending inside the last group (7 is not a multiple of 2)
    ("ragged_bf16_d128_yarn", {"STATEKV_ATTN_SPLITS": "1"}),
]


@pytest.mark.parametrize("name,env", SHAPES, ids=["one_split", "three_splits_one_rsplit",
                                                  "few_score_slots", "d128_one_split"])
def test_launch_shape_overrides(name, env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    wl = SMALL[name]
    chk = StepCheck(wl, flags=skv.FLAG_ALWAYS_SCORE)
    for _ in range(wl.n_frames):
        rep = chk.step(check=True)
        assert_step_ok(rep, wl.dtype)


# Full per-frame sizes of the five workloads, teacher-forced on sampled frames
# (the fill boundary, the first evicting frames, later frames).
FULL = [
    ("tiny", 0, 8, [0, 1, 2, 3, 7]),
    ("ivl3_1b", 0, 64, [0, 15, 16, 17, 40, 63]),
    ("ivl3_2b", 0, 512, [15, 16, 17, 300, 511]),
    ("ivl3_2b", 27, 24, [16, 23]),
    ("qwen3vl_2b", 0, 40, [0, 3, 4, 5, 21, 39]),
    ("qwen3vl_2b", 27, 8, [4, 7]),
    ("stress", 0, 70, [0, 63, 64, 65, 69]),
]


@pytest.mark.parametrize("name,layer,frames,check", FULL,
                         ids=[f"{c[0]}-L{c[1]}" for c in FULL])
def test_full_size_sampled_frames(name, layer, frames, check):
    wl = CONFIGS[name]
    chk = StepCheck(wl, layer=layer)
    worst = {}
    for n in range(frames):
        rep = chk.step(check=n in check)
        if rep is not None:
            print(name, layer, rep, flush=True)
            assert_step_ok(rep, wl.dtype)
            for key in ("out_err", "score_rel_max", "score_rel_p99", "score_rel_p50"):
                if key in rep:
                    worst[key] = max(worst.get(key, 0.0), rep[key])
    print("worst", name, layer, worst, flush=True)


# Free-running: the GPU and the oracle each carry their own state from frame 0
# on the same seeded frames.  Until the kept sets first differ, both states are
# the same, so every frame's output is compared and the first differing
# selection must lie inside the 1e-6 band around the oracle's B-th score (a
# legitimate divergence); after it the two streams may differ and the run stops.
@pytest.mark.parametrize("name,frames", [("ragged_bf16_d64", 30), ("ragged_bf16_d128_yarn", 20),
                                         ("f32_d128_mha", 20), ("bf16_g16_b_lt_t", 12),
                                         ("bf16_t1_b1", 40), ("ivl3_1b", 64)])
def test_free_running_stream(name, frames):
    wl = (SMALL.get(name) or CONFIGS[name]).replace(n_frames=frames)
    st = make_state(wl)
    fs = FrameStream(wl)
    orc = OracleStream(oracle_cfg(wl))
    tol = 2e-2 if wl.dtype == "bf16" else 1e-5
    first_divergence, worst = None, 0.0
    for n in range(frames):
        Q, K, V = fs.frame(n)
        O = st.prefill_frame(*[to_device(x, wl.dtype) for x in (Q, K, V)], n=n)
        res = orc.step(Q, K, V)
        err = output_error(to_f64(O), res.O_exact)
        worst = max(worst, err)
        assert err < tol, (n, err)
        _, _, pos = st.compressed_view()
        kept = pos.cpu().numpy()
        assert kept.size == res.state.pos.size
        viol = selection_violations(res, kept, wl.budget)
        assert not viol, (n, viol[:10])
        if set(kept.tolist()) != set(res.state.pos.tolist()):
            first_divergence = n
            break
    print(name, "frames", frames, "worst output error", worst,
          "first (in-band) divergence", first_divergence, flush=True)


# Everything is allocated when the state is created: evicting frames and text
# tokens leave the device's free memory unchanged.  A first state runs every
# kernel once beforehand, so that the runtime's lazy loading of code objects
# happens outside the measured region; inputs and outputs are staged before it.
def test_frames_and_text_allocate_nothing():
    import ctypes
    wl = SMALL["ragged_bf16_d64"].replace(n_frames=12)
    fs = FrameStream(wl)
    frames = [[to_device(x, wl.dtype) for x in fs.frame(n)] for n in range(wl.n_frames)]
    gen = torch.Generator().manual_seed(7)
    t, Hq, Hkv, d = 2, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    text = [torch.randn((t, h, d), generator=gen).to(torch.bfloat16).cuda() for h in (Hq, Hkv, Hkv)]
    O = torch.empty((wl.tokens_per_frame, Hq, d), dtype=torch.bfloat16, device="cuda")
    Ot = torch.empty((t, Hq, d), dtype=torch.bfloat16, device="cuda")
    hip = skv._hip_runtime()

    def free_bytes():
        torch.cuda.synchronize()
        free, total = ctypes.c_size_t(), ctypes.c_size_t()
        assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
        return free.value

    for st in (make_state(wl, max_text=4 * t), make_state(wl, max_text=4 * t)):
        st.prefill_frame(*frames[0], n=0, out=O)
        before = free_bytes()
        for n in range(1, wl.n_frames):
            st.prefill_frame(*frames[n], n=n, out=O)
        st.decode(*text, out=Ot)
        st.decode(*text, out=Ot)
        after = free_bytes()
    assert after == before, (before, after)
    _, _, pos = st.compressed_view()
    assert pos.numel() == wl.budget


# The largest pool the single-work-group selection takes: B + T = 32768
# candidates (32 rows per selection thread), teacher-forced at the fill
# boundary and on the first evicting frames.
LARGEST_POOL = _small("largest_pool", 108, n_q_heads=2, n_kv_heads=1, tokens_per_frame=256,
                      budget=32768 - 256, n_frames=130, n_sinks=4)


def test_largest_selection_pool():
    wl = LARGEST_POOL
    chk = StepCheck(wl)
    for n in range(wl.n_frames):
        rep = chk.step(check=n >= 126)
        if rep is not None:
            print(n, rep, flush=True)
            assert_step_ok(rep, wl.dtype)


@pytest.mark.parametrize("name,frames,check,extra", [
    ("ragged_bf16_d64", 9, None, 0),
    ("ragged_bf16_d128_yarn", 8, None, skv.FLAG_ALWAYS_SCORE),
    ("f32_d128_mha", 5, None, 0),
    ("ivl3_1b", 24, [15, 16, 17, 23], 0),
], ids=["bf16_d64", "bf16_d128_scored", "f32", "ivl3_1b"])
def test_recent_window_policy(name, frames, check, extra):
    """Recency window (the ReKV-style baseline): the GPU keeps exactly the last B
    tokens and its outputs match the oracle's recency policy."""
    wl = (SMALL.get(name) or CONFIGS[name]).replace(n_frames=frames)
    chk = StepCheck(wl, flags=skv.FLAG_RECENT_WINDOW | extra)
    T, B = wl.tokens_per_frame, wl.budget
    for n in range(frames):
        rep = chk.step(check=check is None or n in check)
        if rep is None:
            continue
        print(name, rep, flush=True)
        assert_step_ok(rep, wl.dtype)
        _, _, pos = chk.st.compressed_view()
        lo = max(0, (n + 1) * T - B)
        assert sorted(pos.cpu().numpy().tolist()) == list(range(lo, (n + 1) * T))


def test_bursts_are_exercised():
    wl = CONFIGS["qwen3vl_2b"]
    fs = FrameStream(wl, 0)
    assert any(fs.is_burst_frame(n) for n in range(4, 40))


def test_no_eviction_stream_reduces_to_full_attention():
    """B >= N*T: the GPU stream equals the oracle, which equals causal SDPA over
    all tokens (pinned on the CPU)."""
    wl = SMALL["ragged_bf16_d64"].replace(budget=6 * 200 + 5, n_frames=6)
    chk = StepCheck(wl)
    for _ in range(wl.n_frames):
        rep = chk.step(check=True)
        assert_step_ok(rep, wl.dtype)
    _, _, pos = chk.st.compressed_view()
    assert pos.cpu().numpy().tolist() == list(range(6 * 200))   # nothing evicted or moved


@pytest.mark.parametrize("T,B,before", [(8, 13, 2), (64, 1500, 24)], ids=["b13", "b1500"])
def test_exact_ties_keep_the_oldest(T, B, before):
    """All-zero queries: every state key and the frame's first key tie bit-exactly;
    with one slot too few the newest of them is evicted, exactly as the oracle.
    With B = 1500 the tie (1501 keys) is larger than the selection's candidate
    buffer, so the tie is broken by the refinement over positions."""
    wl = _small("ties", 106, n_q_heads=2, n_kv_heads=1, tokens_per_frame=T, budget=B,
                n_frames=before + 1, n_sinks=0)
    st = make_state(wl)
    cfg = oracle_cfg(wl)
    fs = FrameStream(wl)
    for n in range(before):
        st.prefill_frame(*[to_device(x, wl.dtype) for x in fs.frame(n)], n=n)
    Q, K, V = fs.frame(before)
    Q = np.zeros_like(Q)
    prior = gpu_state_as_oracle(st)
    assert prior.pos.size == B
    st.prefill_frame(*[to_device(x, wl.dtype) for x in (Q, K, V)], n=before)
    res = frame_step(cfg, prior, Q, K, V, before)
    _, _, pos = st.compressed_view()
    assert sorted(pos.cpu().numpy().tolist()) == sorted(res.state.pos.tolist())
    sc = st.scores()
    s = sc["scores"].cpu().numpy()
    assert len(set(s[:B + 1].tolist())) == 1       # B state keys + frame key 0
    assert sorted(res.state.pos.tolist()) == sorted(prior.pos.tolist())


def test_two_runs_are_bitwise_identical():
    wl = SMALL["ragged_bf16_d128_yarn"]
    outs = []
    for _ in range(2):
        st = make_state(wl)
        fs = FrameStream(wl)
        os_ = [st.prefill_frame(*[to_device(x, wl.dtype) for x in fs.frame(n)], n=n).cpu()
               for n in range(wl.n_frames)]
        k, v, pos = st.compressed_view()
        sc = st.scores()
        outs.append((os_, k.cpu(), v.cpu(), pos.cpu(), sc["scores"].cpu()))
        st.close()
    a, b = outs
    for x, y in zip(a[0], b[0]):
        assert torch.equal(x, y)
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x, y)


def test_side_stream_run_matches_default_stream():
    """The state takes torch's current stream at creation: a stream run on a
    side stream (inputs uploaded and outputs read on it) gives the same bits
    as on the default stream."""
    wl = SMALL["ragged_bf16_d64"]
    outs = []
    for side in (False, True):
        stream = torch.cuda.Stream() if side else torch.cuda.current_stream()
        with torch.cuda.stream(stream):
            st = make_state(wl)
            fs = FrameStream(wl)
            os_ = [st.prefill_frame(*[to_device(x, wl.dtype) for x in fs.frame(n)], n=n).cpu()
                   for n in range(wl.n_frames)]
            k, v, pos = st.compressed_view()
            dk, dv = st.detailed_view()
            outs.append((os_, k.cpu(), v.cpu(), pos.cpu(), dk.cpu(), dv.cpu()))
            st.close()
    a, b = outs
    for x, y in zip(a[0], b[0]):
        assert torch.equal(x, y)
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x, y)


def _run_bits(st, wl, frames_on):
    """Steps every frame of wl with the inputs uploaded, and the output read, on
    the stream frames_on(n) returns; returns the outputs and the final state."""
    fs = FrameStream(wl)
    outs = []
    for n in range(wl.n_frames):
        with torch.cuda.stream(frames_on(n)):
            x = [to_device(a, wl.dtype) for a in fs.frame(n)]
            outs.append(st.prefill_frame(*x, n=n).cpu())
    k, v, pos = st.compressed_view()
    return outs, (k.cpu(), v.cpu(), pos.cpu())


def test_state_stream_differs_from_current_stream():
    """A state created on the default stream, stepped while torch's current
    stream is a side stream (inputs produced and outputs read there): the
    binding orders the state's stream after the side stream and the side stream
    after the step, so the bits equal an all-default-stream run."""
    wl = SMALL["ragged_bf16_d64"]
    default = torch.cuda.current_stream()
    ref = _run_bits(make_state(wl), wl, lambda n: default)
    side = torch.cuda.Stream()
    st = make_state(wl)                       # state stream: the default stream
    assert st.stream == default
    got = _run_bits(st, wl, lambda n: side)
    for x, y in zip(ref[0], got[0]):
        assert torch.equal(x, y)
    for x, y in zip(ref[1], got[1]):
        assert torch.equal(x, y)


def test_set_stream_between_frames():
    """statekv_set_stream between frames (alternating two side streams, no host
    synchronisation): the new stream is ordered after the old one's work."""
    wl = SMALL["ragged_bf16_d64"]
    default = torch.cuda.current_stream()
    ref = _run_bits(make_state(wl), wl, lambda n: default)
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    st = make_state(wl)

    def on(n):
        st.set_stream(sides[n % 2])
        return sides[n % 2]

    got = _run_bits(st, wl, on)
    for x, y in zip(ref[0], got[0]):
        assert torch.equal(x, y)
    for x, y in zip(ref[1], got[1]):
        assert torch.equal(x, y)


def test_out_of_order_and_capacity_errors_leave_state_unchanged():
    wl = SMALL["tiny"].replace(n_frames=2)
    st = make_state(wl)
    fs = FrameStream(wl)
    f0 = [to_device(x, wl.dtype) for x in fs.frame(0)]
    with pytest.raises(skv.StateKVError) as e:
        st.prefill_frame(*f0, n=1)
    assert e.value.code == skv.STATEKV_EORDER
    st.prefill_frame(*f0, n=0)
    st.prefill_frame(*[to_device(x, wl.dtype) for x in fs.frame(1)], n=1)
    with pytest.raises(skv.StateKVError) as e:
        st.prefill_frame(*f0, n=2)
    assert e.value.code == skv.STATEKV_ECAPACITY
    _, _, pos = st.compressed_view()
    assert pos.numel() == 32


def test_nonfinite_input_is_reported():
    wl = SMALL["tiny"]
    st = make_state(wl)
    Q, K, V = FrameStream(wl).frame(0)
    K = K.copy()
    K[3, 0, 5] = np.nan
    st.prefill_frame(*[to_device(x, wl.dtype) for x in (Q, K, V)], n=0)
    with pytest.raises(skv.StateKVError) as e:
        st.compressed_view()
    assert e.value.code == skv.STATEKV_ENONFINITE


def test_binding_rejects_bad_tensors():
    wl = SMALL["tiny"]
    st = make_state(wl)
    Q, K, V = [to_device(x, wl.dtype) for x in FrameStream(wl).frame(0)]
    with pytest.raises(ValueError):
        st.prefill_frame(Q.to(torch.bfloat16), K, V, n=0)
    with pytest.raises(ValueError):
        st.prefill_frame(Q[:, :1], K, V, n=0)
    with pytest.raises(ValueError):
        st.prefill_frame(Q.cpu(), K, V, n=0)
