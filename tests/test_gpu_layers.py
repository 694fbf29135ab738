"""Layer stacks: L independent layers stepped together by one state, every
frame-step kernel covering all layers in one launch (needs an MI355X).

Layer l of a stack takes its own seeded stream, and each checked layer is
compared with the oracle exactly as a single-layer state is (teacher-forced
frames; the bars of test_gpu_parity: output error, bit-exact D rows and state
rows, selections outside the 1e-6 band, scores).  Distinct streams per layer
make any mix-up of layers (a wrong layer offset in a kernel) show as a
mismatch.  The text phase over each layer's D is checked the same way.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream, text_tokens
from gpu_helpers import (OUT_TOL, StepCheck, assert_step_ok, make_state, oracle_cfg, output_error,
                         to_device, to_f64)
from oracle import decode_step
from test_gpu_decode import _frame_rows_exact
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


SMALL_STACKS = [
    # (config, layers, flags)
    ("tiny", 3, skv.FLAG_ALWAYS_SCORE),
    ("ragged_bf16_d64", 3, skv.FLAG_ALWAYS_SCORE),
    ("ragged_bf16_d128_yarn", 4, 0),
    ("f32_d128_mha", 2, skv.FLAG_ALWAYS_SCORE),
    ("bf16_t1_b1", 5, 0),
    ("bf16_rows99_splits", 3, 0),
    ("ragged_bf16_d64", 3, skv.FLAG_RECENT_WINDOW),
]


@pytest.mark.parametrize("name,layers,flags", SMALL_STACKS,
                         ids=[f"{c[0]}-L{c[1]}-f{c[2]}" for c in SMALL_STACKS])
def test_small_stack_every_frame(name, layers, flags):
    wl = SMALL[name]
    chk = StepCheck(wl, flags=flags, layers=layers)
    for _ in range(wl.n_frames):
        for rep in chk.step(check=True):
            print(rep, flush=True)
            assert_step_ok(rep, wl.dtype)
    if flags & skv.FLAG_RECENT_WINDOW:
        T, B, n = wl.tokens_per_frame, wl.budget, wl.n_frames
        for l in range(layers):
            _, _, pos = chk.st.compressed_view(l)
            assert sorted(pos.cpu().numpy().tolist()) == list(range(max(0, n * T - B), n * T))


# Full per-layer sizes: the fill boundary and the first evicting frames, on
# the first, a middle and the last layer of the stack.
FULL_STACKS = [
    # (config, layers, frames, check frames, check layers)
    ("ivl3_1b", 4, 20, [15, 16, 19], None),
    ("ivl3_2b", 28, 18, [16, 17], [0, 13, 27]),
    ("qwen3vl_2b", 28, 6, [4, 5], [0, 27]),
    ("stress", 2, 66, [64, 65], None),
]


@pytest.mark.parametrize("name,layers,frames,check,check_layers", FULL_STACKS,
                         ids=[f"{c[0]}-L{c[1]}" for c in FULL_STACKS])
def test_full_size_stack(name, layers, frames, check, check_layers):
    wl = CONFIGS[name]
    chk = StepCheck(wl, layers=layers, check_layers=check_layers, max_frames=frames)
    worst = 0.0
    for n in range(frames):
        reps = chk.step(check=n in check)
        for rep in reps or []:
            print(name, rep, flush=True)
            assert_step_ok(rep, wl.dtype)
            worst = max(worst, rep["out_err"])
    print("worst", name, layers, worst, flush=True)


@pytest.mark.parametrize("name,layers,frames,chunks", [
    ("ragged_bf16_d64", 3, 6, [1, 3, 200, 1]),
    ("ragged_bf16_d128_yarn", 2, 7, [1, 96, 1]),
    ("f32_d128_mha", 3, 5, [1, 33, 2]),
], ids=["bf16_d64", "bf16_d128", "f32"])
def test_stack_text_phase(name, layers, frames, chunks):
    """Text chunks (one token: the fused kernel; long chunks: pass 1 over D and
    the merge) on every layer of a stack, against the oracle over that layer's D."""
    wl = SMALL[name]
    T = wl.tokens_per_frame
    cfg = oracle_cfg(wl)
    st = make_state(wl, max_frames=frames, max_text=sum(chunks), layers=layers)
    streams = [FrameStream(wl, l) for l in range(layers)]
    for n in range(frames):
        fr = [fs.frame(n) for fs in streams]
        st.prefill_frame(*[to_device(np.stack([f[i] for f in fr]), wl.dtype) for i in range(3)], n)
    D = []
    for l in range(layers):
        dk, dv = st.detailed_view(l)
        assert _frame_rows_exact(cfg, dk, dv, range(frames), streams[l], T)
        D.append([to_f64(dk), to_f64(dv)])
    pos = frames * T
    for t in chunks:
        toks = [text_tokens(wl, pos, t, layer=l) for l in range(layers)]
        O = st.decode(*[to_device(np.stack([x[i] for x in toks]), wl.dtype) for i in range(3)])
        torch.cuda.synchronize()
        for l in range(layers):
            res = decode_step(cfg, D[l][0], D[l][1], *toks[l])
            err = output_error(to_f64(O[l]), res.O_exact)
            print(name, "layer", l, "chunk", t, "at", pos, "out_err", err, flush=True)
            assert err <= OUT_TOL[wl.dtype], (l, t, pos, err)
            dk, dv = st.detailed_view(l)
            assert np.array_equal(to_f64(dk[pos:pos + t]), res.K_rot)
            assert np.array_equal(to_f64(dv[pos:pos + t]), res.V)
            D[l][0] = np.concatenate([D[l][0], res.K_rot])
            D[l][1] = np.concatenate([D[l][1], res.V])
        pos += t


def test_stack_rejects_single_layer_shapes():
    wl = SMALL["ragged_bf16_d64"]
    st = make_state(wl, max_frames=2, layers=2)
    Q, K, V = FrameStream(wl).frame(0)
    with pytest.raises(ValueError):
        st.prefill_frame(to_device(Q, wl.dtype), to_device(K, wl.dtype), to_device(V, wl.dtype), 0)
    with pytest.raises(ValueError):
        st.compressed_view(2)
