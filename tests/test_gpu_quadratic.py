"""The quadratic baseline at the stress shape (needs an MI355X): one-shot full
causal attention over all 512 x 256 = 131072 tokens of the stress stream,
run as one frame of a state that never evicts (B = N*T).

Bars, against the oracle's definition of the step computed from the raw
inputs (no GPU value enters the reference):
  * rotated keys in D: bit-exact on sampled tokens;
  * O on sampled (token, head) rows: ||O - O_ref||_inf / ||O_ref||_inf <= 2e-2,
    with O_ref = softmax(sigma * Q_rot K_rot^T over keys 0..t) V in fp64.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import CONFIGS, stream_tokens
from gpu_helpers import OUT_TOL, to_device, to_f64
from oracle import rope_cos_sin, rope_rotate, yarn_inv_freq, yarn_logit_scale

pytestmark = pytest.mark.gpu


def test_one_shot_full_causal_attention_stress_shape():
    wl = CONFIGS["stress"]
    N, T = wl.n_frames, wl.tokens_per_frame
    L = N * T
    Hq, Hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    G = Hq // Hkv
    Q, K, V = stream_tokens(wl, N)
    print("inputs generated", L, flush=True)
    st = skv.StateKV(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, tokens_per_frame=L, max_frames=1,
                     budget=L, alpha=wl.alpha, dtype=wl.dtype, rope_base=wl.rope_base,
                     rope_orig_ctx=wl.rope_orig_ctx)
    O = st.prefill_frame(to_device(Q, wl.dtype), to_device(K, wl.dtype), to_device(V, wl.dtype), 0)
    torch.cuda.synchronize()
    dk, _ = st.detailed_view()
    print("gpu done", flush=True)

    inv = yarn_inv_freq(d, wl.rope_base, wl.alpha, wl.rope_orig_ctx)
    sigma = yarn_logit_scale(d, wl.alpha)
    heads = [0, 13, 31]
    groups = sorted({h // G for h in heads})
    # Rotated keys of every token for the sampled KV heads, from the raw inputs.
    cos, sin = rope_cos_sin(np.arange(L), inv)
    K_rot = rope_rotate(K[:, groups], cos, sin, wl.dtype)          # [L][len(groups)][d]
    tokens = [0, 1, 255, 256, 4099, 65535, 98304, L - 1]
    dk_s = to_f64(dk[tokens][:, groups])
    assert np.array_equal(dk_s, K_rot[tokens]), "rotated keys in D differ from the oracle"
    Q_rot = rope_rotate(Q[tokens], cos[tokens], sin[tokens], wl.dtype)   # [len(tokens)][Hq][d]
    Vd = V.astype(np.float64)
    O_gpu = to_f64(O[tokens])
    worst = 0.0
    for a, t in enumerate(tokens):
        for h in heads:
            gi = groups.index(h // G)
            logits = sigma * (K_rot[: t + 1, gi] @ Q_rot[a, h])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            o_ref = p @ Vd[: t + 1, h // G]
            err = np.abs(O_gpu[a, h] - o_ref).max() / np.abs(o_ref).max()
            worst = max(worst, err)
            assert err <= OUT_TOL[wl.dtype], (t, h, err)
    print("worst sampled output error", worst, flush=True)
    st.close()
