"""The C ABI library loads and exports what include/statekv.h declares; host-side
argument checks reject bad calls before touching the device.  No compute."""
import ctypes
import math
import os

import pytest

import kv_cache_compression_statekv_amd as skv


def test_every_declared_function_is_exported():
    lib = skv.load_library()
    names = skv.declared_functions()
    assert {"statekv_create", "statekv_prefill_frame", "statekv_decode",
            "statekv_compressed_view", "statekv_detailed_view", "statekv_destroy"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_error_strings():
    for code in range(0, -8, -1):
        assert skv.error_string(code) and skv.error_string(code) != "unknown error"
    assert skv.error_string(-99) == "unknown error"


def _cfg(**kw):
    base = dict(n_q_heads=4, n_kv_heads=2, head_dim=64, tokens_per_frame=16, max_frames=4,
                dtype=skv.DTYPE_BF16, rope_base=1e6, rope_orig_ctx=32768, max_text=0)
    base.update(kw)
    return skv.LayerCfg(**base)


@pytest.mark.parametrize("bad", [
    dict(n_q_heads=0), dict(n_kv_heads=0), dict(n_q_heads=6, n_kv_heads=4),
    dict(head_dim=96), dict(head_dim=32), dict(tokens_per_frame=0), dict(max_frames=0),
    dict(dtype=7), dict(rope_base=1.0), dict(rope_base=math.inf), dict(rope_orig_ctx=0),
    dict(max_text=-1),
    # frame tokens fit 32-bit positions, frames plus text do not
    dict(tokens_per_frame=1 << 16, max_frames=(1 << 15) - 1, max_text=1 << 16),
])
def test_create_rejects_bad_config(bad):
    lib = skv.load_library()
    h = ctypes.c_void_p()
    cfg = _cfg(**bad)
    assert lib.statekv_create(ctypes.byref(cfg), 64, 1.0, ctypes.byref(h)) == skv.STATEKV_EINVAL
    assert not h.value


@pytest.mark.parametrize("budget,alpha,frames", [(0, 1.0, 4), (-5, 1.0, 4), (64, 0.5, 4),
                                                 (64, math.nan, 4), (64, math.inf, 4),
                                                 # evicting stream whose pool exceeds 32768
                                                 (32768, 1.0, 4096)])
def test_create_rejects_bad_budget_or_alpha(budget, alpha, frames):
    lib = skv.load_library()
    h = ctypes.c_void_p()
    cfg = _cfg(max_frames=frames)
    assert lib.statekv_create(ctypes.byref(cfg), budget, alpha, ctypes.byref(h)) == skv.STATEKV_EINVAL


def test_create_accepts_full_attention_budget_beyond_pool_limit():
    """A budget that holds every token never selects, so the 32768-candidate
    limit of the selection does not apply (here: no GPU, so creation stops at
    the device, after validation)."""
    lib = skv.load_library()
    h = ctypes.c_void_p()
    cfg = _cfg(max_frames=4096)      # 65536 tokens
    rc = lib.statekv_create(ctypes.byref(cfg), 65536, 1.0, ctypes.byref(h))
    assert rc != skv.STATEKV_EINVAL
    if rc == skv.STATEKV_OK:
        lib.statekv_destroy(h)


@pytest.mark.parametrize("name,mirror", [("statekv_layer_cfg", "LayerCfg"),
                                         ("statekv_view", "View"),
                                         ("statekv_scores_view", "ScoresView")])
def test_struct_mirrors_match_the_header(name, mirror):
    """The ctypes mirrors of the ABI structs have the header's fields, in order."""
    import re
    text = open(skv.HEADER).read()
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(\w+)\s*;", body)
    assert fields == [f[0] for f in getattr(skv, mirror)._fields_]


@pytest.mark.parametrize("layers", [-1, 257])
def test_create_rejects_bad_layer_counts(layers):
    lib = skv.load_library()
    h = ctypes.c_void_p()
    cfg = _cfg(n_layers=layers)
    assert lib.statekv_create(ctypes.byref(cfg), 64, 1.0, ctypes.byref(h)) == skv.STATEKV_EINVAL


def test_null_arguments_are_rejected():
    lib = skv.load_library()
    h = ctypes.c_void_p()
    assert lib.statekv_create(None, 64, 1.0, ctypes.byref(h)) == skv.STATEKV_EINVAL
    cfg = _cfg()
    assert lib.statekv_create(ctypes.byref(cfg), 64, 1.0, None) == skv.STATEKV_EINVAL
    assert lib.statekv_prefill_frame(None, None, None, None, 0, None) == skv.STATEKV_EINVAL
    assert lib.statekv_prefill_frame_static(None, None, None, None, 0, None) == skv.STATEKV_EINVAL
    assert lib.statekv_decode(None, None, None, None, 1, None) == skv.STATEKV_EINVAL
    v = skv.View()
    assert lib.statekv_compressed_view(None, ctypes.byref(v)) == skv.STATEKV_EINVAL
    assert lib.statekv_detailed_view(None, ctypes.byref(v)) == skv.STATEKV_EINVAL
    sv = skv.ScoresView()
    assert lib.statekv_scores(None, ctypes.byref(sv)) == skv.STATEKV_EINVAL
    assert lib.statekv_set_flags(None, 0) == skv.STATEKV_EINVAL
    assert lib.statekv_set_stream(None, None) == skv.STATEKV_EINVAL
    assert lib.statekv_kernel_times(None, None, None, 0, 0) == skv.STATEKV_EINVAL
    lib.statekv_destroy(None)


def test_product_path_never_reaches_the_oracle():
    # No module of the package imports the CPU oracle, and a missing library
    # is an error rather than a silent fallback.
    import ast
    import glob
    import kv_cache_compression_statekv_amd as skv
    pkg = os.path.dirname(skv.__file__)
    for path in glob.glob(os.path.join(pkg, "*.py")):
        tree = ast.parse(open(path).read())
        for node in ast.walk(tree):
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            assert not any(n.split(".")[0] == "oracle" for n in names), (path, names)


def test_missing_library_is_an_error(monkeypatch, tmp_path):
    import kv_cache_compression_statekv_amd as skv
    monkeypatch.setattr(skv, "_lib", None)
    monkeypatch.setattr(skv, "library_path", lambda: str(tmp_path / "libstatekv.so"))
    with pytest.raises(RuntimeError, match="not built"):
        skv.load_library(build_if_missing=False)
