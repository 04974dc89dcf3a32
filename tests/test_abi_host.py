"""Host-only checks of the C-ABI library: it loads, exports every symbol include/mk.h declares, and its
scheduler builds valid plans for every workload shape (no GPU calls)."""
import ctypes
import os
import re

import pytest

import persistent_megakernel_decode_amd as mkd
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^\s*(?:mk_status|const char\*|void)\s+(mk_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = mkd.lib()
    declared = _declared_functions()
    assert set(declared) == set(mkd.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_struct_sizes_match_header_layout():
    # mk_model_desc is 92 bytes of fields padded to 96; the library itself rejects any struct_size
    # other than its own sizeof (see test_host_rejects_out_of_contract_descriptions / mk_plan calls)
    assert ctypes.sizeof(mkd.mk_model_desc) == 96
    assert ctypes.sizeof(mkd.mk_layer_weights) == 15 * 8
    assert ctypes.sizeof(mkd.mk_kv_cache) == 48


def _desc(cfg, max_ctx):
    s = synth.shape_of(cfg, max_ctx)
    return mkd.make_desc(s["n_layers"], s["hidden"], s["vocab"], s["ffn"], s["n_q_heads"], s["n_kv_heads"],
                         s["head_dim"], s["qk_norm"], s["tied"], s["rms_eps"], s["rope_base"], s["layer_kinds"],
                         s["max_batch"], s["max_ctx"], s["n_delta_heads"], s["delta_dk"], s["delta_dv"],
                         s["conv_width"])


@pytest.mark.parametrize("name", ["tiny", "0.6b", "8b", "13b", "hybrid"])
def test_plan_is_valid_and_balanced(name):
    cfg = synth.CONFIGS[name]
    info = mkd.mk_plan(_desc(cfg, 4096 + 256), 256)
    assert info.errors == 0, mkd.mk_last_error()
    assert info.n_stages >= 3 * cfg.n_layers
    if name != "tiny":  # every unit streams the same weight bytes to within a row group per stage
        assert info.max_cu_bytes <= 1.03 * info.mean_cu_bytes


def test_plan_for_other_unit_counts():
    for n in (1, 7, 80, 304):
        info = mkd.mk_plan(_desc(synth.CONFIGS["tiny"], 512), n)
        assert info.errors == 0, mkd.mk_last_error()


def test_host_rejects_out_of_contract_descriptions():
    cfg = synth.CONFIGS["tiny"]
    bad = [dict(head_dim=96), dict(max_batch=0), dict(max_batch=9), dict(hidden=252), dict(n_kv_heads=3)]
    for kw in bad:
        c = cfg.replace(**{k: v for k, v in kw.items() if k != "max_batch"})
        d = _desc(c, 512)
        if "max_batch" in kw:
            d.max_batch = kw["max_batch"]
        with pytest.raises(mkd.MKError):
            mkd.mk_plan(d, 256)
    d = _desc(cfg, 512)
    d.abi_version = 99
    with pytest.raises(mkd.MKError) as e:
        mkd.mk_plan(d, 256)
    assert e.value.status == mkd.MK_ERR_INVALID_ARG


def test_trace_calls_reject_null_arguments():
    """The trace entry points answer a null context or buffer with MK_ERR_INVALID_ARG before any
    GPU call."""
    L = mkd.lib()
    n = ctypes.c_size_t(0)
    assert L.mk_trace_words(None, ctypes.byref(n)) == mkd.MK_ERR_INVALID_ARG
    assert L.mk_trace_words(None, None) == mkd.MK_ERR_INVALID_ARG
    buf = (ctypes.c_uint32 * 8)()
    assert L.mk_copy_trace(None, buf, 8) == mkd.MK_ERR_INVALID_ARG
