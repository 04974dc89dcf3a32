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
    # mk_model_desc is 104 bytes (weight_format at 92, n_experts and top_k last); the library itself
    # rejects any struct_size other than its own sizeof (see test_host_rejects_out_of_contract_descriptions)
    assert ctypes.sizeof(mkd.mk_model_desc) == 104
    assert mkd.mk_model_desc.weight_format.offset == 92 and mkd.mk_model_desc.top_k.offset == 100
    assert ctypes.sizeof(mkd.mk_layer_weights) == (15 + 10 + 1) * 8  # 15 tensors, 10 scale pointers, the router
    assert ctypes.sizeof(mkd.mk_kv_cache) == 48


def _desc(cfg, max_ctx):
    s = synth.shape_of(cfg, max_ctx)
    return mkd.make_desc(s["n_layers"], s["hidden"], s["vocab"], s["ffn"], s["n_q_heads"], s["n_kv_heads"],
                         s["head_dim"], s["qk_norm"], s["tied"], s["rms_eps"], s["rope_base"], s["layer_kinds"],
                         s["max_batch"], s["max_ctx"], s["n_delta_heads"], s["delta_dk"], s["delta_dv"],
                         s["conv_width"], weight_format={"fp8": mkd.MK_WEIGHTS_FP8_E4M3,
                                                         "fp4": mkd.MK_WEIGHTS_FP4_MX}.get(cfg.weights, 0),
                         n_experts=cfg.n_experts, top_k=cfg.top_k)


def _proj_bytes(cfg, per_weight, per_row):
    """The model's projection bytes (attention models), per_weight bytes a weight plus per_row a row."""
    H, F, d = cfg.hidden, cfg.ffn, cfg.head_dim
    mats = [(cfg.n_q_heads * d, H), (cfg.n_kv_heads * d, H), (cfg.n_kv_heads * d, H), (H, cfg.n_q_heads * d),
            (F, H), (F, H), (H, F)]
    return cfg.n_layers * sum(r * (c * per_weight + per_row) for r, c in mats)


@pytest.mark.parametrize("name", ["tiny", "0.6b", "8b", "13b"])
def test_fp8_plan_streams_one_byte_per_weight(name):
    """fp8 projections: the plan checks, and streams one byte per weight plus a 4-byte scale per row
    (the LM head stays bf16), against 2 bytes per weight for the bf16 model."""
    cfg = synth.CONFIGS[name]
    lm = cfg.vocab * cfg.hidden * 2
    for c, per_weight, per_row in ((cfg, 2, 0), (cfg.replace(weights="fp8"), 1, 4)):
        info = mkd.mk_plan(_desc(c, 4096 + 256), 256)
        assert info.errors == 0, mkd.mk_last_error()
        assert info.weight_bytes == lm + _proj_bytes(c, per_weight, per_row)
        if name != "tiny":
            assert info.max_cu_bytes <= 1.03 * info.mean_cu_bytes


def test_fp8_out_of_contract_descriptions():
    """fp8 weights: an input length that is not a multiple of 16 (of 512 at batch width 8) is
    MK_ERR_UNSUPPORTED; an unknown weight format is MK_ERR_INVALID_ARG; every batch width plans."""
    cfg = synth.CONFIGS["tiny"].replace(weights="fp8")
    for b in (2, 3, 4):
        assert mkd.mk_plan(_desc(cfg.replace(batch=b, ctx=[128] * b), 512), 256).errors == 0
    for c in (cfg.replace(hidden=264), cfg.replace(batch=8, ctx=[128] * 8)):  # (hidden 256: not a multiple of 512)
        with pytest.raises(mkd.MKError) as e:
            mkd.mk_plan(_desc(c, 512), 256)
        assert e.value.status == mkd.MK_ERR_UNSUPPORTED
    d = _desc(cfg, 512)
    d.weight_format = 7
    with pytest.raises(mkd.MKError) as e:
        mkd.mk_plan(d, 256)
    assert e.value.status == mkd.MK_ERR_INVALID_ARG


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


def test_library_imports_no_device_allocator():
    """The library never allocates device memory itself (every buffer is the caller's, or the static
    scratch of mk_create_static): its dynamic imports hold no hipMalloc / hipFree family call."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not available")
    out = subprocess.run([nm, "-D", "--undefined-only", mkd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    imported = {l.split()[-1].split("@")[0] for l in out.splitlines() if l.strip()}
    assert "hipGetSymbolAddress" in imported
    assert not {s for s in imported if s.startswith("hip") and ("Malloc" in s or "Free" in s or "Alloc" in s)}


@pytest.mark.parametrize("name", ["tiny", "0.6b", "8b"])
def test_fp4_plan_streams_half_a_byte_per_weight(name):
    """MX fp4 projections (one sequence): the plan checks, and streams half a byte per weight plus one
    E8M0 scale byte per 32 weights (the LM head stays bf16)."""
    cfg = synth.CONFIGS[name].replace(weights="fp4")
    lm = cfg.vocab * cfg.hidden * 2
    info = mkd.mk_plan(_desc(cfg, 4096 + 256), 256)
    assert info.weight_bytes == lm + _proj_bytes(cfg, 0.5 + 1 / 32, 0)


def test_fp4_refuses_more_than_one_sequence_and_partial_blocks():
    cfg = synth.CONFIGS["tiny"].replace(weights="fp4")
    with pytest.raises(mkd.MKError) as e:
        mkd.mk_plan(_desc(cfg.replace(batch=2, ctx=[128, 128]), 512), 256)
    assert e.value.status == mkd.MK_ERR_UNSUPPORTED and "max_batch" in str(e.value)
    with pytest.raises(mkd.MKError) as e:  # hidden 272: rows of 272 weights are not whole blocks of 32
        mkd.mk_plan(_desc(cfg.replace(hidden=272), 512), 256)
    assert e.value.status == mkd.MK_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,batch", [("tiny-moe", 1), ("tiny-moe", 4), ("moe", 1)])
def test_moe_plan_checks_and_streams_every_expert_once(name, batch):
    """Mixture-of-experts layers: a router stage and one gate / up and one down op per compute unit
    that cover a row tile of every expert; the plan checks and accounts every expert's bytes once."""
    cfg = (synth.SMALL.get(name) or synth.CONFIGS[name]).replace(batch=batch)
    info = mkd.mk_plan(_desc(cfg, 4096 + 256), 256)
    assert info.errors == 0, mkd.mk_last_error()  # (includes: every workspace address relocatable)
    H, F, d, E = cfg.hidden, cfg.ffn, cfg.head_dim, cfg.n_experts
    per_layer = (E * H + E * 3 * F * H + (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d * H + H * cfg.n_q_heads * d) * 2
    assert info.weight_bytes == cfg.vocab * H * 2 + cfg.n_layers * per_layer
    assert info.max_cu_bytes <= 1.05 * info.weight_bytes / 256 + 2 * E * 3 * F * 2 * 4


def test_moe_refuses_unsupported_shapes():
    cfg = synth.SMALL["tiny-moe"]
    for bad in (cfg.replace(batch=8, ctx=[128] * 8), cfg.replace(top_k=9, n_experts=12), cfg.replace(n_experts=6),
                cfg.replace(n_experts=68, top_k=2)):
        with pytest.raises(mkd.MKError) as e:
            mkd.mk_plan(_desc(bad, 512), 256)
        assert e.value.status == mkd.MK_ERR_UNSUPPORTED
