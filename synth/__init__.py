"""Seeded synthetic inputs for the decode step: model shapes, weights, caches.

This module only draws numbers and lays them out; it holds none of the
decode arithmetic.  Both the oracle harness and the GPU path consume what it
produces, so neither side generates its own inputs.

The five model shapes follow the workloads the persistent-decode-megakernel
pages evaluate (ForgeMegakernel abstract: decode of 0.6B-13B models; the
MK-KDA pull request for the gated delta-rule layer), with the sizes fixed in
the workload table this project measures.
"""
from __future__ import annotations

import ctypes
import dataclasses
import hashlib
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

ATTN, DELTA = 0, 1


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, u64, dbl = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_double
        L.synth_normal_bf16.argtypes = [vp, sz, u64, u64, dbl, dbl]
        L.synth_normal_f32.argtypes = [vp, sz, u64, u64, dbl, dbl]
        L.synth_uniform_bf16.argtypes = [vp, sz, u64, u64, dbl, dbl]
        L.synth_u32.argtypes = [vp, sz, u64, u64]
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_fp8_codes.argtypes = [vp, sz, u64, u64]
        for f in (L.synth_normal_bf16, L.synth_normal_f32, L.synth_uniform_bf16, L.synth_u32, L.synth_philox4x32_10,
                  L.synth_fp8_codes):
            f.restype = None
        _lib = L
    return _lib


def stream_id(name: str) -> int:
    """64-bit stream id of a tensor name (first 8 bytes of its SHA-256)."""
    return int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")


def normal_bf16(shape, seed: int, name: str, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(out.ctypes.data, out.size, seed, stream_id(name), mean, std)
    return out


def normal_f32(shape, seed: int, name: str, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(out.ctypes.data, out.size, seed, stream_id(name), mean, std)
    return out


def uniform_bf16(shape, seed: int, name: str, lo: float, hi: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_uniform_bf16(out.ctypes.data, out.size, seed, stream_id(name), lo, hi)
    return out


def u32(n: int, seed: int, name: str) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().synth_u32(out.ctypes.data, n, seed, stream_id(name))
    return out


def fp8_codes(shape, seed: int, name: str) -> np.ndarray:
    """Random E4M3 fp8 weight codes (uint8; no NaN codes), see synth_fp8_codes in gen.c."""
    out = np.empty(shape, dtype=np.uint8)
    lib().synth_fp8_codes(out.ctypes.data, out.size, seed, stream_id(name))
    return out


def philox(ctr, key) -> List[int]:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return [int(v) for v in o]


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Model shapes
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Config:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 1e4
    qk_norm: int = 0
    tied: int = 0
    layer_kinds: Optional[List[int]] = None  # None = all attention
    n_delta_heads: int = 0
    delta_dk: int = 0
    delta_dv: int = 0
    conv_width: int = 0
    # run
    batch: int = 1
    ctx: Optional[List[int]] = None          # context already cached per sequence
    ctx_range: Optional[tuple] = None        # (lo, hi) inclusive, drawn per sequence
    steps: int = 8
    seed: int = 0
    page_size: int = 16
    shuffle_pages: bool = False
    gain_range: Optional[tuple] = None       # None = unit norm gains
    weights: str = "bf16"                    # projections: "bf16", "fp8" (+ fp32 row scales), "fp4" (+ E8M0 block scales)
    n_experts: int = 0                       # > 0: every MLP is top_k of n_experts experts of width ffn
    top_k: int = 0

    def kinds(self) -> List[int]:
        return list(self.layer_kinds) if self.layer_kinds is not None else [ATTN] * self.n_layers

    @property
    def n_attn_layers(self) -> int:
        return sum(1 for k in self.kinds() if k == ATTN)

    @property
    def n_delta_layers(self) -> int:
        return sum(1 for k in self.kinds() if k == DELTA)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def hybrid_kinds(n_layers: int) -> List[int]:
    """Every 4th layer (l with (l+1) % 4 == 0) is full attention, the rest delta-rule."""
    return [ATTN if (l + 1) % 4 == 0 else DELTA for l in range(n_layers)]


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768,
                   vocab=1024, rope_base=1e4, batch=1, ctx=[128], steps=8, seed=0),
    "0.6b": Config("0.6b", n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=3072,
                   vocab=151936, qk_norm=1, tied=1, rope_base=1e4, batch=1, ctx=[1024], steps=64, seed=1),
    "8b": Config("8b", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                 vocab=128256, rope_base=5e5, batch=1, ctx=[4096], steps=128, seed=2),
    "13b": Config("13b", n_layers=40, hidden=5120, n_q_heads=40, n_kv_heads=40, head_dim=128, ffn=13824,
                  vocab=32000, rope_base=1e4, batch=8, ctx_range=(512, 4096), steps=64, seed=3,
                  shuffle_pages=True),
    "hybrid": Config("hybrid", n_layers=24, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=6144,
                     vocab=65536, rope_base=1e4, layer_kinds=hybrid_kinds(24), n_delta_heads=16,
                     delta_dk=128, delta_dv=128, conv_width=4, batch=4, ctx=[2048] * 4, steps=64, seed=4),
}


# the 8B shape with every projection in fp8 (E4M3 codes, fp32 row scales); LM head, embedding and
# KV cache bf16
CONFIGS["8b-fp8"] = CONFIGS["8b"].replace(name="8b-fp8", weights="fp8")
CONFIGS["13b-fp8"] = CONFIGS["13b"].replace(name="13b-fp8", weights="fp8")
# a mixture-of-experts decoder: 16 layers, hidden 2048, GQA 16/4, every MLP 8 of 64 experts of
# width 1024 (the layer shape of the small open MoE models), batch 1, ctx 4096
CONFIGS["moe"] = Config("moe", n_layers=16, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=1024,
                        vocab=50304, rope_base=1e4, batch=1, ctx=[4096], steps=64, seed=5, n_experts=64, top_k=8)
# the 8B shape with MX fp4 projections (E2M1, E8M0 scales per 32 weights)
CONFIGS["8b-fp4"] = CONFIGS["8b"].replace(name="8b-fp4", weights="fp4")


def context_lengths(cfg: Config) -> List[int]:
    """Cached tokens per sequence before the first decode step."""
    if cfg.ctx is not None:
        assert len(cfg.ctx) == cfg.batch
        return list(cfg.ctx)
    lo, hi = cfg.ctx_range
    draws = u32(cfg.batch, cfg.seed, "ctx_lens")
    return [int(lo + (int(d) % (hi - lo + 1))) for d in draws]


def first_tokens(cfg: Config) -> np.ndarray:
    return (u32(cfg.batch, cfg.seed, "first_tokens") % np.uint32(cfg.vocab)).astype(np.int32)


def permutation(n: int, seed: int, name: str) -> np.ndarray:
    """Seeded Fisher-Yates permutation of range(n)."""
    draws = u32(max(n, 1), seed, name)
    p = np.arange(n, dtype=np.int32)
    for i in range(n - 1, 0, -1):
        j = int(draws[i]) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


# --------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------
WEIGHT_STD = 0.02


def _gain(cfg: Config, n: int, name: str) -> np.ndarray:
    if cfg.gain_range is None:
        return np.full(n, 0x3F80, dtype=np.uint16)  # bf16 1.0
    lo, hi = cfg.gain_range
    return uniform_bf16(n, cfg.seed, name, lo, hi)


# fp8 projections: the drawn codes' values have an RMS of about 142 (the exponent spread of
# synth_fp8_codes), so row scales of FP8_SCALE * U[0.5, 1.5) give weights of about WEIGHT_STD.
FP8_SCALE = WEIGHT_STD / 142.0


# fp4 projections: uniform random E2M1 nibbles (RMS of their values 2.93) with E8M0 block scales 2^-8
# or 2^-7 drawn per block of 32 weights (RMS 0.0062), so the weights have an RMS of 0.018, about the
# bf16 models' WEIGHT_STD.
FP4_SCALE_E = (119, 120)


def _proj(cfg: Config, L: dict, name: str, rows: int, cols: int, prefix: str) -> None:
    """One projection matrix: bf16 N(0, WEIGHT_STD); fp8 codes with one fp32 scale per row; or fp4
    E2M1 codes packed two per byte (low nibble first) with one E8M0 scale byte per 32 weights."""
    if cfg.weights == "fp4":
        if cols % 32:
            raise ValueError(f"{name}: fp4 rows of {cols} weights are not whole blocks of 32")
        L[name] = u32(rows * cols // 8, cfg.seed, prefix + name).view(np.uint8).reshape(rows, cols // 2)
        e = u32(rows * cols // 32, cfg.seed, prefix + name + "_scale") % len(FP4_SCALE_E)
        L[name + "_scale"] = (np.uint8(FP4_SCALE_E[0]) + e.astype(np.uint8)).reshape(rows, cols // 32)
    elif cfg.weights == "fp8":
        L[name] = fp8_codes((rows, cols), cfg.seed, prefix + name)
        u = u32(rows, cfg.seed, prefix + name + "_scale").astype(np.float64) / 4294967296.0
        L[name + "_scale"] = (FP8_SCALE * (0.5 + u)).astype(np.float32)
    else:
        L[name] = normal_bf16((rows, cols), cfg.seed, prefix + name, WEIGHT_STD)


def make_weights(cfg: Config) -> dict:
    """Host (numpy) weights in PyTorch Linear layout [out, in]: bf16 bit patterns, except that with
    cfg.weights == "fp8" every projection matrix is E4M3 codes (uint8) with fp32 row scales
    ("<name>_scale"); embedding, LM head, norm gains and conv taps stay bf16."""
    if cfg.weights not in ("bf16", "fp8", "fp4"):
        raise ValueError(f"weight format {cfg.weights!r}")
    s, H, d = cfg.seed, cfg.hidden, cfg.head_dim
    w = {"embed": normal_bf16((cfg.vocab, H), s, "embed", WEIGHT_STD),
         "final_norm": _gain(cfg, H, "final_norm"), "format": cfg.weights}
    w["lm_head"] = w["embed"] if cfg.tied else normal_bf16((cfg.vocab, H), s, "lm_head", WEIGHT_STD)
    layers = []
    for l, kind in enumerate(cfg.kinds()):
        p = f"layer{l}."
        L = {"attn_norm": _gain(cfg, H, p + "attn_norm"), "mlp_norm": _gain(cfg, H, p + "mlp_norm")}
        if cfg.n_experts:  # router and expert-major expert weights (bf16)
            if cfg.weights != "bf16":
                raise ValueError("mixture-of-experts models take bf16 weights")
            E, F = cfg.n_experts, cfg.ffn
            L["w_router"] = normal_bf16((E, H), s, p + "w_router", WEIGHT_STD)
            L["w_gate"] = normal_bf16((E, F, H), s, p + "w_gate", WEIGHT_STD)
            L["w_up"] = normal_bf16((E, F, H), s, p + "w_up", WEIGHT_STD)
            L["w_down"] = normal_bf16((E, H, F), s, p + "w_down", WEIGHT_STD)
        else:
            _proj(cfg, L, "w_gate", cfg.ffn, H, p)
            _proj(cfg, L, "w_up", cfg.ffn, H, p)
            _proj(cfg, L, "w_down", H, cfg.ffn, p)
        if kind == ATTN:
            _proj(cfg, L, "wq", cfg.n_q_heads * d, H, p)
            _proj(cfg, L, "wk", cfg.n_kv_heads * d, H, p)
            _proj(cfg, L, "wv", cfg.n_kv_heads * d, H, p)
            _proj(cfg, L, "wo", H, cfg.n_q_heads * d, p)
            if cfg.qk_norm:
                L["q_norm"] = _gain(cfg, d, p + "q_norm")
                L["k_norm"] = _gain(cfg, d, p + "k_norm")
        else:
            nh, dk, dv = cfg.n_delta_heads, cfg.delta_dk, cfg.delta_dv
            C = nh * (2 * dk + dv)
            _proj(cfg, L, "w_qkv_delta", C, H, p)
            _proj(cfg, L, "w_gates", 2 * nh, H, p)
            L["conv_w"] = normal_bf16((C, cfg.conv_width), s, p + "conv_w", WEIGHT_STD)
            _proj(cfg, L, "wo_delta", H, nh * dv, p)
        layers.append(L)
    w["layers"] = layers
    return w


# --------------------------------------------------------------------------
# KV cache, page table and recurrent states
# --------------------------------------------------------------------------
def make_cache(cfg: Config, ctx_lens: List[int], extra_tokens: int, prompt_mode: bool = False) -> dict:
    """Paged bf16 KV cache holding random K/V for positions < ctx_lens[b] (random-cache mode).

    Pages are page_size positions; each sequence owns ceil((ctx+extra)/page_size) pages, taken from
    a seeded permutation of page ids when cfg.shuffle_pages, else in order.  With prompt_mode the
    cache starts empty (zeros) and the recurrent states start at zero.
    """
    B, ps = cfg.batch, cfg.page_size
    need = [-(-(c + extra_tokens) // ps) for c in ctx_lens]
    max_pages_per_seq = max(need)
    num_pages = sum(need)
    ids = permutation(num_pages, cfg.seed, "page_perm") if cfg.shuffle_pages else np.arange(num_pages, dtype=np.int32)
    table = np.full((B, max_pages_per_seq), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :need[b]] = ids[o:o + need[b]]
        o += need[b]
    nA, Hkv, d = cfg.n_attn_layers, cfg.n_kv_heads, cfg.head_dim
    shape = (nA, num_pages, Hkv, ps, d)
    k_pages = np.zeros(shape, dtype=np.uint16)
    v_pages = np.zeros(shape, dtype=np.uint16)
    if not prompt_mode:
        for a in range(nA):
            for b in range(B):
                n = ctx_lens[b]
                if n == 0:
                    continue
                kk = normal_bf16((n, Hkv, d), cfg.seed, f"k_cache.{a}.{b}")
                vv = normal_bf16((n, Hkv, d), cfg.seed, f"v_cache.{a}.{b}")
                for pg in range(-(-n // ps)):
                    lo, hi = pg * ps, min(n, pg * ps + ps)
                    phys = table[b, pg]
                    k_pages[a, phys, :, :hi - lo, :] = kk[lo:hi].transpose(1, 0, 2)
                    v_pages[a, phys, :, :hi - lo, :] = vv[lo:hi].transpose(1, 0, 2)
    cache = {"k_pages": k_pages, "v_pages": v_pages, "page_table": table, "num_pages": num_pages,
             "max_pages_per_seq": max_pages_per_seq}
    nD = cfg.n_delta_layers
    if nD:
        nh, dk, dv, W = cfg.n_delta_heads, cfg.delta_dk, cfg.delta_dv, cfg.conv_width
        C = nh * (2 * dk + dv)
        if prompt_mode:
            cache["delta_state"] = np.zeros((nD, B, nh, dv, dk), dtype=np.float32)
            cache["conv_state"] = np.zeros((nD, B, C, W - 1), dtype=np.float32)
        else:
            cache["delta_state"] = normal_f32((nD, B, nh, dv, dk), cfg.seed, "delta_state")
            cache["conv_state"] = normal_f32((nD, B, C, W - 1), cfg.seed, "conv_state")
    return cache


# Small shapes for the oracle's own pins and for GPU parity at tile-spanning sizes.
SMALL: Dict[str, Config] = {
    # dense GQA, unit-test gains drawn U(0.5, 1.5) so a dropped gain cannot pass
    "tiny-gain": CONFIGS["tiny"].replace(name="tiny-gain", gain_range=(0.5, 1.5)),
    # per-head q/k norm and tied embeddings (the 0.6B family) at toy size
    "tiny-qknorm": CONFIGS["tiny"].replace(name="tiny-qknorm", qk_norm=1, tied=1, gain_range=(0.5, 1.5)),
    # hybrid: layers 0-2 delta rule, layer 3 full attention
    "tiny-hybrid": Config("tiny-hybrid", n_layers=4, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                          vocab=512, layer_kinds=hybrid_kinds(4), n_delta_heads=2, delta_dk=32, delta_dv=32,
                          conv_width=4, batch=2, ctx=[16, 16], steps=4, seed=5, gain_range=(0.5, 1.5)),
    # mixture of experts: 8 experts of width 256, top 2
    "tiny-moe": CONFIGS["tiny"].replace(name="tiny-moe", ffn=256, n_experts=8, top_k=2, gain_range=(0.5, 1.5),
                                        seed=6),
}


def shape_of(cfg: Config, max_ctx: int) -> dict:
    """Model-description fields for the megakernel's C ABI (include/mk.h, mk_model_desc)."""
    return dict(n_layers=cfg.n_layers, hidden=cfg.hidden, vocab=cfg.vocab, ffn=cfg.ffn, n_q_heads=cfg.n_q_heads,
                n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, qk_norm=cfg.qk_norm, tied=cfg.tied,
                rms_eps=cfg.rms_eps, rope_base=cfg.rope_base, layer_kinds=cfg.kinds(), max_batch=cfg.batch,
                max_ctx=max_ctx, n_delta_heads=cfg.n_delta_heads, delta_dk=cfg.delta_dk, delta_dv=cfg.delta_dv,
                conv_width=cfg.conv_width, page_size=cfg.page_size, weights=cfg.weights, n_experts=cfg.n_experts,
                top_k=cfg.top_k)
