"""Decode-step oracle -- TEST INFRASTRUCTURE ONLY.

ctypes binding of liboracle.so (oracle.c): a plain, slow CPU decode step
with fp64 accumulation, written from the definition of the decode step and
sharing no code with the GPU path.  Only tests/, the smoke check and the
bench's CPU-baseline leg may import this package.

ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract): an
independent mid-state test oracle derives the intermediate states of the
megakernel and checks error and precision; ``DecodeOracle.step`` returns
those mid-states on request.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    hdr = os.path.join(_HERE, "oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class OrcModel(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("vocab", ctypes.c_int), ("ffn", ctypes.c_int),
                ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("qk_norm", ctypes.c_int), ("tied_embeddings", ctypes.c_int),
                ("rms_eps", ctypes.c_double), ("rope_base", ctypes.c_double),
                ("n_delta_heads", ctypes.c_int), ("delta_dk", ctypes.c_int), ("delta_dv", ctypes.c_int),
                ("conv_width", ctypes.c_int), ("layer_kind", P), ("page_size", ctypes.c_int),
                ("delta_decay_first", ctypes.c_int), ("weight_format", ctypes.c_int),
                ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int)]


W_BF16, W_FP8, W_FP4 = 0, 1, 2  # orc_model.weight_format


_LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "w_qkv_delta", "w_gates", "conv_w",
                 "wo_delta", "mlp_norm", "w_gate", "w_up", "w_down"]


# projections that are fp8 codes with fp32 row scales ("<name>_scale") when the weights are fp8, or
# packed E2M1 codes with E8M0 block scales ("<name>_scale", uint8 [rows][cols / 32]) when fp4
PROJ_FIELDS = ["wq", "wk", "wv", "wo", "w_qkv_delta", "w_gates", "wo_delta", "w_gate", "w_up", "w_down"]


class OrcLayer(ctypes.Structure):
    _fields_ = [(f, P) for f in _LAYER_FIELDS] + [("s_" + f, P) for f in PROJ_FIELDS] + [("w_router", P)]


class OrcWeights(ctypes.Structure):
    _fields_ = [("embed", P), ("final_norm", P), ("lm_head", P), ("layers", P)]


class OrcCache(ctypes.Structure):
    _fields_ = [("k_pages", P), ("v_pages", P), ("num_pages", ctypes.c_int), ("max_pages_per_seq", ctypes.c_int),
                ("page_table", P), ("delta_state", P), ("conv_state", P), ("max_batch", ctypes.c_int)]


class OrcDump(ctypes.Structure):
    _fields_ = [("x_mixer", P), ("x_mlp", P), ("mixer_o", P), ("mlp_m", P), ("final_r", P), ("router", P),
                ("sel", P), ("force", P)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_rmsnorm.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P]
        L.orc_matvec.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
        L.orc_matvec_fp8.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P]
        L.orc_matvec_fp8.restype = None
        L.orc_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_e4m3.restype = ctypes.c_double
        L.orc_e2m1.argtypes = [ctypes.c_uint8]
        L.orc_e2m1.restype = ctypes.c_double
        L.orc_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_e8m0.restype = ctypes.c_double
        L.orc_matvec_fp4.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P]
        L.orc_matvec_fp4.restype = None
        L.orc_moe_select.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        L.orc_moe_select.restype = None
        L.orc_moe_weights.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.orc_moe_weights.restype = None
        L.orc_rope.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.orc_attend.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P, P]
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_sigmoid.argtypes = [ctypes.c_double]
        L.orc_sigmoid.restype = ctypes.c_double
        L.orc_conv_step.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P]
        L.orc_delta_step.argtypes = [P, P, P, P, ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, P]
        L.orc_delta_mixer.argtypes = [P, P, P, P, P, P, P]
        L.orc_delta_mixer.restype = None
        L.orc_decode_step.argtypes = [P, P, P, P, P, P, ctypes.c_int, P, P]
        L.orc_decode_step.restype = ctypes.c_int
        L.orc_argmax.argtypes = [P, ctypes.c_int]
        L.orc_argmax.restype = ctypes.c_int
        for f in (L.orc_rmsnorm, L.orc_matvec, L.orc_rope, L.orc_attend, L.orc_conv_step, L.orc_delta_step):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- blocks
def rmsnorm(x, gain_bf16=None, eps=1e-6) -> np.ndarray:
    x = _c(x, np.float32)
    g = None if gain_bf16 is None else _c(gain_bf16, np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(y))
    return y


def matvec(W_bf16, x) -> np.ndarray:
    W = _c(W_bf16, np.uint16)
    x = _c(x, np.float32)
    y = np.empty(W.shape[0], dtype=np.float32)
    lib().orc_matvec(_ptr(W), _ptr(x), W.shape[0], W.shape[1], _ptr(y))
    return y


def e4m3(code: int) -> float:
    """The value of one OCP E4M3 fp8 code (NaN for 0x7F / 0xFF)."""
    return lib().orc_e4m3(int(code))


def matvec_fp8(W_codes, scale, x) -> np.ndarray:
    """y[r] = scale[r] * sum_k e4m3(W[r][k]) x[k]."""
    W = _c(W_codes, np.uint8)
    s = _c(scale, np.float32)
    x = _c(x, np.float32)
    y = np.empty(W.shape[0], dtype=np.float32)
    lib().orc_matvec_fp8(_ptr(W), _ptr(s), _ptr(x), W.shape[0], W.shape[1], _ptr(y))
    return y


def e2m1(code: int) -> float:
    """The value of one MX E2M1 code (low 4 bits)."""
    return lib().orc_e2m1(int(code))


def e8m0(e: int) -> float:
    """The value of one MX E8M0 scale byte (NaN for 0xFF)."""
    return lib().orc_e8m0(int(e))


def matvec_fp4(W_packed, S, x) -> np.ndarray:
    """y[r] = sum_k e8m0(S[r][k // 32]) e2m1(code(r, k)) x[k], codes packed two per byte, low nibble first."""
    W = _c(W_packed, np.uint8)
    S = _c(S, np.uint8)
    x = _c(x, np.float32)
    y = np.empty(W.shape[0], dtype=np.float32)
    lib().orc_matvec_fp4(_ptr(W), _ptr(S), _ptr(x), W.shape[0], x.size, _ptr(y))
    return y


def moe_select(logits, k: int) -> np.ndarray:
    """The k largest router logits' experts, descending, ties to the lower index."""
    v = _c(logits, np.float32)
    sel = np.empty(k, dtype=np.int32)
    lib().orc_moe_select(_ptr(v), v.size, k, _ptr(sel))
    return sel


def moe_weights(logits, sel) -> np.ndarray:
    """softmax over all router logits, renormalised over the chosen experts `sel`."""
    v = _c(logits, np.float32)
    sel = _c(sel, np.int32)
    w = np.empty(sel.size, dtype=np.float64)
    lib().orc_moe_weights(_ptr(v), v.size, sel.size, _ptr(sel), _ptr(w))
    return w


def rope(u, pos: int, base: float) -> np.ndarray:
    u = _c(u, np.float32).copy()
    lib().orc_rope(_ptr(u), u.size, pos, base)
    return u


def attend(q, K_bf16, V_bf16):
    """Single-head attention over rows of K, V ([n, d] bf16).  Returns (o, probs)."""
    q = _c(q, np.float32)
    K = _c(K_bf16, np.uint16)
    V = _c(V_bf16, np.uint16)
    n, d = K.shape
    kp = (ctypes.c_void_p * n)(*[K.ctypes.data + j * d * 2 for j in range(n)])
    vp = (ctypes.c_void_p * n)(*[V.ctypes.data + j * d * 2 for j in range(n)])
    o = np.empty(d, dtype=np.float32)
    pr = np.empty(n, dtype=np.float64)
    lib().orc_attend(_ptr(q), ctypes.cast(kp, P), ctypes.cast(vp, P), n, d, _ptr(o), _ptr(pr))
    return o, pr


def silu(z: float) -> float:
    return lib().orc_silu(z)


def sigmoid(z: float) -> float:
    return lib().orc_sigmoid(z)


def conv_step(u, conv_w_bf16, state):
    """Returns (y, new_state); state is [C][W-1] fp32 (not modified)."""
    u = _c(u, np.float32)
    w = _c(conv_w_bf16, np.uint16)
    st = _c(state, np.float32).copy()
    C, W = w.shape
    y = np.empty(C, dtype=np.float32)
    lib().orc_conv_step(_ptr(u), _ptr(w), _ptr(st), C, W, _ptr(y))
    return y, st


def delta_step(st, q, k, v, g, beta, decay_first=0):
    """st = S^T [dv][dk] fp32.  Returns (new st, o[dv])."""
    st = _c(st, np.float32).copy()
    dv, dk = st.shape
    o = np.empty(dv, dtype=np.float32)
    lib().orc_delta_step(_ptr(st), _ptr(_c(q, np.float32)), _ptr(_c(k, np.float32)), _ptr(_c(v, np.float32)),
                         float(g), float(beta), dk, dv, int(decay_first), _ptr(o))
    return st, o


def bf16(x) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest even), via the oracle's own routine."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().orc_f32_to_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def argmax(v) -> int:
    v = _c(v, np.float32)
    return lib().orc_argmax(_ptr(v), v.size)


# ---------------------------------------------------------------- model
class DecodeOracle:
    """Runs orc_decode_step over a model whose weights and cache are numpy arrays.

    The oracle owns private copies of the mutable cache state (KV pages, conv and delta states),
    so it evolves its own history next to the GPU's.
    """

    def __init__(self, cfg, weights: dict, cache: dict, decay_first: int = 0):
        self.cfg = cfg
        self.w = weights
        self.kinds = np.asarray(cfg.kinds(), dtype=np.int32)
        m = OrcModel()
        m.n_layers, m.hidden, m.vocab, m.ffn = cfg.n_layers, cfg.hidden, cfg.vocab, cfg.ffn
        m.n_q_heads, m.n_kv_heads, m.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        m.qk_norm, m.tied_embeddings = cfg.qk_norm, cfg.tied
        m.rms_eps, m.rope_base = cfg.rms_eps, cfg.rope_base
        m.n_delta_heads, m.delta_dk, m.delta_dv, m.conv_width = cfg.n_delta_heads, cfg.delta_dk, cfg.delta_dv, cfg.conv_width
        m.layer_kind = self.kinds.ctypes.data
        m.page_size = cfg.page_size
        m.delta_decay_first = decay_first
        fmt = weights.get("format", "bf16")
        fp8, fp4 = fmt == "fp8", fmt == "fp4"
        m.weight_format = W_FP8 if fp8 else (W_FP4 if fp4 else W_BF16)
        m.n_experts, m.top_k = getattr(cfg, "n_experts", 0), getattr(cfg, "top_k", 0)
        self.m = m
        self.layers = (OrcLayer * cfg.n_layers)()
        for l, L in enumerate(weights["layers"]):
            for f in _LAYER_FIELDS:
                if f in L:
                    want = np.uint8 if (fp8 or fp4) and f in PROJ_FIELDS else np.uint16
                    if L[f].dtype != want:
                        raise TypeError(f"layer {l} {f}: {L[f].dtype}, expected {np.dtype(want)}")
                    setattr(self.layers[l], f, L[f].ctypes.data)
            if fp8 or fp4:
                for f in PROJ_FIELDS:
                    if f in L:
                        sc = L[f + "_scale"]
                        shape = (L[f].shape[0],) if fp8 else (L[f].shape[0], L[f].shape[1] * 2 // 32)
                        if sc.dtype != (np.float32 if fp8 else np.uint8) or sc.shape != shape:
                            raise TypeError(f"layer {l} {f}_scale: {'fp32' if fp8 else 'uint8'} {list(shape)} expected")
                        setattr(self.layers[l], "s_" + f, sc.ctypes.data)
            if m.n_experts:
                E, F, H = m.n_experts, cfg.ffn, cfg.hidden
                for f, shape in (("w_router", (E, H)), ("w_gate", (E, F, H)), ("w_up", (E, F, H)), ("w_down", (E, H, F))):
                    if L[f].dtype != np.uint16 or L[f].shape != shape or not L[f].flags.c_contiguous:
                        raise TypeError(f"layer {l} {f}: bf16 {list(shape)} expected")
                self.layers[l].w_router = L["w_router"].ctypes.data
        ow = OrcWeights()
        ow.embed = weights["embed"].ctypes.data
        ow.final_norm = weights["final_norm"].ctypes.data
        ow.lm_head = weights["lm_head"].ctypes.data
        ow.layers = ctypes.cast(self.layers, P)
        self.ow = ow
        self.k_pages = cache["k_pages"].copy()
        self.v_pages = cache["v_pages"].copy()
        self.page_table = np.ascontiguousarray(cache["page_table"], dtype=np.int32)
        self.delta_state = cache["delta_state"].copy() if "delta_state" in cache else None
        self.conv_state = cache["conv_state"].copy() if "conv_state" in cache else None
        oc = OrcCache()
        oc.k_pages, oc.v_pages = self.k_pages.ctypes.data, self.v_pages.ctypes.data
        oc.num_pages, oc.max_pages_per_seq = int(cache["num_pages"]), int(cache["max_pages_per_seq"])
        oc.page_table = self.page_table.ctypes.data
        oc.delta_state = _ptr(self.delta_state)
        oc.conv_state = _ptr(self.conv_state)
        oc.max_batch = self.page_table.shape[0]
        self.oc = oc

    @property
    def mix_dim(self) -> int:
        c = self.cfg
        return max(c.n_q_heads * c.head_dim, c.n_delta_heads * c.delta_dv)

    def delta_mixer(self, layer: int, u, a, conv_state, delta_state):
        """The delta-rule mixer of layer `layer` for one sequence, from given projections u [C] and gate
        logits a [2 heads], conv state [C][W-1] and S^T [heads][dv][dk] (none modified).
        Returns (o [heads*dv], new conv state, new S^T)."""
        c = self.cfg
        cs = _c(conv_state, np.float32).copy()
        st = _c(delta_state, np.float32).copy()
        o = np.empty(c.n_delta_heads * c.delta_dv, dtype=np.float32)
        lib().orc_delta_mixer(ctypes.byref(self.m), self.w["layers"][layer]["conv_w"].ctypes.data,
                              _ptr(_c(u, np.float32)), _ptr(_c(a, np.float32)), _ptr(cs), _ptr(st), _ptr(o))
        return o, cs, st

    def step(self, tokens, positions, ctx_lens, dump: bool = False, force_experts=None):
        """One decode step.  Returns logits [B, V] (and a dict of mid-states when dump).  For
        mixture-of-experts models the mid-states include the router logits "router" [L, B, E] and the
        oracle's own expert choice "sel" [L, B, k]; force_experts [L, B, k] makes it use those experts
        instead of its own choice."""
        c = self.cfg
        tokens = _c(tokens, np.int32)
        positions = _c(positions, np.int32)
        ctx_lens = _c(ctx_lens, np.int32)
        B = tokens.size
        logits = np.empty((B, c.vocab), dtype=np.float32)
        d = None
        arrs = {}
        if dump:
            arrs = {"x_mixer": np.zeros((c.n_layers, B, c.hidden), np.float32),
                    "x_mlp": np.zeros((c.n_layers, B, c.hidden), np.float32),
                    "mixer_o": np.zeros((c.n_layers, B, self.mix_dim), np.float32),
                    "mlp_m": np.zeros((c.n_layers, B, c.ffn), np.float32),
                    "final_r": np.zeros((B, c.hidden), np.float32)}
            if self.m.n_experts:
                arrs["router"] = np.zeros((c.n_layers, B, self.m.n_experts), np.float32)
                arrs["sel"] = np.zeros((c.n_layers, B, self.m.top_k), np.int32)
        if arrs or force_experts is not None:
            d = OrcDump(**{k: v.ctypes.data for k, v in arrs.items()})
            if force_experts is not None:
                fe = np.ascontiguousarray(force_experts, dtype=np.int32)
                if fe.shape != (c.n_layers, B, self.m.top_k) or fe.min() < 0 or fe.max() >= self.m.n_experts:
                    raise ValueError("force_experts: [n_layers, batch, top_k] expert ids expected")
                d.force = fe.ctypes.data
                self._force_keep = fe
        rc = lib().orc_decode_step(ctypes.byref(self.m), ctypes.byref(self.ow), ctypes.byref(self.oc),
                                   tokens.ctypes.data, positions.ctypes.data, ctx_lens.ctypes.data, B,
                                   logits.ctypes.data, ctypes.byref(d) if d is not None else None)
        if rc != 0:
            raise ValueError(f"orc_decode_step rejected its inputs (code {rc})")
        return (logits, arrs) if dump else logits
