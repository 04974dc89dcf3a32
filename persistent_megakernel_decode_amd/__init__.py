"""Persistent decode megakernel for AMD MI355X (gfx950) -- Python binding.

A thin ctypes layer over libmk.so, whose C ABI is include/mk.h.  Every step
of the decode path runs inside the HIP megakernel; this module only moves
arguments across the boundary.  PyTorch supplies device memory and streams.

The library is required: importing this package without a built libmk.so
raises, and there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_ABI_VERSION = 3
MK_WEIGHTS_BF16, MK_WEIGHTS_FP8_E4M3, MK_WEIGHTS_FP4_MX = 0, 1, 2
MK_OK, MK_ERR_INVALID_ARG, MK_ERR_UNSUPPORTED, MK_ERR_HIP, MK_ERR_DEVICE_INPUT, MK_ERR_TIMEOUT, MK_ERR_STATE = \
    0, -1, -2, -3, -4, -5, -6
MK_LAYER_ATTN, MK_LAYER_DELTA = 0, 1
MK_MID_X_MIXER, MK_MID_X_MLP, MK_MID_MIXER_O, MK_MID_MLP_M, MK_MID_PROJ, MK_MID_EMBED, MK_MID_ROUTER = 0, 1, 2, 3, 4, 5, 6

STATUS_NAMES = {0: "MK_OK", -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_UNSUPPORTED", -3: "MK_ERR_HIP",
                -4: "MK_ERR_DEVICE_INPUT", -5: "MK_ERR_TIMEOUT", -6: "MK_ERR_STATE"}

P = ctypes.c_void_p
I32 = ctypes.c_int32


class mk_model_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
                ("n_layers", I32), ("hidden", I32), ("vocab", I32), ("ffn", I32),
                ("n_q_heads", I32), ("n_kv_heads", I32), ("head_dim", I32), ("qk_norm", I32),
                ("tied_embeddings", I32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("n_delta_heads", I32), ("delta_dk", I32), ("delta_dv", I32), ("conv_width", I32),
                ("layer_kind", P), ("max_batch", I32), ("max_ctx", I32), ("page_size", I32),
                ("weight_format", I32), ("n_experts", I32), ("top_k", I32)]


LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "w_qkv_delta", "w_gates", "conv_w",
                "wo_delta", "mlp_norm", "w_gate", "w_up", "w_down"]


# projection matrices: bf16, or fp8 E4M3 codes with fp32 row scales "<name>_scale"
PROJ_FIELDS = ["wq", "wk", "wv", "wo", "w_qkv_delta", "w_gates", "wo_delta", "w_gate", "w_up", "w_down"]


class mk_layer_weights(ctypes.Structure):
    _fields_ = [(f, P) for f in LAYER_FIELDS] + [(f + "_scale", P) for f in PROJ_FIELDS] + [("w_router", P)]


class mk_weights(ctypes.Structure):
    _fields_ = [("embed", P), ("final_norm", P), ("lm_head", P), ("layers", P)]


class mk_kv_cache(ctypes.Structure):
    _fields_ = [("k_pages", P), ("v_pages", P), ("num_pages", I32), ("max_pages_per_seq", I32),
                ("page_table", P), ("delta_state", P), ("conv_state", P)]


class mk_plan_info(ctypes.Structure):
    _fields_ = [("n_cus", I32), ("n_ops", I32), ("n_stages", I32), ("max_ops_per_cu", I32),
                ("weight_bytes", ctypes.c_double), ("max_cu_bytes", ctypes.c_double),
                ("mean_cu_bytes", ctypes.c_double), ("errors", I32)]


class mk_emu_config(ctypes.Structure):
    _fields_ = [("n_cus", I32), ("n_launches", I32), ("batch", P), ("ctx_lens", P), ("seed", ctypes.c_uint64),
                ("flags", ctypes.c_uint32)]


class mk_emu_report(ctypes.Structure):
    _fields_ = [("ops_run", ctypes.c_int64), ("polls", ctypes.c_int64), ("stale_accepts", ctypes.c_int64),
                ("unsynced_reads", ctypes.c_int64), ("double_writes", ctypes.c_int64),
                ("unwritten_cells", ctypes.c_int64), ("deadlocks", I32), ("first_bad_launch", I32)]


MK_EMU_COUNTERS, MK_EMU_IDLE_ITEMS_SILENT, MK_EMU_DEAD_ROWS_SILENT, MK_EMU_STALL_ONE_OP = 1, 2, 4, 8

EXPORTED = ["mk_workspace_size", "mk_create", "mk_decode_step", "mk_sync_status", "mk_reset", "mk_last_error",
            "mk_destroy", "mk_plan", "mk_emulate", "mk_copy_midstate", "mk_trace_words", "mk_copy_trace",
            "mk_create_static", "mk_decode_steps", "mk_stream_read", "mk_decode_window"]
MK_STATIC_SCRATCH_BYTES = 64 << 20
MK_MAX_STEPS = 4096
MK_MAX_WINDOW = 8
TRACE_WORDS = 8  # per-op trace record (mk_internal.h)

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with persistent_megakernel_decode_amd/build.py "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        L.mk_workspace_size.argtypes = [ctypes.POINTER(mk_model_desc), ctypes.POINTER(ctypes.c_size_t)]
        L.mk_create.argtypes = [ctypes.POINTER(mk_model_desc), ctypes.POINTER(mk_weights),
                                ctypes.POINTER(mk_kv_cache), P, ctypes.c_size_t, ctypes.POINTER(P)]
        L.mk_create_static.argtypes = [ctypes.POINTER(mk_model_desc), ctypes.POINTER(mk_weights),
                                       ctypes.POINTER(mk_kv_cache), ctypes.POINTER(P)]
        L.mk_decode_step.argtypes = [P, P, P, P, I32, P, P]
        L.mk_decode_steps.argtypes = [P, P, P, P, I32, I32, P, P, P]
        L.mk_stream_read.argtypes = [P, ctypes.c_size_t, P, I32, P]
        L.mk_decode_window.argtypes = [P, P, P, P, I32, I32, P, P]
        L.mk_sync_status.argtypes = [P]
        L.mk_reset.argtypes = [P]
        L.mk_last_error.argtypes = []
        L.mk_last_error.restype = ctypes.c_char_p
        L.mk_destroy.argtypes = [P]
        L.mk_destroy.restype = None
        L.mk_plan.argtypes = [ctypes.POINTER(mk_model_desc), I32, ctypes.POINTER(mk_plan_info)]
        L.mk_emulate.argtypes = [ctypes.POINTER(mk_model_desc), ctypes.POINTER(mk_emu_config),
                                 ctypes.POINTER(mk_emu_report)]
        L.mk_copy_midstate.argtypes = [P, I32, I32, P, ctypes.c_size_t, P]
        L.mk_trace_words.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.mk_copy_trace.argtypes = [P, P, ctypes.c_size_t]
        for f in ("mk_workspace_size", "mk_create", "mk_create_static", "mk_decode_step", "mk_decode_steps", "mk_stream_read", "mk_decode_window", "mk_sync_status", "mk_reset", "mk_plan",
                  "mk_emulate", "mk_copy_midstate", "mk_trace_words", "mk_copy_trace"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


class MKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mk_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def check(status: int, where: str) -> None:
    if status != MK_OK:
        raise MKError(status, where)


# ---------------------------------------------------------------- C-ABI wrappers (same names)
def make_desc(n_layers, hidden, vocab, ffn, n_q_heads, n_kv_heads, head_dim, qk_norm, tied_embeddings, rms_eps,
              rope_base, layer_kinds: Sequence[int], max_batch, max_ctx, n_delta_heads=0, delta_dk=0, delta_dv=0,
              conv_width=0, page_size=16, weight_format=MK_WEIGHTS_BF16, n_experts=0, top_k=0):
    kinds = (I32 * n_layers)(*layer_kinds)
    d = mk_model_desc(MK_ABI_VERSION, ctypes.sizeof(mk_model_desc), n_layers, hidden, vocab, ffn, n_q_heads,
                      n_kv_heads, head_dim, qk_norm, tied_embeddings, rms_eps, rope_base, n_delta_heads, delta_dk,
                      delta_dv, conv_width, ctypes.cast(kinds, P), max_batch, max_ctx, page_size, weight_format,
                      n_experts, top_k)
    d._kinds = kinds  # keep the array alive with the struct
    return d


def mk_workspace_size(desc: mk_model_desc) -> int:
    n = ctypes.c_size_t(0)
    check(lib().mk_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "mk_workspace_size")
    return n.value


def mk_plan(desc: mk_model_desc, n_cus: int) -> mk_plan_info:
    info = mk_plan_info()
    check(lib().mk_plan(ctypes.byref(desc), n_cus, ctypes.byref(info)), "mk_plan")
    return info


def mk_emulate(desc: mk_model_desc, n_cus: int, batches: Sequence[int], ctx_lens: Sequence[Sequence[int]],
               seed: int = 0, flags: int = 0):
    """Replay the compiled queues over a launch sequence on the CPU (no GPU).  ctx_lens[i] lists the
    context lengths of launch i (at least batches[i] entries).  Returns (report, findings text)."""
    import numpy as np
    n = len(batches)
    mb = desc.max_batch
    bt = np.ascontiguousarray(batches, dtype=np.int32)
    cl = np.zeros((max(n, 1), mb), dtype=np.int32)
    for i, row in enumerate(ctx_lens):
        cl[i, :min(len(row), mb)] = list(row)[:mb]
    cfg = mk_emu_config(n_cus, n, bt.ctypes.data, cl.ctypes.data, seed, flags)
    rep = mk_emu_report()
    check(lib().mk_emulate(ctypes.byref(desc), ctypes.byref(cfg), ctypes.byref(rep)), "mk_emulate")
    return rep, mk_last_error()


def mk_create(desc, weights: mk_weights, cache: mk_kv_cache, workspace_ptr: int, workspace_bytes: int) -> int:
    out = P()
    check(lib().mk_create(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(cache), workspace_ptr,
                          workspace_bytes, ctypes.byref(out)), "mk_create")
    return out.value


def mk_create_static(desc, weights: mk_weights, cache: mk_kv_cache) -> int:
    """mk_create with the library's static device scratch as the workspace (no allocation)."""
    out = P()
    check(lib().mk_create_static(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(out)),
          "mk_create_static")
    return out.value


def mk_decode_step(ctx: int, tokens_ptr: int, positions_ptr: int, ctx_lens_ptr: int, batch: int, logits_ptr: int,
                   stream: int = 0) -> int:
    return lib().mk_decode_step(ctx, tokens_ptr, positions_ptr, ctx_lens_ptr, batch, logits_ptr, stream or None)


def mk_decode_steps(ctx: int, tokens_ptr: int, positions_ptr: int, ctx_lens_ptr: int, batch: int, n_steps: int,
                    logits_ptr: int, tokens_out_ptr: int, stream: int = 0) -> int:
    return lib().mk_decode_steps(ctx, tokens_ptr, positions_ptr, ctx_lens_ptr, batch, n_steps, logits_ptr,
                                 tokens_out_ptr, stream or None)


def mk_decode_window(ctx: int, tokens_ptr: int, positions_ptr: int, ctx_lens_ptr: int, batch: int, window: int,
                     logits_ptr: int, stream: int = 0) -> int:
    return lib().mk_decode_window(ctx, tokens_ptr, positions_ptr, ctx_lens_ptr, batch, window, logits_ptr,
                                  stream or None)


def mk_stream_read(buf_ptr: int, nbytes: int, out_ptr: int, blocks: int, stream: int = 0) -> int:
    return lib().mk_stream_read(buf_ptr, nbytes, out_ptr, blocks, stream or None)


def mk_sync_status(ctx: int) -> int:
    return lib().mk_sync_status(ctx)


def mk_reset(ctx: int) -> int:
    return lib().mk_reset(ctx)


def mk_last_error() -> str:
    return lib().mk_last_error().decode(errors="replace")


def mk_destroy(ctx: int) -> None:
    lib().mk_destroy(ctx)


def mk_copy_midstate(ctx: int, kind: int, layer: int, dst_ptr: int, count: int, stream: int = 0) -> int:
    return lib().mk_copy_midstate(ctx, kind, layer, dst_ptr, count, stream or None)


# ---------------------------------------------------------------- device-resident model
class DecodeContext:
    """Owns the device tensors of one model and its mk_ctx.

    `weights` / `cache` are dicts of host numpy arrays (bf16 as uint16; with shape["weights"] ==
    "fp8" the projections as uint8 E4M3 codes with float32 "<name>_scale" row scales; "fp4" as packed
    uint8 E2M1 codes with uint8 E8M0 "<name>_scale" block scales) in the layout
    include/mk.h documents; they are copied to `device` once.  Only memory and the stream come from
    PyTorch.
    """

    ARENA_ALIGN = 2 << 20  # weights sit 2 MiB-aligned in one arena allocation

    def __init__(self, shape: dict, weights: dict, cache: dict, device: str = "cuda:0", arena: bool = True,
                 static_workspace: bool = False):
        import numpy as np
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.shape = dict(shape)
        i16 = torch.int16
        self.tensors: Dict[str, "torch.Tensor"] = {}
        keep: List = self.tensors.setdefault("_all", [])
        self.arena = None
        wfmt = shape.get("weights", "bf16")
        fp8, fp4 = wfmt == "fp8", wfmt == "fp4"
        if arena:  # one allocation for every weight tensor
            arrays = [weights["embed"], weights["final_norm"]] + ([] if shape["tied"] else [weights["lm_head"]])
            for L in weights["layers"]:
                arrays += [L[f] for f in LAYER_FIELDS + ["w_router"] if f in L]
                if fp8 or fp4:
                    arrays += [L[f + "_scale"] for f in PROJ_FIELDS if f in L]
            A = self.ARENA_ALIGN
            total = sum((a.nbytes + A - 1) // A * A for a in arrays) + A
            self.arena = torch.empty(total, dtype=torch.uint8, device=self.device)
            self._arena_off = (-self.arena.data_ptr()) % A

        def dev(a, dt=None):
            if self.arena is not None and dt in (i16, "raw"):
                n = a.nbytes
                view = self.arena[self._arena_off:self._arena_off + n]
                self._arena_off += (n + self.ARENA_ALIGN - 1) // self.ARENA_ALIGN * self.ARENA_ALIGN
                view.copy_(torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)))
                x = view.view(torch.int16) if dt is i16 else view
            elif dt == "raw":
                x = torch.from_numpy(np.ascontiguousarray(a)).to(self.device)
            else:
                x = torch.from_numpy(a).to(self.device) if dt is None else torch.from_numpy(a).view(dt).to(self.device)
            keep.append(x)
            return x

        s = self.shape
        self.desc = make_desc(s["n_layers"], s["hidden"], s["vocab"], s["ffn"], s["n_q_heads"], s["n_kv_heads"],
                              s["head_dim"], s["qk_norm"], s["tied"], s["rms_eps"], s["rope_base"], s["layer_kinds"],
                              s["max_batch"], s["max_ctx"], s.get("n_delta_heads", 0), s.get("delta_dk", 0),
                              s.get("delta_dv", 0), s.get("conv_width", 0), s.get("page_size", 16),
                              MK_WEIGHTS_FP8_E4M3 if fp8 else (MK_WEIGHTS_FP4_MX if fp4 else MK_WEIGHTS_BF16),
                              s.get("n_experts", 0), s.get("top_k", 0))
        self.embed = dev(weights["embed"], i16)
        final_norm = dev(weights["final_norm"], i16)
        lm = self.embed if s["tied"] else dev(weights["lm_head"], i16)
        self.layers = (mk_layer_weights * s["n_layers"])()
        for l, L in enumerate(weights["layers"]):
            for f in LAYER_FIELDS:
                if f in L:
                    if (fp8 or fp4) and f in PROJ_FIELDS:
                        if L[f].dtype != np.uint8 or L[f + "_scale"].dtype != (np.float32 if fp8 else np.uint8):
                            raise TypeError(f"layer {l} {f}: {wfmt} weights are uint8 codes with "
                                            f"{'float32 row' if fp8 else 'uint8 E8M0 block'} scales")
                        setattr(self.layers[l], f, dev(L[f], "raw").data_ptr())
                        setattr(self.layers[l], f + "_scale", dev(L[f + "_scale"], "raw").data_ptr())
                    else:
                        setattr(self.layers[l], f, dev(L[f], i16).data_ptr())
            if "w_router" in L:  # mixture of experts: expert-major w_gate / w_up / w_down above
                self.layers[l].w_router = dev(L["w_router"], i16).data_ptr()
        self.w = mk_weights(self.embed.data_ptr(), final_norm.data_ptr(), lm.data_ptr(), ctypes.cast(self.layers, P))
        self.k_pages = torch.from_numpy(cache["k_pages"]).view(i16).to(self.device)
        self.v_pages = torch.from_numpy(cache["v_pages"]).view(i16).to(self.device)
        keep += [self.k_pages, self.v_pages]
        self.page_table = dev(cache["page_table"])
        self.delta_state = dev(cache["delta_state"]) if "delta_state" in cache else None
        self.conv_state = dev(cache["conv_state"]) if "conv_state" in cache else None
        self.c = mk_kv_cache(self.k_pages.data_ptr(), self.v_pages.data_ptr(), int(cache["num_pages"]),
                             int(cache["max_pages_per_seq"]), self.page_table.data_ptr(),
                             self.delta_state.data_ptr() if self.delta_state is not None else None,
                             self.conv_state.data_ptr() if self.conv_state is not None else None)
        with torch.cuda.device(self.device):
            self.ws_bytes = mk_workspace_size(self.desc)
            if static_workspace:  # the library's static scratch: no workspace tensor
                self.workspace = None
                self.ctx = mk_create_static(self.desc, self.w, self.c)
            else:
                self.workspace = torch.zeros(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
                base = self.workspace.data_ptr()
                self.ws_ptr = (base + 255) // 256 * 256
                self.ctx = mk_create(self.desc, self.w, self.c, self.ws_ptr, self.ws_bytes)
        B = s["max_batch"]
        self.tokens = torch.zeros(B, dtype=torch.int32, device=self.device)
        self.positions = torch.zeros(B, dtype=torch.int32, device=self.device)
        self.ctx_lens = torch.zeros(B, dtype=torch.int32, device=self.device)
        self.logits = torch.zeros((B, s["vocab"]), dtype=torch.float32, device=self.device)

    def stream_ptr(self, stream=None) -> int:
        st = stream if stream is not None else self.torch.cuda.current_stream(self.device)
        return int(st.cuda_stream)

    def step(self, tokens, positions, ctx_lens, stream=None) -> int:
        """Enqueue one decode step from host lists (copied into device int32 arrays first)."""
        B = len(tokens)
        T = self.torch
        self.tokens[:B].copy_(T.as_tensor(list(tokens), dtype=T.int32))
        self.positions[:B].copy_(T.as_tensor(list(positions), dtype=T.int32))
        self.ctx_lens[:B].copy_(T.as_tensor(list(ctx_lens), dtype=T.int32))
        return mk_decode_step(self.ctx, self.tokens.data_ptr(), self.positions.data_ptr(), self.ctx_lens.data_ptr(),
                              B, self.logits.data_ptr(), self.stream_ptr(stream))

    def step_device(self, batch: int, stream=None) -> int:
        """Enqueue one decode step reading the device arrays self.tokens / positions / ctx_lens as they are."""
        return mk_decode_step(self.ctx, self.tokens.data_ptr(), self.positions.data_ptr(), self.ctx_lens.data_ptr(),
                              batch, self.logits.data_ptr(), self.stream_ptr(stream))

    def steps(self, tokens, positions, ctx_lens, n_steps: int, stream=None):
        """Enqueue n_steps greedy decode steps in one launch from host lists.  Returns (status,
        logits [n_steps][batch][vocab], tokens_out [n_steps][batch]): device tensors this call
        allocates, valid once the stream has run the launch."""
        B = len(tokens)
        T = self.torch
        self.tokens[:B].copy_(T.as_tensor(list(tokens), dtype=T.int32))
        self.positions[:B].copy_(T.as_tensor(list(positions), dtype=T.int32))
        self.ctx_lens[:B].copy_(T.as_tensor(list(ctx_lens), dtype=T.int32))
        logits = T.empty((n_steps, B, self.shape["vocab"]), dtype=T.float32, device=self.device)
        toks = T.empty((n_steps, B), dtype=T.int32, device=self.device)
        rc = mk_decode_steps(self.ctx, self.tokens.data_ptr(), self.positions.data_ptr(), self.ctx_lens.data_ptr(),
                             B, n_steps, logits.data_ptr(), toks.data_ptr(), self.stream_ptr(stream))
        return rc, logits, toks

    def window(self, tokens, positions, ctx_lens, stream=None):
        """Enqueue one verify-window step from host data: tokens [batch][window], positions and
        ctx_lens [batch] (of window token 0).  Returns (status, logits [batch][window][vocab]), the
        logits a device tensor this call allocates."""
        T = self.torch
        tk = T.as_tensor(tokens, dtype=T.int32)
        B, W = int(tk.shape[0]), int(tk.shape[1])
        toks = T.zeros(max(4, B * W), dtype=T.int32, device=self.device)
        toks[:B * W].copy_(tk.reshape(-1))
        self.positions[:B].copy_(T.as_tensor(list(positions), dtype=T.int32))
        self.ctx_lens[:B].copy_(T.as_tensor(list(ctx_lens), dtype=T.int32))
        logits = T.empty((B, W, self.shape["vocab"]), dtype=T.float32, device=self.device)
        self._window_tokens = toks  # kept alive until the launch has run
        rc = mk_decode_window(self.ctx, toks.data_ptr(), self.positions.data_ptr(), self.ctx_lens.data_ptr(), B, W,
                              logits.data_ptr(), self.stream_ptr(stream))
        return rc, logits

    def sync(self) -> int:
        return mk_sync_status(self.ctx)

    def reset(self) -> int:
        return mk_reset(self.ctx)

    def midstate(self, kind: int, layer: int, width: int, batch: int):
        out = self.torch.empty((batch, width), dtype=self.torch.float32, device=self.device)
        check(mk_copy_midstate(self.ctx, kind, layer, out.data_ptr(), batch * width, self.stream_ptr()),
              "mk_copy_midstate")
        return out

    def trace(self) -> dict:
        """Per-op timing of the last step (the context must have been created with MK_TRACE=1):
        queue offsets per CU and, per op, opcode, stage, the compute waves' start / inputs-ready / end
        stamps (100 MHz GPU clock, low 32 bits) and the loader wave's first-issue / last-issue stamps
        and the ticks it spent blocked on a full ring while issuing the op."""
        import numpy as np
        n = ctypes.c_size_t(0)
        check(lib().mk_trace_words(self.ctx, ctypes.byref(n)), "mk_trace_words")
        buf = np.zeros(n.value, np.uint32)
        check(lib().mk_copy_trace(self.ctx, buf.ctypes.data, n.value), "mk_copy_trace")
        n_ops, n_cus = int(buf[0]), int(buf[1])
        off = buf[2:3 + n_cus].astype(np.int64)
        rec = buf[3 + n_cus:].reshape(n_ops, TRACE_WORDS)
        cu = np.repeat(np.arange(n_cus), np.diff(off))
        return {"n_cus": n_cus, "queue_off": off, "cu": cu, "opcode": rec[:, 0] >> 16,
                "stage": (rec[:, 0] & 0xFFFF).astype(np.int16), "t": rec[:, 1:4].astype(np.int64),
                "loader": rec[:, 4:7].astype(np.int64)}

    def close(self) -> None:
        if getattr(self, "ctx", None):
            mk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
