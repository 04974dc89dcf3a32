"""Brute-force full-sequence recomputation -- TEST INFRASTRUCTURE ONLY.

An independent check of the decode oracle (oracle.c): NumPy float64, the
whole token sequence at once, causal mask instead of a KV cache, and the
gated delta rule in its closed product form instead of the step recurrence.
It shares no code with oracle.c.  Used on tiny shapes only.

Readings it follows (the pages print no model equations): RMSNorm
x * (mean x^2 + eps)^-1/2 * gain; rotate-half RoPE with angle
pos * base^(-2i/d); scores scaled by 1/sqrt(d); query head h reads KV head
floor(h * Hkv / Hq); cached K/V rounded to bf16 before use.  Delta-rule
layer (MK-KDA pull request, github choiceoh/stkernel #230, phase chain;
update S <- g S + beta k (v^T - k^T S)): SiLU after a causal depthwise conv,
per-head L2 norm of q and k, q scaled by dk^-1/2, g and beta sigmoids of
the gates projection [g | beta].  Mixture-of-experts MLP (top-k gating as in
Mixtral / OLMoE): router logits of the normalised input, the k largest (ties
to the lower index), softmax weights renormalised over those k, and the sum of
the chosen SwiGLU experts' outputs weighted by them.
"""
from __future__ import annotations

import numpy as np


def _f(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rms(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def rope_all(u: np.ndarray, base: float) -> np.ndarray:
    """u: [T, heads, d]; position t for row t."""
    T, _, d = u.shape
    half = d // 2
    inv = base ** (-2.0 * np.arange(half) / d)
    ang = np.arange(T)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def attention_layer(cfg, L, R):
    T = R.shape[0]
    d, Hq, Hkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    Q = (R @ _f(L["wq"]).T).reshape(T, Hq, d)
    K = (R @ _f(L["wk"]).T).reshape(T, Hkv, d)
    V = (R @ _f(L["wv"]).T).reshape(T, Hkv, d)
    if cfg.qk_norm:
        Q = rms(Q, _f(L["q_norm"]), cfg.rms_eps)
        K = rms(K, _f(L["k_norm"]), cfg.rms_eps)
    Q = rope_all(Q, cfg.rope_base)
    K = round_bf16(rope_all(K, cfg.rope_base))
    V = round_bf16(V)
    mask = np.tril(np.ones((T, T), dtype=bool))
    O = np.zeros((T, Hq, d))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        S = (Q[:, h, :] @ K[:, g, :].T) / np.sqrt(d)
        S = np.where(mask, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        Pm = np.exp(S)
        Pm /= Pm.sum(axis=1, keepdims=True)
        O[:, h, :] = Pm @ V[:, g, :]
    return O.reshape(T, Hq * d)


def delta_layer(cfg, L, R, S0=None, conv0=None, decay_first=False):
    """Full-sequence gated delta-rule layer.

    S0: initial S^T per head [heads, dv, dk] (None = 0); conv0: initial conv window [C, W-1] (None = 0).
    Returns (outputs [T, heads*dv], final S^T [heads, dv, dk], final conv window [C, W-1]).
    """
    T = R.shape[0]
    nh, dk, dv, W = cfg.n_delta_heads, cfg.delta_dk, cfg.delta_dv, cfg.conv_width
    C = nh * (2 * dk + dv)
    U = R @ _f(L["w_qkv_delta"]).T            # [T, C]
    A = R @ _f(L["w_gates"]).T                # [T, 2 nh]
    pre = np.zeros((W - 1, C)) if conv0 is None else np.asarray(conv0, np.float64).T
    Upad = np.concatenate([pre, U], axis=0)   # zero (or given) left padding, oldest first
    cw = _f(L["conv_w"])                      # [C, W]
    Y = np.stack([np.sum(Upad[t:t + W, :].T * cw, axis=1) for t in range(T)])  # full causal conv1d
    Y = silu(Y)
    conv_final = Upad[-(W - 1):, :].T.copy()
    out = np.zeros((T, nh * dv))
    S_final = np.zeros((nh, dv, dk))
    eye = np.eye(dk)
    for h in range(nh):
        q = Y[:, h * dk:(h + 1) * dk]
        k = Y[:, nh * dk + h * dk: nh * dk + (h + 1) * dk]
        v = Y[:, 2 * nh * dk + h * dv: 2 * nh * dk + (h + 1) * dv]
        q = q / np.sqrt(np.sum(q * q, axis=1, keepdims=True) + 1e-6) / np.sqrt(dk)
        k = k / np.sqrt(np.sum(k * k, axis=1, keepdims=True) + 1e-6)
        g = sigmoid(A[:, h])
        beta = sigmoid(A[:, nh + h])
        # A_s = g_s I - beta_s k_s k_s^T (literal update) or g_s (I - beta_s k_s k_s^T) (decay first)
        As = [(g[s] * (eye - beta[s] * np.outer(k[s], k[s]))) if decay_first
              else (g[s] * eye - beta[s] * np.outer(k[s], k[s])) for s in range(T)]
        S0h = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[h], np.float64).T  # S = (S^T)^T
        for t in range(T):
            # S_t = sum_{s<=t} (A_t ... A_{s+1}) beta_s k_s v_s^T + (A_t ... A_0) S0
            St = np.zeros((dk, dv))
            Pm = eye.copy()                     # A_t ... A_{s+1}, built from the left end inward
            for s in range(t, -1, -1):
                St += Pm @ (beta[s] * np.outer(k[s], v[s]))
                Pm = Pm @ As[s]
            St += Pm @ S0h
            out[t, h * dv:(h + 1) * dv] = St.T @ q[t]
            if t == T - 1:
                S_final[h] = St.T
    return out, S_final, conv_final


def moe_mlp(cfg, L, R):
    """Mixture-of-experts MLP of every position of R [T, H]: each row routed on its own."""
    E, k = cfg.n_experts, cfg.top_k
    Z = R @ _f(L["w_router"]).T                  # [T, E] router logits
    Wg, Wu, Wd = _f(L["w_gate"]), _f(L["w_up"]), _f(L["w_down"])
    out = np.zeros_like(R)
    for t in range(R.shape[0]):
        z = Z[t]
        chosen = np.lexsort((np.arange(E), -z))[:k]   # descending logit, ties to the lower index
        p = np.exp(z - z.max())
        p = p / p.sum()
        g = p[chosen] / p[chosen].sum()
        for e, ge in zip(chosen, g):
            m = silu(Wg[e] @ R[t]) * (Wu[e] @ R[t])
            out[t] += ge * (Wd[e] @ m)
    return out


def forward(cfg, w, tokens, S0=None, conv0=None, decay_first=False):
    """Logits of the last position after running the whole sequence `tokens` (prompt mode).

    S0 / conv0: optional initial delta / conv states per delta layer ([nD][heads, dv, dk], [nD][C, W-1]).
    Returns (logits [V], per-layer residual after each MLP [L][H] at the last position, final states).
    """
    T = len(tokens)
    X = _f(w["embed"])[np.asarray(tokens)]
    xs = []
    states = []
    idx = 0
    for l, kind in enumerate(cfg.kinds()):
        L = w["layers"][l]
        R = rms(X, _f(L["attn_norm"]), cfg.rms_eps)
        if kind == 0:
            X = X + attention_layer(cfg, L, R) @ _f(L["wo"]).T
        else:
            O, Sf, cf = delta_layer(cfg, L, R, None if S0 is None else S0[idx], None if conv0 is None else conv0[idx],
                                    decay_first)
            states.append((Sf, cf))
            idx += 1
            X = X + O @ _f(L["wo_delta"]).T
        R = rms(X, _f(L["mlp_norm"]), cfg.rms_eps)
        if getattr(cfg, "n_experts", 0):
            X = X + moe_mlp(cfg, L, R)
        else:
            M = silu(R @ _f(L["w_gate"]).T) * (R @ _f(L["w_up"]).T)
            X = X + M @ _f(L["w_down"]).T
        xs.append(X[-1].copy())
    r = rms(X[-1], _f(w["final_norm"]), cfg.rms_eps)
    logits = _f(w["lm_head"]) @ r
    return logits, xs, states
