"""Pins of the oracle's low-bit weight paths: fp8 (E4M3 codes with fp32 row scales) and MX fp4 (E2M1
codes with E8M0 scales per block of 32).

The code table is pinned to PyTorch's own float8_e4m3fn type (a library decoding of the same OCP
format, independent of oracle.c) and to values the format fixes; the projection to a brute-force
product of those library-decoded values; and the whole decode step to the bf16 path (itself pinned
by oracle_pins and the brute-force recomputation): with power-of-two row scales every fp8 weight is
exactly a bf16 number, and the fp8 model must give the bf16 model's logits bit for bit.  A slip in
the code table, a scale applied by column or to the wrong projection, or a projection left on the
bf16 path fails one of these.  fp4: the E2M1 table against the format's eight magnitudes, E8M0
against PyTorch's float8_e8m0fnu, the block-scaled product against a float64 product of weights
unpacked here, one block scale moving one row by that block's share, and the decode step bit for bit
against the bf16 model holding the same (exactly representable) weights.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def torch_e4m3(codes) -> np.ndarray:
    """PyTorch's decoding of E4M3 codes (float8_e4m3fn), widened to float64."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_table_matches_pytorch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_e4m3(codes)
    got = np.array([oracle.e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # -0 at 0x80


def test_e4m3_values_the_format_fixes():
    # OCP 8-bit floating point, E4M3: bias 7, largest finite 448 (0x7E), NaN at S.1111.111 only,
    # smallest subnormal 2^-9, smallest normal 2^-6
    assert oracle.e4m3(0x38) == 1.0 and oracle.e4m3(0xB8) == -1.0
    assert oracle.e4m3(0x7E) == 448.0 and oracle.e4m3(0xFE) == -448.0
    assert np.isnan(oracle.e4m3(0x7F)) and np.isnan(oracle.e4m3(0xFF))
    assert oracle.e4m3(0x78) == 256.0  # exponent field 15 is finite apart from mantissa 7
    assert oracle.e4m3(0x01) == 2.0 ** -9 and oracle.e4m3(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x00) == 0.0 and np.signbit(oracle.e4m3(0x80))
    # positive codes increase strictly with the code up to 448: the encoding is sign-magnitude
    v = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(v, v[1:]))


def test_generated_codes_are_finite_and_spread():
    c = synth.fp8_codes(200_000, 3, "pin")
    v = torch_e4m3(c)
    assert not np.isnan(v).any()
    e = (c >> 3) & 15
    assert e.max() == 14 and (e <= 1).any()  # the bottom fields (subnormal at 0) appear too
    # field e has probability 2^(e-15): halves per step below the top
    h = np.bincount(e, minlength=16)
    assert 0.45 < h[14] / c.size < 0.55 and 0.2 < h[13] / c.size < 0.3


def test_matvec_fp8_is_the_scaled_product():
    rng = np.random.default_rng(7)
    W = synth.fp8_codes((7, 33), 1, "mv")
    s = rng.uniform(0.5, 2.0, 7).astype(np.float32)
    x = rng.standard_normal(33).astype(np.float32)
    want = s.astype(np.float64) * (torch_e4m3(W) @ x.astype(np.float64))
    got = oracle.matvec_fp8(W, s, x)
    assert np.allclose(got, want, rtol=1e-6, atol=0)
    # all-ones codes: each row is its scale times the sum of the inputs
    ones = np.full((3, 33), 0x38, np.uint8)
    assert np.allclose(oracle.matvec_fp8(ones, s[:3], x), s[:3] * x.astype(np.float64).sum(), rtol=1e-6)


def _pow2_scales(w: dict, seed: int) -> dict:
    """The fp8 weights with every row scale replaced by a power of two, 2^-12 .. 2^-5 (drawn per row)."""
    out = dict(w)
    out["layers"] = []
    for l, L in enumerate(w["layers"]):
        L = dict(L)
        for f in oracle.PROJ_FIELDS:
            if f in L:
                k = synth.u32(L[f].shape[0], seed, f"pow2.{l}.{f}") % 8
                L[f + "_scale"] = (2.0 ** -(5.0 + k)).astype(np.float32)
        out["layers"].append(L)
    return out


def _as_bf16(w: dict) -> dict:
    """The same model with every fp8 projection widened to bf16 (exact: an E4M3 value times a power
    of two has at most four significant bits), through PyTorch's decoding."""
    out = dict(w, format="bf16")
    out["layers"] = []
    for L in w["layers"]:
        L = dict(L)
        for f in oracle.PROJ_FIELDS:
            if f in L:
                v = torch_e4m3(L[f]) * L.pop(f + "_scale").astype(np.float64)[:, None]
                b = torch.from_numpy(v).to(torch.bfloat16)
                assert np.array_equal(b.to(torch.float64).numpy(), v)  # exact
                L[f] = b.view(torch.int16).numpy().view(np.uint16)
        out["layers"].append(L)
    return out


@pytest.mark.parametrize("name", ["tiny-gain", "tiny-qknorm", "tiny-hybrid"])
def test_fp8_step_equals_bf16_step_at_power_of_two_scales(name):
    cfg = synth.SMALL[name].replace(weights="fp8")
    w8 = _pow2_scales(synth.make_weights(cfg), cfg.seed)
    wb = _as_bf16(w8)
    ctx = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx, 2)
    o8, ob = oracle.DecodeOracle(cfg, w8, cache), oracle.DecodeOracle(cfg.replace(weights="bf16"), wb, cache)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    for s in range(2):
        pos = [c + s for c in ctx]
        a = o8.step(toks, pos, [p + 1 for p in pos])
        b = ob.step(toks, pos, [p + 1 for p in pos])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {s}"
        toks = [oracle.argmax(r) for r in a]
    if o8.delta_state is not None:
        assert np.array_equal(o8.delta_state, ob.delta_state)
        assert np.array_equal(o8.conv_state, ob.conv_state)


def test_fp8_scales_are_per_row_of_each_projection():
    """Doubling one projection's scale of one row changes that projection's output row only: the
    oracle's logits move, and restoring it restores them bit for bit."""
    cfg = synth.SMALL["tiny-gain"].replace(weights="fp8")
    w = synth.make_weights(cfg)
    ctx = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx, 1)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    base = oracle.DecodeOracle(cfg, w, cache).step(toks, ctx, [c + 1 for c in ctx])
    for f in ("wv", "w_down"):
        L = w["layers"][1]
        keep = L[f + "_scale"].copy()
        L[f + "_scale"][3] *= 2.0
        moved = oracle.DecodeOracle(cfg, w, cache).step(toks, ctx, [c + 1 for c in ctx])
        L[f + "_scale"][:] = keep
        assert not np.array_equal(moved, base), f
        again = oracle.DecodeOracle(cfg, w, cache).step(toks, ctx, [c + 1 for c in ctx])
        assert np.array_equal(again, base)


# ------------------------------------------------------------------ MX fp4 (E2M1 + E8M0 block scales)
def test_e2m1_values_the_format_fixes():
    # OCP Microscaling formats, E2M1: the eight magnitudes 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6
    # and their negatives (the sign bit is bit 3); no infinities, no NaN
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = [oracle.e2m1(c) for c in range(16)]
    assert got[:8] == want and got[8:] == [-v for v in want]
    assert np.signbit(oracle.e2m1(8)) and not np.signbit(oracle.e2m1(0))
    assert oracle.e2m1(0x17) == oracle.e2m1(0x7)  # only the low 4 bits count


def test_e8m0_matches_pytorch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got[255])
    assert np.array_equal(got[:255], ref[:255])
    assert oracle.e8m0(127) == 1.0 and oracle.e8m0(0) == 2.0 ** -127


def fp4_values(W_packed, S) -> np.ndarray:
    """Weights of an fp4 matrix in float64, unpacked here by nibble (low first) with the format's value
    table and PyTorch's E8M0 decoding."""
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
    W = np.asarray(W_packed, np.uint8)
    codes = np.stack([W & 15, W >> 4], axis=-1).reshape(W.shape[0], -1)
    v = table[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    sc = torch.from_numpy(np.ascontiguousarray(S)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return v * np.repeat(sc, 32, axis=1)


def test_matvec_fp4_is_the_block_scaled_product():
    rng = np.random.default_rng(9)
    cfg = synth.CONFIGS["tiny"].replace(weights="fp4")
    L = {}
    synth._proj(cfg, L, "w", 7, 96, "pin.")
    x = rng.standard_normal(96).astype(np.float32)
    want = fp4_values(L["w"], L["w_scale"]) @ x.astype(np.float64)
    assert np.allclose(oracle.matvec_fp4(L["w"], L["w_scale"], x), want, rtol=1e-6, atol=0)
    # one block's scale doubled moves only that row, by that block's share
    S2 = L["w_scale"].copy()
    S2[3, 1] += 1
    d = oracle.matvec_fp4(L["w"], S2, x).astype(np.float64) - oracle.matvec_fp4(L["w"], L["w_scale"], x)
    blk = fp4_values(L["w"], L["w_scale"])[3, 32:64] @ x[32:64].astype(np.float64)
    assert np.allclose(d[3], blk, rtol=1e-5) and np.count_nonzero(d) == 1


def _fp4_as_bf16(w: dict) -> dict:
    """The fp4 model with every projection widened to bf16 (exact: an E2M1 value times a power of two)."""
    out = dict(w, format="bf16")
    out["layers"] = []
    for L in w["layers"]:
        L = dict(L)
        for f in oracle.PROJ_FIELDS:
            if f in L:
                v = fp4_values(L[f], L.pop(f + "_scale"))
                b = torch.from_numpy(v).to(torch.bfloat16)
                assert np.array_equal(b.to(torch.float64).numpy(), v)
                L[f] = b.view(torch.int16).numpy().view(np.uint16)
        out["layers"].append(L)
    return out


@pytest.mark.parametrize("name", ["tiny-gain", "tiny-qknorm"])
def test_fp4_step_equals_bf16_step(name):
    cfg = synth.SMALL[name].replace(weights="fp4")
    w4 = synth.make_weights(cfg)
    wb = _fp4_as_bf16(w4)
    ctx = synth.context_lengths(cfg)
    cache = synth.make_cache(cfg, ctx, 2)
    o4, ob = oracle.DecodeOracle(cfg, w4, cache), oracle.DecodeOracle(cfg.replace(weights="bf16"), wb, cache)
    toks = [int(t) for t in synth.first_tokens(cfg)]
    for s in range(2):
        pos = [c + s for c in ctx]
        a = o4.step(toks, pos, [p + 1 for p in pos])
        b = ob.step(toks, pos, [p + 1 for p in pos])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {s}"
        toks = [oracle.argmax(r) for r in a]
