"""The seeded generator itself: Philox4x32-10 known answers and draw statistics."""
import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors published with the Philox definition (Random123 kat_vectors).
    assert synth.philox([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_normal_statistics_and_determinism():
    z = synth.normal_f32(400_000, 7, "t")
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.array_equal(z[:1000], synth.normal_f32(1000, 7, "t"))  # prefix-stable (counter-based)
    w = synth.bf16_to_f32(synth.normal_bf16(100_000, 7, "w", 0.02))
    assert abs(w.std() - 0.02) < 0.001


def test_cache_layout_and_page_permutation():
    cfg = synth.CONFIGS["tiny"].replace(batch=3, ctx=[5, 40, 17], shuffle_pages=True)
    cache = synth.make_cache(cfg, cfg.ctx, 8)
    t = cache["page_table"]
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(cache["num_pages"]))  # a permutation of page ids
    # K of sequence 1 at position 33 lives at (page_table[1][2], slot 1)
    kk = synth.normal_bf16((40, cfg.n_kv_heads, cfg.head_dim), cfg.seed, "k_cache.0.1")
    assert np.array_equal(cache["k_pages"][0, t[1, 2], :, 1, :], kk[33])
