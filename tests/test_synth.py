"""The seeded input generators: published SplitMix64 outputs, determinism, distributions."""
import numpy as np
import torch

import moe_synth as synth


def test_splitmix64_published_first_outputs():
    # SplitMix64 seeded with 0 starts 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4 (Vigna's reference generator).
    assert synth.splitmix64_py(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64_py(0, 1) == 0x6E789E6AA1B965F4


def test_torch_words_match_python_definition():
    for key in (0, 1, 0xFFFFFFFFFFFFFFFF, synth.derive_key(3, 4, 5)):
        for start in (0, 12345, 10**10):
            got = synth.splitmix64_words(key, start, 64).tolist()
            want = [synth._signed(synth.splitmix64_py(key, start + i)) for i in range(64)]
            assert got == want


def test_code_bytes_little_endian_words():
    key = synth.derive_key(9)
    out = torch.empty(16, dtype=torch.uint8)
    synth.fill_code_bytes(out, key)
    w0 = synth.splitmix64_py(key, 0)
    assert out[:8].tolist() == [(w0 >> (8 * j)) & 0xFF for j in range(8)]


def test_expert_slices_match_whole_layer():
    wl = synth.WORKLOADS["tiny"]
    full = synth.layer_weights(wl, 0)
    for mat in synth.MATRICES:
        for g in (0, 3, wl.experts):
            c, s = synth.expert_matrix(wl, 0, mat, g)
            assert torch.equal(c, full[mat][0][g]) and torch.equal(s, full[mat][1][g])


def test_distributions():
    wl = synth.WORKLOADS["tiny"]
    full = synth.layer_weights(wl, 0)
    codes = full["gate"][0].numpy().reshape(-1)
    nib = np.concatenate([codes & 15, codes >> 4])
    hist = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(hist - 1 / 16) < 0.01)
    sc = full["down"][1].numpy().reshape(-1)
    assert sc.min() == 123 and sc.max() == 127
    assert np.all(np.abs(np.bincount(sc - 123, minlength=5) / sc.size - 0.2) < 0.03)
    wr = synth.router_weights(synth.WORKLOADS["decode_t8"])
    assert abs(wr.std() - 0.02) < 2e-4 and abs(wr.mean()) < 2e-4


def test_determinism_and_distinct_streams():
    a = synth.tokens("decode_t8", layer=0, step=0)
    b = synth.tokens("decode_t8", layer=0, step=0)
    c = synth.tokens("decode_t8", layer=1, step=0)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    c1, _ = synth.expert_matrix("decode_t8", 0, "gate", 5)
    c2, _ = synth.expert_matrix("decode_t8", 1, "gate", 5)
    assert not torch.equal(c1, c2)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -2.5, 1 + 2 ** -7 + 2 ** -9], np.float32)
    bits = synth.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); 1+2^-7+2^-9 rounds to 1+2^-7
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x3F81]


def test_fp8_shared_expert_draws():
    wl = synth.custom_workload("fp8_small", 256, 4, 2, 1, 384, 4, shared_fp8=True)
    assert wl.fp4_groups == 4 and wl.groups == 5
    w = synth.shared_fp8_weights(wl, 0)
    for mat, (n, k) in (("gate", (384, 256)), ("up", (384, 256)), ("down", (256, 384))):
        c, s = w[mat]
        assert c.shape == (n, k) and c.dtype == torch.uint8
        assert s.shape == (n // 128, k // 128) and s.dtype == torch.float32
        assert not ((c & 0x7F) == 0x7F).any()                   # no NaN pattern is drawn
        assert len(torch.unique(c)) == 254                       # every finite code occurs
        assert (s >= 2.0 ** -8).all() and (s < 1.5 * 2.0 ** -7).all()
        c2, s2 = synth.shared_fp8_matrix(wl, 0, mat)
        assert torch.equal(c, c2) and torch.equal(s, s2)         # deterministic
    # FP4 arrays hold the routed experts only, with the same bytes a per-group draw gives
    fp4 = synth.layer_weights(wl, 0)
    assert fp4["gate"][0].shape[0] == 4
    c, sc = synth.expert_matrix(wl, 0, "down", 3)
    assert torch.equal(fp4["down"][0][3], c) and torch.equal(fp4["down"][1][3], sc)
    g = synth.LazyExperts(wl, 0)[4]
    assert g["up"][0] == "fp8" and np.array_equal(g["up"][1], w["up"][0].numpy())


def test_fp8_flag_leaves_other_workload_ids_alone():
    a = synth.custom_workload("w", 256, 4, 2, 1, 128, 4)
    b = synth.custom_workload("w", 256, 4, 2, 1, 128, 4, shared_fp8=True)
    assert synth._wl_id(a) != synth._wl_id(b)
    assert synth.WORKLOADS["decode_t8"].fp4_groups == 257


def test_chain_inputs_are_seeded_and_shaped():
    wl = synth.WORKLOADS["chained_decode_16l"]
    h = synth.residual_input(wl, step=3)
    assert h.shape == (1, 4096) and h.dtype == np.float32
    assert np.array_equal(h, synth.residual_input(wl, step=3))
    assert not np.array_equal(h, synth.residual_input(wl, step=4))
    g = synth.norm_weight(wl, 5)
    assert g.shape == (4096,) and g.dtype == np.float32 and abs(g.mean() - 1) < 0.01 and 0.08 < g.std() < 0.12
    assert not np.array_equal(g, synth.norm_weight(wl, 6))
    # workloads without the later fields keep the ids they had before those fields existed
    a = synth.custom_workload("w", 256, 4, 2, 1, 128, 4)
    assert synth._wl_id(a) == synth._wl_id(synth.custom_workload("w", 256, 4, 2, 1, 128, 4, chained=False))
