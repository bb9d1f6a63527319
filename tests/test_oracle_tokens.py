"""Oracle token arithmetic against the numbers the pages print."""
import oracle as O
import pfgen


def test_tokens_per_block(golden):
    g = golden["tokens_per_block"]
    assert O.tokens_per_block(**g["inputs"]) == g["value"] == 6240


def test_compressed_tokens(golden):
    g = golden["compressed_tokens"]
    assert O.compressed_tokens(**g["inputs"]) == g["value"] == 182


def test_compressed_tokens_latent_form():
    # "Feature Fusion" restates N_c on the latent grid as floor(T/2) floor(H/8) floor(W/8);
    # the patch embedding halves each spatial side, so H = 2h = 60 and W = 2w = 104.
    assert (4 // 2) * (60 // 8) * (104 // 8) == O.compressed_tokens(4, 30, 52)


def test_context_size(golden):
    g = golden["context_size"]
    assert O.context_size(**g["inputs"]) == g["value"] == 27872


def test_uncompressed_context(golden):
    g = golden["uncompressed_tokens_2min"]
    inp = g["inputs"]
    tokens = inp["blocks"] * O.tokens_per_block(inp["block_frames"], inp["h"], inp["w"])
    assert tokens == 748800
    assert abs(tokens - g["value_approx"]) <= g["tolerance"]
    gb = golden["uncompressed_kv_gb"]
    nbytes = O.kv_cache_bytes(tokens, **gb["inputs"])
    assert abs(nbytes / 1e9 - gb["value_approx"]) <= gb["tolerance"]


def test_sink_share(golden):
    n = O.tokens_per_block(4, 30, 52)
    sink = (golden["sink_share_below"]["inputs"]["n_sink_frames"] // 4) * n
    assert sink == 12480
    assert sink / (120 * n) < golden["sink_share_below"]["value"]


def test_rope_split(golden):
    g = golden["rope_split"]
    assert [O.T_DIMS, O.H_DIMS, O.W_DIMS] == g["value"]
    assert sum(g["value"]) == g["total"] == O.HEAD_DIM


def test_reduction_ratios(golden):
    ratio = O.tokens_per_block(4, 30, 52) / O.compressed_tokens(4, 30, 52)
    assert abs(ratio / golden["token_reduction_approx"]["value"] - 1) < 0.1
    f = golden["volume_reduction"]["factors"]
    assert f[0] * f[1] * f[2] == golden["volume_reduction"]["value"]


def test_config_shapes():
    assert (pfgen.C0.n, pfgen.C0.n_c, pfgen.C0.n_keys) == (256, 8, 1056)
    assert (pfgen.C1.n, pfgen.C1.n_c, pfgen.C1.n_keys) == (6240, 182, 27872)
    assert pfgen.C1.n_keys == O.context_size(8, 16, 4, 4, 30, 52)
    assert pfgen.C2.n_keys == 27872 and pfgen.C2.pool_blocks == 116
    # C2's history: 2 sink + 116 pool + 1 recent + 1 current = 120 blocks
    assert 2 + 116 + 1 + 1 == 120
    assert pfgen.C4.n_sink + pfgen.C4.n_recent + pfgen.C4.n == 748800
