"""bench.py's host-side accounting (no GPU): the algorithmic flops and bytes it divides by,
against counts made here from the shapes (per layer, per product) and brute force."""
import bench
import ttt_workloads as W


def test_step_flops_per_token_at_the_760m_shape():
    """Per token: the up and down products of 3 blocks forward (2 x 2dm each), dA, G2, G1
    backward in every block and dHn in the two upper ones (2dm each), logits and dY (2Vd each)."""
    d, m, V = 1536, 6144, 32000
    fwd = 3 * (2 * d * m + 2 * d * m)
    bwd = 3 * (3 * 2 * d * m) + 2 * (2 * d * m)
    head = 2 * V * d + 2 * V * d
    assert bench.alg_flops_per_token(W.preset("s760m")) == fwd + bwd + head == 517472256


def test_decode_bytes_per_token():
    """One decoded token reads each weight once: bf16 fast tensors as two terms (W0, rn(D)),
    the LM head, and for the fuller block the static MLP, [Wq Wk Wv], Wo and a full window of
    keys and values (hi and lo terms)."""
    d, m, V = 1536, 6144, 32000
    fast = 2 * (2 * d * m * 2)  # W1 and W2, two bf16 terms each
    assert bench.decode_bytes_per_token(W.preset("s760m")) == 3 * fast + V * d * 2 == 324796416
    w = W.preset("e2e760m")
    d, m, ms, k = w.d_model, w.d_hidden, w.static_hidden, w.swa_window
    per_block = 2 * (2 * d * m * 2) + 2 * d * ms * 2 + 4 * d * d * 2 + 4 * k * d * 2
    assert bench.decode_bytes_per_token(w) == 3 * per_block + w.vocab * d * 2 == 626786304


def test_visible_keys_brute_force():
    w = W.preset("e2e760m", swa_window=5)
    for pos, n in [(0, 12), (3, 4), (40, 7)]:
        brute = sum(len([kk for kk in range(p + 1) if p - kk < 5]) for p in range(pos, pos + n))
        assert bench.visible_keys(w, pos, n) == brute


def test_attention_flops_of_the_timed_steps():
    """Past the first window every query sees the whole window: the forward core is 4d flops
    per visible key, so a launch (one block, one chunk) is 4 d b k."""
    w = W.preset("e2e760m")
    launches = w.n_chunks * w.n_blocks
    full = bench.e2e_flops_per_step(w, w.n_tokens)["attn_fwd"] / launches
    assert full == 4 * w.d_model * w.chunk * w.swa_window
    first = bench.e2e_flops_per_step(w, 0)["attn_fwd"] / launches
    assert first < full  # the first pass over the stream starts with short windows
