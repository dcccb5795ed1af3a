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
    """The method reads each weight once per decoded token, in one bf16 copy: the fast tensors
    W1 and W2 of every block, the LM head, and for the fuller block the static MLP, [Wq Wk Wv],
    Wo and one copy of a full window's keys and values (about 211 MB and 419 MB)."""
    d, m, V = 1536, 6144, 32000
    fast = 2 * (d * m * 2)  # W1 and W2, one bf16 copy each
    assert bench.decode_bytes_per_token(W.preset("s760m")) == 3 * fast + V * d * 2 == 211550208
    w = W.preset("e2e760m")
    d, m, ms, k = w.d_model, w.d_hidden, w.static_hidden, w.swa_window
    per_block = 2 * (d * m * 2) + 2 * d * ms * 2 + 4 * d * d * 2 + 2 * k * d * 2
    assert bench.decode_bytes_per_token(w) == 3 * per_block + w.vocab * d * 2 == 419168256


def test_decode_implementation_bytes_per_token():
    """What the implementation reads: bf16 fast tensors as two terms (W0, rn(D)); the keys and
    values in one half-precision copy (as many bytes as the method's bf16 copy)."""
    d, m, V = 1536, 6144, 32000
    fast = 2 * (2 * d * m * 2)
    assert bench.decode_impl_bytes_per_token(W.preset("s760m")) == 3 * fast + V * d * 2 == 324796416
    w = W.preset("e2e760m")
    d, m, ms, k = w.d_model, w.d_hidden, w.static_hidden, w.swa_window
    per_block = 2 * (2 * d * m * 2) + 2 * d * ms * 2 + 4 * d * d * 2 + 2 * k * d * 2
    assert bench.decode_impl_bytes_per_token(w) == 3 * per_block + w.vocab * d * 2 == 475791360


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


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(monkeypatch):
    """roofline.traffic comes from the committed counter summaries, which record the sha256 of
    the sources the counters were taken on: a line's dominant kind has a figure while the
    sources read as recorded, and none once they read differently (the attention forward is
    checked against its own sources, the GEMM kinds against the GEMM sources)."""
    import os
    import re
    kinds = [("s760m", "up"), ("single", "ce_fwd"), ("s125m", "dw"), ("inplace", "ce_fwd"), ("e2e760m", "attn")]
    for wl, kind in kinds:
        text = open(os.path.join(bench.ROOT, "profiles", f"traffic_{wl}.md")).read()
        rec = {lab: re.search(rf"^{lab}_sources_sha256:\s*([0-9a-f]{{64}})", text, re.M).group(1)
               for lab in ("gemm", "attention") if re.search(rf"^{lab}_sources_sha256:", text, re.M)}
        as_recorded = lambda src: rec["attention"] if src == bench.ATTENTION_SOURCES else rec["gemm"]
        monkeypatch.setattr(bench, "sources_sha256", as_recorded)
        t = bench.measured_traffic(wl, kind)
        assert t is not None and t > 0, (wl, kind)
        assert bench.measured_traffic(wl, "no_such_kind") is None
        monkeypatch.setattr(bench, "sources_sha256", lambda src: "0" * 64)
        assert bench.measured_traffic(wl, kind) is None, (wl, kind)
    assert bench.measured_traffic("no_such_workload", "up") is None
