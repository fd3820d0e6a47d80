"""GPU parity of the language-model decoder step against the oracle
(oracle.decoder), through the C ABI.

  * a small geometry (d 256, 4/2 heads of 128, FFN 512, vocab 1024, 2 layers),
    fp16 and bf16: a 37-row prompt in one call (tiled products), then single
    rows (skinny matrix-vector kernels) continuing it; a 9-row prompt on the
    skinny path; three sequences of different lengths in one call, then one
    decode step with a row each; a 600-row prompt and decode steps past it
    (attention over three 256-key chunks);
  * the card's full width (d 2048, 16/8 heads, FFN 6144, vocab 151 936) with
    two layers: prompt + decode steps against the oracle, and a 3-row step of
    three sequences (up to four rows the output and down projections compute
    their input -- the attention combine, SwiGLU -- themselves);
  * the card's 28 layers: a 16-row decode step equals each row alone
    (bitwise), and argmax equals the host's argmax of the returned logits;
  * steps with one row per sequence (queries and the new key / value computed
    inside the attention kernel) equal two rows of one sequence in one call
    (separate Q/K-norm pass), bitwise.
Logits are compared row by row: cosine >= 0.999 and max |diff| <= 0.02 RMS.
"""

import sys

import numpy as np
import pytest

import synth
from oracle import decoder as OD
from tests.helpers import assert_bf16_rows

pytestmark = pytest.mark.gpu

SMALL = dict(vocab=1024, d_model=256, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=128, d_ffn=512)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class GpuDecoder:
    def __init__(self, geom, weights, dt_name, max_seqs, max_pos):
        import torch
        import windowed_attention_audio_amd as W
        self.W = W
        self.geom = geom
        dt = W.MT_F16 if dt_name == "f16" else W.MT_BF16
        self.cfg = W.decoder_config(geom, dt)
        dev = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in weights.values()]
        self.dec = W.mt_decoder_create(self.cfg, dev)
        torch.cuda.synchronize()
        del dev
        self.max_seqs, self.max_pos = max_seqs, max_pos
        self.cache = torch.zeros(W.mt_decoder_cache_bytes(self.dec, max_seqs, max_pos), dtype=torch.uint8,
                                 device="cuda")

    def step(self, x, seq, pos):
        import torch
        xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        logits, nxt = self.W.mt_decode(self.dec, xt, seq, pos, self.cache, self.max_seqs, self.max_pos)
        torch.cuda.synchronize()
        return logits.cpu().numpy(), nxt.cpu().numpy()


def check_logits(gpu, ref, nxt, what):
    r = assert_bf16_rows(gpu, ref, what=what)
    assert np.array_equal(nxt, np.argmax(gpu, axis=1)), f"{what}: argmax differs from the returned logits"
    return r


@pytest.fixture(scope="module")
def small_w():
    return synth.make_decoder_weights(SMALL, bf16=True, seed=31)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_small_prompt_then_decode(small_w, dt):
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    toks = np.random.default_rng(1).integers(0, SMALL["vocab"], 42)
    x = OD.embed(toks, P)
    g = GpuDecoder(SMALL, small_w, dt, 2, 64)
    cache = OD.empty_cache(SMALL)
    say(f"decoder small {dt}: 37-row prompt (tiled path)")
    gl, nx = g.step(x[:37], [1] * 37, list(range(37)))
    check_logits(gl, OD.forward(x[:37], P, SMALL, cache), nx, "prompt")
    for i in range(37, 42):
        gl, nx = g.step(x[i:i + 1], [1], [i])
        r = check_logits(gl, OD.forward(x[i:i + 1], P, SMALL, cache), nx, f"decode pos {i}")
    say(f"  last step: cos {r['cos'].min():.6f} worst {r['maxabs_rms'].max():.4f}")


def test_small_short_prompt_on_skinny_path(small_w):
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    toks = np.random.default_rng(2).integers(0, SMALL["vocab"], 9)
    x = OD.embed(toks, P)
    g = GpuDecoder(SMALL, small_w, "f16", 1, 32)
    say("decoder small: 9-row prompt (skinny path)")
    gl, nx = g.step(x, [0] * 9, list(range(9)))
    check_logits(gl, OD.forward(x, P, SMALL, OD.empty_cache(SMALL)), nx, "9-row prompt")


def test_small_three_sequences(small_w):
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    lens = [10, 20, 5]
    rng = np.random.default_rng(3)
    xs = [OD.embed(rng.integers(0, SMALL["vocab"], n + 1), P) for n in lens]
    g = GpuDecoder(SMALL, small_w, "bf16", 4, 64)
    slots = [3, 0, 2]
    x = np.concatenate([xi[:n] for xi, n in zip(xs, lens)])
    seq = sum(([s] * n for s, n in zip(slots, lens)), [])
    pos = sum((list(range(n)) for n in lens), [])
    say("decoder small: 3 prompts in one call, then one step each")
    gl, nx = g.step(x, seq, pos)
    caches = [OD.empty_cache(SMALL) for _ in lens]
    ref = np.concatenate([OD.forward(xi[:n], P, SMALL, c) for xi, n, c in zip(xs, lens, caches)])
    check_logits(gl, ref, nx, "3 prompts")
    gl, nx = g.step(np.stack([xi[n] for xi, n in zip(xs, lens)]), slots, lens)
    ref = np.concatenate([OD.forward(xi[n:n + 1], P, SMALL, c) for xi, n, c in zip(xs, lens, caches)])
    check_logits(gl, ref, nx, "3 decode rows")


def test_fused_qk_equals_separate_pass(small_w):
    """With one row per sequence the attention kernel computes the queries and
    the new key / value itself; two rows of one sequence in one call take the
    separate Q/K-norm pass (the second row attends to the first one's new
    entry).  The same two rows in two calls must give the same bits."""
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    x = OD.embed(np.random.default_rng(6).integers(0, SMALL["vocab"], 12), P)
    say("decoder small: 2 rows of one sequence in one call vs two calls")
    ga = GpuDecoder(SMALL, small_w, "bf16", 1, 64)
    gb = GpuDecoder(SMALL, small_w, "bf16", 1, 64)
    ga.step(x[:10], [0] * 10, list(range(10)))
    gb.step(x[:10], [0] * 10, list(range(10)))
    la, na = ga.step(x[10:12], [0, 0], [10, 11])
    lb0, nb0 = gb.step(x[10:11], [0], [10])
    lb1, nb1 = gb.step(x[11:12], [0], [11])
    assert np.array_equal(la[0], lb0[0]) and np.array_equal(la[1], lb1[0])
    assert na[0] == nb0[0] and na[1] == nb1[0]


def test_small_long_context(small_w):
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    toks = np.random.default_rng(4).integers(0, SMALL["vocab"], 603)
    x = OD.embed(toks, P)
    g = GpuDecoder(SMALL, small_w, "f16", 1, 1024)
    cache = OD.empty_cache(SMALL)
    say("decoder small: 600-row prompt, 3 decode steps (3 key chunks)")
    gl, nx = g.step(x[:600], [0] * 600, list(range(600)))
    ref = OD.forward(x[:600], P, SMALL, cache)
    check_logits(gl[::37], ref[::37], nx[::37], "600-row prompt (sampled rows)")
    for i in range(600, 603):
        gl, nx = g.step(x[i:i + 1], [0], [i])
        check_logits(gl, OD.forward(x[i:i + 1], P, SMALL, cache), nx, f"decode pos {i}")


def test_full_width_two_layers():
    geom = dict(synth.DEC_GEOM, n_layers=2)
    say("decoder full width, 2 layers: weights")
    w = synth.make_decoder_weights(geom, bf16=True, seed=5)
    P = {k: v.astype(np.float64) for k, v in w.items()}
    toks = np.random.default_rng(5).integers(0, geom["vocab"], 22)
    x = OD.embed(toks, P)
    g = GpuDecoder(geom, w, "f16", 1, 64)
    cache = OD.empty_cache(geom)
    say("  20-row prompt, 2 decode steps")
    gl, nx = g.step(x[:20], [0] * 20, list(range(20)))
    check_logits(gl, OD.forward(x[:20], P, geom, cache), nx, "full-width prompt")
    for i in (20, 21):
        gl, nx = g.step(x[i:i + 1], [0], [i])
        r = check_logits(gl, OD.forward(x[i:i + 1], P, geom, cache), nx, f"full-width decode {i}")
    say(f"  cos {r['cos'].min():.6f} worst {r['maxabs_rms'].max():.4f}")


def test_full_width_three_rows_fused_products():
    """At most four rows the output and down projections compute their input
    (the attention combine, SwiGLU) inside the product; at full width both
    apply.  Three sequences, then one 3-row step, against the oracle."""
    geom = dict(synth.DEC_GEOM, n_layers=2)
    say("decoder full width, 2 layers: 3 prompts, then a 3-row step")
    w = synth.make_decoder_weights(geom, bf16=True, seed=9)
    P = {k: v.astype(np.float64) for k, v in w.items()}
    lens = [7, 70, 2]  # 1, 2 and 1 chunks of 64 keys at the step
    rng = np.random.default_rng(9)
    xs = [OD.embed(rng.integers(0, geom["vocab"], n + 1), P) for n in lens]
    g = GpuDecoder(geom, w, "f16", 3, 128)
    slots = [1, 2, 0]
    caches = [OD.empty_cache(geom) for _ in lens]
    for xi, n, c, sl in zip(xs, lens, caches, slots):
        g.step(xi[:n], [sl] * n, list(range(n)))
        OD.forward(xi[:n], P, geom, c)
    gl, nx = g.step(np.stack([xi[n] for xi, n in zip(xs, lens)]), slots, lens)
    ref = np.concatenate([OD.forward(xi[n:n + 1], P, geom, c) for xi, n, c in zip(xs, lens, caches)])
    r = check_logits(gl, ref, nx, "3-row step")
    say(f"  cos {r['cos'].min():.6f} worst {r['maxabs_rms'].max():.4f}")


def test_full_geometry_batch_equals_single():
    import torch
    geom = synth.DEC_GEOM
    say("decoder 28 layers: weights")
    w = synth.make_decoder_weights(geom, bf16=True, seed=6)
    g = GpuDecoder(geom, w, "bf16", 16, 128)
    emb = w["embed.weight"]
    rng = np.random.default_rng(6)
    # 16 sequences with prompts of 3..18 rows in one call, then a 16-row step
    lens = [3 + i for i in range(16)]
    x = np.concatenate([emb[rng.integers(0, geom["vocab"], n)] for n in lens])
    seq = sum(([s] * n for s, n in enumerate(lens)), [])
    pos = sum((list(range(n)) for n in lens), [])
    say("  16 prompts in one call")
    g.step(x, seq, pos)
    snap = g.cache.clone()
    step_x = emb[rng.integers(0, geom["vocab"], 16)]
    say("  16-row decode step vs each row alone")
    gl, nx = g.step(step_x, list(range(16)), lens)
    assert np.isfinite(gl).all()
    for s in (0, 7, 15):
        g.cache.copy_(snap)
        l1, n1 = g.step(step_x[s:s + 1], [s], [lens[s]])
        assert np.array_equal(l1[0], gl[s]), f"row {s}"
        assert n1[0] == nx[s]
    torch.cuda.synchronize()


def test_decode_step_graph_replays_match_eager(small_w):
    """The decode step captured in a HIP graph (as the benchmark times it):
    every replay, with eager work between replays, equals the eager step."""
    import torch
    import windowed_attention_audio_amd as W
    g = GpuDecoder(SMALL, small_w, "bf16", 4, 64)
    rng = np.random.default_rng(8)
    emb = small_w["embed.weight"]
    g.step(emb[rng.integers(0, SMALL["vocab"], 40)], sum(([s] * 10 for s in range(4)), []), list(range(10)) * 4)
    x = torch.from_numpy(np.ascontiguousarray(emb[rng.integers(0, SMALL["vocab"], 4)])).cuda()
    seq, pos = [0, 1, 2, 3], [10] * 4
    ws = torch.empty(W.mt_decode_workspace_size(g.dec, seq, pos, 4, 64), dtype=torch.uint8, device="cuda")
    logits = torch.empty((4, SMALL["vocab"]), dtype=torch.float32, device="cuda")
    nxt = torch.empty(4, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        W.mt_decode(g.dec, x, seq, pos, g.cache, 4, 64, logits, nxt, ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = logits.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        W.mt_decode(g.dec, x, seq, pos, g.cache, 4, 64, logits, nxt, ws,
                    stream=torch.cuda.current_stream())
    for i in range(3):
        logits.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, eager), f"replay {i}"
        _ = (x * 2.0).sum().item()  # eager work between replays


def test_zero_layer_decoder_is_the_tied_head(small_w):
    geom = dict(SMALL, n_layers=0)
    w = {k: v for k, v in small_w.items() if not k.startswith("layers.")}
    P = {k: v.astype(np.float64) for k, v in w.items()}
    x = OD.embed(np.arange(5) * 100, P)
    g = GpuDecoder(geom, w, "f16", 1, 8)
    gl, nx = g.step(x, [0] * 5, list(range(5)))
    check_logits(gl, OD.forward(x, P, geom, OD.empty_cache(geom)), nx, "0-layer")


def test_decode_rejections(small_w):
    import torch
    import windowed_attention_audio_amd as W
    g = GpuDecoder(SMALL, small_w, "bf16", 2, 16)
    x = torch.zeros((2, SMALL["d_model"]), dtype=torch.float32, device="cuda")
    for seq, pos, what in (([0, 0], [3, 3], "duplicate (seq, pos)"), ([0, 2], [0, 0], "seq >= max_seqs"),
                           ([0, 1], [0, 16], "pos >= max_pos"), ([0, -1], [0, 0], "negative seq")):
        with pytest.raises(W.MtError) as e:
            W.mt_decode(g.dec, x, seq, pos, g.cache, 2, 16)
        assert e.value.status == W.MT_ERR_INVALID_ARG, what
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(W.MtError) as e:
        W.mt_decode(g.dec, x, [0, 1], [0, 0], g.cache, 2, 16, ws=ws)
    assert e.value.status == W.MT_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_small_wide_decode_batch(small_w):
    """40 sequences: 3-row prompts in one call (tiled path), then a 40-row
    decode step (skinny path, three 16-row tiles sharing weight fragments):
    the oracle per sequence, and bitwise equality with a one-row step."""
    P = {k: v.astype(np.float64) for k, v in small_w.items()}
    B = 40
    rng = np.random.default_rng(9)
    xs = [OD.embed(rng.integers(0, SMALL["vocab"], 4), P) for _ in range(B)]
    g = GpuDecoder(SMALL, small_w, "bf16", B, 8)
    say("decoder small: 40 prompts of 3 rows, then a 40-row step")
    g.step(np.concatenate([x[:3] for x in xs]), sum(([s] * 3 for s in range(B)), []), [0, 1, 2] * B)
    snap = g.cache.clone()
    gl, nx = g.step(np.stack([x[3] for x in xs]), list(range(B)), [3] * B)
    caches = [OD.empty_cache(SMALL) for _ in range(B)]
    for s in range(B):
        OD.forward(xs[s][:3], P, SMALL, caches[s])
    ref = np.concatenate([OD.forward(xs[s][3:4], P, SMALL, caches[s]) for s in range(B)])
    check_logits(gl, ref, nx, "40-row step")
    g.cache.copy_(snap)
    l1, n1 = g.step(xs[17][3:4], [17], [3])
    assert np.array_equal(l1[0], gl[17]) and n1[0] == nx[17]
