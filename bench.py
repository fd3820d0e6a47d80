"""Throughput of the windowed-attention audio encoder on one MI355X.

A step is one pass of the whole forward path over one batch: waveform ->
log-mel (mt_logmel) -> conv front-end, 32 windowed-attention layers and the
encoder head (mt_encode).  The workload is 16 clips of 30 s of synthetic
16 kHz audio (sum of three tones plus noise, 20 % silent gaps), bf16-valued
weights, window 104 encoder frames.  The headline runs fp16 matrix operands
with fp32 accumulation: the 16-bit operand type that meets the parity bar on
every workload (bf16 activations miss it on the 32-clip adapter workload; the
bf16-operand throughput is reported beside it as `bf16_operands`).
Inputs are resident in device memory before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  `value` is encoder audio-seconds per second over the
median step of the K timed steps (each step bracketed by its own pair of HIP
events on the launch stream; no stage timer is armed meanwhile).
`roofline` describes the dominant kernel (the FFN up-projection GEMM with
fused bias + GELU), its launches timed with HIP events on the launch stream
in a separate pass of the same steps; `cpu_baseline` times the CPU oracle on
one clip of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0

# HBM traffic of one fc1 launch, from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE) of `bench.py --only headline --steps 1 --warmup 1
# --copy-probe`, each scaled by what the same counter read for the probe's
# 256 MiB device copy (profiles/encoder_16x30s_traffic.md).  Keyed by a hash
# of the GEMM kernel sources: after any change to them the figure is stale and
# reported as null.
FC1_TRAFFIC = {
    "3cf03dce31711dd5": {"fetch_KiB": 69949.6, "write_KiB": 72480.0,
                         "fetch_scale": 262144 / 131087.375, "write_scale": 262144 / 262144.0},
}


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "windowed_attention_audio_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def fc1_traffic_bytes():
    t = FC1_TRAFFIC.get(gemm_source_hash())
    if t is None:
        return None
    return round(1024 * (t["fetch_KiB"] * t["fetch_scale"] + t["write_KiB"] * t["write_scale"]))


def algorithmic_flops(geom, lens_T, window):
    """Multiply-add count x 2 of one forward pass (excluding the log-mel)."""
    C, D, F, O, A = (geom[k] for k in ("conv_ch", "d_model", "d_ffn", "d_out", "adapter_hidden"))
    L = geom["n_layers"]
    tot = dict(conv1=0, conv2=0, conv3=0, conv_out=0, qkv=0, attn=0, o=0, ffn=0, head=0, adapter=0)
    for T in lens_T:
        T1 = (T + 1) // 2
        T2 = (T1 + 1) // 2
        N = (T2 + 1) // 2
        tot["conv1"] += 2 * 9 * C * T1 * 64
        tot["conv2"] += 2 * 9 * C * C * T2 * 32
        tot["conv3"] += 2 * 9 * C * C * N * 16
        tot["conv_out"] += 2 * 16 * C * D * N
        tot["qkv"] += L * 2 * N * D * 3 * D
        tot["o"] += L * 2 * N * D * D
        tot["ffn"] += L * 2 * 2 * N * D * F
        ws = [min(window, N - s) for s in range(0, N, window)]
        tot["attn"] += L * sum(4 * w * w * D for w in ws)
        tot["head"] += 2 * N * D * (D + O)
        tot["adapter"] += 2 * N * O * 3 * A
    return tot


def cpu_baseline(clip, weights, geom, window, min_seconds=10.0, max_clips=4):
    """The oracle (NumPy float64) on whole clips of the workload, until about
    min_seconds of CPU time have passed."""
    import numpy as np  # noqa: F401
    from oracle import encoder as OE
    from oracle import logmel as OL
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] + [1])
        libs = [p for p in info if p.get("user_api") == "blas"]
        if libs:
            blas = "%s %s (%s)" % (libs[0].get("internal_api"), libs[0].get("version"),
                                   os.path.basename(libs[0].get("filepath", "")))
    except Exception:
        cores = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    P = OE.as_f64(weights)
    done, t0 = 0, time.perf_counter()
    while True:
        mel = OL.log_mel(clip)
        OE.encode_clip(mel, P, geom, window)
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or done >= max_clips:
            break
    audio = done * len(clip) / 16000.0
    return {"value": audio / el, "unit": "audio-s/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} x 30 s clip (clip 0 of the 16 x 30 s workload): log-mel + "
                      f"full encoder in NumPy float64, {el:.1f} s wall",
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(), "blas": blas}


def stream_measure(W, enc, synth, torch, np, chunks=(8, 32), reps=4):
    """mt_encode_stream on the 10-minute stream (window 104) with chunk_windows
    windows per chunk, against mt_logmel + mt_encode of the whole stream: time
    per encode and workspace bytes."""
    wl = synth.workload(3)
    wav = synth.make_clips(wl)[0]
    n = len(wav)
    dwav = torch.from_numpy(wav).cuda()
    T = W.mt_mel_frames(n)
    N = W.mt_encoder_frames(T)
    out = torch.empty((N, enc.d_out), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {"workload": wl.name, "audio_s": n / 16000.0,
           "peak_note": "peak_bytes: the most device memory torch held during the measurement "
                        "(waveform, output, workspaces; the library allocates none), packed "
                        "weights excluded (weights_bytes)",
           "weights_bytes": enc.packed.numel()}
    base = torch.cuda.memory_allocated()
    for cw in chunks:
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        nb = W.mt_encode_stream_workspace_size(enc, n, wl.window, cw)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        ms = timed(lambda: W.mt_encode_stream(enc, dwav, wl.window, cw, out=out, ws=ws,
                                              stream=stream))
        res[f"chunk{cw}"] = {"ms": round(ms, 3), "audio_s_per_s": round(n / 16000.0 / (ms * 1e-3), 1),
                             "workspace_bytes": nb,
                             "peak_bytes": torch.cuda.max_memory_allocated() - base + dwav.numel() * 4
                             + out.numel() * 4}
        del ws
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    mel = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    ws_m = torch.empty(W.mt_logmel_workspace_size([n]), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(W.mt_encode_workspace_size(enc, [T], wl.window), dtype=torch.uint8,
                       device="cuda")

    def whole():
        W.mt_logmel(dwav, [n], mel=mel, ws=ws_m, stream=stream)
        W.mt_encode(enc, mel, [T], wl.window, out=out, ws=ws_e, stream=stream)

    ms = timed(whole)
    res["whole"] = {"ms": round(ms, 3), "audio_s_per_s": round(n / 16000.0 / (ms * 1e-3), 1),
                    "workspace_bytes": ws_m.numel() + ws_e.numel() + mel.numel() * 4,
                    "peak_bytes": torch.cuda.max_memory_allocated() - base + dwav.numel() * 4
                    + out.numel() * 4}
    # live: the stream pushed in 1 s pieces as it "arrives" (each window
    # encoded once its samples are in), bounded state
    piece = 16000
    live_state = W.mt_stream_state_bytes(enc, wl.window, piece)
    lout = torch.empty((N, enc.d_out), dtype=torch.float32, device="cuda")

    def live():
        stl = W.LiveStream(enc, wl.window, piece)
        r = 0
        for i in range(0, n, piece):
            m = min(piece, n - i)
            got = stl.pending_frames(m)
            stl.push(dwav[i:i + m], out=lout[r:], stream=stream)
            r += got
        stl.finish(out=lout[r:], stream=stream)
        stl.close()

    live()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    live()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lms = e0.elapsed_time(e1)
    res["live_1s_pushes"] = {"ms": round(lms, 3), "audio_s_per_s": round(n / 16000.0 / (lms * 1e-3), 1),
                             "host_wall_ms": round(wall * 1e3, 3), "state_bytes": live_state,
                             "windows": (N + wl.window - 1) // wl.window,
                             "note": "one window (8.32 s of audio) encoded per call as soon as its samples "
                                     "are in; running-maximum log clamp"}
    # log-mel alone on the stream (the HBM-bound stage): per call, median of reps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(41)]
    for _ in range(5):
        W.mt_logmel(dwav, [n], mel=mel, ws=ws_m, stream=stream)
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(40):
        W.mt_logmel(dwav, [n], mel=mel, ws=ws_m, stream=stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(40))
    mel_ms = per[len(per) // 2]
    alg = 4 * n + 4 * 128 * T
    res["logmel"] = {"ms_median": round(mel_ms, 4), "algorithmic_bytes": alg,
                     "GBps": round(alg / (mel_ms * 1e-3) / 1e9, 1),
                     "frac_of_8TBps": round(alg / (mel_ms * 1e-3) / 8e12, 4)}
    return res


def splice_measure(W, frames, lens_T, synth, torch, np, vocab=151936, audio_token=151646, reps=20):
    """mt_prompt_embed: the 16 x 30 s batch's encoder frames spliced into 16
    ChatML-shaped prompts (one token sequence) with a [151936, 2048] fp16
    table; achieved GB/s (rows written + rows read)."""
    d = frames.shape[1]
    table = torch.randn((vocab, d), dtype=torch.float16, device="cuda")
    toks, rows = [], 0
    for i, t in enumerate(lens_T):
        nf = W.mt_encoder_frames(t)
        toks += synth.prompt_tokens(nf, vocab, audio_token, seed=100 + i)
        rows += nf
    out = torch.empty((len(toks), d), dtype=torch.float32, device="cuda")
    ws = torch.empty(W.mt_prompt_embed_workspace_size(len(toks)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    audio = frames[:rows]
    for _ in range(3):
        W.mt_prompt_embed(toks, table, audio, audio_token, out=out, ws=ws, stream=stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        W.mt_prompt_embed(toks, table, audio, audio_token, out=out, ws=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = len(toks) * d * 4 + rows * d * 4 + (len(toks) - rows) * d * 2
    del table
    return {"tokens": len(toks), "audio_rows": rows, "ms": round(ms, 4),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
            "note": "includes the host-side row map upload (kernel arguments)"}


def flops_2x(geom, lens_T):
    """Multiply-add count x 2 of one forward pass of the 2x-front-end encoder
    with full attention (excluding the log-mel)."""
    D, F, L = geom["d_model"], geom["d_ffn"], geom["n_layers"]
    tot = dict(conv1=0, conv2=0, qkv=0, attn=0, o=0, ffn=0)
    for T in lens_T:
        N = (T + 1) // 2
        tot["conv1"] += 2 * T * 3 * geom["n_mels"] * D
        tot["conv2"] += 2 * N * 3 * D * D
        tot["qkv"] += L * 2 * N * D * 3 * D
        tot["o"] += L * 2 * N * D * D
        tot["ffn"] += L * 2 * 2 * N * D * F
        tot["attn"] += L * 4 * N * N * D
    return tot


def measure_2x(W, synth, torch, wav, lens, lens_T, mel, ws_mel, steps=10, warmup=2):
    """The full-attention encoder with the 2x conv front-end at the 32 x 1280
    geometry (32 layers, 20 heads, FFN 5120) on the same 16 x 30 s batch: log-mel
    + encode per step, fp16 operands."""
    geom = synth.WHISPER_LARGE_GEOM
    weights = synth.make_weights(geom, bf16=True)
    dev_w = [torch.from_numpy(v).cuda() for v in weights.values()]
    enc = W.mt_encoder_create(W.encoder_config(geom, W.MT_F16), dev_w)
    torch.cuda.synchronize()
    del dev_w
    full = 1 << 30
    M = sum(W.mt_encoder_frames_for(W.MT_FRONTEND_CONV1D_2X, t) for t in lens_T)
    out = torch.empty((M, geom["d_model"]), dtype=torch.float32, device="cuda")
    ws = torch.empty(W.mt_encode_workspace_size(enc, lens_T, full), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        W.mt_logmel(wav, lens, mel=mel, ws=ws_mel, stream=stream)
        W.mt_encode(enc, mel, lens_T, full, out=out, ws=ws, stream=stream)

    for _ in range(warmup):
        step()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    stages = {}
    for st in ("mel16", "conv1", "conv2", "ln1", "qkv", "attn", "o", "ln2", "fc1", "fc2", "ln_post"):
        W.mt_trace_arm(st, max_launches=64)
        W.mt_trace_collect()
        step()
        torch.cuda.synchronize()
        t, _ = W.mt_trace_collect()
        stages[st] = round(t, 4)
    W.mt_trace_arm(None)
    fl = sum(flops_2x(geom, lens_T).values())
    enc.close()
    return {"workload": "16x30s_conv1d_2x_32x1280_full_attention", "encoder_frames": M,
            "ms_per_step": round(ms, 4), "audio_s_per_s": round(sum(lens) / 16000.0 / (ms * 1e-3), 1),
            "step_tflops": round(fl / (ms * 1e-3) / 1e12, 1), "breakdown_ms_per_step": stages}


def measure_varlen_adapter(W, synth, torch, np, weights, steps=5, warmup=2):
    """The 32-clip variable-length packed batch (durations uniform in 2-60 s,
    window 52) through the whole path with the SwiGLU adapter: audio-s/s of
    log-mel + encoder + head + adapter, and the adapter's two products
    (gate/up with the SwiGLU epilogue, down) against the MFMA peak."""
    wl = synth.workload(4)
    geom = synth.geom_for(wl)
    wts = synth.with_adapter(weights, geom, bf16=True)
    lens = wl.n_samples
    lens_T = [n // 160 for n in lens]
    dev_w = [torch.from_numpy(v).cuda() for v in wts.values()]
    enc = W.mt_encoder_create(W.encoder_config(geom, W.MT_F16), dev_w)
    torch.cuda.synchronize()
    del dev_w
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    wav = torch.from_numpy(np.concatenate(synth.make_clips(wl))).cuda()
    mel = torch.empty((sum(lens_T), 128), dtype=torch.float32, device="cuda")
    M = sum(W.mt_encoder_frames(t) for t in lens_T)
    out = torch.empty((M, geom["d_out"]), dtype=torch.float32, device="cuda")
    ws_mel = torch.empty(W.mt_logmel_workspace_size(lens), dtype=torch.uint8, device="cuda")
    ws_enc = torch.empty(W.mt_encode_workspace_size(enc, lens_T, wl.window), dtype=torch.uint8,
                         device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        W.mt_logmel(wav, lens, mel=mel, ws=ws_mel, stream=stream)
        W.mt_encode(enc, mel, lens_T, wl.window, out=out, ws=ws_enc, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    stage = {}
    for st in ("adapter_gu", "adapter_down"):
        W.mt_trace_arm(st, max_launches=8)
        W.mt_trace_collect()
        step()
        torch.cuda.synchronize()
        stage[st] = round(W.mt_trace_collect()[0], 4)
    W.mt_trace_arm(None)
    flops = algorithmic_flops(geom, lens_T, wl.window)
    ad_ms = stage["adapter_gu"] + stage["adapter_down"]
    res = {"workload": wl.name, "clips": len(lens), "audio_s": round(sum(lens) / 16000.0, 2),
           "window": wl.window, "encoder_frames": M, "ms_per_step": round(ms, 4),
           "audio_s_per_s": round(sum(lens) / 16000.0 / (ms * 1e-3), 1),
           "step_tflops": round(sum(flops.values()) / (ms * 1e-3) / 1e12, 1),
           "adapter_ms": stage,
           "adapter_tflops": round(flops["adapter"] / (ad_ms * 1e-3) / 1e12, 1),
           "adapter_frac": round(flops["adapter"] / (ad_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "peak_bytes": torch.cuda.max_memory_allocated() - base,
           "weights_bytes": enc.packed.numel(),
           "peak_note": "peak_bytes: the most device memory torch held for the workload "
                        "(waveform, log-mel, output, workspaces), packed weights excluded"}
    del enc, wav, mel, out, ws_mel, ws_enc
    torch.cuda.synchronize()
    return res


def measure_decoder(W, synth, torch, ctx=400, batches=(1, 16, 64), reps=20):
    """The language-model decoder step (Qwen3-1.7B geometry, bf16 weights,
    seeded N(0, 0.02^2) weights drawn on the device) over B sequences whose
    KV cache holds a ctx-position prompt: ms per step eager and as a replayed
    HIP graph, tokens/s, and HBM bytes per step (every weight once, the KV
    entries each row reads) against the 8 TB/s peak."""
    import numpy as np
    geom = synth.DEC_GEOM
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    dev = []
    for name, shape in synth.decoder_weight_names(geom):
        if len(shape) == 1:
            dev.append(1.0 + 0.1 * torch.randn(shape, generator=gen, device="cuda"))
        else:
            dev.append(torch.randn(shape, generator=gen, device="cuda") * (1.0 if name == "embed.weight" else 0.02))
    cfg = W.decoder_config(geom, W.MT_BF16)
    dec = W.mt_decoder_create(cfg, dev)
    torch.cuda.synchronize()
    del dev
    Bmax = max(batches)
    cache = torch.zeros(W.mt_decoder_cache_bytes(dec, Bmax, ctx + 8), dtype=torch.uint8, device="cuda")
    emb = W.mt_decoder_embedding(dec)
    # prompts: ctx positions of every sequence, one call per sequence
    for sq in range(Bmax):
        x = emb[torch.randint(0, geom["vocab"], (ctx,), generator=gen, device="cuda")].float()
        W.mt_decode(dec, x, [sq] * ctx, list(range(ctx)), cache, Bmax, ctx + 8)
    torch.cuda.synchronize()
    weight_bytes = 2 * sum(int(np.prod(s)) for n, s in synth.decoder_weight_names(geom) if len(s) > 1)
    kv_row = geom["n_layers"] * 2 * geom["n_kv_heads"] * geom["head_dim"] * 2  # bytes per cached position
    out = {"workload": "decode_step_qwen3_1.7b_bf16_ctx%d" % ctx, "weight_bytes": weight_bytes}
    for B in batches:
        x = emb[torch.randint(0, geom["vocab"], (B,), generator=gen, device="cuda")].float().contiguous()
        seq, pos = list(range(B)), [ctx] * B
        ws = torch.empty(W.mt_decode_workspace_size(dec, seq, pos, Bmax, ctx + 8), dtype=torch.uint8, device="cuda")
        logits = torch.empty((B, geom["vocab"]), dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream()

        def step():
            W.mt_decode(dec, x, seq, pos, cache, Bmax, ctx + 8, logits, nxt, ws, stream=torch.cuda.current_stream())

        for _ in range(3):
            step()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) / reps
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        ref = logits.clone()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(logits, ref))
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / reps
        nbytes = weight_bytes + B * (ctx + 1) * kv_row
        out["B%d" % B] = {"ms_eager": round(eager, 4), "ms_graph": round(gms, 4),
                          "tokens_per_s": round(B / (gms * 1e-3), 1), "hbm_bytes": nbytes,
                          "GBps": round(nbytes / (gms * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(nbytes / (gms * 1e-3) / 8e12, 4),
                          "graph_replay_equals_eager": same}
        del graph
    dec.close()
    return out


def timed_steps(torch, fn, stream, steps):
    """Runs fn() `steps` times, each bracketed by HIP events recorded on
    `stream`; returns (median ms, mean ms, per-step ms)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    srt = sorted(per)
    med = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
    return med, evs[0].elapsed_time(evs[-1]) / steps, per


def graph_replay(torch, fn, reps=50, warmup=10):
    """Captures fn() (launches on the current stream) into a HIP graph and
    times `reps` replays after `warmup`: (median ms, replay output equals the
    eager output bitwise) -- fn returns the output tensor."""
    stream = torch.cuda.current_stream()
    ref = fn().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref))
    med, _, _ = timed_steps(torch, g.replay, stream, reps)
    torch.cuda.synchronize()
    same = same and bool(torch.equal(out, ref))
    del g
    return med, same


def latency_single_clip(W, synth, torch, np, weights_bf16):
    """Time to a usable result for one clip: the 1 s clip with fp32 operands
    (its own fp32 weights) and the 30 s clip with fp16 operands; mt_logmel +
    mt_encode per call, eager and replayed as a HIP graph."""
    res = {}
    for cid, dt_name in ((0, "f32"), (1, "f16")):
        wl = synth.workload(cid)
        geom = synth.geom_for(wl)
        if dt_name == "f32":
            wts = synth.make_weights(geom, bf16=False)
            dt = W.MT_F32
        else:
            wts = weights_bf16
            dt = W.MT_F16
        dev_w = [torch.from_numpy(v).cuda() for v in wts.values()]
        enc = W.mt_encoder_create(W.encoder_config(geom, dt), dev_w)
        torch.cuda.synchronize()
        del dev_w
        wav = torch.from_numpy(synth.make_clips(wl)[0]).cuda()
        n = wav.numel()
        T = n // 160
        mel = torch.empty((T, 128), dtype=torch.float32, device="cuda")
        out = torch.empty((W.mt_encoder_frames(T), geom["d_out"]), dtype=torch.float32, device="cuda")
        ws_m = torch.empty(W.mt_logmel_workspace_size([n]), dtype=torch.uint8, device="cuda")
        ws_e = torch.empty(W.mt_encode_workspace_size(enc, [T], wl.window), dtype=torch.uint8, device="cuda")

        def call():
            s = torch.cuda.current_stream()
            W.mt_logmel(wav, [n], mel=mel, ws=ws_m, stream=s)
            W.mt_encode(enc, mel, [T], wl.window, out=out, ws=ws_e, stream=s)
            return out

        for _ in range(5):
            call()
        eager, _, _ = timed_steps(torch, call, torch.cuda.current_stream(), 30)
        gms, same = graph_replay(torch, call, reps=30)
        res[wl.name] = {"operands": dt_name, "ms_eager_median": round(eager, 4),
                        "ms_graph_median": round(gms, 4), "graph_equals_eager": same,
                        "audio_s_per_s_graph": round(n / 16000.0 / (gms * 1e-3), 1)}
        enc.close()
        del enc, wav, mel, out, ws_m, ws_e
        torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--operands", choices=["f16", "bf16"], default="f16")
    ap.add_argument("--only", choices=["2x", "decoder", "varlen", "headline", "mel"],
                    help="run only this measurement and print its JSON (for profiling)")
    ap.add_argument("--no-decoder", action="store_true",
                    help="skip the language-model decoder step")
    ap.add_argument("--no-2x", action="store_true",
                    help="skip the 2x-front-end full-attention workload")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the bounded-memory stream measurement (10-minute stream)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the 32-clip variable-length workload with the adapter")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the graph replay, bf16-operand and single-clip latency lines")
    ap.add_argument("--copy-probe", action="store_true",
                    help="before the steps, copy 256 MiB device-to-device once (a kernel of known "
                         "traffic, to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(clips are independent: a multi-GPU run is data-parallel with no "
              "collective, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import windowed_attention_audio_amd as W

    torch.cuda.set_device(0)
    wl = synth.workload(2)
    geom = synth.geom_for(wl)
    clips = synth.make_clips(wl)
    weights = synth.make_weights(geom, bf16=True)
    lens = wl.n_samples
    lens_T = [n // 160 for n in lens]
    window = wl.window

    dev_w = [torch.from_numpy(v).cuda() for v in weights.values()]
    op_dt = W.MT_F16 if args.operands == "f16" else W.MT_BF16
    enc = W.mt_encoder_create(W.encoder_config(geom, op_dt), dev_w)
    torch.cuda.synchronize()
    wav = torch.from_numpy(np.concatenate(clips)).cuda()
    mel = torch.empty((sum(lens_T), 128), dtype=torch.float32, device="cuda")
    M = sum(W.mt_encoder_frames(t) for t in lens_T)
    out = torch.empty((M, geom["d_out"]), dtype=torch.float32, device="cuda")
    ws_mel = torch.empty(W.mt_logmel_workspace_size(lens), dtype=torch.uint8, device="cuda")
    ws_enc = torch.empty(W.mt_encode_workspace_size(enc, lens_T, window), dtype=torch.uint8,
                         device="cuda")
    stream = torch.cuda.current_stream()

    def step_on(e, s):
        W.mt_logmel(wav, lens, mel=mel, ws=ws_mel, stream=s)
        W.mt_encode(e, mel, lens_T, window, out=out, ws=ws_enc, stream=s)
        return out

    def step():
        return step_on(enc, stream)

    if args.only == "2x":
        del dev_w
        print(json.dumps(measure_2x(W, synth, torch, wav, lens, lens_T, mel, ws_mel)), flush=True)
        return
    if args.only == "decoder":
        del dev_w
        print(json.dumps(measure_decoder(W, synth, torch)), flush=True)
        return
    if args.only == "varlen":
        del dev_w
        print(json.dumps(measure_varlen_adapter(W, synth, torch, np, weights)), flush=True)
        return
    if args.only == "mel":
        # the log-mel stage alone: the 16 x 30 s batch, then the 10-minute
        # stream, `steps` calls each after `warmup` (for counter profiles)
        del dev_w
        w3 = synth.make_clips(synth.workload(3))[0]
        wav3 = torch.from_numpy(w3).cuda()
        n3 = wav3.numel()
        mel3 = torch.empty((n3 // 160, 128), dtype=torch.float32, device="cuda")
        ws3 = torch.empty(W.mt_logmel_workspace_size([n3]), dtype=torch.uint8, device="cuda")
        res = {}
        for name, fn, alg in (
                ("16x30s", lambda: W.mt_logmel(wav, lens, mel=mel, ws=ws_mel, stream=stream),
                 4 * sum(lens) + 4 * 128 * sum(lens_T)),
                ("600s_stream", lambda: W.mt_logmel(wav3, [n3], mel=mel3, ws=ws3, stream=stream),
                 4 * n3 + 4 * 128 * (n3 // 160))):
            for _ in range(args.warmup):
                fn()
            med, _, _ = timed_steps(torch, fn, stream, args.steps)
            res[name] = {"ms_median": round(med, 4), "algorithmic_bytes": alg,
                         "GBps": round(alg / (med * 1e-3) / 1e9, 1)}
        print(json.dumps(res), flush=True)
        return

    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed steps: no stage timer armed
    ms, ms_mean, per_step = timed_steps(torch, step, stream, args.steps)

    audio_s = sum(lens) / 16000.0
    flops = algorithmic_flops(geom, lens_T, window)
    total_flops = sum(flops.values())
    if args.only == "headline":
        print(json.dumps({"ms_per_step": round(ms, 4), "value": round(audio_s / (ms * 1e-3), 2)}),
              flush=True)
        return

    # ---- fc1 (the roofline kernel): its launches timed in a separate pass
    fc1_steps = 5
    W.mt_trace_arm("fc1", max_launches=geom["n_layers"] * fc1_steps + 8)
    W.mt_trace_collect()
    for _ in range(fc1_steps):
        step()
    torch.cuda.synchronize()
    fc1_ms, fc1_n = W.mt_trace_collect()
    W.mt_trace_arm(None)
    fc1_flops = 2.0 * M * geom["d_ffn"] * geom["d_model"]
    fc1_avg = fc1_ms / max(fc1_n, 1)
    fc1_tflops = fc1_flops / (fc1_avg * 1e-3) / 1e12

    breakdown = {}
    if not args.no_breakdown:
        stages = ["mel", "mel_norm", "conv1", "conv2", "conv3", "conv_out", "ln1", "qkv", "attn",
                  "o", "ln2", "fc1", "fc2", "ln_post", "proj1", "proj2"]
        for st in stages:
            W.mt_trace_arm(st, max_launches=64)
            W.mt_trace_collect()
            step()
            torch.cuda.synchronize()
            t, n = W.mt_trace_collect()
            breakdown[st] = round(t, 4)
        W.mt_trace_arm(None)
        mel_bytes = 4 * sum(lens) + 4 * 128 * sum(lens_T)
        breakdown["mel_GBps"] = round(mel_bytes / ((breakdown["mel"] + breakdown["mel_norm"]) * 1e-3) / 1e9, 1)

    res = {
        "metric": "encoder audio-sec/sec (batch 16 x 30 s clips, bf16-valued weights, fp16 matrix "
                  "operands, fp32 accumulate); % of 16-bit MFMA peak",
        "value": round(audio_s / (ms * 1e-3), 2),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_min_max": [round(min(per_step), 4), round(max(per_step), 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.operands,
        "data": "synthetic (seeded tones + noise + silent gaps; seeded random weights)",
        "config": {"workload": wl.name.replace("bf16", "bf16w_%s_operands" % args.operands),
                   "clips": len(lens), "clip_seconds": 30, "window": window,
                   "weights": "bf16 values", "operands": args.operands, "accumulate": "f32",
                   "mel_frames": sum(lens_T), "encoder_frames": M, "layers": geom["n_layers"]},
        "mfma_frac": round(total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_tflops": round(total_flops / (ms * 1e-3) / 1e12, 1),
        "roofline": {"kernel": "fc1 (FFN up-projection GEMM + bias + GELU, M=%d N=%d K=%d)"
                               % (M, geom["d_ffn"], geom["d_model"]),
                     "bound": "mfma", "achieved": round(fc1_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fc1_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": fc1_traffic_bytes(), "avg_launch_ms": round(fc1_avg, 5),
                     "launches": fc1_n, "timing": "separate pass of %d steps" % fc1_steps,
                     "algorithmic_bytes": 2 * (M * geom["d_model"] + geom["d_ffn"] * geom["d_model"]
                                               + M * geom["d_ffn"])},
    }
    if breakdown:
        res["breakdown_ms_per_step"] = breakdown
        gemm_st = ["conv2", "conv3", "conv_out", "qkv", "attn", "o", "fc1", "fc2", "proj1", "proj2"]
        g_ms = sum(breakdown[s] for s in gemm_st)
        g_fl = sum(flops[k] for k in ("conv2", "conv3", "conv_out", "qkv", "attn", "o", "ffn", "head"))
        res["gemm_attn_frac"] = round(g_fl / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    if not args.no_extra:
        gms, same = graph_replay(torch, lambda: step_on(enc, torch.cuda.current_stream()), reps=50,
                                 warmup=10)
        res["graph_replay"] = {"ms_per_step_median": round(gms, 4), "replays": 50, "warmup": 10,
                               "audio_s_per_s": round(audio_s / (gms * 1e-3), 1),
                               "equals_eager": same}
        # the same batch with bf16 activations at the matrix cores
        enc_b = W.mt_encoder_create(W.encoder_config(geom, W.MT_BF16 if op_dt == W.MT_F16 else W.MT_F16),
                                    dev_w)
        torch.cuda.synchronize()
        for _ in range(5):
            step_on(enc_b, stream)
        bms, _, _ = timed_steps(torch, lambda: step_on(enc_b, stream), stream, 20)
        res["bf16_operands" if op_dt == W.MT_F16 else "f16_operands"] = {
            "ms_per_step_median": round(bms, 4), "audio_s_per_s": round(audio_s / (bms * 1e-3), 1),
            "mfma_frac": round(total_flops / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "parity": "bf16 activations: within the bar on the 16 x 30 s batch and the 10-minute "
                      "stream, outside it (max|d|/RMS > 0.02) on the 32-clip adapter workload"}
        enc_b.close()
        del enc_b
    del dev_w
    torch.cuda.synchronize()
    if not args.no_extra:
        res["single_clip_latency"] = latency_single_clip(W, synth, torch, np, weights)
    if not args.no_stream:
        res["stream_10min"] = stream_measure(W, enc, synth, torch, np)
        res["prompt_splice"] = splice_measure(W, out, lens_T, synth, torch, np)
    if not args.no_varlen:
        res["varlen_adapter"] = measure_varlen_adapter(W, synth, torch, np, weights)
    if not args.no_2x:
        res["conv1d_2x_16x30s"] = measure_2x(W, synth, torch, wav, lens, lens_T, mel, ws_mel)
    if not args.no_decoder:
        res["decoder_step"] = measure_decoder(W, synth, torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(clips[0], weights, geom, window)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
