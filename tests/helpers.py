"""Shared helpers of the test-suite: tolerances and GPU-side runners.

Tolerances (the parity bar of this encoder):
  log-mel            max |gpu - oracle| <= 1e-4 over every valid entry
  fp32 encoder       per row ||gpu - ref|| / ||ref|| <= 1e-3
  16-bit encoder     per row cosine >= 0.999 and max |gpu - ref| <= 0.02 * RMS(ref row)
                     (bf16-valued weights; matrix operands fp16 or bf16)
Padded rows must be exactly zero.
"""

import numpy as np

MEL_TOL = 1e-4
F32_REL_TOL = 1e-3
BF16_COS = 0.999
BF16_MAXABS_RMS = 0.02


def row_metrics(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = gpu - ref
    nref = np.linalg.norm(ref, axis=1)
    rel = np.linalg.norm(d, axis=1) / np.maximum(nref, 1e-30)
    cos = (gpu * ref).sum(1) / np.maximum(np.linalg.norm(gpu, axis=1) * nref, 1e-30)
    rms = nref / np.sqrt(ref.shape[1])
    maxabs_rms = np.abs(d).max(axis=1) / np.maximum(rms, 1e-30)
    return dict(rel=rel, cos=cos, maxabs_rms=maxabs_rms)


def assert_f32_rows(gpu, ref, tol=F32_REL_TOL, what=""):
    m = row_metrics(gpu, ref)
    worst = m["rel"].max()
    assert worst <= tol, f"{what}: worst per-row relative L2 {worst:.3e} > {tol:.1e}"
    return m


def assert_bf16_rows(gpu, ref, what=""):
    m = row_metrics(gpu, ref)
    cmin = m["cos"].min()
    amax = m["maxabs_rms"].max()
    assert cmin >= BF16_COS, f"{what}: min per-row cosine {cmin:.6f} < {BF16_COS}"
    assert amax <= BF16_MAXABS_RMS, f"{what}: max |diff| / RMS {amax:.4f} > {BF16_MAXABS_RMS}"
    return m


class GpuModel:
    """Weights on the device plus an encoder handle, built once per geometry."""

    def __init__(self, geom, dtype_name, weights: dict, with_head=True):
        import torch
        import windowed_attention_audio_amd as W
        self.W = W
        self.geom = geom
        self.dt = {"bf16": W.MT_BF16, "f16": W.MT_F16, "f32": W.MT_F32}[dtype_name]
        self.cfg = W.encoder_config(geom, self.dt, with_head=with_head)
        self.dev_weights = [torch.from_numpy(np.ascontiguousarray(v)).cuda()
                            for v in weights.values()]
        self.enc = W.mt_encoder_create(self.cfg, self.dev_weights)
        torch.cuda.synchronize()
        # the source tensors may be dropped once create() has finished
        self.dev_weights = None

    def encode(self, mel_list, window, layout=0):
        import torch
        W = self.W
        lens = [m.shape[0] for m in mel_list]
        if layout == W.MT_PACKED:
            mel = torch.from_numpy(np.concatenate(mel_list).astype(np.float32)).cuda()
        else:
            tmax = max(lens)
            arr = np.zeros((len(lens), tmax, 128), np.float32)
            for i, m in enumerate(mel_list):
                arr[i, :m.shape[0]] = m
            mel = torch.from_numpy(arr).cuda()
        out = W.mt_encode(self.enc, mel, lens, window, layout=layout)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def split_rows(packed: np.ndarray, ns):
    out, r = [], 0
    for n in ns:
        out.append(packed[r:r + n])
        r += n
    return out


def gpu_logmel(wavs, layout=0):
    import torch
    import windowed_attention_audio_amd as W
    lens = [len(w) for w in wavs]
    if layout == W.MT_PACKED:
        wav = torch.from_numpy(np.concatenate(wavs).astype(np.float32)).cuda()
    else:
        arr = np.zeros((len(wavs), max(lens)), np.float32)
        for i, w in enumerate(wavs):
            arr[i, :len(w)] = w
        wav = torch.from_numpy(arr).cuda()
    mel = W.mt_logmel(wav, lens, layout=layout)
    torch.cuda.synchronize()
    return mel.cpu().numpy()
