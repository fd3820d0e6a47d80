"""CPU oracle for the audio-encoder forward pass.  TEST INFRASTRUCTURE ONLY.

Plain, slow NumPy float64 code written from the pages' description of the
model (the model card "MOSS-Transcribe-preview-2B-GGUF": Architecture table,
"Implementation notes (correctness)" and the gotcha list).  It shares no code
with the HIP library and imports nothing from it; only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may call it.

Modules
  logmel   waveform -> normalised log-mel frames
  encoder  log-mel -> encoder frames (conv front-end, windowed-attention
           tower, head, optional SwiGLU adapter)
  encoder2x  log-mel -> encoder frames of the full-attention variant with a
             2x time-downsampling front-end (page "CrisperWhisper -> ONNX
             (with cross-attentions)": whisper geometries)
  live     one long stream encoded window by window as its audio arrives
           (the clip maximum of the log clamp read as a causal running
           maximum)
  prompt   adapter frames spliced into the prompt's token embeddings
  decoder  the language-model decoder (Qwen3-1.7B geometry) over a KV cache

Every function below is pinned by tests under ``tests/`` that check it against
closed forms, invariants, brute force, or an independent library routine.
"""

from . import logmel, encoder, encoder2x, live, prompt, decoder  # noqa: F401
