"""f64 CPU oracle for the chunked streaming DiT denoising step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it.

Source: HeyGen, "Avatar inference at scale".  The model architecture section
says the generator is a diffusion transformer trained with flow matching and
conditioned on rich reference tokens.  The pipeline loop section says the
reference is encoded once per request, and that the audio-to-video stage runs
a multi-step diffusion pass conditioned on the previous chunk's boundary frames.
The pages give no block internals, so every constant below (norm type, RoPE
split, modulation order, GELU form, schedule) is a stated reading, chosen as the
plainest one consistent with them.

The boundary continuity section adds interpolation (I) chunks between ordinary
N-chunks, anchored on the neighbouring N-chunks' frames (anchor_context,
interp_stream).

Parity status: every function is pinned by a CPU test (brute-force attention,
softmax normalisation, masked-joint vs cached-KV equivalence with and without
the interpolation anchor, chunked == unchunked, closed-form Euler,
constant-velocity model, uniform attention, RoPE and RMSNorm identities,
zero-gate identity, key-permutation and time-shift invariance).  Against
the pages themselves parity is unpinned: they print no values.
"""
from .dit import *  # noqa: F401,F403
