"""MI355X-native chunked streaming DiT denoising step (gfx950 HIP kernels + C ABI).

The compute lives in libditchunk.so (built by chunked_streaming_dit_amd.build); this
package is its ctypes binding.  The first call into it loads the library and raises
if it is missing: there is no fallback path.
"""
from ._lib import DitError, lib  # noqa: F401
from .dit import AUDIO_HELD, ChunkConfig, DitChunk, fm_euler_step, fm_noise_to, grid, ops, torch_dtype  # noqa: F401
