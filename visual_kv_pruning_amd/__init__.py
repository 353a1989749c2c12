"""svlm: MI355X-native (gfx950) hot path of verifier-guided visual-token / KV
selection and draft/verify decode attention for lossless speculative decoding
of video LLMs.

The compute lives in libsvlm.so (hand-written HIP, C ABI in include/svlm.h);
``visual_kv_pruning_amd.ops`` holds thin torch-facing wrappers.  Importing the
package does not load the library; the first call does, and fails loudly if
it is missing.
"""
from . import _lib  # noqa: F401
