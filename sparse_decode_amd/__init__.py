"""MI355X-native KV-cache compression hot path: window scoring, top-k selection,
compacting gather and GQA decode attention as hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/kvc.h``.

``sparse_decode_amd.kvc`` is the thin Python binding of that library (argument
marshalling only); ``sparse_decode_amd.synth`` draws seeded synthetic inputs.
Submodules are imported on demand so that drawing inputs never loads the GPU
library.
"""

__all__ = ["kvc", "synth"]
