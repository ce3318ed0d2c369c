"""tp_vocab_logits_amd -- the one-shot Lamport-mailbox gather of vocab-parallel
lm_head logits, built for MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (``include/hg.h``,
``libhg.so``); this package is the thin Python binding over it. Importing the
package loads nothing: :class:`HeadGather` and :mod:`._lib` load the shared
library on first use and raise if it is missing -- there is no fallback path.
"""

import importlib

__all__ = ["HeadGather", "HgError", "lib", "synthetic"]

_LAZY = {"HeadGather": ("head_gather", "HeadGather"), "HgError": ("_lib", "HgError"),
         "lib": ("_lib", None), "synthetic": ("synthetic", None)}


def __getattr__(name):
    if name not in _LAZY:
        raise AttributeError(name)
    module, attr = _LAZY[name]
    mod = importlib.import_module(f"{__name__}.{module}")
    return mod if attr is None else getattr(mod, attr)
