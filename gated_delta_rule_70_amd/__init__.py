"""Gated delta rule for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of include/gdr.h
(``libgdr.so`` in this directory, built by ``python -m gated_delta_rule_70_amd.build``).
``chunk_fwd`` and ``decode_step`` are its Python binding (``binding.py``); ``inputs`` holds
the seeded synthetic workloads.
"""

_BINDING = ("chunk_fwd", "decode_step", "selftest_mfma", "GdrError")


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
