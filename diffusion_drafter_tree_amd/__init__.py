"""MI355X-native DARTree draft-tree construction round.

The hot path is hand-written HIP for gfx950 behind a C ABI (libdartree.so).
``ops`` is the thin torch-facing binding; ``inputs`` draws seeded synthetic
rounds. Importing the package does not load the library; the first call
into ``ops`` does, and fails loudly when it is missing.
"""
__all__ = ["inputs", "ops"]
