"""BPT (Blockwise Parallel Transformer) layer forward for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``); ``bpt`` is its thin Python binding. ``synth`` draws seeded inputs and
``accounting`` holds the FLOP and memory formulas.
"""
