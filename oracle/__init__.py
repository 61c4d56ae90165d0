"""Float64 CPU oracle of the Thinformer / Thinformer Express attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never calls it and
shares no code with it: no kernels, helpers, tables or constant generators.

What is defined here, and where the definition comes from:

* ``philox``      counter-based uniforms, Philox4x64-10 as published by Salmon,
                  Moraes, Dror and Shaw ("Parallel random numbers: as easy as
                  1, 2, 3", SC'11).  Pinned against NumPy's ``Philox`` bit
                  generator, an independent library implementation.
* ``kernel_halving``  the key-value attention kernel kappa_att and one kernel
                  halving (self-balancing walk) pass.  Named on "Express
                  Language Modeling", section "Thinformer Express"; the walk
                  itself follows the published kernel-thinning papers
                  (Dwivedi and Mackey, "Kernel Thinning"; Shetty, Dwivedi and
                  Mackey, "Distribution Compression in Near-linear Time").
* ``compress``    the unmasked (Thinformer) coreset: a recursive four-way
                  split with one halving at every merge.
* ``express``     the causal EXPRESS weighted cache (exact, thin, HALVE
                  phases), "Express Language Modeling", section
                  "Methodology / The EXPRESS Meta-Procedure".
* ``attention``   weighted-coreset softmax attention, exact attention
                  (written separately) and the error metrics.
* ``forward``     the whole path as the library exposes it, including GQA,
                  sampled outputs and the replay of another implementation's
                  halving decisions.

All arithmetic is float64; inputs are upcast exactly from float32 / bfloat16.
Parity status of each function is stated in its docstring; "parity unpinned"
marks results that no page, closed form or library routine fixes.
"""
