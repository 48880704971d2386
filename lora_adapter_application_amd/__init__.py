"""MI355X (gfx950) multi-adapter LoRA apply path.

The product is the C-ABI library ``liblora_mi355x.so`` (``include/lora_mi355x.h``),
built from ``csrc/`` by ``build.py``.  ``binding`` is its ctypes binding;
``synth`` draws seeded synthetic inputs; ``lru`` is the host-side slot-residency
driver used by the churn benchmark.  Importing the package loads nothing: the
library is loaded on first use and its absence raises.
"""
