"""MI355X-native (gfx950) compressed sparse attention (CSA) and heavily
compressed attention (HCA), prefill and decode, over a paged compressed cache.

  binding   -- ctypes binding of libcsahca.so (the HIP library, include/csahca.h);
               importing it fails loudly if the library is not built
  layers    -- per-layer orchestration of the library calls (prefill, decode step)
  configs   -- the workload presets
  synth     -- seeded synthetic inputs (random draws only)
  build     -- compiles csrc/*.hip for gfx950 into libcsahca.so
"""
