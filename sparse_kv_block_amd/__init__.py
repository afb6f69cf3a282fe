"""MI355X-native look-ahead sparse decode step (OasisKV-style) for gfx950.

Submodules:
  configs  workload shapes
  gen      seeded synthetic inputs (no method arithmetic)
  lib      thin ctypes binding over the C-ABI library liboasis.so
  build    compiles the HIP sources into liboasis.so
"""
