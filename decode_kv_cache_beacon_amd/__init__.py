"""MI355X-native decode-time KV-cache eviction pass (BeaconKV hot path).

Submodules:
  beaconkv -- ctypes binding of the C-ABI library libbeaconkv.so (HIP kernels
              for gfx950); importing it fails loudly if the library is absent.
  synth    -- seeded synthetic inputs shaped like the pages' workloads.
  build    -- compiles the HIP library in-tree with hipcc.
"""
__all__ = ["beaconkv", "synth", "build"]
