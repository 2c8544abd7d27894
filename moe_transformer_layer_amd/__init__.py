"""One DeepSeek-V4.1-style decode layer (M <= 48 rows) as one persistent HIP
launch on MI355X (gfx950).

Submodules:
  dsl    -- ctypes binding of the C ABI in include/dsl.h (libdsl.so, built in-tree)
  synth  -- seeded synthetic inputs in the layer's stored formats
The binding is imported on demand so that synth stays usable without the
shared library.
"""
