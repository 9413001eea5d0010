"""Speculative KV coding on MI355X: lossless KV-cache compression with a HIP
range coder behind a C ABI (include/skv.h).  `skv` is the binding, `synth`
makes seeded synthetic caches."""
