"""MI355X-native hot path of the Tessera potential: Hilbert-ordered neighbour rebuild and
equivariant-attention energy/forces, as HIP kernels behind the C ABI in include/tess.h.

Submodules: ``tess`` (ctypes binding of libtess.so), ``workloads`` (seeded synthetic
inputs), ``build`` (hipcc build of libtess.so)."""
