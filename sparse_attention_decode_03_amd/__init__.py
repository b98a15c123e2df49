"""MI355X-native DSA decode hot path: lightning-indexer scores, exact top-k
selection and FP8 paged NoPE-MLA gather-attend, as hand-written HIP kernels for
gfx950 behind a C ABI (include/dsa.h). `dsa` is the thin ctypes binding;
`workloads` draws the seeded synthetic inputs."""
