"""MI355X-native InfiniGen decode hot path: HIP kernels behind a C ABI (include/ig.h)."""
