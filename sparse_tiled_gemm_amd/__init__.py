"""MI355X (gfx950) tiled GEMM D = A*B + C with a fused epilogue and a 2:4
structured-sparse-A variant.  The compute path is the HIP library
libstgemm.so behind the C ABI in include/gemm.h; `gemm` is its binding."""
