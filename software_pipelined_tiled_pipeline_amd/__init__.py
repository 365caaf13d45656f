"""pgemm: software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950)."""
