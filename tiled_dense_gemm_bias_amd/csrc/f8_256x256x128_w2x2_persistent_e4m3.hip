// 8-bit-input GEMM instances (gemm_f8.hpp), E4M3 operands: fp16 / bf16 bias and
// output x six activations.
#include "gba_registry.hpp"

GBA_F8_ENTRY(f8_e4m3, 0)
