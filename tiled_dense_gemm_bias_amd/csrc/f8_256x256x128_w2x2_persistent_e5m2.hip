// 8-bit-input GEMM instances (gemm_f8.hpp), E5M2 operands: fp16 / bf16 bias and
// output x six activations.
#include "gba_registry.hpp"

GBA_F8_ENTRY(f8_e5m2, 1)
