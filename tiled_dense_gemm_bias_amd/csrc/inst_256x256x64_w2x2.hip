// Kernel instances of the 256x256x64 tile, 2x2 waves.
#include "gba_registry.hpp"

GBA_SCHEDULE_ENTRY(s_256x256x64_w2x2, 256, 256, 64, 2, 2, 4)
