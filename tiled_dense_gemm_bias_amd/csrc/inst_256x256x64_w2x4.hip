// Kernel instances of the 256x256x64 tile, 2x4 waves.
#include "gba_registry.hpp"

GBA_SCHEDULE_ENTRY(s_256x256x64_w2x4, 256, 256, 64, 2, 4, 4)
