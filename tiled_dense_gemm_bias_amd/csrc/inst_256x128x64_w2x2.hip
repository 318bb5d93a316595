// Kernel instances of the 256x128x64 tile, 2x2 waves.
#include "gba_registry.hpp"

GBA_SCHEDULE_ENTRY(s_256x128x64_w2x2, 256, 128, 64, 2, 2, 4)
