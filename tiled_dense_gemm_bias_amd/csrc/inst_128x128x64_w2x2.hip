// Kernel instances of the 128x128x64 tile, 2x2 waves.
#include "gba_registry.hpp"

GBA_SCHEDULE_ENTRY(s_128x128x64_w2x2, 128, 128, 64, 2, 2, 8)
