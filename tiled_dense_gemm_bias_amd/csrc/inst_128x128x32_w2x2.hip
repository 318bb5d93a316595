// Kernel instances of the 128x128x32 tile, 2x2 waves.
#include "gba_registry.hpp"

GBA_SCHEDULE_ENTRY(s_128x128x32_w2x2, 128, 128, 32, 2, 2, 8)
