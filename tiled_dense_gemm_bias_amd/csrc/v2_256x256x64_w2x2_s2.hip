// Direct-to-LDS kernel instances: 256x256x64 tile, 2x2 waves, 2 LDS stages.
#include "gba_registry.hpp"

GBA_V2_SCHEDULE_ENTRY(d_256x256x64_w2x2_s2, 256, 256, 64, 2, 2, 2, 4)
