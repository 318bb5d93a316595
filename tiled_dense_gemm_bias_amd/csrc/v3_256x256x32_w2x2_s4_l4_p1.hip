// Interleaved direct-to-LDS kernel instances: 256x256x32 tile, 2x2 waves,
// 4 LDS stages, 4 loader waves, loads spread over 1 MFMA steps.
#include "gba_registry.hpp"

GBA_V3_SCHEDULE_ENTRY(i_256x256x32_w2x2_s4_l4_p1, 256, 256, 32, 2, 2, 4, 4, 1, 4)
