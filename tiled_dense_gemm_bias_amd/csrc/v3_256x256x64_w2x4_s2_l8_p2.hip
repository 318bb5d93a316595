// Interleaved direct-to-LDS kernel instances: 256x256x64 tile, 2x4 waves,
// 2 LDS stages, 8 loader waves, loads spread over 2 MFMA steps.
#include "gba_registry.hpp"

GBA_V3_SCHEDULE_ENTRY(i_256x256x64_w2x4_s2_l8_p2, 256, 256, 64, 2, 4, 2, 8, 2, 4)
