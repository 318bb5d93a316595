// Interleaved direct-to-LDS kernel instances: 256x256x64 tile, 2x2 waves,
// 2 LDS stages, 4 loader waves, loads spread over 1 MFMA step(s), 16x16x32 MFMAs.
#include "gba_registry.hpp"

GBA_V3_SCHEDULE_ENTRY_TBA(i_256x256x64_w2x2_s2_l4_p1_m16, 256, 256, 64, 2, 2, 2, 4, 1, 4)
