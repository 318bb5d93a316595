// Interleaved direct-to-LDS kernel instances: 128x128x64 tile, 2x2 waves,
// 4 LDS stages, 4 loader waves, loads spread over 1 MFMA step(s), 16x16x32 MFMAs;
// also the split-K first pass, and A stored (K,M). The built-in choice for shapes too small for
// 256-wide tiles: the fourth stage keeps more loads in flight (10-20 % faster
// than three stages at 1024^3 and 2048^3).
#include "gba_registry.hpp"

GBA_V3_SCHEDULE_ENTRY_TBPA(i_128x128x64_w2x2_s4_l4_p1_m16, 128, 128, 64, 2, 2, 4, 4, 1, 8)
