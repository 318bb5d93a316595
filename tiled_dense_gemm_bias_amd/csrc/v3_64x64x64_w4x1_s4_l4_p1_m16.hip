// Interleaved direct-to-LDS kernel instances: 64x64x64 tile, 4x1 waves (16 rows
// of C each), 4 LDS stages, 4 loader waves, loads spread over 1 MFMA step(s),
// 16x16x32 MFMAs; also the split-K first pass. For shapes whose 128x128 tiles
// leave most CUs idle (1024^2 outputs: 64 tiles of 128^2 against 256 of 64^2).
// No A stored (K,M) variant: its transposing reads need 16 chunks per k row.
#include "gba_registry.hpp"

GBA_V3_SCHEDULE_ENTRY_TBP(i_64x64x64_w4x1_s4_l4_p1_m16, 64, 64, 64, 4, 1, 4, 4, 1, 8)
