// Persistent interleaved kernel instances: 256x256x64 tiles, 2x2 waves, 2 LDS
// stages, 16x16x32 MFMAs, one workgroup per CU walking its tiles.
#include "gba_registry.hpp"

GBA_V5_SCHEDULE_ENTRY(p_256x256x64_w2x2, 256, 256, 2, 2, 4)
