// Per-window tile kernel.  Placeholder until written.
#include "tile_common.h"
hipError_t launch_tile_window(const TileArgs&, hipStream_t) { return hipErrorNotSupported; }
