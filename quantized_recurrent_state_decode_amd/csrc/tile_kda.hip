// STEP KDA tile kernel (row-level mixed widths).  Placeholder until written.
#include "tile_common.h"
hipError_t launch_tile_kda(const TileArgs&, hipStream_t) { return hipErrorNotSupported; }
