// Prefill-chunk indexer scores on MFMA (gfx950): placeholder unit, filled in
// with the bf16 GEMM of the chunk's per-group query sums against the slab.
#include "tkv_dev.h"
#include "tkv_launch.h"
