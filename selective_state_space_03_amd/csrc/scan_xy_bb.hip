// Fused-scan kernels for x/z stored as bf16 and y stored as bf16.
#define SSM_SCAN_XT bf16s
#define SSM_SCAN_YT bf16s
#include "scan_fused_impl.h"
