// Fused-scan kernels for x/z stored as fp32 and y stored as bf16.
#define SSM_SCAN_XT float
#define SSM_SCAN_YT bf16s
#include "scan_fused_impl.h"
