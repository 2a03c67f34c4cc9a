// Fused-scan kernels for x/z stored as bf16 and y stored as fp32.
#define SSM_SCAN_XT bf16s
#define SSM_SCAN_YT float
#include "scan_fused_impl.h"
