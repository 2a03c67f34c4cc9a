// Fused-scan kernels for x/z stored as fp32 and y stored as fp32.
#define SSM_SCAN_XT float
#define SSM_SCAN_YT float
#include "scan_fused_impl.h"
