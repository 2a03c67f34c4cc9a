// Internal interface between the host ABI (api.cpp) and the kernel launchers
// (*.hip).  Not installed; the public interface is include/ssm_mi355x.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

// ---- fused scan ----------------------------------------------------------
// B, C and the rank-1 dt input are repacked per (batch, t) into one fp32 row
// so the scan kernel reads them with wave-uniform scalar loads.
constexpr int kScanN = 16;          // d_state handled by the fused scan
constexpr int kBcrRow = 48;         // floats per packed row: B[16] C[16] r pad
constexpr int kScanMaxSplit = 16;   // segments per workgroup (one wave each)
constexpr int kConvK = 4;

struct ScanKernelArgs {
  const void* x;
  const void* z;
  const void* dt;        // full-width dt (DTM 1/2); unused for rank-1
  void* y;
  const float* bcr;      // (batch*seqlen, kBcrRow)
  const float* A;        // (dim, 16)
  const float* D;        // (dim) or null
  const float* dt_w;     // (dim) or null
  const float* dt_bias;  // (dim) or null
  const float* conv_w;   // (dim, 4) or null
  const float* conv_b;   // (dim) or null
  const float* conv_cache_in;
  float* conv_cache_out;
  const float* state_in;
  float* state_out;
  int batch, seqlen, dim, n_egroups, seg_len, nseg;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus, has_z;
};

struct ScanLaunch {
  ScanKernelArgs k;
  int x_dtype, y_dtype, bc_dtype;
  int dt_mode;  // 0 rank-1 f32, 1 full f32, 2 full bf16
  bool conv;
  const void* B;
  const void* C;
  const float* r;  // rank-1 dt input (batch, seqlen) or null
  float* bcr_out;  // workspace
};

size_t scan_bcr_bytes(int batch, int seqlen);
hipError_t launch_scan(const ScanLaunch& l, hipStream_t stream);

// ---- decode step ---------------------------------------------------------
struct DecodeKernelArgs {
  const void* x;
  const void* z;
  const void* dt;
  const void* B;
  const void* C;
  void* y;
  const float* A;
  const float* D;
  const float* dt_w;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;
  float* conv_cache;
  float* state;
  int batch, dim;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus, has_z;
};

struct DecodeLaunch {
  DecodeKernelArgs k;
  int x_dtype, y_dtype, bc_dtype, dt_mode;
  bool conv;
};

hipError_t launch_decode(const DecodeLaunch& l, hipStream_t stream);

// ---- chunked SSD ---------------------------------------------------------
constexpr int kSsdN = 64;
constexpr int kSsdQ = 128;
constexpr int kSsdMaxP = 128;

struct ChunkKernelArgs {
  const void* x;
  const float* dt;
  const float* dt_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* state_in;
  float* state_out;
  void* out;
  float* ws;  // workspace
  int batch, seqlen, nheads, headdim, ngroups, nchunks, d_per_channel;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus;
};

struct ChunkLaunch {
  ChunkKernelArgs k;
  int x_dtype, bc_dtype, out_dtype;
};

size_t chunk_workspace_bytes(int batch, int seqlen, int nheads, int headdim, int ngroups);
hipError_t launch_chunk(const ChunkLaunch& l, hipStream_t stream);

}  // namespace ssm
