// Internal interface between the host ABI (api.cpp) and the kernel launchers
// (*.hip).  Not installed; the public interface is include/ssm_mi355x.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

// Caller-supplied HIP events recorded around the main kernel of the next
// entry-point calls on this thread (null: nothing recorded).
struct TimingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
TimingEvents timing_events();

// Launches `launch` on `s` between the timing events, when set.
template <typename F>
hipError_t timed_launch(hipStream_t s, F&& launch) {
  const TimingEvents ev = timing_events();
  if (ev.start != nullptr) {
    const hipError_t e = hipEventRecord(ev.start, s);
    if (e != hipSuccess) return e;
  }
  launch();
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && ev.stop != nullptr) err = hipEventRecord(ev.stop, s);
  return err;
}

// ---- fused scan ----------------------------------------------------------
// B and C are repacked per (batch, t) into one fp32 row [B0..B15, C0..C15] so
// the scan kernel reads them with wave-uniform scalar loads.  A second set of
// rows holds them rescaled for the scaled-state form of the recurrence (see
// scan_fused_impl.h): B_t[n] q_n^-(j+1) and C_t[n] q_n^(j+1), where
// q_n = exp(dt_max A[0, n]) and j = t mod kScanResc, next to a table of q_n^k
// for k = 0..kScanResc.
constexpr int kScanN = 16;         // d_state handled by the fused scan
constexpr int kBcRow = 32;         // floats per packed row
constexpr int kScanMaxSplit = 32;  // time segments per sequence
constexpr unsigned kScanCuSlots = 256;  // compute units the scan's workgroups go round (MI355X)
constexpr int kConvK = 4;
constexpr int kScanBlk = 4;        // steps per tile of prefetched vector loads
constexpr int kScanResc = 2 * kScanBlk;  // steps between rescalings of the scaled state (a pair of tiles); segments start at multiples of it
constexpr int kScanTab = (kScanResc + 1) * kScanN;  // floats of the q_n^k table
constexpr int kScanHead = kScanN + kConvK - 1;      // floats per lane of a saved segment-0 start

struct ScanKernelArgs {
  const void* x;
  const void* z;
  const void* dt;        // rank-1 r (batch, seqlen) f32, or full (batch, seqlen, dim)
  void* y;
  const float* bc;       // packed rows (batch*seqlen + padding, kBcRow)
  const float* bcg;      // the rescaled rows, same shape; null: no scaled-state form
  const float* qtab;     // q_n^k, [k][n] for k = 0..kScanResc
  float* summ;           // per-segment summaries (time split only)
  float* head;           // segment 0's starting state and conv window, saved by the summary pass
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
  bool zoh;     // zero-order-hold input coefficient instead of dt
  const void* B;
  const void* C;
  float* bc_out;   // = k.bc, written by the packing kernel
  float* bcg_out;  // = k.bcg (or null), written by the packing kernel
  float* qtab_out; // = k.qtab, written by the packing kernel with bcg_out
};

struct bf16s;
size_t scan_workspace_bytes(int batch, int seqlen, int dim, int nseg);
// Turns the segment summaries into the state entering each segment, in place
// (slot k then holds the state entering segment k+1).
hipError_t launch_scan_compose(const ScanKernelArgs& a, hipStream_t stream);
template <typename XT, typename YT>
hipError_t launch_scan_xy(const ScanLaunch& l, hipStream_t stream);
template <typename XT, typename YT>
int scan_occupancy_xy(const ScanLaunch& l);
// Workgroups of the full-segment scan kernel that the current device holds at
// once (CUs x resident workgroups per CU), or 0 when it cannot be queried.
long scan_resident_waves(const ScanLaunch& l);
// Workspace layout of a scan call: plain rows, rescaled rows, the q_n^k
// table, then (time split only) the segment summaries and the saved starts
// of segment 0.
size_t scan_bcg_offset(int batch, int seqlen);
size_t scan_qtab_offset(int batch, int seqlen);
size_t scan_summary_offset(int batch, int seqlen);
size_t scan_head_offset(int batch, int seqlen, int dim, int nseg);
hipError_t launch_scan(const ScanLaunch& l, hipStream_t stream);
// The no-allocation scan entry point's scratch: a file-scope device array of
// kScanScratchBytes (one copy per device, held until the process ends).
// Writes its device address on the current device to *ptr; the address is
// looked up once per device (hipGetSymbolAddress) and kept.
constexpr size_t kScanScratchBytes = size_t(64) << 20;
hipError_t scan_scratch(void** ptr);

// ---- blocked scan (scan_blocked.hip) ---------------------------------------
// The whole sequence in one pass of 16-step blocks, 16 channels per wave, the
// saturated blocks' recurrence as matrix-core products of per-block tables
// (see scan_blocked.hip).  Takes bf16 x / z / E-wide dt, no conv, Euler, dim a
// multiple of 64.
constexpr int kBlkT = 16;           // steps per block
constexpr int kBlkRec = 5120;       // bytes of a (batch, block) table record
constexpr int kBlkQv = 16 + (kBlkT + 1) * kScanN + 1;  // floats: log2 q_n, q_n^k (k = 0..16), flag
constexpr long kBlkAutoGroups = 3L * kScanCuSlots;  // 64-channel groups from which the library chooses it

struct ScanBlkArgs {
  const uint16_t* x;    // u (batch, L, E) bf16
  const uint16_t* z;    // (batch, L, E) bf16 or null
  const uint16_t* dt;   // pre-activation (batch, L, E) bf16
  void* y;
  const unsigned char* rec;  // (batch, nrec) records, written by the packing kernel
  const float* qv;           // kBlkQv floats, written by the packing kernel
  const float* A;            // (dim, 16)
  const float* D;            // (dim) or null
  const float* dt_bias;      // (dim) or null
  const float* state_in;
  float* state_out;
  int batch, seqlen, dim, nrec;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus;
};

struct ScanBlkLaunch {
  ScanBlkArgs k;
  int y_dtype, bc_dtype;
  const void* B;
  const void* C;
  unsigned char* rec_out;  // = k.rec
  float* qv_out;           // = k.qv
};

inline int scan_blk_records(int seqlen) { return (seqlen + kBlkT - 1) / kBlkT; }
size_t scan_blk_qv_offset(int batch, int seqlen);
size_t scan_blk_workspace_bytes(int batch, int seqlen);
hipError_t launch_scan_blocked(const ScanBlkLaunch& l, hipStream_t stream);

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
  bool zoh;  // zero-order-hold input coefficient instead of dt
};

hipError_t launch_decode(const DecodeLaunch& l, hipStream_t stream);

// ---- chunked SSD ---------------------------------------------------------
constexpr int kSsdN = 64;
constexpr int kSsdQ = 128;
constexpr int kSsdMaxP = 128;
constexpr int kSsdMaxSeg = 16;
constexpr int kSsdPiece = 16;  // chunks per segment summary piece

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
  const void* z;  // gate (Bt, L, H, P) or null
  float* ws;  // workspace: segment states and piece summaries (nseg > 1)
  int batch, seqlen, nheads, headdim, ngroups, nchunks, d_per_channel, z_bf16;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus;
  int nseg, cps, ppseg;  // segments per sequence, chunks per segment, summary pieces per segment
};

// How a sequence of the chunked scan is cut into segments (one workgroup per
// batch, head and segment).
struct ChunkSplit {
  int nseg, cps, ppseg;
};
ChunkSplit chunk_split(int batch, int seqlen, int nheads, int headdim, int segments);

struct ChunkLaunch {
  ChunkKernelArgs k;
  int x_dtype, bc_dtype, out_dtype;
};

size_t chunk_workspace_bytes(int batch, int seqlen, int nheads, int headdim, int segments);
hipError_t launch_chunk(const ChunkLaunch& l, hipStream_t stream);

// ---- chunked SSD, the other shapes (ssd_generic.hip) -----------------------
// Any chunk size up to kSsdGenMaxQ, d_state up to kSsdGenMaxN, headdim up to
// kSsdGenMaxP, x / B / C / z in fp32 or bf16; fp32 vector arithmetic.
constexpr int kSsdGenMaxQ = 256;
constexpr int kSsdGenMaxN = 128;
constexpr int kSsdGenMaxP = 128;

struct ChunkGenericArgs {
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
  const void* z;
  float* chunk_state;  // workspace (batch, nchunks, H, P, N): chunk states, then the states entering each chunk
  float* chunk_decay;  // workspace (batch, nchunks, H): e^{sum over the chunk of dt A_h}
  int batch, seqlen, nheads, headdim, ngroups, d_state, chunk_size, nchunks, d_per_channel;
  int x_bf16, bc_bf16, z_bf16, out_bf16, dt_softplus;
  float dt_min, dt_max, sp_lo, sp_hi;
};

size_t chunk_generic_workspace_bytes(int batch, int seqlen, int nheads, int headdim, int d_state, int chunk_size);
size_t chunk_generic_decay_offset(int batch, int seqlen, int nheads, int headdim, int d_state, int chunk_size);
hipError_t launch_chunk_generic(const ChunkGenericArgs& a, hipStream_t stream);

// ---- SSD-form decode step ------------------------------------------------
struct ChunkDecodeKernelArgs {
  const void* x;        // (Bt, H, P)
  const float* dt;      // (Bt, H) raw
  const float* dt_bias; // (H) or null
  const float* A;       // (H)
  const void* B;        // (Bt, G, N)
  const void* C;
  const float* D;       // (H) or (H, P) or null
  const void* z;        // (Bt, H, P) or null
  float* state;         // (Bt, H, P, N), in place
  void* out;            // (Bt, H, P)
  unsigned rows;        // Bt * H * P
  int nheads, headdim, ngroups, heads_per_group, d_per_channel, z_bf16;
  float dt_min, dt_max, sp_lo, sp_hi;
  int dt_softplus;
};

struct ChunkDecodeLaunch {
  ChunkDecodeKernelArgs k;
  int x_dtype, bc_dtype, out_dtype, d_state;
};

hipError_t launch_chunk_decode(const ChunkDecodeLaunch& l, hipStream_t stream);

// ---- backward of the scan stage --------------------------------------------
constexpr int kBwdSeg = 16;     // time steps per segment (states recomputed in registers)
constexpr int kBwdRun = 4;      // segments one wave of the main pass walks, last to first
constexpr int kBwdWg = 4;       // 16-channel groups per main-pass workgroup (one wave each)
constexpr int kBwdPe = 24;      // per-(batch, segment run, channel) partial: dA[16], dD, ddt_w, ddt_bias, dconv_w[4], dconv_b

struct BwdArgs {
  // forward inputs
  const void* x;
  const void* dt;
  const float* dt_w;
  const float* dt_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* conv_w;
  const float* conv_b;
  const float* conv_cache_in;
  const float* state_in;
  // incoming gradients
  const void* dy;
  const float* dstate_out;
  // gradients (fp32; null: not written)
  float *dx, *dz, *ddt, *ddt_w, *ddt_bias, *dA, *dB, *dC, *dD, *dconv_w, *dconv_b, *dconv_cache, *dstate_in;
  // workspace
  // xb: the conv-output gradient of the first 3 steps of every run
  float *hs, *qs, *sdt, *xb, *pB, *pC, *pr, *pe;
  int batch, seqlen, dim, nseg, ngroups16;
  int x_bf16, dt_bf16, dt_rank1, bc_bf16, dy_bf16, dt_softplus;
  float dt_min, dt_max;
};

int bwd_segments(int seqlen);
// Segment runs (kBwdRun segments each) and main-pass channel blocks (kBwdWg
// groups of 16 channels each): the granularity of the partial sums.
__host__ __device__ inline int bwd_runs(int nseg) { return (nseg + kBwdRun - 1) / kBwdRun; }
__host__ __device__ inline int bwd_blocks64(int dim) { return ((dim + 15) / 16 + kBwdWg - 1) / kBwdWg; }
hipError_t launch_scan_bwd(const BwdArgs& a, hipStream_t stream);

// ---- projection GEMM: C = A W^T --------------------------------------------
// A (M, K) bf16 or f32 with row stride lda; W (N, K) bf16 with row stride ldw;
// output columns [0, n_split) go to C0 (row stride ldc0), [n_split, N) to C1
// (row stride ldc1, column index n - n_split).  Requires K % 8 == 0, N % 4 ==
// 0, n_split == N or n_split % 256 == 0, 16-byte aligned rows and pointers.
// A workspace (ws, ws_bytes) lets a shape with too few output tiles for the
// chip split K and add fp32 partials; without one it runs unsplit.
struct GemmArgs {
  const void* A;
  const uint16_t* W;
  void* C0;
  void* C1;
  float* ws;
  size_t ws_bytes;
  int lda, ldw, ldc0, ldc1;
  int M, N, K, n_split;
  int kchunk;  // set by the launcher
};

// Workspace for the fastest split of this shape (0: none needed).
size_t gemm_workspace_bytes(int M, int N, int K, int a_dtype);
hipError_t launch_gemm(const GemmArgs& g, int a_dtype, int out_dtype, hipStream_t stream);

// ---- x_proj of the layer (conv + SiLU recomputed from x) -------------------
struct XprojArgs {
  const float* x;              // (T, E) x_branch, T = batch * seqlen
  const float* conv_w;         // (E, 4)
  const float* conv_b;         // (E) or null
  const float* conv_cache_in;  // (batch, E, 3) or null (zeros)
  const uint16_t* w_x;         // (nout, E) bf16
  float* part;                 // partial sums (splits, T, 48)
  float* B;                    // (T, d_state)
  float* C;                    // (T, d_state)
  float* dt_raw;               // (T)
  int batch, seqlen, dim, d_state, nout;
};

int xproj_splits(int tokens, int dim);
size_t xproj_partial_bytes(int tokens, int dim);
hipError_t launch_xproj(const XprojArgs& a, hipStream_t stream);

}  // namespace ssm
