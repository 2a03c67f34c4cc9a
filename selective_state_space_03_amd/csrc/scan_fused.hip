// Fused selective scan for gfx950 (host dispatch and the B/C packing kernel;
// the scan kernels are in scan_fused_impl.h): causal depthwise conv1d (k=4) + SiLU, the
// step size dt = clip(softplus(dt_proj + dt_bias), lo, hi), the diagonal
// recurrence h_t = exp(dt*A) h_{t-1} + dt*B_t*u_t with readout
// y_t = C_t . h_t + D*u_t, and the gate y * SiLU(z), in one pass over HBM.
//
// Page "Axon-SSM: selective state space model": section "Algorithm" (the
// dataflow x_branch -> conv1d -> SiLU -> scan -> y * SiLU(z)), "SSM scan"
// (sequential over seq_len), "JIT-compiled kernels" (_ssm_fma = dA*h + dB*x_t
// fused with no intermediate tensors; _compute_dt = clip(softplus(dt +
// dt_bias))), "Autoregressive decoding" (prefill builds conv_cache from the last
// K-1 positions).  Page "What is the Mamba model?", sections "Parallel
// prefix-scan" and "chunkscan": the sequence is cut into segments scanned in
// parallel, each reduced to its affine map (prod exp(dt A), h_end from 0), the
// maps composed in order, and every segment re-run from its incoming state.
//
// Mapping: one lane = one (batch, channel); its 16 fp32 states stay in VGPRs
// for the whole segment.  A workgroup is one wave of 64 consecutive channels,
// so each x/dt/z/y access of a step is one contiguous 128- or 256-byte
// segment, issued as a buffer load whose per-lane offset never changes (the
// step's position travels in the scalar offset).  B_t and C_t are the same for
// every channel of a batch row: they are packed once into 128-byte fp32 rows
// (plain, and rescaled for the scaled-state form) that each step reads with
// scalar loads (see scan_fused_impl.h).
//
// Time split (nseg > 1): launch 1 reduces segments 0..nseg-2 to their
// summaries (segment 0 from the true initial state, the others from zero);
// a small launch composes them in order into every segment's incoming state;
// the last launch runs all segments in full.  Summaries travel through the
// workspace.
#include <mutex>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

// Workspace of ssm_scan_fwd_noalloc (packed and rescaled B/C rows, the decay
// table, segment summaries), for callers that cannot allocate device memory.
// In host code this name is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress on each device (scan_scratch) and
// is the only form in which host code hands the array to a kernel.
static __device__ __align__(256) unsigned char scratch[kScanScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Pack B and C (bf16 or fp32) into fp32 rows [B0..B15, C0..C15].  With
// outg: also the rows of the scaled-state form, B_t[n] q_n^-(j+1) and
// C_t[n] q_n^(j+1) with q_n = exp(dt_max A[0, n]) and j = t mod kScanResc,
// and the table qtab[k][n] = q_n^k (k = 0..kScanResc).  The factors are
// exponentials taken in double precision and rounded once, so a product
// q^-(i+1) q^(j+1) or q^-(i+1) q^k is the decay over its steps to within a
// few fp32 roundings.  The grid has at least 256 threads, so the table is
// always complete.
template <typename BT>
__global__ void pack_bc_kernel(const BT* __restrict__ B, const BT* __restrict__ C, float* __restrict__ out,
                               float* __restrict__ outg, float* __restrict__ qtab, const float* __restrict__ A,
                               float dt_max, int seqlen, size_t rows) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (outg && i < static_cast<size_t>(kScanTab)) {
    const int k = static_cast<int>(i) / kScanN, n = static_cast<int>(i) % kScanN;
    qtab[i] = static_cast<float>(exp(static_cast<double>(k) * dt_max * A[n]));
  }
  if (i >= rows * kBcRow) return;
  const size_t row = i / kBcRow;
  const int col = static_cast<int>(i % kBcRow);
  const float v = col < kScanN ? to_f32(B[row * kScanN + col]) : to_f32(C[row * kScanN + col - kScanN]);
  out[i] = v;
  if (outg) {
    const int j = static_cast<int>(row % static_cast<size_t>(seqlen)) % kScanResc + 1;
    const int n = col % kScanN;
    const double e = (col < kScanN ? -j : j) * static_cast<double>(dt_max) * A[n];
    outg[i] = static_cast<float>(static_cast<double>(v) * exp(e));
  }
}

// One row more than there are tokens: each step also loads the next step's
// row, which after the last token is this padding row.
size_t bc_bytes(int batch, int seqlen) {
  const size_t rows = static_cast<size_t>(batch) * seqlen + 1;
  return (rows * kBcRow * sizeof(float) + 255) & ~static_cast<size_t>(255);
}
constexpr size_t kQtabBytes = (kScanTab * sizeof(float) + 255) & ~static_cast<size_t>(255);

// Affine composition of the segment summaries, one thread per (batch,
// channel, state): slot 0 already holds segment 0's end state (it started from
// the true initial state), and for k = 1 .. nseg-2 the state entering segment
// k+1 is exp(A sum dt_k) h + h_end_k, written over slot k.  Every summary is
// loaded before the chain starts, so the chain waits for memory once.
// Block: 64 channels x 4 states; grid: (batch x channel groups, 4).
__global__ __launch_bounds__(256) void scan_compose_kernel(ScanKernelArgs a) {
  constexpr int K = kScanMaxSplit - 1;  // summary slots at most
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int gid = blockIdx.x;  // batch * n_egroups + channel group
  const int g = gid % a.n_egroups;
  const int e = min(g * 64 + lane, a.dim - 1);
  const int nk = a.nseg - 1;   // slots in use
  float* summ = a.summ + static_cast<size_t>(gid) * nk * (kScanN + 1) * 64;
  const float al2 = a.A[static_cast<size_t>(e) * kScanN + n] * kLog2e;
  float hend[K], sd[K];
#pragma unroll
  for (int k = 1; k < K; ++k) {
    if (k < nk) {
      const float* sk = summ + static_cast<size_t>(k) * (kScanN + 1) * 64;
      hend[k] = sk[n * 64 + lane];
      sd[k] = sk[kScanN * 64 + lane];
    }
  }
  float h = summ[n * 64 + lane];
#pragma unroll
  for (int k = 1; k < K; ++k) {
    if (k < nk) {
      h = fmaf(exp2_fast(al2 * sd[k]), h, hend[k]);
      summ[static_cast<size_t>(k) * (kScanN + 1) * 64 + n * 64 + lane] = h;
    }
  }
}

}  // namespace

hipError_t launch_scan_compose(const ScanKernelArgs& a, hipStream_t stream) {
  if (a.nseg <= 2) return hipSuccess;  // slot 0 is already the state entering segment 1
  const unsigned groups = static_cast<unsigned>(a.batch) * static_cast<unsigned>(a.n_egroups);
  hipLaunchKernelGGL(scan_compose_kernel, dim3(groups, kScanN / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

size_t scan_head_offset(int batch, int seqlen, int dim, int nseg) {
  const size_t groups = static_cast<size_t>(batch) * ((dim + 63) / 64);
  return scan_summary_offset(batch, seqlen) + groups * (nseg - 1) * (kScanN + 1) * 64 * sizeof(float);
}

size_t scan_workspace_bytes(int batch, int seqlen, int dim, int nseg) {
  if (batch <= 0 || seqlen <= 0) return 0;
  if (nseg <= 1) return scan_summary_offset(batch, seqlen);
  // summaries, then segment 0's starting state and conv window per lane
  const size_t groups = static_cast<size_t>(batch) * ((dim + 63) / 64);
  return scan_head_offset(batch, seqlen, dim, nseg) + groups * kScanHead * 64 * sizeof(float);
}

size_t scan_bcg_offset(int batch, int seqlen) { return bc_bytes(batch, seqlen); }
size_t scan_qtab_offset(int batch, int seqlen) { return 2 * bc_bytes(batch, seqlen); }
size_t scan_summary_offset(int batch, int seqlen) { return 2 * bc_bytes(batch, seqlen) + kQtabBytes; }

hipError_t scan_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

long scan_resident_waves(const ScanLaunch& l) {
  // CU count per device, asked once (no runtime query inside stream capture)
  static int cu_count[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int cus = __atomic_load_n(&cu_count[dev], __ATOMIC_RELAXED);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    __atomic_store_n(&cu_count[dev], cus, __ATOMIC_RELAXED);
  }
  int per_cu;
  if (l.x_dtype == kBF16)
    per_cu = l.y_dtype == kBF16 ? scan_occupancy_xy<bf16s, bf16s>(l) : scan_occupancy_xy<bf16s, float>(l);
  else
    per_cu = l.y_dtype == kBF16 ? scan_occupancy_xy<float, bf16s>(l) : scan_occupancy_xy<float, float>(l);
  return static_cast<long>(cus) * per_cu;
}

hipError_t launch_scan(const ScanLaunch& l, hipStream_t stream) {
  const size_t rows = static_cast<size_t>(l.k.batch) * l.k.seqlen;
  if (rows > 0) {
    const size_t total = rows * kBcRow;
    const unsigned threads = 256;
    const unsigned blocks = static_cast<unsigned>((total + threads - 1) / threads);
    if (l.bc_dtype == kBF16) {
      hipLaunchKernelGGL(pack_bc_kernel<bf16s>, dim3(blocks), dim3(threads), 0, stream,
                         static_cast<const bf16s*>(l.B), static_cast<const bf16s*>(l.C), l.bc_out, l.bcg_out,
                         l.qtab_out, l.k.A, l.k.dt_max, l.k.seqlen, rows);
    } else {
      hipLaunchKernelGGL(pack_bc_kernel<float>, dim3(blocks), dim3(threads), 0, stream,
                         static_cast<const float*>(l.B), static_cast<const float*>(l.C), l.bc_out, l.bcg_out,
                         l.qtab_out, l.k.A, l.k.dt_max, l.k.seqlen, rows);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (l.x_dtype == kBF16) {
    return l.y_dtype == kBF16 ? launch_scan_xy<bf16s, bf16s>(l, stream) : launch_scan_xy<bf16s, float>(l, stream);
  }
  return l.y_dtype == kBF16 ? launch_scan_xy<float, bf16s>(l, stream) : launch_scan_xy<float, float>(l, stream);
}

}  // namespace ssm
