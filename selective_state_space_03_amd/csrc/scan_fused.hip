// Fused selective scan for gfx950: causal depthwise conv1d (k=4) + SiLU, the
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
// prefix-scan" and "chunkscan": the sequence split into segments scanned in
// parallel, each reduced to an affine map (prod dA, h_end), the maps combined
// in order, and each segment re-run from its incoming state.
//
// Mapping: one lane = one (batch, channel); its 16 fp32 states live in VGPRs
// for the whole sequence.  B_t, C_t (and the rank-1 dt input r_t) are the same
// for every channel of a batch row, so they are read with wave-uniform scalar
// loads from a packed fp32 row.  A wave covers 64 consecutive channels, so
// every x/dt/z/y access of a wave is one contiguous 128- or 256-byte segment.
// A workgroup holds `nseg` waves on the same 64 channels, wave w scanning time
// segment w; the segments' affine summaries meet in LDS.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kTile = 4;  // time steps whose loads are issued one tile ahead

// Pack B, C (bf16 or fp32) and the rank-1 dt input r into fp32 rows of
// kBcrRow floats: [B0..B15, C0..C15, r, 0...].
template <typename BT>
__global__ void pack_bcr_kernel(const BT* __restrict__ B, const BT* __restrict__ C, const float* __restrict__ r,
                                float* __restrict__ out, size_t rows) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (i >= rows * kBcrRow) return;
  const size_t row = i / kBcrRow;
  const int col = static_cast<int>(i % kBcrRow);
  float v = 0.0f;
  if (col < kScanN) {
    v = to_f32(B[row * kScanN + col]);
  } else if (col < 2 * kScanN) {
    v = to_f32(C[row * kScanN + col - kScanN]);
  } else if (col == 2 * kScanN && r != nullptr) {
    v = r[row];
  }
  out[i] = v;
}

struct LaneCtx {
  int b, e;
  bool act;
  float al2[kScanN];  // A[e, n] * log2(e)
  float d, dtw, dtb;
  float cw0, cw1, cw2, cw3, cb;
};

// Raw (pre-conv) input at time p for this lane: x when p >= 0, otherwise the
// cache entry K-1+p (oldest first), or 0 at a fresh prefill.
template <typename XT>
__device__ __forceinline__ float raw_at(const ScanKernelArgs& a, const XT* __restrict__ x, const LaneCtx& c, int p) {
  if (p >= a.seqlen) return 0.0f;  // only reachable for an empty segment, whose window is unused
  if (p >= 0) return to_f32(x[(static_cast<size_t>(c.b) * a.seqlen + p) * a.dim + c.e]);
  if (a.conv_cache_in == nullptr) return 0.0f;
  return a.conv_cache_in[(static_cast<size_t>(c.b) * a.dim + c.e) * (kConvK - 1) + (kConvK - 1 + p)];
}

// Packed-row floats one step reads: B[16], C[16] and, for rank-1 dt, r.
template <int DTM>
constexpr int row_floats() {
  return DTM == 0 ? 2 * kScanN + 1 : 2 * kScanN;
}

template <int K>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&r)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) r[i] = p[i];
}

// Scan time steps [t0, t1) of one lane.  FULL: readout, gate and store y.
// Otherwise (summary pass): state update only, accumulating sum(dt) so the
// segment's decay product is exp(A * sum dt).
//
// Each step is laid out in phases separated by scheduling barriers so that the
// wave-uniform row (B_t, C_t, r_t) of the next step is requested as soon as the
// current row is dead and lands while the row-independent work of the next
// step (conv, dt, decay factors, gate) runs; the row lives in one set of SGPRs.
template <typename XT, typename YT, int DTM, bool CONV, bool POW, bool FULL>
__device__ __forceinline__ void run_segment(const ScanKernelArgs& a, const LaneCtx& c, const XT* __restrict__ x,
                                            const XT* __restrict__ z, const void* __restrict__ dtp,
                                            const float* __restrict__ bcr, YT* __restrict__ y, int t0, int t1,
                                            float (&h)[kScanN], float (&win)[3], float& sdt) {
  using DT = typename std::conditional<DTM == 2, bf16s, float>::type;
  constexpr int RF = row_floats<DTM>();
  const DT* __restrict__ dtv_p = static_cast<const DT*>(dtp);
  const size_t E = static_cast<size_t>(a.dim);
  const size_t lane_base = static_cast<size_t>(c.b) * a.seqlen * E + c.e;
  const float* __restrict__ bcr_b = bcr + static_cast<size_t>(c.b) * a.seqlen * kBcrRow;
  const bool has_z = FULL && a.has_z;
  const bool sp = a.dt_softplus;
  if (t0 >= t1) return;

  auto load_tile = [&](int tb, XT (&xs)[kTile], DT (&ds)[kTile], XT (&zs)[kTile]) {
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      const int t = min(tb + i, t1 - 1);
      const size_t idx = lane_base + static_cast<size_t>(t) * E;
      xs[i] = x[idx];
      if (DTM != 0) ds[i] = dtv_p[idx];
      if (has_z) zs[i] = z[idx];
    }
  };
  auto row_at = [&](int t) { return bcr_b + static_cast<size_t>(t) * kBcrRow; };

  float row[RF];
  auto step = [&](int t, XT xr, DT dr, XT zr, bool next) {
    // phase 1: everything that does not need the row (except rank-1 dt)
    float u = to_f32(xr);
    if (CONV) {
      const float xc = fmaf(c.cw0, win[0], fmaf(c.cw1, win[1], fmaf(c.cw2, win[2], fmaf(c.cw3, u, c.cb))));
      win[0] = win[1];
      win[1] = win[2];
      win[2] = u;
      u = silu(xc);
    }
    const float gate = has_z ? silu(to_f32(zr)) : 1.0f;
    float pre;
    if constexpr (DTM == 0) {
      pre = fmaf(c.dtw, row[2 * kScanN], c.dtb);
    } else {
      pre = to_f32(dr) + c.dtb;
    }
    const float dt = sp ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                        : dt_clip(pre, a.dt_min, a.dt_max);
    if (!FULL) sdt += dt;
    const float dtu = dt * u;
    float dA[kScanN];
    if (POW) {
      // A[e, n] = (n+1) A[e, 0] for every n: exp(dt A[e,n]) = r^(n+1) with
      // r = exp(dt A[e,0]); the powers come from a depth-5 product tree.
      dA[0] = exp2_fast(dt * c.al2[0]);
#pragma unroll
      for (int k = 1; k < kScanN; ++k) dA[k] = (k & 1) ? dA[(k - 1) / 2] * dA[(k - 1) / 2] : dA[k - 1] * dA[0];
    } else {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) dA[n] = exp2_fast(dt * c.al2[n]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 2: state update and readout with the row
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < kScanN; ++n) {
      h[n] = fmaf(dA[n], h[n], dtu * row[n]);
      if (FULL) acc = fmaf(row[kScanN + n], h[n], acc);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 3: the row is dead; request the next one
    if (next) load_row(row_at(t + 1), row);
    __builtin_amdgcn_sched_barrier(0);
    // phase 4: skip term, gate, store
    if (FULL) {
      acc = fmaf(c.d, u, acc) * gate;
      if (c.act) st<YT>(y, lane_base + static_cast<size_t>(t) * E, acc);
    }
  };

  XT xv[kTile];
  DT dv[kTile];
  XT zv[kTile];
  load_tile(t0, xv, dv, zv);
  load_row(row_at(t0), row);
  int tb = t0;
  // Full tiles: the next tile's vector loads are in flight while this tile computes.
  for (; tb + kTile <= t1; tb += kTile) {
    XT xn[kTile];
    DT dn[kTile];
    XT zn[kTile];
    if (tb + kTile < t1) load_tile(tb + kTile, xn, dn, zn);
#pragma unroll
    for (int i = 0; i < kTile; ++i) step(tb + i, xv[i], dv[i], zv[i], tb + i + 1 < t1);
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      xv[i] = xn[i];
      if (DTM != 0) dv[i] = dn[i];
      if (has_z) zv[i] = zn[i];
    }
  }
  // Ragged tail: fewer than kTile steps, already loaded into xv/dv/zv and row.
#pragma unroll
  for (int i = 0; i < kTile - 1; ++i) {
    if (tb + i < t1) step(tb + i, xv[i], dv[i], zv[i], tb + i + 1 < t1);
  }
}

template <typename XT, typename YT, int DTM, bool CONV>
__global__ __launch_bounds__(64 * kScanMaxSplit) void scan_kernel(ScanKernelArgs a, const XT* __restrict__ x,
                                                                   const XT* __restrict__ z,
                                                                   const void* __restrict__ dtp,
                                                                   const float* __restrict__ bcr,
                                                                   YT* __restrict__ y) {
  __shared__ float s_h[kScanMaxSplit - 1][kScanN][64];
  __shared__ float s_sdt[kScanMaxSplit - 1][64];

  const int lane = threadIdx.x & 63;
  const int seg = uniform(threadIdx.x >> 6);
  const int g = uniform(blockIdx.x % a.n_egroups);
  LaneCtx c;
  c.b = uniform(blockIdx.x / a.n_egroups);
  const int e_raw = g * 64 + lane;
  c.act = e_raw < a.dim;
  c.e = c.act ? e_raw : a.dim - 1;

  bool prog = true;
  const float a0 = a.A[static_cast<size_t>(c.e) * kScanN];
#pragma unroll
  for (int n = 0; n < kScanN; ++n) {
    const float an = a.A[static_cast<size_t>(c.e) * kScanN + n];
    c.al2[n] = an * kLog2e;
    prog = prog && (an == static_cast<float>(n + 1) * a0);
  }
  c.d = a.D ? a.D[c.e] : 0.0f;
  c.dtw = a.dt_w ? a.dt_w[c.e] : 0.0f;
  c.dtb = a.dt_bias ? a.dt_bias[c.e] : 0.0f;
  if (CONV) {
    c.cw0 = a.conv_w[c.e * kConvK + 0];
    c.cw1 = a.conv_w[c.e * kConvK + 1];
    c.cw2 = a.conv_w[c.e * kConvK + 2];
    c.cw3 = a.conv_w[c.e * kConvK + 3];
    c.cb = a.conv_b ? a.conv_b[c.e] : 0.0f;
  } else {
    c.cw0 = c.cw1 = c.cw2 = c.cw3 = c.cb = 0.0f;
  }
  const bool use_pow = __all(prog);

  const int t0 = seg * a.seg_len;
  const int t1 = min(t0 + a.seg_len, a.seqlen);
  float win0[3] = {0.0f, 0.0f, 0.0f};
  if (CONV) {
    win0[0] = raw_at<XT>(a, x, c, t0 - 3);
    win0[1] = raw_at<XT>(a, x, c, t0 - 2);
    win0[2] = raw_at<XT>(a, x, c, t0 - 1);
  }
  float win[3] = {win0[0], win0[1], win0[2]};
  float h[kScanN];
  const size_t sbase = (static_cast<size_t>(c.b) * a.dim + c.e) * kScanN;
#pragma unroll
  for (int n = 0; n < kScanN; ++n) h[n] = (seg == 0 && a.state_in) ? a.state_in[sbase + n] : 0.0f;
  float sdt = 0.0f;

#define SSM_RUN(FULLV)                                                                                   \
  do {                                                                                                   \
    if (use_pow)                                                                                         \
      run_segment<XT, YT, DTM, CONV, true, FULLV>(a, c, x, z, dtp, bcr, y, t0, t1, h, win, sdt);         \
    else                                                                                                 \
      run_segment<XT, YT, DTM, CONV, false, FULLV>(a, c, x, z, dtp, bcr, y, t0, t1, h, win, sdt);        \
  } while (0)

  if (a.nseg == 1) {
    SSM_RUN(true);
  } else {
    if (seg == 0) {
      SSM_RUN(true);  // segment 0 starts from the true state: its end state is final
    } else {
      SSM_RUN(false);  // local summary from h = 0
    }
    if (seg < a.nseg - 1) {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) s_h[seg][n][lane] = h[n];
      s_sdt[seg][lane] = sdt;
    }
    __syncthreads();
    if (seg > 0) {
      // state entering this segment: fold the summaries of segments 1..seg-1
      // onto segment 0's end state, in order: h <- exp(A * sum dt) h + h_end.
#pragma unroll
      for (int n = 0; n < kScanN; ++n) h[n] = s_h[0][n][lane];
      for (int j = 1; j < seg; ++j) {
        const float sd = s_sdt[j][lane];
#pragma unroll
        for (int n = 0; n < kScanN; ++n) h[n] = fmaf(exp2_fast(c.al2[n] * sd), h[n], s_h[j][n][lane]);
      }
      win[0] = win0[0];
      win[1] = win0[1];
      win[2] = win0[2];
      SSM_RUN(true);
    }
  }
#undef SSM_RUN

  if (seg == a.nseg - 1 && c.act) {
    if (a.state_out) {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) a.state_out[sbase + n] = h[n];
    }
    if (CONV && a.conv_cache_out) {
      const size_t cbase = (static_cast<size_t>(c.b) * a.dim + c.e) * (kConvK - 1);
      a.conv_cache_out[cbase + 0] = win[0];
      a.conv_cache_out[cbase + 1] = win[1];
      a.conv_cache_out[cbase + 2] = win[2];
    }
  }
}

template <typename XT, typename YT, int DTM, bool CONV>
hipError_t launch_scan_t(const ScanLaunch& l, hipStream_t stream) {
  const ScanKernelArgs& a = l.k;
  const unsigned blocks = static_cast<unsigned>(a.batch) * static_cast<unsigned>(a.n_egroups);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((scan_kernel<XT, YT, DTM, CONV>), dim3(blocks), dim3(64 * a.nseg), 0, stream, a,
                     static_cast<const XT*>(a.x), static_cast<const XT*>(a.z), a.dt, a.bcr,
                     static_cast<YT*>(a.y));
  return hipGetLastError();
}

template <typename XT, typename YT, int DTM>
hipError_t pick_conv(const ScanLaunch& l, hipStream_t s) {
  return l.conv ? launch_scan_t<XT, YT, DTM, true>(l, s) : launch_scan_t<XT, YT, DTM, false>(l, s);
}

template <typename XT, typename YT>
hipError_t pick_dt(const ScanLaunch& l, hipStream_t s) {
  switch (l.dt_mode) {
    case 0: return pick_conv<XT, YT, 0>(l, s);
    case 1: return pick_conv<XT, YT, 1>(l, s);
    default: return pick_conv<XT, YT, 2>(l, s);
  }
}

}  // namespace

size_t scan_bcr_bytes(int batch, int seqlen) {
  return static_cast<size_t>(batch) * static_cast<size_t>(seqlen) * kBcrRow * sizeof(float);
}

hipError_t launch_scan(const ScanLaunch& l, hipStream_t stream) {
  const size_t rows = static_cast<size_t>(l.k.batch) * l.k.seqlen;
  if (rows > 0) {
    const size_t total = rows * kBcrRow;
    const unsigned threads = 256;
    const unsigned blocks = static_cast<unsigned>((total + threads - 1) / threads);
    if (l.bc_dtype == kBF16) {
      hipLaunchKernelGGL(pack_bcr_kernel<bf16s>, dim3(blocks), dim3(threads), 0, stream,
                         static_cast<const bf16s*>(l.B), static_cast<const bf16s*>(l.C), l.r, l.bcr_out, rows);
    } else {
      hipLaunchKernelGGL(pack_bcr_kernel<float>, dim3(blocks), dim3(threads), 0, stream,
                         static_cast<const float*>(l.B), static_cast<const float*>(l.C), l.r, l.bcr_out, rows);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (l.x_dtype == kBF16) {
    return l.y_dtype == kBF16 ? pick_dt<bf16s, bf16s>(l, stream) : pick_dt<bf16s, float>(l, stream);
  }
  return l.y_dtype == kBF16 ? pick_dt<float, bf16s>(l, stream) : pick_dt<float, float>(l, stream);
}

}  // namespace ssm
