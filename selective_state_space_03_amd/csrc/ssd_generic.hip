// Multi-head chunked scan (SSD form) for the shapes the tuned MFMA kernel of
// ssd_chunk.hip does not take: any chunk size up to 256, any d_state and
// headdim up to 128, x / B / C / z in fp32 or bf16.  Same computation, in
// fp32 on the vector ALUs, as three launches:
//
//   1. per (batch, chunk, head): the chunk's own final state from zero,
//        S_c[p, n] = sum_s e^{dA[Q-1] - dA[s]} dt[s] x[s, p] B[s, n],
//      and its decay e^{dA[Q-1]};
//   2. per (batch, head, p, n): the chunks in order, S <- e^{dA[Q-1]} S + S_c
//      (the inter-chunk scan over chunk-final states), leaving in chunk c's
//      slot the state that enters chunk c;
//   3. per (batch, chunk, head): the chunk's outputs,
//        out[l, p] = sum_{s<=l} (C[l] . B[s]) e^{dA[l] - dA[s]} dt[s] x[s, p]
//                  + e^{dA[l]} sum_n C[l, n] S_in[p, n] + D x[l, p],
//      gated by SiLU(z) when z is given.
//
// Page "What is the Mamba model?", sections "chunkscan" (intra-chunk scan,
// inter-chunk scan over the chunk-final states, combination) and "chunkscan
// implementation (TileLang)" (the chunk output formula), with dA the
// inclusive cumulative sum of dt A_h inside the chunk.  The cumulative sums
// are taken in fp64 and only their differences are rounded to fp32 before the
// exponential: a difference of two fp32 sums near the end of a long chunk
// would carry an absolute error of an ulp of the sum (3e-5 at |dA| = 400) into
// every decay factor.  A sequence that is not a whole number of chunks ends
// with a shorter chunk handled by the same formulas over its own length.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kGT = 256;        // threads per workgroup
constexpr int kGRows = 32;      // token positions per tile
constexpr int kPad = 1;         // padding of LDS rows (a column walk across rows spreads over the banks)
constexpr int kAccS = kSsdGenMaxP * kSsdGenMaxN / kGT;  // chunk-state outputs per thread at most
constexpr int kAccO = kGRows * kSsdGenMaxP / kGT;        // chunk outputs per thread at most

__device__ __forceinline__ float ldv(const void* p, size_t i, int bf16) {
  return bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16)
              : static_cast<const float*>(p)[i];
}

// (batch, chunk, head) of a workgroup, head fastest.
__device__ __forceinline__ void decode_bch(const ChunkGenericArgs& a, int& b, int& c, int& h) {
  int id = blockIdx.x;
  h = id % a.nheads;
  id /= a.nheads;
  c = id % a.nchunks;
  b = id / a.nchunks;
}

// dt of every position of the chunk into dts[], and the inclusive cumulative
// sum of dt A_h into cum[] (fp64).  Wave 0 scans: each lane sums four
// consecutive positions, the lanes' totals are scanned with shuffles, and
// every lane adds its prefix back.  Ends with a barrier.
__device__ void chunk_prologue(const ChunkGenericArgs& a, int b, int h, int t0, int qc, float* dts, double* cum) {
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.0f;
  for (int s = threadIdx.x; s < qc; s += kGT) {
    const float pre = a.dt[(static_cast<size_t>(b) * a.seqlen + t0 + s) * a.nheads + h] + dtb;
    dts[s] = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                           : dt_clip(pre, a.dt_min, a.dt_max);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const double Ah = static_cast<double>(a.A[h]);
    double v[4];
    double run = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * lane + j;
      run += (s < qc) ? static_cast<double>(dts[s]) * Ah : 0.0;
      v[j] = run;
    }
    double pre = run;  // inclusive scan of the lanes' totals
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(pre, off, 64);
      if (lane >= off) pre += o;
    }
    const double base = pre - run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * lane + j;
      if (s < qc) cum[s] = base + v[j];
    }
  }
  __syncthreads();
}

// e^{d} for an fp64 exponent difference: rounded to fp32 once, then the
// transcendental unit.
__device__ __forceinline__ float exp_diff(double d) {
  return exp2_fast(static_cast<float>(d * 1.4426950408889634));
}

__global__ __launch_bounds__(kGT) void ssdg_state_kernel(ChunkGenericArgs a) {
  __shared__ double cum[kSsdGenMaxQ];
  __shared__ float dts[kSsdGenMaxQ];
  __shared__ float w[kSsdGenMaxQ];
  __shared__ float xs[kGRows][kSsdGenMaxP + kPad];
  __shared__ float bs[kGRows][kSsdGenMaxN + kPad];
  int b, c, h;
  decode_bch(a, b, c, h);
  const int H = a.nheads, P = a.headdim, N = a.d_state, Q = a.chunk_size;
  const int g = h / (H / a.ngroups);
  const int t0 = c * Q, qc = min(Q, a.seqlen - t0);
  chunk_prologue(a, b, h, t0, qc, dts, cum);
  const double last = cum[qc - 1];
  for (int s = threadIdx.x; s < qc; s += kGT) w[s] = exp_diff(last - cum[s]) * dts[s];
  const size_t bch = (static_cast<size_t>(b) * a.nchunks + c) * H + h;
  if (threadIdx.x == 0) a.chunk_decay[bch] = exp_diff(last);
  const int nout = P * N;
  float acc[kAccS];
#pragma unroll
  for (int k = 0; k < kAccS; ++k) acc[k] = 0.0f;
  for (int s0 = 0; s0 < qc; s0 += kGRows) {
    const int rows = min(kGRows, qc - s0);
    __syncthreads();  // w is written; the previous tile has been read
    for (int i = threadIdx.x; i < rows * P; i += kGT) {
      const int r = i / P, p = i % P;
      const size_t t = static_cast<size_t>(b) * a.seqlen + t0 + s0 + r;
      xs[r][p] = ldv(a.x, (t * H + h) * P + p, a.x_bf16) * w[s0 + r];
    }
    for (int i = threadIdx.x; i < rows * N; i += kGT) {
      const int r = i / N, n = i % N;
      const size_t t = static_cast<size_t>(b) * a.seqlen + t0 + s0 + r;
      bs[r][n] = ldv(a.B, (t * a.ngroups + g) * N + n, a.bc_bf16);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kAccS; ++k) {
      const int o = threadIdx.x + k * kGT;
      if (o < nout) {
        const int p = o / N, n = o % N;
        float v = acc[k];
        for (int r = 0; r < rows; ++r) v = fmaf(xs[r][p], bs[r][n], v);
        acc[k] = v;
      }
    }
  }
  float* out = a.chunk_state + bch * nout;
#pragma unroll
  for (int k = 0; k < kAccS; ++k) {
    const int o = threadIdx.x + k * kGT;
    if (o < nout) out[o] = acc[k];
  }
}

// One thread per (batch, head, p, n): the chunks in order.  Slot c of the
// chunk states is overwritten with the state entering chunk c.
__global__ __launch_bounds__(kGT) void ssdg_pass_kernel(ChunkGenericArgs a) {
  const int H = a.nheads, nout = a.headdim * a.d_state;
  const size_t e = static_cast<size_t>(blockIdx.x) * kGT + threadIdx.x;
  const size_t per_batch = static_cast<size_t>(H) * nout;
  if (e >= static_cast<size_t>(a.batch) * per_batch) return;
  const int b = static_cast<int>(e / per_batch);
  const size_t rem = e % per_batch;
  const int h = static_cast<int>(rem / nout);
  const int o = static_cast<int>(rem % nout);
  float S = a.state_in ? a.state_in[e] : 0.0f;
#pragma unroll 4
  for (int c = 0; c < a.nchunks; ++c) {
    const size_t bch = (static_cast<size_t>(b) * a.nchunks + c) * H + h;
    float* slot = a.chunk_state + bch * nout + o;
    const float sc = *slot;
    const float dec = a.chunk_decay[bch];
    *slot = S;
    S = fmaf(dec, S, sc);
  }
  if (a.state_out) a.state_out[e] = S;
}

template <typename OT>
__global__ __launch_bounds__(kGT) void ssdg_out_kernel(ChunkGenericArgs a) {
  __shared__ double cum[kSsdGenMaxQ];
  __shared__ float dts[kSsdGenMaxQ];
  __shared__ float sin_[kSsdGenMaxP * kSsdGenMaxN];       // state entering the chunk, [p][n]
  __shared__ float cs[kGRows][kSsdGenMaxN + kPad];        // C rows of the output block
  __shared__ float bs[kGRows][kSsdGenMaxN + kPad];        // B rows of the source block
  __shared__ float xs[kGRows][kSsdGenMaxP + kPad];        // x rows of the source block
  __shared__ float m[kGRows][kGRows + kPad];              // masked, decayed C B^T dt of the two blocks
  int b, c, h;
  decode_bch(a, b, c, h);
  const int H = a.nheads, P = a.headdim, N = a.d_state, Q = a.chunk_size;
  const int g = h / (H / a.ngroups);
  const int t0 = c * Q, qc = min(Q, a.seqlen - t0);
  chunk_prologue(a, b, h, t0, qc, dts, cum);
  const size_t bch = (static_cast<size_t>(b) * a.nchunks + c) * H + h;
  const float* sslot = a.chunk_state + bch * P * N;
  for (int i = threadIdx.x; i < P * N; i += kGT) sin_[i] = sslot[i];
  const float dhead = (a.D && !a.d_per_channel) ? a.D[h] : 0.0f;
  const size_t tb = static_cast<size_t>(b) * a.seqlen + t0;  // first token of the chunk
  for (int l0 = 0; l0 < qc; l0 += kGRows) {
    const int lr = min(kGRows, qc - l0);
    __syncthreads();  // sin_ is written; the previous block's tiles have been read
    for (int i = threadIdx.x; i < lr * N; i += kGT) {
      const int r = i / N, n = i % N;
      cs[r][n] = ldv(a.C, ((tb + l0 + r) * a.ngroups + g) * N + n, a.bc_bf16);
    }
    __syncthreads();
    // the incoming state's readout, e^{dA[l]} C[l] . S_in[p]
    float acc[kAccO];
#pragma unroll
    for (int k = 0; k < kAccO; ++k) {
      const int o = threadIdx.x + k * kGT;
      acc[k] = 0.0f;
      if (o < lr * P) {
        const int r = o / P, p = o % P;
        float v = 0.0f;
        for (int n = 0; n < N; ++n) v = fmaf(cs[r][n], sin_[p * N + n], v);
        acc[k] = v * exp_diff(cum[l0 + r]);
      }
    }
    // the intra-chunk sum over source blocks up to the diagonal one
    for (int s0 = 0; s0 < l0 + lr; s0 += kGRows) {
      const int sr = min(kGRows, qc - s0);
      __syncthreads();  // the previous source block has been read
      for (int i = threadIdx.x; i < sr * N; i += kGT) {
        const int r = i / N, n = i % N;
        bs[r][n] = ldv(a.B, ((tb + s0 + r) * a.ngroups + g) * N + n, a.bc_bf16);
      }
      for (int i = threadIdx.x; i < sr * P; i += kGT) {
        const int r = i / P, p = i % P;
        xs[r][p] = ldv(a.x, ((tb + s0 + r) * H + h) * P + p, a.x_bf16);
      }
      __syncthreads();
      for (int i = threadIdx.x; i < kGRows * kGRows; i += kGT) {
        const int r = i / kGRows, q = i % kGRows;
        const int l = l0 + r, s = s0 + q;
        float v = 0.0f;
        if (r < lr && q < sr && s <= l) {
          float dot = 0.0f;
          for (int n = 0; n < N; ++n) dot = fmaf(cs[r][n], bs[q][n], dot);
          v = dot * exp_diff(cum[l] - cum[s]) * dts[s];
        }
        m[r][q] = v;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kAccO; ++k) {
        const int o = threadIdx.x + k * kGT;
        if (o < lr * P) {
          const int r = o / P, p = o % P;
          float v = acc[k];
          for (int q = 0; q < sr; ++q) v = fmaf(m[r][q], xs[q][p], v);
          acc[k] = v;
        }
      }
    }
    // skip, gate, store
#pragma unroll
    for (int k = 0; k < kAccO; ++k) {
      const int o = threadIdx.x + k * kGT;
      if (o < lr * P) {
        const int r = o / P, p = o % P;
        const size_t idx = ((tb + l0 + r) * H + h) * P + p;
        const float dv = a.D ? (a.d_per_channel ? a.D[h * P + p] : dhead) : 0.0f;
        float y = fmaf(dv, ldv(a.x, idx, a.x_bf16), acc[k]);
        if (a.z) y *= silu(ldv(a.z, idx, a.z_bf16));
        st<OT>(a.out, idx, y);
      }
    }
  }
}

}  // namespace

size_t chunk_generic_workspace_bytes(int batch, int seqlen, int nheads, int headdim, int d_state, int chunk_size) {
  if (batch <= 0 || seqlen <= 0 || chunk_size <= 0) return 0;
  const size_t nch = (static_cast<size_t>(seqlen) + chunk_size - 1) / chunk_size;
  const size_t bch = static_cast<size_t>(batch) * nch * nheads;
  const size_t states = (bch * headdim * d_state * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return states + ((bch * sizeof(float) + 255) & ~static_cast<size_t>(255));
}

size_t chunk_generic_decay_offset(int batch, int seqlen, int nheads, int headdim, int d_state, int chunk_size) {
  const size_t nch = (static_cast<size_t>(seqlen) + chunk_size - 1) / chunk_size;
  const size_t bch = static_cast<size_t>(batch) * nch * nheads;
  return (bch * headdim * d_state * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

// With no token (nchunks = 0) only the pass kernel runs: it hands the
// incoming state (or zeros) to state_out.
hipError_t launch_chunk_generic(const ChunkGenericArgs& a, hipStream_t stream) {
  const unsigned bch = static_cast<unsigned>(static_cast<size_t>(a.batch) * a.nchunks * a.nheads);
  const size_t elems = static_cast<size_t>(a.batch) * a.nheads * a.headdim * a.d_state;
  if (elems == 0) return hipSuccess;
  if (bch > 0) {
    hipLaunchKernelGGL(ssdg_state_kernel, dim3(bch), dim3(kGT), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(ssdg_pass_kernel, dim3(static_cast<unsigned>((elems + kGT - 1) / kGT)), dim3(kGT), 0, stream,
                     a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || bch == 0) return err;
  return timed_launch(stream, [&] {
    if (a.out_bf16)
      hipLaunchKernelGGL(ssdg_out_kernel<bf16s>, dim3(bch), dim3(kGT), 0, stream, a);
    else
      hipLaunchKernelGGL(ssdg_out_kernel<float>, dim3(bch), dim3(kGT), 0, stream, a);
  });
}

}  // namespace ssm
