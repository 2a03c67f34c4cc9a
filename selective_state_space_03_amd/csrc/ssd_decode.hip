// One decode step of the multi-head (SSD-form) scan, in place, for gfx950.
//
// Page "What is the Mamba model?", section "chunkscan": the chunked scan hands
// a per-head state of shape (headdim, d_state) from chunk to chunk; a single
// new token advances that state by one step of the recurrence it summarises,
// with the head's scalar A:
//   S[p][n] <- e^{dt A_h} S[p][n] + dt x[p] B[n]
//   out[p]   = (sum_n C[n] S[p][n] + D x[p]) * SiLU(z[p])   (gate optional)
// which is the chunk formula of that section with a chunk of one token.
//
// The step reads and writes the whole (batch, H, P, N) fp32 state once, so it
// is bound by HBM bandwidth.  N / 8 lanes share one state row (b, h, p): each
// owns 8 consecutive states (two 16-byte non-temporal accesses), so a wave
// covers a contiguous span of rows, and the readout is summed across the
// row's lanes with log2(N / 8) cross-lane adds (N = 8 SPL LPR in the kernel's
// terms, SPL = 8).  B and C rows are shared by
// all P rows of a head (and by all heads of a group) and come from the caches.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// K consecutive elements (K a multiple of 4) from an aligned address
template <int K>
__device__ __forceinline__ void loadk(const float* p, float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    const float4 a = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
}

template <int K>
__device__ __forceinline__ void loadk(const bf16s* p, float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K / 4; ++i) {
    const uint2 r = reinterpret_cast<const uint2*>(p)[i];
    v[4 * i] = __uint_as_float(r.x << 16);
    v[4 * i + 1] = __uint_as_float(r.x & 0xffff0000u);
    v[4 * i + 2] = __uint_as_float(r.y << 16);
    v[4 * i + 3] = __uint_as_float(r.y & 0xffff0000u);
  }
}

// SPL states per lane, LPR = N / SPL lanes per state row; 256 threads hold
// 256 / LPR rows.
template <typename XT, typename BT, typename OT, int N, int SPL>
__global__ __launch_bounds__(256) void ssd_decode_kernel(ChunkDecodeKernelArgs a) {
  constexpr int LPR = N / SPL;
  const int q = threadIdx.x % LPR;
  // rows r = (b H + h) P + p; batch * H * P < 2^31
  const uint32_t rows = a.rows;
  const uint32_t r_raw = blockIdx.x * (256u / LPR) + threadIdx.x / LPR;
  const bool act = r_raw < rows;
  const uint32_t r = act ? r_raw : rows - 1;
  const uint32_t P = static_cast<uint32_t>(a.headdim), H = static_cast<uint32_t>(a.nheads);
  const uint32_t bh = r / P;
  const uint32_t p = r - bh * P;
  const uint32_t b = bh / H;
  const uint32_t h = bh - b * H;
  const uint32_t g = h / static_cast<uint32_t>(a.heads_per_group);

  float4* __restrict__ st4 = reinterpret_cast<float4*>(a.state) + (static_cast<size_t>(r) * N + SPL * q) / 4;
  float sv[SPL];
#pragma unroll
  for (int i = 0; i < SPL / 4; ++i) {
    const float4 v = load_stream(st4 + i);
    sv[4 * i] = v.x; sv[4 * i + 1] = v.y; sv[4 * i + 2] = v.z; sv[4 * i + 3] = v.w;
  }

  const float pre = a.dt[bh] + (a.dt_bias ? a.dt_bias[h] : 0.0f);
  const float dt = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                 : dt_clip(pre, a.dt_min, a.dt_max);
  const float dA = exp2_fast(dt * (a.A[h] * kLog2e));
  const float xv = ld<XT>(a.x, r);
  const float dtx = dt * xv;

  float bv[SPL], cv[SPL];
  const size_t bc0 = (static_cast<size_t>(b) * a.ngroups + g) * N + SPL * q;
  loadk<SPL>(static_cast<const BT*>(a.B) + bc0, bv);
  loadk<SPL>(static_cast<const BT*>(a.C) + bc0, cv);

  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    sv[j] = fmaf(dA, sv[j], dtx * bv[j]);
    acc = fmaf(cv[j], sv[j], acc);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, LPR);

  if (!act) return;
#pragma unroll
  for (int i = 0; i < SPL / 4; ++i)
    store_stream(st4 + i, make_float4(sv[4 * i], sv[4 * i + 1], sv[4 * i + 2], sv[4 * i + 3]));
  if (q == 0) {
    const float d = a.D ? (a.d_per_channel ? a.D[static_cast<size_t>(h) * P + p] : a.D[h]) : 0.0f;
    float y = fmaf(d, xv, acc);
    if (a.z) y *= silu(a.z_bf16 ? ld<bf16s>(a.z, r) : ld<float>(a.z, r));
    st<OT>(a.out, r, y);
  }
}

// States per lane.  At batch 64, 80 heads x 96, N 64 (state 126 MB) the step
// ran at 49.9 us with 8 (5.1 TB/s, the rate of a plain device copy on the same
// machine), 53.1 us with 4 and 87.9 us with 16 (too few waves in flight).
constexpr int kSpl = 8;

template <typename XT, typename BT, typename OT, int N>
hipError_t go(const ChunkDecodeLaunch& l, hipStream_t s) {
  constexpr int spl = kSpl < N ? kSpl : N;
  constexpr unsigned kRowsPerBlock = 256 / (N / spl);
  const unsigned blocks = (l.k.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  return timed_launch(s, [&] {
    hipLaunchKernelGGL((ssd_decode_kernel<XT, BT, OT, N, spl>), dim3(blocks), dim3(256), 0, s, l.k);
  });
}

template <typename XT, typename BT, typename OT>
hipError_t pick_n(const ChunkDecodeLaunch& l, hipStream_t s) {
  switch (l.d_state) {
    case 16: return go<XT, BT, OT, 16>(l, s);
    case 32: return go<XT, BT, OT, 32>(l, s);
    case 64: return go<XT, BT, OT, 64>(l, s);
    default: return go<XT, BT, OT, 128>(l, s);
  }
}

template <typename XT, typename BT>
hipError_t pick_out(const ChunkDecodeLaunch& l, hipStream_t s) {
  return l.out_dtype == kBF16 ? pick_n<XT, BT, bf16s>(l, s) : pick_n<XT, BT, float>(l, s);
}

template <typename XT>
hipError_t pick_bc(const ChunkDecodeLaunch& l, hipStream_t s) {
  return l.bc_dtype == kBF16 ? pick_out<XT, bf16s>(l, s) : pick_out<XT, float>(l, s);
}

}  // namespace

hipError_t launch_chunk_decode(const ChunkDecodeLaunch& l, hipStream_t stream) {
  if (l.k.rows == 0) return hipSuccess;
  return l.x_dtype == kBF16 ? pick_bc<bf16s>(l, stream) : pick_bc<float>(l, stream);
}

}  // namespace ssm
