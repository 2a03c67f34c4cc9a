// One autoregressive decode step, in place, for gfx950.
//
// Page "Axon-SSM: selective state space model", section "Autoregressive
// decoding": concatenate conv_cache with the new token, run exactly one step
// of the scan from the previous ssm_state, return the updated
// [conv_cache, ssm_state].  Per channel: window = (cache[0..2], x) -> causal
// depthwise conv (k=4) + SiLU -> dt = clip(softplus(dt_proj + dt_bias)) ->
// h = exp(dt*A) h + dt*B*u -> y = (C . h + D*u) * SiLU(z); cache <- window[1..3].
//
// The step reads and writes the whole (batch, E, 16) fp32 state, so it is
// bound by HBM bandwidth.  Four lanes share one (batch, channel): each owns 4
// of its 16 states, so every state load and store is one 16-byte access per
// lane and a wave's accesses cover one contiguous 1 KiB span.  The readout is
// summed across the four lanes with two cross-lane adds.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// The state is read once and written once per step, with non-temporal
// accesses (load_stream / store_stream): they keep it from displacing the
// parameters (A, conv weights, ...) that every step re-reads from the caches,
// and measured ~12% faster at batch 64.

// 4 consecutive elements from a 4-element-aligned address
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x;
  v[1] = f.y;
  v[2] = f.z;
  v[3] = f.w;
}

__device__ __forceinline__ void load4(const bf16s* p, float (&v)[4]) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(r.x << 16);
  v[1] = __uint_as_float(r.x & 0xffff0000u);
  v[2] = __uint_as_float(r.y << 16);
  v[3] = __uint_as_float(r.y & 0xffff0000u);
}

// ZOH: B enters as ((e^{dt A} - 1) / A) B u instead of dt B u.
template <typename XT, typename YT, typename BT, int DTM, bool CONV, bool ZOH>
__global__ __launch_bounds__(256) void decode_kernel(DecodeKernelArgs a) {
  using DT = typename std::conditional<DTM == 2, bf16s, float>::type;
  const int q = threadIdx.x & 3;
  // (b, e) flattened; batch * dim < 2^31, so 32-bit index arithmetic
  const uint32_t total = static_cast<uint32_t>(a.batch) * static_cast<uint32_t>(a.dim);
  const uint32_t ch_raw = blockIdx.x * 64u + (threadIdx.x >> 2);
  const bool act = ch_raw < total;
  const uint32_t ch = act ? ch_raw : total - 1;
  const uint32_t b = ch / static_cast<uint32_t>(a.dim);
  const uint32_t e = ch - b * static_cast<uint32_t>(a.dim);

  float4* __restrict__ state4 = reinterpret_cast<float4*>(a.state);
  const float4 hs = load_stream(state4 + static_cast<size_t>(ch) * 4 + q);
  const float4 a4 = reinterpret_cast<const float4*>(a.A)[static_cast<size_t>(e) * 4 + q];
  const float xr = ld<XT>(a.x, ch);

  float c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
  float u = xr;
  if (CONV) {
    // lanes 0..2 of the quad each load one cache entry; the quad shares them
    const float cq = q < 3 ? __builtin_nontemporal_load(a.conv_cache + static_cast<size_t>(ch) * 3 + q) : 0.0f;
    c0 = __shfl(cq, 0, 4);
    c1 = __shfl(cq, 1, 4);
    c2 = __shfl(cq, 2, 4);
    const float4 w = reinterpret_cast<const float4*>(a.conv_w)[e];
    const float cb = a.conv_b ? a.conv_b[e] : 0.0f;
    const float xc = fmaf(w.x, c0, fmaf(w.y, c1, fmaf(w.z, c2, fmaf(w.w, xr, cb))));
    u = silu(xc);
  }
  const float dtb = a.dt_bias ? a.dt_bias[e] : 0.0f;
  const float pre = (DTM == 0) ? fmaf(a.dt_w[e], static_cast<const float*>(a.dt)[b], dtb)
                               : to_f32(static_cast<const DT*>(a.dt)[ch]) + dtb;
  const float dt = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                 : dt_clip(pre, a.dt_min, a.dt_max);
  const float dtu = dt * u;

  // this lane's 4 entries of B and C: one aligned 4-element load each
  float bq[4], cq4[4];
  load4(static_cast<const BT*>(a.B) + static_cast<size_t>(b) * kScanN + 4 * q, bq);
  load4(static_cast<const BT*>(a.C) + static_cast<size_t>(b) * kScanN + 4 * q, cq4);
  const float hin[4] = {hs.x, hs.y, hs.z, hs.w};
  const float av[4] = {a4.x, a4.y, a4.z, a4.w};
  float hout[4];
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float an = exp2_fast(dt * (av[j] * kLog2e));
    if (ZOH) {
      const float coef = dt * zoh_phi(dt * av[j], an);
      hout[j] = fmaf(an, hin[j], (coef * u) * bq[j]);
    } else {
      hout[j] = fmaf(an, hin[j], dtu * bq[j]);
    }
    acc = fmaf(cq4[j], hout[j], acc);
  }
  acc += __shfl_xor(acc, 1, 4);
  acc += __shfl_xor(acc, 2, 4);

  if (!act) return;
  store_stream(state4 + static_cast<size_t>(ch) * 4 + q, make_float4(hout[0], hout[1], hout[2], hout[3]));
  if (q == 0) {
    float yv = fmaf(a.D ? a.D[e] : 0.0f, u, acc);
    if (a.has_z) yv *= silu(ld<XT>(a.z, ch));
    st<YT>(a.y, ch, yv);
  }
  if (CONV && q < 3) {
    const float nv = (q == 0) ? c1 : (q == 1) ? c2 : xr;
    __builtin_nontemporal_store(nv, a.conv_cache + static_cast<size_t>(ch) * 3 + q);
  }
}

template <typename XT, typename YT, typename BT, int DTM>
hipError_t go(const DecodeLaunch& l, hipStream_t s) {
  const size_t total = static_cast<size_t>(l.k.batch) * l.k.dim;
  const unsigned blocks = static_cast<unsigned>((total + 63) / 64);
  return timed_launch(s, [&] {
    if (l.zoh) {
      if (l.conv)
        hipLaunchKernelGGL((decode_kernel<XT, YT, BT, DTM, true, true>), dim3(blocks), dim3(256), 0, s, l.k);
      else
        hipLaunchKernelGGL((decode_kernel<XT, YT, BT, DTM, false, true>), dim3(blocks), dim3(256), 0, s, l.k);
    } else if (l.conv) {
      hipLaunchKernelGGL((decode_kernel<XT, YT, BT, DTM, true, false>), dim3(blocks), dim3(256), 0, s, l.k);
    } else {
      hipLaunchKernelGGL((decode_kernel<XT, YT, BT, DTM, false, false>), dim3(blocks), dim3(256), 0, s, l.k);
    }
  });
}

template <typename XT, typename YT, typename BT>
hipError_t pick_dt(const DecodeLaunch& l, hipStream_t s) {
  switch (l.dt_mode) {
    case 0: return go<XT, YT, BT, 0>(l, s);
    case 1: return go<XT, YT, BT, 1>(l, s);
    default: return go<XT, YT, BT, 2>(l, s);
  }
}

template <typename XT, typename YT>
hipError_t pick_bc(const DecodeLaunch& l, hipStream_t s) {
  return l.bc_dtype == kBF16 ? pick_dt<XT, YT, bf16s>(l, s) : pick_dt<XT, YT, float>(l, s);
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& l, hipStream_t stream) {
  if (l.x_dtype == kBF16) {
    return l.y_dtype == kBF16 ? pick_bc<bf16s, bf16s>(l, stream) : pick_bc<bf16s, float>(l, stream);
  }
  return l.y_dtype == kBF16 ? pick_bc<float, bf16s>(l, stream) : pick_bc<float, float>(l, stream);
}

}  // namespace ssm
