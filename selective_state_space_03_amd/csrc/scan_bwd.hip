// Backward of the scan stage for gfx950, with recomputation.
//
// Page "Mamba/SSM basics" (molayo), the section after "Technical details":
// production training recomputes intermediate states in the backward pass
// instead of materialising them in HBM.  Here nothing of size (L, E, N) is
// stored: the sequence is cut into segments of kSeg steps and
//   1. bwd_summary: per segment, the state at its end starting from zero and
//      the reverse-time gradient at its start starting from zero (both linear
//      in what enters the segment), and the sum of dt over it;
//   2. bwd_compose: per (batch, channel, state), the state entering every
//      segment (forward through the segments, from the initial state) and
//      the gradient entering every segment from its right (backward, from the
//      gradient on the final state), which also gives the initial state's
//      gradient;
//   3. bwd_main: a wave walks a run of kBwdRun segments, last to first; per
//      segment the states of its kSeg steps are recomputed into registers
//      and walked backward, producing every gradient of the step, and the
//      reverse-time gradient passes on to the segment before in registers
//      (only the run's last segment takes it from the composition).
//      Gradients summed over channels (B, C, a rank-1 dt) are summed over the
//      wave's 16 channels in registers and over the workgroup's kBwdWg waves
//      in LDS, and leave as one partial per (step, 64 channels); gradients
//      summed over time (A, D, dt_w, dt_bias, the conv weights and bias)
//      leave as one partial per run.  The conv's transpose is applied on the
//      way: walking backward, the four lanes of a channel hold the conv-output
//      gradients of steps t .. t+3, so dx_t is a quad sum; only the first three
//      steps of a run are kept, for the last three dx of the run before it;
//   4. the run-boundary terms of dx, the conv cache's gradient and the
//      reductions, all in a fixed order.
// A wave first stages its segment's inputs in LDS (x with the conv's three
// earlier steps, dt's pre-activation, dy, z for its 16 channels; B and C of
// the segment), with coalesced loads issued together, so the steps read LDS
// instead of waiting on a dozen dependent global loads each.
// Reverse recurrence (G_t = dL/dh_t, Q_t = a_t G_t, a_t = exp(dt_t A)):
//   G_t = dyc_t C_t + Q_{t+1},  dyc_t = dy_t SiLU(z_t),  Q at the end = dL/dh_L.
// Lanes: 4 per (batch, channel), each holding 4 of the 16 states, so a
// segment's 16 recomputed states take 64 registers per lane (32 steps spilled
// the history to scratch memory) and the sums over states are two cross-lane
// adds.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kSeg = kBwdSeg;  // steps per segment (16)

__device__ __forceinline__ float ldx(const void* p, size_t i, bool bf) {
  return bf ? ld<bf16s>(p, i) : ld<float>(p, i);
}

// 4 consecutive entries (f32 or bf16) from a 4-element-aligned address
__device__ __forceinline__ void load4v(const void* p, size_t i, bool bf, float (&v)[4]) {
  if (bf) {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

__device__ __forceinline__ float dsilu(float x) {
  const float s = rcp_fast(1.0f + exp2_fast(-x * kLog2e));
  return s * (1.0f + x * (1.0f - s));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// sum over the 4 lanes of a channel (DPP quad permutations 1 0 3 2, 2 3 0 1)
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v;
}

// v of the same lane in the other 16-lane row of its pair (rows 0 <-> 1,
// 2 <-> 3) and in the other 32-lane half, by the permlane swaps, each added
// to v
__device__ __forceinline__ float add_row_swap(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, static_cast<int>(p[0])) + __builtin_bit_cast(float, static_cast<int>(p[1]));
}
__device__ __forceinline__ float add_half_swap(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, static_cast<int>(p[0])) + __builtin_bit_cast(float, static_cast<int>(p[1]));
}

// sum over the 16 channels of the wave (lanes with the same state quarter):
// the 4 channels of a 16-lane row by DPP row rotations, then across rows
__device__ __forceinline__ float chan_sum(float v) {
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return add_half_swap(add_row_swap(v));
}


// One segment's inputs for the 16 channels of a wave, with the per-channel
// quantities of each step computed once (not by each of a channel's four
// lanes).  Rows past the end of the sequence are not read.
struct SegStage {
  float xr[kSeg + 3][16];  // raw x at t0 - 3 + i (the conv cache or zeros before the start)
  float u[kSeg][16];       // u_t = SiLU(conv) (or x)
  float dt[kSeg][16];      // dt_t
  float dpf[kSeg][16];     // d dt / d pre: softplus' strictly inside the clip, else 0
  float dyc[kSeg][16];     // dy_t SiLU(z_t) (or dy_t)
  float dzf[kSeg][16];     // dy_t SiLU'(z_t)
  float dsx[kSeg][16];     // SiLU'(conv output) (or 1)
  float B[kSeg][kScanN];
  float C[kSeg][kScanN];
};

// Stage segment [t0, t1) of batch b for channel group gw: lane (r, j) loads
// channel j of rows r, r + 4, ... and computes those rows' per-channel
// quantities (with FULL, also the derivative factors only the main pass
// uses); B and C rows are contiguous (4 values a lane).
template <bool FULL>
__device__ __forceinline__ void stage_segment(const BwdArgs& a, int b, int gw, int t0, int t1, SegStage& S) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, r = lane >> 4;
  const int e = min(16 * gw + j, a.dim - 1);
  const size_t row0 = static_cast<size_t>(b) * a.seqlen;
  const float dtw = a.dt_rank1 ? a.dt_w[e] : 0.0f;
  const float dtb = a.dt_bias ? a.dt_bias[e] : 0.0f;
#pragma unroll
  for (int i0 = 0; i0 < kSeg + 3; i0 += 4) {
    const int i = i0 + r;
    const int t = t0 - 3 + i;
    if (i < kSeg + 3 && t < t1) {
      float v = 0.0f;
      if (t >= 0)
        v = ldx(a.x, (row0 + t) * a.dim + e, a.x_bf16);
      else if (a.conv_cache_in)
        v = a.conv_cache_in[(static_cast<size_t>(b) * a.dim + e) * 3 + (3 + t)];
      S.xr[i][j] = v;
    }
  }
  float pre[kSeg / 4], dy[kSeg / 4], z[kSeg / 4];
#pragma unroll
  for (int k = 0; k < kSeg / 4; ++k) {
    const int t = t0 + r + 4 * k;
    pre[k] = dy[k] = z[k] = 0.0f;
    if (t < t1) {
      const size_t be = (row0 + t) * a.dim + e;
      pre[k] = a.dt_rank1 ? fmaf(dtw, static_cast<const float*>(a.dt)[row0 + t], dtb) : ldx(a.dt, be, a.dt_bf16) + dtb;
      dy[k] = ldx(a.dy, be, a.dy_bf16);
      if (a.z) z[k] = ldx(a.z, be, a.x_bf16);
    }
  }
  if (t0 + (lane >> 2) < t1) {
    float v[4];
    const size_t o = (row0 + t0) * kScanN + 4 * lane;
    load4v(a.B, o, a.bc_bf16, v);
    *reinterpret_cast<float4*>(&S.B[lane >> 2][4 * (lane & 3)]) = make_float4(v[0], v[1], v[2], v[3]);
    load4v(a.C, o, a.bc_bf16, v);
    *reinterpret_cast<float4*>(&S.C[lane >> 2][4 * (lane & 3)]) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // the wave's own LDS writes complete before its reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f;
  if (a.conv_w) {
    const float4 w = reinterpret_cast<const float4*>(a.conv_w)[e];
    cw[0] = w.x;
    cw[1] = w.y;
    cw[2] = w.z;
    cw[3] = w.w;
    cb = a.conv_b ? a.conv_b[e] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kSeg / 4; ++k) {
    const int i = r + 4 * k;
    if (t0 + i < t1) {
      float u, dsx = 1.0f;
      if (a.conv_w) {
        const float xc = fmaf(cw[0], S.xr[i][j], fmaf(cw[1], S.xr[i + 1][j], fmaf(cw[2], S.xr[i + 2][j],
                                                                                 fmaf(cw[3], S.xr[i + 3][j], cb))));
        u = silu(xc);
        if (FULL) dsx = dsilu(xc);
      } else {
        u = S.xr[i + 3][j];
      }
      float sp, dsp = 1.0f;
      if (a.dt_softplus) {
        sp = softplus(pre[k]);
        if (FULL) dsp = rcp_fast(1.0f + exp2_fast(-pre[k] * kLog2e));
      } else {
        sp = pre[k];
      }
      S.u[i][j] = u;
      S.dt[i][j] = fminf(fmaxf(sp, a.dt_min), a.dt_max);
      S.dyc[i][j] = a.z ? dy[k] * silu(z[k]) : dy[k];
      if (FULL) {
        const bool inside = sp > a.dt_min && sp < a.dt_max;
        S.dpf[i][j] = inside ? dsp : 0.0f;
        S.dsx[i][j] = dsx;
        S.dzf[i][j] = a.z ? dy[k] * dsilu(z[k]) : 0.0f;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Per-lane context: which (batch, channel, state quarter) and its constants.
struct Lane {
  const BwdArgs& a;
  int b, e, q, gw;
  bool act;
  float Al2[4], An[4];  // A[e][4q + j] log2(e), A[e][4q + j]
  float dtw, d;
  float wt;             // conv weight 3 - q: the tap that meets the conv-output gradient of step t + q

  // live: the wave has a channel group (false for the spare waves of a
  // ragged last workgroup, which compute on a valid group and write nothing)
  __device__ Lane(const BwdArgs& args, int b_, int gw_, bool live = true) : a(args), b(b_), gw(gw_) {
    const int lane = threadIdx.x & 63;
    q = lane & 3;
    const int e_raw = 16 * gw + (lane >> 2);
    act = live && e_raw < a.dim;
    e = act ? e_raw : a.dim - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      An[j] = a.A[static_cast<size_t>(e) * kScanN + 4 * q + j];
      Al2[j] = An[j] * kLog2e;
    }
    dtw = a.dt_rank1 ? a.dt_w[e] : 0.0f;
    d = a.D ? a.D[e] : 0.0f;
    wt = a.conv_w ? a.conv_w[static_cast<size_t>(e) * 4 + (3 - q)] : 0.0f;
  }
  __device__ size_t be(int t) const { return (static_cast<size_t>(b) * a.seqlen + t) * a.dim + e; }
  // staged value of step i of the segment for this lane's channel (slot lane / 4)
  __device__ static float at(const float (*M)[16], int i) { return M[i][(threadIdx.x & 63) >> 2]; }
  __device__ void sbc(const float (*M)[kScanN], int i, float (&v)[4]) const {
    const float4 f = *reinterpret_cast<const float4*>(&M[i][4 * q]);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  __device__ void decay(float dt, float (&av)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = exp2_fast(dt * Al2[j]);
  }
};

// wave -> (batch, channel group of 16, segment)
__device__ __forceinline__ void wave_ids(const BwdArgs& a, int& b, int& gw, int& s) {
  int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  gw = w % a.ngroups16;
  w /= a.ngroups16;
  b = w % a.batch;
  s = w / a.batch;
}

__global__ __launch_bounds__(256) void bwd_summary(BwdArgs a) {
  __shared__ SegStage stage[4];
  int b, gw, s;
  wave_ids(a, b, gw, s);
  if (s >= a.nseg) return;
  const Lane c(a, b, gw);
  const int t0 = s * kSeg, t1 = min(a.seqlen, t0 + kSeg);
  SegStage& S = stage[threadIdx.x >> 6];
  stage_segment<false>(a, b, gw, t0, t1, S);
  // the decays of the forward walk are kept for the backward one
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sdt = 0.0f;
  float ah[kSeg][4];
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    if (t0 + i < t1) {
      float bv[4];
      const float u = Lane::at(S.u, i);
      const float dt = Lane::at(S.dt, i);
      c.sbc(S.B, i, bv);
      c.decay(dt, ah[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = fmaf(ah[i][j], h[j], dt * u * bv[j]);
      sdt += dt;
    }
  }
  float Q[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = kSeg - 1; i >= 0; --i) {
    if (t0 + i < t1) {
      float cv[4];
      c.sbc(S.C, i, cv);
      const float dyc = Lane::at(S.dyc, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) Q[j] = ah[i][j] * fmaf(dyc, cv[j], Q[j]);
    }
  }
  if (!c.act) return;
  const size_t o = ((static_cast<size_t>(b) * a.nseg + s) * a.dim + c.e) * kScanN + 4 * c.q;
  *reinterpret_cast<float4*>(a.hs + o) = make_float4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<float4*>(a.qs + o) = make_float4(Q[0], Q[1], Q[2], Q[3]);
  if (c.q == 0) a.sdt[(static_cast<size_t>(b) * a.nseg + s) * a.dim + c.e] = sdt;
}

// one thread per (batch, channel, state)
__global__ __launch_bounds__(256) void bwd_compose(BwdArgs a) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = static_cast<size_t>(a.batch) * a.dim * kScanN;
  if (i >= total) return;
  const int n = static_cast<int>(i % kScanN);
  const int e = static_cast<int>((i / kScanN) % a.dim);
  const int b = static_cast<int>(i / (static_cast<size_t>(kScanN) * a.dim));
  const float al2 = a.A[static_cast<size_t>(e) * kScanN + n] * kLog2e;
  auto at = [&](int s) { return ((static_cast<size_t>(b) * a.nseg + s) * a.dim + e) * kScanN + n; };
  auto sd = [&](int s) { return a.sdt[(static_cast<size_t>(b) * a.nseg + s) * a.dim + e]; };
  // blocks of 8 segments: the block's loads are all issued before its chain
  constexpr int kB = 8;
  float hcur = a.state_in ? a.state_in[(static_cast<size_t>(b) * a.dim + e) * kScanN + n] : 0.0f;
  for (int s0 = 0; s0 < a.nseg; s0 += kB) {
    float loc[kB], dec[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = min(s0 + k, a.nseg - 1);
      loc[k] = a.hs[at(s)];
      dec[k] = sd(s);
    }
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      if (s0 + k < a.nseg) {
        a.hs[at(s0 + k)] = hcur;  // the state entering segment s0 + k
        hcur = fmaf(exp2_fast(al2 * dec[k]), hcur, loc[k]);
      }
    }
  }
  float qcur = a.dstate_out ? a.dstate_out[(static_cast<size_t>(b) * a.dim + e) * kScanN + n] : 0.0f;
  for (int s0 = a.nseg - 1; s0 >= 0; s0 -= kB) {
    float loc[kB], dec[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int s = max(s0 - k, 0);
      loc[k] = a.qs[at(s)];
      dec[k] = sd(s);
    }
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      if (s0 - k >= 0) {
        // the gradient entering segment s0 - k from its right, kept where a
        // run of the main pass starts (its last segment)
        const int s = s0 - k;
        if (s % kBwdRun == kBwdRun - 1 || s == a.nseg - 1) a.qs[at(s)] = qcur;
        qcur = fmaf(exp2_fast(al2 * dec[k]), qcur, loc[k]);
      }
    }
  }
  if (a.dstate_in) a.dstate_in[(static_cast<size_t>(b) * a.dim + e) * kScanN + n] = qcur;
}

// Workgroup (block of kBwdWg channel groups, batch, run of segments); wave
// w takes group kBwdWg * block + w.  Three waves per SIMD.
__global__ __launch_bounds__(256, 3) void bwd_main(BwdArgs a) {
  __shared__ SegStage stage[4];
  // per wave and step of the segment: dB over its 16 channels, then dC, then
  // the rank-1 dt's channel sum (rows padded to 16-byte multiples)
  constexpr int kPart = 2 * kScanN + 1, kPartRow = (kPart + 3) / 4 * 4;
  __shared__ float part[kBwdWg][kSeg][kPartRow];
  static_assert(kBwdWg == 4, "one wave per group, four waves per workgroup");
  const int wave = threadIdx.x >> 6;
  const int nblk = bwd_blocks64(a.dim);
  int blk = blockIdx.x;
  const int gq = blk % nblk;
  blk /= nblk;
  const int b = blk % a.batch;
  const int run = blk / a.batch;
  const int gw_raw = gq * kBwdWg + wave;
  const bool live = gw_raw < a.ngroups16;
  const int gw = live ? gw_raw : a.ngroups16 - 1;
  const Lane c(a, b, gw, live);
  SegStage& S = stage[wave];
  const int lane = threadIdx.x & 63;
  const int s_lo = run * kBwdRun, s_hi = min(a.nseg, s_lo + kBwdRun) - 1;
  const float actf = c.act ? 1.0f : 0.0f;
  float Q[4];
  {
    const size_t so = ((static_cast<size_t>(b) * a.nseg + s_hi) * a.dim + c.e) * kScanN + 4 * c.q;
    const float4 qv = *reinterpret_cast<const float4*>(a.qs + so);
    Q[0] = qv.x; Q[1] = qv.y; Q[2] = qv.z; Q[3] = qv.w;
  }
  float dA[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dD = 0.0f, ddtw = 0.0f, ddtb = 0.0f;
  // conv: lane q's weight gradient dw[q], the bias gradient, and the
  // conv-output gradient of step t + q (zero past the run's end)
  float dwq = 0.0f, dbq = 0.0f, win = 0.0f;
  const int run_t0 = s_lo * kSeg;
#pragma unroll 1
  for (int s = s_hi; s >= s_lo; --s) {
    const int t0 = s * kSeg, t1 = min(a.seqlen, t0 + kSeg);
    stage_segment<true>(a, b, gw, t0, t1, S);
    float hin[4];
    {
      const size_t so = ((static_cast<size_t>(b) * a.nseg + s) * a.dim + c.e) * kScanN + 4 * c.q;
      const float4 hv = *reinterpret_cast<const float4*>(a.hs + so);
      hin[0] = hv.x; hin[1] = hv.y; hin[2] = hv.z; hin[3] = hv.w;
    }
    // the segment's states, recomputed
    float hist[kSeg][4];
    {
      float h[4] = {hin[0], hin[1], hin[2], hin[3]};
#pragma unroll
      for (int i = 0; i < kSeg; ++i) {
        if (t0 + i < t1) {
          float bv[4], av[4];
          const float u = Lane::at(S.u, i);
          const float dt = Lane::at(S.dt, i);
          c.sbc(S.B, i, bv);
          c.decay(dt, av);
#pragma unroll
          for (int j = 0; j < 4; ++j) h[j] = fmaf(av[j], h[j], dt * u * bv[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[i][j] = h[j];
      }
    }
#pragma unroll
    for (int i = kSeg - 1; i >= 0; --i) {
      if (t0 + i >= t1) continue;
      const int t = t0 + i;
      float hprev[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) hprev[j] = i > 0 ? hist[i - 1][j] : hin[j];
      float bv[4], cv[4], av[4];
      const float u = Lane::at(S.u, i);
      const float dt = Lane::at(S.dt, i);
      c.sbc(S.B, i, bv);
      c.sbc(S.C, i, cv);
      c.decay(dt, av);
      const float dyc = Lane::at(S.dyc, i);
      float G[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) G[j] = fmaf(dyc, cv[j], Q[j]);
      // dz = dy * yc * SiLU'(z), yc = C . h_t + D u
      if (a.z) {
        float yp = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) yp = fmaf(cv[j], hist[i][j], yp);
        const float yc = fmaf(c.d, u, quad_sum(yp));
        if (a.dz && c.act && c.q == 0) a.dz[c.be(t)] = Lane::at(S.dzf, i) * yc;
      }
      float pdt = 0.0f, pdu = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pdt = fmaf(G[j], fmaf(c.An[j] * av[j], hprev[j], u * bv[j]), pdt);
        pdu = fmaf(G[j] * dt, bv[j], pdu);
        dA[j] = fmaf(G[j] * dt * av[j], hprev[j], dA[j]);
      }
      const float ddt = quad_sum(pdt);
      const float du = fmaf(dyc, c.d, quad_sum(pdu));
      // dB_t = sum_e G dt u, dC_t = sum_e dyc h_t: this wave's 16 channels,
      // into LDS (lanes 0..3 hold states 4 lane .. 4 lane + 3)
      float sB[4], sC[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sB[j] = chan_sum(actf * G[j] * dt * u);
        sC[j] = chan_sum(actf * dyc * hist[i][j]);
      }
      if (lane < 4) {
        *reinterpret_cast<float4*>(&part[wave][i][4 * lane]) = make_float4(sB[0], sB[1], sB[2], sB[3]);
        *reinterpret_cast<float4*>(&part[wave][i][kScanN + 4 * lane]) = make_float4(sC[0], sC[1], sC[2], sC[3]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) Q[j] = av[j] * G[j];
      dD = fmaf(dyc, u, dD);
      const float dpre = ddt * Lane::at(S.dpf, i);
      ddtb += dpre;
      if (a.dt_rank1) {
        const float r = static_cast<const float*>(a.dt)[static_cast<size_t>(b) * a.seqlen + t];
        ddtw = fmaf(dpre, r, ddtw);
        const float sr = chan_sum(c.q == 0 ? actf * dpre * c.dtw : 0.0f);
        if (lane == 0) part[wave][i][2 * kScanN] = sr;
      } else if (a.ddt && c.act && c.q == 0) {
        a.ddt[c.be(t)] = dpre;
      }
      if (a.conv_w) {
        const float dxc = du * Lane::at(S.dsx, i);  // dL / d(conv output) at t
        const float v = c.q == 0 ? dxc : win;       // lane q: that of step t + q
        // dx_t = w3 dxc_t + w2 dxc_{t+1} + w1 dxc_{t+2} + w0 dxc_{t+3}; for
        // the last three steps of a run the terms past its end are added
        // by bwd_conv_fix
        const float dxt = quad_sum(c.wt * v);
        win = dpp<0x90>(v);                         // quad_perm 0 0 1 2: lane q <- lane q - 1
        dwq = fmaf(dxc, S.xr[i + c.q][(threadIdx.x & 63) >> 2], dwq);  // tap q meets raw x_{t-3+q}
        dbq += dxc;
        if (c.act && c.q == 0) {
          if (a.dx) a.dx[c.be(t)] = dxt;
          if (t - run_t0 < 3)
            a.xb[((static_cast<size_t>(b) * bwd_runs(a.nseg) + run) * 3 + (t - run_t0)) * a.dim + c.e] = dxc;
        }
      } else if (c.act && c.q == 0 && a.dx) {
        a.dx[c.be(t)] = du;
      }
    }
    // the workgroup's partials of this segment: summed over its waves in a
    // fixed order, one row per (step, block of 64 channels)
    __syncthreads();
    const int nb = t1 - t0;
    for (int k = threadIdx.x; k < nb * kPart; k += 256) {
      const int i = k / kPart, v = k % kPart;
      const float sum = ((part[0][i][v] + part[1][i][v]) + part[2][i][v]) + part[3][i][v];
      const size_t row = static_cast<size_t>(b) * a.seqlen + t0 + i;
      if (v < kScanN) a.pB[(row * nblk + gq) * kScanN + v] = sum;
      else if (v < 2 * kScanN) a.pC[(row * nblk + gq) * kScanN + (v - kScanN)] = sum;
      else if (a.dt_rank1) a.pr[row * nblk + gq] = sum;
    }
    __syncthreads();
  }
  if (!c.act) return;
  float* pe = a.pe + ((static_cast<size_t>(b) * bwd_runs(a.nseg) + run) * a.dim + c.e) * kBwdPe;
  *reinterpret_cast<float4*>(pe + 4 * c.q) = make_float4(dA[0], dA[1], dA[2], dA[3]);
  pe[19 + c.q] = dwq;
  if (c.q == 0) {
    pe[16] = dD;
    pe[17] = ddtw;
    pe[18] = ddtb;
    pe[23] = dbq;
  }
}

// The conv terms that cross a run boundary, one thread per (batch, run,
// channel): the last three dx of the run before run r > 0 take the terms of
// the first three conv-output gradients of run r; run 0's three give the
// conv cache's gradient (cache entry j is x at j - 3: sum_{k <= j} w_k dxc_{j-k}).
__global__ __launch_bounds__(256) void bwd_conv_fix(BwdArgs a) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const int runs = bwd_runs(a.nseg);
  if (i >= static_cast<size_t>(a.batch) * runs * a.dim) return;
  const int e = static_cast<int>(i % a.dim);
  const int r = static_cast<int>((i / a.dim) % runs);
  const int b = static_cast<int>(i / (static_cast<size_t>(a.dim) * runs));
  const int R = r * kBwdRun * kSeg;  // first step of run r
  const float4 w4 = reinterpret_cast<const float4*>(a.conv_w)[e];
  const float w[4] = {w4.x, w4.y, w4.z, w4.w};
  float g[3];
#pragma unroll
  for (int k = 0; k < 3; ++k)
    g[k] = R + k < a.seqlen ? a.xb[((static_cast<size_t>(b) * runs + r) * 3 + k) * a.dim + e] : 0.0f;
  if (r == 0) {
    if (a.dconv_cache) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k <= j; ++k) v = fmaf(g[j - k], w[k], v);
        a.dconv_cache[(static_cast<size_t>(b) * a.dim + e) * 3 + j] = v;
      }
    }
    return;
  }
  if (!a.dx) return;
  float* dx = a.dx + (static_cast<size_t>(b) * a.seqlen + R) * a.dim + e;
  dx[-3 * static_cast<ptrdiff_t>(a.dim)] += w[0] * g[0];
  dx[-2 * static_cast<ptrdiff_t>(a.dim)] += fmaf(w[0], g[1], w[1] * g[0]);
  dx[-1 * static_cast<ptrdiff_t>(a.dim)] += fmaf(w[0], g[2], fmaf(w[1], g[1], w[2] * g[0]));
}

// sums over the 64-channel blocks, one workgroup per (b, t) row: thread
// (slice, n) adds the blocks slice, slice + 16, ... of dB and dC, then the 16
// slices are added in order (the rank-1 dt the same way over 256 slices)
__global__ __launch_bounds__(256) void bwd_reduce_bc(BwdArgs a) {
  __shared__ float sb[16][kScanN], sc[16][kScanN], sr[256];
  const size_t row = blockIdx.x;
  const int n = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int nblk = bwd_blocks64(a.dim);
  const float* pb = a.pB + row * nblk * kScanN;
  const float* pc = a.pC + row * nblk * kScanN;
  float vb = 0.0f, vc = 0.0f;
  for (int g = sl; g < nblk; g += 16) {
    vb += pb[g * kScanN + n];
    vc += pc[g * kScanN + n];
  }
  sb[sl][n] = vb;
  sc[sl][n] = vc;
  float vr = 0.0f;
  if (a.dt_rank1) {
    for (int g = threadIdx.x; g < nblk; g += 256) vr += a.pr[row * nblk + g];
  }
  sr[threadIdx.x] = vr;
  __syncthreads();
  if (threadIdx.x < kScanN) {
    float tb = 0.0f, tc = 0.0f;
    for (int k = 0; k < 16; ++k) {
      tb += sb[k][threadIdx.x];
      tc += sc[k][threadIdx.x];
    }
    if (a.dB) a.dB[row * kScanN + threadIdx.x] = tb;
    if (a.dC) a.dC[row * kScanN + threadIdx.x] = tc;
  }
  if (threadIdx.x == 0 && a.dt_rank1 && a.ddt) {
    float t = 0.0f;
    for (int k = 0; k < 256; ++k) t += sr[k];
    a.ddt[row] = t;
  }
}

// sums over (batch, segment run) of the per-channel gradients; one thread
// per (channel, item)
__global__ __launch_bounds__(256) void bwd_reduce_e(BwdArgs a) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<size_t>(a.dim) * kBwdPe) return;
  const int e = static_cast<int>(i / kBwdPe), j = static_cast<int>(i % kBwdPe);
  float* out = nullptr;
  if (j < kScanN) out = a.dA ? a.dA + static_cast<size_t>(e) * kScanN + j : nullptr;
  else if (j == 16) out = a.dD ? a.dD + e : nullptr;
  else if (j == 17) out = a.ddt_w ? a.ddt_w + e : nullptr;
  else if (j == 18) out = a.ddt_bias ? a.ddt_bias + e : nullptr;
  else if (j < 23) out = a.dconv_w ? a.dconv_w + static_cast<size_t>(e) * 4 + (j - 19) : nullptr;
  else out = a.dconv_b ? a.dconv_b + e : nullptr;
  if (!out) return;
  const int runs = bwd_runs(a.nseg);
  float v = 0.0f;
  for (int b = 0; b < a.batch; ++b)
#pragma unroll 8
    for (int r = 0; r < runs; ++r) v += a.pe[((static_cast<size_t>(b) * runs + r) * a.dim + e) * kBwdPe + j];
  *out = v;
}

unsigned blocks_for(size_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

int bwd_segments(int seqlen) { return (seqlen + kSeg - 1) / kSeg; }

hipError_t launch_scan_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seqlen == 0) return hipSuccess;
  const size_t waves = static_cast<size_t>(a.batch) * a.ngroups16 * a.nseg;
  const unsigned wblocks = static_cast<unsigned>((waves + 3) / 4);
  const unsigned mblocks = static_cast<unsigned>(static_cast<size_t>(a.batch) * bwd_blocks64(a.dim) * bwd_runs(a.nseg));
  hipLaunchKernelGGL(bwd_summary, dim3(wblocks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_compose, dim3(blocks_for(static_cast<size_t>(a.batch) * a.dim * kScanN)), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = timed_launch(s, [&] { hipLaunchKernelGGL(bwd_main, dim3(mblocks), dim3(256), 0, s, a); });
  if (e != hipSuccess) return e;
  const size_t bt = static_cast<size_t>(a.batch) * a.seqlen;
  if (a.conv_w) {
    hipLaunchKernelGGL(bwd_conv_fix, dim3(blocks_for(static_cast<size_t>(a.batch) * bwd_runs(a.nseg) * a.dim)),
                       dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_reduce_bc, dim3(static_cast<unsigned>(bt)), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_e, dim3(blocks_for(static_cast<size_t>(a.dim) * kBwdPe)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ssm
