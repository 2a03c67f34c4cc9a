// Fused selective scan for gfx950 (kernel templates; included once per
// storage-type pair by the scan_xy_*.hip units): causal depthwise conv1d (k=4) + SiLU, the
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
// and each step reads its row with two scalar loads into SGPRs, which the
// VALU takes as operands directly (an LDS broadcast would move 64 copies of
// every value through the LDS return path, which then limits the loop).
//
// Time split (nseg > 1): launch 1 reduces segments 0..nseg-2 to their
// summaries (segment 0 from the true initial state, the others from zero), a
// small launch composes them in order into every segment's incoming state
// (scan_fused.hip), and launch 3 runs all segments in full.  Summaries travel
// through the workspace.
//
// Scaled-state form.  When A[e, n] is the same in all channels of the wave
// (A[e, n] = A[0, n]; the initialisation A_log = log(1..N) has this) and dt
// has a finite upper clip, the upper-clip decay q_n = exp(dt_max A[0, n]) is
// uniform across the wave.  Inside a period of kScanResc steps starting at
// t0 the lane keeps g_n = h_n(t) q_n^-(t - t0 + 1) instead of h_n(t); then
//   g_n <- g_n + dt u B'_n                    (step at the upper clip)
//   g_n <- g_n exp((dt - dt_max) A[e, n]) + dt u B'_n   (any other step)
//   y = sum_n C'_n g_n + D u
// with B'_n = B_n q_n^-(t - t0 + 1) and C'_n = C_n q_n^(t - t0 + 1) taken
// from the rescaled rows, and at the end of the period h_n = g_n q_n^k for the
// k steps taken.  It is the same recurrence regrouped: the decay of a step
// moves into the row factors, so a step at the clip costs one FMA per state
// for the update instead of a multiply and an FMA.  The factors stay within
// exp(+-32) (checked per wave, else the plain form runs).
#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kBlk = kScanBlk;          // steps per block: one tile of vector loads
constexpr unsigned kCuSlots = kScanCuSlots;  // compute units the workgroups go round (MI355X)
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: the store is dropped
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family

using rsrc_t = __amdgpu_buffer_rsrc_t;
// Memory the kernel never writes, in the constant address space: uniform
// loads from it become scalar loads.
typedef __attribute__((address_space(4))) float cfloat;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <typename T>
struct BufIO;

template <>
struct BufIO<float> {
  using raw = uint32_t;
  static constexpr uint32_t bytes = 4;
  __device__ static raw load(rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
  }
  __device__ static float f32(raw v) { return __uint_as_float(v); }
  __device__ static void store(float v, rsrc_t r, uint32_t vo, uint32_t so) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, vo, so, 0);
  }
};

template <>
struct BufIO<bf16s> {
  using raw = uint16_t;
  static constexpr uint32_t bytes = 2;
  __device__ static raw load(rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
  }
  __device__ static float f32(raw v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static void store(float v, rsrc_t r, uint32_t vo, uint32_t so) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, vo, so, 0);
  }
};

struct LaneCtx {
  int b, e;
  bool act;
  float al0;              // A[e, 0] * log2(e)
  float d, dtw, dtb;
  float cw0, cw1, cw2, cw3, cb;
};

// kMain: a whole sequence (nseg == 1) or, after kPass1, segments 1..nseg-1.
// dA[n] = exp(dt A[e, n]).  POW: A[e, n] = (n+1) A[e, 0] for every n, so
// exp(dt A[e, n]) = r^(n+1) with r = exp(dt A[e, 0]), the powers taken by a
// depth-5 product tree.  Otherwise one exponential per state, with A[e, n]
// log2(e) read back from the wave's LDS copy ([n / 4][lane] float4s).
template <bool POW>
__device__ __forceinline__ void decay(float dt, float al0, const float4* al2, float (&dA)[kScanN]) {
  if (POW) {
    dA[0] = exp2_fast(dt * al0);
#pragma unroll
    for (int k = 1; k < kScanN; ++k) dA[k] = (k & 1) ? dA[(k - 1) / 2] * dA[(k - 1) / 2] : dA[k - 1] * dA[0];
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = al2[q * 64 + lane];
      dA[4 * q + 0] = exp2_fast(dt * v.x);
      dA[4 * q + 1] = exp2_fast(dt * v.y);
      dA[4 * q + 2] = exp2_fast(dt * v.z);
      dA[4 * q + 3] = exp2_fast(dt * v.w);
    }
  }
}

enum Mode { kPass1 = 1, kMain = 2 };

// ZOH: B enters as ((e^{dt A} - 1) / A) B u (zero-order hold) instead of
// dt B u.
template <typename XT, typename YT, int DTM, bool CONV, bool GATE, bool ZOH>
struct Scan {
  using DT = typename std::conditional<DTM == 2, bf16s, float>::type;
  using XIO = BufIO<XT>;
  using DIO = BufIO<DT>;
  using YIO = BufIO<YT>;
  static constexpr bool kWideDt = DTM != 0;                            // dt given per channel
  static constexpr bool kDtSharesX = kWideDt && DIO::bytes == XIO::bytes;  // same byte offsets as x

  const ScanKernelArgs& a;
  const LaneCtx c;
  rsrc_t rx, rz, rdt, ry;
  const cfloat* rows;              // this batch row's packed B/C rows (constant memory)
  const cfloat* rows_g;            // the same rows rescaled for the scaled-state form
  const cfloat* qtab;              // q_n^k as [k][n], k = 0..kScanResc
  uint32_t vo_x[kBlk];             // per-lane byte offset of step i of a tile (x and z)
  uint32_t vo_d[kBlk];             // the same for an E-wide dt of another element size
  uint32_t vy;                     // per-lane byte offset in a y row; out of range for idle lanes
  uint32_t rb_x, rb_dt, rb_y;      // bytes per time step
  float dt_min, dt_max, sp_lo, sp_hi;
  float sat_pre;                   // pre-activations at or above this give dt = dt_max
  bool dt_softplus;
  const float4* al2;               // A[e, n] log2(e) as [n / 4][lane] float4s (LDS)
  float4* sat4;                    // exp(dt_max A[e, n]), the same layout (LDS; plain form)

  __device__ Scan(const ScanKernelArgs& a_, const LaneCtx& c_, const float4* al2_, float4* sat4_)
      : a(a_), c(c_), al2(al2_), sat4(sat4_) {
    const uint32_t L = a.seqlen, E = a.dim;
    const size_t tok0 = static_cast<size_t>(c.b) * L;  // first token of this batch row
    // each descriptor covers this batch row (the per-lane offsets are range
    // checked against it; the scalar step offsets stay inside it by
    // construction, see load_block)
    rx = make_rsrc(static_cast<const char*>(a.x) + tok0 * E * XIO::bytes, L * E * XIO::bytes);
    rz = make_rsrc(static_cast<const char*>(a.z ? a.z : a.x) + tok0 * E * XIO::bytes, L * E * XIO::bytes);
    ry = make_rsrc(static_cast<char*>(a.y) + tok0 * E * YIO::bytes, L * E * YIO::bytes);
    rb_x = E * XIO::bytes;
    rb_y = E * YIO::bytes;
    if constexpr (kWideDt) {
      rdt = make_rsrc(static_cast<const char*>(a.dt) + tok0 * E * DIO::bytes, L * E * DIO::bytes);
      rb_dt = E * DIO::bytes;
    } else {
      // the rank-1 input r[b, t]: every lane loads the same word (a vector
      // load, so it is prefetched with the tile and waited for in order)
      rdt = make_rsrc(static_cast<const float*>(a.dt) + tok0, L * 4u);
      rb_dt = 4;
    }
    rows = (const cfloat*)(a.bc + tok0 * kBcRow);
    rows_g = (const cfloat*)(a.bcg ? a.bcg + tok0 * kBcRow : a.bc);
    qtab = (const cfloat*)(a.qtab ? a.qtab : a.bc);
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      vo_x[i] = static_cast<uint32_t>(c.e) * XIO::bytes + i * rb_x;
      vo_d[i] = (kWideDt ? static_cast<uint32_t>(c.e) * DIO::bytes : 0u) + i * rb_dt;
    }
    vy = c.act ? static_cast<uint32_t>(c.e) * YIO::bytes : kOob;
    dt_min = a.dt_min;
    dt_max = a.dt_max;
    sp_lo = a.sp_lo;
    sp_hi = a.sp_hi;
    dt_softplus = a.dt_softplus != 0;
    sat_pre = dt_softplus ? sp_hi : dt_max;
  }

  // Raw (pre-conv) input at time p: x when p >= 0, the cache entry K-1+p
  // (oldest first) before the sequence, 0 at a fresh prefill.
  __device__ __forceinline__ float raw_at(int p) const {
    if (p >= a.seqlen) return 0.0f;  // only reachable for an empty segment
    if (p >= 0) return XIO::f32(XIO::load(rx, vo_x[0], static_cast<uint32_t>(p) * rb_x));
    if (a.conv_cache_in == nullptr) return 0.0f;
    return a.conv_cache_in[(static_cast<size_t>(c.b) * a.dim + c.e) * (kConvK - 1) + (kConvK - 1 + p)];
  }

  struct Tile {
    typename XIO::raw x[kBlk];
    typename DIO::raw d[kBlk];
    typename XIO::raw z[kBlk];
  };

  // Loads of steps tb .. tb+kBlk-1.  Steps past the segment are loaded too
  // (and never used).  The buffer range check covers the per-lane offset
  // but not the scalar one, so a tile reaching past the end of the batch row
  // (the last one of a sequence) takes its rows one by one, clamped to the
  // last row: every access stays inside the tensor.
  template <bool FULL>
  __device__ __forceinline__ void load_block(int tb, Tile& T) const {
    constexpr bool has_z = FULL && GATE;
    if (tb + kBlk <= a.seqlen) {
      const uint32_t sx = static_cast<uint32_t>(tb) * rb_x;
      const uint32_t sd = static_cast<uint32_t>(tb) * rb_dt;
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        T.x[i] = XIO::load(rx, vo_x[i], sx);
        T.d[i] = DIO::load(rdt, kDtSharesX ? vo_x[i] : vo_d[i], kDtSharesX ? sx : sd);
        if (has_z) T.z[i] = XIO::load(rz, vo_x[i], sx);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        const uint32_t r = static_cast<uint32_t>(min(tb + i, a.seqlen - 1));
        T.x[i] = XIO::load(rx, vo_x[0], r * rb_x);
        T.d[i] = DIO::load(rdt, kDtSharesX ? vo_x[0] : vo_d[0], r * (kDtSharesX ? rb_x : rb_dt));
        if (has_z) T.z[i] = XIO::load(rz, vo_x[0], r * rb_x);
      }
    }
  }

  // B_t (the first half of the packed row of step t) into SGPRs: wave-uniform
  // scalar loads.  G: the rescaled row.
  template <bool G>
  __device__ __forceinline__ void load_b(int t, float (&bv)[kScanN]) const {
    const cfloat* row = (G ? rows_g : rows) + static_cast<size_t>(t) * kBcRow;
#pragma unroll
    for (int n = 0; n < kScanN; ++n) bv[n] = row[n];
  }

  // One step with B_t in bv.  C_t is loaded at the start of the step (it is
  // first needed by the readout at its end), B_{t+1} after the readout, so
  // its latency is covered by the row-independent work at the start of the
  // next step and at most one row of each is held in SGPRs.  FULL: readout,
  // skip, gate, store.  Otherwise state update only and the running sum of
  // dt for the segment's decay product.  G: h holds the scaled state g and
  // the rows are the rescaled ones.
  template <bool POW, bool FULL, bool G>
  __device__ __forceinline__ void step(int t, const Tile& T, int i, float (&h)[kScanN], float (&win)[3],
                                       float& sdt, const float (&asat)[kScanN], const float (&zsat)[kScanN],
                                       float (&bv)[kScanN], float (&bn)[kScanN]) const {
    constexpr bool has_z = FULL && GATE;
    // the summary pass holds no C row, so its B rows are double-buffered:
    // B_{t+1} is requested a whole step before it is used
    if (!FULL) load_b<G>(t + 1, bn);
    float cv[kScanN];
    if (FULL) {
      const cfloat* row = (G ? rows_g : rows) + static_cast<size_t>(t) * kBcRow;
#pragma unroll
      for (int n = 0; n < kScanN; ++n) cv[n] = row[kScanN + n];
    }
    float u = XIO::f32(T.x[i]);
    if (CONV) {
      const float xc = fmaf(c.cw0, win[0], fmaf(c.cw1, win[1], fmaf(c.cw2, win[2], fmaf(c.cw3, u, c.cb))));
      win[0] = win[1];
      win[1] = win[2];
      win[2] = u;
      u = silu(xc);
    }
    const float pre = kWideDt ? DIO::f32(T.d[i]) + c.dtb : fmaf(c.dtw, DIO::f32(T.d[i]), c.dtb);
    // dt = clip(softplus(pre), lo, hi).  When every lane of the wave is at or
    // beyond the upper threshold, dt is dt_max everywhere (exact: softplus is
    // increasing) and the decay factors are the per-segment exp(dt_max A).
    // Otherwise lanes beyond either threshold take the clip value, softplus
    // runs only if some lane lies inside the band, and the decay factors are
    // computed for the step.  Both branches update h in place
    // (h = (a h) + dt u B).
    const float gate = has_z ? silu(XIO::f32(T.z[i])) : 1.0f;
    // G: the branches only set dt u and, off the clip, scale g in place; the
    // FMA with B' after them is common, so g stays in one set of registers
    float dtu_g = 0.0f;
    if (__all(pre >= sat_pre)) {
      if (!FULL) sdt += dt_max;
      if (G) {
        dtu_g = dt_max * u;
      } else if (ZOH) {
#pragma unroll
        for (int n = 0; n < kScanN; ++n) h[n] = fmaf(zsat[n] * u, bv[n], asat[n] * h[n]);
      } else {
        // the clip decays come from LDS: held in registers through the loop
        // they would cost the kernel a wave per SIMD
        const float dtu = dt_max * u;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = sat4[q * 64 + lane];
          h[4 * q + 0] = fmaf(dtu, bv[4 * q + 0], v.x * h[4 * q + 0]);
          h[4 * q + 1] = fmaf(dtu, bv[4 * q + 1], v.y * h[4 * q + 1]);
          h[4 * q + 2] = fmaf(dtu, bv[4 * q + 2], v.z * h[4 * q + 2]);
          h[4 * q + 3] = fmaf(dtu, bv[4 * q + 3], v.w * h[4 * q + 3]);
        }
      }
    } else {
      float dt;
      if (dt_softplus) {
        dt = (pre >= sp_hi) ? dt_max : dt_min;
        const bool mid = (pre > sp_lo) && (pre < sp_hi);
        if (__any(mid)) {
          const float sp = softplus(pre);
          dt = mid ? __builtin_amdgcn_fmed3f(sp, dt_min, dt_max) : dt;
        }
      } else {
        dt = __builtin_amdgcn_fmed3f(pre, dt_min, dt_max);
      }
      if (!FULL) sdt += dt;
      const float dtu = dt * u;
      float dA[kScanN];
      // G: the decay relative to the clip's, exp((dt - dt_max) A) >= 1
      decay<POW>(G ? dt - dt_max : dt, c.al0, al2, dA);
      if (ZOH && !G) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = al2[q * 64 + lane];  // A log2(e)
          const float av[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = 4 * q + r;
            const float coef = dt * zoh_phi(dt * av[r] * kLn2, dA[n]);
            h[n] = fmaf(coef * u, bv[n], dA[n] * h[n]);
          }
        }
      } else if (G) {
        dtu_g = dtu;
#pragma unroll
        for (int n = 0; n < kScanN; ++n) h[n] *= dA[n];
      } else {
#pragma unroll
        for (int n = 0; n < kScanN; ++n) h[n] = fmaf(dtu, bv[n], dA[n] * h[n]);
      }
      // keeps this update in its branch (merged with the other one, the decay
      // factors would be copied into common registers every step)
#pragma unroll
      for (int n = 0; n < kScanN; ++n) asm volatile("" : "+v"(h[n]));
    }
    if (G) {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) h[n] = fmaf(dtu_g, bv[n], h[n]);
    }
    if (!FULL) {
      // nothing reads the state between steps of the summary pass; pin it
      // here, or the compiler interleaves several steps of the recurrence and
      // runs out of registers
#pragma unroll
      for (int n = 0; n < kScanN; ++n) asm volatile("" : "+v"(h[n]));
    }
    if (FULL) {
      // B_t is dead once the state is updated: B_{t+1} goes into the same
      // registers now, and its latency is covered by the readout, the store
      // and the start of the next step
      __builtin_amdgcn_sched_barrier(0);
      load_b<G>(t + 1, bv);
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int n = 0; n < kScanN; ++n) acc[n & 3] = fmaf(cv[n], h[n], acc[n & 3]);
      const float yv = fmaf(c.d, u, (acc[0] + acc[1]) + (acc[2] + acc[3])) * gate;
      YIO::store(yv, ry, vy, static_cast<uint32_t>(t) * rb_y);
    }
  }

  // The kBlk steps of a full tile.  The scheduling barrier keeps each step's
  // scalar loads inside the step (hoisted across steps they would need a
  // second set of SGPRs).
  template <bool POW, bool FULL, bool G>
  __device__ __forceinline__ void block(int tb, const Tile& T, float (&h)[kScanN], float (&win)[3],
                                        float& sdt, const float (&asat)[kScanN], const float (&zsat)[kScanN],
                                        float (&bv0)[kScanN], float (&bv1)[kScanN]) const {
    static_assert(kBlk % 2 == 0, "every tile starts with B in the first buffer");
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      if (FULL || (i & 1) == 0) step<POW, FULL, G>(tb + i, T, i, h, win, sdt, asat, zsat, bv0, bv1);
      else step<POW, FULL, G>(tb + i, T, i, h, win, sdt, asat, zsat, bv1, bv0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The steps tb .. t1-1 (fewer than kBlk) of an already loaded tile.
  template <bool POW, bool FULL, bool G>
  __device__ __forceinline__ void partial(int tb, int t1, const Tile& T, float (&h)[kScanN], float (&win)[3],
                                          float& sdt, const float (&asat)[kScanN], const float (&zsat)[kScanN],
                                          float (&bv0)[kScanN], float (&bv1)[kScanN]) const {
#pragma unroll
    for (int i = 0; i < kBlk - 1; ++i) {
      if (tb + i < t1) {
        if (FULL || (i & 1) == 0) step<POW, FULL, G>(tb + i, T, i, h, win, sdt, asat, zsat, bv0, bv1);
        else step<POW, FULL, G>(tb + i, T, i, h, win, sdt, asat, zsat, bv1, bv0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Scan steps [t0, t1) from state h.  Two tiles alternate: while one is
  // consumed the next one's loads are in flight, and as the roles swap by
  // program position no register copy ever waits on a load.  G: the
  // scaled-state form (t0 is a multiple of kScanResc = 2 tiles); h is
  // rescaled back after every pair of tiles and at the end.
  template <bool POW, bool FULL, bool G>
  __device__ __forceinline__ void run(int t0, int t1, float (&h)[kScanN], float (&win)[3], float& sdt) const {
    static_assert(kScanResc == 2 * kBlk, "a rescaling period is the loop's pair of tiles");
    if (t0 >= t1) return;
    const int nfull = (t1 - t0) / kBlk;
    float asat[kScanN];             // exp(dt_max A[e, n]): the decay on the upper clip
    if (G) {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) asat[n] = 0.0f;
    } else {
      decay<POW>(dt_max, c.al0, al2, asat);
      if (!ZOH) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sat4[q * 64 + lane] = make_float4(asat[4 * q], asat[4 * q + 1], asat[4 * q + 2], asat[4 * q + 3]);
      }
    }
    float zsat[kScanN];             // ZOH: (exp(dt_max A[e, n]) - 1) / A[e, n]
    if (ZOH && !G) {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = al2[q * 64 + lane];
        const float av[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) zsat[4 * q + r] = dt_max * zoh_phi(dt_max * av[r] * kLn2, asat[4 * q + r]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < kScanN; ++n) zsat[n] = 0.0f;
    }
    float bv[kScanN], bw[kScanN];   // B of the current step (and, summary pass, of the next)
    load_b<G>(t0, bv);
    Tile A, B;
    load_block<FULL>(t0, A);
    int tb = t0;
    int k = 0;
#pragma unroll 1
    for (; k + 2 <= nfull; k += 2) {
      load_block<FULL>(tb + kBlk, B);
      block<POW, FULL, G>(tb, A, h, win, sdt, asat, zsat, bv, bw);
      load_block<FULL>(tb + 2 * kBlk, A);
      block<POW, FULL, G>(tb + kBlk, B, h, win, sdt, asat, zsat, bv, bw);
      if (G) {
        // h = g q^kScanResc: the period is over
#pragma unroll
        for (int n = 0; n < kScanN; ++n) h[n] *= qtab[kScanResc * kScanN + n];
      }
      tb += 2 * kBlk;
    }
    if (k < nfull) {
      load_block<FULL>(tb + kBlk, B);
      block<POW, FULL, G>(tb, A, h, win, sdt, asat, zsat, bv, bw);
      partial<POW, FULL, G>(tb + kBlk, t1, B, h, win, sdt, asat, zsat, bv, bw);
    } else {
      partial<POW, FULL, G>(tb, t1, A, h, win, sdt, asat, zsat, bv, bw);
    }
    if (G) {
      // the t1 - tb (< kScanResc) steps of the last, unfinished period
      const cfloat* q = qtab + (t1 - tb) * kScanN;
#pragma unroll
      for (int n = 0; n < kScanN; ++n) h[n] *= q[n];
    }
  }

  // run() in the variant the wave qualifies for (no scaled-state form with ZOH)
  template <bool FULL>
  __device__ __forceinline__ void run_any(bool pow, bool g, int t0, int t1, float (&h)[kScanN], float (&win)[3],
                                          float& sdt) const {
    if constexpr (!ZOH) {
      if (g) {
        if (pow) run<true, FULL, true>(t0, t1, h, win, sdt);
        else run<false, FULL, true>(t0, t1, h, win, sdt);
        return;
      }
    }
    if (pow) run<true, FULL, false>(t0, t1, h, win, sdt);
    else run<false, FULL, false>(t0, t1, h, win, sdt);
  }
};

template <typename XT, typename YT, int DTM, bool CONV, bool GATE, bool ZOH, int MODE>
__global__ __launch_bounds__(64, 3) void scan_kernel(ScanKernelArgs a) {
  const int lane = threadIdx.x;
  // block -> (segment, batch, channel group).  Workgroups are handed out
  // round-robin, so block i runs on compute unit i % kCuSlots (8 XCDs x 32
  // CUs on MI355X, measured) in round i / kCuSlots.  The blocks of one CU
  // get consecutive positions of the (segment, batch, channel group) order,
  // channel groups fastest, so the waves a CU holds walk the same B/C rows
  // and find them in its scalar cache.  Any CU count gives a bijection.
  const unsigned nblk = gridDim.x;
  const unsigned full = nblk / kCuSlots, rem = nblk % kCuSlots;
  const unsigned slot = blockIdx.x % kCuSlots, round = blockIdx.x / kCuSlots;
  int bid = static_cast<int>(slot * full + min(slot, rem) + round);
  const int g = uniform(bid % a.n_egroups);
  bid /= a.n_egroups;
  LaneCtx c;
  c.b = uniform(bid % a.batch);
  const int seg = uniform(bid / a.batch);
  const int e_raw = g * 64 + lane;
  c.act = e_raw < a.dim;
  c.e = c.act ? e_raw : a.dim - 1;

  __shared__ float4 s_al2[4 * 64];
  __shared__ float4 s_sat[4 * 64];
  bool prog = true;
  bool same = true;    // A[e, :] = A[0, :]
  float span = 0.0f;   // max_n |A[0, n]|
  const float a0 = a.A[static_cast<size_t>(c.e) * kScanN];
  float al2v[kScanN];
#pragma unroll
  for (int n = 0; n < kScanN; ++n) {
    const float an = a.A[static_cast<size_t>(c.e) * kScanN + n];
    const float ar = a.A[n];
    al2v[n] = an * kLog2e;
    prog = prog && (an == static_cast<float>(n + 1) * a0);
    same = same && (an == ar);
    span = fmaxf(span, fabsf(ar));
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    s_al2[q * 64 + lane] = make_float4(al2v[4 * q], al2v[4 * q + 1], al2v[4 * q + 2], al2v[4 * q + 3]);
  c.al0 = al2v[0];
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
  // the scaled-state form: rescaled rows present (finite dt_max, Euler), A
  // the same in every channel of the wave, factors within exp(+-32)
  const bool use_g = !ZOH && a.bcg != nullptr && __all(same) && kScanResc * fabsf(a.dt_max) * span <= 32.0f;
  const Scan<XT, YT, DTM, CONV, GATE, ZOH> S(a, c, s_al2, s_sat);
  const int t0 = seg * a.seg_len;
  const int t1 = min(t0 + a.seg_len, a.seqlen);
  const size_t sbase = (static_cast<size_t>(c.b) * a.dim + c.e) * kScanN;
  // summaries: [(b, g)][segment][16 states + sum dt][lane]
  float* summ = a.summ + (static_cast<size_t>(c.b) * a.n_egroups + g) * (a.nseg - 1) * (kScanN + 1) * 64;
  // segment 0's starting state and conv window: [(b, g)][16 states + 3][lane]
  float* head = a.head + (static_cast<size_t>(c.b) * a.n_egroups + g) * kScanHead * 64;
  // With a time split, the last segment of the full pass writes the final
  // state and conv cache, which may be the very buffers the initial ones are
  // read from (in-place update), and nothing orders it after segment 0 of the
  // same pass.  So only the summary pass reads the initial state and cache;
  // it saves them for segment 0 of the full pass.
  const bool saved_start = MODE == kMain && seg == 0 && a.nseg > 1;
  float win[3] = {0.0f, 0.0f, 0.0f};
  if (CONV) {
    if (saved_start) {
      win[0] = head[(kScanN + 0) * 64 + lane];
      win[1] = head[(kScanN + 1) * 64 + lane];
      win[2] = head[(kScanN + 2) * 64 + lane];
    } else {
      win[0] = S.raw_at(t0 - 3);
      win[1] = S.raw_at(t0 - 2);
      win[2] = S.raw_at(t0 - 1);
    }
  }
  float h[kScanN];
  float sdt = 0.0f;

  if (MODE == kMain && seg > 0) {
    // state entering this segment, left in slot seg-1 by the composition of
    // the summaries (scan_compose_kernel)
    const float* sin = summ + static_cast<size_t>(seg - 1) * (kScanN + 1) * 64;
#pragma unroll
    for (int n = 0; n < kScanN; ++n) h[n] = sin[n * 64 + lane];
  } else if (saved_start) {
#pragma unroll
    for (int n = 0; n < kScanN; ++n) h[n] = head[n * 64 + lane];
  } else {
#pragma unroll
    for (int n = 0; n < kScanN; ++n) h[n] = (seg == 0 && a.state_in) ? a.state_in[sbase + n] : 0.0f;
  }

  if (MODE == kPass1 && seg == 0) {
#pragma unroll
    for (int n = 0; n < kScanN; ++n) head[n * 64 + lane] = h[n];
    head[(kScanN + 0) * 64 + lane] = win[0];
    head[(kScanN + 1) * 64 + lane] = win[1];
    head[(kScanN + 2) * 64 + lane] = win[2];
  }

  if (MODE == kPass1) {
    // summary of segments 0..nseg-2: the end state from the true initial state
    // (segment 0) or from zero (the others), and the sum of dt
    S.template run_any<false>(use_pow, use_g, t0, t1, h, win, sdt);
    float* ss = summ + static_cast<size_t>(seg) * (kScanN + 1) * 64;
#pragma unroll
    for (int n = 0; n < kScanN; ++n) ss[n * 64 + lane] = h[n];
    ss[kScanN * 64 + lane] = sdt;
    return;
  }
  S.template run_any<true>(use_pow, use_g, t0, t1, h, win, sdt);
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

template <typename XT, typename YT, int DTM, bool CONV, bool GATE, bool ZOH>
hipError_t launch_scan_t(const ScanLaunch& l, hipStream_t stream) {
  const ScanKernelArgs& a = l.k;
  const unsigned groups = static_cast<unsigned>(a.batch) * static_cast<unsigned>(a.n_egroups);
  if (groups == 0) return hipSuccess;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((scan_kernel<XT, YT, DTM, CONV, GATE, ZOH, kPass1>), dim3(groups * (a.nseg - 1)), dim3(64), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = launch_scan_compose(a, stream);
    if (err != hipSuccess) return err;
  }
  return timed_launch(stream, [&] {
    hipLaunchKernelGGL((scan_kernel<XT, YT, DTM, CONV, GATE, ZOH, kMain>), dim3(groups * a.nseg), dim3(64), 0, stream,
                       a);
  });
}

template <typename XT, typename YT, int DTM, bool CONV, bool GATE>
hipError_t pick_zoh(const ScanLaunch& l, hipStream_t s) {
  return l.zoh ? launch_scan_t<XT, YT, DTM, CONV, GATE, true>(l, s) : launch_scan_t<XT, YT, DTM, CONV, GATE, false>(l, s);
}

template <typename XT, typename YT, int DTM, bool CONV>
hipError_t pick_gate(const ScanLaunch& l, hipStream_t s) {
  return l.k.has_z ? pick_zoh<XT, YT, DTM, CONV, true>(l, s) : pick_zoh<XT, YT, DTM, CONV, false>(l, s);
}

template <typename XT, typename YT, int DTM>
hipError_t pick_conv(const ScanLaunch& l, hipStream_t s) {
  return l.conv ? pick_gate<XT, YT, DTM, true>(l, s) : pick_gate<XT, YT, DTM, false>(l, s);
}

template <typename XT, typename YT>
hipError_t pick_dt(const ScanLaunch& l, hipStream_t s) {
  switch (l.dt_mode) {
    case 0: return pick_conv<XT, YT, 0>(l, s);
    case 1: return pick_conv<XT, YT, 1>(l, s);
    default: return pick_conv<XT, YT, 2>(l, s);
  }
}

// Resident workgroups (one wave each) per CU of the full-segment kernel of a
// variant, from the runtime's occupancy calculator; cached per variant.
template <typename XT, typename YT, int DTM, bool CONV, bool GATE, bool ZOH>
int occupancy_t() {
  static int cached = 0;
  int n = __atomic_load_n(&cached, __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_kernel<XT, YT, DTM, CONV, GATE, ZOH, kMain>, 64, 0) !=
          hipSuccess ||
      n <= 0)
    return 0;
  __atomic_store_n(&cached, n, __ATOMIC_RELAXED);
  return n;
}

template <typename XT, typename YT, int DTM, bool CONV>
int occ_gate(const ScanLaunch& l) {
  if (l.zoh) return l.k.has_z ? occupancy_t<XT, YT, DTM, CONV, true, true>() : occupancy_t<XT, YT, DTM, CONV, false, true>();
  return l.k.has_z ? occupancy_t<XT, YT, DTM, CONV, true, false>() : occupancy_t<XT, YT, DTM, CONV, false, false>();
}

template <typename XT, typename YT, int DTM>
int occ_conv(const ScanLaunch& l) {
  return l.conv ? occ_gate<XT, YT, DTM, true>(l) : occ_gate<XT, YT, DTM, false>(l);
}

}  // namespace

// Launch for one (x dtype, y dtype) pair; defined in scan_xy_*.hip.
template <>
hipError_t launch_scan_xy<SSM_SCAN_XT, SSM_SCAN_YT>(const ScanLaunch& l, hipStream_t stream) {
  return pick_dt<SSM_SCAN_XT, SSM_SCAN_YT>(l, stream);
}

template <>
int scan_occupancy_xy<SSM_SCAN_XT, SSM_SCAN_YT>(const ScanLaunch& l) {
  switch (l.dt_mode) {
    case 0: return occ_conv<SSM_SCAN_XT, SSM_SCAN_YT, 0>(l);
    case 1: return occ_conv<SSM_SCAN_XT, SSM_SCAN_YT, 1>(l);
    default: return occ_conv<SSM_SCAN_XT, SSM_SCAN_YT, 2>(l);
  }
}

}  // namespace ssm
