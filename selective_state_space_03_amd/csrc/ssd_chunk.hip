// Multi-head chunked scan (SSD form) for gfx950, with MFMA for the dense
// contractions.
//
// Page "What is the Mamba model?", sections "chunkscan" and "chunkscan
// implementation": the sequence is cut into chunks of Q tokens; inside a chunk
//   out[l] = sum_{s<=l} cb[l,s] e^{dA[l]-dA[s]} dt[s] x[s]     (intra-chunk)
//          + e^{dA[l]} C[l] prev_states                        (earlier chunks)
//          + D x[l]                                            (skip)
// with cb = C B^T and dA the inclusive cumulative sum of dt * A_h; the chunks are
// taken in order and each hands its final state to the next (the inter-chunk
// scan): prev_states <- e^{dA[Q-1]} prev_states + sum_s e^{dA[Q-1]-dA[s]} dt[s]
// x[s] (outer) B[s], which is the unrolled product-sum form applied to a chunk.
//
// Mapping: one workgroup (4 waves) per (batch, head, 16- or 32-wide slice of
// headdim) walks all chunks in order, so the state (PT x N, fp32) stays in MFMA
// accumulators and the outer chunk loop of the page runs on the device.  Per
// chunk: C, B (both layouts), x (transposed) and the dt cumsum are staged in
// LDS while the next chunk's loads are in flight; each wave owns two 16-row
// blocks of the chunk (rows w and 7-w, equal causal work):
//   cb^T blocks   = B_J C_I^T            v_mfma_f32_16x16x32_bf16
//   M (masked)    = cb . 2^(dA_l - dA_s) . dt_s, the exponent masked to -inf
//                   for s > l before the exponential
//   intra         = M X_J                v_mfma_f32_16x16x16_bf16, M split hi+lo
//   state readout = C_I S^T              v_mfma_f32_16x16x32_bf16, S split hi+lo
//   state update  = (w.x)^T B            v_mfma_f32_16x16x32_bf16, w.x split hi+lo
// where the hi/lo split (a bf16 value plus the bf16 of its remainder) keeps the
// operands that are not exact bf16 inputs at about 16 mantissa bits.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kQ = kSsdQ;  // 128 tokens per chunk
constexpr int kN = kSsdN;  // 64 states
constexpr int kRowN = kN + 8;   // padded LDS row of N bf16 (144 bytes)
constexpr int kRowQ = kQ + 8;   // padded LDS row of Q bf16 (272 bytes)
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Column of element s in row r of the transposed tiles (Bt, Xt): the 16-byte
// blocks of a row are permuted by the row's 8-row group, so the transposing
// stores (one row per 8-row group across the lanes of a wave) fall in
// different banks.  Reads of 4 or 8 consecutive elements inside one block stay
// contiguous.
__device__ __forceinline__ int swz(int r, int s) { return ((((s >> 3) ^ (r >> 3)) & 15) << 3) | (s & 7); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = bf16_bits(v);
  lo = bf16_bits(v - bf16_val(hi));
}

template <int PT>
struct alignas(16) Smem {
  uint16_t C[kQ][kRowN];    // C chunk, row-major [l][n]
  uint16_t B[kQ][kRowN];    // B chunk, row-major [s][n]
  uint16_t Bt[kN][kRowQ];   // B chunk transposed [n][swz(n, s)]
  uint16_t Xt[PT][kRowQ];   // x chunk slice transposed [p][swz(p, s)]
  uint16_t XWh[PT][kRowQ];  // wS[s] x[s][p], transposed, bf16 high part
  uint16_t XWl[PT][kRowQ];  //                              bf16 low part
  uint16_t Shi[PT][kRowN];  // state entering the chunk, [p][n], bf16 high part
  uint16_t Slo[PT][kRowN];  //                                   bf16 low part
  float O[kQ][PT + 4];      // the chunk's output tile, stored to HBM row by row
  float EL[8][kQ];          // 2^(dA[l] - dA[16 J]) for l >= 16 J
  float ESD[kQ];            // 2^(dA[16 (s / 16)] - dA[s]) dt[s]
  float dA[kQ];             // inclusive cumsum of dt * A * log2(e)
  float dt[kQ];             // dt after softplus and clip
  float wS[kQ];             // 2^(dA[Q-1] - dA[s]) * dt[s]: state-update weights
  float eA[kQ];             // 2^dA[l]: decay of the incoming state
};

// Workgroup of NW = 4 * (PT / 16) waves.  Loads: C and B as 16-byte pieces,
// RPT consecutive rows per thread (so B can be written transposed with one
// LDS store per n); x two rows per thread.
template <int PT>
struct Shape {
  static constexpr int NPT = PT / 16;        // 16-wide subtiles of the headdim slice
  static constexpr int NW = 4 * NPT;         // waves
  static constexpr int NT = 64 * NW;         // threads
  static constexpr int RPT = 1024 / NT;      // rows of C / B per thread (8 pieces per row)
  static constexpr int XPR = PT / 8;         // x pieces per row
  static constexpr int XT = 64 * XPR;        // threads loading x (2 rows each)
};

template <int PT>
struct ChunkRegs {
  uint4 c[Shape<PT>::RPT], b[Shape<PT>::RPT], x[2];
  float dt;
  int valid;  // tokens of this chunk inside the sequence (fewer in a ragged last chunk)
};

// GATE: the output is multiplied by SiLU(z).  Whole chunks run in the loop;
// a ragged last chunk (L not a multiple of Q) runs after it in its own copy
// of the chunk step, so the loop carries no row tests.
template <typename OT, int PT, bool GATE>
__global__ __launch_bounds__(Shape<PT>::NT) void ssd_kernel(ChunkKernelArgs a) {
  using Sh = Shape<PT>;
  constexpr int NPT = Sh::NPT, NW = Sh::NW, NT = Sh::NT, RPT = Sh::RPT, XPR = Sh::XPR;
  __shared__ Smem<PT> sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;

  const int ntiles = a.headdim / PT;
  int bid = blockIdx.x;
  const int ptile = bid % ntiles;
  bid /= ntiles;
  const int h = bid % a.nheads;
  const int b = bid / a.nheads;
  const int g = h / (a.nheads / a.ngroups);
  const int p0 = ptile * PT;
  const int H = a.nheads, P = a.headdim, G = a.ngroups, L = a.seqlen;
  const float Al2 = a.A[h] * kLog2e;
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.0f;
  // The decay between positions s <= l of a chunk is 2^(dA[l] - dA[s]).  It is
  // factored through the start of s's 16-block, 2^(dA[l] - dA[16 J]) times
  // 2^(dA[16 J] - dA[s]), two tables shared by the workgroup, when the second
  // factor cannot overflow: |dt A| log2(e) below 6 per step (the 15 steps of a
  // block then stay under 2^90).  Otherwise each element takes its own
  // exponential.
  const bool factored = a.dt_max * fabsf(Al2) < 6.0f;

  const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(a.x);
  const uint16_t* __restrict__ Bg = static_cast<const uint16_t*>(a.B);
  const uint16_t* __restrict__ Cg = static_cast<const uint16_t*>(a.C);

  const int rg = tid >> 3, pc = tid & 7;            // C / B: row group, 8-column piece
  const int rgx = tid / XPR, pcx = tid % XPR;       // x: row pair, 8-column piece
  const bool xload = tid < Sh::XT;

  // Rows past the end of the sequence (the ragged last chunk) load as zeros,
  // and their dt is set to 0 below: they add nothing to the state, do not
  // decay it, and their outputs are not stored.
  auto load_chunk = [&](int c, ChunkRegs<PT>& R, auto ragged) {
    constexpr bool kRag = decltype(ragged)::value;
    // chunk bases are wave-uniform; per-lane offsets fit in 32 bits
    const size_t tok = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
    R.valid = kRag ? L - c * kQ : kQ;
    const uint16_t* Cc = Cg + (tok * G + g) * kN;
    const uint16_t* Bc = Bg + (tok * G + g) * kN;
    const uint16_t* xc = xg + (tok * H + h) * P + p0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RPT * rg + i;
      const int o = r * G * kN + 8 * pc;
      const bool in = !kRag || r < R.valid;
      R.c[i] = load16_if(Cc + o, in);
      R.b[i] = load16_if(Bc + o, in);
    }
    if (xload) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 2 * rgx + i;
        const bool in = !kRag || r < R.valid;
        R.x[i] = load16_if(xc + r * H * P + 8 * pcx, in);
      }
    }
    if (tid < R.valid) R.dt = a.dt[tok * H + h + tid * H];
  };

  // bf16 j of a 16-byte piece
  auto half = [](const uint4& v, int j) -> uint32_t {
    return (reinterpret_cast<const uint32_t*>(&v)[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
  };

  auto store_chunk = [&](const ChunkRegs<PT>& R, auto ragged) {
    constexpr bool kRag = decltype(ragged)::value;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      *reinterpret_cast<uint4*>(&sm.C[RPT * rg + i][8 * pc]) = R.c[i];
      *reinterpret_cast<uint4*>(&sm.B[RPT * rg + i][8 * pc]) = R.b[i];
    }
    // B transposed: RPT consecutive s for each of the 8 n of this piece
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (RPT == 4) {
        const uint32_t lo = half(R.b[0], j) | (half(R.b[1], j) << 16);
        const uint32_t hi = half(R.b[2], j) | (half(R.b[3], j) << 16);
        *reinterpret_cast<uint2*>(&sm.Bt[8 * pc + j][swz(8 * pc + j, 4 * rg)]) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(&sm.Bt[8 * pc + j][swz(8 * pc + j, 2 * rg)]) = half(R.b[0], j) | (half(R.b[1], j) << 16);
      }
    }
    if (xload) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint32_t*>(&sm.Xt[8 * pcx + j][swz(8 * pcx + j, 2 * rgx)]) = half(R.x[0], j) | (half(R.x[1], j) << 16);
    }
    if (tid < kQ) {
      const float pre = R.dt + dtb;
      const float d = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                    : __builtin_amdgcn_fmed3f(pre, a.dt_min, a.dt_max);
      sm.dt[tid] = !kRag || tid < R.valid ? d : 0.0f;
    }
  };

  // State block of this wave: n in [16 nb, 16 nb + 16), p in [16 ps, 16 ps + 16);
  // lane holds S[p = 16 ps + 4 lg + r][n = 16 nb + li].
  const int nb = w & 3, ps = w >> 2;
  f32x4 S;
  const size_t sbase = ((static_cast<size_t>(b) * H + h) * P + p0) * kN;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 16 * ps + 4 * lg + r;
    S[r] = a.state_in ? a.state_in[sbase + static_cast<size_t>(p) * kN + 16 * nb + li] : 0.0f;
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * ps + 4 * lg + r;
      uint16_t hi, lo;
      split_bf16(S[r], hi, lo);
      sm.Shi[p][16 * nb + li] = hi;
      sm.Slo[p][16 * nb + li] = lo;
    }
  };
  publish_state();

  // Output items of this wave: 16-row block I of the chunk and 16-column
  // subtile pt; (w, 0) and (7 - w, NPT - 1) have 9 causal 16x16 blocks
  // between them, for every wave.
  const int I0 = w, I1 = 7 - w;
  const int pt1 = NPT - 1;
  float dv0 = 0.0f, dv1 = 0.0f;  // D for the lane's output column of each item
  if (a.D) {
    const int pa = p0 + li, pb = p0 + 16 * pt1 + li;
    dv0 = a.d_per_channel ? a.D[static_cast<size_t>(h) * P + pa] : a.D[h];
    dv1 = a.d_per_channel ? a.D[static_cast<size_t>(h) * P + pb] : a.D[h];
  }

  ChunkRegs<PT> R;
  const int nfull = L / kQ;  // whole chunks; a ragged one follows when L % Q != 0
  // One chunk step: stage chunk c (already in R) in LDS, prefetch the next
  // whole chunk, emit the chunk's outputs and advance the state.
  auto chunk_step = [&](const int c, auto ragged) {
    constexpr bool kRag = decltype(ragged)::value;
    __syncthreads();  // the previous chunk's LDS readers are done
    store_chunk(R, ragged);
    if (!kRag && c + 1 < nfull) load_chunk(c + 1, R, std::false_type{});
    __syncthreads();

    // Every wave scans the chunk's log2 decays in registers (lane: steps
    // 2 lane and 2 lane + 1), then writes its share of the tables.
    {
      const float2 dt2 = *reinterpret_cast<const float2*>(&sm.dt[2 * lane]);
      const float v0 = dt2.x * Al2, v1 = dt2.y * Al2;
      float incl = v0 + v1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const float d0 = incl - v1, d1 = incl;  // dA[2 lane], dA[2 lane + 1]
      const float last = __shfl(incl, 63);
      // 16-blocks: wave w fills EL[J] for J = w, w + NW, ...
#pragma unroll
      for (int J = w; J < 8; J += NW) {
        const float ref = __shfl(d0, 8 * J);  // dA[16 J]
        if (2 * lane >= 16 * J) {
          sm.EL[J][2 * lane] = exp2_fast(d0 - ref);
          sm.EL[J][2 * lane + 1] = exp2_fast(d1 - ref);
        }
      }
      if (w == 0) {
        const float ref = __shfl(d0, 8 * (lane >> 3));  // dA at the start of this lane's 16-block
        sm.ESD[2 * lane] = exp2_fast(ref - d0) * dt2.x;
        sm.ESD[2 * lane + 1] = exp2_fast(ref - d1) * dt2.y;
        sm.dA[2 * lane] = d0;
        sm.dA[2 * lane + 1] = d1;
      } else if (w == 1) {
        sm.eA[2 * lane] = exp2_fast(d0);
        sm.eA[2 * lane + 1] = exp2_fast(d1);
        sm.wS[2 * lane] = exp2_fast(last - d0) * dt2.x;
        sm.wS[2 * lane + 1] = exp2_fast(last - d1) * dt2.y;
      }
    }
    __syncthreads();

    // x weighted for the state update, split into bf16 high and low parts:
    // XW[p][s] = wS[s] x[s][p] (every thread a few elements)
#pragma unroll
    for (int idx = tid; idx < PT * (kQ / 8); idx += NT) {
      const int p = idx / (kQ / 8), s0 = 8 * (idx % (kQ / 8));
      const bf16x8 xr = *reinterpret_cast<const bf16x8*>(&sm.Xt[p][swz(p, s0)]);
      const float4 w0 = *reinterpret_cast<const float4*>(&sm.wS[s0]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sm.wS[s0 + 4]);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      bf16x8 hi8, lo8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = static_cast<float>(xr[j]) * wv[j];
        const __bf16 hv = static_cast<__bf16>(v);
        hi8[j] = hv;
        lo8[j] = static_cast<__bf16>(v - static_cast<float>(hv));
      }
      *reinterpret_cast<bf16x8*>(&sm.XWh[p][s0]) = hi8;
      *reinterpret_cast<bf16x8*>(&sm.XWl[p][s0]) = lo8;
    }

    // Intra-chunk sums of both items: 16x16 blocks J = 0..I of each, walked
    // together (k-th block of each item in step k) with the LDS operands of
    // step k + 1 loaded while step k computes.  M = cb . decay . dt, masked
    // on the diagonal block, split into bf16 high and low parts for the MFMA.
    struct Ops {
      float el;     // factored: 2^(dA[l] - dA[16 J]); otherwise dA[l]
      float4 e4;    // factored: 2^(dA[16 J] - dA[s]) dt[s]; otherwise dA[s]
      s16x4 xv;     // x[s][p] for the MFMA B operand
    };
    auto load_ops = [&](int I, int J, int pt) {
      Ops o;
      const int l_row = 16 * I + li, s0 = 16 * J + 4 * lg;
      o.el = factored ? sm.EL[J][l_row] : sm.dA[l_row];
      o.e4 = *reinterpret_cast<const float4*>(factored ? &sm.ESD[s0] : &sm.dA[s0]);
      o.xv = *reinterpret_cast<const s16x4*>(&sm.Xt[16 * pt + li][swz(16 * pt + li, s0)]);
      return o;
    };
    // cb^T block (I, J) from the B rows of block J and the C rows of block I:
    // cb[r] = cb[l = 16 I + li][s = 16 J + 4 lg + r]
    auto intra = [&](int I, int J, const bf16x8 (&bj)[2], const bf16x8 (&ci)[2], const Ops& o, f32x4& acc_hi,
                     f32x4& acc_lo) {
      f32x4 cb = {0.0f, 0.0f, 0.0f, 0.0f};
      cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bj[0], ci[0], cb, 0, 0, 0);
      cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bj[1], ci[1], cb, 0, 0, 0);
      const int l_row = 16 * I + li;
      const float ev[4] = {o.e4.x, o.e4.y, o.e4.z, o.e4.w};
      float dv4[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (!factored) {
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dt[16 * J + 4 * lg]);
        dv4[0] = d4.x; dv4[1] = d4.y; dv4[2] = d4.z; dv4[3] = d4.w;
      }
      s16x4 mhi, mlo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = factored ? cb[r] * o.el * ev[r] : cb[r] * exp2_fast(o.el - ev[r]) * dv4[r];
        // causal mask (only the diagonal block has s > l), applied after the
        // product so a masked overflow never reaches the sum
        const float mv = (J < I || 16 * J + 4 * lg + r <= l_row) ? m : 0.0f;
        uint16_t hi, lo;
        split_bf16(mv, hi, lo);
        mhi[r] = static_cast<short>(hi);
        mlo[r] = static_cast<short>(lo);
      }
      acc_hi = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mhi, o.xv, acc_hi, 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mlo, o.xv, acc_lo, 0, 0, 0);
    };
    auto rows16 = [&](const uint16_t (*M)[kRowN], int blk, bf16x8 (&v)[2]) {
      v[0] = *reinterpret_cast<const bf16x8*>(&M[16 * blk + li][8 * lg]);
      v[1] = *reinterpret_cast<const bf16x8*>(&M[16 * blk + li][32 + 8 * lg]);
    };
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 a0h = zero4, a0l = zero4, a1h = zero4, a1l = zero4;
    {
      bf16x8 c0[2], c1[2], bj[2];
      rows16(sm.C, I0, c0);
      rows16(sm.C, I1, c1);
      rows16(sm.B, 0, bj);
      Ops o0 = load_ops(I0, 0, 0), o1 = load_ops(I1, 0, pt1);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // block k + 1's operands while block k computes (past an item's
        // diagonal they are valid LDS, loaded and not used)
        const int kn = k < 7 ? k + 1 : 7;
        bf16x8 bn[2];
        rows16(sm.B, kn, bn);
        const Ops n0 = load_ops(I0, kn, 0), n1 = load_ops(I1, kn, pt1);
        if (k <= I0) intra(I0, k, bj, c0, o0, a0h, a0l);
        if (k <= I1) intra(I1, k, bj, c1, o1, a1h, a1l);
        bj[0] = bn[0];
        bj[1] = bn[1];
        o0 = n0;
        o1 = n1;
      }
    }

    // Readout of the incoming state, (C_I S^T)[l][p] scaled by 2^dA[l], plus
    // the skip, into the LDS output tile.  Lane holds rows l = 16 I + 4 lg + r
    // at column p = 16 pt + li.
    auto finish = [&](const int I, const int pt, const f32x4& acc_hi, const f32x4& acc_lo, const float dv) {
      f32x4 sr_hi = zero4, sr_lo = zero4;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sm.C[16 * I + li][32 * kk + 8 * lg]);
        const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&sm.Shi[16 * pt + li][32 * kk + 8 * lg]);
        const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&sm.Slo[16 * pt + li][32 * kk + 8 * lg]);
        sr_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, sh, sr_hi, 0, 0, 0);
        sr_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, sl, sr_lo, 0, 0, 0);
      }
      const int p = 16 * pt + li;
      const float4 e4 = *reinterpret_cast<const float4*>(&sm.eA[16 * I + 4 * lg]);
      const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
      const s16x4 xv = *reinterpret_cast<const s16x4*>(&sm.Xt[p][swz(p, 16 * I + 4 * lg)]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float xr = bf16_val(static_cast<uint16_t>(xv[r]));
        sm.O[16 * I + 4 * lg + r][p] = fmaf(dv, xr, fmaf(ev[r], sr_hi[r] + sr_lo[r], acc_hi[r] + acc_lo[r]));
      }
    };
    // The output pieces: thread tid stores 8 values of row l = tid / PPR (all
    // of the tile's pieces, one per thread).  Its gate values are fetched
    // here so that their latency overlaps the state readout.
    constexpr int PPR = PT / 8;  // 8-value pieces per row
    static_assert(kQ * PPR == NT, "one output piece per thread");
    const int ol = tid / PPR, oq = tid % PPR;
    const size_t tok0 = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
    const size_t e0 = ((tok0 + ol) * H + h) * P + p0 + 8 * oq;
    const bool orow = !kRag || ol < L - c * kQ;
    uint4 zr0 = make_uint4(0u, 0u, 0u, 0u), zr1 = zr0;
    if constexpr (GATE) {
      if (orow) {
        if (a.z_bf16) {
          zr0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.z) + e0);
        } else {
          zr0 = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.z) + e0);
          zr1 = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.z) + e0 + 4);
        }
      }
    }
    finish(I0, 0, a0h, a0l, dv0);
    finish(I1, pt1, a1h, a1l, dv1);
    __syncthreads();  // output tile and XW complete; every wave is done reading Shi/Slo

    // ---- the output tile to HBM: whole 16-byte pieces of each row (rows of
    // the sequence only), times SiLU(z) when gated
    if (orow) {
      const float4 v0 = *reinterpret_cast<const float4*>(&sm.O[ol][8 * oq]);
      const float4 v1 = *reinterpret_cast<const float4*>(&sm.O[ol][8 * oq + 4]);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if constexpr (GATE) {
        float zv[8];
        if (a.z_bf16) {
          const uint32_t zw[4] = {zr0.x, zr0.y, zr0.z, zr0.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            zv[2 * j] = __uint_as_float(zw[j] << 16);
            zv[2 * j + 1] = __uint_as_float(zw[j] & 0xffff0000u);
          }
        } else {
          const uint32_t zw[8] = {zr0.x, zr0.y, zr0.z, zr0.w, zr1.x, zr1.y, zr1.z, zr1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) zv[j] = __uint_as_float(zw[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= silu(zv[j]);
      }
      if constexpr (sizeof(OT) == 4) {
        float* o = static_cast<float*>(a.out) + e0;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        uint4 o;
        o.x = bf16_bits(v[0]) | (static_cast<uint32_t>(bf16_bits(v[1])) << 16);
        o.y = bf16_bits(v[2]) | (static_cast<uint32_t>(bf16_bits(v[3])) << 16);
        o.z = bf16_bits(v[4]) | (static_cast<uint32_t>(bf16_bits(v[5])) << 16);
        o.w = bf16_bits(v[6]) | (static_cast<uint32_t>(bf16_bits(v[7])) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + e0) = o;
      }
    }

    // ---- state update of this wave's block: S <- 2^dA[Q-1] S + XW^T B
    const float dlast = exp2_fast(sm.dA[kQ - 1]);
    f32x4 acc_hi = S * dlast, acc_lo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int s0 = 32 * kk + 8 * lg;
      const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&sm.XWh[16 * ps + li][s0]);
      const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&sm.XWl[16 * ps + li][s0]);
      const bf16x8 bt = *reinterpret_cast<const bf16x8*>(&sm.Bt[16 * nb + li][swz(16 * nb + li, s0)]);
      acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bt, acc_hi, 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bt, acc_lo, 0, 0, 0);
    }
    S = acc_hi + acc_lo;
    publish_state();
  };
  if (nfull > 0) load_chunk(0, R, std::false_type{});
  for (int c = 0; c < nfull; ++c) chunk_step(c, std::false_type{});
  if (nfull * kQ < L) {
    load_chunk(nfull, R, std::true_type{});
    chunk_step(nfull, std::true_type{});
  }

  if (a.state_out) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * ps + 4 * lg + r;
      a.state_out[sbase + static_cast<size_t>(p) * kN + 16 * nb + li] = S[r];
    }
  }
}

template <typename OT, int PT>
hipError_t go(const ChunkLaunch& l, hipStream_t s) {
  const ChunkKernelArgs& k = l.k;
  const unsigned blocks = static_cast<unsigned>(k.batch) * k.nheads * (k.headdim / PT);
  if (blocks == 0) return hipSuccess;
  return timed_launch(s, [&] {
    if (k.z != nullptr)
      hipLaunchKernelGGL((ssd_kernel<OT, PT, true>), dim3(blocks), dim3(Shape<PT>::NT), 0, s, k);
    else
      hipLaunchKernelGGL((ssd_kernel<OT, PT, false>), dim3(blocks), dim3(Shape<PT>::NT), 0, s, k);
  });
}

}  // namespace

size_t chunk_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_chunk(const ChunkLaunch& l, hipStream_t stream) {
  const bool p32 = l.k.headdim % 32 == 0;
  if (l.out_dtype == kBF16) return p32 ? go<bf16s, 32>(l, stream) : go<bf16s, 16>(l, stream);
  return p32 ? go<float, 32>(l, stream) : go<float, 16>(l, stream);
}

}  // namespace ssm
