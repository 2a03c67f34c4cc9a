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
  uint16_t Bt[kN][kRowQ];   // B chunk transposed [n][s]
  uint16_t Xt[PT][kRowQ];   // x chunk slice transposed [p][s]
  uint16_t Shi[PT][kRowN];  // state entering the chunk, [p][n], bf16 high part
  uint16_t Slo[PT][kRowN];  //                                   bf16 low part
  float dA[kQ];             // inclusive cumsum of dt * A * log2(e)
  float dt[kQ];             // dt after softplus and clip
  float wS[kQ];             // 2^(dA[Q-1] - dA[s]) * dt[s]: state-update weights
  float eA[kQ];             // 2^dA[l]: decay of the incoming state
};

// Registers holding one chunk's global loads until they are stored to LDS.
struct ChunkRegs {
  uint4 c[4], b[4], x[4];
  float dt;
};

template <typename OT, int PT>
__global__ __launch_bounds__(256) void ssd_kernel(ChunkKernelArgs a) {
  constexpr int NPT = PT / 16;  // 16-wide subtiles of the headdim slice
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

  const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(a.x);
  const uint16_t* __restrict__ Bg = static_cast<const uint16_t*>(a.B);
  const uint16_t* __restrict__ Cg = static_cast<const uint16_t*>(a.C);

  // load assignment: thread -> 4 consecutive rows x 8 columns (16 bytes)
  const int rg = tid >> 3, pc = tid & 7;               // C / B: 32 row groups x 8 pieces
  constexpr int XPC = PT / 8;                          // x pieces per row
  const int rgx = tid / XPC, pcx = tid % XPC;          // x: 32 row groups x XPC pieces
  const bool xload = tid < 32 * XPC;

  auto load_chunk = [&](int c, ChunkRegs& R) {
    const size_t tok = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t row = tok + 4 * rg + i;
      R.c[i] = *reinterpret_cast<const uint4*>(Cg + (row * G + g) * kN + 8 * pc);
      R.b[i] = *reinterpret_cast<const uint4*>(Bg + (row * G + g) * kN + 8 * pc);
    }
    if (xload) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t row = tok + 4 * rgx + i;
        R.x[i] = *reinterpret_cast<const uint4*>(xg + (row * H + h) * P + p0 + 8 * pcx);
      }
    }
    if (tid < kQ) R.dt = a.dt[(tok + tid) * H + h];
  };

  auto store_chunk = [&](const ChunkRegs& R) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&sm.C[4 * rg + i][8 * pc]) = R.c[i];
      *reinterpret_cast<uint4*>(&sm.B[4 * rg + i][8 * pc]) = R.b[i];
    }
    // B transposed: 4 consecutive s for each of the 8 n of this piece
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = (j & 1) * 16;
      uint32_t lo = ((reinterpret_cast<const uint32_t*>(&R.b[0])[j >> 1] >> sh) & 0xffffu) |
                    (((reinterpret_cast<const uint32_t*>(&R.b[1])[j >> 1] >> sh) & 0xffffu) << 16);
      uint32_t hi = ((reinterpret_cast<const uint32_t*>(&R.b[2])[j >> 1] >> sh) & 0xffffu) |
                    (((reinterpret_cast<const uint32_t*>(&R.b[3])[j >> 1] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<uint2*>(&sm.Bt[8 * pc + j][4 * rg]) = make_uint2(lo, hi);
    }
    if (xload) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = (j & 1) * 16;
        uint32_t lo = ((reinterpret_cast<const uint32_t*>(&R.x[0])[j >> 1] >> sh) & 0xffffu) |
                      (((reinterpret_cast<const uint32_t*>(&R.x[1])[j >> 1] >> sh) & 0xffffu) << 16);
        uint32_t hi = ((reinterpret_cast<const uint32_t*>(&R.x[2])[j >> 1] >> sh) & 0xffffu) |
                      (((reinterpret_cast<const uint32_t*>(&R.x[3])[j >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&sm.Xt[8 * pcx + j][4 * rgx]) = make_uint2(lo, hi);
      }
    }
    if (tid < kQ) {
      const float pre = R.dt + dtb;
      const float d = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                    : __builtin_amdgcn_fmed3f(pre, a.dt_min, a.dt_max);
      sm.dt[tid] = d;
      sm.wS[tid] = d * Al2;  // per-step log2 decay, scanned below
    }
  };

  // state accumulators: wave w owns n in [16w, 16w+16) for every p subtile;
  // lane holds S[p = 16pt + 4lg + r][n = 16w + li]
  f32x4 S[NPT];
  const size_t sbase = ((static_cast<size_t>(b) * H + h) * P + p0) * kN;
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pt + 4 * lg + r;
      S[pt][r] = a.state_in ? a.state_in[sbase + static_cast<size_t>(p) * kN + 16 * w + li] : 0.0f;
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pt + 4 * lg + r;
        uint16_t hi, lo;
        split_bf16(S[pt][r], hi, lo);
        sm.Shi[p][16 * w + li] = hi;
        sm.Slo[p][16 * w + li] = lo;
      }
    }
  };
  publish_state();

  const float* Dp = a.D;
  ChunkRegs R;
  load_chunk(0, R);
  for (int c = 0; c < a.nchunks; ++c) {
    __syncthreads();  // previous chunk's LDS readers are done
    store_chunk(R);
    if (c + 1 < a.nchunks) load_chunk(c + 1, R);
    __syncthreads();
    if (w == 0) {
      // inclusive scan of the per-step log2 decays: two steps per lane
      const float v0 = sm.wS[2 * lane], v1 = sm.wS[2 * lane + 1];
      float incl = v0 + v1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const float excl = incl - (v0 + v1);
      const float d0 = excl + v0, d1 = incl;
      const float last = __shfl(incl, 63);
      sm.dA[2 * lane] = d0;
      sm.dA[2 * lane + 1] = d1;
      sm.eA[2 * lane] = exp2_fast(d0);
      sm.eA[2 * lane + 1] = exp2_fast(d1);
      sm.wS[2 * lane] = exp2_fast(last - d0) * sm.dt[2 * lane];
      sm.wS[2 * lane + 1] = exp2_fast(last - d1) * sm.dt[2 * lane + 1];
    }
    __syncthreads();
    const size_t tok0 = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;

    // ---- output rows: blocks I = w and 7 - w
#pragma unroll 1
    for (int bi = 0; bi < 2; ++bi) {
      const int I = bi == 0 ? w : 7 - w;
      const int l_row = 16 * I + li;  // row of cb held by this lane in the M layout
      const float dAl = sm.dA[l_row];
      f32x4 acc[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int J = 0; J <= I; ++J) {
        f32x4 cbt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sm.B[16 * J + li][32 * kk + 8 * lg]);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sm.C[16 * I + li][32 * kk + 8 * lg]);
          cbt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, cbt, 0, 0, 0);
        }
        // cbt[r] = cb[l = 16I + li][s = 16J + 4lg + r]
        const float4 dAs = *reinterpret_cast<const float4*>(&sm.dA[16 * J + 4 * lg]);
        const float4 dts = *reinterpret_cast<const float4*>(&sm.dt[16 * J + 4 * lg]);
        const float dAsv[4] = {dAs.x, dAs.y, dAs.z, dAs.w};
        const float dtsv[4] = {dts.x, dts.y, dts.z, dts.w};
        s16x4 mhi, mlo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * J + 4 * lg + r;
          const float ex = (s <= l_row) ? dAl - dAsv[r] : kNegInf;  // mask before the exponential
          const float m = cbt[r] * exp2_fast(ex) * dtsv[r];
          uint16_t hi, lo;
          split_bf16(m, hi, lo);
          mhi[r] = static_cast<short>(hi);
          mlo[r] = static_cast<short>(lo);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const s16x4 xv = *reinterpret_cast<const s16x4*>(&sm.Xt[16 * pt + li][16 * J + 4 * lg]);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mhi, xv, acc[pt], 0, 0, 0);
          acc[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mlo, xv, acc[pt], 0, 0, 0);
        }
      }
      // readout of the incoming state: (C_I S^T)[l][p], scaled by 2^dA[l]
      const float4 e4 = *reinterpret_cast<const float4*>(&sm.eA[16 * I + 4 * lg]);
      const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        f32x4 sr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sm.C[16 * I + li][32 * kk + 8 * lg]);
          const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&sm.Shi[16 * pt + li][32 * kk + 8 * lg]);
          const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&sm.Slo[16 * pt + li][32 * kk + 8 * lg]);
          sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, sh, sr, 0, 0, 0);
          sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, sl, sr, 0, 0, 0);
        }
        // lane holds rows l = 16I + 4lg + r at column p = 16pt + li
        const int p = 16 * pt + li;
        const s16x4 xv = *reinterpret_cast<const s16x4*>(&sm.Xt[p][16 * I + 4 * lg]);
        const float dv = Dp ? (a.d_per_channel ? Dp[static_cast<size_t>(h) * P + p0 + p] : Dp[h]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int l = 16 * I + 4 * lg + r;
          const float xr = bf16_val(static_cast<uint16_t>(xv[r]));
          const float yv = fmaf(dv, xr, fmaf(ev[r], sr[r], acc[pt][r]));
          const size_t o = ((tok0 + l) * H + h) * P + p0 + p;
          if constexpr (sizeof(OT) == 4) {
            static_cast<float*>(a.out)[o] = yv;
          } else {
            static_cast<uint16_t*>(a.out)[o] = bf16_bits(yv);
          }
        }
      }
    }

    __syncthreads();  // every wave is done reading Shi/Slo
    // ---- state update: S <- 2^dA[Q-1] S + (wS . x)^T B
    const float dlast = exp2_fast(sm.dA[kQ - 1]);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      f32x4 acc = S[pt] * dlast;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int s0 = 32 * kk + 8 * lg;
        const bf16x8 xr = *reinterpret_cast<const bf16x8*>(&sm.Xt[16 * pt + li][s0]);
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
        const bf16x8 bt = *reinterpret_cast<const bf16x8*>(&sm.Bt[16 * w + li][s0]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi8, bt, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo8, bt, acc, 0, 0, 0);
      }
      S[pt] = acc;
    }
    publish_state();
  }

  if (a.state_out) {
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pt + 4 * lg + r;
        a.state_out[sbase + static_cast<size_t>(p) * kN + 16 * w + li] = S[pt][r];
      }
    }
  }
}

template <typename OT, int PT>
hipError_t go(const ChunkLaunch& l, hipStream_t s) {
  const ChunkKernelArgs& k = l.k;
  const unsigned blocks = static_cast<unsigned>(k.batch) * k.nheads * (k.headdim / PT);
  if (blocks == 0) return hipSuccess;
  return timed_launch(s, [&] { hipLaunchKernelGGL((ssd_kernel<OT, PT>), dim3(blocks), dim3(256), 0, s, k); });
}

}  // namespace

size_t chunk_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_chunk(const ChunkLaunch& l, hipStream_t stream) {
  const bool p32 = l.k.headdim % 32 == 0;
  if (l.out_dtype == kBF16) return p32 ? go<bf16s, 32>(l, stream) : go<bf16s, 16>(l, stream);
  return p32 ? go<float, 32>(l, stream) : go<float, 16>(l, stream);
}

}  // namespace ssm
