// Projection GEMMs of the layer for gfx950: C = A W^T with W (N, K) in bf16
// (a weight stored as (out, in)), A (M, K) in bf16 or fp32, fp32 accumulation.
//
// Page "Axon-SSM: selective state space model", section "Algorithm": in_proj
// (D -> 2E, split into x_branch and z) and out_proj (E -> D) are dense
// projections of every token.  They are the only dense contractions of the
// layer and run on the matrix cores:
//   v_mfma_f32_16x16x32_bf16, a 64x64 tile per wave, 4 waves per workgroup
//   (128x128 output tile), K in steps of 64 staged in LDS (double-buffered,
//   the next step's global loads in flight during the current step's MFMAs).
// An fp32 A operand (the scan output feeding out_proj) is split on its way
// into LDS into a bf16 high part and the bf16 of the remainder, and both are
// multiplied (about 16 mantissa bits, so the product keeps fp32-level
// accuracy); a bf16 A (the layer input) is used as it is.
// The MFMA takes W rows as its first operand and A rows as its second, so each
// lane ends with 4 consecutive output columns of one row: 16-byte (fp32) or
// 8-byte (bf16) stores.  Columns n >= n_split go to a second output (in_proj's
// z half), so the split costs nothing.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <type_traits>

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 (144 bytes: rows land on different banks)
constexpr int kThreads = 256;

template <bool SPLIT>
struct GemmSmem {
  uint16_t A[2][kBM][kPitch];
  uint16_t Alo[SPLIT ? 2 : 1][SPLIT ? kBM : 1][kPitch];
  uint16_t W[2][kBN][kPitch];
};

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// Global -> register staging of one K step.
template <typename AT>
struct Stage {
  // bf16 A: 4 pieces of 8; fp32 A: 8 pieces of 4
  static constexpr int kAPieces = std::is_same<AT, float>::value ? 8 : 4;
  uint4 a[kAPieces];
  uint4 w[4];
};

template <typename AT, typename OT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  constexpr bool kSplit = std::is_same<AT, float>::value;
  __shared__ GemmSmem<kSplit> sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;

  // Tile order: each XCD (workgroups are dealt to the 8 XCDs in turn) takes a
  // contiguous range of tiles, and inside it the M tiles of one N tile are
  // consecutive, so a W tile is fetched once per L2 and reused.
  const int tiles_m = (g.M + kBM - 1) / kBM;
  int t;
  {
    const int n = gridDim.x, per = n / 8, rem = n % 8;
    const int x = blockIdx.x % 8, s = blockIdx.x / 8;
    t = (x < rem) ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
  }
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;

  Stage<AT> st;
  // bf16 pieces: row = idx / 8, 8-element piece = idx % 8 (a row of the K step
  // is 8 pieces: 128 contiguous bytes per 8 threads)
  auto gload = [&](int k0) {
    if constexpr (kSplit) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = tid + kThreads * i, r = idx >> 4, pc = idx & 15;
        const int m = m0 + r, k = k0 + 4 * pc;
        st.a[i] = load16_if(static_cast<const float*>(g.A) + static_cast<size_t>(m) * g.lda + k, m < g.M && k < g.K);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i, r = idx >> 3, pc = idx & 7;
        const int m = m0 + r, k = k0 + 8 * pc;
        st.a[i] = load16_if(static_cast<const uint16_t*>(g.A) + static_cast<size_t>(m) * g.lda + k,
                            m < g.M && k < g.K);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i, r = idx >> 3, pc = idx & 7;
      const int n = n0 + r, k = k0 + 8 * pc;
      st.w[i] = load16_if(g.W + static_cast<size_t>(n) * g.ldw + k, n < g.N && k < g.K);
    }
  };
  auto sstore = [&](int buf) {
    if constexpr (kSplit) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = tid + kThreads * i, r = idx >> 4, pc = idx & 15;
        const float v[4] = {__uint_as_float(st.a[i].x), __uint_as_float(st.a[i].y), __uint_as_float(st.a[i].z),
                            __uint_as_float(st.a[i].w)};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi[j] = bf16_rne(v[j]);
          lo[j] = bf16_rne(v[j] - __uint_as_float(hi[j] << 16));
        }
        *reinterpret_cast<uint2*>(&sm.A[buf][r][4 * pc]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        *reinterpret_cast<uint2*>(&sm.Alo[buf][r][4 * pc]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i, r = idx >> 3, pc = idx & 7;
        *reinterpret_cast<uint4*>(&sm.A[buf][r][8 * pc]) = st.a[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i, r = idx >> 3, pc = idx & 7;
      *reinterpret_cast<uint4*>(&sm.W[buf][r][8 * pc]) = st.w[i];
    }
  };

  // wave tile: rows [64 wm, 64 wm + 64) of A, rows [64 wn, 64 wn + 64) of W
  const int wm = w & 1, wn = w >> 1;
  f32x4 acc[4][4];  // [j: W 16-block][i: A 16-block]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int k = 32 * kk + 8 * lg;
      bf16x8 wf[4], af[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = *reinterpret_cast<const bf16x8*>(&sm.W[buf][64 * wn + 16 * j + li][k]);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(&sm.A[buf][64 * wm + 16 * i + li][k]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
      if constexpr (kSplit) {
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(&sm.Alo[buf][64 * wm + 16 * i + li][k]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc[j][i], 0, 0, 0);
      }
    }
  };

  const int KT = (g.K + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload((kt + 1) * kBK);
    compute(kt & 1);
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // acc[j][i] lane (li, lg): rows m = m0 + 64 wm + 16 i + li, columns
  // n = n0 + 64 wn + 16 j + 4 lg + r (r = 0..3)
  const bool second = n0 >= g.n_split;
  void* out = second ? g.C1 : g.C0;
  const int ncol0 = second ? n0 - g.n_split : n0;
  const int ncols = second ? g.N - g.n_split : g.n_split;
  const int ldc = second ? g.ldc1 : g.ldc0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 64 * wm + 16 * i + li;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = ncol0 + 64 * wn + 16 * j + 4 * lg;
      if (c >= ncols) continue;  // ncols % 4 == 0: a 4-column piece is all in or all out
      const f32x4 v = acc[j][i];
      const size_t o = static_cast<size_t>(m) * ldc + c;
      if constexpr (std::is_same<OT, float>::value) {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
            make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
      }
    }
  }
}

template <typename AT, typename OT>
hipError_t go(const GemmArgs& g, hipStream_t s) {
  const unsigned tiles = static_cast<unsigned>((g.M + kBM - 1) / kBM) * static_cast<unsigned>((g.N + kBN - 1) / kBN);
  if (tiles == 0 || g.K == 0) return hipSuccess;
  return timed_launch(s, [&] { hipLaunchKernelGGL((gemm_kernel<AT, OT>), dim3(tiles), dim3(kThreads), 0, s, g); });
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int a_dtype, int out_dtype, hipStream_t stream) {
  if (a_dtype == kBF16) return out_dtype == kBF16 ? go<bf16s, bf16s>(g, stream) : go<bf16s, float>(g, stream);
  return out_dtype == kBF16 ? go<float, bf16s>(g, stream) : go<float, float>(g, stream);
}

}  // namespace ssm
