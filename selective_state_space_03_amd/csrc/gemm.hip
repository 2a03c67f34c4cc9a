// Projection GEMMs of the layer for gfx950: C = A W^T with W (N, K) in bf16
// (a weight stored as (out, in)), A (M, K) in bf16 or fp32, fp32 accumulation.
//
// Page "Axon-SSM: selective state space model", section "Algorithm": in_proj
// (D -> 2E, split into x_branch and z) and out_proj (E -> D) are dense
// projections of every token.  They are the only dense contractions of the
// layer and run on the matrix cores:
//   v_mfma_f32_32x32x16_bf16, a 128x64 tile per wave (128 accumulator
//   registers), 8 waves per workgroup (256x256 output tile, two waves per SIMD
//   so one computes while the other waits on LDS), K in steps staged in LDS
//   (double-buffered, the next step's global loads in flight during the
//   current step's MFMAs; fragments of the next MFMA sub-step read from LDS
//   while the current one computes).  Measured against one 128x128 wave per
//   SIMD: in_proj 221 vs 233 us, out_proj 200 vs 228 us.
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

#include <algorithm>
#include <type_traits>

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef GEMM_WN
#define GEMM_WN 4
#endif
constexpr int kWavesN = GEMM_WN;           // waves along N (2 along M)
constexpr int kThreads = 128 * kWavesN;    // 8 waves: 2 x 4 over the output tile

// GM x GN 32x32 MFMA blocks per wave (wave tile 32 GM rows of A by 32 GN rows
// of W), so the workgroup tile is BM = 64 GM by BN = 64 GN; K steps of BK.
template <int GM, int GN, int BK, bool SPLIT>
struct Cfg {
  static constexpr int BM = 64 * GM, BN = 32 * GN * kWavesN;
  static constexpr int kPitch = BK + 8;  // LDS row pitch in bf16 (rows land on different banks)
  static constexpr int APR = SPLIT ? BK / 4 : BK / 8;  // 16-byte pieces per A row of a K step
  static constexpr int WPR = BK / 8;
  static constexpr int AP = BM * APR / kThreads;  // A pieces per thread
  static constexpr int WP = BN * WPR / kThreads;
  static_assert(BM * APR % kThreads == 0 && BN * WPR % kThreads == 0, "whole pieces per thread");
};

template <int GM, int GN, int BK, bool SPLIT>
struct GemmSmem {
  using C = Cfg<GM, GN, BK, SPLIT>;
  uint16_t A[2][C::BM][C::kPitch];
  uint16_t Alo[SPLIT ? 2 : 1][SPLIT ? C::BM : 1][C::kPitch];
  uint16_t W[2][C::BN][C::kPitch];
};

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// blockIdx.x -> tile: each XCD (workgroups are dealt to the 8 XCDs in turn)
// takes a contiguous range of tiles, and inside it the M tiles of one N tile
// are consecutive, so a W tile is fetched once per L2 and reused.
__device__ __forceinline__ int xcd_tile() {
  const int n = gridDim.x, per = n / 8, rem = n % 8;
  const int x = blockIdx.x % 8, s = blockIdx.x / 8;
  return (x < rem) ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
}

// K split: blockIdx.y takes K range [ky Kc, min(K, (ky + 1) Kc)) and, when
// there is more than one range, writes its fp32 partial tile to ws[ky]
// (M x N); gemm_reduce adds the partials in order.
// EDGE: the shape has partial tiles (M, N or K not a multiple of the tile),
// so loads and stores are guarded; otherwise they are not.
//
// v_mfma_f32_32x32x16_bf16 with W rows as the first operand and A rows as the
// second: lane l supplies row l % 32 of its operand at k = 8 (l / 32) .. + 7,
// and holds in accumulator register r the output (n = 8 (r / 4) + 4 (l / 32)
// + r % 4, m = l % 32) of the block, i.e. four runs of 4 consecutive columns.
#ifndef GEMM_WPE
#define GEMM_WPE 2
#endif
template <typename AT, typename OT, int GM, int GN, int BK, bool EDGE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GEMM_WPE, GEMM_WPE))) void gemm_kernel(GemmArgs g) {
  constexpr bool kSplit = std::is_same<AT, float>::value;
  static_assert(BK % 16 == 0, "whole MFMA K steps");
  using C = Cfg<GM, GN, BK, kSplit>;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ GemmSmem<GM, GN, BK, kSplit> sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int t = xcd_tile();
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;
  const int kbeg = blockIdx.y * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);

  uint4 sa[C::AP], sw[C::WP];
  // A guarded piece is loaded from a clamped (valid) address and zeroed after,
  // which keeps the loads free of branches.
  auto piece = [&](const char* base, size_t ld_bytes, int row, int rows, int col_bytes, int k, int klim) -> uint4 {
    if constexpr (!EDGE) {
      return *reinterpret_cast<const uint4*>(base + static_cast<size_t>(row) * ld_bytes + col_bytes);
    } else {
      const bool ok = row < rows && k < klim;
      const int rc = ok ? row : 0;
      const int cc = ok ? col_bytes : 0;
      uint4 v = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(rc) * ld_bytes + cc);
      if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
      return v;
    }
  };
  const char* Ab = static_cast<const char*>(g.A);
  const char* Wb = reinterpret_cast<const char*>(g.W);
  constexpr int kAes = kSplit ? 4 : 2;  // bytes per A element
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
      const int idx = tid + kThreads * i, r = idx / C::APR, pc = idx % C::APR;
      const int k = k0 + (kSplit ? 4 : 8) * pc;
      sa[i] = piece(Ab, static_cast<size_t>(g.lda) * kAes, m0 + r, g.M, k * kAes, k, kend);
    }
#pragma unroll
    for (int i = 0; i < C::WP; ++i) {
      const int idx = tid + kThreads * i, r = idx / C::WPR, pc = idx % C::WPR;
      const int k = k0 + 8 * pc;
      sw[i] = piece(Wb, static_cast<size_t>(g.ldw) * 2, n0 + r, g.N, k * 2, k, kend);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
      const int idx = tid + kThreads * i, r = idx / C::APR, pc = idx % C::APR;
      if constexpr (kSplit) {
        const float v[4] = {__uint_as_float(sa[i].x), __uint_as_float(sa[i].y), __uint_as_float(sa[i].z),
                            __uint_as_float(sa[i].w)};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi[j] = bf16_rne(v[j]);
          lo[j] = bf16_rne(v[j] - __uint_as_float(hi[j] << 16));
        }
        *reinterpret_cast<uint2*>(&sm.A[buf][r][4 * pc]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        *reinterpret_cast<uint2*>(&sm.Alo[buf][r][4 * pc]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      } else {
        *reinterpret_cast<uint4*>(&sm.A[buf][r][8 * pc]) = sa[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::WP; ++i) {
      const int idx = tid + kThreads * i, r = idx / C::WPR, pc = idx % C::WPR;
      *reinterpret_cast<uint4*>(&sm.W[buf][r][8 * pc]) = sw[i];
    }
  };

  // wave tile: A rows [32 GM wm, +32 GM), W rows [32 GN wn, +32 GN)
  const int wm = w & 1, wn = w >> 1;
  f32x16 acc[GN][GM];
#pragma unroll
  for (int j = 0; j < GN; ++j)
#pragma unroll
    for (int i = 0; i < GM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // One K step from LDS buffer buf in MFMA sub-steps of 16: the fragments of
  // sub-step kk + 1 are read while those of kk feed the matrix cores, and the
  // scheduler is told to interleave the two.
  struct Frags {
    bf16x8 w[GN], a[GM], alo[kSplit ? GM : 1];
  };
  auto read_frags = [&](int buf, int kk, Frags& f) {
    const int k = 16 * kk + 8 * lh;
#pragma unroll
    for (int j = 0; j < GN; ++j) f.w[j] = *reinterpret_cast<const bf16x8*>(&sm.W[buf][32 * GN * wn + 32 * j + l32][k]);
#pragma unroll
    for (int i = 0; i < GM; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(&sm.A[buf][32 * GM * wm + 32 * i + l32][k]);
    if constexpr (kSplit) {
#pragma unroll
      for (int i = 0; i < GM; ++i)
        f.alo[i] = *reinterpret_cast<const bf16x8*>(&sm.Alo[buf][32 * GM * wm + 32 * i + l32][k]);
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int j = 0; j < GN; ++j)
#pragma unroll
      for (int i = 0; i < GM; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[j], f.a[i], acc[j][i], 0, 0, 0);
    if constexpr (kSplit) {
#pragma unroll
      for (int j = 0; j < GN; ++j)
#pragma unroll
        for (int i = 0; i < GM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[j], f.alo[i], acc[j][i], 0, 0, 0);
    }
  };
  constexpr int kReads = GN + GM * (kSplit ? 2 : 1);
  constexpr int kMfmas = GN * GM * (kSplit ? 2 : 1);
  constexpr int kPer = kMfmas / kReads > 0 ? kMfmas / kReads : 1;
  auto compute = [&](int buf) {
    Frags f[2];
    read_frags(buf, 0, f[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) {
        read_frags(buf, kk + 1, f[(kk + 1) & 1]);
        mfmas(f[kk & 1]);
#pragma unroll
        for (int r = 0; r < kReads; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
        }
        if (kMfmas > kPer * kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kPer * kReads, 0);
      } else {
        mfmas(f[kk & 1]);
      }
    }
  };

  const int KT = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  if (KT > 0) {
    gload(kbeg);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kbeg + (kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // acc[j][i] lane (l32, lh), register 4 q + e: row m = m0 + 32 GM wm + 32 i
  // + l32, column n = n0 + 32 GN wn + 32 j + 8 q + 4 lh + e
  const int mb = m0 + 32 * GM * wm + l32;
  const int nb = 32 * GN * wn + 4 * lh;
  if (gridDim.y > 1) {  // fp32 partial of this K range
    float* part = g.ws + static_cast<size_t>(blockIdx.y) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < GM; ++i) {
      const int m = mb + 32 * i;
      if (EDGE && m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < GN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + nb + 32 * j + 8 * q;
          if (EDGE && n >= g.N) continue;
          const f32x16& v = acc[j][i];
          *reinterpret_cast<float4*>(part + static_cast<size_t>(m) * g.N + n) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
    }
    return;
  }
  const bool second = n0 >= g.n_split;
  void* out = second ? g.C1 : g.C0;
  const int ncol0 = second ? n0 - g.n_split : n0;
  const int ncols = second ? g.N - g.n_split : g.n_split;
  const int ldc = second ? g.ldc1 : g.ldc0;
#pragma unroll
  for (int i = 0; i < GM; ++i) {
    const int m = mb + 32 * i;
    if (EDGE && m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < GN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = ncol0 + nb + 32 * j + 8 * q;
        if (EDGE && c >= ncols) continue;  // ncols % 4 == 0: a 4-column piece is all in or all out
        const f32x16& v = acc[j][i];
        const size_t o = static_cast<size_t>(m) * ldc + c;
        if constexpr (std::is_same<OT, float>::value) {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + o) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
              make_uint2(bf16_rne(v[4 * q]) | (bf16_rne(v[4 * q + 1]) << 16),
                         bf16_rne(v[4 * q + 2]) | (bf16_rne(v[4 * q + 3]) << 16));
        }
      }
  }
}

// Sum of the K-range partials (in range order) into the outputs, 4 columns a
// thread.
template <typename OT>
__global__ __launch_bounds__(256) void gemm_reduce(GemmArgs g, int parts) {
  const size_t q = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;  // 4-column piece
  const size_t total = static_cast<size_t>(g.M) * (g.N / 4);
  if (q >= total) return;
  const size_t m = q / (g.N / 4);
  const int n = static_cast<int>(q - m * (g.N / 4)) * 4;
  const size_t plane = static_cast<size_t>(g.M) * g.N;
  float4 s = reinterpret_cast<const float4*>(g.ws)[q];
  for (int p = 1; p < parts; ++p) {
    const float4 v = reinterpret_cast<const float4*>(g.ws + p * plane)[q];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const bool second = n >= g.n_split;
  void* out = second ? g.C1 : g.C0;
  const size_t o = m * (second ? g.ldc1 : g.ldc0) + (second ? n - g.n_split : n);
  if constexpr (std::is_same<OT, float>::value) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = s;
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
        make_uint2(bf16_rne(s.x) | (bf16_rne(s.y) << 16), bf16_rne(s.z) | (bf16_rne(s.w) << 16));
  }
}

#ifndef GEMM_FM
#define GEMM_FM 4
#endif
#ifndef GEMM_FN
#define GEMM_FN 2
#endif
#ifndef GEMM_BK
#define GEMM_BK 64
#endif
#ifndef GEMM_SPLIT_BK
#define GEMM_SPLIT_BK 32
#endif

// K ranges for a shape: one when the tiles alone fill the chip, else enough to
// reach about 240 workgroups (one per CU, 256 CUs), keeping each range at
// least 1024 deep; only as many as the workspace holds partials for.
int k_parts(int M, int N, int K, bool split_a, size_t ws_bytes) {
  const int BM = 64 * GEMM_FM, BN = 32 * GEMM_FN * kWavesN;
  (void)split_a;
  const long tiles = static_cast<long>((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles >= 160 || K < 2048) return 1;
  int parts = static_cast<int>(std::min<long>((240 + tiles - 1) / tiles, K / 1024));
  const size_t plane = static_cast<size_t>(M) * N * 4;
  while (parts > 1 && static_cast<size_t>(parts) * plane > ws_bytes) --parts;
  return std::max(parts, 1);
}

template <typename AT, typename OT>
hipError_t go(const GemmArgs& g0, hipStream_t s) {
  constexpr bool kSplit = std::is_same<AT, float>::value;
  constexpr int FM = GEMM_FM, FN = GEMM_FN, BK = kSplit ? GEMM_SPLIT_BK : GEMM_BK;
  using C = Cfg<FM, FN, BK, kSplit>;
  GemmArgs g = g0;
  const unsigned tiles = static_cast<unsigned>((g.M + C::BM - 1) / C::BM) * static_cast<unsigned>((g.N + C::BN - 1) / C::BN);
  if (tiles == 0) return hipSuccess;
  const int parts = k_parts(g.M, g.N, g.K, kSplit, g.ws != nullptr ? g.ws_bytes : 0);
  g.kchunk = (g.K + parts * BK - 1) / (parts * BK) * BK;
  // whole tiles everywhere (the K ranges included): the unguarded kernel
  if (g.n_split != g.N && g.n_split % C::BN != 0) return hipErrorInvalidValue;  // a tile would straddle the split
  const bool edge = g.M % C::BM != 0 || g.N % C::BN != 0 || g.K % g.kchunk != 0;
  hipError_t e = timed_launch(s, [&] {
    if (edge)
      hipLaunchKernelGGL((gemm_kernel<AT, OT, FM, FN, BK, true>), dim3(tiles, parts), dim3(kThreads), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_kernel<AT, OT, FM, FN, BK, false>), dim3(tiles, parts), dim3(kThreads), 0, s, g);
  });
  if (e != hipSuccess || parts == 1) return e;
  const size_t pieces = static_cast<size_t>(g.M) * (g.N / 4);
  hipLaunchKernelGGL((gemm_reduce<OT>), dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, s, g, parts);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int a_dtype) {
  const int parts = k_parts(M, N, K, a_dtype == kF32, ~static_cast<size_t>(0));
  return parts > 1 ? static_cast<size_t>(parts) * M * N * 4 : 0;
}

hipError_t launch_gemm(const GemmArgs& g, int a_dtype, int out_dtype, hipStream_t stream) {
  if (a_dtype == kBF16) return out_dtype == kBF16 ? go<bf16s, bf16s>(g, stream) : go<bf16s, float>(g, stream);
  return out_dtype == kBF16 ? go<float, bf16s>(g, stream) : go<float, float>(g, stream);
}

}  // namespace ssm
