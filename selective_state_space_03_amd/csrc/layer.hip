// x_proj of the layer for gfx950: B, C and dt_raw of every token from the
// post-conv activation, with the conv recomputed on the fly.
//
// Page "Axon-SSM: selective state space model", section "Algorithm": the
// x_branch goes through the causal depthwise conv1d (k=4) and SiLU, and x_proj
// (E -> 2 d_state + 1) of that activation u gives B, C and dt_raw, in that
// order.  Here
//   u[t, e] = SiLU(sum_k conv_w[e, k] x[t - 3 + k, e] + conv_b[e])
//   xp[t, j] = sum_e u[t, e] W_x[j, e]
// is one pass over x: each wave takes 16 tokens; per 32 channels a lane forms
// u for one token and 8 channels (its own x row plus the three rows before it,
// which come from the neighbouring lanes of its 16-lane row by DPP shifts, or
// from memory / the conv cache / zeros for the first lanes), splits u into a
// bf16 value and the bf16 of its remainder, and feeds both to
// v_mfma_f32_16x16x32_bf16 against W_x rows (j, 16 per block, 3 blocks for the
// 33 outputs).  The channel range is split over blockIdx.y; each range writes
// fp32 partials (tokens x 48) and xproj_reduce adds them in range order into
// B (T, N), C (T, N) and dt_raw (T).
#include <algorithm>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kJ = 48;         // x_proj outputs padded to 3 blocks of 16
constexpr int kTokTile = 64;   // tokens per workgroup (4 waves x 16)

__device__ __forceinline__ uint16_t bf16_rne16(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// value of the lane li - k of the same 16-lane row (row_shr:k); lanes li < k
// keep `old`
template <int K>
__device__ __forceinline__ float shr(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               0x110 + K, 0xF, 0xF, false));
}

__global__ __launch_bounds__(256) void xproj_kernel(XprojArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int T = a.batch * a.seqlen;
  const int tok_raw = blockIdx.x * kTokTile + 16 * w + li;
  const bool tok_ok = tok_raw < T;
  const int tok = tok_ok ? tok_raw : T - 1;
  const int b = tok / a.seqlen, t = tok - b * a.seqlen;  // position inside its sequence
  const int E = a.dim;
  const int steps = (E / 32 + gridDim.y - 1) / gridDim.y;
  const int e_beg = blockIdx.y * steps * 32;
  const int e_end = min(E, e_beg + steps * 32);

  f32x4 acc[3];
#pragma unroll
  for (int jt = 0; jt < 3; ++jt) acc[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const float* xrow = a.x + static_cast<size_t>(tok) * E;
  // this lane's 8 channels of the token's row at e; the next step's are
  // requested before the current step is worked on, so the stream from
  // memory overlaps the arithmetic
  auto load_row = [&](int e, float (&v)[8]) {
    const float4 p0 = *reinterpret_cast<const float4*>(xrow + e);
    const float4 p1 = *reinterpret_cast<const float4*>(xrow + e + 4);
    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
  };
  float nxt[8];
  if (e_beg < e_end) load_row(e_beg + 8 * lg, nxt);
  for (int e0 = e_beg; e0 < e_end; e0 += 32) {
    const int e = e0 + 8 * lg;  // this lane's 8 channels
    float cur[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) cur[c] = nxt[c];
    if (e0 + 32 < e_end) load_row(e + 32, nxt);
    // rows t-1, t-2, t-3: from lanes li-1.. of this row; lanes whose source is
    // outside the row (li < k) read memory; positions before the sequence
    // start read the conv cache (oldest first) or zeros
    float prev[3][8];
#pragma unroll
    for (int k = 1; k <= 3; ++k) {
      float own[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) own[c] = 0.0f;
      if (li < k || t < k) {
        if (t >= k) {
          const float* pr = xrow - static_cast<size_t>(k) * E + e;
#pragma unroll
          for (int c = 0; c < 8; ++c) own[c] = pr[c];
        } else if (a.conv_cache_in != nullptr) {
          const float* cc = a.conv_cache_in + (static_cast<size_t>(b) * E + e) * 3 + (3 + t - k);
#pragma unroll
          for (int c = 0; c < 8; ++c) own[c] = cc[3 * c];
        }
      }
      const bool take_own = li < k || t < k;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v;
        if (k == 1) v = shr<1>(own[c], cur[c]);
        else if (k == 2) v = shr<2>(own[c], cur[c]);
        else v = shr<3>(own[c], cur[c]);
        prev[k - 1][c] = take_own ? own[c] : v;
      }
    }
    // conv + SiLU, then the bf16 value / remainder pair for the MFMA
    bf16x8 uh, ul;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 wk = reinterpret_cast<const float4*>(a.conv_w)[e + c];
      float s = a.conv_b ? a.conv_b[e + c] : 0.0f;
      s = fmaf(wk.x, prev[2][c], s);
      s = fmaf(wk.y, prev[1][c], s);
      s = fmaf(wk.z, prev[0][c], s);
      s = fmaf(wk.w, cur[c], s);
      const float u = silu(s);
      const uint16_t hi = bf16_rne16(u);
      const uint16_t lo = bf16_rne16(u - __uint_as_float(static_cast<uint32_t>(hi) << 16));
      uh[c] = __builtin_bit_cast(__bf16, hi);
      ul[c] = __builtin_bit_cast(__bf16, lo);
    }
#pragma unroll
    for (int jt = 0; jt < 3; ++jt) {
      const int j = 16 * jt + li;
      bf16x8 wv;
      if (j < a.nout) {
        wv = *reinterpret_cast<const bf16x8*>(a.w_x + static_cast<size_t>(j) * E + e);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) wv[c] = static_cast<__bf16>(0.0f);
      }
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, uh, acc[jt], 0, 0, 0);
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, ul, acc[jt], 0, 0, 0);
    }
  }
  // acc[jt] lane (li, lg): outputs j = 16 jt + 4 lg + r of token tok
  if (!tok_ok) return;
  float* part = a.part + (static_cast<size_t>(blockIdx.y) * T + tok) * kJ;
#pragma unroll
  for (int jt = 0; jt < 3; ++jt)
    *reinterpret_cast<float4*>(part + 16 * jt + 4 * lg) = make_float4(acc[jt][0], acc[jt][1], acc[jt][2], acc[jt][3]);
}

// B[t, n] = xp[t, n], C[t, n] = xp[t, N + n], dt_raw[t] = xp[t, 2N]: partials
// added in range order
__global__ __launch_bounds__(256) void xproj_reduce(XprojArgs a, int parts) {
  const int T = a.batch * a.seqlen;
  const size_t q = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q >= static_cast<size_t>(T) * a.nout) return;
  const int tok = static_cast<int>(q / a.nout), j = static_cast<int>(q % a.nout);
  float s = 0.0f;
  // loads issued eight at a time, the additions still in range order
#pragma unroll 8
  for (int p = 0; p < parts; ++p) s += a.part[(static_cast<size_t>(p) * T + tok) * kJ + j];
  const int N = a.d_state;
  if (j < N) a.B[static_cast<size_t>(tok) * N + j] = s;
  else if (j < 2 * N) a.C[static_cast<size_t>(tok) * N + j - N] = s;
  else a.dt_raw[tok] = s;
}

}  // namespace

int xproj_splits(int tokens, int dim) {
  const int tiles = (tokens + kTokTile - 1) / kTokTile;
  const int ksteps = dim / 32;
  int s = std::max(1, std::min(ksteps, (768 + tiles - 1) / tiles));  // 768 workgroups: 3 waves per SIMD
  const int per = (ksteps + s - 1) / s;
  return (ksteps + per - 1) / per;  // no empty range
}

size_t xproj_partial_bytes(int tokens, int dim) {
  return static_cast<size_t>(xproj_splits(tokens, dim)) * tokens * kJ * 4;
}

hipError_t launch_xproj(const XprojArgs& a, hipStream_t s) {
  const int T = a.batch * a.seqlen;
  if (T == 0) return hipSuccess;
  const int parts = xproj_splits(T, a.dim);
  const unsigned tiles = static_cast<unsigned>((T + kTokTile - 1) / kTokTile);
  hipLaunchKernelGGL(xproj_kernel, dim3(tiles, parts), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = static_cast<size_t>(T) * a.nout;
  hipLaunchKernelGGL(xproj_reduce, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a, parts);
  return hipGetLastError();
}

}  // namespace ssm
