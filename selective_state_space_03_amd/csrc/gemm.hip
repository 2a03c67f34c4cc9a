// Projection GEMMs of the layer: C = A W^T with W (N, K) in bf16 (a weight
// stored as (out, in)), A (M, K) in bf16 or fp32, fp32 accumulation.
//
// Page "Axon-SSM: selective state space model", section "Algorithm": in_proj
// (D -> 2E, split into x_branch and z) and out_proj (E -> D) are dense
// projections of every token, plain GEMMs with nothing to fuse, so they go to
// the ROCm GEMM library (hipBLASLt) on the matrix cores.  What is done here:
//   * the layout: row-major C = A W^T is the column-major product
//     C^T = W A^T, i.e. hipBLASLt's D = op(W) op(A) with op(W) = T on W seen
//     column-major (K x N) and A seen column-major (K x M);
//   * in_proj's output columns >= n_split go to a second buffer (z): one call
//     per half, on the matching rows of W;
//   * an fp32 A (the scan output feeding out_proj) is split into a bf16 value
//     and the bf16 of its remainder (about 16 mantissa bits, so the product
//     keeps fp32-level accuracy), and the two halves are multiplied in turn,
//     the second accumulating onto the first (beta = 1) in fp32;
//   * plans (descriptors, layouts and the library's first heuristic choice
//     among algorithms that need no workspace) are made once per shape and
//     device and kept.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace ssm {
namespace {

// fp32 A -> bf16 value and bf16 remainder, 4 elements a thread
__global__ __launch_bounds__(256) void split_hi_lo(const float* __restrict__ A, int lda, int M, int K,
                                                   uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const size_t q = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const int kq = K / 4;
  if (q >= static_cast<size_t>(M) * kq) return;
  const int m = static_cast<int>(q / kq), k = 4 * static_cast<int>(q % kq);
  const float4 v = *reinterpret_cast<const float4*>(A + static_cast<size_t>(m) * lda + k);
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f[j]));
    l[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f[j] - __uint_as_float(h[j] << 16)));
  }
  const size_t o = static_cast<size_t>(m) * K + k;
  *reinterpret_cast<uint2*>(hi + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  *reinterpret_cast<uint2*>(lo + o) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// fp32 (M, N) contiguous -> bf16 rows of pitch ldc, 4 elements a thread
__global__ __launch_bounds__(256) void to_bf16(const float* __restrict__ T, int M, int N, uint16_t* __restrict__ C,
                                               int ldc) {
  const size_t q = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const int nq = N / 4;
  if (q >= static_cast<size_t>(M) * nq) return;
  const int m = static_cast<int>(q / nq), n = 4 * static_cast<int>(q % nq);
  const float4 v = *reinterpret_cast<const float4*>(T + static_cast<size_t>(m) * N + n);
  const uint32_t b0 = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.x));
  const uint32_t b1 = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.y));
  const uint32_t b2 = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.z));
  const uint32_t b3 = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v.w));
  *reinterpret_cast<uint2*>(C + static_cast<size_t>(m) * ldc + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
}

unsigned blocks_for(size_t n) { return static_cast<unsigned>((n + 255) / 256); }

// ---- hipBLASLt plans ------------------------------------------------------
struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t lw = nullptr, la = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};

// (device, M, N, K, lda, ldw, ldc, output type, accumulate)
using PlanKey = std::tuple<int, int, int, int, int, int, int, int, int>;

std::mutex g_lt_mutex;
hipblasLtHandle_t g_lt_handle[64] = {};
std::map<PlanKey, Plan> g_plans;

hipError_t lt_status(hipblasStatus_t s) { return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorUnknown; }

// The plan for D (M x N row-major, pitch ldc, type out) = A (M x K bf16, pitch
// lda) * W (N x K bf16, pitch ldw)^T (+ D when acc).
hipError_t get_plan(int M, int N, int K, int lda, int ldw, int ldc, int out_dtype, bool acc, const Plan** plan,
                    hipblasLtHandle_t* handle) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_lt_mutex);
  if (g_lt_handle[dev] == nullptr) {
    e = lt_status(hipblasLtCreate(&g_lt_handle[dev]));
    if (e != hipSuccess) return e;
  }
  *handle = g_lt_handle[dev];
  const PlanKey key{dev, M, N, K, lda, ldw, ldc, out_dtype, acc ? 1 : 0};
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *plan = &it->second;
    return hipSuccess;
  }
  Plan p;
  const hipDataType dt = out_dtype == kBF16 ? HIP_R_16BF : HIP_R_32F;
  auto fail = [&](hipError_t err) {
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
    if (p.lw) hipblasLtMatrixLayoutDestroy(p.lw);
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
    return err;
  };
  if ((e = lt_status(hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F))) != hipSuccess) return fail(e);
  const hipblasOperation_t tw = HIPBLAS_OP_T, ta = HIPBLAS_OP_N;
  if ((e = lt_status(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &tw, sizeof(tw)))) !=
      hipSuccess)
    return fail(e);
  if ((e = lt_status(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &ta, sizeof(ta)))) !=
      hipSuccess)
    return fail(e);
  if ((e = lt_status(hipblasLtMatrixLayoutCreate(&p.lw, HIP_R_16BF, K, N, ldw))) != hipSuccess) return fail(e);
  if ((e = lt_status(hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, M, lda))) != hipSuccess) return fail(e);
  if ((e = lt_status(hipblasLtMatrixLayoutCreate(&p.lc, dt, N, M, ldc))) != hipSuccess) return fail(e);
  hipblasLtMatmulPreference_t pref = nullptr;
  if ((e = lt_status(hipblasLtMatmulPreferenceCreate(&pref))) != hipSuccess) return fail(e);
  const uint64_t no_ws = 0;
  e = lt_status(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                                      sizeof(no_ws)));
  hipblasLtMatmulHeuristicResult_t res{};
  int found = 0;
  if (e == hipSuccess)
    e = lt_status(hipblasLtMatmulAlgoGetHeuristic(*handle, p.desc, p.lw, p.la, p.lc, p.lc, pref, 1, &res, &found));
  hipblasLtMatmulPreferenceDestroy(pref);
  if (e != hipSuccess) return fail(e);
  if (found < 1) return fail(hipErrorNotSupported);
  p.algo = res.algo;
  auto ins = g_plans.emplace(key, p);
  *plan = &ins.first->second;
  return hipSuccess;
}

hipError_t matmul(const uint16_t* A, int lda, const uint16_t* W, int ldw, void* D, int ldc, int M, int N, int K,
                  int out_dtype, bool acc, hipStream_t s) {
  const Plan* p = nullptr;
  hipblasLtHandle_t h = nullptr;
  hipError_t e = get_plan(M, N, K, lda, ldw, ldc, out_dtype, acc, &p, &h);
  if (e != hipSuccess) return e;
  const float alpha = 1.0f, beta = acc ? 1.0f : 0.0f;
  return lt_status(hipblasLtMatmul(h, p->desc, &alpha, W, p->lw, A, p->la, &beta, D, p->lc, D, p->lc, &p->algo,
                                   nullptr, 0, s));
}

size_t split_bytes(int M, int K) { return (static_cast<size_t>(M) * K * 2 + 255) & ~static_cast<size_t>(255); }

}  // namespace

// fp32 A: its bf16 value and remainder (M x K each), and an fp32 (M x N)
// product for a bf16 output.
size_t gemm_workspace_bytes(int M, int N, int K, int a_dtype) {
  if (a_dtype != kF32) return 0;
  return 2 * split_bytes(M, K) + static_cast<size_t>(M) * N * 4;
}

hipError_t launch_gemm(const GemmArgs& g, int a_dtype, int out_dtype, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  hipError_t r = hipSuccess;  // the library calls' status (timed_launch reports launch errors)
  if (a_dtype == kBF16) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const int n0 = g.C1 ? g.n_split : g.N;
    const hipError_t e = timed_launch(stream, [&] {
      r = matmul(A, g.lda, g.W, g.ldw, g.C0, g.ldc0, g.M, n0, g.K, out_dtype, false, stream);
      if (r == hipSuccess && g.C1)
        r = matmul(A, g.lda, g.W + static_cast<size_t>(n0) * g.ldw, g.ldw, g.C1, g.ldc1, g.M, g.N - n0, g.K,
                   out_dtype, false, stream);
    });
    return r != hipSuccess ? r : e;
  }
  // fp32 A: split, then value and remainder products accumulated in fp32
  if (g.C1 || g.K % 4 != 0 || g.lda % 4 != 0 || g.N % 4 != 0) return hipErrorInvalidValue;
  if (g.ws == nullptr || g.ws_bytes < gemm_workspace_bytes(g.M, g.N, g.K, kF32)) return hipErrorInvalidValue;
  char* ws = reinterpret_cast<char*>(g.ws);
  uint16_t* hi = reinterpret_cast<uint16_t*>(ws);
  uint16_t* lo = reinterpret_cast<uint16_t*>(ws + split_bytes(g.M, g.K));
  float* tmp = reinterpret_cast<float*>(ws + 2 * split_bytes(g.M, g.K));
  hipLaunchKernelGGL(split_hi_lo, dim3(blocks_for(static_cast<size_t>(g.M) * (g.K / 4))), dim3(256), 0, stream,
                     static_cast<const float*>(g.A), g.lda, g.M, g.K, hi, lo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool direct = out_dtype == kF32;
  void* D = direct ? g.C0 : tmp;
  const int ldd = direct ? g.ldc0 : g.N;
  e = timed_launch(stream, [&] {
    r = matmul(hi, g.K, g.W, g.ldw, D, ldd, g.M, g.N, g.K, kF32, false, stream);
    if (r == hipSuccess) r = matmul(lo, g.K, g.W, g.ldw, D, ldd, g.M, g.N, g.K, kF32, true, stream);
  });
  if (r != hipSuccess) return r;
  if (e != hipSuccess || direct) return e;
  hipLaunchKernelGGL(to_bf16, dim3(blocks_for(static_cast<size_t>(g.M) * (g.N / 4))), dim3(256), 0, stream, tmp, g.M,
                     g.N, static_cast<uint16_t*>(g.C0), g.ldc0);
  return hipGetLastError();
}

}  // namespace ssm
