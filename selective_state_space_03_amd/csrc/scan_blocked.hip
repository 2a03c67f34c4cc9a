// Blocked selective scan for gfx950: the diagonal recurrence
// h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t with readout
// y_t = (C_t . h_t + D u_t) SiLU(z_t) and dt = clip(softplus(dt_raw + dt_bias),
// dt_min, dt_max), over the whole sequence in one pass of 16-step blocks.
//
// Page "Axon-SSM: selective state space model": sections "Algorithm" (the
// recurrence, readout and gate) and "JIT-compiled kernels" (_compute_dt).
// Page "What is the Mamba model?", section "chunkscan": inside a block the
// outputs are the readout of the state entering the block plus a causal
// product of the block's own inputs, and the state leaving the block is the
// entering one decayed plus the block's inputs weighted by their decay to the
// block's end.
//
// Scaled form.  When A[e, :] = A[0, :] in every channel and dt sits at its
// upper clip, the step decay q_n = exp(dt_max A[0, n]) is the same in every
// channel.  Inside a block starting at t0, with g_n(t) = h_n(t) q_n^-(t-t0+1),
//   g(t) = h(t0 - 1) + sum_{s <= t} dt_max u_s B'_s,    B'_s = B_s q^-(s-t0+1)
//   y(t) = C'_t . g(t) + D u_t,                         C'_t = C_t q^(t-t0+1)
//   h(t0 + 15) = q^16 g(t0 + 15)
// so for a 16 x 16 tile (steps x channels) of a block at the clip
//   Y  = C' H0 + M U,          M[t][s] = dt_max sum_n C_t[n] B_s[n] q_n^(t-s), s <= t
//   H1 = q^16 (H0 + B''^T U),  B''_s = dt_max B'_s
// matrix products with K = 16 states or 16 steps (v_mfma_f32_16x16x32_bf16).
// C', M and B'' depend on the batch row and the block only: a packing kernel
// writes them once per call, from double-precision exponentials, as bf16
// hi + lo pairs (lo = bf16 of the remainder) in the matrix cores' operand
// order, next to fp32 rows of B' and C'.  U is the bf16 input itself, so the
// products C'hi H0hi + C'lo H0hi + C'hi H0lo and Mhi U + Mlo U keep about 16
// mantissa bits.
//
// Steps off the clip.  Most tiles that hold any have one or two such steps
// (the bulk recipe: 13 % of tiles, four in five with a single step).  The
// block's products are then taken as if every step were at the clip, and
// each step s off the clip, in order, adds to every later scaled state of
// its channel the difference d = (f - 1) g(s-1) + (dt - dt_max) u B'_s with
// f = exp((dt - dt_max) A): one more update product for g(s-1) and one more
// readout product C' d.  A tile with more than four such steps (or A differing across
// channels, or factors out of range, or a partial last block) runs step by
// step on the same registers: lane (r, e) holds states 4r..4r+3 of channel e,
// and the four lanes' partial readouts of a channel are summed by a
// transposing reduction of permlane swaps that lands y in the same lane
// layout as the matrix-core path.
//
// Mapping: a workgroup of 4 waves takes 64 consecutive channels of one batch
// row, wave w the channels 16w..16w+15.  Per block the workgroup stages u,
// dt and z (16 rows of 128 bytes each) and the block's table record in LDS
// with 8- and 16-byte loads issued three blocks ahead, and writes y back
// through LDS as whole 128-byte rows.  The workgroups one CU holds at once
// take adjacent channel groups, so together they read whole 512-byte pieces
// of each row (measured: 128-byte pieces from scattered CUs stream at 3.7
// TB/s, adjacent ones at 4.3, one 16-channel wave per workgroup at 2 TB/s).
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kT = kBlkT;       // steps per block
constexpr int kN = kScanN;      // states
constexpr int kThreads = 256;   // 4 waves x 16 channels
constexpr int kCh = 64;         // channels per workgroup
constexpr int kFbRow = kCh / 4 + 1;  // padded row of the per-wave step table (float2)
constexpr int kMaxOff = 4;      // steps off the clip a tile's block corrects after its products
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: loads 0, stores dropped
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family

// record of one (batch row, block), bytes
constexpr int kRecTC = 0;     // [lane][8 bf16]: C' hi | lo, operand A of the readout
constexpr int kRecTM = 1024;  // M hi | lo, operand A of the in-block product
constexpr int kRecTB = 2048;  // B'' hi | lo, operand A of the state update
constexpr int kRecRB = 3072;  // B' fp32 [step][state]
constexpr int kRecRC = 4096;  // C' fp32 [step][state]
static_assert(kRecRC + kT * kN * 4 == kBlkRec, "record layout");
// per-call values, floats
constexpr int kQvLog = 0;                         // log2 q_n (0: scaled form off)
constexpr int kQvPow = kN;                        // q_n^k as [k][n], k = 0..16
constexpr int kQvFlag = kQvPow + (kT + 1) * kN;   // 1: scaled form on
static_assert(kQvFlag + 1 == kBlkQv, "per-call values");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

// Raw buffer descriptor over [p, p + bytes).  The words pass through
// readfirstlane so the compiler knows they are uniform.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           kRsrcWord3);
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

// v = hi + lo to about 16 bits: hi = bf16(v), lo = bf16 of the remainder
// (taken in double)
__device__ __forceinline__ void split_d(double v, uint16_t& hi, uint16_t& lo) {
  hi = bf16_bits(static_cast<float>(v));
  lo = bf16_bits(static_cast<float>(v - static_cast<double>(bf16_val(hi))));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// (bf16(a), bf16(b)) in one word, a in the low half; and the pair of
// remainders
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing sum over the four 16-lane rows: x_j holds, in row r', a partial
// sum of item j; the result holds in row r the total of item r.
//   permlane32_swap(a, b): a <- [a.r0 a.r1 b.r0 b.r1], b <- [a.r2 a.r3 b.r2 b.r3]
//   permlane16_swap(a, b): a <- [a.r0 b.r0 a.r2 b.r2], b <- [a.r1 b.r1 a.r3 b.r3]
__device__ __forceinline__ float pair_sum(float a, float b, bool half) {
  const int ia = __builtin_bit_cast(int, a), ib = __builtin_bit_cast(int, b);
  if (half) {
    const auto p = __builtin_amdgcn_permlane32_swap(ia, ib, false, false);
    return __builtin_bit_cast(float, static_cast<int>(p[0])) + __builtin_bit_cast(float, static_cast<int>(p[1]));
  }
  const auto p = __builtin_amdgcn_permlane16_swap(ia, ib, false, false);
  return __builtin_bit_cast(float, static_cast<int>(p[0])) + __builtin_bit_cast(float, static_cast<int>(p[1]));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
// v OR-ed with the same lane of the other three 16-lane rows
__device__ __forceinline__ uint32_t or_rows(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane16_swap(static_cast<int>(v), static_cast<int>(v), false, false);
  v = static_cast<uint32_t>(p[0]) | static_cast<uint32_t>(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(static_cast<int>(v), static_cast<int>(v), false, false);
  return static_cast<uint32_t>(q[0]) | static_cast<uint32_t>(q[1]);
}

__device__ __forceinline__ float row_transpose_sum(float x0, float x1, float x2, float x3) {
  const float s02 = pair_sum(x0, x2, true);   // [x0(r0+r2) x0(r1+r3) x2(r0+r2) x2(r1+r3)]
  const float s13 = pair_sum(x1, x3, true);   // the same for x1, x3
  return pair_sum(s02, s13, false);           // [sum x0, sum x1, sum x2, sum x3]
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}
// rows 1 and 3 receive rows 0 and 2 (rows 0 and 2 keep their own)
__device__ __forceinline__ float from_row_below(float x) {
  const int i = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, static_cast<int>(__builtin_amdgcn_permlane16_swap(i, i, false, false)[0]));
}
// row 1 in every row
__device__ __forceinline__ float row1_everywhere(float x) {
  const int i = __builtin_bit_cast(int, x);
  const int y = static_cast<int>(__builtin_amdgcn_permlane32_swap(i, i, false, false)[0]);
  return __builtin_bit_cast(float, static_cast<int>(__builtin_amdgcn_permlane16_swap(y, y, false, false)[1]));
}
// x of lane i of this lane's quad
__device__ __forceinline__ float quad_lane(float x, int i) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (i) {
    case 0: r = __builtin_amdgcn_update_dpp(0, v, 0x00, 0xF, 0xF, false); break;  // quad_perm [0, 0, 0, 0]
    case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false); break;  // quad_perm [1, 1, 1, 1]
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false); break;  // quad_perm [2, 2, 2, 2]
    default: r = __builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false); break;  // quad_perm [3, 3, 3, 3]
  }
  return __builtin_bit_cast(float, r);
}
// row q (1 .. 3) receives row q - 1: rows 1 and 3 from the pair swap, row 2
// from the half swap of the pair swap's odd rows (each swap of a register
// with itself)
__device__ __forceinline__ float from_row_above(float x, int q) {
  const int i = __builtin_bit_cast(int, x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(i, i, false, false);  // [x0 x0 x2 x2], [x1 x1 x3 x3]
  const int o = static_cast<int>(p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(o, o, false, false);  // [x1 x1 x1 x1], ...
  // both swaps run with every lane active: a swap sunk into the branch of a
  // row's choice would not see the rows it reads from
  int r1 = static_cast<int>(p16[0]), r2 = static_cast<int>(p32[0]);
  asm volatile("" : "+v"(r1), "+v"(r2));
  return __builtin_bit_cast(float, q == 2 ? r2 : r1);
}
// x of lane src (any lane of the wave)
__device__ __forceinline__ float lane_val(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// The 4-element units of a step row (8 bytes in bf16, 16 in fp32) are
// XOR-permuted by the row's group of four, so the four rows a wave reads in
// one instruction (steps 4r + i, r = 0..3) fall on different banks.
__device__ __forceinline__ int swz(int s) { return ((s >> 2) & 3) << 2; }

// ---- per-call tables -------------------------------------------------------
// One workgroup per (batch row, block); thread (s, n) = (tid / 16, tid % 16).
// The scaled form is on when dt_max is finite and 16 dt_max max|A[0, n]| <= 32
// (factors within e^+-32); otherwise q := 1, the rows are B and C themselves
// and the matrix-core tables are zero (unused).
template <typename BT>
__global__ __launch_bounds__(256) void pack_blk_kernel(const BT* __restrict__ B, const BT* __restrict__ C,
                                                       const float* __restrict__ A, float dt_max, int seqlen,
                                                       int nrec, unsigned char* __restrict__ rec,
                                                       float* __restrict__ qv) {
  __shared__ double qp[kT + 1][kN];  // q_n^k
  __shared__ double qm[kT + 1][kN];  // q_n^-k
  __shared__ float sB[kT][kN], sC[kT][kN];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / nrec, blk = blockIdx.x % nrec;
  const int t0 = blk * kT;
  const int T = min(kT, seqlen - t0);
  const int s = tid >> 4, n = tid & 15;
  // this thread's B and C entries are requested first, so their loads are in
  // flight while A and the decay tables are formed
  // (a step past the end reads the block's first row and is zeroed below:
  // no branch, so nothing waits for these loads before the tables)
  const bool in = s < T;
  const size_t o = (static_cast<size_t>(b) * seqlen + t0 + (in ? s : 0)) * kN + n;
  const BT braw = B[o], craw = C[o];
  const double dm = dt_max;
  double amax = 0.0;
  for (int n = 0; n < kN; ++n) amax = fmax(amax, fabs(static_cast<double>(A[n])));
  const bool ok = __builtin_isfinite(dm) && 16.0 * dm * amax <= 32.0;
  for (int i = tid; i < (kT + 1) * kN; i += 256) {
    const int k = i / kN, n = i % kN;
    const double x = ok ? k * dm * static_cast<double>(A[n]) : 0.0;
    qp[k][n] = exp(x);
    qm[k][n] = exp(-x);
  }
  sB[s][n] = in ? to_f32(braw) : 0.0f;
  sC[s][n] = in ? to_f32(craw) : 0.0f;
  __syncthreads();
  unsigned char* R = rec + (static_cast<size_t>(b) * nrec + blk) * kBlkRec;
  const double bs = static_cast<double>(sB[s][n]) * qm[s + 1][n];  // B'_s[n]
  const double cs = static_cast<double>(sC[s][n]) * qp[s + 1][n];  // C'_s[n]
  reinterpret_cast<float*>(R + kRecRB)[s * kN + n] = static_cast<float>(bs);
  reinterpret_cast<float*>(R + kRecRC)[s * kN + n] = static_cast<float>(cs);
  uint16_t hi, lo;
  // C'[t = s][n]: lane 16 (n / 4) + t, k slots n % 4 (hi) and 4 + n % 4 (lo)
  split_d(cs, hi, lo);
  uint16_t* tc = reinterpret_cast<uint16_t*>(R + kRecTC) + (16 * (n >> 2) + s) * 8 + (n & 3);
  tc[0] = hi;
  tc[4] = lo;
  // B''[s][n]: lane 16 (s / 4) + n, k slots s % 4 and 4 + s % 4
  split_d(ok ? dm * bs : 0.0, hi, lo);
  uint16_t* tb = reinterpret_cast<uint16_t*>(R + kRecTB) + (16 * (s >> 2) + n) * 8 + (s & 3);
  tb[0] = hi;
  tb[4] = lo;
  // M[t][s'] with (t, s') = (tid / 16, tid % 16): lane 16 (s' / 4) + t
  {
    const int t = s, sp = n;
    double m = 0.0;
    if (ok && sp <= t && t < T) {
      for (int k = 0; k < kN; ++k)
        m = fma(static_cast<double>(sC[t][k]) * static_cast<double>(sB[sp][k]), qp[t - sp][k], m);
      m *= dm;
    }
    split_d(m, hi, lo);
    uint16_t* tm = reinterpret_cast<uint16_t*>(R + kRecTM) + (16 * (sp >> 2) + t) * 8 + (sp & 3);
    tm[0] = hi;
    tm[4] = lo;
  }
  if (blockIdx.x == 0) {
    if (tid < kN) qv[kQvLog + tid] = ok ? static_cast<float>(dm * static_cast<double>(A[tid]) * 1.4426950408889634) : 0.0f;
    for (int i = tid; i < (kT + 1) * kN; i += 256) qv[kQvPow + i] = static_cast<float>(qp[i / kN][i % kN]);
    if (tid == 0) qv[kQvFlag] = ok ? 1.0f : 0.0f;
  }
}

// Position in the (batch row, channel group) order of workgroup i of n.
// Workgroups go to the XCDs round-robin (i mod 8) and within an XCD to its 32
// CUs round-robin ((i / 8) mod 32), one of a few rounds.  XCD x takes a
// contiguous range of positions (with 8 batch rows: one row, so its L2 holds
// that row's table records), and each of its CUs a run of consecutive
// positions within it, so the workgroups a CU holds at once read adjacent
// 128-byte pieces of the same rows.
//
// Within a run the positions are handed out worst first: ranked by the
// smallest dt_bias among their 64 channels (ties by position), the lowest goes
// to round 0.  A channel whose bias sits low has dt below its upper clip on
// many steps, so its wave takes the per-step corrections on most blocks and
// its workgroup runs longest; the oldest waves of a SIMD win its issue
// arbitration, so a slow workgroup started first ends sooner.  The ranks are
// a permutation of the run's rounds (a strict order), so the mapping stays a
// bijection onto the positions.  skey: 4 floats of LDS; every thread of the
// workgroup calls this (it holds a barrier).
__device__ __forceinline__ unsigned blk_position(unsigned i, unsigned n, unsigned ngroups, const float* bias,
                                                 float* skey) {
  constexpr unsigned kXcd = 8, kCus = kScanCuSlots / kXcd;
  const unsigned x = i % kXcd, k = i / kXcd;
  const unsigned cnt = n / kXcd + (x < n % kXcd ? 1u : 0u);
  const unsigned start = x * (n / kXcd) + min(x, n % kXcd);
  const unsigned c = k % kCus, round = k / kCus;
  const unsigned full = cnt / kCus, rem = cnt % kCus;
  const unsigned run0 = start + c * full + min(c, rem);
  const unsigned len = full + (c < rem ? 1u : 0u);  // rounds of this CU slot: round < len
  if (bias == nullptr || len < 2 || len > 4) return run0 + round;
  // wave j: the smallest bias of the run's position j (NaN counts as +inf)
  const unsigned tid = threadIdx.x, wv = tid >> 6;
  float v = INFINITY;
  if (wv < len) v = bias[((run0 + wv) % ngroups) * kCh + (tid & 63)];
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  if ((tid & 63) == 0) skey[wv] = v != v ? INFINITY : v;
  __syncthreads();
  unsigned sel = 0;
  for (unsigned j = 0; j < len; ++j) {
    unsigned rank = 0;
    for (unsigned m = 0; m < len; ++m) rank += (skey[m] < skey[j] || (skey[m] == skey[j] && m < j)) ? 1u : 0u;
    if (rank == round) sel = j;
  }
  return run0 + sel;
}

template <typename YT>
struct alignas(16) BlkSmem {
  uint16_t in[2][3][kT][kCh];       // u, dt, z of a block (bf16), units permuted by swz
  unsigned char rec[2][kBlkRec];    // the block's record
  YT yt[2][kT][kCh];                // y of a block, units permuted by swz
  float2 fb[4][kT][kFbRow];         // per wave: (dt u, dt) of [step][channel]
};

template <typename YT>
struct YUnit;
template <>
struct YUnit<bf16s> {
  typedef uint2 type;
  __device__ static void store(rsrc_t r, uint32_t vo, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, vo, 0, 0);
  }
  __device__ static void put(bf16s* p, float v) { p->bits = bf16_bits(v); }
};
template <>
struct YUnit<float> {
  typedef uint4 type;
  __device__ static void store(rsrc_t r, uint32_t vo, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, vo, 0, 0);
  }
  __device__ static void put(float* p, float v) { *p = v; }
};

// Loads of one block held in registers until they are written to LDS.
struct Stage {
  uint2 u, d, z;
  uint4 r16;
  uint32_t r4;
};

__device__ __forceinline__ uint2 ld64(rsrc_t r, uint32_t vo) {
  const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, vo, 0, 0));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld128(rsrc_t r, uint32_t vo) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename YT, bool GATE>
__global__ __launch_bounds__(kThreads, 4) void scan_blk_kernel(ScanBlkArgs a) {
  __shared__ BlkSmem<YT> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l >> 4, e = l & 15;
  const unsigned ngroups = static_cast<unsigned>(a.dim) / kCh;
  __shared__ float skey[4];
  const unsigned pos = blk_position(blockIdx.x, gridDim.x, ngroups, a.dt_bias, skey);
  const int b = static_cast<int>(pos / ngroups);
  const int g = static_cast<int>(pos % ngroups);
  const int c = g * kCh + 16 * w + e;  // this lane's channel; its states are 4r..4r+3
  const uint32_t L = a.seqlen, E = a.dim;
  const size_t tok0 = static_cast<size_t>(b) * L;
  const int nb = a.nrec;
  const rsrc_t rx = make_rsrc(a.x + tok0 * E, L * E * 2u);
  const rsrc_t rd = make_rsrc(a.dt + tok0 * E, L * E * 2u);
  const rsrc_t rz = make_rsrc((GATE ? a.z : a.x) + tok0 * E, L * E * 2u);
  const rsrc_t ry = make_rsrc(static_cast<char*>(a.y) + tok0 * E * sizeof(YT), L * E * static_cast<uint32_t>(sizeof(YT)));
  const rsrc_t rr = make_rsrc(a.rec + static_cast<size_t>(b) * nb * kBlkRec, static_cast<uint32_t>(nb) * kBlkRec);

  // staging: this lane moves 4 consecutive channels (unit e) of step row 4w + r
  // (the unit's element offset in a step row of the batch row's u / dt / z,
  // and its position in the LDS row)
  const int srow = 4 * w + r;
  const uint32_t sel = static_cast<uint32_t>(srow) * E + static_cast<uint32_t>(g * kCh + 4 * e);
  const int su = (e ^ swz(srow)) * 4;
  const uint32_t blk_el = kT * E;  // elements of one block of a batch row's u, dt, z or y
  auto issue = [&](int j, Stage& S) {
    const bool in = j >= 0 && j < nb;
    const uint32_t vo = in ? (static_cast<uint32_t>(j) * blk_el + sel) * 2u : kOob;
    S.u = ld64(rx, vo);
    S.d = ld64(rd, vo);
    if (GATE) S.z = ld64(rz, vo);
    const uint32_t vr = in ? static_cast<uint32_t>(j) * kBlkRec : kOob;
    S.r16 = ld128(rr, vr + (in ? tid * 16u : 0u));
    S.r4 = __builtin_amdgcn_raw_buffer_load_b32(rr, vr + (in ? 4096u + tid * 4u : 0u), 0, 0);
  };
  auto commit = [&](int buf, const Stage& S) {
    *reinterpret_cast<uint2*>(&sm.in[buf][0][srow][su]) = S.u;
    *reinterpret_cast<uint2*>(&sm.in[buf][1][srow][su]) = S.d;
    if (GATE) *reinterpret_cast<uint2*>(&sm.in[buf][2][srow][su]) = S.z;
    *reinterpret_cast<uint4*>(&sm.rec[buf][tid * 16]) = S.r16;
    *reinterpret_cast<uint32_t*>(&sm.rec[buf][4096 + tid * 4]) = S.r4;
  };
  // y of block j leaves in two parts: its LDS read goes out first after a
  // barrier (ahead of the staging writes, so its latency overlaps them), the
  // store once the staging is written
  auto read_y = [&](int j) { return *reinterpret_cast<const typename YUnit<YT>::type*>(&sm.yt[j & 1][srow][su]); };
  auto put_y = [&](int j, const typename YUnit<YT>::type& v) {
    const bool in = j >= 0;
    const uint32_t vo = in ? (static_cast<uint32_t>(j) * blk_el + sel) * static_cast<uint32_t>(sizeof(YT)) : kOob;
    YUnit<YT>::store(ry, vo, v);
  };

  // per-lane constants
  // (vector types, so that no per-lane array is left in scratch memory)
  const float* Ac = a.A + static_cast<size_t>(c) * kN + 4 * r;
  f32x4 al, cq, q16, G;
  bool same = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float av = Ac[i];
    same = same && av == a.A[4 * r + i];
    al[i] = av * kLog2e;
    cq[i] = a.qv[kQvLog + 4 * r + i];
    q16[i] = a.qv[kQvPow + kT * kN + 4 * r + i];
  }
  const bool scaled = a.qv[kQvFlag] != 0.0f;
  // per state n: log2 decay per unit dt and log2 q, of A's row 0 (the row
  // every channel has where they are used), for the one-channel path
  __shared__ float s_al[kN], s_cq[kN];
  if (tid < kN) {
    s_al[tid] = a.A[tid] * kLog2e;
    s_cq[tid] = a.qv[kQvLog + tid];
  }
  // steps at the clip need no factor and full blocks at the clip take the
  // matrix cores when the scaled form holds for every channel of the wave
  const bool clip_free = scaled && __all(same);
  const float dcoef = a.D ? a.D[c] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[c] : 0.0f;
  const float sat_pre = a.dt_softplus ? a.sp_hi : a.dt_max;
  const float dt_max = a.dt_max;
  const size_t so = (static_cast<size_t>(b) * E + c) * kN + 4 * r;
#pragma unroll
  for (int i = 0; i < 4; ++i) G[i] = a.state_in ? a.state_in[so + i] : 0.0f;

  // inputs at lane (r, e): steps 4r + i of channel c; unit 4w + e / 4 of the row
  const int cu = 4 * w + (e >> 2), ce = e & 3;
  auto compute = [&](int j, int buf) {
    const int T = min(kT, static_cast<int>(L) - kT * j);
    // (vector types: an element picked by a uniform index stays in registers)
    // (u of steps 4r, 4r + 1 and 4r + 2, 4r + 3 as two packed pairs, read
    // straight into the halves of a word)
    u32x2 up;
    f32x4 uf, pre, zf;
    bool sat[4];
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const int idx = ((cu ^ swz(4 * r + i)) << 2) + ce;
      u16x2 p;
      p.x = sm.in[buf][0][4 * r + i][idx];
      p.y = sm.in[buf][0][4 * r + i + 1][idx];
      up[i >> 1] = __builtin_bit_cast(uint32_t, p);
      uf[i] = __uint_as_float(up[i >> 1] << 16);
      uf[i + 1] = __uint_as_float(up[i >> 1] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * r + i;
      const int idx = ((cu ^ swz(s)) << 2) + ce;
      pre[i] = bf16_val(sm.in[buf][1][s][idx]) + bias;
      zf[i] = GATE ? bf16_val(sm.in[buf][2][s][idx]) : 0.0f;
      sat[i] = pre[i] >= sat_pre;
    }
    // the steps of the wave's tile with some channel off the clip (bit t):
    // each lane's bits at 4r + i, OR-ed over its row (DPP rotations) and over
    // the rows (permlane swaps)
    uint32_t off;
    {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) v |= sat[i] ? 0u : (1u << i);
      v <<= 4 * r;
      v |= dpp_u32<0x121>(v);  // row_ror:1
      v |= dpp_u32<0x122>(v);  // row_ror:2
      v |= dpp_u32<0x124>(v);  // row_ror:4
      v |= dpp_u32<0x128>(v);  // row_ror:8
      v = or_rows(v);
      off = __builtin_amdgcn_readfirstlane(v);
    }
    // the channels of the tile with a step off the clip (bit e)
    uint32_t chm;
    {
      const uint64_t m = __ballot(!(sat[0] && sat[1] && sat[2] && sat[3]));
      chm = static_cast<uint32_t>(m | (m >> 16) | (m >> 32) | (m >> 48)) & 0xffffu;
    }
    const bool whole = clip_free && T == kT;
    // y of the block's steps, and the state leaving it before the rescale
    // (one multiply after the three paths join, into the loop's register)
    f32x4 yv, Hn;
    // The block's matrix products: the readout C' H + M U and the update
    // H + B''^T U (not rescaled), U = the tile's u kept on steps lo..hi.
    const uint4 tc = *reinterpret_cast<const uint4*>(&sm.rec[buf][kRecTC + l * 16]);
    auto u_kept = [&](int lo, int hi) {
      uint32_t km[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) km[i] = (4 * r + i >= lo && 4 * r + i <= hi) ? 0xffffu << (16 * (i & 1)) : 0u;
      const uint32_t uw0 = up[0] & (km[0] | km[1]), uw1 = up[1] & (km[2] | km[3]);
      return as_bf16x8(make_uint4(uw0, uw1, uw0, uw1));
    };
    // C' H for a state H (its bf16 hi + lo): C'hi Hhi + C'lo Hhi, then C'hi Hlo
    // (the second half of k is zero)
    auto readout = [&](const f32x4& H) {
      uint32_t h01, l01, h23, l23;
      split2(H[0], H[1], h01, l01);
      split2(H[2], H[3], h23, l23);
      f32x4 Y = {0.0f, 0.0f, 0.0f, 0.0f};
      Y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tc), as_bf16x8(make_uint4(h01, h23, h01, h23)), Y, 0, 0, 0);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(tc.x, tc.y, tc.x, tc.y)),
                                                     as_bf16x8(make_uint4(l01, l23, 0u, 0u)), Y, 0, 0, 0);
    };
    auto update = [&](const f32x4& H, const bf16x8& uu) {
      const uint4 tb = *reinterpret_cast<const uint4*>(&sm.rec[buf][kRecTB + l * 16]);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tb), uu, H, 0, 0, 0);
    };
    auto products = [&](const f32x4& H0, f32x4& Y, f32x4& H1) {
      const uint4 tm = *reinterpret_cast<const uint4*>(&sm.rec[buf][kRecTM + l * 16]);
      const bf16x8 uu = u_kept(0, kT - 1);
      Y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tm), uu, readout(H0), 0, 0, 0);
      H1 = update(H0, uu);
    };
    // (dt u, dt) of the wave's tile into its LDS table, for steps taken one at a time
    float2* fbw = &sm.fb[w][0][0];
    const float* RB = reinterpret_cast<const float*>(&sm.rec[buf][kRecRB]);
    const float* RC = reinterpret_cast<const float*>(&sm.rec[buf][kRecRC]);
    auto fill_table = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dt = a.dt_softplus ? dt_softplus_clip(pre[i], a.dt_min, dt_max, a.sp_lo, a.sp_hi)
                                       : dt_clip(pre[i], a.dt_min, dt_max);
        fbw[(4 * r + i) * kFbRow + e] = make_float2(dt * uf[i], dt);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    };
    // (dt u, dt) of the next step, read from LDS one step ahead: its use
    // opens a step, so a read issued with the step's own B' and C' rows would
    // stall every step for a whole LDS round trip (the rows are used later
    // in the step; reading them ahead as well leaves too few registers)
    float2 vn;
    // one step on the scaled state: the factor exp((dt - dt_max) A) where dt
    // is off the clip (exp(dt A) without the scaled form), then dt u B'; the
    // lane's part of the readout C' . g
    auto step = [&](int s) {
      const float2 v = vn;
      const float4 b4 = *reinterpret_cast<const float4*>(&RB[s * kN + 4 * r]);
      const float4 c4 = *reinterpret_cast<const float4*>(&RC[s * kN + 4 * r]);
      if (s + 1 < kT) vn = fbw[(s + 1) * kFbRow + e];
      const bool need = !(clip_free && v.y == dt_max);
      if (__any(need)) {
        // the factors for every lane, then kept where needed (no branch)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = exp2_fast(fmaf(v.y, al[i], -cq[i]));
          G[i] *= need ? f : 1.0f;
        }
      }
      G[0] = fmaf(v.x, b4.x, G[0]);
      G[1] = fmaf(v.x, b4.y, G[1]);
      G[2] = fmaf(v.x, b4.z, G[2]);
      G[3] = fmaf(v.x, b4.w, G[3]);
      return fmaf(c4.x, G[0], fmaf(c4.y, G[1], fmaf(c4.z, G[2], c4.w * G[3])));
    };
    if (whole && off == 0) {
      // every step at the clip: the block's products
      products(G, yv, Hn);
    } else if (whole && __builtin_popcount(chm) == 1 && __builtin_popcount(off) >= 3) {
      // Every step off the clip in the tile (three or more: with fewer the
      // per-step corrections below cost less) is in one channel, ec.  The
      // tile's products (as if at the clip) serve the other fifteen; channel
      // ec's block is taken again with the lanes on its states and steps:
      // lane (q, n) runs state n over steps 4q .. 4q + 3 from zero (the
      // scaled form's step, g = f g + dt u B'_s), the four quarters' maps
      // x -> P x + Q are composed in row order across the rows, the state
      // entering each quarter follows from the one entering the block, and
      // the readout C'_t . g(t) is summed over the sixteen states of a row.
      products(G, yv, Hn);
      const int ec = __builtin_ctz(chm);
      // lane indices formed again from an opaque copy of the lane id: formed
      // from the kernel's own, their addresses would be held through the loop
      int lo = l;
      asm volatile("" : "+v"(lo));
      const int qr = lo >> 4, ne = lo & 15;
      // state ne of channel ec entering the block: component ne % 4 of lane
      // 16 (ne / 4) + ec
      const int hs = 16 * (ne >> 2) + ec;
      float g0 = lane_val(G[0], hs), g1 = lane_val(G[1], hs), g2 = lane_val(G[2], hs), g3 = lane_val(G[3], hs);
      asm volatile("" : "+v"(g0), "+v"(g1), "+v"(g2), "+v"(g3));  // (read with every lane active)
      const float h0 = (ne & 2) ? ((ne & 1) ? g3 : g2) : ((ne & 1) ? g1 : g0);
      const float bc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bias), ec));
      const int cuc = 4 * w + (ec >> 2), cec = ec & 3;
      // dt and dt u of step 4 qr + ne % 4 of channel ec, formed once per
      // lane and handed to the other lanes of its quad (each quad runs the
      // row's four steps)
      float dts, dus;
      {
        const int sq = 4 * qr + (ne & 3);
        const int idx = ((cuc ^ swz(sq)) << 2) + cec;
        const float us = bf16_val(sm.in[buf][0][sq][idx]);
        const float ps = bf16_val(sm.in[buf][1][sq][idx]) + bc;
        if (a.dt_softplus) {
          float sp = fminf(fmaxf(softplus(ps), a.dt_min), dt_max);
          asm volatile("" : "+v"(sp));  // formed for every lane: no branch around it
          dts = ps >= a.sp_hi ? dt_max : (ps <= a.sp_lo ? a.dt_min : sp);
        } else {
          dts = dt_clip(ps, a.dt_min, dt_max);
        }
        dus = dts * us;
      }
      f32x4 gq, pq;
      float gl = 0.0f, pl = 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int st = 4 * qr + i;
        const float dt = quad_lane(dts, i), du = quad_lane(dus, i);
        const float f = dt == dt_max ? 1.0f : exp2_fast(fmaf(dt, s_al[ne], -s_cq[ne]));
        gl = fmaf(f, gl, du * RB[st * kN + ne]);
        pl *= f;
        gq[i] = gl;
        pq[i] = pl;
      }
      // inclusive composition over the rows: rows 1 and 3 after rows 0 and
      // 2, then rows 2 and 3 after rows 0 .. 1
      float P = pq[3], Q = gq[3];
      {
        float Pb = from_row_below(P), Qb = from_row_below(Q);
        asm volatile("" : "+v"(Pb), "+v"(Qb));  // (formed with every lane active)
        const bool odd = (qr & 1) != 0;
        Q = odd ? fmaf(P, Qb, Q) : Q;
        P = odd ? P * Pb : P;
        float P1 = row1_everywhere(P), Q1 = row1_everywhere(Q);
        asm volatile("" : "+v"(P1), "+v"(Q1));
        const bool hi = qr >= 2;
        Q = hi ? fmaf(P, Q1, Q) : Q;
        P = hi ? P * P1 : P;
      }
      const float hout = fmaf(P, h0, Q);  // state ne after quarter qr
      float hin_up = from_row_above(hout, qr);
      asm volatile("" : "+v"(hin_up));  // (formed with every lane active)
      const float hin = qr == 0 ? h0 : hin_up;
      const bool mine = ne == ec;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float yr = row_sum16(RC[(4 * qr + i) * kN + ne] * fmaf(pq[i], hin, gq[i]));  // y of step 4qr + i
        asm volatile("" : "+v"(yr));  // (summed with every lane active)
        yv[i] = mine ? yr : yv[i];
      }
      // the state leaving the block: state 4qr + j of channel ec is in lane 48 + 4qr + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float hj = lane_val(hout, 48 + 4 * qr + j);
        asm volatile("" : "+v"(hj));  // (read with every lane active)
        Hn[j] = mine ? hj : Hn[j];
      }
    } else if (whole && __builtin_popcount(off) <= kMaxOff) {
      // The block's products as if at the clip, then for each step s off the
      // clip (in order) the difference it makes to the scaled state,
      //   d = (f - 1) g(s-1) + (dt - dt_max) u B'_s,   f = exp((dt - dt_max) A),
      // which every later state of the block carries: y_t += C'_t . d for
      // t >= s, and the state leaving the block gains d.
      // u and the pre-activation of step st of this lane's channel, read
      // again from the block's LDS copy (the four lanes of a channel read
      // one address)
      auto off_step = [&](int st, float& du, f32x4& fm1) {
        const int idx = ((cu ^ swz(st)) << 2) + ce;
        const float us = bf16_val(sm.in[buf][0][st][idx]);
        const float ps = bf16_val(sm.in[buf][1][st][idx]) + bias;
        float dt;
        if (a.dt_softplus) {
          float sp = fminf(fmaxf(softplus(ps), a.dt_min), dt_max);
          asm volatile("" : "+v"(sp));  // formed for every lane: no branch around it
          dt = ps >= a.sp_hi ? dt_max : (ps <= a.sp_lo ? a.dt_min : sp);
        } else {
          dt = dt_clip(ps, a.dt_min, dt_max);
        }
        const bool need = dt != dt_max;
        du = (dt - dt_max) * us;
#pragma unroll
        for (int i = 0; i < 4; ++i) fm1[i] = need ? exp2_fast(fmaf(dt, al[i], -cq[i])) - 1.0f : 0.0f;
      };
      // y_t += C'_t . d for t >= st: the readout with C' rows t < st zeroed
      // (lane l carries row l % 16 of the A operand), accumulated into y
      auto add_readout = [&](const f32x4& d, int st) {
        const uint4 tcm = (l & 15) >= st ? tc : make_uint4(0u, 0u, 0u, 0u);
        uint32_t h01, l01, h23, l23;
        split2(d[0], d[1], h01, l01);
        split2(d[2], d[3], h23, l23);
        yv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tcm), as_bf16x8(make_uint4(h01, h23, h01, h23)), yv, 0, 0, 0);
        yv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(tcm.x, tcm.y, tcm.x, tcm.y)),
                                                     as_bf16x8(make_uint4(l01, l23, 0u, 0u)), yv, 0, 0, 0);
      };
      auto diff = [&](int st, const f32x4& dprev, float du, const f32x4& fm1, const f32x4& Hs) {
        const float4 b4 = *reinterpret_cast<const float4*>(&RB[st * kN + 4 * r]);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = fmaf(fm1[i], Hs[i] + dprev[i], du * bv[i]);
        return d;
      };
      // the first step off the clip in straight-line code beside the products
      const int st0 = __builtin_ctz(off);
      float du0;
      f32x4 fm10, H1;
      off_step(st0, du0, fm10);
      const f32x4 Hs0 = update(G, u_kept(0, st0 - 1));  // g(st0 - 1)
      products(G, yv, H1);
      f32x4 dsum = diff(st0, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, du0, fm10, Hs0);
      add_readout(dsum, st0);
      // the others in order: g(s-1) from the products plus the earlier differences
      for (uint32_t rest = off & (off - 1); rest != 0; rest &= rest - 1) {
        const int st = __builtin_ctz(rest);
        float du;
        f32x4 fm1;
        off_step(st, du, fm1);
        const f32x4 d = diff(st, dsum, du, fm1, update(G, u_kept(0, st - 1)));
        dsum += d;
        add_readout(d, st);
      }
      Hn = H1 + dsum;
    } else {
      // step by step through the whole block
      fill_table();
      vn = fbw[e];
      float P[kT];
      auto pinned = [&](int s) {
        P[s] = step(s);
        // formed here: sunk to its use after the loop, it would keep every
        // step's C' row and state copy alive
        asm volatile("" : "+v"(P[s]));
      };
      if (T == kT) {
#pragma unroll
        for (int s = 0; s < kT; ++s) pinned(s);
      } else {
#pragma unroll
        for (int s = 0; s < kT; ++s) {
          P[s] = 0.0f;
          if (s < T) pinned(s);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) yv[i] = row_transpose_sum(P[i], P[4 + i], P[8 + i], P[12 + i]);
      Hn = G;
    }
    if (T == kT) {
      G = Hn * q16;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) G[i] = Hn[i] * a.qv[kQvPow + T * kN + 4 * r + i];
    }
    // y = (C . h + D u) SiLU(z), written to the block's y tile
    const int yidx = ((cu ^ swz(4 * r)) << 2) + ce;  // (the same unit position in the lane's four rows)
    auto y_at = [&](int i) {
      const float v = fmaf(dcoef, uf[i], yv[i]);
      return GATE ? v * silu(zf[i]) : v;
    };
    if constexpr (sizeof(YT) == 2) {
      // two steps per conversion, the halves to two rows
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint32_t pk = pk_bf16(y_at(i), y_at(i + 1));
        sm.yt[buf][4 * r + i][yidx].bits = static_cast<uint16_t>(pk);
        sm.yt[buf][4 * r + i + 1][yidx].bits = static_cast<uint16_t>(pk >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) YUnit<YT>::put(&sm.yt[buf][4 * r + i][yidx], y_at(i));
    }
  };

  // Block j's loads go out three blocks ahead (two register sets), its LDS
  // copy one block ahead (two LDS buffers); one barrier per block.  The loop
  // starts two trips early (blocks < 0 load and store nothing, compute
  // nothing) instead of having a prologue, and always runs both halves (its
  // only exit is at the end): the waits the compiler places for the register
  // set being copied then leave the other set's loads in flight.
  Stage S0 = {}, S1 = {};
  // the per-lane constants' loads complete here, so none is in flight on
  // entry either
  __builtin_amdgcn_s_waitcnt(0);
  for (int k = -4; k < nb; k += 2) {
    __syncthreads();
    {
      const auto yu = read_y(k - 1);
      commit(1, S1);  // block k + 1
      put_y(k - 1, yu);
    }
    issue(k + 3, S1);
    if (k >= 0) compute(k, 0);
    __syncthreads();
    {
      const auto yu = read_y(k);
      commit(0, S0);  // block k + 2
      put_y(k, yu);
    }
    issue(k + 4, S0);
    if (k + 1 >= 0 && k + 1 < nb) compute(k + 1, 1);
  }
  // with an even count the last block was computed in a second half
  if ((nb & 1) == 0) {
    __syncthreads();
    put_y(nb - 1, read_y(nb - 1));
  }
  if (a.state_out) {
    // the offset formed again from an opaque copy of the thread id: kept from
    // the start, it would hold two registers through the loop
    int t = tid;
    asm volatile("" : "+v"(t));
    const int c2 = g * kCh + 16 * (t >> 6) + (t & 15);
    const size_t so2 = (static_cast<size_t>(b) * E + c2) * kN + 4 * ((t >> 4) & 3);
    *reinterpret_cast<f32x4*>(a.state_out + so2) = G;
  }
}

template <typename YT, bool GATE>
void launch_main(const ScanBlkArgs& k, hipStream_t stream) {
  const unsigned groups = static_cast<unsigned>(k.batch) * static_cast<unsigned>(k.dim / kCh);
  hipLaunchKernelGGL((scan_blk_kernel<YT, GATE>), dim3(groups), dim3(kThreads), 0, stream, k);
}

}  // namespace

size_t scan_blk_qv_offset(int batch, int seqlen) {
  const size_t rec = static_cast<size_t>(batch) * scan_blk_records(seqlen) * kBlkRec;
  return (rec + 255) & ~static_cast<size_t>(255);
}

size_t scan_blk_workspace_bytes(int batch, int seqlen) {
  if (batch <= 0 || seqlen <= 0) return 0;
  return scan_blk_qv_offset(batch, seqlen) + ((kBlkQv * sizeof(float) + 255) & ~static_cast<size_t>(255));
}

hipError_t launch_scan_blocked(const ScanBlkLaunch& l, hipStream_t stream) {
  const ScanBlkArgs& k = l.k;
  if (k.batch <= 0 || k.seqlen <= 0) return hipSuccess;
  const unsigned packs = static_cast<unsigned>(k.batch) * static_cast<unsigned>(k.nrec);
  if (l.bc_dtype == kBF16) {
    hipLaunchKernelGGL(pack_blk_kernel<bf16s>, dim3(packs), dim3(256), 0, stream, static_cast<const bf16s*>(l.B),
                       static_cast<const bf16s*>(l.C), k.A, k.dt_max, k.seqlen, k.nrec, l.rec_out, l.qv_out);
  } else {
    hipLaunchKernelGGL(pack_blk_kernel<float>, dim3(packs), dim3(256), 0, stream, static_cast<const float*>(l.B),
                       static_cast<const float*>(l.C), k.A, k.dt_max, k.seqlen, k.nrec, l.rec_out, l.qv_out);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return timed_launch(stream, [&] {
    if (l.y_dtype == kBF16)
      k.z ? launch_main<bf16s, true>(k, stream) : launch_main<bf16s, false>(k, stream);
    else
      k.z ? launch_main<float, true>(k, stream) : launch_main<float, false>(k, stream);
  });
}

}  // namespace ssm
