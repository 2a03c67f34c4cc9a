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
// Mapping.  One workgroup (8 waves) per (batch, head, segment of the
// sequence) walks the segment's chunks in order with the head's whole state
// (P x N, fp32) in MFMA accumulators, so C B^T and the decay-weighted matrix M
// of a chunk are formed once per head (they do not depend on the headdim
// column).  Waves 0-3 form the chunk's outputs; waves 4-7 own the state (one
// 16-wide n-block each), load and stage the chunks, scan the decays and
// advance the state while waves 0-3 compute, one wave of each kind per SIMD.  The incoming state of every segment but the first comes from two
// small launches before it: ssd_summary_kernel reduces pieces of up to 16
// chunks to (state reached from zero, total log2 decay) -- the state update
// alone, parallel over pieces -- and ssd_compose_kernel chains them per state
// element in order, S <- 2^decay S + S_piece, which is the same recurrence
// taken a piece at a time.
//
// Per chunk: the state waves stage C, B (both layouts), x (transposed) and dt
// in LDS while the next chunk's loads are in flight, scan dt * A in registers
// and fill the decay tables; output wave q owns the 16-row blocks q and 7 - q
// of the chunk (9 causal blocks, the same for every wave) for all 16-wide
// headdim strips, and for each block J <= I
//   cb^T block     = B_J C_I^T              v_mfma_f32_16x16x32_bf16
//   M (masked)     = cb . 2^(dA_l - dA_s) . dt_s, the skip D on its diagonal
//   out^T[strip]  += X_J^T M^T              v_mfma_f32_16x16x32_bf16, M hi + lo as K = 32
// then the readout of the incoming state, (S C_I^T) scaled by 2^dA[l]
// (v_mfma_f32_16x16x32_bf16, S split hi + lo), and the state update
//   S <- 2^dA[Q-1] S + X^T (w . B)          v_mfma_f32_16x16x32_bf16, w.B hi + lo
// with w[s] = 2^(dA[Q-1] - dA[s]) dt[s].  The hi/lo split (a bf16 value plus
// the bf16 of its remainder) keeps the operands that are not exact bf16 inputs
// at about 16 mantissa bits.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <algorithm>
#include <type_traits>

namespace ssm {
namespace {

constexpr int kQ = kSsdQ;        // 128 tokens per chunk
constexpr int kN = kSsdN;        // 64 states
constexpr int kRowN = kN + 8;    // padded LDS row of N bf16 (144 bytes)
constexpr int kRowQ = kQ + 8;    // padded LDS row of Q bf16 (272 bytes)
constexpr int kThreads = 512;    // 8 waves
constexpr int kPiece = kSsdPiece;  // chunks per summary piece
constexpr int kMaxSeg = kSsdMaxSeg;  // segments per sequence at most
#ifndef SSD_KUNROLL
#define SSD_KUNROLL 1
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family
// The descriptor's words pass through readfirstlane: they are uniform, and
// the compiler must know it, or it wraps every load in a loop over the
// distinct descriptors of the wave's lanes.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kRsrcWord3);
}
// 16 bytes at byte offset vo + so of a raw buffer
__device__ __forceinline__ uint4 ld128(rsrc_t r, uint32_t vo, uint32_t so) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Column of element s in row r of the transposed tiles (Bt, Xt): the 16-byte
// blocks of a row are permuted by the row's 8-row group, so the transposing
// stores fall in different banks.  Reads of 4 or 8 consecutive elements
// inside one block stay contiguous.
__device__ __forceinline__ int swz(int r, int s) { return ((((s >> 3) ^ (r >> 3)) & 15) << 3) | (s & 7); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = bf16_bits(v);
  lo = bf16_bits(v - bf16_val(hi));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// (bf16(a), bf16(b)) in one word, a in the low half (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// hi/lo split of a pair: hi = bf16 of each, lo = bf16 of each remainder
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// bf16 j of a 16-byte piece
__device__ __forceinline__ uint32_t half16(const uint4& v, int j) {
  return (reinterpret_cast<const uint32_t*>(&v)[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
}

constexpr int kIoThreads = 256;  // threads of the state waves (4 x 64)

// Decay tables of one chunk
struct alignas(16) DecayTables {
  float EL[8][kQ];  // 2^(dA[l] - dA[16 J]) for l >= 16 J
  float ESD[kQ];    // 2^(dA[16 (s / 16)] - dA[s]) dt[s]
  float dA[kQ];     // inclusive cumsum of dt * A * log2(e)
  float dt[kQ];     // dt after softplus and clip
  float wS[kQ];     // 2^(dA[Q-1] - dA[s]) * dt[s]: state-update weights
  float eA[kQ];     // 2^dA[l]: decay of the incoming state (eA[Q-1]: of the whole chunk)
};

// The chunk's tiles, and NB copies of the incoming state and of the decay
// tables (two: those of the next chunk are written while the current ones
// are read).
template <int NS, int NB>
struct alignas(16) HeadSmem {
  uint16_t C[kQ][kRowN];             // C chunk, row-major [l][n]
  uint16_t B[kQ][kRowN];             // B chunk, row-major [s][n]
  uint16_t Bt[kN][kRowQ];            // B chunk transposed [n][swz(n, s)]
  uint16_t Xt[16 * NS][kRowQ];       // x chunk transposed [p][swz(p, s)]
  uint16_t Shi[NB][16 * NS][kRowN];  // state entering the chunk, [p][n], bf16 high part
  uint16_t Slo[NB][16 * NS][kRowN];  //                                   bf16 low part
  DecayTables tb[NB];
};
constexpr size_t kLdsBytes = 160 * 1024;
template <int NS>
constexpr int kStateBuffers = sizeof(HeadSmem<NS, 2>) <= kLdsBytes ? 2 : 1;

template <int NS>
struct alignas(16) SummSmem {
  uint16_t Bt[kN][kRowQ];
  uint16_t Xt[16 * NS][kRowQ];
  float dt[kQ];
  float wS[kQ];
};

// A chunk in registers, loaded by NT threads: RPT rows of C and B and XI
// (row pair, 8-column piece) items of x per thread.  Headdim P = 16 NS.
template <int NS, int NT>
struct ChunkRegs {
  static constexpr int RPT = 1024 / NT;
  static constexpr int XI = (128 * NS + NT - 1) / NT;
  uint4 c[RPT], b[RPT], x[XI][2];
  float dt;
  int valid;  // tokens of this chunk inside the sequence (fewer in a ragged last chunk)
};

// Workspace (floats): the state entering segments 1 .. nseg-1, then the
// piece summaries (state from zero) and the pieces' log2 decays.
__host__ __device__ inline size_t ws_sin_floats(const ChunkKernelArgs& a) {
  return static_cast<size_t>(a.batch) * a.nheads * (a.nseg - 1) * a.headdim * kN;
}
__host__ __device__ inline size_t ws_piece_floats(const ChunkKernelArgs& a) {
  return static_cast<size_t>(a.batch) * a.nheads * (a.nseg - 1) * a.ppseg * a.headdim * kN;
}
__host__ __device__ inline size_t ws_dec_floats(const ChunkKernelArgs& a) {
  return static_cast<size_t>(a.batch) * a.nheads * (a.nseg - 1) * a.ppseg;
}

// Shared pieces of both kernels: chunk loads into registers, their LDS
// stores, the dt scan and the state-update MFMAs.
template <int NS, int NT>
struct ChunkIo {
  using Regs = ChunkRegs<NS, NT>;
  static constexpr int RPT = Regs::RPT, XI = Regs::XI;
  const ChunkKernelArgs& a;
  int b, h, g;
  // Buffer descriptors of this (batch, head)'s x, B, C and dt rows.  Whole
  // chunks are read through them: the lane's offset is fixed for the whole
  // walk and the chunk's position goes in the scalar offset, so a chunk's
  // loads need no per-chunk address arithmetic.  (With 64-bit addresses
  // formed per chunk, registers still read by loads in flight were
  // overwritten and every such reuse waited for those loads.)
  rsrc_t rx, rb, rc, rdt;

  __device__ ChunkIo(const ChunkKernelArgs& args, int b_, int h_)
      : a(args), b(b_), h(h_), g(h_ / (args.nheads / args.ngroups)) {
    constexpr size_t P = 16 * NS;
    const size_t L = a.seqlen, H = a.nheads, G = a.ngroups;
    const size_t L1 = L > 0 ? L - 1 : 0;
    rx = make_rsrc(static_cast<const uint16_t*>(a.x) + (b * L * H + h) * P,
                   static_cast<uint32_t>((L1 * H * P + P) * 2));
    rb = make_rsrc(static_cast<const uint16_t*>(a.B) + (b * L * G + g) * kN,
                   static_cast<uint32_t>((L1 * G * kN + kN) * 2));
    rc = make_rsrc(static_cast<const uint16_t*>(a.C) + (b * L * G + g) * kN,
                   static_cast<uint32_t>((L1 * G * kN + kN) * 2));
    rdt = make_rsrc(a.dt + b * L * H + h, static_cast<uint32_t>((L1 * H + 1) * 4));
  }

  // The lane's byte offsets for whole-chunk loads (io thread tid).
  struct Offs {
    uint32_t bc[RPT];
    uint32_t x[XI][2];
    uint32_t dt;
  };
  __device__ __forceinline__ Offs offsets(int tid) const {
    constexpr int P = 16 * NS;
    const int rg = tid >> 3, pc = tid & 7;
    const int H = a.nheads, G = a.ngroups;
    Offs o;
#pragma unroll
    for (int i = 0; i < RPT; ++i) o.bc[i] = static_cast<uint32_t>(((RPT * rg + i) * G * kN + 8 * pc) * 2);
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int q = tid + NT * i;
      const int rgx = q / (2 * NS), pcx = q % (2 * NS);
#pragma unroll
      for (int e = 0; e < 2; ++e) o.x[i][e] = static_cast<uint32_t>(((2 * rgx + e) * H * P + 8 * pcx) * 2);
    }
    o.dt = static_cast<uint32_t>(tid * H * 4);
    return o;
  }

  // Part k of load_whole: 0 the C rows, 1 the B rows, 2 + i the x slot i,
  // 2 + XI the dt row.
  template <bool WITH_C, bool WITH_DT = true>
  __device__ __forceinline__ void load_whole_part(int c, Regs& R, const Offs& o, int tid, int k) const {
    constexpr uint32_t P = 16 * NS;
    const uint32_t H = a.nheads, G = a.ngroups;
    const uint32_t row0 = static_cast<uint32_t>(c) * kQ;
    const uint32_t sbc = row0 * G * kN * 2, sx = row0 * H * P * 2, sdt = row0 * H * 4;
    R.valid = kQ;
    if (k == 0) {
      if constexpr (WITH_C) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) R.c[i] = ld128(rc, o.bc[i], sbc);
      }
    } else if (k == 1) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) R.b[i] = ld128(rb, o.bc[i], sbc);
    } else if (k < 2 + XI) {
#pragma unroll
      for (int i = 0; i < XI; ++i) {
        if (k == 2 + i && (XI * NT == 128 * NS || tid + NT * i < 128 * NS)) {
#pragma unroll
          for (int e = 0; e < 2; ++e) R.x[i][e] = ld128(rx, o.x[i][e], sx);
        }
      }
    } else if (WITH_DT && tid < kQ) {
      R.dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdt, o.dt, sdt, 0));
    }
  }

  // A whole chunk c through the descriptors (io thread tid, offsets o).
  template <bool WITH_C, bool WITH_DT = true>
  __device__ __forceinline__ void load_whole(int c, Regs& R, const Offs& o, int tid) const {
    constexpr uint32_t P = 16 * NS;
    const uint32_t H = a.nheads, G = a.ngroups;
    const uint32_t row0 = static_cast<uint32_t>(c) * kQ;
    const uint32_t sbc = row0 * G * kN * 2, sx = row0 * H * P * 2, sdt = row0 * H * 4;
    R.valid = kQ;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if constexpr (WITH_C) R.c[i] = ld128(rc, o.bc[i], sbc);
      R.b[i] = ld128(rb, o.bc[i], sbc);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      if (XI * NT == 128 * NS || tid + NT * i < 128 * NS) {
#pragma unroll
        for (int e = 0; e < 2; ++e) R.x[i][e] = ld128(rx, o.x[i][e], sx);
      }
    }
    if (WITH_DT && tid < kQ) R.dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdt, o.dt, sdt, 0));
  }

  // Rows past the end of the sequence (a ragged last chunk) load as zeros;
  // their dt is set to 0 when stored, so they neither add to nor decay the
  // state.  Rows of C are loaded when WITH_C.
  template <bool kRag, bool WITH_C, bool WITH_DT = true>
  __device__ __forceinline__ void load(int c, Regs& R, int tid) const {
    constexpr int P = 16 * NS;
    const int rg = tid >> 3, pc = tid & 7;  // C / B: row group, 8-column piece
    const int L = a.seqlen, H = a.nheads, G = a.ngroups;
    const size_t tok = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
    R.valid = kRag ? L - c * kQ : kQ;
    const uint16_t* Cc = static_cast<const uint16_t*>(a.C) + (tok * G + g) * kN;
    const uint16_t* Bc = static_cast<const uint16_t*>(a.B) + (tok * G + g) * kN;
    const uint16_t* xc = static_cast<const uint16_t*>(a.x) + (tok * H + h) * P;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RPT * rg + i;
      const int o = r * G * kN + 8 * pc;
      const bool in = !kRag || r < R.valid;
      if constexpr (WITH_C) R.c[i] = load16_if(Cc + o, in);
      R.b[i] = load16_if(Bc + o, in);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int q = tid + NT * i;
      if (XI * NT == 128 * NS || q < 128 * NS) {
        const int rgx = q / (2 * NS), pcx = q % (2 * NS);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * rgx + e;
          const bool in = !kRag || r < R.valid;
          R.x[i][e] = load16_if(xc + static_cast<size_t>(r) * H * P + 8 * pcx, in);
        }
      }
    }
    if (WITH_DT && tid < R.valid) R.dt = a.dt[(tok + tid) * H + h];
  }

  template <bool kRag, bool WITH_C, bool WITH_DT = true>
  __device__ __forceinline__ void store(const Regs& R, uint16_t (*C)[kRowN], uint16_t (*B)[kRowN],
                                        uint16_t (*Bt)[kRowQ], uint16_t (*Xt)[kRowQ], float* dts, float dtb,
                                        int tid) const {
    const int rg = tid >> 3, pc = tid & 7;
    if constexpr (WITH_C) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        *reinterpret_cast<uint4*>(&C[RPT * rg + i][8 * pc]) = R.c[i];
        *reinterpret_cast<uint4*>(&B[RPT * rg + i][8 * pc]) = R.b[i];
      }
    }
    // B transposed: RPT consecutive s for each of the 8 n of this piece
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (RPT == 4) {
        const uint32_t lo = half16(R.b[0], j) | (half16(R.b[1], j) << 16);
        const uint32_t hi = half16(R.b[2], j) | (half16(R.b[3], j) << 16);
        *reinterpret_cast<uint2*>(&Bt[8 * pc + j][swz(8 * pc + j, 4 * rg)]) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(&Bt[8 * pc + j][swz(8 * pc + j, 2 * rg)]) =
            half16(R.b[0], j) | (half16(R.b[1], j) << 16);
      }
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int q = tid + NT * i;
      if (XI * NT == 128 * NS || q < 128 * NS) {
        const int rgx = q / (2 * NS), pcx = q % (2 * NS);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint32_t*>(&Xt[8 * pcx + j][swz(8 * pcx + j, 2 * rgx)]) =
              half16(R.x[i][0], j) | (half16(R.x[i][1], j) << 16);
      }
    }
    if (WITH_DT && tid < kQ) {
      const float pre = R.dt + dtb;
      const float d = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                    : __builtin_amdgcn_fmed3f(pre, a.dt_min, a.dt_max);
      dts[tid] = !kRag || tid < R.valid ? d : 0.0f;
    }
  }
};

// Inclusive scan of the chunk's dt * A * log2(e) across a wave: lane holds
// steps 2 lane and 2 lane + 1 (d0, d1); `last` is the chunk total.
struct Scan2 {
  float v0, v1, d0, d1, last;
};
// v of the lane selected by DPP control CTRL in the rows of ROWS; 0 where
// the source lane does not exist or the row is not selected
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp0(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, true));
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of row 0 (2) added to row 1 (3), then lane
// 31 to rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp0<0x111, 0xF>(v);  // row_shr:1
  v += dpp0<0x112, 0xF>(v);  // row_shr:2
  v += dpp0<0x114, 0xF>(v);  // row_shr:4
  v += dpp0<0x118, 0xF>(v);  // row_shr:8
  v += dpp0<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp0<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ Scan2 scan_chunk(const float* dts, int lane, float Al2) {
  const float2 dt2 = *reinterpret_cast<const float2*>(&dts[2 * lane]);
  Scan2 r;
  r.v0 = dt2.x;
  r.v1 = dt2.y;
  const float a0 = dt2.x * Al2, a1 = dt2.y * Al2;
  const float incl = wave_prefix_sum(a0 + a1);
  r.d0 = incl - a1;
  r.d1 = incl;
  r.last = lane_value(incl, 63);
  return r;
}

// State update of the blocks (pb = pb0 + PSTRIDE j < NS, nb) a wave owns:
// S[j] <- dlast S[j] + sum_s x[s][p] (wS[s] B[s][n]), formed as the
// transpose (w.B)^T x so that the lane holds four consecutive n of one p:
// S[p = 16 pb + li][n = 16 nb + 4 lg + r], which it publishes with one
// 8-byte store per half.
// between(j) runs after the products of block j (the main kernel issues the
// next chunk's loads there, a part at a time, so their issue overlaps the
// matrix products instead of preceding them).
template <int NS, int NB, int PSTRIDE, typename Between>
__device__ __forceinline__ void state_update(f32x4 (&S)[NB], float dlast, const uint16_t (*Bt)[kRowQ],
                                             const uint16_t (*Xt)[kRowQ], const float* wS, int nb, int pb0, int li,
                                             int lg, Between&& between) {
  const int nrow = 16 * nb + li;
  bf16x8 bwh[4], bwl[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int s0 = 32 * kk + 8 * lg;
    const bf16x8 bt = *reinterpret_cast<const bf16x8*>(&Bt[nrow][swz(nrow, s0)]);
    const float4 w0 = *reinterpret_cast<const float4*>(&wS[s0]);
    const float4 w1 = *reinterpret_cast<const float4*>(&wS[s0 + 4]);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint4 bw = __builtin_bit_cast(uint4, bt);
    const uint32_t bwd[4] = {bw.x, bw.y, bw.z, bw.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      split2(__uint_as_float(bwd[j] << 16) * wv[2 * j], __uint_as_float(bwd[j] & 0xffff0000u) * wv[2 * j + 1], hi[j],
             lo[j]);
    bwh[kk] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    bwl[kk] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int pb = pb0 + PSTRIDE * j;
    if (pb < NS) {
      const int prow = 16 * pb + li;
      f32x4 acc_hi = S[j] * dlast, acc_lo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&Xt[prow][swz(prow, 32 * kk + 8 * lg)]);
        acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwh[kk], xa, acc_hi, 0, 0, 0);
        acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bwl[kk], xa, acc_lo, 0, 0, 0);
      }
      S[j] = acc_hi + acc_lo;
    }
    between(j);
  }
}

// Workgroup order.  Workgroups are handed to the 8 XCDs in turn, so block
// index i runs on XCD i % 8.  A head's x slice (P bf16 per token) shares its
// 128-byte lines with the neighbouring heads', so when the head count is a
// multiple of 8, the heads are cut into 8 runs of consecutive heads and run m
// goes to XCD m (neighbours share that XCD's L2).  The batch varies next,
// then the segment (main kernel) or the summary piece, slowest.
__device__ __forceinline__ void decode_heads(const ChunkKernelArgs& a, int bid, int& h, int& rest) {
  if (a.nheads % 8 == 0) {
    const int run = a.nheads / 8;
    const int xcd = bid & 7;
    rest = bid >> 3;
    h = xcd * run + rest % run;
    rest /= run;
  } else {
    h = bid % a.nheads;
    rest = bid / a.nheads;
  }
}
__device__ __forceinline__ void decode_bid(const ChunkKernelArgs& a, int bid, int& b, int& h, int& k) {
  int rest;
  decode_heads(a, bid, h, rest);
  b = rest % a.batch;
  k = rest / a.batch;
}

// ---- main kernel --------------------------------------------------------
// GATE: the output is multiplied by SiLU(z).  Whole chunks run in the loop;
// a ragged last chunk (L not a multiple of Q) runs after it in its own copy
// of the chunk step, so the loop carries no row tests.
template <typename OT, int NS, bool GATE>
__global__ __launch_bounds__(kThreads) void ssd_kernel(ChunkKernelArgs a) {
  constexpr int P = 16 * NS;
  using Io = ChunkIo<NS, kIoThreads>;
  constexpr int NB = kStateBuffers<NS>;
  __shared__ HeadSmem<NS, NB> sm;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, held in a scalar register
  const bool sw = w >= 4;    // state wave (n-block w - 4); else output wave (row blocks w, 7 - w)
  const int u = w & 3;

  int b, h, seg;
  decode_bid(a, blockIdx.x, b, h, seg);
  const int H = a.nheads, L = a.seqlen;
  const float Al2 = a.A[h] * kLog2e;
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.0f;
  // The decay between positions s <= l of a chunk is 2^(dA[l] - dA[s]).  It is
  // factored through the start of s's 16-block, 2^(dA[l] - dA[16 J]) times
  // 2^(dA[16 J] - dA[s]), two tables shared by the workgroup, when neither
  // factor can overflow: |dt A| log2(e) below 6 per step (the 15 steps of a
  // block then stay under 2^90 either way).  Otherwise each element takes its
  // own exponential.  |dt| is bounded by |dt_max| after a softplus (dt > 0 up
  // to the upper clip, or dt = dt_max when that clip is negative) and by the
  // larger of the two clip magnitudes without one (dt may be negative).
  const float dt_abs = a.dt_softplus ? fabsf(a.dt_max) : fmaxf(fabsf(a.dt_min), fabsf(a.dt_max));
  const bool factored = dt_abs * fabsf(Al2) < 6.0f;
  const Io io(a, b, h);

  // chunks of this segment: [c_beg, c_end); whole ones below nfull
  const int nfull = L / kQ;
  const int c_beg = seg * a.cps;
  const int c_end = min(a.nchunks, c_beg + a.cps);
  const int c_whole = min(c_end, nfull);

  const size_t bh = static_cast<size_t>(b) * H + h;

  // Output waves: 16-row blocks I0 = w and I1 = 7 - w.  D per head is added
  // on the diagonal of M; D per channel after the sums.
  const int I0 = u, I1 = 7 - u;
  const bool dch = a.D != nullptr && a.d_per_channel;
  const float dhead = (a.D != nullptr && !a.d_per_channel) ? a.D[h] : 0.0f;

  // The two kinds of wave run loops of their own (same chunks, two barriers
  // per chunk), so neither holds the other's registers.  Chunk c uses state
  // and table buffer c % NB.  With two buffers the state waves write the
  // next chunk's tables and incoming state while the output waves work on
  // the current chunk; with one, between the chunk's last barrier and the
  // staging of the next.
  if (sw) {
    // The state, held by the state waves: p-blocks 0..NS-1 of n-block u; the
    // lane holds S[p = 16 j + li][n = 16 u + 4 lg + r].
    f32x4 S[NS];
    auto publish_state = [&](int buf, int li, int lg) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int p = 16 * j + li, n0 = 16 * u + 4 * lg;
        uint32_t h01, l01, h23, l23;
        split2(S[j][0], S[j][1], h01, l01);
        split2(S[j][2], S[j][3], h23, l23);
        *reinterpret_cast<uint2*>(&sm.Shi[buf][p][n0]) = make_uint2(h01, h23);
        *reinterpret_cast<uint2*>(&sm.Slo[buf][p][n0]) = make_uint2(l01, l23);
      }
    };
    // dt of chunk c for state wave 0: lane holds rows 2 lane and 2 lane + 1
    // lane offsets of those rows in the head's dt descriptor (whole chunks)
    const uint32_t vdt0 = static_cast<uint32_t>(2 * (threadIdx.x & 63) * H * 4);
    const uint32_t vdt1 = vdt0 + static_cast<uint32_t>(H * 4);
    auto load_dt = [&](int c, int lane, bool whole) {
      const size_t tok = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
      float2 r = make_float2(0.0f, 0.0f);
      if (whole) {
        const uint32_t so = static_cast<uint32_t>(c) * kQ * H * 4;
        r.x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(io.rdt, vdt0, so, 0));
        r.y = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(io.rdt, vdt1, so, 0));
      } else {
        const int valid = min(kQ, L - c * kQ);
        if (2 * lane < valid) r.x = a.dt[(tok + 2 * lane) * H + h];
        if (2 * lane + 1 < valid) r.y = a.dt[(tok + 2 * lane + 1) * H + h];
      }
      return r;
    };
    // decay tables of chunk c (raw dt in dt2) into buffer buf, by state wave
    // 0: the chunk's log2 decays scanned across its lanes
    auto tables = [&](int c, int buf, float2 dt2, int lane) {
      const int valid = min(kQ, L - c * kQ);
      auto dt_of = [&](float raw, int row) {
        const float pre = raw + dtb;
        const float d = a.dt_softplus ? dt_softplus_clip(pre, a.dt_min, a.dt_max, a.sp_lo, a.sp_hi)
                                      : __builtin_amdgcn_fmed3f(pre, a.dt_min, a.dt_max);
        return row < valid ? d : 0.0f;  // rows past the end neither add nor decay
      };
      const float v0 = dt_of(dt2.x, 2 * lane), v1 = dt_of(dt2.y, 2 * lane + 1);
      const float a0 = v0 * Al2, a1 = v1 * Al2;
      const float incl = wave_prefix_sum(a0 + a1);
      const float d0 = incl - a1, d1 = incl, last = lane_value(incl, 63);
      DecayTables& t = sm.tb[buf];
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        const float ref = lane_value(d0, 8 * J);  // dA[16 J]
        if (2 * lane >= 16 * J)
          *reinterpret_cast<float2*>(&t.EL[J][2 * lane]) = make_float2(exp2_fast(d0 - ref), exp2_fast(d1 - ref));
      }
      const float r16 = __shfl(d0, 8 * (lane >> 3));  // dA at the start of this lane's 16-block
      *reinterpret_cast<float2*>(&t.ESD[2 * lane]) = make_float2(exp2_fast(r16 - d0) * v0, exp2_fast(r16 - d1) * v1);
      *reinterpret_cast<float2*>(&t.dA[2 * lane]) = make_float2(d0, d1);
      *reinterpret_cast<float2*>(&t.dt[2 * lane]) = make_float2(v0, v1);
      *reinterpret_cast<float2*>(&t.eA[2 * lane]) = make_float2(exp2_fast(d0), exp2_fast(d1));
      *reinterpret_cast<float2*>(&t.wS[2 * lane]) =
          make_float2(exp2_fast(last - d0) * v0, exp2_fast(last - d1) * v1);
    };

    typename Io::Regs R;
    float2 dtn = make_float2(0.0f, 0.0f);  // raw dt of the next chunk (state wave 0)
    // dt first: the tables wait for it, and loads complete in order, so
    // issued last it would hold the tables until the whole chunk had landed
    const typename Io::Offs offs = io.offsets(threadIdx.x - kIoThreads);
    auto load_chunk = [&](int c, int tid) {
      if (u == 0) dtn = load_dt(c, tid & 63, c < nfull);
      if (c >= nfull)
        io.template load<true, true, false>(c, R, tid - kIoThreads);
      else
        io.template load_whole<true, false>(c, R, offs, tid - kIoThreads);
    };
    {
      const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
      const float* s_in = seg == 0 ? (a.state_in ? a.state_in + bh * P * kN : nullptr)
                                   : a.ws + (bh * (a.nseg - 1) + (seg - 1)) * P * kN;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[j][r] = s_in != nullptr ? s_in[static_cast<size_t>(16 * j + li) * kN + 16 * u + 4 * lg + r] : 0.0f;
      // the loads of S complete here on every path: otherwise the wait for
      // them is placed at S's first use inside the chunk loop, where it runs
      // every chunk and also waits for the next chunk's loads in flight
#pragma unroll
      for (int j = 0; j < NS; ++j) asm volatile("" : "+v"(S[j]));
      if (c_beg < c_end) {
        load_chunk(c_beg, threadIdx.x);
        publish_state(c_beg % NB, li, lg);
        if (u == 0) tables(c_beg, c_beg % NB, dtn, lane);
      }
    }
    for (int c = c_beg; c < c_end; ++c) {
      // Lane indexes re-derived from an opaque copy of the thread id: the LDS
      // and global offsets built from them are then formed inside the loop
      // instead of being hoisted out of it, which would hold some hundred
      // registers across the whole loop.
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
      const int buf = c % NB, nbuf = (c + 1) % NB;
      // ---- stage the chunk (every reader of the previous chunk's tiles
      // passed the last barrier)
      io.template store<false, true, false>(R, sm.C, sm.B, sm.Bt, sm.Xt, nullptr, dtb, tid - kIoThreads);
      __syncthreads();
      // the next chunk's loads, in flight while the chunk is processed
      // ---- state update (registers), with the next chunk's loads issued
      // between its blocks (a ragged next chunk: all before it); published
      // for the next chunk once the output waves no longer read the buffer
      const bool more = c + 1 < c_end, whole_next = c + 1 < nfull;
      if (more && whole_next) {
        // dt first: the tables wait only for it (loads complete in order)
        state_update<NS, NS, 1>(S, sm.tb[buf].eA[kQ - 1], sm.Bt, sm.Xt, sm.tb[buf].wS, u, 0, li, lg, [&](int j) {
          constexpr int kParts = 3 + Io::XI;  // dt, C rows, B rows, the x slots
#pragma unroll
          for (int k = 0; k < kParts; ++k)
            if (k == j || (j == NS - 1 && k > j)) {
              if (k == 0) {
                if (u == 0) dtn = load_dt(c + 1, lane, true);
              } else {
                io.template load_whole_part<true, false>(c + 1, R, offs, tid - kIoThreads, k - 1);
              }
            }
        });
      } else {
        if (more) load_chunk(c + 1, tid);  // the ragged last chunk
        state_update<NS, NS, 1>(S, sm.tb[buf].eA[kQ - 1], sm.Bt, sm.Xt, sm.tb[buf].wS, u, 0, li, lg, [](int) {});
      }
      if constexpr (NB == 2) {
        publish_state(nbuf, li, lg);
        if (u == 0 && c + 1 < c_end) tables(c + 1, nbuf, dtn, lane);
        __syncthreads();
      } else {
        __syncthreads();
        publish_state(nbuf, li, lg);
        if (u == 0 && c + 1 < c_end) tables(c + 1, nbuf, dtn, lane);
      }
    }
    if (a.state_out && seg == a.nseg - 1) {
      const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.state_out[bh * P * kN + static_cast<size_t>(16 * j + li) * kN + 16 * u + 4 * lg + r] = S[j][r];
    }
    return;
  }

  auto out_step = [&](const int c, auto ragged) {
    constexpr bool kRag = decltype(ragged)::value;
    int tid = threadIdx.x;  // opaque copy, as in the state waves' loop
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const size_t tok0 = static_cast<size_t>(b) * L + static_cast<size_t>(c) * kQ;
    const int valid = kRag ? L - c * kQ : kQ;
    // gate values of item it (row l = 16 I + li, columns 16 st + 4 lg .. + 3),
    // fetched before its sums so that their latency overlaps them
    auto load_gate = [&](int it, uint4 (&zr)[NS]) {
      const int l = 16 * (it ? I1 : I0) + li;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        zr[t] = make_uint4(0u, 0u, 0u, 0u);
        if (!kRag || l < valid) {
          const size_t e = ((tok0 + l) * H + h) * P + 16 * t + 4 * lg;
          if (a.z_bf16) {
            const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.z) + e);
            zr[t].x = v.x;
            zr[t].y = v.y;
          } else {
            zr[t] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.z) + e);
          }
        }
      }
    };
    __syncthreads();  // the chunk, its tables and its incoming state are in place
    const DecayTables& tb = sm.tb[c % NB];
    const uint16_t (*Shi)[kRowN] = sm.Shi[c % NB];
    const uint16_t (*Slo)[kRowN] = sm.Slo[c % NB];
    // ---- outputs.  Intra-chunk sums of one item (16-row block I): blocks
    // J = 0..I in a software pipeline -- in step J the C B^T product of
    // block J + 1 is issued, the LDS operands of blocks J + 1 (decays,
    // x^T) and J + 2 (B rows) are fetched, and block J's M is formed and
    // multiplied -- with the diagonal block (masked, D on its diagonal)
    // peeled off the loop.
    struct Ops {
      float el;         // factored: 2^(dA[l] - dA[16 J]); otherwise dA[l]
      float4 e4;        // factored: 2^(dA[16 J] - dA[s]) dt[s]; otherwise dA[s]
      s16x4 xv[NS];     // x^T[p][s] fragments of the strips
    };
    auto rows16 = [&](const uint16_t (*M)[kRowN], int blk, bf16x8 (&v)[2]) {
      v[0] = *reinterpret_cast<const bf16x8*>(&M[16 * blk + li][8 * lg]);
      v[1] = *reinterpret_cast<const bf16x8*>(&M[16 * blk + li][32 + 8 * lg]);
    };
    auto load_ops = [&](int I, int J, Ops& o, auto fac) {
      constexpr bool kFac = decltype(fac)::value;
      const int l_row = 16 * I + li, s0 = 16 * J + 4 * lg;
      o.el = kFac ? tb.EL[J][l_row] : tb.dA[l_row];
      o.e4 = *reinterpret_cast<const float4*>(kFac ? &tb.ESD[s0] : &tb.dA[s0]);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const int prow = 16 * t + li;
        o.xv[t] = *reinterpret_cast<const s16x4*>(&sm.Xt[prow][swz(prow, s0)]);
      }
    };
    auto cbT = [&](const bf16x8 (&bj)[2], const bf16x8 (&ci)[2]) {
      f32x4 cb = {0.0f, 0.0f, 0.0f, 0.0f};
      cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bj[0], ci[0], cb, 0, 0, 0);
      cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bj[1], ci[1], cb, 0, 0, 0);
      return cb;
    };
    // block (I, J): lane holds cb[l = 16 I + li][s = 16 J + 4 lg + r], which
    // is the B operand M^T[s][l] of the x^T M^T product as it stands
    auto block = [&](int J, const f32x4& cb, const Ops& o, f32x4 (&acc)[NS], auto fac, auto diag) {
      constexpr bool kFac = decltype(fac)::value;
      constexpr bool kDiag = decltype(diag)::value;
      const float ev[4] = {o.e4.x, o.e4.y, o.e4.z, o.e4.w};
      float m[4];
      if constexpr (kFac) {
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = cb[r] * o.el * ev[r];
      } else {
        const float4 d4 = *reinterpret_cast<const float4*>(&tb.dt[16 * J + 4 * lg]);
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = cb[r] * exp2_fast(o.el - ev[r]) * dv4[r];
      }
      if constexpr (kDiag) {
        // causal mask, applied after the product so a masked overflow never
        // reaches the sum; the per-head skip D on the diagonal
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 4 * lg + r;
          m[r] = s < li ? m[r] : (s == li ? m[r] + dhead : 0.0f);
        }
      }
      uint32_t h01, l01, h23, l23;
      split2(m[0], m[1], h01, l01);
      split2(m[2], m[3], h23, l23);
      // hi and lo as one K = 32 product: the lane's k slots 0-3 carry
      // (x, M hi) and slots 4-7 (x, M lo) for the same four s
      const bf16x8 mhl = __builtin_bit_cast(bf16x8, make_uint4(h01, h23, l01, l23));
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const uint2 xu = __builtin_bit_cast(uint2, o.xv[t]);
        const bf16x8 xx = __builtin_bit_cast(bf16x8, make_uint4(xu.x, xu.y, xu.x, xu.y));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xx, mhl, acc[t], 0, 0, 0);
      }
    };
    auto item = [&](const int I, const bf16x8 (&ci)[2], f32x4 (&acc)[NS], auto fac) {
      bf16x8 b0[2], b1[2];
      Ops cur, nxt;
      rows16(sm.B, 0, b0);
      rows16(sm.B, I > 0 ? 1 : 0, b1);
      load_ops(I, 0, cur, fac);
      f32x4 cb = cbT(b0, ci);
      // one off-diagonal step: block J from (cb, o), block J + 1's operands into o2
      auto step = [&](int J, const Ops& o, Ops& o2) {
        const f32x4 cbn = cbT(b1, ci);    // block J + 1
        rows16(sm.B, min(J + 2, 7), b1);  // block J + 2 (loaded, not used, past the diagonal)
        load_ops(I, J + 1, o2, fac);
        block(J, cb, o, acc, fac, std::false_type{});
        cb = cbn;
      };
      // two steps per trip so that the operand sets swap roles instead of
      // being copied
      int J = 0;
      for (; J + 2 <= I; J += 2) {
        step(J, cur, nxt);
        step(J + 1, nxt, cur);
      }
      if (J < I) {
        step(J, cur, nxt);
        block(I, cb, nxt, acc, fac, std::true_type{});
      } else {
        block(I, cb, cur, acc, fac, std::true_type{});
      }
    };

    // Readout of the incoming state, (S C_I^T)[p][l] scaled by 2^dA[l],
    // added to the sums; then the per-channel skip, the gate and the
    // store.  The lane holds rows p = 16 st + 4 lg + r of column
    // l = 16 I + li.
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto finish = [&](const int it, const bf16x8 (&ci)[2], f32x4 (&acc)[NS], const uint4 (&zr)[NS], auto per_ch) {
      constexpr bool kDch = decltype(per_ch)::value;
      const int I = it ? I1 : I0;
      const int l = 16 * I + li;
      const float eAl = tb.eA[l];
      const bool orow = !kRag || l < valid;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        f32x4 sr_hi = zero4, sr_lo = zero4;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&Shi[16 * st + li][32 * kk + 8 * lg]);
          const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&Slo[16 * st + li][32 * kk + 8 * lg]);
          sr_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sh, ci[kk], sr_hi, 0, 0, 0);
          sr_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl, ci[kk], sr_lo, 0, 0, 0);
        }
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(eAl, sr_hi[r] + sr_lo[r], acc[st][r]);
        if constexpr (kDch) {
          const float4 d4 = *reinterpret_cast<const float4*>(a.D + static_cast<size_t>(h) * P + 16 * st + 4 * lg);
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int p = 16 * st + 4 * lg + r;
            v[r] = fmaf(dv[r], bf16_val(sm.Xt[p][swz(p, l)]), v[r]);
          }
        }
        if constexpr (GATE) {
          float zv[4];
          if (a.z_bf16) {
            zv[0] = __uint_as_float(zr[st].x << 16);
            zv[1] = __uint_as_float(zr[st].x & 0xffff0000u);
            zv[2] = __uint_as_float(zr[st].y << 16);
            zv[3] = __uint_as_float(zr[st].y & 0xffff0000u);
          } else {
            zv[0] = __uint_as_float(zr[st].x);
            zv[1] = __uint_as_float(zr[st].y);
            zv[2] = __uint_as_float(zr[st].z);
            zv[3] = __uint_as_float(zr[st].w);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] *= silu(zv[r]);
        }
        if (orow) {
          const size_t e = ((tok0 + l) * H + h) * P + 16 * st + 4 * lg;
          if constexpr (sizeof(OT) == 4) {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + e) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + e) =
                make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
          }
        }
      }
    };
    // each item's sums, then its outputs
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int I = it ? I1 : I0;
      f32x4 acc[NS];
#pragma unroll
      for (int t = 0; t < NS; ++t) acc[t] = zero4;
      uint4 zr[NS];
      if constexpr (GATE) load_gate(it, zr);
      bf16x8 ci[2];
      rows16(sm.C, I, ci);
      if (factored)
        item(I, ci, acc, std::true_type{});
      else
        item(I, ci, acc, std::false_type{});
      if (dch)
        finish(it, ci, acc, zr, std::true_type{});
      else
        finish(it, ci, acc, zr, std::false_type{});
    }
    __syncthreads();  // the chunk's tiles, tables and state have been read
  };
  for (int c = c_beg; c < c_whole; ++c) out_step(c, std::false_type{});
  if (c_end > nfull && c_beg <= nfull) out_step(nfull, std::true_type{});
}

// ---- segment pieces: state reached from zero and total log2 decay --------
// Workgroup (piece j of segment k < nseg - 1, batch, head); the piece covers
// chunks [k cps + j kPiece, min(k cps + (j + 1) kPiece, (k + 1) cps)), all
// whole (the ragged chunk, if any, is the last chunk of the last segment).
// Four waves; wave w owns n-block w of the piece's state for all p-blocks.
template <int NS>
__global__ __launch_bounds__(kIoThreads) void ssd_summary_kernel(ChunkKernelArgs a) {
  constexpr int P = 16 * NS;
  using Io = ChunkIo<NS, kIoThreads>;
  __shared__ SummSmem<NS> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
  const int lane = tid & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;

  const int npieces = (a.nseg - 1) * a.ppseg;
  int h, rest;
  decode_heads(a, blockIdx.x, h, rest);
  const int b = rest % a.batch;
  const int piece = rest / a.batch;
  const int seg = piece / a.ppseg, j = piece % a.ppseg;
  const int c_beg = seg * a.cps + j * kPiece;
  const int c_end = min(c_beg + kPiece, (seg + 1) * a.cps);
  const float Al2 = a.A[h] * kLog2e;
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const Io io(a, b, h);

  f32x4 S[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) S[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float dec = 0.0f;

  typename Io::Regs R;
  const typename Io::Offs offs = io.offsets(tid);
  if (c_beg < c_end) io.template load_whole<false>(c_beg, R, offs, tid);
  for (int c = c_beg; c < c_end; ++c) {
    int tid = threadIdx.x;  // opaque copy: offsets formed inside the loop (see ssd_kernel)
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    __syncthreads();  // the previous chunk's LDS readers are done
    io.template store<false, false>(R, nullptr, nullptr, sm.Bt, sm.Xt, sm.dt, dtb, tid);
    if (c + 1 < c_end) io.template load_whole<false>(c + 1, R, offs, tid);
    __syncthreads();
    const Scan2 sc = scan_chunk(sm.dt, lane, Al2);
    if (w == 0) {
      sm.wS[2 * lane] = exp2_fast(sc.last - sc.d0) * sc.v0;
      sm.wS[2 * lane + 1] = exp2_fast(sc.last - sc.d1) * sc.v1;
    }
    dec += sc.last;
    __syncthreads();
    state_update<NS, NS, 1>(S, exp2_fast(sc.last), sm.Bt, sm.Xt, sm.wS, w, 0, li, lg, [](int) {});
  }

  const size_t bh = static_cast<size_t>(b) * a.nheads + h;
  const size_t slot = bh * npieces + piece;
  float* out = a.ws + ws_sin_floats(a) + slot * P * kN;
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[static_cast<size_t>(16 * t + li) * kN + 16 * w + 4 * lg + r] = S[t][r];
  if (tid == 0) a.ws[ws_sin_floats(a) + ws_piece_floats(a) + slot] = dec;
}

// ---- state entering each segment: the pieces chained in order ------------
// Thread per (batch, head, state element); S <- 2^decay S + S_piece over the
// pieces of segments 0 .. nseg - 2, starting from state_in (or zeros).
__global__ __launch_bounds__(256) void ssd_compose_kernel(ChunkKernelArgs a) {
  const int PN = a.headdim * kN;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= PN) return;
  const size_t bh = blockIdx.y;
  const int npieces = (a.nseg - 1) * a.ppseg;
  float s = a.state_in ? a.state_in[bh * PN + e] : 0.0f;
  const float* pieces = a.ws + ws_sin_floats(a) + bh * npieces * PN;
  const float* decs = a.ws + ws_sin_floats(a) + ws_piece_floats(a) + bh * npieces;
  float* sin = a.ws + bh * (a.nseg - 1) * PN;
  for (int k = 0; k < a.nseg - 1; ++k) {
    for (int j = 0; j < a.ppseg; ++j) {
      const int pc = k * a.ppseg + j;
      s = fmaf(exp2_fast(decs[pc]), s, pieces[static_cast<size_t>(pc) * PN + e]);
    }
    sin[static_cast<size_t>(k) * PN + e] = s;
  }
}

template <int NS>
int resident_blocks_per_cu() {
  static int cached = 0;
  int v = __atomic_load_n(&cached, __ATOMIC_RELAXED);
  if (v > 0) return v;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ssd_kernel<bf16s, NS, false>, kThreads, 0) != hipSuccess ||
      n <= 0)
    n = 1;
  __atomic_store_n(&cached, n, __ATOMIC_RELAXED);
  return n;
}

int resident_blocks(int headdim) {
  static int cu_count[64] = {};
  int dev = 0;
  int cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    int c = __atomic_load_n(&cu_count[dev], __ATOMIC_RELAXED);
    if (c <= 0 && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      __atomic_store_n(&cu_count[dev], c, __ATOMIC_RELAXED);
    if (c > 0) cus = c;
  }
  int per = 1;
  switch (headdim / 16) {
    case 1: per = resident_blocks_per_cu<1>(); break;
    case 2: per = resident_blocks_per_cu<2>(); break;
    case 3: per = resident_blocks_per_cu<3>(); break;
    case 4: per = resident_blocks_per_cu<4>(); break;
    case 5: per = resident_blocks_per_cu<5>(); break;
    case 6: per = resident_blocks_per_cu<6>(); break;
    case 7: per = resident_blocks_per_cu<7>(); break;
    default: per = resident_blocks_per_cu<8>(); break;
  }
  return cus * per;
}

template <typename OT, int NS>
hipError_t go(const ChunkLaunch& l, hipStream_t s) {
  const ChunkKernelArgs& k = l.k;
  const unsigned heads = static_cast<unsigned>(k.batch) * k.nheads;
  if (heads == 0) return hipSuccess;
  if (k.nseg > 1) {
    const unsigned pieces = heads * static_cast<unsigned>((k.nseg - 1) * k.ppseg);
    hipLaunchKernelGGL((ssd_summary_kernel<NS>), dim3(pieces), dim3(kIoThreads), 0, s, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned pn = static_cast<unsigned>(k.headdim * kN);
    hipLaunchKernelGGL(ssd_compose_kernel, dim3((pn + 255) / 256, heads), dim3(256), 0, s, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned blocks = heads * static_cast<unsigned>(k.nseg);
  return timed_launch(s, [&] {
    if (k.z != nullptr)
      hipLaunchKernelGGL((ssd_kernel<OT, NS, true>), dim3(blocks), dim3(kThreads), 0, s, k);
    else
      hipLaunchKernelGGL((ssd_kernel<OT, NS, false>), dim3(blocks), dim3(kThreads), 0, s, k);
  });
}

template <typename OT>
hipError_t go_ns(const ChunkLaunch& l, hipStream_t s) {
  switch (l.k.headdim / 16) {
    case 1: return go<OT, 1>(l, s);
    case 2: return go<OT, 2>(l, s);
    case 3: return go<OT, 3>(l, s);
    case 4: return go<OT, 4>(l, s);
    case 5: return go<OT, 5>(l, s);
    case 6: return go<OT, 6>(l, s);
    case 7: return go<OT, 7>(l, s);
    case 8: return go<OT, 8>(l, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Segments per sequence: the caller's count (at most one per chunk), else
// enough (batch, head, segment) workgroups to fill the device once, with at
// least 8 chunks per segment.
ChunkSplit chunk_split(int batch, int seqlen, int nheads, int headdim, int segments) {
  ChunkSplit sp{1, 0, 0};
  const int nchunks = (seqlen + kQ - 1) / kQ;
  sp.cps = nchunks;
  const long heads = static_cast<long>(batch) * nheads;
  if (heads <= 0 || nchunks < 2 || headdim <= 0) return sp;
  int s;
  if (segments > 0) {
    s = std::min(segments, nchunks);
  } else {
    if (nchunks < 16) return sp;
    const long slots = resident_blocks(headdim);
    s = heads >= slots ? 1 : static_cast<int>(slots / heads);
    s = std::min(std::min(s, kMaxSeg), nchunks / 8);
  }
  if (s <= 1) return sp;
  sp.cps = (nchunks + s - 1) / s;
  sp.nseg = (nchunks + sp.cps - 1) / sp.cps;
  sp.ppseg = (sp.cps + kPiece - 1) / kPiece;
  return sp;
}

size_t chunk_workspace_bytes(int batch, int seqlen, int nheads, int headdim, int segments) {
  const ChunkSplit sp = chunk_split(batch, seqlen, nheads, headdim, segments);
  if (sp.nseg <= 1) return 0;
  ChunkKernelArgs a{};
  a.batch = batch;
  a.nheads = nheads;
  a.headdim = headdim;
  a.nseg = sp.nseg;
  a.ppseg = sp.ppseg;
  return (ws_sin_floats(a) + ws_piece_floats(a) + ws_dec_floats(a)) * sizeof(float);
}

hipError_t launch_chunk(const ChunkLaunch& l, hipStream_t stream) {
  if (l.out_dtype == kBF16) return go_ns<bf16s>(l, stream);
  return go_ns<float>(l, stream);
}

}  // namespace ssm
