// Host side of the C ABI declared in include/ssm_mi355x.h: argument
// validation (pure host code, runs without a GPU), workspace sizing, variant
// choice and launch on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "../../include/ssm_mi355x.h"
#include "ssm_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local ssm::TimingEvents g_timing;

ssm_status_t fail(ssm_status_t s, const char* fmt, const char* what) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, what);
  g_last_error = buf;
  return s;
}

ssm_status_t ok() {
  g_last_error.clear();
  return SSM_OK;
}

bool valid_dtype(int32_t d) { return d == SSM_F32 || d == SSM_BF16; }
size_t esize(int32_t d) { return d == SSM_BF16 ? 2 : 4; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outward-rounded thresholds of the softplus/clip shortcut: pre >= sp_hi
// guarantees softplus(pre) >= hi, pre <= sp_lo guarantees softplus(pre) <= lo.
void softplus_thresholds(float lo, float hi, float* sp_lo, float* sp_hi) {
  const float inf = std::numeric_limits<float>::infinity();
  if (!(hi < inf)) {
    *sp_hi = inf;
  } else if (hi <= 0.0f) {
    *sp_hi = -inf;
  } else {
    const double t = std::log(std::expm1(static_cast<double>(hi)));
    float f = static_cast<float>(t);
    if (static_cast<double>(f) < t) f = std::nextafter(f, inf);
    *sp_hi = std::nextafter(f, inf);  // one more ulp of margin for the fp32 comparison
  }
  if (!(lo > 0.0f)) {
    *sp_lo = -inf;
  } else if (!(lo < inf)) {
    *sp_lo = inf;
  } else {
    const double t = std::log(std::expm1(static_cast<double>(lo)));
    float f = static_cast<float>(t);
    if (static_cast<double>(f) > t) f = std::nextafter(f, -inf);
    *sp_lo = std::nextafter(f, -inf);
  }
}

ssm_status_t check_dt_bounds(float lo, float hi) {
  if (std::isnan(lo) || std::isnan(hi)) return fail(SSM_ERR_INVALID_ARG, "%s is NaN", "dt_min/dt_max");
  if (lo > hi) return fail(SSM_ERR_INVALID_ARG, "%s: dt_min > dt_max", "dt bounds");
  return SSM_OK;
}

// ---------------------------------------------------------------- scan

// Number of time segments.  A wave issues at most about one VALU instruction
// every 9 cycles on its own and needs 2-3 companions on its SIMD to keep the
// VALU busy, so the split makes batch * channel groups * segments as large as
// the device holds at once for the full-segment kernel (its resident
// workgroups per CU from the occupancy calculator, times the CUs: 3 x 1024 on
// MI355X at the kernels' register use), and no larger: one more segment past
// that runs as a second, mostly idle round.  Segments keep at least 32 steps
// (the summary pass and the composition cost a fixed amount per segment), and
// every segment past the first starts at t >= 4, so only the first reads the
// conv cache (which the last one may overwrite in place).
// Segment length for s segments: ceil(L / s) rounded up to whole rescaling
// periods of the scaled-state form (two load tiles), so every segment starts
// where the rescaled B/C rows start a period and only the last one ends
// inside it.
int scan_seg_len(int L, int s) {
  const int seg = (L + s - 1) / s;
  return (seg + ssm::kScanResc - 1) / ssm::kScanResc * ssm::kScanResc;
}

// The kernel variant a call selects (what the occupancy depends on).
ssm::ScanLaunch scan_variant(const ssm_scan_params_t* p) {
  ssm::ScanLaunch l{};
  l.x_dtype = p->x_dtype;
  l.y_dtype = p->y_dtype;
  l.bc_dtype = p->bc_dtype;
  l.dt_mode = p->dt_rank1 ? 0 : (p->dt_dtype == SSM_BF16 ? 2 : 1);
  l.conv = p->conv_w != nullptr;
  l.zoh = p->discretization == SSM_ZOH;
  l.k.has_z = p->z ? 1 : 0;
  return l;
}

int scan_split(const ssm_scan_params_t* p) {
  const int L = p->seqlen;
  if (p->batch <= 0 || L <= 0 || p->dim <= 0) return 1;  // no work: nothing to split, no workspace
  int s = p->time_split;
  if (s <= 0) {
    const long groups = static_cast<long>(p->batch) * ((p->dim + 63) / 64);
    long slots = ssm::scan_resident_waves(scan_variant(p));
    if (slots <= 0) slots = 3 * 1024;  // no device to ask: MI355X at 3 waves per SIMD
    s = groups >= slots ? 1 : static_cast<int>(slots / groups);
    s = std::min(s, std::max(1, L / 32));
  }
  s = std::min(std::min(s, ssm::kScanMaxSplit), std::max(1, L / 4));
  if (s <= 1) return 1;
  const int seg = scan_seg_len(L, s);
  return (L + seg - 1) / seg;
}

// The blocked single-pass kernel (scan_blocked.hip) takes bf16 u and z, an
// E-wide bf16 dt, no conv, Euler, whole 64-channel groups, and the alignment
// of its 8- and 16-byte accesses.
bool scan_blocked_fits(const ssm_scan_params_t* p) {
  const auto al = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; };
  return p->x_dtype == SSM_BF16 && (!p->z || p->z_dtype == SSM_BF16) && !p->dt_rank1 && p->dt_dtype == SSM_BF16 &&
         !p->conv_w && p->discretization == SSM_EULER && p->d_state == ssm::kScanN && p->dim > 0 &&
         p->dim % 64 == 0 && al(p->x, 8) && al(p->z, 8) && al(p->dt, 8) &&
         al(p->y, p->y_dtype == SSM_BF16 ? 8 : 16) && al(p->ssm_state_out, 16);
}

// Whether a call runs the blocked kernel: asked for (time_split =
// SSM_SCAN_BLOCKED), or chosen (time_split = 0) when it fits and the batch's
// channel groups fill every CU three times over (below that the time-split
// kernels keep more waves busy).
bool scan_blocked(const ssm_scan_params_t* p) {
  if (p->batch <= 0 || p->seqlen <= 0) return false;
  if (p->time_split == SSM_SCAN_BLOCKED) return true;
  return p->time_split == 0 && scan_blocked_fits(p) &&
         static_cast<long>(p->batch) * (p->dim / 64) >= ssm::kBlkAutoGroups;
}

size_t scan_ws(const ssm_scan_params_t* p) {
  if (scan_blocked(p)) return ssm::scan_blk_workspace_bytes(p->batch, p->seqlen);
  return ssm::scan_workspace_bytes(p->batch, p->seqlen, p->dim, scan_split(p));
}

ssm_status_t scan_check(const ssm_scan_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_scan_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->discretization != SSM_EULER && p->discretization != SSM_ZOH)
    return fail(SSM_ERR_INVALID_ARG, "%s must be SSM_EULER or SSM_ZOH", "discretization");
  if (p->batch < 0 || p->seqlen < 0 || p->dim <= 0)
    return fail(SSM_ERR_INVALID_ARG, "%s: negative size or dim <= 0", "batch/seqlen/dim");
  if (p->d_state <= 0) return fail(SSM_ERR_INVALID_ARG, "%s must be positive", "d_state");
  if (p->d_state != ssm::kScanN) return fail(SSM_ERR_UNSUPPORTED, "%s must be 16", "d_state");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->y_dtype) || !valid_dtype(p->bc_dtype) ||
      !valid_dtype(p->dt_dtype) || (p->z && !valid_dtype(p->z_dtype)))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/y/bc/dt/z_dtype");
  if (p->z && p->z_dtype != p->x_dtype) return fail(SSM_ERR_UNSUPPORTED, "%s must equal x_dtype", "z_dtype");
  if (p->time_split < SSM_SCAN_BLOCKED || p->time_split > ssm::kScanMaxSplit)
    return fail(SSM_ERR_INVALID_ARG, "%s must be in [-1, 32]", "time_split");
  if (p->time_split == SSM_SCAN_BLOCKED && !scan_blocked_fits(p))
    return fail(SSM_ERR_UNSUPPORTED,
                "%s: the blocked scan takes bf16 x/z, E-wide bf16 dt, no conv, Euler, dim % 64 == 0, x/z/dt/y "
                "8-byte and ssm_state_out 16-byte aligned (fp32 y: 16-byte)",
                "time_split = SSM_SCAN_BLOCKED");
  if (!p->A) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "A");
  if (p->conv_w) {
    if (p->conv_k != ssm::kConvK) return fail(SSM_ERR_UNSUPPORTED, "%s must be 4", "conv_k");
  } else if (p->conv_cache_in || p->conv_cache_out || p->conv_b) {
    return fail(SSM_ERR_INVALID_ARG, "%s given without conv_w", "conv_b/conv_cache");
  }
  if (p->dt_rank1) {
    if (p->dt_dtype != SSM_F32) return fail(SSM_ERR_UNSUPPORTED, "%s: rank-1 dt input must be f32", "dt_dtype");
    if (!p->dt_w) return fail(SSM_ERR_INVALID_ARG, "%s is NULL with dt_rank1", "dt_w");
  }
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  const size_t Bt = p->batch, L = p->seqlen, E = p->dim, N = p->d_state;
  const size_t tok = Bt * L;
  if (tok > 0) {
    if (!p->x) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x");
    if (!p->y) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "y");
    if (!p->B || !p->C) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "B/C");
    if (!p->dt) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "dt");
  }
  if (Bt * ((E + 63) / 64) * ssm::kScanMaxSplit > 0x7fffffffULL)
    return fail(SSM_ERR_UNSUPPORTED, "%s too large", "batch*dim");
  if ((L + 64) * E * 4 >= 0x80000000ULL)
    return fail(SSM_ERR_UNSUPPORTED, "%s: one batch row must stay under 2 GiB", "seqlen*dim");
  const Range y{p->y, tok * E * esize(p->y_dtype)};
  const Range ins[] = {
      {p->x, tok * E * esize(p->x_dtype)},
      {p->z, p->z ? tok * E * esize(p->z_dtype) : 0},
      {p->dt, p->dt_rank1 ? tok * 4 : tok * E * esize(p->dt_dtype)},
      {p->B, tok * N * esize(p->bc_dtype)},
      {p->C, tok * N * esize(p->bc_dtype)},
      {p->A, E * N * 4},
      {p->D, p->D ? E * 4 : 0},
      {p->ssm_state_in, p->ssm_state_in ? Bt * E * N * 4 : 0},
      {p->ssm_state_out, p->ssm_state_out ? Bt * E * N * 4 : 0},
      {p->conv_cache_in, p->conv_cache_in ? Bt * E * 3 * 4 : 0},
      {p->conv_cache_out, p->conv_cache_out ? Bt * E * 3 * 4 : 0},
      {p->workspace, p->workspace_bytes},
  };
  for (const Range& r : ins)
    if (overlaps(y, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "y");
  if (p->ssm_state_out && p->ssm_state_out != p->ssm_state_in &&
      overlaps({p->ssm_state_out, Bt * E * N * 4}, {p->ssm_state_in, p->ssm_state_in ? Bt * E * N * 4 : 0}))
    return fail(SSM_ERR_INVALID_ARG, "%s partially overlaps ssm_state_in", "ssm_state_out");
  const size_t need = scan_ws(p);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(SSM_ERR_WORKSPACE, "%s is missing or smaller than ssm_scan_workspace_size()", "workspace");
  if (p->workspace && (reinterpret_cast<uintptr_t>(p->workspace) & 255))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 256-byte aligned", "workspace");
  return SSM_OK;
}

// ---------------------------------------------------------------- decode

ssm_status_t decode_check(const ssm_decode_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_decode_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->discretization != SSM_EULER && p->discretization != SSM_ZOH)
    return fail(SSM_ERR_INVALID_ARG, "%s must be SSM_EULER or SSM_ZOH", "discretization");
  if (p->batch < 0 || p->dim <= 0) return fail(SSM_ERR_INVALID_ARG, "%s: negative size or dim <= 0", "batch/dim");
  if (p->d_state <= 0) return fail(SSM_ERR_INVALID_ARG, "%s must be positive", "d_state");
  if (p->d_state != ssm::kScanN) return fail(SSM_ERR_UNSUPPORTED, "%s must be 16", "d_state");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->y_dtype) || !valid_dtype(p->bc_dtype) ||
      !valid_dtype(p->dt_dtype) || (p->z && !valid_dtype(p->z_dtype)))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/y/bc/dt/z_dtype");
  if (p->z && p->z_dtype != p->x_dtype) return fail(SSM_ERR_UNSUPPORTED, "%s must equal x_dtype", "z_dtype");
  if (!p->A) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "A");
  if (p->conv_w) {
    if (p->conv_k != ssm::kConvK) return fail(SSM_ERR_UNSUPPORTED, "%s must be 4", "conv_k");
    if (p->batch > 0 && !p->conv_cache) return fail(SSM_ERR_INVALID_ARG, "%s is NULL with conv_w", "conv_cache");
  } else if (p->conv_cache || p->conv_b) {
    return fail(SSM_ERR_INVALID_ARG, "%s given without conv_w", "conv_b/conv_cache");
  }
  if (p->dt_rank1) {
    if (p->dt_dtype != SSM_F32) return fail(SSM_ERR_UNSUPPORTED, "%s: rank-1 dt input must be f32", "dt_dtype");
    if (!p->dt_w) return fail(SSM_ERR_INVALID_ARG, "%s is NULL with dt_rank1", "dt_w");
  }
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  const size_t Bt = p->batch, E = p->dim, N = p->d_state;
  if (Bt > 0) {
    if (!p->x || !p->y || !p->B || !p->C || !p->dt || !p->ssm_state)
      return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x/y/B/C/dt/ssm_state");
  }
  if (Bt * E > 0x7fffffffULL) return fail(SSM_ERR_UNSUPPORTED, "%s too large", "batch*dim");
  if (Bt > 0 && ((reinterpret_cast<uintptr_t>(p->ssm_state) | reinterpret_cast<uintptr_t>(p->A) |
                  reinterpret_cast<uintptr_t>(p->conv_w)) & 15))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "ssm_state/A/conv_w");
  if (Bt > 0 && ((reinterpret_cast<uintptr_t>(p->B) | reinterpret_cast<uintptr_t>(p->C)) & (p->bc_dtype == SSM_BF16 ? 7 : 15)))
    return fail(SSM_ERR_INVALID_ARG, "%s must be aligned to 4 elements", "B/C");
  const Range y{p->y, Bt * E * esize(p->y_dtype)};
  const Range ins[] = {
      {p->x, Bt * E * esize(p->x_dtype)},
      {p->z, p->z ? Bt * E * esize(p->z_dtype) : 0},
      {p->dt, p->dt_rank1 ? Bt * 4 : Bt * E * esize(p->dt_dtype)},
      {p->B, Bt * N * esize(p->bc_dtype)},
      {p->C, Bt * N * esize(p->bc_dtype)},
      {p->A, E * N * 4},
      {p->ssm_state, Bt * E * N * 4},
      {p->conv_cache, p->conv_cache ? Bt * E * 3 * 4 : 0},
  };
  for (const Range& r : ins)
    if (overlaps(y, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "y");
  return SSM_OK;
}

// ---------------------------------------------------------------- chunked SSD

// The tuned MFMA kernel takes N = 64, chunk_size = 128, bf16 x and B/C and a
// headdim that is a multiple of 16 up to 128; every other supported shape
// runs the vector-ALU chunked kernels of ssd_generic.hip.
bool chunk_tuned(const ssm_chunk_params_t* p) {
  return p->d_state == ssm::kSsdN && p->chunk_size == ssm::kSsdQ && p->x_dtype == SSM_BF16 &&
         p->bc_dtype == SSM_BF16 && p->headdim % 16 == 0 && p->headdim <= ssm::kSsdMaxP;
}

void chunk_plan(const ssm_chunk_params_t* p, ssm::ChunkGenericArgs& g, ssm::ChunkLaunch& l);
ssm_status_t debug_chunk(const ssm_chunk_params_t* p, const ssm::ChunkGenericArgs& g, const ssm::ChunkLaunch& l);

size_t chunk_ws(const ssm_chunk_params_t* p) {
  if (p->batch <= 0 || p->seqlen <= 0) return 0;
  if (!chunk_tuned(p))
    return ssm::chunk_generic_workspace_bytes(p->batch, p->seqlen, p->nheads, p->headdim, p->d_state,
                                              p->chunk_size);
  return ssm::chunk_workspace_bytes(p->batch, p->seqlen, p->nheads, p->headdim, p->segments);
}

ssm_status_t chunk_check(const ssm_chunk_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_chunk_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->ngroups <= 0 ||
      p->d_state <= 0 || p->chunk_size <= 0)
    return fail(SSM_ERR_INVALID_ARG, "%s: negative or zero size", "dims");
  if (p->nheads % p->ngroups != 0) return fail(SSM_ERR_INVALID_ARG, "%s", "nheads must be a multiple of ngroups");
  if (p->segments < 0 || p->segments > ssm::kSsdMaxSeg)
    return fail(SSM_ERR_INVALID_ARG, "%s must be in [0, 16]", "segments");
  if (p->d_state > ssm::kSsdGenMaxN) return fail(SSM_ERR_UNSUPPORTED, "%s must be at most 128", "d_state");
  if (p->chunk_size > ssm::kSsdGenMaxQ) return fail(SSM_ERR_UNSUPPORTED, "%s must be at most 256", "chunk_size");
  if (p->headdim > ssm::kSsdMaxP) return fail(SSM_ERR_UNSUPPORTED, "%s must be at most 128", "headdim");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->bc_dtype) || !valid_dtype(p->out_dtype))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/bc/out_dtype");
  if (p->z && !valid_dtype(p->z_dtype)) return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "z_dtype");
  // whole chunks are read through buffer descriptors of one batch row with
  // 32-bit byte offsets
  if (static_cast<unsigned long long>(p->seqlen) *
          std::max<unsigned long long>(static_cast<unsigned long long>(p->nheads) * p->headdim,
                                       static_cast<unsigned long long>(p->ngroups) * p->d_state) * 2ull >
      0xffffffffull)
    return fail(SSM_ERR_UNSUPPORTED, "%s", "one batch row of x, B or C must stay below 4 GiB (seqlen too long)");
  if (chunk_tuned(p) &&
      ((reinterpret_cast<uintptr_t>(p->x) | reinterpret_cast<uintptr_t>(p->B) | reinterpret_cast<uintptr_t>(p->C) |
        reinterpret_cast<uintptr_t>(p->out) | reinterpret_cast<uintptr_t>(p->z)) & 15))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "x/B/C/out/z");
  if (!chunk_tuned(p) &&
      ((reinterpret_cast<uintptr_t>(p->x) & (esize(p->x_dtype) - 1)) |
       (reinterpret_cast<uintptr_t>(p->B) & (esize(p->bc_dtype) - 1)) |
       (reinterpret_cast<uintptr_t>(p->C) & (esize(p->bc_dtype) - 1)) |
       (reinterpret_cast<uintptr_t>(p->out) & (esize(p->out_dtype) - 1)) |
       (p->z ? reinterpret_cast<uintptr_t>(p->z) & (esize(p->z_dtype) - 1) : 0)))
    return fail(SSM_ERR_INVALID_ARG, "%s must be aligned to their element size", "x/B/C/out/z");
  if (!p->A) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "A");
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  const size_t Bt = p->batch, L = p->seqlen, H = p->nheads, P = p->headdim, G = p->ngroups, N = p->d_state;
  const size_t tok = Bt * L;
  if (tok > 0 && (!p->x || !p->out || !p->B || !p->C || !p->dt))
    return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x/out/B/C/dt");
  const Range out{p->out, tok * H * P * esize(p->out_dtype)};
  const Range ins[] = {
      {p->x, tok * H * P * esize(p->x_dtype)},
      {p->dt, tok * H * 4},
      {p->B, tok * G * N * esize(p->bc_dtype)},
      {p->C, tok * G * N * esize(p->bc_dtype)},
      {p->A, H * 4},
      {p->D, p->D ? (p->d_per_channel ? H * P * 4 : H * 4) : 0},
      {p->dt_bias, p->dt_bias ? H * 4 : 0},
      {p->state_in, p->state_in ? Bt * H * P * N * 4 : 0},
      {p->state_out, p->state_out ? Bt * H * P * N * 4 : 0},
      {p->workspace, p->workspace_bytes},
      {p->z, p->z ? tok * H * P * esize(p->z_dtype) : 0},
  };
  for (const Range& r : ins)
    if (overlaps(out, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "out");
  if (p->state_out && p->state_out != p->state_in &&
      overlaps({p->state_out, Bt * H * P * N * 4}, {p->state_in, p->state_in ? Bt * H * P * N * 4 : 0}))
    return fail(SSM_ERR_INVALID_ARG, "%s partially overlaps state_in", "state_out");
  const size_t need = chunk_ws(p);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(SSM_ERR_WORKSPACE, "%s is missing or smaller than ssm_chunk_scan_workspace_size()", "workspace");
  if (p->workspace && (reinterpret_cast<uintptr_t>(p->workspace) & 255))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 256-byte aligned", "workspace");
  return SSM_OK;
}

// ---------------------------------------------------------------- SSD decode

ssm_status_t chunk_decode_check(const ssm_chunk_decode_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_chunk_decode_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->batch < 0 || p->nheads <= 0 || p->headdim <= 0 || p->ngroups <= 0 || p->d_state <= 0)
    return fail(SSM_ERR_INVALID_ARG, "%s: negative or zero size", "dims");
  if (p->nheads % p->ngroups != 0) return fail(SSM_ERR_INVALID_ARG, "%s", "nheads must be a multiple of ngroups");
  if (p->d_state != 16 && p->d_state != 32 && p->d_state != 64 && p->d_state != 128)
    return fail(SSM_ERR_UNSUPPORTED, "%s must be 16, 32, 64 or 128", "d_state");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->bc_dtype) || !valid_dtype(p->out_dtype) ||
      (p->z && !valid_dtype(p->z_dtype)))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/bc/out/z_dtype");
  if (!p->A) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "A");
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  const size_t Bt = p->batch, H = p->nheads, P = p->headdim, G = p->ngroups, N = p->d_state;
  const size_t rows = Bt * H * P;
  if (rows > 0x7fffffffULL) return fail(SSM_ERR_UNSUPPORTED, "%s too large", "batch*nheads*headdim");
  if (Bt == 0) return SSM_OK;
  if (!p->x || !p->out || !p->B || !p->C || !p->dt || !p->state)
    return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x/out/B/C/dt/state");
  if (reinterpret_cast<uintptr_t>(p->state) & 15)
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "state");
  if ((reinterpret_cast<uintptr_t>(p->B) | reinterpret_cast<uintptr_t>(p->C)) & (p->bc_dtype == SSM_BF16 ? 15 : 31))
    return fail(SSM_ERR_INVALID_ARG, "%s must be aligned to 8 elements", "B/C");
  const Range out{p->out, rows * esize(p->out_dtype)};
  const Range ins[] = {
      {p->x, rows * esize(p->x_dtype)},
      {p->dt, Bt * H * 4},
      {p->dt_bias, p->dt_bias ? H * 4 : 0},
      {p->A, H * 4},
      {p->B, Bt * G * N * esize(p->bc_dtype)},
      {p->C, Bt * G * N * esize(p->bc_dtype)},
      {p->D, p->D ? (p->d_per_channel ? H * P * 4 : H * 4) : 0},
      {p->z, p->z ? rows * esize(p->z_dtype) : 0},
      {p->state, rows * N * 4},
  };
  for (const Range& r : ins)
    if (overlaps(out, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "out");
  return SSM_OK;
}

// ---------------------------------------------------------------- projections

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

ssm_status_t linear_check(const ssm_linear_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_linear_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->rows < 0 || p->in_features <= 0 || p->out_features <= 0)
    return fail(SSM_ERR_INVALID_ARG, "%s: negative or zero size", "rows/in_features/out_features");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->out_dtype))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/out_dtype");
  if (p->in_features % 8 != 0) return fail(SSM_ERR_UNSUPPORTED, "%s must be a multiple of 8", "in_features");
  if (p->out_features % 4 != 0) return fail(SSM_ERR_UNSUPPORTED, "%s must be a multiple of 4", "out_features");
  if (p->rows == 0) return SSM_OK;
  if (!p->x || !p->weight || !p->out) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x/weight/out");
  if (!aligned16(p->x) || !aligned16(p->weight) || !aligned16(p->out))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "x/weight/out");
  const size_t M = p->rows, K = p->in_features, N = p->out_features;
  const Range out{p->out, M * N * esize(p->out_dtype)};
  if (overlaps(out, {p->x, M * K * esize(p->x_dtype)}) || overlaps(out, {p->weight, N * K * 2}))
    return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "out");
  if (p->workspace) {
    if (reinterpret_cast<uintptr_t>(p->workspace) & 255)
      return fail(SSM_ERR_INVALID_ARG, "%s must be 256-byte aligned", "workspace");
    const Range ws{p->workspace, p->workspace_bytes};
    if (overlaps(ws, out) || overlaps(ws, {p->x, M * K * esize(p->x_dtype)}) || overlaps(ws, {p->weight, N * K * 2}))
      return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "workspace");
  }
  const size_t need = ssm::gemm_workspace_bytes(p->rows, p->out_features, p->in_features, p->x_dtype);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(SSM_ERR_WORKSPACE, "%s is missing or smaller than ssm_linear_workspace_size()", "workspace");
  return SSM_OK;
}

// ---------------------------------------------------------------- layer

// The layer's workspace: activations between the steps, then the scratch of
// the scan and of the projections (each piece 256-byte aligned).
struct LayerWs {
  size_t x, z, y, part, B, C, r, scan, gemm, total;
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// The scan step of the layer as an ssm_scan_fwd call on the workspace's
// activations (x_branch, z, B, C, dt_raw and y in fp32).
ssm_scan_params_t layer_scan_params(const ssm_layer_params_t* p, char* ws, const LayerWs& o) {
  ssm_scan_params_t sp{};
  sp.struct_size = sizeof(ssm_scan_params_t);
  sp.batch = p->batch;
  sp.seqlen = p->seqlen;
  sp.dim = p->dim;
  sp.d_state = p->d_state;
  sp.conv_k = p->conv_k;
  sp.x = ws ? ws + o.x : nullptr;
  sp.x_dtype = SSM_F32;
  sp.conv_w = p->conv_w;
  sp.conv_b = p->conv_b;
  sp.conv_cache_in = p->conv_cache_in;
  sp.conv_cache_out = p->conv_cache_out;
  sp.dt = ws ? ws + o.r : nullptr;
  sp.dt_dtype = SSM_F32;
  sp.dt_rank1 = 1;
  sp.dt_w = p->dt_w;
  sp.dt_bias = p->dt_bias;
  sp.dt_softplus = p->dt_softplus;
  sp.dt_min = p->dt_min;
  sp.dt_max = p->dt_max;
  sp.A = p->A;
  sp.B = ws ? ws + o.B : nullptr;
  sp.C = ws ? ws + o.C : nullptr;
  sp.bc_dtype = SSM_F32;
  sp.D = p->D;
  sp.z = ws ? ws + o.z : nullptr;
  sp.z_dtype = SSM_F32;
  sp.ssm_state_in = p->ssm_state_in;
  sp.ssm_state_out = p->ssm_state_out;
  sp.y = ws ? ws + o.y : nullptr;
  sp.y_dtype = SSM_F32;
  sp.time_split = 0;
  sp.workspace = ws ? ws + o.scan : nullptr;
  sp.workspace_bytes = o.gemm - o.scan;
  return sp;
}

LayerWs layer_ws(const ssm_layer_params_t* p) {
  LayerWs o{};
  const size_t T = static_cast<size_t>(p->batch) * p->seqlen, E = p->dim, N = p->d_state, Dm = p->d_model;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  o.x = take(T * E * 4);
  o.z = take(T * E * 4);
  o.y = take(T * E * 4);
  o.part = take(T > 0 ? ssm::xproj_partial_bytes(static_cast<int>(T), p->dim) : 0);
  o.B = take(T * N * 4);
  o.C = take(T * N * 4);
  o.r = take(T * 4);
  o.scan = off;
  ssm_scan_params_t sp = layer_scan_params(p, nullptr, o);
  off += align256(T > 0 ? ssm_scan_workspace_size(&sp) : 0);
  o.gemm = off;
  size_t g = 0;
  if (T > 0) {
    g = std::max(ssm::gemm_workspace_bytes(static_cast<int>(T), static_cast<int>(2 * E), static_cast<int>(Dm), SSM_BF16),
                 ssm::gemm_workspace_bytes(static_cast<int>(T), static_cast<int>(Dm), static_cast<int>(E), SSM_F32));
  }
  off += align256(g);
  o.total = off;
  return o;
}

ssm_status_t layer_check(const ssm_layer_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_layer_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->batch < 0 || p->seqlen < 0 || p->d_model <= 0 || p->dim <= 0 || p->d_state <= 0)
    return fail(SSM_ERR_INVALID_ARG, "%s: negative or zero size", "dims");
  if (p->d_state != ssm::kScanN) return fail(SSM_ERR_UNSUPPORTED, "%s must be 16", "d_state");
  if (p->conv_k != ssm::kConvK) return fail(SSM_ERR_UNSUPPORTED, "%s must be 4", "conv_k");
  if (p->dim % 256 != 0) return fail(SSM_ERR_UNSUPPORTED, "%s must be a multiple of 256", "dim");
  if (p->d_model % 8 != 0) return fail(SSM_ERR_UNSUPPORTED, "%s must be a multiple of 8", "d_model");
  if (!valid_dtype(p->hidden_dtype) || !valid_dtype(p->out_dtype))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "hidden/out_dtype");
  if (!p->w_in || !p->conv_w || !p->w_x || !p->dt_w || !p->A || !p->w_out)
    return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "w_in/conv_w/w_x/dt_w/A/w_out");
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  if (!aligned16(p->w_in) || !aligned16(p->conv_w) || !aligned16(p->w_x) || !aligned16(p->A) || !aligned16(p->w_out))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "weights/conv_w/A");
  const size_t T = static_cast<size_t>(p->batch) * p->seqlen;
  if (T == 0) return SSM_OK;
  if (T * static_cast<size_t>(p->dim) > 0x7fffffffULL)
    return fail(SSM_ERR_UNSUPPORTED, "%s too large", "batch*seqlen*dim");
  if (!p->hidden || !p->out) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "hidden/out");
  if (!aligned16(p->hidden) || !aligned16(p->out))
    return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "hidden/out");
  const size_t E = p->dim, N = p->d_state, Dm = p->d_model;
  const Range out{p->out, T * Dm * esize(p->out_dtype)};
  const Range ins[] = {
      {p->hidden, T * Dm * esize(p->hidden_dtype)}, {p->w_in, 2 * E * Dm * 2}, {p->conv_w, E * 4 * 4},
      {p->conv_b, p->conv_b ? E * 4 : 0},          {p->w_x, (2 * N + 1) * E * 2}, {p->dt_w, E * 4},
      {p->dt_bias, p->dt_bias ? E * 4 : 0},        {p->A, E * N * 4},        {p->D, p->D ? E * 4 : 0},
      {p->w_out, Dm * E * 2},
      {p->conv_cache_in, p->conv_cache_in ? p->batch * E * 3 * 4 : 0},
      {p->conv_cache_out, p->conv_cache_out ? p->batch * E * 3 * 4 : 0},
      {p->ssm_state_in, p->ssm_state_in ? p->batch * E * N * 4 : 0},
      {p->ssm_state_out, p->ssm_state_out ? p->batch * E * N * 4 : 0},
  };
  for (const Range& r : ins)
    if (overlaps(out, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "out");
  const LayerWs o = layer_ws(p);
  if (!p->workspace || p->workspace_bytes < o.total)
    return fail(SSM_ERR_WORKSPACE, "%s is missing or smaller than ssm_layer_workspace_size()", "workspace");
  if (reinterpret_cast<uintptr_t>(p->workspace) & 255)
    return fail(SSM_ERR_INVALID_ARG, "%s must be 256-byte aligned", "workspace");
  const Range ws{p->workspace, o.total};
  if (overlaps(ws, out)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "workspace");
  for (const Range& r : ins)
    if (overlaps(ws, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "workspace");
  // the scan step's own constraints (cache/state aliasing and alignment)
  char* wsp = static_cast<char*>(p->workspace);
  ssm_scan_params_t sp = layer_scan_params(p, wsp, o);
  return scan_check(&sp);
}

// ---------------------------------------------------------------- scan backward

struct BwdWs {
  size_t hs, qs, sdt, xb, pB, pC, pr, pe, total;
};

BwdWs bwd_ws(const ssm_scan_bwd_params_t* p) {
  BwdWs o{};
  const size_t Bt = p->batch, L = p->seqlen, E = p->dim, N = ssm::kScanN;
  const size_t S = L > 0 ? ssm::bwd_segments(p->seqlen) : 0, R = ssm::bwd_runs(static_cast<int>(S));
  const size_t G = ssm::bwd_blocks64(p->dim);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  o.hs = take(Bt * S * E * N * 4);
  o.qs = take(Bt * S * E * N * 4);
  o.sdt = take(Bt * S * E * 4);
  o.xb = take(p->conv_w ? Bt * R * 3 * E * 4 : 0);
  o.pB = take(Bt * L * G * N * 4);
  o.pC = take(Bt * L * G * N * 4);
  o.pr = take(p->dt_rank1 ? Bt * L * G * 4 : 0);
  o.pe = take(Bt * R * E * ssm::kBwdPe * 4);
  o.total = off;
  return o;
}

void bwd_plan(const ssm_scan_bwd_params_t* p, ssm::BwdArgs& a);
ssm_status_t debug_bwd(const ssm_scan_bwd_params_t* p, const ssm::BwdArgs& a);

ssm_status_t bwd_check(const ssm_scan_bwd_params_t* p) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_scan_bwd_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->batch < 0 || p->seqlen < 0 || p->dim <= 0) return fail(SSM_ERR_INVALID_ARG, "%s: negative size or dim <= 0", "dims");
  if (p->d_state != ssm::kScanN) return fail(SSM_ERR_UNSUPPORTED, "%s must be 16", "d_state");
  if (!valid_dtype(p->x_dtype) || !valid_dtype(p->bc_dtype) || !valid_dtype(p->dt_dtype) ||
      !valid_dtype(p->dy_dtype) || (p->z && !valid_dtype(p->z_dtype)))
    return fail(SSM_ERR_INVALID_ARG, "%s: unknown dtype", "x/bc/dt/dy/z_dtype");
  if (p->z && p->z_dtype != p->x_dtype) return fail(SSM_ERR_UNSUPPORTED, "%s must equal x_dtype", "z_dtype");
  if (!p->A) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "A");
  if (p->conv_w) {
    if (p->conv_k != ssm::kConvK) return fail(SSM_ERR_UNSUPPORTED, "%s must be 4", "conv_k");
    if (!aligned16(p->conv_w)) return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "conv_w");
  } else if (p->conv_b || p->conv_cache_in || p->dconv_w || p->dconv_b || p->dconv_cache) {
    return fail(SSM_ERR_INVALID_ARG, "%s given without conv_w", "conv_b/conv_cache_in/dconv_*");
  }
  if (p->dt_rank1) {
    if (p->dt_dtype != SSM_F32) return fail(SSM_ERR_UNSUPPORTED, "%s: rank-1 dt input must be f32", "dt_dtype");
    if (!p->dt_w) return fail(SSM_ERR_INVALID_ARG, "%s is NULL with dt_rank1", "dt_w");
  } else if (p->ddt_w) {
    return fail(SSM_ERR_INVALID_ARG, "%s needs a rank-1 dt", "ddt_w");
  }
  if (p->dz && !p->z) return fail(SSM_ERR_INVALID_ARG, "%s given without z", "dz");
  ssm_status_t s = check_dt_bounds(p->dt_min, p->dt_max);
  if (s != SSM_OK) return s;
  const size_t Bt = p->batch, L = p->seqlen, E = p->dim, N = ssm::kScanN;
  if (Bt * L * E > 0x7fffffffULL) return fail(SSM_ERR_UNSUPPORTED, "%s too large", "batch*seqlen*dim");
  if (Bt * L == 0) return SSM_OK;
  if (!p->x || !p->B || !p->C || !p->dt || !p->dy) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "x/B/C/dt/dy");
  if (!aligned16(p->A)) return fail(SSM_ERR_INVALID_ARG, "%s must be 16-byte aligned", "A");
  if ((reinterpret_cast<uintptr_t>(p->B) | reinterpret_cast<uintptr_t>(p->C)) & (p->bc_dtype == SSM_BF16 ? 7 : 15))
    return fail(SSM_ERR_INVALID_ARG, "%s must be aligned to 4 elements", "B/C");
  const size_t xe = esize(p->x_dtype);
  const Range ins[] = {
      {p->x, Bt * L * E * xe},
      {p->z, p->z ? Bt * L * E * xe : 0},
      {p->dt, p->dt_rank1 ? Bt * L * 4 : Bt * L * E * esize(p->dt_dtype)},
      {p->dy, Bt * L * E * esize(p->dy_dtype)},
      {p->B, Bt * L * N * esize(p->bc_dtype)},
      {p->C, Bt * L * N * esize(p->bc_dtype)},
      {p->A, E * N * 4},
      {p->ssm_state_in, p->ssm_state_in ? Bt * E * N * 4 : 0},
      {p->dstate_out, p->dstate_out ? Bt * E * N * 4 : 0},
      {p->conv_cache_in, p->conv_cache_in ? Bt * E * 3 * 4 : 0},
  };
  const Range outs[] = {
      {p->dx, p->dx ? Bt * L * E * 4 : 0},        {p->dz, p->dz ? Bt * L * E * 4 : 0},
      {p->ddt, p->ddt ? (p->dt_rank1 ? Bt * L * 4 : Bt * L * E * 4) : 0},
      {p->ddt_w, p->ddt_w ? E * 4 : 0},           {p->ddt_bias, p->ddt_bias ? E * 4 : 0},
      {p->dA, p->dA ? E * N * 4 : 0},             {p->dB, p->dB ? Bt * L * N * 4 : 0},
      {p->dC, p->dC ? Bt * L * N * 4 : 0},        {p->dD, p->dD ? E * 4 : 0},
      {p->dconv_w, p->dconv_w ? E * 4 * 4 : 0},   {p->dconv_b, p->dconv_b ? E * 4 : 0},
      {p->dconv_cache, p->dconv_cache ? Bt * E * 3 * 4 : 0},
      {p->dstate_in, p->dstate_in ? Bt * E * N * 4 : 0},
  };
  const size_t n_out = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < n_out; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps an input", "a gradient output");
    for (size_t j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return fail(SSM_ERR_INVALID_ARG, "%s overlap each other", "gradient outputs");
  }
  const BwdWs o = bwd_ws(p);
  if (!p->workspace || p->workspace_bytes < o.total)
    return fail(SSM_ERR_WORKSPACE, "%s is missing or smaller than ssm_scan_bwd_workspace_size()", "workspace");
  if (reinterpret_cast<uintptr_t>(p->workspace) & 255)
    return fail(SSM_ERR_INVALID_ARG, "%s must be 256-byte aligned", "workspace");
  const Range ws{p->workspace, o.total};
  for (const Range& r : ins)
    if (overlaps(ws, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "workspace");
  for (const Range& r : outs)
    if (overlaps(ws, r)) return fail(SSM_ERR_INVALID_ARG, "%s overlaps another tensor", "workspace");
  return SSM_OK;
}

ssm_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(SSM_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
}

}  // namespace

namespace ssm {
TimingEvents timing_events() { return g_timing; }
static_assert(kScanScratchBytes == SSM_SCAN_NOALLOC_MAX_BYTES, "scratch size in the header and the library differ");
}  // namespace ssm

extern "C" {

ssm_status_t ssm_scan_check(const ssm_scan_params_t* p) {
  const ssm_status_t s = scan_check(p);
  return s == SSM_OK ? ok() : s;
}

size_t ssm_scan_workspace_size(const ssm_scan_params_t* p) {
  if (!p || p->struct_size != sizeof(ssm_scan_params_t)) return 0;
  return scan_ws(p);
}

}  // extern "C"

namespace {

// The launch plan of a validated scan call (its workspace already in place).
void scan_plan(const ssm_scan_params_t* p, ssm::ScanLaunch& l) {
  l = ssm::ScanLaunch{};
  ssm::ScanKernelArgs& k = l.k;
  k.x = p->x;
  k.z = p->z;
  k.dt = p->dt;
  k.y = p->y;
  k.bc = static_cast<const float*>(p->workspace);
  k.A = p->A;
  k.D = p->D;
  k.dt_w = p->dt_rank1 ? p->dt_w : nullptr;
  k.dt_bias = p->dt_bias;
  k.conv_w = p->conv_w;
  k.conv_b = p->conv_b;
  k.conv_cache_in = p->conv_cache_in;
  k.conv_cache_out = p->conv_cache_out;
  k.state_in = p->ssm_state_in;
  k.state_out = p->ssm_state_out;
  k.batch = p->batch;
  k.seqlen = p->seqlen;
  k.dim = p->dim;
  k.n_egroups = (p->dim + 63) / 64;
  k.nseg = scan_split(p);
  k.seg_len = p->seqlen > 0 ? (k.nseg > 1 ? scan_seg_len(p->seqlen, k.nseg) : p->seqlen) : 0;
  k.summ = k.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(p->workspace) +
                                                 ssm::scan_summary_offset(p->batch, p->seqlen))
                      : nullptr;
  k.head = k.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(p->workspace) +
                                                 ssm::scan_head_offset(p->batch, p->seqlen, p->dim, k.nseg))
                      : nullptr;
  k.dt_min = p->dt_min;
  k.dt_max = p->dt_max;
  softplus_thresholds(p->dt_min, p->dt_max, &k.sp_lo, &k.sp_hi);
  k.dt_softplus = p->dt_softplus ? 1 : 0;
  k.has_z = p->z ? 1 : 0;
  const ssm::ScanLaunch v = scan_variant(p);
  l.x_dtype = v.x_dtype;
  l.y_dtype = v.y_dtype;
  l.bc_dtype = v.bc_dtype;
  l.dt_mode = v.dt_mode;
  l.conv = v.conv;
  l.zoh = v.zoh;
  l.B = p->B;
  l.C = p->C;
  l.bc_out = static_cast<float*>(p->workspace);
  // the scaled-state form needs a finite upper clip (its rescaling factors are
  // powers of exp(dt_max A)); the kernels also check, per wave, that A is the
  // same in every channel and that the factors stay in range
  if (p->discretization == SSM_EULER && std::isfinite(p->dt_max) && p->seqlen > 0 && p->batch > 0) {
    char* ws = static_cast<char*>(p->workspace);
    l.bcg_out = reinterpret_cast<float*>(ws + ssm::scan_bcg_offset(p->batch, p->seqlen));
    l.qtab_out = reinterpret_cast<float*>(ws + ssm::scan_qtab_offset(p->batch, p->seqlen));
  }
  k.bcg = l.bcg_out;
  k.qtab = l.qtab_out;
}

// The launch plan of a validated call of the blocked kernel.
void scan_blk_plan(const ssm_scan_params_t* p, ssm::ScanBlkLaunch& l) {
  l = ssm::ScanBlkLaunch{};
  ssm::ScanBlkArgs& k = l.k;
  k.x = static_cast<const uint16_t*>(p->x);
  k.z = static_cast<const uint16_t*>(p->z);
  k.dt = static_cast<const uint16_t*>(p->dt);
  k.y = p->y;
  char* ws = static_cast<char*>(p->workspace);
  l.rec_out = reinterpret_cast<unsigned char*>(ws);
  l.qv_out = reinterpret_cast<float*>(ws + ssm::scan_blk_qv_offset(p->batch, p->seqlen));
  k.rec = l.rec_out;
  k.qv = l.qv_out;
  k.A = p->A;
  k.D = p->D;
  k.dt_bias = p->dt_bias;
  k.state_in = p->ssm_state_in;
  k.state_out = p->ssm_state_out;
  k.batch = p->batch;
  k.seqlen = p->seqlen;
  k.dim = p->dim;
  k.nrec = ssm::scan_blk_records(p->seqlen);
  k.dt_min = p->dt_min;
  k.dt_max = p->dt_max;
  softplus_thresholds(p->dt_min, p->dt_max, &k.sp_lo, &k.sp_hi);
  k.dt_softplus = p->dt_softplus ? 1 : 0;
  l.y_dtype = p->y_dtype;
  l.bc_dtype = p->bc_dtype;
  l.B = p->B;
  l.C = p->C;
}

ssm_status_t debug_scan(const ssm_scan_params_t* p, const ssm::ScanLaunch& l);
ssm_status_t debug_scan_blk(const ssm_scan_params_t* p, const ssm::ScanBlkLaunch& l);

// The launch of a validated scan call (its workspace already in place).
ssm_status_t scan_launch(const ssm_scan_params_t* p, void* stream) {
  if (scan_blocked(p)) {
    ssm::ScanBlkLaunch bl;
    scan_blk_plan(p, bl);
    const ssm_status_t d = debug_scan_blk(p, bl);
    if (d != SSM_OK) return d;
    return hip_status(ssm::launch_scan_blocked(bl, static_cast<hipStream_t>(stream)));
  }
  ssm::ScanLaunch l;
  scan_plan(p, l);
  const ssm_status_t d = debug_scan(p, l);
  if (d != SSM_OK) return d;
  if (p->batch == 0) return ok();
  return hip_status(ssm::launch_scan(l, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ssm_status_t ssm_scan_fwd(const ssm_scan_params_t* p, void* stream) {
  const ssm_status_t s = scan_check(p);
  if (s != SSM_OK) return s;
  return scan_launch(p, stream);
}

ssm_status_t ssm_scan_fwd_noalloc(const ssm_scan_params_t* p, void* stream) {
  if (!p) return fail(SSM_ERR_INVALID_ARG, "%s is NULL", "params");
  if (p->struct_size != sizeof(ssm_scan_params_t))
    return fail(SSM_ERR_INVALID_ARG, "%s does not match this library", "struct_size");
  if (p->workspace || p->workspace_bytes)
    return fail(SSM_ERR_INVALID_ARG, "%s must be NULL and 0: this entry point uses the library's own scratch",
                "workspace/workspace_bytes");
  // sizes first, so a request past the scratch fails before the device is touched
  if (p->batch >= 0 && p->seqlen >= 0 && p->dim > 0 && p->d_state == ssm::kScanN &&
      p->time_split >= SSM_SCAN_BLOCKED && p->time_split <= ssm::kScanMaxSplit) {
    const size_t need = scan_ws(p);
    if (need > ssm::kScanScratchBytes) {
      char buf[192];
      std::snprintf(buf, sizeof(buf), "needs %zu bytes of scratch; ssm_scan_fwd_noalloc holds at most %zu",
                    need, static_cast<size_t>(ssm::kScanScratchBytes));
      return fail(SSM_ERR_WORKSPACE, "%s", buf);
    }
  }
  void* scratch = nullptr;
  const hipError_t e = ssm::scan_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e);
  ssm_scan_params_t q = *p;
  q.workspace = scratch;
  q.workspace_bytes = ssm::kScanScratchBytes;
  const ssm_status_t s = scan_check(&q);
  if (s != SSM_OK) return s;
  return scan_launch(&q, stream);
}

ssm_status_t ssm_decode_check(const ssm_decode_params_t* p) {
  const ssm_status_t s = decode_check(p);
  return s == SSM_OK ? ok() : s;
}

ssm_status_t ssm_decode_step(const ssm_decode_params_t* p, void* stream) {
  const ssm_status_t s = decode_check(p);
  if (s != SSM_OK) return s;
  if (p->batch == 0) return ok();
  ssm::DecodeLaunch l{};
  ssm::DecodeKernelArgs& k = l.k;
  k.x = p->x;
  k.z = p->z;
  k.dt = p->dt;
  k.B = p->B;
  k.C = p->C;
  k.y = p->y;
  k.A = p->A;
  k.D = p->D;
  k.dt_w = p->dt_rank1 ? p->dt_w : nullptr;
  k.dt_bias = p->dt_bias;
  k.conv_w = p->conv_w;
  k.conv_b = p->conv_b;
  k.conv_cache = p->conv_cache;
  k.state = p->ssm_state;
  k.batch = p->batch;
  k.dim = p->dim;
  k.dt_min = p->dt_min;
  k.dt_max = p->dt_max;
  softplus_thresholds(p->dt_min, p->dt_max, &k.sp_lo, &k.sp_hi);
  k.dt_softplus = p->dt_softplus ? 1 : 0;
  k.has_z = p->z ? 1 : 0;
  l.x_dtype = p->x_dtype;
  l.y_dtype = p->y_dtype;
  l.bc_dtype = p->bc_dtype;
  l.dt_mode = p->dt_rank1 ? 0 : (p->dt_dtype == SSM_BF16 ? 2 : 1);
  l.conv = p->conv_w != nullptr;
  l.zoh = p->discretization == SSM_ZOH;
  return hip_status(ssm::launch_decode(l, static_cast<hipStream_t>(stream)));
}

ssm_status_t ssm_chunk_scan_check(const ssm_chunk_params_t* p) {
  const ssm_status_t s = chunk_check(p);
  return s == SSM_OK ? ok() : s;
}

size_t ssm_chunk_scan_workspace_size(const ssm_chunk_params_t* p) {
  if (!p || p->struct_size != sizeof(ssm_chunk_params_t)) return 0;
  if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->ngroups <= 0) return 0;
  return chunk_ws(p);
}

ssm_status_t ssm_chunk_scan_fwd(const ssm_chunk_params_t* p, void* stream) {
  const ssm_status_t s = chunk_check(p);
  if (s != SSM_OK) return s;
  if (p->batch == 0) return ok();
  ssm::ChunkGenericArgs g{};
  ssm::ChunkLaunch l{};
  chunk_plan(p, g, l);
  const ssm_status_t d = debug_chunk(p, g, l);
  if (d != SSM_OK) return d;
  if (!chunk_tuned(p)) return hip_status(ssm::launch_chunk_generic(g, static_cast<hipStream_t>(stream)));
  return hip_status(ssm::launch_chunk(l, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The launch plan of a validated chunked-scan call: g for the vector-ALU path,
// l for the tuned matrix-core one (the one chunk_tuned(p) picks is filled).
void chunk_plan(const ssm_chunk_params_t* p, ssm::ChunkGenericArgs& g, ssm::ChunkLaunch& l) {
  if (!chunk_tuned(p)) {
    g.x = p->x;
    g.dt = p->dt;
    g.dt_bias = p->dt_bias;
    g.A = p->A;
    g.B = p->B;
    g.C = p->C;
    g.D = p->D;
    g.state_in = p->state_in;
    g.state_out = p->state_out;
    g.out = p->out;
    g.z = p->z;
    g.chunk_state = static_cast<float*>(p->workspace);
    g.chunk_decay = reinterpret_cast<float*>(static_cast<char*>(p->workspace) +
                                             ssm::chunk_generic_decay_offset(p->batch, p->seqlen, p->nheads,
                                                                             p->headdim, p->d_state, p->chunk_size));
    g.batch = p->batch;
    g.seqlen = p->seqlen;
    g.nheads = p->nheads;
    g.headdim = p->headdim;
    g.ngroups = p->ngroups;
    g.d_state = p->d_state;
    g.chunk_size = p->chunk_size;
    g.nchunks = (p->seqlen + p->chunk_size - 1) / p->chunk_size;
    g.d_per_channel = p->d_per_channel ? 1 : 0;
    g.x_bf16 = p->x_dtype == SSM_BF16;
    g.bc_bf16 = p->bc_dtype == SSM_BF16;
    g.z_bf16 = p->z && p->z_dtype == SSM_BF16;
    g.out_bf16 = p->out_dtype == SSM_BF16;
    g.dt_softplus = p->dt_softplus ? 1 : 0;
    g.dt_min = p->dt_min;
    g.dt_max = p->dt_max;
    softplus_thresholds(p->dt_min, p->dt_max, &g.sp_lo, &g.sp_hi);
    return;
  }
  ssm::ChunkKernelArgs& k = l.k;
  k.x = p->x;
  k.dt = p->dt;
  k.dt_bias = p->dt_bias;
  k.A = p->A;
  k.B = p->B;
  k.C = p->C;
  k.D = p->D;
  k.state_in = p->state_in;
  k.state_out = p->state_out;
  k.out = p->out;
  k.ws = static_cast<float*>(p->workspace);
  k.batch = p->batch;
  k.seqlen = p->seqlen;
  k.nheads = p->nheads;
  k.headdim = p->headdim;
  k.ngroups = p->ngroups;
  k.nchunks = (p->seqlen + p->chunk_size - 1) / p->chunk_size;
  const ssm::ChunkSplit sp = ssm::chunk_split(p->batch, p->seqlen, p->nheads, p->headdim, p->segments);
  k.nseg = sp.nseg;
  k.cps = sp.cps;
  k.ppseg = sp.ppseg;
  k.z = p->z;
  k.z_bf16 = p->z && p->z_dtype == SSM_BF16 ? 1 : 0;
  k.d_per_channel = p->d_per_channel ? 1 : 0;
  k.dt_min = p->dt_min;
  k.dt_max = p->dt_max;
  softplus_thresholds(p->dt_min, p->dt_max, &k.sp_lo, &k.sp_hi);
  k.dt_softplus = p->dt_softplus ? 1 : 0;
  l.x_dtype = p->x_dtype;
  l.bc_dtype = p->bc_dtype;
  l.out_dtype = p->out_dtype;
}

}  // namespace

extern "C" {

ssm_status_t ssm_chunk_decode_check(const ssm_chunk_decode_params_t* p) {
  const ssm_status_t s = chunk_decode_check(p);
  return s == SSM_OK ? ok() : s;
}

ssm_status_t ssm_chunk_decode_step(const ssm_chunk_decode_params_t* p, void* stream) {
  const ssm_status_t s = chunk_decode_check(p);
  if (s != SSM_OK) return s;
  if (p->batch == 0) return ok();
  ssm::ChunkDecodeLaunch l{};
  ssm::ChunkDecodeKernelArgs& k = l.k;
  k.x = p->x;
  k.dt = p->dt;
  k.dt_bias = p->dt_bias;
  k.A = p->A;
  k.B = p->B;
  k.C = p->C;
  k.D = p->D;
  k.z = p->z;
  k.state = p->state;
  k.out = p->out;
  k.rows = static_cast<unsigned>(static_cast<size_t>(p->batch) * p->nheads * p->headdim);
  k.nheads = p->nheads;
  k.headdim = p->headdim;
  k.ngroups = p->ngroups;
  k.heads_per_group = p->nheads / p->ngroups;
  k.d_per_channel = p->d_per_channel ? 1 : 0;
  k.z_bf16 = p->z && p->z_dtype == SSM_BF16 ? 1 : 0;
  k.dt_min = p->dt_min;
  k.dt_max = p->dt_max;
  softplus_thresholds(p->dt_min, p->dt_max, &k.sp_lo, &k.sp_hi);
  k.dt_softplus = p->dt_softplus ? 1 : 0;
  l.x_dtype = p->x_dtype;
  l.bc_dtype = p->bc_dtype;
  l.out_dtype = p->out_dtype;
  l.d_state = p->d_state;
  return hip_status(ssm::launch_chunk_decode(l, static_cast<hipStream_t>(stream)));
}

ssm_status_t ssm_linear_check(const ssm_linear_params_t* p) {
  const ssm_status_t s = linear_check(p);
  return s == SSM_OK ? ok() : s;
}

ssm_status_t ssm_linear_fwd(const ssm_linear_params_t* p, void* stream) {
  const ssm_status_t s = linear_check(p);
  if (s != SSM_OK) return s;
  if (p->rows == 0) return ok();
  ssm::GemmArgs g{};
  g.A = p->x;
  g.W = static_cast<const uint16_t*>(p->weight);
  g.C0 = p->out;
  g.C1 = nullptr;
  g.lda = p->in_features;
  g.ldw = p->in_features;
  g.ldc0 = g.ldc1 = p->out_features;
  g.M = p->rows;
  g.N = p->out_features;
  g.K = p->in_features;
  g.n_split = p->out_features;
  g.ws = static_cast<float*>(p->workspace);
  g.ws_bytes = p->workspace ? p->workspace_bytes : 0;
  return hip_status(ssm::launch_gemm(g, p->x_dtype, p->out_dtype, static_cast<hipStream_t>(stream)));
}

size_t ssm_linear_workspace_size(const ssm_linear_params_t* p) {
  if (!p || p->struct_size != sizeof(ssm_linear_params_t)) return 0;
  if (p->rows <= 0 || p->in_features <= 0 || p->out_features <= 0) return 0;
  return ssm::gemm_workspace_bytes(p->rows, p->out_features, p->in_features, p->x_dtype);
}

ssm_status_t ssm_layer_check(const ssm_layer_params_t* p) {
  const ssm_status_t s = layer_check(p);
  return s == SSM_OK ? ok() : s;
}

size_t ssm_layer_workspace_size(const ssm_layer_params_t* p) {
  if (!p || p->struct_size != sizeof(ssm_layer_params_t)) return 0;
  if (p->batch < 0 || p->seqlen < 0 || p->d_model <= 0 || p->dim <= 0 || p->d_state != ssm::kScanN) return 0;
  if (p->conv_k != ssm::kConvK) return 0;
  return layer_ws(p).total;
}

ssm_status_t ssm_layer_fwd(const ssm_layer_params_t* p, void* stream) {
  const ssm_status_t s = layer_check(p);
  if (s != SSM_OK) return s;
  const int T = p->batch * p->seqlen;
  if (T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const LayerWs o = layer_ws(p);
  char* ws = static_cast<char*>(p->workspace);
  // the caller's timing events bracket the whole layer, not its inner launches
  const ssm::TimingEvents ev = g_timing;
  g_timing = ssm::TimingEvents{};
  auto done = [&](ssm_status_t r) {
    g_timing = ev;
    return r;
  };
  if (ev.start) {
    const hipError_t e = hipEventRecord(ev.start, st);
    if (e != hipSuccess) return done(hip_status(e));
  }
  // 1. in_proj: columns [0, E) -> x_branch, [E, 2E) -> z (fp32)
  ssm::GemmArgs gi{};
  gi.A = p->hidden;
  gi.W = static_cast<const uint16_t*>(p->w_in);
  gi.C0 = ws + o.x;
  gi.C1 = ws + o.z;
  gi.ws = reinterpret_cast<float*>(ws + o.gemm);
  gi.ws_bytes = o.total - o.gemm;
  gi.lda = p->d_model;
  gi.ldw = p->d_model;
  gi.ldc0 = gi.ldc1 = p->dim;
  gi.M = T;
  gi.N = 2 * p->dim;
  gi.K = p->d_model;
  gi.n_split = p->dim;
  hipError_t e = ssm::launch_gemm(gi, p->hidden_dtype, SSM_F32, st);
  if (e != hipSuccess) return done(hip_status(e));
  // 2. conv + SiLU + x_proj -> B, C, dt_raw
  ssm::XprojArgs xa{};
  xa.x = reinterpret_cast<const float*>(ws + o.x);
  xa.conv_w = p->conv_w;
  xa.conv_b = p->conv_b;
  xa.conv_cache_in = p->conv_cache_in;
  xa.w_x = static_cast<const uint16_t*>(p->w_x);
  xa.part = reinterpret_cast<float*>(ws + o.part);
  xa.B = reinterpret_cast<float*>(ws + o.B);
  xa.C = reinterpret_cast<float*>(ws + o.C);
  xa.dt_raw = reinterpret_cast<float*>(ws + o.r);
  xa.batch = p->batch;
  xa.seqlen = p->seqlen;
  xa.dim = p->dim;
  xa.d_state = p->d_state;
  xa.nout = 2 * p->d_state + 1;
  e = ssm::launch_xproj(xa, st);
  if (e != hipSuccess) return done(hip_status(e));
  // 3. the scan (conv + SiLU again from x_branch, dt, recurrence, D, gate)
  ssm_scan_params_t sp = layer_scan_params(p, ws, o);
  const ssm_status_t ss = ssm_scan_fwd(&sp, stream);
  if (ss != SSM_OK) return done(ss);
  // 4. out_proj from the fp32 y
  ssm::GemmArgs go{};
  go.A = ws + o.y;
  go.W = static_cast<const uint16_t*>(p->w_out);
  go.C0 = p->out;
  go.C1 = nullptr;
  go.ws = reinterpret_cast<float*>(ws + o.gemm);
  go.ws_bytes = o.total - o.gemm;
  go.lda = p->dim;
  go.ldw = p->dim;
  go.ldc0 = go.ldc1 = p->d_model;
  go.M = T;
  go.N = p->d_model;
  go.K = p->dim;
  go.n_split = p->d_model;
  e = ssm::launch_gemm(go, SSM_F32, p->out_dtype, st);
  if (e != hipSuccess) return done(hip_status(e));
  if (ev.stop) {
    e = hipEventRecord(ev.stop, st);
    if (e != hipSuccess) return done(hip_status(e));
  }
  return done(ok());
}

ssm_status_t ssm_scan_bwd_check(const ssm_scan_bwd_params_t* p) {
  const ssm_status_t s = bwd_check(p);
  return s == SSM_OK ? ok() : s;
}

size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_params_t* p) {
  if (!p || p->struct_size != sizeof(ssm_scan_bwd_params_t)) return 0;
  if (p->batch < 0 || p->seqlen < 0 || p->dim <= 0) return 0;
  return bwd_ws(p).total;
}

ssm_status_t ssm_scan_bwd(const ssm_scan_bwd_params_t* p, void* stream) {
  const ssm_status_t s = bwd_check(p);
  if (s != SSM_OK) return s;
  if (static_cast<size_t>(p->batch) * p->seqlen == 0) return ok();
  ssm::BwdArgs a{};
  bwd_plan(p, a);
  const ssm_status_t d = debug_bwd(p, a);
  if (d != SSM_OK) return d;
  return hip_status(ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The launch plan of a validated backward call.
void bwd_plan(const ssm_scan_bwd_params_t* p, ssm::BwdArgs& a) {
  const BwdWs o = bwd_ws(p);
  char* ws = static_cast<char*>(p->workspace);
  auto wf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  a = ssm::BwdArgs{};
  a.x = p->x;
  a.dt = p->dt;
  a.dt_w = p->dt_rank1 ? p->dt_w : nullptr;
  a.dt_bias = p->dt_bias;
  a.A = p->A;
  a.B = p->B;
  a.C = p->C;
  a.D = p->D;
  a.z = p->z;
  a.conv_w = p->conv_w;
  a.conv_b = p->conv_b;
  a.conv_cache_in = p->conv_cache_in;
  a.state_in = p->ssm_state_in;
  a.dy = p->dy;
  a.dstate_out = p->dstate_out;
  a.dx = p->dx;
  a.dz = p->dz;
  a.ddt = p->ddt;
  a.ddt_w = p->ddt_w;
  a.ddt_bias = p->ddt_bias;
  a.dA = p->dA;
  a.dB = p->dB;
  a.dC = p->dC;
  a.dD = p->dD;
  a.dconv_w = p->dconv_w;
  a.dconv_b = p->dconv_b;
  a.dconv_cache = p->dconv_cache;
  a.dstate_in = p->dstate_in;
  a.hs = wf(o.hs);
  a.qs = wf(o.qs);
  a.sdt = wf(o.sdt);
  a.xb = p->conv_w ? wf(o.xb) : nullptr;
  a.pB = wf(o.pB);
  a.pC = wf(o.pC);
  a.pr = p->dt_rank1 ? wf(o.pr) : nullptr;
  a.pe = wf(o.pe);
  a.batch = p->batch;
  a.seqlen = p->seqlen;
  a.dim = p->dim;
  a.nseg = ssm::bwd_segments(p->seqlen);
  a.ngroups16 = (p->dim + 15) / 16;
  a.x_bf16 = p->x_dtype == SSM_BF16;
  a.dt_bf16 = p->dt_dtype == SSM_BF16;
  a.dt_rank1 = p->dt_rank1 ? 1 : 0;
  a.bc_bf16 = p->bc_dtype == SSM_BF16;
  a.dy_bf16 = p->dy_dtype == SSM_BF16;
  a.dt_softplus = p->dt_softplus ? 1 : 0;
  a.dt_min = p->dt_min;
  a.dt_max = p->dt_max;
}

}  // namespace

extern "C" {

const char* ssm_status_string(int32_t status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
    case SSM_ERR_INTERNAL: return "SSM_ERR_INTERNAL";
    default: return "unknown status";
  }
}

const char* ssm_last_error(void) { return g_last_error.c_str(); }

int32_t ssm_abi_version(void) { return SSM_ABI_VERSION; }

void ssm_set_timing_events(void* start, void* stop) {
  g_timing.start = static_cast<hipEvent_t>(start);
  g_timing.stop = static_cast<hipEvent_t>(stop);
}

size_t ssm_params_sizeof(int32_t which) {
  switch (which) {
    case 0: return sizeof(ssm_scan_params_t);
    case 1: return sizeof(ssm_decode_params_t);
    case 2: return sizeof(ssm_chunk_params_t);
    case 3: return sizeof(ssm_chunk_decode_params_t);
    case 4: return sizeof(ssm_linear_params_t);
    case 5: return sizeof(ssm_layer_params_t);
    case 6: return sizeof(ssm_scan_bwd_params_t);
    default: return 0;
  }
}

}  // extern "C"

// ---------------------------------------------------------------- debug build
// With SSM_DEBUG the host checks every launch plan before it goes out against
// the buffers the call describes, restating from the kernels' own indexing what
// each of them touches: the mapping from block ids to work items is a
// bijection, segments, chunks and summary pieces tile the sequence as the
// kernels assume, and every workspace region a kernel indexes is 256-byte
// aligned, inside the workspace and disjoint from the others.  Without
// SSM_DEBUG the checks compile to nothing.

namespace {

#ifdef SSM_DEBUG
std::atomic<long> g_debug_checks{0};

ssm_status_t dbg_fail(const char* what) { return fail(SSM_ERR_INTERNAL, "debug check failed: %s", what); }

struct Region {
  const char* what;
  size_t off, bytes;
};

ssm_status_t dbg_regions(const Region* r, int n, size_t ws_bytes) {
  for (int i = 0; i < n; ++i) {
    if (r[i].bytes == 0) continue;
    if (r[i].off % 256) return dbg_fail(r[i].what);
    if (r[i].off > ws_bytes || r[i].bytes > ws_bytes - r[i].off) return dbg_fail(r[i].what);
    for (int j = 0; j < i; ++j)
      if (r[j].bytes && r[i].off < r[j].off + r[j].bytes && r[j].off < r[i].off + r[i].bytes)
        return dbg_fail(r[i].what);
  }
  return SSM_OK;
}

bool dbg_same(const void* arg, const void* base, size_t off) {
  return arg == static_cast<const void*>(static_cast<const char*>(base) + off);
}

// The scan kernels' block ids -> positions of the (segment, batch, channel
// group) order over nblk blocks (CU slot i % 256, round i / 256, the slots'
// runs of consecutive positions): a permutation of [0, nblk).
bool dbg_scan_mapping(long nblk) {
  if (nblk <= 0) return true;
  std::vector<unsigned char> seen(static_cast<size_t>(nblk), 0);
  const long slots = ssm::kScanCuSlots, full = nblk / slots, rem = nblk % slots;
  for (long i = 0; i < nblk; ++i) {
    const long slot = i % slots, round = i / slots;
    const long bid = slot * full + std::min(slot, rem) + round;
    if (bid < 0 || bid >= nblk || seen[static_cast<size_t>(bid)]) return false;
    seen[static_cast<size_t>(bid)] = 1;
  }
  return true;
}

// The chunked scan's block ids -> (batch, head, segment or piece k) over
// batch x heads x nk blocks (heads in runs of H / 8 per XCD when H % 8 == 0):
// each item exactly once.
bool dbg_chunk_mapping(long batch, long heads, long nk) {
  const long n = batch * heads * nk;
  if (n <= 0) return true;
  std::vector<unsigned char> seen(static_cast<size_t>(n), 0);
  for (long bid = 0; bid < n; ++bid) {
    long h, rest;
    if (heads % 8 == 0) {
      const long run = heads / 8;
      rest = bid >> 3;
      h = (bid & 7) * run + rest % run;
      rest /= run;
    } else {
      h = bid % heads;
      rest = bid / heads;
    }
    const long b = rest % batch, k = rest / batch;
    if (h >= heads || k >= nk) return false;
    const size_t item = static_cast<size_t>((k * batch + b) * heads + h);
    if (seen[item]) return false;
    seen[item] = 1;
  }
  return true;
}
#endif

ssm_status_t debug_scan(const ssm_scan_params_t* p, const ssm::ScanLaunch& l) {
#ifdef SSM_DEBUG
  const ssm::ScanKernelArgs& k = l.k;
  const long Bt = p->batch, L = p->seqlen, E = p->dim;
  if (static_cast<long>(k.n_egroups) * 64 < E || static_cast<long>(k.n_egroups - 1) * 64 >= E)
    return dbg_fail("scan: 64-channel groups do not cover the channels exactly");
  if (Bt > 0 && L > 0) {
    if (k.nseg < 1 || k.nseg > ssm::kScanMaxSplit) return dbg_fail("scan: segment count");
    if (k.nseg == 1) {
      if (k.seg_len != L) return dbg_fail("scan: one segment must span the sequence");
    } else {
      if (k.seg_len % ssm::kScanResc) return dbg_fail("scan: segments must start on a rescaling period");
      if (k.seg_len < ssm::kConvK)
        return dbg_fail("scan: a segment past the first starts before step 3 (only segment 0 may read the conv cache)");
      if (static_cast<long>(k.nseg - 1) * k.seg_len >= L || static_cast<long>(k.nseg) * k.seg_len < L)
        return dbg_fail("scan: segments do not tile the sequence (one empty or steps left over)");
    }
    const long groups = Bt * k.n_egroups;
    if (!dbg_scan_mapping(groups * (k.nseg - 1)) || !dbg_scan_mapping(groups * k.nseg))
      return dbg_fail("scan: block mapping is not a bijection");
    // every step also reads the next step's row: batch x L + 1 rows
    const size_t rows = (static_cast<size_t>(Bt) * L + 1) * ssm::kBcRow * sizeof(float);
    const size_t bcg = ssm::scan_bcg_offset(p->batch, p->seqlen), qt = ssm::scan_qtab_offset(p->batch, p->seqlen);
    const size_t so = ssm::scan_summary_offset(p->batch, p->seqlen);
    if (bcg < rows) return dbg_fail("scan: packed B/C rows region too small");
    if (!dbg_same(k.bc, p->workspace, 0)) return dbg_fail("scan: packed rows pointer");
    Region r[5];
    int n = 0;
    r[n++] = {"scan: packed B/C rows region", 0, rows};
    if (k.bcg) {
      if (!dbg_same(k.bcg, p->workspace, bcg) || !dbg_same(k.qtab, p->workspace, qt))
        return dbg_fail("scan: rescaled rows / table pointers");
      if (so - qt < ssm::kScanTab * sizeof(float)) return dbg_fail("scan: q^k table region too small");
      r[n++] = {"scan: rescaled rows region", bcg, rows};
      r[n++] = {"scan: q^k table region", qt, ssm::kScanTab * sizeof(float)};
    }
    if (k.nseg > 1) {
      const size_t ho = ssm::scan_head_offset(p->batch, p->seqlen, p->dim, k.nseg);
      const size_t sb = static_cast<size_t>(groups) * (k.nseg - 1) * (ssm::kScanN + 1) * 64 * sizeof(float);
      const size_t hb = static_cast<size_t>(groups) * ssm::kScanHead * 64 * sizeof(float);
      if (!dbg_same(k.summ, p->workspace, so) || !dbg_same(k.head, p->workspace, ho))
        return dbg_fail("scan: summary / saved-start pointers");
      r[n++] = {"scan: segment summaries region", so, sb};
      r[n++] = {"scan: saved segment-0 start region", ho, hb};
    }
    const ssm_status_t s = dbg_regions(r, n, p->workspace_bytes);
    if (s != SSM_OK) return s;
  }
  g_debug_checks.fetch_add(1, std::memory_order_relaxed);
#else
  (void)p;
  (void)l;
#endif
  return SSM_OK;
}

ssm_status_t debug_scan_blk(const ssm_scan_params_t* p, const ssm::ScanBlkLaunch& l) {
#ifdef SSM_DEBUG
  const ssm::ScanBlkArgs& k = l.k;
  const long Bt = p->batch, L = p->seqlen, E = p->dim;
  if (E % 64) return dbg_fail("blocked scan: channels are not whole 64-channel groups");
  if (static_cast<long>(k.nrec) * ssm::kBlkT < L || static_cast<long>(k.nrec - 1) * ssm::kBlkT >= L)
    return dbg_fail("blocked scan: blocks do not tile the sequence");
  // workgroup i -> position in the (batch row, channel group) order: XCD
  // i % 8 takes a contiguous range, each of its 32 CUs ((i / 8) % 32) a run
  // within it, round (i / 8) / 32 of the run; each position once.  The kernel
  // hands a run's positions to its rounds in an order taken from dt_bias (a
  // permutation of 0 .. len - 1), so the runs must partition the positions
  // and every round must fall inside its run.
  const long groups = E / 64, n = Bt * groups;
  std::vector<unsigned char> seen(static_cast<size_t>(n), 0);
  for (long i = 0; i < n; ++i) {
    const long x = i % 8, k = i / 8;
    const long cnt = n / 8 + (x < n % 8 ? 1 : 0), start = x * (n / 8) + std::min(x, n % 8);
    const long c = k % 32, round = k / 32, full = cnt / 32, rem = cnt % 32;
    const long len = full + (c < rem ? 1 : 0);
    const long p = start + c * full + std::min(c, rem) + round;
    if (round >= len || p < 0 || p >= n || seen[static_cast<size_t>(p)]) return dbg_fail("blocked scan: workgroup mapping");
    seen[static_cast<size_t>(p)] = 1;
  }
  // every batch row's buffer range stays below 2^31 bytes (32-bit offsets)
  const size_t ybytes = p->y_dtype == SSM_BF16 ? 2 : 4;
  if (static_cast<size_t>(L) * E * ybytes >= 0x80000000ULL) return dbg_fail("blocked scan: batch row range");
  const size_t recb = static_cast<size_t>(Bt) * k.nrec * ssm::kBlkRec;
  const size_t qo = ssm::scan_blk_qv_offset(p->batch, p->seqlen);
  if (!dbg_same(k.rec, p->workspace, 0) || !dbg_same(k.qv, p->workspace, qo)) return dbg_fail("blocked scan: workspace pointers");
  const Region r[2] = {{"blocked scan: block records region", 0, recb},
                       {"blocked scan: per-call values region", qo, ssm::kBlkQv * sizeof(float)}};
  const ssm_status_t s = dbg_regions(r, 2, p->workspace_bytes);
  if (s != SSM_OK) return s;
  g_debug_checks.fetch_add(1, std::memory_order_relaxed);
#else
  (void)p;
  (void)l;
#endif
  return SSM_OK;
}

ssm_status_t debug_chunk(const ssm_chunk_params_t* p, const ssm::ChunkGenericArgs& g, const ssm::ChunkLaunch& l) {
#ifdef SSM_DEBUG
  const long Bt = p->batch, L = p->seqlen, H = p->nheads;
  if (!chunk_tuned(p)) {
    const long Q = g.chunk_size, nch = g.nchunks;
    if (nch * Q < L || (nch > 0 && (nch - 1) * Q >= L)) return dbg_fail("chunked scan: chunks do not tile the sequence");
    const size_t st = static_cast<size_t>(Bt) * nch * H * g.headdim * g.d_state * sizeof(float);
    const size_t dec_off = ssm::chunk_generic_decay_offset(p->batch, p->seqlen, p->nheads, p->headdim, p->d_state,
                                                           p->chunk_size);
    if (nch > 0) {
      if (!dbg_same(g.chunk_state, p->workspace, 0) || !dbg_same(g.chunk_decay, p->workspace, dec_off))
        return dbg_fail("chunked scan: workspace pointers");
      const Region r[2] = {{"chunked scan: chunk states region", 0, st},
                           {"chunked scan: chunk decays region", dec_off, static_cast<size_t>(Bt) * nch * H * sizeof(float)}};
      const ssm_status_t s = dbg_regions(r, 2, p->workspace_bytes);
      if (s != SSM_OK) return s;
    }
  } else {
    const ssm::ChunkKernelArgs& k = l.k;
    const long nch = k.nchunks;
    if (nch * ssm::kSsdQ < L || (nch > 0 && (nch - 1) * ssm::kSsdQ >= L))
      return dbg_fail("chunked scan: chunks do not tile the sequence");
    if (k.nseg < 1 || k.nseg > ssm::kSsdMaxSeg) return dbg_fail("chunked scan: segment count");
    if (static_cast<long>(k.nseg) * k.cps < nch || (k.nseg > 1 && static_cast<long>(k.nseg - 1) * k.cps >= nch))
      return dbg_fail("chunked scan: segments do not tile the chunks");
    if (!dbg_chunk_mapping(Bt, H, k.nseg)) return dbg_fail("chunked scan: main-kernel block mapping");
    if (k.nseg > 1) {
      if (static_cast<long>(k.ppseg) * ssm::kSsdPiece < k.cps || static_cast<long>(k.ppseg - 1) * ssm::kSsdPiece >= k.cps)
        return dbg_fail("chunked scan: summary pieces do not tile a segment");
      if (!dbg_chunk_mapping(Bt, H, static_cast<long>(k.nseg - 1) * k.ppseg))
        return dbg_fail("chunked scan: summary-kernel block mapping");
      // the states entering segments 1.., the pieces' states, their decays
      const size_t pn = static_cast<size_t>(k.headdim) * ssm::kSsdN;
      const size_t sin = static_cast<size_t>(Bt) * H * (k.nseg - 1) * pn;
      const size_t pieces = static_cast<size_t>(Bt) * H * (k.nseg - 1) * k.ppseg;
      const size_t need = (sin + pieces * pn + pieces) * sizeof(float);
      if (!dbg_same(k.ws, p->workspace, 0) || need > p->workspace_bytes)
        return dbg_fail("chunked scan: segment workspace runs past the workspace");
    }
  }
  g_debug_checks.fetch_add(1, std::memory_order_relaxed);
#else
  (void)p;
  (void)g;
  (void)l;
#endif
  return SSM_OK;
}

ssm_status_t debug_bwd(const ssm_scan_bwd_params_t* p, const ssm::BwdArgs& a) {
#ifdef SSM_DEBUG
  const size_t Bt = p->batch, L = p->seqlen, E = p->dim, N = ssm::kScanN;
  const long S = a.nseg, R = ssm::bwd_runs(a.nseg), G64 = ssm::bwd_blocks64(p->dim);
  if (S * ssm::kBwdSeg < static_cast<long>(L) || (S - 1) * ssm::kBwdSeg >= static_cast<long>(L))
    return dbg_fail("backward: segments do not tile the sequence");
  if (R * ssm::kBwdRun < S || (R - 1) * ssm::kBwdRun >= S) return dbg_fail("backward: runs do not tile the segments");
  if (static_cast<long>(a.ngroups16) * 16 < static_cast<long>(E) || static_cast<long>(a.ngroups16 - 1) * 16 >= static_cast<long>(E))
    return dbg_fail("backward: 16-channel groups do not cover the channels exactly");
  if (G64 * ssm::kBwdWg < a.ngroups16 || (G64 - 1) * ssm::kBwdWg >= a.ngroups16)
    return dbg_fail("backward: workgroups of four groups do not cover the groups exactly");
  const BwdWs o = bwd_ws(p);
  const void* ws = p->workspace;
  if (!dbg_same(a.hs, ws, o.hs) || !dbg_same(a.qs, ws, o.qs) || !dbg_same(a.sdt, ws, o.sdt) ||
      !dbg_same(a.pB, ws, o.pB) || !dbg_same(a.pC, ws, o.pC) || !dbg_same(a.pe, ws, o.pe) ||
      (a.xb && !dbg_same(a.xb, ws, o.xb)) || (a.pr && !dbg_same(a.pr, ws, o.pr)))
    return dbg_fail("backward: workspace pointers");
  const Region r[8] = {
      {"backward: segment states region", o.hs, Bt * S * E * N * 4},
      {"backward: segment gradients region", o.qs, Bt * S * E * N * 4},
      {"backward: segment dt sums region", o.sdt, Bt * S * E * 4},
      {"backward: run-start conv gradients region", o.xb, a.xb ? Bt * R * 3 * E * 4 : 0},
      {"backward: dB partials region", o.pB, Bt * L * G64 * N * 4},
      {"backward: dC partials region", o.pC, Bt * L * G64 * N * 4},
      {"backward: rank-1 dt partials region", o.pr, a.pr ? Bt * L * G64 * 4 : 0},
      {"backward: per-run channel partials region", o.pe, Bt * R * E * ssm::kBwdPe * 4},
  };
  const ssm_status_t s = dbg_regions(r, 8, p->workspace_bytes);
  if (s != SSM_OK) return s;
  g_debug_checks.fetch_add(1, std::memory_order_relaxed);
#else
  (void)p;
  (void)a;
#endif
  return SSM_OK;
}

}  // namespace

extern "C" {

long ssm_debug_checks(void) {
#ifdef SSM_DEBUG
  return g_debug_checks.load(std::memory_order_relaxed);
#else
  return -1;
#endif
}

ssm_status_t ssm_debug_check_scan(const ssm_scan_params_t* p) {
#ifdef SSM_DEBUG
  const ssm_status_t s = scan_check(p);
  if (s != SSM_OK) return s;
  if (scan_blocked(p)) {
    ssm::ScanBlkLaunch bl;
    scan_blk_plan(p, bl);
    return debug_scan_blk(p, bl);
  }
  ssm::ScanLaunch l;
  scan_plan(p, l);
  return debug_scan(p, l);
#else
  (void)p;
  return fail(SSM_ERR_UNSUPPORTED, "%s", "this build has no debug checks (SSM_DEBUG)");
#endif
}

ssm_status_t ssm_debug_check_chunk(const ssm_chunk_params_t* p) {
#ifdef SSM_DEBUG
  const ssm_status_t s = chunk_check(p);
  if (s != SSM_OK || p->batch == 0) return s;
  ssm::ChunkGenericArgs g{};
  ssm::ChunkLaunch l{};
  chunk_plan(p, g, l);
  return debug_chunk(p, g, l);
#else
  (void)p;
  return fail(SSM_ERR_UNSUPPORTED, "%s", "this build has no debug checks (SSM_DEBUG)");
#endif
}

ssm_status_t ssm_debug_check_scan_bwd(const ssm_scan_bwd_params_t* p) {
#ifdef SSM_DEBUG
  const ssm_status_t s = bwd_check(p);
  if (s != SSM_OK || static_cast<size_t>(p->batch) * p->seqlen == 0) return s;
  ssm::BwdArgs a{};
  bwd_plan(p, a);
  return debug_bwd(p, a);
#else
  (void)p;
  return fail(SSM_ERR_UNSUPPORTED, "%s", "this build has no debug checks (SSM_DEBUG)");
#endif
}

}  // extern "C"
