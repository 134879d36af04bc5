// dp_api.hip -- C ABI of libdp.so (declared in include/dp.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, then enqueues the kernels of dp_kernels.hpp on the caller's
// stream and returns.  The library allocates no device memory for a call and
// keeps no state between calls (a dp_pipeline is the caller's object), except
// the fixed `scratch` array of the no-alloc packed forward.
#include <algorithm>
#include <mutex>
#include <new>
#include <limits.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "dp.h"
#include "dp_bwd.hpp"
#include "dp_kernels.hpp"

DP_DECLARE_LAUNCHERS(f32, 16)
DP_DECLARE_LAUNCHERS(f32, 32)
DP_DECLARE_LAUNCHERS(f32, 64)
DP_DECLARE_LAUNCHERS(f32, 128)
DP_DECLARE_LAUNCHERS(bf16, 16)
DP_DECLARE_LAUNCHERS(bf16, 32)
DP_DECLARE_LAUNCHERS(bf16, 64)
DP_DECLARE_LAUNCHERS(bf16, 128)
DP_DECLARE_BWD_LAUNCHER(f32, 16)
DP_DECLARE_BWD_LAUNCHER(f32, 32)
DP_DECLARE_BWD_LAUNCHER(f32, 64)
DP_DECLARE_BWD_LAUNCHER(f32, 128)
DP_DECLARE_BWD_LAUNCHER(bf16, 16)
DP_DECLARE_BWD_LAUNCHER(bf16, 32)
DP_DECLARE_BWD_LAUNCHER(bf16, 64)
DP_DECLARE_BWD_LAUNCHER(bf16, 128)

// Chunk-offset table of the no-alloc packed forward (dp_fwd_varlen_noalloc_bf16).
constexpr int kScratchInts = DP_NOALLOC_MAX_SEQS + 1;
static_assert(kScratchInts % 64 == 0, "scratch is a whole number of 256-byte blocks");
static __device__ __align__(256) int scratch[kScratchInts];

namespace {

constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr size_t kWsAlign = 256;

struct Shape {
  int n_h, B, H, L, dk, dv, chunk;
};

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_shape(const Shape& s) {
  if (s.n_h <= 0 || s.B <= 0 || s.H <= 0 || s.L < 0 || s.dk <= 0 || s.dv <= 0 || s.chunk <= 0)
    return DP_EINVAL;
  if (!dim_ok(s.dk) || !dim_ok(s.dv)) return DP_ENOTSUP;
  if (s.chunk != 16 && s.chunk != 32 && s.chunk != 64) return DP_ENOTSUP;
  if (s.n_h > 64) return DP_ENOTSUP;
  const long long N = (long long)s.L * s.n_h;
  if (N > (long long)INT_MAX - 64) return DP_ENOTSUP;  // sub-step indices are 32-bit
  const long long nc = (N + s.chunk - 1) / s.chunk;
  if ((long long)s.B * s.H * nc > (long long)INT_MAX) return DP_ENOTSUP;  // grid size
  if ((long long)s.B * s.H * 8 > (long long)INT_MAX) return DP_ENOTSUP;
  // byte offsets within a chunk's readout rows are 32-bit: 64 rows x H dv x 4 bytes
  if ((long long)s.H * s.dv * 64 * 4 > (long long)INT_MAX) return DP_ENOTSUP;
  return DP_OK;
}

int num_chunks(const Shape& s) {
  const long long N = (long long)s.L * s.n_h;
  return (int)((N + s.chunk - 1) / s.chunk);
}

size_t ws_t_bytes(const Shape& s, int elem) {
  return align_up((size_t)s.B * s.H * num_chunks(s) * s.chunk * s.chunk * elem, kWsAlign);
}

// Readout rows a chunk can hold (ceil(C / n_h)), rounded up to MFMA tiles.
int readout_rows(int C, int n_h) {
  const int r = (C + n_h - 1) / n_h;
  return r >= C ? C : ((r + 15) / 16) * 16;
}

// bf16: one operand block per chunk (dp_prep_kernel's output), sized for the
// write-key form where that runs on the same kernels (its block adds the write
// keys), so that one workspace size serves dp_fwd_* and dp_fwd_wk_*; it also
// covers the T / (1/|k|, G) layout of the other write-key shapes.  fp32: T
// and (1/|k|, G).
size_t ws_blocks_bytes(const Shape& s) {
  const bool asym = dp::chain_asym_ok(s.dk, s.chunk);
  const dp::Chunk16Layout W = dp::chunk16_layout(s.dk, s.chunk, readout_rows(s.chunk, s.n_h), asym);
  return align_up((size_t)s.B * s.H * num_chunks(s) * W.bytes, kWsAlign);
}

// One fp32 slot per lane of every scan wavefront (at most dv / 16 per head).
size_t ws_sink_bytes(const Shape& s) { return align_up((size_t)s.B * s.H * (s.dv / 16) * 64 * 4, kWsAlign); }

// The per-channel-gate form (UT / scan kernels) keeps T, the per-sub-step
// scalars and the readout scores (RT x C) per chunk, then the gated operands
// the UT kernel writes for the scan: read and write keys (the layout of k),
// readout queries (the layout of q) and the state decay per chunk (dk fp32).
size_t ws_s_bytes(const Shape& s) { return align_up((size_t)s.B * s.H * num_chunks(s) * s.chunk * sizeof(float2), kWsAlign); }
struct CgWs {
  size_t p, kg, qg, dec;
};
CgWs cg_ws(const Shape& s, int elem) {
  CgWs w;
  const size_t nch = (size_t)s.B * s.H * num_chunks(s);
  w.p = align_up(nch * readout_rows(s.chunk, s.n_h) * s.chunk * elem, kWsAlign);
  w.kg = align_up((size_t)s.B * s.L * s.H * s.n_h * s.dk * elem, kWsAlign);
  w.qg = align_up((size_t)s.B * s.L * s.H * s.dk * elem, kWsAlign);
  w.dec = align_up(nch * s.dk * 4, kWsAlign);
  return w;
}
size_t ws_cg_bytes(const Shape& s, int elem) {
  const CgWs w = cg_ws(s, elem);
  return ws_t_bytes(s, elem) + ws_s_bytes(s) + w.p + 2 * w.kg + w.qg + w.dec;
}

size_t ws_total(const Shape& s, int elem) {
  const size_t cg = ws_cg_bytes(s, elem);
  size_t base = elem == 2 ? ws_blocks_bytes(s) + ws_sink_bytes(s) : ws_t_bytes(s, elem) + ws_s_bytes(s);
  return base > cg ? base : cg;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int a16(int x) { return (x + 15) & ~15; }

// Magic number for s / d, 0 <= s < 2^31, 1 <= d <= 64: with l = ceil(log2 d),
// shift = 31 + l and magic = ceil(2^shift / d), s / d == (s * magic) >> shift
// (the rounding error s * (magic * d - 2^shift) / (d 2^shift) stays below 1/d).
void fastdiv_magic(int d, uint32_t* magic, int* shift) {
  int l = 0;
  while ((1 << l) < d) ++l;
  const int sh = 31 + l;
  const unsigned long long m = ((1ull << sh) + (unsigned long long)d - 1) / (unsigned long long)d;
  *magic = (uint32_t)m;
  *shift = sh;
}

// Fill the scan kernel's LDS offsets; returns total bytes.
int scan_layout(dp::FwdArgs& a, int elem, int DK, int C, int BV) {
  const int VE = 16 / elem;
  const int LDK = DK + VE, LDC = C + VE;
  int off = 0;
  auto take = [&](int bytes) {
    const int o = off;
    off += a16(bytes);
    return o;
  };
  const bool cg = a.ga != nullptr;
  a.oK = take(C * LDK * elem);
  a.oKt = (a.asym || cg) ? take(C * LDK * elem) : a.oK;
  // the readout queries are dead after the first phase of a chunk and Up / Us
  // are written after it: they share one region
  const int q_bytes = a.RT * LDK * elem, u_bytes = a16(BV * LDC * elem);
  a.oQ = take(q_bytes > 2 * u_bytes ? q_bytes : 2 * u_bytes);
  a.oUo = a.oQ;
  a.oUs = a.oQ + u_bytes;
  a.oT = take(C * LDC * elem);
  a.oHt = take(BV * LDK * elem);
  a.oXt = take(BV * LDC * elem);
  a.oP = take(a.RT * LDC * elem);
  a.oV = take(C * (BV + 4) * 4);
  a.oG = take(C * 4);
  a.oEG = take(C * 4);
  a.oEL = take(C * 4);
  a.oLoc = take(a.RT * 4);
  a.oRow = take(2 * C * 8);
  a.oTok = take(2 * a.RT * 8);
  a.oDec = cg ? take(DK * 4) : 0;
  return off;
}

int ut_lds(int elem, int DK, int C, int asym, int cg = 0) { return dp::ut_lds_bytes(elem, DK, C, asym, cg); }

// Value-block width of the scan: the widest BV (fewer redundant key-side
// products per head) that still gives at least one workgroup per CU
// (256 CUs), else the narrowest.  DP_SCAN_BV overrides it (16, 32 or 64).
int pick_bv(int BH, int dv) {
  const char* env = getenv("DP_SCAN_BV");
  if (env != nullptr) {
    const int v = atoi(env);
    if ((v == 16 || v == 32 || v == 64) && v <= dv) return v;
  }
  for (int bv = 64; bv >= 16; bv >>= 1) {
    if (bv > dv) continue;
    if ((long long)BH * (dv / bv) >= 256) return bv;
  }
  return 16;
}

// Value columns per workgroup of the bf16 scan (16 per wavefront, 1, 2 or 4
// wavefronts): the widest that still gives at least one workgroup per CU
// (256 CUs), else one wavefront.  DP_SCAN_NW overrides it (1, 2 or 4).
int pick_bv16(int BH, int dv) {
  const char* env = getenv("DP_SCAN_NW");
  if (env != nullptr) {
    const int nw = atoi(env);
    if ((nw == 1 || nw == 2 || nw == 4) && 16 * nw <= dv) return 16 * nw;
  }
  for (int nw = 4; nw >= 1; nw >>= 1) {
    if (16 * nw > dv) continue;
    if ((long long)BH * (dv / (16 * nw)) >= 256) return 16 * nw;
  }
  return 16;
}

// Can this call run the fused kernel?  bf16, symmetric keys, dk and chunk
// multiples of 32 and both stages in one call.
bool fused_possible(int elem, bool asym, int dk, int chunk, int flags) {
  return elem == 2 && !asym && dp::fused_ok(dk, chunk) && (flags & DP_STAGE_ALL) == DP_STAGE_ALL;
}

// Does it?  Each workgroup of the fused kernel builds its chunk's operands
// itself, so a head split over several workgroups (value-column blocks) builds
// them once per block; the prep / chain pair builds them once per chunk and
// is faster there.  The fused kernel is the default only where one workgroup
// holds all dv columns of a head (dv <= 32); DP_FWD_SPLIT and DP_FWD_FUSED
// override the choice.
bool use_fused(int elem, bool asym, int dk, int dv, int chunk, int flags) {
  if (!fused_possible(elem, asym, dk, chunk, flags) || (flags & DP_FWD_SPLIT) != 0) return false;
  return (flags & DP_FWD_FUSED) != 0 || dv <= 32;
}

// Flag checks shared by the forward entry points: known bits, one stage at
// least, not both path overrides, and a forced fused path only where it exists.
int check_fwd_flags(int elem, bool asym, int dk, int chunk, int flags) {
  if ((flags & ~(DP_STAGE_ALL | DP_OUT_F32 | DP_FWD_SPLIT | DP_FWD_FUSED)) != 0) return DP_EINVAL;
  if ((flags & DP_STAGE_ALL) == 0) return DP_EINVAL;
  if ((flags & DP_FWD_SPLIT) != 0 && (flags & DP_FWD_FUSED) != 0) return DP_EINVAL;
  if ((flags & DP_FWD_FUSED) != 0 && !fused_possible(elem, asym, dk, chunk, flags)) return DP_ENOTSUP;
  return DP_OK;
}

// Choose BV and fill the scan layout of `a` (a.RT, a.asym, a.fused and a.ga must be set).
int plan(dp::FwdArgs& a, int elem, int dk, int chunk, int* BV_out, int* lds_out) {
  if (a.ga != nullptr) {  // per-channel gate: the UT / scan kernels for either input type
    int BV = pick_bv(a.B * a.H, a.dv);
    int lds = 0;
    for (;; BV >>= 1) {
      if (BV < 16) return DP_ENOTSUP;
      lds = scan_layout(a, elem, dk, chunk, BV);
      if (lds <= kMaxLds) break;
    }
    if (ut_lds(elem, dk, chunk, a.asym, 1) > kMaxLds) return DP_ENOTSUP;
    a.nvb = a.dv / BV;
    *BV_out = BV;
    *lds_out = lds;
    return DP_OK;
  }
  if (a.fused) {
    // one or two consumer wavefronts: all of dv up to 32 columns in one workgroup
    int BV = a.dv <= 32 ? a.dv : pick_bv16(a.B * a.H, a.dv);
    if (BV > 32) BV = 32;
    while (dp::fused_layout(dk, chunk, a.RT, BV).bytes > kMaxLds && BV > 16) BV >>= 1;
    if (dp::fused_layout(dk, chunk, a.RT, BV).bytes > kMaxLds) return DP_ENOTSUP;
    a.nvb = a.dv / BV;
    *BV_out = BV;
    *lds_out = dp::fused_layout(dk, chunk, a.RT, BV).bytes;
    return DP_OK;
  }
  if (elem == 2 && (!a.asym || dp::chain_asym_ok(dk, chunk))) {
    const bool asym = a.asym != 0;
    int BV = pick_bv16(a.B * a.H, a.dv);
    while (dp::chain_lds_bytes(dk, chunk, a.RT, BV, asym) > kMaxLds && BV > 16) BV >>= 1;
    if (dp::chain_lds_bytes(dk, chunk, a.RT, BV, asym) > kMaxLds) return DP_ENOTSUP;
    if (dp::prep_lds_bytes(dk, chunk, a.RT, asym) > kMaxLds) return DP_ENOTSUP;
    a.nvb = a.dv / BV;
    *BV_out = BV;
    *lds_out = dp::chain_lds_bytes(dk, chunk, a.RT, BV, asym);
    return DP_OK;
  }
  if (elem == 2) {
    int BV = pick_bv16(a.B * a.H, a.dv);
    dp::Scan16Layout L = dp::scan16_layout(dk, chunk, BV, a.RT, a.asym);
    while (L.total > kMaxLds && BV > 16) {  // fewer value columns, smaller buffers
      BV >>= 1;
      L = dp::scan16_layout(dk, chunk, BV, a.RT, a.asym);
    }
    if (L.total > kMaxLds) return DP_ENOTSUP;
    if (ut_lds(elem, dk, chunk, a.asym) > kMaxLds) return DP_ENOTSUP;
    a.nvb = a.dv / BV;
    *BV_out = BV;
    *lds_out = L.total;
    return DP_OK;
  }
  int BV = pick_bv(a.B * a.H, a.dv);
  int lds = 0;
  for (;; BV >>= 1) {
    if (BV < 16) return DP_ENOTSUP;
    lds = scan_layout(a, elem, dk, chunk, BV);
    if (lds <= kMaxLds) break;
  }
  if (ut_lds(elem, dk, chunk, a.asym) > kMaxLds) return DP_ENOTSUP;
  a.nvb = a.dv / BV;
  *BV_out = BV;
  *lds_out = lds;
  return DP_OK;
}

hipError_t dispatch_fwd(int elem, int dk, const dp::FwdArgs& a, int C, int BV, int lds,
                        int stages, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 16: return dp_launch_fwd_f32_16(a, C, BV, lds, stages, st);
      case 32: return dp_launch_fwd_f32_32(a, C, BV, lds, stages, st);
      case 64: return dp_launch_fwd_f32_64(a, C, BV, lds, stages, st);
      case 128: return dp_launch_fwd_f32_128(a, C, BV, lds, stages, st);
    }
  } else {
    switch (dk) {
      case 16: return dp_launch_fwd_bf16_16(a, C, BV, lds, stages, st);
      case 32: return dp_launch_fwd_bf16_32(a, C, BV, lds, stages, st);
      case 64: return dp_launch_fwd_bf16_64(a, C, BV, lds, stages, st);
      case 128: return dp_launch_fwd_bf16_128(a, C, BV, lds, stages, st);
    }
  }
  return hipErrorInvalidValue;
}

// Phase 1 in 64-token chunks (dk >= 64): its workspace per call of L tokens.
struct P1cWs {
  size_t tm, v, fac, gt, dstart, gam, restart, cbase, total;
};
// nbh heads, nch chunks over all heads, ncb ints of per-sequence chunk offsets
P1cWs p1c_ws_n(size_t nbh, size_t nch, int dk, size_t ncb) {
  P1cWs w;
  w.tm = align_up(nch * dp::kP1Chunk * dp::kP1Chunk * 4, kWsAlign);
  w.v = align_up(nch * dp::kP1Chunk * 4, kWsAlign);
  w.fac = align_up(nch * dp::kP1Chunk * 16, kWsAlign);
  w.gt = align_up(nch * 4, kWsAlign);
  w.dstart = align_up(nch * dk * 4, kWsAlign);
  w.gam = w.v;
  w.restart = align_up(nbh * 4, kWsAlign);
  w.cbase = align_up(ncb * 4, kWsAlign);
  w.total = dk >= 64 ? w.tm + w.v + w.fac + w.gt + w.dstart + w.gam + w.restart + w.cbase : 0;
  return w;
}
P1cWs p1c_ws(int B, int H, int L, int dk) {
  const size_t nbh = (size_t)B * H;
  return p1c_ws_n(nbh, nbh * ((L + dp::kP1Chunk - 1) / dp::kP1Chunk), dk, 0);
}
// packed: nseq sequences over T tokens, at most ceil(T / C) + nseq chunks per head
P1cWs p1c_ws_var(int nseq, int H, int T, int dk) {
  return p1c_ws_n((size_t)nseq * H, (size_t)H * ((T + dp::kP1Chunk - 1) / dp::kP1Chunk + nseq), dk,
                  (size_t)nseq + 1);
}
// point a's chunked-form buffers into ws (p1c_ws(B, H, L, dk).total bytes, or
// p1c_ws_var(B, H, L, dk).total with packed sequences)
void p1c_bind(dp::PrecondArgs& a, char* ws, int dk) {
  const P1cWs w = a.cu != nullptr ? p1c_ws_var(a.B, a.H, a.L, dk) : p1c_ws(a.B, a.H, a.L, dk);
  char* o = ws;
  a.wsTm = reinterpret_cast<float*>(o);
  o += w.tm;
  a.wsV = reinterpret_cast<float*>(o);
  o += w.v;
  a.wsFac = reinterpret_cast<float4*>(o);
  o += w.fac;
  a.wsGT = reinterpret_cast<float*>(o);
  o += w.gt;
  a.dstart = reinterpret_cast<float*>(o);
  o += w.dstart;
  a.gam = reinterpret_cast<float*>(o);
  o += w.gam;
  a.restart = reinterpret_cast<int*>(o);
  o += w.restart;
  a.cbase = a.cu != nullptr ? reinterpret_cast<int*>(o) : nullptr;
}

hipError_t dispatch_precond_chunked(int elem, int dk, const dp::PrecondArgs& a, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 64: return dp_launch_precond_chunked_f32_64(a, st);
      case 128: return dp_launch_precond_chunked_f32_128(a, st);
    }
  } else {
    switch (dk) {
      case 64: return dp_launch_precond_chunked_bf16_64(a, st);
      case 128: return dp_launch_precond_chunked_bf16_128(a, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_precond(int elem, int dk, const dp::PrecondArgs& a, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 16: return dp_launch_precond_f32_16(a, st);
      case 32: return dp_launch_precond_f32_32(a, st);
      case 64: return dp_launch_precond_f32_64(a, st);
      case 128: return dp_launch_precond_f32_128(a, st);
    }
  } else {
    switch (dk) {
      case 16: return dp_launch_precond_bf16_16(a, st);
      case 32: return dp_launch_precond_bf16_32(a, st);
      case 64: return dp_launch_precond_bf16_64(a, st);
      case 128: return dp_launch_precond_bf16_128(a, st);
    }
  }
  return hipErrorInvalidValue;
}

// Ls, t0: the call covers tokens t0 .. t0 + L - 1 of sequences Ls tokens long
// (0, 0: the whole sequences).  dry: validate and plan only, enqueue nothing.
int fwd_impl(int elem, const void* q, const void* k, const void* kt, const void* v,
             const float* beta, const float* g, int n_h, int B, int H, int L, int dk, int dv,
             int chunk, void* out, float* final_state, const float* h0, void* workspace,
             size_t workspace_bytes, int flags, dp_stream stream, int Ls = 0, int t0 = 0,
             bool dry = false, const float* ga = nullptr) {
  const Shape s{n_h, B, H, L, dk, dv, chunk};
  int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  rc = check_fwd_flags(elem, kt != nullptr, dk, chunk, flags);
  if (rc != DP_OK) return rc;
  const int stages = flags & DP_STAGE_ALL;
  // with L == 0 the per-token tensors are empty and may be null
  if (L > 0 && (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || out == nullptr))
    return DP_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (kt != nullptr && !aligned16(kt)))
    return DP_EINVAL;
  if (ga != nullptr && (flags & DP_FWD_FUSED) != 0) return DP_ENOTSUP;  // the fused kernel has no channel gate
  const bool fused = ga == nullptr && use_fused(elem, kt != nullptr, dk, dv, chunk, flags);
  const size_t need = fused ? 0 : ws_total(s, elem);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return DP_EWORKSPACE;
  if (need > 0 && ((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;

  dp::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.kt = kt;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.out = out;
  a.fstate = final_state;
  if (!fused) {
    a.wsT = workspace;
    a.wsS = reinterpret_cast<float2*>(static_cast<char*>(workspace) + ws_t_bytes(s, elem));
    if (elem == 2) a.sink = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_blocks_bytes(s));
    if (ga != nullptr) {
      const CgWs w = cg_ws(s, elem);
      char* base = static_cast<char*>(workspace) + ws_t_bytes(s, elem) + ws_s_bytes(s);
      a.wsP = base;
      a.wsKg = base + w.p;
      a.wsKtg = base + w.p + w.kg;
      a.wsQg = base + w.p + 2 * w.kg;
      a.wsDec = reinterpret_cast<float*>(base + w.p + 2 * w.kg + w.qg);
    }
  }
  a.ga = ga;
  a.N = L * n_h;
  a.B = B;
  a.H = H;
  a.L = L;
  a.n_h = n_h;
  a.dv = dv;
  a.nc = num_chunks(s);
  a.RT = readout_rows(chunk, n_h);
  a.asym = kt != nullptr ? 1 : 0;
  a.out_f32 = (elem == 4 || (flags & DP_OUT_F32) != 0) ? 1 : 0;
  a.Ls = Ls;
  a.t0 = t0;
  a.fused = fused ? 1 : 0;
  fastdiv_magic(n_h, &a.nh_magic, &a.nh_shift);

  int BV = 0, lds = 0;
  rc = plan(a, elem, dk, chunk, &BV, &lds);
  if (rc != DP_OK || dry) return rc;

  int run = stages;
  if (a.nc == 0) run &= ~DP_STAGE_UT;  // nothing to transform; the scan copies h0
  const hipError_t e = dispatch_fwd(elem, dk, a, chunk, BV, lds, run,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

// Packed variable-length sequences (bf16, symmetric keys).  The operand blocks
// are sized for the worst case over all splits of T tokens into nseq sequences,
// H (ceil(T n_h / C) + nseq) blocks; then the per-sequence first chunks
// (nseq + 1 ints) and the sink.
struct VarShape {
  int n_h, nseq, H, T, dk, dv, chunk;
};

int check_varlen(const VarShape& v) {
  if (v.n_h <= 0 || v.nseq <= 0 || v.H <= 0 || v.T < 0 || v.dk <= 0 || v.dv <= 0 || v.chunk <= 0)
    return DP_EINVAL;
  const Shape s{v.n_h, v.nseq, v.H, 0, v.dk, v.dv, v.chunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  const long long N = (long long)v.T * v.n_h;
  if (N > (long long)INT_MAX - 64) return DP_ENOTSUP;
  const long long nwork = (long long)v.H * ((N + v.chunk - 1) / v.chunk + v.nseq);
  if (nwork > (long long)INT_MAX) return DP_ENOTSUP;
  return DP_OK;
}

long long varlen_nwork(const VarShape& v) {
  const long long N = (long long)v.T * v.n_h;
  return (long long)v.H * ((N + v.chunk - 1) / v.chunk + v.nseq);
}

size_t varlen_blocks_bytes(const VarShape& v) {
  // sized for the write-key form wherever it runs (as ws_blocks_bytes), so
  // one size serves both forward forms
  const bool asym = dp::chain_asym_ok(v.dk, v.chunk);
  const dp::Chunk16Layout W = dp::chunk16_layout(v.dk, v.chunk, readout_rows(v.chunk, v.n_h), asym);
  return align_up((size_t)varlen_nwork(v) * W.bytes, kWsAlign);
}
size_t varlen_cbase_bytes(const VarShape& v) { return align_up((size_t)(v.nseq + 1) * 4, kWsAlign); }
// fp32 inputs (UT / scan kernels): T (C x C fp32) and the per-sub-step
// scalars (C float2) of every work item, then the first chunks
size_t varlen_t32_bytes(const VarShape& v) {
  return align_up((size_t)varlen_nwork(v) * v.chunk * v.chunk * 4, kWsAlign);
}
size_t varlen_s32_bytes(const VarShape& v) {
  return align_up((size_t)varlen_nwork(v) * v.chunk * sizeof(float2), kWsAlign);
}
size_t varlen_ws_total16(const VarShape& v) {
  return varlen_blocks_bytes(v) + varlen_cbase_bytes(v) +
         align_up((size_t)v.nseq * v.H * (v.dv / 16) * 64 * 4, kWsAlign);
}
size_t varlen_ws_total32(const VarShape& v) {
  return varlen_t32_bytes(v) + varlen_s32_bytes(v) + varlen_cbase_bytes(v);
}
// one size serves both input types and both packed forms
size_t varlen_ws_total(const VarShape& v) { return std::max(varlen_ws_total16(v), varlen_ws_total32(v)); }
// the fused kernel needs only the per-sequence first chunks
size_t varlen_ws_need(const VarShape& v, bool fused, int elem) {
  return fused ? varlen_cbase_bytes(v) : elem == 4 ? varlen_ws_total32(v) : varlen_ws_total16(v);
}

// table: when not NULL, the fused kernel's chunk-offset table lives there (at
// least nseq + 1 ints) and no workspace is used.  dry: validate and plan only.
// kt: the write keys (the prep / chain pair's write-key form), or NULL.
int varlen_impl(const void* q, const void* k, const void* v, const float* beta, const float* g,
                const int* cu_seqlens, int nseq, int n_h, int H, int T, int dk, int dv, int chunk,
                void* out, float* final_state, const float* h0, void* workspace,
                size_t workspace_bytes, int flags, dp_stream stream, int* table = nullptr,
                bool dry = false, const void* kt = nullptr, int elem = 2) {
  const VarShape vs{n_h, nseq, H, T, dk, dv, chunk};
  int rc = check_varlen(vs);
  if (rc != DP_OK) return rc;
  const bool asym = kt != nullptr;
  rc = check_fwd_flags(elem, asym, dk, chunk, flags);
  if (rc != DP_OK) return rc;
  // bf16: the packed write-key form runs on the prep / chain pair only
  if (elem == 2 && asym && !dp::chain_asym_ok(dk, chunk)) return DP_ENOTSUP;
  const int stages = flags & DP_STAGE_ALL;
  if (cu_seqlens == nullptr) return DP_EINVAL;
  if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || out == nullptr))
    return DP_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(kt)) return DP_EINVAL;
  const bool fused = use_fused(elem, asym, dk, dv, chunk, flags);
  if (table != nullptr) {
    if (!fused) return DP_ENOTSUP;  // only the fused kernel runs on the table alone
  } else {
    const size_t need = varlen_ws_need(vs, fused, elem);
    if (workspace_bytes < need || workspace == nullptr) return DP_EWORKSPACE;
    if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
  }

  dp::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.out = out;
  a.fstate = final_state;
  a.cu = cu_seqlens;
  if (fused) {
    a.cbase = table != nullptr ? table : static_cast<int*>(workspace);
  } else if (elem == 4) {
    a.wsT = workspace;
    a.wsS = reinterpret_cast<float2*>(static_cast<char*>(workspace) + varlen_t32_bytes(vs));
    a.cbase = reinterpret_cast<int*>(static_cast<char*>(workspace) + varlen_t32_bytes(vs) +
                                     varlen_s32_bytes(vs));
  } else {
    a.wsT = workspace;
    a.cbase = reinterpret_cast<int*>(static_cast<char*>(workspace) + varlen_blocks_bytes(vs));
    a.sink = reinterpret_cast<float*>(static_cast<char*>(workspace) + varlen_blocks_bytes(vs) +
                                      varlen_cbase_bytes(vs));
  }
  a.fused = fused ? 1 : 0;
  a.nwork = (int)varlen_nwork(vs);
  a.B = nseq;
  a.H = H;
  a.L = T;  // total tokens (the chunk-offset kernel checks cu[nseq] == T)
  a.n_h = n_h;
  a.dv = dv;
  a.kt = kt;
  a.RT = readout_rows(chunk, n_h);
  a.asym = asym ? 1 : 0;
  a.out_f32 = (elem == 4 || (flags & DP_OUT_F32) != 0) ? 1 : 0;
  fastdiv_magic(n_h, &a.nh_magic, &a.nh_shift);

  int BV = 0, lds = 0;
  rc = plan(a, elem, dk, chunk, &BV, &lds);
  if (rc != DP_OK || dry) return rc;
  const hipError_t e = dispatch_fwd(elem, dk, a, chunk, BV, lds, stages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

// The no-alloc packed forward keeps its chunk-offset table in `scratch`, one
// copy per device, held until the process ends.  In host code `scratch` names
// a host-side stand-in: its device address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is handed to kernels.
constexpr int kMaxScratchDevices = 64;

// device address of this device's `scratch`, or nullptr when the lookup fails
int* scratch_on_current_device() {
  static std::mutex mu;
  static int* addr[kMaxScratchDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = static_cast<int*>(p);
  }
  return addr[dev];
}

hipError_t dispatch_decode(int elem, int dk, const dp::DecodeArgs& a, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 16: return dp_launch_decode_f32_16(a, st);
      case 32: return dp_launch_decode_f32_32(a, st);
      case 64: return dp_launch_decode_f32_64(a, st);
      case 128: return dp_launch_decode_f32_128(a, st);
    }
  } else {
    switch (dk) {
      case 16: return dp_launch_decode_bf16_16(a, st);
      case 32: return dp_launch_decode_bf16_32(a, st);
      case 64: return dp_launch_decode_bf16_64(a, st);
      case 128: return dp_launch_decode_bf16_128(a, st);
    }
  }
  return hipErrorInvalidValue;
}

int decode_impl(int elem, const void* q, const void* k, const void* kt, const void* v,
                const float* beta, const float* g, const float* ga, int n_h, int B, int H, int dk,
                int dv, void* out, float* state, int flags, dp_stream stream) {
  if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || out == nullptr ||
      state == nullptr)
    return DP_EINVAL;
  if (n_h <= 0 || B <= 0 || H <= 0 || dk <= 0 || dv <= 0) return DP_EINVAL;
  if ((flags & ~DP_OUT_F32) != 0) return DP_EINVAL;
  if (!dim_ok(dk) || !dim_ok(dv)) return DP_ENOTSUP;
  if (n_h > 64) return DP_ENOTSUP;
  if ((long long)B * H * 8 > (long long)INT_MAX) return DP_ENOTSUP;  // grid size
  dp::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.kt = kt;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.ga = ga;
  a.out = out;
  a.state = state;
  a.B = B;
  a.H = H;
  a.n_h = n_h;
  a.dv = dv;
  a.out_f32 = (elem == 4 || (flags & DP_OUT_F32) != 0) ? 1 : 0;
  const hipError_t e = dispatch_decode(elem, dk, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

int precond_impl(int elem, const void* k, const float* beta, const float* ret, int flags,
                 int B, int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                 float* d_state, void* kt, bool open_box, dp_stream stream, int Ls = 0, int t0 = 0,
                 bool dry = false, char* p1c = nullptr, const int* cu = nullptr) {
  // with L == 0 the per-token tensors are empty and may be null
  if (d_state == nullptr || (L > 0 && (k == nullptr || beta == nullptr || kt == nullptr))) return DP_EINVAL;
  if (!aligned16(k) || !aligned16(kt)) return DP_EINVAL;
  if (B <= 0 || H <= 0 || L < 0) return DP_EINVAL;
  if ((flags & ~DP_PRECOND_BETA_FREE) != 0) return DP_EINVAL;
  if (!dim_ok(dk)) return DP_ENOTSUP;
  if (!(eps > 0.f) || !(dmin <= dmax) || !(eta == eta)) return DP_EINVAL;
  if (!open_box && !(dmin > 0.f)) return DP_EINVAL;
  if ((long long)B * H * (long long)L > (long long)1 << 40) return DP_ENOTSUP;
  if (L == 0 || dry) return DP_OK;
  dp::PrecondArgs a;
  a.k = k;
  a.beta = beta;
  a.ret = ret;
  a.d = d_state;
  a.kt = kt;
  a.B = B;
  a.H = H;
  a.L = L;
  a.beta_aware = (flags & DP_PRECOND_BETA_FREE) ? 0 : 1;
  a.eta = eta;
  a.dmin = dmin;
  a.dmax = dmax;
  a.eps = eps;
  a.Ls = Ls;
  a.t0 = t0;
  a.cu = cu;  // packed sequences: B of them over L tokens
  // with a workspace for it (p1c_ws, or p1c_ws_var when packed) and dk >= 64,
  // the chunked form, whose hand-over to the exact scan keeps the sequential
  // definition's result
  if (p1c != nullptr && dk >= 64) {
    p1c_bind(a, p1c, dk);
    const hipError_t e = dispatch_precond_chunked(elem, dk, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DP_OK : DP_EHIP;
  }
  const hipError_t e = dispatch_precond(elem, dk, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

// Write-key forward with its phase 1, pipelined over token segments.  Each
// segment is a whole number of chunks (n_h = 1: a chunk is C tokens), so the
// chunks are those of the unsegmented forward.  Phase 1 runs on the caller's
// stream and phase 2 on the stream of a caller-owned dp_pipeline, ordered by
// one event per segment.
constexpr int kMaxSegments = 16;

int seg_len(int L, int chunk, int segments) {
  const int per = (L + segments - 1) / segments;
  const int len = (per + chunk - 1) / chunk * chunk;
  return len > 0 ? len : chunk;
}

}  // namespace

struct dp_pipeline_s {
  int device = -1;
  hipStream_t st2 = nullptr;
  hipEvent_t ev[kMaxSegments + 1] = {};
  std::mutex mu;  // held by a call for its whole enqueue sequence
};

namespace {

void release_pipeline(dp_pipeline p) {
  for (int i = 0; i <= kMaxSegments; ++i)
    if (p->ev[i] != nullptr) (void)hipEventDestroy(p->ev[i]);
  if (p->st2 != nullptr) (void)hipStreamDestroy(p->st2);
  delete p;
}

// Backward: fixed chunk of kBwdChunk sub-steps.  Workspace: T (fp32) and
// (1/|k|, G) per chunk, the chunk-start states, the chunk-end state
// gradients and the pseudo-value gradients.
struct BwdWs {
  size_t t, s, hs, dhe, dup, total;
};

BwdWs bwd_ws(const Shape& s) {
  const size_t nch = (size_t)s.B * s.H * num_chunks(s);
  BwdWs w;
  w.t = align_up(nch * s.chunk * s.chunk * 4, kWsAlign);
  w.s = align_up(nch * s.chunk * sizeof(float2), kWsAlign);
  w.hs = align_up(nch * s.dk * s.dv * 4, kWsAlign);
  w.dhe = w.hs;
  w.dup = align_up(nch * s.chunk * s.dv * 4, kWsAlign);
  w.total = w.t + w.s + w.hs + w.dhe + w.dup;
  return w;
}

hipError_t dispatch_bwd(int elem, int dk, const dp::FwdArgs& fa, const dp::BwdArgs& a, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 16: return dp_launch_bwd_f32_16(fa, a, st);
      case 32: return dp_launch_bwd_f32_32(fa, a, st);
      case 64: return dp_launch_bwd_f32_64(fa, a, st);
      case 128: return dp_launch_bwd_f32_128(fa, a, st);
    }
  } else {
    switch (dk) {
      case 16: return dp_launch_bwd_bf16_16(fa, a, st);
      case 32: return dp_launch_bwd_bf16_32(fa, a, st);
      case 64: return dp_launch_bwd_bf16_64(fa, a, st);
      case 128: return dp_launch_bwd_bf16_128(fa, a, st);
    }
  }
  return hipErrorInvalidValue;
}

int bwd_impl(int elem, const void* q, const void* k, const void* v, const float* beta,
             const float* g, const float* h0, const void* dout, const float* dfinal, int n_h,
             int B, int H, int L, int dk, int dv, float* dq, float* dk_out, float* dv_out,
             float* dbeta, float* dg, float* dh0, void* workspace, size_t workspace_bytes,
             dp_stream stream, const void* kt = nullptr, float* dkt = nullptr, bool wk = false,
             bool dry = false) {
  const Shape s{n_h, B, H, L, dk, dv, dp::kBwdChunk};
  int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  if (L > 0 && (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || dout == nullptr ||
                dq == nullptr || dk_out == nullptr || dv_out == nullptr || dbeta == nullptr))
    return DP_EINVAL;
  if (wk && L > 0 && (kt == nullptr || dkt == nullptr)) return DP_EINVAL;
  if (L > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || (wk && !aligned16(kt))))
    return DP_EINVAL;
  const BwdWs w = bwd_ws(s);
  if (workspace_bytes < w.total || workspace == nullptr) return DP_EWORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);

  dp::FwdArgs fa;
  memset(&fa, 0, sizeof(fa));
  fa.k = k;
  fa.kt = wk ? kt : nullptr;
  fa.asym = wk ? 1 : 0;
  fa.beta = beta;
  fa.g = g;
  fa.wsT = ws;
  fa.wsS = reinterpret_cast<float2*>(ws + w.t);
  fa.N = L * n_h;
  fa.B = B;
  fa.H = H;
  fa.L = L;
  fa.n_h = n_h;
  fa.dv = dv;
  fa.nc = num_chunks(s);
  fastdiv_magic(n_h, &fa.nh_magic, &fa.nh_shift);

  dp::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.kt = wk ? kt : nullptr;
  a.dkt = wk ? dkt : nullptr;
  a.dout = dout;
  a.dfinal = dfinal;
  a.wsT = reinterpret_cast<const float*>(ws);
  a.wsS = fa.wsS;
  // (sized for fp32; the bf16 path stores them in fp16 and uses half)
  a.hs = ws + w.t + w.s;
  a.dhe = ws + w.t + w.s + w.hs;
  a.dup = ws + w.t + w.s + w.hs + w.dhe;
  a.dq = dq;
  a.dk = dk_out;
  a.dv = dv_out;
  a.dbeta = dbeta;
  a.dg = g != nullptr ? dg : nullptr;
  a.dh0 = dh0;
  a.N = fa.N;
  a.B = B;
  a.H = H;
  a.L = L;
  a.n_h = n_h;
  a.dvd = dv;
  a.nc = fa.nc;
  a.RT = readout_rows(dp::kBwdChunk, n_h);
  a.nvb = dv / dp::kBwdBV;
  a.nh_magic = fa.nh_magic;
  a.nh_shift = fa.nh_shift;
  if (a.RT != 16 && a.RT != 32) return DP_ENOTSUP;
  if (dry) return DP_OK;
  const hipError_t e = dispatch_bwd(elem, dk, fa, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

hipError_t dispatch_precond_bwd(int elem, int dk, const dp::PrecondBwdArgs& a, hipStream_t st) {
  if (elem == 4) {
    switch (dk) {
      case 16: return dp_launch_precond_bwd_f32_16(a, st);
      case 32: return dp_launch_precond_bwd_f32_32(a, st);
      case 64: return dp_launch_precond_bwd_f32_64(a, st);
      case 128: return dp_launch_precond_bwd_f32_128(a, st);
    }
  } else {
    switch (dk) {
      case 16: return dp_launch_precond_bwd_bf16_16(a, st);
      case 32: return dp_launch_precond_bwd_bf16_32(a, st);
      case 64: return dp_launch_precond_bwd_bf16_64(a, st);
      case 128: return dp_launch_precond_bwd_bf16_128(a, st);
    }
  }
  return hipErrorInvalidValue;
}

// Gradient of phase 1: the workspace holds d (B H dk f32), the trajectory of
// d (B L H dk f32), the write keys the forward emits again (B L H dk elements
// of the input type; sized for fp32), then for the reverse scan the
// projection mask (B L H dk bytes), the per-token factors (B L H float4) and
// the gradient each token receives (B L H dk f32).  The forward's chunked
// form (dk >= 64) uses the region of the last three before the reverse scan
// needs it, so that region is the larger of the two.
struct PrecondBwdWs {
  size_t d, dtr, kt, msk, fac, gin, rev, total;
};
PrecondBwdWs precond_bwd_ws(int B, int H, int L, int dk) {
  PrecondBwdWs w;
  const size_t n = (size_t)B * L * H;
  w.d = align_up((size_t)B * H * dk * 4, kWsAlign);
  w.dtr = align_up(n * dk * 4, kWsAlign);
  w.kt = w.dtr;
  w.msk = align_up(n * dk, kWsAlign);
  w.fac = align_up(n * 16, kWsAlign);
  w.gin = w.dtr;
  w.rev = std::max(w.msk + w.fac + w.gin, p1c_ws(B, H, L, dk).total);
  w.total = w.d + w.dtr + w.kt + w.rev;
  return w;
}

// Phase 1 forward into `ws` with its trajectory of d: d_1 is d0 (NULL: ones).
hipError_t precond_traj(int elem, const void* k, const float* beta, const float* ret, const float* d0,
                        int flags, int B, int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                        char* ws, void* kt_ws, hipStream_t st) {
  const PrecondBwdWs w = precond_bwd_ws(B, H, L, dk);
  float* dws = reinterpret_cast<float*>(ws);
  if (d0 != nullptr) {
    const hipError_t e = hipMemcpyAsync(dws, d0, (size_t)B * H * dk * 4, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  dp::PrecondArgs a;
  a.k = k;
  a.beta = beta;
  a.ret = ret;
  a.d = dws;
  a.kt = kt_ws;
  a.B = B;
  a.H = H;
  a.L = L;
  a.beta_aware = (flags & DP_PRECOND_BETA_FREE) ? 0 : 1;
  a.eta = eta;
  a.dmin = dmin;
  a.dmax = dmax;
  a.eps = eps;
  a.dtr = reinterpret_cast<float*>(ws + w.d);
  a.d_ones = d0 == nullptr ? 1 : 0;
  if (dk >= 64) {
    p1c_bind(a, ws + w.d + w.dtr + w.kt, dk);
    return dispatch_precond_chunked(elem, dk, a, st);
  }
  return dispatch_precond(elem, dk, a, st);
}

// The reverse scan of phase 1, which adds its key and beta terms into dk_out
// and dbeta.  have_traj: `ws` already holds the trajectory of d (an earlier
// precond_traj on the same inputs); else phase 1 runs again first.
int precond_bwd_impl(int elem, const void* k, const float* beta, const float* ret, const float* d0,
                     const float* dkt, const float* dd_final, int flags, int B, int H, int L, int dk,
                     float eta, float dmin, float dmax, float eps, float* dk_out, float* dbeta,
                     float* dret, float* dd0, char* ws, void* kt_ws, dp_stream stream, bool dry,
                     bool have_traj = false) {
  const PrecondBwdWs w = precond_bwd_ws(B, H, L, dk);
  float* dws = reinterpret_cast<float*>(ws);
  float* dtr = reinterpret_cast<float*>(ws + w.d);
  // the forward's own checks (open box allowed, as for the variants)
  int rc = precond_impl(elem, k, beta, ret, flags, B, H, L, dk, eta, dmin, dmax, eps, dws, kt_ws, true,
                        stream, 0, 0, true);
  if (rc != DP_OK) return rc;
  if (L > 0 && (dkt == nullptr || dk_out == nullptr || dbeta == nullptr)) return DP_EINVAL;
  if (dry) return DP_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // (with L == 0 both kernels run no token: the reverse scan writes dd0 = dd_final)
  if (!have_traj) {
    const hipError_t e = precond_traj(elem, k, beta, ret, d0, flags, B, H, L, dk, eta, dmin, dmax, eps, ws,
                                      kt_ws, st);
    if (e != hipSuccess) return DP_EHIP;
  }
  dp::PrecondBwdArgs g;
  g.k = k;
  g.beta = beta;
  g.ret = ret;
  g.dtr = dtr;
  g.dkt = dkt;
  g.dd_final = dd_final;
  g.dk = dk_out;
  g.dbeta = dbeta;
  g.dret = dret;
  g.dd0 = dd0;
  g.msk = reinterpret_cast<unsigned char*>(ws + w.d + w.dtr + w.kt);
  g.fac = reinterpret_cast<float4*>(ws + w.d + w.dtr + w.kt + w.msk);
  g.gin = reinterpret_cast<float*>(ws + w.d + w.dtr + w.kt + w.msk + w.fac);
  g.B = B;
  g.H = H;
  g.L = L;
  g.beta_aware = (flags & DP_PRECOND_BETA_FREE) ? 0 : 1;
  g.eta = eta;
  g.dmin = dmin;
  g.dmax = dmax;
  g.eps = eps;
  return dispatch_precond_bwd(elem, dk, g, st) == hipSuccess ? DP_OK : DP_EHIP;
}

// The whole OSDN layer's gradient (n_h = 1): phase 1 again, the write-key
// backward, then phase 1's reverse scan into the same dk and dbeta.
struct OsdnBwdWs {
  size_t p1, kt, dkt, bwd, total;
};
OsdnBwdWs osdn_bwd_ws(int B, int H, int L, int dk, int dv) {
  OsdnBwdWs w;
  w.p1 = precond_bwd_ws(B, H, L, dk).total;
  w.kt = align_up((size_t)B * L * H * dk * 4, kWsAlign);
  w.dkt = w.kt;
  const Shape s{1, B, H, L, dk, dv, dp::kBwdChunk};
  w.bwd = bwd_ws(s).total;
  w.total = w.p1 + w.kt + w.dkt + w.bwd;
  return w;
}

int osdn_bwd_impl(int elem, const void* q, const void* k, const void* v, const float* beta,
                  const float* g, const float* h0, const float* ret, const float* d0, const void* dout,
                  const float* dfinal, const float* dd_final, int flags, int B, int H, int L, int dk,
                  int dv, float eta, float dmin, float dmax, float eps, float* dq, float* dk_out,
                  float* dv_out, float* dbeta, float* dg, float* dh0, float* dret, float* dd0,
                  void* workspace, size_t workspace_bytes, dp_stream stream) {
  const Shape s{1, B, H, L, dk, dv, dp::kBwdChunk};
  int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  if (L > 0 && (q == nullptr || v == nullptr || dout == nullptr || dq == nullptr || dv_out == nullptr))
    return DP_EINVAL;
  const OsdnBwdWs w = osdn_bwd_ws(B, H, L, dk, dv);
  if (workspace_bytes < w.total || workspace == nullptr) return DP_EWORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* kt = ws + w.p1;
  float* dkt = reinterpret_cast<float*>(ws + w.p1 + w.kt);
  char* bws = ws + w.p1 + w.kt + w.dkt;
  char* p1ws = ws;
  // every check first: nothing is enqueued when any of them fails
  rc = precond_bwd_impl(elem, k, beta, ret, d0, dkt, dd_final, flags, B, H, L, dk, eta, dmin, dmax, eps,
                        dk_out, dbeta, dret, dd0, p1ws, kt, stream, true);
  if (rc != DP_OK) return rc;
  rc = bwd_impl(elem, q, k, v, beta, g, h0, dout, dfinal, 1, B, H, L, dk, dv, dq, dk_out, dv_out, dbeta, dg,
                dh0, bws, w.bwd, stream, kt, dkt, true, true);
  if (rc != DP_OK) return rc;
  // phase 1 forward: the write keys for the write-key backward, and the trajectory of d
  if (precond_traj(elem, k, beta, ret, d0, flags, B, H, L, dk, eta, dmin, dmax, eps, p1ws, kt,
                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return DP_EHIP;
  rc = bwd_impl(elem, q, k, v, beta, g, h0, dout, dfinal, 1, B, H, L, dk, dv, dq, dk_out, dv_out, dbeta, dg,
                dh0, bws, w.bwd, stream, kt, dkt, true);
  if (rc != DP_OK) return rc;
  return precond_bwd_impl(elem, k, beta, ret, d0, dkt, dd_final, flags, B, H, L, dk, eta, dmin, dmax, eps,
                          dk_out, dbeta, dret, dd0, p1ws, kt, stream, false, true);
}

}  // namespace

extern "C" {

const char* dp_status_str(int status) {
  switch (status) {
    case DP_OK: return "DP_OK";
    case DP_EINVAL: return "DP_EINVAL: invalid argument (null pointer, size or alignment)";
    case DP_ENOTSUP: return "DP_ENOTSUP: unsupported shape (dk/dv/chunk/n_h)";
    case DP_EWORKSPACE: return "DP_EWORKSPACE: workspace missing, misaligned or too small";
    case DP_EHIP: return "DP_EHIP: HIP launch or runtime error";
    case DP_ESCRATCH: return "DP_ESCRATCH: more sequences than the no-alloc entry point's fixed scratch holds";
    default: return "unknown dp status";
  }
}

int dp_fwd_workspace_size(int n_h, int B, int H, int L, int dk, int dv, int chunk,
                          int elem_bytes, size_t* bytes) {
  if (bytes == nullptr) return DP_EINVAL;
  if (elem_bytes != 2 && elem_bytes != 4) return DP_EINVAL;
  const Shape s{n_h, B, H, L, dk, dv, chunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  *bytes = ws_total(s, elem_bytes);
  return DP_OK;
}

int dp_fwd_launch_info(int n_h, int B, int H, int L, int dk, int dv, int chunk, int elem_bytes,
                       int asym, int* info) {
  if (info == nullptr || (elem_bytes != 2 && elem_bytes != 4) || (asym != 0 && asym != 1))
    return DP_EINVAL;
  const Shape s{n_h, B, H, L, dk, dv, chunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  dp::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.H = H;
  a.dv = dv;
  a.RT = readout_rows(chunk, n_h);
  a.asym = asym;
  a.fused = use_fused(elem_bytes, asym != 0, dk, dv, chunk, DP_STAGE_ALL) ? 1 : 0;
  int BV = 0, lds = 0;
  const int prc = plan(a, elem_bytes, dk, chunk, &BV, &lds);
  if (prc != DP_OK) return prc;
  info[0] = BV;
  info[1] = B * H * a.nvb;
  info[2] = a.fused ? 0 : B * H * num_chunks(s);
  info[3] = lds;
  info[4] = a.fused                                               ? 0
            : (elem_bytes == 2 && (!asym || dp::chain_asym_ok(dk, chunk))) ? dp::prep_lds_bytes(dk, chunk, a.RT, asym != 0)
                                                                    : ut_lds(elem_bytes, dk, chunk, asym);
  info[5] = a.RT;
  return DP_OK;
}

int dp_fwd_f32(const float* q, const float* k, const float* v, const float* beta,
               const float* g, int n_h, int B, int H, int L, int dk, int dv, int chunk,
               float* out, float* final_state, const float* h0, void* workspace,
               size_t workspace_bytes, dp_stream stream) {
  return fwd_impl(4, q, k, nullptr, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state,
                  h0, workspace, workspace_bytes, DP_STAGE_ALL, stream);
}

int dp_fwd_bf16(const void* q, const void* k, const void* v, const float* beta,
                const float* g, int n_h, int B, int H, int L, int dk, int dv, int chunk,
                void* out, float* final_state, const float* h0, void* workspace,
                size_t workspace_bytes, dp_stream stream) {
  return fwd_impl(2, q, k, nullptr, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state,
                  h0, workspace, workspace_bytes, DP_STAGE_ALL, stream);
}

int dp_fwd_wk_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, int n_h, int B, int H, int L, int dk,
                  int dv, int chunk, float* out, float* final_state, const float* h0,
                  void* workspace, size_t workspace_bytes, dp_stream stream) {
  if (kt == nullptr) return DP_EINVAL;
  return fwd_impl(4, q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state, h0,
                  workspace, workspace_bytes, DP_STAGE_ALL, stream);
}

int dp_fwd_wk_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, int n_h, int B, int H, int L, int dk,
                   int dv, int chunk, void* out, float* final_state, const float* h0,
                   void* workspace, size_t workspace_bytes, dp_stream stream) {
  if (kt == nullptr) return DP_EINVAL;
  return fwd_impl(2, q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state, h0,
                  workspace, workspace_bytes, DP_STAGE_ALL, stream);
}

int dp_fwd_ex_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, const float* ga, int n_h, int B, int H, int L,
                  int dk, int dv, int chunk, float* out, float* final_state, const float* h0,
                  void* workspace, size_t workspace_bytes, int flags, dp_stream stream) {
  return fwd_impl(4, q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state, h0,
                  workspace, workspace_bytes, flags, stream, 0, 0, false, ga);
}

int dp_fwd_ex_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, const float* ga, int n_h, int B, int H, int L,
                   int dk, int dv, int chunk, void* out, float* final_state, const float* h0,
                   void* workspace, size_t workspace_bytes, int flags, dp_stream stream) {
  return fwd_impl(2, q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, chunk, out, final_state, h0,
                  workspace, workspace_bytes, flags, stream, 0, 0, false, ga);
}

int dp_osdn_precond_f32(const float* k, const float* beta, int B, int H, int L, int dk,
                        float eta, float dmin, float dmax, float eps, float* d_state,
                        float* kt, dp_stream stream) {
  return precond_impl(4, k, beta, nullptr, 0, B, H, L, dk, eta, dmin, dmax, eps, d_state, kt,
                      false, stream);
}

int dp_osdn_precond_bf16(const void* k, const float* beta, int B, int H, int L, int dk,
                         float eta, float dmin, float dmax, float eps, float* d_state,
                         void* kt, dp_stream stream) {
  return precond_impl(2, k, beta, nullptr, 0, B, H, L, dk, eta, dmin, dmax, eps, d_state, kt,
                      false, stream);
}

int dp_osdn_precond_ex_f32(const float* k, const float* beta, const float* r, int flags, int B,
                           int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                           float* d_state, float* kt, dp_stream stream) {
  return precond_impl(4, k, beta, r, flags, B, H, L, dk, eta, dmin, dmax, eps, d_state, kt, true,
                      stream);
}

int dp_osdn_precond_ex_bf16(const void* k, const float* beta, const float* r, int flags, int B,
                            int H, int L, int dk, float eta, float dmin, float dmax, float eps,
                            float* d_state, void* kt, dp_stream stream) {
  return precond_impl(2, k, beta, r, flags, B, H, L, dk, eta, dmin, dmax, eps, d_state, kt, true,
                      stream);
}

int dp_osdn_precond_varlen_workspace_size(int nseq, int H, int T, int dk, size_t* bytes) {
  if (bytes == nullptr || nseq <= 0 || H <= 0 || T < 0) return DP_EINVAL;
  if (!dim_ok(dk)) return DP_ENOTSUP;
  *bytes = p1c_ws_var(nseq, H, T, dk).total;
  return DP_OK;
}

namespace {
int precond_varlen(int elem, const void* k, const float* beta, const float* r, int flags,
                   const int* cu_seqlens, int nseq, int H, int T, int dk, float eta, float dmin,
                   float dmax, float eps, float* d_state, void* kt, void* workspace,
                   size_t workspace_bytes, dp_stream stream) {
  if (cu_seqlens == nullptr || nseq <= 0 || H <= 0 || T < 0) return DP_EINVAL;
  char* p1c = nullptr;
  if (workspace != nullptr && dim_ok(dk)) {
    const size_t need = p1c_ws_var(nseq, H, T, dk).total;
    if (workspace_bytes < need || ((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
    if (need > 0) p1c = static_cast<char*>(workspace);
  }
  if ((long long)H * ((T + dp::kP1Chunk - 1) / dp::kP1Chunk + (long long)nseq) > (long long)INT_MAX)
    return DP_ENOTSUP;
  return precond_impl(elem, k, beta, r, flags, nseq, H, T, dk, eta, dmin, dmax, eps, d_state, kt, true,
                      stream, 0, 0, false, p1c, cu_seqlens);
}
}  // namespace

int dp_osdn_precond_varlen_f32(const float* k, const float* beta, const float* r, int flags,
                               const int* cu_seqlens, int nseq, int H, int T, int dk, float eta,
                               float dmin, float dmax, float eps, float* d_state, float* kt,
                               void* workspace, size_t workspace_bytes, dp_stream stream) {
  return precond_varlen(4, k, beta, r, flags, cu_seqlens, nseq, H, T, dk, eta, dmin, dmax, eps, d_state,
                        kt, workspace, workspace_bytes, stream);
}

int dp_osdn_precond_varlen_bf16(const void* k, const float* beta, const float* r, int flags,
                                const int* cu_seqlens, int nseq, int H, int T, int dk, float eta,
                                float dmin, float dmax, float eps, float* d_state, void* kt,
                                void* workspace, size_t workspace_bytes, dp_stream stream) {
  return precond_varlen(2, k, beta, r, flags, cu_seqlens, nseq, H, T, dk, eta, dmin, dmax, eps, d_state,
                        kt, workspace, workspace_bytes, stream);
}

int dp_osdn_fwd_workspace_size(int B, int H, int L, int dk, int dv, int chunk, int segments,
                               size_t* bytes) {
  if (bytes == nullptr || segments < 1 || segments > kMaxSegments || chunk <= 0 || L < 0) return DP_EINVAL;
  const Shape s{1, B, H, seg_len(L, chunk, segments), dk, dv, chunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  *bytes = align_up(ws_total(s, 2), kWsAlign) + p1c_ws(B, H, s.L, dk).total;
  return DP_OK;
}

int dp_pipeline_create(dp_pipeline* out) {
  if (out == nullptr) return DP_EINVAL;
  *out = nullptr;
  dp_pipeline p = new (std::nothrow) dp_pipeline_s;
  if (p == nullptr) return DP_EHIP;
  bool ok = hipGetDevice(&p->device) == hipSuccess &&
            hipStreamCreateWithFlags(&p->st2, hipStreamNonBlocking) == hipSuccess;
  for (int i = 0; ok && i <= kMaxSegments; ++i)
    ok = hipEventCreateWithFlags(&p->ev[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    release_pipeline(p);
    return DP_EHIP;
  }
  *out = p;
  return DP_OK;
}

int dp_pipeline_destroy(dp_pipeline pipe) {
  if (pipe == nullptr) return DP_OK;
  const hipError_t e = hipStreamSynchronize(pipe->st2);
  release_pipeline(pipe);
  return e == hipSuccess ? DP_OK : DP_EHIP;
}

int dp_osdn_fwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* h0,
                     int B, int H, int L, int dk, int dv, int chunk, float eta, float dmin, float dmax,
                     float eps, float* d_state, void* kt, void* out, float* final_state, void* workspace,
                     size_t workspace_bytes, int segments, dp_pipeline pipe, dp_stream stream) {
  if (segments < 1 || segments > kMaxSegments || chunk <= 0 || L < 0) return DP_EINVAL;
  const int len = seg_len(L, chunk, segments);
  const int nseg = L > 0 ? (L + len - 1) / len : 0;
  const Shape s{1, B, H, len, dk, dv, chunk};
  int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  if (nseg > 1 && final_state == nullptr) return DP_EINVAL;  // the state passes through it
  if (L > 0 && (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || out == nullptr ||
                kt == nullptr || d_state == nullptr))
    return DP_EINVAL;
  // the workspace: one run's forward, then (dk >= 64) one run's chunked phase 1
  const size_t fws = align_up(ws_total(s, 2), kWsAlign);
  const size_t need = fws + p1c_ws(B, H, len, dk).total;
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return DP_EWORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
  char* p1c = p1c_ws(B, H, len, dk).total > 0 ? static_cast<char*>(workspace) + fws : nullptr;
  if (nseg == 0) return fwd_impl(2, q, k, k, v, beta, nullptr, 1, B, H, 0, dk, dv, chunk, out, final_state,
                                 h0, workspace, workspace_bytes, DP_STAGE_ALL, stream);
  // Check every run before enqueueing the first.  The runs differ only in
  // their token count (len, the last one at most len) and offset: a full run
  // passes the same shape, pointer, workspace and plan checks as each of them.
  rc = precond_impl(2, k, beta, nullptr, 0, B, H, len, dk, eta, dmin, dmax, eps, d_state, kt, false,
                    stream, L, 0, true);
  if (rc != DP_OK) return rc;
  rc = fwd_impl(2, q, k, kt, v, beta, nullptr, 1, B, H, len, dk, dv, chunk, out, final_state, h0,
                workspace, fws, DP_STAGE_ALL, stream, L, 0, true);
  if (rc != DP_OK) return rc;
  std::unique_lock<std::mutex> hold;
  if (pipe != nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DP_EHIP;
    if (dev != pipe->device) return DP_EINVAL;
    hold = std::unique_lock<std::mutex>(pipe->mu);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStream_t st2 = pipe != nullptr ? pipe->st2 : st;
  for (int sg = 0; sg < nseg; ++sg) {
    const int t0 = sg * len, n = L - t0 < len ? L - t0 : len;
    rc = precond_impl(2, k, beta, nullptr, 0, B, H, n, dk, eta, dmin, dmax, eps, d_state, kt, false,
                      stream, L, t0, false, p1c);
    if (rc != DP_OK) return rc;
    if (pipe != nullptr && (hipEventRecord(pipe->ev[sg], st) != hipSuccess ||
                            hipStreamWaitEvent(st2, pipe->ev[sg], 0) != hipSuccess))
      return DP_EHIP;
    rc = fwd_impl(2, q, k, kt, v, beta, nullptr, 1, B, H, n, dk, dv, chunk, out, final_state,
                  sg == 0 ? h0 : final_state, workspace, fws, DP_STAGE_ALL, st2, L, t0);
    if (rc != DP_OK) return rc;
  }
  if (pipe != nullptr && (hipEventRecord(pipe->ev[kMaxSegments], st2) != hipSuccess ||
                          hipStreamWaitEvent(st, pipe->ev[kMaxSegments], 0) != hipSuccess))
    return DP_EHIP;
  return DP_OK;
}

int dp_fwd_varlen_workspace_size(int n_h, int nseq, int H, int T, int dk, int dv, int chunk,
                                 size_t* bytes) {
  if (bytes == nullptr) return DP_EINVAL;
  const VarShape vs{n_h, nseq, H, T, dk, dv, chunk};
  const int rc = check_varlen(vs);
  if (rc != DP_OK) return rc;
  *bytes = varlen_ws_total(vs);
  return DP_OK;
}

int dp_fwd_varlen_bf16(const void* q, const void* k, const void* v, const float* beta,
                       const float* g, const int* cu_seqlens, int nseq, int n_h, int H, int T,
                       int dk, int dv, int chunk, void* out, float* final_state, const float* h0,
                       void* workspace, size_t workspace_bytes, int flags, dp_stream stream) {
  return varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out, final_state,
                     h0, workspace, workspace_bytes, flags, stream);
}

int dp_fwd_varlen_f32(const float* q, const float* k, const float* v, const float* beta,
                      const float* g, const int* cu_seqlens, int nseq, int n_h, int H, int T,
                      int dk, int dv, int chunk, float* out, float* final_state, const float* h0,
                      void* workspace, size_t workspace_bytes, int flags, dp_stream stream) {
  return varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out, final_state,
                     h0, workspace, workspace_bytes, flags, stream, nullptr, false, nullptr, 4);
}

int dp_fwd_varlen_wk_f32(const float* q, const float* k, const float* kt, const float* v,
                         const float* beta, const float* g, const int* cu_seqlens, int nseq,
                         int n_h, int H, int T, int dk, int dv, int chunk, float* out,
                         float* final_state, const float* h0, void* workspace,
                         size_t workspace_bytes, int flags, dp_stream stream) {
  if (T > 0 && kt == nullptr) return DP_EINVAL;
  return varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out, final_state,
                     h0, workspace, workspace_bytes, flags, stream, nullptr, false, kt, 4);
}

int dp_fwd_varlen_wk_bf16(const void* q, const void* k, const void* kt, const void* v,
                          const float* beta, const float* g, const int* cu_seqlens, int nseq,
                          int n_h, int H, int T, int dk, int dv, int chunk, void* out,
                          float* final_state, const float* h0, void* workspace,
                          size_t workspace_bytes, int flags, dp_stream stream) {
  if (T > 0 && kt == nullptr) return DP_EINVAL;
  return varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out, final_state,
                     h0, workspace, workspace_bytes, flags, stream, nullptr, false, kt);
}

int dp_fwd_varlen_noalloc_bf16(const void* q, const void* k, const void* v, const float* beta,
                               const float* g, const int* cu_seqlens, int nseq, int n_h, int H,
                               int T, int dk, int dv, int chunk, void* out, float* final_state,
                               const float* h0, int flags, dp_stream stream) {
  if ((flags & ~DP_OUT_F32) != 0) return DP_EINVAL;
  if (nseq > DP_NOALLOC_MAX_SEQS) return DP_ESCRATCH;
  const int f = DP_STAGE_ALL | DP_FWD_FUSED | flags;
  // every check first, before any HIP call; the table address only marks the
  // table-only form here and is not read
  int* const mark = reinterpret_cast<int*>(kWsAlign);
  int rc = varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out,
                       final_state, h0, nullptr, 0, f, stream, mark, true);
  if (rc != DP_OK) return rc;
  int* const table = scratch_on_current_device();
  if (table == nullptr) return DP_EHIP;
  return varlen_impl(q, k, v, beta, g, cu_seqlens, nseq, n_h, H, T, dk, dv, chunk, out, final_state,
                     h0, nullptr, 0, f, stream, table, false);
}

int dp_decode_f32(const float* q, const float* k, const float* kt, const float* v,
                  const float* beta, const float* g, const float* ga, int n_h, int B, int H,
                  int dk, int dv, float* out, float* state, int flags, dp_stream stream) {
  return decode_impl(4, q, k, kt, v, beta, g, ga, n_h, B, H, dk, dv, out, state, flags, stream);
}

int dp_decode_bf16(const void* q, const void* k, const void* kt, const void* v,
                   const float* beta, const float* g, const float* ga, int n_h, int B, int H,
                   int dk, int dv, void* out, float* state, int flags, dp_stream stream) {
  return decode_impl(2, q, k, kt, v, beta, g, ga, n_h, B, H, dk, dv, out, state, flags, stream);
}

int dp_bwd_workspace_size(int n_h, int B, int H, int L, int dk, int dv, size_t* bytes) {
  if (bytes == nullptr) return DP_EINVAL;
  const Shape s{n_h, B, H, L, dk, dv, dp::kBwdChunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  *bytes = bwd_ws(s).total;
  return DP_OK;
}

int dp_bwd_f32(const float* q, const float* k, const float* v, const float* beta, const float* g,
               const float* h0, const float* dout, const float* dfinal, int n_h, int B, int H,
               int L, int dk, int dv, float* dq, float* dk_out, float* dv_out, float* dbeta,
               float* dg, float* dh0, void* workspace, size_t workspace_bytes, dp_stream stream) {
  return bwd_impl(4, q, k, v, beta, g, h0, dout, dfinal, n_h, B, H, L, dk, dv, dq, dk_out, dv_out,
                  dbeta, dg, dh0, workspace, workspace_bytes, stream);
}

int dp_bwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* g,
                const float* h0, const void* dout, const float* dfinal, int n_h, int B, int H,
                int L, int dk, int dv, float* dq, float* dk_out, float* dv_out, float* dbeta,
                float* dg, float* dh0, void* workspace, size_t workspace_bytes, dp_stream stream) {
  return bwd_impl(2, q, k, v, beta, g, h0, dout, dfinal, n_h, B, H, L, dk, dv, dq, dk_out, dv_out,
                  dbeta, dg, dh0, workspace, workspace_bytes, stream);
}

int dp_bwd_wk_f32(const float* q, const float* k, const float* kt, const float* v, const float* beta,
                  const float* g, const float* h0, const float* dout, const float* dfinal, int n_h, int B,
                  int H, int L, int dk, int dv, float* dq, float* dk_out, float* dkt, float* dv_out,
                  float* dbeta, float* dg, float* dh0, void* workspace, size_t workspace_bytes,
                  dp_stream stream) {
  return bwd_impl(4, q, k, v, beta, g, h0, dout, dfinal, n_h, B, H, L, dk, dv, dq, dk_out, dv_out,
                  dbeta, dg, dh0, workspace, workspace_bytes, stream, kt, dkt, true);
}

int dp_bwd_wk_bf16(const void* q, const void* k, const void* kt, const void* v, const float* beta,
                   const float* g, const float* h0, const void* dout, const float* dfinal, int n_h, int B,
                   int H, int L, int dk, int dv, float* dq, float* dk_out, float* dkt, float* dv_out,
                   float* dbeta, float* dg, float* dh0, void* workspace, size_t workspace_bytes,
                   dp_stream stream) {
  return bwd_impl(2, q, k, v, beta, g, h0, dout, dfinal, n_h, B, H, L, dk, dv, dq, dk_out, dv_out,
                  dbeta, dg, dh0, workspace, workspace_bytes, stream, kt, dkt, true);
}

int dp_osdn_precond_bwd_workspace_size(int B, int H, int L, int dk, size_t* bytes) {
  if (bytes == nullptr) return DP_EINVAL;
  if (B <= 0 || H <= 0 || L < 0) return DP_EINVAL;
  if (!dim_ok(dk)) return DP_ENOTSUP;
  if ((long long)B * H * (long long)L > (long long)1 << 40) return DP_ENOTSUP;
  *bytes = precond_bwd_ws(B, H, L, dk).total;
  return DP_OK;
}

static int precond_bwd_entry(int elem, const void* k, const float* beta, const float* r, const float* d0,
                             const float* dkt, const float* dd_final, int flags, int B, int H, int L,
                             int dk, float eta, float dmin, float dmax, float eps, float* dk_out,
                             float* dbeta, float* dret, float* dd0, void* workspace,
                             size_t workspace_bytes, dp_stream stream) {
  size_t need = 0;
  const int rc = dp_osdn_precond_bwd_workspace_size(B, H, L, dk, &need);
  if (rc != DP_OK) return rc;
  if (workspace == nullptr || workspace_bytes < need) return DP_EWORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return DP_EWORKSPACE;
  const PrecondBwdWs w = precond_bwd_ws(B, H, L, dk);
  char* ws = static_cast<char*>(workspace);
  return precond_bwd_impl(elem, k, beta, r, d0, dkt, dd_final, flags, B, H, L, dk, eta, dmin, dmax, eps,
                          dk_out, dbeta, dret, dd0, ws, ws + w.d + w.dtr, stream, false);
}

int dp_osdn_precond_bwd_f32(const float* k, const float* beta, const float* r, const float* d0,
                            const float* dkt, const float* dd_final, int flags, int B, int H, int L,
                            int dk, float eta, float dmin, float dmax, float eps, float* dk_out,
                            float* dbeta, float* dret, float* dd0, void* workspace,
                            size_t workspace_bytes, dp_stream stream) {
  return precond_bwd_entry(4, k, beta, r, d0, dkt, dd_final, flags, B, H, L, dk, eta, dmin, dmax, eps,
                           dk_out, dbeta, dret, dd0, workspace, workspace_bytes, stream);
}

int dp_osdn_precond_bwd_bf16(const void* k, const float* beta, const float* r, const float* d0,
                             const float* dkt, const float* dd_final, int flags, int B, int H, int L,
                             int dk, float eta, float dmin, float dmax, float eps, float* dk_out,
                             float* dbeta, float* dret, float* dd0, void* workspace,
                             size_t workspace_bytes, dp_stream stream) {
  return precond_bwd_entry(2, k, beta, r, d0, dkt, dd_final, flags, B, H, L, dk, eta, dmin, dmax, eps,
                           dk_out, dbeta, dret, dd0, workspace, workspace_bytes, stream);
}

int dp_osdn_bwd_workspace_size(int B, int H, int L, int dk, int dv, size_t* bytes) {
  if (bytes == nullptr) return DP_EINVAL;
  const Shape s{1, B, H, L, dk, dv, dp::kBwdChunk};
  const int rc = check_shape(s);
  if (rc != DP_OK) return rc;
  *bytes = osdn_bwd_ws(B, H, L, dk, dv).total;
  return DP_OK;
}

int dp_osdn_bwd_f32(const float* q, const float* k, const float* v, const float* beta, const float* g,
                    const float* h0, const float* r, const float* d0, const float* dout,
                    const float* dfinal, const float* dd_final, int flags, int B, int H, int L, int dk,
                    int dv, float eta, float dmin, float dmax, float eps, float* dq, float* dk_out,
                    float* dv_out, float* dbeta, float* dg, float* dh0, float* dret, float* dd0,
                    void* workspace, size_t workspace_bytes, dp_stream stream) {
  return osdn_bwd_impl(4, q, k, v, beta, g, h0, r, d0, dout, dfinal, dd_final, flags, B, H, L, dk, dv, eta,
                       dmin, dmax, eps, dq, dk_out, dv_out, dbeta, dg, dh0, dret, dd0, workspace,
                       workspace_bytes, stream);
}

int dp_osdn_bwd_bf16(const void* q, const void* k, const void* v, const float* beta, const float* g,
                     const float* h0, const float* r, const float* d0, const void* dout,
                     const float* dfinal, const float* dd_final, int flags, int B, int H, int L, int dk,
                     int dv, float eta, float dmin, float dmax, float eps, float* dq, float* dk_out,
                     float* dv_out, float* dbeta, float* dg, float* dh0, float* dret, float* dd0,
                     void* workspace, size_t workspace_bytes, dp_stream stream) {
  return osdn_bwd_impl(2, q, k, v, beta, g, h0, r, d0, dout, dfinal, dd_final, flags, B, H, L, dk, dv, eta,
                       dmin, dmax, eps, dq, dk_out, dv_out, dbeta, dg, dh0, dret, dd0, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
