// dp_fused.hpp -- the bf16 forward with symmetric keys in one kernel.
//
// Same chunkwise form as the rest of the library (DeltaProduct study notes
// sec. 2.2 Eq.(3), sec. 2.6 and sec. 4.1; WY/UT chunk form of the OSDN study
// notes sec. 2.5 / App. A.2, with the chunk-local log-gate G):
//
//   A  = E o (Kn Kn^T),  E_ij = e^{G_i - G_j}
//   (I + strict_tril(diag(beta) A)) Up = diag(beta) (V - diag(e^G) Kn H0)
//   O  = diag(e^{G_loc}) Q H0 + P Up,   P = (tril_incl(Q Kn^T) o E) on readout rows
//   H1 = e^{G_last} H0 + Kn^T (diag(e^{G_last - G}) Up)
//
// One workgroup owns one head and 16 NWC value columns, and walks the chunks
// of the head in order.  Nothing is staged through HBM: every operand that
// does not depend on the state is built on chip, from one read of the raw
// keys, queries and beta, while the recurrence runs.
//
// Wavefronts (the first four land on four different SIMDs):
//   consumers  NWC wavefronts, 16 value columns each: the fp32 state slice in
//              registers and the chunk's MFMA steps (X, readout, Up, state).
//   producers  two wavefronts; producer k builds the operands of chunks
//              k, k + 2, k + 4, .. over two periods each:
//                first half  (two periods ahead of the consumers): the Gram
//                            matrix K K^T on bf16 MFMA straight from the raw
//                            key registers, the key norms from its diagonal,
//                            the unit keys and the queries as fp16 tiles, M.
//                second half (one period ahead): the 16 x 16 diagonal blocks
//                            of T = (I + M)^{-1} by forward substitution, the
//                            off-diagonal block of each 32-row half on
//                            split-fp16 MFMA (fp32 accuracy), T diag(beta)
//                            as fp16, and the masked scores P.
//              Each producer loads its next chunk's raw rows into registers
//              as soon as its first half has consumed the current ones.
//   copy       one wavefront: the value tile of each chunk into an LDS ring
//              with direct-to-LDS copies, three chunks ahead, and early
//              single-dword touches of later chunks' rows (into a dummy LDS
//              word) so that the producers' loads find them in L2.
// One workgroup barrier per chunk ("period") orders everything.
//
// The 64-row chunk is solved as two 32-row halves a and b:
//   Ua = (T_aa diag(beta_a)) Xa
//   Ub = (T_bb diag(beta_b)) (Xb - A_ba Ua)
// which is the block forward substitution of (I + M) Up = diag(beta) X.  So
// the off-diagonal 32 x 32 block of T is never formed; the consumers apply
// A_ba instead, with the same number of MFMA steps as T_ba would cost.
#pragma once

#include "dp_fwd16.hpp"

namespace dp {

constexpr int kFusedKQ = 3;    // slots of the key and query rings
constexpr int kFusedT = 2;     // slots of the T, score and scalar rings
constexpr int kFusedV = 3;     // slots of the value ring
constexpr int kFusedAux = 5;   // producer (two pairs) and copy wavefronts besides the consumers
constexpr int kFusedTouchLead = 6;  // chunks between a chunk's L2 touch and its consumption

// The fused kernel needs dk and chunk multiples of 32 (whole 32-deep MFMA steps).
__host__ __device__ constexpr bool fused_ok(int DK, int C) { return DK % 32 == 0 && C % 32 == 0; }

// LDS of dp_fused_kernel: rings of per-chunk operands and two producer scratch areas.
struct FusedLayout {
  int oK, oQ, oT, oP, oS, oV, oW, oD;  // ring bases; producer scratch; touch sink
  int sK, sQ, sT, sP, sS, sV, sW;      // slot sizes
  int wR, wB, wG, wL;                  // scratch: 1/|k|, beta, G, readout locations (M/T blocks at 0)
  int bytes;
};

__host__ __device__ constexpr FusedLayout fused_layout(int DK, int C, int RT, int BV) {
  FusedLayout L{};
  L.sK = C * DK * 2;                    // unit keys, plain blocks (read by rows and transposed)
  L.sQ = RT * DK * 2;                   // readout queries, fragment layout
  L.sT = t_bytes(DK, C);                // T diag(beta) and -A_ba, fragment layout
  L.sP = RT * C * 2;                    // masked scores, fragment layout
  L.sS = ((2 * C + RT) * 4 + 15) & ~15; // e^G, e^{G_last - G}, e^{G_loc}
  L.sV = C * BV * 2;                    // value tile, row-major
  L.wR = (C / 32) * 3 * kPrepBlk * 4;   // three 16 x 16 fp32 blocks per 32-row half
  L.wB = L.wR + C * 4;
  L.wG = L.wB + C * 4;
  L.wL = L.wG + C * 4;
  L.sW = (L.wL + RT * 4 + 32 * 4 + 15) & ~15;  // + role b's copy of half a's 1/|k|
  L.oK = 0;
  L.oQ = L.oK + kFusedKQ * L.sK;
  L.oT = L.oQ + kFusedKQ * L.sQ;
  L.oP = L.oT + kFusedT * L.sT;
  L.oS = L.oP + kFusedT * L.sP;
  L.oV = L.oS + kFusedT * L.sS;
  L.oW = L.oV + kFusedV * L.sV;
  L.oD = L.oW + 2 * L.sW;
  L.bytes = L.oD + 256;
  return L;
}

// Scratch block of the 16 x 16 block (ib, jb) of a 32-row half (ib / 2 == jb / 2, jb <= ib).
__host__ __device__ constexpr int fused_blk(int ib, int jb) { return 3 * (ib / 2) + (ib & 1) + (jb & 1); }

// Every LDS access this wavefront issued has completed; the compiler keeps
// LDS accesses on their side of it.  Orders exchanges between the lanes of
// one wavefront (other wavefronts synchronise through the workgroup barrier).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One single-dword direct-to-LDS load: each lane touches the 4 bytes at `src`
// (bringing its cache line into L2) and drops them into LDS at lds + 4 lane.
__device__ __forceinline__ void touch4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ float vpick(const f32x4_t& v, int e) {
  return e == 0 ? v[0] : (e == 1 ? v[1] : (e == 2 ? v[2] : v[3]));
}

// D += A B for 16 x 16 fp32 operands on fp16 MFMA, each operand split into a
// high and a low fp16 part: A_hi B_hi + A_lo B_hi in one 32-deep step (the two
// parts concatenated along k) and A_hi B_lo in a second, zero-padded 32-deep
// step.  The dropped A_lo B_lo term is 2^-22 of the product: fp32 accuracy at
// fp16 MFMA rate.  Both steps are the same instruction: a 16-deep step that
// accumulates onto a 32-deep step's result with the compiler's one or two wait
// states gave wrong sums on gfx950, while same-instruction chains are exact.
// a: lane (m, g) holds A[m][4g .. 4g+3];  b: lane (n, g) holds B[4g .. 4g+3][n].
__device__ __forceinline__ f32x4_t mm16_split(const f32x4_t& a, const f32x4_t& b, f32x4_t c) {
  const f16x4_t ah = to_h4(a), bh = to_h4(b);
  const f16x4_t al = to_h4(a - __builtin_convertvector(ah, f32x4_t));
  const f16x4_t bl = to_h4(b - __builtin_convertvector(bh, f32x4_t));
  const f16x4_t zero = {0, 0, 0, 0};
  c = mfma32h(cat8(ah, al), cat8(bh, bh), c);
  return mfma32h(cat8(ah, zero), cat8(bl, zero), c);
}

// --------------------------------------------------------------------------
// Consumer step schedule.  Kinds: 0 K H (X), 1 Q H (readout), 2 Ua, 3 Yb = Xb
// - A_ba Ua, 4 Ub, 5 P Up (readout), 6 Kn^T Us (state).  x is the output tile
// (key row tile, readout tile or state tile), k the 32-deep contraction step.
struct FStep {
  int kind, x, k;
};

template <int NCT, int KST, int NRT, int NDT>
struct FSched {
  static constexpr int CH = NCT / 2;
  static constexpr int NS = NCT * KST + NRT * KST + 2 * CH + (CH - 1) * 2 + NRT * CH + NDT * CH;
  FStep s[NS];
  constexpr FSched() : s{} {
    int n = 0;
    // X: the key row tiles of half a first (their X feeds Ua), contraction step outermost
    for (int half = 0; half < CH; ++half)
      for (int k = 0; k < KST; ++k)
        for (int c2 = 0; c2 < 2; ++c2) s[n++] = FStep{0, 2 * half + c2, k};
    for (int c2 = 0; c2 < 2; ++c2) s[n++] = FStep{2, c2, 0};
    const int nq = NRT * KST;
    int qi = 0;
    if (CH == 2) {
      for (; qi < nq / 2; ++qi) s[n++] = FStep{1, qi % NRT, qi / NRT};
      for (int c2 = 0; c2 < 2; ++c2) s[n++] = FStep{3, 2 + c2, 0};
      for (; qi < nq; ++qi) s[n++] = FStep{1, qi % NRT, qi / NRT};
      for (int it = 0; it < NRT; ++it) s[n++] = FStep{5, it, 0};
      for (int dt = 0; dt < NDT / 2; ++dt) s[n++] = FStep{6, dt, 0};
      for (int c2 = 0; c2 < 2; ++c2) s[n++] = FStep{4, 2 + c2, 1};
      for (int dt = NDT / 2; dt < NDT; ++dt) s[n++] = FStep{6, dt, 0};
      for (int it = 0; it < NRT; ++it) s[n++] = FStep{5, it, 1};
      for (int dt = 0; dt < NDT; ++dt) s[n++] = FStep{6, dt, 1};
    } else {
      for (; qi < nq; ++qi) s[n++] = FStep{1, qi % NRT, qi / NRT};
      for (int it = 0; it < NRT; ++it) s[n++] = FStep{5, it, 0};
      for (int dt = 0; dt < NDT; ++dt) s[n++] = FStep{6, dt, 0};
    }
  }
  // does step i complete its output tile (and so trigger a conversion)?
  constexpr bool completes(int i) const {
    const FStep t = s[i];
    if (t.kind == 0 || t.kind == 1) return t.k == KST - 1;
    if (t.kind == 6) return t.k == CH - 1;
    return t.kind != 5;
  }
  // first step that reads the conversion of step i's tile (NS: none in this chunk)
  constexpr int first_use(int i) const {
    const FStep t = s[i];
    for (int j = i + 1; j < NS; ++j) {
      const FStep u = s[j];
      if (t.kind == 0 && t.x < 2 && u.kind == 2) return j;               // xq of half a -> Ua
      if (t.kind == 0 && t.x >= 2 && u.kind == 3 && u.x == t.x) return j; // xb -> Yb
      if (t.kind == 1 && u.kind == 5 && u.x == t.x) return j;            // readout scaling -> P Up
      if (t.kind == 2 && (u.kind == 3 || (u.kind == 5 && u.k == 0) || (u.kind == 6 && u.k == 0))) return j;
      if (t.kind == 3 && u.kind == 4) return j;                          // yq -> Ub
      if (t.kind == 4 && ((u.kind == 5 && u.k == 1) || (u.kind == 6 && u.k == 1))) return j;
    }
    return NS;
  }
};

// Iteration (in steps, before the lookahead shift) at which the conversion of
// step i's tile runs: DL steps after its MFMA, or just before its first use.
// Never earlier than the step after it: conversions run before the MFMA of
// their iteration, so a conversion at step i + 1 follows MFMA i.
template <typename S>
__host__ __device__ constexpr int fconv_at(const S& sc, int i, int DL) {
  const int u = sc.first_use(i);
  const int a = (i + DL) < (u - 1) ? (i + DL) : (u - 1);
  return a > i + 1 ? a : i + 1;
}

// --------------------------------------------------------------------------
template <int DK, int C, int NWC, int NRT, bool GATED>
__global__ __launch_bounds__(64 * (NWC + kFusedAux)) __attribute__((amdgpu_waves_per_eu(1, 2)))
void dp_fused_kernel(FwdArgs p) {
  constexpr int RT = 16 * NRT, BV = 16 * NWC;
  constexpr int NCT = C / 16, NDT = DK / 16, KST = DK / 32, CH = C / 32;
  constexpr FusedLayout F = fused_layout(DK, C, RT, BV);
  static_assert(fused_ok(DK, C), "dk and chunk multiples of 32");
  static_assert(F.sV >= 1024 && F.sV % 1024 == 0, "value tile of whole 1 KB copies");

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware mapping: consecutive workgroup ids go round-robin over the 8
  // XCDs; the value blocks of one head then share an XCD (and its L2) for the
  // key and query rows they all read.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int f = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int bh = f / p.nvb, vb = f % p.nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;
  const SeqGeom sg = seq_geom(p, b, h, C);
  const int nc = sg.nc, N = sg.N, n_h = p.n_h;
  const long long tok0 = (p.cu == nullptr ? tok_base(p, b) : sg.tok) * p.H + h;  // token t: row tok0 + t H
  const bf16_t* const kp = static_cast<const bf16_t*>(p.k);
  const bf16_t* const qp = static_cast<const bf16_t*>(p.q);
  const bf16_t* const vp = static_cast<const bf16_t*>(p.v);
  // row of sub-step s in a [.., H, n_h, *] tensor
  auto sub_row_of = [&](int s) -> long long {
    const int t = fastdiv(s, p.nh_magic, p.nh_shift);
    return (tok0 + (long long)t * p.H) * n_h + (s - t * n_h);
  };

  if (nc == 0) {  // no sub-step: the final state is the initial one
    if (wave < NWC && p.fstate != nullptr) {
      const int col = lane & 15, grp = lane >> 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const long long o = ((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + 16 * wave + col;
          p.fstate[o] = p.h0 != nullptr ? p.h0[o] : 0.f;
        }
    }
    return;
  }

  if (wave >= NWC + 4) {
    // ================================================================ copy wave
    constexpr int NIV = F.sV / 1024;                 // 1 KB copies per value tile
    constexpr int NTK = DK * 2 > 128 ? 2 : 1;        // touches per key / query row (128-byte lines)
    constexpr int NTOUCH = 2 * NTK + 2;              // keys, queries, values, beta
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    auto issue_v = [&](int cc) {
      const uint32_t dst = lds0 + F.oV + (cc % kFusedV) * F.sV;
#pragma unroll
      for (int m = 0; m < NIV; ++m) {
        const int o = 1024 * m + 16 * lane;
        const int r = o / (BV * 2), cv = (o % (BV * 2)) / 2;
        int s = cc * C + r;
        s = s < N ? s : N - 1;  // rows past the end: any valid row (their beta is 0)
        dma16(vp + sub_row_of(s) * p.dv + v0 + cv, dst + 1024 * m);
      }
    };
    auto issue_touch = [&](int cc) {
      const uint32_t dst = lds0 + F.oD;
      int s = cc * C + (lane < C ? lane : C - 1);
      s = s < N ? s : N - 1;
      const long long row = sub_row_of(s);
#pragma unroll
      for (int u = 0; u < NTK; ++u) touch4(kp + row * DK + 64 * u, dst);
      // readout rows of the chunk: sub-steps r0, r0 + n_h, ..
      const int s0 = cc * C;
      const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));
      int sr = r0 + (lane < RT ? lane : RT - 1) * n_h;
      sr = sr < N ? sr : N - 1;
      const long long qrow = tok0 + (long long)fastdiv(sr, p.nh_magic, p.nh_shift) * p.H;
#pragma unroll
      for (int u = 0; u < NTK; ++u) touch4(qp + qrow * DK + 64 * u, dst);
      touch4(vp + row * p.dv + v0, dst);
      touch4(p.beta + row, dst);
    };
    issue_v(0);
    for (int per = -2; per < nc; ++per) {
      const bool iv = per + 3 < nc, it = per + kFusedTouchLead < nc;
      const bool itp = per - 1 >= -2 && per - 1 + kFusedTouchLead < nc;  // the previous period touched
      if (iv) issue_v(per + 3);
      if (it) issue_touch(per + kFusedTouchLead);
      // The value tile of chunk per + 2 (issued last period, before last period's
      // touches) has landed: it is read from the next period on.  Loads retire
      // in order, so the count left in flight is this period's copies and
      // touches and the previous period's touches (they stay in flight for two
      // periods).  it implies itp implies iv.
      if (it)
        wait_vmcnt<NIV + 2 * NTOUCH>();
      else if (itp)
        wait_vmcnt<NIV + NTOUCH>();
      else if (iv)
        wait_vmcnt<NIV>();
      else
        wait_vmcnt<0>();
      if (per + 1 < nc) block_sync_lds();
    }
    wait_vmcnt<0>();
    return;
  }

  if (wave >= NWC) {
    // ================================================================ producers
    // Two pairs of wavefronts; pair pr builds the operands of chunks
    // pr, pr + 2, ..  Within a pair the work of a chunk is split by 32-row
    // half: role a (rb = 0) the rows 0 .. 31, the queries and the per-chunk
    // scalars; role b the rows 32 .. C-1 and the cross block A_ba.  At chunk
    // 32 there is one half and role a does all of it.
    const int pk = wave - NWC;
    const int pr = pk >> 1, rb = pk & 1;
    // lane indices, made opaque inside each half so that the compiler cannot
    // hoist the lane-dependent constants of both halves out of the period loop
    // (they would stay live across it and spill)
    int m = lane & 15, g = lane >> 4;
    unsigned char* const scr = smem + F.oW + pr * F.sW;
    float* const sM = reinterpret_cast<float*>(scr);
    float* const sR = reinterpret_cast<float*>(scr + F.wR);
    float* const sB = reinterpret_cast<float*>(scr + F.wB);
    float* const sG = reinterpret_cast<float*>(scr + F.wG);
    int* const sLoc = reinterpret_cast<int*>(scr + F.wL);
    float* const sRb = reinterpret_cast<float*>(scr + F.wL + RT * 4);  // role b's copy of 1/|k| of half a
    // key row tiles this wave loads: role a tiles 0, 1 (all of them at chunk 32),
    // role b every tile (the cross block needs the rows of half a)
    const int nkt = (CH == 1 || rb == 1) ? NCT : 2;
    // (the unroll of the loads below stops at nkt: the row tile is still a
    // compile-time index of rk)

    // raw operands of this wave's next chunk: lane (m, g) holds, of key row
    // 16 i + m (and readout row 16 it + m), columns 32 t + 8 g .. + 7.  Rows
    // past the chunk's end are read from a valid row and zeroed when the first
    // half consumes them: a select here would wait for the loads and undo the
    // prefetch.
    u32x4_t rk[NCT][KST], rq[NRT][KST];
    float braw = 0.f, graw = 1.f;
    uint32_t rvalid = 0;  // bit i: key row 16 i + m, bit NCT + it: readout row, bit 30: beta, bit 31: gate
    auto load_raw = [&](int cc) {
      const int s0 = cc * C;
      uint32_t vb = 0;
#pragma unroll
      for (int i = 0; i < NCT; ++i) {
        if (i >= nkt) break;
        const int s = s0 + 16 * i + m;
        vb |= (s < N ? 1u : 0u) << i;
        const bf16_t* src = kp + sub_row_of(s < N ? s : N - 1) * DK + 8 * g;
#pragma unroll
        for (int t = 0; t < KST; ++t) rk[i][t] = ld16(src + 32 * t);
      }
      if (rb == 0) {
        const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));
        const int send = min(s0 + C, N);
#pragma unroll
        for (int it = 0; it < NRT; ++it) {
          const int sr = r0 + (16 * it + m) * n_h;
          const bool ok = sr < send;
          vb |= (ok ? 1u : 0u) << (NCT + it);
          const long long row =
              tok0 + (long long)fastdiv(ok ? sr : (r0 < N ? r0 : N - 1), p.nh_magic, p.nh_shift) * p.H;
          const bf16_t* src = qp + row * DK + 8 * g;
#pragma unroll
          for (int t = 0; t < KST; ++t) rq[it][t] = ld16(src + 32 * t);
        }
      }
      const int s = s0 + lane;
      const bool sok = lane < C && s < N;
      const int sc = sok ? s : N - 1;
      const int tt = fastdiv(sc, p.nh_magic, p.nh_shift);
      const int j = sc - tt * n_h;
      const long long tok = tok0 + (long long)tt * p.H;
      vb |= (sok ? 1u : 0u) << 30;
      vb |= (sok && j == 0 ? 1u : 0u) << 31;
      braw = p.beta[tok * n_h + j];
      if constexpr (GATED) graw = p.g[tok];
      rvalid = vb;
    };
    // -A_ba (fp16), role b, from a chunk's first half to its second: lane
    // (m, g) holds row 16 i + m, columns 16 j + 4 g .. + 3, tile (i - 2) * 2 + j
    f16x4_t nab[CH == 2 ? 4 : 1];

    // Gram tile of the raw keys: lane (m, g) holds row 16 i + m, columns
    // 16 j + 4 g .. + 3 (computed as tile (j, i) of the symmetric matrix)
    auto gram = [&](int i, int j) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KST; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, rk[j][t]),
                                                      __builtin_bit_cast(bf16x8_t, rk[i][t]), acc, 0, 0, 0);
      return acc;
    };

    // first half of chunk cc for role RB (a compile-time index: every register
    // array below is indexed by compile-time row tiles)
    auto first_half = [&](int cc, auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      constexpr int NKT = (CH == 1 || RB == 1) ? NCT : 2;  // key row tiles loaded
      constexpr int I0 = (RB == 0 || CH == 1) ? 0 : 2;     // first row tile of the half (role b: never at chunk 32)
      asm volatile("" : "+v"(m), "+v"(g));
      const int s0 = cc * C;
      unsigned char* const sK = smem + F.oK + (cc % kFusedKQ) * F.sK;
      unsigned char* const sQ = smem + F.oQ + (cc % kFusedKQ) * F.sQ;
      float* const sS = reinterpret_cast<float*>(smem + F.oS + (cc % kFusedT) * F.sS);
      // the loaded rows have arrived: zero those past the chunk's end
      const uint32_t vb = rvalid;
#pragma unroll
      for (int i = 0; i < NCT; ++i)
#pragma unroll
        for (int t = 0; t < KST; ++t)
          if (i < NKT && !((vb >> i) & 1u)) rk[i][t] = u32x4_t{0u, 0u, 0u, 0u};
      const float br = ((vb >> 30) & 1u) ? braw : 0.f;
      float lm = 0.f;
      if constexpr (GATED) lm = ((vb >> 31) & 1u) ? logf(fmaxf(graw, FLT_MIN)) : 0.f;
      // 1 / max(|k|, 1e-6) of row 16 i + m: the lane's part of the squared norm
      // by bf16 dot products on the raw registers, summed over the four lanes
      // (m, g) of the row by permlane swaps; published for other lanes' columns
      float rrow[NCT];
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int t = 0; t < KST; ++t)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            // (through a scalar copy: a bit cast of the vector element itself
            // compiled to element 0 for every d)
            const uint32_t w32 = rk[i][t][d];
            bf16x2_t w;
            __builtin_memcpy(&w, &w32, 4);
            ss = __builtin_amdgcn_fdot2_f32_bf16(w, w, ss, false);
          }
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
        rrow[i] = 1.f / fmaxf(sqrtf(ss), 1e-6f);
        if (g == 0) ((RB == 1 && i < 2) ? sRb : sR)[16 * i + m] = rrow[i];
      }
      // diagonal Gram tiles of the half (M's diagonal blocks)
      f32x4_t gd[NCT];
#pragma unroll
      for (int u = 0; u < 2; ++u) gd[I0 + u] = gram(I0 + u, I0 + u);
      // unit keys of the half as fp16, plain blocks of 8 columns (odd blocks' rows permuted by 8)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = I0 + u;
#pragma unroll
        for (int t = 0; t < KST; ++t) {
          float fv[8];
          unpack16(rk[i][t], fv, bf16_t{});
#pragma unroll
          for (int e = 0; e < 8; ++e) fv[e] *= rrow[i];
          const int q = 4 * t + g;
          st_vec16(reinterpret_cast<f16_t*>(sK + blk_pos(q, DK) * C * 16 + ((16 * i + m) ^ (8 * (q & 1))) * 16), fv);
        }
      }
      // off-diagonal Gram tiles this wave needs
      f32x4_t go[NCT][NCT];
      if constexpr (RB == 0 || CH == 1) {
        go[1][0] = gram(1, 0);
      } else {
        go[3][2] = gram(3, 2);
#pragma unroll
        for (int i = 2; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) go[i][j] = gram(i, j);
      }
      if constexpr (RB == 0) {
        // readout queries as fp16, fragment layout: granule (t, g') of a row
        // holds columns 32 t + 4 g' .. + 3 and 32 t + 16 + 4 g' .. + 3
#pragma unroll
        for (int it = 0; it < NRT; ++it)
#pragma unroll
          for (int t = 0; t < KST; ++t) {
            float fv[8];
            const u32x4_t qv = ((vb >> (NCT + it)) & 1u) ? rq[it][t] : u32x4_t{0u, 0u, 0u, 0u};
            unpack16(qv, fv, bf16_t{});
            const int g0 = g < 2 ? 2 * g : 2 * g - 4, hf = g < 2 ? 0 : 8;
            unsigned char* dst = sQ + (4 * t + g0) * RT * 16 + (16 * it + m) * 16 + hf;
            st4(reinterpret_cast<f16_t*>(dst), fv[0], fv[1], fv[2], fv[3]);
            st4(reinterpret_cast<f16_t*>(dst + RT * 16), fv[4], fv[5], fv[6], fv[7]);
          }
      }
      if (cc + 2 < nc) load_raw(cc + 2);  // the raw rows are consumed: fetch this wave's next chunk

      // beta range, cumulative log-gate, readout rows (both roles compute them;
      // role a publishes them for the second half and the consumers)
      const float bc = clamp_keep_nan(br, 0.f, 2.f);
      float G = 0.f;
      if constexpr (GATED) G = wave_inclusive_scan(lm);
      if constexpr (RB == 0) {
        if (lane < C) {
          sB[lane] = bc;
          sG[lane] = G;
        }
        const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));
        const int sr = r0 + lane * n_h;
        const int loc = (lane < RT && sr < min(s0 + C, N)) ? sr - s0 : -1;
        if (lane < RT) sLoc[lane] = loc;
        if constexpr (GATED) {
          const float Gl = __shfl(G, C - 1, 64);
          const float Gloc = __shfl(G, loc >= 0 ? loc : 0, 64);
          if (lane < C) {
            sS[lane] = expf(G);
            sS[C + lane] = expf(Gl - G);
          }
          if (lane < RT) sS[2 * C + lane] = loc >= 0 ? expf(Gloc) : 0.f;
        }
      }
      // A = E o (Kn Kn^T) from a Gram tile: row scale 1/|k_i|, column scale 1/|k_j|,
      // decay e^{G_i - G_j} (beta and G of other lanes through shuffles: role b
      // does not wait for role a's scratch)
      // (tr: the tile is read transposed, as A[16 j + 4 g + e][16 i + m], whose
      // decay is e^{G_{16 j + 4 g + e} - G_{16 i + m}})
      auto scaled = [&](const f32x4_t& a, int i, int j, bool tr) {
        const int jj0 = 16 * j + 4 * g;
        const f32x4_t rj = *reinterpret_cast<const f32x4_t*>(((RB == 1 && j < 2) ? sRb : sR) + jj0);
        f32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = a[e] * rrow[i] * rj[e];
        if constexpr (GATED) {
          const float Gi = __shfl(G, 16 * i + m, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = Gi - __shfl(G, jj0 + e, 64);
            o[e] *= expf(tr ? -d : d);
          }
        }
        return o;
      };
      // M = strict_tril(diag(beta) A) on the three blocks of this wave's half
      // (fp32 scratch).  The off-diagonal block is stored as it is (row m,
      // columns 4 g ..), each diagonal block transposed: the symmetric Gram
      // tile's lane (m, g) also holds A[16 i + 4 g + e][16 i + m], which is
      // M^T[16 i + m][16 i + 4 g + e] / beta_{16 i + 4 g + e}, so row m of M^T
      // is again one 16-byte store.  The forward substitution reads M's
      // columns as M^T rows.
      wave_lds_fence();  // this wave's 1/|k| published above
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int i = I0 + (u > 0 ? 1 : 0), j = I0 + (u == 2 ? 1 : 0);
        const f32x4_t a = scaled(i == j ? gd[i] : go[i][j], i, j, i == j);
        const int ii = 16 * i + m, jj0 = 16 * j + 4 * g;
        f32x4_t mv;
        if (i == j) {
          // (the cross-lane reads stay outside the mask: a shuffle under a
          // divergent condition reads inactive lanes' garbage)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float bj = __shfl(bc, jj0 + e, 64);
            mv[e] = (jj0 + e > ii) ? bj * a[e] : 0.f;
          }
        } else {
          const float bi = __shfl(bc, ii, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = bi * a[e];
        }
        *reinterpret_cast<f32x4_t*>(sM + fused_blk(i, j) * kPrepBlk + m * kPrepLdm + 4 * g) = mv;
      }
      if constexpr (CH == 2 && RB == 1) {
#pragma unroll
        for (int i = 2; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) nab[(i - 2) * 2 + j] = to_h4(-scaled(go[i][j], i, j, false));
      }
      wave_lds_fence();
    };

    auto second_half = [&](int cc) {
      asm volatile("" : "+v"(m), "+v"(g));
      unsigned char* const sK = smem + F.oK + (cc % kFusedKQ) * F.sK;
      unsigned char* const sQ = smem + F.oQ + (cc % kFusedKQ) * F.sQ;
      unsigned char* const sT = smem + F.oT + (cc % kFusedT) * F.sT;
      unsigned char* const sP = smem + F.oP + (cc % kFusedT) * F.sP;
      const int hh = (CH == 1) ? 0 : rb;  // the 32-row half this wave solves
      // 1. diagonal blocks D = (I + M_ii)^{-1} of the half by forward
      //    substitution: lane group g < 2 solves block 2 hh + g, lane m one
      //    column of it, by column sweep: once t[j] is final, every later row
      //    takes t[r] -= M[r][j] t[j] (independent updates; M's column j is row
      //    j of the stored M^T, read as a broadcast ahead of its use)
      if (g < 2) {
        float* const blk = sM + fused_blk(2 * hh + g, 2 * hh + g) * kPrepBlk;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = (r == m) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          f32x4_t mc[4];
#pragma unroll
          for (int q = j / 4; q < 4; ++q) mc[q] = *reinterpret_cast<const f32x4_t*>(blk + j * kPrepLdm + 4 * q);
#pragma unroll
          for (int r = j + 1; r < 16; ++r) t[r] = fmaf(-mc[r / 4][r % 4], t[j], t[r]);
        }
        wave_lds_fence();
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[r * kPrepLdm + m] = t[r];
      }
      wave_lds_fence();
      // 2. off-diagonal block of the half: T_10 = -D_1 (M_10 D_0)
      {
        float* const D0 = sM + (3 * hh) * kPrepBlk;
        float* const M10 = sM + (3 * hh + 1) * kPrepBlk;
        float* const D1 = sM + (3 * hh + 2) * kPrepBlk;
        f32x4_t bb;
#pragma unroll
        for (int e = 0; e < 4; ++e) bb[e] = D0[(4 * g + e) * kPrepLdm + m];
        const f32x4_t R = mm16_split(*reinterpret_cast<const f32x4_t*>(M10 + m * kPrepLdm + 4 * g), bb,
                                     f32x4_t{0.f, 0.f, 0.f, 0.f});
        const f32x4_t t10 = mm16_split(*reinterpret_cast<const f32x4_t*>(D1 + m * kPrepLdm + 4 * g), R,
                                       f32x4_t{0.f, 0.f, 0.f, 0.f});
        wave_lds_fence();
#pragma unroll
        for (int e = 0; e < 4; ++e) M10[(4 * g + e) * kPrepLdm + m] = -t10[e];
      }
      wave_lds_fence();
      // 3. T diag(beta) of the half into the T ring (fragment layout; tile hh
      //    stores rows 32 hh .. C-1), and (role b) -A_ba into tile 0 rows 32 .. 63
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = lane + 64 * u;
        const int gq = idx >> 5, rl = idx & 31;
        const int i = 32 * hh + rl, ib = i >> 4;
        const f32x4_t* T0 = reinterpret_cast<const f32x4_t*>(sM + fused_blk(ib, 2 * hh) * kPrepBlk +
                                                              (i & 15) * kPrepLdm + 4 * gq);
        // the (upper) block (2 hh, 2 hh + 1) is zero: read any in-bounds block, then select
        const f32x4_t* T1 = reinterpret_cast<const f32x4_t*>(sM + fused_blk(2 * hh + 1, 2 * hh + 1) * kPrepBlk +
                                                              (i & 15) * kPrepLdm + 4 * gq);
        const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(sB + 32 * hh + 4 * gq);
        const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(sB + 32 * hh + 16 + 4 * gq);
        const f32x4_t x0 = *T0, x1 = *T1;
        const bool up = (ib & 1) == 0;
        float fv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fv[e] = x0[e] * b0[e];
          fv[4 + e] = up ? 0.f : x1[e] * b1[e];
        }
        st_vec16(reinterpret_cast<f16_t*>(sT + t_block_byte(C, hh) + gq * (C - 32 * hh) * 16 + (i - 32 * hh) * 16), fv);
      }
      if constexpr (CH == 2) {
        if (rb == 1) {
#pragma unroll
          for (int i = 2; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              *reinterpret_cast<f16x4_t*>(sT + g * C * 16 + (16 * i + m) * 16 + 8 * j) = nab[(i - 2) * 2 + j];
        }
      }
      // 4. masked, decayed scores of the readout rows, P[i][j] = (q_i . kn_j)
      //    e^{G_loc(i) - G_j} for j <= loc(i): computed transposed (lane (i, g)
      //    gets columns 16 jt + 4 g .. + 3 of row i) from the fp16 tiles.  The
      //    NRT x NCT tiles are split between the two roles.
      const int lrK = lane_row<DK>(C);
      constexpr int NPT = NRT * NCT;
      const int p0 = CH == 1 ? 0 : rb * (NPT / 2), p1 = CH == 1 ? NPT : p0 + NPT / 2;
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        if (pt < p0 || pt >= p1) continue;
        const int it = (NRT >= 2) ? pt / NCT : 0, jt = (NRT >= 2) ? pt % NCT : pt;
        const int i = 16 * it + m;
        const int loc = sLoc[i];
        const float gl = GATED ? sG[loc >= 0 ? loc : 0] : 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KST; ++t) {
          const f16x8_t qf = *reinterpret_cast<const f16x8_t*>(sQ + lane_frag(RT) + it * 256 + 4 * t * RT * 16);
          const unsigned char* kb = sK + lrK + jt * 256 + 4 * t * C * 16;
          const f16x8_t ka = cat8(*reinterpret_cast<const f16x4_t*>(kb), *reinterpret_cast<const f16x4_t*>(kb + C * 16));
          acc = mfma32h(ka, qf, acc);
        }
        const int j0 = 16 * jt + 4 * g;
        float pv[4];
        f32x4_t Gj = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) Gj = *reinterpret_cast<const f32x4_t*>(sG + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (j0 + e <= loc) ? acc[e] * (GATED ? expf(gl - Gj[e]) : 1.f) : 0.f;
        st4(reinterpret_cast<f16_t*>(sP + (4 * (jt >> 1) + g) * RT * 16 + i * 16 + 8 * (jt & 1)), pv[0], pv[1],
            pv[2], pv[3]);
      }
      wave_lds_fence();
    };

    const bool active = CH == 2 || rb == 0;  // at chunk 32 role b has no work
    if (active && pr < nc) load_raw(pr);
    for (int per = -2; per < nc; ++per) {
      const int c1 = per + 2, c2 = per + 1;
      if (active) {
        if (c1 < nc && (c1 & 1) == pr) {
          if (rb == 0)
            first_half(c1, std::integral_constant<int, 0>{});
          else
            first_half(c1, std::integral_constant<int, 1>{});
        } else if (c2 >= 0 && c2 < nc && (c2 & 1) == pr)
          second_half(c2);
      }
      if (per + 1 < nc) block_sync_lds();
    }
    return;
  }

  // ================================================================== consumers
  using Sched = FSched<NCT, KST, NRT, NDT>;
  constexpr Sched SC{};
  constexpr int NS = Sched::NS;
  constexpr int LA = kLookahead, DL = 3;
  constexpr bool EARLY = NCT * KST >= LA;  // the first LA steps are key fragments
  constexpr int TS = t_trimmed(DK, C) ? 32 : 0;
  const int col = lane & 15, grp = lane >> 4;
  const int vw = 16 * wave;
  const int lrK = lane_row<DK>(C);
  const int ltK = lane_tr<DK>(C), ltV = lane_tr_rows<BV>();
  const int ocol = v0 + vw + col;
  f32x4_t hacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    hacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p.h0 != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[dt][e] = p.h0[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + ocol];
    }
  }
  f16x4_t hqn[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) hqn[dt] = to_h4(hacc[dt]);

  const int HD = p.H * p.dv;
  const int es = p.out_f32 ? 4 : 2;
  int voff[NRT][4], voff4[NRT];
#pragma unroll
  for (int it = 0; it < NRT; ++it) {
#pragma unroll
    for (int e = 0; e < 4; ++e) voff[it][e] = ((16 * it + 4 * grp + e) * HD + ocol) * es;
    voff4[it] = ((16 * it + 4 * grp + (col & 3)) * HD + ocol - (col & 3)) * 2;
  }
  const uint32_t qsel = (lane & 1) ? 0x03020706u : 0x05040100u;

  f32x4_t vf[NCT], eg[NCT], el[NCT], egl[NRT];
  float dec = 1.f;
  f16x8_t ring[LA];
  f16x8_t pre[EARLY ? LA : 1];
  struct Ctx {
    uint32_t oK[NCT], oK1[NCT], oT[CH], oQ[NRT], oP[NRT];
    uint32_t sK, sV, sS;
    int t0, nrd;
  };
  auto make_ctx = [&](int cc) __attribute__((always_inline)) {
    Ctx x;
    x.sK = F.oK + (cc % kFusedKQ) * F.sK;
    const uint32_t sQ = F.oQ + (cc % kFusedKQ) * F.sQ;
    const uint32_t sT = F.oT + (cc % kFusedT) * F.sT;
    const uint32_t sP = F.oP + (cc % kFusedT) * F.sP;
    x.sS = F.oS + (cc % kFusedT) * F.sS;
    x.sV = F.oV + (cc % kFusedV) * F.sV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      x.oK[ct] = x.sK + lrK + ct * 256;
      x.oK1[ct] = x.oK[ct] + C * 16;
      asm volatile("" : "+v"(x.oK[ct]), "+v"(x.oK1[ct]));
    }
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      x.oT[t] = sT + t_block_byte(C, t) + (lane >> 4) * (C - TS * t) * 16 + (lane & 15) * 16;
      asm volatile("" : "+v"(x.oT[t]));
    }
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      x.oQ[it] = sQ + lane_frag(RT) + it * 256;
      x.oP[it] = sP + lane_frag(RT) + it * 256;
      asm volatile("" : "+v"(x.oQ[it]), "+v"(x.oP[it]));
    }
    x.t0 = fastdiv(cc * C, p.nh_magic, p.nh_shift);
    x.nrd = fastdiv(min(cc * C + C, N), p.nh_magic, p.nh_shift) - x.t0;
    return x;
  };
  auto load_small = [&](const Ctx& x) {
    const float* sEG = reinterpret_cast<const float*>(smem + x.sS);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // V[16 ct + 4 grp + e][vw + col] (bf16) in accumulator layout
      const s16x4_t vr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(smem + x.sV + ltV + (16 * ct * BV + 16 * wave) * 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[ct][e] = __uint_as_float((uint32_t)(uint16_t)vr[e] << 16);
      if constexpr (GATED) {
        eg[ct] = *reinterpret_cast<const f32x4_t*>(sEG + ct * 16 + 4 * grp);
        el[ct] = *reinterpret_cast<const f32x4_t*>(sEG + C + ct * 16 + 4 * grp);
      }
    }
    if constexpr (GATED) {
#pragma unroll
      for (int it = 0; it < NRT; ++it) egl[it] = *reinterpret_cast<const f32x4_t*>(sEG + 2 * C + it * 16 + 4 * grp);
      dec = sEG[C - 1];
    }
  };
  // A fragment of a key step (kind 0) of the chunk whose contexts are x
  auto key_frag = [&](const Ctx& x, auto ic) -> f16x8_t {
    constexpr int i = decltype(ic)::value;
    constexpr FStep st = SC.s[i];
    constexpr int ko = 4 * st.k * C * 16;
    return cat8(*reinterpret_cast<const f16x4_t*>(smem + x.oK[st.x] + ko),
                *reinterpret_cast<const f16x4_t*>(smem + x.oK1[st.x] + ko));
  };

  // chunk c's values, scalars and first key fragments are read during period
  // c - 1 (chunk 0's between the first two barriers), so that the copy
  // wavefront may refill a value slot in the period after its last read
  block_sync_lds();  // X(-1): chunk 0's keys, scalars and values have landed
  Ctx cur = make_ctx(0);
  load_small(cur);
  if constexpr (EARLY) static_for<LA>([&](auto kc) { pre[decltype(kc)::value] = key_frag(cur, kc); });
  block_sync_lds();  // X(0): chunk 0's T and scores, chunk 1's keys, scalars and values

  for (int c = 0; c < nc; ++c) {
    const long long obase = (tok0 + (long long)cur.t0 * p.H) * p.dv;  // first readout row of the chunk
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(p.out) + obase * es, 0, cur.nrd * HD * es, kBufferDword3);
    Ctx nxt;
    f32x4_t accX[NCT], accU[NCT], accY[NCT], xb[NCT], z[NRT];
    f16x4_t xq[NCT], uq[NCT], usq[NCT], yq[NCT];

    auto load_frag = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr FStep st = SC.s[i];
      f16x8_t fr;
      if constexpr (st.kind == 0) {
        fr = key_frag(cur, ic);
      } else if constexpr (st.kind == 1) {
        fr = *reinterpret_cast<const f16x8_t*>(smem + cur.oQ[st.x] + 4 * st.k * RT * 16);
      } else if constexpr (st.kind == 2 || st.kind == 3) {
        fr = *reinterpret_cast<const f16x8_t*>(smem + cur.oT[0] + (16 * st.x) * 16);
      } else if constexpr (st.kind == 4) {
        fr = *reinterpret_cast<const f16x8_t*>(smem + cur.oT[1] + (16 * st.x - TS) * 16);
      } else if constexpr (st.kind == 5) {
        fr = *reinterpret_cast<const f16x8_t*>(smem + cur.oP[st.x] + 4 * st.k * RT * 16);
      } else {
        const unsigned char* q = smem + cur.sK + ltK + tr_block<DK>(st.x) * C * 16 + 32 * st.k * 16;
        fr = cat8(__builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)q)),
                  __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(q + 256))));
      }
      ring[i % LA] = fr;
    };
    auto mfma_step = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr FStep st = SC.s[i];
      f16x8_t a;
      if constexpr (EARLY && i < LA)
        a = pre[i];
      else
        a = ring[i % LA];
      constexpr f32x4_t Z = {0.f, 0.f, 0.f, 0.f};
      if constexpr (st.kind == 0) {
        accX[st.x] = mfma32h(a, cat8(hqn[2 * st.k], hqn[2 * st.k + 1]), st.k == 0 ? Z : accX[st.x]);
      } else if constexpr (st.kind == 1) {
        z[st.x] = mfma32h(a, cat8(hqn[2 * st.k], hqn[2 * st.k + 1]), st.k == 0 ? Z : z[st.x]);
      } else if constexpr (st.kind == 2) {
        accU[st.x] = mfma32h(a, cat8(xq[0], xq[1]), Z);
      } else if constexpr (st.kind == 3) {
        accY[st.x] = mfma32h(a, cat8(uq[0], uq[1]), xb[st.x]);
      } else if constexpr (st.kind == 4) {
        accU[st.x] = mfma32h(a, cat8(yq[2], yq[3]), Z);
      } else if constexpr (st.kind == 5) {
        z[st.x] = mfma32h(a, cat8(uq[2 * st.k], uq[2 * st.k + 1]), z[st.x]);
      } else {
        if constexpr (GATED && st.k == 0) hacc[st.x] = hacc[st.x] * dec;
        hacc[st.x] = mfma32h(a, cat8(usq[2 * st.k], usq[2 * st.k + 1]), hacc[st.x]);
      }
    };
    auto conv = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr FStep st = SC.s[k];
      if constexpr (st.kind == 0) {
        f32x4_t x;
        if constexpr (GATED)
          x = vf[st.x] - eg[st.x] * accX[st.x];  // accX = Kn H
        else
          x = vf[st.x] - accX[st.x];
        if constexpr (st.x < 2) {
          xq[st.x] = to_h4(x);
          asm volatile("" : "+v"(xq[st.x]));
        } else {
          xb[st.x] = x;
        }
      } else if constexpr (st.kind == 1) {
        if constexpr (GATED) z[st.x] = z[st.x] * egl[st.x];
      } else if constexpr (st.kind == 2 || st.kind == 4) {
        uq[st.x] = to_h4(accU[st.x]);
        asm volatile("" : "+v"(uq[st.x]));
        if constexpr (GATED) {
          usq[st.x] = to_h4(accU[st.x] * el[st.x]);
          asm volatile("" : "+v"(usq[st.x]));
        } else {
          usq[st.x] = uq[st.x];
        }
      } else if constexpr (st.kind == 3) {
        yq[st.x] = to_h4(accY[st.x]);
        asm volatile("" : "+v"(yq[st.x]));
      } else if constexpr (st.kind == 6) {
        hqn[st.x] = to_h4(hacc[st.x]);
        asm volatile("" : "+v"(hqn[st.x]));
      }
    };
    constexpr int NSP = EARLY ? (NS + LA - 1) / LA * LA : NS;
    static_for<NSP + LA + DL>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      // conversions due in this iteration
      static_for<DL + 1>([&](auto wc) {
        constexpr int k = i - LA - DL + decltype(wc)::value;
        if constexpr (k >= 0 && k < NS) {
          if constexpr (SC.completes(k) && fconv_at(SC, k, DL) + LA == i) conv(std::integral_constant<int, k>{});
        }
      });
      if constexpr (i >= LA && i - LA < NS) mfma_step(std::integral_constant<int, i - LA>{});
      if constexpr (i == LA + 2) nxt = make_ctx(c + 1 < nc ? c + 1 : c);
      if constexpr (EARLY) {
        if constexpr (i >= LA && i < NS) load_frag(std::integral_constant<int, i>{});
        if constexpr (i >= NSP && i < NSP + LA) pre[i - NSP] = key_frag(nxt, std::integral_constant<int, i - NSP>{});
      } else {
        if constexpr (i < NS) load_frag(std::integral_constant<int, i>{});
      }
      if constexpr (i == NS + LA) load_small(nxt);  // past this chunk's last use of them
      sched_fence();
    });
    // readout rows, stored after the chunk's products; rows from nrd on fall
    // outside the buffer resource's bound and are dropped
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      if (p.out_f32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z[it][e]), orsrc, voff[it][e], 0, 0);
      } else {
        uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{z[it][0], z[it][1]}, bf16x2_t));
        uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{z[it][2], z[it][3]}, bf16x2_t));
        const uint32_t x0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p0, 0x4E, 0xF, 0xF, false);  // lane ^ 2
        const uint32_t x1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p1, 0x4E, 0xF, 0xF, false);
        if (lane & 2)
          p0 = x1;
        else
          p1 = x0;
        const uint32_t y0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p0, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        const uint32_t y1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p1, 0xB1, 0xF, 0xF, false);
        p0 = __builtin_amdgcn_perm(y0, p0, qsel);
        p1 = __builtin_amdgcn_perm(y1, p1, qsel);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{p0, p1}, orsrc, voff4[it], 0, 0);
      }
    }
    if (c + 1 < nc) block_sync_lds();  // X(c + 1)
    cur = nxt;
  }

  if (p.fstate != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.fstate[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + ocol] = hacc[dt][e];
  }
}

template <int DK, int C, int NWC, int NRT, bool GATED>
hipError_t launch_fused_g(const FwdArgs& a, hipStream_t st) {
  static const bool attr =
      allow_big_lds(reinterpret_cast<const void*>(&dp_fused_kernel<DK, C, NWC, NRT, GATED>));
  (void)attr;
  const long long nwg = (long long)a.B * a.H * a.nvb;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((dp_fused_kernel<DK, C, NWC, NRT, GATED>), dim3((unsigned)nwg), dim3(64 * (NWC + kFusedAux)),
                     fused_layout(DK, C, 16 * NRT, 16 * NWC).bytes, st, a);
  return hipGetLastError();
}

template <int DK, int C, int NRT>
hipError_t launch_fused(const FwdArgs& a, int BV, hipStream_t st) {
  // readout tiles ceil(C / n_h) rounded to 16: 1, 2 or 4 at chunk 64, 1 or 2 at
  // chunk 32; at most two consumer wavefronts (with the four producers and the
  // copy wavefront, more would put three wavefronts on a SIMD and cap the registers)
  if constexpr (fused_ok(DK, C) && NRT != 3) {
    const bool gated = a.g != nullptr;
    switch (BV) {
      case 16: return gated ? launch_fused_g<DK, C, 1, NRT, true>(a, st) : launch_fused_g<DK, C, 1, NRT, false>(a, st);
      case 32: return gated ? launch_fused_g<DK, C, 2, NRT, true>(a, st) : launch_fused_g<DK, C, 2, NRT, false>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dp
