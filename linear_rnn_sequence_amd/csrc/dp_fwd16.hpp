// dp_fwd16.hpp -- the bf16 forward with symmetric keys: a parallel chunk-prep
// kernel and a register-resident chunk scan fed by direct-to-LDS copies.
//
// Same chunkwise form as the rest of the library (DeltaProduct study notes
// sec. 2.2 Eq.(3), sec. 2.6 and sec. 4.1; chunkwise WY/UT form of the OSDN
// study notes sec. 2.5 / App. A.2, with the chunk-local log-gate G):
//
//   T  = (I + strict_tril(diag(beta) (E o Kn Kn^T)))^{-1}
//   Up = (T diag(beta)) (V - diag(e^G) Kn H0)
//   O  = diag(e^{G_loc}) Q H0 + P Up,   P = (tril_incl(Q Kn^T) o E) on readout rows
//   H1 = e^{G_last} H0 + Kn^T (diag(e^{G_last - G}) Up)
//
// dp_prep_kernel (one workgroup per chunk, all chunks in parallel) computes
// every operand that does not depend on the state and writes it to the
// workspace in its final fp16 form:  T diag(beta), the unit keys Kn, the
// readout queries Q, the masked and decayed scores P, and per-chunk scalars
// (e^G, e^{G_last - G}, e^{G_loc} and the output offset of each readout row).
// dp_chain_kernel then only runs the recurrence: NWC consumer wavefronts keep
// their 16 value columns of the fp32 state in registers, and two copy
// wavefronts stream each chunk's operands (and the values) into a ring of
// LDS stages with global_load_lds_dwordx4, two or three chunks ahead.
// Packed variable-length batches run the same two kernels: every sequence is
// chunked from its own first sub-step (SeqGeom), so no chunk spans two.
//
// Tile layout ("block-major"): a tile of R rows and W fp16 columns is stored
// as W/8 blocks of R x 16 bytes (block q holds columns 8q..8q+7 of every row).
// In LDS, the rows of odd blocks are permuted (row r in slot r ^ 8).  Both
// operand read patterns of the scan are then free of bank conflicts: a row
// read (16 rows x 8 bytes of one block per half-wave) touches 256 contiguous
// bytes, and a transposed read (ds_read_b64_tr_b16: 8 rows x 2 adjacent
// blocks per half-wave) touches two 128-byte halves of the 64 banks.  Every
// lane-dependent part of an address is fixed per lane, so all tile offsets
// are instruction immediates.
#pragma once

#include <utility>

#include "dp_device.hpp"

namespace dp {

// Operands that are only read by rows (T diag(beta), Q, P) use, when their
// width W is a multiple of 32, the "fragment" layout: the 16-byte granule
// (t, g) of a row holds columns 32t + 4g .. 32t + 4g + 3 and 32t + 16 + 4g ..
// 32t + 16 + 4g + 3 -- exactly the eight values one lane of group g feeds a
// 32-deep MFMA step -- and granule (t, g) of all rows forms block 4t + g.  A
// fragment is then one 16-byte read, and 16 lanes read 256 contiguous bytes.
// The keys (read by rows and transposed) stay in plain blocks of 8 columns.
__host__ __device__ constexpr bool frag_layout(int W) { return W % 32 == 0; }
// byte offset, inside a row's granules, of column c (fragment layout)
__host__ __device__ constexpr int frag_col_byte(int c) {
  return ((c >> 4) & 1) * 8 + (c & 3) * 2;
}
// block index of column c (fragment layout)
__host__ __device__ constexpr int frag_col_block(int c) { return 4 * (c >> 5) + ((c & 15) >> 2); }

// T diag(beta) is block lower-triangular.  When the chunk scan runs its
// pipelined body (dk and chunk multiples of 32) and the chunk has more than
// one 32-column tile, the fragment-layout blocks of column tile t keep only
// rows 32 t .. C-1 (the rows above are zero): block 4t + g then starts at
// t_block_byte(C, t) + g (C - 32 t) 16 and row i sits (i - 32 t) 16 bytes in.
__host__ __device__ constexpr bool t_trimmed(int DK, int C) { return DK % 32 == 0 && C % 32 == 0 && C > 32; }
__host__ __device__ constexpr int t_block_byte(int C, int t) {
  return 4 * 16 * (t * C - 16 * t * (t - 1));  // sum over t' < t of 4 (C - 32 t') 16
}
__host__ __device__ constexpr int t_bytes(int DK, int C) {
  return t_trimmed(DK, C) ? t_block_byte(C, C / 32) : C * C * 2;
}

// Byte offsets of one chunk's operand block (workspace and LDS stage alike).
// With a separate write key (asym) the block also holds the write keys Kw,
// which the state update reads transposed in place of Kn.
struct Chunk16Layout {
  int oT, oK, oKW, oQ, oP, oS;  // T diag(beta), Kn, Kw (= oK when symmetric), readout Q, scores P, scalars
  int oEG, oEL, oEGL, oOff;     // scalars (relative to oS)
  int bytes;                    // whole block, a multiple of 16
};

__host__ __device__ constexpr Chunk16Layout chunk16_layout(int DK, int C, int RT, bool asym = false) {
  Chunk16Layout L{};
  L.oT = 0;
  L.oK = L.oT + t_bytes(DK, C);
  L.oKW = asym ? L.oK + C * DK * 2 : L.oK;
  L.oQ = L.oKW + C * DK * 2;
  L.oP = L.oQ + RT * DK * 2;
  L.oS = L.oP + RT * C * 2;
  L.oEG = 0;
  L.oEL = 4 * C;
  L.oEGL = 8 * C;
  L.oOff = (8 * C + 4 * RT + 7) & ~7;
  L.bytes = L.oS + ((L.oOff + 8 * RT + 15) & ~15);
  return L;
}

// LDS of dp_chain_kernel: kStages copies of (chunk block, value tile).
// Four stages (three chunks in flight) when they fit the 160 KB of LDS, else
// three, else two (the write-key block at one readout per sub-step).
__host__ __device__ constexpr int chain_stage_bytes(int DK, int C, int RT, int BV, bool asym = false) {
  return chunk16_layout(DK, C, RT, asym).bytes + C * BV * 2;
}
__host__ __device__ constexpr int chain_stages(int DK, int C, int RT, int BV, bool asym = false) {
  return 4 * chain_stage_bytes(DK, C, RT, BV, asym) <= 160 * 1024   ? 4
         : 3 * chain_stage_bytes(DK, C, RT, BV, asym) <= 160 * 1024 ? 3
                                                                     : 2;
}
// Lookahead (in MFMA steps) of the pipelined chunk body.
constexpr int kLookahead = 8;
// Pipelined body (dk and chunk multiples of 32), four stages, and the first
// kLookahead steps are key fragments (C/16 key tiles of dk/32 steps each).
__host__ __device__ constexpr bool chain_early(int DK, int C, int STG) {
  return DK % 32 == 0 && C % 32 == 0 && STG == 4 && (C / 16) * (DK / 32) >= kLookahead;
}
__host__ __device__ constexpr int chain_lds_bytes(int DK, int C, int RT, int BV, bool asym = false) {
  return chain_stages(DK, C, RT, BV, asym) * chain_stage_bytes(DK, C, RT, BV, asym);
}
// The write-key form runs on the prep / chain pair only with the chain's
// pipelined body (dk and chunk multiples of 32).
__host__ __device__ constexpr bool chain_asym_ok(int DK, int C) { return DK % 32 == 0 && C % 32 == 0; }

// LDS of dp_prep_kernel.  Region 0 holds the fp16 key and query rows while
// M and the scores are formed, then fp32 T and the partial-sum tiles of the
// blocked inverse; after it come fp32 M, beta, G and the readout locations.
// M is kept as its lower-triangular 16 x 16 blocks only (block (i, j), j <= i,
// at index i (i + 1) / 2 + j, rows kPrepLdm floats apart, blocks kPrepBlk
// floats apart), which keeps five workgroups resident per CU at dk = 128,
// chunk 64.
constexpr int kPrepLdm = 20;  // 20 n mod 64 is distinct for n < 16: conflict-free row reads
// 8 floats of padding per block: the diagonal blocks 0, 2, 5, 9 that the four
// lane groups of the forward substitution read in step start on banks 0, 16,
// 40 and 8 (with 320 they would all start on bank 0: a 4-way conflict)
constexpr int kPrepBlk = 16 * kPrepLdm + 8;
__host__ __device__ constexpr int prep_mblock(int i, int j) { return i * (i + 1) / 2 + j; }
__host__ __device__ constexpr int prep_m_bytes(int C) {
  return (C / 16) * (C / 16 + 1) / 2 * kPrepBlk * 4;
}
// With dk a multiple of 32 the readout queries never touch LDS: each
// wavefront loads its MFMA fragments of them straight into registers (and
// writes them to the operand block from there).  T is kept packed like M.
__host__ __device__ constexpr bool prep_q_in_regs(int DK) { return DK % 32 == 0; }
// With write keys, region 0 also holds their fp16 rows (after the query rows).
__host__ __device__ constexpr int prep_rows_bytes(int DK, int C, int RT, bool asym) {
  return C * (DK + 8) * 2 + (prep_q_in_regs(DK) ? 0 : RT * (DK + 8) * 2) + (asym ? C * (DK + 8) * 2 : 0);
}
__host__ __device__ constexpr int prep_region0_bytes(int DK, int C, int RT, bool asym = false) {
  return prep_rows_bytes(DK, C, RT, asym) > (prep_m_bytes(C) + 4 * 16 * 17 * 4) ? prep_rows_bytes(DK, C, RT, asym)
                                                                               : (prep_m_bytes(C) + 4 * 16 * 17 * 4);
}
__host__ __device__ constexpr int prep_lds_bytes(int DK, int C, int RT, bool asym = false) {
  return prep_region0_bytes(DK, C, RT, asym) + prep_m_bytes(C) + 2 * C * 4 + RT * 4;
}

// ---------------------------------------------------------------------------
// dp_prep_kernel: one chunk per workgroup.  ASYM: the write keys kt are
// given (used as they are): M pairs the read keys Kn (rows) with the write
// keys (columns), the scores pair the queries with the write keys, and the
// block carries the write keys for the chain's state update.
template <int DK, int C, int NRT, bool ASYM = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void dp_prep_kernel(FwdArgs p) {
  constexpr int RT = 16 * NRT;
  constexpr int TPR = DK / 8;  // 16-byte granules per key row
  constexpr int LDK = DK + 8;
  constexpr int NT = C / 16;
  constexpr int KV = C * TPR, KIT = (KV + 255) / 256;
  constexpr int QV = RT * TPR, QIT = (QV + 255) / 256;
  constexpr Chunk16Layout W = chunk16_layout(DK, C, RT, ASYM);
  static_assert(TPR <= 64 && 64 % TPR == 0, "row group must fit in a wavefront");

  extern __shared__ __align__(16) unsigned char smem[];
  f16_t* sK = reinterpret_cast<f16_t*>(smem);  // region 0, until M and P are formed
  f16_t* sQ = sK + C * LDK;
  // write-key rows (fp16, as given); the read keys stand in for them when symmetric
  f16_t* sKW = ASYM ? sQ + (prep_q_in_regs(DK) ? 0 : RT * LDK) : sK;
  float* sTf = reinterpret_cast<float*>(smem);  // region 0, from the inverse on (packed blocks)
  float* sSc = sTf + prep_m_bytes(C) / 4;
  float* sA = reinterpret_cast<float*>(smem + prep_region0_bytes(DK, C, RT, ASYM));
  float* sB = sA + prep_m_bytes(C) / 4;
  float* sG = sB + C;
  int* sLoc = reinterpret_cast<int*>(sG + C);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long chunk = blockIdx.x;  // operand block index
  int b, h, c;
  if (p.cu == nullptr) {
    const int bh = (int)(chunk / p.nc);
    c = (int)(chunk % p.nc);
    b = bh / p.H;
    h = bh % p.H;
  } else {
    // sequence d owns blocks cbase[d] H .. cbase[d+1] H - 1 (head-major inside)
    if (chunk >= (long long)p.cbase[p.B] * p.H) return;  // past the last block: nothing to do
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)p.cbase[mid] * p.H <= chunk) lo = mid; else hi = mid - 1;
    }
    b = lo;
    const int ncd = p.cbase[b + 1] - p.cbase[b];
    const int rel = (int)(chunk - (long long)p.cbase[b] * p.H);
    h = rel / ncd;
    c = rel % ncd;
  }
  const SeqGeom sg = seq_geom(p, b, h, C);
  const int N = sg.N;
  const int s0 = c * C, n_h = p.n_h;
  const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));  // first readout
  const long long tok0 = sg.tok * p.H + h;  // token (sequence start, head h)
  const bf16_t* kp = static_cast<const bf16_t*>(p.k);
  const bf16_t* kwp = static_cast<const bf16_t*>(p.kt);
  const bf16_t* qp = static_cast<const bf16_t*>(p.q);
  unsigned char* wsc = static_cast<unsigned char*>(p.wsT) + chunk * W.bytes;

  // 1. global loads: key rows, readout query rows, beta, gate.  Every lane
  //    loads on every path: rows past the end (or the padding of a ragged
  //    chunk) read the chunk's first sub-step, which exists, and are masked
  //    where the value is first used.  (A load inside a branch joins a
  //    zero-initialised copy of its register, and that copy waits for the
  //    load at once: the loads would go out as several round trips.)
  constexpr bool QREG = prep_q_in_regs(DK);
  constexpr int QKS = DK / 32;  // 32-deep steps of a query fragment row
  u32x4_t rk[KIT], rq[QIT], rkw[ASYM ? KIT : 1];
  bool kin[KIT], qin[QREG ? NRT : QIT];
  auto sub_row = [&](int s) {  // row of sub-step s in the [.., n_h, DK] tensors, without the column
    const int t = fastdiv(s, p.nh_magic, p.nh_shift);
    return ((tok0 + (long long)t * p.H) * n_h + (s - t * n_h)) * DK;
  };
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * 256;
    const int r = idx / TPR, cg = idx % TPR;
    const int s = s0 + r;
    kin[it] = idx < KV && s < N;
    const long long row = sub_row(kin[it] ? s : s0) + cg * 8;
    rk[it] = ld16(kp + row);
    if constexpr (ASYM) rkw[it] = ld16(kwp + row);
  }
  // beta and the gate of sub-step tid (threads tid < C; the others read sub-step s0)
  const bool bin = tid < C && s0 + tid < N;
  float braw, graw = 1.f;
  bool gin;
  {
    const int s = bin ? s0 + tid : s0;
    const int t = fastdiv(s, p.nh_magic, p.nh_shift);
    const int j = s - t * n_h;
    const long long tok = tok0 + (long long)t * p.H;
    braw = p.beta[tok * n_h + j];
    if (p.g != nullptr) graw = p.g[tok];
    gin = bin && j == 0 && p.g != nullptr;
  }

  // queries: loaded with the keys (one memory round trip per chunk) when
  // their fragments fit the registers (up to two row tiles), else once the
  // key rows are in LDS (fewer registers live at once).
  // QREG: the fragment (row 16 it + n, step t) of lane (n, g) -- columns
  // 32 t + 4 g .. + 3 and 32 t + 16 + 4 g .. + 3 -- as raw bf16
  constexpr bool QEARLY = NRT <= 2;
  u32x4_t qr[QREG ? NRT : 1][QREG ? QKS : 1];
  auto load_queries = [&]() {
    if constexpr (QREG) {
#pragma unroll
      for (int it = 0; it < NRT; ++it) {
        const int i = it * 16 + (lane & 15);
        const int s = r0 + i * n_h;
        const bool ok = s < s0 + C && s < N;
        qin[it] = ok;  // masked where the fragments are converted
        const long long tk = tok0 + (long long)fastdiv(ok ? s : s0, p.nh_magic, p.nh_shift) * p.H;
#pragma unroll
        for (int t = 0; t < QKS; ++t) {
          const bf16_t* src = qp + tk * DK + 32 * t + 4 * (lane >> 4);
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 16);
          qr[it][t] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < QIT; ++it) {
        const int idx = tid + it * 256;
        const int i = idx / TPR, cg = idx % TPR;
        const int s = r0 + i * n_h;
        qin[it] = idx < QV && s < s0 + C && s < N;  // masked where the rows are stored
        const long long tk = tok0 + (long long)fastdiv(qin[it] ? s : s0, p.nh_magic, p.nh_shift) * p.H;
        rq[it] = ld16(qp + tk * DK + cg * 8);
      }
    }
  };
  if constexpr (QEARLY) load_queries();

  // 2. unit keys (row norms by a TPR-lane reduction) and queries, as fp16 rows
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * 256;
    const int r = idx / TPR, cg = idx % TPR;
    float f[8];
    unpack16(rk[it], f, bf16_t{});
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = kin[it] ? f[e] : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    ss = dpp_group_sum<TPR>(ss);
    const float rinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f));  // 1 / max(|k|, 1e-6)
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= rinv;
    if (idx < KV) st_vec16(sK + r * LDK + cg * 8, f);
    if constexpr (ASYM) {
      unpack16(rkw[it], f, bf16_t{});
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = kin[it] ? f[e] : 0.f;
      if (idx < KV) st_vec16(sKW + r * LDK + cg * 8, f);
    }
  }
  if constexpr (!QEARLY) load_queries();
  f16x8_t qf[QREG ? NRT : 1][QREG ? QKS : 1];  // QREG: fp16 query fragments
  if constexpr (QREG) {
#pragma unroll
    for (int it = 0; it < NRT; ++it)
#pragma unroll
      for (int t = 0; t < QKS; ++t) {
        float f[8];
        unpack16(qr[it][t], f, bf16_t{});
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[it][t][e] = (f16_t)(qin[it] ? f[e] : 0.f);
      }
  } else {
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int idx = tid + it * 256;
      const int i = idx / TPR, cg = idx % TPR;
      float f[8];
      unpack16(rq[it], f, bf16_t{});
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = qin[it] ? f[e] : 0.f;
      if (idx < QV) st_vec16(sQ + i * LDK + cg * 8, f);
    }
  }

  // 3. beta range, cumulative log-gate and the per-chunk scalars (wave 0)
  if (wave == 0) {
    const float lam = gin ? logf(fmaxf(graw, FLT_MIN)) : 0.f;
    const float G = p.g != nullptr ? wave_inclusive_scan(lam) : 0.f;  // no gate: all zero
    const float Gl = __shfl(G, C - 1, 64);
    float* sEG = reinterpret_cast<float*>(wsc + W.oS + W.oEG);
    float* sEL = reinterpret_cast<float*>(wsc + W.oS + W.oEL);
    float* sEGL = reinterpret_cast<float*>(wsc + W.oS + W.oEGL);
    long long* sOff = reinterpret_cast<long long*>(wsc + W.oS + W.oOff);
    if (lane < C) {
      sB[lane] = clamp_keep_nan(bin ? braw : 0.f, 0.f, 2.f);  // 0 past the end
      sG[lane] = G;
      sEG[lane] = expf(G);
      sEL[lane] = expf(Gl - G);
    }
    const int s = r0 + lane * n_h;
    const bool ok = lane < RT && s < s0 + C && s < N;
    const int loc = ok ? s - s0 : 0;
    const float Gloc = __shfl(G, loc, 64);
    if (lane < RT) {
      sLoc[lane] = ok ? loc : -1;
      sEGL[lane] = ok ? expf(Gloc) : 0.f;
      sOff[lane] = ok ? (tok0 + (long long)fastdiv(s, p.nh_magic, p.nh_shift) * p.H) * p.dv : -1ll;
    }
  }
  __syncthreads();

  // 4. Kn and Q to the workspace, block-major (16 consecutive rows of a block
  //    per quarter-wave: contiguous global stores, conflict-free LDS reads)
  for (int idx = tid; idx < KV; idx += 256) {
    const int q = idx / C, r = idx % C;
    st16(wsc + W.oK + (q * C + r) * 16, ld16(sK + r * LDK + q * 8));
    if constexpr (ASYM) st16(wsc + W.oKW + (q * C + r) * 16, ld16(sKW + r * LDK + q * 8));
  }
  if constexpr (QREG) {
    // fragment layout: block 4 t + g holds lane (n, g)'s fragment of step t, row 16 it + n
#pragma unroll
    for (int t = 0; t < QKS; ++t) {
      if ((t & 3) != wave) continue;  // every wavefront holds every fragment: wave t % 4 writes step t
#pragma unroll
      for (int it = 0; it < NRT; ++it)
        st16(wsc + W.oQ + ((4 * t + (lane >> 4)) * RT + it * 16 + (lane & 15)) * 16,
             __builtin_bit_cast(u32x4_t, qf[it][t]));
    }
  } else {
    for (int idx = tid; idx < QV; idx += 256) {
      const int q = idx / RT, i = idx % RT;
      st16(wsc + W.oQ + (q * RT + i) * 16, ld16(sQ + i * LDK + q * 8));
    }
  }

  // 5. masked, decayed scores of the readout rows:  P[i][j] = (q_i . kn_j)
  //    e^{G_loc(i) - G_j} for j <= loc(i).  Computed transposed (lane: four
  //    consecutive j of one i) and stored block-major in 8-byte pieces.
  auto p_tile = [&](int it, int jt, f32x4_t acc) {
    const int i = it * 16 + (lane & 15);
    const int loc = sLoc[i];
    const int j0 = jt * 16 + 4 * (lane >> 4);
    const float gl = loc >= 0 ? sG[loc] : 0.f;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + e;
      pv[e] = (j <= loc) ? acc[e] * (p.g != nullptr ? expf(gl - sG[j]) : 1.f) : 0.f;
    }
    const int pblk = frag_layout(C) ? frag_col_block(j0) : (j0 >> 3);
    const int pbyte = frag_layout(C) ? frag_col_byte(j0) : (j0 & 7) * 2;
    st4(reinterpret_cast<f16_t*>(wsc + W.oP + (pblk * RT + i) * 16 + pbyte), pv[0], pv[1], pv[2], pv[3]);
  };
  if constexpr (QREG) {
    // the query fragments are registers: the row tile it is a compile-time index
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      for (int jt = wave; jt < NT; jt += 4) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < QKS; ++t)
          acc = mfma32h(lds_a32(sKW, LDK, jt * 16 + (lane & 15), 32 * t), qf[it][t], acc);
        p_tile(it, jt, acc);
      }
    }
  } else {
    for (int tile = wave; tile < NRT * NT; tile += 4) {
      const int it = tile / NT, jt = tile % NT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_ll<DK>(acc, sKW, LDK, jt * 16 + (lane & 15), sQ, LDK, it * 16 + (lane & 15));
      p_tile(it, jt, acc);
    }
  }
  // 6. M = strict_tril(diag(beta) (E o Kn Kn^T)) on MFMA, lower blocks only
  for (int tile = wave; tile < NT * (NT + 1) / 2; tile += 4) {
    int ti = 0;
    while (prep_mblock(ti + 1, 0) <= tile) ++ti;
    const int tj = tile - prep_mblock(ti, 0);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_ll<DK>(acc, sK, LDK, ti * 16 + (lane & 15), sKW, LDK, tj * 16 + (lane & 15));
    const int jj = tj * 16 + (lane & 15);
    float* mb = sA + tile * kPrepBlk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = ti * 16 + 4 * (lane >> 4) + e;
      float val = 0.f;
      if (jj < ii) val = sB[ii] * (p.g != nullptr ? expf(sG[ii] - sG[jj]) : 1.f) * acc[e];
      mb[(4 * (lane >> 4) + e) * kPrepLdm + (lane & 15)] = val;
    }
  }
  __syncthreads();

  // 7. T = (I + M)^{-1} (fp32), blocked over 16 x 16 tiles: diagonal tiles by
  //    forward substitution (one 16-lane group per tile, one column per
  //    lane), then the off-diagonal tiles level by level (i - j = 1, 2, ..):
  //    T_ij = -T_ii sum_{k=j}^{i-1} M_ik T_kj  on fp32 MFMA.
  if (wave == 0) {
    const int gb = lane >> 4, cc = lane & 15;
    if (gb < NT) {
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == cc) ? 1.f : 0.f;
        const float* ar = sA + prep_mblock(gb, gb) * kPrepBlk + i * kPrepLdm;
#pragma unroll
        for (int j = 0; j < i; ++j) acc = fmaf(-ar[j], t[j], acc);
        t[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTf[prep_mblock(gb, gb) * kPrepBlk + i * kPrepLdm + cc] = t[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int dist = 1; dist < NT; ++dist) {
    const int j = wave, i = wave + dist;
    float* sS = sSc + wave * 16 * 17;
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb)
        acc = mm_tile_tb<float, 16>(acc, sA + prep_mblock(i, kb) * kPrepBlk, kPrepLdm, 0,
                                    sTf + prep_mblock(kb, j) * kPrepBlk, kPrepLdm, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sS[(4 * (lane >> 4) + e) * 17 + (lane & 15)] = acc[e];
    }
    __syncthreads();
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<float, 16>(acc, sTf + prep_mblock(i, i) * kPrepBlk, kPrepLdm, 0, sS, 17, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sTf[prep_mblock(i, j) * kPrepBlk + (4 * (lane >> 4) + e) * kPrepLdm + (lane & 15)] = -acc[e];
    }
    __syncthreads();
  }
  // 8. T diag(beta) to the workspace, block-major (upper tiles zero, or left
  //    out in the trimmed layout: granule idx is then tile t's block g, row i)
  constexpr bool TRIM = t_trimmed(DK, C);
  static_assert(!TRIM || C == 64, "the trimmed layout has two tile rows");
  for (int idx = tid; idx < t_bytes(DK, C) / 16; idx += 256) {
    int q = idx / C, i = idx % C;
    if constexpr (TRIM) {
      int t = 0;
      while (t + 1 < C / 32 && idx >= t_block_byte(C, t + 1) / 16) ++t;
      // rows = C - 32 t: a select of constant divisions, not a division by a variable
      const int rel = idx - t_block_byte(C, t) / 16;
      q = 4 * t + (t == 0 ? rel / C : rel / (C - 32));
      i = 32 * t + (t == 0 ? rel % C : rel % (C - 32));
    }
    // The reads are unconditional: for any row block ib and column block jb
    // below C/16, prep_mblock(ib, jb) stays inside the packed lower blocks, so
    // an upper block reads a stored block and the select drops it.  The
    // compiler then fetches four adjacent columns per 16-byte read, one LDS
    // round trip per granule (a guarded read waits once per element).
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = frag_layout(C) ? 32 * (q >> 2) + 4 * (q & 3) + (e & 3) + 16 * (e >> 2) : q * 8 + e;
      const float tv = sTf[prep_mblock(i >> 4, j >> 4) * kPrepBlk + (i & 15) * kPrepLdm + (j & 15)] * sB[j];
      f[e] = ((j >> 4) > (i >> 4)) ? 0.f : tv;
    }
    st_vec16(reinterpret_cast<f16_t*>(wsc + W.oT + idx * 16), f);
  }
}

// ---------------------------------------------------------------------------
// dp_chain_kernel: the sequential part, one workgroup per (head, BV columns).
//
// LDS tile layout.  A tile of R rows and W columns arrives block-major (W/8
// blocks of R x 16 bytes).  In LDS (a) the rows of logically odd blocks are
// permuted, row r in slot r ^ 8, and (b) when W is a multiple of 32 the blocks
// of each group of four are stored in the order 0, 2, 1, 3.  With (b) the two
// 8-byte halves of an MFMA A fragment (columns 32t + 4g.. and 32t + 16 + 4g..)
// sit exactly one block apart, so one ds_read2_b64 fetches a fragment into
// consecutive registers.  The value tile is the exception: it is row-major
// (BV columns per sub-step), so that each direct-to-LDS copy moves whole rows.

// physical position of logical block q in a region of W columns (an involution)
__host__ __device__ constexpr int blk_pos(int q, int W) {
  return (W % 32 == 0) ? ((q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1)) : q;
}

// Lane part of a row read (A fragment of a 32- or 16-deep step): lane
// (n = l & 15, g = l >> 4) reads row row0 + n, logical blocks 4t + (g >> 1)
// (and 4t + 2 + (g >> 1)), 8-byte half (g & 1).
template <int W>
__device__ __forceinline__ int lane_row(int rows) {
  const int l = threadIdx.x & 63, n = l & 15, g = l >> 4, hi = g >> 1;
  return blk_pos(hi, W) * rows * 16 + (n ^ (8 * hi)) * 16 + 8 * (g & 1);
}
// Lane part of a transposed read (ds_read_b64_tr_b16): source lane i = 4e + a
// of group g points at row j0 + 4g + e, columns d0 + 4a .. d0 + 4a + 3, i.e.
// logical block d0 / 8 + (a >> 1), 8-byte half (a & 1).
template <int W>
__device__ __forceinline__ int lane_tr(int rows) {
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4, e = i >> 2, a = i & 3, hi = a >> 1;
  return blk_pos(hi, W) * rows * 16 + ((4 * g + e) ^ (8 * hi)) * 16 + 8 * (a & 1);
}
// Lane part of a transposed read of a row-major tile W columns wide (W * 2
// bytes per row): source lane i = 4e + a of group g points at row 4g + e,
// columns 4a .. 4a + 3 (plus the tile's row and column offsets).
template <int W>
__device__ __forceinline__ int lane_tr_rows() {
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4, e = i >> 2, a = i & 3;
  return ((4 * g + e) * W + 4 * a) * 2;
}
// block offset (immediate part) of logical block pair base 2 * dt (d0 = 16 dt)
template <int W>
__host__ __device__ constexpr int tr_block(int dt) {
  return (W % 32 == 0) ? 4 * (dt >> 1) + (dt & 1) : 2 * dt;
}

// A fragments of a 16 x K operand from block-major rows (K = W of the region).
template <int ROWS, int K, bool FRAG>
struct RowFrags {
  f16x8_t f[K / 32 > 0 ? K / 32 : 1];
  f16x4_t r;  // the last 16 of the contraction when K % 32 == 16
  // `off`: LDS byte offset of this 16-row tile, lane part included (lane_frag
  // for the fragment layout, lane_row otherwise).  In the plain layout the two
  // halves of a fragment are one block apart; each half gets its own opaque
  // base so that they stay two ds_read_b64 (a paired ds_read2 of this pattern
  // is bank-conflicted four ways).
  __device__ __forceinline__ void load(const unsigned char* lds, uint32_t off) {
    if constexpr (FRAG) {
      asm volatile("" : "+v"(off));
#pragma unroll
      for (int t = 0; t < K / 32; ++t) f[t] = *reinterpret_cast<const f16x8_t*>(lds + off + 4 * t * ROWS * 16);
    } else {
      uint32_t off1 = off + ROWS * 16;
      asm volatile("" : "+v"(off), "+v"(off1));
#pragma unroll
      for (int t = 0; t < K / 32; ++t)
        f[t] = cat8(*reinterpret_cast<const f16x4_t*>(lds + off + 4 * t * ROWS * 16),
                    *reinterpret_cast<const f16x4_t*>(lds + off1 + 4 * t * ROWS * 16));
      if constexpr (K % 32 == 16) r = *reinterpret_cast<const f16x4_t*>(lds + off + ((K - 16) / 8) * ROWS * 16);
    }
  }
  __device__ __forceinline__ f32x4_t mma(f32x4_t acc, const f16x4_t* b) const {
#pragma unroll
    for (int t = 0; t < K / 32; ++t) acc = mfma32h(f[t], cat8(b[2 * t], b[2 * t + 1]), acc);
    if constexpr (K % 32 == 16) acc = mfma16h(r, b[K / 16 - 1], acc);
    return acc;
  }
};
// Lane part of a row read in the fragment layout: lane (n, g) reads row n of block g.
__device__ __forceinline__ int lane_frag(int rows) {
  const int l = threadIdx.x & 63;
  return (l >> 4) * rows * 16 + (l & 15) * 16;
}

// A fragments of the transpose (16 x K) of block-major rows 0..K-1, columns
// d0..d0+15 of a region W columns wide.
template <int ROWS, int W, int K>
struct TrFrags {
  f16x8_t f[K / 32 > 0 ? K / 32 : 1];
  f16x4_t r;
  __device__ __forceinline__ static f16x4_t rd(const unsigned char* p) {
    return __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
  }
  __device__ __forceinline__ void load(const unsigned char* base, int dt) {
    const unsigned char* p = base + tr_block<W>(dt) * ROWS * 16;
#pragma unroll
    for (int t = 0; t < K / 32; ++t) f[t] = cat8(rd(p + 32 * t * 16), rd(p + (32 * t + 16) * 16));
    if constexpr (K % 32 == 16) r = rd(p + (K - 16) * 16);
  }
  __device__ __forceinline__ f32x4_t mma(f32x4_t acc, const f16x4_t* b) const {
#pragma unroll
    for (int t = 0; t < K / 32; ++t) acc = mfma32h(f[t], cat8(b[2 * t], b[2 * t + 1]), acc);
    if constexpr (K % 32 == 16) acc = mfma16h(r, b[K / 16 - 1], acc);
    return acc;
  }
};

// One direct-to-LDS copy: each lane moves 16 bytes from `src` to LDS byte
// address lds + 16 * lane.  Written as inline assembly: completion is tracked
// by the caller's explicit vmcnt waits (the compiler's own tracking of the
// builtin inserts a full vmcnt(0) wait whenever it reuses an address register,
// which would serialize the copy pipeline).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// keep the scheduler from moving instructions across this point
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, each with a compile-time index
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Order of the MFMA steps inside one product of the pipelined chain body: step
// j of a product with `ntile` output tiles and `nk` 32-deep contraction steps
// works on tile step_tile(j) and contraction step step_k(j).  The contraction
// step is outermost, so consecutive MFMAs accumulate into different tiles and
// none waits for the result of the one before it; a tile is complete at its
// last contraction step.
__host__ __device__ constexpr int step_tile(int j, int ntile) { return j % ntile; }
__host__ __device__ constexpr int step_k(int j, int ntile) { return j / ntile; }

// Step schedule of the pipelined chain body (see dp_chain_kernel): phase
// starts S2, S3, S4 and end NS; a tile conversion for step k runs in
// iteration min(k + LA + DL, next phase start + LA).
template <int S2, int S3, int S4, int NS, int LA, int DL>
__host__ __device__ constexpr int chain_conv_iter(int k) {
  const int nxt = k < S2 ? S2 : (k < S3 ? S3 : (k < S4 ? S4 : NS));
  return (k + LA + DL) < (nxt + LA) ? (k + LA + DL) : (nxt + LA);
}

// Copy wavefronts per dp_chain_kernel workgroup: one wavefront issues about one
// 1 KB direct-to-LDS copy per ~60 cycles, so the copies of a chunk are split.
constexpr int kChainCopyWaves = 2;

// Third descriptor word of a raw (stride 0) gfx9 buffer resource: 32-bit data
// format; the hardware then bounds each access by the resource's byte size.
constexpr int kBufferDword3 = 0x00020000;

// ASYM: the state update reads the block's write keys (transposed) where the
// symmetric form reads Kn; everything else is the same.
template <int DK, int C, int NWC, int NRT, bool GATED, bool ASYM = false>
__global__ __launch_bounds__(64 * (NWC + kChainCopyWaves)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dp_chain_kernel(FwdArgs p) {
  constexpr int RT = 16 * NRT, BV = 16 * NWC;
  constexpr int NCT = C / 16, NDT = DK / 16;
  constexpr Chunk16Layout W = chunk16_layout(DK, C, RT, ASYM);
  constexpr int STG = chain_stages(DK, C, RT, BV, ASYM);  // LDS ring stages
  // With four stages and a pipelined body whose first kLookahead steps are
  // key fragments, the consumers read the next chunk's first operands while
  // finishing the current one, so each chunk must land one chunk earlier.
  constexpr bool EARLY = chain_early(DK, C, STG);
  constexpr int VB = C * BV * 2;                      // value tile bytes
  constexpr int STAGE = W.bytes + VB;
  // Bytes of each block the scan reads: the ungated pipelined body needs none
  // of the per-chunk scalars at the block's end (its decay factors are all 1
  // and it bounds the readout rows itself), so its copies stop before them.
  constexpr bool PIPE = DK % 32 == 0 && C % 32 == 0;
  static_assert(!ASYM || PIPE, "the write-key form runs on the pipelined body only");
  constexpr int CB = (PIPE && !GATED) ? W.oS : W.bytes;
  constexpr int NIB = (CB + 1023) / 1024;             // copies per chunk block
  constexpr int NIV = VB / 1024 > 0 ? VB / 1024 : 1;  // copies per value tile
  constexpr int VPI = VB >= 1024 ? 64 : VB / 16;      // lanes per value copy
  constexpr int NI = NIB + NIV;
  constexpr int NCW = kChainCopyWaves;
  // copies of copy wavefront w: indices m = w, w + NCW, .. of the NI copies
  constexpr int NI0 = (NI + NCW - 1) / NCW, NI1 = NI / NCW;
  static_assert(NCW == 2, "two copy wavefronts");
  static_assert((STG - 2) * NI0 < 64, "copies in flight exceed the vmcnt range");
  static_assert(VB % 16 == 0 && (VB < 1024 || VB % 1024 == 0), "value tile");

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware mapping: consecutive workgroup ids go round-robin over the 8
  // XCDs, so spread ids so that the value blocks of one head share an XCD
  // (and its L2) for the operand blocks they all read.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int f = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int bh = f / p.nvb, vb = f % p.nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;
  const SeqGeom sg = seq_geom(p, b, h, C);
  const int nc = sg.nc, N = sg.N;
  const unsigned char* wsh = static_cast<const unsigned char*>(p.wsT) + sg.blk0 * W.bytes;

  if (wave >= NWC) {
    // =============================================================== copy waves
    // Source offset of each lane in each copy of the chunk block: in the
    // plain-layout tiles, LDS slot (physical block, row slot) holds logical
    // block blk_pos(physical) and row slot ^ 8 for odd logical blocks; the
    // fragment-layout tiles and the scalars are copied as they are.
    const int cw = wave - NWC;
    int soff[NIB];
    // Readout rows past ceil(C / n_h), the most any chunk has, are padding in
    // the Q and P tiles: their lanes copy nothing (the LDS rows keep whatever
    // they held; they only ever feed output rows that are never stored).
    const int rmax = (C + p.n_h - 1) / p.n_h;
    bool keep[NIB];
#pragma unroll
    for (int m = 0; m < NIB; ++m) {
      const int o = 1024 * m + 16 * lane;
      int src = o;
      auto region = [&](int start, int rows, int cols) {
        if (!frag_layout(cols) && o >= start && o < start + rows * cols * 2) {
          const int rel = o - start, pb = rel / (rows * 16), rs = (rel / 16) % rows;
          const int q = blk_pos(pb, cols);
          src = start + q * rows * 16 + (rs ^ (8 * (q & 1))) * 16;
        }
      };
      region(W.oT, C, C);
      // the keys keep the plain layout whatever their width (they are also read
      // transposed); so do the write keys
      auto keys = [&](int start) {
        if (o >= start && o < start + C * DK * 2) {
          const int rel = o - start, pb = rel / (C * 16), rs = (rel / 16) % C;
          const int q = blk_pos(pb, DK);
          src = start + q * C * 16 + (rs ^ (8 * (q & 1))) * 16;
        }
      };
      keys(W.oK);
      if constexpr (ASYM) keys(W.oKW);
      region(W.oQ, RT, DK);
      region(W.oP, RT, C);
      soff[m] = src;
      keep[m] = true;
      // (fragment-layout tiles are copied as they are: LDS row = tile row)
      if (frag_layout(DK) && o >= W.oQ && o < W.oQ + RT * DK * 2 && ((o - W.oQ) / 16) % RT >= rmax) keep[m] = false;
      if (frag_layout(C) && o >= W.oP && o < W.oP + RT * C * 2 && ((o - W.oP) / 16) % RT >= rmax) keep[m] = false;
    }
    const bf16_t* vp = static_cast<const bf16_t*>(p.v) + v0;
    const long long tok0 = sg.tok * p.H + h;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;  // LDS byte address of the ring
    // copies of chunk c issued by copy wavefront CW: index m = CW, CW + NCW, ..
    auto issue = [&](auto cwc, int c) {
      constexpr int CW = decltype(cwc)::value;
      const uint32_t st = lds0 + (uint32_t)((c % STG) * STAGE);
      const unsigned char* src = wsh + (long long)c * W.bytes;
      static_for<NIB>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m % NCW == CW) {
          if (1024 * m + 16 * lane < CB && keep[m]) dma16(src + soff[m], st + 1024 * m);
        }
      });
      // value tile, row-major (BV * 2 bytes per sub-step): each copy moves
      // whole runs of BV columns of consecutive sub-steps
      static_for<NIV>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr ((NIB + m) % NCW == CW) {
          const int o = 1024 * m + 16 * lane;
          const int r = o / (BV * 2), cv = (o % (BV * 2)) / 2;  // tile row, first column
          int s = c * C + r;
          s = s < N ? s : N - 1;  // rows past the end: any valid row (their beta is 0)
          const int t = fastdiv(s, p.nh_magic, p.nh_shift);
          const long long row = (tok0 + (long long)t * p.H) * p.n_h + (s - t * p.n_h);
          if (lane < VPI) dma16(vp + row * p.dv + cv, st + W.bytes + 1024 * m);
        }
      });
    };
    auto run = [&](auto cwc) {
      constexpr int CW = decltype(cwc)::value;
      constexpr int NMINE = CW == 0 ? NI0 : NI1;  // copies per chunk of this wavefront
      // wait until at most `ahead` chunks' copies of this wavefront are in flight
      auto wait_ahead = [&](int ahead) {
        if (ahead >= 2) {
          wait_vmcnt<(STG > 3 ? 2 : 1) * NMINE>();
        } else if (ahead == 1) {
          wait_vmcnt<NMINE>();
        } else {
          wait_vmcnt<0>();
        }
      };
      // at X(c) chunk c has landed, and chunk c + 1 too when EARLY
      constexpr int LEAD = EARLY ? 1 : 0;
      const int pre = nc < STG - 1 ? nc : STG - 1;  // chunks 0 .. STG-2 up front
      for (int j = 0; j < pre; ++j) issue(cwc, j);
      if (nc > 0) {
        const int a0 = pre - 1 - LEAD;
        wait_ahead(a0 > 0 ? a0 : 0);
        block_sync_lds();  // X(0)
      }
      for (int c = 0; c + 1 < nc; ++c) {
        if (c + STG - 1 < nc) issue(cwc, c + STG - 1);  // into the stage chunk c - 1 used
        const int last = c + STG - 1 < nc ? c + STG - 1 : nc - 1;
        const int a = last - (c + 1 + LEAD);
        wait_ahead(a > 0 ? a : 0);
        block_sync_lds();  // X(c + 1)
      }
    };
    if (cw == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});
    return;
  }

  // ==================================================================== consumers
  const int col = lane & 15, grp = lane >> 4;
  const int vw = 16 * wave;  // this wavefront's columns inside the block
  const int lrK = lane_row<DK>(C);
  const int lrT = frag_layout(C) ? lane_frag(C) : lane_row<C>(C);
  const int lrQ = frag_layout(DK) ? lane_frag(RT) : lane_row<DK>(RT);
  const int lrP = frag_layout(C) ? lane_frag(RT) : lane_row<C>(RT);
  const int ltK = lane_tr<DK>(C), ltV = lane_tr_rows<BV>();
  const int ocol = v0 + vw + col;  // output column of this lane
  float* const sink = p.sink + ((long long)f * NWC + wave) * 64 + lane;
  f32x4_t hacc[NDT];
  f16x4_t hq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    hacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p.h0 != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[dt][e] = p.h0[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + vw + col];
    }
    hq[dt] = to_h4(hacc[dt]);
  }
  if constexpr (DK % 32 == 0 && C % 32 == 0) {
    // Software-pipelined chunk body.  The MFMA steps of a chunk run in a fixed
    // order -- Kn H (X), Q H (readout), T X (Up), P Up (readout), Kn^T Us
    // (state) -- and the A fragment of step i is read LA steps ahead.  The
    // tile conversions that feed later products run DL steps after the MFMA
    // that completes the tile, or at the start of the product that needs
    // them, whichever comes first; each converted tile is pinned where it is
    // made (an empty asm), so the compiler cannot sink the state's
    // conversions past the chunk's barrier.
    constexpr int KST = DK / 32, CST = C / 32;
    constexpr int S1 = NCT * KST, S2 = S1 + NRT * KST, S3 = S2 + NCT * CST, S4 = S3 + NRT * CST;
    constexpr int NS = S4 + NDT * CST;
    constexpr int LA = kLookahead, DL = 4;
    constexpr bool TRIM = t_trimmed(DK, C);
    constexpr int TS = TRIM ? 32 : 0;  // first stored row of T tile t is TS t
    // Readout row i of a chunk is token t0 + i: consecutive tokens, H dv
    // elements apart in out.  Each chunk stores through a buffer resource
    // based at its first row and bounded by its nrd rows, so this lane's
    // element of row 16 it + 4 grp + e sits at a byte offset that is the
    // same for every chunk, and the padding rows (from nrd on) fall outside
    // the bound, where the hardware drops the store.
    const int HD = p.H * p.dv;
    const int es = p.out_f32 ? 4 : 2;
    int voff[NRT][4], voff4[NRT];
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
#pragma unroll
      for (int e = 0; e < 4; ++e) voff[it][e] = ((16 * it + 4 * grp + e) * HD + ocol) * es;
      // after the quad transpose (bf16): row 16 it + 4 grp + (col & 3), columns from ocol - (col & 3)
      voff4[it] = ((16 * it + 4 * grp + (col & 3)) * HD + ocol - (col & 3)) * 2;
    }
    // byte selector of the second transpose step: even lanes keep their low
    // halves and take the partner's low halves above them, odd lanes the highs
    const uint32_t qsel = (lane & 1) ? 0x03020706u : 0x05040100u;
    f16x4_t hqn[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) hqn[dt] = to_h4(hacc[dt]);
    // step list padded to a multiple of LA: the next chunk's step k then lands
    // in ring slot k % LA, the slot its MFMA reads
    constexpr int NSP = EARLY ? (NS + LA - 1) / LA * LA : NS;
    static_assert(!EARLY || S1 >= LA, "early fragments must be key fragments");
    f32x4_t vf[NCT], eg[NCT], el[NCT], egl[NRT];
    float dec = 1.f;
    f16x8_t ring[LA];
    // the first LA fragments of the next chunk, read during this one (EARLY): a
    // loop-carried array of its own, written once per chunk, so that the
    // compiler keeps it in place across the back edge
    f16x8_t pre[EARLY ? LA : 1];
    // per-chunk small operands of the chunk in stage byte offset `so`
    auto load_small = [&](uint32_t so) {
      const unsigned char* st = smem + so;
      const float* sEG = reinterpret_cast<const float*>(st + W.oS + W.oEG);
      const float* sEL = reinterpret_cast<const float*>(st + W.oS + W.oEL);
      const float* sEGL = reinterpret_cast<const float*>(st + W.oS + W.oEGL);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        // V[16 ct + 4 grp + e][vw + col] (bf16) in accumulator layout
        const s16x4_t vr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(st + W.bytes + ltV + (16 * ct * BV + 16 * wave) * 2));
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[ct][e] = __uint_as_float((uint32_t)(uint16_t)vr[e] << 16);
        if constexpr (GATED) {
          eg[ct] = *reinterpret_cast<const f32x4_t*>(sEG + ct * 16 + 4 * grp);
          el[ct] = *reinterpret_cast<const f32x4_t*>(sEL + ct * 16 + 4 * grp);
        }
      }
#pragma unroll
      for (int it = 0; it < NRT; ++it) {
        if constexpr (GATED) egl[it] = *reinterpret_cast<const f32x4_t*>(sEGL + it * 16 + 4 * grp);
      }
      if constexpr (GATED) dec = sEG[C - 1];
    };
    // key fragment k (< LA) of the chunk whose key tiles start at ok / ok1
    auto key_frag = [&](const uint32_t* ok, const uint32_t* ok1, auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ct = step_tile(k, NCT), ko = 4 * step_k(k, NCT) * C * 16;
      pre[k] = cat8(*reinterpret_cast<const f16x4_t*>(smem + ok[ct] + ko),
                    *reinterpret_cast<const f16x4_t*>(smem + ok1[ct] + ko));
    };
    if (nc > 0) block_sync_lds();  // X(0)
    if constexpr (EARLY) {
      if (nc > 0) {  // chunk 0's small operands and first LA fragments (stage 0)
        uint32_t ok[NCT], ok1[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          ok[ct] = W.oK + lrK + ct * 256;
          ok1[ct] = ok[ct] + C * 16;
          asm volatile("" : "+v"(ok[ct]), "+v"(ok1[ct]));
        }
        load_small(0);
        static_for<LA>([&](auto kc) { key_frag(ok, ok1, kc); });
      }
    }
    // Per-chunk context: LDS offsets of the chunk's stage (opaque, so that the
    // two halves of a key fragment keep their own bases) and its readout rows.
    // The context of chunk c + 1 is built while chunk c runs, so that little
    // is left between the chunk barrier and the next products.
    struct ChunkCtx {
      uint32_t so, oK[NCT], oK1[NCT], oT[CST], oQ[NRT], oP[NRT];
      int t0, nrd;  // readout rows i < nrd are the tokens t0 + i
    };
    auto make_ctx = [&](int cc) __attribute__((always_inline)) {
      ChunkCtx x;
      x.so = (uint32_t)((cc % STG) * STAGE);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        x.oK[ct] = x.so + W.oK + lrK + ct * 256;
        x.oK1[ct] = x.oK[ct] + C * 16;  // second half of each key fragment: one block on
        asm volatile("" : "+v"(x.oK[ct]), "+v"(x.oK1[ct]));
      }
      // T diag(beta): one base per 32-column tile t (rows from 32 t on when trimmed)
#pragma unroll
      for (int t = 0; t < CST; ++t) {
        x.oT[t] = x.so + W.oT + (TRIM ? t_block_byte(C, t) : 4 * t * C * 16) + (lane >> 4) * (C - TS * t) * 16 +
                  (lane & 15) * 16;
        asm volatile("" : "+v"(x.oT[t]));
      }
#pragma unroll
      for (int it = 0; it < NRT; ++it) {
        x.oQ[it] = x.so + W.oQ + lrQ + it * 256;
        x.oP[it] = x.so + W.oP + lrP + it * 256;
        asm volatile("" : "+v"(x.oQ[it]), "+v"(x.oP[it]));
      }
      x.t0 = fastdiv(cc * C, p.nh_magic, p.nh_shift);
      x.nrd = fastdiv(min(cc * C + C, N), p.nh_magic, p.nh_shift) - x.t0;
      return x;
    };
    ChunkCtx cur = make_ctx(0);
    for (int c = 0; c < nc; ++c) {
      const uint32_t so = cur.so;
      const unsigned char* st = smem + so;
      const uint32_t *oK = cur.oK, *oK1 = cur.oK1, *oT = cur.oT, *oQ = cur.oQ, *oP = cur.oP;
      const long long rowbase = ((sg.tok + cur.t0) * p.H + h) * p.dv;
      const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<char*>(p.out) + rowbase * es, 0, cur.nrd * HD * es, kBufferDword3);
      // the next chunk's context (this chunk's again after the last: its reads are then unused)
      ChunkCtx nxt;
      if constexpr (!EARLY) load_small(so);

      f32x4_t accX[NCT], accU[NCT], z[NRT];
      f16x4_t xq[NCT], uq[NCT], usq[NCT];
      auto load_frag = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i >= S2 && i < S3 && TRIM && step_tile(i - S2, NCT) < 2 * step_k(i - S2, NCT)) {
          return;  // zero tile of T diag(beta): no read, no product
        }
        f16x8_t fr;
        if constexpr (i < S1) {
          constexpr int ct = step_tile(i, NCT), ko = 4 * step_k(i, NCT) * C * 16;
          fr = cat8(*reinterpret_cast<const f16x4_t*>(smem + oK[ct] + ko),
                    *reinterpret_cast<const f16x4_t*>(smem + oK1[ct] + ko));
        } else if constexpr (i < S2) {
          constexpr int j = i - S1;
          fr = *reinterpret_cast<const f16x8_t*>(smem + oQ[step_tile(j, NRT)] + 4 * step_k(j, NRT) * RT * 16);
        } else if constexpr (i < S3) {
          constexpr int j = i - S2;
          constexpr int ct = step_tile(j, NCT), t = step_k(j, NCT);
          fr = *reinterpret_cast<const f16x8_t*>(smem + oT[t] + (16 * ct - TS * t) * 16);
        } else if constexpr (i < S4) {
          constexpr int j = i - S3;
          fr = *reinterpret_cast<const f16x8_t*>(smem + oP[step_tile(j, NRT)] + 4 * step_k(j, NRT) * RT * 16);
        } else {
          constexpr int j = i - S4;
          const unsigned char* q =
              st + W.oKW + ltK + tr_block<DK>(step_tile(j, NDT)) * C * 16 + 32 * step_k(j, NDT) * 16;
          fr = cat8(__builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)q)),
                    __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(q + 256))));
        }
        ring[i % LA] = fr;
      };
      auto mfma_step = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        f16x8_t a;
        if constexpr (EARLY && i < LA)
          a = pre[i];
        else
          a = ring[i % LA];
        if constexpr (i < S1) {
          constexpr int ct = step_tile(i, NCT), t = step_k(i, NCT);
          accX[ct] = mfma32h(a, cat8(hqn[2 * t], hqn[2 * t + 1]), t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : accX[ct]);
        } else if constexpr (i < S2) {
          constexpr int j = i - S1, it = step_tile(j, NRT), t = step_k(j, NRT);
          z[it] = mfma32h(a, cat8(hqn[2 * t], hqn[2 * t + 1]), t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : z[it]);
        } else if constexpr (i < S3) {
          constexpr int j = i - S2, ct = step_tile(j, NCT), t = step_k(j, NCT);
          if constexpr (!(TRIM && ct < 2 * t))
            accU[ct] = mfma32h(a, cat8(xq[2 * t], xq[2 * t + 1]), t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : accU[ct]);
        } else if constexpr (i < S4) {
          constexpr int j = i - S3, it = step_tile(j, NRT), t = step_k(j, NRT);
          z[it] = mfma32h(a, cat8(uq[2 * t], uq[2 * t + 1]), z[it]);
        } else {
          constexpr int j = i - S4, dt = step_tile(j, NDT), t = step_k(j, NDT);
          if constexpr (GATED && t == 0) hacc[dt] = hacc[dt] * dec;
          hacc[dt] = mfma32h(a, cat8(usq[2 * t], usq[2 * t + 1]), hacc[dt]);
        }
      };
      auto conv = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < S1) {
          if constexpr (step_k(k, NCT) == KST - 1) {
            constexpr int ct = step_tile(k, NCT);
            if constexpr (GATED)
              xq[ct] = to_h4(vf[ct] - eg[ct] * accX[ct]);  // accX = Kn H
            else
              xq[ct] = to_h4(vf[ct] - accX[ct]);
            asm volatile("" : "+v"(xq[ct]));
          }
        } else if constexpr (k < S2) {
          if constexpr (step_k(k - S1, NRT) == KST - 1) {
            constexpr int it = step_tile(k - S1, NRT);
            if constexpr (GATED) z[it] = z[it] * egl[it];  // e^{G_loc} = 1 without a gate
          }
        } else if constexpr (k < S3) {
          if constexpr (step_k(k - S2, NCT) == CST - 1) {
            constexpr int ct = step_tile(k - S2, NCT);
            uq[ct] = to_h4(accU[ct]);
            asm volatile("" : "+v"(uq[ct]));
            if constexpr (GATED) {
              usq[ct] = to_h4(accU[ct] * el[ct]);
              asm volatile("" : "+v"(usq[ct]));
            } else {
              usq[ct] = uq[ct];
            }
          }
        } else if constexpr (k < S4) {
          // the readout tiles are stored after the chunk's last product (below)
        } else {
          if constexpr (step_k(k - S4, NDT) == CST - 1) {
            constexpr int dt = step_tile(k - S4, NDT);
            hqn[dt] = to_h4(hacc[dt]);
            asm volatile("" : "+v"(hqn[dt]));
          }
        }
      };
      static_for<NSP + LA + DL>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        // conversions due in this iteration: steps k in [i - LA - DL, i - LA]
        static_for<DL + 1>([&](auto wc) {
          constexpr int k = i - LA - DL + decltype(wc)::value;
          if constexpr (k >= 0 && k < NS) {
            if constexpr (chain_conv_iter<S2, S3, S4, NS, LA, DL>(k) == i) conv(std::integral_constant<int, k>{});
          }
        });
        if constexpr (i >= LA && i - LA < NS) mfma_step(std::integral_constant<int, i - LA>{});
        if constexpr (i == LA + 2) nxt = make_ctx(c + 1 < nc ? c + 1 : c);
        if constexpr (EARLY) {
          // steps 0 .. LA-1 were read during the previous chunk
          if constexpr (i >= LA && i < NS) load_frag(std::integral_constant<int, i>{});
          if constexpr (i >= NSP && i < NSP + LA) key_frag(nxt.oK, nxt.oK1, std::integral_constant<int, i - NSP>{});
          if constexpr (i == NS + LA) load_small(nxt.so);  // past this chunk's last use of them
        } else {
          if constexpr (i < NS) load_frag(std::integral_constant<int, i>{});
        }
        sched_fence();
      });
      // Readout rows, stored once the chunk's products are issued: the copy
      // wavefronts' transfers of a later chunk, issued after the previous
      // barrier, have left the vector-memory path by now, so the stores do not
      // queue behind them.  Rows from nrd on are padding: out of the
      // resource's bound, dropped.
#pragma unroll
      for (int it = 0; it < NRT; ++it) {
        if (p.out_f32) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z[it][e]), orsrc, voff[it][e], 0, 0);
        } else {
          // bf16: transpose each quad of lanes' 4 x 4 values (lane 4q + a of a
          // group holds rows 4g + e of column 4q + a; afterwards row 4g + a of
          // columns 4q .. 4q + 3), so one 8-byte store per lane writes the tile
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
  } else {
  if (nc > 0) block_sync_lds();  // X(0)
  for (int c = 0; c < nc; ++c) {
    const uint32_t so = (uint32_t)((c % STG) * STAGE);
    const unsigned char* st = smem + so;
    const float* sEG = reinterpret_cast<const float*>(st + W.oS + W.oEG);
    const float* sEL = reinterpret_cast<const float*>(st + W.oS + W.oEL);
    const float* sEGL = reinterpret_cast<const float*>(st + W.oS + W.oEGL);
    const long long* sOff = reinterpret_cast<const long long*>(st + W.oS + W.oOff);

    // ---- operands of X and of the readout's Q H, all issued before the first product
    RowFrags<C, DK, false> fk[NCT];
    RowFrags<RT, DK, frag_layout(DK)> fq[NRT];
    s16x4_t vr[NCT];
    f32x4_t eg[NCT], egl[NRT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      fk[ct].load(smem, so + W.oK + lrK + ct * 256);
      vr[ct] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(st + W.bytes + ltV + (16 * ct * BV + 16 * wave) * 2));
      eg[ct] = *reinterpret_cast<const f32x4_t*>(sEG + ct * 16 + 4 * grp);
    }
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      fq[it].load(smem, so + W.oQ + lrQ + it * 256);
      egl[it] = *reinterpret_cast<const f32x4_t*>(sEGL + it * 16 + 4 * grp);
    }
    RowFrags<C, C, frag_layout(C)> ft[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) ft[ct].load(smem, so + W.oT + lrT + ct * 256);
    sched_fence();

    // ---- X = V - diag(e^G) (Kn H);  Z = diag(e^{G_loc}) Q H  (both read H)
    f16x4_t xq[NCT];
    f32x4_t z[NRT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f32x4_t acc = fk[ct].mma(f32x4_t{0.f, 0.f, 0.f, 0.f}, hq);
      f32x4_t x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __uint_as_float((uint32_t)(uint16_t)vr[ct][e] << 16) - eg[ct][e] * acc[e];
      xq[ct] = to_h4(x);
    }
#pragma unroll
    for (int it = 0; it < NRT; ++it) z[it] = fq[it].mma(f32x4_t{0.f, 0.f, 0.f, 0.f}, hq) * egl[it];
    // operands of the readout's P Up, issued while X and Up are computed
    RowFrags<RT, C, frag_layout(C)> fp[NRT];
    long long off[NRT][4];
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      fp[it].load(smem, so + W.oP + lrP + it * 256);
#pragma unroll
      for (int e = 0; e < 4; ++e) off[it][e] = sOff[it * 16 + 4 * grp + e];
    }
    f32x4_t el[NCT];
    if constexpr (GATED) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) el[ct] = *reinterpret_cast<const f32x4_t*>(sEL + ct * 16 + 4 * grp);
    }
    sched_fence();

    // ---- Up = (T diag(beta)) X;  Us = diag(e^{G_last - G}) Up
    f16x4_t uq[NCT], usq[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f32x4_t acc = ft[ct].mma(f32x4_t{0.f, 0.f, 0.f, 0.f}, xq);
      uq[ct] = to_h4(acc);
      if constexpr (GATED)
        usq[ct] = to_h4(acc * el[ct]);
      else
        usq[ct] = uq[ct];
    }
    // operands of the state update, issued while the readout is computed
    TrFrags<C, DK, C> fkt[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) fkt[dt].load(st + W.oK + ltK, dt);
    sched_fence();

    // ---- H = e^{G_last} H + Kn^T Us;  O = Z + P Up for the readout rows, written
    //      out (rows of missing readouts go to this lane's slot of the sink)
    const float dec = sEG[C - 1];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if constexpr (GATED) hacc[dt] = hacc[dt] * dec;
      hacc[dt] = fkt[dt].mma(hacc[dt], usq);
    }
#pragma unroll
    for (int it = 0; it < NRT; ++it) z[it] = fp[it].mma(z[it], uq);
    if (p.out_f32) {
#pragma unroll
      for (int it = 0; it < NRT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(off[it][e] >= 0 ? static_cast<float*>(p.out) + off[it][e] + ocol : sink) = z[it][e];
    } else {
#pragma unroll
      for (int it = 0; it < NRT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(off[it][e] >= 0 ? static_cast<bf16_t*>(p.out) + off[it][e] + ocol : reinterpret_cast<bf16_t*>(sink)) =
              __builtin_bit_cast(bf16_t, (__bf16)z[it][e]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) hq[dt] = to_h4(hacc[dt]);
    if (c + 1 < nc) block_sync_lds();  // X(c + 1)
  }

  }

  if (p.fstate != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.fstate[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + vw + col] = hacc[dt][e];
  }
}

}  // namespace dp
