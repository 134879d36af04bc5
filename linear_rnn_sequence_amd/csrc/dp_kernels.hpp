// dp_kernels.hpp -- gfx950 kernels of the chunkwise DeltaProduct forward.
//
// The forward follows the DeltaProduct study notes (arXiv 2502.10297v7):
// sec. 2.2 Eq.(3) (n_h ordered generalized-Householder sub-steps per token),
// sec. 2.6 (per-token gate before the sub-steps, readout H^T q) and sec. 4.1
// (the sequence expanded to L*n_h interleaved sub-steps, gate (g,1,..,1),
// only each token's last sub-step read out), computed in the chunkwise WY/UT
// form of the OSDN study notes (arXiv 2605.13473v1) sec. 2.5 (App.A.2),
// extended with the chunk-local cumulative log-gate G (E_ij = e^{G_i - G_j}):
//
//   M  = strict_tril(diag(beta) (E o Kn Kw^T)),  T = (I + M)^{-1}
//   Up = T diag(beta) (V - diag(e^G) Kn H0)                 (pseudo-values)
//   O  = diag(e^G) Q H0 + (tril_incl(Q Kw^T) o E) Up         (readout rows)
//   H1 = e^{G_last} H0 + (diag(e^{G_last - G}) Kw)^T Up
//
// with Kn the unit read keys and Kw the write keys (Kw = Kn, or the OSDN
// write keys, OSDN notes sec. 2.2).  W = T diag(beta e^G) Kn is never formed:
// Up is computed as (T diag(beta)) (V - diag(e^G) Kn H0), which needs the
// state only through one C x dk x BV product per chunk.
//
// Kernel pairs: the bf16 forward with symmetric keys runs dp_prep_kernel and
// dp_chain_kernel (dp_fwd16.hpp); the fp32 forward and the bf16 write-key
// forward run these two launches:
//   dp_ut_kernel    one workgroup per chunk (all chunks in parallel): gathers
//                   the chunk's sub-steps straight from the token-major
//                   tensors (the interleave is pure addressing), normalises
//                   keys, clamps beta, builds the log-gate cumsum, forms M on
//                   MFMA and solves T in fp32; writes T diag(beta) and the
//                   per-sub-step scalars (1/|k|, G) to the workspace.
//   dp_scan_kernel  one workgroup per (head, block of BV value columns),
//                   sequential over the chunks: the fp32 dk x BV state lives
//                   in MFMA accumulators; per chunk it computes Up, the
//                   readout rows and the state update on MFMA; at the end it
//                   writes the final state.
//   (dp_scan16_kernel is the bf16 form of the scan, for the write-key path.)
// dp_precond_kernel is the OSDN phase-1 scan, dp_decode_kernel (dp_decode.hpp)
// the one-token decode step, dp_varlen_chunks_kernel the first chunk of every
// packed sequence.
//
// Precision: on the bf16 path the inputs are bf16, every accumulation and the
// carried state are fp32, and the MFMA operands that are computed (T diag(beta),
// the state copy, X, Up, the masked scores, the normalised keys) are fp16 -- the
// same MFMA rate as bf16 with 3 more mantissa bits.  The fp32 path uses fp32
// MFMA throughout.
#pragma once

#include <float.h>

#include <type_traits>

#include "dp_device.hpp"

namespace dp {

constexpr int kThreads = 256;  // 4 wavefronts

// MFMA operand type for computed operands: fp16 on the bf16 path, fp32 on the fp32 path.
template <typename T>
struct OpType {
  using type = T;
};
template <>
struct OpType<bf16_t> {
  using type = f16_t;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* kt;  // write keys (asymmetric) or nullptr
  const void* v;
  const float* beta;
  const float* g;   // nullptr: no gate
  const float* h0;  // nullptr: zero initial state
  void* out;
  float* fstate;    // nullptr: final state not returned
  void* wsT;        // [B*H*nc][C][C]: T diag(beta), operand type (fp16 / fp32)
  float2* wsS;      // [B*H*nc][C]: (1/|k|, G)
  float* sink;      // one slot per scan lane for outputs of rows that are not read out
  int N;            // L * n_h sub-steps per head
  int B, H, L, n_h, dv, nc, RT, nvb, asym;
  int out_f32;      // 1: out is fp32 whatever the input type
  // Packed variable-length sequences (bf16 symmetric path): sequence d is
  // tokens cu[d] .. cu[d+1]-1 of a [T, H, ...] batch, with its own state; B is
  // then the number of sequences and cbase[d] the first chunk of sequence d
  // (workspace, filled on the device).  cu == nullptr: B sequences of L tokens.
  const int* cu;
  int* cbase;
  int nwork;        // prep work items (varlen: an upper bound; extra items exit)
  uint32_t nh_magic;  // s / n_h == fastdiv(s, nh_magic, nh_shift) for 0 <= s < 2^31
  int nh_shift;
  // A call on tokens t0 .. t0 + L - 1 of sequences Ls tokens long (the UT and
  // scan kernels of the fixed-length paths): token t of batch row b is row
  // (b Ls + t0 + t) of the token-major tensors.  Ls = 0: Ls = L, t0 = 0.
  int Ls = 0, t0 = 0;
  // bf16 with symmetric keys: 1 runs the single fused kernel (dp_fused.hpp),
  // 0 the chunk-prep kernel then the chain kernel with operand blocks in HBM
  int fused = 0;
  // per-key-channel gate alpha [B, L, H, dk] (the KDA host) or nullptr; with it
  // the UT kernel also writes each chunk's readout scores to wsP (RT x C)
  const float* ga = nullptr;
  void* wsP = nullptr;
  // per-channel gate: operands the UT kernel writes for the scan, in the
  // input layouts and type: read keys e^G o kn and write keys e^{G_C - G} o w
  // ([B, L, H, n_h, dk]), readout queries e^{G_loc} o q ([B, L, H, dk]), and
  // the chunk's state decay e^{G_C} ([B*H*nc][dk] fp32)
  void* wsKg = nullptr;
  void* wsKtg = nullptr;
  void* wsQg = nullptr;
  float* wsDec = nullptr;
  // dp_scan_kernel LDS byte offsets (oDec: the per-channel state decay, dk floats)
  int oK, oKt, oQ, oT, oHt, oXt, oUo, oUs, oP, oV, oG, oEG, oEL, oLoc, oRow, oTok, oDec;
};

// First token row of batch row b (see FwdArgs::Ls).
template <typename A>
__host__ __device__ __forceinline__ long long tok_base(const A& p, int b) {
  return (long long)b * (p.Ls > 0 ? p.Ls : p.L) + p.t0;
}

struct PrecondArgs {
  const void* k;
  const float* beta;
  const float* ret;  // [B, L, H] retention of d (APF), or nullptr
  float* d;
  void* kt;
  int B, H, L;
  int beta_aware;    // 0: the beta-free phase-1 step
  float eta, dmin, dmax, eps;
  int Ls = 0, t0 = 0;  // a call on tokens t0 .. t0 + L - 1 of Ls-token sequences (0: Ls = L)
  float* dtr = nullptr;  // [B, L, H, dk] fp32: d_t of every token (before its update), or nullptr
  int d_ones = 0;        // 1: the scan starts from d = 1 (p.d is then written only)
  // the chunked form (dp_precond_chunk.hpp), per 64-token chunk of each head
  float* wsTm = nullptr;    // [B*H*nc][64][64] (I + L diag(c2))^-1
  float* wsV = nullptr;     // [B*H*nc][64] its product with L w
  float4* wsFac = nullptr;  // [B*H*nc][64] (1/max(|k|, 1e-6), w, c2, G) per token
  float* wsGT = nullptr;    // [B*H*nc] the chunk's total log-retention
  float* dstart = nullptr;  // [B*H*nc][dk] d at each chunk start
  float* gam = nullptr;     // [B*H*nc][64] w - c2 a per token
  // [B*H] first chunk whose check failed (nc: none): with it, dp_precond_kernel
  // runs the exact scan from that chunk's start d and leaves other heads alone
  int* restart = nullptr;
  // packed sequences: B of them along one axis of L tokens, sequence b being
  // tokens cu[b] .. cu[b+1]-1 (device memory), or nullptr; with the chunked
  // form also cbase[B+1], the first 64-token chunk of every sequence
  const int* cu = nullptr;
  int* cbase = nullptr;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// Geometry of sequence d of head h: token offset of its first token, sub-steps,
// chunks and the index of its first operand block (blocks are sequence-major,
// then head, then chunk).
struct SeqGeom {
  long long tok;
  int N, nc;
  long long blk0;
};
__device__ __forceinline__ SeqGeom seq_geom(const FwdArgs& p, int d, int h, int C) {
  SeqGeom g;
  if (p.cu == nullptr) {
    g.tok = tok_base(p, d);  // a token run (FwdArgs::Ls, t0) starts t0 tokens into its sequence
    g.N = p.N;
    g.nc = p.nc;
    g.blk0 = ((long long)d * p.H + h) * p.nc;
  } else {
    // the chunk count comes from cbase, which is all zero for malformed offsets:
    // such a sequence then has no chunk and nothing of it is read
    g.nc = p.cbase[d + 1] - p.cbase[d];
    g.tok = g.nc > 0 ? p.cu[d] : 0;
    g.N = g.nc > 0 ? (p.cu[d + 1] - p.cu[d]) * p.n_h : 0;
    g.blk0 = (long long)p.cbase[d] * p.H + (long long)h * g.nc;
  }
  return g;
}

// Work item `chunk` of a per-chunk kernel -> head bh (sequence-major) and its
// chunk c.  Packed sequences: sequence d owns items cbase[d] H .. cbase[d+1] H
// - 1, head-major inside; false past the last one (the grid is an upper bound).
__device__ __forceinline__ bool chunk_item(const FwdArgs& p, long long chunk, int& bh, int& c) {
  if (p.cu == nullptr) {
    bh = (int)(chunk / p.nc);
    c = (int)(chunk % p.nc);
    return true;
  }
  if (chunk >= (long long)p.cbase[p.B] * p.H) return false;
  int lo = 0, hi = p.B - 1;  // the last sequence whose first item is <= chunk: it has chunks
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)p.cbase[mid] * p.H <= chunk) lo = mid; else hi = mid - 1;
  }
  const int ncd = p.cbase[lo + 1] - p.cbase[lo];
  const int rel = (int)(chunk - (long long)p.cbase[lo] * p.H);
  bh = lo * p.H + rel / ncd;
  c = rel % ncd;
  return true;
}

// Row of sub-step s of a head whose token 0 is token `tok` in a [.., H, n_h, *]
// token-major tensor: ((tok + t) H + h) n_h + j with t = s / n_h, j = s % n_h.
__device__ __forceinline__ long long sub_row_at(const FwdArgs& p, long long tok, int s, int h) {
  const int t = fastdiv(s, p.nh_magic, p.nh_shift);
  return ((tok + t) * p.H + h) * p.n_h + (s - t * p.n_h);
}

// Row of sub-step s of head (b, h) in a [B, L, H, n_h, *] tensor:
// ((b L + t) H + h) n_h + j with t = s / n_h, j = s % n_h.
__device__ __forceinline__ long long sub_row(const FwdArgs& p, int s, int b, int h) {
  const int t = fastdiv(s, p.nh_magic, p.nh_shift);
  const int j = s - t * p.n_h;
  return ((tok_base(p, b) + t) * p.H + h) * p.n_h + j;
}

// LDS bytes of dp_ut_kernel: K (and Kw) rows, fp32 M, 3 scalar vectors,
// fp32 T and the per-wave partial-sum tiles of the blocked inverse; with a
// per-channel gate (cg) both key regions and the cumulative log-gates G
// (C x (dk + 4) fp32).  With 16-bit inputs the rebased fp16 operand rows of
// M's off-diagonal tiles (C x (dk + 8)) use the space of T and the inverse's
// scratch, which are not needed until M is complete.
__host__ __device__ constexpr int ut_gam_ld(int DK) { return DK + 4; }
__host__ __device__ constexpr int ut_cg_op_ld(int DK) { return DK + 8; }
__host__ __device__ constexpr int ut_lds_bytes(int elem, int DK, int C, int asym, int cg = 0) {
  return align16((asym || cg ? 2 : 1) * C * (DK + 16 / elem) * elem) + align16(C * (C + 4) * 4) +
         3 * C * 4 + C * (C + 4) * 4 + 4 * 16 * 17 * 4 + (cg ? C * ut_gam_ld(DK) * 4 : 0);
}

// ---------------------------------------------------------------------------
// dp_ut_kernel: per-chunk prep + UT transform.
// WT is the workspace type of T's output and TB selects T diag(beta) (the
// forward's operand) or T itself (the backward, which also needs T alone).
//
// CG: a per-key-channel gate alpha (the KDA host of the OSDN notes, sec. 2.7:
// H <- Diag(alpha_t) H before a token's sub-steps).  With G_s the chunk-local
// cumulative log-gate of each key channel (the scalar gate folded in), a chunk
// is the ungated write-key form for the read keys e^{G_s} o kn_s and the write
// keys e^{-G_s} o w_s, so that
//   M_ij = beta_i sum_c kn_i[c] w_j[c] e^{G_i[c] - G_j[c]}          (j < i)
//   P_rj = sum_c q_r[c] w_j[c] e^{G_loc(r)[c] - G_j[c]}             (j <= loc(r))
// Every factor is e^{G_a - G_b} with a >= b, at most 1: each entry is summed
// pair by pair with its own factors, so no scaling can overflow however fast a
// channel decays.  The scores go to wsP for the scan, and with them the
// operands the scan then uses as they are (each factor again at most 1): the
// read keys e^{G_s} o kn_s (wsKg), the write keys e^{G_C - G_s} o w_s
// (wsKtg), the readout queries e^{G_loc} o q (wsQg) and e^{G_C} (wsDec).
template <typename T, int DK, int C, typename WT = typename OpType<T>::type, bool TB = true, bool CG = false>
__global__ __launch_bounds__(kThreads) void dp_ut_kernel(FwdArgs p) {
  using OT = WT;
  constexpr int VE = Vec<T>::N;
  constexpr int LDK = DK + VE;  // 16-byte row pad
  constexpr int LDA = C + 4;
  constexpr int NT = C / 16;
  constexpr int TPR = DK / VE;  // threads per key row (<= 32)
  constexpr int KV = C * TPR;   // 16-byte vectors in a key tile
  constexpr int KIT = (KV + kThreads - 1) / kThreads;
  static_assert(TPR <= 64 && (64 % TPR) == 0, "row group must fit in a wavefront");

  extern __shared__ __align__(16) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem);
  T* sKt = sK + C * LDK;
  const T* sKw = p.asym ? sKt : sK;
  float* sA = reinterpret_cast<float*>(smem + align16((p.asym || CG ? 2 : 1) * C * LDK * (int)sizeof(T)));
  float* sR = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(sA) + align16(C * LDA * 4));
  float* sB = sR + C;
  float* sG = sB + C;
  float* sTf = sG + C;         // C x LDA fp32: T
  float* sSc = sTf + C * LDA;  // 4 x 16 x 17 fp32: per-wave partial sums
  float* sGam = sSc + 4 * 16 * 17;  // CG: C x ut_gam_ld(DK) fp32, cumulative log-gates
  constexpr int LDG = ut_gam_ld(DK);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long chunk = blockIdx.x;
  int bh, c;
  if (!chunk_item(p, chunk, bh, c)) return;
  const int b = bh / p.H, h = bh % p.H;
  const SeqGeom sg = seq_geom(p, b, h, C);  // packed: this sequence's tokens and sub-steps
  const int N = sg.N;
  const int s0 = c * C;
  const T* kp = static_cast<const T*>(p.k);
  const T* ktp = static_cast<const T*>(p.kt);

  // 1. issue every global load of the chunk first: key rows, beta, gate
  u32x4_t rk[KIT], rkt[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * kThreads;
    const int r = idx / TPR, cg = idx % TPR;
    const int s = s0 + r;
    rk[it] = u32x4_t{0u, 0u, 0u, 0u};
    rkt[it] = u32x4_t{0u, 0u, 0u, 0u};
    if (idx < KV && s < N) {
      const long long off = sub_row_at(p, sg.tok, s, h) * DK + cg * VE;
      rk[it] = ld16(kp + off);
      if (p.asym) rkt[it] = ld16(ktp + off);
    }
  }
  float braw = 0.f, lam = 0.f;
  bool first = false;
  if (tid < C && s0 + tid < N) {
    const int s = s0 + tid;
    const int t = fastdiv(s, p.nh_magic, p.nh_shift);
    const int j = s - t * p.n_h;
    const long long tok = (sg.tok + t) * p.H + h;
    braw = p.beta[tok * p.n_h + j];
    first = (j == 0);
    if (p.g != nullptr && first) lam = logf(fmaxf(p.g[tok], FLT_MIN));
  }
  // 2. key tiles to LDS; row norms by a TPR-lane reduction (every lane joins)
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * kThreads;
    const int r = idx / TPR, cg = idx % TPR;
    if (idx < KV) {
      st16(sK + r * LDK + cg * VE, rk[it]);
      if (p.asym) st16(sKt + r * LDK + cg * VE, rkt[it]);
      else if (CG) st16(sKt + r * LDK + cg * VE, rk[it]);  // write keys: the keys (normalised below)
    }
    float f[VE];
    unpack16(rk[it], f, T{});
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) ss = fmaf(f[e], f[e], ss);
    if constexpr (TPR <= 16)
      ss = dpp_group_sum<TPR>(ss);  // inside one DPP row
    else
      ss = group_sum<TPR>(ss);
    if (idx < KV && cg == 0) sR[r] = (s0 + r < N) ? 1.f / fmaxf(sqrtf(ss), 1e-6f) : 0.f;
  }
  // 3. beta range and chunk-local cumulative log-gate (C <= 64: wave 0)
  if (wave == 0) {
    const float G = p.g != nullptr ? wave_inclusive_scan(lam) : 0.f;  // no gate: all zero
    if (lane < C) {
      sB[lane] = clamp_keep_nan(braw, 0.f, 2.f);
      sG[lane] = G;
    }
  }
  if constexpr (CG) {
    // log-gate of each (sub-step, key channel) of the chunk, all threads at
    // once: log alpha_t + log g_t at a token's first sub-step, 0 on the others
    // and past the end (the loads are unconditional, at a valid address, so
    // that they are all in flight together)
    const long long tokb = sg.tok * p.H + h;
    constexpr int GIT = C * DK / kThreads;
    static_assert(C * DK % kThreads == 0, "gate tile");
#pragma unroll 8
    for (int it = 0; it < GIT; ++it) {
      const int idx = tid + it * kThreads;
      const int r = idx / DK, ch = idx % DK;
      const int s = s0 + r;
      const int t = fastdiv(min(s, N - 1), p.nh_magic, p.nh_shift);
      const bool first = s < N && s == t * p.n_h;
      const long long tok = tokb + (long long)t * p.H;
      float l = logf(fmaxf(p.ga[tok * DK + ch], FLT_MIN));
      if (p.g != nullptr) l += logf(fmaxf(p.g[tok], FLT_MIN));
      sGam[r * LDG + ch] = first ? l : 0.f;
    }
    block_sync_lds();
    // cumulative over the chunk's sub-steps, one key channel per thread
    if (tid < DK) {
      float acc = 0.f;
#pragma unroll 8
      for (int r = 0; r < C; ++r) {
        acc += sGam[r * LDG + tid];
        sGam[r * LDG + tid] = acc;
      }
    }
  }
  block_sync_lds();
  // (CG: the scan reads pre-normalised keys, so its key scale is 1 on rows in range)
  if (tid < C) p.wsS[chunk * C + tid] = CG ? make_float2(s0 + tid < N ? 1.f : 0.f, 0.f) : make_float2(sR[tid], sG[tid]);

  if constexpr (CG) {
    // 4'. M_ij (j < i); symmetric keys are normalised here (sR), write keys
    //     used as given.  With fp32 inputs, and on the diagonal 16 x 16 tiles,
    //     pair by pair over the key channels.  With 16-bit inputs the tiles
    //     below the diagonal run on MFMA: for block row a (rows i >= r = 16 a)
    //     and columns j < r, e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j} with
    //     both factors at most 1, so the rebased rows kn_i o e^{G_i - G_r} and
    //     w_j o e^{G_r - G_j} are fp16 operands of one product.
    constexpr bool MM = sizeof(OT) == 2;
    constexpr int NPAIR = C * (C - 1) / 2, DPAIR = 16 * 15 / 2;
    for (int pr = tid; pr < C * C; pr += kThreads) sA[(pr / C) * LDA + pr % C] = 0.f;
    block_sync_lds();
    auto pair_sum = [&](int i, int j) {
      float acc = 0.f;
#pragma unroll 4
      for (int c = 0; c < DK; ++c)
        acc = fmaf(to_f32(sK[i * LDK + c]) * to_f32(sKt[j * LDK + c]), __expf(sGam[i * LDG + c] - sGam[j * LDG + c]),
                   acc);
      sA[i * LDA + j] = sB[i] * sR[i] * (p.asym ? 1.f : sR[j]) * acc;
    };
    auto tri = [](int q) {  // q -> (i, j), j < i, in row-major order of the strict lower triangle
      int i = (int)((1.f + sqrtf(1.f + 8.f * (float)q)) * 0.5f);
      while (i * (i - 1) / 2 > q) --i;
      while ((i + 1) * i / 2 <= q) ++i;
      return make_int2(i, q - i * (i - 1) / 2);
    };
    if constexpr (!MM) {
      for (int pr = tid; pr < NPAIR; pr += kThreads) {
        const int2 ij = tri(pr);
        pair_sum(ij.x, ij.y);
      }
    } else {
      for (int pr = tid; pr < NT * DPAIR; pr += kThreads) {
        const int2 ij = tri(pr % DPAIR);
        const int base = 16 * (pr / DPAIR);
        pair_sum(base + ij.x, base + ij.y);
      }
      constexpr int LDO = ut_cg_op_ld(DK);
      static_assert(C * LDO * (int)sizeof(OT) <= (C * LDA + 4 * 16 * 17) * 4, "operand rows fit T's space");
      OT* sOa = reinterpret_cast<OT*>(sTf);  // 16 rebased key rows, then up to C - 16 write rows
      OT* sOb = sOa + 16 * LDO;
      for (int a = 1; a < NT; ++a) {
        const int r = 16 * a;
        for (int idx = tid; idx < (16 + r) * DK; idx += kThreads) {
          const int row = idx / DK, ch = idx % DK;
          if (row < 16) {
            const int i = r + row;
            sOa[row * LDO + ch] =
                from_f32<OT>(to_f32(sK[i * LDK + ch]) * sR[i] * __expf(sGam[i * LDG + ch] - sGam[r * LDG + ch]));
          } else {
            const int j = row - 16;
            const float wj = to_f32(sKt[j * LDK + ch]) * (p.asym ? 1.f : sR[j]);
            sOb[j * LDO + ch] = from_f32<OT>(wj * __expf(sGam[r * LDG + ch] - sGam[j * LDG + ch]));
          }
        }
        block_sync_lds();
        if (wave < a) {  // tile (a, wave)
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
          acc = mm_tile<OT, DK>(acc, sOa, LDO, 0, sOb, LDO, wave * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = r + 4 * (lane >> 4) + e;
            sA[i * LDA + wave * 16 + (lane & 15)] = sB[i] * acc[e];
          }
        }
        block_sync_lds();  // the operand rows are rebased again for the next block row
      }
    }
    // the scan's key operands: e^{G_s} o kn_s and e^{G_C - G_s} o w_s, rows in range
    {
      OT* kg = static_cast<OT*>(p.wsKg);  // in the operand type, as the scan's LDS tiles
      OT* ktg = static_cast<OT*>(p.wsKtg);
      const float* gC = sGam + (C - 1) * LDG;
      for (int idx = tid; idx < KV; idx += kThreads) {
        const int r = idx / TPR, cg = idx % TPR;
        const int s = s0 + r;
        if (s < N) {
          const float* gr = sGam + r * LDG + cg * VE;
          const float rr = sR[r], rw = p.asym ? 1.f : sR[r];
          float fk[VE], fw[VE];
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            fk[e] = to_f32(sK[r * LDK + cg * VE + e]) * rr * __expf(gr[e]);
            fw[e] = to_f32(sKt[r * LDK + cg * VE + e]) * rw * __expf(gC[cg * VE + e] - gr[e]);
          }
          const long long off = sub_row_at(p, sg.tok, s, h) * DK + cg * VE;
          st_vec16(kg + off, fk);
          st_vec16(ktg + off, fw);
        }
      }
      if (tid < DK) p.wsDec[chunk * DK + tid] = __expf(gC[tid]);
    }
    block_sync_lds();
    // 4''. readout scores P_rj (j <= loc(r)) to wsP; the query rows take the
    //      key rows' place (the keys are done)
    const int n_h = p.n_h;
    const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));
    const int RT = p.RT;
    const T* qp = static_cast<const T*>(p.q);
    for (int idx = tid; idx < RT * TPR; idx += kThreads) {
      const int r = idx / TPR, cg = idx % TPR;
      const int s = r0 + r * n_h;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (s < s0 + C && s < N) {
        const long long tok = (sg.tok + fastdiv(s, p.nh_magic, p.nh_shift)) * p.H + h;
        v = ld16(qp + tok * DK + cg * VE);
        // the scan's readout query: e^{G_loc} o q
        float fq[VE];
        unpack16(v, fq, T{});
        const float* gl = sGam + (s - s0) * LDG + cg * VE;
#pragma unroll
        for (int e = 0; e < VE; ++e) fq[e] *= __expf(gl[e]);
        st_vec16(static_cast<OT*>(p.wsQg) + tok * DK + cg * VE, fq);
      }
      st16(sK + r * LDK + cg * VE, v);
    }
    block_sync_lds();
    OT* wp = static_cast<OT*>(p.wsP) + chunk * RT * C;
    for (int e = tid; e < RT * C; e += kThreads) {
      const int r = e / C, j = e % C;
      const int s = r0 + r * n_h;
      const int loc = (s < s0 + C && s < N) ? s - s0 : -1;
      float acc = 0.f;
      if (j <= loc) {
        const float rw = p.asym ? 1.f : sR[j];
#pragma unroll 4
        for (int c = 0; c < DK; ++c)
          acc = fmaf(to_f32(sK[r * LDK + c]) * to_f32(sKt[j * LDK + c]),
                     __expf(sGam[loc * LDG + c] - sGam[j * LDG + c]), acc);
        acc *= rw;
      }
      wp[e] = from_f32<OT>(acc);
    }
  } else {
  // 4. M = strict_tril(diag(beta) (E o Kn Kw^T)) on MFMA (lower tiles only)
  for (int tile = wave; tile < NT * NT; tile += 4) {
    const int ti = tile / NT, tj = tile % NT;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) acc = mm_tile<T, DK>(acc, sK, LDK, ti * 16, sKw, LDK, tj * 16);
    const int jj = tj * 16 + (lane & 15);
    const float rw = p.asym ? 1.f : sR[jj];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ii = ti * 16 + 4 * (lane >> 4) + e;
      float val = 0.f;
      if (jj < ii) val = sB[ii] * sR[ii] * rw * expf(sG[ii] - sG[jj]) * acc[e];
      sA[ii * LDA + jj] = val;
    }
  }
  }
  block_sync_lds();

  // 5. T = (I + M)^{-1} (fp32), blocked over 16 x 16 tiles:
  //    diagonal tiles D_b = (I + M_bb)^{-1} by forward substitution (one
  //    16-lane group per tile, one column per lane), then the off-diagonal
  //    tiles level by level (i - j = 1, 2, ..):
  //    T_ij = -D_i sum_{k=j}^{i-1} M_ik T_kj  on fp32 MFMA.
  if (wave == 0) {
    const int gb = lane >> 4, cc = lane & 15;
    if (gb < NT) {
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == cc) ? 1.f : 0.f;
        const float* ar = sA + (gb * 16 + i) * LDA + gb * 16;
#pragma unroll
        for (int j = 0; j < i; ++j) acc = fmaf(-ar[j], t[j], acc);
        t[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTf[(gb * 16 + i) * LDA + gb * 16 + cc] = t[i];
    }
  }
  block_sync_lds();
#pragma unroll
  for (int dist = 1; dist < NT; ++dist) {
    const int j = wave, i = wave + dist;  // NT - dist <= 3 tiles per level
    float* sS = sSc + wave * 16 * 17;
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb)
        acc = mm_tile_tb<float, 16>(acc, sA + i * 16 * LDA + kb * 16, LDA, 0,
                                    sTf + kb * 16 * LDA + j * 16, LDA, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sS[(4 * (lane >> 4) + e) * 17 + (lane & 15)] = acc[e];
    }
    block_sync_lds();
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<float, 16>(acc, sTf + i * 16 * LDA + i * 16, LDA, 0, sS, 17, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sTf[(i * 16 + 4 * (lane >> 4) + e) * LDA + j * 16 + (lane & 15)] = -acc[e];
    }
    block_sync_lds();
  }
  // 6. T diag(beta) (or T) -> workspace in the operand type, 8 columns per store
  //    (upper tiles are zero)
  {
    OT* wt = static_cast<OT*>(p.wsT) + chunk * C * C;
    constexpr int NV8 = C * C / 8;
    for (int v8 = tid; v8 < NV8; v8 += kThreads) {
      const int i = v8 / (C / 8), j0 = (v8 % (C / 8)) * 8;
      // unconditional reads (T is a full C x LDA matrix in LDS) and a select:
      // the compiler then fetches the eight values in 16-byte reads with one
      // wait, where a guarded read waits once per element
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const float tv = sTf[i * LDA + j] * (TB ? sB[j] : 1.f);
        f[e] = ((j >> 4) > (i >> 4)) ? 0.f : tv;
      }
      if constexpr (sizeof(OT) == 2) {
        st_vec16(wt + i * C + j0, f);
      } else {
        st_vec16(wt + i * C + j0, f);
        st_vec16(wt + i * C + j0 + 4, f + 4);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dp_scan_kernel: sequential chunk scan for one (head, value block).
//
// Software pipeline: the global loads of chunk c+1 (key rows, T diag(beta),
// gates, readout queries, values) are issued into registers after chunk c's
// tiles are committed to LDS and land while chunk c is computed.  Every load
// is unconditional (rows past the end are clamped to row 0 and zeroed when
// committed), so no wait is forced before the compute.  Row indices of the
// next chunk's sub-steps and readout tokens are computed once per chunk into
// LDS.  All barriers order LDS only.  NRT = readout-row tiles per chunk.
//
// CG (per-key-channel gate, see dp_ut_kernel): the scan runs on the UT
// kernel's gated operands (read keys e^{G_s} o kn_s, write keys
// e^{G_C - G_s} o w_s, readout queries e^{G_loc} o q, passed as k, kt and q
// of a write-key launch) and its scores (wsP), with no scalar-gate factors;
// the state's rows decay by e^{G_C} (wsDec).  Every factor is at most 1.
template <typename T, int DK, int C, int BV, int NRT, bool CG = false>
__global__ __launch_bounds__(kThreads) void dp_scan_kernel(FwdArgs p) {
  using OT = typename OpType<T>::type;  // MFMA operand type
  static_assert(sizeof(OT) == sizeof(T), "operand and input types share a width");
  constexpr int VE = Vec<T>::N;
  constexpr int LDK = DK + VE;  // rows of dk operands + 16 B
  constexpr int LDC = C + VE;   // rows of C operands + 16 B
  constexpr int LDV = BV + 4;   // fp32 value rows
  constexpr int RT = NRT * 16;
  constexpr int NCT = C / 16, NVT = BV / 16, NDT = DK / 16;
  constexpr int NYT = NCT * NVT;  // X and Up tiles
  constexpr int YPW = (NYT + 3) / 4;
  constexpr int NPT = NCT * NRT;  // score tiles
  constexpr int PPW = (NPT + 3) / 4;
  constexpr int NZT = NRT * NVT;  // readout tiles
  constexpr int ZPW = (NZT + 3) / 4;
  constexpr int NHT = NDT * NVT;  // state tiles
  constexpr int HPW = (NHT + 3) / 4;
  constexpr int TPR = DK / VE;   // 16-byte vectors per key / query row
  constexpr int TPRC = C / VE;   // per T row
  constexpr int BVV = BV / VE;   // per value row
  constexpr int KV = C * TPR, KIT = (KV + kThreads - 1) / kThreads;
  constexpr int QV = RT * TPR, QIT = (QV + kThreads - 1) / kThreads;
  constexpr int TV = C * TPRC, TIT = (TV + kThreads - 1) / kThreads;
  constexpr int VV = C * BVV, VIT = (VV + kThreads - 1) / kThreads;

  extern __shared__ __align__(16) unsigned char smem[];
  OT* sK = reinterpret_cast<OT*>(smem + p.oK);    // unit read keys
  OT* sKt = reinterpret_cast<OT*>(smem + p.oKt);  // write keys (asymmetric)
  OT* sQ = reinterpret_cast<OT*>(smem + p.oQ);    // readout queries
  OT* sT = reinterpret_cast<OT*>(smem + p.oT);    // T diag(beta)
  OT* sHt = reinterpret_cast<OT*>(smem + p.oHt);  // H^T (operand copy of the fp32 state)
  OT* sXt = reinterpret_cast<OT*>(smem + p.oXt);  // X^T
  OT* sUo = reinterpret_cast<OT*>(smem + p.oUo);  // Up^T
  OT* sUs = reinterpret_cast<OT*>(smem + p.oUs);  // (diag(e^{G_last - G}) Up)^T
  OT* sP = reinterpret_cast<OT*>(smem + p.oP);    // masked, gated scores
  float* sV = reinterpret_cast<float*>(smem + p.oV);    // values, C x LDV fp32
  float* sG = reinterpret_cast<float*>(smem + p.oG);    // G
  float* sEG = reinterpret_cast<float*>(smem + p.oEG);  // e^G
  float* sEL = reinterpret_cast<float*>(smem + p.oEL);  // e^{G_last - G}
  int* sLoc = reinterpret_cast<int*>(smem + p.oLoc);    // readout row -> sub-step in chunk
  long long* sRow = reinterpret_cast<long long*>(smem + p.oRow);  // [2][C] sub-step rows
  long long* sTok = reinterpret_cast<long long*>(smem + p.oTok);  // [2][RT] readout tokens
  float* sDec = reinterpret_cast<float*>(smem + p.oDec);          // CG: e^{G_C} per key channel
  const OT* sKw = (p.asym || CG) ? sKt : sK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  // XCD-aware mapping: consecutive workgroup ids go round-robin over the 8
  // XCDs, so spread ids so that the value blocks of one head share an XCD
  // (and its L2) for the key / T / query tiles they all read.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int f = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int bh = f / p.nvb, vb = f % p.nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;
  const SeqGeom sg = seq_geom(p, b, h, C);  // packed: this sequence's tokens, sub-steps, chunks
  const int n_h = p.n_h, nc = sg.nc, N = sg.N;
  const T* kp = static_cast<const T*>(p.k);
  const T* ktp = static_cast<const T*>(p.kt);
  const T* vp = static_cast<const T*>(p.v) + v0;
  const T* qp = static_cast<const T*>(p.q);
  const OT* wsT = static_cast<const OT*>(p.wsT) + sg.blk0 * C * C;
  const OT* wsP = static_cast<const OT*>(p.wsP) + sg.blk0 * RT * C;
  const float2* wsS = p.wsS + sg.blk0 * C;
  const long long tok0 = sg.tok * p.H + h;  // token (b, 0, h)

  // row indices of chunk c's sub-steps / readout tokens into buffer c & 1
  auto index_chunk = [&](int c) {
    const int s0 = c * C;
    long long* rows = sRow + (c & 1) * C;
    long long* toks = sTok + (c & 1) * RT;
    if (tid < C) {
      const int s = s0 + tid;
      long long row = 0;
      if (s < N) {
        const int t = fastdiv(s, p.nh_magic, p.nh_shift);
        row = (tok0 + (long long)t * p.H) * n_h + (s - t * n_h);
      }
      rows[tid] = row;
    }
    if (tid < RT) {
      const int r0 = s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h));
      const int s = r0 + tid * n_h;
      toks[tid] = (s < s0 + C && s < N) ? tok0 + (long long)fastdiv(s, p.nh_magic, p.nh_shift) * p.H
                                           : -1;
    }
  };

  // ---- prefetch registers (one chunk)
  constexpr int PV = RT * TPRC, PIT = (PV + kThreads - 1) / kThreads;  // CG scores
  u32x4_t rk[KIT], rkt[KIT], rq[QIT], rt[TIT], rvv[VIT], rp[CG ? PIT : 1];
  float rinv[KIT];
  float rg, rdec = 1.f;

  auto prefetch = [&](int c) {
    const long long* rows = sRow + (c & 1) * C;
    const long long* toks = sTok + (c & 1) * RT;
    const OT* tsrc = wsT + (long long)c * C * C;
    const float2* ssrc = wsS + (long long)c * C;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int idx = (KV % kThreads == 0) ? tid + it * kThreads : min(tid + it * kThreads, KV - 1);
      const int r = idx / TPR, cg = idx % TPR;
      const long long off = rows[r] * DK + cg * VE;
      rk[it] = ld16(kp + off);
      if (p.asym) rkt[it] = ld16(ktp + off);
      rinv[it] = ssrc[r].x;
    }
#pragma unroll
    for (int it = 0; it < TIT; ++it) {
      const int idx = (TV % kThreads == 0) ? tid + it * kThreads : min(tid + it * kThreads, TV - 1);
      rt[it] = ld16(tsrc + idx * VE);
    }
    if constexpr (CG) {
      const OT* psrc = wsP + (long long)c * RT * C;
#pragma unroll
      for (int it = 0; it < PIT; ++it) {
        const int idx = (PV % kThreads == 0) ? tid + it * kThreads : min(tid + it * kThreads, PV - 1);
        rp[it] = ld16(psrc + idx * VE);
      }
    }
    rg = ssrc[min(tid, C - 1)].y;
    if constexpr (CG) rdec = p.wsDec[(sg.blk0 + c) * DK + min(tid, DK - 1)];
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int idx = (QV % kThreads == 0) ? tid + it * kThreads : min(tid + it * kThreads, QV - 1);
      const int i = idx / TPR, cg = idx % TPR;
      const long long tk = toks[i];
      rq[it] = ld16(qp + (tk < 0 ? 0 : tk) * DK + cg * VE);
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = (VV % kThreads == 0) ? tid + it * kThreads : min(tid + it * kThreads, VV - 1);
      const int r = idx / BVV, cv = idx % BVV;
      rvv[it] = ld16(vp + rows[r] * p.dv + cv * VE);
    }
  };

  // ---- registers -> LDS (chunk c); also index chunk c+1
  auto commit = [&](int c) {
    const int s0 = c * C;
    const long long* toks = sTok + (c & 1) * RT;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int idx = tid + it * kThreads;
      const int r = idx / TPR, cg = idx % TPR;
      if (KV % kThreads == 0 || idx < KV) {
        // (CG: the UT kernel's gated operands, stored in the operand type)
        using LT = std::conditional_t<CG, OT, T>;
        float fv[VE];
        unpack16(rk[it], fv, LT{});
#pragma unroll
        for (int e = 0; e < VE; ++e) fv[e] *= rinv[it];  // 1/|k|, 0 past the end
        st_vec16(sK + r * LDK + cg * VE, fv);
        if (CG && !p.asym) st_vec16(sKt + r * LDK + cg * VE, fv);  // write keys: the unit keys
        if (p.asym) {
          unpack16(rkt[it], fv, LT{});
          const float keep = (s0 + r < N) ? 1.f : 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) fv[e] *= keep;
          st_vec16(sKt + r * LDK + cg * VE, fv);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < TIT; ++it) {
      const int idx = tid + it * kThreads;
      const int r = idx / TPRC, cg = idx % TPRC;
      if (TV % kThreads == 0 || idx < TV) st16(sT + r * LDC + cg * VE, rt[it]);
    }
    if constexpr (CG) {
#pragma unroll
      for (int it = 0; it < PIT; ++it) {
        const int idx = tid + it * kThreads;
        const int r = idx / TPRC, cg = idx % TPRC;
        if (PV % kThreads == 0 || idx < PV) st16(sP + r * LDC + cg * VE, rp[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int idx = tid + it * kThreads;
      const int i = idx / TPR, cg = idx % TPR;
      if (QV % kThreads == 0 || idx < QV) {
        float fv[VE];
        unpack16(rq[it], fv, std::conditional_t<CG, OT, T>{});
        const float keep = toks[i] >= 0 ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) fv[e] *= keep;
        st_vec16(sQ + i * LDK + cg * VE, fv);
      }
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + it * kThreads;
      const int r = idx / BVV, cv = idx % BVV;
      if (VV % kThreads == 0 || idx < VV) {
        float fv[VE];
        unpack16(rvv[it], fv, T{});
        const float keep = (s0 + r < N) ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          st4(sV + r * LDV + cv * VE + e, fv[e] * keep, fv[e + 1] * keep, fv[e + 2] * keep,
              fv[e + 3] * keep);
      }
    }
    if (tid < C) {
      sG[tid] = rg;
      sEG[tid] = expf(rg);
    }
    if (CG && tid < DK) sDec[tid] = rdec;
    if (tid < RT) sLoc[tid] = toks[tid] >= 0 ? (s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h)) + tid * n_h) - s0 : -1;
    if (c + 1 < nc) index_chunk(c + 1);
  };

  // state H (dk x BV, fp32) in accumulators: wave owns tiles wave + 4u
  f32x4_t hacc[HPW];
#pragma unroll
  for (int u = 0; u < HPW; ++u) {
    hacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int tile = wave + 4 * u;
    if (tile < NHT) {
      const int dt = tile / NVT, nt = tile % NVT;
      if (p.h0 != nullptr) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hacc[u][e] = p.h0[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + nt * 16 + col];
      }
      st4(sHt + (nt * 16 + col) * LDK + dt * 16 + 4 * grp, hacc[u][0], hacc[u][1], hacc[u][2],
          hacc[u][3]);
    }
  }

  if (nc > 0) {
    index_chunk(0);
    block_sync_lds();
    prefetch(0);
  }
  for (int c = 0; c < nc; ++c) {
    const int s0 = c * C;
    block_sync_lds();  // the previous chunk is done with every tile below
    commit(c);
    block_sync_lds();
    if (c + 1 < nc) prefetch(c + 1);

    // ---- phase 1: X = V - diag(e^G) (Kn H0);  P^T = Kw Q^T (masked, gated);  Z = Q H0
    if (tid < C) sEL[tid] = expf(sG[C - 1] - sG[tid]);
#pragma unroll
    for (int u = 0; u < YPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NYT) {
        const int ct = tile / NVT, nt = tile % NVT;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_tile<OT, DK>(acc, sK, LDK, ct * 16, sHt, LDK, nt * 16);
        const int r0 = ct * 16 + 4 * grp;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sV[(r0 + e) * LDV + nt * 16 + col] - (CG ? 1.f : sEG[r0 + e]) * acc[e];
        st4(sXt + (nt * 16 + col) * LDC + r0, x[0], x[1], x[2], x[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < (CG ? 0 : PPW); ++u) {  // CG: the scores came with the chunk
      const int tile = wave + 4 * u;
      if (tile < NPT) {
        const int jt = tile / NRT, it = tile % NRT;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_tile<OT, DK>(acc, sKw, LDK, jt * 16, sQ, LDK, it * 16);
        const int i = it * 16 + col;
        const int loc = sLoc[i];
        const float gl = loc >= 0 ? sG[loc] : 0.f;
        const int j0 = jt * 16 + 4 * grp;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (j0 + e <= loc) ? acc[e] * expf(gl - sG[j0 + e]) : 0.f;
        st4(sP + i * LDC + j0, pv[0], pv[1], pv[2], pv[3]);
      }
    }
    f32x4_t zacc[ZPW];
#pragma unroll
    for (int u = 0; u < ZPW; ++u) {
      zacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int tile = wave + 4 * u;
      if (tile < NZT) {
        const int it = tile / NVT, nt = tile % NVT;
        zacc[u] = mm_tile<OT, DK>(zacc[u], sQ, LDK, it * 16, sHt, LDK, nt * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int loc = sLoc[it * 16 + 4 * grp + e];
          zacc[u][e] *= (loc >= 0) ? (CG ? 1.f : sEG[loc]) : 0.f;
        }
      }
    }
    block_sync_lds();

    // ---- phase 2: Up = (T diag(beta)) X ; copies for the readout and the update
#pragma unroll
    for (int u = 0; u < YPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NYT) {
        const int ct = tile / NVT, nt = tile % NVT;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = mm_tile<OT, C>(acc, sT, LDC, ct * 16, sXt, LDC, nt * 16);
        const int rowoff = (nt * 16 + col) * LDC + ct * 16 + 4 * grp;
        st4(sUo + rowoff, acc[0], acc[1], acc[2], acc[3]);
        const int j0 = ct * 16 + 4 * grp;
        if constexpr (CG)
          st4(sUs + rowoff, acc[0], acc[1], acc[2], acc[3]);  // the decay is in the write keys
        else
          st4(sUs + rowoff, acc[0] * sEL[j0], acc[1] * sEL[j0 + 1], acc[2] * sEL[j0 + 2],
              acc[3] * sEL[j0 + 3]);
      }
    }
    block_sync_lds();

    // ---- phase 3: O = Z + P Up (written out);  H = e^{G_last} H + Kw^T Us
#pragma unroll
    for (int u = 0; u < ZPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NZT) {
        const int it = tile / NVT, nt = tile % NVT;
        zacc[u] = mm_tile<OT, C>(zacc[u], sP, LDC, it * 16, sUo, LDC, nt * 16);
        const long long* toks = sTok + (c & 1) * RT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const long long tk = toks[it * 16 + 4 * grp + e];
          if (tk >= 0) {
            const long long o = tk * p.dv + v0 + nt * 16 + col;
            if (p.out_f32)
              static_cast<float*>(p.out)[o] = zacc[u][e];
            else
              static_cast<T*>(p.out)[o] = from_f32<T>(zacc[u][e]);
          }
        }
      }
    }
    const float dec = sEG[C - 1];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NHT) {
        const int dt = tile / NVT, nt = tile % NVT;
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[u][e] *= CG ? sDec[dt * 16 + 4 * grp + e] : dec;
        hacc[u] = mm_tile_ta<OT, C>(hacc[u], sKw, LDK, dt * 16, sUs, LDC, nt * 16);
        st4(sHt + (nt * 16 + col) * LDK + dt * 16 + 4 * grp, hacc[u][0], hacc[u][1], hacc[u][2],
            hacc[u][3]);
      }
    }
    (void)s0;
  }

  if (p.fstate != nullptr) {
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NHT) {
        const int dt = tile / NVT, nt = tile % NVT;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.fstate[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + nt * 16 + col] = hacc[u][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dp_scan16_kernel: warp-specialised, register-resident chunk scan of the
// bf16 path.
//
// A workgroup takes one head and 16*NWC value columns with NWC consumer and
// NWP producer wavefronts.
//  * Each consumer owns 16 value columns and keeps, in accumulator registers,
//    its slice of the fp32 state H (dk x 16) and, per chunk, X, Up and the
//    readout tiles.  Those are the B operands of all of its products (fp16,
//    see mm_ar / mm_atr), so the chain  H -> X = V - e^G Kn H ->
//    Up = (T diag(beta)) X -> H' = e^{G_last} H + Kw^T (e^{G_last - G} Up)
//    has no LDS traffic of its own.
//  * Producers load chunk c+1 from HBM, normalise the keys, convert keys,
//    queries and values to fp16, commit them with T diag(beta) and the gate
//    scales to the other LDS buffer and compute the chunk's masked scores
//    P = (Q Kw^T) o E, while the consumers work on chunk c.  Keys are
//    normalised before they become fp16 operands (scaling an fp16 operand
//    by 1/|k| instead could overflow for tiny keys).
//  * Consumers read their value columns with one transposed LDS read per
//    16 rows, which lands them directly in accumulator layout.
// Two LDS buffers, two barriers per chunk:
//   X(c) | producers: commit(c+1)     | consumers: X, Up, Q H   of chunk c
//   Y(c) | producers: scores(c+1)     | consumers: P Up, state  of chunk c
// LDS layout of one buffer (byte offsets).
struct Scan16Layout {
  int K, Kt, T, Q, P, V, G, EG, EL, Loc, Tok, buf, total;
};

__host__ __device__ constexpr Scan16Layout scan16_layout(int DK, int C, int BV, int RT, int asym) {
  Scan16Layout L{};
  int off = 0;
  L.K = off;   off += align16(C * (DK + 8) * 2);
  L.Kt = off;  off += asym ? align16(C * (DK + 8) * 2) : 0;
  L.T = off;   off += align16(C * (C + 8) * 2);
  L.Q = off;   off += align16(RT * (DK + 8) * 2);
  L.P = off;   off += align16(RT * (C + 8) * 2);
  L.V = off;   off += align16(C * (BV + 8) * 2);
  L.G = off;   off += align16(C * 4);
  L.EG = off;  off += align16(C * 4);
  L.EL = off;  off += align16(C * 4);
  L.Loc = off; off += align16(RT * 4);
  L.Tok = off; off += align16(RT * 8);
  L.buf = off;
  L.total = 2 * off;
  if (!asym) L.Kt = L.K;
  return L;
}

template <int DK, int C, int NWC, int NWP, int NRT, bool ASYM>
__global__ __launch_bounds__(64 * (NWC + NWP)) void dp_scan16_kernel(FwdArgs p) {
  using T = bf16_t;
  constexpr int NPR = 64 * NWP;  // producer threads
  constexpr int BV = 16 * NWC;
  constexpr int VE = 8;
  constexpr int LDK = DK + 8, LDC = C + 8;
  constexpr int RT = 16 * NRT;
  constexpr int NCT = C / 16, NDT = DK / 16;
  constexpr int LDV = BV + 8;
  constexpr int TPR = DK / VE, TPRC = C / VE, BVV = BV / VE;
  constexpr int KV = C * TPR, KIT = (KV + NPR - 1) / NPR;
  constexpr int QV = RT * TPR, QIT = (QV + NPR - 1) / NPR;
  constexpr int TV = C * TPRC, TIT = (TV + NPR - 1) / NPR;
  constexpr int VV = C * BVV, VIT = (VV + NPR - 1) / NPR;
  constexpr int NPT = NCT * NRT, PPW = (NPT + NWP - 1) / NWP;
  constexpr Scan16Layout Lo = scan16_layout(DK, C, BV, RT, ASYM ? 1 : 0);

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool consumer = wave < NWC;
  const int col = lane & 15, grp = lane >> 4;
  // XCD-aware mapping: consecutive workgroup ids go round-robin over the 8
  // XCDs, so spread ids so that the value blocks of one head share an XCD
  // (and its L2) for the key / T / query tiles they all read.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int f = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int bh = f / p.nvb, vb = f % p.nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;  // first value column of the workgroup
  const int n_h = p.n_h, nc = p.nc;
  const long long tok0 = tok_base(p, b) * p.H + h;  // token (b, 0, h)
  auto first_readout = [&](int s0) { return s0 + (n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * n_h)); };
  auto buffer = [&](int c) { return smem + (c & 1) * Lo.buf; };

  if (!consumer) {
    // =================================================================== producers
    const int ptid = tid - 64 * NWC;
    const int pw = wave - NWC;
    const T* kp = static_cast<const T*>(p.k);
    const T* ktp = static_cast<const T*>(p.kt);
    const T* qp = static_cast<const T*>(p.q);
    const T* vp = static_cast<const T*>(p.v) + v0;
    const f16_t* wsT = static_cast<const f16_t*>(p.wsT) + (long long)bh * nc * C * C;
    const float2* wsS = p.wsS + (long long)bh * nc * C;
    auto row_of = [&](int s) -> long long {  // row of sub-step s (row 0 past the end)
      if (s >= p.N) return 0;
      const int t = fastdiv(s, p.nh_magic, p.nh_shift);
      return (tok0 + (long long)t * p.H) * n_h + (s - t * n_h);
    };

    u32x4_t rk[KIT], rkt[ASYM ? KIT : 1], rq[QIT], rt[TIT], rv[VIT];
    float rinv[KIT];
    float rg = 0.f, rgl = 0.f;
    auto load = [&](int c) {
      const int s0 = c * C;
      const float2* ss = wsS + (long long)c * C;
#pragma unroll
      for (int it = 0; it < KIT; ++it) {
        const int idx = (KV % NPR == 0) ? ptid + it * NPR : min(ptid + it * NPR, KV - 1);
        const int r = idx / TPR, cg = idx % TPR;
        const long long off = row_of(s0 + r) * DK + cg * VE;
        rk[it] = ld16(kp + off);
        if constexpr (ASYM) rkt[it] = ld16(ktp + off);
        rinv[it] = ss[r].x;  // 0 past the end
      }
      const f16_t* tsrc = wsT + (long long)c * C * C;
#pragma unroll
      for (int it = 0; it < TIT; ++it) {
        const int idx = (TV % NPR == 0) ? ptid + it * NPR : min(ptid + it * NPR, TV - 1);
        rt[it] = ld16(tsrc + idx * VE);
      }
      const int r0 = first_readout(s0);
#pragma unroll
      for (int it = 0; it < QIT; ++it) {
        const int idx = (QV % NPR == 0) ? ptid + it * NPR : min(ptid + it * NPR, QV - 1);
        const int i = idx / TPR, cg = idx % TPR;
        const int s = r0 + i * n_h;
        const long long tk =
            (s < s0 + C && s < p.N) ? tok0 + (long long)fastdiv(s, p.nh_magic, p.nh_shift) * p.H : 0;
        rq[it] = ld16(qp + tk * DK + cg * VE);
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int idx = (VV % NPR == 0) ? ptid + it * NPR : min(ptid + it * NPR, VV - 1);
        const int r = idx / BVV, cv = idx % BVV;
        rv[it] = ld16(vp + row_of(s0 + r) * p.dv + cv * VE);
      }
      rg = ss[min(ptid, C - 1)].y;
      rgl = ss[C - 1].y;
    };
    auto commit = [&](int c) {
      unsigned char* B = buffer(c);
      f16_t* sK = reinterpret_cast<f16_t*>(B + Lo.K);
      f16_t* sKt = reinterpret_cast<f16_t*>(B + Lo.Kt);
      f16_t* sT = reinterpret_cast<f16_t*>(B + Lo.T);
      f16_t* sQ = reinterpret_cast<f16_t*>(B + Lo.Q);
      f16_t* sV = reinterpret_cast<f16_t*>(B + Lo.V);
      float* sG = reinterpret_cast<float*>(B + Lo.G);
      float* sEG = reinterpret_cast<float*>(B + Lo.EG);
      float* sEL = reinterpret_cast<float*>(B + Lo.EL);
      int* sLoc = reinterpret_cast<int*>(B + Lo.Loc);
      long long* sTok = reinterpret_cast<long long*>(B + Lo.Tok);
      const int s0 = c * C;
      const int r0 = first_readout(s0);
#pragma unroll
      for (int it = 0; it < KIT; ++it) {
        const int idx = ptid + it * NPR;
        const int r = idx / TPR, cg = idx % TPR;
        if (KV % NPR == 0 || idx < KV) {
          // rows past the end hold row 0 of the tensor and 1/|k| = 0; their
          // beta is 0 too, so their pseudo-values vanish and scores mask them
          float fv[VE];
          unpack16(rk[it], fv, T{});
#pragma unroll
          for (int e = 0; e < VE; ++e) fv[e] *= rinv[it];
          st_vec16(sK + r * LDK + cg * VE, fv);
          if constexpr (ASYM) {
            unpack16(rkt[it], fv, T{});
            st_vec16(sKt + r * LDK + cg * VE, fv);
          }
        }
      }
#pragma unroll
      for (int it = 0; it < TIT; ++it) {
        const int idx = ptid + it * NPR;
        const int r = idx / TPRC, cg = idx % TPRC;
        if (TV % NPR == 0 || idx < TV) st16(sT + r * LDC + cg * VE, rt[it]);
      }
#pragma unroll
      for (int it = 0; it < QIT; ++it) {
        const int idx = ptid + it * NPR;
        const int i = idx / TPR, cg = idx % TPR;
        if (QV % NPR == 0 || idx < QV) {  // rows of missing readouts are masked later
          float fv[VE];
          unpack16(rq[it], fv, T{});
          st_vec16(sQ + i * LDK + cg * VE, fv);
        }
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int idx = ptid + it * NPR;
        const int r = idx / BVV, cv = idx % BVV;
        if (VV % NPR == 0 || idx < VV) {
          const float keep = (s0 + r < p.N) ? 1.f : 0.f;
          float fv[VE];
          unpack16(rv[it], fv, T{});
#pragma unroll
          for (int e = 0; e < VE; ++e) fv[e] *= keep;
          st_vec16(sV + r * LDV + cv * VE, fv);
        }
      }
      if (ptid < C) {
        sG[ptid] = rg;
        sEG[ptid] = expf(rg);
        sEL[ptid] = expf(rgl - rg);
      }
      if (ptid < RT) {
        const int s = r0 + ptid * n_h;
        const bool ok = s < s0 + C && s < p.N;
        sLoc[ptid] = ok ? s - s0 : -1;
        sTok[ptid] = ok ? tok0 + (long long)fastdiv(s, p.nh_magic, p.nh_shift) * p.H : -1;
      }
    };
    // masked, gated scores P^T[j][i] = (Kw_j . q_i) e^{G_loc(i) - G_j} for j <= loc(i)
    auto scores = [&](int c) {
      unsigned char* B = buffer(c);
      const f16_t* sKw = reinterpret_cast<const f16_t*>(B + Lo.Kt);
      const f16_t* sQ = reinterpret_cast<const f16_t*>(B + Lo.Q);
      f16_t* sP = reinterpret_cast<f16_t*>(B + Lo.P);
      const float* sG = reinterpret_cast<const float*>(B + Lo.G);
      const int* sLoc = reinterpret_cast<const int*>(B + Lo.Loc);
#pragma unroll
      for (int u = 0; u < PPW; ++u) {
        const int tile = pw + NWP * u;
        if (tile < NPT) {
          const int jt = tile / NRT, it = tile % NRT;
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
          acc = mm_ll<DK>(acc, sKw, LDK, jt * 16 + col, sQ, LDK, it * 16 + col);
          const int i = it * 16 + col;
          const int loc = sLoc[i];
          const float gl = loc >= 0 ? sG[loc] : 0.f;
          const int j0 = jt * 16 + 4 * grp;
          const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(sG + j0);
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = (j0 + e <= loc) ? acc[e] * expf(gl - g4[e]) : 0.f;
          st4(sP + i * LDC + j0, pv[0], pv[1], pv[2], pv[3]);
        }
      }
    };

    // prologue: chunk 0 committed and scored before the consumers start
    if (nc > 0) {
      load(0);
      commit(0);
      if (nc > 1) load(1);
    }
    block_sync_lds();  // P0
    if (nc > 0) scores(0);
    for (int c = 0; c < nc; ++c) {
      block_sync_lds();  // X(c)
      if (c + 1 < nc) {
        commit(c + 1);
        if (c + 2 < nc) load(c + 2);
      }
      block_sync_lds();  // Y(c)
      if (c + 1 < nc) scores(c + 1);
    }
    return;
  }

  // ===================================================================== consumers
  const int vw = 16 * wave;  // this wavefront's columns inside the block
  f32x4_t hacc[NDT];
  f16x4_t hq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    hacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p.h0 != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hacc[dt][e] = p.h0[((long long)bh * DK + dt * 16 + 4 * grp + e) * p.dv + v0 + vw + col];
    }
    hq[dt] = to_h4(hacc[dt]);
  }
  block_sync_lds();  // P0
  for (int c = 0; c < nc; ++c) {
    unsigned char* B = buffer(c);
    const f16_t* sK = reinterpret_cast<const f16_t*>(B + Lo.K);
    const f16_t* sKw = reinterpret_cast<const f16_t*>(B + Lo.Kt);
    const f16_t* sT = reinterpret_cast<const f16_t*>(B + Lo.T);
    const f16_t* sQ = reinterpret_cast<const f16_t*>(B + Lo.Q);
    const f16_t* sP = reinterpret_cast<const f16_t*>(B + Lo.P);
    const f16_t* sV = reinterpret_cast<const f16_t*>(B + Lo.V);
    const float* sEG = reinterpret_cast<const float*>(B + Lo.EG);
    const float* sEL = reinterpret_cast<const float*>(B + Lo.EL);
    const int* sLoc = reinterpret_cast<const int*>(B + Lo.Loc);
    const long long* sTok = reinterpret_cast<const long long*>(B + Lo.Tok);
    block_sync_lds();  // X(c): chunk c's tiles and scores are in LDS

    // ---- X = V - diag(e^G) (Kn H)
    f16x4_t xq[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_ar<DK>(acc, sK, LDK, ct * 16 + col, hq);
      const f32x4_t eg = *reinterpret_cast<const f32x4_t*>(sEG + ct * 16 + 4 * grp);
      const f16x4_t v4 = lds_t16(sV, LDV, vw, ct * 16);  // V[16 ct + 4 grp + e][vw + col]
      f32x4_t x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (float)v4[e] - eg[e] * acc[e];
      xq[ct] = to_h4(x);
    }
    // ---- Up = (T diag(beta)) X; Us = diag(e^{G_last - G}) Up
    f16x4_t uq[NCT], usq[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_ar<C>(acc, sT, LDC, ct * 16 + col, xq);
      const f32x4_t el = *reinterpret_cast<const f32x4_t*>(sEL + ct * 16 + 4 * grp);
      uq[ct] = to_h4(acc);
      usq[ct] = to_h4(acc * el);
    }
    // ---- diag(e^G) Q H for the readout rows
    f32x4_t z[NRT];
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      z[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      z[it] = mm_ar<DK>(z[it], sQ, LDK, it * 16 + col, hq);
      const int4 loc4 = *reinterpret_cast<const int4*>(sLoc + it * 16 + 4 * grp);
      z[it][0] *= loc4.x >= 0 ? sEG[loc4.x] : 0.f;
      z[it][1] *= loc4.y >= 0 ? sEG[loc4.y] : 0.f;
      z[it][2] *= loc4.z >= 0 ? sEG[loc4.z] : 0.f;
      z[it][3] *= loc4.w >= 0 ? sEG[loc4.w] : 0.f;
    }
    block_sync_lds();  // Y(c)

    // ---- O = diag(e^G) Q H + P Up, written out
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      z[it] = mm_ar<C>(z[it], sP, LDC, it * 16 + col, uq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long long tk = sTok[it * 16 + 4 * grp + e];
        if (tk >= 0) {
          const long long o = tk * p.dv + v0 + vw + col;
          if (p.out_f32)
            static_cast<float*>(p.out)[o] = z[it][e];
          else
            static_cast<T*>(p.out)[o] = from_f32<T>(z[it][e]);
        }
      }
    }
    // ---- H = e^{G_last} H + Kw^T Us
    const float dec = sEG[C - 1];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      hacc[dt] = hacc[dt] * dec;
      hacc[dt] = mm_atr<C>(hacc[dt], sKw, LDK, dt * 16, usq);
      hq[dt] = to_h4(hacc[dt]);
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

// ---------------------------------------------------------------------------
// dp_precond_kernel: OSDN phase 1 (OSDN notes sec. 2.3-2.4, Alg.1), with the
// optional APF retention of d (sec. 2.6: d_{t+1} = P[r_t d_t + step]) and the
// beta-free step of the 1.3B configuration (sec. 2.7: beta taken as 1 in the
// phase-1 step only).
// A head's dk coordinates are spread over LPH = min(dk, 64) lanes (dk/LPH
// each), 64/LPH heads per wavefront; each head is a sequential scan over its
// L tokens.  Tokens come in blocks of PF, loaded one block ahead.  The part of
// a token that does not depend on d -- the key norm, the unit key kh,
// s = kh o kh, its sum and the step factor eta beta / max(sum s, eps) -- runs
// LAH tokens ahead of the sequential part, which is <d, s> (one head sum),
// the update of d and the store of the write key d o kh.

// Sum over the LPH lanes of a head (LPH = 16, 32 or 64): within each DPP row
// (lane ^ 1, lane ^ 2, the mirrored quad, the mirrored half), then across row
// pairs and halves by permlane swaps.  Every lane of the head ends with the
// same value.
template <int LPH>
__device__ __forceinline__ float head_sum(float x) {
  static_assert(LPH == 16 || LPH == 32 || LPH == 64, "lanes per head");
  auto dpp_add = [](float v, auto ctrl) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x = dpp_add(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  x = dpp_add(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  x = dpp_add(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  x = dpp_add(x, std::integral_constant<int, 0x140>{});  // row_mirror
  if constexpr (LPH >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LPH == 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// clamp to [lo, hi]; NaN stays NaN
__device__ __forceinline__ float med3_keep_nan(float x, float lo, float hi) {
  return x != x ? x : __builtin_amdgcn_fmed3f(x, lo, hi);
}

template <typename T, int DK>
__global__ __launch_bounds__(64) void dp_precond_kernel(PrecondArgs p) {
  constexpr int LPH = DK < 64 ? DK : 64;  // lanes per head
  constexpr int EPL = DK / LPH;           // coordinates per lane (1 or 2)
  constexpr int HPW = 64 / LPH;           // heads per wavefront
  constexpr int PF = 32;                  // tokens per block
  constexpr int LAH = 3, NSL = LAH + 1;   // look-ahead of the d-independent part
  static_assert(EPL == 1 || EPL == 2, "coordinates per lane");
  const int lane = threadIdx.x & 63;
  const int sl = lane % LPH;
  const long long nbh = (long long)p.B * p.H;
  const long long bh_raw = (long long)blockIdx.x * HPW + lane / LPH;
  const bool active = bh_raw < nbh;
  const long long bh = active ? bh_raw : 0;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  // this head's tokens: L of them from token tb (packed: sequence b's own run;
  // offsets outside 0 = cu[0], cu[b] <= cu[b+1] <= cu[B] = L make it empty)
  int L = p.L;
  long long tb = tok_base(p, b);
  if (p.cu != nullptr) {
    const int lo = p.cu[b], hi = p.cu[b + 1];
    const bool ok = p.cu[0] == 0 && p.cu[p.B] == p.L && 0 <= lo && lo <= hi && hi <= p.L;
    tb = ok ? lo : 0;
    L = ok ? hi - lo : 0;
  }
  // token t of this head: row ((tb + t) H + h) of the token-major tensors
  const long long row0 = tb * p.H + h;
  const T* kp = static_cast<const T*>(p.k) + row0 * DK + sl * EPL;
  T* ktp = static_cast<T*>(p.kt) + row0 * DK + sl * EPL;
  const float* bp = p.beta + row0;
  const float* rp = p.ret != nullptr ? p.ret + row0 : nullptr;
  const long long kstride = (long long)p.H * DK;

  float d[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) d[e] = p.d_ones ? 1.f : p.d[bh * DK + sl * EPL + e];
  // d_t of token t, kept for the backward when asked for
  float* const dtp = p.dtr != nullptr ? p.dtr + row0 * DK + sl * EPL : nullptr;
  auto store_d = [&](int t) {
    if constexpr (EPL == 2)
      *reinterpret_cast<float2*>(dtp + t * kstride) = make_float2(d[0], d[1]);
    else
      dtp[t * kstride] = d[0];
  };

  // write key d o kh (EPL values, stored together) at dst
  auto store_kt_at = [&](T* dst, const float* kh) {
    T o[EPL];
    if constexpr (sizeof(T) == 2 && EPL == 2) {
      const bf16x2_t v = __builtin_convertvector(f32x2_t{d[0] * kh[0], d[1] * kh[1]}, bf16x2_t);
      __builtin_memcpy(o, &v, 4);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = from_f32<T>(d[e] * kh[e]);
    }
    __builtin_memcpy(__builtin_assume_aligned(dst, EPL * sizeof(T)), o, EPL * sizeof(T));
  };
  // write key d o kh of token t (EPL values, stored together)
  auto store_kt = [&](int t, const float* kh) {
    T o[EPL];
    if constexpr (sizeof(T) == 2 && EPL == 2) {
      const bf16x2_t v = __builtin_convertvector(f32x2_t{d[0] * kh[0], d[1] * kh[1]}, bf16x2_t);
      __builtin_memcpy(o, &v, 4);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = from_f32<T>(d[e] * kh[e]);
    }
    __builtin_memcpy(__builtin_assume_aligned(ktp + t * kstride, EPL * sizeof(T)), o, EPL * sizeof(T));
  };

  if constexpr (LPH == 64) {
    // One head per wavefront (the grid has one per head: every lane is active).
    // Lane j also owns token t0 + j of the block: it
    // loads that token's whole key row, beta and retention one block ahead
    // and forms the token's scalars (1/max(|k|, 1e-6), the step factor, the
    // clamped beta); the sequential part reads them with v_readlane.
    if (!active) return;
    constexpr int PB = sizeof(T) == 2 ? 64 : 32;  // tokens per block
    // after the chunked form: start at the head's first failed chunk, or not at all
    int tbeg = 0;
    if (p.restart != nullptr) {
      // the head's chunks: nc of them from blk0 (packed: sequence b's, head-major)
      int nc = (p.L + 63) / 64;
      long long blk0 = bh * nc;
      if (p.cu != nullptr) {
        nc = p.cbase[b + 1] - p.cbase[b];
        blk0 = (long long)p.cbase[b] * p.H + (long long)h * nc;
      }
      const int sc = p.restart[bh];
      if (sc >= nc) return;
      tbeg = sc * 64;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d[e] = p.dstart[(blk0 + sc) * DK + sl * EPL + e];
    }
    constexpr int RB = DK * (int)sizeof(T);       // bytes per key row
    static_assert(RB % 16 == 0, "key rows in 16-byte pieces");
    const T* krow = static_cast<const T*>(p.k) + row0 * DK;
    uint4 rowraw[RB / 16];
    float bnx = 0.f, rnx = 1.f;
    auto load_rows = [&](int t0) {
      const int t = t0 + lane;
      if (lane < PB && t < L) {
        const uint4* src = reinterpret_cast<const uint4*>(krow + t * kstride);
#pragma unroll
        for (int q = 0; q < RB / 16; ++q) rowraw[q] = src[q];
        bnx = bp[(long long)t * p.H];
        rnx = rp != nullptr ? rp[(long long)t * p.H] : 1.f;
      } else {
#pragma unroll
        for (int q = 0; q < RB / 16; ++q) rowraw[q] = uint4{0u, 0u, 0u, 0u};
        bnx = 0.f;
        rnx = 1.f;
      }
    };
    T sc[PB][EPL], sn[PB][EPL];  // this lane's coordinates of every token, current and next block
    auto load_slices = [&](int t0, T (&sv)[PB][EPL]) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (t0 + i < L)
          __builtin_memcpy(sv[i], __builtin_assume_aligned(kp + (t0 + i) * kstride, EPL * sizeof(T)), EPL * sizeof(T));
        else
#pragma unroll
          for (int e = 0; e < EPL; ++e) sv[i][e] = T{};
      }
    };
    float rv, wv, bwv, rtv;  // this lane's token scalars (current block): 1/|k|, w, beta w, r
    auto token_scalars = [&]() {
      const T* kv = reinterpret_cast<const T*>(rowraw);
      float n4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < DK; ++e) n4[e & 3] = fmaf(to_f32(kv[e]), to_f32(kv[e]), n4[e & 3]);
      const float n2 = (n4[0] + n4[1]) + (n4[2] + n4[3]);
      rv = __builtin_amdgcn_rsqf(fmaxf(n2, 1e-12f));  // 1 / max(|k|, 1e-6)
      const float ns = n2 * rv * rv;                  // |kh|^2
      const float bt = p.beta_aware ? clamp_keep_nan(bnx, 0.f, 2.f) : 1.f;
      wv = p.eta * bt * __builtin_amdgcn_rcpf(fmaxf(ns, p.eps));
      bwv = bt * wv;  // coef = w (1 - beta <d, s>) = w - (beta w) <d, s>
      rtv = rnx;
    };
    auto lane_val = [](float x, int i) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i)); };
    // RET: a retention gate is given (else r = 1 and d is not rescaled)
    auto run_block = [&](auto fullc, auto retc, int t0) {
      constexpr bool FULL = decltype(fullc)::value, RET = decltype(retc)::value;
      T* kto = ktp + t0 * kstride;  // write key of token t0 + i at kto + i kstride
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const int t = t0 + i;
        if (FULL || t < L) {
          const float r = lane_val(rv, i), w = lane_val(wv, i), bw = lane_val(bwv, i);
          float kh[EPL], sq[EPL], ds = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            kh[e] = to_f32(sc[i][e]) * r;
            sq[e] = kh[e] * kh[e];
            ds = fmaf(d[e], sq[e], ds);
          }
          ds = head_sum<LPH>(ds);
          store_kt_at(kto, kh);
          kto += kstride;
          if (dtp != nullptr) store_d(t);
          const float coef = fmaf(-bw, ds, w);
          if constexpr (RET) {
            const float rt = lane_val(rtv, i);
#pragma unroll
            for (int e = 0; e < EPL; ++e) d[e] = med3_keep_nan(fmaf(coef, sq[e], rt * d[e]), p.dmin, p.dmax);
          } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) d[e] = med3_keep_nan(fmaf(coef, sq[e], d[e]), p.dmin, p.dmax);
          }
        }
      }
    };
    load_rows(tbeg);
    load_slices(tbeg, sc);
    for (int t0 = tbeg; t0 < L; t0 += PB) {
      token_scalars();
      if (t0 + PB < L) {
        load_rows(t0 + PB);
        load_slices(t0 + PB, sn);
      }
      const bool full = t0 + PB <= L;
      if (rp != nullptr) {
        if (full)
          run_block(std::true_type{}, std::true_type{}, t0);
        else
          run_block(std::false_type{}, std::true_type{}, t0);
      } else {
        if (full)
          run_block(std::true_type{}, std::false_type{}, t0);
        else
          run_block(std::false_type{}, std::false_type{}, t0);
      }
#pragma unroll
      for (int i = 0; i < PB; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) sc[i][e] = sn[i][e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) p.d[bh * DK + sl * EPL + e] = d[e];
    return;
  }

  // raw key slice, beta and retention of the tokens of one block
  struct Raw {
    T k[PF][EPL];
    float beta[PF], ret[PF];
  };
  auto load_block = [&](int t0, Raw& r) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int t = t0 + i;
      if (t < L) {
        __builtin_memcpy(r.k[i], __builtin_assume_aligned(kp + t * kstride, EPL * sizeof(T)), EPL * sizeof(T));
        r.beta[i] = bp[(long long)t * p.H];
        r.ret[i] = rp != nullptr ? rp[(long long)t * p.H] : 1.f;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) r.k[i][e] = T{};
        r.beta[i] = 0.f;
        r.ret[i] = 1.f;
      }
    }
  };
  Raw cur, nxt;
  // FULL: every token of the block is below L (no per-token checks)
  auto run_block = [&](auto fullc, int t0) {
    constexpr bool FULL = decltype(fullc)::value;
    float kh[NSL][EPL], s[NSL][EPL], w[NSL], bt[NSL];
    auto prep_tok = [&](int i) {
      const int q = i % NSL;
      float n2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) n2 = fmaf(to_f32(cur.k[i][e]), to_f32(cur.k[i][e]), n2);
      n2 = head_sum<LPH>(n2);
      const float r = __builtin_amdgcn_rsqf(fmaxf(n2, 1e-12f));  // 1 / max(|k|, 1e-6)
      float ns = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kh[q][e] = to_f32(cur.k[i][e]) * r;
        s[q][e] = kh[q][e] * kh[q][e];
        ns += s[q][e];
      }
      ns = head_sum<LPH>(ns);
      bt[q] = p.beta_aware ? clamp_keep_nan(cur.beta[i], 0.f, 2.f) : 1.f;
      w[q] = p.eta * bt[q] * __builtin_amdgcn_rcpf(fmaxf(ns, p.eps));
    };
#pragma unroll
    for (int i = 0; i < LAH; ++i) prep_tok(i);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (i + LAH < PF) prep_tok(i + LAH);
      const int q = i % NSL;
      const int t = t0 + i;
      if (FULL || t < L) {
        float ds = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ds = fmaf(d[e], s[q][e], ds);
        ds = head_sum<LPH>(ds);
        // emit the write key with the current d_t
        if (active) store_kt(t, kh[q]);
        if (active && dtp != nullptr) store_d(t);
        const float coef = w[q] * (1.f - bt[q] * ds);
        // retention scales d_t (exactly 1 without the gate), the step uses d_t
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[e] = med3_keep_nan(fmaf(coef, s[q][e], cur.ret[i] * d[e]), p.dmin, p.dmax);
      }
    }
  };
  load_block(0, cur);
  for (int t0 = 0; t0 < L; t0 += PF) {
    if (t0 + PF < L) load_block(t0 + PF, nxt);
    if (t0 + PF <= L)
      run_block(std::true_type{}, t0);
    else
      run_block(std::false_type{}, t0);
    cur = nxt;
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) p.d[bh * DK + sl * EPL + e] = d[e];
  }
}

// ---------------------------------------------------------------------------
// dp_varlen_chunks_kernel: first chunk of every packed sequence,
//   cbase[d] = sum over d' < d of ceil((cu[d'+1] - cu[d']) n_h / C),  d = 0 .. nseq,
// in one workgroup (each thread a contiguous run of sequences, then a scan of
// the run totals).  Offsets that are not 0 = cu[0] <= cu[1] <= .. <= cu[nseq]
// = T make every sequence empty (cbase all zero): nothing is then read or
// written beyond the initial state.
template <int C>
__global__ __launch_bounds__(256) void dp_varlen_chunks_kernel(const int* cu, int nseq, int n_h, int T, int* cbase) {
  __shared__ long long run[256];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int per = (nseq + 255) / 256;
  const int lo = tid * per < nseq ? tid * per : nseq;
  const int hi = lo + per < nseq ? lo + per : nseq;
  if (tid == 0) bad = (cu[0] != 0 || cu[nseq] != T) ? 1 : 0;
  __syncthreads();
  long long sum = 0;
  int mybad = 0;
  for (int d = lo; d < hi; ++d) {
    const int len = cu[d + 1] - cu[d];
    if (len < 0) mybad = 1;
    sum += ((long long)(len > 0 ? len : 0) * n_h + C - 1) / C;
  }
  if (mybad) atomicOr(&bad, 1);
  run[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    long long acc = 0;
    for (int i = 0; i < 256; ++i) {
      const long long x = run[i];
      run[i] = acc;
      acc += x;
    }
  }
  __syncthreads();
  long long acc = run[tid];
  const bool ok = bad == 0;
  for (int d = lo; d < hi; ++d) {
    cbase[d] = ok ? (int)acc : 0;
    const int len = cu[d + 1] - cu[d];
    acc += ((long long)(len > 0 ? len : 0) * n_h + C - 1) / C;
  }
  if (tid == 255) cbase[nseq] = ok ? (int)acc : 0;
}

// ---------------------------------------------------------------------------
// Host-side launchers (instantiated per element type and key dimension).

// Raise a kernel's dynamic-LDS limit to the gfx950 maximum (best effort: a
// refusal is cleared here and surfaces, if it matters, as a launch error).
inline bool allow_big_lds(const void* fn) {
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) (void)hipGetLastError();
  return e == hipSuccess;
}

}  // namespace dp

#include "dp_fwd16.hpp"
#include "dp_fused.hpp"
#include "dp_decode.hpp"
#include "dp_precond_chunk.hpp"

namespace dp {

template <typename T, int DK, int C>
hipError_t launch_ut(const FwdArgs& a, hipStream_t st) {
  const int lds = ut_lds_bytes((int)sizeof(T), DK, C, a.asym);
  static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_ut_kernel<T, DK, C>));
  (void)attr;
  long long nchunks = (long long)a.B * a.H * a.nc;
  if (a.cu != nullptr) {  // packed sequences: per-sequence chunk counts first
    hipLaunchKernelGGL((dp_varlen_chunks_kernel<C>), dim3(1), dim3(256), 0, st, a.cu, a.B, a.n_h, a.L, a.cbase);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    nchunks = a.nwork;
  }
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL((dp_ut_kernel<T, DK, C>), dim3((unsigned)nchunks), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <typename T, int DK, int C, int BV, int NRT>
hipError_t launch_scan(const FwdArgs& a, int lds, hipStream_t st) {
  static const bool attr =
      allow_big_lds(reinterpret_cast<const void*>(&dp_scan_kernel<T, DK, C, BV, NRT>));
  (void)attr;
  const long long nwg = (long long)a.B * a.H * a.nvb;
  hipLaunchKernelGGL((dp_scan_kernel<T, DK, C, BV, NRT>), dim3((unsigned)nwg), dim3(kThreads), lds,
                     st, a);
  return hipGetLastError();
}

template <typename T, int DK, int C, int BV>
hipError_t launch_scan_nrt(const FwdArgs& a, int lds, hipStream_t st) {
  switch (a.RT / 16) {
    case 1: return launch_scan<T, DK, C, BV, 1>(a, lds, st);
    case 2: if constexpr (C >= 32) return launch_scan<T, DK, C, BV, 2>(a, lds, st); break;
    case 3: if constexpr (C >= 64) return launch_scan<T, DK, C, BV, 3>(a, lds, st); break;
    case 4: if constexpr (C >= 64) return launch_scan<T, DK, C, BV, 4>(a, lds, st); break;
  }
  return hipErrorInvalidValue;
}

// Per-key-channel gate (either input type): dp_ut_kernel and dp_scan_kernel in
// their CG form, operands in the input's operand type.
template <typename T, int DK, int C>
hipError_t launch_ut_cg(const FwdArgs& a, hipStream_t st) {
  using OT = typename OpType<T>::type;
  const int lds = ut_lds_bytes((int)sizeof(T), DK, C, a.asym, 1);
  static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_ut_kernel<T, DK, C, OT, true, true>));
  (void)attr;
  const long long nchunks = (long long)a.B * a.H * a.nc;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL((dp_ut_kernel<T, DK, C, OT, true, true>), dim3((unsigned)nchunks), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <typename T, int DK, int C, int BV, int NRT>
hipError_t launch_scan_cg(const FwdArgs& a, int lds, hipStream_t st) {
  static const bool attr =
      allow_big_lds(reinterpret_cast<const void*>(&dp_scan_kernel<T, DK, C, BV, NRT, true>));
  (void)attr;
  const long long nwg = (long long)a.B * a.H * a.nvb;
  hipLaunchKernelGGL((dp_scan_kernel<T, DK, C, BV, NRT, true>), dim3((unsigned)nwg), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <typename T, int DK, int C, int BV>
hipError_t launch_scan_cg_nrt(const FwdArgs& a, int lds, hipStream_t st) {
  switch (a.RT / 16) {
    case 1: return launch_scan_cg<T, DK, C, BV, 1>(a, lds, st);
    case 2: if constexpr (C >= 32) return launch_scan_cg<T, DK, C, BV, 2>(a, lds, st); break;
    case 3: if constexpr (C >= 64) return launch_scan_cg<T, DK, C, BV, 3>(a, lds, st); break;
    case 4: if constexpr (C >= 64) return launch_scan_cg<T, DK, C, BV, 4>(a, lds, st); break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK, int C>
hipError_t launch_cg(const FwdArgs& a, int BV, int lds_scan, int stages, hipStream_t st) {
  if ((stages & 1) && a.nc > 0) {
    const hipError_t e = launch_ut_cg<T, DK, C>(a, st);
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    // the scan reads the UT kernel's gated operands as its write-key inputs
    FwdArgs s = a;
    s.k = a.wsKg;
    s.kt = a.wsKtg;
    s.q = a.wsQg;
    s.asym = 1;
    switch (BV) {
      case 16: return launch_scan_cg_nrt<T, DK, C, 16>(s, lds_scan, st);
      case 32: return launch_scan_cg_nrt<T, DK, C, 32>(s, lds_scan, st);
      case 64: return launch_scan_cg_nrt<T, DK, C, 64>(s, lds_scan, st);
      default: return hipErrorInvalidValue;
    }
  }
  return hipSuccess;
}

// Producer wavefronts per workgroup of dp_scan16_kernel for NWC consumers.
constexpr int scan16_producers(int nwc) { return nwc >= 2 ? 2 : 1; }

template <int DK, int C, int NWC, int NRT>
hipError_t launch_scan16(const FwdArgs& a, int lds, hipStream_t st) {
  constexpr int NWP = scan16_producers(NWC);
  const long long nwg = (long long)a.B * a.H * a.nvb;
  if (a.asym) {
    static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_scan16_kernel<DK, C, NWC, NWP, NRT, true>));
    (void)attr;
    hipLaunchKernelGGL((dp_scan16_kernel<DK, C, NWC, NWP, NRT, true>), dim3((unsigned)nwg), dim3(64 * (NWC + NWP)),
                       lds, st, a);
  } else {
    static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_scan16_kernel<DK, C, NWC, NWP, NRT, false>));
    (void)attr;
    hipLaunchKernelGGL((dp_scan16_kernel<DK, C, NWC, NWP, NRT, false>), dim3((unsigned)nwg), dim3(64 * (NWC + NWP)),
                       lds, st, a);
  }
  return hipGetLastError();
}

template <int DK, int C, int NWC>
hipError_t launch_scan16_nrt(const FwdArgs& a, int lds, hipStream_t st) {
  switch (a.RT / 16) {
    case 1: return launch_scan16<DK, C, NWC, 1>(a, lds, st);
    case 2: if constexpr (C >= 32) return launch_scan16<DK, C, NWC, 2>(a, lds, st); break;
    case 3: if constexpr (C >= 64) return launch_scan16<DK, C, NWC, 3>(a, lds, st); break;
    case 4: if constexpr (C >= 64) return launch_scan16<DK, C, NWC, 4>(a, lds, st); break;
  }
  return hipErrorInvalidValue;
}

// Scan launch: the bf16 path uses the register-resident dp_scan16_kernel with
// BV / 16 wavefronts per workgroup; the fp32 path the LDS-staged dp_scan_kernel.
template <typename T, int DK, int C>
hipError_t launch_scan_any(const FwdArgs& a, int BV, int lds, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    switch (BV) {
      case 16: return launch_scan16_nrt<DK, C, 1>(a, lds, st);
      case 32: return launch_scan16_nrt<DK, C, 2>(a, lds, st);
      case 64: return launch_scan16_nrt<DK, C, 4>(a, lds, st);
    }
  } else {
    switch (BV) {
      case 16: return launch_scan_nrt<T, DK, C, 16>(a, lds, st);
      case 32: return launch_scan_nrt<T, DK, C, 32>(a, lds, st);
      case 64: return launch_scan_nrt<T, DK, C, 64>(a, lds, st);
    }
  }
  return hipErrorInvalidValue;
}

// bf16: dp_prep_kernel then dp_chain_kernel (symmetric keys, or write keys
// with dk and chunk multiples of 32).
template <int DK, int C, int NRT, bool ASYM>
hipError_t launch_prep(const FwdArgs& a, hipStream_t st) {
  static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_prep_kernel<DK, C, NRT, ASYM>));
  (void)attr;
  if (a.cu != nullptr) {
    hipLaunchKernelGGL((dp_varlen_chunks_kernel<C>), dim3(1), dim3(256), 0, st, a.cu, a.B, a.n_h, a.L, a.cbase);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nchunks = a.cu != nullptr ? (long long)a.nwork : (long long)a.B * a.H * a.nc;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL((dp_prep_kernel<DK, C, NRT, ASYM>), dim3((unsigned)nchunks), dim3(256),
                     prep_lds_bytes(DK, C, 16 * NRT, ASYM), st, a);
  return hipGetLastError();
}

template <int DK, int C, int NWC, int NRT, bool GATED, bool ASYM>
hipError_t launch_chain_g(const FwdArgs& a, hipStream_t st) {
  static const bool attr =
      allow_big_lds(reinterpret_cast<const void*>(&dp_chain_kernel<DK, C, NWC, NRT, GATED, ASYM>));
  (void)attr;
  const long long nwg = (long long)a.B * a.H * a.nvb;
  hipLaunchKernelGGL((dp_chain_kernel<DK, C, NWC, NRT, GATED, ASYM>), dim3((unsigned)nwg),
                     dim3(64 * (NWC + kChainCopyWaves)), chain_lds_bytes(DK, C, 16 * NRT, 16 * NWC, ASYM), st, a);
  return hipGetLastError();
}

template <int DK, int C, int NWC, int NRT, bool ASYM>
hipError_t launch_chain(const FwdArgs& a, hipStream_t st) {
  return a.g != nullptr ? launch_chain_g<DK, C, NWC, NRT, true, ASYM>(a, st)
                        : launch_chain_g<DK, C, NWC, NRT, false, ASYM>(a, st);
}

template <int DK, int C, int NRT, bool ASYM>
hipError_t launch_pair16_nrt(const FwdArgs& a, int BV, int stages, hipStream_t st) {
  if (!ASYM && a.fused) {
    if (a.cu != nullptr) {  // packed sequences: per-sequence chunk counts first
      hipLaunchKernelGGL((dp_varlen_chunks_kernel<C>), dim3(1), dim3(256), 0, st, a.cu, a.B, a.n_h, a.L, a.cbase);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return launch_fused<DK, C, NRT>(a, BV, st);
  }
  if (stages & 1) {
    const hipError_t e = launch_prep<DK, C, NRT, ASYM>(a, st);
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    switch (BV) {
      case 16: return launch_chain<DK, C, 1, NRT, ASYM>(a, st);
      case 32: return launch_chain<DK, C, 2, NRT, ASYM>(a, st);
      case 64: return launch_chain<DK, C, 4, NRT, ASYM>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  return hipSuccess;
}

template <int DK, int C, bool ASYM>
hipError_t launch_pair16(const FwdArgs& a, int BV, int stages, hipStream_t st) {
  switch (a.RT / 16) {
    case 1: return launch_pair16_nrt<DK, C, 1, ASYM>(a, BV, stages, st);
    case 2: if constexpr (C >= 32) return launch_pair16_nrt<DK, C, 2, ASYM>(a, BV, stages, st); break;
    case 3: if constexpr (C >= 64) return launch_pair16_nrt<DK, C, 3, ASYM>(a, BV, stages, st); break;
    case 4: if constexpr (C >= 64) return launch_pair16_nrt<DK, C, 4, ASYM>(a, BV, stages, st); break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK>
hipError_t launch_fwd_dk(const FwdArgs& a, int C, int BV, int lds_scan, int stages, hipStream_t st) {
  hipError_t e = hipSuccess;
#define DP_CASE_C(CC)                                                          \
  case CC:                                                                     \
    if (a.ga != nullptr) return launch_cg<T, DK, CC>(a, BV, lds_scan, stages, st); \
    if constexpr (sizeof(T) == 2) {                                            \
      if (!a.asym) return launch_pair16<DK, CC, false>(a, BV, stages, st);     \
      if constexpr (chain_asym_ok(DK, CC))                                     \
        return launch_pair16<DK, CC, true>(a, BV, stages, st);                 \
    }                                                                          \
    if (stages & 1) {                                                          \
      e = launch_ut<T, DK, CC>(a, st);                                         \
      if (e != hipSuccess) return e;                                           \
    }                                                                          \
    if (stages & 2) e = launch_scan_any<T, DK, CC>(a, BV, lds_scan, st);      \
    return e;
  switch (C) {
    DP_CASE_C(16)
    DP_CASE_C(32)
    DP_CASE_C(64)
    default:
      return hipErrorInvalidValue;
  }
#undef DP_CASE_C
}

template <typename T, int DK>
hipError_t launch_precond_dk(const PrecondArgs& a, hipStream_t st) {
  const long long nbh = (long long)a.B * a.H;
  constexpr int HPW = 64 / (DK < 64 ? DK : 64);  // heads per wavefront
  const unsigned blocks = (unsigned)((nbh + HPW - 1) / HPW);
  hipLaunchKernelGGL((dp_precond_kernel<T, DK>), dim3(blocks), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace dp

// Per-(type, dk) entry points, each defined in its own translation unit so
// that the instantiations compile in parallel.
#define DP_DECLARE_LAUNCHERS(TNAME, DK)                                                        \
  hipError_t dp_launch_fwd_##TNAME##_##DK(const dp::FwdArgs& a, int C, int BV, int lds_scan,   \
                                          int stages, hipStream_t st);                         \
  hipError_t dp_launch_precond_##TNAME##_##DK(const dp::PrecondArgs& a, hipStream_t st);   \
  hipError_t dp_launch_precond_chunked_##TNAME##_##DK(const dp::PrecondArgs& a, hipStream_t st); \
  hipError_t dp_launch_decode_##TNAME##_##DK(const dp::DecodeArgs& a, hipStream_t st);

#define DP_DEFINE_LAUNCHERS(T, TNAME, DK)                                                      \
  hipError_t dp_launch_fwd_##TNAME##_##DK(const dp::FwdArgs& a, int C, int BV, int lds_scan,   \
                                          int stages, hipStream_t st) {                        \
    return dp::launch_fwd_dk<T, DK>(a, C, BV, lds_scan, stages, st);                           \
  }                                                                                            \
  hipError_t dp_launch_precond_##TNAME##_##DK(const dp::PrecondArgs& a, hipStream_t st) {      \
    return dp::launch_precond_dk<T, DK>(a, st);                                                \
  }                                                                                            \
  hipError_t dp_launch_precond_chunked_##TNAME##_##DK(const dp::PrecondArgs& a, hipStream_t st) { \
    return dp::launch_precond_chunked_if<T, DK>(a, st);                                        \
  }                                                                                            \
  hipError_t dp_launch_decode_##TNAME##_##DK(const dp::DecodeArgs& a, hipStream_t st) {        \
    return dp::launch_decode_dk<T, DK>(a, st);                                                 \
  }
