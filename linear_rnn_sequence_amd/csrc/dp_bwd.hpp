// dp_bwd.hpp -- gfx950 kernels of the chunkwise DeltaProduct backward.
//
// The gradient of the forward of the DeltaProduct study notes (arXiv
// 2502.10297v7: sec. 2.2 Eq.(3) sub-steps, sec. 2.6 gate and readout, sec. 4.1
// the expanded sequence) w.r.t. q, the raw keys, v, the raw beta, the gate
// and the initial state, for symmetric keys.  It is the reverse-mode
// derivative of the chunkwise form (OSDN study notes, arXiv 2605.13473v1,
// sec. 2.5 / App.A.2, with the chunk-local log-gate G).  Per chunk, with the
// chunk-start state H0, Tb = T diag(beta):
//
//   X  = V - diag(e^G) K H0             Up = Tb X
//   H1 = e^{G_C} H0 + K^T diag(e^{G_C - G}) Up
//   O  = diag(e^{G_l}) Q H0 + P Up,      P_rj = e^{G_l - G_j} q_r.k_j  (j <= l)
//
// (l the readout sub-step of row r).  Given dH1 and dO, reverse mode gives
//
//   dUp = diag(e^{G_C - G}) K dH1 + P^T dO          dX = Tb^T dUp  (= dV)
//   dH0 = e^{G_C} dH1 + Q^T diag(e^{G_l}) dO - K^T diag(e^G) dX
//   dTb = dUp X^T,  dT = dTb diag(beta),  dM = -T^T dT T^T  (strictly lower)
//
// and the key, query, beta and log-gate terms collected in
// dp_bwd_chunk_kernel.  Three launches:
//   dp_ut_kernel<.., float, false>  T (fp32) and (1/|k|, G) per chunk
//   dp_bwd_scans_kernel    the two sequential scans side by side, one role
//                          per workgroup: sequential over chunks in reverse,
//                          dH1 and dUp of every chunk -> workspace and dH0 of
//                          chunk 0 -> dh0 (bwd_dstate_body); sequential over
//                          chunks, the forward's chunk-start states H0 ->
//                          workspace (bwd_states_body)
//   dp_bwd_chunk_kernel    one workgroup per chunk, all in parallel: dq, dk,
//                          dv, dbeta, dg from H0, dH1, dUp and the chunk
// The state and its gradient are kept in fp32, and every product accumulates
// in fp32; the MFMA operands are the input's operand type (fp16 for bf16
// inputs, as the forward uses; fp32 for fp32 inputs).
//
// ASYM: write keys W given apart from the read keys (the OSDN write-key
// forward, sec. 2.5 phase 2): M = strict_tril(diag(beta)(E o K W^T)), the
// state update and the readout scores use W, X and the state read use K.
// The formulas above then split the key gradient in two:
//   dK = -diag(e^G) dX H0^T + Z W                         (read keys)
//   dW = diag(e^{G_C - G}) Up dH1^T + Gm^T Q + Z^T K       (write keys, as given)
// with S = K W^T in the beta and gate terms and Q W^T in the scores.
#pragma once

#include "dp_kernels.hpp"

namespace dp {

constexpr int kBwdChunk = 32;  // sub-steps per chunk of the backward
constexpr int kBwdBV = 16;     // value columns per block

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;       // nullptr: no gate
  const float* h0;      // nullptr: zero initial state
  const void* kt;       // ASYM: [B, L, H, n_h, dk] write keys, input type
  float* dkt;           // ASYM: [B, L, H, n_h, dk] their gradient
  const void* dout;     // [B, L, H, dv], input type
  const float* dfinal;  // [B, H, dk, dv] or nullptr (zero)
  const float* wsT;     // [B*H*nc][C][C] T (fp32)
  const float2* wsS;    // [B*H*nc][C] (1/|k|, G)
  // in the MFMA operand type (the per-chunk kernel's only use of them is as
  // operands): fp16 for bf16 inputs, fp32 for fp32 inputs
  void* hs;             // [B*H*nc][dk][dv] chunk-start states
  void* dhe;            // [B*H*nc][dk][dv] gradients of the chunk-end states
  void* dup;            // [B*H*nc][C][dv] gradients of the pseudo-values
  float* dq;            // [B, L, H, dk]
  float* dk;            // [B, L, H, n_h, dk]
  float* dv;            // [B, L, H, n_h, dv]
  float* dbeta;         // [B, L, H, n_h]
  float* dg;            // [B, L, H] or nullptr
  float* dh0;           // [B, H, dk, dv] or nullptr
  int N, B, H, L, n_h, dvd, nc, RT, nvb;
  uint32_t nh_magic;
  int nh_shift;
};

// acc += A * B, A read transposed (element (m, k) at a[k * lda + ra + m]) and
// B read k-major (element (k, n) at b[k * ldb + rb + n]).
template <typename T, int K>
__device__ __forceinline__ f32x4_t mm_tile_tt(f32x4_t acc, const T* a, int lda, int ra, const T* b, int ldb,
                                              int rb) {
  using M = Mfma<T>;
  static_assert(K % M::KS == 0 || K % M::KS == 16, "contraction length");
#pragma unroll
  for (int k0 = 0; k0 + M::KS <= K; k0 += M::KS)
    acc = M::mma(M::load_t(a, lda, ra, k0), M::load_t(b, ldb, rb, k0), acc);
  if constexpr (K % M::KS == 16)
    acc = M::mma4(M::load4_t(a, lda, ra, K - 16), M::load4_t(b, ldb, rb, K - 16), acc);
  return acc;
}
template <int K>
__device__ __forceinline__ f32x4_t mm_tile_tt(f32x4_t acc, const float* a, int lda, int ra, const float* b,
                                              int ldb, int rb) {
  return mm_tile_tt<float, K>(acc, a, lda, ra, b, ldb, rb);
}

// Row pitch (elements) of an LDS operand buffer of n columns: n plus 16 bytes.
template <typename OT>
__host__ __device__ constexpr int bwd_ld(int n) {
  return n + 16 / (int)sizeof(OT);
}

// Sum over the 16 lanes of one lane group (one accumulator row of a tile).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}
// Sum over the 4 lane groups (one accumulator column of a tile, per e).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Per-chunk indexing shared by the backward kernels: row of each sub-step in
// the [B, L, H, n_h, *] tensors (-1 past the end), token of each readout row
// (-1 when the row is empty) and its sub-step within the chunk.
struct BwdChunkMeta {
  long long* row;  // [C]
  long long* tok;  // [RT]
  int* loc;        // [RT]
};

template <int C>
__device__ __forceinline__ void bwd_index_chunk(const BwdArgs& p, int b, int h, int c, int RT,
                                                const BwdChunkMeta& m) {
  const int tid = threadIdx.x;
  const int s0 = c * C;
  const long long tok0 = (long long)b * p.L * p.H + h;
  if (tid < C) {
    const int s = s0 + tid;
    long long row = -1;
    if (s < p.N) {
      const int t = fastdiv(s, p.nh_magic, p.nh_shift);
      row = (tok0 + (long long)t * p.H) * p.n_h + (s - t * p.n_h);
    }
    m.row[tid] = row;
  }
  if (tid < RT) {
    const int r0 = s0 + (p.n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * p.n_h));
    const int s = r0 + tid * p.n_h;
    const bool ok = s < s0 + C && s < p.N;
    m.tok[tid] = ok ? tok0 + (long long)fastdiv(s, p.nh_magic, p.nh_shift) * p.H : -1;
    m.loc[tid] = ok ? s - s0 : -1;
  }
}

// ---------------------------------------------------------------------------
// Software pipelining of the two sequential kernels.  While a chunk is
// computed from LDS, every thread already holds its slice of the next
// chunk's operands in registers (loaded with the widest aligned loads); after
// the chunk's last barrier it writes them to LDS.  One thread per C/256 of a
// sub-step row: thread t covers row t / TPR, elements (t % TPR) * E ..

// E consecutive stored elements of T, read with loads as wide as their
// alignment allows (E * sizeof(T) bytes, at most 16 at a time).
template <typename T, int E>
struct RawSlice {
  T v[E];
  __device__ __forceinline__ void load(const T* src) {
    constexpr int NB = E * (int)sizeof(T);
    constexpr int AL = NB >= 16 ? 16 : NB;
    __builtin_memcpy(v, __builtin_assume_aligned(src, AL), NB);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = T{};
  }
  // zero unless `in` (a select per element: no branch around the load before it)
  __device__ __forceinline__ void keep(bool in) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = in ? v[i] : T{};
  }
  __device__ __forceinline__ float operator[](int i) const { return to_f32(v[i]); }
};

// Row of sub-step s of head (b, h) in the [B, L, H, n_h, *] tensors, or -1 past the end.
__device__ __forceinline__ long long bwd_row(const BwdArgs& p, int b, int h, int s) {
  if (s >= p.N) return -1;
  const int t = fastdiv(s, p.nh_magic, p.nh_shift);
  return (((long long)b * p.L + t) * p.H + h) * p.n_h + (s - t * p.n_h);
}

// Readout row rr of chunk c: its token's row in the [B, L, H, *] tensors and
// its sub-step inside the chunk, or (-1, -1) when the chunk has no such row.
__device__ __forceinline__ void bwd_readout(const BwdArgs& p, int b, int h, int c, int C, int rr, long long* tok,
                                            int* loc) {
  const int s0 = c * C;
  const int r0 = s0 + (p.n_h - 1 - (s0 - fastdiv(s0, p.nh_magic, p.nh_shift) * p.n_h));
  const int s = r0 + rr * p.n_h;
  const bool ok = s < s0 + C && s < p.N;
  *tok = ok ? ((long long)b * p.L + fastdiv(s, p.nh_magic, p.nh_shift)) * p.H + h : -1;
  *loc = ok ? s - s0 : -1;
}

// The operands every sequential kernel needs per chunk: the thread's slice of
// the unit keys (with 1/|k| of its row), its four entries of T, and for
// threads t < C the scalars of sub-step t (the raw beta, G, G of the chunk's
// last).  Every lane loads on every path (rows past the end read row 0, in
// bounds, and are zeroed by a select), so the compiler counts the loads in
// flight exactly and waits only where a value is used, a chunk later; beta
// is clamped where it is committed.
template <typename T, int DK, int C, bool ASYM = false>
struct BwdChunkCommon {
  static constexpr int TPR = 256 / C;  // threads per sub-step row
  static constexpr int EK = DK / TPR;  // key elements per thread
  static_assert(C * C == 4 * 256 && EK >= 1 && DK % TPR == 0, "32-sub-step chunks, 256 threads");
  RawSlice<T, EK> k;
  RawSlice<T, ASYM ? EK : 1> w;  // ASYM: the write-key slice of the same row
  float rinv;  // 1/|k| of the key row (0 past the end)
  float4 t;    // T entries 4 tid .. 4 tid + 3
  float beta, g, gl;
  __device__ __forceinline__ void load(const BwdArgs& p, int b, int h, int c, long long chunk) {
    const int tid = threadIdx.x;
    const long long row = bwd_row(p, b, h, c * C + tid / TPR);
    const bool in = row >= 0;
    const long long rr = in ? row : 0;
    k.load(static_cast<const T*>(p.k) + rr * DK + (tid % TPR) * EK);
    k.keep(in);
    if constexpr (ASYM) {
      w.load(static_cast<const T*>(p.kt) + rr * DK + (tid % TPR) * EK);
      w.keep(in);
    }
    const float ri = p.wsS[chunk * C + tid / TPR].x;
    rinv = in ? ri : 0.f;
    t = *reinterpret_cast<const float4*>(p.wsT + chunk * C * C + 4 * tid);
    const int ts = tid & (C - 1);  // threads t < C keep sub-step t's scalars
    const long long rs = bwd_row(p, b, h, c * C + ts);
    const float bt = p.beta[rs >= 0 ? rs : 0];
    beta = rs >= 0 ? bt : 0.f;
    g = p.wsS[chunk * C + ts].y;
    gl = p.wsS[chunk * C + C - 1].y;
  }
  template <int LDK, int LDC, typename OT>
  __device__ __forceinline__ void commit(OT* sK, OT* sT, OT* sW = nullptr) const {
    const int tid = threadIdx.x;
    OT* kd = sK + (tid / TPR) * LDK + (tid % TPR) * EK;
#pragma unroll
    for (int i = 0; i < EK; ++i) kd[i] = from_f32<OT>(k[i] * rinv);
    if constexpr (ASYM) {
      OT* wd = sW + (tid / TPR) * LDK + (tid % TPR) * EK;
#pragma unroll
      for (int i = 0; i < EK; ++i) wd[i] = from_f32<OT>(w[i]);
    }
    OT* td = sT + ((4 * tid) / C) * LDC + (4 * tid) % C;
    td[0] = from_f32<OT>(t.x);
    td[1] = from_f32<OT>(t.y);
    td[2] = from_f32<OT>(t.z);
    td[3] = from_f32<OT>(t.w);
  }
};

// ---------------------------------------------------------------------------
// The forward's chunk-start states: one workgroup per (head, block of BV value
// columns), sequential over the chunks.  Each wavefront keeps the fp32 state
// tiles it owns in registers; LDS holds their operand copy.
template <typename T, int DK, int C, int BV, bool ASYM>
__host__ __device__ constexpr int bwd_states_lds_bytes() {
  using OT = typename OpType<T>::type;
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(BV), LDF = BV + 4;
  return ((ASYM ? 2 : 1) * C * LDK + C * LDC + DK * LDB + 2 * C * LDB) * (int)sizeof(OT) + (C * LDF + 3 * C) * 4;
}

template <typename T, int DK, int C, int BV, bool ASYM>
__device__ __forceinline__ void bwd_states_body(const BwdArgs& p, unsigned char* smb, const int wg) {
  using OT = typename OpType<T>::type;  // MFMA operand type
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(BV), LDF = BV + 4;
  constexpr int NCT = C / 16, NDT = DK / 16, NVT = BV / 16;
  constexpr int NHT = NDT * NVT, HPW = (NHT + 3) / 4;  // state tiles, per wavefront
  using Common = BwdChunkCommon<T, DK, C, ASYM>;
  constexpr int TPR = Common::TPR, EV = BV / TPR;
  static_assert(EV >= 1 && BV % TPR == 0, "value slice");
  OT* sK = reinterpret_cast<OT*>(smb);  // C x LDK unit read keys
  OT* sW = sK + C * LDK;                // ASYM: write keys
  OT* sT = sW + (ASYM ? C * LDK : 0);
  OT* sHo = sT + C * LDC;  // operand copy of the state
  OT* sXb = sHo + DK * LDB;
  OT* sU = sXb + C * LDB;
  float* sV = reinterpret_cast<float*>(sU + C * LDB);  // the values (fp32)
  float* sB = sV + C * LDF;
  float* sEG = sB + C;
  float* sEL = sEG + C;
  OT* const sKw = ASYM ? sW : sK;  // the keys the state update writes with

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nvb = p.dvd / BV;
  const int bh = wg / nvb, vb = wg % nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;
  const T* vp = static_cast<const T*>(p.v);

  // the operands of the next chunk, in registers (one chunk of this scan is
  // long enough to cover the loads)
  struct Next {
    Common x;
    RawSlice<T, EV> v;
  };
  Next nb;
  auto prefetch = [&](Next& nx, int c) {
    const long long chunk = (long long)bh * p.nc + c;
    nx.x.load(p, b, h, c, chunk);
    const long long row = bwd_row(p, b, h, c * C + tid / TPR);
    nx.v.load(vp + (row >= 0 ? row : 0) * p.dvd + v0 + (tid % TPR) * EV);
    nx.v.keep(row >= 0);
  };

  // the fp32 state: tile wave + 4u of the DK x BV block, rows 4 grp + e, column col
  f32x4_t hacc[HPW];
#pragma unroll
  for (int u = 0; u < HPW; ++u) {
    const int tile = wave + 4 * u;
    hacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tile < NHT) {
      const int dt = tile / NVT, nt = tile % NVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = dt * 16 + 4 * grp + e, n = nt * 16 + col;
        if (p.h0 != nullptr) hacc[u][e] = p.h0[((long long)bh * DK + d) * p.dvd + v0 + n];
        sHo[d * LDB + n] = from_f32<OT>(hacc[u][e]);
      }
    }
  }
  if (p.nc > 0) prefetch(nb, 0);
  auto body = [&](Next& nx, int c) {
    const long long chunk = (long long)bh * p.nc + c;
    __syncthreads();  // the previous chunk is done with every buffer
    nx.x.template commit<LDK, LDC>(sK, sT, sW);
    {
      float* vd = sV + (tid / TPR) * LDF + (tid % TPR) * EV;
#pragma unroll
      for (int i = 0; i < EV; ++i) vd[i] = nx.v[i];
    }
    if (tid < C) {
      sB[tid] = clamp_keep_nan(nx.x.beta, 0.f, 2.f);
      sEG[tid] = expf(nx.x.g);
      sEL[tid] = expf(nx.x.gl - nx.x.g);
    }
    // the state at the chunk start, from the tiles each wavefront holds
    OT* hdst = static_cast<OT*>(p.hs) + chunk * DK * p.dvd + v0;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NHT) {
        const int dt = tile / NVT, nt = tile % NVT;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hdst[(long long)(dt * 16 + 4 * grp + e) * p.dvd + nt * 16 + col] = from_f32<OT>(hacc[u][e]);
      }
    }
    __syncthreads();
    prefetch(nx, min(c + 1, p.nc - 1));  // lands while this chunk is computed (the last one again at the end)
    // beta X = beta (V - diag(e^G) K H0)
    for (int tile = wave; tile < NCT * NVT; tile += 4) {
      const int ct = tile / NVT, nt = tile % NVT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, DK>(acc, sK, LDK, ct * 16, sHo, LDB, nt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = ct * 16 + 4 * grp + e, n = nt * 16 + col;
        sXb[r * LDB + n] = from_f32<OT>(sB[r] * (sV[r * LDF + n] - sEG[r] * acc[e]));
      }
    }
    __syncthreads();
    // diag(e^{G_C - G}) Up, Up = T (beta X)
    for (int tile = wave; tile < NCT * NVT; tile += 4) {
      const int ct = tile / NVT, nt = tile % NVT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, C>(acc, sT, LDC, ct * 16, sXb, LDB, nt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = ct * 16 + 4 * grp + e;
        sU[r * LDB + nt * 16 + col] = from_f32<OT>(sEL[r] * acc[e]);
      }
    }
    __syncthreads();
    // H = e^{G_C} H + W^T (diag(e^{G_C - G}) Up): each wavefront its own tiles
    const float egl = sEG[C - 1];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NHT) {
        const int dt = tile / NVT, nt = tile % NVT;
        f32x4_t acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = egl * hacc[u][e];
        acc = mm_tile_tt<OT, C>(acc, sKw, LDK, dt * 16, sU, LDB, nt * 16);
        hacc[u] = acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) sHo[(dt * 16 + 4 * grp + e) * LDB + nt * 16 + col] = from_f32<OT>(acc[e]);
      }
    }
  };
  for (int c = 0; c < p.nc; ++c) body(nb, c);
}

// ---------------------------------------------------------------------------
// The reverse chunk scan of the state gradient (bwd_dstate_body), one
// workgroup per (head, block of BV value columns), chunks last to first.
// Writes dH1 (the gradient of each chunk's end state) and dUp per chunk, and
// the gradient of the initial state.
// LDS of the state-gradient scan (dynamic: with the write keys it passes 64 KB):
// the operand buffers in OT, then the fp32 state gradient and the scalars.
template <typename OT, int DK, int C, int BV, int RT, bool ASYM>
__host__ __device__ constexpr int bwd_dstate_lds_bytes() {
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(BV);
  return ((ASYM ? 2 : 1) * C * LDK + RT * LDK + C * LDC + RT * LDC + DK * LDB + 2 * RT * LDB + 2 * C * LDB) *
             (int)sizeof(OT) +
         (DK * (BV + 4) + 4 * C) * 4 + RT * 4;
}

template <typename T, int DK, int C, int BV, int NRT, bool ASYM>
__device__ __forceinline__ void bwd_dstate_body(const BwdArgs& p, unsigned char* smb, const int wg) {
  using OT = typename OpType<T>::type;  // MFMA operand type
  constexpr int RT = 16 * NRT;
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(BV), LDF = BV + 4;
  constexpr int NCT = C / 16, NDT = DK / 16, NVT = BV / 16;
  using Common = BwdChunkCommon<T, DK, C, ASYM>;
  constexpr int TPQ = 256 / RT, EQ = DK / TPQ, EO = BV / TPQ;  // per readout row
  static_assert(EQ >= 1 && EO >= 1 && DK % TPQ == 0 && BV % TPQ == 0, "readout slices");
  OT* sK = reinterpret_cast<OT*>(smb);  // C x LDK unit read keys
  OT* sW = sK + C * LDK;                // ASYM: C x LDK write keys
  OT* sQ = sW + (ASYM ? C * LDK : 0);
  OT* sT = sQ + RT * LDK;
  OT* sP = sT + C * LDC;
  OT* sdHo = sP + RT * LDC;  // operand copy of the state gradient
  OT* sdO = sdHo + DK * LDB;
  OT* sdOe = sdO + RT * LDB;
  OT* sdUp = sdOe + RT * LDB;
  OT* sdX = sdUp + C * LDB;
  float* sdH = reinterpret_cast<float*>(sdX + C * LDB);  // the fp32 state gradient
  float* sB = sdH + DK * LDF;
  float* sG = sB + C;
  float* sEG = sG + C;
  float* sEL = sEG + C;
  int* sLoc = reinterpret_cast<int*>(sEL + C);
  OT* const sKw = ASYM ? sW : sK;  // the keys of the state update and the scores

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int bh = wg / p.nvb, vb = wg % p.nvb;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = vb * BV;
  const T* dop = static_cast<const T*>(p.dout);
  const T* qp = static_cast<const T*>(p.q);

  // the operands of the next chunk, in registers (one chunk of this scan is
  // long enough to cover the loads)
  struct Next {
    Common x;
    RawSlice<T, EQ> q;
    RawSlice<T, EO> o;
    int loc;
    float g;  // G at the readout row's sub-step
  };
  Next nb;
  auto prefetch = [&](Next& nx, int c) {
    const long long chunk = (long long)bh * p.nc + c;
    nx.x.load(p, b, h, c, chunk);
    long long tok;
    bwd_readout(p, b, h, c, C, tid / TPQ, &tok, &nx.loc);
    const bool in = tok >= 0;  // loads on every path, then selects (as in BwdChunkCommon)
    const long long tt = in ? tok : 0;
    nx.q.load(qp + tt * DK + (tid % TPQ) * EQ);
    nx.q.keep(in);
    nx.o.load(dop + tt * p.dvd + v0 + (tid % TPQ) * EO);
    nx.o.keep(in);
    const float gg = p.wsS[chunk * C + (in ? nx.loc : 0)].y;
    nx.g = in ? gg : 0.f;
  };

  for (int idx = tid; idx < DK * BV; idx += 256) {
    const int d = idx / BV, n = idx % BV;
    const float x = p.dfinal != nullptr ? p.dfinal[((long long)bh * DK + d) * p.dvd + v0 + n] : 0.f;
    sdH[d * LDF + n] = x;
    sdHo[d * LDB + n] = from_f32<OT>(x);
  }
  if (p.nc > 0) prefetch(nb, p.nc - 1);
  auto body = [&](Next& nx, int c) {
    const long long chunk = (long long)bh * p.nc + c;
    __syncthreads();  // the previous chunk is done with every buffer
    nx.x.template commit<LDK, LDC>(sK, sT, sW);
    {
      const int rr = tid / TPQ, q0 = (tid % TPQ) * EQ, o0 = (tid % TPQ) * EO;
#pragma unroll
      for (int i = 0; i < EQ; ++i) sQ[rr * LDK + q0 + i] = from_f32<OT>(nx.q[i]);
      const float e = nx.loc >= 0 ? expf(nx.g) : 0.f;
#pragma unroll
      for (int i = 0; i < EO; ++i) {
        sdO[rr * LDB + o0 + i] = from_f32<OT>(nx.o[i]);
        sdOe[rr * LDB + o0 + i] = from_f32<OT>(e * nx.o[i]);
      }
      if (tid % TPQ == 0) sLoc[rr] = nx.loc;
    }
    if (tid < C) {
      sB[tid] = clamp_keep_nan(nx.x.beta, 0.f, 2.f);
      sG[tid] = nx.x.g;
      sEG[tid] = expf(nx.x.g);
      sEL[tid] = expf(nx.x.gl - nx.x.g);
    }
    // the gradient of the chunk's end state
    OT* ddst = static_cast<OT*>(p.dhe) + chunk * DK * p.dvd + v0;
    for (int idx = tid; idx < DK * BV; idx += 256) {
      const int d = idx / BV, n = idx % BV;
      ddst[(long long)d * p.dvd + n] = sdHo[d * LDB + n];
    }
    __syncthreads();
    prefetch(nx, max(c - 1, 0));  // lands while this chunk is computed (the first one again at the end)
    // P = masked, gated scores (RT x C)
    for (int tile = wave; tile < NRT * NCT; tile += 4) {
      const int rt = tile / NCT, ct = tile % NCT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile<OT, DK>(acc, sQ, LDK, rt * 16, sKw, LDK, ct * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rt * 16 + 4 * grp + e, j = ct * 16 + col;
        const int l = sLoc[r];
        // read for every lane (in bounds), then masked: no per-lane branch around the reads
        const float ex = expf(sG[max(l, 0)] - sG[j]);
        sP[r * LDC + j] = from_f32<OT>((l >= 0 && j <= l) ? acc[e] * ex : 0.f);
      }
    }
    __syncthreads();
    // dUp = diag(e^{G_C - G}) W dH1 + P^T dO
    for (int tile = wave; tile < NCT * NVT; tile += 4) {
      const int ct = tile / NVT, nt = tile % NVT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, DK>(acc, sKw, LDK, ct * 16, sdHo, LDB, nt * 16);
      acc2 = mm_tile_tt<OT, RT>(acc2, sP, LDC, ct * 16, sdO, LDB, nt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ct * 16 + 4 * grp + e, n = nt * 16 + col;
        const float du = sEL[j] * acc[e] + acc2[e];
        sdUp[j * LDB + n] = from_f32<OT>(du);
        static_cast<OT*>(p.dup)[(chunk * C + j) * p.dvd + v0 + n] = from_f32<OT>(du);
      }
    }
    __syncthreads();
    // diag(e^G) dX,  dX = Tb^T dUp = diag(beta) T^T dUp
    for (int tile = wave; tile < NCT * NVT; tile += 4) {
      const int ct = tile / NVT, nt = tile % NVT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tt<OT, C>(acc, sT, LDC, ct * 16, sdUp, LDB, nt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ct * 16 + 4 * grp + e;
        sdX[j * LDB + nt * 16 + col] = from_f32<OT>(sEG[j] * sB[j] * acc[e]);
      }
    }
    __syncthreads();
    // dH0 = e^{G_C} dH1 + Q^T diag(e^{G_l}) dO - K^T diag(e^G) dX
    const float egl = sEG[C - 1];
    for (int tile = wave; tile < NDT * NVT; tile += 4) {
      const int dt = tile / NVT, nt = tile % NVT;
      f32x4_t acc, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = egl * sdH[(dt * 16 + 4 * grp + e) * LDF + nt * 16 + col];
      acc = mm_tile_tt<OT, RT>(acc, sQ, LDK, dt * 16, sdOe, LDB, nt * 16);
      acc2 = mm_tile_tt<OT, C>(acc2, sK, LDK, dt * 16, sdX, LDB, nt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = acc[e] - acc2[e];
        sdH[(dt * 16 + 4 * grp + e) * LDF + nt * 16 + col] = x;
        sdHo[(dt * 16 + 4 * grp + e) * LDB + nt * 16 + col] = from_f32<OT>(x);
      }
    }
  };
  for (int c = p.nc - 1; c >= 0; --c) body(nb, c);
  __syncthreads();
  if (p.dh0 != nullptr) {
    for (int idx = tid; idx < DK * BV; idx += 256) {
      const int d = idx / BV, n = idx % BV;
      p.dh0[((long long)bh * DK + d) * p.dvd + v0 + n] = sdH[d * LDF + n];
    }
  }
}

// ---------------------------------------------------------------------------
// dp_bwd_scans_kernel: the two sequential scans in one launch.  The reverse
// scan of dH needs neither the forward's states nor their scan, so the
// workgroups take one role each and run side by side: the first B*H*(dv/16)
// the state gradient (16 value columns each, the longer scan, dispatched
// first), the rest the chunk-start states (BVS value columns each).
template <typename T, int DK, int C, int BVS, int NRT, bool ASYM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void dp_bwd_scans_kernel(BwdArgs p) {
  extern __shared__ __align__(16) unsigned char smb[];
  const int nd = p.B * p.H * p.nvb;
  if ((int)blockIdx.x < nd)
    bwd_dstate_body<T, DK, C, kBwdBV, NRT, ASYM>(p, smb, (int)blockIdx.x);
  else
    bwd_states_body<T, DK, C, BVS, ASYM>(p, smb, (int)blockIdx.x - nd);
}

// ---------------------------------------------------------------------------
// dp_bwd_chunk_kernel: the per-chunk gradients, one workgroup per chunk.
//
// The value columns are taken in blocks of 16: each block's X, Up and dX are
// formed in LDS and folded into register accumulators (fixed tile ownership
// per wavefront) of
//   dXH = dX H0^T (C x DK)   Y = Up dH1^T (C x DK)   A = dO H0^T (RT x DK)
//   dP = dO Up^T (RT x C)    dTb = dUp X^T (C x C)   <dH1, H0>
// after which the key, query, beta and log-gate gradients follow:
//   dq_r  = e^{G_l} A_r + sum_j Gm_rj k_j,     Gm_rj = e^{G_l - G_j} dP_rj (j <= l)
//   dkn   = -diag(e^G) dXH + diag(e^{G_C - G}) Y + Gm^T Q + Z K + Z^T K
//   Z_ij  = F_ij beta_i e^{G_i - G_j},  F = strict_tril(-T^T (dTb diag(beta)) T^T)
//   dbeta_j = sum_i dTb_ij T_ij + sum_i' F_ji' e^{G_j - G_i'} S_ji'   (S = K K^T)
//   dG    = the gate terms of each product, then dlog g = reverse cumsum of dG
// and finally the key normalisation, the beta clamp and the log of the gate.
// LDS of dp_bwd_chunk_kernel: the operand buffers in OT, then fp32 scalars and
// the row indices.
template <typename OT, int DK, int C, int RT, bool ASYM = false>
__host__ __device__ constexpr int bwd_chunk_lds_bytes() {
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(16);
  return ((ASYM ? 2 : 1) * C * LDK + RT * LDK + 3 * C * LDC + RT * LDC + 2 * DK * LDB + 6 * C * LDB +
          RT * LDB) * (int)sizeof(OT) +
         8 * C * 4 + C * 8 + RT * 12;
}

template <typename T, int DK, int C, int NRT, bool ASYM = false>
__global__ __launch_bounds__(256) void dp_bwd_chunk_kernel(BwdArgs p) {
  using OT = typename OpType<T>::type;  // MFMA operand type
  constexpr int BV = 16;
  constexpr int RT = 16 * NRT;
  constexpr int LDK = bwd_ld<OT>(DK), LDC = bwd_ld<OT>(C), LDB = bwd_ld<OT>(BV);
  constexpr int NCT = C / 16, NDT = DK / 16;
  constexpr int NKD = NCT * NDT, KPW = (NKD + 3) / 4;  // C x DK tiles
  constexpr int NQD = NRT * NDT, QPW = (NQD + 3) / 4;  // RT x DK tiles
  constexpr int NCC = NCT * NCT, NRC = NRT * NCT;
  static_assert(NCC <= 4 && NRC <= 4 && 2 * NCT <= 4, "one C x C and one RT x C tile per wavefront");

  extern __shared__ __align__(16) unsigned char smb[];
  OT* sK = reinterpret_cast<OT*>(smb);  // C x LDK unit keys
  OT* sWk = sK + C * LDK;               // ASYM: C x LDK write keys
  OT* sQ = sWk + (ASYM ? C * LDK : 0);  // RT x LDK readout queries
  OT* sT = sQ + RT * LDK;               // C x LDC  T
  OT* sA = sT + C * LDC;                // C x LDC  dT, then Z
  OT* sW = sA + C * LDC;                // C x LDC  T^T dT
  OT* sGm = sW + C * LDC;               // RT x LDC gated, masked dP
  OT* sH0 = sGm + RT * LDC;             // DK x LDB
  OT* sdHe = sH0 + DK * LDB;            // DK x LDB
  OT* sV = sdHe + DK * LDB;             // C x LDB
  OT* sdUp = sV + C * LDB;
  OT* sX = sdUp + C * LDB;
  OT* sXb = sX + C * LDB;  // beta X
  OT* sUp = sXb + C * LDB;
  OT* sdX = sUp + C * LDB;
  OT* sdO = sdX + C * LDB;                             // RT x LDB
  float* sB = reinterpret_cast<float*>(sdO + RT * LDB);  // C scalars each
  float* sG = sB + C;
  float* sEG = sG + C;
  float* sEL = sEG + C;
  float* sRinv = sEL + C;
  float* sDB = sRinv + C;  // dbeta accumulator
  float* sDG = sDB + C;    // dG accumulator
  float* sRD = sDG + C;    // k . dkn per row
  long long* sRow = reinterpret_cast<long long*>(sRD + C);
  long long* sTok = sRow + C;
  int* sLoc = reinterpret_cast<int*>(sTok + RT);
  OT* const sKw = ASYM ? sWk : sK;  // the keys of M's right side, the state update and the scores

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const long long chunk = blockIdx.x;
  const int bh = (int)(chunk / p.nc), c = (int)(chunk % p.nc);
  const int b = bh / p.H, h = bh % p.H;
  const T* vp = static_cast<const T*>(p.v);
  const T* dop = static_cast<const T*>(p.dout);
  const BwdChunkMeta meta{sRow, sTok, sLoc};
  const OT* hsrc = static_cast<const OT*>(p.hs) + chunk * DK * p.dvd;
  const OT* dhsrc = static_cast<const OT*>(p.dhe) + chunk * DK * p.dvd;
  const OT* dusrc = static_cast<const OT*>(p.dup) + chunk * C * p.dvd;
  // The next value block's operands, in registers: thread t holds EH
  // consecutive columns of row t / TPH of H0 and dH1, EV of sub-step row
  // t / TPR of V and dUp, and EO of readout row t / TPQ of dO.
  constexpr int TPH = 256 / DK, EH = BV / TPH;
  constexpr int TPR = 256 / C, EV = BV / TPR;
  constexpr int TPQ = 256 / RT, EO = BV / TPQ;
  static_assert(EH >= 1 && EV >= 1 && EO >= 1, "block slices");
  const int hd = tid / TPH, hn = (tid % TPH) * EH;
  const int vr = tid / TPR, vn = (tid % TPR) * EV;
  const int orr = tid / TPQ, on = (tid % TPQ) * EO;
  const long long vrow = bwd_row(p, b, h, c * C + vr);
  long long otok;
  int oloc;
  bwd_readout(p, b, h, c, C, orr, &otok, &oloc);
  RawSlice<OT, EH> nh0, ndh;
  RawSlice<T, EV> nv;
  RawSlice<OT, EV> ndu;
  RawSlice<T, EO> ndo;
  // every lane loads on every path (rows past the end read row 0, in bounds,
  // then a select zeroes them), so the compiler's wait counts stay exact
  const bool vin = vrow >= 0, oin = otok >= 0;
  const long long vrr = vin ? vrow : 0, orow = oin ? otok : 0;
  auto prefetch = [&](int vb) {
    const int v0 = vb * BV;
    nh0.load(hsrc + (long long)hd * p.dvd + v0 + hn);
    ndh.load(dhsrc + (long long)hd * p.dvd + v0 + hn);
    ndu.load(dusrc + (long long)vr * p.dvd + v0 + vn);
    nv.load(vp + vrr * p.dvd + v0 + vn);
    nv.keep(vin);
    ndo.load(dop + orow * p.dvd + v0 + on);
    ndo.keep(oin);
  };
  // the chunk's scalars first (committed at once), then its keys, T and readout
  // queries and value block 0, which land while the chunk's scores are formed
  const float2 sc = p.wsS[chunk * C + (tid & (C - 1))];
  BwdChunkCommon<T, DK, C, ASYM> cx;
  cx.load(p, b, h, c, chunk);
  constexpr int EQ = DK / TPQ;
  RawSlice<T, EQ> cq;
  cq.load(static_cast<const T*>(p.q) + orow * DK + (tid % TPQ) * EQ);
  cq.keep(oin);
  if (p.nvb > 0) prefetch(0);

  bwd_index_chunk<C>(p, b, h, c, RT, meta);
  if (tid < C) {
    sRinv[tid] = sc.x;
    sG[tid] = sc.y;
    sDB[tid] = 0.f;
    sDG[tid] = 0.f;
    sRD[tid] = 0.f;
  }
  __syncthreads();
  if (tid < C) {
    sB[tid] = clamp_keep_nan(cx.beta, 0.f, 2.f);
    sEG[tid] = expf(sG[tid]);
    sEL[tid] = expf(sG[C - 1] - sG[tid]);
  }
  cx.template commit<LDK, LDC>(sK, sT, sWk);
#pragma unroll
  for (int i = 0; i < EQ; ++i) sQ[orr * LDK + (tid % TPQ) * EQ + i] = from_f32<OT>(cq[i]);
  __syncthreads();

  // S = K W^T (tile `wave`) and Q W^T (tile `wave` when < NRC), kept in registers (W = K when symmetric)
  const int cit = wave / NCT, cjt = wave % NCT;  // the C x C tile of this wavefront
  const int rrt = wave / NCT, rct = wave % NCT;  // the RT x C tile of this wavefront
  f32x4_t accS = {0.f, 0.f, 0.f, 0.f}, accQK = {0.f, 0.f, 0.f, 0.f};
  if (wave < NCC) accS = mm_tile<OT, DK>(accS, sK, LDK, cit * 16, sKw, LDK, cjt * 16);
  if (wave < NRC) accQK = mm_tile<OT, DK>(accQK, sQ, LDK, rrt * 16, sKw, LDK, rct * 16);

  f32x4_t aXH[KPW], aY[KPW], aA[QPW];
  f32x4_t aP = {0.f, 0.f, 0.f, 0.f}, aTb = {0.f, 0.f, 0.f, 0.f};
  static_assert(BV == 16, "16-column value blocks");
#pragma unroll
  for (int u = 0; u < KPW; ++u) aXH[u] = aY[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < QPW; ++u) aA[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float hdot = 0.f;

  for (int vb = 0; vb < p.nvb; ++vb) {
    const int v0 = vb * BV;
#pragma unroll
    for (int i = 0; i < EH; ++i) {
      sH0[hd * LDB + hn + i] = from_f32<OT>(nh0[i]);
      sdHe[hd * LDB + hn + i] = from_f32<OT>(ndh[i]);
      hdot = fmaf(nh0[i], ndh[i], hdot);
    }
#pragma unroll
    for (int i = 0; i < EV; ++i) {
      sV[vr * LDB + vn + i] = from_f32<OT>(nv[i]);
      sdUp[vr * LDB + vn + i] = from_f32<OT>(ndu[i]);
    }
#pragma unroll
    for (int i = 0; i < EO; ++i) sdO[orr * LDB + on + i] = from_f32<OT>(ndo[i]);
    __syncthreads();
    prefetch(min(vb + 1, p.nvb - 1));  // lands while this block is computed (the last one again at the end)
    if (wave < NCT) {
      // X = V - diag(e^G) K H0
      const int ct = wave;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, DK>(acc, sK, LDK, ct * 16, sH0, LDB, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = ct * 16 + 4 * grp + e;
        const float x = to_f32(sV[r * LDB + col]) - sEG[r] * acc[e];
        sX[r * LDB + col] = from_f32<OT>(x);
        sXb[r * LDB + col] = from_f32<OT>(sB[r] * x);
      }
    } else if (wave < 2 * NCT) {
      // dX = diag(beta) T^T dUp, which is dv
      const int ct = wave - NCT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tt<OT, C>(acc, sT, LDC, ct * 16, sdUp, LDB, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ct * 16 + 4 * grp + e;
        const float dx = sB[j] * acc[e];
        sdX[j * LDB + col] = from_f32<OT>(dx);
        if (sRow[j] >= 0) p.dv[sRow[j] * p.dvd + v0 + col] = dx;
      }
    }
    __syncthreads();
    if (wave < NCT) {
      // Up = T (beta X)
      const int ct = wave;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, C>(acc, sT, LDC, ct * 16, sXb, LDB, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sUp[(ct * 16 + 4 * grp + e) * LDB + col] = from_f32<OT>(acc[e]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NKD) {
        const int ct = tile / NDT, dt = tile % NDT;
        aXH[u] = mm_tile<OT, BV>(aXH[u], sdX, LDB, ct * 16, sH0, LDB, dt * 16);
        aY[u] = mm_tile<OT, BV>(aY[u], sUp, LDB, ct * 16, sdHe, LDB, dt * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      const int tile = wave + 4 * u;
      if (tile < NQD) {
        const int rt = tile / NDT, dt = tile % NDT;
        aA[u] = mm_tile<OT, BV>(aA[u], sdO, LDB, rt * 16, sH0, LDB, dt * 16);
      }
    }
    if (wave < NRC) aP = mm_tile<OT, BV>(aP, sdO, LDB, rrt * 16, sUp, LDB, rct * 16);
    if (wave < NCC) aTb = mm_tile<OT, BV>(aTb, sdUp, LDB, cit * 16, sX, LDB, cjt * 16);
    __syncthreads();  // the next block overwrites the block buffers
  }

  // <dH1, H0>: block sum into the gate gradient of the chunk's last sub-step
  hdot = sum16(hdot);
  hdot += __shfl_xor(hdot, 16);
  hdot += __shfl_xor(hdot, 32);
  if (lane == 0) atomicAdd(&sDG[C - 1], sEG[C - 1] * hdot);

  // dT = dTb diag(beta) -> sA;  dbeta_j += sum_i dTb_ij T_ij
  if (wave < NCC) {
    const int j = cjt * 16 + col;
    float cs = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = cit * 16 + 4 * grp + e;
      cs = fmaf(aTb[e], to_f32(sT[i * LDC + j]), cs);
      sA[i * LDC + j] = from_f32<OT>(aTb[e] * sB[j]);
    }
    cs = sum_groups(cs);
    if (grp == 0) atomicAdd(&sDB[j], cs);
  }
  __syncthreads();
  // T^T dT -> sW
  if (wave < NCC) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile_tt<OT, C>(acc, sT, LDC, cit * 16, sA, LDC, cjt * 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) sW[(cit * 16 + 4 * grp + e) * LDC + cjt * 16 + col] = from_f32<OT>(acc[e]);
  }
  __syncthreads();
  // F = -(T^T dT) T^T (strictly lower); the M terms of dbeta and dG; Z -> sA
  if (wave < NCC) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile<OT, C>(acc, sW, LDC, cit * 16, sT, LDC, cjt * 16);
    const int j = cjt * 16 + col;
    float csum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = cit * 16 + 4 * grp + e;
      const bool ok = j < i && sRow[i] >= 0;
      const float exr = expf(sG[i] - sG[j]);  // every lane reads, then the mask selects
      const float ex = ok ? exr : 0.f;
      const float fm = ok ? -acc[e] * ex : 0.f;  // F_ij e^{G_i - G_j}
      const float z = fm * sB[i];
      const float zs = z * accS[e];
      const float rb = sum16(fm * accS[e]);
      const float rg = sum16(zs);
      if (col == 0) {
        atomicAdd(&sDB[i], rb);
        atomicAdd(&sDG[i], rg);
      }
      csum += zs;
      sA[i * LDC + j] = from_f32<OT>(z);
    }
    csum = sum_groups(csum);
    if (grp == 0) atomicAdd(&sDG[j], -csum);
  }
  // Gm = e^{G_l - G_j} dP (j <= l); the score terms of dG
  if (wave < NRC) {
    const int j = rct * 16 + col;
    float csum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rrt * 16 + 4 * grp + e;
      const int l = sLoc[r];
      const bool ok = l >= 0 && j <= l;
      const float exr = expf(sG[max(l, 0)] - sG[j]);  // in bounds for every lane; masked below
      const float gm = ok ? aP[e] * exr : 0.f;
      const float pr = gm * accQK[e];
      const float rs = sum16(pr);
      if (col == 0 && l >= 0) atomicAdd(&sDG[l], rs);
      csum += pr;
      sGm[r * LDC + j] = from_f32<OT>(gm);
    }
    csum = sum_groups(csum);
    if (grp == 0) atomicAdd(&sDG[j], -csum);
  }
  __syncthreads();
  // dq = diag(e^{G_l}) A + Gm W;  dG_l += e^{G_l} q_r . A_r
  float* dqp = p.dq;
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const int tile = wave + 4 * u;
    if (tile < NQD) {
      const int rt = tile / NDT, dt = tile % NDT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<OT, C>(acc, sGm, LDC, rt * 16, sKw, LDK, dt * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rt * 16 + 4 * grp + e, d = dt * 16 + col;
        const int l = sLoc[r];
        const float el = l >= 0 ? sEG[l] : 0.f;
        const float a = aA[u][e];
        const float qd = sum16(to_f32(sQ[r * LDK + d]) * a * el);
        if (l >= 0) {
          dqp[sTok[r] * DK + d] = el * a + acc[e];
          if (col == 0) atomicAdd(&sDG[l], qd);
        }
      }
    }
  }
  // dkn = -diag(e^G) dXH + diag(e^{G_C - G}) Y + Gm^T Q + Z K + Z^T K, and its gate terms;
  // ASYM: dkn = -diag(e^G) dXH + Z W (read keys), and the write keys' gradient
  // diag(e^{G_C - G}) Y + Gm^T Q + Z^T K goes out as it is
  f32x4_t dkn[KPW];
  float glast = 0.f;
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int tile = wave + 4 * u;
    dkn[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tile < NKD) {
      const int ct = tile / NDT, dt = tile % NDT;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (ASYM) {
        f32x4_t accw = {0.f, 0.f, 0.f, 0.f};
        accw = mm_tile_tt<OT, RT>(accw, sGm, LDC, ct * 16, sQ, LDK, dt * 16);
        accw = mm_tile_tt<OT, C>(accw, sA, LDC, ct * 16, sK, LDK, dt * 16);
        acc = mm_tile_tb<OT, C>(acc, sA, LDC, ct * 16, sWk, LDK, dt * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = ct * 16 + 4 * grp + e, d = dt * 16 + col;
          const float kv = to_f32(sK[j * LDK + d]), wv = to_f32(sWk[j * LDK + d]);
          const float xh = aXH[u][e], y = aY[u][e];
          const float dk = acc[e] - sEG[j] * xh;
          dkn[u][e] = dk;
          const long long rw = sRow[j];
          if (rw >= 0) p.dkt[rw * DK + d] = accw[e] + sEL[j] * y;
          const float gj = sum16(-sEG[j] * kv * xh - sEL[j] * wv * y);
          const float rd = sum16(kv * dk);
          glast = fmaf(sEL[j], wv * y, glast);
          if (col == 0) {
            atomicAdd(&sDG[j], gj);
            atomicAdd(&sRD[j], rd);
          }
        }
      } else {
        acc = mm_tile_tt<OT, RT>(acc, sGm, LDC, ct * 16, sQ, LDK, dt * 16);
        acc = mm_tile_tb<OT, C>(acc, sA, LDC, ct * 16, sK, LDK, dt * 16);
        acc = mm_tile_tt<OT, C>(acc, sA, LDC, ct * 16, sK, LDK, dt * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = ct * 16 + 4 * grp + e, d = dt * 16 + col;
          const float kv = to_f32(sK[j * LDK + d]);
          const float xh = aXH[u][e], y = aY[u][e];
          const float dk = acc[e] - sEG[j] * xh + sEL[j] * y;
          dkn[u][e] = dk;
          const float gj = sum16(-sEG[j] * kv * xh - sEL[j] * kv * y);
          const float rd = sum16(kv * dk);
          glast = fmaf(sEL[j], kv * y, glast);
          if (col == 0) {
            atomicAdd(&sDG[j], gj);
            atomicAdd(&sRD[j], rd);
          }
        }
      }
    }
  }
  glast = sum16(glast);
  glast += __shfl_xor(glast, 16);
  glast += __shfl_xor(glast, 32);
  if (lane == 0) atomicAdd(&sDG[C - 1], glast);
  __syncthreads();
  // raw-key gradient through k / max(|k|, 1e-6)
  const float rclamp = 1.f / 1e-6f;
#pragma unroll
  for (int u = 0; u < KPW; ++u) {
    const int tile = wave + 4 * u;
    if (tile < NKD) {
      const int ct = tile / NDT, dt = tile % NDT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ct * 16 + 4 * grp + e, d = dt * 16 + col;
        const long long rw = sRow[j];
        if (rw >= 0) {
          const float ri = sRinv[j];
          const float proj = ri < rclamp ? to_f32(sK[j * LDK + d]) * sRD[j] : 0.f;
          p.dk[rw * DK + d] = ri * (dkn[u][e] - proj);
        }
      }
    }
  }
  // dbeta through the clamp; dlog g = reverse cumsum of dG over the chunk
  if (wave == 0) {
    const int i = lane;
    float x = (i < C) ? sDG[i] : 0.f;
    // suffix sum over lanes i .. C-1
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off);
      if (i + off < 64) x += y;
    }
    if (i < C && sRow[i] >= 0) {
      const long long rw = sRow[i];
      const float braw = p.beta[rw];
      p.dbeta[rw] = (braw >= 0.f && braw <= 2.f) ? sDB[i] : 0.f;
      if (p.g != nullptr && p.dg != nullptr && (rw % p.n_h) == 0) {
        const long long tk = rw / p.n_h;
        const float gv = p.g[tk];
        p.dg[tk] = gv >= FLT_MIN ? x / gv : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gradient of OSDN phase 1 (OSDN study notes sec. 2.5, closing paragraph: the
// write key kt_t = d_t o kh_t passes its gradient into d_t and k_t, and the
// gradient of d runs back through the recursion of sec. 2.4, with the
// retention of sec. 2.6 and the beta-free step of sec. 2.7).  Per token, with
// s = kh o kh, n = sum s, nb = max(n, eps), a = bu <d, s>,
// coef = eta bu (1 - a) / nb, x = r d + coef s and the gradient gd' on d_{t+1}:
//   gx  = gd' where dmin <= x <= dmax (else 0)
//   gd  = r gx - (eta bu^2 / nb) <gx, s> s + kh o gkt
//   gr  = <gx, d>,   gbu = <gx, s> eta (1 - 2a) / nb
//   gs  = coef gx + <gx, s> (-(eta bu^2 / nb) d - [n > eps] coef / nb)
//   gkh = 2 kh o gs + d o gkt,  then the normalisation kh = k / max(|k|, 1e-6)
// Only gd runs through the tokens, so three launches share the work:
//   dp_precond_bwd_factors_kernel (parallel over tokens): the projection mask
//     of every (token, coordinate) and the factors (1/|k|, r, eta bu^2 / nb);
//   dp_precond_bwd_chain_kernel (sequential per head, last token first): the
//     chain alone, gx, <gx, s> (one head sum) and gd, storing the gradient each
//     token receives;
//   dp_precond_bwd_grads_kernel (parallel over tokens): the key, beta and
//     retention gradients of every token from the gradient it received.
// The lane layout is the forward's (LPH lanes per head, EPL coordinates per
// lane).  d_t comes from the trajectory the forward kernel stored.  dk and
// dbeta are accumulated into (they already hold the write-key forward's
// gradients), dret and dd0 written.
struct PrecondBwdArgs {
  const void* k;          // [B, L, H, dk] raw keys
  const float* beta;      // [B, L, H]
  const float* ret;       // [B, L, H] or nullptr
  const float* dtr;       // [B, L, H, dk] d_t of every token
  const float* dkt;       // [B, L, H, dk] gradient on the write keys
  const float* dd_final;  // [B, H, dk] or nullptr (zero)
  float* dk;              // [B, L, H, dk], accumulated into
  float* dbeta;           // [B, L, H], accumulated into
  float* dret;            // [B, L, H] or nullptr
  float* dd0;             // [B, H, dk] or nullptr
  unsigned char* msk;     // [B, L, H, dk] 1 where the token's step stays inside the box
  float4* fac;            // [B, L, H] (1/max(|k|, 1e-6), r, eta bu^2 / nb, 0)
  float* gin;             // [B, L, H, dk] the gradient on d_{t+1} that token t receives
  int B, H, L, beta_aware;
  float eta, dmin, dmax, eps;
};

constexpr int kP1Tokens = 64;  // tokens per workgroup of the two parallel kernels

// The per-token factors of the step, as the forward forms them.
template <int LPH, int EPL>
struct P1Tok {
  float kh[EPL], sq[EPL], rinv, coef, c2, fb, cn;
  bool tiny;
};
template <typename T, int LPH, int EPL>
__device__ __forceinline__ P1Tok<LPH, EPL> p1_token(const T (&k)[EPL], const float (&d)[EPL], float beta,
                                                    const PrecondBwdArgs& p) {
  P1Tok<LPH, EPL> o;
  float n2 = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) n2 = fmaf(to_f32(k[e]), to_f32(k[e]), n2);
  n2 = head_sum<LPH>(n2);
  o.rinv = __builtin_amdgcn_rsqf(fmaxf(n2, 1e-12f));  // 1 / max(|k|, 1e-6)
  o.tiny = !(n2 > 1e-12f);
  const float ns = n2 * o.rinv * o.rinv;  // |kh|^2
  float ds = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    o.kh[e] = to_f32(k[e]) * o.rinv;
    o.sq[e] = o.kh[e] * o.kh[e];
    ds = fmaf(d[e], o.sq[e], ds);
  }
  ds = head_sum<LPH>(ds);
  const float bu = p.beta_aware ? clamp_keep_nan(beta, 0.f, 2.f) : 1.f;
  const float a = bu * ds;
  const float rn = __builtin_amdgcn_rcpf(fmaxf(ns, p.eps));
  o.coef = p.eta * bu * (1.f - a) * rn;
  o.c2 = p.eta * bu * bu * rn;
  o.fb = p.eta * (1.f - 2.f * a) * rn;
  o.cn = ns > p.eps ? o.coef * rn : 0.f;
  return o;
}

// Lane geometry shared by the three kernels: HPW heads per wavefront.
template <int DK>
struct P1Lanes {
  static constexpr int LPH = DK < 64 ? DK : 64, EPL = DK / LPH, HPW = 64 / LPH;
  static_assert(EPL == 1 || EPL == 2, "coordinates per lane");
};

template <typename T, int DK>
__global__ __launch_bounds__(64) void dp_precond_bwd_factors_kernel(PrecondBwdArgs p) {
  using G = P1Lanes<DK>;
  constexpr int LPH = G::LPH, EPL = G::EPL, HPW = G::HPW;
  const int lane = threadIdx.x & 63, sl = lane % LPH;
  const int nblk = (p.L + kP1Tokens - 1) / kP1Tokens;
  const long long nbh = (long long)p.B * p.H;
  const long long bh_raw = (long long)(blockIdx.x / nblk) * HPW + lane / LPH;
  const int t0 = (int)(blockIdx.x % nblk) * kP1Tokens;
  const bool active = bh_raw < nbh;
  const long long bh = active ? bh_raw : 0;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const long long row0 = (long long)b * p.L * p.H + h, kstride = (long long)p.H * DK;
  const T* kp = static_cast<const T*>(p.k) + row0 * DK + sl * EPL;
  const float* dtp = p.dtr + row0 * DK + sl * EPL;
  const int t1 = min(t0 + kP1Tokens, p.L);
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    T kv[EPL];
    float dv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      kv[e] = kp[t * kstride + e];
      dv[e] = dtp[t * kstride + e];
    }
    const long long rw = row0 + (long long)t * p.H;
    const float r = p.ret != nullptr ? p.ret[rw] : 1.f;
    const P1Tok<LPH, EPL> f = p1_token<T, LPH, EPL>(kv, dv, p.beta[rw], p);
    if (active) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = fmaf(f.coef, f.sq[e], r * dv[e]);
        p.msk[rw * DK + sl * EPL + e] = (x >= p.dmin && x <= p.dmax) ? 1 : 0;
      }
      if (sl == 0) p.fac[rw] = make_float4(f.rinv, r, f.c2, 0.f);
    }
  }
}

template <typename T, int DK>
__global__ __launch_bounds__(64) void dp_precond_bwd_chain_kernel(PrecondBwdArgs p) {
  using G = P1Lanes<DK>;
  constexpr int LPH = G::LPH, EPL = G::EPL, HPW = G::HPW;
  constexpr int PB = 16;  // tokens per block (<= LPH: lane j of a head holds token j's factors)
  static_assert(PB <= LPH, "one factor lane per token");
  const int lane = threadIdx.x & 63, sl = lane % LPH, hl = lane - sl;
  const long long nbh = (long long)p.B * p.H;
  const long long bh_raw = (long long)blockIdx.x * HPW + lane / LPH;
  const bool active = bh_raw < nbh;
  const long long bh = active ? bh_raw : 0;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const long long row0 = (long long)b * p.L * p.H + h, kstride = (long long)p.H * DK;
  const T* kp = static_cast<const T*>(p.k) + row0 * DK + sl * EPL;
  const float* gkp = p.dkt + row0 * DK + sl * EPL;
  const unsigned char* mp = p.msk + row0 * DK + sl * EPL;
  float* gip = p.gin + row0 * DK + sl * EPL;

  float gd[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) gd[e] = p.dd_final != nullptr ? p.dd_final[bh * DK + sl * EPL + e] : 0.f;

  struct Blk {
    T k[PB][EPL];
    float gk[PB][EPL];
    unsigned char m[PB][EPL];
    float4 f;  // lane j of the head: token t0 + j's factors
  };
  auto load = [&](int t0, Blk& r) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int t = t0 + i;
      const bool ok = t < p.L;
      const long long o = (long long)(ok ? t : 0) * kstride;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        r.k[i][e] = kp[o + e];
        r.gk[i][e] = gkp[o + e];
        r.m[i][e] = mp[o + e];
      }
    }
    const int tj = t0 + (sl < PB ? sl : 0);
    r.f = p.fac[row0 + (long long)(tj < p.L ? tj : 0) * p.H];
  };
  auto run_block = [&](const Blk& c, int t0) {
#pragma unroll
    for (int i = PB - 1; i >= 0; --i) {
      const int t = t0 + i;
      if (t < p.L) {
        // token t's factors from lane i of the head: with one head per
        // wavefront a scalar read of that lane, else a lane shuffle
        float rinv, rt, c2;
        if constexpr (LPH == 64) {
          rinv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c.f.x), i));
          rt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c.f.y), i));
          c2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c.f.z), i));
        } else {
          rinv = __shfl(c.f.x, hl + i);
          rt = __shfl(c.f.y, hl + i);
          c2 = __shfl(c.f.z, hl + i);
        }
        float kh[EPL], sq[EPL], gx[EPL], gxs = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          kh[e] = to_f32(c.k[i][e]) * rinv;
          sq[e] = kh[e] * kh[e];
          gx[e] = c.m[i][e] ? gd[e] : 0.f;
          gxs = fmaf(gx[e], sq[e], gxs);
        }
        gxs = head_sum<LPH>(gxs);
        if (active) {
          if constexpr (EPL == 2)
            *reinterpret_cast<float2*>(gip + t * kstride) = make_float2(gd[0], gd[1]);
          else
            gip[t * kstride] = gd[0];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) gd[e] = fmaf(rt, gx[e], fmaf(-c2 * gxs, sq[e], kh[e] * c.gk[i][e]));
      }
    }
  };
  // Two register sets, each loaded one block ahead of its use, and the loop
  // over pairs of blocks: every load is issued on every path (the last one
  // clamped to block 0) and no loaded set is copied, so the compiler counts
  // the loads in flight exactly and waits only for the block it runs.
  const int nblk = (p.L + PB - 1) / PB;
  Blk ba, bb;
  int blk = nblk - 1;
  if (nblk > 0) load(blk * PB, ba);
  for (; blk >= 1; blk -= 2) {
    load((blk - 1) * PB, bb);  // lands while block blk runs
    run_block(ba, blk * PB);
    load(max(blk - 2, 0) * PB, ba);
    run_block(bb, (blk - 1) * PB);
  }
  if (blk == 0) run_block(ba, 0);
  if (active && p.dd0 != nullptr) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) p.dd0[bh * DK + sl * EPL + e] = gd[e];
  }
}

template <typename T, int DK>
__global__ __launch_bounds__(64) void dp_precond_bwd_grads_kernel(PrecondBwdArgs p) {
  using G = P1Lanes<DK>;
  constexpr int LPH = G::LPH, EPL = G::EPL, HPW = G::HPW;
  const int lane = threadIdx.x & 63, sl = lane % LPH;
  const int nblk = (p.L + kP1Tokens - 1) / kP1Tokens;
  const long long nbh = (long long)p.B * p.H;
  const long long bh_raw = (long long)(blockIdx.x / nblk) * HPW + lane / LPH;
  const int t0 = (int)(blockIdx.x % nblk) * kP1Tokens;
  const bool active = bh_raw < nbh;
  const long long bh = active ? bh_raw : 0;
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  const long long row0 = (long long)b * p.L * p.H + h, kstride = (long long)p.H * DK;
  const long long c0 = row0 * DK + sl * EPL;
  const T* kp = static_cast<const T*>(p.k) + c0;
  const int t1 = min(t0 + kP1Tokens, p.L);
#pragma unroll 2
  for (int t = t0; t < t1; ++t) {
    const long long o = (long long)t * kstride;
    T kv[EPL];
    float dv[EPL], gk[EPL], gi[EPL], dk0[EPL];
    bool in[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      kv[e] = kp[o + e];
      dv[e] = p.dtr[c0 + o + e];
      gk[e] = p.dkt[c0 + o + e];
      gi[e] = p.gin[c0 + o + e];
      dk0[e] = p.dk[c0 + o + e];
      in[e] = p.msk[c0 + o + e] != 0;
    }
    const long long rw = row0 + (long long)t * p.H;
    const float braw = p.beta[rw];
    const P1Tok<LPH, EPL> f = p1_token<T, LPH, EPL>(kv, dv, braw, p);
    float gx[EPL], gxs = 0.f, gr = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      gx[e] = in[e] ? gi[e] : 0.f;
      gxs = fmaf(gx[e], f.sq[e], gxs);
      gr = fmaf(gx[e], dv[e], gr);
    }
    gxs = head_sum<LPH>(gxs);
    if (p.dret != nullptr) gr = head_sum<LPH>(gr);
    float gkh[EPL], pp = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float gs = fmaf(f.coef, gx[e], gxs * fmaf(-f.c2, dv[e], -f.cn));
      gkh[e] = fmaf(2.f * f.kh[e], gs, dv[e] * gk[e]);
      pp = fmaf(f.kh[e], gkh[e], pp);
    }
    pp = head_sum<LPH>(pp);
    if (active) {
      const float proj = f.tiny ? 0.f : pp;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p.dk[c0 + o + e] = dk0[e] + (gkh[e] - f.kh[e] * proj) * f.rinv;
      if (sl == 0) {
        if (p.beta_aware && braw >= 0.f && braw <= 2.f) p.dbeta[rw] += gxs * f.fb;
        if (p.dret != nullptr) p.dret[rw] = p.ret != nullptr ? gr : 0.f;
      }
    }
  }
}

template <typename T, int DK>
hipError_t launch_precond_bwd_dk(const PrecondBwdArgs& a, hipStream_t st) {
  using G = P1Lanes<DK>;
  const long long nbh = (long long)a.B * a.H;
  const unsigned groups = (unsigned)((nbh + G::HPW - 1) / G::HPW);
  const unsigned nblk = (unsigned)((a.L + kP1Tokens - 1) / kP1Tokens);
  if (groups == 0) return hipSuccess;
  if (nblk > 0) {
    hipLaunchKernelGGL((dp_precond_bwd_factors_kernel<T, DK>), dim3(groups * nblk), dim3(64), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dp_precond_bwd_chain_kernel<T, DK>), dim3(groups), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nblk == 0) return e;
  hipLaunchKernelGGL((dp_precond_bwd_grads_kernel<T, DK>), dim3(groups * nblk), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launch of the four kernels.
template <typename T, int DK, int BVS, int NRT, bool ASYM>
hipError_t launch_bwd_scans(const BwdArgs& a, hipStream_t st) {
  using OT = typename OpType<T>::type;
  constexpr int C = kBwdChunk;
  constexpr int l1 = bwd_dstate_lds_bytes<OT, DK, C, kBwdBV, 16 * NRT, ASYM>();
  constexpr int l2 = bwd_states_lds_bytes<T, DK, C, BVS, ASYM>();
  constexpr int lds = l1 > l2 ? l1 : l2;
  static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_bwd_scans_kernel<T, DK, C, BVS, NRT, ASYM>));
  (void)attr;
  const unsigned nwg = (unsigned)(a.B * a.H * (a.nvb + a.dvd / BVS));
  hipLaunchKernelGGL((dp_bwd_scans_kernel<T, DK, C, BVS, NRT, ASYM>), dim3(nwg), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <typename T, int DK, bool ASYM>
hipError_t launch_bwd_form(const FwdArgs& fa, const BwdArgs& a, hipStream_t st) {
  constexpr int C = kBwdChunk;
  const long long nchunks = (long long)a.B * a.H * a.nc;
  if (nchunks > 0) {
    const int lds = ut_lds_bytes((int)sizeof(T), DK, C, ASYM);
    static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_ut_kernel<T, DK, C, float, false>));
    (void)attr;
    hipLaunchKernelGGL((dp_ut_kernel<T, DK, C, float, false>), dim3((unsigned)nchunks), dim3(kThreads), lds, st, fa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.B * a.H * a.nvb > 0) {
    // the chunk-start states in blocks of 32 value columns where dv allows
    hipError_t e;
    if (a.dvd >= 32)
      e = a.RT == 16 ? launch_bwd_scans<T, DK, 32, 1, ASYM>(a, st) : launch_bwd_scans<T, DK, 32, 2, ASYM>(a, st);
    else
      e = a.RT == 16 ? launch_bwd_scans<T, DK, 16, 1, ASYM>(a, st) : launch_bwd_scans<T, DK, 16, 2, ASYM>(a, st);
    if (e != hipSuccess) return e;
  }
  if (nchunks > 0) {
    if (a.RT == 16) {
      static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_bwd_chunk_kernel<T, DK, C, 1, ASYM>));
      (void)attr;
      constexpr int lds = bwd_chunk_lds_bytes<typename OpType<T>::type, DK, C, 16, ASYM>();
      hipLaunchKernelGGL((dp_bwd_chunk_kernel<T, DK, C, 1, ASYM>), dim3((unsigned)nchunks), dim3(256), lds, st, a);
    } else {
      static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_bwd_chunk_kernel<T, DK, C, 2, ASYM>));
      (void)attr;
      constexpr int lds = bwd_chunk_lds_bytes<typename OpType<T>::type, DK, C, 32, ASYM>();
      hipLaunchKernelGGL((dp_bwd_chunk_kernel<T, DK, C, 2, ASYM>), dim3((unsigned)nchunks), dim3(256), lds, st, a);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int DK>
hipError_t launch_bwd_dk(const FwdArgs& fa, const BwdArgs& a, hipStream_t st) {
  return a.kt != nullptr ? launch_bwd_form<T, DK, true>(fa, a, st) : launch_bwd_form<T, DK, false>(fa, a, st);
}

}  // namespace dp

#define DP_DEFINE_BWD_LAUNCHER(T, TNAME, DK)                                                     \
  hipError_t dp_launch_bwd_##TNAME##_##DK(const dp::FwdArgs& fa, const dp::BwdArgs& a, hipStream_t st) { \
    return dp::launch_bwd_dk<T, DK>(fa, a, st);                                                  \
  }                                                                                              \
  hipError_t dp_launch_precond_bwd_##TNAME##_##DK(const dp::PrecondBwdArgs& a, hipStream_t st) {  \
    return dp::launch_precond_bwd_dk<T, DK>(a, st);                                              \
  }
#define DP_DECLARE_BWD_LAUNCHER(TNAME, DK)                                                                 \
  hipError_t dp_launch_bwd_##TNAME##_##DK(const dp::FwdArgs& fa, const dp::BwdArgs& a, hipStream_t st); \
  hipError_t dp_launch_precond_bwd_##TNAME##_##DK(const dp::PrecondBwdArgs& a, hipStream_t st);
