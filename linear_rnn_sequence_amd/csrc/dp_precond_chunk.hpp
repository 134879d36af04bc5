// dp_precond_chunk.hpp -- OSDN phase 1 in 64-token chunks (gfx950).
//
// Phase 1 (OSDN study notes sec. 2.4, Alg.1, with the retention of sec. 2.6
// and the beta-free step of sec. 2.7) is, per head and token t,
//   kt_t = d_t o kh_t,  a_t = <d_t, s_t>,  s_t = kh_t o kh_t,
//   d_{t+1} = P[ r_t d_t + (w_t - c2_t a_t) s_t ],
// w_t = eta bu_t / max(|kh_t|^2, eps), c2_t = bu_t w_t.  While the projection P
// onto the box leaves every coordinate alone the step is linear in d (the
// notes: affine without the clamp, piecewise affine with it).  Over a chunk
// of T tokens from d_0, with G_t the cumulative log-retention before token t:
//   d_t = e^{G_t} d_0 + sum_{u<t} e^{G_t - G_{u+1}} (w_u - c2_u a_u) s_u,
//   (I + L diag(c2)) a = e^G o (S d_0) + L w,   L_tu = e^{G_t - G_{u+1}} <s_t, s_u>  (u < t)
// The matrix depends on the keys, beta and r only, so it is inverted for every
// chunk in parallel (dp_p1_ut_kernel); the sequential part per head is then
// three small products per chunk (dp_p1_chain_kernel): p = S d_0, a = Tm
// (e^G o p) + v, and the end-of-chunk d.  dp_p1_emit_kernel replays each
// chunk coordinate by coordinate from its start d (a_t known), emits the write
// keys and checks that no step came within a margin of the box (or is NaN).
// A head whose check fails anywhere runs the exact sequential scan again from
// the first such chunk's start (dp_precond_kernel with PrecondArgs::restart),
// so the result is the sequential definition's whichever way it is reached.
// The notes state phase 1's depth as the sequence length; this form keeps that
// definition and only shortens the work on the sequential path while no
// clamp binds.  Used for dk >= 64 (one head per wavefront in the fallback).
#pragma once

namespace dp {

constexpr int kP1Chunk = 64;  // tokens per chunk
constexpr int kP1Ld = kP1Chunk + 4;

// N (4 or 8) values as fp16 at p (8 or 16 bytes, aligned to that)
template <int N>
__device__ __forceinline__ void st_f16s(f16_t* p, const float* f) {
  if constexpr (N == 8) {
    st_vec16(p, f);
  } else {
    f16x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (f16_t)f[i];
    *reinterpret_cast<f16x4_t*>(p) = v;
  }
}

// --------------------------------------------------------------------------
// dp_p1_ut_kernel: one workgroup per (head, chunk), all in parallel.
// Where a head's chunks live.  Fixed length: B H heads of L tokens, nc =
// ceil(L / C) chunks each, chunk c of head bh at bh nc + c.  Packed sequences
// (p.cu; p.cbase from dp_varlen_chunks_kernel with n_h = 1): sequence s has
// cbase[s+1] - cbase[s] chunks per head, stored head by head from cbase[s] H.
// All-zero offsets (what that kernel leaves for malformed cu) make every
// sequence empty.
struct P1Head {
  long long row0;  // token-major row of the head's first token
  long long blk0;  // its first chunk in the per-chunk arrays
  int L, nc;       // its tokens and chunks
};
__device__ __forceinline__ P1Head p1_head(const PrecondArgs& p, long long bh) {
  const int b = (int)(bh / p.H), h = (int)(bh % p.H);
  P1Head g;
  if (p.cu == nullptr) {
    g.L = p.L;
    g.nc = (p.L + kP1Chunk - 1) / kP1Chunk;
    g.row0 = tok_base(p, b) * p.H + h;
    g.blk0 = bh * g.nc;
  } else {
    g.nc = p.cbase[b + 1] - p.cbase[b];
    g.L = g.nc > 0 ? p.cu[b + 1] - p.cu[b] : 0;
    g.row0 = (g.nc > 0 ? (long long)p.cu[b] : 0ll) * p.H + h;
    g.blk0 = (long long)p.cbase[b] * p.H + (long long)h * g.nc;
  }
  return g;
}
// Work item w of the per-chunk kernels -> head bh and chunk c; false past the
// last chunk (packed: the grid is an upper bound).
__device__ __forceinline__ bool p1_item(const PrecondArgs& p, long long w, long long& bh, int& c) {
  if (p.cu == nullptr) {
    const int nc = (p.L + kP1Chunk - 1) / kP1Chunk;
    bh = w / nc;
    c = (int)(w % nc);
    return true;
  }
  if (w >= (long long)p.cbase[p.B] * p.H) return false;
  // the last sequence s with cbase[s] H <= w; it has chunks, since cbase[s+1] H > w
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)p.cbase[mid] * p.H <= w) lo = mid; else hi = mid - 1;
  }
  const int ncs = p.cbase[lo + 1] - p.cbase[lo];
  const long long rel = w - (long long)p.cbase[lo] * p.H;
  bh = (long long)lo * p.H + rel / ncs;
  c = (int)(rel % ncs);
  return true;
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void dp_p1_ut_kernel(PrecondArgs p) {
  constexpr int C = kP1Chunk, LDM = kP1Ld, NT = C / 16;
  constexpr int VE = Vec<T>::N;
  constexpr int TPR = DK / VE;   // 16-byte granules per key row
  constexpr int KV = C * TPR, KIT = (KV + 255) / 256;
  static_assert(TPR <= 64 && 64 % TPR == 0, "row group must fit in a wavefront");
  // The squared unit keys s, scaled by 2^10 (into fp16's normal range), as
  // fp16 pairs hi + lo: the Gram matrix is hi hi' + hi lo' + lo hi' on fp16
  // MFMA (the dropped lo lo' is 2^-22 of a term: fp32 accuracy).  They are
  // dead once the Gram tiles are in registers: M, Tm and the inverse's
  // scratch take their place (about 40 KB in all: four workgroups per CU).
  constexpr int LDH = DK + 8;  // fp16 row stride (16-byte rows)
  constexpr int NMT = 2 * C * LDM + 4 * 16 * 17;
  constexpr int NBIG = C * LDH > NMT ? C * LDH : NMT;  // floats
  __shared__ __align__(16) float sBig[NBIG];
  f16_t* const sSh = reinterpret_cast<f16_t*>(sBig);
  f16_t* const sSl = sSh + C * LDH;
  float* const sTm = sBig;
  float* const sM = sBig + C * LDM;
  float* const sSc = sBig + 2 * C * LDM;
  __shared__ float sN[C], sRinv[C], sW[C], sC2[C], sG[C + 1], sLw[C];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  long long bh;
  int c;
  if (!p1_item(p, blockIdx.x, bh, c)) return;
  const P1Head hg = p1_head(p, bh);
  const long long chunk = hg.blk0 + c;
  const long long row0 = hg.row0;
  const int L = hg.L;
  const int t0 = c * C;
  const T* kp = static_cast<const T*>(p.k);

  // 1. key rows -> squared unit keys (fp16 pairs) and the row norms
  u32x4_t rk[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * 256;
    const int r = idx / TPR, cg = idx % TPR;
    rk[it] = u32x4_t{0u, 0u, 0u, 0u};
    if (idx < KV && t0 + r < L) rk[it] = ld16(kp + (row0 + (long long)(t0 + r) * p.H) * DK + cg * VE);
  }
  float braw = 0.f, rr = 1.f;
  if (tid < C && t0 + tid < L) {
    const long long rw = row0 + (long long)(t0 + tid) * p.H;
    braw = p.beta[rw];
    if (p.ret != nullptr) rr = p.ret[rw];
  }
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + it * 256;
    const int r = idx / TPR, cg = idx % TPR;
    float f[VE];
    unpack16(rk[it], f, T{});
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) ss = fmaf(f[e], f[e], ss);
    if constexpr (TPR <= 16)
      ss = dpp_group_sum<TPR>(ss);
    else
      ss = group_sum<TPR>(ss);
    const float rinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f));  // 1 / max(|k|, 1e-6)
    if (idx < KV) {
      float hi[VE], lo[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float a = f[e] * rinv;
        const float sc = a * a * 1024.f;
        hi[e] = (float)(f16_t)sc;
        lo[e] = sc - hi[e];
      }
      st_f16s<VE>(sSh + r * LDH + cg * VE, hi);
      st_f16s<VE>(sSl + r * LDH + cg * VE, lo);
      if (cg == 0) {
        sN[r] = ss * rinv * rinv;  // |kh|^2, as the sequential scan forms it
        sRinv[r] = rinv;
      }
    }
  }
  __syncthreads();
  // 2. per-token factors and the cumulative log-retention (G_0 = 0)
  if (wave == 0) {
    const bool ok = lane < C && t0 + lane < L;
    float w = 0.f, c2 = 0.f, lr = 0.f;
    if (ok) {
      const float bu = p.beta_aware ? clamp_keep_nan(braw, 0.f, 2.f) : 1.f;
      w = p.eta * bu * __builtin_amdgcn_rcpf(fmaxf(sN[lane], p.eps));
      c2 = bu * w;
      lr = logf(fmaxf(rr, FLT_MIN));
    }
    const float incl = wave_inclusive_scan(lr);
    if (lane < C) {
      sW[lane] = w;
      sC2[lane] = c2;
      sG[lane] = incl - lr;
    }
    if (lane == C - 1) sG[C] = incl;
  }
  __syncthreads();
  // 3. L (gated Gram matrix of the squared keys, strictly lower): wave w forms
  //    the tiles of column block w in registers, then (once no wave reads the
  //    keys any more) writes them over the keys' space
  static_assert(NT == 4, "one column block of tiles per wave");
  f32x4_t acc[NT];
#pragma unroll
  for (int ti = 0; ti < NT; ++ti) {
    acc[ti] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (wave <= ti) {
      acc[ti] = mm_tile<f16_t, DK>(acc[ti], sSh, LDH, ti * 16, sSh, LDH, wave * 16);
      acc[ti] = mm_tile<f16_t, DK>(acc[ti], sSh, LDH, ti * 16, sSl, LDH, wave * 16);
      acc[ti] = mm_tile<f16_t, DK>(acc[ti], sSl, LDH, ti * 16, sSh, LDH, wave * 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int ti = 0; ti < NT; ++ti) {
    const int u = wave * 16 + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = ti * 16 + 4 * grp + e;
      sM[t * LDM + u] = (u < t) ? __expf(sG[t] - sG[u + 1]) * (acc[ti][e] * 0x1p-20f) : 0.f;
    }
  }
  __syncthreads();
  // L w, and M = L diag(c2) in place: four threads per row, each a quarter of it
  {
    const int t = tid >> 2, q = tid & 3;
    float lw = 0.f;
#pragma unroll
    for (int u = q * (C / 4); u < (q + 1) * (C / 4); ++u) {
      const float l = sM[t * LDM + u];
      lw = fmaf(l, sW[u], lw);
      sM[t * LDM + u] = l * sC2[u];
    }
    lw += __shfl_xor(lw, 1);
    lw += __shfl_xor(lw, 2);
    if (q == 0) sLw[t] = lw;
  }
  __syncthreads();
  // 4. Tm = (I + M)^{-1}: diagonal 16 x 16 blocks by forward substitution (one
  //    16-lane group per block, one column per lane), then the off-diagonal
  //    blocks level by level, Tm_ij = -Tm_ii sum_{k=j}^{i-1} M_ik Tm_kj
  if (wave == 0) {
    const int gb = lane >> 4, cc = lane & 15;
    if (gb < NT) {
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == cc) ? 1.f : 0.f;
        const float* ar = sM + (gb * 16 + i) * LDM + gb * 16;
#pragma unroll
        for (int j = 0; j < i; ++j) acc = fmaf(-ar[j], t[j], acc);
        t[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTm[(gb * 16 + i) * LDM + gb * 16 + cc] = t[i];
    }
  }
  // the upper blocks of Tm are zero
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx / C, j = idx % C;
    if ((j >> 4) > (i >> 4)) sTm[i * LDM + j] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int dist = 1; dist < NT; ++dist) {
    const int j = wave, i = wave + dist;
    float* sX = sSc + wave * 16 * 17;
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb)
        acc = mm_tile_tb<float, 16>(acc, sM + i * 16 * LDM + kb * 16, LDM, 0, sTm + kb * 16 * LDM + j * 16, LDM, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(4 * grp + e) * 17 + col] = acc[e];
    }
    __syncthreads();
    if (i < NT) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mm_tile_tb<float, 16>(acc, sTm + i * 16 * LDM + i * 16, LDM, 0, sX, 17, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sTm[(i * 16 + 4 * grp + e) * LDM + j * 16 + col] = -acc[e];
    }
    __syncthreads();
  }
  // 5. outputs: Tm, v = Tm (L w), the per-token factors and the chunk's total log-retention
  float* tm = p.wsTm + chunk * C * C;
  for (int idx = tid; idx < C * C / 4; idx += 256) {
    const int i = (4 * idx) / C, j = (4 * idx) % C;
    *reinterpret_cast<float4*>(tm + 4 * idx) = *reinterpret_cast<const float4*>(sTm + i * LDM + j);
  }
  {  // v_t = sum_u Tm_tu (L w)_u: four threads per row
    const int t = tid >> 2, q = tid & 3;
    float v = 0.f;
#pragma unroll
    for (int u = q * (C / 4); u < (q + 1) * (C / 4); ++u) v = fmaf(sTm[t * LDM + u], sLw[u], v);
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    if (q == 0) p.wsV[chunk * C + t] = v;
  }
  if (tid < C) p.wsFac[chunk * C + tid] = make_float4(sRinv[tid], sW[tid], sC2[tid], sG[tid]);
  if (tid == 0) p.wsGT[chunk] = sG[C];
}

// --------------------------------------------------------------------------
// dp_p1_chain_kernel: one workgroup per head, sequential over its chunks.  The
// chunk's squared unit keys and Tm stay in registers where they were loaded
// (a row group of DK / (16 / sizeof(T)) lanes per key row, 16 lanes per Tm
// row); the products are lane partials summed within the group by DPP, and
// the end-of-chunk d sums the row groups' partials through LDS.  Its barriers
// order LDS only, so the loads of the chunk after next stay in flight; every
// global load and store in the loop is issued by every lane on every path
// (clamped addresses, duplicate stores of equal values), so the compiler
// counts the loads in flight exactly and waits only for the ones it uses.
template <typename T, int DK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dp_p1_chain_kernel(PrecondArgs p) {
  constexpr int C = kP1Chunk;
  constexpr int VE = Vec<T>::N;
  constexpr int TPR = DK / VE;           // lanes per key row
  constexpr int KIT = C * TPR / 256;     // key rows per thread
  constexpr int RPI = 256 / TPR;         // key rows per pass of the workgroup (row groups)
  constexpr int TMIT = C * C / 4 / 256;  // Tm rows per thread (four values each)
  static_assert(C * TPR == 256 * KIT && TMIT == 4 && TPR <= 64 && 64 % TPR == 0, "thread layout");
  __shared__ __align__(16) float sPart[RPI * DK];
  __shared__ __align__(16) float sRhs[C];
  __shared__ float sD[DK], sCoef[C], sW[C], sC2[C], sG[C + 1], sV[C];

  const int tid = threadIdx.x, cg = tid % TPR, rg = tid / TPR;
  const long long bh = blockIdx.x;
  const P1Head hg = p1_head(p, bh);
  const int nc = hg.nc, L = hg.L;
  const long long row0 = hg.row0;
  const T* kp = static_cast<const T*>(p.k);

  // a chunk's operands in registers: two sets, loaded two chunks ahead of use
  struct Stage {
    u32x4_t rk[KIT];    // key granule of rows rg + RPI it
    float4 rf[KIT];     // their factors (1/|k|, w, c2, G)
    float4 rtm[TMIT];   // Tm row tid / 16 + 16 it, columns 4 (tid % 16) ..
    float4 rfac;        // factors of row tid (tid < C)
    float rv, rgt;
  };
  auto prefetch = [&](Stage& S, int c) {  // 0 <= c < nc
    const long long chunk = hg.blk0 + c;
    const int t0 = c * C;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int r = rg + RPI * it;
      const int tr = min(t0 + r, L - 1);  // rows past the end: loaded in bounds, then zeroed
      const u32x4_t v = ld16(kp + (row0 + (long long)tr * p.H) * DK + cg * VE);
      const bool in = t0 + r < L;
      S.rk[it] = u32x4_t{in ? v[0] : 0u, in ? v[1] : 0u, in ? v[2] : 0u, in ? v[3] : 0u};
      S.rf[it] = p.wsFac[chunk * C + r];
    }
#pragma unroll
    for (int it = 0; it < TMIT; ++it)
      S.rtm[it] = reinterpret_cast<const float4*>(p.wsTm + chunk * C * C)[tid + it * 256];
    S.rfac = p.wsFac[chunk * C + (tid & (C - 1))];
    S.rv = p.wsV[chunk * C + (tid & (C - 1))];
    S.rgt = p.wsGT[chunk];
  };

  if (tid < DK) sD[tid] = p.d_ones ? 1.f : p.d[bh * DK + tid];
  if (tid == 0) p.restart[bh] = nc;
  auto body = [&](Stage& S, int c) {
    const long long chunk = hg.blk0 + c;
    block_sync_lds();  // d of this chunk's start is in sD; the last chunk's reads are done
    if (tid < C) {
      sW[tid] = S.rfac.y;
      sC2[tid] = S.rfac.z;
      sG[tid] = S.rfac.w;
      sV[tid] = S.rv;
    }
    if (tid == 0) sG[C] = S.rgt;
    p.dstart[chunk * DK + tid % DK] = sD[tid % DK];
    // the squared unit keys of this thread's rows and columns
    float sv[KIT][VE];
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      float f[VE];
      unpack16(S.rk[it], f, T{});
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float a = f[e] * S.rf[it].x;
        sv[it][e] = a * a;
      }
    }
    float dv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) dv[e] = sD[cg * VE + e];
    // p_t = <s_t, d_0>, rhs_t = e^{G_t} p_t
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc = fmaf(sv[it][e], dv[e], acc);
      if constexpr (TPR <= 16)
        acc = dpp_group_sum<TPR>(acc);
      else
        acc = group_sum<TPR>(acc);
      if (cg == 0) sRhs[rg + RPI * it] = __expf(S.rf[it].w) * acc;
    }
    block_sync_lds();
    // a = Tm rhs + v;  gamma = w - c2 a;  coef_u = e^{G_C - G_{u+1}} gamma_u
    {
      const float4 rh = reinterpret_cast<const float4*>(sRhs)[tid & 15];
#pragma unroll
      for (int it = 0; it < TMIT; ++it) {
        const float4 tm = S.rtm[it];
        float x = fmaf(tm.x, rh.x, fmaf(tm.y, rh.y, fmaf(tm.z, rh.z, tm.w * rh.w)));
        x = dpp_group_sum<16>(x);
        const int i = (tid >> 4) + 16 * it;
        // every lane of the row's group holds the sum: all store the same values
        const float gm = fmaf(-sC2[i], x + sV[i], sW[i]);
        p.gam[chunk * C + i] = gm;
        sCoef[i] = __expf(sG[C] - sG[i + 1]) * gm;
      }
    }
    prefetch(S, min(c + 2, nc - 1));  // lands while this chunk and the next are computed
    block_sync_lds();
    // d_C = e^{G_C} d_0 + sum_u coef_u s_u: each row group's partial, then their sum
    {
      float part[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) part[e] = 0.f;
#pragma unroll
      for (int it = 0; it < KIT; ++it) {
        const float cf = sCoef[rg + RPI * it];
#pragma unroll
        for (int e = 0; e < VE; ++e) part[e] = fmaf(cf, sv[it][e], part[e]);
      }
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(sPart + rg * DK + cg * VE + e) =
            make_float4(part[e], part[e + 1], part[e + 2], part[e + 3]);
    }
    block_sync_lds();
    if (tid < DK) {
      float x = __expf(sG[C]) * sD[tid];
#pragma unroll 8
      for (int q = 0; q < RPI; ++q) x += sPart[q * DK + tid];
      sD[tid] = x;
    }
  };
  Stage sa, sb;
  if (nc > 0) {
    prefetch(sa, 0);
    __builtin_amdgcn_sched_barrier(0);  // the second set's loads after all of the first's, as in the loop
    prefetch(sb, min(1, nc - 1));
  }
  // pairs of chunks, then an odd last one (the loop's back edge follows the
  // second set's chunk only, so the wait counts at its head are exact)
  int c = 0;
  for (; c + 1 < nc; c += 2) {
    body(sa, c);
    body(sb, c + 1);
  }
  if (c < nc) body(sa, c);
  block_sync_lds();
  if (tid < DK) p.d[bh * DK + tid] = sD[tid];
}

// --------------------------------------------------------------------------
// dp_p1_emit_kernel: one workgroup per (head, chunk), all in parallel; thread j
// replays coordinate j of the chunk from its start d with the solved a_t,
// emits the write keys (and d_t when asked), and checks every step against
// the box with a margin.  A failing chunk marks its head for the exact scan.
// The chunk's keys and factors are staged in LDS first (one memory round trip).
template <typename T, int DK>
__global__ __launch_bounds__(DK) void dp_p1_emit_kernel(PrecondArgs p) {
  constexpr int C = kP1Chunk;
  constexpr int VE = Vec<T>::N;
  constexpr int TPR = DK / VE, KV = C * TPR, KIT = (KV + DK - 1) / DK;
  __shared__ __align__(16) T sK[C * DK];
  __shared__ float4 sFac[C];
  __shared__ float sGam[C], sR[C];
  const int j = threadIdx.x;
  long long bh;
  int c;
  if (!p1_item(p, blockIdx.x, bh, c)) return;
  const P1Head hg = p1_head(p, bh);
  const long long chunk = hg.blk0 + c;
  const long long row0 = hg.row0;
  const int t0 = c * C, n = min(C, hg.L - t0);
  const long long ks = (long long)p.H * DK;
  const T* kp = static_cast<const T*>(p.k) + (row0 + (long long)t0 * p.H) * DK;
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = j + it * DK;
    const int r = idx / TPR, cg = idx % TPR;
    if (idx < KV && r < n) st16(sK + r * DK + cg * VE, ld16(kp + r * ks + cg * VE));
  }
  if (j < n) {
    sFac[j] = p.wsFac[chunk * C + j];
    sGam[j] = p.gam[chunk * C + j];
    sR[j] = p.ret != nullptr ? p.ret[row0 + (long long)(t0 + j) * p.H] : 1.f;
  }
  float d = p.dstart[chunk * DK + j];
  __syncthreads();
  T* ktp = static_cast<T*>(p.kt) + (row0 + (long long)t0 * p.H) * DK + j;
  float* dtp = p.dtr != nullptr ? p.dtr + (row0 + (long long)t0 * p.H) * DK + j : nullptr;
  // a step within this margin of a finite bound is not trusted to the chunked form
  // (an infinite bound keeps no margin: -inf + inf would be NaN and fail every step)
  const float lo = isfinite(p.dmin) ? p.dmin + 1e-5f * fmaxf(1.f, fabsf(p.dmin)) : p.dmin;
  const float hi = isfinite(p.dmax) ? p.dmax - 1e-5f * fmaxf(1.f, fabsf(p.dmax)) : p.dmax;
  bool ok = true;
#pragma unroll 8
  for (int i = 0; i < n; ++i) {
    const float kh = to_f32(sK[i * DK + j]) * sFac[i].x;
    ktp[i * ks] = from_f32<T>(d * kh);
    if (dtp != nullptr) dtp[i * ks] = d;
    const float x = fmaf(sGam[i], kh * kh, sR[i] * d);
    ok = ok && (x >= lo && x <= hi);
    d = x;
  }
  if (__any(!ok) && (j & 63) == 0) atomicMin(&p.restart[bh], c);
}

template <typename T, int DK>
hipError_t launch_precond_chunked(const PrecondArgs& a, hipStream_t st) {
  static_assert(DK >= 64, "the exact fallback runs one head per wavefront");
  const long long nbh = (long long)a.B * a.H;
  if (nbh == 0) return hipSuccess;
  // per-chunk work items: every chunk of every head (packed: an upper bound,
  // ceil(L / C) + B chunks per head, the extra items exit)
  long long nwork = nbh * ((a.L + kP1Chunk - 1) / kP1Chunk);
  if (a.cu != nullptr) {
    hipLaunchKernelGGL((dp_varlen_chunks_kernel<kP1Chunk>), dim3(1), dim3(256), 0, st, a.cu, a.B, 1, a.L,
                       a.cbase);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    nwork = (long long)a.H * ((a.L + kP1Chunk - 1) / kP1Chunk + a.B);
  }
  if (nwork > 0) {
    hipLaunchKernelGGL((dp_p1_ut_kernel<T, DK>), dim3((unsigned)nwork), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dp_p1_chain_kernel<T, DK>), dim3((unsigned)nbh), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nwork == 0) return e;
  hipLaunchKernelGGL((dp_p1_emit_kernel<T, DK>), dim3((unsigned)nwork), dim3(DK), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the exact scan from the first chunk that failed the check (heads with none return at once)
  hipLaunchKernelGGL((dp_precond_kernel<T, DK>), dim3((unsigned)nbh), dim3(64), 0, st, a);
  return hipGetLastError();
}

// dk < 64 has no chunked form (several heads share a wavefront in the exact scan)
template <typename T, int DK>
hipError_t launch_precond_chunked_if(const PrecondArgs& a, hipStream_t st) {
  if constexpr (DK >= 64)
    return launch_precond_chunked<T, DK>(a, st);
  else
    return hipErrorInvalidValue;
}

}  // namespace dp
