// dp_decode.hpp -- one recurrent decode step of DeltaProduct on gfx950.
//
// Every head applies one token's n_h ordered generalized-Householder
// sub-steps to its resident fp32 state and reads the state out
// (DeltaProduct study notes, arXiv 2502.10297v7: sec. 2.2 Eq.(3), the
// per-token pseudocode of sec. 2.6 with its optional gate, applied once
// before the first sub-step; the asymmetric write key of the OSDN study
// notes, arXiv 2605.13473v1, sec. 2.2 Eqs.(2)/(5), and its KDA host's
// per-key-channel decay, sec. 2.7):
//
//   H <- g H, H <- Diag(alpha) H               (when the gates are given)
//   for j < n_h:  e = v_j - H^T kn_j,   H <- H + clamp(b_j, 0, 2) kw_j e^T
//   o = H^T q
//
// with kn_j = k_j / max(|k_j|, 1e-6) and kw_j = kn_j, or the write key as
// given.  This is the plain sequential definition, not the chunkwise form:
// one token has no intra-chunk parallelism to exploit, and the cost is the
// state's round trip through HBM (2 dk dv 4 bytes per head), so the kernel
// is laid out for that stream.
//
// Layout of work: a workgroup owns one head and CW consecutive value columns
// (CW = min(dv, 64)); each of its 256 or 512 threads holds one column of RP
// consecutive state rows in registers, so every load and store of a row of
// the state is one contiguous CW * 4-byte segment per wavefront.  The column
// sums H^T k and H^T q reduce the threads' row partials through LDS (one
// barrier each, alternating two buffers).
#pragma once

namespace dp {

struct DecodeArgs {
  const void* q;    // [B, H, dk]        T
  const void* k;    // [B, H, n_h, dk]   T (raw keys)
  const void* kt;   // [B, H, n_h, dk]   T write keys, or nullptr
  const void* v;    // [B, H, n_h, dv]   T
  const float* beta;  // [B, H, n_h]
  const float* g;     // [B, H] or nullptr
  const float* ga;    // [B, H, dk] per-key-channel gate or nullptr
  void* out;          // [B, H, dv]      T, or fp32 when out_f32
  float* state;       // [B, H, dk, dv]  in/out
  int B, H, n_h, dv, out_f32;
};

// Threads per workgroup: 512 where the head slice holds at least 512 state
// elements (16 rows of a column per thread at dk = 128, CW = 64), else 256.
__host__ __device__ constexpr int decode_threads(int dk, int cw) { return dk * cw >= 512 ? 512 : 256; }

// LDS floats of dp_decode_kernel: read keys and write keys (n_h x DK each),
// q (DK), the block's value columns (n_h x CW), 1/|k| and beta (n_h each),
// two reduction buffers (one float per thread each).
__host__ __device__ constexpr int decode_lds_floats(int dk, int cw, int n_h, int asym) {
  return n_h * dk * (1 + asym) + dk + n_h * cw + 2 * n_h + 2 * decode_threads(dk, cw);
}

template <typename T, int DK, int CW>
__global__ __launch_bounds__(512) void dp_decode_kernel(DecodeArgs p) {
  constexpr int NTH = decode_threads(DK, CW);
  constexpr int NRG = NTH / CW;  // row groups
  constexpr int RP = DK / NRG;              // state rows per thread
  static_assert(RP >= 1 && DK % NRG == 0, "row split");
  extern __shared__ float dsm[];
  const int tid = threadIdx.x;
  const int cl = tid % CW, rg = tid / CW;
  const int nvb = p.dv / CW;
  const long long bh = blockIdx.x / nvb;
  const int col = (blockIdx.x % nvb) * CW + cl;
  const int n_h = p.n_h;
  const bool asym = p.kt != nullptr;

  float* sK = dsm;
  float* sW = sK + n_h * DK;               // write keys (asymmetric only)
  float* sQ = sW + (asym ? n_h * DK : 0);
  float* sV = sQ + DK;
  float* sR = sV + n_h * CW;               // 1 / max(|k|, 1e-6)
  float* sB = sR + n_h;                    // clamped beta
  float* sRed = sB + n_h;                  // [2][NRG][CW]

  // the state rows of this thread, issued first: they are the long pole
  float* st = p.state + bh * DK * p.dv + (long long)(rg * RP) * p.dv + col;
  float hs[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) hs[i] = st[(long long)i * p.dv];

  const T* kp = static_cast<const T*>(p.k) + bh * n_h * DK;
  for (int x = tid; x < n_h * DK; x += NTH) sK[x] = to_f32(kp[x]);
  if (asym) {
    const T* wp = static_cast<const T*>(p.kt) + bh * n_h * DK;
    for (int x = tid; x < n_h * DK; x += NTH) sW[x] = to_f32(wp[x]);
  }
  const T* qp = static_cast<const T*>(p.q) + bh * DK;
  for (int x = tid; x < DK; x += NTH) sQ[x] = to_f32(qp[x]);
  const T* vp = static_cast<const T*>(p.v) + bh * n_h * p.dv + (col - cl);
  for (int x = tid; x < n_h * CW; x += NTH) sV[x] = to_f32(vp[(long long)(x / CW) * p.dv + x % CW]);
  for (int j = tid; j < n_h; j += NTH) sB[j] = clamp_keep_nan(p.beta[bh * n_h + j], 0.f, 2.f);
  const float gt = p.g != nullptr ? p.g[bh] : 1.f;
  block_sync_lds();

  // key norms: wavefront w takes sub-steps w, w + 4, ...
  const int wave = tid >> 6, lane = tid & 63;
  for (int j = wave; j < n_h; j += NTH / 64) {
    float s = 0.f;
    for (int x = lane; x < DK; x += 64) s = fmaf(sK[j * DK + x], sK[j * DK + x], s);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) sR[j] = 1.f / fmaxf(sqrtf(s), 1e-6f);
  }

  if (p.g != nullptr) {
#pragma unroll
    for (int i = 0; i < RP; ++i) hs[i] *= gt;
  }
  if (p.ga != nullptr) {  // Diag(alpha) H: state row r scales by alpha[r]
    const float* al = p.ga + bh * DK + rg * RP;
#pragma unroll
    for (int i = 0; i < RP; ++i) hs[i] *= al[i];
  }
  block_sync_lds();

  // column sum over all row groups of this thread's column; buffer `buf`
  auto colsum = [&](float part, int buf) {
    float* red = sRed + buf * NRG * CW;
    red[rg * CW + cl] = part;
    block_sync_lds();
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < NRG; ++r) s += red[r * CW + cl];
    return s;
  };

  int buf = 0;
  for (int j = 0; j < n_h; ++j) {
    const float* kr = sK + j * DK + rg * RP;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) part = fmaf(hs[i], kr[i], part);
    const float rj = sR[j];
    const float e = sV[j * CW + cl] - colsum(part, buf) * rj;  // v - H^T kn
    buf ^= 1;
    const float be = sB[j] * e;
    if (asym) {
      const float* wr = sW + j * DK + rg * RP;
#pragma unroll
      for (int i = 0; i < RP; ++i) hs[i] = fmaf(wr[i], be, hs[i]);
    } else {
#pragma unroll
      for (int i = 0; i < RP; ++i) hs[i] = fmaf(kr[i] * rj, be, hs[i]);
    }
  }

  float part = 0.f;
#pragma unroll
  for (int i = 0; i < RP; ++i) part = fmaf(hs[i], sQ[rg * RP + i], part);
  const float o = colsum(part, buf);
#pragma unroll
  for (int i = 0; i < RP; ++i) st[(long long)i * p.dv] = hs[i];
  if (rg == 0) {
    if (p.out_f32)
      static_cast<float*>(p.out)[bh * p.dv + col] = o;
    else
      static_cast<T*>(p.out)[bh * p.dv + col] = from_f32<T>(o);
  }
}

template <typename T, int DK, int CW>
hipError_t launch_decode_cw(const DecodeArgs& a, hipStream_t st) {
  const long long blocks = (long long)a.B * a.H * (a.dv / CW);
  static const bool attr = allow_big_lds(reinterpret_cast<const void*>(&dp_decode_kernel<T, DK, CW>));
  (void)attr;
  const int lds = 4 * decode_lds_floats(DK, CW, a.n_h, a.kt != nullptr ? 1 : 0);
  hipLaunchKernelGGL((dp_decode_kernel<T, DK, CW>), dim3((unsigned)blocks), dim3(decode_threads(DK, CW)), lds, st,
                     a);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_decode_dk(const DecodeArgs& a, hipStream_t st) {
  switch (a.dv) {
    case 16: return launch_decode_cw<T, DK, 16>(a, st);
    case 32: return launch_decode_cw<T, DK, 32>(a, st);
    default: return launch_decode_cw<T, DK, 64>(a, st);  // dv in {64, 128}
  }
}

}  // namespace dp
