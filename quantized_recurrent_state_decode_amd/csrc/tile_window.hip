// Per-window decode (LeapQuant notes Sec. 2.3-2.6, GDN scalar gate).
//
// A head keeps a fixed INT8 boundary S0 = diag(C) (Z/127) diag(B) and the
// records (alpha_j, kt_j = beta_j k_j, u_j) of the tokens since the last
// rebuild.  With Gamma_{a:b} = alpha_b ... alpha_a (1 when a > b):
//   S_l^T x = Gamma_{1:l} S0^T x + sum_{j<=l} u_j (kt_j . Gamma_{j+1:l} x)
// Token i = l + 1:
//   u_i = v_i - S_{i-1}^T (alpha_i k_i)          (stored as float32)
//   o_i = S_i^T q_i                               (the head output)
// and when the window holds p records the dense state
//   S_p = Gamma_{1:p} S0 + sum_j Gamma_{j+1:p} kt_j u_j^T
// is rebuilt and re-encoded with key-row smoothing and per-column INT8
// (Sec. 2.5, App. B.3): C_a = max(sqrt(mean_j |S_aj|), c_floor),
// T = diag(C)^-1 S, B_j = max_a |T_aj|, Z = clamp(rne(127 T / B), +-127).
//
// S0^T x costs one fused multiply-add per boundary element for each of the
// two read vectors; lanes own 2 columns x 32 rows of the INT8 boundary
// (blocked layout), so the reduction over rows is lane-local plus one LDS
// combine across row blocks.
#include "tile_common.h"

using namespace sqk;

namespace {

constexpr int kMaxP = 32;

template <int DK, int DV>
struct SmemWin {
  float x1[DK], qv[DK], ktn[DK];   // alpha_i k_i, q_i, beta_i k_i (float32)
  float cx1[DK], cq[DK];           // C_a x1_a, C_a q_a
  float rowf[DK];                  // per-row factor of the rebuild / 1 / C_a
  float kr[kMaxP][DK];             // Gamma_{j+1:L} kt_j for the rebuild
  float al[kMaxP];                 // record decays
  float g1[kMaxP + 1], g2[kMaxP + 1];
  float dots[2 * kMaxP];
  float unew[DV];
  float2 colA[DK / 32][DV / 2];
  float rowt[DK / 32][32][DV / 2 + 1];
};

struct WinPtrs {
  int* ell;
  float* alpha;
  unsigned char* Z;
  float *C, *B, *K, *U;
};

__device__ __forceinline__ WinPtrs win_ptrs(unsigned char* base, int zoff, int DK, int DV, int P) {
  WinPtrs w;
  w.ell = reinterpret_cast<int*>(base);
  w.alpha = reinterpret_cast<float*>(base + 16);
  w.Z = base + zoff;
  w.C = reinterpret_cast<float*>(base + zoff + DK * DV);
  w.B = w.C + DK;
  w.K = w.B + DV;
  w.U = w.K + P * DK;
  return w;
}

// Wave-wide sum of a float (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// x holds S (fp32) in the lane layout; re-encode it into the head and reset
// the window.  All threads of the workgroup call this.
template <int DK, int DV>
__device__ __forceinline__ void encode_boundary(float (&x)[64], const WinPtrs& wp, float c_floor,
                                                SmemWin<DK, DV>& sm, int P, bool clear_records) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 32; ++m) sm.rowt[rb][m][p] = fabsf(x[2 * m]) + fabsf(x[2 * m + 1]);
  __syncthreads();
  {
    constexpr int LPR = NP / 32;
    const int m = p & 31, part = p >> 5;
    float s = 0.f;
#pragma unroll 8
    for (int pp = 0; pp < 32; ++pp) s += sm.rowt[rb][m][part * 32 + pp];
    if constexpr (LPR == 2) s += __shfl_xor(s, 32);
    if (part == 0) {
      const int a = 32 * rb + m;
      const float ca = fmaxf(sqrtf(s / (float)DV), c_floor);
      wp.C[a] = ca;
      sm.rowf[a] = 1.0f / ca;
    }
  }
  __syncthreads();
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float ic = sm.rowf[32 * rb + m];
    x[2 * m] *= ic;
    x[2 * m + 1] *= ic;
    m0 = fmaxf(m0, fabsf(x[2 * m]));
    m1 = fmaxf(m1, fabsf(x[2 * m + 1]));
  }
  sm.colA[rb][p] = make_float2(m0, m1);
  __syncthreads();
  float b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    b0 = fmaxf(b0, sm.colA[r][p].x);
    b1 = fmaxf(b1, sm.colA[r][p].y);
  }
  const float s0 = b0 > 0.f ? 127.0f / b0 : 0.f, s1 = b1 > 0.f ? 127.0f / b1 : 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    x[2 * m] = fminf(fmaxf(rintf(x[2 * m] * s0), -127.f), 127.f) + 128.f;
    x[2 * m + 1] = fminf(fmaxf(rintf(x[2 * m + 1] * s1), -127.f), 127.f) + 128.f;
  }
  uint32_t wd[16];
  pack_codes<8>(x, wd);
  store_chunk<8, NP>(wp.Z, rb, p, wd);
  if (rb == 0) *reinterpret_cast<float2*>(wp.B + j0) = make_float2(b0, b1);
  if (t == 0) wp.ell[0] = 0;
  if (clear_records) {
    if (t < 3) wp.ell[1 + t] = 0;
    for (int i = t; i < P; i += NT) wp.alpha[i] = 0.f;
    for (int i = t; i < P * (DK + DV); i += NT) wp.K[i] = 0.f;  // K and U are contiguous
  }
}

// Rebuild the dense state of L records into x (lane layout).  Records 0..L-2
// come from the head; record L-1 comes from LDS when `last_in_lds`.
template <int DK, int DV>
__device__ __forceinline__ void rebuild(float (&x)[64], const WinPtrs& wp, int L, bool last_in_lds,
                                        SmemWin<DK, DV>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NT = G::NT;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  // suffix products: factor of record j is prod_{m=j+1}^{L-1} al[m]
  if (t == 0) {
    float g = 1.f;
    for (int j = L - 1; j >= 0; --j) {
      sm.g1[j] = g;
      g *= sm.al[j];
    }
    sm.g1[kMaxP] = g;  // Gamma over all L records
  }
  __syncthreads();
  for (int i = t; i < L * DK; i += NT) {
    const int j = i / DK, a = i - j * DK;
    const float kt = (last_in_lds && j == L - 1) ? sm.ktn[a] : wp.K[j * DK + a];
    sm.kr[j][a] = sm.g1[j] * kt;
  }
  if (t < DK) sm.rowf[t] = sm.g1[kMaxP] * wp.C[t] * (1.0f / 127.0f);
  __syncthreads();
  const float2 bb = *reinterpret_cast<const float2*>(wp.B + j0);
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float f = sm.rowf[32 * rb + m];
    x[2 * m] = f * bb.x * (x[2 * m] - 128.f);
    x[2 * m + 1] = f * bb.y * (x[2 * m + 1] - 128.f);
  }
  for (int j = 0; j < L; ++j) {
    const float2 u = (last_in_lds && j == L - 1)
                         ? make_float2(sm.unew[j0], sm.unew[j0 + 1])
                         : *reinterpret_cast<const float2*>(wp.U + j * DV + j0);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float k = sm.kr[j][32 * rb + m];
      x[2 * m] = fmaf(k, u.x, x[2 * m]);
      x[2 * m + 1] = fmaf(k, u.y, x[2 * m + 1]);
    }
  }
}

template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void window_tile_kernel(TileArgs a) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT, NW = NT / 64;
  __shared__ SmemWin<DK, DV> sm;
  const int tile = blockIdx.x;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (a.op == OP_DECODE && t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    return;
  }
  const int P = a.P.p;
  const WinPtrs wp = win_ptrs(base, a.P.r_off[h], DK, DV, P);
  const int op = a.op;
  float x[64];
  if (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float2 v2 = *reinterpret_cast<const float2*>(X + (32 * rb + m) * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    encode_boundary<DK, DV>(x, wp, a.P.c_floor, sm, P, true);
    return;
  }
  // records held; a value outside [0, p) is not a state this library writes,
  // it is clamped so that every access stays inside the head
  const int ell = min(max(wp.ell[0], 0), P - 1);
  {
    uint32_t wd[16];
    load_chunk<8, NP>(wp.Z, rb, p, wd);
    unpack_codes<8>(wd, x);  // Z + 128
  }
  if (op == OP_UNPACK || op == OP_FLUSH) {
    if (op == OP_FLUSH && ell == 0) return;
    if (t < ell) sm.al[t] = wp.alpha[t];
    __syncthreads();
    rebuild<DK, DV>(x, wp, ell, false, sm);
    if (op == OP_FLUSH) {
      encode_boundary<DK, DV>(x, wp, a.P.c_floor, sm, P, false);
      return;
    }
    float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m)
      *reinterpret_cast<float2*>(S + (32 * rb + m) * DV + j0) = make_float2(x[2 * m], x[2 * m + 1]);
    return;
  }
  // ---- decode token i = ell + 1 (record index ell, 0-based)
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  const float alpha = a.gate[tile], beta = a.beta[tile];
  if (t < ell) sm.al[t] = wp.alpha[t];
  if (t == 0) sm.al[ell] = alpha;
  if (t < DK) {
    const float kk = a.k[tk + t], qq = a.q[tk + t], ca = wp.C[t];
    const float x1 = alpha * kk, kn = beta * kk;
    sm.x1[t] = x1;
    sm.qv[t] = qq;
    sm.ktn[t] = kn;
    sm.cx1[t] = ca * x1;
    sm.cq[t] = ca * qq;
    wp.K[ell * DK + t] = kn;  // the new record's key (record slot ell is free)
  }
  __syncthreads();
  if (t == 0) {
    // g1[j] = prod_{m=j+1}^{ell-1} al[m] (for u_i), g2[j] = prod_{m=j+1}^{ell} al[m] (for o_i);
    // index kMaxP holds the products over all records (Gamma_{1:i-1}, Gamma_{1:i})
    float g = 1.f;
    for (int j = ell - 1; j >= 0; --j) {
      sm.g1[j] = g;
      g *= sm.al[j];
    }
    sm.g1[kMaxP] = g;
    g = 1.f;
    for (int j = ell; j >= 0; --j) {
      sm.g2[j] = g;
      g *= sm.al[j];
    }
    sm.g2[kMaxP] = g;
  }
  // dot products kt_j . x1 (j < ell) and kt_j . q (j <= ell), one task per wave
  {
    const int w = t >> 6, lane = t & 63;
    for (int task = w; task < 2 * ell + 2; task += NW) {
      const int j = task >> 1;
      const float* xv = (task & 1) ? sm.qv : sm.x1;
      float s = 0.f;
      for (int r = lane; r < DK; r += 64) {
        const float kt = j == ell ? sm.ktn[r] : wp.K[j * DK + r];
        s = fmaf(kt, xv[r], s);
      }
      s = wave_sum(s);
      if (lane == 0) sm.dots[task] = s;
    }
  }
  // boundary readouts: sum_a Z_aj (C_a x_a), for x = x1 and x = q
  float s10 = 0.f, s11 = 0.f, s20 = 0.f, s21 = 0.f, c1s = 0.f, c2s = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float f1 = sm.cx1[32 * rb + m], f2 = sm.cq[32 * rb + m];
    s10 = fmaf(f1, x[2 * m], s10);
    s11 = fmaf(f1, x[2 * m + 1], s11);
    s20 = fmaf(f2, x[2 * m], s20);
    s21 = fmaf(f2, x[2 * m + 1], s21);
    c1s += f1;
    c2s += f2;
  }
  s10 = fmaf(-128.f, c1s, s10);
  s11 = fmaf(-128.f, c1s, s11);
  s20 = fmaf(-128.f, c2s, s20);
  s21 = fmaf(-128.f, c2s, s21);
  // two column vectors combine through LDS: x1-part in colA, q-part in rowt scratch
  sm.colA[rb][p] = make_float2(s10, s11);
  reinterpret_cast<float2*>(&sm.rowt[0][0][0])[rb * NP + p] = make_float2(s20, s21);
  __syncthreads();
  if (rb == 0) {
    float r10 = 0.f, r11 = 0.f, r20 = 0.f, r21 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      r10 += sm.colA[r][p].x;
      r11 += sm.colA[r][p].y;
      const float2 q2 = reinterpret_cast<const float2*>(&sm.rowt[0][0][0])[r * NP + p];
      r20 += q2.x;
      r21 += q2.y;
    }
    const float2 bb = *reinterpret_cast<const float2*>(wp.B + j0);
    const float f0 = bb.x * (1.0f / 127.0f), f1 = bb.y * (1.0f / 127.0f);
    float pv0 = sm.g1[kMaxP] * f0 * r10, pv1 = sm.g1[kMaxP] * f1 * r11;
    float o0 = sm.g2[kMaxP] * f0 * r20, o1 = sm.g2[kMaxP] * f1 * r21;
    for (int j = 0; j < ell; ++j) {
      const float2 u = *reinterpret_cast<const float2*>(wp.U + j * DV + j0);
      const float d1 = sm.g1[j] * sm.dots[2 * j], d2 = sm.g2[j] * sm.dots[2 * j + 1];
      pv0 = fmaf(u.x, d1, pv0);
      pv1 = fmaf(u.y, d1, pv1);
      o0 = fmaf(u.x, d2, o0);
      o1 = fmaf(u.y, d2, o1);
    }
    const float2 vv = *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float u0 = vv.x - pv0, u1 = vv.y - pv1;
    const float dn = sm.dots[2 * ell + 1];  // kt_i . q
    o0 = fmaf(u0, dn, o0);
    o1 = fmaf(u1, dn, o1);
    *reinterpret_cast<float2*>(wp.U + ell * DV + j0) = make_float2(u0, u1);
    *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(o0, o1);
    sm.unew[j0] = u0;
    sm.unew[j0 + 1] = u1;
  }
  if (ell + 1 < P) {
    if (t == 0) {
      wp.alpha[ell] = alpha;
      wp.ell[0] = ell + 1;
    }
    return;
  }
  // the window is full: rebuild S_p and re-encode the boundary
  __syncthreads();
  rebuild<DK, DV>(x, wp, P, true, sm);
  encode_boundary<DK, DV>(x, wp, a.P.c_floor, sm, P, false);
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((window_tile_kernel<DK, DV>), dim3(a.n_tiles), dim3((DK / 32) * (DV / 2)), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_window(const TileArgs& a, hipStream_t s) {
  if (a.P.p > kMaxP || a.P.p < 1) return hipErrorInvalidValue;
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(a, s);
  return hipErrorInvalidValue;
}
