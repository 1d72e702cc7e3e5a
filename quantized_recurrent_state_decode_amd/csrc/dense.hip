// Full-precision (fp32 state) gated delta-rule decode step: the FP32-state
// baseline the pages compare against (STEPQuant Sec. 5.1; LeapQuant notes
// Sec. 3.3), and the way large workloads build their warm-up states.
//   X = D S + beta k (v - (D S)^T k)^T,  y = X^T q,  S <- X (in place).
// Same lane geometry as the packed kernels: lane (rb, p) owns rows
// 32 rb .. 32 rb + 31 of columns 2p, 2p+1.
#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void dense_kernel(
    int kind, int H, float* S, long long n_slots, const int* slots, const float* q,
    const float* k, const float* v, const float* beta, const float* gate, float* y) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  __shared__ float kd[DK], bk[DK], qq[DK];
  __shared__ float2 col[NRB][NP];
  const int tile = blockIdx.x, bi = tile / H, h = tile - bi * H;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  const int slot = slots[bi];
  if (slot < 0 || (long long)slot >= n_slots) {
    if (t < DV) y[tv + t] = __builtin_nanf("");
    return;
  }
  float* St = S + ((long long)slot * H + h) * DK * DV;
  if (t < DK) {
    const float g = kind == SQ_KIND_GDN ? gate[tile] : gate[tk + t];
    const float kk = k[tk + t];
    kd[t] = kk * g;
    bk[t] = beta[tile] * kk;
    qq[t] = q[tk + t];
  }
  float x[64];
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float2 v2 = *reinterpret_cast<const float2*>(St + (32 * rb + m) * DV + j0);
    x[2 * m] = v2.x;
    x[2 * m + 1] = v2.y;
  }
  __syncthreads();
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float kk = kd[32 * rb + m];
    a0 = fmaf(kk, x[2 * m], a0);
    a1 = fmaf(kk, x[2 * m + 1], a1);
  }
  col[rb][p] = make_float2(a0, a1);
  __syncthreads();
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    d0 += col[r][p].x;
    d1 += col[r][p].y;
  }
  const float2 vv = *reinterpret_cast<const float2*>(v + tv + j0);
  const float e0 = vv.x - d0, e1 = vv.y - d1;
  const float ga = kind == SQ_KIND_GDN ? gate[tile] : 0.f;
  float y0 = 0.f, y1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int i = 32 * rb + m;
    const float g = kind == SQ_KIND_GDN ? ga : gate[tk + i];
    const float b = bk[i], qv = qq[i];
    const float v0 = fmaf(g, x[2 * m], b * e0);
    const float v1 = fmaf(g, x[2 * m + 1], b * e1);
    y0 = fmaf(qv, v0, y0);
    y1 = fmaf(qv, v1, y1);
    *reinterpret_cast<float2*>(St + i * DV + j0) = make_float2(v0, v1);
  }
  __syncthreads();
  col[rb][p] = make_float2(y0, y1);
  __syncthreads();
  if (rb == 0) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      s0 += col[r][p].x;
      s1 += col[r][p].y;
    }
    *reinterpret_cast<float2*>(y + tv + j0) = make_float2(s0, s1);
  }
}

template <int DK, int DV>
hipError_t launch(int kind, int H, float* S, long long n_slots, const int* slots, int B,
                  const float* q, const float* k, const float* v, const float* beta,
                  const float* gate, float* y, hipStream_t s) {
  hipLaunchKernelGGL((dense_kernel<DK, DV>), dim3(B * H), dim3((DK / 32) * (DV / 2)), 0, s, kind, H, S,
                     n_slots, slots, q, k, v, beta, gate, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_step(int kind, int H, int dk, int dv, float* S, long long n_slots,
                             const int* slots, int B, const float* q, const float* k,
                             const float* v, const float* beta, const float* gate, float* y,
                             hipStream_t s) {
  if (dk == 128 && dv == 128) return launch<128, 128>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  return hipErrorInvalidValue;
}
