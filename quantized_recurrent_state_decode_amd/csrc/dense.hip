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

// Prefill of one chunk: T tokens of the recurrence per (sequence, head) tile
// with the state held in registers for the whole chunk (the prefill step of
// the serving flow, "unpack active states, run the chunk kernel, pack
// boundary states", STEPQuant App. F.1).  Inputs are [B][T][H][...]; the
// output y_t of every token is written; the final state replaces S.  Row
// constants of token s (g_i, beta k_i, q_i, g_i k_i) are staged three tokens
// ahead in LDS, and the update of token s also forms the key-retrieval
// partials of token s + 1, so one workgroup barrier per token suffices.
template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void prefill_kernel(
    int kind, int H, int T, float* S, const float* q, const float* k, const float* v,
    const float* beta, const float* gate, float* y) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  __shared__ float4 rc[3][DK];                 // g, beta k, q, g k of a token's rows
  __shared__ float2 colD[2][NRB][NP], colY[2][NRB][NP];
  const int tile = blockIdx.x, bi = tile / H, h = tile - bi * H;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  float* St = S + (long long)tile * DK * DV;
  const long long base = (long long)bi * T * H + h;   // token s of this tile: base + s H
  auto stage = [&](int s) {
    if (t < DK) {
      const long long th = base + (long long)s * H, tk = th * DK;
      const float g = kind == SQ_KIND_GDN ? gate[th] : gate[tk + t];
      const float kk = k[tk + t];
      rc[s % 3][t] = make_float4(g, beta[th] * kk, q[tk + t], g * kk);
    }
  };
  float x[64];
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float2 v2 = *reinterpret_cast<const float2*>(St + (r0 + m) * DV + j0);
    x[2 * m] = v2.x;
    x[2 * m + 1] = v2.y;
  }
  stage(0);
  if (T > 1) stage(1);
  __syncthreads();
  {  // key retrieval partials of token 0
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float w = rc[0][r0 + m].w;
      a0 = fmaf(w, x[2 * m], a0);
      a1 = fmaf(w, x[2 * m + 1], a1);
    }
    colD[0][rb][p] = make_float2(a0, a1);
  }
  __syncthreads();
  for (int s = 0; s < T; ++s) {
    // the buffer of token s + 2 last held token s - 1, read before the barrier
    if (s + 2 < T) stage(s + 2);
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      d0 += colD[s & 1][r][p].x;
      d1 += colD[s & 1][r][p].y;
    }
    if (s > 0 && rb == 0) {  // the previous token's output
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        o0 += colY[(s - 1) & 1][r][p].x;
        o1 += colY[(s - 1) & 1][r][p].y;
      }
      *reinterpret_cast<float2*>(y + (base + (long long)(s - 1) * H) * DV + j0) =
          make_float2(o0, o1);
    }
    const float2 vv = *reinterpret_cast<const float2*>(v + (base + (long long)s * H) * DV + j0);
    const float e0 = vv.x - d0, e1 = vv.y - d1;
    float y0 = 0.f, y1 = 0.f, n0 = 0.f, n1 = 0.f;
    const int cur = s % 3, nxt = (s + 1) % 3;
    if (s + 1 < T) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float4 c = rc[cur][r0 + m];
        const float wn = rc[nxt][r0 + m].w;
        const float v0 = fmaf(c.x, x[2 * m], c.y * e0);
        const float v1 = fmaf(c.x, x[2 * m + 1], c.y * e1);
        x[2 * m] = v0;
        x[2 * m + 1] = v1;
        y0 = fmaf(c.z, v0, y0);
        y1 = fmaf(c.z, v1, y1);
        n0 = fmaf(wn, v0, n0);
        n1 = fmaf(wn, v1, n1);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float4 c = rc[cur][r0 + m];
        const float v0 = fmaf(c.x, x[2 * m], c.y * e0);
        const float v1 = fmaf(c.x, x[2 * m + 1], c.y * e1);
        x[2 * m] = v0;
        x[2 * m + 1] = v1;
        y0 = fmaf(c.z, v0, y0);
        y1 = fmaf(c.z, v1, y1);
      }
    }
    colY[s & 1][rb][p] = make_float2(y0, y1);
    colD[(s + 1) & 1][rb][p] = make_float2(n0, n1);
    __syncthreads();
  }
  if (rb == 0) {
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      o0 += colY[(T - 1) & 1][r][p].x;
      o1 += colY[(T - 1) & 1][r][p].y;
    }
    *reinterpret_cast<float2*>(y + (base + (long long)(T - 1) * H) * DV + j0) = make_float2(o0, o1);
  }
#pragma unroll
  for (int m = 0; m < 32; ++m)
    *reinterpret_cast<float2*>(St + (r0 + m) * DV + j0) = make_float2(x[2 * m], x[2 * m + 1]);
}

template <int DK, int DV>
hipError_t launch_prefill(int kind, int H, int B, int T, float* S, const float* q, const float* k,
                          const float* v, const float* beta, const float* gate, float* y,
                          hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(B * H), dim3((DK / 32) * (DV / 2)), 0, s, kind,
                     H, T, S, q, k, v, beta, gate, y);
  return hipGetLastError();
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

hipError_t launch_prefill_chunk(int kind, int H, int dk, int dv, int B, int T, float* S,
                                const float* q, const float* k, const float* v, const float* beta,
                                const float* gate, float* y, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_prefill<128, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 64) return launch_prefill<64, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 128 && dv == 64) return launch_prefill<128, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 128) return launch_prefill<64, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  return hipErrorInvalidValue;
}
