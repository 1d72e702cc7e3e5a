// Calibration statistics on the GPU (STEPQuant "Lifetime-aware Bit
// Allocation", Sec. 4, Eqs. 6-8; row impact, Sec. 4.1 and App. B-C).
//
// * Gate statistics of one calibration step over n sequences: the sum of
//   log r_{t,u} per unit (r = alpha_t for a GDN head, d_{t,i} for a KDA key
//   row) and the sum of g_{t,i}^2 per key row, with the transported query
//   g_t = A_t^T q_t = D_t (q_t - beta_t k_t (k_t . q_t)).  One workgroup owns
//   a head's accumulators, so the sums are deterministic; the arithmetic is
//   float64 (the inputs are float32, exact in float64).
// * Distortion: the squared error of packed STEP heads (written by the
//   library's own quantizer, quantize-only) against the dense tiles they were
//   quantized from, summed per unit (a whole head, or one key row) in float64.
//   The dequantized value is r_i c_j z_ij / q_b.
#include "tile_common.h"

using namespace sqk;

namespace {

// Sum of v over the workgroup (DK lanes, DK / 64 waves), returned to all lanes.
template <int DK>
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int o = 1; o < 64 && o < DK; o <<= 1) v += __shfl_xor(v, o);
  constexpr int NW = DK / 64 > 0 ? DK / 64 : 1;
  if (NW == 1) return v;
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  return s;
}

template <int DK>
__global__ __launch_bounds__(DK) void calib_gate_kernel(int kind, int H, int n, const float* q,
                                                        const float* k, const float* beta,
                                                        const float* gate, double* log_sum,
                                                        double* om_sum) {
  __shared__ double red[DK / 64 > 0 ? DK / 64 : 1];
  const int h = blockIdx.x, i = threadIdx.x;
  double ls = 0.0, om = 0.0;
  for (int s = 0; s < n; ++s) {
    const long long th = (long long)s * H + h, tk = th * DK;
    const double qi = q[tk + i], ki = k[tk + i];
    const double kq = block_sum<DK>(ki * qi, red);
    const double d = kind == SQ_KIND_GDN ? (double)gate[th] : (double)gate[tk + i];
    const double g = d * (qi - (double)beta[th] * ki * kq);
    om += g * g;
    if (kind == SQ_KIND_KDA || i == 0) ls += log(d);
  }
  om_sum[(long long)h * DK + i] += om;
  if (kind == SQ_KIND_KDA) log_sum[(long long)h * DK + i] += ls;
  else if (i == 0) log_sum[h] += ls;
}

template <int DK, int DV, int BITS>
__device__ __forceinline__ void dist_tile(const DevPlan& P, int tile, int h, const unsigned char* head,
                                          const float* S, int per_row, double* dist,
                                          double* rows) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  const double qb = (double)((1 << (BITS - 1)) - 1), off = (double)(1 << (BITS - 1));
  const __half* r_ptr = reinterpret_cast<const __half*>(head + P.r_off[h]);
  const __half* c_ptr = reinterpret_cast<const __half*>(head + P.c_off[h]);
  uint32_t wd[2 * BITS];
  load_chunk<BITS, NP>(head, rb, p, wd);
  float z[64];
  unpack_codes<BITS>(wd, z);  // offset-binary: z + 2^(BITS-1)
  const double c0 = __half2float(c_ptr[j0]), c1 = __half2float(c_ptr[j0 + 1]);
  const float* X = S + (long long)tile * DK * DV;
  for (int m = 0; m < 32; ++m) {
    const int i = r0 + m;
    const double ri = __half2float(r_ptr[i]);
    const float2 xv = *reinterpret_cast<const float2*>(X + (long long)i * DV + j0);
    const double e0 = ri * c0 * ((double)z[2 * m] - off) / qb - (double)xv.x;
    const double e1 = ri * c1 * ((double)z[2 * m + 1] - off) / qb - (double)xv.y;
    atomicAdd(&rows[i], e0 * e0 + e1 * e1);
  }
}

template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void calib_dist_kernel(
    DevPlan P, int n_tiles, const unsigned char* packed, long long stride, const float* S,
    int per_row, double* dist) {
  __shared__ double rows[DK];
  const int tile = blockIdx.x, h = tile % P.H, t = threadIdx.x;
  constexpr int NT = (DK / 32) * (DV / 2);
  for (int i = t; i < DK; i += NT) rows[i] = 0.0;
  __syncthreads();
  const unsigned char* head = packed + (long long)tile * stride;
  switch (P.head_bits[h]) {
    case 2: dist_tile<DK, DV, 2>(P, tile, h, head, S, per_row, dist, rows); break;
    case 4: dist_tile<DK, DV, 4>(P, tile, h, head, S, per_row, dist, rows); break;
    case 6: dist_tile<DK, DV, 6>(P, tile, h, head, S, per_row, dist, rows); break;
    case 8: dist_tile<DK, DV, 8>(P, tile, h, head, S, per_row, dist, rows); break;
    default: break;
  }
  __syncthreads();
  if (per_row) {
    for (int i = t; i < DK; i += NT) atomicAdd(&dist[(long long)h * DK + i], rows[i]);
  } else if (t == 0) {
    double s = 0.0;
    for (int i = 0; i < DK; ++i) s += rows[i];
    atomicAdd(&dist[h], s);
  }
}

template <int DK, int DV>
hipError_t launch_dist(const DevPlan& P, int n_tiles, const unsigned char* packed, long long stride,
                       const float* S, int per_row, double* dist, hipStream_t s) {
  hipLaunchKernelGGL((calib_dist_kernel<DK, DV>), dim3(n_tiles), dim3((DK / 32) * (DV / 2)), 0, s,
                     P, n_tiles, packed, stride, S, per_row, dist);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calib_gate(int kind, int H, int dk, int n, const float* q, const float* k,
                             const float* beta, const float* gate, double* log_sum,
                             double* om_sum, hipStream_t s) {
  if (dk == 128)
    hipLaunchKernelGGL((calib_gate_kernel<128>), dim3(H), dim3(128), 0, s, kind, H, n, q, k, beta,
                       gate, log_sum, om_sum);
  else if (dk == 64)
    hipLaunchKernelGGL((calib_gate_kernel<64>), dim3(H), dim3(64), 0, s, kind, H, n, q, k, beta,
                       gate, log_sum, om_sum);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_calib_dist(const DevPlan& P, int n_tiles, const unsigned char* packed,
                             long long stride, const float* S, int per_row, double* dist,
                             hipStream_t s) {
  if (P.dk == 128 && P.dv == 128) return launch_dist<128, 128>(P, n_tiles, packed, stride, S, per_row, dist, s);
  if (P.dk == 64 && P.dv == 64) return launch_dist<64, 64>(P, n_tiles, packed, stride, S, per_row, dist, s);
  if (P.dk == 128 && P.dv == 64) return launch_dist<128, 64>(P, n_tiles, packed, stride, S, per_row, dist, s);
  if (P.dk == 64 && P.dv == 128) return launch_dist<64, 128>(P, n_tiles, packed, stride, S, per_row, dist, s);
  return hipErrorInvalidValue;
}
