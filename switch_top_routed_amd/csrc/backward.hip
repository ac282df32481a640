// Backward pass of the Switch top-1 MoE layer.
//
// The gate value multiplies the expert output, so the gradient reaches the
// router through it (Switch Transformers summary page, Switch-layer passage);
// the auxiliary loss reaches it through P only, f being a count (same page,
// Eq. 4 passage); the training step backpropagates into router and experts
// ("MoE expert capacity factor and token dropping" page, training-step
// flowchart).  With O = ReLU(X W1) W2 per expert and y = s O (s = gate or 1):
//   U  = dY W2^T              dg_t = <U_t, H_t>        dZ = s U * [H > 0]
//   dW2 = H^T (s dY)          dW1 = X^T dZ             dX_e = dZ W1^T
//   dlogit_t = p_t * (dp_t - <p_t, dp_t>),  dp_ti = [i = e_t] dg_t + dl_aux N f_i / T
//   dW_g = dlogit^T x,  db = sum_t dlogit_t,  dx_t = dX_e + dlogit_t W_g (+ dy_t
//   for dropped tokens and with the residual flag) (+ the shared expert's dX).
// H is the forward's saved hidden activation (bf16 for bf16 layers), so the
// ReLU pattern is the one the forward used.
//
// This file holds the generic kernels: a tiled fp32-accumulating GEMM over any
// operand orientation (row gathers through token_of_slot, per-expert row or
// reduction extents from kept_count), the per-slot dZ / dg rows, the router
// softmax gradient, column sums and the final dx assembly.  Every reduction has
// a fixed order (no atomics), so results are bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = (uint16_t)f2bf(v); }

constexpr int kGT = 64;   // output tile edge
constexpr int kGK = 16;   // reduction chunk

// physical row of operand row `r` of batch b
__device__ __forceinline__ int64_t op_row(const GemmOperand& o, int b, int C, int r) {
  return o.gather != nullptr ? (int64_t)o.gather[(int64_t)b * C + r] : (int64_t)r;
}

}  // namespace

// out[b][m][n] = sum_k A_b(m, k) B_b(k, n), fp32 accumulation in ascending k.
// A_b(m, k) = A[a_base + row(i) * lda + j] with (i, j) = trans ? (k, m) : (m, k),
// B_b(k, n) likewise with (i, j) = trans ? (n, k) : (k, n); row(i) is
// gather[b * C + i] or i (then a_base = b * bstride).  extent: 1 -> M_b =
// min(kept[b], C), 2 -> K_b = min(kept[b], C).  Rows m >= M_b are not written.
template <typename TA, typename TB, typename TO>
__global__ __launch_bounds__(256) void gemm_generic(GemmOperand a, GemmOperand b, GemmOut o, int M, int Nn, int K,
                                                    int C, const int32_t* __restrict__ kept, int extent) {
  __shared__ float As[kGK][kGT + 4];
  __shared__ float Bs[kGK][kGT + 4];
  const int bt = blockIdx.z;
  const int n0 = blockIdx.x * kGT;
  int Mb = M, Kb = K;
  if (extent != 0) {
    int kc = kept[bt];
    kc = kc < 0 ? 0 : (kc > C ? C : kc);
    if (extent == 1) Mb = kc < M ? kc : M;
    else Kb = kc < K ? kc : K;
  }
  // grid.y row tiles stride over M (M may exceed 65535 tiles)
  for (int64_t m0l = (int64_t)blockIdx.y * kGT; m0l < Mb; m0l += (int64_t)gridDim.y * kGT) {
  const int m0 = (int)m0l;
  const TA* A = static_cast<const TA*>(a.ptr) + (a.gather != nullptr ? 0 : (int64_t)bt * a.bstride);
  const TB* B = static_cast<const TB*>(b.ptr) + (b.gather != nullptr ? 0 : (int64_t)bt * b.bstride);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kb; k0 += kGK) {
    // 64 x 16 elements of each operand, 4 per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      // A: element (m = m0 + mm, k = k0 + kk)
      {
        int mm, kk;
        if (a.trans) {  // consecutive threads along m (the contiguous index)
          mm = e & 63;
          kk = e >> 6;
        } else {
          kk = e & 15;
          mm = e >> 4;
        }
        const int m = m0 + mm, k = k0 + kk;
        float v = 0.f;
        if (m < Mb && k < Kb) {
          const int i = a.trans ? k : m, j = a.trans ? m : k;
          v = ld<TA>(A, op_row(a, bt, C, i) * a.ld + j);
        }
        As[kk][mm] = v;
      }
      // B: element (k = k0 + kk, n = n0 + nn)
      {
        int nn, kk;
        if (b.trans) {
          kk = e & 15;
          nn = e >> 4;
        } else {
          nn = e & 63;
          kk = e >> 6;
        }
        const int n = n0 + nn, k = k0 + kk;
        float v = 0.f;
        if (n < Nn && k < Kb) {
          const int i = b.trans ? n : k, j = b.trans ? k : n;
          const int64_t r = op_row(b, bt, C, i);
          v = ld<TB>(B, r * b.ld + j);
          if (b.row_scale != nullptr) v *= b.row_scale[r];
        }
        Bs[kk][nn] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty + 16 * i];
        bv[i] = Bs[kk][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  TO* out = static_cast<TO*>(o.ptr) + (int64_t)bt * o.bstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= Mb) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n < Nn) st<TO>(out, (int64_t)m * o.ld + n, acc[i][j]);
    }
  }
  }
}

// One workgroup per filled slot row (e, s): dZ = scale * U * [H > 0] and
// dg[e*C + s] = sum_f U * H (fixed order: per-thread strided sums, then the
// wave butterfly, then waves in order).  scale = gate[token] or 1.
template <typename TH>
__global__ __launch_bounds__(256) void dz_rows(const float* __restrict__ U, const TH* __restrict__ H,
                                               TH* __restrict__ dZ, float* __restrict__ dg,
                                               const int32_t* __restrict__ kept, const int32_t* __restrict__ tos,
                                               const float* __restrict__ gate, int C, int dff) {
  __shared__ float part[4];
  const int e = blockIdx.y, s = blockIdx.x;
  int kc = kept[e];
  kc = kc > C ? C : kc;
  if (s >= kc) return;
  const int64_t row = (int64_t)e * C + s;
  const float scale = gate != nullptr ? gate[tos[row]] : 1.f;
  float sum = 0.f;
  for (int f = threadIdx.x; f < dff; f += 256) {
    const float u = U[row * dff + f], h = ld<TH>(H, row * dff + f);
    sum = fmaf(u, h, sum);
    st<TH>(dZ, row * dff + f, h > 0.f ? scale * u : 0.f);
  }
  if (dg == nullptr) return;
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) dg[row] = ((part[0] + part[1]) + part[2]) + part[3];
}

// One wave per token: dlogit_t = p_t * (dp_t - <p_t, dp_t>) with
// dp_ti = [i = e_t] dg_t + dl_aux * N * f_i / T.
__global__ __launch_bounds__(256) void router_grad(const float* __restrict__ probs, const int32_t* __restrict__ eid,
                                                   const int32_t* __restrict__ slot, const float* __restrict__ dg,
                                                   int nparts, const float* __restrict__ f,
                                                   const float* __restrict__ dl_aux, int64_t T, int N, int C,
                                                   float* __restrict__ dlogit) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float caux = dl_aux != nullptr ? dl_aux[0] * (float)N / (float)T : 0.f;
  const int e = eid[t], s = slot[t];
  float dgt = 0.f;
  if (dg != nullptr && s >= 0)  // the slot's partial sums, in order
    for (int p = 0; p < nparts; ++p) dgt += dg[((int64_t)e * C + s) * nparts + p];
  float dot = 0.f;
  for (int i = lane; i < N; i += 64) {
    const float dp = (i == e ? dgt : 0.f) + caux * f[i];
    dot = fmaf(probs[t * N + i], dp, dot);
  }
  dot = wave_sum(dot);
  for (int i = lane; i < N; i += 64) {
    const float p = probs[t * N + i];
    const float dp = (i == e ? dgt : 0.f) + caux * f[i];
    dlogit[t * N + i] = p * (dp - dot);
  }
}

// Column sums of a [T, N] fp32 matrix in two fixed-order passes: partial[c][n]
// over 256-row chunks, then out[n] = sum_c partial[c][n] in ascending c.
__global__ __launch_bounds__(256) void colsum_partial(const float* __restrict__ a, int64_t T, int N,
                                                      float* __restrict__ partial) {
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (n >= N) return;
  const int64_t t0 = (int64_t)blockIdx.x * 256;
  const int64_t t1 = t0 + 256 < T ? t0 + 256 : T;
  float s = 0.f;
  for (int64_t t = t0; t < t1; ++t) s += a[t * N + n];
  partial[(int64_t)blockIdx.x * N + n] = s;
}

__global__ __launch_bounds__(256) void colsum_final(const float* __restrict__ partial, int chunks, int N,
                                                    float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += partial[(int64_t)c * N + n];
  out[n] = s;
}

// One workgroup per token: dx_t = sum_i dlogit_ti W_g[i] (ascending i)
// + dX_e[e_t, slot_t] (kept) + dy_t (dropped, or every token with the residual
// flag) + dx_shared_t; rounded once to the layer dtype.
template <typename TX>
__global__ __launch_bounds__(256) void dx_assemble(const float* __restrict__ dlogit, const TX* __restrict__ wg,
                                                   const float* __restrict__ dxe, const TX* __restrict__ dy,
                                                   const float* __restrict__ dxs, const int32_t* __restrict__ eid,
                                                   const int32_t* __restrict__ slot, int64_t T, int d, int N, int C,
                                                   int residual_all, TX* __restrict__ dx) {
  extern __shared__ float dl[];
  const int64_t t = blockIdx.x;
  for (int i = threadIdx.x; i < N; i += 256) dl[i] = dlogit[t * N + i];
  __syncthreads();
  const int s = slot[t];
  const int64_t row = s >= 0 ? (int64_t)eid[t] * C + s : -1;
  const bool pass = s < 0 || residual_all;
  for (int k = threadIdx.x; k < d; k += 256) {
    float v = 0.f;
    for (int i = 0; i < N; ++i) v = fmaf(dl[i], ld<TX>(wg, (int64_t)i * d + k), v);
    if (row >= 0) v += dxe[row * d + k];
    if (pass) v += ld<TX>(dy, t * d + k);
    if (dxs != nullptr) v += dxs[t * d + k];
    st<TX>(dx, t * d + k, v);
  }
}

// ----------------------------------------------------------------------------
template <typename TA, typename TB, typename TO>
static hipError_t gemm_t(const GemmOperand& a, const GemmOperand& b, const GemmOut& o, int batches, int M, int Nn,
                         int K, int C, const int32_t* kept, int extent, hipStream_t st) {
  if (batches <= 0 || M <= 0 || Nn <= 0) return hipSuccess;
  const int mt = (M + kGT - 1) / kGT;
  dim3 grid((unsigned)((Nn + kGT - 1) / kGT), (unsigned)(mt < 65535 ? mt : 65535), (unsigned)batches);
  hipLaunchKernelGGL((gemm_generic<TA, TB, TO>), grid, dim3(256), 0, st, a, b, o, M, Nn, K, C, kept, extent);
  return hipGetLastError();
}

hipError_t launch_gemm_generic(const GemmOperand& a, int a_f32, const GemmOperand& b, const GemmOut& o, int o_f32,
                               int dtype, int batches, int M, int Nn, int K, int C, const int32_t* kept, int extent,
                               hipStream_t st) {
  if (dtype == 0) return gemm_t<float, float, float>(a, b, o, batches, M, Nn, K, C, kept, extent, st);
  if (a_f32) {
    if (o_f32) return gemm_t<float, uint16_t, float>(a, b, o, batches, M, Nn, K, C, kept, extent, st);
    return gemm_t<float, uint16_t, uint16_t>(a, b, o, batches, M, Nn, K, C, kept, extent, st);
  }
  if (o_f32) return gemm_t<uint16_t, uint16_t, float>(a, b, o, batches, M, Nn, K, C, kept, extent, st);
  return gemm_t<uint16_t, uint16_t, uint16_t>(a, b, o, batches, M, Nn, K, C, kept, extent, st);
}

hipError_t launch_dz_rows(const float* U, const void* H, void* dZ, float* dg, const int32_t* kept,
                          const int32_t* tos, const float* gate, int N, int C, int dff, int dtype, hipStream_t st) {
  dim3 grid((unsigned)C, (unsigned)N);
  if (dtype == 0)
    hipLaunchKernelGGL(dz_rows<float>, grid, dim3(256), 0, st, U, static_cast<const float*>(H),
                       static_cast<float*>(dZ), dg, kept, tos, gate, C, dff);
  else
    hipLaunchKernelGGL(dz_rows<uint16_t>, grid, dim3(256), 0, st, U, static_cast<const uint16_t*>(H),
                       static_cast<uint16_t*>(dZ), dg, kept, tos, gate, C, dff);
  return hipGetLastError();
}

hipError_t launch_router_grad(const float* probs, const int32_t* eid, const int32_t* slot, const float* dg,
                              int nparts, const float* f, const float* dl_aux, int64_t T, int N, int C,
                              float* dlogit, hipStream_t st) {
  hipLaunchKernelGGL(router_grad, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, probs, eid, slot, dg, nparts, f,
                     dl_aux, T, N, C, dlogit);
  return hipGetLastError();
}

size_t colsum_scratch_bytes(int64_t T, int N) { return (size_t)((T + 255) / 256) * N * 4; }

hipError_t launch_colsum(const float* a, int64_t T, int N, float* scratch, float* out, hipStream_t st) {
  const int chunks = (int)((T + 255) / 256);
  hipLaunchKernelGGL(colsum_partial, dim3((unsigned)chunks, (unsigned)((N + 255) / 256)), dim3(256), 0, st, a, T, N,
                     scratch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, scratch, chunks, N, out);
  return hipGetLastError();
}

hipError_t launch_dx_assemble(const float* dlogit, const void* wg, const float* dxe, const void* dy, const float* dxs,
                              const int32_t* eid, const int32_t* slot, int64_t T, int d, int N, int C,
                              int residual_all, void* dx, int dtype, hipStream_t st) {
  const size_t lds = (size_t)N * 4;
  if (dtype == 0)
    hipLaunchKernelGGL(dx_assemble<float>, dim3((unsigned)T), dim3(256), lds, st, dlogit,
                       static_cast<const float*>(wg), dxe, static_cast<const float*>(dy), dxs, eid, slot, T, d, N, C,
                       residual_all, static_cast<float*>(dx));
  else
    hipLaunchKernelGGL(dx_assemble<uint16_t>, dim3((unsigned)T), dim3(256), lds, st, dlogit,
                       static_cast<const uint16_t*>(wg), dxe, static_cast<const uint16_t*>(dy), dxs, eid, slot, T, d,
                       N, C, residual_all, static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

}  // namespace swm
