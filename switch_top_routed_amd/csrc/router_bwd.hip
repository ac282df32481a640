// Router backward on MFMA for bf16 layers: dW_g = dlogit^T x and the token
// gradient dx = dlogit W_g + (the other terms of dx), with the router kept in
// fp32 (Switch Transformers summary page, selective-precision passage: the
// router computes in float32 even in a bfloat16 model).
//
// dlogit is fp32.  It enters the bf16 MFMA as two bf16 planes, hi = bf16(v) and
// lo = bf16(v - hi), whose sum carries 16 significant bits; x and W_g are bf16,
// so each product is exact in fp32 and the contraction is accurate to fp32
// accumulation.  Planes are [T][NP] with NP = N rounded up to 64 (zero columns).
//
// dW_g: workgroups own (64 experts x 64 model columns, one token chunk); both
// operands sit in LDS as [token][64] tiles and are read with transposing reads
// (8 consecutive tokens per lane); the chunk partials [S][N][d] are summed in a
// fixed order by a second kernel.  dx: workgroups own 64 tokens x 64 columns;
// W_g chunks of 64 experts sit in LDS (transposing reads), the dlogit rows are
// read straight from memory (8 consecutive experts per lane), and the epilogue
// adds the expert, pass-through and shared-expert terms before one rounding.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

typedef short v4i16_r __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_r lds_v4i16_r;

__device__ __forceinline__ u32x2 tr_read_r(const unsigned char* lds) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_r*)lds));
}

// byte offset of 16-byte chunk q of row m in a [rows][64] bf16 LDS tile (the
// swizzle keeps 16-row direct reads and 4-row transposing reads conflict-free)
__device__ __forceinline__ int rlds_off(int m, int q) {
  const int g = ((m >> 2) & 3) | (((m >> 1) & 1) << 2);
  return m * 128 + ((q ^ g) << 4);
}

// transposing-read address: k-step rows 8 kg + 4 h + (c >> 2), columns 16 t + 4 (c & 3)
__device__ __forceinline__ int rtr_off(int row0, int kg, int h, int c, int t) {
  const int m = row0 + 8 * kg + 4 * h + (c >> 2);
  const int col = 16 * t + 4 * (c & 3);
  return rlds_off(m, col >> 3) + ((col >> 2) & 1) * 8;
}

}  // namespace

// One wave per token: dlogit (fp32 [T][N]) and its hi / lo bf16 planes
// ([T][NP], zero beyond N).
__global__ __launch_bounds__(256) void router_split(const float* __restrict__ dlogit, int64_t T, int N, int NP,
                                                    uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int i = lane; i < NP; i += 64) {
    const float v = i < N ? dlogit[t * N + i] : 0.f;
    const uint32_t h = f2bf(v);
    hi[t * NP + i] = (uint16_t)h;
    lo[t * NP + i] = (uint16_t)f2bf(v - bf2f(h));
  }
}

// partial[s][i][k] = sum over tokens t of chunk s of (hi + lo)[t][i] x[t][k];
// block (ib, kb, s): experts 64 ib .., columns 64 kb .., tokens s * TC ..
// Computed transposed (rows k, columns i) so that each lane stores 4
// consecutive k of one expert (16 bytes).
__global__ __launch_bounds__(256) void router_dwg_partial(const uint16_t* __restrict__ hi,
                                                          const uint16_t* __restrict__ lo,
                                                          const uint16_t* __restrict__ x, int64_t T, int N, int NP,
                                                          int d, int TC, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) unsigned char xs[32 * 128], hs[32 * 128], ls[32 * 128];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4, w = tid >> 6;
  const int i0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int64_t t0 = (int64_t)blockIdx.z * TC;
  int64_t t1 = t0 + TC;
  if (t1 > T) t1 = T;
  f32x4 acc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  // thread -> (row r, chunk q) of the 32 x 64 tiles
  const int r = tid >> 3, q = tid & 7;
  for (int64_t tb = t0; tb < t1; tb += 32) {
    const int64_t t = tb + r;
    u32x4 vx = {0u, 0u, 0u, 0u}, vh = vx, vl = vx;
    if (t < t1) {
      vx = *reinterpret_cast<const u32x4*>(x + t * d + k0 + q * 8);
      vh = *reinterpret_cast<const u32x4*>(hi + t * NP + i0 + q * 8);
      vl = *reinterpret_cast<const u32x4*>(lo + t * NP + i0 + q * 8);
    }
    __syncthreads();  // the previous step's reads are done
    *reinterpret_cast<u32x4*>(xs + rlds_off(r, q)) = vx;
    *reinterpret_cast<u32x4*>(hs + rlds_off(r, q)) = vh;
    *reinterpret_cast<u32x4*>(ls + rlds_off(r, q)) = vl;
    __syncthreads();
    // A = x^T (rows k: this wave's 16 columns), B = dlogit (columns i: 4 tiles)
    u32x2 a0 = tr_read_r(xs + rtr_off(0, kg, 0, c, w)), a1 = tr_read_r(xs + rtr_off(0, kg, 1, c, w));
    const u32x4 af = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      u32x2 b0 = tr_read_r(hs + rtr_off(0, kg, 0, c, it)), b1 = tr_read_r(hs + rtr_off(0, kg, 1, c, it));
      acc[it] = mfma_bf16_16x16x32(af, u32x4{b0[0], b0[1], b1[0], b1[1]}, acc[it]);
      b0 = tr_read_r(ls + rtr_off(0, kg, 0, c, it));
      b1 = tr_read_r(ls + rtr_off(0, kg, 1, c, it));
      acc[it] = mfma_bf16_16x16x32(af, u32x4{b0[0], b0[1], b1[0], b1[1]}, acc[it]);
    }
  }
  // lane: rows k = k0 + 16 w + 4 kg + j, column i = i0 + 16 it + c
  float* base = partial + (int64_t)blockIdx.z * N * d;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = i0 + 16 * it + c;
    if (i < N) *reinterpret_cast<f32x4*>(base + (int64_t)i * d + k0 + 16 * w + 4 * kg) = acc[it];
  }
}

// dW_g[i][k] = sum_s partial[s][i][k], ascending s
__global__ __launch_bounds__(256) void router_dwg_reduce(const float* __restrict__ partial, int S, int64_t n,
                                                         float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int p = 0; p < S; ++p) s += partial[(int64_t)p * n + j];
  out[j] = s;
}

// dx for 64 tokens x 64 columns: dx^T[k][t] = sum_i W_g[i][k] (hi + lo)[t][i],
// then + dX_e[e_t, slot_t] (kept) + dy_t (dropped, or all with the residual
// flag) + dx_shared_t, rounded once to bf16.
__global__ __launch_bounds__(256) void router_dx(const uint16_t* __restrict__ hi, const uint16_t* __restrict__ lo,
                                                 const uint16_t* __restrict__ wg, const float* __restrict__ dxe,
                                                 const uint16_t* __restrict__ dy, const float* __restrict__ dxs,
                                                 const int32_t* __restrict__ eid, const int32_t* __restrict__ slot,
                                                 int64_t T, int d, int N, int NP, int C, int residual_all,
                                                 uint16_t* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) unsigned char ws_[64 * 128];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int k0 = blockIdx.y * 64;
  const int64_t tok = t0 + 16 * w + c;  // this lane's token (B column)
  const bool tok_ok = tok < T;
  f32x4 acc[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ib = 0; ib < NP; ib += 64) {
    __syncthreads();
    for (int p = tid; p < 64 * 8; p += 256) {  // W_g rows ib .. ib+63, columns k0 .. k0+63
      const int r = p >> 3, q = p & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ib + r < N) v = *reinterpret_cast<const u32x4*>(wg + (int64_t)(ib + r) * d + k0 + q * 8);
      *reinterpret_cast<u32x4*>(ws_ + rlds_off(r, q)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 bh = {0u, 0u, 0u, 0u}, bl = bh;
      if (tok_ok) {
        bh = *reinterpret_cast<const u32x4*>(hi + tok * NP + ib + 32 * ks + 8 * kg);
        bl = *reinterpret_cast<const u32x4*>(lo + tok * NP + ib + 32 * ks + 8 * kg);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const u32x2 a0 = tr_read_r(ws_ + rtr_off(32 * ks, kg, 0, c, kt));
        const u32x2 a1 = tr_read_r(ws_ + rtr_off(32 * ks, kg, 1, c, kt));
        const u32x4 af = {a0[0], a0[1], a1[0], a1[1]};
        acc[kt] = mfma_bf16_16x16x32(af, bh, acc[kt]);
        acc[kt] = mfma_bf16_16x16x32(af, bl, acc[kt]);
      }
    }
  }
  // lane: columns k = k0 + 16 kt + 4 kg + j of token `tok`
  if (!tok_ok) return;
  const int s = slot[tok];
  const int64_t row = s >= 0 ? (int64_t)eid[tok] * C + s : -1;
  const bool pass = s < 0 || residual_all;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int k = k0 + 16 * kt + 4 * kg;
    float v[4] = {acc[kt][0], acc[kt][1], acc[kt][2], acc[kt][3]};
    if (row >= 0) {
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(dxe + row * d + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += e4[j];
    }
    if (pass) {
      const u32x2 y2 = *reinterpret_cast<const u32x2*>(dy + tok * d + k);
      v[0] += bf2f(y2[0] & 0xffffu);
      v[1] += bf2f(y2[0] >> 16);
      v[2] += bf2f(y2[1] & 0xffffu);
      v[3] += bf2f(y2[1] >> 16);
    }
    if (dxs != nullptr) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(dxs + tok * d + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += s4[j];
    }
    u32x2 o;
    o[0] = pack_bf2(v[0], v[1]);
    o[1] = pack_bf2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(dx + tok * d + k) = o;
  }
}

// ----------------------------------------------------------------------------
RouterBwdPlan router_bwd_plan(int64_t T, int N, int d) {
  RouterBwdPlan p{};
  p.NP = (N + 63) / 64 * 64;
  const int64_t base = (int64_t)(p.NP / 64) * (d / 64);
  // token chunks: enough workgroups to fill the device (>= 1024), chunks of at
  // least 128 tokens (a multiple of 32), at most 64 chunks
  int64_t S = (1024 + base - 1) / base;
  if (S > 64) S = 64;
  int64_t tc = (T + S - 1) / S;
  if (tc < 128) tc = 128;
  tc = (tc + 31) / 32 * 32;
  p.TC = (int)tc;
  p.S = (int)((T + tc - 1) / tc);
  p.planes_bytes = (size_t)T * p.NP * 2;
  p.partial_bytes = (size_t)p.S * N * d * 4;
  return p;
}

hipError_t launch_router_bwd_mfma(const RouterBwdPlan& p, const float* dlogit, const void* x, const void* wg,
                                  const float* dxe, const void* dy, const float* dxs, const int32_t* eid,
                                  const int32_t* slot, int64_t T, int d, int N, int C, int residual_all,
                                  uint16_t* hi, uint16_t* lo, float* partial, float* dw_gate, void* dx,
                                  hipStream_t st) {
  hipLaunchKernelGGL(router_split, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, dlogit, T, N, p.NP, hi, lo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_dwg_partial, dim3((unsigned)(p.NP / 64), (unsigned)(d / 64), (unsigned)p.S), dim3(256), 0,
                     st, hi, lo, static_cast<const uint16_t*>(x), T, N, p.NP, d, p.TC, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = (int64_t)N * d;
  hipLaunchKernelGGL(router_dwg_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, partial, p.S, n, dw_gate);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(router_dx, dim3((unsigned)((T + 63) / 64), (unsigned)(d / 64)), dim3(256), 0, st, hi, lo,
                     static_cast<const uint16_t*>(wg), dxe, static_cast<const uint16_t*>(dy), dxs, eid, slot, T, d,
                     N, p.NP, C, residual_all, static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

}  // namespace swm
