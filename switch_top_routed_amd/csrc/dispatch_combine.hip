// Dispatch into the fixed per-expert buffers and combine back to token order.
//
// Sources: "MoE expert capacity factor and token dropping" page, Where
// capacity comes from (fixed per-expert slots give a static shape) and After
// overflow (overflowing tokens bypass the expert on the residual path);
// "Top-1 Routing" page, Core mechanism (y = E(x), or gate * E(x) in other
// implementations) and Token Dropping; Switch Transformers summary page,
// Switch-layer passage (gate value as the multiplier) and expert-capacity
// passage (dropped tokens pass straight to the next layer).
//
// Both kernels are pure HBM streams: one wave per row, 16-byte vector loads
// and stores, consecutive lanes on consecutive 16-byte chunks of a row.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kRowThreads = 256;  // 4 rows per workgroup

__global__ __launch_bounds__(kRowThreads) void dispatch_rows(const u32x4* __restrict__ x, int64_t T, int chunks,
                                                             const int32_t* __restrict__ token_of_slot,
                                                             const int32_t* __restrict__ kept_count, int N, int C,
                                                             u32x4* __restrict__ expert_in) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row < (int64_t)N * C) {
    const int e = (int)(row / C), s = (int)(row - (int64_t)e * C);
    if (s < kept_count[e]) {
      const int32_t t = token_of_slot[row];
      if (t >= 0 && t < T) {
        const u32x4* src = x + (int64_t)t * chunks;
        u32x4* dst = expert_in + row * chunks;
        for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
      }
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void combine_rows(const u32x4* __restrict__ eo, const u32x4* __restrict__ x,
                                                            const u32x4* __restrict__ sh, int64_t T, int chunks,
                                                            const int32_t* __restrict__ eid,
                                                            const int32_t* __restrict__ slot,
                                                            const float* __restrict__ gate, int N, int C,
                                                            uint32_t flags, u32x4* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int s = slot[t];
  const int e = s >= 0 ? eid[t] : 0;
  const bool kept = s >= 0 && s < C && e >= 0 && e < N;
  const float scale = (flags & SWITCH_GATE_SCALE) ? gate[t] : 1.0f;
  const bool res = (flags & SWITCH_RESIDUAL_ALL) != 0;
  const u32x4* xr = x + t * chunks;
  const u32x4* orow = eo + ((int64_t)e * C + (kept ? s : 0)) * chunks;
  const u32x4* srow = sh ? sh + t * chunks : nullptr;
  u32x4* yr = y + t * chunks;
  const bool need_x = !kept || res;  // a kept token without the residual flag never reads x
  constexpr int U = 4;               // chunks per lane in flight
  for (int c0 = lane; c0 < chunks; c0 += 64 * U) {
    u32x4 xv[U], ov[U], sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      const bool in = c < chunks;
      xv[u] = (in && need_x) ? xr[c] : u32x4{0u, 0u, 0u, 0u};
      ov[u] = (in && kept) ? orow[c] : u32x4{0u, 0u, 0u, 0u};
      sv[u] = (in && sh) ? srow[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= chunks) break;
      if (!kept && !sh) {
        yr[c] = xv[u];  // dropped token: bit copy of its input
        continue;
      }
      float v[BF16 ? 8 : 4];
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = bf2f(xv[u][q] & 0xffffu);
          v[2 * q + 1] = bf2f(xv[u][q] >> 16);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __uint_as_float(xv[u][q]);
      }
      if (kept) {
        float o[BF16 ? 8 : 4];
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[2 * q] = bf2f(ov[u][q] & 0xffffu);
            o[2 * q + 1] = bf2f(ov[u][q] >> 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = __uint_as_float(ov[u][q]);
        }
#pragma unroll
        for (int q = 0; q < (BF16 ? 8 : 4); ++q) v[q] = res ? v[q] + scale * o[q] : scale * o[q];
      }
      if (sh) {
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] += bf2f(sv[u][q] & 0xffffu);
            v[2 * q + 1] += bf2f(sv[u][q] >> 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] += __uint_as_float(sv[u][q]);
        }
      }
      u32x4 out;
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = pack_bf2(v[2 * q], v[2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(v[q]);
      }
      yr[c] = out;
    }
  }
}

hipError_t launch_dispatch(const void* x, int dtype, int64_t T, int d, const int32_t* token_of_slot,
                           const int32_t* kept_count, int N, int C, void* expert_in, hipStream_t st) {
  const int esz = dtype == 1 ? 2 : 4;
  const int chunks = d * esz / 16;
  const int64_t rows = (int64_t)N * C;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  hipLaunchKernelGGL(dispatch_rows, dim3(grid), dim3(kRowThreads), 0, st, static_cast<const u32x4*>(x), T, chunks,
                     token_of_slot, kept_count, N, C, static_cast<u32x4*>(expert_in));
  return hipGetLastError();
}

hipError_t launch_combine(const void* expert_out, const void* x, const void* shared_out, int dtype, int64_t T, int d,
                          const int32_t* expert_id, const int32_t* slot, const float* gate, int N, int C,
                          uint32_t flags, void* y, hipStream_t st) {
  const int esz = dtype == 1 ? 2 : 4;
  const int chunks = d * esz / 16;
  const unsigned grid = (unsigned)((T + 3) / 4);
  auto* eo = static_cast<const u32x4*>(expert_out);
  auto* xx = static_cast<const u32x4*>(x);
  auto* sh = static_cast<const u32x4*>(shared_out);
  auto* yy = static_cast<u32x4*>(y);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_rows<true>, dim3(grid), dim3(kRowThreads), 0, st, eo, xx, sh, T, chunks, expert_id,
                       slot, gate, N, C, flags, yy);
  else
    hipLaunchKernelGGL(combine_rows<false>, dim3(grid), dim3(kRowThreads), 0, st, eo, xx, sh, T, chunks, expert_id,
                       slot, gate, N, C, flags, yy);
  return hipGetLastError();
}

}  // namespace swm
