// Expert FFN: out[e, s] = ReLU(in[e, s] . W1[e]) . W2[e] over the filled slots
// of the active experts only.
//
// Source: "Top-1 Routing" page, Key parameters and compute (each expert is a
// two-layer FFN, biases ignored; 2 x d_model x d_ff weights per expert); the
// activation is ReLU.  "MoE expert capacity factor and token dropping" page,
// Where capacity comes from (the grouped GEMM runs on the fixed [N, C, d]
// buffers).
//
// bf16 kernel (both GEMMs): a weight-streaming grouped GEMM on MFMA
// v_mfma_f32_16x16x32_bf16.  With at most C tokens per expert the GEMMs read
// every weight byte once for a few dozen FLOPs, so they are bound by HBM on the
// weights; the kernel is built to stream them:
//  * W is row-major [K][Ncols] (Ncols contiguous), but an MFMA operand wants
//    8 consecutive k per lane.  Lane l (c = l & 15, kg = l >> 4) loads the 16
//    bytes at columns 8c..8c+7 of the 8 rows 8kg..8kg+7 of a 32 x 128 weight
//    block (8 fully used 256-byte row segments per instruction across the
//    wave), then transposes that 8 x 8 bf16 tile in registers.  Column j of
//    the tile becomes the B operand of MFMA j, whose 16 output columns are the
//    physical columns 8c + j: the weights never touch LDS, and the 8
//    accumulators of a lane hold 8 consecutive output columns of one row, so
//    the results leave as 16-byte stores.
//  * A = token rows (k contiguous), 16 rows per MFMA tile, up to MT tiles per
//    item.  Rows at or beyond kept_count are neither loaded nor stored, and
//    tiles beyond kept_count are skipped, so empty capacity slots cost nothing.
//  * Work item = (active expert, m-chunk of MT*16 rows, 128-column block,
//    k-split).  The 4 waves of a workgroup take every 4th 32-deep k-step of
//    the item and meet in LDS (fixed-order sum).  Workgroups are persistent and
//    walk the item list.  When few experts are active (skewed routing, decode
//    batches) the items are also split along K so that ~1k items exist; each
//    split writes an fp32 partial tile and the last workgroup to finish a tile
//    (agent-scope counter) sums the partials in split order and applies the
//    epilogue.  The split factor is derived on the device from n_active, so
//    nothing is synchronised with the host.
// fp32 kernel: plain fp32 FMA, one workgroup per (slot row, expert).
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kFfnThreads = 256;

// in[r] = 8 bf16 of row r (two per dword); out[j] = the 8 rows of column j
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = in[2 * q][p], b = in[2 * q + 1][p];
      out[2 * p][q] = (a & 0xffffu) | (b << 16);
      out[2 * p + 1][q] = (a >> 16) | (b & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ void load_wblock(u32x4 (&br)[8], const uint16_t* p, int64_t ld) {
#pragma unroll
  for (int r = 0; r < 8; ++r) br[r] = *reinterpret_cast<const u32x4*>(p + r * ld);
}

__device__ __forceinline__ u32x4 pack8(const float (&v)[8], bool relu) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float lo = v[2 * q], hi = v[2 * q + 1];
    if (relu) {
      lo = fmaxf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
    }
    o[q] = pack_bf2(lo, hi);
  }
  return o;
}

// split factor along K, identical in every workgroup of a launch
__device__ __forceinline__ int split_factor(int64_t base, int target, int smax, int ksteps, int64_t part_tiles) {
  if (base <= 0 || base >= target) return 1;
  int64_t s = (target + base - 1) / base;
  if (s > smax) s = smax;
  if (s > ksteps / 4) s = ksteps / 4;
  if (s > part_tiles / base) s = part_tiles / base;
  return s < 1 ? 1 : (int)s;
}

// phase 1: H = ReLU(X . W1) (K = d_model, Ncols = d_ff)
// phase 2: Y = H . W2      (K = d_ff,    Ncols = d_model)
// Phase 1 with a K split leaves fp32 partial tiles in part1 and no bf16 H; phase
// 2 then sums those partials (split order), applies ReLU and rounds to bf16 as
// it loads its A operand.  Phase 1 also clears the phase-2 tile counters.
template <int MT>
__global__ __launch_bounds__(kFfnThreads, MT <= 2 ? 2 : 1) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
    float* __restrict__ part1, float* __restrict__ part2, int32_t* __restrict__ cnt2, int64_t n_cnt2,
    const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    int N, int C, int K, int Ncols, int phase, int mch, int target, int smax, int64_t part_tiles) {
  __shared__ float red[4 * 4 * 8 * 64];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, kg = lane >> 4;
  if (phase == 1)
    for (int64_t i = (int64_t)blockIdx.x * kFfnThreads + tid; i < n_cnt2; i += (int64_t)gridDim.x * kFfnThreads)
      cnt2[i] = 0;
  const int NCB = Ncols >> 7;
  int n_act = n_active[0];
  if (n_act > N) n_act = N;
  const int ksteps = K >> 5;
  const int64_t base = (int64_t)n_act * NCB * mch;
  if (base <= 0) return;
  const int S = split_factor(base, target, smax, ksteps, part_tiles);
  // phase 2: how phase 1 was split (its K = Ncols here, its Ncols = K here)
  const int S1 = phase == 2 ? split_factor((int64_t)n_act * (K >> 7) * mch, target, smax, Ncols >> 5, part_tiles) : 1;
  const bool relu_out = phase == 1;
  const int64_t items = base * S;
  constexpr int kTile = MT * 16 * 128;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  float* part = phase == 1 ? part1 : part2;

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int mc = (int)(item % mch);
    int64_t r = item / mch;
    const int s = (int)(r % S);
    r /= S;
    const int cb = (int)(r % NCB);
    const int a = (int)(r / NCB);
    const int64_t tile = ((int64_t)a * NCB + cb) * mch + mc;
    const int e = active[a];
    if (e < 0 || e >= N) continue;
    const int m0 = mc * MT * 16;
    int kept = kept_count[e];
    if (kept > C) kept = C;
    int rows = kept - m0;
    if (rows > MT * 16) rows = MT * 16;
    if (rows <= 0) continue;
    const int mtc = (rows + 15) >> 4;
    const int ks0 = (int)((int64_t)ksteps * s / S), ks1 = (int)((int64_t)ksteps * (s + 1) / S);

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int rr = mt * 16 + c;
      aval[mt] = rr < rows;
      arow[mt] = A + ((int64_t)e * C + m0 + (aval[mt] ? rr : 0)) * K + kg * 8;
    }
    // phase-1 partial tiles of this expert / m-chunk: tile1 = (a * (K/128) + ks/4) * mch + mc
    const float* p1 = part1 + (((int64_t)a * (K >> 7)) * mch + mc) * S1 * kTile;
    const uint16_t* wb = W + (int64_t)e * K * Ncols + (int64_t)(kg * 8) * Ncols + cb * 128 + c * 8;

    int ks = ks0 + w;
    u32x4 br[8];
    if (ks < ks1) load_wblock(br, wb + (int64_t)ks * 32 * Ncols, Ncols);
    for (; ks < ks1; ks += 4) {
      u32x4 av[MT];
      if (S1 == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = (mt < mtc && aval[mt]) ? *reinterpret_cast<const u32x4*>(arow[mt] + ks * 32) : zero;
      } else {
        const float* pk = p1 + (int64_t)(ks >> 2) * mch * S1 * kTile + (ks & 3) * 32 + kg * 8;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          av[mt] = zero;
          if (mt < mtc && aval[mt]) {
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const float* pr = pk + (mt * 16 + c) * 128;
            for (int s1 = 0; s1 < S1; ++s1) {
              const f32x4 q0 = *reinterpret_cast<const f32x4*>(pr + (int64_t)s1 * kTile);
              const f32x4 q1 = *reinterpret_cast<const f32x4*>(pr + (int64_t)s1 * kTile + 4);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] += q0[q];
                v[4 + q] += q1[q];
              }
            }
            av[mt] = pack8(v, true);
          }
        }
      }
      u32x4 bn[8];
      if (ks + 4 < ks1) load_wblock(bn, wb + (int64_t)(ks + 4) * 32 * Ncols, Ncols);
      u32x4 bt[8];
      transpose8x8(br, bt);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mtc) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[mt][j] = mfma_bf16_16x16x32(av[mt], bt[j], acc[mt][j]);
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) br[q] = bn[q];
    }

    // cross-wave sum in LDS, one 16-row tile at a time; wave w finishes row 4*kg + w
    const int rl_base = kg * 4 + w;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mtc) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((w * 4 + i) * 8 + j) * 64 + lane] = acc[mt][j][i];
        __syncthreads();
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = ((red[((0 * 4 + w) * 8 + j) * 64 + lane] + red[((1 * 4 + w) * 8 + j) * 64 + lane]) +
                  red[((2 * 4 + w) * 8 + j) * 64 + lane]) +
                 red[((3 * 4 + w) * 8 + j) * 64 + lane];
        __syncthreads();
        const int rl = mt * 16 + rl_base;
        if (rl < rows) {
          if (S == 1) {
            *reinterpret_cast<u32x4*>(out + ((int64_t)e * C + m0 + rl) * Ncols + cb * 128 + c * 8) =
                pack8(v, relu_out);
          } else {
            float* pp = part + (tile * S + s) * kTile + rl * 128 + c * 8;
            *reinterpret_cast<f32x4*>(pp) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(pp + 4) = f32x4{v[4], v[5], v[6], v[7]};
          }
        }
      }
    }
    if (S > 1 && phase == 2) {
      // the last of the S workgroups of this tile sums the partials in split order
      __threadfence();
      __syncthreads();
      if (tid == 0) s_last = (atomicAdd(&cnt2[tile], 1) == S - 1) ? 1 : 0;
      __syncthreads();
      if (s_last) {
        __threadfence();
        for (int idx = tid; idx < rows * 16; idx += kFfnThreads) {
          const int rl = idx >> 4, cc = (idx & 15) * 8;
          float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int s2 = 0; s2 < S; ++s2) {
            const float* pp = part + (tile * S + s2) * kTile + rl * 128 + cc;
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(pp);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(pp + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] += q0[q];
              v[4 + q] += q1[q];
            }
          }
          *reinterpret_cast<u32x4*>(out + ((int64_t)e * C + m0 + rl) * Ncols + cb * 128 + cc) = pack8(v, false);
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void ffn_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                    float* __restrict__ out, const int32_t* __restrict__ kept_count,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, int N, int C, int K,
                                                    int Ncols, int relu) {
  const int a = blockIdx.y;
  if (a >= n_active[0]) return;
  const int e = active[a];
  if (e < 0 || e >= N) return;
  const int row = blockIdx.x;
  if (row >= kept_count[e] || row >= C) return;
  const float* ar = A + ((int64_t)e * C + row) * K;
  const float* wb = W + (int64_t)e * K * Ncols;
  float* orow = out + ((int64_t)e * C + row) * Ncols;
  for (int col = threadIdx.x; col < Ncols; col += 256) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(ar[k], wb[(int64_t)k * Ncols + col], acc);
    orow[col] = relu ? fmaxf(acc, 0.f) : acc;
  }
}

__global__ void dense_plan(int32_t* kept, int32_t* active, int32_t* n_active, int32_t M) {
  if (threadIdx.x == 0) {
    kept[0] = M;
    active[0] = 0;
    n_active[0] = 1;
  }
}

// ----------------------------------------------------------------------------
FfnPlan ffn_plan(int N, int C, int d, int dff, int dtype) {
  FfnPlan pl{};
  size_t off = 0;
  const size_t esz = dtype == 1 ? 2 : 4;
  pl.off_h = off;
  off = align_up(off + (size_t)N * C * dff * esz);
  if (dtype == 1) {
    pl.mt = C <= 16 ? 1 : C <= 32 ? 2 : C <= 48 ? 3 : 4;
    pl.mch = (C + pl.mt * 16 - 1) / (pl.mt * 16);
    pl.grid = 1024;
    pl.target = 1024;
    pl.smax = 16;
    // a split only happens when base < target, so base * S < 2 * target tiles
    pl.part_tiles = 2 * (int64_t)pl.target;
    pl.n_counters = (int64_t)N * (d / 128) * pl.mch;
    const size_t part_bytes = (size_t)pl.part_tiles * pl.mt * 16 * 128 * 4;
    pl.off_part = off;
    off = align_up(off + part_bytes);
    pl.off_part2 = off;
    off = align_up(off + part_bytes);
    pl.off_cnt2 = off;
    off = align_up(off + (size_t)pl.n_counters * 4);
  }
  pl.bytes = off;
  return pl;
}

hipError_t launch_dense_plan(int32_t* kept, int32_t* active, int32_t* n_active, int32_t M, hipStream_t st) {
  hipLaunchKernelGGL(dense_plan, dim3(1), dim3(64), 0, st, kept, active, n_active, M);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_gemm(const FfnPlan& pl, const void* A, const void* W, void* out, char* ws,
                              const int32_t* kept, const int32_t* active, const int32_t* n_active, int N, int C, int K,
                              int Ncols, int phase, hipStream_t st) {
  hipLaunchKernelGGL((ffn_gemm_bf16<MT>), dim3(pl.grid), dim3(kFfnThreads), 0, st, static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(out),
                     reinterpret_cast<float*>(ws + pl.off_part), reinterpret_cast<float*>(ws + pl.off_part2),
                     reinterpret_cast<int32_t*>(ws + pl.off_cnt2), pl.n_counters, kept, active, n_active, N, C, K,
                     Ncols, phase, pl.mch, pl.target, pl.smax, pl.part_tiles);
  return hipGetLastError();
}

static hipError_t gemm_bf16(const FfnPlan& pl, const void* A, const void* W, void* out, char* ws, const int32_t* kept,
                            const int32_t* active, const int32_t* n_active, int N, int C, int K, int Ncols, int phase,
                            hipStream_t st) {
  switch (pl.mt) {
    case 1: return launch_gemm<1>(pl, A, W, out, ws, kept, active, n_active, N, C, K, Ncols, phase, st);
    case 2: return launch_gemm<2>(pl, A, W, out, ws, kept, active, n_active, N, C, K, Ncols, phase, st);
    case 3: return launch_gemm<3>(pl, A, W, out, ws, kept, active, n_active, N, C, K, Ncols, phase, st);
    default: return launch_gemm<4>(pl, A, W, out, ws, kept, active, n_active, N, C, K, Ncols, phase, st);
  }
}

hipError_t launch_ffn(const FfnPlan& pl, const void* xin, const void* w1, const void* w2, int dtype, int N, int C, int d,
                      int dff, const int32_t* kept_count, const int32_t* active, const int32_t* n_active, void* xout,
                      char* ws, hipStream_t st) {
  void* h = ws + pl.off_h;
  if (dtype == 0) {
    hipLaunchKernelGGL(ffn_gemm_f32, dim3((unsigned)C, (unsigned)N), dim3(256), 0, st, static_cast<const float*>(xin),
                       static_cast<const float*>(w1), static_cast<float*>(h), kept_count, active, n_active, N, C, d,
                       dff, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ffn_gemm_f32, dim3((unsigned)C, (unsigned)N), dim3(256), 0, st, static_cast<const float*>(h),
                       static_cast<const float*>(w2), static_cast<float*>(xout), kept_count, active, n_active, N, C,
                       dff, d, 0);
    return hipGetLastError();
  }
  hipError_t e = gemm_bf16(pl, xin, w1, h, ws, kept_count, active, n_active, N, C, d, dff, 1, st);
  if (e != hipSuccess) return e;
  return gemm_bf16(pl, h, w2, xout, ws, kept_count, active, n_active, N, C, dff, d, 2, st);
}

}  // namespace swm
