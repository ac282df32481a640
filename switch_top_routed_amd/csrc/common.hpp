// Internal device helpers for the gfx950 kernels (wave64, MFMA).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// Wave reductions on DPP lane moves (no LDS traffic; a ds_bpermute shuffle
// costs an LDS round trip per step): quad swaps (lane ^ 1, lane ^ 2), the half-
// row and row mirrors (the 8- and 16-lane groups), then row broadcasts of lanes
// 15 and 31 into the rows above.  Lane 63 ends with the whole wave's result,
// which is read back as a wave-uniform value, so every lane returns the same
// bits.  All 64 lanes must be active.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_move(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppBcast15 = 0x142, kDppBcast31 = 0x143;

__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(dpp_move<kDppQuadXor1>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppQuadXor2>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppHalfMirror>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppMirror>(0, __float_as_int(v)));
  v += __int_as_float(dpp_move<kDppBcast15, 0xa>(0, __float_as_int(v)));  // rows 1, 3 (+0 elsewhere)
  v += __int_as_float(dpp_move<kDppBcast31, 0xc>(0, __float_as_int(v)));  // rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_int(int v) {
  v += dpp_move<kDppQuadXor1>(0, v);
  v += dpp_move<kDppQuadXor2>(0, v);
  v += dpp_move<kDppHalfMirror>(0, v);
  v += dpp_move<kDppMirror>(0, v);
  v += dpp_move<kDppBcast15, 0xa>(0, v);
  v += dpp_move<kDppBcast31, 0xc>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}

// (value, index) arg-max over the wave; equal values resolve to the lower index.
// Lanes a broadcast step does not write get their own pair back (no change).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& idx) {
  const float ov = __int_as_float(dpp_move<CTRL, ROW_MASK>(__float_as_int(v), __float_as_int(v)));
  const int oi = dpp_move<CTRL, ROW_MASK>(idx, idx);
  if (ov > v || (ov == v && oi < idx)) {
    v = ov;
    idx = oi;
  }
}
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
  argmax_step<kDppQuadXor1, 0xf>(v, idx);
  argmax_step<kDppQuadXor2, 0xf>(v, idx);
  argmax_step<kDppHalfMirror, 0xf>(v, idx);
  argmax_step<kDppMirror, 0xf>(v, idx);
  argmax_step<kDppBcast15, 0xa>(v, idx);
  argmax_step<kDppBcast31, 0xc>(v, idx);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  idx = __builtin_amdgcn_readlane(idx, 63);
}

// hist[digit] += 1 for every active lane (digit < 256); the lanes of a wave
// with the same digit are counted together, one LDS atomic per distinct digit
// and wave.  Every lane of the wave must call it.
__device__ __forceinline__ void hist_add_wave(int* hist, uint32_t digit, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t same = __ballot(active);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (digit >> b) & 1u;
    const uint64_t m = __ballot(active && bit);
    same &= bit ? m : ~m;
  }
  if (active && __ffsll((unsigned long long)same) - 1 == lane) atomicAdd(&hist[digit], __popcll(same));
}

// One step of a descending radix select over a 256-bin histogram in LDS, run
// by all 64 lanes of one wave: the bin that holds the need-th largest key
// (1-based, counting from bin 255 down) and need minus the keys in the bins
// above it.  Bin 0 takes whatever remains.  The result is the same on every
// lane.
__device__ __forceinline__ void radix_pick_desc(const int* hist, int need, int* bin, int* rem) {
  const int lane = threadIdx.x & 63;
  int h[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // lane l holds bins 255 - 4l .. 252 - 4l
    h[q] = hist[255 - 4 * lane - q];
    s += h[q];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  int run = incl - s, b = 0, r = 0;
  bool found = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bq = 255 - 4 * lane - q;
    if (!found && (bq == 0 || run + h[q] >= need)) {
      b = bq;
      r = need - run;
      found = true;
    }
    if (!found) run += h[q];
  }
  const uint64_t ok = __ballot(incl >= need);
  const int L = ok ? __ffsll((unsigned long long)ok) - 1 : 63;
  *bin = __shfl(b, L, kWave);
  *rem = __shfl(r, L, kWave);
}

// Exclusive prefix sum over a block of up to 1024 threads (blockDim.x multiple
// of 64).  `wsum` is LDS scratch of >= 16 ints.  Returns the exclusive prefix;
// *total receives the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int s = wsum[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Register transposes of bf16 tiles (for B operands stored [K][N]).
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

// in[r] = 4 bf16 of row r (two per dword); out[j] = the 8 rows of column j
__device__ __forceinline__ void transpose8x4(const u32x2 (&in)[8], u32x4 (&out)[4]) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = in[2 * q][p], b = in[2 * q + 1][p];
      out[2 * p][q] = (a & 0xffffu) | (b << 16);
      out[2 * p + 1][q] = (a >> 16) | (b & 0xffff0000u);
    }
  }
}

}  // namespace swm
