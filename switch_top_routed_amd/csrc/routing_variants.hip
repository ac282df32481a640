// Routing variants next to top-1 ("Top-1 Routing" page, introduction and
// Variants section): top-K token choice (each token picks its K highest-logit
// experts; top-2 as in GShard) and expert choice (each expert picks its top
// tokens, balanced by construction).  Capacity, buffers and the expert FFN are
// those of the top-1 layer.
//
// Top-K: the router writes each token's K choices also in choice-major order
// (j * T + t), so the slot assignment of the top-1 layer ranks the K T
// assignments as one list of "virtual tokens" (every first choice before every
// second choice under token order); topk_fixup turns virtual indices back into
// token rows and [T, K] slots.
// Expert choice: ec_select gives each expert its min(C, T) highest-probability
// tokens (ties to the lower token), ranked by descending probability: a 4-pass
// 8-bit radix select of the threshold on the fp32 bit patterns (positive floats
// order like their bits), an ordered compaction of the tokens above it (and of
// the lowest-index tokens equal to it), and ranks by counting.  Integer LDS
// atomics only count; every output position comes from a scan, so the result
// is deterministic.
// combine_picks sums each token's kept picks in pick order (choice j, or expert
// index), with the gate or 1, in fp32; a token without a kept pick passes
// through unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kMaxPicks = 1024;  // picks per token: K (top-K) or up to N (expert choice)

// slot[t * K + j] = slot_v[j * T + t]; token_of_slot entries v -> v mod T
__global__ __launch_bounds__(256) void topk_fixup(const int32_t* __restrict__ slot_v, int64_t T, int K,
                                                  int32_t* __restrict__ tos, int64_t NC, int32_t* __restrict__ slot) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < T * K) {
    const int64_t t = i / K, j = i - t * K;
    slot[i] = slot_v[j * T + t];
  }
  if (i < NC) {
    const int32_t v = tos[i];
    if (v >= 0) tos[i] = (int32_t)(v % T);
  }
}

// pick[t][i] = -1 for every (t, i); n_dropped = 0
__global__ __launch_bounds__(256) void ec_clear(int32_t* __restrict__ pick, int64_t n, int32_t* __restrict__ n_dropped) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) pick[i] = -1;
  if (i == 0) n_dropped[0] = 0;
}

// One workgroup (1024 threads) per expert i over its probability row
// probs_t[i][0..T): token_of_slot[i][rank], pick[t][i] = rank, kept_count[i],
// active[i] = i (every expert is full).
__global__ __launch_bounds__(1024) void ec_select(const float* __restrict__ probs_t, int64_t T, int N, int C,
                                                  int32_t* __restrict__ tos, int32_t* __restrict__ pick,
                                                  int32_t* __restrict__ kept_count, int32_t* __restrict__ active,
                                                  int32_t* __restrict__ n_active) {
  extern __shared__ uint32_t ec_lds[];  // sel_key[k], sel_tok[k]
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need, s_base, s_eqbase;
  const int e = blockIdx.x, tid = threadIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(probs_t) + (int64_t)e * T;
  const int k = (int)(T < C ? T : C);
  uint32_t* sel_key = ec_lds;
  int* sel_tok = reinterpret_cast<int*>(ec_lds + k);

  // ---- radix select: the k-th largest key (with multiplicity) ----
  if (tid == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_need = k;  // rank (1-based, from the top) still to locate inside the current prefix
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += 1024) hist[b] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int64_t t0 = 0; t0 < T; t0 += 1024) {  // the same trip count on every lane
      const int64_t t = t0 + tid;
      const uint32_t v = t < T ? key[t] : 0u;
      hist_add_wave(hist, (v >> shift) & 255u, t < T && (v & mask) == prefix);
    }
    __syncthreads();
    if (tid < 64) {
      int b, need;
      radix_pick_desc(hist, s_need, &b, &need);
      if (tid == 0) {
        s_need = need;
        s_prefix = prefix | ((uint32_t)b << shift);
        s_mask = mask | (255u << shift);
      }
    }
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int eq_take = s_need;  // how many keys equal to thr are taken (lowest tokens first)

  // ---- ordered compaction: keys > thr, and the first eq_take keys == thr ----
  if (tid == 0) {
    s_base = 0;
    s_eqbase = 0;
  }
  __syncthreads();
  for (int64_t t0 = 0; t0 < T; t0 += 1024) {
    const int64_t t = t0 + tid;
    const uint32_t v = t < T ? key[t] : 0u;
    const int is_eq = (t < T && v == thr) ? 1 : 0;
    int tot_eq;
    const int eq_rank = s_eqbase + block_exclusive_scan(is_eq, wsum, &tot_eq);
    const int take = (t < T && (v > thr || (is_eq && eq_rank < eq_take))) ? 1 : 0;
    int tot;
    const int pos = s_base + block_exclusive_scan(take, wsum, &tot);
    if (take) {
      sel_key[pos] = v;
      sel_tok[pos] = (int)t;
    }
    __syncthreads();
    if (tid == 0) {
      s_base += tot;
      s_eqbase += tot_eq;
    }
    __syncthreads();
  }

  // ---- ranks by counting: (key descending, token ascending) ----
  for (int a = tid; a < k; a += 1024) {
    const uint32_t ka = sel_key[a];
    const int ta = sel_tok[a];
    int r = 0;
    for (int b = 0; b < k; ++b) {
      const uint32_t kb = sel_key[b];
      r += (kb > ka || (kb == ka && sel_tok[b] < ta)) ? 1 : 0;
    }
    tos[(int64_t)e * C + r] = ta;
    pick[(int64_t)ta * N + e] = r;
  }
  for (int s = k + tid; s < C; s += 1024) tos[(int64_t)e * C + s] = -1;
  if (tid == 0) {
    kept_count[e] = k;
    active[e] = e;
    if (e == 0) n_active[0] = N;
  }
}

// One wave per token.  MODE 0 (top-K): picks (expert_id, slot, gate)[t * K + j];
// MODE 1 (expert choice): pick[t][i] >= 0 with gate probs_t[i][t].  In MODE 1 the
// number of kept picks goes to npick[t] and tokens without one are counted in
// n_dropped (integer atomic: order-independent).
template <bool BF16, int MODE>
__global__ __launch_bounds__(256) void combine_picks(const u32x4* __restrict__ expert_out, const u32x4* __restrict__ x,
                                                     const u32x4* __restrict__ shared, int64_t T, int chunks, int K,
                                                     const int32_t* __restrict__ eid, const int32_t* __restrict__ slot,
                                                     const float* __restrict__ gate, const int32_t* __restrict__ pick,
                                                     const float* __restrict__ probs_t, int N, int C, uint32_t flags,
                                                     int32_t* __restrict__ npick, int32_t* __restrict__ n_dropped,
                                                     u32x4* __restrict__ y) {
  __shared__ int pk_e[4][kMaxPicks];
  __shared__ int pk_s[4][kMaxPicks];
  __shared__ float pk_g[4][kMaxPicks];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  if (t >= T) return;
  const bool gs = (flags & SWITCH_GATE_SCALE) != 0, res = (flags & SWITCH_RESIDUAL_ALL) != 0;
  // this token's kept picks, in pick order
  int np = 0;
  if (MODE == 0) {
    for (int j = 0; j < K; ++j) {
      const int s = slot[t * K + j];
      if (s >= 0) {
        if (lane == 0) {
          pk_e[w][np] = eid[t * K + j];
          pk_s[w][np] = s;
          pk_g[w][np] = gs ? gate[t * K + j] : 1.f;
        }
        ++np;
      }
    }
  } else {
    for (int i0 = 0; i0 < N; i0 += 64) {
      const int i = i0 + lane;
      const int s = i < N ? pick[t * N + i] : -1;
      const uint64_t m = __ballot(s >= 0);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (s >= 0) {
        pk_e[w][np + before] = i;
        pk_s[w][np + before] = s;
        pk_g[w][np + before] = gs ? probs_t[(int64_t)i * T + t] : 1.f;
      }
      np += __popcll(m);
    }
    if (lane == 0) {
      npick[t] = np;
      if (np == 0) atomicAdd(n_dropped, 1);
    }
  }
  // the pick lists are per wave: a wave-scope fence orders this wave's LDS
  // writes before its reads (no workgroup barrier: other waves may have exited)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const u32x4* xr = x + t * chunks;
  const u32x4* sr = shared != nullptr ? shared + t * chunks : nullptr;
  u32x4* yr = y + t * chunks;
  constexpr int EPV = BF16 ? 8 : 4;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 xv = xr[c];
    if (np == 0 && sr == nullptr) {
      yr[c] = xv;  // no kept pick: bit copy of the input
      continue;
    }
    float xf[EPV], acc[EPV];
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xf[2 * q] = bf2f(xv[q] & 0xffffu);
        xf[2 * q + 1] = bf2f(xv[q] >> 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) xf[q] = __uint_as_float(xv[q]);
    }
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    for (int p = 0; p < np; ++p) {
      const u32x4 ov = expert_out[((int64_t)pk_e[w][p] * C + pk_s[w][p]) * chunks + c];
      const float g = pk_g[w][p];
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += g * bf2f(ov[q] & 0xffffu);
          acc[2 * q + 1] += g * bf2f(ov[q] >> 16);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += g * __uint_as_float(ov[q]);
      }
    }
    float v[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) v[q] = np == 0 ? xf[q] : (res ? acc[q] + xf[q] : acc[q]);
    if (sr != nullptr) {
      const u32x4 sv = sr[c];
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += bf2f(sv[q] & 0xffffu);
          v[2 * q + 1] += bf2f(sv[q] >> 16);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += __uint_as_float(sv[q]);
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

// ----------------------------------------------------------------------------
hipError_t launch_topk_fixup(const int32_t* slot_v, int64_t T, int K, int32_t* tos, int64_t NC, int32_t* slot,
                             hipStream_t st) {
  const int64_t n = T * K > NC ? T * K : NC;
  hipLaunchKernelGGL(topk_fixup, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slot_v, T, K, tos, NC, slot);
  return hipGetLastError();
}

size_t ec_select_lds_bytes(int64_t T, int C) {
  const int64_t k = T < C ? T : C;
  return (size_t)k * 8;
}

hipError_t launch_ec_select(const float* probs_t, int64_t T, int N, int C, int32_t* tos, int32_t* pick,
                            int32_t* kept_count, int32_t* active, int32_t* n_active, int32_t* n_dropped,
                            hipStream_t st) {
  const int64_t n = T * N;
  hipLaunchKernelGGL(ec_clear, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pick, n, n_dropped);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ec_select, dim3((unsigned)N), dim3(1024), ec_select_lds_bytes(T, C), st, probs_t, T, N, C, tos,
                     pick, kept_count, active, n_active);
  return hipGetLastError();
}

hipError_t launch_combine_picks(int mode, const void* expert_out, const void* x, const void* shared_out, int dtype,
                                int64_t T, int d, int K, const int32_t* eid, const int32_t* slot, const float* gate,
                                const int32_t* pick, const float* probs_t, int N, int C, uint32_t flags,
                                int32_t* npick, int32_t* n_dropped, void* y, hipStream_t st) {
  const int esz = dtype == 1 ? 2 : 4;
  const int chunks = d * esz / 16;
  const unsigned grid = (unsigned)((T + 3) / 4);
  auto* eo = static_cast<const u32x4*>(expert_out);
  auto* xx = static_cast<const u32x4*>(x);
  auto* sh = static_cast<const u32x4*>(shared_out);
  auto* yy = static_cast<u32x4*>(y);
#define SWM_COMBINE(B, M)                                                                                          \
  hipLaunchKernelGGL((combine_picks<B, M>), dim3(grid), dim3(256), 0, st, eo, xx, sh, T, chunks, K, eid, slot, gate, \
                     pick, probs_t, N, C, flags, npick, n_dropped, yy)
  if (dtype == 1) {
    if (mode == 0) SWM_COMBINE(true, 0);
    else SWM_COMBINE(true, 1);
  } else {
    if (mode == 0) SWM_COMBINE(false, 0);
    else SWM_COMBINE(false, 1);
  }
#undef SWM_COMBINE
  return hipGetLastError();
}

}  // namespace swm
