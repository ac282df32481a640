// Expanded Drop: capacity-aware re-routing of overflow tokens at inference
// ("MoE expert capacity factor and token dropping" page, inference section:
// tokens dropped by a full expert consider further experts of their candidate
// set, so that the spare capacity of lightly loaded experts is used).
//
// Round 0 is the top-1 capacity assignment.  In round r every token still
// without a slot applies to its candidate r (the router's r-th highest logit),
// and each expert fills its free slots with that round's applicants in the
// layer's priority order, after the slots already taken.  One launch per round:
//   expand_round    - one workgroup (1024 threads) per expert finds its
//                     applicants in ascending token order (ballots per wave,
//                     one LDS scan per 16K tokens).  Token order: the first
//                     `free` of them take the slots in that same pass.  Gate
//                     order: the applicants (their keys and tokens in LDS up to
//                     4096 of them, else a list in the workspace) go through a
//                     4-pass 8-bit radix select of the threshold key on the fp32
//                     bit patterns of p (ties go to the lower token, which is
//                     list order; histogram atomics aggregated per wave and
//                     digit), an ordered gather of the taken ones and ranks by
//                     counting.  Integer LDS atomics only count.
//   expand_finalize - the active list, n_active and n_dropped from the final
//                     kept counts.
// Only workgroup i writes expert i's slots, kept count and the rows of its
// applicants (an applicant's candidate r is one expert), so one round's
// workgroups never touch the same data.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {
constexpr int kXdThreads = 1024;
constexpr int kXdWaves = kXdThreads / 64;
constexpr int kXdSub = 16;     // 1024-token chunks per list-building step
constexpr int kXdCache = 4096;  // gate order: applicants whose key and token stay in LDS
}  // namespace

// ev, gv: candidate r of every token and p there (rows r*T of the router's
// choice-major candidate lists).  list: this expert's scratch row [T] (gate
// order only).
__global__ __launch_bounds__(kXdThreads) void expand_round(const int32_t* __restrict__ ev,
                                                           const float* __restrict__ gv, int64_t T, int C,
                                                           int gate_order, int32_t* __restrict__ slot,
                                                           int32_t* __restrict__ expert_id, float* __restrict__ gate,
                                                           int32_t* __restrict__ tos,
                                                           int32_t* __restrict__ kept_count,
                                                           int32_t* __restrict__ list_all) {
  // gate order: akey[kXdCache], atok[kXdCache], then sel_key[room], sel_tok[room]
  extern __shared__ uint32_t xd_lds[];
  __shared__ int woff[kXdSub * kXdWaves];
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ int s_total;
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need, s_base, s_eqbase;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kept0 = kept_count[e];
  const int room = C - kept0;
  if (room <= 0) return;  // uniform over the workgroup
  int32_t* list = list_all + (int64_t)e * T;
  uint32_t* akey = xd_lds;
  int* atok = reinterpret_cast<int*>(xd_lds + kXdCache);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- applicants of this round in ascending token order; with token order
  // the first `room` of them take the free slots right here ----
  int n_app = 0;
  for (int64_t c0 = 0; c0 < T; c0 += (int64_t)kXdSub * kXdThreads) {
    bool f[kXdSub];
    uint64_t m[kXdSub];
#pragma unroll
    for (int j = 0; j < kXdSub; ++j) {
      const int64_t t = c0 + (int64_t)j * kXdThreads + tid;
      f[j] = t < T && ev[t] == e;
    }
#pragma unroll
    for (int j = 0; j < kXdSub; ++j) {
      const int64_t t = c0 + (int64_t)j * kXdThreads + tid;
      f[j] = f[j] && slot[t] < 0;
      m[j] = __ballot(f[j]);
      if (lane == 0) woff[j * kXdWaves + w] = __popcll(m[j]);
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of the 256 counts, chunk-major then wave
      int v[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = woff[lane * 4 + q];
        s += v[q];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      int run = incl - s;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        woff[lane * 4 + q] = run;
        run += v[q];
      }
      if (lane == 63) s_total = incl;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kXdSub; ++j) {
      if (f[j]) {
        const int64_t t = c0 + (int64_t)j * kXdThreads + tid;
        const int pos = n_app + woff[j * kXdWaves + w] + __popcll(m[j] & below);
        if (!gate_order) {
          if (pos < room) {
            const int s = kept0 + pos;
            slot[t] = s;
            tos[(int64_t)e * C + s] = (int32_t)t;
            expert_id[t] = e;
            gate[t] = gv[t];
          }
        } else {
          list[pos] = (int32_t)t;
          if (pos < kXdCache) {
            akey[pos] = __float_as_uint(gv[t]);
            atok[pos] = (int)t;
          }
        }
      }
    }
    n_app += s_total;
    __syncthreads();  // woff and s_total are rewritten by the next step
  }
  const int take = n_app < room ? n_app : room;
  if (!gate_order) {
    if (tid == 0) kept_count[e] = kept0 + take;
    return;
  }
  if (take == 0) return;
  const bool cached = n_app <= kXdCache;
  if (!cached) __threadfence_block();  // the list is read back by other threads of this workgroup
  __syncthreads();
  auto key_at = [&](int a) -> uint32_t { return cached ? akey[a] : __float_as_uint(gv[list[a]]); };
  auto tok_at = [&](int a) -> int { return cached ? atok[a] : list[a]; };

  // ---- the threshold: keys > thr are taken, and the first eq_take keys == thr ----
  uint32_t thr = 0u;
  int eq_take = take;
  if (take < n_app) {
    if (tid == 0) {
      s_prefix = 0u;
      s_mask = 0u;
      s_need = take;
    }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = tid; b < 256; b += kXdThreads) hist[b] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int a0 = 0; a0 < n_app; a0 += kXdThreads) {  // the same trip count on every lane
        const int a = a0 + tid;
        const uint32_t v = a < n_app ? key_at(a) : 0u;
        hist_add_wave(hist, (v >> shift) & 255u, a < n_app && (v & mask) == prefix);
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
    thr = s_prefix;
    eq_take = s_need;
  }

  // ---- ordered gather of the taken applicants ----
  uint32_t* sel_key = xd_lds + 2 * kXdCache;
  int* sel_tok = reinterpret_cast<int*>(sel_key + room);
  if (tid == 0) {
    s_base = 0;
    s_eqbase = 0;
  }
  __syncthreads();
  for (int a0 = 0; a0 < n_app; a0 += kXdThreads) {
    const int a = a0 + tid;
    const uint32_t v = a < n_app ? key_at(a) : 0u;
    const int is_eq = (a < n_app && v == thr) ? 1 : 0;
    int tot_eq;
    const int eq_rank = s_eqbase + block_exclusive_scan(is_eq, wsum, &tot_eq);
    const int tk = (a < n_app && (v > thr || (is_eq && eq_rank < eq_take))) ? 1 : 0;
    int tot;
    const int pos = s_base + block_exclusive_scan(tk, wsum, &tot);
    if (tk) {
      sel_key[pos] = v;
      sel_tok[pos] = tok_at(a);
    }
    __syncthreads();
    if (tid == 0) {
      s_base += tot;
      s_eqbase += tot_eq;
    }
    __syncthreads();
  }

  // ---- slots: rank by (key descending, token ascending) ----
  for (int a = tid; a < take; a += kXdThreads) {
    const uint32_t ka = sel_key[a];
    const int ta = sel_tok[a];
    int r = 0;
    for (int b = 0; b < take; ++b) {
      const uint32_t kb = sel_key[b];
      r += (kb > ka || (kb == ka && sel_tok[b] < ta)) ? 1 : 0;
    }
    const int s = kept0 + r;
    slot[ta] = s;
    tos[(int64_t)e * C + s] = ta;
    expert_id[ta] = e;
    gate[ta] = gv[ta];
  }
  if (tid == 0) kept_count[e] = kept0 + take;
}

// term != NULL (token order, whose assignment left its cross-expert step to
// this kernel): also L_aux = N sum_i f_i P_i from term[i] = f_i P_i through
// route_finalize's tree (xor tree inside each wave, then the wave sums in
// wave order).
__global__ __launch_bounds__(1024) void expand_finalize(const int32_t* __restrict__ kept_count, int N, int64_t T,
                                                        int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                                        int32_t* __restrict__ n_dropped,
                                                        const double* __restrict__ term, float* __restrict__ l_aux) {
  __shared__ int wsum[16];
  __shared__ double sl[16];
  const int n = threadIdx.x;
  if (term != nullptr) {
    double t = n < N ? term[n] : 0.0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    if ((n & 63) == 0) sl[n >> 6] = t;
    __syncthreads();
    if (n == 0) {
      double a = 0.0;
      for (int i = 0; i < 16; ++i) a += sl[i];
      l_aux[0] = (float)((double)N * a);
    }
  }
  const int kept = n < N ? kept_count[n] : 0;
  int tot_active, tot_kept;
  const int pos = block_exclusive_scan(kept > 0 ? 1 : 0, wsum, &tot_active);
  block_exclusive_scan(kept, wsum, &tot_kept);
  if (n < N && kept > 0) active[pos] = n;
  if (n == 0) {
    n_active[0] = tot_active;
    n_dropped[0] = (int32_t)(T - tot_kept);
  }
}

// ----------------------------------------------------------------------------
size_t expand_lds_bytes(int C, int gate_order) { return gate_order ? (size_t)kXdCache * 8 + (size_t)C * 8 : 0; }

hipError_t launch_expand(const int32_t* ev_cm, const float* gv_cm, int64_t T, int N, int C, int M, int gate_order,
                         int32_t* slot, int32_t* expert_id, float* gate, int32_t* tos, int32_t* kept_count,
                         int32_t* active, int32_t* n_active, int32_t* n_dropped, int32_t* list, hipStream_t st,
                         const double* term, float* l_aux) {
  for (int r = 1; r < M; ++r) {
    hipLaunchKernelGGL(expand_round, dim3((unsigned)N), dim3(kXdThreads), expand_lds_bytes(C, gate_order), st, ev_cm + r * T,
                       gv_cm + r * T, T, C, gate_order, slot, expert_id, gate, tos, kept_count, list);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(expand_finalize, dim3(1), dim3(1024), 0, st, kept_count, N, T, active, n_active, n_dropped, term,
                     l_aux);
  return hipGetLastError();
}

}  // namespace swm
