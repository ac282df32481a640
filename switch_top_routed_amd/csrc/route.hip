// Router: logits W_g.x (+b), softmax, top-1 argmax, gate value, and the
// per-expert load statistics f_i, P_i and L_aux = N * sum_i f_i P_i.
//
// Sources: "Top-1 Routing" concept page, Core mechanism (gate, softmax,
// argmax, gate value) and Load balancing (f_i, P_i, L_aux); Switch
// Transformers summary page, Eq. 4 passage (the same loss, alpha left to the
// caller) and selective-precision passage (router computed in fp32).
//
// bf16 operands meet on MFMA v_mfma_f32_16x16x32_bf16: a bf16 x bf16 product is
// exact in fp32 and accumulation is fp32, so this is the fp32 router of the
// selective-precision passage evaluated on bf16-stored inputs.
//
// Two shapes:
//  * fused (T >= 2048 tokens): one workgroup owns TM x 16 tokens and all N
//    experts; the 4 waves split the expert tiles, logits meet in LDS, then each
//    wave takes whole tokens for the softmax/argmax (wave reductions) and
//    accumulates sum_t p[t, i] and the per-expert counts in registers; the 4
//    waves' partials are summed in LDS in a fixed order and written once per
//    workgroup.
//  * split (few tokens, e.g. a 128-token decode batch): the token tiles alone
//    cannot fill 256 CUs, so the K dimension is cut into chunks, partial logits
//    go to the workspace, and a second kernel sums them in chunk order and runs
//    the same epilogue.
// A final single-workgroup kernel reduces the per-workgroup partials in a
// fixed order (fp64) into routed_count, f, P and L_aux.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

constexpr int kRouteThreads = 256;
constexpr size_t kRouteXlMax = 64 * 1024;  // token rows staged in LDS up to this many bytes per workgroup

namespace {
typedef __attribute__((address_space(3))) void lds_void_rt;
// gfx950 builtin in a plain function (a kernel template naming it directly
// loses its host launch stub): 16 bytes per lane, lane i lands at lds + 16 i
__device__ __forceinline__ void rt_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_rt*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void rt_dma16_so(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_rt*)lds, 16, voff, soff, 0, 0);
}
}  // namespace

// logits for `rows` tokens live in LDS lg[m * ldl + n] (no bias yet)
// lg must hold >= 8 * N floats; it is reused for the cross-wave partial sums.
// J = experts per lane (N <= 64 * J).
template <int J>
__device__ void route_epilogue(float* lg, int ldl, int rows, int64_t t0, int64_t T, int N,
                               const float* __restrict__ bias, int32_t* __restrict__ expert_id,
                               float* __restrict__ gate, float* __restrict__ part_p, int32_t* __restrict__ part_cnt,
                               int64_t blk, const RouteExtra& ex) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float bs[J], ps[J];
  int cn[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int n = lane + 64 * j;
    bs[j] = (bias != nullptr && n < N) ? bias[n] : 0.f;
    ps[j] = 0.f;
    cn[j] = 0;
  }
  for (int m = w; m < rows; m += 4) {
    const int64_t t = t0 + m;
    if (t >= T) break;
    float v[J];
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int n = lane + 64 * j;
      v[j] = (n < N) ? lg[m * ldl + n] + bs[j] : -INFINITY;
      if (n < N && v[j] > best) {  // ascending n: keeps the lowest index on ties
        best = v[j];
        bi = n;
      }
    }
    wave_argmax(best, bi);
    float lv[J];  // logits, kept for the further choices of top-K
#pragma unroll
    for (int j = 0; j < J; ++j) lv[j] = v[j];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int n = lane + 64 * j;
      v[j] = (n < N) ? __expf(v[j] - best) : 0.f;
      s += v[j];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;  // p at the argmax: exp(0) / s
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int n = lane + 64 * j;
      ps[j] += v[j] * inv;
      cn[j] += (n == bi) ? 1 : 0;
      if (ex.probs != nullptr && n < N) ex.probs[t * N + n] = v[j] * inv;
      if (ex.probs_t != nullptr && n < N) ex.probs_t[(int64_t)n * T + t] = v[j] * inv;
    }
    if (ex.K <= 1 || ex.expand) {
      if (lane == 0) {
        expert_id[t] = bi;
        gate[t] = inv;
        if (ex.ev_cm != nullptr) {
          ex.ev_cm[t] = bi;
          ex.gv_cm[t] = inv;
        }
      }
    }
    if (ex.K > 1) {
      // top-K: choice r is the largest logit not chosen yet (ties to the lower
      // index); its gate is p at that expert.  With ex.expand the further
      // choices are only candidates: they are neither counted nor written to
      // expert_id / gate
      // tk bit j: expert lane + 64 j is chosen already; lane r < K keeps choice r
      uint32_t tk = 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) tk |= (lane + 64 * j == bi) ? (1u << j) : 0u;
      int my_e = bi;
      float my_g = inv;
      float gsum = inv;
      for (int r = 1; r < ex.K; ++r) {
        float bv = -INFINITY;
        int bx = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int n = lane + 64 * j;
          if (n < N && !((tk >> j) & 1u) && lv[j] > bv) {
            bv = lv[j];
            bx = n;
          }
        }
        wave_argmax(bv, bx);
        // p of the chosen expert, from the lane that holds it
        float mine = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if (lane + 64 * j == bx) {
            mine = v[j] * inv;
            tk |= 1u << j;
            if (!ex.expand) cn[j] += 1;
          }
        }
        const float pr = __shfl(mine, bx & 63, 64);
        if (lane == r) {
          my_e = bx;
          my_g = pr;
        }
        gsum += pr;
      }
      if (ex.expand) {
        if (lane >= 1 && lane < ex.K) {
          ex.ev_cm[(int64_t)lane * T + t] = my_e;
          ex.gv_cm[(int64_t)lane * T + t] = my_g;
        }
      } else if (lane < ex.K) {
        const float g = ex.renorm ? my_g * (1.0f / gsum) : my_g;
        expert_id[t * ex.K + lane] = my_e;
        gate[t * ex.K + lane] = g;
        if (ex.ev_cm != nullptr) {
          ex.ev_cm[(int64_t)lane * T + t] = my_e;
          ex.gv_cm[(int64_t)lane * T + t] = g;
        }
      }
    }
  }
  __syncthreads();  // every wave is done reading the logits
  float* red_p = lg;
  int* red_c = reinterpret_cast<int*>(lg + 4 * N);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int n = lane + 64 * j;
    if (n < N) {
      red_p[w * N + n] = ps[j];
      red_c[w * N + n] = cn[j];
    }
  }
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += kRouteThreads) {
    part_p[blk * N + n] = ((red_p[n] + red_p[N + n]) + red_p[2 * N + n]) + red_p[3 * N + n];
    part_cnt[blk * N + n] = red_c[n] + red_c[N + n] + red_c[2 * N + n] + red_c[3 * N + n];
  }
}

// The plain top-1 case of the same epilogue (no probabilities out, no further
// choices) for 16, 32 or 64 tokens and N <= 128 (logits rows of ldl <= 128
// floats, ldl a multiple of 16).  The general one walks the tokens one per wave
// and step, and each token costs a whole-wave arg-max and sum (12 dependent
// lane exchanges); at 16 tokens per wave that took about 12 us of a 60 us
// route call on 16384 x 5120 tokens.  Here TPT = 256 / ROWS consecutive lanes
// share a token, so a token needs log2(TPT) exchanges and all of a wave's
// tokens run at once.  The results are bit-identical to route_epilogue's, so
// the two can serve the same layer in different calls:
//  * lane-slot l (0..63) holds experts l and l + 64, as a lane does there; the
//    lane of a token with index q takes the slots q L .. q L + L - 1 (L = 64 /
//    TPT) and the exp-sum is the same balanced tree over the slots in order
//    (slot sums, then pairs of adjacent blocks), its upper levels across the
//    TPT lanes;
//  * the block's sum of p per expert is the same ((S0 + S1) + S2) + S3 with
//    S_w summed over tokens w, w + 4, ... in order.
// The probabilities overwrite the logits for the column sums.  tok: ROWS ints
// (16-byte aligned) and red: 512 floats of LDS scratch outside the logits.
template <int ROWS>
__device__ void route_epilogue_top1(float* lg, int ldl, int* tok, float* red, int rows, int64_t t0, int N,
                                    const float* __restrict__ bias, int32_t* __restrict__ expert_id,
                                    float* __restrict__ gate, float* __restrict__ part_p,
                                    int32_t* __restrict__ part_cnt, int64_t blk, int32_t* __restrict__ ev_cm,
                                    float* __restrict__ gv_cm) {
  constexpr int TPT = kRouteThreads / ROWS;  // lanes per token
  constexpr int L = 64 / TPT;                // lane-slots per lane
  constexpr int CH = L / 4;                  // 16-byte chunks per half (experts < 64, >= 64)
  static_assert(TPT == 4 || TPT == 8 || TPT == 16, "16, 32 or 64 tokens per workgroup");
  const int m = threadIdx.x / TPT, q = threadIdx.x % TPT;
  // chunk i of a half is read at position (i + rot) % CH, which puts the lanes
  // of an LDS request on distinct 16-byte bank groups (16 lanes over 256 bytes,
  // and any 8 over 128)
  int rot = 0;
  if constexpr (TPT == 4) rot = ((m & 3) + 2 * (q >> 1)) & 3;
  if constexpr (TPT == 8) rot = ((m & 1) + (q >> 2)) & 1;
  const float* row = lg + m * ldl + q * L;
  float lo[L], hi[L];  // experts q L + i and 64 + q L + i
  int nb[2][CH];
  float best = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int cc = CH > 1 ? (i + rot) % CH : 0;
      const int n0 = hh * 64 + q * L + cc * 4;
      nb[hh][i] = n0;
      // chunks at or past N (then also past the row's ldl floats) are not read
      const f32x4 x4 = n0 < N ? *reinterpret_cast<const f32x4*>(row + hh * 64 + cc * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int n = n0 + u;
        const float val = n < N ? x4[u] + (bias != nullptr ? bias[n] : 0.f) : -INFINITY;
        if (hh == 0) lo[i * 4 + u] = val;  // register slot i: chunk cc (see the sums)
        else hi[i * 4 + u] = val;
        if (n < N && (val > best || (val == best && n < bi))) {
          best = val;
          bi = n;
        }
      }
    }
  argmax_step<kDppQuadXor1, 0xf>(best, bi);
  argmax_step<kDppQuadXor2, 0xf>(best, bi);
  if constexpr (TPT >= 8) argmax_step<kDppHalfMirror, 0xf>(best, bi);
  if constexpr (TPT == 16) argmax_step<kDppMirror, 0xf>(best, bi);
  // exp, then the slot sums in slot order (register chunk i holds slots of
  // chunk (i + rot) % CH, so slot j of this lane is chunk j / 4 - rot)
  float e[2][L];
  float sl[L];
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      e[0][i * 4 + u] = __expf(lo[i * 4 + u] - best);  // -inf (n >= N) -> 0
      e[1][i * 4 + u] = __expf(hi[i * 4 + u] - best);
    }
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int i = CH > 1 ? (j - rot + CH) % CH : 0;  // register chunk holding slot chunk j
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int r = 0; r < CH; ++r)
        if (r == i) {
          a0 = e[0][r * 4 + u];
          a1 = e[1][r * 4 + u];
        }
      sl[j * 4 + u] = a0 + a1;
    }
  }
#pragma unroll
  for (int w2 = 1; w2 < L; w2 *= 2)
#pragma unroll
    for (int i = 0; i < L; i += 2 * w2) sl[i] = sl[i] + sl[i + w2];
  float sum = sl[0];
  sum += __int_as_float(dpp_move<kDppQuadXor1>(0, __float_as_int(sum)));
  sum += __int_as_float(dpp_move<kDppQuadXor2>(0, __float_as_int(sum)));
  if constexpr (TPT >= 8) sum += __int_as_float(dpp_move<kDppHalfMirror>(0, __float_as_int(sum)));
  if constexpr (TPT == 16) sum += __int_as_float(dpp_move<kDppMirror>(0, __float_as_int(sum)));
  const float inv = 1.0f / sum;
  const bool valid = m < rows;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      f32x4 p4;
#pragma unroll
      for (int u = 0; u < 4; ++u) p4[u] = e[hh][i * 4 + u] * inv;
      if (nb[hh][i] < N) *reinterpret_cast<f32x4*>(lg + m * ldl + nb[hh][i]) = p4;
    }
  if (q == 0) {
    tok[m] = valid ? bi : -1;
    if (valid) {
      expert_id[t0 + m] = bi;
      gate[t0 + m] = inv;
      if (ev_cm != nullptr) {
        ev_cm[t0 + m] = bi;
        gv_cm[t0 + m] = inv;
      }
    }
  }
  __syncthreads();
  {
    // fixed trip counts, so that all reads of a loop are in flight together
    // (a loop bounded by rows waited for each read in turn)
    const int n = threadIdx.x & 127, h = threadIdx.x >> 7;
    float s0 = 0.f, s1 = 0.f;  // S_{2h}, S_{2h+1}
    int cn = 0;
    if (n < N) {
#pragma unroll
      for (int k = 0; k < ROWS / 4; ++k) {
        const int m0 = 4 * k + 2 * h;
        const float a = lg[m0 * ldl + n], b = lg[(m0 + 1) * ldl + n];
        if (m0 < rows) s0 += a;
        if (m0 + 1 < rows) s1 += b;
      }
      if (h == 0) {
#pragma unroll
        for (int k = 0; k < ROWS / 4; ++k) {  // token ids past rows are -1
          const u32x4 t4 = *reinterpret_cast<const u32x4*>(tok + 4 * k);
          cn += ((int)t4[0] == n ? 1 : 0) + ((int)t4[1] == n ? 1 : 0) + ((int)t4[2] == n ? 1 : 0) +
                ((int)t4[3] == n ? 1 : 0);
        }
      }
    }
    red[(2 * h) * 128 + n] = s0;
    red[(2 * h + 1) * 128 + n] = s1;
    if (h == 0 && n < N) part_cnt[blk * N + n] = cn;
  }
  __syncthreads();
  if (threadIdx.x < N) {
    const int n = threadIdx.x;
    part_p[blk * N + n] = ((red[n] + red[128 + n]) + red[256 + n]) + red[384 + n];
  }
}

// plain top-1: no per-token probabilities, further choices or candidates
__device__ __forceinline__ bool route_plain_top1(const RouteExtra& ex) {
  return ex.K <= 1 && !ex.expand && ex.probs == nullptr && ex.probs_t == nullptr;
}

// ----------------------------------------------------------------------------
// fused bf16 router.  lane l: c = l & 15 selects the A row / B column, kg = l >> 4
// selects 8 consecutive k.  A = x rows (k contiguous), B = W_g^T, whose
// fragment is 8 consecutive k of one W_g row (also contiguous).
// ----------------------------------------------------------------------------
// XL: the workgroup's token rows are copied to LDS once (direct global-to-LDS
// loads, 16-byte chunks of each row XOR-swizzled by the row's low 4 bits so
// that 16 rows read at one k fall on distinct banks) and the k-loop streams
// only W_g.  Without it every wave streams the rows too, and because loads
// retire in order each step also waits for its rows' first trip from HBM.
template <int TM, int NG, int J, bool XL>
__global__ __launch_bounds__(kRouteThreads) void route_fused_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias, int64_t T, int d,
    int N, int32_t* __restrict__ expert_id, float* __restrict__ gate, float* __restrict__ part_p,
    int32_t* __restrict__ part_cnt, RouteExtra ex) {
  extern __shared__ float smem[];
  const int NT = (N + 15) >> 4;
  const int ldl = NT * 16;
  float* lg = smem;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * TM * 16;
  const int ksteps = d >> 5;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // Operands through buffer loads: rows past T or N get a lane offset beyond the
  // descriptor's extent and read zeros, so the k-loop needs no branches and the
  // loads of RP steps stay in flight ahead of the MFMAs (a register ring).
  constexpr int RP = TM >= 4 ? 4 : 8;  // a 12-deep ring with XL measured slower (16.7 against 15.5 us)
  const int64_t rows_here = (T - t0) < TM * 16 ? (T - t0) : TM * 16;
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + t0 * d), (short)0, (int)(rows_here * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wg), (short)0, (int)((int64_t)N * d * 2), 0x00020000);
  const int kpad = (ksteps + RP - 1) / RP * RP;
  const int cpr = d >> 3;  // 16-byte chunks per row (a multiple of 16: d % 128 == 0)
  unsigned char* xt = reinterpret_cast<unsigned char*>(smem + TM * 16 * ldl);
  if (XL) {
    const int nb = TM * 16 * cpr / 64;  // 1 KB blocks of the tile
    for (int b = w; b < nb; b += 4) {
      const int q = b * 64 + lane, r = q / cpr, kc = (q - r * cpr) ^ (r & 15);
      rt_dma16(xres, xt + b * 1024, r < rows_here ? (r * d + kc * 8) * 2 : 0x7ffffff0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
    __syncthreads();
  }
  for (int ntb = w * NG; ntb < NT; ntb += 4 * NG) {
    f32x4 acc[TM][NG];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    int b_voff[NG], a_voff[TM];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int n = (ntb + g) * 16 + c;
      b_voff[g] = n < N ? (n * d + kg * 8) * 2 : 0x7ffffff0;
    }
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
      const int r = mt * 16 + c;
      a_voff[mt] = r < rows_here ? (r * d + kg * 8) * 2 : 0x7ffffff0;
    }
    u32x4 ra[RP][TM], rb[RP][NG];
    auto load = [&](int slot, int ks) {
      const int so = (ks < ksteps ? ks : ksteps - 1) * 64;  // past the end: re-read the last step
#pragma unroll
      for (int mt = 0; mt < TM; ++mt)
        if (!XL)
          ra[slot][mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, a_voff[mt], so, 0));
#pragma unroll
      for (int g = 0; g < NG; ++g)
        rb[slot][g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, b_voff[g], so, 0));
    };
#pragma unroll
    for (int s0 = 0; s0 < RP - 1; ++s0) load(s0, s0);
    for (int it = 0; it < kpad; it += RP) {
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int ks = it + u;
        load((u + RP - 1) % RP, ks + RP - 1);
        __builtin_amdgcn_sched_barrier(0);
        const bool live = ks < ksteps;
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
          u32x4 a;
          if (XL) {
            const int r = mt * 16 + c, kc = ((ks < ksteps ? ks : 0) * 4 + kg) ^ (r & 15);
            a = *reinterpret_cast<const u32x4*>(xt + (r * cpr + kc) * 16);
          } else {
            a = ra[u][mt];
          }
          a = live ? a : zero;
#pragma unroll
          for (int g = 0; g < NG; ++g) acc[mt][g] = mfma_bf16_16x16x32(a, rb[u][g], acc[mt][g]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (ntb + g < NT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lg[(mt * 16 + kg * 4 + i) * ldl + (ntb + g) * 16 + c] = acc[mt][g][i];
        }
      }
  }
  __syncthreads();
  if (N <= 128 && route_plain_top1(ex)) {  // scratch after the logits (the staged rows, if any, are dead)
    float* scr = smem + TM * 16 * ldl;
    route_epilogue_top1<TM * 16>(lg, ldl, reinterpret_cast<int*>(scr), scr + 64, (int)rows_here, t0, N, bias,
                                 expert_id, gate, part_p, part_cnt, blockIdx.x, ex.ev_cm, ex.gv_cm);
  } else {
    route_epilogue<J>(lg, ldl, TM * 16, t0, T, N, bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex);
  }
}

// ----------------------------------------------------------------------------
// K-sliced bf16 router for many tokens with long rows (the 16384 x 5120 layer):
// the 4 waves of a workgroup split K into quarters, and each wave covers every
// expert tile (N <= 128) of the workgroup's 16 TM tokens.  The fused kernel
// above splits the expert tiles instead, so all 4 waves stream the same token
// rows and a CU keeps only (RP - 1) steps x 16 TM x 64 bytes of distinct x in
// flight; here each wave streams its own quarter of the rows, 4x the distinct
// bytes in flight per CU for the same ring depth, which is what an HBM-bound
// read of 16 TM rows x d needs.  One workgroup per CU (the 128 accumulator
// registers plus a 4-step ring take more than half the register file).  The
// quarters' partial logits meet in LDS and are summed in wave order, then the
// shared epilogue runs.
// ----------------------------------------------------------------------------
template <int TM, int J>
__global__ __launch_bounds__(kRouteThreads, 1) void route_kslice_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias, int64_t T, int d,
    int N, int32_t* __restrict__ expert_id, float* __restrict__ gate, float* __restrict__ part_p,
    int32_t* __restrict__ part_cnt, RouteExtra ex) {
  constexpr int NT = 8;  // expert tiles: N <= 128
  constexpr int ldl = NT * 16;
  constexpr int RP = 4;  // register ring depth (RP - 1 steps of loads ahead)
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * TM * 16;
  const int ksteps = d >> 5;
  const int ks0 = ksteps * w / 4, nks = ksteps * (w + 1) / 4 - ks0;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int64_t rows_here = (T - t0) < TM * 16 ? (T - t0) : TM * 16;
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + t0 * d), (short)0, (int)(rows_here * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wg), (short)0, (int)((int64_t)N * d * 2), 0x00020000);
  int a_voff[TM], b_voff[NT];
#pragma unroll
  for (int mt = 0; mt < TM; ++mt) {
    const int r = mt * 16 + c;
    a_voff[mt] = r < rows_here ? (r * d + kg * 8) * 2 : 0x7ffffff0;
  }
#pragma unroll
  for (int g = 0; g < NT; ++g) {
    const int n = g * 16 + c;
    b_voff[g] = n < N ? (n * d + kg * 8) * 2 : 0x7ffffff0;
  }
  f32x4 acc[TM][NT];
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[RP][TM], rb[RP][NT];
  auto load = [&](int slot, int s) {
    const int so = (ks0 + (s < nks ? s : nks - 1)) * 64;  // past the end: re-read the last step
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
      ra[slot][mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, a_voff[mt], so, 0));
#pragma unroll
    for (int g = 0; g < NT; ++g)
      rb[slot][g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, b_voff[g], so, 0));
  };
#pragma unroll
  for (int s0 = 0; s0 < RP - 1; ++s0) load(s0, s0);
  const int kpad = (nks + RP - 1) / RP * RP;
  for (int it = 0; it < kpad; it += RP) {
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      const int ks = it + u;
      load((u + RP - 1) % RP, ks + RP - 1);
      __builtin_amdgcn_sched_barrier(0);
      const bool live = ks < nks;
#pragma unroll
      for (int mt = 0; mt < TM; ++mt) {
        const u32x4 a = live ? ra[u][mt] : zero;
#pragma unroll
        for (int g = 0; g < NT; ++g) acc[mt][g] = mfma_bf16_16x16x32(a, rb[u][g], acc[mt][g]);
      }
    }
  }
  // the quarters' partial logits, each in its own LDS region, summed in wave order
  constexpr int REG = TM * 16 * ldl;
  float* mine = smem + w * REG;
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int g = 0; g < NT; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[(mt * 16 + kg * 4 + i) * ldl + g * 16 + c] = acc[mt][g][i];
  __syncthreads();
  for (int q = threadIdx.x; q < REG; q += kRouteThreads)
    smem[q] = ((smem[q] + smem[REG + q]) + smem[2 * REG + q]) + smem[3 * REG + q];
  __syncthreads();
  if (route_plain_top1(ex)) {  // the other quarters' regions are free for its scratch
    const int64_t rows_here = (T - t0) < TM * 16 ? (T - t0) : TM * 16;
    route_epilogue_top1<TM * 16>(smem, ldl, reinterpret_cast<int*>(smem + REG), smem + 2 * REG, (int)rows_here, t0, N,
                                 bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex.ev_cm, ex.gv_cm);
  } else {
    route_epilogue<J>(smem, ldl, TM * 16, t0, T, N, bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex);
  }
}

// ----------------------------------------------------------------------------
// Streaming bf16 router for many tokens with long rows (the 16384 x 5120
// layer; d % 1024 == 0), where reading x from HBM is the whole cost: the
// workgroup's 16 TM token rows are staged in LDS chunk by chunk (KC = 256 k
// per row) by direct global-to-LDS loads, whole 512-byte row segments per
// chunk, with three chunks in flight while a fourth is multiplied, so a CU
// keeps 3 x 16 TM x 512 bytes of distinct x in flight.  The 4 waves split the
// expert tiles (N <= 128: two 16-expert tiles each); each wave holds its W_g
// fragments for a whole chunk in registers (from L2), loaded one chunk ahead
// into a second register set.  Loads retire in order, so one wait per chunk
// covers the chunk's W_g and x.  The four chunk buffers are separate LDS
// arrays named by compile-time indices, so the compiler's wait counts see
// that a fragment read does not alias the loads in flight to the other
// buffers.  16-byte pieces of a staged row are XOR-swizzled by the row's low
// 4 bits, so the 16 rows an A-fragment read touches fall on distinct banks.
// ----------------------------------------------------------------------------
#define SWM_RT_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

// W_g in MFMA-fragment order for the streaming kernel: fragment (k-step ks,
// expert tile g) is 64 lanes x 16 bytes, lane (c, kg) holding W_g[16 g + c,
// 32 ks + 8 kg .. + 7] (zero past N), so that a wave reads each fragment as
// one contiguous 1 KB (whole cache lines) instead of 16 half-lines.
__global__ __launch_bounds__(256) void route_wg_frag(const uint16_t* __restrict__ wg, int d, int N,
                                                     u32x4* __restrict__ wgf) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // fragment element
  const int64_t total = (int64_t)8 * (d / 32) * 64;
  if (i >= total) return;
  const int lane = (int)(i & 63), g = (int)((i >> 6) & 7), ks = (int)(i >> 9);
  const int n = g * 16 + (lane & 15), k = ks * 32 + (lane >> 4) * 8;
  wgf[i] = n < N ? *reinterpret_cast<const u32x4*>(wg + (int64_t)n * d + k) : u32x4{0u, 0u, 0u, 0u};
}

template <int TM, int J>
__global__ __launch_bounds__(kRouteThreads, 1) void route_stream_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias, int64_t T, int d,
    int N, int32_t* __restrict__ expert_id, float* __restrict__ gate, float* __restrict__ part_p,
    int32_t* __restrict__ part_cnt, RouteExtra ex, const u32x4* __restrict__ wgf) {
  constexpr int NG = 2;                 // expert tiles per wave: 4 waves x 2 x 16 = 128 experts
  constexpr int KC = 256;               // k per chunk
  constexpr int KS = KC / 32;           // 32-deep MFMA steps per chunk
  constexpr int ROWS = TM * 16;         // tokens per workgroup
  constexpr int CB = ROWS * KC * 2;     // bytes of one staged chunk
  constexpr int DW = CB / 1024 / 4;     // 1 KB global-to-LDS loads per wave per chunk
  constexpr int CPR = KC / 8;           // 16-byte pieces per staged row
  constexpr int RB = KC * 2;            // bytes per staged row
  constexpr int WAIT = 2 * DW + KS * NG;  // loads issued after a chunk's W_g (see the loop)
  static_assert(WAIT <= 63, "vmcnt range");
  constexpr int ldl = 128;              // logits row stride (N <= 128)
  static_assert(ROWS * ldl * 4 <= CB, "the logits fit the first chunk buffer");
  __shared__ __attribute__((aligned(1024))) unsigned char xb0[CB];
  __shared__ __attribute__((aligned(1024))) unsigned char xb1[CB];
  __shared__ __attribute__((aligned(1024))) unsigned char xb2[CB];
  __shared__ __attribute__((aligned(1024))) unsigned char xb3[CB];
  auto xbuf = [&](int i) -> unsigned char* { return i == 0 ? xb0 : i == 1 ? xb1 : i == 2 ? xb2 : xb3; };
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * ROWS;
  const int64_t rows_here = (T - t0) < ROWS ? (T - t0) : ROWS;
  const int nch = d / KC;
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + t0 * d), (short)0, (int)(rows_here * d * 2), 0x00020000);
  // W_g in fragment order (route_wg_frag): 8 tiles x d / 32 k-steps x 1 KB
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(wgf), (short)0,
                                                                        (int)((int64_t)8 * (d / 32) * 1024), 0x00020000);
  // x: load i of this wave fills staged piece p = (w DW + i) 64 + lane, i.e.
  // row p / CPR, stored piece p % CPR, which holds global piece (p % CPR) ^ (row & 15)
  int x_voff[DW];
#pragma unroll
  for (int i = 0; i < DW; ++i) {
    const int p = (w * DW + i) * 64 + lane, r = p / CPR, q = (p % CPR) ^ (r & 15);
    x_voff[i] = r < rows_here ? (r * d + q * 8) * 2 : 0x7ffffff0;
  }
  int b_voff[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) b_voff[g] = ((w * NG + g) * 64 + lane) * 16;
  auto issue_x = [&](int buf, int ch) {  // past the last chunk: re-read it (cache hits)
    const int so = (ch < nch ? ch : nch - 1) * RB;
    unsigned char* xb = xbuf(buf);
#pragma unroll
    for (int i = 0; i < DW; ++i) rt_dma16_so(xres, xb + (w * DW + i) * 1024, x_voff[i], so);
  };
  u32x4 wr0[KS][NG], wr1[KS][NG];
  auto issue_w = [&](u32x4 (&wr)[KS][NG], int ch) {
    const int so = (ch < nch ? ch : nch - 1) * KS * 8 * 1024;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        wr[ks][g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, b_voff[g], so + ks * 8 * 1024, 0));
  };
  f32x4 acc[TM][NG];
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[mt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&wr)[KS][NG], int buf) {
    const unsigned char* xb = xbuf(buf);
    u32x4 a[2][TM];
    auto read_a = [&](u32x4 (&dst)[TM], int ks) {  // row mt 16 + c: its swizzle key (row & 15) is c
#pragma unroll
      for (int mt = 0; mt < TM; ++mt)
        dst[mt] = *reinterpret_cast<const u32x4*>(xb + (mt * 16 + c) * RB + (((ks * 4 + kg) ^ c) << 4));
    };
    read_a(a[0], 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) read_a(a[(ks + 1) & 1], ks + 1);
#pragma unroll
      for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[mt][g] = mfma_bf16_16x16x32(a[ks & 1][mt], wr[ks][g], acc[mt][g]);
    }
    // instruction order (0x100: LDS reads, 0x008: MFMAs): the first step's
    // reads, then per step the next step's reads ahead of this step's MFMAs.
    // Left to itself the scheduler put each read right before its MFMAs and
    // waited for it there, one LDS round trip per two MFMAs (67 -> 60 us per
    // route call on 16384 x 5120 tokens)
    __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, TM * NG, 0);
    }
  };
  // chunk ch = ch0 + u (buffer u): every wave is done with chunk ch - 1, whose
  // buffer takes chunk ch + 3; issue W_g of ch + 1 and x of ch + 3, wait for
  // W_g and x of ch (WAIT loads were issued after W_g of ch), publish x of ch,
  // multiply.  The W_g loads go out before the x loads: loads retire in order,
  // so an x load the compiler placed among them would be waited for one chunk
  // later with the W_g (54.5 -> 53.4 us per route call on 16384 x 5120 tokens)
  auto body = [&](u32x4 (&cur)[KS][NG], u32x4 (&nxt)[KS][NG], int u, int ch) {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_w(nxt, ch + 1);
    asm volatile("" ::: "memory");
    issue_x((u + 3) & 3, ch + 3);
    SWM_RT_WAIT_VMCNT_LGKM0(WAIT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    compute(cur, u);
  };
  issue_w(wr0, 0);
  issue_x(0, 0);
  issue_x(1, 1);
  issue_x(2, 2);
  // nch is a multiple of 4 (d % 1024 == 0): buffer and register-set indices
  // stay compile-time constants and the loop has no inner branch (a branch
  // would let the compiler sink the next chunk's W_g loads down to their use)
  for (int ch = 0; ch < nch; ch += 4) {
    body(wr0, wr1, 0, ch);
    body(wr1, wr0, 1, ch + 1);
    body(wr0, wr1, 2, ch + 2);
    body(wr1, wr0, 3, ch + 3);
  }
  SWM_RT_WAIT_VMCNT_LGKM0(0);  // no load may still be writing LDS
  __syncthreads();
  float* lg = reinterpret_cast<float*>(xb0);  // the staged chunks are dead now
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[(mt * 16 + kg * 4 + i) * ldl + (w * NG + g) * 16 + c] = acc[mt][g][i];
  __syncthreads();
  if (route_plain_top1(ex))  // the other chunk buffers are free for its scratch
    route_epilogue_top1<ROWS>(lg, ldl, reinterpret_cast<int*>(xb1), reinterpret_cast<float*>(xb2), (int)rows_here, t0, N,
                              bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex.ev_cm, ex.gv_cm);
  else
    route_epilogue<J>(lg, ldl, ROWS, t0, T, N, bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex);
}

// ----------------------------------------------------------------------------
// split path: partial logits plog[s][t][n] over k-chunk s
// ----------------------------------------------------------------------------
template <int NG>
__global__ __launch_bounds__(kRouteThreads) void route_logits_split_bf16(const uint16_t* __restrict__ x,
                                                                         const uint16_t* __restrict__ wg, int64_t T,
                                                                         int d, int N, int S,
                                                                         float* __restrict__ plog) {
  const int NT = (N + 15) >> 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int s = blockIdx.y;
  const int ksteps = d >> 5;
  const int ks0 = (int)((int64_t)ksteps * s / S), ks1 = (int)((int64_t)ksteps * (s + 1) / S);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int64_t row = t0 + c;
  const bool avalid = row < T;
  const uint16_t* ap = x + (avalid ? row : 0) * (int64_t)d + kg * 8;
  for (int ntb = w * NG; ntb < NT; ntb += 4 * NG) {
    f32x4 acc[NG];
    const uint16_t* bp[NG];
    bool bvalid[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int n = (ntb + g) * 16 + c;
      bvalid[g] = (ntb + g) < NT && n < N;
      bp[g] = wg + (int64_t)(bvalid[g] ? n : 0) * d + kg * 8;
    }
    for (int ks = ks0; ks < ks1; ++ks) {
      const u32x4 a = avalid ? *reinterpret_cast<const u32x4*>(ap + ks * 32) : zero;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const u32x4 b = bvalid[g] ? *reinterpret_cast<const u32x4*>(bp[g] + ks * 32) : zero;
        acc[g] = mfma_bf16_16x16x32(a, b, acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int n = (ntb + g) * 16 + c;
      if ((ntb + g) < NT && n < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = t0 + kg * 4 + i;
          if (t < T) plog[((int64_t)s * T + t) * N + n] = acc[g][i];
        }
      }
    }
  }
}

template <int J>
__global__ __launch_bounds__(kRouteThreads) void route_softmax_split(const float* __restrict__ plog, int S, int64_t T,
                                                                     int N, const float* __restrict__ bias,
                                                                     int32_t* __restrict__ expert_id,
                                                                     float* __restrict__ gate,
                                                                     float* __restrict__ part_p,
                                                                     int32_t* __restrict__ part_cnt, RouteExtra ex) {
  // one token per workgroup: its N logits are sums over the S k-chunks, in
  // chunk order, with 8 independent loads in flight per expert
  extern __shared__ float smem[];
  float* lg = smem;
  const int64_t t = blockIdx.x;
  for (int n = threadIdx.x; n < N; n += kRouteThreads) {
    const float* p = plog + t * N + n;
    const int64_t stride = T * N;
    float v = 0.f;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = p[(s + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) v += q[u];
    }
    for (; s < S; ++s) v += p[s * stride];
    lg[n] = v;
  }
  __syncthreads();
  route_epilogue<J>(lg, N, 1, t, T, N, bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex);
}

// ----------------------------------------------------------------------------
// fp32 router: plain fp32 FMA dot products (sequential in k), same epilogue
// ----------------------------------------------------------------------------
template <int J>
__global__ __launch_bounds__(kRouteThreads) void route_f32(const float* __restrict__ x, const float* __restrict__ wg,
                                                           const float* __restrict__ bias, int64_t T, int d, int N,
                                                           int32_t* __restrict__ expert_id, float* __restrict__ gate,
                                                           float* __restrict__ part_p,
                                                           int32_t* __restrict__ part_cnt, RouteExtra ex) {
  extern __shared__ float smem[];
  const int ldl = N;
  float* lg = smem;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  for (int idx = threadIdx.x; idx < 16 * N; idx += kRouteThreads) {
    const int m = idx / N, n = idx - m * N;
    const int64_t t = t0 + m;
    float acc = 0.f;
    if (t < T) {
      const float* xr = x + t * d;
      const float* wr = wg + (int64_t)n * d;
      for (int k = 0; k < d; ++k) acc = fmaf(xr[k], wr[k], acc);
    }
    lg[m * ldl + n] = acc;
  }
  __syncthreads();
  route_epilogue<J>(lg, ldl, 16, t0, T, N, bias, expert_id, gate, part_p, part_cnt, blockIdx.x, ex);
}

// ----------------------------------------------------------------------------
// fixed-order reduction of the per-workgroup partials
// ----------------------------------------------------------------------------
// thread tid: expert n = tid % NP (consecutive lanes read consecutive experts, so
// every load is coalesced), block group g = tid / NP takes blocks g, g + G, ...
// (NP = N rounded up to 64, G = 1024 / NP); the G partial sums are combined in g
// order, the N products in a fixed tree order.
// Fixed-order reduction of the per-workgroup partials (blockDim = 1024), shared
// by route_finalize and route_assign_token.  Thread tid: expert n = tid % NP
// (consecutive lanes read consecutive experts: coalesced), group g = tid / NP
// (NP = N rounded up to 64, G = 1024 / NP groups) owns the contiguous tile range
// [b0, b1), read 16 tiles at a time.  Group sums meet in LDS in group order; the N products go through
// a fixed tree.  P_i: fp64 sums in tile order.  cnt_out (LDS, >= 1024 ints)
// receives each thread's count over its range.
__device__ __forceinline__ void finalize_partials(const float* __restrict__ part_p,
                                                  const int32_t* __restrict__ part_cnt, int64_t nblk, int64_t T,
                                                  int N, int NP, int32_t* __restrict__ routed_count,
                                                  float* __restrict__ f, float* __restrict__ P,
                                                  float* __restrict__ l_aux, int* cnt_out, int K = 1) {
  __shared__ double sp[1024];
  __shared__ double sl[16];
  const int tid = threadIdx.x;
  const int G = 1024 / NP;
  const int n = tid % NP, g = tid / NP;
  const int64_t per = (nblk + G - 1) / G;
  const int64_t b0 = (int64_t)g * per, b1 = (b0 + per < nblk) ? b0 + per : nblk;
  double accp = 0.0;
  int accc = 0;
  if (n < N && g < G) {
    for (int64_t b = b0; b < b1; b += 16) {  // 16 coalesced loads of each array in flight
      float pv[16];
      int cv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bool in = b + u < b1;
        pv[u] = in ? part_p[(b + u) * N + n] : 0.f;
        cv[u] = in ? part_cnt[(b + u) * N + n] : 0;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        accp += (double)pv[u];
        accc += cv[u];
      }
    }
  }
  sp[tid] = accp;
  cnt_out[tid] = accc;
  __syncthreads();
  double term = 0.0;
  if (tid < N) {
    double s = 0.0;
    long long cnum = 0;
    for (int i = 0; i < G; ++i) {
      s += sp[i * NP + tid];
      cnum += cnt_out[i * NP + tid];
    }
    const double fn = (double)cnum / ((double)K * (double)T);  // K assignments per token
    const double pn = s / (double)T;
    routed_count[tid] = (int32_t)cnum;
    f[tid] = (float)fn;
    P[tid] = (float)pn;
    term = fn * pn;
  }
  // L_aux: a fixed xor tree inside each wave, then the 16 wave sums in wave order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) term += __shfl_xor(term, o, 64);
  if ((tid & 63) == 0) sl[tid >> 6] = term;
  __syncthreads();
  if (tid == 0) {
    double a = 0.0;
    for (int i = 0; i < 16; ++i) a += sl[i];
    l_aux[0] = (float)((double)N * a);
  }
}

__global__ __launch_bounds__(1024) void route_finalize(const float* __restrict__ part_p,
                                                       const int32_t* __restrict__ part_cnt, int64_t nblk, int64_t T,
                                                       int N, int NP, int32_t* __restrict__ routed_count,
                                                       float* __restrict__ f, float* __restrict__ P,
                                                       float* __restrict__ l_aux, int K) {
  __shared__ int cnt[1024];
  finalize_partials(part_p, part_cnt, nblk, T, N, NP, routed_count, f, P, l_aux, cnt, K);
}

// Token-order capacity and slots, one workgroup per expert ("Top-1 Routing"
// page, Token Dropping: an expert keeps its first C tokens in token order).
// Workgroup e (NT threads) finds the tokens routed to e in ascending token
// order (ballots per wave, one LDS scan per 16 NT tokens); the r-th of them takes slot r if
// r < C and is dropped otherwise.  Top-K (K > 1): the list is the K T choices
// in choice-major order v = j T + t (every first choice before every second
// one), expert_id is that [K, T] list, and choice v's slot goes to
// slot[t K + j] and its token_of_slot entry is t.  It also reduces expert e's router partials
// into routed_count, f and P, in the same order as route_finalize (group g of
// G = 1024 / NP owns a contiguous tile range summed in tile order, then the
// groups in group order), so both give the same bits, and leaves f_e * P_e in
// term[e] for assign_token_finalize.  Every token is routed to exactly one
// expert, so each slot[t] and token_of_slot row has exactly one writer.
namespace {
constexpr int kAtSub = 16;  // NT-token chunks per LDS scan
}  // namespace

template <int NT, bool MULTI>
__global__ __launch_bounds__(NT) void assign_token_expert(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_cnt, int64_t nblk, int64_t T, int K_, int N,
    int NP, int C, const int32_t* __restrict__ expert_id, int32_t* __restrict__ routed_count, float* __restrict__ f,
    float* __restrict__ P, double* __restrict__ term, int32_t* __restrict__ slot, int32_t* __restrict__ token_of_slot,
    int32_t* __restrict__ kept_count) {
  __shared__ int woff[kAtSub * (NT / 64)];
  __shared__ float cp[NT];
  __shared__ int cc[NT];
  __shared__ double sp[16];
  __shared__ int sc[16];
  __shared__ int s_total;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int K = MULTI ? K_ : 1;  // choices per token (top-K); 1 compiles the top-1 path
  const int64_t TV = T * K;  // choices in the list
  // the first chunk's expert ids are loaded together with the first tiles
  int ev0[kAtSub];
#pragma unroll
  for (int j = 0; j < kAtSub; ++j) {
    const int64_t v = (int64_t)j * NT + tid;
    ev0[j] = v < TV ? expert_id[v] : -1;
  }

  // statistics of expert e: the tiles' partials pass through LDS NT at a
  // time; group g = tid < G adds the part of its tile range in each chunk
  const int G = 1024 / NP;
  const int64_t per = (nblk + G - 1) / G;
  const int64_t b0 = (int64_t)tid * per, b1 = (b0 + per < nblk) ? b0 + per : nblk;
  double accp = 0.0;
  int accc = 0;
  for (int64_t c0 = 0; c0 < nblk; c0 += NT) {
    const int64_t b = c0 + tid;
    cp[tid] = b < nblk ? part_p[b * N + e] : 0.f;
    cc[tid] = b < nblk ? part_cnt[b * N + e] : 0;
    __syncthreads();
    if (tid < G) {
      const int64_t lo = b0 > c0 ? b0 : c0, hi = b1 < c0 + NT ? b1 : c0 + NT;
      for (int64_t q = lo; q < hi; ++q) {
        accp += (double)cp[q - c0];
        accc += cc[q - c0];
      }
    }
    __syncthreads();
  }
  if (tid < G) {
    sp[tid] = accp;
    sc[tid] = accc;
  }

  // slots: the tokens of expert e in ascending token order
  int n_seen = 0;
  for (int64_t c0 = 0; c0 < TV; c0 += (int64_t)kAtSub * NT) {
    bool fl[kAtSub];
    uint64_t m[kAtSub];
#pragma unroll
    for (int j = 0; j < kAtSub; ++j) {
      const int64_t v = c0 + (int64_t)j * NT + tid;
      fl[j] = c0 == 0 ? ev0[j] == e : (v < TV && expert_id[v] == e);
    }
#pragma unroll
    for (int j = 0; j < kAtSub; ++j) {
      m[j] = __ballot(fl[j]);
      if (lane == 0) woff[j * (NT / 64) + w] = __popcll(m[j]);
    }
    __syncthreads();
    if (w == 0) {  // exclusive scan of the kAtSub x NT / 64 counts, chunk-major then wave
      constexpr int Q = kAtSub * (NT / 64) / 64;  // counts per lane
      int v[Q], sum = 0;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        v[q] = woff[lane * Q + q];
        sum += v[q];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      int run = incl - sum;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        woff[lane * Q + q] = run;
        run += v[q];
      }
      if (lane == 63) s_total = incl;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kAtSub; ++j) {
      if (fl[j]) {
        const int64_t v = c0 + (int64_t)j * NT + tid;
        // choice-major position -> (token, choice); K T < 2^31 on this path (x
        // itself is under 2^31 bytes), so 32-bit division suffices
        int64_t t = v;
        int ch = 0;
        if (MULTI) {
          ch = (int)((uint32_t)v / (uint32_t)T);
          t = v - (int64_t)ch * T;
        }
        const int r = n_seen + woff[j * (NT / 64) + w] + __popcll(m[j] & below);
        if (r < C) {
          slot[t * K + ch] = r;
          token_of_slot[(int64_t)e * C + r] = (int32_t)t;
        } else {
          slot[t * K + ch] = -1;
        }
      }
    }
    n_seen += s_total;
    __syncthreads();  // woff and s_total are rewritten by the next chunk
  }
  const int kept = n_seen < C ? n_seen : C;
  for (int r = kept + tid; r < C; r += NT) token_of_slot[(int64_t)e * C + r] = -1;
  if (tid == 0) {
    double sum = 0.0;
    long long cnum = 0;
    for (int g = 0; g < G; ++g) {
      sum += sp[g];
      cnum += sc[g];
    }
    const double fn = (double)cnum / ((double)K * (double)T);  // K choices per token
    const double pn = sum / (double)T;
    routed_count[e] = (int32_t)cnum;
    f[e] = (float)fn;
    P[e] = (float)pn;
    term[e] = fn * pn;
    kept_count[e] = kept;
  }
}

// The cross-expert results of the token-order assignment (one workgroup of
// 1024 threads, N <= 1024): the active list in expert order, n_active,
// n_dropped = T - sum of kept counts, and L_aux = N * sum_i f_i P_i through the
// same fixed tree as route_finalize (xor tree inside each wave, then the 16
// wave sums in wave order).
__global__ __launch_bounds__(1024) void assign_token_finalize(const int32_t* __restrict__ kept_count,
                                                              const double* __restrict__ term, int N, int64_t T,
                                                              float* __restrict__ l_aux, int32_t* __restrict__ active,
                                                              int32_t* __restrict__ n_active,
                                                              int32_t* __restrict__ n_dropped) {
  __shared__ int wsum[16];
  __shared__ double sl[16];
  const int n = threadIdx.x;
  const int kept = n < N ? kept_count[n] : 0;
  double tm = n < N ? term[n] : 0.0;
  int tot_active, tot_kept;
  const int pos = block_exclusive_scan(kept > 0 ? 1 : 0, wsum, &tot_active);
  block_exclusive_scan(kept, wsum, &tot_kept);
  if (n < N && kept > 0) active[pos] = n;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tm += __shfl_xor(tm, o, 64);
  if ((n & 63) == 0) sl[n >> 6] = tm;
  __syncthreads();
  if (n == 0) {
    double a = 0.0;
    for (int i = 0; i < 16; ++i) a += sl[i];
    l_aux[0] = (float)((double)N * a);
    n_active[0] = tot_active;
    n_dropped[0] = (int32_t)(T - tot_kept);
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
// the streaming kernel (rows staged in LDS chunks) takes the K-sliced plans with d % 1024 == 0
static bool route_streams(const RoutePlan& pl, int d) { return pl.split == 0 && pl.kslice && d % 1024 == 0; }

RoutePlan route_plan(int64_t T, int d, int N, int dtype) {
  RoutePlan pl{};
  const int64_t tiles16 = (T + 15) / 16;
  if (dtype == 1 && tiles16 >= 128) {
    const int NT = (N + 15) / 16;
    int tm = 1;
    for (int c : {2, 4})
      if ((T + c * 16 - 1) / (c * 16) >= 256 && (size_t)c * 16 * NT * 16 * 4 <= 64 * 1024) tm = c;
    pl.split = 0;
    pl.tm = tm;
    pl.nblk = (T + tm * 16 - 1) / (tm * 16);
    // K-sliced kernel: long rows (>= 64 k-steps, 16 per wave) and N <= 128
    pl.kslice = tm >= 2 && N <= 128 && d >= 2048;
  } else if (dtype == 1) {
    // split path: 16-token tiles x S k-chunks for the logits, then one
    // workgroup per token for the chunk sums and the softmax
    const int ksteps = d / 32;
    int64_t s = (256 + tiles16 - 1) / tiles16;
    if (s > ksteps) s = ksteps;
    if (s > 32) s = 32;
    if (s < 1) s = 1;
    pl.split = (int)s;
    pl.tm = 1;
    pl.nblk = T;
  } else {
    pl.split = 0;
    pl.tm = 1;
    pl.nblk = tiles16;
  }
  size_t off = 0;
  pl.off_part_p = off;
  off = align_up(off + (size_t)pl.nblk * N * 4);
  pl.off_part_cnt = off;
  off = align_up(off + (size_t)pl.nblk * N * 4);
  pl.off_logits = off;
  if (pl.split > 0) off = align_up(off + (size_t)pl.split * T * N * 4);
  pl.off_wgf = off;
  if (route_streams(pl, d)) off = align_up(off + (size_t)8 * (d / 32) * 1024);  // 8 expert tiles x k-steps x 1 KB
  pl.tile_rows = pl.split == 0 ? pl.tm * 16 : (dtype == 1 ? 1 : 16);
  pl.bytes = off;
  return pl;
}

template <int J>
static hipError_t launch_route_j(const RoutePlan& pl, const void* x, const void* wg, const float* bias, int64_t T,
                                 int d, int N, int dtype, int32_t* expert_id, float* gate, float* part_p,
                                 int32_t* part_cnt, char* ws, hipStream_t st,
                                 const RouteExtra& ex) {
  if (dtype == 1 && pl.split == 0) {
    const int NT = (N + 15) / 16;
    // the logits, then the top-1 epilogue's scratch (64 token ids, 512 sums)
    const size_t lds = (size_t)pl.tm * 16 * NT * 16 * 4 + 4096;
    const size_t xl_bytes = (size_t)pl.tm * 16 * d * 2;  // the token rows of a workgroup
    // the XOR swizzle of the staged rows (row & 15 over 16-byte chunks) is a
    // bijection only when a row holds a multiple of 16 chunks: d % 128 == 0
    const bool xl = xl_bytes <= kRouteXlMax && d % 128 == 0;
    dim3 grid((unsigned)pl.nblk);
    auto* xb = static_cast<const uint16_t*>(x);
    auto* wb = static_cast<const uint16_t*>(wg);
    if (J != 2 && pl.kslice) return hipErrorInvalidValue;  // the plan takes these kernels for N <= 128 only
    if constexpr (J == 2) {
    if (route_streams(pl, d)) {  // static LDS: four staged chunks
      u32x4* wgf = reinterpret_cast<u32x4*>(ws + pl.off_wgf);
      const int64_t frag = (int64_t)8 * (d / 32) * 64;
      hipLaunchKernelGGL(route_wg_frag, dim3((unsigned)((frag + 255) / 256)), dim3(256), 0, st, wb, d, N, wgf);
      if (pl.tm == 4)
        hipLaunchKernelGGL((route_stream_bf16<4, J>), grid, dim3(kRouteThreads), 0, st, xb, wb, bias, T, d, N,
                           expert_id, gate, part_p, part_cnt, ex, wgf);
      else
        hipLaunchKernelGGL((route_stream_bf16<2, J>), grid, dim3(kRouteThreads), 0, st, xb, wb, bias, T, d, N,
                           expert_id, gate, part_p, part_cnt, ex, wgf);
      return hipGetLastError();
    }
    if (pl.kslice) {
      const size_t klds = (size_t)4 * pl.tm * 16 * 128 * 4;  // four quarters' partial logits
      if (pl.tm == 4)
        hipLaunchKernelGGL((route_kslice_bf16<4, J>), grid, dim3(kRouteThreads), klds, st, xb, wb, bias, T, d, N,
                           expert_id, gate, part_p, part_cnt, ex);
      else
        hipLaunchKernelGGL((route_kslice_bf16<2, J>), grid, dim3(kRouteThreads), klds, st, xb, wb, bias, T, d, N,
                           expert_id, gate, part_p, part_cnt, ex);
      return hipGetLastError();
    }
    }
    if (pl.tm == 4)
      hipLaunchKernelGGL((route_fused_bf16<4, 2, J, false>), grid, dim3(kRouteThreads), lds, st, xb, wb, bias, T, d, N,
                         expert_id, gate, part_p, part_cnt, ex);
    else if (pl.tm == 2)
      hipLaunchKernelGGL((route_fused_bf16<2, 2, J, false>), grid, dim3(kRouteThreads), lds, st, xb, wb, bias, T, d, N,
                         expert_id, gate, part_p, part_cnt, ex);
    else if (xl)
      hipLaunchKernelGGL((route_fused_bf16<1, 2, J, true>), grid, dim3(kRouteThreads), lds + xl_bytes, st, xb, wb, bias,
                         T, d, N, expert_id, gate, part_p, part_cnt, ex);
    else
      hipLaunchKernelGGL((route_fused_bf16<1, 2, J, false>), grid, dim3(kRouteThreads), lds, st, xb, wb, bias, T, d, N,
                         expert_id, gate, part_p, part_cnt, ex);
  } else if (dtype == 1) {
    float* plog = reinterpret_cast<float*>(ws + pl.off_logits);
    hipLaunchKernelGGL((route_logits_split_bf16<2>), dim3((unsigned)((T + 15) / 16), (unsigned)pl.split), dim3(kRouteThreads),
                       0, st, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), T, d, N, pl.split,
                       plog);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)8 * N * 4;  // the epilogue reuses it for the cross-wave partials
    hipLaunchKernelGGL(route_softmax_split<J>, dim3((unsigned)pl.nblk), dim3(kRouteThreads), lds, st, plog, pl.split,
                       T, N, bias, expert_id, gate, part_p, part_cnt, ex);
  } else {
    const size_t lds = (size_t)16 * N * 4;
    hipLaunchKernelGGL(route_f32<J>, dim3((unsigned)pl.nblk), dim3(kRouteThreads), lds, st,
                       static_cast<const float*>(x), static_cast<const float*>(wg), bias, T, d, N, expert_id, gate,
                       part_p, part_cnt, ex);
  }
  return hipGetLastError();
}

hipError_t launch_route(const RoutePlan& pl, const void* x, const void* wg, const float* bias, int64_t T, int d, int N,
                        int dtype, int32_t* expert_id, float* gate, int32_t* routed_count, float* f, float* P,
                        float* l_aux, char* ws, hipStream_t st, bool stats_later, const RouteExtra& ex) {
  float* part_p = reinterpret_cast<float*>(ws + pl.off_part_p);
  int32_t* part_cnt = reinterpret_cast<int32_t*>(ws + pl.off_part_cnt);
  hipError_t e;
  if (N <= 128)
    e = launch_route_j<2>(pl, x, wg, bias, T, d, N, dtype, expert_id, gate, part_p, part_cnt, ws, st, ex);
  else if (N <= 512)
    e = launch_route_j<8>(pl, x, wg, bias, T, d, N, dtype, expert_id, gate, part_p, part_cnt, ws, st, ex);
  else
    e = launch_route_j<16>(pl, x, wg, bias, T, d, N, dtype, expert_id, gate, part_p, part_cnt, ws, st, ex);
  if (e != hipSuccess) return e;
  if (stats_later) return hipSuccess;  // the statistics come from launch_assign_token
  const int NP = (N + 63) / 64 * 64;
  hipLaunchKernelGGL(route_finalize, dim3(1), dim3(1024), 0, st, part_p, part_cnt, pl.nblk, T, N, NP, routed_count, f,
                     P, l_aux, (ex.K < 1 || ex.expand) ? 1 : ex.K);
  return hipGetLastError();
}

hipError_t launch_assign_token(const RoutePlan& pl, int64_t T, int K, int N, int C, const int32_t* expert_id, double* term,
                               int32_t* routed_count, float* f, float* P, float* l_aux, int32_t* slot,
                               int32_t* token_of_slot, int32_t* kept_count, int32_t* n_dropped, int32_t* active,
                               int32_t* n_active, char* ws, hipStream_t st, bool finalize) {
  const float* part_p = reinterpret_cast<const float*>(ws + pl.off_part_p);
  const int32_t* part_cnt = reinterpret_cast<const int32_t*>(ws + pl.off_part_cnt);
  const int NP = (N + 63) / 64 * 64;
  // 256-thread workgroups for short lists (measured on the 384-expert decode
  // batch, T = 128: 15.7 against 22.7 us for the assignment stage); 1024 threads
  // otherwise (top-2 on the base layer, 8192 choices: 17.2 against 25.8 us)
#define SWM_ASSIGN_TOKEN(NTH, MULTI)                                                                              \
  hipLaunchKernelGGL((assign_token_expert<NTH, MULTI>), dim3((unsigned)N), dim3(NTH), 0, st, part_p, part_cnt, pl.nblk, \
                     T, K, N, NP, C, expert_id, routed_count, f, P, term, slot, token_of_slot, kept_count)
  if (T * K <= 2048) {
    if (K > 1) SWM_ASSIGN_TOKEN(256, true);
    else SWM_ASSIGN_TOKEN(256, false);
  } else {
    if (K > 1) SWM_ASSIGN_TOKEN(1024, true);
    else SWM_ASSIGN_TOKEN(1024, false);
  }
#undef SWM_ASSIGN_TOKEN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !finalize) return e;
  hipLaunchKernelGGL(assign_token_finalize, dim3(1), dim3(1024), 0, st, kept_count, term, N, T * K, l_aux, active,
                     n_active, n_dropped);
  return hipGetLastError();
}

}  // namespace swm
