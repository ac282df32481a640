// Fused expert backward on MFMA: one pass over an expert weight matrix computes
// both the activation gradient that multiplies it and its own gradient.
//
// Per expert e with kept rows m (its filled slots), gate scale s_m (gate value
// or 1) and the forward's hidden activation H (Switch Transformers summary
// page, Switch-layer passage: the gate value multiplies the expert output;
// "Top-1 Routing" page, Key parameters and compute: two-layer ReLU FFN):
//   pass over W2[e] (rows f = d_ff, columns k = d_model), Q = dY rows, S = s*H:
//     U^T[f][m] = sum_k W2[f][k] dY[m][k]     -> dZ = s U [H > 0], dg partials
//     dW2[f][k] = sum_m (s H)[m][f] dY[m][k]
//   pass over W1[e] (rows k = d_model, columns f = d_ff), Q = dZ rows, S = X:
//     dX^T[k][m] = sum_f W1[k][f] dZ[m][f]    -> dX_e (fp32)
//     dW1[k][f]  = sum_m X[m][k] dZ[m][f]
// A workgroup (4 waves) owns 64 consecutive rows of the weight matrix and walks
// its columns in 64-wide chunks, so every weight byte is read once and every
// gradient byte written once; the token rows (Q, S) come from L2.
//  * Weight fragments go from global memory straight into registers (16 bytes
//    per lane: 8 consecutive columns of one row, which is an MFMA operand
//    as is), STAGES chunks ahead.
//  * The Q chunk (rows m, 64 columns) sits in LDS and is read two ways: 16-byte
//    rows for U^T / dX^T (B operand: 8 consecutive columns of one row m), and
//    ds_read_b64_tr_b16 transposing reads for the weight gradient (A operand:
//    8 consecutive m of one column).  S (rows m, the workgroup's 64 weight
//    rows) is staged once and read transposed as the B operand.  16-byte chunk
//    q of LDS row m sits at q ^ g(m), g(m) = ((m >> 2) & 3) | (((m >> 1) & 1) << 2):
//    16 consecutive rows land on 16 distinct 16-byte bank groups (direct reads)
//    and the 4 rows x 2 chunks of a transposing read on 8 (conflict-free).
//  * Outputs: lane (c, kg) of an MFMA D tile holds rows 4kg..4kg+3 of column c,
//    so U^T / dX^T are computed with rows = weight rows (each lane stores 4
//    consecutive elements); the weight-gradient tile is computed transposed and
//    passes through LDS so that its stores write whole 128-byte rows.
// Rows m at or beyond kept_count are zero in LDS and never stored.
// ACC (the caller's accumulate flag): each weight-gradient piece is added to
// what the buffer holds (fp32 sum of the two bf16 values, rounded once) instead
// of overwriting it; experts that kept no token are not visited at all.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

typedef short v4i16_b __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_b lds_v4i16_b;

// ds_read_b64_tr_b16 in a plain function (a kernel template that names a gfx950
// builtin directly loses its host launch stub)
__device__ __forceinline__ u32x2 tr_read(const unsigned char* lds) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_b*)lds));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// byte offset of 16-byte chunk q of row m in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int lds_off(int m, int q) {
  const int g = ((m >> 2) & 3) | (((m >> 1) & 1) << 2);
  return m * 128 + ((q ^ g) << 4);
}

constexpr int kBwdXcds = 8;

}  // namespace

// MODE 2: pass over W2 (epilogue dZ, dg partials); MODE 1: pass over W1
// (epilogue dX_e).  MT = 16-row tiles of m (kept <= 16 MT); MQ = m rows in LDS
// (a multiple of 32: whole MFMA k-steps for the weight gradient).
template <int MT, int MODE, int STAGES, bool ACC>
__global__ __launch_bounds__(256, 2) void bwd_expert_fused(
    const uint16_t* __restrict__ Wt, int rows, int cols,
    const uint16_t* __restrict__ Q, const int32_t* __restrict__ q_gather,      // Q rows: gathered or [N][C][cols]
    const uint16_t* __restrict__ S, const int32_t* __restrict__ s_gather,      // S rows: gathered or [N][C][rows]
    const float* __restrict__ s_scale,                                         // per token (gate) or NULL
    uint16_t* __restrict__ G,                                                  // [N][rows][cols]
    uint16_t* __restrict__ dZ, const uint16_t* __restrict__ H, float* __restrict__ dgp,  // MODE 2
    float* __restrict__ dXe,                                                   // MODE 1
    const int32_t* __restrict__ kept_count, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ tos, int N, int C, int64_t q_rows) {
  constexpr int MQ = (MT * 16 + 31) / 32 * 32;
  constexpr int KSM = MQ / 32;  // m k-steps of the weight gradient
  __shared__ __attribute__((aligned(16))) unsigned char qt[2][MQ * 128];
  // the S tile is staged in the second Q buffer: it is read into sfrag before
  // the first Q chunk goes to the first buffer, and the second is written only
  // at the end of the first chunk's step.  The 20 KB this saves lets a third
  // workgroup onto each CU at 160 rows (large layer: w2 pass 6.01 -> 5.75 ms,
  // w1 pass 5.45 -> 5.12 ms)
  unsigned char* const stile = qt[1];
  __shared__ float red[4][MT * 16];
  __shared__ __attribute__((aligned(16))) unsigned char gstage[4 * 16 * 144];

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RB = rows >> 6;
  int n_act = n_active[0];
  if (n_act > N) n_act = N;
  const int64_t items = (int64_t)n_act * RB;
  // contiguous item ranges per XCD (blockIdx % 8): an expert's row blocks share
  // the L2 that holds its token rows
  const int nx = (gridDim.x % kBwdXcds == 0) ? kBwdXcds : 1;
  const int64_t per_x = (items + nx - 1) / nx;
  const int64_t local = blockIdx.x / nx;
  const int64_t item = (int64_t)(blockIdx.x % nx) * per_x + local;
  if (local >= per_x || item >= items) return;
  const int a = (int)(item / RB), rb = (int)(item - (int64_t)a * RB);
  const int e = __builtin_amdgcn_readfirstlane(active[a]);
  if (e < 0 || e >= N) return;
  int kept = __builtin_amdgcn_readfirstlane(kept_count[e]);
  if (kept > C) kept = C;
  if (kept > MT * 16) kept = MT * 16;  // the launcher picks MT >= C
  if (kept <= 0) return;
  const int r0 = rb * 64;
  const int64_t slot0 = (int64_t)e * C;

  // ---- S tile: rows m < kept, columns r0 .. r0+63, scaled by s_m (MODE 2) ----
  for (int p = tid; p < MQ * 8; p += 256) {
    const int m = p >> 3, q = p & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < kept) {
      const int64_t srow = s_gather != nullptr ? (int64_t)s_gather[slot0 + m] : slot0 + m;
      v = *reinterpret_cast<const u32x4*>(S + srow * rows + r0 + q * 8);
      if (s_scale != nullptr) {
        const float sc = s_scale[tos[slot0 + m]];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = pack_bf2(sc * bf2f(v[u] & 0xffffu), sc * bf2f(v[u] >> 16));
      }
    }
    *reinterpret_cast<u32x4*>(stile + lds_off(m, q)) = v;
  }

  // ---- Q chunk loader: rows m < kept, columns chunk*64 .. +63.  Buffer loads
  // without branches (rows at or beyond kept get an offset past the descriptor
  // and read as zero), so the compiler's wait counts keep the weight stream in
  // flight across them.
  constexpr int QP = (MQ * 8 + 255) / 256;  // 16-byte pieces per thread
  const __amdgpu_buffer_rsrc_t qres =
      q_gather != nullptr ? rsrc(Q, (int64_t)q_rows * cols * 2) : rsrc(Q + slot0 * cols, (int64_t)kept * cols * 2);
  int q_voff[QP], q_lds[QP];
#pragma unroll
  for (int i = 0; i < QP; ++i) {
    const int p = tid + 256 * i, m = p >> 3, q = p & 7;
    q_lds[i] = p < MQ * 8 ? lds_off(m, q) : -1;
    q_voff[i] = 0x7ffffff0;
    if (p < MQ * 8 && m < kept) {
      const int64_t src = q_gather != nullptr ? (int64_t)q_gather[slot0 + m] : (int64_t)m;
      q_voff[i] = (int)((src * cols + q * 8) * 2);
    }
  }
  auto load_q = [&](u32x4 (&dst)[QP], int chunk) {
#pragma unroll
    for (int i = 0; i < QP; ++i) dst[i] = bload16(qres, q_voff[i], chunk * 128);
  };
  auto store_q = [&](const u32x4 (&src)[QP], int buf) {
#pragma unroll
    for (int i = 0; i < QP; ++i)
      if (q_lds[i] >= 0) *reinterpret_cast<u32x4*>(&qt[buf][q_lds[i]]) = src[i];
  };

  // ---- weight fragments: row r0 + 16 w + c, columns chunk*64 + 32 ks + 8 kg ----
  const __amdgpu_buffer_rsrc_t wres = rsrc(Wt + (int64_t)e * rows * cols, (int64_t)rows * cols * 2);
  const int w_voff = ((r0 + 16 * w + c) * cols + 8 * kg) * 2;
  const int nch = cols >> 6;
  auto load_w = [&](u32x4 (&dst)[2], int chunk) {
    const int ch = chunk < nch ? chunk : nch - 1;  // past the end: re-read the last chunk (cache hit)
    dst[0] = bload16(wres, w_voff, ch * 128);
    dst[1] = bload16(wres, w_voff, ch * 128 + 64);
  };

  f32x4 accP[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) accP[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment offsets inside a Q chunk / the S tile
  int qb_off[MT][2];  // B of U^T / dX^T: row m = 16 mt + c, chunk 4 ks + kg
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qb_off[mt][ks] = lds_off(16 * mt + c, 4 * ks + kg);
  // transposing reads: row m = 32 ksm + 8 kg + 4 h + (c >> 2), columns 16 t + 4 (c & 3)
  auto tr_off = [&](int ksm, int h, int t) {
    const int m = 32 * ksm + 8 * kg + 4 * h + (c >> 2);
    const int col = 16 * t + 4 * (c & 3);
    return lds_off(m, col >> 3) + ((col >> 2) & 1) * 8;
  };
  u32x4 sfrag[KSM];  // B of the weight gradient: S[m][r0 + 16 w + c], fixed for the whole walk
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < KSM; ++ks) {
    const u32x2 lo = tr_read(stile + tr_off(ks, 0, w)), hi = tr_read(stile + tr_off(ks, 1, w));
    sfrag[ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }

  u32x4 wbuf[STAGES][2];
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) load_w(wbuf[s], s);
  {
    u32x4 q0[QP];
    load_q(q0, 0);
    store_q(q0, 0);
  }
  __syncthreads();

  uint16_t* gbase = G + (int64_t)e * rows * cols + (int64_t)(r0 + 16 * w) * cols;
  const int nch_pad = (nch + STAGES - 1) / STAGES * STAGES;
  for (int it = 0; it < nch_pad; it += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int ch = it + u;
      if (ch < nch) {  // uniform
        // the next Q chunk first, then the weight prefetch: waiting for the Q
        // loads at the end of this step leaves the weight loads in flight
        u32x4 qn[QP];
        load_q(qn, ch + 1 < nch ? ch + 1 : ch);
        load_w(wbuf[(u + STAGES - 1) % STAGES], ch + STAGES - 1);
        const unsigned char* qb = qt[ch & 1];
        // U^T / dX^T: rows r (this wave's 16), columns m
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const u32x4 bq = *reinterpret_cast<const u32x4*>(qb + qb_off[mt][ks]);
            accP[mt] = mfma_bf16_16x16x32(wbuf[u][ks], bq, accP[mt]);
          }
        // weight gradient, transposed: rows = the chunk's 64 columns (4 tiles),
        // columns = this wave's 16 weight rows.  The 16 x 64 tile goes through
        // the wave's own LDS region (row stride 144 bytes: conflict-free 8-byte
        // writes), then leaves as 8 whole 128-byte rows per store instruction
        // (partial-line stores cost more than half the pass time).
        {
          unsigned char* gs = gstage + w * 16 * 144;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
              const u32x2 lo = tr_read(qb + tr_off(ks, 0, t)), hi = tr_read(qb + tr_off(ks, 1, t));
              g = mfma_bf16_16x16x32(u32x4{lo[0], lo[1], hi[0], hi[1]}, sfrag[ks], g);
            }
            // lane: chunk columns 16 t + 4 kg + i of weight row 16 w + c
            u32x2 o;
            o[0] = pack_bf2(g[0], g[1]);
            o[1] = pack_bf2(g[2], g[3]);
            *reinterpret_cast<u32x2*>(gs + c * 144 + (16 * t + 4 * kg) * 2) = o;
          }
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            const int row = 8 * hlf + (lane >> 3), q = lane & 7;
            u32x4 v = *reinterpret_cast<const u32x4*>(gs + row * 144 + q * 16);
            uint16_t* gp = gbase + (int64_t)row * cols + ch * 64 + q * 8;
            if constexpr (ACC) {  // accumulate: the stored gradient plus this one, summed in fp32
              const u32x4 old = *reinterpret_cast<const u32x4*>(gp);
#pragma unroll
              for (int u = 0; u < 4; ++u)
                v[u] = pack_bf2(bf2f(old[u] & 0xffffu) + bf2f(v[u] & 0xffffu), bf2f(old[u] >> 16) + bf2f(v[u] >> 16));
            }
            *reinterpret_cast<u32x4*>(gp) = v;
          }
        }
        if (ch + 1 < nch) store_q(qn, (ch + 1) & 1);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: accP[mt] = P^T[r = r0 + 16 w + 4 kg + i][m = 16 mt + c] ----
  const int rr = r0 + 16 * w + 4 * kg;
  if constexpr (MODE == 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
      float part = 0.f;
      if (m < kept) {
        const int64_t row = slot0 + m;
        const float sc = s_scale != nullptr ? s_scale[tos[row]] : 1.f;
        const u32x2 hv = *reinterpret_cast<const u32x2*>(H + row * rows + rr);
        float hf[4] = {bf2f(hv[0] & 0xffffu), bf2f(hv[0] >> 16), bf2f(hv[1] & 0xffffu), bf2f(hv[1] >> 16)};
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          part = fmaf(accP[mt][i], hf[i], part);
          z[i] = hf[i] > 0.f ? sc * accP[mt][i] : 0.f;
        }
        u32x2 o;
        o[0] = pack_bf2(z[0], z[1]);
        o[1] = pack_bf2(z[2], z[3]);
        *reinterpret_cast<u32x2*>(dZ + row * rows + rr) = o;
      }
      // sum over kg (lanes c, c+16, c+32, c+48), then over the 4 waves in order
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (kg == 0) red[w][m] = part;
    }
    __syncthreads();
    for (int m = tid; m < kept; m += 256)
      dgp[(slot0 + m) * RB + rb] = ((red[0][m] + red[1][m]) + red[2][m]) + red[3][m];
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
      if (m < kept)
        *reinterpret_cast<f32x4*>(dXe + (slot0 + m) * rows + rr) = accP[mt];
    }
  }
}

// zero the weight gradients of experts that kept no token (dW1 and dW2 of one
// expert are `per` elements each)
__global__ __launch_bounds__(256) void zero_idle_experts(uint16_t* __restrict__ g1, uint16_t* __restrict__ g2,
                                                         const int32_t* __restrict__ kept_count, int64_t per) {
  const int e = blockIdx.y;
  if (kept_count[e] > 0) return;
  const int64_t n16 = per / 8;  // 16-byte pieces
  u32x4* a = reinterpret_cast<u32x4*>(g1 + (int64_t)e * per);
  u32x4* b = reinterpret_cast<u32x4*>(g2 + (int64_t)e * per);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    a[i] = z;
    b[i] = z;
  }
}

// ----------------------------------------------------------------------------
// m up to 160 rows (10 MFMA tiles of accumulators); the token matrices dy and x
// addressed through 32-bit buffer offsets
bool fused_expert_bwd_applies(int64_t T, int C, int d, int dff) {
  return C <= 160 && d % 64 == 0 && dff % 64 == 0 && T * d * 2 < ((int64_t)1 << 31);
}

template <int MT, int MODE, bool ACC>
static hipError_t launch_fused_acc(const ExpertBwdArgs& A, hipStream_t st) {
  const int rows = MODE == 2 ? A.dff : A.d, cols = MODE == 2 ? A.d : A.dff;
  int64_t grid = (int64_t)A.N * (rows / 64);
  grid = (grid + kBwdXcds - 1) / kBwdXcds * kBwdXcds;
  const auto* W = static_cast<const uint16_t*>(MODE == 2 ? A.w2 : A.w1);
  if (MODE == 2)
    hipLaunchKernelGGL((bwd_expert_fused<MT, 2, 3, ACC>), dim3((unsigned)grid), dim3(256), 0, st, W, rows, cols,
                       static_cast<const uint16_t*>(A.dy), A.tos, static_cast<const uint16_t*>(A.h), nullptr,
                       A.gate, static_cast<uint16_t*>(A.dw2), static_cast<uint16_t*>(A.dz),
                       static_cast<const uint16_t*>(A.h), A.dgp, nullptr, A.kept, A.active, A.n_active, A.tos, A.N,
                       A.C, A.T);
  else
    hipLaunchKernelGGL((bwd_expert_fused<MT, 1, 3, ACC>), dim3((unsigned)grid), dim3(256), 0, st, W, rows, cols,
                       static_cast<const uint16_t*>(A.dz), nullptr, static_cast<const uint16_t*>(A.x), A.tos,
                       nullptr, static_cast<uint16_t*>(A.dw1), nullptr, nullptr, nullptr, A.dxe, A.kept, A.active,
                       A.n_active, A.tos, A.N, A.C, (int64_t)0);
  return hipGetLastError();
}

template <int MT, int MODE>
static hipError_t launch_fused_mt(const ExpertBwdArgs& A, hipStream_t st) {
  return A.accum ? launch_fused_acc<MT, MODE, true>(A, st) : launch_fused_acc<MT, MODE, false>(A, st);
}

template <int MODE>
static hipError_t launch_fused(const ExpertBwdArgs& A, hipStream_t st) {
  const int mt = (A.C + 15) / 16;
  if (mt <= 1) return launch_fused_mt<1, MODE>(A, st);
  if (mt <= 2) return launch_fused_mt<2, MODE>(A, st);
  if (mt <= 3) return launch_fused_mt<3, MODE>(A, st);
  if (mt <= 4) return launch_fused_mt<4, MODE>(A, st);
  if (mt <= 6) return launch_fused_mt<6, MODE>(A, st);
  if (mt <= 8) return launch_fused_mt<8, MODE>(A, st);
  return launch_fused_mt<10, MODE>(A, st);
}

hipError_t launch_zero_idle_experts(const ExpertBwdArgs& A, hipStream_t st) {
  hipLaunchKernelGGL(zero_idle_experts, dim3(64, (unsigned)A.N), dim3(256), 0, st, static_cast<uint16_t*>(A.dw1),
                     static_cast<uint16_t*>(A.dw2), A.kept, (int64_t)A.d * A.dff);
  return hipGetLastError();
}

hipError_t launch_expert_bwd_pass(const ExpertBwdArgs& A, int which, hipStream_t st) {
  return which == 2 ? launch_fused<2>(A, st) : launch_fused<1>(A, st);
}

}  // namespace swm
