// Dense LDS-tiled MFMA GEMMs for the shared expert's backward: the shared
// dense expert ("Top-1 Routing" page, History: an always-on shared expert) is
// y += ReLU(x Ws1) Ws2 on every token, so its gradients are four dense GEMMs
// over all T tokens, each with 2 T d d_ff FLOP:
//   dZs = (dY Ws2^T) * [Hs > 0]     A = dY [T][d],    B = Ws2 stored [d_ff][d]   (B transposed)
//   dXs = dZs Ws1^T  (fp32)          A = dZs [T][d_ff], B = Ws1 stored [d][d_ff]   (B transposed)
//   dWs2 = Hs^T dY                   A = Hs stored [T][d_ff] (A transposed), B = dY [T][d]
//   dWs1 = x^T dZs                   A = x stored [T][d] (A transposed),     B = dZs [T][d_ff]
// The kernel is the direct-to-LDS tile of the forward's expert GEMM with both
// operand orientations: an operand whose rows run along K (A [M][K], or B
// stored [N][K]) sits in LDS as 16-row blocks of 64 bytes per 32-deep step and
// is read with 16-byte direct reads; an operand whose rows are K-rows (B
// [K][N], or A stored [K][M]) sits as 32 K-rows and is read with the
// transposing ds_read_b64_tr_b16.  Both layouts fill 1 KB LDS blocks, so the
// loads, stages and wait counts are those of the forward tile: every load is a
// buffer load straight into LDS, S stages keep S - 1 steps in flight, and one
// barrier per step publishes a stage without draining the loads behind it.
#include "common.hpp"
#include "kernels.hpp"

namespace swm {

namespace {

constexpr int kDenseXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dn_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// row tiles: 16-byte chunk q of row r at r * 64 + ((q ^ swz(r)) << 4)
__device__ __forceinline__ int dn_row_swz(int r) {
  return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 1) ^ (r >> 3) ^ (r >> 6)) & 1) << 1);
}
// K-row tiles: 16-byte chunk c of K-row k at k * row_bytes + ((c ^ swz(k)) << 4)
__device__ __forceinline__ int dn_k_swz(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }

#define SWM_DN_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

typedef short v4i16_dn __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_dn;
typedef __attribute__((address_space(3))) v4i16_dn lds_v4i16_dn;

// gfx950 builtins in plain functions (a kernel template naming them directly
// loses its host launch stub)
__device__ __forceinline__ void dn_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_dn*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ u32x2 dn_tr16(const unsigned char* lds) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_dn*)lds));
}

}  // namespace

// out[M][Ncols] = A . B over K.  AT: A stored [K][M]; BNT: B stored [Ncols][K].
// EPI 0: bf16 out; 1: fp32 out; 2: bf16 out times [H[m][n] > 0] (H bf16 [M][Ncols]).
// A workgroup (2 WN waves, 2 x WN) owns a BM x TN tile, BM = 32 MTW, TN = 16 NJ WN.
template <int MTW, int NJ, int S, bool AT, bool BNT, int EPI, int WN>
__global__ __launch_bounds__(128 * WN, WN > 2 ? 1 : 2) void dense_tile_dma(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                         void* __restrict__ out, const uint16_t* __restrict__ H, int M,
                                                         int K, int Ncols, int mch) {
  constexpr int BM = 32 * MTW, TN = 16 * NJ * WN, NWV = 2 * WN;
  constexpr int AB = BM / 16, WB = TN / 16, NB = AB + WB;
  constexpr int LW = (NB + NWV - 1) / NWV;
  static_assert(NB >= NWV, "every wave loads at least one block");
  constexpr int ARB = BM * 2, BRB = TN * 2;  // bytes per K-row of a K-row tile
  constexpr int SB = NB * 1024;
  static_assert(S >= 2 && S <= 4, "2 to 4 LDS stages");
  __shared__ __attribute__((aligned(1024))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[S > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[S > 3 ? SB : 16];
  auto stage = [&](int i) -> unsigned char* { return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3; };

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int NT = Ncols / TN;
  const int64_t tiles = (int64_t)mch * NT;
  const int nx = (gridDim.x % kDenseXcds == 0) ? kDenseXcds : 1;
  const int64_t per_x = (tiles + nx - 1) / nx;
  const int64_t local = blockIdx.x / nx;
  const int64_t tile = (int64_t)(blockIdx.x % nx) * per_x + local;
  if (local >= per_x || tile >= tiles) return;
  // up to 8 m-chunks walk the column blocks together (shared panels in L2)
  const int GM = mch < 8 ? mch : 8;
  const int grp = (int)(tile / ((int64_t)GM * NT));
  const int gm_here = (mch - grp * GM) < GM ? (mch - grp * GM) : GM;
  const int in_g = (int)(tile - (int64_t)grp * GM * NT);
  const int mc = grp * GM + in_g % gm_here;
  const int nt = in_g / gm_here;
  const int m0 = mc * BM;
  int rows = M - m0;
  if (rows > BM) rows = BM;
  const int n0 = nt * TN;
  const int ksteps = K >> 5;

  // descriptors: row-major-along-K A covers this tile's rows only (rows beyond
  // M read zero); K-row operands cover the whole matrix
  const __amdgpu_buffer_rsrc_t ares =
      AT ? dn_rsrc(A, (int64_t)K * M * 2) : dn_rsrc(A + (int64_t)m0 * K, (int64_t)rows * K * 2);
  const __amdgpu_buffer_rsrc_t bres = dn_rsrc(B, (int64_t)K * Ncols * 2);

  int voff[LW], lds_blk[LW], stp[LW];
  bool is_a[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    int j = w + NWV * i;
    if (j >= NB) j -= NWV;  // repeats block j - NWV: same bytes to the same place
    lds_blk[i] = j * 1024;
    is_a[i] = j < AB;
    if (j < AB) {
      if (!AT) {  // 16 rows of 64 bytes
        const int r = 16 * j + (lane >> 2), q = (lane & 3) ^ dn_row_swz(r);
        voff[i] = r < rows ? (r * K + q * 8) * 2 : 0x7ffffff0;
        stp[i] = 64;
      } else {    // K-rows of BM columns
        const int o = j * 1024 + lane * 16;
        const int k = o / ARB, pc = (o % ARB) >> 4, lc = pc ^ dn_k_swz(k);
        voff[i] = (k * M + m0 + lc * 8) * 2;
        stp[i] = 32 * M * 2;
      }
    } else {
      const int jb = j - AB;
      if (BNT) {  // 16 rows (columns n) of 64 bytes
        const int r = 16 * jb + (lane >> 2), q = (lane & 3) ^ dn_row_swz(r);
        voff[i] = ((n0 + r) * K + q * 8) * 2;
        stp[i] = 64;
      } else {    // K-rows of TN columns
        const int o = jb * 1024 + lane * 16;
        const int k = o / BRB, pc = (o % BRB) >> 4, lc = pc ^ dn_k_swz(k);
        voff[i] = (k * Ncols + n0 + lc * 8) * 2;
        stp[i] = 32 * Ncols * 2;
      }
    }
  }
  auto issue = [&](int st, int s) {
    const int sc = s < ksteps ? s : ksteps - 1;  // past the end: re-read the last step (cache hit)
    unsigned char* base = stage(st);
#pragma unroll
    for (int i = 0; i < LW; ++i) dn_dma16(is_a[i] ? ares : bres, base + lds_blk[i], voff[i], sc * stp[i]);
  };

  // fragment addresses inside a stage
  int a_rd[MTW][2], b_rd[NJ][2];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!AT) {
        const int r = wm * (BM / 2) + mt * 16 + c;
        a_rd[mt][h] = r * 64 + ((kg ^ dn_row_swz(r)) << 4);
      } else {
        const int k = 8 * kg + 4 * h + (c >> 2);
        const int m = wm * (BM / 2) + mt * 16 + 4 * (c & 3);
        a_rd[mt][h] = k * ARB + (((m >> 3) ^ dn_k_swz(k)) << 4) + ((m >> 2) & 1) * 8;
      }
    }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (BNT) {
        const int r = wn * 16 * NJ + 16 * j + c;
        b_rd[j][h] = AB * 1024 + r * 64 + ((kg ^ dn_row_swz(r)) << 4);
      } else {
        const int k = 8 * kg + 4 * h + (c >> 2);
        const int n = wn * 16 * NJ + 16 * j + 4 * (c & 3);
        b_rd[j][h] = AB * 1024 + k * BRB + (((n >> 3) ^ dn_k_swz(k)) << 4) + ((n >> 2) & 1) * 8;
      }
    }

  f32x4 acc[MTW][NJ];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st) {
    const unsigned char* base = stage(st);
    u32x4 bf[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (BNT) {
        bf[j] = *reinterpret_cast<const u32x4*>(base + b_rd[j][0]);
      } else {
        const u32x2 l2 = dn_tr16(base + b_rd[j][0]), h2 = dn_tr16(base + b_rd[j][1]);
        bf[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      u32x4 af;
      if (!AT) {
        af = *reinterpret_cast<const u32x4*>(base + a_rd[mt][0]);
      } else {
        const u32x2 l2 = dn_tr16(base + a_rd[mt][0]), h2 = dn_tr16(base + a_rd[mt][1]);
        af = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[mt][j] = mfma_bf16_16x16x32(af, bf[j], acc[mt][j]);
    }
  };
  auto step_sync = [&]() {
    SWM_DN_WAIT_VMCNT_LGKM0((S - 2) * LW);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int s0 = 0; s0 < S - 1; ++s0) issue(s0, s0);
  int it = 0;
  for (; it + S <= ksteps; it += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      step_sync();
      issue((u + S - 1) % S, it + u + S - 1);
      compute(u);
    }
  }
#pragma unroll
  for (int u = 0; u < S - 1; ++u) {
    if (it + u < ksteps) {
      step_sync();
      issue((u + S - 1) % S, it + u + S - 1);
      compute(u);
    }
  }
  SWM_DN_WAIT_VMCNT_LGKM0(0);  // no load may still be writing LDS when the workgroup exits
  __syncthreads();              // every wave is done with the stages: they now stage the output

  // A lane holds rows 4 kg + i of each 16-row tile and column c of each
  // 16-column tile.  Each 16-row slice of the wave's tile goes through an LDS
  // region of its own (rows padded by 16 bytes so that the four kg row groups
  // fall on different banks) and leaves as 16-byte non-temporal stores over
  // whole 128-byte lines.  EPI 2 applies the mask to the staged chunk, from a
  // 16-byte load of the same chunk of H.
  constexpr int EB = EPI == 1 ? 4 : 2;        // output bytes per element
  constexpr int ROWB = 16 * NJ * EB + 16;     // staged row: the wave's 16 NJ columns
  constexpr int CH = 16 * NJ * EB / 16;       // 16-byte chunks per staged row
  constexpr int WPS = SB / (16 * ROWB);        // waves staged per LDS stage
  static_assert(WPS * S >= NWV, "every wave's staging fits the stages");
  unsigned char* ost = stage(w / WPS) + (w % WPS) * 16 * ROWB;
  const int64_t col0 = (int64_t)n0 + wn * 16 * NJ;
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        unsigned char* p = ost + (kg * 4 + i) * ROWB + (16 * j + c) * EB;
        if (EPI == 1)
          *reinterpret_cast<float*>(p) = acc[mt][j][i];
        else
          *reinterpret_cast<uint16_t*>(p) = (uint16_t)f2bf(acc[mt][j][i]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q0 = 0; q0 < 16 * CH; q0 += 64) {
      const int q = q0 + lane, r = q / CH, ch = q - r * CH;
      const int rl = wm * (BM / 2) + mt * 16 + r;
      u32x4 v = *reinterpret_cast<const u32x4*>(ost + r * ROWB + ch * 16);
      if (rl < rows) {
        const int64_t off = (int64_t)(m0 + rl) * Ncols + col0 + ch * (16 / EB);  // elements
        if (EPI == 2) {  // keep where H > 0: bf16 bits in (0, 0x7f80] (positive, up to +inf)
          const u32x4 h = *reinterpret_cast<const u32x4*>(H + off);
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const uint32_t lo = h[q2] & 0xffffu, hi = h[q2] >> 16;
            const uint32_t keep = ((lo - 1u) < 0x7f80u ? 0x0000ffffu : 0u) | ((hi - 1u) < 0x7f80u ? 0xffff0000u : 0u);
            v[q2] &= keep;
          }
        }
        if (EPI == 1)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<float*>(out) + off));
        else
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + off));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next slice overwrites the region
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ----------------------------------------------------------------------------
// 128 x 256 tiles on 8 waves (2 x 4, each 64 x 64), 3 stages: the forward's shared-FFN configuration
template <bool AT, bool BNT, int EPI>
static hipError_t launch_dense(const void* A, const void* B, void* out, const void* H, int M, int K, int Ncols,
                               hipStream_t st) {
  constexpr int MTW = 4, NJ = 4, S = 3, WN = 4, BM = 32 * MTW, TN = 16 * NJ * WN;
  const int mch = (M + BM - 1) / BM;
  int64_t grid = (int64_t)mch * (Ncols / TN);
  grid = (grid + kDenseXcds - 1) / kDenseXcds * kDenseXcds;
  hipLaunchKernelGGL((dense_tile_dma<MTW, NJ, S, AT, BNT, EPI, WN>), dim3((unsigned)grid), dim3(128 * WN), 0, st,
                     static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), out,
                     static_cast<const uint16_t*>(H), M, K, Ncols, mch);
  return hipGetLastError();
}

// the tiles need whole 32-deep steps and whole 128-row / 256-column blocks
// where an operand is addressed by K-rows, and every matrix under 2^31 bytes
// for the 32-bit buffer offsets
bool dense_bwd_applies(int64_t T, int d, int dffs) {
  const int64_t lim = (int64_t)1 << 31;
  return T % 128 == 0 && d % 256 == 0 && dffs % 256 == 0 && T * d * 2 < lim && T * dffs * 2 < lim &&
         (int64_t)d * dffs * 2 < lim;
}

hipError_t launch_shared_bwd_dense(const void* x, const void* dy, const void* ws1, const void* ws2, const void* hs,
                                   void* dzs, float* dxs, void* dws1, void* dws2, int64_t T, int d, int dffs,
                                   hipStream_t st) {
  const int Ti = (int)T;
  // dZs [T][dffs] = (dY Ws2^T) * [Hs > 0]
  hipError_t e = launch_dense<false, true, 2>(dy, ws2, dzs, hs, Ti, d, dffs, st);
  if (e != hipSuccess) return e;
  // dWs2 [dffs][d] = Hs^T dY
  if ((e = launch_dense<true, false, 0>(hs, dy, dws2, nullptr, dffs, Ti, d, st)) != hipSuccess) return e;
  // dWs1 [d][dffs] = x^T dZs
  if ((e = launch_dense<true, false, 0>(x, dzs, dws1, nullptr, d, Ti, dffs, st)) != hipSuccess) return e;
  // dXs [T][d] = dZs Ws1^T (fp32)
  return launch_dense<false, true, 1>(dzs, ws1, dxs, nullptr, Ti, dffs, d, st);
}

}  // namespace swm
