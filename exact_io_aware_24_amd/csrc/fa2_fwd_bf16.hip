// Exact attention forward, bf16 inputs, bf16 MFMA on gfx950 (CDNA4).
//
// What is computed (per batch*head, per query block of 128 rows):
//   for each K/V tile of BC keys (the inner loop of FlashAttention-2's order:
//   query blocks outside, K/V blocks inside -- itimpress.au page
//   "FlashAttention scaling, multi-GPU training and weight quantisation",
//   section 1):
//     S  = K_tile . Q_block^T            bf16 MFMA, fp32 accumulate
//     m' = max(m, rowmax(S) * c)          c = scale * log2(e)   (base-2 units)
//     P~ = 2^(S*c - m')                   fp32, hardware exp2
//     l  = l * 2^(m - m') + rowsum(P~)
//     O~ = O~ * 2^(m - m') + P~ . V_tile  P~ rounded to bf16, MFMA, fp32 acc
//   and after the last tile O = O~ / l, lse = (m + log2 l) * ln 2.
// The running (m, l, O~) update is the two-block online-softmax merge of the
// shakilmahmud.com page "Large language models part 06: FlashAttention --
// GPU SRAM, tiling, online softmax", section 2, with O~ kept unnormalised so
// that the single division by l happens once at the end (FlashAttention-2's
// reduction of non-matmul work, the same itimpress.au section).  One
// workgroup per (batch*head, query block) spreads one head over many compute
// units (improvement 2 of the "FlashAttention-2 (BN)" wiki article).
//
// gfx950 mapping (this library's design, not the pages'):
//  * 256 threads = 4 wave64s; wave w owns query rows [32w, 32w+32) of the
//    block, so the softmax statistics of a row never leave its wave (the
//    wiki article's improvement 3: no shared-memory exchange between warps
//    for the softmax).
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//    32 queries held in registers for the whole kernel.  In the 32x32 result
//    each lane holds ONE query (lane % 32) and 16 keys, so the row max and
//    row sum are in-lane reductions plus a single v_permlane32_swap between
//    the two half-waves, and the rescale factor is a per-lane scalar.
//  * The K rows feeding MFMA row m are permuted (bits 2 and 3 of m swapped)
//    so that the eight keys a lane holds for each 16-key step are contiguous;
//    the fp32 result registers then convert directly into the B operand of
//    O^T += V^T P^T, and V^T is read with one 16-byte LDS load per operand.
//  * K is staged row-major and V transposed (V^T, keys contiguous) in LDS,
//    both with XOR swizzles of their 16-byte chunks so that every 8-lane
//    phase of a 128-bit LDS access touches 32 distinct banks.  The next tile
//    is fetched from HBM into registers while the current one is consumed;
//    LDS is double-buffered, one barrier per tile.
//  * Causal: tiles past a wave's last query are skipped (the wave only
//    helps to stage them); the mask is applied only in tiles that cross the
//    diagonal or the ragged end of the sequence.  Query blocks are issued
//    longest first.
//  * Workgroup ids are remapped so that the blocks of one head run on the
//    same XCD (hardware deals workgroups round-robin over the 8 XCDs), which
//    keeps that head's K/V in one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = kBf16RowsPerBlock;  // 128 query rows per workgroup
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

struct Params {
  const uint16_t *q, *k, *v;
  void *o;
  float *lse;
  int n;          // sequence length
  int n_qblocks;  // ceil(n / 128)
  int total;      // bh * n_qblocks (grid size)
  float c;        // scale * log2(e)
};

// Keys per K/V tile: 64 at d = 128, 128 at d = 64 (16 KB of K and 16 KB of V
// either way, 32 MFMA per wave per tile).
template <int D>
struct TileCfg {
  static constexpr int BC = (D == 128) ? 64 : 128;
};

// Row permutation inside each 16-row group: swap bits 2 and 3.
__device__ __forceinline__ int perm16(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Swizzle of V^T rows: 16-byte chunk j of row c lives at chunk j ^ vsw(c).
__device__ __forceinline__ int vsw(int c) { return (c ^ (c >> 3)) & 7; }

// Both half-waves combined: returns (x of lanes 0-31, x of lanes 32-63) as
// seen from every lane.
__device__ __forceinline__ void halves(float x, float &lo, float &hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

template <int D, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(Params p) {
  constexpr int BC = TileCfg<D>::BC;
  constexpr int KCH = D / 8;                        // 16-byte chunks per K row
  constexpr int KMASK = (KCH < 16 ? KCH : 16) - 1;  // K swizzle width
  constexpr int NKT = BC / 32;                      // 32-key sub-tiles
  constexpr int NDT = D / 16;                       // 16-dim MFMA k-steps
  constexpr int NCT = D / 32;                       // 32-wide O^T row tiles
  constexpr int KLOADS = BC * KCH / kThreads;       // 16-byte K chunks/thread
  constexpr int VCOLS = D / 4;                      // 4-column V groups
  static_assert(KLOADS * kThreads == BC * KCH, "K tile split");
  static_assert((BC / 8) * VCOLS == kThreads, "V tile split");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * BC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int lr = lane & 31;  // query column of this lane in S^T / O^T
  const int hh = lane >> 5;  // half-wave

  // ---- workgroup -> (head, query block) --------------------------------
  const int w = blockIdx.x;
  const int per_xcd = p.total >> 3;
  int logical = w;
  if (w < (per_xcd << 3)) logical = (w & 7) * per_xcd + (w >> 3);
  const int bh = logical / p.n_qblocks;
  const int qbl = logical - bh * p.n_qblocks;
  const int qb = CAUSAL ? (p.n_qblocks - 1 - qbl) : qbl;

  const int N = p.n;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const uint16_t *__restrict__ qh = p.q + head;
  const uint16_t *__restrict__ kh = p.k + head;
  const uint16_t *__restrict__ vh = p.v + head;
  const int q0 = qb * kRows;      // first query of the block
  const int qw = q0 + wv * 32;    // first query of this wave
  const int qi = qw + lr;         // this lane's query

  // ---- Q into registers (B operand of S^T = K Q^T) ---------------------
  float c = p.c;
  uint32_t qflip = 0;
  if (c < 0.f) {  // exact: negate q (bf16 sign bit) and use -c
    c = -c;
    qflip = 0x80008000u;
  }
  bf16x8 qreg[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) {
      x = *reinterpret_cast<const u32x4 *>(qh + static_cast<size_t>(qi) * D +
                                            16 * t + 8 * hh);
      x ^= qflip;
    }
    qreg[t] = __builtin_bit_cast(bf16x8, x);
  }

  // ---- tile staging ----------------------------------------------------
  const int kend = CAUSAL ? min(N, q0 + kRows) : N;
  const int ntiles = (kend + BC - 1) / BC;

  u32x4 kpre[KLOADS];
  u32x2 vpre[8];
  const int vcc = tid % VCOLS;  // this thread's 4-column group of V
  const int vjg = tid / VCOLS;  // and its 8-key group

  auto gload = [&](int j0) {
#pragma unroll
    for (int it = 0; it < KLOADS; ++it) {
      const int id = tid + kThreads * it;
      const int row = id / KCH, ch = id % KCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j0 + row < N)
        x = *reinterpret_cast<const u32x4 *>(
            kh + static_cast<size_t>(j0 + row) * D + ch * 8);
      kpre[it] = x;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = j0 + vjg * 8 + r;
      u32x2 x = {0u, 0u};
      if (row < N)
        x = *reinterpret_cast<const u32x2 *>(vh + static_cast<size_t>(row) * D +
                                              vcc * 4);
      vpre[r] = x;
    }
  };

  auto swrite = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KLOADS; ++it) {
      const int id = tid + kThreads * it;
      const int row = id / KCH, ch = id % KCH;
      const int pos = ch ^ (perm16(row) & KMASK);
      *reinterpret_cast<u32x4 *>(&Ks[buf][row * D + pos * 8]) = kpre[it];
    }
    // 8 keys x 4 columns -> 4 columns x 8 keys (bf16 transpose in registers)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 outv;
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t a = (e < 2) ? vpre[2 * pr].x : vpre[2 * pr].y;
        const uint32_t b = (e < 2) ? vpre[2 * pr + 1].x : vpre[2 * pr + 1].y;
        outv[pr] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                           : ((a & 0xffffu) | (b << 16));
      }
      const int col = vcc * 4 + e;
      const int pos = vjg ^ vsw(col);
      *reinterpret_cast<u32x4 *>(&Vs[buf][col * BC + pos * 8]) = outv;
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();

  f32x16 oacc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[ct][r] = 0.f;
  float m_run = -INFINITY;  // running max, base-2 scaled units
  float l_run = 0.f;        // this half-wave's share of the running sum

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BC;
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) gload(j0 + BC);

    const bool active = !CAUSAL || j0 <= qw + 31;
    if (active) {
      // -- S^T = K Q^T ---------------------------------------------------
      f32x16 s[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        const uint16_t *krow = &Ks[buf][(32 * kt + perm16(lr)) * D];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int pos = (2 * dt + hh) ^ (lr & KMASK);
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + pos * 8);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[dt], s[kt],
                                                          0, 0, 0);
        }
      }
      // -- mask (diagonal / ragged tiles only) ---------------------------
      // register r of sub-tile kt holds key j0 + 32kt + 16(r/8) + 8hh + r%8
      const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * kt + 16 * (r >> 3) + 8 * hh + (r & 7);
            if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
          }
      }
      // -- online softmax --------------------------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      float mlo, mhi;
      halves(mx, mlo, mhi);
      mx = fmaxf(mlo, mhi);
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float m_new = fmaxf(m_run, m_tile);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      bf16x8 pb[NKT][2];
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sv = s[kt][8 * u + e];
            float x = fast_exp2(__builtin_fmaf(sv, c, -m_use));
            if (need_mask) x = (sv == -INFINITY) ? 0.f : x;
            rs += x;
            pb[kt][u][e] = static_cast<__bf16>(x);
          }
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;

      // -- O^T += V^T P^T --------------------------------------------------
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int chunk = 4 * kt + 2 * u + hh;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const int col = 32 * ct + lr;
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                &Vs[buf][col * BC + (chunk ^ vsw(col)) * 8]);
            oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, pb[kt][u], oacc[ct], 0, 0, 0);
          }
        }
    }

    if (more) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, lse ----------------------------------------
  float llo, lhi;
  halves(l_run, llo, lhi);
  const float l_tot = llo + lhi;
  const float inv = 1.0f / l_tot;
  if (qi < N) {
    // O^T register r of row tile ct holds column 32ct + 8(r/4) + 4hh + r%4
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = 32 * ct + 8 * a + 4 * hh;
        const size_t off = static_cast<size_t>(qi) * D + col;
        if (O32) {
          f32x4 ov;
#pragma unroll
          for (int b = 0; b < 4; ++b) ov[b] = oacc[ct][4 * a + b] * inv;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + head + off) = ov;
        } else {
          __bf16 ob[4];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            ob[b] = static_cast<__bf16>(oacc[ct][4 * a + b] * inv);
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.o) + head + off) =
              __builtin_bit_cast(u32x2, ob);
        }
      }
    if (p.lse && hh == 0)
      p.lse[static_cast<size_t>(bh) * N + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool O32>
hipError_t launch(const Params &prm, hipStream_t s) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, O32>), dim3(prm.total),
                     dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Params &prm, bool causal, bool o32, hipStream_t s) {
  if (causal)
    return o32 ? launch<D, true, true>(prm, s) : launch<D, true, false>(prm, s);
  return o32 ? launch<D, false, true>(prm, s) : launch<D, false, false>(prm, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, bool o32, hipStream_t s) {
  Params prm;
  prm.q = static_cast<const uint16_t *>(a.q);
  prm.k = static_cast<const uint16_t *>(a.k);
  prm.v = static_cast<const uint16_t *>(a.v);
  prm.o = a.o;
  prm.lse = a.lse;
  prm.n = a.n;
  prm.n_qblocks = (a.n + kRows - 1) / kRows;
  prm.total = a.bh * prm.n_qblocks;
  prm.c = a.scale * kLog2e;
  if (a.d == 128) return launch_d<128>(prm, a.causal, o32, s);
  return launch_d<64>(prm, a.causal, o32, s);
}

}  // namespace fa2
