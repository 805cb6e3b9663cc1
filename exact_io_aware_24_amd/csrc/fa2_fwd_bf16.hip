// Exact attention forward, bf16 inputs, bf16 MFMA on gfx950 (CDNA4).
//
// What is computed (per batch*head, per query block of 128 rows):
//   for each K/V tile of BC keys (the inner loop of FlashAttention-2's order:
//   query blocks outside, K/V blocks inside -- itimpress.au page
//   "FlashAttention scaling, multi-GPU training and weight quantisation",
//   section 1):
//     S  = K_tile . Q_block^T            bf16 MFMA, fp32 accumulate
//     mt = rowmax(S) * c                  c = scale * log2(e)   (base-2 units)
//     if mt > m + 8 for any row of the wave:   (lazy rescale, see below)
//         a = 2^(m - max(m, mt)); m = max(m, mt); l *= a; O~ *= a
//     P~ = 2^(S*c - m)                    fp32, hardware exp2
//     l  = l + rowsum(P~)
//     O~ = O~ + P~ . V_tile               P~ rounded to bf16, MFMA, fp32 acc
//   and after the last tile O = O~ / l, lse = (m + log2 l) * ln 2.
// The running (m, l, O~) update is the two-block online-softmax merge of the
// shakilmahmud.com page "Large language models part 06: FlashAttention --
// GPU SRAM, tiling, online softmax", section 2, with O~ kept unnormalised so
// that the single division by l happens once at the end (FlashAttention-2's
// reduction of non-matmul work, the same itimpress.au section).  One
// workgroup per (batch*head, query block) spreads one head over many compute
// units (improvement 2 of the "FlashAttention-2 (BN)" wiki article).
//
// Lazy rescale: the merge is exact for ANY common reference value m, not only
// the true running maximum, as long as the same m is used for l and O~.  The
// reference is therefore raised only when a tile's maximum exceeds it by more
// than 8 (a factor 256), which keeps every P~ <= 2^8 (no overflow, the same
// relative bf16 precision) and skips the O~ rescale on most tiles.
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
//    phase of a 128-bit LDS access touches 32 distinct banks.  Swizzles use
//    only lane bits that leave compile-time parts of the address additive,
//    so almost every LDS access is a per-lane base plus an immediate.
//  * Global loads are raw buffer loads with the per-head extent as the
//    buffer size: rows past the end of the sequence read as zero in hardware,
//    with no branches.  The next tile is fetched into registers while the
//    current one is consumed; LDS is double-buffered, one barrier per tile.
//  * Causal: tiles past a wave's last query are skipped by that wave (it only
//    helps to stage them); the mask is applied only in the tiles that cross
//    the diagonal or the ragged end of the sequence, which run in a separate
//    loop after the unmasked ones.  Query blocks are issued longest first.
//  * Workgroup ids are remapped so that the blocks of one head run on the
//    same XCD (hardware deals workgroups round-robin over the 8 XCDs), which
//    keeps that head's K/V in one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kRows = kBf16RowsPerBlock;  // 128 query rows per workgroup
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;
constexpr float kRescaleThreshold = 8.0f;  // base-2 units: P~ <= 256
// Buffer descriptor word 3: 32-bit data format, raw (untyped) addressing.
constexpr int kBufWord3 = 0x00020000;

struct Params {
  const uint16_t *q, *k, *v;
  void *o;
  float *lse;
  int n;          // sequence length
  int n_qblocks;  // ceil(n / 128)
  int total;      // bh * n_qblocks (grid size)
  float c;        // scale * log2(e)
};

template <int D>
struct Cfg {
  static constexpr int BC = (D == 128) ? 64 : 128;  // keys per tile
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int NKT = BC / 32;               // 32-key sub-tiles
  static constexpr int NDT = D / 16;                // 16-dim MFMA k-steps
  static constexpr int NCT = D / 32;                // 32-wide O^T row tiles
  static constexpr int KLOADS = BC * KCH / kThreads;
  static constexpr int VCOLS = D / 4;               // 4-column V groups
  static constexpr int TILE = BC * D;               // elements per K or V tile
  static constexpr int TILE_BYTES = TILE * 2;       // 16 KB either way
  static_assert(KLOADS * kThreads == BC * KCH, "K tile split");
  static_assert((BC / 8) * VCOLS == kThreads, "V tile split");
  static_assert(kThreads / KCH * D * 2 == 4096, "K load stride");
};

// Row permutation inside each 16-row group: swap bits 2 and 3.
__device__ __forceinline__ int perm16(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Swizzle of V^T rows (columns of V): 16-byte chunk j of row c is stored at
// chunk j ^ vsw(c).  It uses bits 0-4 of c only, so rows 32 apart share it.
__device__ __forceinline__ int vsw(int c) { return (c & 7) ^ ((c >> 3) & 3); }

// (x of lanes 0-31, x of lanes 32-63) as seen from every lane.
__device__ __forceinline__ void halves(float x, float &lo, float &hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

template <typename T>
__device__ __forceinline__ T lds_load(const char *base, int byte_off) {
  return *reinterpret_cast<const T *>(base + byte_off);
}
template <typename T>
__device__ __forceinline__ void lds_store(char *base, int byte_off, T v) {
  *reinterpret_cast<T *>(base + byte_off) = v;
}

// Everything one wave needs while it walks the K/V tiles.
template <int D>
struct WaveState {
  bf16x8 qreg[Cfg<D>::NDT];
  f32x16 oacc[Cfg<D>::NCT];
  float m_run;  // reference max (base-2 scaled units)
  float l_run;  // this half-wave's share of the running sum
};

// Per-thread byte offsets that stay fixed for the whole kernel.
template <int D>
struct Offsets {
  int k_rd[4];  // K operand reads, 16-dim steps 0..3 (steps 4..7 at +128 B)
  int v_rd[4];  // V^T operand reads, (sub-tile parity, 16-key half) 0..3
  int k_wr;     // K staging write (loads it = 0..3 at +4096 B each)
  int v_wr[4];  // V^T staging writes, columns 4*vcc + e
  int k_ld;     // K buffer-load offset within a tile
  int v_ld;     // V buffer-load offset within a tile (rows r at +r*D*2)
};

template <int D>
__device__ __forceinline__ void gload(const __amdgpu_buffer_rsrc_t &rk,
                                      const __amdgpu_buffer_rsrc_t &rv,
                                      const Offsets<D> &off, int tile_byte,
                                      u32x4 (&kpre)[Cfg<D>::KLOADS],
                                      u32x2 (&vpre)[8]) {
#pragma unroll
  for (int it = 0; it < Cfg<D>::KLOADS; ++it)
    kpre[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off.k_ld,
                                                     tile_byte + it * 4096, 0);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    vpre[r] = __builtin_amdgcn_raw_buffer_load_b64(rv, off.v_ld + r * D * 2,
                                                   tile_byte, 0);
}

template <int D, int BUF>
__device__ __forceinline__ void swrite(char *smem, const Offsets<D> &off,
                                       const u32x4 (&kpre)[Cfg<D>::KLOADS],
                                       const u32x2 (&vpre)[8]) {
  using C = Cfg<D>;
  char *kb = smem + BUF * C::TILE_BYTES;
  char *vb = smem + (2 + BUF) * C::TILE_BYTES;
#pragma unroll
  for (int it = 0; it < C::KLOADS; ++it) lds_store(kb, off.k_wr + it * 4096, kpre[it]);
  // 8 keys x 4 columns -> 4 columns x 8 keys (bf16 transpose in registers)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u32x4 outv;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const uint32_t a = (e < 2) ? vpre[2 * pr].x : vpre[2 * pr].y;
      const uint32_t b = (e < 2) ? vpre[2 * pr + 1].x : vpre[2 * pr + 1].y;
      outv[pr] = (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                         : __builtin_amdgcn_perm(b, a, 0x05040100u);
    }
    lds_store(vb, off.v_wr[e], outv);
  }
}

// One K/V tile for one wave.  MASKED tiles apply the causal / sequence-end
// mask; unmasked tiles need no compare at all.
template <int D, bool CAUSAL, bool MASKED, int BUF>
__device__ __forceinline__ void tile(const char *smem, const Offsets<D> &off,
                                     WaveState<D> &st, float c, int j0, int N,
                                     int qi, int hh) {
  using C = Cfg<D>;
  const char *kb = smem + BUF * C::TILE_BYTES;
  const char *vb = smem + (2 + BUF) * C::TILE_BYTES;

  // -- S^T = K Q^T ---------------------------------------------------------
  f32x16 s[C::NKT];
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
    // operands in groups of four: 16 registers in flight, not 32
#pragma unroll
    for (int g = 0; g < C::NDT; g += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = lds_load<bf16x8>(kb, off.k_rd[i] + (g >> 2) * 128 + kt * 32 * D * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], st.qreg[g + i],
                                                        s[kt], 0, 0, 0);
    }
  }

  // -- mask: register r of sub-tile kt holds key j0 + 32kt + 16(r/8) + 8hh + r%8
  if (MASKED) {
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kt + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
      }
  }

  // -- online softmax --------------------------------------------------------
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  float mlo, mhi;
  halves(mx, mlo, mhi);
  mx = fmaxf(mlo, mhi);
  const float m_tile = (MASKED && mx == -INFINITY) ? -INFINITY : mx * c;
  if (__builtin_amdgcn_ballot_w64(m_tile > st.m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(st.m_run, m_tile);
    const float alpha =
        (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[ct][r] *= alpha;
  }
  const float mu = (MASKED && st.m_run == -INFINITY) ? 0.f : st.m_run;

  bf16x8 pb[C::NKT][2];
  float rs = 0.f;
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sv = s[kt][8 * u + e];
        float x = fast_exp2(__builtin_fmaf(sv, c, -mu));
        if (MASKED) x = (sv == -INFINITY) ? 0.f : x;
        rs += x;
        pb[kt][u][e] = static_cast<__bf16>(x);
      }
  st.l_run += rs;

  // -- O^T += V^T P^T ----------------------------------------------------------
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 a[C::NCT];
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
        a[ct] = lds_load<bf16x8>(vb, off.v_rd[(kt & 1) * 2 + u] + (kt >> 1) * 128 +
                                         ct * 32 * C::BC * 2);
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
        st.oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ct], pb[kt][u],
                                                              st.oacc[ct], 0, 0, 0);
    }
}

template <int D, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[4 * C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int lr = lane & 31;  // query column of this lane in S^T / O^T
  const int hh = lane >> 5;  // half-wave

  // ---- workgroup -> (head, query block) ----------------------------------
  const int w = blockIdx.x;
  const int per_xcd = p.total >> 3;
  int logical = w;
  if (w < (per_xcd << 3)) logical = (w & 7) * per_xcd + (w >> 3);
  const int bh = logical / p.n_qblocks;
  const int qbl = logical - bh * p.n_qblocks;
  const int qb = CAUSAL ? (p.n_qblocks - 1 - qbl) : qbl;

  const int N = p.n;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int head_bytes = N * D * 2;  // < 2^32 - 2^17 (host-validated)
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.q + head), 0, head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.k + head), 0, head_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(p.v + head), 0, head_bytes, kBufWord3);

  const int q0 = qb * kRows;      // first query of the block
  const int qw = q0 + wv * 32;    // first query of this wave
  const int qi = qw + lr;         // this lane's query

  // ---- fixed offsets -------------------------------------------------------
  Offsets<D> off;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    off.k_rd[i] = (perm16(lr) * D + (((2 * i + hh) ^ (lr & 7)) * 8)) * 2;
    const int chunk = 2 * i + hh;  // (sub-tile parity, half) -> 16-B chunk
    off.v_rd[i] = (lr * C::BC + ((chunk ^ vsw(lr)) * 8)) * 2;
  }
  {
    const int row = tid / C::KCH, ch = tid % C::KCH;
    off.k_wr = (row * D + ((ch ^ (perm16(row) & 7)) * 8)) * 2;
    off.k_ld = (row * D + ch * 8) * 2;
    const int vcc = tid % C::VCOLS, vjg = tid / C::VCOLS;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = vcc * 4 + e;
      off.v_wr[e] = (col * C::BC + ((vjg ^ vsw(col)) * 8)) * 2;
    }
    off.v_ld = ((vjg * 8) * D + vcc * 4) * 2;
  }

  // ---- Q into registers (B operand of S^T = K Q^T) -------------------------
  WaveState<D> st;
  float c = p.c;
  uint32_t qflip = 0;
  if (c < 0.f) {  // exact: negate q (bf16 sign bit) and use -c
    c = -c;
    qflip = 0x80008000u;
  }
  const int q_ld = (qi * D + 8 * hh) * 2;
#pragma unroll
  for (int t = 0; t < C::NDT; ++t) {
    u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, q_ld + 32 * t, 0, 0);
    x ^= qflip;
    st.qreg[t] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[ct][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  // ---- tile schedule -------------------------------------------------------
  // Tiles [0, n_full) need no mask for any row of the block; the rest (the
  // diagonal band when causal, the ragged end of the sequence) are masked.
  const int kend = CAUSAL ? min(N, q0 + kRows) : N;
  const int ntiles = (kend + C::BC - 1) / C::BC;
  int n_full = CAUSAL ? (q0 + 1) / C::BC : N / C::BC;
  if (n_full > ntiles) n_full = ntiles;
  if (n_full * C::BC > N) n_full = N / C::BC;

  u32x4 kpre[C::KLOADS];
  u32x2 vpre[8];
  gload<D>(rk, rv, off, 0, kpre, vpre);
  swrite<D, 0>(smem, off, kpre, vpre);
  __syncthreads();

  auto step = [&](auto buf_tag, auto masked_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int j0 = t * C::BC;
    const bool more = t + 1 < ntiles;
    if (more) gload<D>(rk, rv, off, (j0 + C::BC) * D * 2, kpre, vpre);
    if (!MASKED || !CAUSAL || j0 <= qw + 31)
      tile<D, CAUSAL, MASKED, BUF>(smem, off, st, c, j0, N, qi, hh);
    if (more) swrite<D, 1 - BUF>(smem, off, kpre, vpre);
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  int t = 0;
  for (; t + 2 <= n_full; t += 2) {
    step(B0{}, Unmasked{}, t);
    step(B1{}, Unmasked{}, t + 1);
  }
  if (t < n_full) {
    step(B0{}, Unmasked{}, t);
    ++t;
  }
  for (; t < ntiles; ++t) {
    if (t & 1)
      step(B1{}, Masked{}, t);
    else
      step(B0{}, Masked{}, t);
  }

  // ---- epilogue: O = O~ / l, lse ---------------------------------------------
  float llo, lhi;
  halves(st.l_run, llo, lhi);
  const float l_tot = llo + lhi;
  const float inv = 1.0f / l_tot;
  if (qi < N) {
    // O^T register r of row tile ct holds column 32ct + 8(r/4) + 4hh + r%4
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = 32 * ct + 8 * a + 4 * hh;
        const size_t o_off = head + static_cast<size_t>(qi) * D + col;
        if (O32) {
          f32x4 ov;
#pragma unroll
          for (int b = 0; b < 4; ++b) ov[b] = st.oacc[ct][4 * a + b] * inv;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + o_off) = ov;
        } else {
          __bf16 ob[4];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            ob[b] = static_cast<__bf16>(st.oacc[ct][4 * a + b] * inv);
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.o) + o_off) =
              __builtin_bit_cast(u32x2, ob);
        }
      }
    if (p.lse && hh == 0)
      p.lse[static_cast<size_t>(bh) * N + qi] = (st.m_run + log2f(l_tot)) * kLn2;
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
