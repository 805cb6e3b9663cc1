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
//     l  = l + rowsum(P~)                 (for the lse)
//     lb = lb + rowsum(bf16(P~))          (the normaliser of O~)
//     O~ = O~ + bf16(P~) . V_tile         MFMA, fp32 acc
//   and after the last tile O = O~ / lb, lse = (m + log2 l) * ln 2.
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
// Normaliser: O~ is divided by the sum of the bf16-rounded P~ that multiplied
// V (v_dot2 of each rounded pair against (1, 1)), so the weights applied to
// V sum to one exactly.  Dividing by the sum of the unrounded values instead
// leaves the rounding of a dominant P~ -- anywhere in (1, 2^8] under the lazy
// rescale, not exactly 1 -- in O undiluted, up to 2^-8 of |V|, which exceeds
// the stated tolerance on sharp softmaxes (the x20 outlier rows).  The lse
// keeps the fp32 sum of the unrounded values.  The rounded normaliser does
// not cover every input: when two keys of similar weight dominate a row and
// the later one exceeds the reference by less than 8, both of their P~ are
// rounded, and at very sharp softmaxes (scales of about seven times
// 1/sqrt(d)) the output can pass the element-wise tolerance by up to about
// a fifth.  A reference kept at the exact running maximum (rescaling on every
// increase) avoids that at about 6 % of the throughput.
//
// gfx950 mapping (this library's design, not the pages'), fwd_bf16_kernel
// (d = 128; d = 64 runs fwd_small_kernel, further down):
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
//  * K and V go from HBM straight into LDS (buffer_load ... lds: no register
//    staging), issued one tile ahead and double-buffered, one barrier per
//    tile.  Each tile's loads go through a raw buffer descriptor that starts
//    at the tile and ends at the end of the head, so rows past the end of
//    the sequence read as zero in hardware, with no branches.
//  * K is stored row-major with its 16-byte granules XOR-swizzled by the row,
//    so the 16 lanes of each phase of a 128-bit read hit 16 distinct bank
//    groups.  V is stored in blocks of 32 columns (each key's 64 bytes
//    contiguous inside a block) and read with ds_read_b64_tr_b16, which
//    transposes 16-lane groups in flight: each lane receives one column of
//    four consecutive keys, exactly the A operand of O^T += V^T P^T, whose B
//    operand is the S^T result converted in place to bf16.  All V reads are
//    one per-lane base plus immediates, and conflict-free.
//  * Causal: tiles past a wave's last query are skipped by that wave (it only
//    helps to stage them); the mask is applied only in the tiles that cross
//    the diagonal or the ragged end of the sequence, which run in a separate
//    loop after the unmasked ones.  Query blocks are issued longest first.
//  * Workgroup ids are remapped so that the blocks of one head run on the
//    same XCD (hardware deals workgroups round-robin over the 8 XCDs), which
//    keeps that head's K/V in one L2.
//
// The same kernel serves the general forward (fa2_fwd_splitkv): Nq queries
// against Nk keys (causal: query i sits at key position i + Nk - Nq), K/V
// heads shared by groups of query heads, and the key tiles of a query block
// split into ranges handled by separate workgroups, each writing fp32
// partial (O, lse) that merge_splits_kernel combines with the online-softmax
// merge of the shakilmahmud.com page's section 2.  Tile indices stay global
// (masks and loads are unchanged); waves whose rows all lie past Nq only
// help with the loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kRows = kBf16RowsPerBlock;  // 128 query rows per workgroup
constexpr float kRescaleThreshold = 8.0f;  // base-2 units: P~ <= 256

struct Params {
  const uint16_t *q, *k, *v;
  void *o;               // final output, or fp32 partial outputs per split
  float *lse;            // final lse, or partial lse per split (may be null)
  int nq;                // query rows per head
  int nk;                // key rows per head
  int h;                 // query heads per batch index
  int group;             // query heads per K/V head
  int n_qblocks;         // ceil(nq / 128)
  int n_splits;          // key ranges per query block (1: no split)
  int tiles_per_split;   // key tiles per range
  int total;             // bh * n_qblocks * n_splits (work items)
  int persist;           // 1: the grid walks the items (see the kernel)
  int no_skip;           // 1: causal blocks also run the key tiles past
                         // their diagonal, every score masked (test switch)
  size_t o_split_stride;    // elements between the partial outputs of splits
  size_t lse_split_stride;  // same for lse
  float c;               // scale * log2(e)
};

// Tile configuration of fwd_bf16_kernel, which runs d = 128 only (d = 64
// runs fwd_small_kernel with its own SmallCfg).
template <int D>
struct Cfg {
  static_assert(D == 128, "fwd_bf16_kernel is the d = 128 kernel");
  static constexpr int BC = 64;                     // keys per tile
  static constexpr int KCH = D / 8;                 // 16-byte granules per K row
  static constexpr int NKT = BC / 32;               // 32-key sub-tiles
  static constexpr int NDT = D / 16;                // 16-dim MFMA k-steps
  static constexpr int NCT = D / 32;                // 32-wide O^T row tiles
  static constexpr int TILE_BYTES = BC * D * 2;     // 16 KB for K or V
  static constexpr int K_ROWS_PER_LOAD = 64 / KCH;  // rows per 1 KB wave load
  static_assert(TILE_BYTES == 16 * 1024, "one tile = 16 wave loads of 1 KB");
};

// K granule swizzle: granule j of row r is stored at position j ^ kswz(r).
// With 16 granules per row (d = 128) one row fills the 64 banks; with 8
// (d = 64) two rows share them, so the row pair index is used.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Everything one wave needs while it walks the K/V tiles.
template <int D>
struct WaveState {
  bf16x8 qreg[Cfg<D>::NDT];
  f32x16 oacc[Cfg<D>::NCT];
  float m_run;  // reference max (base-2 scaled units)
  float l_run;  // this half-wave's share of the running sum
  float lr_run; // the same for the bf16-rounded P~ (the normaliser of O~)
};

// Per-thread byte offsets fixed for the whole kernel.
template <int D>
struct Offsets {
  int k_rd[Cfg<D>::NDT];  // K operand reads per 16-dim step
  int v_rd;               // V transposed reads (all others are immediates)
  int k_ld[4];            // K loads within a tile, one per wave load
  int v_ld[4];            // V loads within a tile, one per wave load
};

// The four 1 KB loads of K, and of V, that this wave issues for one tile
// (bytes [tile_byte, ...) of the head; rows past its end load as zeros).
// LDS destinations are wave-uniform (they go to M0).
template <int D>
__device__ __forceinline__ void issue_k(const uint16_t *k, int head_bytes,
                                        const Offsets<D> &off, char *kbuf,
                                        int wv, int tile_byte) {
  const u32x4 rk = tile_desc(k, head_bytes, tile_byte);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int inst = 4 * wv + it;
    const int vo = off.k_ld[it];
    dma16(rk, vo, 0, lds_addr(kbuf + inst * 1024));
  }
}

template <int D>
__device__ __forceinline__ void issue_v(const uint16_t *v, int head_bytes,
                                        const Offsets<D> &off, char *vbuf,
                                        int wv, int tile_byte) {
  using C = Cfg<D>;
  const u32x4 rv = tile_desc(v, head_bytes, tile_byte);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    // block of 32 columns = wave, 16-key group = it
    const int vo = off.v_ld[it];
    dma16(rv, vo, 0, lds_addr(vbuf + wv * C::BC * 64 + it * 1024));
  }
}

// S^T = K Q^T for one tile: MFMA row m of sub-tile kt is key j0 + 32kt + m.
// The K operands are read from LDS one group of four ahead of the MFMAs
// that consume them, so the LDS latency hides under the previous group.
template <int D>
__device__ __forceinline__ void scores(const char *kb, const Offsets<D> &off,
                                       const bf16x8 (&qreg)[Cfg<D>::NDT],
                                       f32x16 (&s)[Cfg<D>::NKT]) {
  using C = Cfg<D>;
  constexpr int G = C::NDT / 4;   // groups of four k-steps per sub-tile
  constexpr int NG = C::NKT * G;  // groups per tile
  bf16x8 a[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[0][i] = lds_load<bf16x8>(kb, off.k_rd[i]);
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    if (grp + 1 < NG) {
      const int kt1 = (grp + 1) / G, g1 = ((grp + 1) % G) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[(grp + 1) & 1][i] =
            lds_load<bf16x8>(kb, off.k_rd[g1 + i] + kt1 * 32 * D * 2);
    }
    pin_lds_mfma();
    const int kt = grp / G, g = (grp % G) * 4;
    if (g == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[grp & 1][i], qreg[g + i],
                                                      s[kt], 0, 0, 0);
  }
}

// Mask (MASKED tiles only), row max, and the lazy update of the reference
// max for one tile of scores.  When a row's tile max exceeds the reference
// by more than the threshold the whole wave raises it, rescales l and O~ by
// the same factor (the merge is exact for any common reference) and goes
// on; otherwise nothing changes and the exponentials of this tile are taken
// against the old reference (they stay <= 2^8).  Called as soon as a tile's
// scores exist, one iteration before their exponentials, so that the
// iteration body that follows has no branch between its MFMAs and its
// exponentials.
template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void softmax_max(f32x16 (&s)[Cfg<D>::NKT],
                                            WaveState<D> &st, float c, int j0,
                                            int N, int qi, int hh) {
  using C = Cfg<D>;
  // register r of sub-tile kt holds key j0 + 32kt + 8(r/4) + 4hh + r%4
  if (MASKED) {
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
      }
  }
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
    st.lr_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[ct][r] *= alpha;
  }
}

// P~ = 2^(S c - mu), summed in fp32 into l (the log-sum-exp needs the
// unrounded values) and rounded to bf16 for the P.V product.  16-key step u
// of sub-tile kt takes registers 8u..8u+7: keys 32kt + 16u + 8a + 4hh + b for
// element 4a + b, which is the B operand of the P.V MFMA (k index
// 8hh + 4a + b) as it is.
template <int D, bool MASKED>
__device__ __forceinline__ void softmax_exp(const f32x16 (&s)[Cfg<D>::NKT],
                                            float mu, float c,
                                            bf16x8 (&pb)[Cfg<D>::NKT][2],
                                            float &l_run, float &lr_run) {
  using C = Cfg<D>;
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
  l_run += rs;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float rr = lr_run;
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pb[kt][u][e], pb[kt][u][e + 1]};
        rr = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rr, false);
      }
  lr_run = rr;
}

// O^T += V^T P^T: A operand = columns 32ct + lane%32 of the keys above,
// read transposed from LDS one 16-key step ahead of the MFMAs that use it.
template <int D>
__device__ __forceinline__ void pv(const char *vb, const Offsets<D> &off,
                                   const bf16x8 (&pb)[Cfg<D>::NKT][2],
                                   f32x16 (&oacc)[Cfg<D>::NCT]) {
  using C = Cfg<D>;
  constexpr int NS = 2 * C::NKT;  // 16-key steps per tile
  bf16x8 a[2][C::NCT];
  auto read = [&](int step, bf16x8 (&dst)[C::NCT]) {
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      const int imm = ct * C::BC * 64 + 16 * step * 64;
      const s16x4 lo = lds_read_tr(vb, off.v_rd + imm);
      const s16x4 hi = lds_read_tr(vb, off.v_rd + imm + 8 * 64);
      dst[ct] = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  read(0, a[0]);
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    if (st + 1 < NS) read(st + 1, a[(st + 1) & 1]);
    pin_lds_mfma();
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
      oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a[st & 1][ct], pb[st >> 1][st & 1], oacc[ct], 0, 0, 0);
  }
}

template <int D, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  // [K buffer 0][K buffer 1][V buffer 0][V buffer 1], 16 KB each
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;  // query column of this lane in S^T / O^T
  const int hh = lane >> 5;  // half-wave

  const int Nq = p.nq, Nk = p.nk;
  // causal: query i sits at key position i + Nk - Nq (the last query sees
  // every key; with Nq == Nk, query i sees keys 0..i)
  const int qoff = Nk - Nq;
  const int head_bytes = Nk * D * 2;  // < 2^31 (host-validated)

  // ---- fixed offsets -------------------------------------------------------
  Offsets<D> off;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
    off.k_rd[dt] = (lr * D + (((2 * dt + hh) ^ kswz<D>(lr)) * 8)) * 2;
  {
    // transposed V reads: lane s of a 16-lane group g supplies key 4hh + s/4
    // (plus the step's base key) and columns 16(g&1) + 4(s%4) .. +3
    const int g = lane >> 4, sl = lane & 15;
    off.v_rd = (4 * hh + (sl >> 2)) * 64 + (g & 1) * 32 + (sl & 3) * 8;
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (4 * wv + it) * C::K_ROWS_PER_LOAD + lane / C::KCH;
    const int pos = lane % C::KCH;
    off.k_ld[it] = row * D * 2 + ((pos ^ kswz<D>(row)) * 16);
  }
  {
#pragma unroll
    for (int it = 0; it < 4; ++it)
      off.v_ld[it] = (16 * it + lane / 4) * D * 2 + (4 * wv + (lane & 3)) * 16;
  }

  float c = p.c;
  uint32_t qflip = 0;
  if (c < 0.f) {  // exact: negate q (bf16 sign bit) and use -c
    c = -c;
    qflip = 0x80008000u;
  }

  auto kbuf = [&](int i) { return smem + i * C::TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * C::TILE_BYTES; };

  // ---- work items ----------------------------------------------------------
  // An item is (batch*head, query block, key range).  Without p.persist each
  // workgroup takes one item, ids remapped so that each XCD runs a
  // contiguous range of them.  With it, a grid of two workgroups per compute
  // unit walks the items: the workgroups of XCD x (hardware deals workgroup
  // w to XCD w % 8) take the contiguous items [x*total/8, (x+1)*total/8),
  // workgroup j of the XCD item r*per + j in round r, the order reversed on
  // odd rounds so that a long causal block is paired with a short one.  The
  // loads of an item's first tiles and of its Q rows are then issued during
  // the last tile of the item before (see the general loop).
  const int per = static_cast<int>(gridDim.x >> 3);
  const int xj = static_cast<int>(blockIdx.x >> 3);
  const int xcd = static_cast<int>(blockIdx.x & 7);
  const int ilo = static_cast<int>(static_cast<int64_t>(xcd) * p.total / 8);
  const int ilen = static_cast<int>(static_cast<int64_t>(xcd + 1) * p.total / 8) - ilo;
  auto item_at = [&](int r) -> int {
    if (!p.persist) return r == 0 ? xcd_remap(blockIdx.x, p.total) : -1;
    const int local = r * per + ((r & 1) ? per - 1 - xj : xj);
    return local < ilen ? ilo + local : -1;
  };
  // item -> key range, batch*head, first query row
  auto decode = [&](int logical, int &split, int &bh, int &q0) {
    split = 0;
    if (p.n_splits > 1) {
      split = logical % p.n_splits;
      logical /= p.n_splits;
    }
    bh = logical / p.n_qblocks;
    const int qbl = logical - bh * p.n_qblocks;
    q0 = (CAUSAL ? (p.n_qblocks - 1 - qbl) : qbl) * kRows;
  };
  // K/V head shared by `group` consecutive query heads (grouped-query
  // attention; 1 = one K/V head per query head)
  auto kv_head = [&](int bh) -> size_t {
    const int kvbh = p.group == 1 ? bh : (bh / p.h) * (p.h / p.group) + (bh % p.h) / p.group;
    return static_cast<size_t>(kvbh) * Nk * D;
  };
  // key tiles the query block starting at q0 needs (causal: up to its last query)
  auto block_tiles = [&](int q0) -> int {
    const int kend = CAUSAL && !p.no_skip ? max(0, min(Nk, q0 + kRows + qoff)) : Nk;
    return (kend + C::BC - 1) / C::BC;
  };

  // Q into registers (B operand of S^T = K Q^T); the sign flip of a negative
  // scale is applied at the start of the item, once the rows have arrived
  WaveState<D> st;
  auto load_q = [&](int bh, int q0) {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.q + static_cast<size_t>(bh) * Nq * D), 0, Nq * D * 2,
        kBufWord3);
    const int q_ld = ((q0 + wv * 32 + lr) * D + 8 * hh) * 2;
#pragma unroll
    for (int t = 0; t < C::NDT; ++t)
      st.qreg[t] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, q_ld + 32 * t, 0, 0));
  };

  bool pre = false;  // this item's Q, K/V(0) and K(1) were issued already
  bool handed = false;
  int logical = item_at(0);
  for (int r = 0; logical >= 0; ++r) {
    const int nxt = item_at(r + 1);
    int split, bh, q0;
    decode(logical, split, bh, q0);
    const size_t qhead = static_cast<size_t>(bh) * Nq * D;
    const size_t kvhead = kv_head(bh);
    const uint16_t *kh = p.k + kvhead;
    const uint16_t *vh = p.v + kvhead;
    const int qw = q0 + wv * 32;    // first query of this wave
    const int qi = qw + lr;         // this lane's query
    const int qpos = qi + qoff;     // its position among the keys

    if (!pre) load_q(bh, q0);
#pragma unroll
    for (int t = 0; t < C::NDT; ++t)
      st.qreg[t] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, st.qreg[t]) ^ qflip);
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) st.oacc[ct][r2] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    st.lr_run = 0.f;

    // ---- tile schedule -----------------------------------------------------
    // Software pipeline: iteration t computes the scores of tile t+1 (K one
    // tile ahead in LDS) while it runs the softmax of tile t and the P.V
    // product with V(t); the loads of K(t+2) and V(t+1) are in flight
    // meanwhile.  Tiles are numbered over the whole key range; this item
    // takes tiles [tb, ntiles) of it (all of them unless the keys are split).
    // Tiles below n_full need no mask for any row of the block; the rest (the
    // diagonal band when causal, the ragged end of the keys) are masked.
    const int tb = split * p.tiles_per_split;
    const int ntiles = min(block_tiles(q0), tb + p.tiles_per_split);
    const int n_full = CAUSAL ? max(0, (q0 + qoff + 1) / C::BC) : Nk / C::BC;
    // waves with no query rows (short query blocks) only help with the loads
    const bool live = qw < Nq;
    // tiles this wave needs (causal: keys up to its last query)
    const int w_tiles = !live ? tb
                        : CAUSAL && !p.no_skip ? min(ntiles, (qw + 31 + qoff) / C::BC + 1)
                                               : ntiles;
    // branch-free main loop: tiles t and t+1 unmasked
    const int n_main = live ? min(n_full, ntiles) - 1 : tb;
    f32x16 sa[C::NKT], sb[C::NKT];

    if (tb < ntiles) {  // (an empty key range leaves l = 0: O = 0, lse = -inf)
    // Rows past the end of the sequence load as zeros; clear LDS first so
    // that no tile can ever expose uninitialised bits, whatever the hardware
    // does with out-of-range lanes.  (Never with p.persist.)
    if (Nk % C::BC != 0) {
      for (int i = tid; i < 4 * C::TILE_BYTES / 16; i += kThreads)
        reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    // prologue: K(tb), V(tb) -> buffers 0; then K(tb+1) in flight while S(tb)
    // is computed.  Buffer parity is (t - tb) & 1.
    if (!pre) {
      issue_k<D>(kh, head_bytes, off, kbuf(0), wv, tb * C::BC * D * 2);
      issue_v<D>(vh, head_bytes, off, vbuf(0), wv, tb * C::BC * D * 2);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!pre && tb + 1 < ntiles)
      issue_k<D>(kh, head_bytes, off, kbuf(1), wv, (tb + 1) * C::BC * D * 2);
    if (tb < w_tiles) {
      scores<D>(kbuf(0), off, st.qreg, sa);
      if (tb < n_full)
        softmax_max<D, CAUSAL, false>(sa, st, c, tb * C::BC, Nk, qpos, hh);
      else
        softmax_max<D, CAUSAL, true>(sa, st, c, tb * C::BC, Nk, qpos, hh);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // one pipelined iteration; CUR holds S(t), NXT receives S(t+1)
    auto step = [&](auto par_tag, int t, f32x16(&cur)[C::NKT],
                    f32x16(&nxt)[C::NKT]) {
      constexpr int P = decltype(par_tag)::value;  // (t - tb) & 1
      const int j0 = t * C::BC;
      if (t + 2 < ntiles) issue_k<D>(kh, head_bytes, off, kbuf(P), wv, (j0 + 2 * C::BC) * D * 2);
      issue_v<D>(vh, head_bytes, off, vbuf(1 - P), wv, (j0 + C::BC) * D * 2);
      scores<D>(kbuf(1 - P), off, st.qreg, nxt);
      bf16x8 pb[C::NKT][2];
      softmax_exp<D, false>(cur, st.m_run, c, pb, st.l_run, st.lr_run);
      pv<D>(vbuf(P), off, pb, st.oacc);
      softmax_max<D, CAUSAL, false>(nxt, st, c, j0 + C::BC, Nk, qpos, hh);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    int t = tb;
    for (; t + 2 <= n_main; t += 2) {
      step(P0{}, t, sa, sb);
      step(P1{}, t + 1, sb, sa);
    }
    if (t < n_main) {
      step(P0{}, t, sa, sb);
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) sa[kt] = sb[kt];
      ++t;
    }
    // general loop: masked tiles, waves that stop early, the last tile.  In
    // the last tile no K buffer is read and only V buffer p is, so the next
    // item's Q rows, K(0), K(1) and (when p == 1) V(0) are issued there;
    // that iteration then skips its wait for loads, which the next item's
    // prologue waits for.  (Items start at tile 0 when p.persist is set.)
    bool v_next = false;  // V(0) of the next item issued
    for (; t < ntiles; ++t) {
      const int j0 = t * C::BC;
      const int pr = (t - tb) & 1;
      const bool hand_over = nxt >= 0 && t + 1 == ntiles;
      if (t + 2 < ntiles) issue_k<D>(kh, head_bytes, off, kbuf(pr), wv, (j0 + 2 * C::BC) * D * 2);
      if (t + 1 < ntiles) issue_v<D>(vh, head_bytes, off, vbuf(1 - pr), wv, (j0 + C::BC) * D * 2);
      if (t + 1 < w_tiles) scores<D>(kbuf(1 - pr), off, st.qreg, sb);
      if (hand_over) {
        int split2, bh2, q02;
        decode(nxt, split2, bh2, q02);
        load_q(bh2, q02);
        const size_t kv2 = kv_head(bh2);
        issue_k<D>(p.k + kv2, head_bytes, off, kbuf(0), wv, 0);
        if (block_tiles(q02) > 1)
          issue_k<D>(p.k + kv2, head_bytes, off, kbuf(1), wv, C::BC * D * 2);
        if (pr == 1) {
          issue_v<D>(p.v + kv2, head_bytes, off, vbuf(0), wv, 0);
          v_next = true;
        }
        handed = true;
      }
      if (t < w_tiles) {
        const float mu = (st.m_run == -INFINITY) ? 0.f : st.m_run;
        bf16x8 pb[C::NKT][2];
        softmax_exp<D, true>(sa, mu, c, pb, st.l_run, st.lr_run);
        pv<D>(vbuf(pr), off, pb, st.oacc);
      }
      if (t + 1 < w_tiles)
        softmax_max<D, CAUSAL, true>(sb, st, c, j0 + C::BC, Nk, qpos, hh);
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) sa[kt] = sb[kt];
      if (!hand_over) __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (nxt >= 0 && !v_next) {  // V buffer 0 was read by the last tile
      int split2, bh2, q02;
      decode(nxt, split2, bh2, q02);
      issue_v<D>(p.v + kv_head(bh2), head_bytes, off, vbuf(0), wv, 0);
    }
    }  // tb < ntiles

    // ---- epilogue: O = O~ / l, lse -------------------------------------------
    float llo, lhi, rlo, rhi;
    halves(st.l_run, llo, lhi);
    halves(st.lr_run, rlo, rhi);
    const float l_tot = llo + lhi;
    const float lr_tot = rlo + rhi;
    // a row that saw no key (only possible within one key range of a split,
    // or causal with more queries than keys): O = 0, lse = -inf
    const float inv = lr_tot > 0.f ? 1.0f / lr_tot : 0.f;
    if (qi < Nq) {
      const size_t head = qhead + split * p.o_split_stride;
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
        p.lse[split * p.lse_split_stride + static_cast<size_t>(bh) * Nq + qi] =
            l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
    logical = nxt;
    pre = handed;
    handed = false;
  }
}

// ---- d = 64: four waves per SIMD ---------------------------------------------------
//
// At d = 64 a score costs half the matrix work of d = 128 for the same
// softmax work, so the kernel is bound by its VALU issue: what pays is more
// waves to issue from and less VALU work per score.  fwd_small_kernel keeps
// the work items, the per-wave ownership of 32 query rows, the operand
// layouts and the normaliser of fwd_bf16_kernel, with
//  * 64-key tiles double-buffered in LDS (2 x 16 KB) and no score of the next
//    tile in flight: 120-128 VGPRs, four waves per SIMD;
//  * the checked softmax: a tile's exponentials are taken against the
//    current reference first, and only if some lane's sum of them exceeds
//    2^16 (or is not finite: the first tile, whose reference is still -inf)
//    does the wave find the tile's row maxima, raise the reference to them,
//    rescale l, the rounded sum and O~, and take the exponentials again.
//    Every P~ that reaches the sums is then <= 2^16; the row maximum (16
//    max3 per lane and tile, a cross-lane step, a ballot) leaves the common
//    path.  With O~ divided by the sum of the rounded P~, a single dominant
//    P~ away from 1 costs no accuracy; two near-tied dominant keys still
//    carry both roundings, as under the lazy rule of the d = 128 kernel.
constexpr int kSmallTile = 64;
constexpr float kCheckedSumLimit = 65536.0f;  // 2^16

template <int D, int BC_>
struct SmallCfg {
  static constexpr int BC = BC_;                      // keys per tile
  static constexpr int NKT = BC / 32;                 // 32-key sub-tiles
  static constexpr int KCH = D / 8;                   // 16-byte granules per K row
  static constexpr int NDT = D / 16;                  // 16-dim MFMA k-steps (S)
  static constexpr int NCT = D / 32;                  // 32-wide O^T row tiles
  static constexpr int TILE_BYTES = BC * D * 2;       // K or V tile
  static constexpr int NLOAD = TILE_BYTES / 1024 / 4; // 1 KB loads per wave per operand
  static constexpr int K_ROWS_PER_LOAD = 64 / KCH;    // K rows per 1 KB load
  static constexpr int VGROUPS = BC / 16;             // 16-key groups per V column block
  static constexpr int NSTAGE = 2;                   // double-buffered
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K then V
  static_assert(NLOAD >= 1 && NLOAD * 4 * 1024 == TILE_BYTES, "tile loads");
};

template <int D, int BC>
struct SmallOffsets {
  using C = SmallCfg<D, BC>;
  int k_rd[C::NDT];
  int v_rd;
  int k_ld[C::NLOAD], v_ld[C::NLOAD];
  int k_dst[C::NLOAD], v_dst[C::NLOAD];
};

template <int D, int BC>
__device__ __forceinline__ void issue_small_tile(const uint16_t *kh, const uint16_t *vh,
                                            int head_bytes, const SmallOffsets<D, BC> &off,
                                            char *stage, int tile_byte) {
  using C = SmallCfg<D, BC>;
  const u32x4 rk = tile_desc(kh, head_bytes, tile_byte);
  const u32x4 rv = tile_desc(vh, head_bytes, tile_byte);
#pragma unroll
  for (int it = 0; it < C::NLOAD; ++it)
    dma16(rk, off.k_ld[it], 0, lds_addr(stage + off.k_dst[it]));
#pragma unroll
  for (int it = 0; it < C::NLOAD; ++it)
    dma16(rv, off.v_ld[it], 0, lds_addr(stage + C::TILE_BYTES + off.v_dst[it]));
}

template <int D, int BC>
struct SmallState {
  using C = SmallCfg<D, BC>;
  bf16x8 qreg[C::NDT];
  f32x16 oacc[C::NCT];
  float m_run, l_run, lr_run;
};

// S^T of one tile (MFMA), mask, checked softmax, sums, P~.V (MFMA).
template <int D, int BC, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void small_tile(const char *sb, const SmallOffsets<D, BC> &off,
                                      SmallState<D, BC> &st, float c, int j0, int N, int qi,
                                      int hh) {
  using C = SmallCfg<D, BC>;
  f32x16 s[C::NKT];
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
      const bf16x8 a = lds_load<bf16x8>(sb, off.k_rd[dt] + kt * 32 * D * 2);
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qreg[dt], s[kt], 0, 0, 0);
    }
  if (MASKED) {
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
      }
  }
  auto raise = [&]() {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    float mlo, mhi;
    halves(mx, mlo, mhi);
    mx = fmaxf(mlo, mhi);
    const float m_tile = (MASKED && mx == -INFINITY) ? -INFINITY : mx * c;
    return m_tile;
  };
  auto rescale = [&](float m_tile) {
    const float m_new = fmaxf(st.m_run, m_tile);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
    st.lr_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[ct][r] *= alpha;
  };
  bf16x8 pb[C::NKT][2];
  auto exps = [&](float mu) -> float {
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
    return rs;
  };
  float rs = exps(st.m_run);
  if (__builtin_amdgcn_ballot_w64(!(rs <= kCheckedSumLimit))) {
    rescale(raise());
    rs = exps(st.m_run == -INFINITY ? 0.f : st.m_run);
  }
  st.l_run += rs;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float rr = st.lr_run;
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pb[kt][u][e], pb[kt][u][e + 1]};
        rr = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rr, false);
      }
  st.lr_run = rr;
  const char *vb = sb + C::TILE_BYTES;
#pragma unroll
  for (int ks = 0; ks < 2 * C::NKT; ++ks) {
    bf16x8 a[C::NCT];
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      const int imm = ct * C::BC * 64 + 16 * ks * 64;
      const s16x4 lo = lds_read_tr(vb, off.v_rd + imm);
      const s16x4 hi = lds_read_tr(vb, off.v_rd + imm + 8 * 64);
      a[ct] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
      st.oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ct], pb[ks >> 1][ks & 1],
                                                            st.oacc[ct], 0, 0, 0);
  }
}

template <int D, int BC, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 4) void fwd_small_kernel(Params p) {
  using C = SmallCfg<D, BC>;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int hh = lane >> 5;
  const int Nq = p.nq, Nk = p.nk;
  const int qoff = Nk - Nq;
  const int head_bytes = Nk * D * 2;

  SmallOffsets<D, BC> off;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
    off.k_rd[dt] = (lr * D + (((2 * dt + hh) ^ kswz<D>(lr)) * 8)) * 2;
  {
    const int g = lane >> 4, sl = lane & 15;
    off.v_rd = (4 * hh + (sl >> 2)) * 64 + (g & 1) * 32 + (sl & 3) * 8;
  }
#pragma unroll
  for (int it = 0; it < C::NLOAD; ++it) {
    const int inst = wv * C::NLOAD + it;
    const int row = inst * C::K_ROWS_PER_LOAD + lane / C::KCH;
    const int pos = lane % C::KCH;
    off.k_ld[it] = row * D * 2 + ((pos ^ kswz<D>(row)) * 16);
    off.k_dst[it] = inst * 1024;
    const int cg = inst / C::VGROUPS, kb = inst % C::VGROUPS;
    off.v_ld[it] = (16 * kb + lane / 4) * D * 2 + (4 * cg + (lane & 3)) * 16;
    off.v_dst[it] = cg * C::BC * 64 + kb * 1024;
  }
  float c = p.c;
  uint32_t qflip = 0;
  if (c < 0.f) {
    c = -c;
    qflip = 0x80008000u;
  }
  auto stage = [&](int t) { return smem + (t % C::NSTAGE) * C::STAGE_BYTES; };
  int split, bh, q0;
  {
    int logical = xcd_remap(blockIdx.x, p.total);
    split = 0;
    if (p.n_splits > 1) {
      split = logical % p.n_splits;
      logical /= p.n_splits;
    }
    bh = logical / p.n_qblocks;
    const int qbl = logical - bh * p.n_qblocks;
    q0 = (CAUSAL ? (p.n_qblocks - 1 - qbl) : qbl) * kRows;
  }
  const int kvbh = p.group == 1 ? bh : (bh / p.h) * (p.h / p.group) + (bh % p.h) / p.group;
  const size_t kvhead = static_cast<size_t>(kvbh) * Nk * D;
  const uint16_t *kh = p.k + kvhead;
  const uint16_t *vh = p.v + kvhead;
  const int qw = q0 + wv * 32;
  const int qi = qw + lr;
  const int qpos = qi + qoff;
  SmallState<D, BC> st;
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.q + static_cast<size_t>(bh) * Nq * D), 0, Nq * D * 2,
        kBufWord3);
    const int q_ld = ((qw + lr) * D + 8 * hh) * 2;
#pragma unroll
    for (int t = 0; t < C::NDT; ++t)
      st.qreg[t] = __builtin_bit_cast(
          bf16x8, __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rq, q_ld + 32 * t, 0, 0)) ^ qflip);
  }
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[ct][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.lr_run = 0.f;
  const int kend = CAUSAL && !p.no_skip ? max(0, min(Nk, q0 + kRows + qoff)) : Nk;
  const int tb = split * p.tiles_per_split;
  const int ntiles = min((kend + C::BC - 1) / C::BC, tb + p.tiles_per_split);
  const int n_full = CAUSAL ? max(0, (q0 + qoff + 1) / C::BC) : Nk / C::BC;
  const bool live = qw < Nq;
  const int w_tiles = !live ? tb
                      : CAUSAL && !p.no_skip ? min(ntiles, (qw + 31 + qoff) / C::BC + 1)
                                             : ntiles;
  const int n_main = live ? min(n_full, ntiles) : tb;
  if (tb < ntiles) {
    if (Nk % C::BC != 0) {
      for (int i = tid; i < C::NSTAGE * C::STAGE_BYTES / 16; i += kThreads)
        reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    issue_small_tile<D, BC>(kh, vh, head_bytes, off, stage(tb), tb * C::BC * D * 2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&](auto masked_tag, int t) {
      constexpr bool M = decltype(masked_tag)::value;
      const int j0 = t * C::BC;
      if (t + 1 < ntiles)
        issue_small_tile<D, BC>(kh, vh, head_bytes, off, stage(t + 1), (j0 + C::BC) * D * 2);
      if (t < w_tiles) small_tile<D, BC, CAUSAL, M>(stage(t), off, st, c, j0, Nk, qpos, hh);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    using F = std::integral_constant<bool, false>;
    using T = std::integral_constant<bool, true>;
    int t = tb;
    for (; t < n_main; ++t) step(F{}, t);
    for (; t < ntiles; ++t) step(T{}, t);
  }
  float llo, lhi, rlo, rhi;
  halves(st.l_run, llo, lhi);
  halves(st.lr_run, rlo, rhi);
  const float l_tot = llo + lhi;
  const float lr_tot = rlo + rhi;
  const float inv = lr_tot > 0.f ? 1.0f / lr_tot : 0.f;
  if (qi < Nq) {
    const size_t head = static_cast<size_t>(bh) * Nq * D + split * p.o_split_stride;
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
          for (int b = 0; b < 4; ++b) ob[b] = static_cast<__bf16>(st.oacc[ct][4 * a + b] * inv);
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.o) + o_off) =
              __builtin_bit_cast(u32x2, ob);
        }
      }
    if (p.lse && hh == 0)
      p.lse[split * p.lse_split_stride + static_cast<size_t>(bh) * Nq + qi] =
          l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---- merge of key ranges -----------------------------------------------------
//
// Key range s of a query row left O_s = O~_s / l_s (fp32) and lse_s = m_s +
// ln l_s (base e).  The two-block merge of the shakilmahmud.com page "Large
// language models part 06: FlashAttention -- GPU SRAM, tiling, online
// softmax", section 2, applied to all ranges at once: with m = max_s lse_s,
//   l = sum_s exp(lse_s - m),  O = sum_s exp(lse_s - m) O_s / l,
//   lse = m + ln l.
// A range that saw no key of the row has lse_s = -inf and weight 0.
template <int D, bool O32>
__global__ __launch_bounds__(kThreads) void merge_splits_kernel(
    const float *o_part, const float *lse_part, void *o, float *lse,
    int64_t rows, int n_splits, size_t o_stride, size_t lse_stride) {
  constexpr int LPR = 32;      // lanes per row
  constexpr int CPL = D / LPR;  // columns per lane
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / LPR) +
                      threadIdx.x / LPR;
  const int col = (threadIdx.x % LPR) * CPL;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, lse_part[s * lse_stride + row]);
  float acc[CPL], l = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float ls = lse_part[s * lse_stride + row];
      if (ls == -INFINITY) continue;
      const float w = __expf(ls - m);
      l += w;
      const float *src = o_part + s * o_stride + row * D + col;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(w, src[c], acc[c]);
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const size_t dst = static_cast<size_t>(row) * D + col;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (O32)
      static_cast<float *>(o)[dst + c] = acc[c] * inv;
    else
      static_cast<__bf16 *>(o)[dst + c] = static_cast<__bf16>(acc[c] * inv);
  }
  if (lse && col == 0) lse[row] = l > 0.f ? m + __logf(l) : -INFINITY;
}

// d = 128: fwd_bf16_kernel (two waves per SIMD, 64-key tiles, S(t+1) in
// flight); d = 64: fwd_small_kernel (four waves per SIMD, 64-key tiles).
template <int D, bool CAUSAL, bool O32>
hipError_t launch(const Params &prm, int grid, hipStream_t s) {
  unsigned pad = 0;
  if constexpr (D == 64) {
    const hipError_t e = debug_lds_pad(
        reinterpret_cast<const void *>(&fwd_small_kernel<D, kSmallTile, CAUSAL, O32>), &pad);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_small_kernel<D, kSmallTile, CAUSAL, O32>), dim3(grid),
                       dim3(kThreads), pad, s, prm);
  } else {
    const hipError_t e =
        debug_lds_pad(reinterpret_cast<const void *>(&fwd_bf16_kernel<D, CAUSAL, O32>), &pad);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, O32>), dim3(grid),
                       dim3(kThreads), pad, s, prm);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Params &prm, int grid, bool causal, bool o32, hipStream_t s) {
  if (causal)
    return o32 ? launch<D, true, true>(prm, grid, s) : launch<D, true, false>(prm, grid, s);
  return o32 ? launch<D, false, true>(prm, grid, s) : launch<D, false, false>(prm, grid, s);
}

// Compute units of the current device (cached per device; 0 if unknown).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D>
hipError_t launch_merge(const FwdArgs &a, bool o32, size_t o_stride,
                        size_t lse_stride, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.bh) * a.nq;
  const int rpb = kThreads / 32;
  const dim3 grid(static_cast<unsigned>((rows + rpb - 1) / rpb));
  if (o32)
    hipLaunchKernelGGL((merge_splits_kernel<D, true>), grid, dim3(kThreads), 0, s,
                       a.o_part, a.lse_part, a.o, a.lse, rows, a.n_splits,
                       o_stride, lse_stride);
  else
    hipLaunchKernelGGL((merge_splits_kernel<D, false>), grid, dim3(kThreads), 0, s,
                       a.o_part, a.lse_part, a.o, a.lse, rows, a.n_splits,
                       o_stride, lse_stride);
  return hipGetLastError();
}

}  // namespace

// Workspace of fa2_fwd_splitkv_noalloc, one copy per device for the life of
// the process.  Host code never uses the name itself as an address (on the
// host it is only a stand-in): fwd_scratch() looks the device address up.
static __device__ __align__(256) float scratch[kFwdScratchBytes / sizeof(float)];

hipError_t fwd_scratch(float **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = static_cast<float *>(addr[dev]);
  return hipSuccess;
}

// FA2_DEBUG_NO_SKIP=1 in the environment (read at every call) makes causal
// query blocks run the key tiles past their diagonal too, through the masked
// path, where every score is hidden and adds exactly zero: a test of the
// tile skipping, which must not change any output.
static int debug_no_skip() {
  const char *e = std::getenv("FA2_DEBUG_NO_SKIP");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

hipError_t debug_lds_pad(const void *kernel, unsigned *pad) {
  *pad = 0;
  const char *e = std::getenv("FA2_DEBUG_ONE_WG_PER_CU");
  if (e == nullptr || e[0] != '1' || e[1] != '\0') return hipSuccess;
  hipFuncAttributes fa;
  const hipError_t r = hipFuncGetAttributes(&fa, kernel);
  if (r != hipSuccess) return r;
  constexpr size_t kTarget = 84u * 1024;  // > 160 KB / 2
  *pad = fa.sharedSizeBytes < kTarget ? static_cast<unsigned>(kTarget - fa.sharedSizeBytes) : 0;
  return hipSuccess;
}

hipError_t launch_fwd_bf16(const FwdArgs &a, bool o32, hipStream_t s) {
  Params prm;
  prm.q = static_cast<const uint16_t *>(a.q);
  prm.k = static_cast<const uint16_t *>(a.k);
  prm.v = static_cast<const uint16_t *>(a.v);
  prm.nq = a.nq;
  prm.nk = a.nk;
  prm.h = a.h;
  prm.group = a.group;
  prm.n_qblocks = (a.nq + kRows - 1) / kRows;
  prm.n_splits = a.n_splits;
  const int bc = a.d == 128 ? Cfg<128>::BC : kSmallTile;
  const int key_tiles = (a.nk + bc - 1) / bc;
  prm.tiles_per_split = (key_tiles + a.n_splits - 1) / a.n_splits;
  prm.total = a.bh * prm.n_qblocks * a.n_splits;
  prm.c = a.scale * kLog2e;
  prm.no_skip = debug_no_skip();
  // A grid of two workgroups per compute unit walks the items when there
  // are more items than that and every item starts at key tile 0 with whole
  // tiles (d = 128, one key range, equal query and key lengths, no ragged
  // tile) -- and only for causal attention with at most 64 query blocks per
  // head, where hiding each block's first loads and pairing long with short
  // blocks measured faster.  Elsewhere (uniform blocks, or blocks so long
  // that speed differences between workgroups outweigh the saved latency)
  // the hardware's dynamic dispatch of one workgroup per item measured
  // as fast or faster.
  prm.persist = 0;
  int grid = prm.total;
  const int slots = (2 * cu_count()) & ~7;
  if (a.d == 128 && a.causal && prm.n_qblocks <= 64 && a.n_splits == 1 &&
      a.nq == a.nk && a.nk % bc == 0 && slots >= 8 && prm.total > slots) {
    prm.persist = 1;
    grid = slots;
  }
  if (a.n_splits == 1) {
    prm.o = a.o;
    prm.lse = a.lse;
    prm.o_split_stride = prm.lse_split_stride = 0;
    if (a.d == 128) return launch_d<128>(prm, grid, a.causal, o32, s);
    return launch_d<64>(prm, grid, a.causal, o32, s);
  }
  // key ranges into the fp32 partial buffers, then the merge
  prm.o = a.o_part;
  prm.lse = a.lse_part;
  prm.o_split_stride = static_cast<size_t>(a.bh) * a.nq * a.d;
  prm.lse_split_stride = static_cast<size_t>(a.bh) * a.nq;
  hipError_t e = a.d == 128 ? launch_d<128>(prm, grid, a.causal, true, s)
                            : launch_d<64>(prm, grid, a.causal, true, s);
  if (e != hipSuccess) return e;
  return a.d == 128 ? launch_merge<128>(a, o32, prm.o_split_stride, prm.lse_split_stride, s)
                    : launch_merge<64>(a, o32, prm.o_split_stride, prm.lse_split_stride, s);
}

}  // namespace fa2
