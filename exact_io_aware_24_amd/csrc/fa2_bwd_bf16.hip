// Exact attention backward, bf16 inputs, bf16 MFMA on gfx950 (CDNA4).
//
// What is computed (per batch*head; P is never stored, it is recomputed
// tile by tile from the forward's log-sum-exp -- the recomputation idea of
// the unite.ai page "Flash Attention: revolutionising transformer
// efficiency", section "Enter Flash Attention"):
//
//   P_ij  = exp(scale q_i.k_j - lse_i)       (0 where the causal mask hides j)
//   D_i   = dO_i . O_i                       (= sum_j P_ij dP_ij, since O = PV)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_i dS_ij q_i
//
// These are the exact gradients of the forward definition; the pages give no
// backward formula beyond the recomputation.  Three kernels, in stream
// order, none with atomics (results are bit-reproducible):
//   delta_kernel : D_i from the bf16 O and dO rows (fp32 sums);
//   dkdv_kernel  : one workgroup per 128 keys; K and V stay in registers
//                  while Q, dO (and their lse, D) stream through LDS in
//                  tiles of 64 queries;
//   dq_kernel    : one workgroup per 128 queries; Q and dO stay in registers
//                  while K and V stream through LDS in tiles of 64 keys --
//                  the forward kernel's query-block parallelism (improvement
//                  2 of the "FlashAttention-2 (BN)" wiki article).
// Splitting dQ from dK/dV recomputes S and dP once more but needs neither
// atomics nor a dQ accumulation buffer.
//
// Grouped K/V heads (query head h reads K/V head h / (H / H_kv)): dQ needs
// only that index map; dK and dV of a shared head are sums over its group of
// query heads.  A dkdv_kernel workgroup streams the query tiles of every
// head of one range of the group in turn, accumulating in the same
// registers; with one range per group it writes dK/dV directly, with several
// each range writes an fp32 partial and reduce_parts_kernel adds the
// partials in range order (deterministic, no atomics).  Causal with several
// heads per range, dkdv_pair_kernel does the same for two key blocks per
// workgroup, ordered so that a range's workgroups read the same query tiles
// at the same time (see there).
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16): A lane l holds A[l%32][8(l/32)
// .. +7], B lane l holds B[8(l/32) .. +7][l%32], the result register r of
// lane l is D[8(r/4) + 4(l/32) + r%4][l%32].  Each kernel computes its
// products so that lane l%32 owns one row of what it accumulates (a query in
// dq_kernel, a key in dkdv_kernel) and the result registers of one product
// are, converted to bf16, the B operand of the next one as they stand.
//
// LDS tiles use one layout for every operand ("block-swizzled"): a tile of
// R rows x d columns is stored as d/32 blocks of R rows x 64 bytes, and the
// four 16-byte chunks of each 64-byte row segment are XOR-permuted by
// (row / 4) % 4.  Row reads (ds_read_b128: 16 lanes, 16 rows, the same
// chunk) and transposed reads (ds_read_b64_tr_b16: 4 consecutive rows, 32
// bytes each per 16 lanes) then both hit distinct banks, so each tile is
// stored once and read both ways.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kBlk = kBf16BwdRowsPerBlock;  // 128 queries (dq) / keys (dkdv)
constexpr int kTileRows = 64;               // rows of a streamed LDS tile

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dout;
  const float *lse;
  float *delta;
  void *dq, *dk, *dv;
  float *dk_part, *dv_part;  // [n_gsplits][B*H_kv][N][d] (n_gsplits > 1)
  size_t part_stride;        // B*H_kv*N*d
  int n;          // sequence length
  int n_blocks;   // ceil(n / 128)
  int total;      // B*H*n_blocks (dq grid size)
  int total_kv;   // dkdv grid size: B*H_kv*n_gsplits*n_blocks, or with
                  // paired key blocks B*H_kv*n_gsplits*ceil(n_blocks / 2)
  int h;          // query heads per batch index
  int group;      // query heads per K/V head
  int n_gsplits;  // ranges of a group's query heads
  float c;        // scale * log2(e)
  float scale;
};

// K/V head read by query head bh (both counted over B*H / B*H_kv).
__device__ __forceinline__ int kv_head(int bh, int h, int group) {
  return group == 1 ? bh : (bh / h) * (h / group) + (bh % h) / group;
}

template <int D>
struct BCfg {
  static constexpr int NDT = D / 16;                      // 16-column k-steps
  static constexpr int NCT = D / 32;                      // 32-column blocks
  static constexpr int BLOCK_BYTES = kTileRows * 64;      // one column block
  static constexpr int TILE_BYTES = NCT * BLOCK_BYTES;    // 16 KB (d=128)
  static constexpr int PIECES = TILE_BYTES / 1024;        // 1 KB wave loads
  static constexpr int PPW = PIECES / 4;                  // per wave
};

// ---- block-swizzled tile addressing ----------------------------------------

// Byte offset of the 16-byte chunk holding columns [8ch', 8ch'+8) of column
// block cb, row r (logical chunk ch, 0..3).
__device__ __forceinline__ int blk_off(int r, int cb, int ch) {
  return cb * kTileRows * 64 + r * 64 + ((ch ^ ((r >> 2) & 3)) * 16);
}

// Per-lane offsets fixed for a whole kernel.
template <int D>
struct TileOffsets {
  int rd[2];       // row reads: k-step parity 0 / 1 (other steps: immediates)
  int tr[2];       // transposed reads: lo (rows +0..3), hi (rows +8..11)
  int ld[BCfg<D>::PPW];  // byte offset of this lane's 16 bytes from the
                         // tile's first row, per wave load
};

template <int D>
__device__ __forceinline__ TileOffsets<D> tile_offsets(int lane, int wv) {
  using C = BCfg<D>;
  TileOffsets<D> t;
  const int lr = lane & 31, hh = lane >> 5;
  // row read of row lr, columns 16ks + 8hh: chunk 2(ks&1) + hh of block ks/2
  t.rd[0] = blk_off(lr, 0, hh);
  t.rd[1] = blk_off(lr, 0, 2 + hh);
  // transposed read: lane (g, s) of 16-lane group g addresses row 4hh + s/4
  // (+8 for hi) and columns 16(g&1) + 4(s%4) .. +3 of a block; the row's
  // swizzle key (row / 4) % 4 is hh (lo) or hh + 2 (hi)
  const int g = lane >> 4, s = lane & 15;
  const int ch = 2 * (g & 1) + ((s & 3) >> 1);
  t.tr[0] = (4 * hh + (s >> 2)) * 64 + ((ch ^ hh) * 16) + (s & 1) * 8;
  t.tr[1] = (8 + 4 * hh + (s >> 2)) * 64 + ((ch ^ (hh + 2)) * 16) + (s & 1) * 8;
  // wave load `it`: 16 rows x 64 bytes of one column block, lane i to LDS
  // position 16 i, i.e. row i/4 of the piece, stored chunk i%4, which holds
  // logical chunk (i%4) ^ (row/4 % 4)
#pragma unroll
  for (int it = 0; it < C::PPW; ++it) {
    const int pc = wv * C::PPW + it;
    const int cb = pc >> 2, rb = pc & 3;
    const int row = rb * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    t.ld[it] = row * D * 2 + cb * 64 + chunk * 16;
  }
  return t;
}

// This wave's share of one tile: rows [row0, row0 + 64) of the head at
// `base` (rows past its end load as zeros).
template <int D>
__device__ __forceinline__ void issue_tile(const uint16_t *base, int head_bytes,
                                           const TileOffsets<D> &o, char *buf,
                                           int wv, int row0) {
  using C = BCfg<D>;
  const u32x4 rsrc = tile_desc(base, head_bytes, row0 * D * 2);
#pragma unroll
  for (int it = 0; it < C::PPW; ++it) {
    const int pc = wv * C::PPW + it;
    const int cb = pc >> 2, rb = pc & 3;
    const int vo = o.ld[it];
    dma16(rsrc, vo, 0, lds_addr(buf + cb * C::BLOCK_BYTES + rb * 1024));
  }
}

// A operand of a product over the columns: row `row_base + lane%32` of the
// tile, k-step ks (columns 16ks + 8hh .. +7).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char *buf,
                                              const TileOffsets<D> &o,
                                              int row_base, int ks) {
  return lds_load<bf16x8>(buf, o.rd[ks & 1] + (ks >> 1) * BCfg<D>::BLOCK_BYTES +
                                   row_base * 64);
}

// A operand of a product over the rows: column 32ct + lane%32 of the tile,
// rows 16 step + 4hh + 0..3 (transposed read lo) and 16 step + 8 + 4hh +
// 0..3 (hi).  That is the row order of registers 8u .. 8u+7 of a 32x32
// result whose rows are the same tile rows, so such a result, converted to
// bf16, is the matching B operand as it stands.
template <int D>
__device__ __forceinline__ bf16x8 col_operand(const char *buf,
                                              const TileOffsets<D> &o, int ct,
                                              int step) {
  const int base = ct * BCfg<D>::BLOCK_BYTES + step * 16 * 64;
  const s16x4 lo = lds_read_tr(buf, o.tr[0] + base);
  const s16x4 hi = lds_read_tr(buf, o.tr[1] + base);
  return __builtin_bit_cast(
      bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes (8 bf16) of row `row` of a head, columns 8hh + 16t, for every t:
// the B operand of a product over the columns, held in registers.
template <int D>
__device__ __forceinline__ void load_row_operand(const uint16_t *head_base,
                                                 int head_bytes, int row,
                                                 int hh, bf16x8 (&r)[D / 16]) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(head_base), 0, head_bytes, kBufWord3);
  const int off = (row * D + 8 * hh) * 2;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    r[t] = __builtin_bit_cast(bf16x8,
                              __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * t, 0, 0));
}

// Store a 32-row x d accumulator held transposed (register r of column block
// ct = column 32ct + 8(r/4) + 4hh + r%4 of this lane's row), times `mul`.
template <int D, bool O32>
__device__ __forceinline__ void store_rows(void *out, size_t row_elem, int hh,
                                           const f32x16 (&acc)[D / 32],
                                           float mul) {
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const size_t off = row_elem + 32 * ct + 8 * a + 4 * hh;
      if (O32) {
        f32x4 v;
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = acc[ct][4 * a + b] * mul;
        *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + off) = v;
      } else {
        __bf16 v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = static_cast<__bf16>(acc[ct][4 * a + b] * mul);
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(out) + off) =
            __builtin_bit_cast(u32x2, v);
      }
    }
}

// ---- D_i = dO_i . O_i -------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(const uint16_t *o,
                                                         const uint16_t *dout,
                                                         float *delta,
                                                         int64_t rows) {
  constexpr int LPR = D / 8;           // lanes per row, 8 elements each
  constexpr int RPB = kThreads / LPR;  // rows per workgroup
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(o + row * D + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(a[w] & 0xffff0000u),
                           __uint_as_float(b[w] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---- dK, dV -----------------------------------------------------------------
//
// One step of the dK/dV accumulation: the tile of 64 queries (Q, dO, lse in
// base-2 units, D) in LDS at qb/ob/lb/db against this wave's 32 keys
// (k0 + 32w .. +31, K and V in registers), as two 32-query halves:
//   S  = Q K^T      A = Q rows (LDS),  B = K (registers)  -> lane = key
//   dP = dO V^T     A = dO rows (LDS), B = V (registers)
//   P = exp2(S c - lse log2 e), dS = P (dP - D)
//   dV^T += dO^T P  A = dO columns (transposed LDS reads), B = P (bf16)
//   dK^T += Q^T dS  A = Q columns,                        B = dS (bf16)
// MASKED: the tile holds a query before one of the block's keys (causal) --
// a compile-time switch, so that the other tiles carry no mask
// instructions.  A wave whose keys all come after every query of the tile
// has nothing to do.
template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void dkdv_tile(const char *qb, const char *ob,
                                          const char *lb, const char *db,
                                          const TileOffsets<D> &off,
                                          const bf16x8 (&kreg)[D / 16],
                                          const bf16x8 (&vreg)[D / 16],
                                          f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                          float c, int t, int kw, int kj, int hh) {
  using C = BCfg<D>;
  if (CAUSAL && t * kTileRows + kTileRows - 1 < kw) return;
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // 32-query halves of the tile
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NDT; ++ks) {
      s = mfma(row_operand<D>(qb, off, 32 * h, ks), kreg[ks], s);
      dp = mfma(row_operand<D>(ob, off, 32 * h, ks), vreg[ks], dp);
    }
    // register r holds query 32h + 8(r/4) + 4hh + r%4 of the tile
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int qrow = 32 * h + 8 * a + 4 * hh;
      const f32x4 l4 = lds_load<f32x4>(lb, qrow * 4);  // lse log2(e)
      const f32x4 d4 = lds_load<f32x4>(db, qrow * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a + e;
        float x = fast_exp2(__builtin_fmaf(s[r], c, -l4[e]));
        if (MASKED && kj > t * kTileRows + qrow + e) x = 0.f;
        const float ds = x * (dp[r] - d4[e]);
        pb[r >> 3][r & 7] = static_cast<__bf16>(x);
        sb[r >> 3][r & 7] = static_cast<__bf16>(ds);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        dv[ct] = mfma(col_operand<D>(ob, off, ct, 2 * h + u), pb[u], dv[ct]);
        dk[ct] = mfma(col_operand<D>(qb, off, ct, 2 * h + u), sb[u], dk[ct]);
      }
  }
}

//
// Workgroup: 128 keys of one K/V head, wave w owns keys k0 + 32w + lane%32,
// and one range of the query heads that read this K/V head (all of them, or
// one of n_gsplits ranges).  K and V of those keys are B operands held in
// registers; for each query head of the range and each of its tiles of 64
// queries (two 32-query halves):
//   S  = Q K^T      A = Q rows (LDS),  B = K (registers)  -> lane = key
//   dP = dO V^T     A = dO rows (LDS), B = V (registers)
//   P = exp2(S c - lse log2 e), dS = P (dP - D)
//   dV^T += dO^T P  A = dO columns (transposed LDS reads), B = P (bf16)
//   dK^T += Q^T dS  A = Q columns,                        B = dS (bf16)
// The lse and D values of a tile are staged in LDS next to it (rows past
// the sequence end read as 0, which gives them zero weight because their
// Q and dO rows are zero too).  (The tile step is written out here rather
// than called as dkdv_tile: through the function the register allocator
// placed a spill in the unmasked tile loop of the causal d = 128 variants.)
template <int D, bool CAUSAL, bool O32, bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void dkdv_kernel(BwdParams p) {
  using C = BCfg<D>;
  // [Q 0][Q 1][dO 0][dO 1][lse 0][lse 1][D 0][D 1] (statistics: 1 KB each,
  // of which the first 256 bytes are used)
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES + 4 * 1024];
  auto qbuf = [&](int i) { return smem + i * C::TILE_BYTES; };
  auto obuf = [&](int i) { return smem + (2 + i) * C::TILE_BYTES; };
  auto lbuf = [&](int i) { return smem + 4 * C::TILE_BYTES + i * 1024; };
  auto dbuf = [&](int i) { return smem + 4 * C::TILE_BYTES + (2 + i) * 1024; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, p.total_kv);
  const int unit = logical / p.n_blocks;        // (K/V head, query-head range)
  const int kb = logical - unit * p.n_blocks;   // causal: block 0 is heaviest
  const int kvbh = unit / p.n_gsplits;
  const int gs = unit - kvbh * p.n_gsplits;
  const int hkv = p.h / p.group;
  const int g_lo = gs * p.group / p.n_gsplits;
  const int ng = (gs + 1) * p.group / p.n_gsplits - g_lo;  // >= 1
  const int qbh0 = (kvbh / hkv) * p.h + (kvbh % hkv) * p.group + g_lo;
  const int N = p.n;
  const size_t head = static_cast<size_t>(kvbh) * N * D;
  const int head_bytes = N * D * 2;
  const int k0 = kb * kBlk;
  const int kw = k0 + 32 * wv;
  const int kj = kw + lr;

  bf16x8 kreg[C::NDT], vreg[C::NDT];
  load_row_operand<D>(p.k + head, head_bytes, kj, hh, kreg);
  load_row_operand<D>(p.v + head, head_bytes, kj, hh, vreg);
  f32x16 dk[C::NCT], dv[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[ct][r] = dv[ct][r] = 0.f;

  const TileOffsets<D> off = tile_offsets<D>(lane, wv);
  // statistics: wave 0 loads lse, wave 1 loads D; lanes 16.. read past the
  // end of the buffer (zero) into the unused part of the staging area
  const int st_off = lane < 16 ? lane * 16 : 0x7ffffff0;

  // query tiles: causal -> from the tile holding query k0
  const int nt = (N + kTileRows - 1) / kTileRows;
  const int t0 = CAUSAL ? k0 / kTileRows : 0;
  // tiles below this one contain a query before one of the block's keys
  const int t_full = CAUSAL ? (k0 + kBlk - 1 + kTileRows - 1) / kTileRows : 0;

  // tile t of query head qbh0 + g
  auto issue = [&](int g, int t, int buf) {
    const size_t rows = static_cast<size_t>(qbh0 + g) * N;
    issue_tile<D>(p.q + rows * D, head_bytes, off, qbuf(buf), wv, t * kTileRows);
    issue_tile<D>(p.dout + rows * D, head_bytes, off, obuf(buf), wv, t * kTileRows);
    if (wv == 0)
      dma16(tile_desc(p.lse + rows, N * 4, t * kTileRows * 4), st_off, 0,
            lds_addr(lbuf(buf)));
    if (wv == 1)
      dma16(tile_desc(p.delta + rows, N * 4, t * kTileRows * 4), st_off, 0,
            lds_addr(dbuf(buf)));
  };

  if (N % kTileRows != 0) {  // ragged end: never expose stale LDS bits
    for (int i = tid; i < (4 * C::TILE_BYTES + 4 * 1024) / 16; i += kThreads)
      reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  // Wave 0 stages each tile's lse; once its load has landed (its own wait),
  // and before the barrier that publishes the tile, it turns the 64 values
  // into base-2 units in place, so that no wave multiplies them per element.
  auto lse_to_base2 = [&](int buf) {
    if (wv == 0) {
      float *l = reinterpret_cast<float *>(lbuf(buf)) + lane;
      *l = *l * kLog2e;
    }
  };
  // Order of the (head, query tile) steps.  One query head: tiles upward
  // from the block's first.  Several (GROUPED): tiles from the last one down
  // to the block's first, the range's heads interleaved at each tile, so
  // that every workgroup of a (K/V head, head range) starts at the same tile
  // and they move down together: a tile's Q and dO are fetched once for all
  // of them and stay in L2 while they are read (walking up head by head,
  // each workgroup starts at its own diagonal tile, and the range's Q/dO,
  // twice an XCD's L2, is streamed again for every workgroup).
  if (t0 < nt) issue(0, GROUPED ? nt - 1 : t0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  lse_to_base2(0);
  __syncthreads();

  const float c = p.c;
  // One (head, tile) step, the next pair's tile prefetched (tiles
  // descending, heads ascending within a tile).  MASKED: the tile holds a
  // query before one of the block's keys (causal, t < t_full) -- a
  // compile-time switch, so that the other tiles carry no mask
  // instructions.
  int b = 0;
  auto step = [&](auto masked_tag, int g, int t) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    bool next;
    if (GROUPED) {
      next = g + 1 < ng || t > t0;
      if (g + 1 < ng) issue(g + 1, t, b ^ 1);
      else if (t > t0) issue(0, t - 1, b ^ 1);
    } else {
      next = t + 1 < nt || g + 1 < ng;
      if (t + 1 < nt) issue(g, t + 1, b ^ 1);
      else if (g + 1 < ng) issue(g + 1, t0, b ^ 1);
    }
    // this wave's keys all come after every query of the tile: nothing to do
    const bool skip = CAUSAL && (t * kTileRows + kTileRows - 1 < kw);
    if (!skip) {
      const char *qb = qbuf(b), *ob = obuf(b);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // 32-query halves of the tile
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::NDT; ++ks) {
          s = mfma(row_operand<D>(qb, off, 32 * h, ks), kreg[ks], s);
          dp = mfma(row_operand<D>(ob, off, 32 * h, ks), vreg[ks], dp);
        }
        // register r holds query 32h + 8(r/4) + 4hh + r%4 of the tile
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int qrow = 32 * h + 8 * a + 4 * hh;
          const f32x4 l4 = lds_load<f32x4>(lbuf(b), qrow * 4);  // lse log2(e)
          const f32x4 d4 = lds_load<f32x4>(dbuf(b), qrow * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * a + e;
            float x = fast_exp2(__builtin_fmaf(s[r], c, -l4[e]));
            if (MASKED && kj > t * kTileRows + qrow + e) x = 0.f;
            const float ds = x * (dp[r] - d4[e]);
            pb[r >> 3][r & 7] = static_cast<__bf16>(x);
            sb[r >> 3][r & 7] = static_cast<__bf16>(ds);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int ct = 0; ct < C::NCT; ++ct) {
            dv[ct] = mfma(col_operand<D>(ob, off, ct, 2 * h + u), pb[u], dv[ct]);
            dk[ct] = mfma(col_operand<D>(qb, off, ct, 2 * h + u), sb[u], dk[ct]);
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (next) lse_to_base2(b ^ 1);
    __syncthreads();
    b ^= 1;
  };
  const int t_mask_end = CAUSAL ? min(t_full, nt) : t0;
  if constexpr (GROUPED) {
    for (int t = nt - 1; t >= t_mask_end; --t)
      for (int g = 0; g < ng; ++g) step(std::false_type{}, g, t);
    for (int t = t_mask_end - 1; t >= t0; --t)
      for (int g = 0; g < ng; ++g) step(std::true_type{}, g, t);
  } else {
    for (int g = 0; g < ng; ++g) {
      int t = t0;
      for (; t < t_mask_end; ++t) step(std::true_type{}, g, t);
      for (; t < nt; ++t) step(std::false_type{}, g, t);
    }
  }

  if (kj < N) {
    const size_t row = head + static_cast<size_t>(kj) * D;
    if (p.n_gsplits == 1) {
      store_rows<D, O32>(p.dk, row, hh, dk, p.scale);
      store_rows<D, O32>(p.dv, row, hh, dv, 1.0f);
    } else {
      const size_t part = static_cast<size_t>(gs) * p.part_stride;
      store_rows<D, true>(p.dk_part + part, row, hh, dk, p.scale);
      store_rows<D, true>(p.dv_part + part, row, hh, dv, 1.0f);
    }
  }
}

// Causal dK/dV with grouped K/V heads (a range of several query heads per
// workgroup): each workgroup takes key blocks j and n_blocks - 1 - j in
// turn, which together span the same number of query tiles for every j, so
// the n_blocks / 2 workgroups of a (K/V head, head range) start together
// and end together.  The first block is walked downward from the last
// query tile to its diagonal, the second upward from its diagonal to the
// last tile, the range's heads interleaved at each tile: at the workgroups'
// s-th tile step every first block is at tile nt - 1 - s and every second
// block at tile s - 2, so a unit reads two tiles per head at a time, whose
// Q and dO are fetched once and stay in L2 while all of them read it (one
// block per workgroup, the blocks that start as slots free up each stream
// the range's Q and dO on their own).  The tile steps are dkdv_tile's.
template <int D, bool O32>
__global__ __launch_bounds__(kThreads, 2) void dkdv_pair_kernel(BwdParams p) {
  using C = BCfg<D>;
  // [Q 0][Q 1][dO 0][dO 1][lse 0][lse 1][D 0][D 1], as in dkdv_kernel
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES + 4 * 1024];
  auto qbuf = [&](int i) { return smem + i * C::TILE_BYTES; };
  auto obuf = [&](int i) { return smem + (2 + i) * C::TILE_BYTES; };
  auto lbuf = [&](int i) { return smem + 4 * C::TILE_BYTES + i * 1024; };
  auto dbuf = [&](int i) { return smem + 4 * C::TILE_BYTES + (2 + i) * 1024; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int pairs = (p.n_blocks + 1) / 2;
  const int logical = xcd_remap(blockIdx.x, p.total_kv);
  const int unit = logical / pairs;             // (K/V head, query-head range)
  const int jb = logical - unit * pairs;
  const int kvbh = unit / p.n_gsplits;
  const int gs = unit - kvbh * p.n_gsplits;
  const int hkv = p.h / p.group;
  const int g_lo = gs * p.group / p.n_gsplits;
  const int ng = (gs + 1) * p.group / p.n_gsplits - g_lo;  // >= 1
  const int qbh0 = (kvbh / hkv) * p.h + (kvbh % hkv) * p.group + g_lo;
  const int N = p.n;
  const size_t head = static_cast<size_t>(kvbh) * N * D;
  const int head_bytes = N * D * 2;
  const TileOffsets<D> off = tile_offsets<D>(lane, wv);
  const int st_off = lane < 16 ? lane * 16 : 0x7ffffff0;
  const int nt = (N + kTileRows - 1) / kTileRows;

  auto issue = [&](int g, int t, int buf) {
    const size_t rows = static_cast<size_t>(qbh0 + g) * N;
    issue_tile<D>(p.q + rows * D, head_bytes, off, qbuf(buf), wv, t * kTileRows);
    issue_tile<D>(p.dout + rows * D, head_bytes, off, obuf(buf), wv, t * kTileRows);
    if (wv == 0)
      dma16(tile_desc(p.lse + rows, N * 4, t * kTileRows * 4), st_off, 0,
            lds_addr(lbuf(buf)));
    if (wv == 1)
      dma16(tile_desc(p.delta + rows, N * 4, t * kTileRows * 4), st_off, 0,
            lds_addr(dbuf(buf)));
  };
  if (N % kTileRows != 0) {
    for (int i = tid; i < (4 * C::TILE_BYTES + 4 * 1024) / 16; i += kThreads)
      reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  auto lse_to_base2 = [&](int buf) {
    if (wv == 0) {
      float *l = reinterpret_cast<float *>(lbuf(buf)) + lane;
      *l = *l * kLog2e;
    }
  };
  const float c = p.c;
  int b = 0;  // LDS buffer of the current step

  auto run_block = [&](auto down_tag, int kb) {
    constexpr bool down = decltype(down_tag)::value;
    const int k0 = kb * kBlk;
    const int kw = k0 + 32 * wv;
    const int kj = kw + lr;
    bf16x8 kreg[C::NDT], vreg[C::NDT];
    load_row_operand<D>(p.k + head, head_bytes, kj, hh, kreg);
    load_row_operand<D>(p.v + head, head_bytes, kj, hh, vreg);
    f32x16 dk[C::NCT], dv[C::NCT];
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[ct][r] = dv[ct][r] = 0.f;
    const int t0 = k0 / kTileRows;
    const int t_mask_end = min((k0 + kBlk - 1 + kTileRows - 1) / kTileRows, nt);

    // step (g, t), the next one (gn, tn) prefetched into the other buffer
    auto step = [&](auto masked_tag, int g, int t, int gn, int tn) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      if (gn >= 0) issue(gn, tn, b ^ 1);
      dkdv_tile<D, true, MASKED>(qbuf(b), obuf(b), lbuf(b), dbuf(b), off, kreg, vreg, dk,
                                 dv, c, t, kw, kj, hh);
      __builtin_amdgcn_s_waitcnt(0);
      if (gn >= 0) lse_to_base2(b ^ 1);
      __syncthreads();
      b ^= 1;
    };
    // tiles lo .. hi in the walk's direction, each with the range's heads
    constexpr int dt = down ? -1 : 1;
    const int t_last = down ? t0 : nt - 1;
    auto walk = [&](auto masked_tag, int lo, int hi) {
      if (lo > hi) return;
      const int t_end = down ? lo : hi;
      for (int t = down ? hi : lo;; t += dt) {
        for (int g = 0; g < ng; ++g) {
          const bool lg = g + 1 == ng;
          const int gn = !lg ? g + 1 : (t != t_last ? 0 : -1);
          step(masked_tag, g, t, gn, lg ? t + dt : t);
        }
        if (t == t_end) break;
      }
    };
    // this block's first step, into the current buffer (free: the previous
    // block's last step prefetched nothing and ended with a barrier)
    issue(0, down ? nt - 1 : t0, b);
    __builtin_amdgcn_s_waitcnt(0);
    lse_to_base2(b);
    __syncthreads();
    if constexpr (down) {
      walk(std::false_type{}, t_mask_end, nt - 1);
      walk(std::true_type{}, t0, t_mask_end - 1);
    } else {
      walk(std::true_type{}, t0, t_mask_end - 1);
      walk(std::false_type{}, t_mask_end, nt - 1);
    }
    if (kj < N) {
      const size_t row = head + static_cast<size_t>(kj) * D;
      if (p.n_gsplits == 1) {
        store_rows<D, O32>(p.dk, row, hh, dk, p.scale);
        store_rows<D, O32>(p.dv, row, hh, dv, 1.0f);
      } else {
        const size_t pofs = static_cast<size_t>(gs) * p.part_stride;
        store_rows<D, true>(p.dk_part + pofs, row, hh, dk, p.scale);
        store_rows<D, true>(p.dv_part + pofs, row, hh, dv, 1.0f);
      }
    }
  };
  run_block(std::true_type{}, jb);
  if (2 * jb + 1 != p.n_blocks) run_block(std::false_type{}, p.n_blocks - 1 - jb);
}

// dK or dV from the fp32 partials of the n_gsplits query-head ranges:
// out[e] = sum over s of part[s][e], in increasing s.
template <bool O32>
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float *part,
                                                           size_t stride,
                                                           int n_parts,
                                                           size_t n_vec4,
                                                           void *out) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n_vec4;
       i += static_cast<size_t>(gridDim.x) * 256) {
    f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
    for (int s = 1; s < n_parts; ++s) {
      const f32x4 x = reinterpret_cast<const f32x4 *>(part + s * stride)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += x[e];
    }
    if (O32) {
      reinterpret_cast<f32x4 *>(out)[i] = acc;
    } else {
      __bf16 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[e]);
      reinterpret_cast<u32x2 *>(out)[i] = __builtin_bit_cast(u32x2, v);
    }
  }
}

// ---- dQ ---------------------------------------------------------------------
//
// Workgroup: 128 queries of one head, wave w owns queries q0 + 32w +
// lane%32; Q and dO of those queries are B operands in registers.  For each
// tile of 64 keys (two 32-key halves):
//   S^T  = K Q^T     A = K rows (LDS), B = Q (registers)  -> lane = query
//   dP^T = V dO^T    A = V rows (LDS), B = dO (registers)
//   P = exp2(S c - lse log2 e), dS = P (dP - D)
//   dQ^T += K^T dS^T A = K columns (transposed LDS reads), B = dS (bf16)
template <int D, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdParams p) {
  using C = BCfg<D>;
  // [K 0][K 1][V 0][V 1]
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];
  auto kbuf = [&](int i) { return smem + i * C::TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * C::TILE_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, p.total);
  const int bh = logical / p.n_blocks;
  const int qbl = logical - bh * p.n_blocks;
  const int qb = CAUSAL ? (p.n_blocks - 1 - qbl) : qbl;  // longest first
  const int N = p.n;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const size_t kvhead = static_cast<size_t>(kv_head(bh, p.h, p.group)) * N * D;
  const int head_bytes = N * D * 2;
  const int q0 = qb * kBlk;
  const int qw = q0 + 32 * wv;
  const int qi = qw + lr;

  bf16x8 qreg[C::NDT], oreg[C::NDT];
  load_row_operand<D>(p.q + head, head_bytes, qi, hh, qreg);
  load_row_operand<D>(p.dout + head, head_bytes, qi, hh, oreg);
  float lse2 = 0.f, dlt = 0.f;  // rows past the end: Q = dO = 0 -> dS = 0
  if (qi < N) {
    lse2 = p.lse[static_cast<size_t>(bh) * N + qi] * kLog2e;
    dlt = p.delta[static_cast<size_t>(bh) * N + qi];
  }
  f32x16 dq[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[ct][r] = 0.f;

  const uint16_t *kh = p.k + kvhead, *vh = p.v + kvhead;
  const TileOffsets<D> off = tile_offsets<D>(lane, wv);

  const int kend = CAUSAL ? min(N, q0 + kBlk) : N;
  const int nt = (kend + kTileRows - 1) / kTileRows;
  int n_full = CAUSAL ? (q0 + 1) / kTileRows : N / kTileRows;
  if (n_full > nt) n_full = nt;
  const int w_tiles = CAUSAL ? min(nt, (qw + 31) / kTileRows + 1) : nt;

  if (N % kTileRows != 0) {
    for (int i = tid; i < 4 * C::TILE_BYTES / 16; i += kThreads)
      reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  issue_tile<D>(kh, head_bytes, off, kbuf(0), wv, 0);
  issue_tile<D>(vh, head_bytes, off, vbuf(0), wv, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float c = p.c;
  // One tile; MASKED (the tiles from n_full on: the diagonal band, the
  // ragged end) is a compile-time switch, so that the other tiles carry no
  // mask instructions.
  auto step = [&](auto masked_tag, int t) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int b = t & 1;
    if (t + 1 < nt) {
      issue_tile<D>(kh, head_bytes, off, kbuf(b ^ 1), wv, (t + 1) * kTileRows);
      issue_tile<D>(vh, head_bytes, off, vbuf(b ^ 1), wv, (t + 1) * kTileRows);
    }
    if (t < w_tiles) {
      const char *kbp = kbuf(b), *vbp = vbuf(b);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // 32-key halves of the tile
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::NDT; ++ks) {
          s = mfma(row_operand<D>(kbp, off, 32 * h, ks), qreg[ks], s);
          dp = mfma(row_operand<D>(vbp, off, 32 * h, ks), oreg[ks], dp);
        }
        // register r holds key 32h + 8(r/4) + 4hh + r%4 of the tile
        bf16x8 sb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          if (MASKED) {
            const int key = t * kTileRows + 32 * h + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= N || (CAUSAL && key > qi)) x = 0.f;
          }
          sb[r >> 3][r & 7] = static_cast<__bf16>(x * (dp[r] - dlt));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int ct = 0; ct < C::NCT; ++ct)
            dq[ct] = mfma(col_operand<D>(kbp, off, ct, 2 * h + u), sb[u], dq[ct]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int t = 0;
  for (; t < n_full; ++t) step(std::false_type{}, t);
  for (; t < nt; ++t) step(std::true_type{}, t);

  if (qi < N)
    store_rows<D, O32>(p.dq, head + static_cast<size_t>(qi) * D, hh, dq, p.scale);
}

template <int D, bool CAUSAL, bool O32>
hipError_t launch(const BwdParams &prm, int64_t rows, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 8);
  hipLaunchKernelGGL((delta_kernel<D>), dim3((rows + RPB - 1) / RPB), dim3(kThreads),
                     0, s, prm.o, prm.dout, prm.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned pad = 0;
  if (CAUSAL && prm.group > prm.n_gsplits) {  // paired blocks, several heads per range
    e = debug_lds_pad(reinterpret_cast<const void *>(&dkdv_pair_kernel<D, O32>), &pad);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_pair_kernel<D, O32>), dim3(prm.total_kv), dim3(kThreads), pad, s,
                       prm);
  } else if (prm.group > prm.n_gsplits) {  // some range holds several query heads
    e = debug_lds_pad(reinterpret_cast<const void *>(&dkdv_kernel<D, CAUSAL, O32, true>), &pad);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, O32, true>), dim3(prm.total_kv),
                       dim3(kThreads), pad, s, prm);
  } else {
    e = debug_lds_pad(reinterpret_cast<const void *>(&dkdv_kernel<D, CAUSAL, O32, false>),
                      &pad);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, O32, false>), dim3(prm.total_kv),
                       dim3(kThreads), pad, s, prm);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prm.n_gsplits > 1) {
    const size_t n_vec4 = prm.part_stride / 4;
    const size_t blocks = std::min<size_t>((n_vec4 + 255) / 256, 8192);
    for (int i = 0; i < 2; ++i) {
      hipLaunchKernelGGL((reduce_parts_kernel<O32>), dim3(blocks), dim3(256), 0, s,
                         i == 0 ? prm.dk_part : prm.dv_part, prm.part_stride,
                         prm.n_gsplits, n_vec4, i == 0 ? prm.dk : prm.dv);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  e = debug_lds_pad(reinterpret_cast<const void *>(&dq_kernel<D, CAUSAL, O32>), &pad);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL, O32>), dim3(prm.total), dim3(kThreads),
                     pad, s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdParams &prm, int64_t rows, bool causal, bool o32,
                    hipStream_t s) {
  if (causal)
    return o32 ? launch<D, true, true>(prm, rows, s) : launch<D, true, false>(prm, rows, s);
  return o32 ? launch<D, false, true>(prm, rows, s) : launch<D, false, false>(prm, rows, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs &a, bool o32, hipStream_t s) {
  BwdParams prm;
  prm.q = static_cast<const uint16_t *>(a.q);
  prm.k = static_cast<const uint16_t *>(a.k);
  prm.v = static_cast<const uint16_t *>(a.v);
  prm.o = static_cast<const uint16_t *>(a.o);
  prm.dout = static_cast<const uint16_t *>(a.dout);
  prm.lse = a.lse;
  prm.delta = a.delta;
  prm.dq = a.dq;
  prm.dk = a.dk;
  prm.dv = a.dv;
  prm.n = a.n;
  prm.n_blocks = (a.n + kBlk - 1) / kBlk;
  prm.total = a.bh * prm.n_blocks;
  prm.h = a.h;
  prm.group = a.group;
  prm.n_gsplits = a.n_gsplits;
  // causal with several query heads per range: dkdv_pair_kernel, one
  // workgroup per pair of key blocks
  const bool paired = a.causal && a.group > a.n_gsplits;
  prm.total_kv = a.bh / a.group * a.n_gsplits *
                 (paired ? (prm.n_blocks + 1) / 2 : prm.n_blocks);
  prm.part_stride = static_cast<size_t>(a.bh / a.group) * a.n * a.d;
  prm.dk_part = a.dkv_part;
  prm.dv_part = a.dkv_part ? a.dkv_part + static_cast<size_t>(a.n_gsplits) * prm.part_stride
                           : nullptr;
  prm.c = a.scale * kLog2e;
  prm.scale = a.scale;
  const int64_t rows = static_cast<int64_t>(a.bh) * a.n;
  if (a.d == 128) return launch_d<128>(prm, rows, a.causal, o32, s);
  return launch_d<64>(prm, rows, a.causal, o32, s);
}

}  // namespace fa2
