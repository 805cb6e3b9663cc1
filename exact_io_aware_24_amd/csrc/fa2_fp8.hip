// FP8 forward: block quantisation with incoherent processing, and attention
// on the FP8 MFMA of gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4, twice the
// bf16 rate).
//
// Recipe (FlashAttention-3's FP8 path as the itimpress.au page
// "FlashAttention scaling, multi-GPU training and weight quantisation",
// section 1, describes it): small tiles are scaled independently (block
// quantisation), and Q and K are multiplied by a random orthogonal matrix
// before quantising so that outliers are spread over all channels
// (incoherent processing).  Here:
//   * the orthogonal matrix is diag(signs) H / sqrt(d), H the Walsh-Hadamard
//     matrix: the quantiser applies the signs and the unnormalised fast
//     transform (add/sub butterflies in fp32, stages h = 1, 2, 4, ...), and
//     the two 1/sqrt(d) factors become scale / d in the attention kernel;
//   * each block (128 rows of Q, 64 rows of K or V) gets a power-of-two
//     scale 2^e, the smallest with max|x| <= 448 * 2^e, and is stored as
//     e4m3(x * 2^-e) (round to nearest even);
//   * the attention kernel folds the Q and K exponents into the exp2
//     constant of each tile, and each V tile's exponent into the exp2
//     argument as an exact shift relative to the head's largest one, so
//     O~ accumulates sum_t P_t V_t 2^-e_max with P_t kept <= 2^8 < 448.
// P is rounded to e4m3 for the P.V product; everything else is fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cfloat>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 256;
constexpr int kRows = kFp8RowsPerBlock;  // 128 query rows per workgroup
constexpr int kTile = kFp8KvRowsPerBlock;  // 64 keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;

// ---- quantiser ----------------------------------------------------------------

// Smallest e with amax <= 448 * 2^e: amax = m 2^E (0.5 <= m < 1) and
// 448 = 0.875 * 2^9, so e = E - 9 if m <= 0.875, else E - 8 (0 for amax 0).
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  return m <= 0.875f ? E - 9 : E - 8;
}

// Four floats to four e4m3 codes, byte i = code of x_i (round to nearest
// even; the magnitudes here never exceed 448).  The first conversion writes
// the low half-word and the second the high one, so the register's prior
// contents never reach the result: it starts from whatever the register
// holds (an empty asm that only claims to define it, tied to x0 so that
// every call gets its own) rather than from a zero that costs a move.
__device__ __forceinline__ int cvt_fp8x4(float x0, float x1, float x2, float x3) {
  int any;
  asm("; fp8 pack start" : "=v"(any) : "v"(x0));
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, any, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

// One workgroup per (head, block of R rows).  Four lanes per row, D/4
// values per lane (contiguous): the transform's stages h < D/4 run inside a
// lane, the last two (h = D/4, D/2) pair the lanes of a row, which form one
// quad, exchanged by DPP quad permutes.  In a cross-lane butterfly the lane
// holding the pair's upper element negates its value and adds its
// partner's: b + (-a) is exactly b - a, the same fp32 operations in the
// same order as the in-lane stages.
template <int D, int R>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t *x, uint8_t *codes, int *exps, const float *signs, int n,
    int nblocks) {
  constexpr int EPL = D / 4;           // values per lane
  constexpr int RPP = kThreads / 4;    // rows per pass
  constexpr int PASSES = R / RPP;
  static_assert(PASSES >= 1 && R % RPP == 0, "block rows");
  __shared__ float wmax[kThreads / 64];
  const int bh = blockIdx.x / nblocks;
  const int blk = blockIdx.x - bh * nblocks;
  const int part = threadIdx.x & 3;
  const size_t head = static_cast<size_t>(bh) * n * D;
  // sign flips of this lane's columns as a bit mask: ballots over the
  // wave's lanes give columns 0-63 and 64-127, each lane takes its slice
  uint32_t neg = 0;
  if (signs) {
    const int l = threadIdx.x & 63;
    const uint64_t lo = __builtin_amdgcn_ballot_w64(signs[l] < 0.f);
    uint64_t hi = 0;
    if (D == 128) hi = __builtin_amdgcn_ballot_w64(signs[64 + l] < 0.f);
    const uint64_t word = (part * EPL < 64) ? lo : hi;
    neg = static_cast<uint32_t>(word >> ((part * EPL) & 63));
    if (EPL < 32) neg &= (1u << EPL) - 1u;
  }
  float y[PASSES][EPL];
  float amax = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = blk * R + ps * RPP + (threadIdx.x >> 2);
    u32x4 raw[EPL / 8];
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) raw[c] = u32x4{0u, 0u, 0u, 0u};
    if (row < n) {
#pragma unroll
      for (int c = 0; c < EPL / 8; ++c)
        raw[c] = *reinterpret_cast<const u32x4 *>(
            x + head + static_cast<size_t>(row) * D + part * EPL + 8 * c);
    }
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        y[ps][8 * c + 2 * w] = __uint_as_float(raw[c][w] << 16);
        y[ps][8 * c + 2 * w + 1] = __uint_as_float(raw[c][w] & 0xffff0000u);
      }
    if (signs) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        y[ps][e] = __uint_as_float(__float_as_uint(y[ps][e]) ^ (((neg >> e) & 1u) << 31));
#pragma unroll
      for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (!(i & h)) {
            const float a = y[ps][i], b2 = y[ps][i + h];
            y[ps][i] = a + b2;
            y[ps][i + h] = a - b2;
          }
      // h = EPL: partner lane part ^ 1; h = 2 EPL: part ^ 2
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bool upper = (part >> st) & 1;
        const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int mine = __float_as_int(y[ps][i]);
          const int other = st == 0 ? __builtin_amdgcn_update_dpp(0, mine, 0xB1, 0xF, 0xF, false)
                                    : __builtin_amdgcn_update_dpp(0, mine, 0x4E, 0xF, 0xF, false);
          y[ps][i] = __int_as_float(other) + __uint_as_float(__float_as_uint(y[ps][i]) ^ flip);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(y[ps][i]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = block_exponent(amax);
  const float inv = ldexpf(1.f, -e);
  if (threadIdx.x == 0) exps[static_cast<size_t>(bh) * nblocks + blk] = e;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = blk * R + ps * RPP + (threadIdx.x >> 2);
    u32x4 out[EPL / 16];
#pragma unroll
    for (int c = 0; c < EPL / 16; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float *v4 = &y[ps][16 * c + 4 * w];
        out[c][w] = static_cast<uint32_t>(cvt_fp8x4(v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv));
      }
    if (row < n) {
#pragma unroll
      for (int c = 0; c < EPL / 16; ++c)
        *reinterpret_cast<u32x4 *>(codes + head + static_cast<size_t>(row) * D + part * EPL + 16 * c) = out[c];
    }
  }
}

// ---- attention -------------------------------------------------------------------

struct Fp8Params {
  const uint8_t *q, *k, *v;
  const int *qe, *ke, *ve;  // block exponents
  void *o;
  float *lse;
  int n;
  int n_qblocks;  // ceil(n / 128)
  int n_tiles;    // ceil(n / 64)
  int total;      // bh * n_qblocks (grid size)
  float c;        // scale * log2(e); the caller divides scale by d when Q
                  // and K were rotated
};

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 operands (format 0), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f,
                                                          0, 0x7f7f7f7f);
}

// LDS tiles of 64 rows x D bytes, 16-byte chunks XOR-permuted by row:
//   K (row reads, 16 lanes = 16 rows per phase): chunk ^ kswz(row);
//   V (8-bit transposed reads, 8 rows x 2 chunks per 32 lanes): chunk ^ vswz(row).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)) : (2 * ((r >> 3) & 1));
}

template <int D>
struct Fp8Cfg {
  static constexpr int CPR = D / 16;            // 16-byte chunks per row
  static constexpr int TILE_BYTES = kTile * D;  // 8 KB at d = 128
  static constexpr int LOADS = TILE_BYTES / 1024 / 4;  // 1 KB loads per wave
  static constexpr int STEPS = D / 64;          // MFMA k-steps for S
  static constexpr int NCT = D / 32;            // 32-column blocks of O
};

template <int D>
__device__ __forceinline__ void issue_tile8(const uint8_t *base, int head_bytes,
                                            int tile_byte, char *buf, int wv,
                                            bool vlayout) {
  using C = Fp8Cfg<D>;
  const u32x4 rs = tile_desc(base, head_bytes, tile_byte);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) {
    const int piece = wv * C::LOADS + it;           // 1 KB piece of the tile
    const int row = piece * (64 / C::CPR) + lane / C::CPR;
    const int pos = lane % C::CPR;
    const int chunk = pos ^ (vlayout ? vswz<D>(row) : kswz<D>(row));
    dma16(rs, row * D + chunk * 16, 0, lds_addr(buf + piece * 1024));
  }
}

template <int D, bool CAUSAL, bool O32>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(Fp8Params p) {
  using C = Fp8Cfg<D>;
  // [K 0][K 1][V 0][V 1], 64 rows x D bytes each
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE_BYTES];
  auto kbuf = [&](int i) { return smem + i * C::TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * C::TILE_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, p.total);
  const int bh = logical / p.n_qblocks;
  const int qbl = logical - bh * p.n_qblocks;
  const int qb = CAUSAL ? (p.n_qblocks - 1 - qbl) : qbl;
  const int N = p.n;
  const size_t head = static_cast<size_t>(bh) * N * D;  // elements (= code bytes)
  const int head_bytes = N * D;
  const int q0 = qb * kRows;
  const int qw = q0 + 32 * wv;
  const int qi = qw + lr;

  // block exponents: Q's for this block, K's and V's per tile; the head's
  // largest V exponent is the reference of the exact per-tile shifts
  const int eq = p.qe[static_cast<size_t>(bh) * p.n_qblocks + qb];
  const int *kex = p.ke + static_cast<size_t>(bh) * p.n_tiles;
  const int *vex = p.ve + static_cast<size_t>(bh) * p.n_tiles;
  int em = -100000;
  for (int i = lane; i < p.n_tiles; i += 64) em = max(em, vex[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) em = max(em, __shfl_xor(em, m, 64));
  em = __builtin_amdgcn_readfirstlane(em);

  // Q: B operand of S^T = K Q^T, bytes 64 step + 32 hh .. +31 of row qi
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.q + head), 0, head_bytes, kBufWord3);
  // a negative scale is taken exactly as -|scale| on negated q (e4m3 sign
  // bits), so that the row maximum of the scores is the maximum of the
  // logits
  float cq = p.c;
  uint32_t qflip = 0;
  if (cq < 0.f) {
    cq = -cq;
    qflip = 0x80808080u;
  }
  i32x8 qreg[C::STEPS];
#pragma unroll
  for (int st = 0; st < C::STEPS; ++st) {
    const int off = qi * D + 64 * st + 32 * hh;
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0) ^ qflip;
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0) ^ qflip;
    qreg[st] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // K row reads: row lr (+32 kt), chunks 4 step + 2 hh + {0, 1}
  int krd[C::STEPS][2];
#pragma unroll
  for (int st = 0; st < C::STEPS; ++st)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      krd[st][h2] = lr * D + (((4 * st + 2 * hh + h2) ^ kswz<D>(lr)) * 16);
  // V transposed reads (8-bit): within a 16-lane group g, lane s addresses
  // row 4hh + (s/2)%4 + 8(s/8) (+16 per read) and the 8 bytes at column
  // 32ct + 16(g&1) + 8(s&1); lane L then holds column 32ct + L of rows
  // 4hh + e%4 + 8(e/4), e = 0..7 -- the key order of the P operand
  int vrd[C::NCT];
  {
    const int g = lane >> 4, s = lane & 15;
    const int row = 4 * hh + ((s >> 1) & 3) + 8 * (s >> 3);
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
      vrd[ct] = row * D + (((2 * ct + (g & 1)) ^ vswz<D>(row)) * 16) + 8 * (s & 1);
  }

  // The running reference starts at the lowest finite float instead of
  // -inf: every finite logit exceeds it by more than the rescale threshold,
  // so a lane's first visible key raises it, and neither m_run - shift nor
  // m_run - m_new can form inf - inf (no selects on the tile path).
  float m_run = -FLT_MAX, l_run = 0.f;
  f32x16 oacc[C::NCT];
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[ct][r] = 0.f;

  const int kend = CAUSAL ? min(N, q0 + kRows) : N;
  const int ntiles = (kend + kTile - 1) / kTile;
  int n_full = CAUSAL ? (q0 + 1) / kTile : N / kTile;
  if (n_full > ntiles) n_full = ntiles;
  const int w_tiles = CAUSAL ? min(ntiles, (qw + 31) / kTile + 1) : ntiles;

  if (N % kTile != 0) {
    for (int i = tid; i < 4 * C::TILE_BYTES / 16; i += kThreads)
      reinterpret_cast<u32x4 *>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  issue_tile8<D>(p.k + head, head_bytes, 0, kbuf(0), wv, false);
  issue_tile8<D>(p.v + head, head_bytes, 0, vbuf(0), wv, true);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // one tile; MASKED (diagonal or ragged tiles) is a compile-time switch so
  // that the unmasked tiles carry no mask or select instructions
  // ct_c: this tile's scores -> base-2 logits; ishift (<= 0): its V
  // exponent relative to the head's largest
  auto tile = [&](auto masked_tag, int t, const char *kb, const char *vb,
                  float ct_c, int ishift) {
    constexpr bool masked = decltype(masked_tag)::value;
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int st = 0; st < C::STEPS; ++st) {
        const u32x4 lo = lds_load<u32x4>(kb, krd[st][0] + kt * 32 * D);
        const u32x4 hi = lds_load<u32x4>(kb, krd[st][1] + kt * 32 * D);
        const i32x8 a = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kt] = mfma_fp8(a, qreg[st], s[kt]);
      }
    }
    // register r of sub-tile kt holds key 64t + 32kt + 8(r/4) + 4hh + r%4
    if (masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * kTile + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    float mlo, mhi;
    halves(mx, mlo, mhi);
    mx = fmaxf(mlo, mhi);
    const float m_tile = (masked && mx == -INFINITY) ? -INFINITY : mx * ct_c;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ct][r] *= alpha;
    }
    const float mu = m_run - static_cast<float>(ishift);
    float x[2][16];
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = fast_exp2(__builtin_fmaf(s[kt][r], ct_c, -mu));
        if (masked) v = s[kt][r] == -INFINITY ? 0.f : v;
        x[kt][r] = v;
        rs += v;
      }
    l_run += ldexpf(rs, -ishift);  // P = P' 2^-shift
    // P' (<= 2^8) as e4m3, key order 32kt + 8a + 4hh + b -> byte 16kt + 4a + b
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kt = w >> 2, r0 = 4 * (w & 3);
      pb[w] = cvt_fp8x4(x[kt][r0], x[kt][r0 + 1], x[kt][r0 + 2], x[kt][r0 + 3]);
    }
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      i32x2 r4[4];
#pragma unroll
      for (int rd = 0; rd < 4; ++rd)
        r4[rd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2 *)(vb + vrd[ct] + rd * 16 * D));
      const i32x8 a = i32x8{r4[0][0], r4[0][1], r4[1][0], r4[1][1],
                            r4[2][0], r4[2][1], r4[3][0], r4[3][1]};
      oacc[ct] = mfma_fp8(a, pb, oacc[ct]);
    }
  };

  // tile t + 1 into the other buffers, and its exponents (loaded with the
  // tile so that they have arrived by the barrier that publishes it; a
  // later load would make the in-order counter wait for the prefetch too)
  int ek_n = ntiles > 0 ? kex[0] : 0, ev_n = ntiles > 0 ? vex[0] : 0;
  // the tile constants are formed after the barrier, once the exponents are
  // known to have arrived
  auto consts = [&](float &ct_c, int &ishift) {
    ct_c = ldexpf(cq, eq + ek_n);
    ishift = ev_n - em;
  };
  float ct_c = 0.f;
  int shift = 0;
  auto prefetch = [&](int t) {
    if (t + 1 < ntiles) {
      const int nb = (t + 1) & 1;
      issue_tile8<D>(p.k + head, head_bytes, (t + 1) * kTile * D, kbuf(nb), wv, false);
      issue_tile8<D>(p.v + head, head_bytes, (t + 1) * kTile * D, vbuf(nb), wv, true);
      ek_n = kex[t + 1];
      ev_n = vex[t + 1];
    }
  };
  // unmasked tiles (every wave needs them), then the diagonal / ragged ones
  // The empty asm uses the exponents right after each barrier: any wait the
  // compiler adds for them lands there (where the counter is already zero)
  // and not after the next prefetch, which volatile asm cannot pass.
  auto arrived = [&]() { asm volatile("" : : "v"(ek_n), "v"(ev_n)); };
  arrived();
  int t = 0;
  for (; t < n_full; ++t) {
    consts(ct_c, shift);
    prefetch(t);
    tile(std::false_type{}, t, kbuf(t & 1), vbuf(t & 1), ct_c, shift);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    arrived();
  }
  for (; t < ntiles; ++t) {
    consts(ct_c, shift);
    prefetch(t);
    if (t < w_tiles) tile(std::true_type{}, t, kbuf(t & 1), vbuf(t & 1), ct_c, shift);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    arrived();
  }

  float llo, lhi;
  halves(l_run, llo, lhi);
  const float l_tot = llo + lhi;
  // O~ = 2^-em sum_t P_t V_t
  const float inv = l_tot > 0.f ? ldexpf(1.f, em) / l_tot : 0.f;
  if (qi < N) {
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = 32 * ct + 8 * a + 4 * hh;
        const size_t o_off = head + static_cast<size_t>(qi) * D + col;
        if (O32) {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = oacc[ct][4 * a + e] * inv;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + o_off) = ov;
        } else {
          __bf16 ob[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[e] = static_cast<__bf16>(oacc[ct][4 * a + e] * inv);
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.o) + o_off) =
              __builtin_bit_cast(u32x2, ob);
        }
      }
    if (p.lse && hh == 0)
      p.lse[static_cast<size_t>(bh) * N + qi] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int R>
hipError_t launch_q(const QuantArgs &a, hipStream_t s) {
  const int nb = (a.n + R - 1) / R;
  hipLaunchKernelGGL((quantize_kernel<D, R>), dim3(a.bh * nb), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(a.x), static_cast<uint8_t *>(a.codes),
                     a.exps, a.signs, a.n, nb);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool O32>
hipError_t launch_f(const Fp8Params &prm, hipStream_t s) {
  unsigned pad = 0;
  const hipError_t e =
      debug_lds_pad(reinterpret_cast<const void *>(&fwd_fp8_kernel<D, CAUSAL, O32>), &pad);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, O32>), dim3(prm.total), dim3(kThreads), pad,
                     s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fd(const Fp8Params &prm, bool causal, bool o32, hipStream_t s) {
  if (causal) return o32 ? launch_f<D, true, true>(prm, s) : launch_f<D, true, false>(prm, s);
  return o32 ? launch_f<D, false, true>(prm, s) : launch_f<D, false, false>(prm, s);
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantArgs &a, hipStream_t s) {
  if (a.d == 128) return a.block_rows == 128 ? launch_q<128, 128>(a, s) : launch_q<128, 64>(a, s);
  return a.block_rows == 128 ? launch_q<64, 128>(a, s) : launch_q<64, 64>(a, s);
}

hipError_t launch_fwd_fp8(const Fp8Args &a, bool o32, hipStream_t s) {
  Fp8Params prm;
  prm.q = static_cast<const uint8_t *>(a.q);
  prm.k = static_cast<const uint8_t *>(a.k);
  prm.v = static_cast<const uint8_t *>(a.v);
  prm.qe = a.qe;
  prm.ke = a.ke;
  prm.ve = a.ve;
  prm.o = a.o;
  prm.lse = a.lse;
  prm.n = a.n;
  prm.n_qblocks = (a.n + kRows - 1) / kRows;
  prm.n_tiles = (a.n + kTile - 1) / kTile;
  prm.total = a.bh * prm.n_qblocks;
  prm.c = a.scale * kLog2e;
  if (a.d == 128) return launch_fd<128>(prm, a.causal, o32, s);
  return launch_fd<64>(prm, a.causal, o32, s);
}

}  // namespace fa2
