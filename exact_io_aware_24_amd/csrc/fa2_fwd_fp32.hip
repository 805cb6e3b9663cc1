// Exact attention forward in fp32 arithmetic throughout (fp32 q, k, v, o).
//
// This path exists for exactness checks on small problems, where bf16
// rounding of the inputs or of the probabilities would hide errors; it is not
// tuned for throughput.  The algorithm is the same tiled online softmax as
// the bf16 MFMA path: query blocks outside, K/V tiles inside (itimpress.au
// page "FlashAttention scaling, multi-GPU training and weight quantisation",
// section 1), the running max / sum / unnormalised output merged tile by tile
// with the two-block rule of section 2 of the shakilmahmud.com page "Large
// language models part 06: FlashAttention -- GPU SRAM, tiling, online
// softmax", and one division by the sum at the end.
//
// Layout: one wave64 per 64 query rows, one query row per lane (q and the
// output accumulator in registers); K and V tiles of 32 keys are staged in
// LDS and read as broadcasts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

constexpr int kThreads = 64;
constexpr int kRows = kFp32RowsPerBlock;  // 64
constexpr int kTile = 32;                 // keys per LDS tile
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

struct Params {
  const float *q, *k, *v;
  float *o;
  float *lse;
  int n;
  int n_qblocks;
  float c;  // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(Params p) {
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / p.n_qblocks;
  const int qb = blockIdx.x - bh * p.n_qblocks;
  const int N = p.n;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int q0 = qb * kRows;
  const int qi = q0 + tid;

  float c = p.c;
  float qsign = 1.f;
  if (c < 0.f) {  // exact: negate q and use -c
    c = -c;
    qsign = -1.f;
  }
  float qv[D], ov[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = (qi < N) ? qsign * p.q[head + static_cast<size_t>(qi) * D + x] : 0.f;
    ov[x] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(N, q0 + kRows) : N;
  for (int j0 = 0; j0 < kend; j0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kThreads) {
      const int r = idx / D, x = idx % D;
      const bool ok = j0 + r < N;
      const size_t g = head + static_cast<size_t>(j0 + r) * D + x;
      Ks[r][x] = ok ? p.k[g] : 0.f;
      Vs[r][x] = ok ? p.v[g] : 0.f;
    }
    __syncthreads();

    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) acc = __builtin_fmaf(qv[x], Ks[j][x], acc);
      const int key = j0 + j;
      const bool masked = key >= N || (CAUSAL && key > qi);
      s[j] = masked ? -INFINITY : acc;
      mx = fmaxf(mx, s[j]);
    }
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_run, m_tile);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      s[j] = (s[j] == -INFINITY) ? 0.f : exp2f(__builtin_fmaf(s[j], c, -m_use));
      rs += s[j];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int x = 0; x < D; ++x) {
      float acc = ov[x] * alpha;
#pragma unroll
      for (int j = 0; j < kTile; ++j) acc = __builtin_fmaf(s[j], Vs[j][x], acc);
      ov[x] = acc;
    }
  }

  if (qi < N) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int x = 0; x < D; ++x)
      p.o[head + static_cast<size_t>(qi) * D + x] = ov[x] * inv;
    if (p.lse)
      p.lse[static_cast<size_t>(bh) * N + qi] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Params &prm, int grid, hipStream_t s) {
  unsigned pad = 0;
  const hipError_t e =
      debug_lds_pad(reinterpret_cast<const void *>(&fwd_fp32_kernel<D, CAUSAL>), &pad);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads),
                     pad, s, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdArgs &a, hipStream_t s) {
  Params prm;
  prm.q = static_cast<const float *>(a.q);
  prm.k = static_cast<const float *>(a.k);
  prm.v = static_cast<const float *>(a.v);
  prm.o = static_cast<float *>(a.o);
  prm.lse = a.lse;
  prm.n = a.nq;  // the fp32 path has equal query and key lengths
  prm.n_qblocks = (a.nq + kRows - 1) / kRows;
  prm.c = a.scale * kLog2e;
  const int grid = a.bh * prm.n_qblocks;
  if (a.d == 128)
    return a.causal ? launch<128, true>(prm, grid, s) : launch<128, false>(prm, grid, s);
  return a.causal ? launch<64, true>(prm, grid, s) : launch<64, false>(prm, grid, s);
}

}  // namespace fa2
