// C-ABI entry points: argument validation (pure host code, before any HIP
// call) and dispatch to the kernel launchers.  The declarations and the full
// contract are in include/fa2.h.
#include "fa2.h"

#include <cmath>
#include <cstdint>

#include "fa2_internal.h"

static_assert(fa2::kFwdScratchBytes == FA2_NOALLOC_WORKSPACE_BYTES,
              "the header states the static workspace size");

#define FA2_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range span(const void *p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool misaligned(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) != 0;
}

// Shared validation of every entry point.  in_bytes / out_bytes are the
// element sizes of q/k/v and of o; rows_per_block is the kernel's query-block
// height (bounds the grid size); max_per_head bounds N*d (the bf16 kernel
// addresses one head with 32-bit byte offsets, including one tile of reads
// past the end that the hardware bounds check turns into zeros).
int validate(const void *q, const void *k, const void *v, const void *o,
             const float *lse, int B, int H, int H_kv, int Nq, int Nk, int d,
             float scale, int in_bytes, int out_bytes, int rows_per_block,
             int64_t max_per_head) {
  if (!q || !k || !v || !o) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || H_kv < 1 || H % H_kv != 0)
    return FA2_ERR_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEADDIM;
  const int64_t bh = static_cast<int64_t>(B) * H;  // < 2^62: no overflow
  const int64_t q_head = static_cast<int64_t>(Nq) * d;
  const int64_t kv_head = static_cast<int64_t>(Nk) * d;
  // bounded factors first, so that no product below can overflow int64
  if (bh > INT32_MAX || q_head > max_per_head || kv_head > max_per_head)
    return FA2_ERR_SHAPE;
  const int64_t blocks = bh * ((static_cast<int64_t>(Nq) + rows_per_block - 1) /
                               rows_per_block);
  if (blocks > INT32_MAX || bh * q_head > FA2_MAX_ELEMS || bh * kv_head > FA2_MAX_ELEMS)
    return FA2_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA2_ERR_SCALE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      (lse && misaligned(lse)))
    return FA2_ERR_ALIGN;
  const int64_t elems = bh * q_head;
  const int64_t kv_elems = static_cast<int64_t>(B) * H_kv * kv_head;
  const Range rq = span(q, elems * in_bytes), rk = span(k, kv_elems * in_bytes),
              rv = span(v, kv_elems * in_bytes), ro = span(o, elems * out_bytes);
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv))
    return FA2_ERR_ALIAS;
  if (lse) {
    const Range rl = span(lse, bh * Nq * static_cast<int64_t>(sizeof(float)));
    if (overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv) ||
        overlaps(rl, ro))
      return FA2_ERR_ALIAS;
  }
  return FA2_OK;
}

fa2::FwdArgs make_args(const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int H, int H_kv, int Nq, int Nk,
                       int d, float scale, int causal) {
  fa2::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.h = H;
  a.group = H / H_kv;
  a.nq = Nq;
  a.nk = Nk;
  a.n_splits = 1;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  return a;
}

// Few queries per head and shared K/V heads (decoding with grouped-query
// attention): the query heads of one K/V head are consecutive in q, o and
// lse, so their rows form one [group * Nq, d] matrix against that K/V head.
// Launched that way, one workgroup takes the rows of a whole group and
// streams the K/V head once per key range instead of once per query head.
// Each row's result is the same computation (rows only move between lanes
// and waves).  Used where every packed row sees the same keys: without a
// mask, or with one query per head, which sees every key when causal.  The
// packed head must still fit the kernel's 32-bit per-head byte offsets (the
// bound validate() applies to one head): with tens of thousands of query
// heads per K/V head it would not, and such calls run unpacked.
void pack_query_heads(fa2::FwdArgs &a) {
  if (a.group == 1 || a.nq >= fa2::kBf16RowsPerBlock || (a.causal && a.nq != 1)) return;
  if (static_cast<int64_t>(a.group) * a.nq * a.d > FA2_MAX_HEAD_ELEMS_BF16) return;
  a.bh /= a.group;
  a.h /= a.group;
  a.nq *= a.group;
  a.group = 1;
  a.causal = false;  // one query per head sees every key
}

// Validation of the backward entry points: every pointer is required (the
// partial-sum workspace only when n_gsplits > 1); the outputs (dq, dk, dv,
// the delta workspace and the partial-sum workspace) may overlap neither an
// input nor each other.
int validate_bwd(const void *q, const void *k, const void *v, const void *o,
                 const void *dout, const float *lse, const float *delta,
                 const void *dq, const void *dk, const void *dv, int B, int H,
                 int H_kv, int N, int d, float scale, int out_bytes,
                 int n_gsplits, const float *dkv_part) {
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv)
    return FA2_ERR_NULL;
  // shape, head dimension, size limits and scale as for the forward
  int rc = validate(q, k, v, o, nullptr, B, H, H_kv, N, N, d, scale, 2, 2,
                    fa2::kBf16BwdRowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc != FA2_OK && rc != FA2_ERR_ALIAS) return rc;
  if (n_gsplits < 1 || n_gsplits > H / H_kv) return FA2_ERR_SHAPE;
  if (n_gsplits > 1 && !dkv_part) return FA2_ERR_NULL;
  if (misaligned(dout) || misaligned(lse) || misaligned(delta) ||
      misaligned(dq) || misaligned(dk) || misaligned(dv) ||
      (n_gsplits > 1 && misaligned(dkv_part)))
    return FA2_ERR_ALIGN;
  const int64_t elems = static_cast<int64_t>(B) * H * N * d;
  const int64_t kv_elems = static_cast<int64_t>(B) * H_kv * N * d;
  const int64_t rows = static_cast<int64_t>(B) * H * N;
  const Range in[6] = {span(q, elems * 2),    span(k, kv_elems * 2),
                       span(v, kv_elems * 2), span(o, elems * 2),
                       span(dout, elems * 2), span(lse, rows * 4)};
  const Range out[5] = {
      span(dq, elems * out_bytes), span(dk, kv_elems * out_bytes),
      span(dv, kv_elems * out_bytes), span(delta, rows * 4),
      span(dkv_part, n_gsplits > 1 ? 2 * n_gsplits * kv_elems * 4 : 0)};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return FA2_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(out[i], out[j])) return FA2_ERR_ALIAS;
  }
  return FA2_OK;
}

fa2::BwdArgs make_bwd_args(const void *q, const void *k, const void *v,
                           const void *o, const void *dout, const float *lse,
                           float *delta, void *dq, void *dk, void *dv, int B,
                           int H, int H_kv, int N, int d, float scale,
                           int causal, int n_gsplits, float *dkv_part) {
  fa2::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.bh = B * H;
  a.h = H;
  a.group = H / H_kv;
  a.n_gsplits = n_gsplits;
  a.dkv_part = n_gsplits > 1 ? dkv_part : nullptr;
  a.n = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  return a;
}

int finish(hipError_t e) { return e == hipSuccess ? FA2_OK : FA2_ERR_HIP; }

// A stream, when given, must belong to the current device: the kernels run
// on the stream's device and address the caller's buffers (and, for the
// allocation-free entry point, the static array) of the current one.
int check_stream(void *stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // the null stream and HIP's implicit default streams are the current device's
  if (st == nullptr || st == hipStreamLegacy || st == hipStreamPerThread) return FA2_OK;
  int cur = -1;
  hipDevice_t sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return FA2_ERR_HIP;
  if (hipStreamGetDevice(st, &sdev) != hipSuccess) return FA2_ERR_HIP;
  return sdev == cur ? FA2_OK : FA2_ERR_DEVICE;
}

}  // namespace

FA2_EXPORT int fa2_fwd(const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int H, int N, int d, float scale,
                       int causal, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H, N, N, d, scale, 2, 2,
                    fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  return finish(fa2::launch_fwd_bf16(
      make_args(q, k, v, o, lse, B, H, H, N, N, d, scale, causal), false,
      static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_fwd_gqa(const void *q, const void *k, const void *v,
                           void *o, float *lse, int B, int H, int H_kv, int N,
                           int d, float scale, int causal, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H_kv, N, N, d, scale, 2, 2,
                    fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  fa2::FwdArgs a = make_args(q, k, v, o, lse, B, H, H_kv, N, N, d, scale, causal);
  pack_query_heads(a);
  return finish(fa2::launch_fwd_bf16(a, false, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_fwd_gqa_o32(const void *q, const void *k, const void *v,
                               float *o, float *lse, int B, int H, int H_kv,
                               int N, int d, float scale, int causal,
                               void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H_kv, N, N, d, scale, 2, 4,
                    fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  fa2::FwdArgs a = make_args(q, k, v, o, lse, B, H, H_kv, N, N, d, scale, causal);
  pack_query_heads(a);
  return finish(fa2::launch_fwd_bf16(a, true, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_fwd_o32(const void *q, const void *k, const void *v,
                           float *o, float *lse, int B, int H, int N, int d,
                           float scale, int causal, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H, N, N, d, scale, 2, 4,
                    fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  return finish(fa2::launch_fwd_bf16(
      make_args(q, k, v, o, lse, B, H, H, N, N, d, scale, causal), true,
      static_cast<hipStream_t>(stream)));
}

// Key ranges of one query block computed by separate workgroups, then
// merged: the same kernel with a key range per workgroup writing fp32
// partial (O, lse), and a merge kernel.  n_splits == 1 is a plain call.
static int splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int H_kv, int Nq, int Nk, int d, float scale,
            int causal, int n_splits, float *o_part, float *lse_part,
            bool o32, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, 2,
                    o32 ? 4 : 2, fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc != FA2_OK) return rc;
  if (n_splits < 1 || n_splits > FA2_MAX_SPLITS) return FA2_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t blocks = bh * ((static_cast<int64_t>(Nq) + fa2::kBf16RowsPerBlock - 1) /
                               fa2::kBf16RowsPerBlock);
  if (blocks * n_splits > INT32_MAX) return FA2_ERR_SHAPE;
  if (n_splits > 1) {
    if (!o_part || !lse_part) return FA2_ERR_NULL;
    if (misaligned(o_part) || misaligned(lse_part)) return FA2_ERR_ALIGN;
    const int64_t rows = bh * Nq;
    const int64_t kv = static_cast<int64_t>(B) * H_kv * Nk * d * 2;
    const Range parts[2] = {span(o_part, n_splits * rows * d * 4),
                            span(lse_part, n_splits * rows * 4)};
    const Range others[5] = {span(q, rows * d * 2), span(k, kv), span(v, kv),
                             span(o, rows * d * (o32 ? 4 : 2)),
                             span(lse ? lse : o_part, lse ? rows * 4 : 0)};
    if (overlaps(parts[0], parts[1])) return FA2_ERR_ALIAS;
    for (const Range &p : parts)
      for (const Range &x : others)
        if (overlaps(p, x)) return FA2_ERR_ALIAS;
  }
  rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  fa2::FwdArgs a = make_args(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal);
  a.n_splits = n_splits;
  a.o_part = o_part;
  a.lse_part = lse_part;
  pack_query_heads(a);
  return finish(fa2::launch_fwd_bf16(a, o32, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_fwd_splitkv(const void *q, const void *k, const void *v,
                               void *o, float *lse, int B, int H, int H_kv,
                               int Nq, int Nk, int d, float scale, int causal,
                               int n_splits, float *o_part, float *lse_part,
                               void *stream) {
  return splitkv(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal,
                 n_splits, o_part, lse_part, false, stream);
}

FA2_EXPORT int fa2_fwd_splitkv_o32(const void *q, const void *k, const void *v,
                                   float *o, float *lse, int B, int H, int H_kv,
                                   int Nq, int Nk, int d, float scale,
                                   int causal, int n_splits, float *o_part,
                                   float *lse_part, void *stream) {
  return splitkv(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal,
                 n_splits, o_part, lse_part, true, stream);
}

// fa2_fwd_splitkv with the partial (O, lse) of the key ranges in the
// library's static per-device workspace instead of caller memory: no
// allocation anywhere on this path.  Every element of the partials that the
// merge reads is written by the range kernel of the same call first, so the
// workspace needs no clearing (it keeps the previous call's values).
FA2_EXPORT int fa2_fwd_splitkv_noalloc(const void *q, const void *k,
                                       const void *v, void *o, float *lse,
                                       int B, int H, int H_kv, int Nq, int Nk,
                                       int d, float scale, int causal,
                                       int n_splits, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, 2, 2,
                    fa2::kBf16RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc != FA2_OK) return rc;
  if (n_splits < 1 || n_splits > FA2_MAX_SPLITS) return FA2_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t blocks = bh * ((static_cast<int64_t>(Nq) + fa2::kBf16RowsPerBlock - 1) /
                               fa2::kBf16RowsPerBlock);
  if (blocks * n_splits > INT32_MAX) return FA2_ERR_SHAPE;
  // [n_splits][B*H][Nq][d] fp32 partial outputs, then [n_splits][B*H][Nq]
  // fp32 partial lse (the first part is a multiple of 256 bytes: d >= 64)
  const int64_t o_floats = static_cast<int64_t>(n_splits) * bh * Nq * d;
  const int64_t l_floats = static_cast<int64_t>(n_splits) * bh * Nq;
  if (n_splits > 1 &&
      (o_floats + l_floats) * 4 > static_cast<int64_t>(FA2_NOALLOC_WORKSPACE_BYTES))
    return FA2_ERR_WORKSPACE;
  rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  fa2::FwdArgs a = make_args(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal);
  a.n_splits = n_splits;
  pack_query_heads(a);
  if (n_splits > 1) {
    float *ws = nullptr;
    if (fa2::fwd_scratch(&ws) != hipSuccess) return FA2_ERR_HIP;
    a.o_part = ws;
    a.lse_part = ws + o_floats;
  }
  return finish(fa2::launch_fwd_bf16(a, false, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_quantize_fp8(const void *x, void *codes, int *exps, int B,
                                int H, int N, int d, int block_rows,
                                const float *signs, void *stream) {
  if (!x || !codes || !exps) return FA2_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || (block_rows != 64 && block_rows != 128))
    return FA2_ERR_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEADDIM;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t nb = (static_cast<int64_t>(N) + block_rows - 1) / block_rows;
  if (bh > INT32_MAX || bh * nb > INT32_MAX || bh * N * d > FA2_MAX_ELEMS)
    return FA2_ERR_SHAPE;
  if (misaligned(x) || misaligned(codes) || (reinterpret_cast<uintptr_t>(exps) & 3) ||
      (signs && (reinterpret_cast<uintptr_t>(signs) & 3)))
    return FA2_ERR_ALIGN;
  const int64_t elems = bh * N * d;
  const Range rx = span(x, elems * 2), rc = span(codes, elems),
              re = span(exps, bh * nb * 4), rs = span(signs, signs ? d * 4 : 0);
  if (overlaps(rc, rx) || overlaps(rc, re) || overlaps(rc, rs) ||
      overlaps(re, rx) || overlaps(re, rs))
    return FA2_ERR_ALIAS;
  const int rc_stream = check_stream(stream);
  if (rc_stream != FA2_OK) return rc_stream;
  fa2::QuantArgs a;
  a.x = x;
  a.codes = codes;
  a.exps = exps;
  a.signs = signs;
  a.bh = static_cast<int>(bh);
  a.n = N;
  a.d = d;
  a.block_rows = block_rows;
  return finish(fa2::launch_quantize_fp8(a, static_cast<hipStream_t>(stream)));
}

static int fwd_fp8(const void *q8, const int *qe, const void *k8, const int *ke,
                   const void *v8, const int *ve, void *o, float *lse, int B,
                   int H, int N, int d, float scale, int rotated, int causal,
                   bool o32, void *stream) {
  if (!qe || !ke || !ve) return FA2_ERR_NULL;
  // shapes, scale, alignment and aliasing of q, k, v, o, lse (1-byte codes)
  int rc = validate(q8, k8, v8, o, lse, B, H, H, N, N, d, scale, 1, o32 ? 4 : 2,
                    fa2::kFp8RowsPerBlock, FA2_MAX_HEAD_ELEMS_BF16);
  if (rc != FA2_OK) return rc;
  if ((reinterpret_cast<uintptr_t>(qe) | reinterpret_cast<uintptr_t>(ke) |
       reinterpret_cast<uintptr_t>(ve)) & 3)
    return FA2_ERR_ALIGN;
  const int64_t bh = static_cast<int64_t>(B) * H;
  const int64_t rows = bh * N;
  const Range out[2] = {span(o, rows * d * (o32 ? 4 : 2)), span(lse, lse ? rows * 4 : 0)};
  const Range ex[3] = {span(qe, bh * ((N + 127) / 128) * 4), span(ke, bh * ((N + 63) / 64) * 4),
                       span(ve, bh * ((N + 63) / 64) * 4)};
  for (const Range &r : out)
    for (const Range &e : ex)
      if (overlaps(r, e)) return FA2_ERR_ALIAS;
  rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  fa2::Fp8Args a;
  a.q = q8;
  a.k = k8;
  a.v = v8;
  a.qe = qe;
  a.ke = ke;
  a.ve = ve;
  a.o = o;
  a.lse = lse;
  a.bh = static_cast<int>(bh);
  a.n = N;
  a.d = d;
  a.scale = rotated ? scale / static_cast<float>(d) : scale;
  a.causal = causal != 0;
  return finish(fa2::launch_fwd_fp8(a, o32, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_fwd_fp8(const void *q8, const int *q_exp, const void *k8,
                           const int *k_exp, const void *v8, const int *v_exp,
                           void *o, float *lse, int B, int H, int N, int d,
                           float scale, int rotated, int causal, void *stream) {
  return fwd_fp8(q8, q_exp, k8, k_exp, v8, v_exp, o, lse, B, H, N, d, scale,
                 rotated, causal, false, stream);
}

FA2_EXPORT int fa2_fwd_fp8_o32(const void *q8, const int *q_exp, const void *k8,
                               const int *k_exp, const void *v8,
                               const int *v_exp, float *o, float *lse, int B,
                               int H, int N, int d, float scale, int rotated,
                               int causal, void *stream) {
  return fwd_fp8(q8, q_exp, k8, k_exp, v8, v_exp, o, lse, B, H, N, d, scale,
                 rotated, causal, true, stream);
}

FA2_EXPORT int fa2_fwd_fp32(const float *q, const float *k, const float *v,
                            float *o, float *lse, int B, int H, int N, int d,
                            float scale, int causal, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, H, N, N, d, scale, 4, 4,
                    fa2::kFp32RowsPerBlock, INT32_MAX);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  return finish(fa2::launch_fwd_fp32(
      make_args(q, k, v, o, lse, B, H, H, N, N, d, scale, causal),
      static_cast<hipStream_t>(stream)));
}

static int bwd(const void *q, const void *k, const void *v, const void *o,
               const void *dout, const float *lse, float *delta, void *dq,
               void *dk, void *dv, int B, int H, int H_kv, int N, int d,
               float scale, int causal, int n_gsplits, float *dkv_part,
               bool o32, void *stream) {
  int rc = validate_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv,
                        N, d, scale, o32 ? 4 : 2, n_gsplits, dkv_part);
  if (rc == FA2_OK) rc = check_stream(stream);
  if (rc != FA2_OK) return rc;
  return finish(fa2::launch_bwd_bf16(
      make_bwd_args(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d,
                    scale, causal, n_gsplits, dkv_part),
      o32, static_cast<hipStream_t>(stream)));
}

FA2_EXPORT int fa2_bwd(const void *q, const void *k, const void *v,
                       const void *o, const void *dout, const float *lse,
                       float *delta, void *dq, void *dk, void *dv, int B, int H,
                       int N, int d, float scale, int causal, void *stream) {
  return bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H, N, d, scale,
             causal, 1, nullptr, false, stream);
}

FA2_EXPORT int fa2_bwd_o32(const void *q, const void *k, const void *v,
                           const void *o, const void *dout, const float *lse,
                           float *delta, float *dq, float *dk, float *dv, int B,
                           int H, int N, int d, float scale, int causal,
                           void *stream) {
  return bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H, N, d, scale,
             causal, 1, nullptr, true, stream);
}

FA2_EXPORT int fa2_bwd_gqa(const void *q, const void *k, const void *v,
                           const void *o, const void *dout, const float *lse,
                           float *delta, void *dq, void *dk, void *dv, int B,
                           int H, int H_kv, int N, int d, float scale,
                           int causal, int n_gsplits, float *dkv_part,
                           void *stream) {
  return bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale,
             causal, n_gsplits, dkv_part, false, stream);
}

FA2_EXPORT int fa2_bwd_gqa_o32(const void *q, const void *k, const void *v,
                               const void *o, const void *dout,
                               const float *lse, float *delta, float *dq,
                               float *dk, float *dv, int B, int H, int H_kv,
                               int N, int d, float scale, int causal,
                               int n_gsplits, float *dkv_part, void *stream) {
  return bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, scale,
             causal, n_gsplits, dkv_part, true, stream);
}

FA2_EXPORT const char *fa2_strerror(int code) {
  switch (code) {
    case FA2_OK: return "success";
    case FA2_ERR_NULL: return "a required pointer is NULL";
    case FA2_ERR_SHAPE:
      return "invalid shape: B, H, N >= 1, H_kv >= 1 dividing H, and the "
             "tensors within the supported size";
    case FA2_ERR_HEADDIM: return "unsupported head dimension (must be 64 or 128)";
    case FA2_ERR_SCALE: return "scale is not finite";
    case FA2_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA2_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA2_ERR_HIP: return "HIP kernel launch failed";
    case FA2_ERR_DEVICE:
      return "the stream belongs to another device than the current HIP device";
    case FA2_ERR_WORKSPACE:
      return "the key-range partials exceed the library's static workspace "
             "(FA2_NOALLOC_WORKSPACE_BYTES)";
    default: return "unknown fa2 error code";
  }
}

FA2_EXPORT int fa2_version(void) { return 8; }
