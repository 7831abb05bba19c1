// jas_api.cpp -- the C ABI of include/jas.h: host-side validation, launch
// geometry, dispatch.  Every check runs on the host before any HIP call; the
// library never allocates, frees or synchronizes.

#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "jas.h"
#include "jas_attn.h"
#include "jas_internal.h"

static_assert(JAS_MAX_KEYS == jas::kMaxStreamKeys, "the public row limit is the streaming kernels'");

namespace {

using jas::Geometry;

struct Dims {
  int64_t rows;     // batch*heads*q_rows
  int64_t span;     // elements from the first row's start to the last row's end
  int64_t esz;      // bytes per element
  int T;            // tiles per row
};

// A C caller may store any int in an enum-typed argument or field; reading
// a value outside the enumerators through the C++ enum type is undefined,
// so values are validated through their bytes.
template <typename E>
int enum_bits(const E &e) {
  static_assert(sizeof(E) == sizeof(int), "the C enums of jas.h are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_add_overflow(a, b, out); }

jas_status_t check_desc(const jas_desc_t *d, Dims *dims) {
  if (!d) return JAS_ERR_NULL_POINTER;
  const int dt = enum_bits(d->dtype);
  if (dt != JAS_DTYPE_F32 && dt != JAS_DTYPE_BF16 && dt != JAS_DTYPE_F16) return JAS_ERR_BAD_DTYPE;
  if (d->flags & ~(uint32_t)(JAS_FLAG_MASK | JAS_FLAG_SINK | JAS_FLAG_CAUSAL | JAS_FLAG_KEY_LEN |
                             JAS_FLAG_LSE))
    return JAS_ERR_BAD_FLAGS;
  if (d->batch < 0 || d->heads < 0 || d->q_rows < 0 || d->keys < 1 || d->ld < d->keys)
    return JAS_ERR_BAD_SHAPE;
  if (d->mask_stride_b < 0 || d->mask_stride_h < 0 || d->mask_stride_q < 0)
    return JAS_ERR_BAD_SHAPE;
  int64_t bh = 0, rows = 0, span = 0, bytes = 0;
  if (!mul_ok(d->batch, d->heads, &bh) || !mul_ok(bh, d->q_rows, &rows)) return JAS_ERR_BAD_SHAPE;
  const int64_t esz = d->dtype == JAS_DTYPE_F32 ? 4 : 2;
  if (rows > 0) {
    if (!mul_ok(rows - 1, d->ld, &span) || !add_ok(span, d->keys, &span) ||
        !mul_ok(span, esz, &bytes))
      return JAS_ERR_BAD_SHAPE;
  }
  if (d->keys > JAS_MAX_KEYS) return JAS_ERR_UNSUPPORTED;
  dims->rows = rows;
  dims->span = span;
  dims->esz = esz;
  dims->T = (int)((d->keys + jas::kTile - 1) / jas::kTile);
  return JAS_OK;
}

// Byte range [lo, hi) of a buffer.
struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void *p, int64_t bytes) {
  const uintptr_t a = (uintptr_t)p;
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Bytes of the mask touched by the shape: the largest addressed element + 1.
jas_status_t mask_bytes(const jas_desc_t *d, int64_t *bytes) {
  int64_t off = d->keys, t = 0;
  const int64_t dims[3] = {d->batch, d->heads, d->q_rows};
  const int64_t strides[3] = {d->mask_stride_b, d->mask_stride_h, d->mask_stride_q};
  for (int i = 0; i < 3; ++i) {
    if (!mul_ok(dims[i] - 1, strides[i], &t) || !add_ok(off, t, &off)) return JAS_ERR_BAD_SHAPE;
  }
  if (!mul_ok(off, 4, bytes)) return JAS_ERR_BAD_SHAPE;
  return JAS_OK;
}

// Rows of whole 16-byte chunks (row length and stride a multiple of the keys
// in a chunk): the shape allows the 16-byte path (the pointers' alignment
// decides the rest).
bool whole_chunk_rows(const jas_desc_t *d) {
  const int64_t kpc = jas::keys_per_chunk(d->dtype);
  return d->keys % kpc == 0 && d->ld % kpc == 0;
}

// What the forward's mask allows: none, a mask, or a mask broadcast over
// queries with no causal flag (consecutive rows of a batch entry and head
// then share one mask row and one visible length).
enum MaskKind { kNoMask = 0, kMask = 1, kSharedMask = 2 };

MaskKind mask_kind(const jas_desc_t *d) {
  if (!(d->flags & JAS_FLAG_MASK)) return kNoMask;
  return (d->mask_stride_q == 0 && !(d->flags & JAS_FLAG_CAUSAL)) ? kSharedMask : kMask;
}

// Rows from which the forward keeps a shared mask row in registers by
// default (then two rows per workgroup, and still 8,192 or more
// workgroups).
constexpr int64_t kMresMinRows = 16384;

// Rows from which the wide streaming backward takes two rows per workgroup
// by default (then still 1,024 or more workgroups, two rounds of the 512
// that fit).
constexpr int64_t kStreamTwoRowsMin = 2048;

// Launch geometry: the override when given (checked), else the default.
// tiles are covered by slots of TPS tiles; a row needs ceil(T/TPS) slots,
// spread over wpr waves holding cpl slots each.
jas_status_t choose_geometry(int dtype, int T, int64_t rows, bool backward, const jas_launch_t *ov,
                             Geometry *g, bool whole_chunks = true, MaskKind mk = kNoMask) {
  const int tps = jas::tiles_per_slot(dtype);
  const int nslots = (T + tps - 1) / tps;
  int ncpl = 0;
  const int *cpls = jas::compiled_cpls(dtype, &ncpl);
  int wpr = ov ? ov->waves_per_row : 0;
  int cpl = ov ? ov->chunks_per_lane : 0;
  int rpb = ov ? ov->rows_per_block : 0;
  int64_t cap = ov ? ov->max_blocks : 0;
  int mres = ov ? ov->mask_in_registers : 0;
  if (wpr < 0 || cpl < 0 || rpb < 0 || cap < 0) return JAS_ERR_UNSUPPORTED;
  if (ov && ov->streaming != 0 && ov->streaming != 1) return JAS_ERR_UNSUPPORTED;
  if (mres < 0 || mres > 2) return JAS_ERR_UNSUPPORTED;
  // a field other than mask_in_registers set: the default does not turn it on
  const bool geo_given = ov && (wpr || cpl || rpb || cap || ov->streaming);
  g->stream = 0;
  g->mres = 0;
  if (T > jas::kMaxTiles || (ov && ov->streaming)) {
    // streaming: one row per workgroup of 4 or 16 waves, the row in segments
    if ((wpr != 0 && wpr != jas::kBlockWaves && wpr != jas::kStreamWideWaves) || rpb > 1 ||
        mres == 1)
      return JAS_ERR_UNSUPPORTED;
    // rows that cannot take 16-byte accesses run the 4-wave workgroup
    if (wpr == 0) wpr = whole_chunks ? jas::default_stream_wpr(dtype, nslots, backward) : jas::kBlockWaves;
    if (cpl == 0) cpl = jas::default_stream_cpl(dtype);
    if (!jas::stream_cpl_compiled(dtype, cpl)) return JAS_ERR_UNSUPPORTED;
    // the wide workgroup is compiled for 16-bit types and the larger segment only
    if (wpr == jas::kStreamWideWaves && (dtype == JAS_DTYPE_F32 || cpl != jas::default_stream_cpl(dtype)))
      return JAS_ERR_UNSUPPORTED;
    int64_t blocks = rows;
    // the wide backward workgroup (66 KB of LDS, two per CU) runs faster
    // taking two rows each than starting a new workgroup per row (65,536-key
    // rows, 8,192 of them: 0.551-0.552 ms against 0.572-0.574)
    if (backward && wpr == jas::kStreamWideWaves && !geo_given && rows >= kStreamTwoRowsMin)
      blocks = (rows + 1) / 2;
    if (cap > 0 && blocks > cap) blocks = cap;
    if (blocks > 0x7fffffff) blocks = 0x7fffffff;
    g->wpr = wpr;
    g->cpl = cpl;
    g->rpb = 1;
    g->blocks = blocks;
    g->stream = 1;
    return JAS_OK;
  }
  if (mres == 1 && wpr == 0) wpr = 2;  // the mask in registers is built for two waves per row
  if (wpr == 0) {
    if (cpl) {
      for (int w : {1, 2, 4})
        if (cpl * w >= nslots) {
          wpr = w;
          break;
        }
    } else {
      wpr = jas::default_wpr(dtype, nslots, backward);
    }
    if (wpr == 0) return JAS_ERR_UNSUPPORTED;
  }
  if (cpl == 0) {
    const int need = (nslots + wpr - 1) / wpr;
    for (int i = 0; i < ncpl; ++i)
      if (cpls[i] >= need) {
        cpl = cpls[i];
        break;
      }
    if (cpl == 0) return JAS_ERR_UNSUPPORTED;
  }
  if (!jas::cpl_compiled(dtype, wpr, cpl) || (int64_t)wpr * cpl < nslots) return JAS_ERR_UNSUPPORTED;
  // the mask in registers: compiled for 16-bit rows on two waves with at
  // most 5 chunks per lane (more would cost a wave per SIMD); rows that
  // cannot take 16-byte accesses run the element-wise forward on the same
  // grid.  By default where consecutive rows share their mask row.
  const bool mres_ok = !backward && dtype != JAS_DTYPE_F32 && mk != kNoMask && wpr == 2 && cpl <= 5;
  if (mres == 1 && !mres_ok) return JAS_ERR_UNSUPPORTED;
  if (mres == 0)
    mres = (!geo_given && mres_ok && whole_chunks && mk == kSharedMask && rows >= kMresMinRows) ? 1 : 2;
  if (mres == 1) {  // one row per workgroup at a time, two rows per workgroup
    if (rpb == 0) rpb = 1;
    if (cap == 0) cap = (rows + 1) / 2;
  }
  if (rpb == 0) rpb = jas::default_rpb(dtype, nslots, wpr, backward);
  if (rpb < 1 || wpr * rpb > jas::kBlockWaves) return JAS_ERR_UNSUPPORTED;
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (cap > 0 && blocks > cap) blocks = cap;
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;  // the workgroups loop over the rest
  g->wpr = wpr;
  g->cpl = cpl;
  g->rpb = rpb;
  g->blocks = blocks;
  g->mres = mres == 1 ? 1 : 0;
  return JAS_OK;
}

jas_status_t fwd_impl(const jas_desc_t *d, const void *scores, const float *mask,
                      const int32_t *key_len, const float *sink, void *probs, float *p_sink,
                      float *lse, const jas_launch_t *launch, void *stream) {
  Dims dm;
  jas_status_t st = check_desc(d, &dm);
  if (st != JAS_OK) return st;
  const bool has_mask = (d->flags & JAS_FLAG_MASK) != 0;
  const bool has_sink = (d->flags & JAS_FLAG_SINK) != 0;
  const bool has_klen = (d->flags & JAS_FLAG_KEY_LEN) != 0;
  const bool has_lse = (d->flags & JAS_FLAG_LSE) != 0;
  if ((!has_mask && mask) || (!has_sink && (sink || p_sink)) || (!has_klen && key_len) ||
      (!has_lse && lse))
    return JAS_ERR_BAD_FLAGS;
  if (dm.rows == 0) return JAS_OK;  // nothing is read or written; row pointers may be NULL
  if (!scores || !probs) return JAS_ERR_NULL_POINTER;
  if (has_mask && !mask) return JAS_ERR_NULL_POINTER;
  if (has_sink && (!sink || !p_sink)) return JAS_ERR_NULL_POINTER;
  if (has_klen && !key_len) return JAS_ERR_NULL_POINTER;
  if (has_lse && !lse) return JAS_ERR_NULL_POINTER;
  if (!aligned(scores, dm.esz) || !aligned(probs, dm.esz) || (mask && !aligned(mask, 4)) ||
      (sink && !aligned(sink, 4)) || (p_sink && !aligned(p_sink, 4)) ||
      (key_len && !aligned(key_len, 4)) || (lse && !aligned(lse, 4)))
    return JAS_ERR_ALIGNMENT;

  const int64_t tbytes = dm.span * dm.esz;
  const Range rs = range_of(scores, tbytes), rp = range_of(probs, tbytes);
  int64_t mb = 0;
  if (has_mask && dm.rows > 0) {
    st = mask_bytes(d, &mb);
    if (st != JAS_OK) return st;
  }
  const Range rm = range_of(mask, has_mask ? mb : 0);
  const Range rk = range_of(sink, has_sink ? d->heads * 4 : 0);
  const Range rps = range_of(p_sink, has_sink ? dm.rows * 4 : 0);
  const Range rkl = range_of(key_len, has_klen ? d->batch * 4 : 0);
  const Range rl = range_of(lse, has_lse ? dm.rows * 4 : 0);
  if (probs != scores && overlap(rp, rs)) return JAS_ERR_ALIASING;
  if (overlap(rp, rm) || overlap(rp, rk) || overlap(rp, rps) || overlap(rp, rkl) ||
      overlap(rp, rl))
    return JAS_ERR_ALIASING;
  if (overlap(rps, rs) || overlap(rps, rm) || overlap(rps, rk) || overlap(rps, rkl) ||
      overlap(rps, rl))
    return JAS_ERR_ALIASING;
  if (overlap(rl, rs) || overlap(rl, rm) || overlap(rl, rk) || overlap(rl, rkl))
    return JAS_ERR_ALIASING;

  Geometry g;
  st = choose_geometry(d->dtype, dm.T, dm.rows, false, launch, &g, whole_chunk_rows(d), mask_kind(d));
  if (st != JAS_OK) return st;
  jas::FwdArgs a;
  a.stash = 0;  // the streaming launcher decides
  a.scores = scores;
  a.probs = probs;
  a.mask = has_mask ? mask : nullptr;
  a.msb = d->mask_stride_b;
  a.msh = d->mask_stride_h;
  a.msq = d->mask_stride_q;
  a.ex = jas::Exclusion{(d->flags & JAS_FLAG_CAUSAL) ? 1 : 0, has_klen ? key_len : nullptr};
  a.sink = has_sink ? sink : nullptr;
  a.p_sink = has_sink ? p_sink : nullptr;
  a.lse = has_lse ? lse : nullptr;
  a.s = jas::RowShape{dm.rows, d->keys, d->ld, d->heads, d->q_rows, dm.T};
  // 16-byte path: every row is whole 16-byte chunks starting on 16-byte
  // boundaries (and so is every mask row); otherwise element-wise access.
  // Both paths compute the same bits.
  const int64_t kpc = jas::keys_per_chunk(d->dtype);
  a.vec_mask = !has_mask || (aligned(mask, 16) && d->mask_stride_b % 4 == 0 &&
                             d->mask_stride_h % 4 == 0 && d->mask_stride_q % 4 == 0);
  a.vec_io = aligned(scores, 16) && aligned(probs, 16) && (d->ld % kpc == 0) &&
             (d->keys % kpc == 0) && a.vec_mask;
  if (jas::launch_fwd(d->dtype, a, g, (hipStream_t)stream) != hipSuccess) return JAS_ERR_HIP;
  return JAS_OK;
}

// The backward.  With `use_scratch` the per-row d_sink shares go to the
// library's static device scratch instead of a caller's workspace (the
// allocation-free entry point): `workspace` is then ignored, and the rows
// are limited to JAS_NOALLOC_MAX_ROWS.
jas_status_t bwd_impl(const jas_desc_t *d, const void *probs, const void *dprobs,
                      const int32_t *key_len, const float *p_sink, void *dscores, float *d_sink,
                      void *workspace, size_t workspace_bytes, const jas_launch_t *launch,
                      void *stream, bool use_scratch = false) {
  Dims dm;
  jas_status_t st = check_desc(d, &dm);
  if (st != JAS_OK) return st;
  const bool has_sink = (d->flags & JAS_FLAG_SINK) != 0;
  const bool has_klen = (d->flags & JAS_FLAG_KEY_LEN) != 0;
  if (!has_klen && key_len) return JAS_ERR_BAD_FLAGS;
  if (dm.rows == 0) {  // nothing is read; only d_sink is written (+0 per head)
    if (!has_sink && (p_sink || d_sink)) return JAS_ERR_BAD_FLAGS;
    if (!has_sink || d->heads == 0) return JAS_OK;
    if (!d_sink) return JAS_ERR_NULL_POINTER;
    if (!aligned(d_sink, 4)) return JAS_ERR_ALIGNMENT;
    jas::DsinkArgs s{nullptr, d_sink, d->batch, d->heads, d->q_rows};
    if (jas::launch_dsink(s, (hipStream_t)stream) != hipSuccess) return JAS_ERR_HIP;
    return JAS_OK;
  }
  if (!probs || !dprobs || !dscores) return JAS_ERR_NULL_POINTER;
  if (has_sink && (!p_sink || !d_sink)) return JAS_ERR_NULL_POINTER;
  if (has_klen && !key_len) return JAS_ERR_NULL_POINTER;
  if (!has_sink && (p_sink || d_sink)) return JAS_ERR_BAD_FLAGS;
  if (!aligned(probs, dm.esz) || !aligned(dprobs, dm.esz) || !aligned(dscores, dm.esz) ||
      (p_sink && !aligned(p_sink, 4)) || (d_sink && !aligned(d_sink, 4)) ||
      (key_len && !aligned(key_len, 4)))
    return JAS_ERR_ALIGNMENT;
  const size_t need = jas_bwd_workspace_bytes(d);
  if (has_sink && use_scratch) {
    if (dm.rows > JAS_NOALLOC_MAX_ROWS) return JAS_ERR_SCRATCH;
    workspace = nullptr;  // the scratch: looked up after validation, and outside every caller buffer
  } else if (has_sink) {
    if (!workspace || workspace_bytes < need) return JAS_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return JAS_ERR_ALIGNMENT;
  }

  const int64_t tbytes = dm.span * dm.esz;
  const Range rp = range_of(probs, tbytes), rg = range_of(dprobs, tbytes);
  const Range rd = range_of(dscores, tbytes);
  const Range rps = range_of(p_sink, has_sink ? dm.rows * 4 : 0);
  const Range rds = range_of(d_sink, has_sink ? d->heads * 4 : 0);
  const Range rw = range_of(workspace, has_sink ? (int64_t)need : 0);
  const Range rkl = range_of(key_len, has_klen ? d->batch * 4 : 0);
  if (dscores != probs && overlap(rd, rp)) return JAS_ERR_ALIASING;
  if (dscores != dprobs && overlap(rd, rg)) return JAS_ERR_ALIASING;
  if (overlap(rd, rps) || overlap(rd, rds) || overlap(rd, rw) || overlap(rd, rkl))
    return JAS_ERR_ALIASING;
  if (overlap(rds, rp) || overlap(rds, rg) || overlap(rds, rps) || overlap(rds, rw) ||
      overlap(rds, rkl))
    return JAS_ERR_ALIASING;
  if (overlap(rw, rp) || overlap(rw, rg) || overlap(rw, rps) || overlap(rw, rkl))
    return JAS_ERR_ALIASING;

  Geometry g;
  st = choose_geometry(d->dtype, dm.T, dm.rows, true, launch, &g, whole_chunk_rows(d));
  if (st != JAS_OK) return st;

  if (has_sink && use_scratch) {
    // every check has passed: find the scratch of the stream's device
    int dev = -1;
    const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    float *sp = nullptr;
    if (e != hipSuccess || jas::scratch_address(dev, &sp) != hipSuccess) return JAS_ERR_HIP;
    workspace = sp;
  }
  {
    jas::BwdArgs a;
    a.stash = 0;  // the streaming launcher decides
    a.probs = probs;
    a.dprobs = dprobs;
    a.dscores = dscores;
    a.p_sink = has_sink ? p_sink : nullptr;
    a.v = has_sink ? static_cast<float *>(workspace) : nullptr;
    a.ex = jas::Exclusion{(d->flags & JAS_FLAG_CAUSAL) ? 1 : 0, has_klen ? key_len : nullptr};
    a.s = jas::RowShape{dm.rows, d->keys, d->ld, d->heads, d->q_rows, dm.T};
    const int64_t kpc = jas::keys_per_chunk(d->dtype);
    a.vec_io = aligned(probs, 16) && aligned(dprobs, 16) && aligned(dscores, 16) &&
               (d->ld % kpc == 0) && (d->keys % kpc == 0);
    if (jas::launch_bwd(d->dtype, a, g, (hipStream_t)stream) != hipSuccess) return JAS_ERR_HIP;
  }
  if (has_sink) {
    jas::DsinkArgs s{static_cast<const float *>(workspace), d_sink, d->batch, d->heads, d->q_rows};
    if (jas::launch_dsink(s, (hipStream_t)stream) != hipSuccess) return JAS_ERR_HIP;
  }
  return JAS_OK;
}

// ---- fused attention -------------------------------------------------------

struct AttnDims {
  int64_t rows;  // batch*heads*q_len
  int T;
};

jas_status_t check_attn_desc(const jas_attn_desc_t *d, AttnDims *dm) {
  if (!d) return JAS_ERR_NULL_POINTER;
  const int dt = enum_bits(d->dtype);
  if (dt != JAS_DTYPE_BF16 && dt != JAS_DTYPE_F16) return JAS_ERR_BAD_DTYPE;
  const uint32_t known = JAS_FLAG_MASK | JAS_FLAG_SINK | JAS_FLAG_CAUSAL | JAS_FLAG_KEY_LEN |
                         JAS_FLAG_LSE | JAS_FLAG_PROBS | JAS_FLAG_SCORES;
  if (d->flags & ~known) return JAS_ERR_BAD_FLAGS;
  if (d->batch < 0 || d->q_len < 0 || d->heads < 1 || d->kv_heads < 1 || d->kv_len < 1 ||
      d->heads % d->kv_heads != 0)
    return JAS_ERR_BAD_SHAPE;
  if (d->mask_stride_b < 0 || d->mask_stride_h < 0 || d->mask_stride_q < 0)
    return JAS_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return JAS_ERR_UNSUPPORTED;
  if (d->kv_len > JAS_ATTN_MAX_KEYS) return JAS_ERR_UNSUPPORTED;
  int64_t t = 0, rows = 0;
  if (!mul_ok(d->batch, d->heads, &t) || !mul_ok(t, d->q_len, &rows)) return JAS_ERR_BAD_SHAPE;
  // one (batch, head)'s Q, K and V are addressed with 32-bit byte offsets
  // (K and V: at most JAS_ATTN_MAX_KEYS x 128 x 2 bytes)
  int64_t qbytes = 0;
  if (!mul_ok(d->q_len, d->head_dim * 2, &qbytes) || qbytes > 0x7fffffff) return JAS_ERR_UNSUPPORTED;
  // so is one (batch, head)'s mask: its last query row ends within 2 GiB
  if (d->flags & JAS_FLAG_MASK) {
    int64_t mq = 0, mext = 0;
    if (!mul_ok(d->q_len > 0 ? d->q_len - 1 : 0, d->mask_stride_q, &mq) ||
        !add_ok(mq, d->kv_len, &mext) || !mul_ok(mext, 4, &mext) || mext > 0x7fffffff)
      return JAS_ERR_UNSUPPORTED;
  }
  const int T = (int)((d->kv_len + jas::kTile - 1) / jas::kTile);
  int64_t probe = 0;
  if (!mul_ok(d->batch, d->kv_heads, &t) || !mul_ok(t, d->kv_len * d->head_dim * 2, &probe))
    return JAS_ERR_BAD_SHAPE;
  if (!mul_ok(rows, d->kv_len * 4, &probe) || !mul_ok(rows, d->head_dim * 2, &probe))
    return JAS_ERR_BAD_SHAPE;
  dm->rows = rows;
  dm->T = T;
  return JAS_OK;
}

jas_status_t attn_fwd_impl(const jas_attn_desc_t *d, const void *q, const void *k, const void *v,
                           const float *mask, const int32_t *key_len, const float *sink,
                           void *out, float *lse, float *p_sink, void *probs, float *scores,
                           int query_blocks, void *stream) {
  AttnDims dm;
  jas_status_t st = check_attn_desc(d, &dm);
  if (st != JAS_OK) return st;
  if (query_blocks < 0 || query_blocks > 2) return JAS_ERR_BAD_FLAGS;
  const uint32_t f = d->flags;
  const bool has_mask = f & JAS_FLAG_MASK, has_sink = f & JAS_FLAG_SINK,
             has_klen = f & JAS_FLAG_KEY_LEN, has_lse = f & JAS_FLAG_LSE,
             has_probs = f & JAS_FLAG_PROBS, has_scores = f & JAS_FLAG_SCORES;
  if ((!has_mask && mask) || (!has_sink && (sink || p_sink)) || (!has_klen && key_len) ||
      (!has_lse && lse) || (!has_probs && probs) || (!has_scores && scores))
    return JAS_ERR_BAD_FLAGS;
  if (dm.rows == 0) return JAS_OK;  // nothing is read or written
  if (!q || !k || !v || !out) return JAS_ERR_NULL_POINTER;
  if ((has_mask && !mask) || (has_sink && (!sink || !p_sink)) || (has_klen && !key_len) ||
      (has_lse && !lse) || (has_probs && !probs) || (has_scores && !scores))
    return JAS_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(out, 2) || (probs && !aligned(probs, 2)) || (mask && !aligned(mask, 4)) ||
      (sink && !aligned(sink, 4)) || (p_sink && !aligned(p_sink, 4)) ||
      (lse && !aligned(lse, 4)) || (scores && !aligned(scores, 4)) ||
      (key_len && !aligned(key_len, 4)))
    return JAS_ERR_ALIGNMENT;

  const int64_t D = d->head_dim;
  const int64_t qbytes = dm.rows * D * 2;
  const int64_t kvbytes = d->batch * d->kv_heads * d->kv_len * D * 2;
  int64_t mb = 0;
  if (has_mask) {
    jas_desc_t md{};
    md.batch = d->batch;
    md.heads = d->heads;
    md.q_rows = d->q_len;
    md.keys = d->kv_len;
    md.mask_stride_b = d->mask_stride_b;
    md.mask_stride_h = d->mask_stride_h;
    md.mask_stride_q = d->mask_stride_q;
    st = mask_bytes(&md, &mb);
    if (st != JAS_OK) return st;
  }
  const Range in[] = {range_of(q, qbytes), range_of(k, kvbytes), range_of(v, kvbytes),
                      range_of(mask, mb), range_of(key_len, has_klen ? d->batch * 4 : 0),
                      range_of(sink, has_sink ? d->heads * 4 : 0)};
  const Range outs[] = {range_of(out, qbytes), range_of(lse, has_lse ? dm.rows * 4 : 0),
                        range_of(p_sink, has_sink ? dm.rows * 4 : 0),
                        range_of(probs, has_probs ? dm.rows * d->kv_len * 2 : 0),
                        range_of(scores, has_scores ? dm.rows * d->kv_len * 4 : 0)};
  for (const Range &o : outs) {
    for (const Range &i : in)
      if (overlap(o, i)) return JAS_ERR_ALIASING;
    for (const Range &o2 : outs)
      if (&o2 != &o && overlap(o, o2)) return JAS_ERR_ALIASING;
  }

  jas::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.mask = has_mask ? mask : nullptr;
  a.msb = d->mask_stride_b;
  a.msh = d->mask_stride_h;
  a.msq = d->mask_stride_q;
  a.ex = jas::Exclusion{(f & JAS_FLAG_CAUSAL) ? 1 : 0, has_klen ? key_len : nullptr};
  a.sink = has_sink ? sink : nullptr;
  a.p_sink = has_sink ? p_sink : nullptr;
  a.lse = has_lse ? lse : nullptr;
  a.probs = has_probs ? probs : nullptr;
  a.scores = has_scores ? scores : nullptr;
  a.scale = d->scale;
  a.B = d->batch;
  a.H = d->heads;
  a.Hkv = d->kv_heads;
  a.Sq = d->q_len;
  a.N = d->kv_len;
  a.D = (int)D;
  a.T = dm.T;
  // one workgroup of 4 waves per 64 * query_blocks queries of a (batch, head)
  if (jas::launch_attn_fwd(d->dtype, a, query_blocks, (hipStream_t)stream) != hipSuccess)
    return JAS_ERR_HIP;
  return JAS_OK;
}

}  // namespace

extern "C" {

jas_status_t jas_fwd(const jas_desc_t *desc, const void *scores, const float *mask,
                     const int32_t *key_len, const float *sink, void *probs, float *p_sink,
                     float *lse, void *stream) {
  return fwd_impl(desc, scores, mask, key_len, sink, probs, p_sink, lse, nullptr, stream);
}

jas_status_t jas_fwd_ex(const jas_desc_t *desc, const void *scores, const float *mask,
                        const int32_t *key_len, const float *sink, void *probs, float *p_sink,
                        float *lse, const jas_launch_t *launch, void *stream) {
  return fwd_impl(desc, scores, mask, key_len, sink, probs, p_sink, lse, launch, stream);
}

size_t jas_bwd_workspace_bytes(const jas_desc_t *desc) {
  Dims dm;
  if (check_desc(desc, &dm) != JAS_OK) return 0;
  if (!(desc->flags & JAS_FLAG_SINK)) return 0;
  const size_t b = (size_t)dm.rows * 4u;
  return (b + 255u) & ~(size_t)255u;
}

jas_status_t jas_bwd(const jas_desc_t *desc, const void *probs, const void *dprobs,
                     const int32_t *key_len, const float *p_sink, void *dscores, float *d_sink,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, workspace,
                  workspace_bytes, nullptr, stream);
}

jas_status_t jas_bwd_ex(const jas_desc_t *desc, const void *probs, const void *dprobs,
                        const int32_t *key_len, const float *p_sink, void *dscores,
                        float *d_sink, void *workspace, size_t workspace_bytes,
                        const jas_launch_t *launch, void *stream) {
  return bwd_impl(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, workspace,
                  workspace_bytes, launch, stream);
}

jas_status_t jas_bwd_noalloc(const jas_desc_t *desc, const void *probs, const void *dprobs,
                             const int32_t *key_len, const float *p_sink, void *dscores,
                             float *d_sink, void *stream) {
  return bwd_impl(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, nullptr, 0, nullptr,
                  stream, true);
}

jas_status_t jas_launch_plan(const jas_desc_t *desc, int backward, const jas_launch_t *launch,
                             jas_launch_t *plan) {
  if (!plan) return JAS_ERR_NULL_POINTER;
  *plan = jas_launch_t{0, 0, 0, 0, 0, 0};
  if (backward != 0 && backward != 1) return JAS_ERR_BAD_FLAGS;
  Dims dm;
  const jas_status_t st = check_desc(desc, &dm);
  if (st != JAS_OK) return st;
  if (dm.rows == 0) return JAS_OK;  // no row kernel runs
  Geometry g;
  const jas_status_t sg =
      choose_geometry(desc->dtype, dm.T, dm.rows, backward != 0, launch, &g, whole_chunk_rows(desc),
                      backward ? kNoMask : mask_kind(desc));
  if (sg != JAS_OK) return sg;
  plan->waves_per_row = g.wpr;
  plan->chunks_per_lane = g.cpl;
  plan->rows_per_block = g.rpb;
  plan->max_blocks = (int32_t)g.blocks;
  plan->streaming = g.stream;
  plan->mask_in_registers = g.mres;
  return JAS_OK;
}

jas_status_t jas_attn_fwd(const jas_attn_desc_t *desc, const void *q, const void *k,
                          const void *v, const float *mask, const int32_t *key_len,
                          const float *sink, void *out, float *lse, float *p_sink, void *probs,
                          float *scores, void *stream) {
  return attn_fwd_impl(desc, q, k, v, mask, key_len, sink, out, lse, p_sink, probs, scores, 0,
                       stream);
}

jas_status_t jas_attn_fwd_ex(const jas_attn_desc_t *desc, const void *q, const void *k,
                             const void *v, const float *mask, const int32_t *key_len,
                             const float *sink, void *out, float *lse, float *p_sink, void *probs,
                             float *scores, int query_blocks, void *stream) {
  return attn_fwd_impl(desc, q, k, v, mask, key_len, sink, out, lse, p_sink, probs, scores,
                       query_blocks, stream);
}

const char *jas_status_str(jas_status_t s) {
  switch (enum_bits(s)) {
    case JAS_OK: return "ok";
    case JAS_ERR_NULL_POINTER: return "a required pointer is NULL";
    case JAS_ERR_BAD_SHAPE: return "invalid shape, row stride or mask stride";
    case JAS_ERR_BAD_DTYPE: return "unknown dtype";
    case JAS_ERR_BAD_FLAGS: return "unknown flag, or a pointer given for a flag that is not set";
    case JAS_ERR_ALIASING: return "an output overlaps another buffer";
    case JAS_ERR_WORKSPACE: return "workspace missing or too small";
    case JAS_ERR_UNSUPPORTED: return "row length or launch geometry not supported";
    case JAS_ERR_HIP: return "the HIP runtime refused a launch";
    case JAS_ERR_ALIGNMENT: return "a pointer is not aligned to its element size";
    case JAS_ERR_SCRATCH: return "more rows than the library's scratch holds (JAS_NOALLOC_MAX_ROWS)";
  }
  return "unknown status";
}

const char *jas_contract(void) {
  return "jas/1 tile=256 tree=balanced-pairwise-by-key fold=left-to-right sink=merged-last "
         "exclusion=suffix(causal,key_len) lse=M+fl(log2(L)*ln2),v_log_f32 "
         "acc=fp32 exp=2^fl(y*log2e),flush<2^-126,v_exp_f32 div=ieee cvt=rne(bf16,f16) "
         "fpcontract=off atomics=none dsink=256-row-chunks,left-fold "
         "attn=qk,pv:mfma_f32_16x16x32(32-per-step,ascending),s=fl(scale*dot),two-pass,"
         "p=rne(dtype) arch=gfx950";
}

}  // extern "C"
