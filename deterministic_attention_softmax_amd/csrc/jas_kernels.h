// jas_kernels.h -- gfx950 kernels of the fixed-order, batch-invariant row
// softmax (forward and backward templates and their launch tables).  Each
// jas_kernels_<dtype>.hip includes this file and instantiates one element
// type, so the instances compile in parallel; jas_launch.hip holds the
// per-head d_sink kernel and the dispatch by dtype.
//
// Method: RL-Kernel PR #453, "[WS1][kernels] Add fixed-order joint-attention
// softmax for Qwen-Image", Summary (fixed-order online softmax over 256-key
// tiles taken left to right, one fixed tree per tile for max and sum, tile
// states merged in order, FP32 intermediates, one conversion at the write;
// fixed-order backward delta = sum(P*dP), dS = P*(dP - delta)).  Sink: ROCm
// TransformerEngine PR #678, Description (one learnable logit per head in the
// denominator, d_sink per head).  Tree shape independent of launch: RL-Kernel
// PR #240, Fixed Reduction Contract.
//
// Mapping to CDNA4.  A row is owned by one wavefront (or by 2 or 4
// wavefronts of one workgroup for long rows).  The row is read as 16-byte
// chunks: a lane's chunk is 8 consecutive bf16 / fp16 keys or 4 consecutive
// fp32 keys, so a 256-key tile is 32 lanes (16-bit types) or 64 lanes (fp32)
// and one wave-wide load ("slot") covers 2 or 1 tiles.  The balanced pairwise tile
// tree is realised exactly: pairwise adds inside the lane over its
// consecutive keys, then across lanes with DPP quad permutes (lane xor 1,
// xor 2), row half-mirror and row mirror (groups of 8 and 16 lanes whose
// values are already uniform within each half), and the gfx950 permlane16 /
// permlane32 swaps for 32 and 64 lanes.  IEEE addition is commutative, so
// every lane of a group ends with the same bits, and the tree is a function
// of key positions only.  Tile states go through LDS to one lane per tile;
// the merge is done as a prefix max across lanes, per-tile rescale factors in
// parallel, then the short serial chain L = L*a_t + q_t that the left fold
// needs.  No MFMA: there is no contraction here, the kernels are bound by HBM
// bandwidth.  No atomics: every output element has one writer.
//
// Built with -ffp-contract=off (no fused multiply-add is formed from a*b+c),
// without fast-math, FP32 denormals preserved.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jas_internal.h"

#if defined(__FAST_MATH__) || (defined(__FINITE_MATH_ONLY__) && __FINITE_MATH_ONLY__)
#error "fast-math changes the arithmetic contract; build without it"
#endif

namespace jas {
namespace {

constexpr float kLog2e = 0x1.715476p+0f;  // binary32 nearest to log2(e)
constexpr float kLn2 = 0x1.62e430p-1f;    // binary32 nearest to ln(2)
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// exp_(y) = 2^fl(y*log2e) with the hardware base-2 exponential, for y <= 0
// or -inf.  The contract flushes results below 2^-126 to +0; v_exp_f32 does
// exactly that on gfx950 (every binary32 exponent from -0 down to -inf was
// checked: +0 below -126, a normal number from -126 up, within 1 ulp of the
// correctly rounded 2^u), so no select is needed.
__device__ __forceinline__ float exp_(float y) { return __builtin_amdgcn_exp2f(y * kLog2e); }

// Round two binary32 to bf16 (round to nearest-even) and pack them, low
// half first: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// Round two binary32 to binary16 (round to nearest-even, subnormals kept,
// overflow to infinity) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Two binary16 (low half first) widened to binary32, exactly.
__device__ __forceinline__ f32x2_t unpack_f16(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

// ln(L) for the row log-sum-exp: the hardware base-2 logarithm times ln 2.
__device__ __forceinline__ float ln_(float L) { return __builtin_amdgcn_logf(L) * kLn2; }

// ---------------------------------------------------------------------------
// Cross-lane steps of the tile tree
// ---------------------------------------------------------------------------

constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- 7-i within 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <- 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xF, 0xF, true));
}

// Returns (value of the even 16-lane row, value of the odd 16-lane row) of
// the lane's 32-lane half, in every lane.
__device__ __forceinline__ f32x2_t rows16_pair(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  return f32x2_t{u2f(p[0]), u2f(p[1])};
}

// Returns (value of lanes 0-31, value of lanes 32-63) in every lane.
__device__ __forceinline__ f32x2_t halves32_pair(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return f32x2_t{u2f(p[0]), u2f(p[1])};
}

// Sum over each aligned 32-lane group, as the top 5 levels of a balanced
// tree whose leaves are the lanes in order.
__device__ __forceinline__ float group32_sum(float v) {
  v = v + dpp<kDppQuadXor1>(v);
  v = v + dpp<kDppQuadXor2>(v);
  v = v + dpp<kDppRowHalfMirror>(v);
  v = v + dpp<kDppRowMirror>(v);
  const f32x2_t p = rows16_pair(v);
  return p[0] + p[1];
}

__device__ __forceinline__ float group64_sum(float v) {
  v = group32_sum(v);
  const f32x2_t p = halves32_pair(v);
  return p[0] + p[1];
}

// max with -0 < +0 and NaN propagation (gfx950 v_maximum3_f32); max is
// exact, so the tree shape cannot change its value.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float group32_max(float v) {
  v = fmax2(v, dpp<kDppQuadXor1>(v));
  v = fmax2(v, dpp<kDppQuadXor2>(v));
  v = fmax2(v, dpp<kDppRowHalfMirror>(v));
  v = fmax2(v, dpp<kDppRowMirror>(v));
  const f32x2_t p = rows16_pair(v);
  return fmax2(p[0], p[1]);
}

__device__ __forceinline__ float group64_max(float v) {
  v = group32_max(v);
  const f32x2_t p = halves32_pair(v);
  return fmax2(p[0], p[1]);
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), lane));
}

// Orders LDS traffic of one wavefront (writes by some lanes, reads by
// others) when a row is owned by a single wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Element layouts
// ---------------------------------------------------------------------------

template <int DT> struct Cfg;
template <> struct Cfg<0> {  // fp32
  static constexpr int KPL = 4;   // keys per 16-byte chunk
  static constexpr int LPT = 64;  // lanes per tile
  static constexpr int TPS = 1;   // tiles per wave-wide chunk
  static constexpr int ESZ = 4;
};
template <> struct Cfg<1> {  // bf16
  static constexpr int KPL = 8;
  static constexpr int LPT = 32;
  static constexpr int TPS = 2;
  static constexpr int ESZ = 2;
};
template <> struct Cfg<2> : Cfg<1> {};  // fp16: the bf16 layout

// Bits of -inf, twice for the 16-bit types (the fill of keys past a row).
template <int DT> constexpr uint32_t kNegInfBits = 0xff800000u;
template <> constexpr uint32_t kNegInfBits<1> = 0xff80ff80u;
template <> constexpr uint32_t kNegInfBits<2> = 0xfc00fc00u;

// A 16-byte chunk as 4 words.
struct Chunk { uint32_t w[4]; };
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element-by-element chunk load for unaligned rows and the tail of a row:
// keys at or past n read as `fill` bits.
template <int DT>
__device__ __forceinline__ Chunk load_chunk_elems(const char *row, int j0, int n, uint32_t fill) {
  Chunk c;
  if constexpr (DT != 0) {
    const uint16_t *e = reinterpret_cast<const uint16_t *>(row);
    const uint32_t f = fill & 0xffffu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 2 * i;
      const uint32_t lo = (j < n) ? e[j] : f;
      const uint32_t hi = (j + 1 < n) ? e[j + 1] : f;
      c.w[i] = lo | (hi << 16);
    }
  } else {
    const uint32_t *e = reinterpret_cast<const uint32_t *>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      c.w[i] = (j < n) ? e[j] : fill;
    }
  }
  return c;
}

template <int DT>
__device__ __forceinline__ void store_chunk_elems(char *row, int j0, int n, const Chunk &c) {
  if constexpr (DT != 0) {
    uint16_t *e = reinterpret_cast<uint16_t *>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 2 * i;
      if (j < n) e[j] = (uint16_t)(c.w[i] & 0xffffu);
      if (j + 1 < n) e[j + 1] = (uint16_t)(c.w[i] >> 16);
    }
  } else {
    uint32_t *e = reinterpret_cast<uint32_t *>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      if (j < n) e[j] = c.w[i];
    }
  }
}

template <int DT>
__device__ __forceinline__ void unpack(const Chunk &c, float (&x)[Cfg<DT>::KPL]) {
  if constexpr (DT == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(c.w[i]);
      x[2 * i + 1] = bf16_hi(c.w[i]);
    }
  } else if constexpr (DT == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t v = unpack_f16(c.w[i]);
      x[2 * i] = v[0];
      x[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = u2f(c.w[i]);
  }
}

template <int DT>
__device__ __forceinline__ Chunk pack(const float (&x)[Cfg<DT>::KPL]) {
  Chunk c;
  if constexpr (DT == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
  } else if constexpr (DT == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = pack_f16(x[2 * i], x[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = f2u(x[i]);
  }
  return c;
}

// Balanced pairwise tree over the lane's consecutive keys (the bottom
// levels of the tile tree).
template <int K>
__device__ __forceinline__ float lane_tree_sum(const float (&x)[K]) {
  if constexpr (K == 4) {
    return (x[0] + x[1]) + (x[2] + x[3]);
  } else {
    return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
  }
}

template <int K>
__device__ __forceinline__ float lane_tree_max(const float (&x)[K]) {
  if constexpr (K == 4) {
    return fmax2(fmax2(fmax2(x[0], x[1]), x[2]), x[3]);
  } else {
    return fmax2(fmax2(fmax2(fmax2(x[0], x[1]), x[2]), fmax2(fmax2(x[3], x[4]), x[5])),
                 fmax2(x[6], x[7]));
  }
}

template <int DT>
__device__ __forceinline__ float tile_sum(float v) {
  if constexpr (Cfg<DT>::LPT == 32) return group32_sum(v);
  else return group64_sum(v);
}

template <int DT>
__device__ __forceinline__ float tile_max(float v) {
  if constexpr (Cfg<DT>::LPT == 32) return group32_max(v);
  else return group64_max(v);
}

template <int WPR>
__device__ __forceinline__ void row_sync() {
  if constexpr (WPR == 1) wave_sync();
  else __syncthreads();
}

// ---------------------------------------------------------------------------
// Row kernels: common indexing
//
// Row r is owned by WPR waves of one workgroup; wave `wir` holds the slots
// gs = s*WPR + wir (s < CPL), slot gs covering tiles gs*TPS .. gs*TPS+TPS-1.
// A lane's chunk starts at key gs*TPS*256 + loff with loff = half*256 +
// cil*KPL.  The wave index is made wave-uniform (readfirstlane) so row
// pointers live in scalar registers and every load is base + 32-bit lane
// offset.  VEC: rows are whole 16-byte chunks on 16-byte boundaries, so a
// chunk is wholly inside or wholly past the row; the row is read and written
// through a buffer resource of the row's size, so lanes past the row read 0
// (replaced by -inf or +0 before use) and their stores are dropped.  !VEC:
// element-wise access.
// ---------------------------------------------------------------------------

template <int DT, int WPR>
struct RowIdx {
  using C = Cfg<DT>;
  int lane, wir, rib, rpb, loff, half, cil;
  __device__ __forceinline__ RowIdx() {
    lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    wir = wave % WPR;
    rib = wave / WPR;
    rpb = blockDim.x / (kWave * WPR);
    half = lane / C::LPT;
    cil = lane % C::LPT;
    loff = half * kTile + cil * C::KPL;
  }
};

// A raw buffer resource over one row (gfx9 family: stride 0, 32-bit
// records).  Loads at or past `bytes` return 0 and stores there are
// dropped, which handles the lanes past the row and the spare rows of a
// workgroup (bytes = 0) without clamps or branches.  The row offset of a
// slot is wave-uniform and goes in the scalar offset; the lane's offset in
// the slot is one VGPR shared by all slots.
constexpr int kBufWord3 = 0x00020000;
constexpr int kAuxNT = 2;  // nontemporal: the row is streamed once

// A cache policy as a type, for lambdas that take it as a compile-time
// argument (the load builtins need an immediate).
template <int V>
struct AuxC {
  static constexpr int value = V;
};

struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void *base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufWord3)) {}
};

template <int AUX>
__device__ __forceinline__ Chunk bload(const Buf &b, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)voff, (int)soff, AUX);
  return Chunk{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ void bstore(const Buf &b, uint32_t voff, uint32_t soff, const Chunk &c) {
  const u32x4 v = {c.w[0], c.w[1], c.w[2], c.w[3]};
  __builtin_amdgcn_raw_buffer_store_b128(v, b.r, (int)voff, (int)soff, kAuxNT);
}

// Visible key prefix of row (b, q): N keys, cut by the causal condition
// key <= N - Sq + q and by the batch entry's key length, clamped to [0, N].
// Wave-uniform.
__device__ __forceinline__ int row_kend(const Exclusion &ex, int N, int64_t Sq, int64_t b,
                                        int64_t q) {
  int64_t k = N;
  if (ex.causal) {
    const int64_t c = q + ((int64_t)N - Sq) + 1;
    k = c < k ? c : k;
  }
  if (ex.key_len) {
    const int64_t l = ex.key_len[b];
    k = l < k ? l : k;
  }
  // a 32-bit scalar from here on: the per-slot comparisons with it stay
  // scalar instead of 64-bit vector compares against hoisted constants
  return __builtin_amdgcn_readfirstlane((int)(k < 0 ? 0 : k));
}

// ---------------------------------------------------------------------------
// Forward
//
// Phase 1 issues every score load of the row before any of it is used, so
// the row's bytes are in flight together; phase 2 reduces each tile (the
// mask row, shared by the rows of a batch and L2-resident, is read one slot
// ahead); the tile states meet in LDS; the merge runs in every wave of the
// row; phase 3 rescales, converts once and stores.
//
// MRES (16-byte rows with a mask): each wave keeps its share of the mask row
// in registers from one of its workgroup's row groups to the next (every
// gridDim-th group, so the workgroups in flight read neighbouring rows), and
// loads it again only when a row's mask row or visible length differs from
// the previous row's: rows that share a mask row (a mask broadcast over
// queries) load it once per workgroup.  The arithmetic is the same.
// ---------------------------------------------------------------------------

template <int DT, int WPR, int CPL, bool VEC, bool MASK, bool EXCL, bool MRES = false>
__global__ __launch_bounds__(kWave * kBlockWaves) void fwd_kernel(const FwdArgs a) {
  using C = Cfg<DT>;
  constexpr int KPL = C::KPL, TPS = C::TPS, ESZ = C::ESZ;
  // keys past the row read as -inf (the max's identity; their e is +0)
  constexpr uint32_t kFill = kNegInfBits<DT>;
  __shared__ float lds_m[kBlockWaves][kMaxTiles];
  __shared__ float lds_l[kBlockWaves][kMaxTiles];

  const RowIdx<DT, WPR> ix;
  const int lane = ix.lane;
  const int T = a.s.T;
  const int N = (int)a.s.N;
  const int nslots = (T + TPS - 1) / TPS;
  const int64_t ngroups = (a.s.rows + ix.rpb - 1) / ix.rpb;
  const bool has_sink = a.sink != nullptr;
  constexpr bool kRes = MRES && MASK && VEC;
  // the mask of the wave's slots (kRes), and the mask row and length it holds
  float4 mres[kRes ? CPL : 1][KPL / 4];
  const float *mheld = nullptr;
  int kheld = -1;

  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t r = grp * ix.rpb + ix.rib;
    const bool active = r < a.s.rows;
    // a workgroup's spare rows read the last row (element-wise path) or see
    // an empty buffer (VEC), and write nothing
    const int64_t rr = active ? r : a.s.rows - 1;
    const char *srow = static_cast<const char *>(a.scores) + rr * a.s.ld * ESZ;
    char *prow = static_cast<char *>(a.probs) + r * a.s.ld * ESZ;
    const float *mrow = nullptr;
    int64_t h = 0;
    int kend = N;  // visible keys: the rest count as -inf and are not read
    if (MASK || has_sink || EXCL) {
      const int64_t q = rr % a.s.Sq;
      const int64_t bh = rr / a.s.Sq;
      h = bh % a.s.H;
      if constexpr (MASK) mrow = a.mask + (bh / a.s.H) * a.msb + h * a.msh + q * a.msq;
      if constexpr (EXCL) kend = row_kend(a.ex, N, a.s.Sq, bh / a.s.H, q);
    }
    // scores (and mask) are read up to the chunk holding the last visible
    // key; the probabilities are written over the whole row
    const int kread = EXCL ? (kend + KPL - 1) / KPL * KPL : N;
    const Buf sbuf(srow, active ? (uint32_t)(kread * ESZ) : 0u);
    const Buf pbuf(prow, active ? (uint32_t)(N * ESZ) : 0u);
    const Buf mbuf(mrow, (MASK && active) ? (uint32_t)(kread * 4) : 0u);
    const uint32_t voff = (uint32_t)(ix.loff * ESZ);
    // this lane's visible keys in the chunk of the slot starting at key sb
    // are the first (lim - sb) of it (compared against constants, so no
    // per-key index is kept live)
    const int lim = kend - ix.loff;

    // ---- phase 1: issue every score load of the row, straight-line (VEC:
    // lanes past the visible prefix read 0 and are overwritten in phase 2) ----
    Chunk raw[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int sb = (s * WPR + ix.wir) * TPS * kTile;
      if constexpr (VEC) raw[s] = bload<kAuxNT>(sbuf, voff, (uint32_t)(sb * ESZ));
      else raw[s] = load_chunk_elems<DT>(srow, sb + ix.loff, kend, kFill);
    }

    // ---- phase 2: per tile max, exponentials, sum ----
    float e[CPL][KPL];
    float4 mv[kRes ? 1 : 2][KPL / 4];  // mask of the current and the next slot (not kRes)
    auto load_mask = [&](int s, float4 (&dst)[KPL / 4]) {
      const uint32_t sb4 = (uint32_t)((s * WPR + ix.wir) * TPS * kTile * 4);
#pragma unroll
      for (int k4 = 0; k4 < KPL / 4; ++k4) {
        const Chunk c = bload<0>(mbuf, (uint32_t)(ix.loff * 4 + 16 * k4), sb4);
        dst[k4] = make_float4(u2f(c.w[0]), u2f(c.w[1]), u2f(c.w[2]), u2f(c.w[3]));
      }
    };
    if constexpr (kRes) {
      if (mrow != mheld || kread != kheld) {  // uniform
#pragma unroll
        for (int s = 0; s < CPL; ++s) load_mask(s, mres[s]);
        mheld = active ? mrow : nullptr;  // a spare row's buffer is empty
        kheld = kread;
      }
    } else if constexpr (MASK && VEC) {
      load_mask(0, mv[0]);
    }
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int gs = s * WPR + ix.wir;
      const int sb = gs * TPS * kTile;
      const int t = gs * TPS + ix.half;
      const int j0 = sb + ix.loff;
      if constexpr (MASK && VEC && !kRes) {
        if (s + 1 < CPL) load_mask(s + 1, mv[(s + 1) & 1]);
      }
      float m = kNegInf, l = 0.0f;
      bool skip = false;
      if constexpr (EXCL) skip = sb >= kend;  // uniform
      if (skip) {  // the whole slot is past the visible keys: not read
#pragma unroll
        for (int k = 0; k < KPL; ++k) e[s][k] = 0.0f;
      } else {
        float x[KPL];
        unpack<DT>(raw[s], x);
        if constexpr (MASK) {
          if constexpr (VEC) {
            const float4 *m4;
            if constexpr (kRes) m4 = mres[s];
            else m4 = mv[s & 1];
#pragma unroll
            for (int k4 = 0; k4 < KPL / 4; ++k4) {
              x[4 * k4 + 0] = x[4 * k4 + 0] + m4[k4].x;
              x[4 * k4 + 1] = x[4 * k4 + 1] + m4[k4].y;
              x[4 * k4 + 2] = x[4 * k4 + 2] + m4[k4].z;
              x[4 * k4 + 3] = x[4 * k4 + 3] + m4[k4].w;
            }
          } else {
#pragma unroll
            for (int k = 0; k < KPL; ++k)
              if (j0 + k < kend) x[k] = x[k] + mrow[j0 + k];
          }
        }
        if constexpr (VEC) {
          if (sb + TPS * kTile > kend) {  // a slot reaching past the row or the cut (uniform)
            if constexpr (EXCL) {
              const int nv = lim - sb;
#pragma unroll
              for (int k = 0; k < KPL; ++k) x[k] = (k < nv) ? x[k] : kNegInf;
            } else {
              const bool inb = j0 < N;  // N is a multiple of the chunk here
#pragma unroll
              for (int k = 0; k < KPL; ++k) x[k] = inb ? x[k] : kNegInf;
            }
          }
        }
        m = tile_max<DT>(lane_tree_max<KPL>(x));
        // a tile whose max is -inf has only -inf keys: subtracting 0 keeps
        // them at -inf and every e at +0, without a -inf - -inf
        const float msafe = (m == kNegInf) ? 0.0f : m;
#pragma unroll
        for (int k = 0; k < KPL; ++k) e[s][k] = exp_(x[k] - msafe);
        l = tile_sum<DT>(lane_tree_sum<KPL>(e[s]));
      }
      if (ix.cil == 0 && t < T) {
        lds_m[ix.rib][t] = m;
        lds_l[ix.rib][t] = l;
      }
    }
    row_sync<WPR>();

    if (active) {
      // ---- merge of the tile states, lane t holds tile t ----
      const float mt = (lane < T) ? lds_m[ix.rib][lane] : kNegInf;
      const float lt = (lane < T) ? lds_l[ix.rib][lane] : 0.0f;
      float Mi = mt;  // running max after tile `lane` (inclusive prefix max)
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) Mi = fmax2(Mi, __shfl_up(Mi, d));
      float Me = __shfl_up(Mi, 1);  // running max before tile `lane`
      if (lane == 0) Me = kNegInf;
      float alpha = 0.0f, qv = 0.0f;
      if (Mi != kNegInf) {
        alpha = (Me == kNegInf) ? 0.0f : exp_(Me - Mi);
        const float beta = (mt == kNegInf) ? 0.0f : exp_(mt - Mi);
        qv = lt * beta;
      }
      float L = 0.0f;
      for (int t = 0; t < T; ++t) {
        const float La = L * readlane(alpha, t);
        L = La + readlane(qv, t);
      }
      float M = readlane(Mi, T - 1);
      float sigma = 0.0f;
      if (has_sink) {
        sigma = a.sink[h];  // one logit per head
        const float Mn = fmax2(M, sigma);
        if (Mn == kNegInf) {
          M = kNegInf;
          L = 0.0f;
        } else {
          const float fa = (M == kNegInf) ? 0.0f : exp_(M - Mn);
          const float fb = (sigma == kNegInf) ? 0.0f : exp_(sigma - Mn);
          const float La = L * fa;
          const float lb = 1.0f * fb;
          L = La + lb;
          M = Mn;
        }
      }
      const float invL = (L == 0.0f) ? 0.0f : 1.0f / L;
      const float ct = (mt == kNegInf) ? 0.0f : exp_(mt - M) * invL;  // tile `lane`'s scale

      // ---- phase 3: rescale, convert once, write ----
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int gs = s * WPR + ix.wir;
        if (gs < nslots) {
          const int sb = gs * TPS * kTile;
          const int j0 = sb + ix.loff;
          float cs = readlane(ct, gs * TPS);
          if constexpr (TPS == 2) {
            const float c1 = readlane(ct, gs * TPS + 1);
            cs = ix.half ? c1 : cs;
          }
          float p[KPL];
#pragma unroll
          for (int k = 0; k < KPL; ++k) p[k] = e[s][k] * cs;
          const Chunk out = pack<DT>(p);
          if constexpr (VEC) bstore(pbuf, voff, (uint32_t)(sb * ESZ), out);
          else store_chunk_elems<DT>(prow, j0, N, out);
        }
      }
      if (has_sink && ix.wir == 0 && lane == 0)
        a.p_sink[r] = (sigma == kNegInf) ? 0.0f : exp_(sigma - M) * invL;
      if (a.lse && ix.wir == 0 && lane == 0)
        a.lse[r] = (L == 0.0f) ? kNegInf : M + ln_(L);
    }
    if constexpr (WPR > 1) __syncthreads();  // LDS is reused by the next row group
    else wave_sync();
  }
}

// ---------------------------------------------------------------------------
// Backward: phase 1 loads P and dP for the whole row, phase 2 forms the tile
// sums of P*dP, the fold runs over the tile sums in order, phase 3 writes dS.
// ---------------------------------------------------------------------------

template <int DT, int WPR, int CPL, bool VEC, bool EXCL>
__global__ __launch_bounds__(kWave * kBlockWaves) void bwd_kernel(const BwdArgs a) {
  using C = Cfg<DT>;
  constexpr int KPL = C::KPL, TPS = C::TPS, ESZ = C::ESZ;
  __shared__ float lds_d[kBlockWaves][kMaxTiles];

  const RowIdx<DT, WPR> ix;
  const int lane = ix.lane;
  const int T = a.s.T;
  const int N = (int)a.s.N;
  const int nslots = (T + TPS - 1) / TPS;
  const int64_t ngroups = (a.s.rows + ix.rpb - 1) / ix.rpb;
  const bool has_sink = a.p_sink != nullptr;

  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t r = grp * ix.rpb + ix.rib;
    const bool active = r < a.s.rows;
    const int64_t rr = active ? r : a.s.rows - 1;  // spare rows (element-wise path)
    const char *prow = static_cast<const char *>(a.probs) + rr * a.s.ld * ESZ;
    const char *grow = static_cast<const char *>(a.dprobs) + rr * a.s.ld * ESZ;
    char *drow = static_cast<char *>(a.dscores) + r * a.s.ld * ESZ;
    int kend = N;  // P is taken as +0 past the visible keys and not read there
    if constexpr (EXCL) {
      const int64_t q = rr % a.s.Sq;
      kend = row_kend(a.ex, N, a.s.Sq, rr / (a.s.Sq * a.s.H), q);
    }
    const int kread = EXCL ? (kend + KPL - 1) / KPL * KPL : N;
    const int lim = kend - ix.loff;  // as in the forward
    const uint32_t row_bytes = active ? (uint32_t)(N * ESZ) : 0u;
    const Buf pbuf(prow, active ? (uint32_t)(kread * ESZ) : 0u);
    const Buf gbuf(grow, row_bytes), dbuf(drow, row_bytes);
    const uint32_t voff = (uint32_t)(ix.loff * ESZ);

    // ---- phase 1: issue every load of the row, straight-line; keys past
    // the row (P: past the visible keys) read as +0 ----
    Chunk rp[CPL], rg[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int sb = (s * WPR + ix.wir) * TPS * kTile;
      if constexpr (VEC) {
        rp[s] = bload<kAuxNT>(pbuf, voff, (uint32_t)(sb * ESZ));
        rg[s] = bload<kAuxNT>(gbuf, voff, (uint32_t)(sb * ESZ));
      } else {
        rp[s] = load_chunk_elems<DT>(prow, sb + ix.loff, kend, 0u);
        rg[s] = load_chunk_elems<DT>(grow, sb + ix.loff, N, 0u);
      }
    }

    // ---- phase 2: tile sums of P*dP; keys past the row count as +0 ----
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int t = (s * WPR + ix.wir) * TPS + ix.half;
      if constexpr (VEC && EXCL) {
        const int sb = (s * WPR + ix.wir) * TPS * kTile;
        if (sb + TPS * kTile > kend && sb < kread) {  // the slot holding the cut (uniform)
          const int nv = lim - sb;  // this lane's visible keys in its chunk
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // keys at or past kend: P = +0
            if constexpr (DT != 0)  // two 16-bit keys per word, low half first
              rp[s].w[i] &= (nv > 2 * i ? 0x0000ffffu : 0u) | (nv > 2 * i + 1 ? 0xffff0000u : 0u);
            else
              rp[s].w[i] = nv > i ? rp[s].w[i] : 0u;
          }
        }
      }
      float p[KPL], g[KPL], pg[KPL];
      unpack<DT>(rp[s], p);
      unpack<DT>(rg[s], g);
#pragma unroll
      for (int k = 0; k < KPL; ++k) pg[k] = p[k] * g[k];
      const float d = tile_sum<DT>(lane_tree_sum<KPL>(pg));
      if (ix.cil == 0 && t < T) lds_d[ix.rib][t] = d;
    }
    row_sync<WPR>();

    if (active) {
      const float dt = (lane < T) ? lds_d[ix.rib][lane] : 0.0f;
      float delta = readlane(dt, 0);  // the fold starts from the first tile's sum
      for (int t = 1; t < T; ++t) delta = delta + readlane(dt, t);

      // ---- phase 3: dS = P * (dP - delta), convert once, write ----
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int gs = s * WPR + ix.wir;
        if (gs < nslots) {
          const int sb = gs * TPS * kTile;
          const int j0 = sb + ix.loff;
          float p[KPL], g[KPL], ds[KPL];
          unpack<DT>(rp[s], p);
          unpack<DT>(rg[s], g);
#pragma unroll
          for (int k = 0; k < KPL; ++k) {
            const float gd = g[k] - delta;
            ds[k] = p[k] * gd;
          }
          const Chunk out = pack<DT>(ds);
          if constexpr (VEC) bstore(dbuf, voff, (uint32_t)(sb * ESZ), out);
          else store_chunk_elems<DT>(drow, j0, N, out);
        }
      }
      if (has_sink && ix.wir == 0 && lane == 0) a.v[r] = -(a.p_sink[r] * delta);
    }
    if constexpr (WPR > 1) __syncthreads();
    else wave_sync();
  }
}

// ---------------------------------------------------------------------------
// Streaming kernels, for rows longer than one pass keeps in registers (and
// for any row when asked for).  A row belongs to one workgroup of 4 waves
// (8 for the 16-bit backward of rows up to 65,536 keys) and is cut into
// segments of WPR x CPL slots.  Pass 1 reduces each segment's tiles exactly
// as the one-pass kernels do and keeps every tile state in LDS; wave 0 then
// folds the states in tile order, 64 tiles at a time with the running state
// carried from block to block (the same left fold); pass 2 writes the
// outputs segment by segment, last segment first: the last one (the last two
// in the forward) is still in registers, the ones just before wait in an
// LDS stash (one segment in the forward, P of two in the 4-wave backward, P
// of one in the 8-wave backward), the others are read again (the forward
// loads the next segment while it writes the current one).  The forward
// recomputes every segment's
// exponentials from the raw chunks and the saved tile maxima -- the same
// operations on the same inputs, so every output has the one-pass kernels'
// bits.
// ---------------------------------------------------------------------------

// Start of the streaming kernels' segment stash in their dynamic LDS, in
// 4-byte words after `used` words of tile states (16-byte aligned).
__host__ __device__ constexpr int stash_offset_words(int used) { return (used + 3) & ~3; }

// The stash holds the raw chunks of the segments just before those that stay
// in registers (the forward keeps the last two, the backward the last one),
// one segment being 256 threads x CPL x 16 bytes; pass 2 reads them from LDS
// instead of reading them again.  Segments of more than 32 KB are not
// stashed, and each direction has its own LDS budget, from measurements on
// MI355X with bf16 rows of 65,536 keys (4 segments of 32 KB; 1, 2 and 3
// segments stashed leave 3 or 4, 2 and 1 workgroups per CU), taken when
// both directions kept only the last segment in registers:
//   forward:  0.422, 0.595, 1.014 ms  -> 1 segment
//   backward: 0.667, 0.639, 0.883 ms  -> 2 segments
// The forward, which keeps a second register set of chunks to load ahead,
// needs the workgroups more than it needs fewer second reads; holding the
// segment before the last in that second set too leaves one segment of the
// four to read twice (0.393 ms against 0.416 ms).
constexpr int kStashSegMaxBytes = 32 * 1024;
constexpr int kStashBudgetFwd = 32 * 1024;
constexpr int kStashBudgetBwd = 64 * 1024;
// the wide workgroup (8 waves, two per CU): one segment of up to 64 KB in
// the stash, in either direction
constexpr int kWideStashSegMaxBytes = 64 * 1024;
constexpr int kWideStashBudget = 64 * 1024;
template <int CPL, int WPR = kBlockWaves>
constexpr size_t stash_bytes() { return (size_t)CPL * kWave * WPR * 16; }

// Segments a streaming row of T tiles is cut into, and how many of them the
// stash holds within `budget` bytes (never more than the row has before its
// last segment).
template <int DT, int CPL, int WPR = kBlockWaves>
__host__ __device__ constexpr int stream_segments(int T) {
  return ((T + Cfg<DT>::TPS - 1) / Cfg<DT>::TPS + WPR * CPL - 1) / (WPR * CPL);
}
// held: segments that stay in registers between the passes (the forward
// keeps the last two, the backward the last one).
template <int DT, int CPL, int WPR = kBlockWaves>
constexpr int stash_segments(int T, int budget, int held) {
  if constexpr (WPR != kBlockWaves) budget = kWideStashBudget;
  const size_t seg_max = WPR == kBlockWaves ? kStashSegMaxBytes : kWideStashSegMaxBytes;
  if (stash_bytes<CPL, WPR>() > seg_max) return 0;
  const int want = stream_segments<DT, CPL, WPR>(T) - held;
  const int fit = (int)((size_t)budget / stash_bytes<CPL, WPR>());
  return want < fit ? (want > 0 ? want : 0) : fit;
}

template <int DT, int CPL, int WPR, bool VEC, bool MASK, bool EXCL>
__global__ __launch_bounds__(kWave * WPR) void fwd_stream_kernel(const FwdArgs a) {
  using C = Cfg<DT>;
  constexpr int KPL = C::KPL, TPS = C::TPS, ESZ = C::ESZ;
  constexpr uint32_t kFill = kNegInfBits<DT>;
  constexpr int SPS = WPR * CPL;  // slots per segment
  extern __shared__ float smem[];
  const int T = a.s.T;
  float *lds_m = smem;            // [T] tile maxima
  float *lds_l = smem + T;        // [T] tile sums
  float *lds_row = smem + 2 * T;  // the row's M and invL
  // a.stash segments' raw chunks, those just before the last segment (the
  // first ones pass 2 would read again), CPL x 256 threads x 16 bytes each,
  // each thread's own
  Chunk *lds_stash = reinterpret_cast<Chunk *>(smem + stash_offset_words(2 * T + 2));

  const RowIdx<DT, WPR> ix;
  const int lane = ix.lane;
  const int N = (int)a.s.N;
  const int nslots = (T + TPS - 1) / TPS;
  const int nseg = (nslots + SPS - 1) / SPS;
  const bool has_sink = a.sink != nullptr;

  for (int64_t r = blockIdx.x; r < a.s.rows; r += gridDim.x) {
    const char *srow = static_cast<const char *>(a.scores) + r * a.s.ld * ESZ;
    char *prow = static_cast<char *>(a.probs) + r * a.s.ld * ESZ;
    const float *mrow = nullptr;
    int64_t h = 0;
    int kend = N;
    if (MASK || has_sink || EXCL) {
      const int64_t q = r % a.s.Sq;
      const int64_t bh = r / a.s.Sq;
      h = bh % a.s.H;
      if constexpr (MASK) mrow = a.mask + (bh / a.s.H) * a.msb + h * a.msh + q * a.msq;
      if constexpr (EXCL) kend = row_kend(a.ex, N, a.s.Sq, bh / a.s.H, q);
    }
    const int kread = EXCL ? (kend + KPL - 1) / KPL * KPL : N;
    const Buf sbuf(srow, (uint32_t)(kread * ESZ));
    const Buf pbuf(prow, (uint32_t)(N * ESZ));
    const Buf mbuf(mrow, MASK ? (uint32_t)(kread * 4) : 0u);
    const uint32_t voff = (uint32_t)(ix.loff * ESZ);
    const int lim = kend - ix.loff;

    // Two register sets of one segment's raw chunks, A and B, taking turns:
    // one is reduced while the next segment loads into the other, so at the
    // end of pass 1 the last two segments are both still in registers.
    // Exponentials are not kept: pass 2 recomputes them for every segment
    // from the raw chunks and the tile maxima, the operations of pass 1 on
    // the same inputs.
    Chunk A[CPL], B[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) A[s] = B[s] = Chunk{{0u, 0u, 0u, 0u}};
    // aux: the cache policy (normal for a segment read again in pass 2, so
    // that the second read can hit the caches; nontemporal for a last read)
    auto load_segment = [&](Chunk (&dst)[CPL], int g, auto aux) {
      constexpr int AX = decltype(aux)::value;
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int sb = (g * SPS + s * WPR + ix.wir) * TPS * kTile;
        if constexpr (VEC) dst[s] = bload<AX>(sbuf, voff, (uint32_t)(sb * ESZ));
        else dst[s] = load_chunk_elems<DT>(srow, sb + ix.loff, kend, kFill);
      }
    };
    // the slot's keys as binary32 with the mask added and every key past
    // the row or the cut at -inf; false when the whole slot is past them
    auto slot_x = [&](int g, int s, const Chunk &raw, float (&x)[KPL]) -> bool {
      const int sb = (g * SPS + s * WPR + ix.wir) * TPS * kTile;
      if (sb >= kend) return false;  // uniform
      const int j0 = sb + ix.loff;
      unpack<DT>(raw, x);
      if constexpr (MASK) {
        if constexpr (VEC) {
#pragma unroll
          for (int k4 = 0; k4 < KPL / 4; ++k4) {
            const Chunk c = bload<0>(mbuf, (uint32_t)(ix.loff * 4 + 16 * k4), (uint32_t)(sb * 4));
            x[4 * k4 + 0] = x[4 * k4 + 0] + u2f(c.w[0]);
            x[4 * k4 + 1] = x[4 * k4 + 1] + u2f(c.w[1]);
            x[4 * k4 + 2] = x[4 * k4 + 2] + u2f(c.w[2]);
            x[4 * k4 + 3] = x[4 * k4 + 3] + u2f(c.w[3]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < KPL; ++k)
            if (j0 + k < kend) x[k] = x[k] + mrow[j0 + k];
        }
      }
      if constexpr (VEC) {
        if (sb + TPS * kTile > kend) {  // the slot reaching past the row or the cut (uniform)
          const int nv = lim - sb;
#pragma unroll
          for (int k = 0; k < KPL; ++k) x[k] = (k < nv) ? x[k] : kNegInf;
        }
      }
      return true;
    };

    // segments wholly past the cut hold only -inf keys: nothing to load
    const int nseg_read = EXCL ? (kend + SPS * TPS * kTile - 1) / (SPS * TPS * kTile) : nseg;
    // the last two segments stay in registers; the stash holds the ones
    // just before them, gs0 .. nseg - 3; the rest are read again
    const int before = nseg > 2 ? nseg - 2 : 0;  // segments before the last two
    const int gs0 = nseg - 2 - (a.stash < before ? a.stash : before);
    auto load_pass1 = [&](Chunk (&dst)[CPL], int g) {
      if (g < gs0) load_segment(dst, g, AuxC<0>{});  // read again in pass 2
      else load_segment(dst, g, AuxC<kAuxNT>{});
    };

    // ---- pass 1: tile states of every segment into LDS ----
    // segment g in c while segment g + 1 loads into n
    // (the scheduling barrier keeps a segment's loads from rising above the
    // work on the one before: three register sets live at once would cost
    // occupancy)
    auto p1seg = [&](Chunk (&c)[CPL], Chunk (&n)[CPL], int g) {
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < nseg_read) load_pass1(n, g + 1);
      if (g >= gs0 && g < nseg - 2 && g < nseg_read) {
        Chunk *st = lds_stash + (g - gs0) * CPL * kWave * WPR;
#pragma unroll
        for (int s = 0; s < CPL; ++s) st[s * kWave * WPR + threadIdx.x] = c[s];
      }
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int t = (g * SPS + s * WPR + ix.wir) * TPS + ix.half;
        float x[KPL];
        float m = kNegInf, l = 0.0f;
        if (slot_x(g, s, c[s], x)) {
          m = tile_max<DT>(lane_tree_max<KPL>(x));
          const float msafe = (m == kNegInf) ? 0.0f : m;
          float e[KPL];
#pragma unroll
          for (int k = 0; k < KPL; ++k) e[k] = exp_(x[k] - msafe);
          l = tile_sum<DT>(lane_tree_sum<KPL>(e));
        }
        if (ix.cil == 0 && t < T) {
          lds_m[t] = m;
          lds_l[t] = l;
        }
      }
    };
    if (nseg_read > 0) load_pass1(A, 0);
    for (int g = 0; g < nseg; g += 2) {  // even segments in A, odd ones in B
      p1seg(A, B, g);
      if (g + 1 < nseg) p1seg(B, A, g + 1);
    }
    __syncthreads();

    // ---- the fold, in tile order, 64 tiles per step (wave 0) ----
    if (ix.wir == 0) {
      float Mc = kNegInf, Lc = 0.0f;  // the state after the tiles folded so far
      for (int b0 = 0; b0 < T; b0 += kWave) {
        const int t = b0 + lane;
        const float mt = (t < T) ? lds_m[t] : kNegInf;
        const float lt = (t < T) ? lds_l[t] : 0.0f;
        float Mi = mt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) Mi = fmax2(Mi, __shfl_up(Mi, d));
        Mi = fmax2(Mi, Mc);               // running max after tile t
        float Me = __shfl_up(Mi, 1);      // running max before tile t
        if (lane == 0) Me = Mc;
        float alpha = 0.0f, qv = 0.0f;
        if (Mi != kNegInf) {
          alpha = (Me == kNegInf) ? 0.0f : exp_(Me - Mi);
          const float beta = (mt == kNegInf) ? 0.0f : exp_(mt - Mi);
          qv = lt * beta;
        }
        const int nt = (T - b0 < kWave) ? T - b0 : kWave;
        float L = Lc;
        for (int i = 0; i < nt; ++i) {
          const float La = L * readlane(alpha, i);
          L = La + readlane(qv, i);
        }
        Lc = L;
        Mc = readlane(Mi, nt - 1);
      }
      float M = Mc, L = Lc;
      float sigma = 0.0f;
      if (has_sink) {
        sigma = a.sink[h];
        const float Mn = fmax2(M, sigma);
        if (Mn == kNegInf) {
          M = kNegInf;
          L = 0.0f;
        } else {
          const float fa = (M == kNegInf) ? 0.0f : exp_(M - Mn);
          const float fb = (sigma == kNegInf) ? 0.0f : exp_(sigma - Mn);
          const float La = L * fa;
          const float lb = 1.0f * fb;
          L = La + lb;
          M = Mn;
        }
      }
      const float invL = (L == 0.0f) ? 0.0f : 1.0f / L;
      if (lane == 0) {
        lds_row[0] = M;
        lds_row[1] = invL;
        if (has_sink) a.p_sink[r] = (sigma == kNegInf) ? 0.0f : exp_(sigma - M) * invL;
        if (a.lse) a.lse[r] = (L == 0.0f) ? kNegInf : M + ln_(L);
      }
    }
    __syncthreads();
    const float M = lds_row[0], invL = lds_row[1];

    // ---- pass 2: rescale, convert once, write; last segment first ----
    // Segment g is written from c; while it is, segment g - 1 comes into n
    // from the stash or a second read (when asked: the segment before the
    // last is already in the other register set).
    auto p2seg = [&](Chunk (&c)[CPL], Chunk (&n)[CPL], int g, bool fetch) {
      __builtin_amdgcn_sched_barrier(0);
      const int gp = g - 1;
      if (fetch && gp >= 0 && gp < nseg_read) {
        if (gp >= gs0) {
          const Chunk *st = lds_stash + (gp - gs0) * CPL * kWave * WPR;
#pragma unroll
          for (int s = 0; s < CPL; ++s) n[s] = st[s * kWave * WPR + threadIdx.x];
        } else {
          load_segment(n, gp, AuxC<kAuxNT>{});
        }
      }
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int gs = g * SPS + s * WPR + ix.wir;
        if (gs < nslots) {
          const int sb = gs * TPS * kTile;
          const int t = gs * TPS + ix.half;
          const float mt = lds_m[t < T ? t : T - 1];
          float e[KPL];
          float x[KPL];
          if (slot_x(g, s, c[s], x)) {
            const float msafe = (mt == kNegInf) ? 0.0f : mt;
#pragma unroll
            for (int k = 0; k < KPL; ++k) e[k] = exp_(x[k] - msafe);
          } else {
#pragma unroll
            for (int k = 0; k < KPL; ++k) e[k] = 0.0f;
          }
          const float cs = (mt == kNegInf) ? 0.0f : exp_(mt - M) * invL;
          float p[KPL];
#pragma unroll
          for (int k = 0; k < KPL; ++k) p[k] = e[k] * cs;
          const Chunk out = pack<DT>(p);
          if constexpr (VEC) bstore(pbuf, voff, (uint32_t)(sb * ESZ), out);
          else store_chunk_elems<DT>(prow, sb + ix.loff, N, out);
        }
      }
    };
    // the last segment into B, the one before it into A
    if (((nseg - 1) & 1) == 0) {
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const Chunk t = A[s];
        A[s] = B[s];
        B[s] = t;
      }
    }
    p2seg(B, A, nseg - 1, false);
    for (int g = nseg - 2; g >= 0; g -= 2) {
      p2seg(A, B, g, true);
      if (g >= 1) p2seg(B, A, g - 1, true);
    }
    __syncthreads();  // LDS is reused by the next row
  }
}

template <int DT, int CPL, int WPR, bool VEC, bool EXCL>
__global__ __launch_bounds__(kWave * WPR) void bwd_stream_kernel(const BwdArgs a) {
  using C = Cfg<DT>;
  constexpr int KPL = C::KPL, TPS = C::TPS, ESZ = C::ESZ;
  constexpr int SPS = WPR * CPL;
  extern __shared__ float smem[];
  const int T = a.s.T;
  float *lds_d = smem;            // [T] tile sums of P*dP
  float *lds_row = smem + T;      // delta
  // a.stash segments' P chunks (as masked), those just before the last
  // segment, each thread's own
  Chunk *lds_stash = reinterpret_cast<Chunk *>(smem + stash_offset_words(T + 1));

  const RowIdx<DT, WPR> ix;
  const int lane = ix.lane;
  const int N = (int)a.s.N;
  const int nslots = (T + TPS - 1) / TPS;
  const int nseg = (nslots + SPS - 1) / SPS;
  const bool has_sink = a.p_sink != nullptr;

  for (int64_t r = blockIdx.x; r < a.s.rows; r += gridDim.x) {
    const char *prow = static_cast<const char *>(a.probs) + r * a.s.ld * ESZ;
    const char *grow = static_cast<const char *>(a.dprobs) + r * a.s.ld * ESZ;
    char *drow = static_cast<char *>(a.dscores) + r * a.s.ld * ESZ;
    int kend = N;
    if constexpr (EXCL) kend = row_kend(a.ex, N, a.s.Sq, r / (a.s.Sq * a.s.H), r % a.s.Sq);
    const int kread = EXCL ? (kend + KPL - 1) / KPL * KPL : N;
    const Buf pbuf(prow, (uint32_t)(kread * ESZ));
    const Buf gbuf(grow, (uint32_t)(N * ESZ)), dbuf(drow, (uint32_t)(N * ESZ));
    const uint32_t voff = (uint32_t)(ix.loff * ESZ);
    const int lim = kend - ix.loff;

    Chunk rp[CPL], rg[CPL];
    // auxp, auxg: cache policies of P and dP, as in the forward
    auto load_segment = [&](int g, auto auxp, auto auxg) {
      constexpr int AP = decltype(auxp)::value, AG = decltype(auxg)::value;
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int sb = (g * SPS + s * WPR + ix.wir) * TPS * kTile;
        if constexpr (VEC) {
          rp[s] = bload<AP>(pbuf, voff, (uint32_t)(sb * ESZ));
          rg[s] = bload<AG>(gbuf, voff, (uint32_t)(sb * ESZ));
          if constexpr (EXCL) {
            if (sb + TPS * kTile > kend && sb < kread) {  // the slot holding the cut (uniform)
              const int nv = lim - sb;
#pragma unroll
              for (int i = 0; i < 4; ++i) {  // keys at or past kend: P = +0
                if constexpr (DT != 0)
                  rp[s].w[i] &= (nv > 2 * i ? 0x0000ffffu : 0u) | (nv > 2 * i + 1 ? 0xffff0000u : 0u);
                else
                  rp[s].w[i] = nv > i ? rp[s].w[i] : 0u;
              }
            }
          }
        } else {
          rp[s] = load_chunk_elems<DT>(prow, sb + ix.loff, kend, 0u);
          rg[s] = load_chunk_elems<DT>(grow, sb + ix.loff, N, 0u);
        }
      }
    };

    auto load_g = [&](int g) {  // dP only, for the segment whose P is in LDS
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int sb = (g * SPS + s * WPR + ix.wir) * TPS * kTile;
        if constexpr (VEC) rg[s] = bload<kAuxNT>(gbuf, voff, (uint32_t)(sb * ESZ));
        else rg[s] = load_chunk_elems<DT>(grow, sb + ix.loff, N, 0u);
      }
    };
    // the stash holds P of segments gs0 .. nseg - 2
    const int gs0 = nseg - 1 - (a.stash < nseg - 1 ? a.stash : nseg - 1);

    // ---- pass 1: tile sums of P*dP into LDS ----
    for (int g = 0; g < nseg; ++g) {
      // P and dP read again in pass 2 keep the normal cache policy
      if (g < gs0) load_segment(g, AuxC<0>{}, AuxC<0>{});
      else if (g < nseg - 1) load_segment(g, AuxC<kAuxNT>{}, AuxC<0>{});
      else load_segment(g, AuxC<kAuxNT>{}, AuxC<kAuxNT>{});
      if (g >= gs0 && g < nseg - 1) {
        Chunk *st = lds_stash + (g - gs0) * CPL * kWave * WPR;
#pragma unroll
        for (int s = 0; s < CPL; ++s) st[s * kWave * WPR + threadIdx.x] = rp[s];
      }
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int t = (g * SPS + s * WPR + ix.wir) * TPS + ix.half;
        float p[KPL], gv[KPL], pg[KPL];
        unpack<DT>(rp[s], p);
        unpack<DT>(rg[s], gv);
#pragma unroll
        for (int k = 0; k < KPL; ++k) pg[k] = p[k] * gv[k];
        const float d = tile_sum<DT>(lane_tree_sum<KPL>(pg));
        if (ix.cil == 0 && t < T) lds_d[t] = d;
      }
    }
    __syncthreads();

    // ---- delta: the tile sums folded left to right from the first (wave 0) ----
    if (ix.wir == 0) {
      float delta = 0.0f;
      for (int b0 = 0; b0 < T; b0 += kWave) {
        const int t = b0 + lane;
        const float dt = (t < T) ? lds_d[t] : 0.0f;
        const int nt = (T - b0 < kWave) ? T - b0 : kWave;
        for (int i = 0; i < nt; ++i) delta = (b0 + i == 0) ? readlane(dt, 0) : delta + readlane(dt, i);
      }
      if (lane == 0) {
        lds_row[0] = delta;
        if (has_sink) a.v[r] = -(a.p_sink[r] * delta);
      }
    }
    __syncthreads();
    const float delta = lds_row[0];

    // ---- pass 2: dS = P * (dP - delta), convert once, write; last segment first ----
    for (int g = nseg - 1; g >= 0; --g) {
      if (g != nseg - 1) {
        if (g >= gs0) {
          const Chunk *st = lds_stash + (g - gs0) * CPL * kWave * WPR;
#pragma unroll
          for (int s = 0; s < CPL; ++s) rp[s] = st[s * kWave * WPR + threadIdx.x];
          load_g(g);
        } else {
          load_segment(g, AuxC<kAuxNT>{}, AuxC<kAuxNT>{});
        }
      }
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int gs = g * SPS + s * WPR + ix.wir;
        if (gs < nslots) {
          const int sb = gs * TPS * kTile;
          float p[KPL], gv[KPL], ds[KPL];
          unpack<DT>(rp[s], p);
          unpack<DT>(rg[s], gv);
#pragma unroll
          for (int k = 0; k < KPL; ++k) {
            const float gd = gv[k] - delta;
            ds[k] = p[k] * gd;
          }
          const Chunk out = pack<DT>(ds);
          if constexpr (VEC) bstore(dbuf, voff, (uint32_t)(sb * ESZ), out);
          else store_chunk_elems<DT>(drow, sb + ix.loff, N, out);
        }
      }
    }
    __syncthreads();  // LDS is reused by the next row
  }
}

// ---------------------------------------------------------------------------
// Launch tables
// ---------------------------------------------------------------------------

// chunks-per-lane sizes compiled for each dtype (register budget: the row's
// share is kept in registers between the reduction and the write); the
// 16-bit types share one list.  The streaming kernels have their own
// (a segment is 4 waves x CPL slots: 64 tiles at the larger size).
constexpr int kCplF32[] = {1, 2, 3, 5, 9, 17};
constexpr int kCplBf16[] = {1, 2, 3, 5, 9};
constexpr int kStreamCplF32[] = {8, 16};
constexpr int kStreamCplBf16[] = {4, 8};

// A kernel whose LDS passes 64 KB asks for the larger allocation (up to the
// 160 KB of a gfx950 CU) before its launch.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// The wide workgroup (8 waves) is built for 16-byte rows only: rows on the
// element-wise path take the 4-wave one, with the same bits.
template <int DT, int CPL, int WPR>
hipError_t launch_fwd_stream(const FwdArgs &a0, const Geometry &g, hipStream_t st) {
  if constexpr (WPR != kBlockWaves) {
    if (!a0.vec_io) return launch_fwd_stream<DT, CPL, kBlockWaves>(a0, g, st);
  }
  const dim3 grid((unsigned)g.blocks), block(kWave * WPR);
  FwdArgs a = a0;
  a.stash = stash_segments<DT, CPL, WPR>(a.s.T, kStashBudgetFwd, 2);
  const size_t lds = (size_t)stash_offset_words(2 * a.s.T + 2) * sizeof(float) +
                     (size_t)a.stash * stash_bytes<CPL, WPR>();
  const bool mask = a.mask != nullptr, excl = a.ex.causal || a.ex.key_len;
#define JAS_FWD_STREAM(V, MK, EX)                                                              \
  do {                                                                                         \
    const hipError_t e = allow_lds(fwd_stream_kernel<DT, CPL, WPR, V, MK, EX>, lds);           \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((fwd_stream_kernel<DT, CPL, WPR, V, MK, EX>), grid, block, lds, st, a); \
  } while (0)
  if (a.vec_io) {
    if (excl) { if (mask) JAS_FWD_STREAM(true, true, true); else JAS_FWD_STREAM(true, false, true); }
    else { if (mask) JAS_FWD_STREAM(true, true, false); else JAS_FWD_STREAM(true, false, false); }
  } else if constexpr (WPR == kBlockWaves) {
    if (excl) { if (mask) JAS_FWD_STREAM(false, true, true); else JAS_FWD_STREAM(false, false, true); }
    else { if (mask) JAS_FWD_STREAM(false, true, false); else JAS_FWD_STREAM(false, false, false); }
  }
#undef JAS_FWD_STREAM
  return hipGetLastError();
}

template <int DT, int CPL, int WPR>
hipError_t launch_bwd_stream(const BwdArgs &a0, const Geometry &g, hipStream_t st) {
  if constexpr (WPR != kBlockWaves) {
    if (!a0.vec_io) return launch_bwd_stream<DT, CPL, kBlockWaves>(a0, g, st);
  }
  const dim3 grid((unsigned)g.blocks), block(kWave * WPR);
  BwdArgs a = a0;
  a.stash = stash_segments<DT, CPL, WPR>(a.s.T, kStashBudgetBwd, 1);
  const size_t lds = (size_t)stash_offset_words(a.s.T + 1) * sizeof(float) +
                     (size_t)a.stash * stash_bytes<CPL, WPR>();
  const bool excl = a.ex.causal || a.ex.key_len;
#define JAS_BWD_STREAM(V, EX)                                                              \
  do {                                                                                     \
    const hipError_t e = allow_lds(bwd_stream_kernel<DT, CPL, WPR, V, EX>, lds);           \
    if (e != hipSuccess) return e;                                                         \
    hipLaunchKernelGGL((bwd_stream_kernel<DT, CPL, WPR, V, EX>), grid, block, lds, st, a); \
  } while (0)
  if (a.vec_io) {
    if (excl) JAS_BWD_STREAM(true, true);
    else JAS_BWD_STREAM(true, false);
  } else if constexpr (WPR == kBlockWaves) {
    if (excl) JAS_BWD_STREAM(false, true);
    else JAS_BWD_STREAM(false, false);
  }
#undef JAS_BWD_STREAM
  return hipGetLastError();
}

// rows with an exclusion (causal or key lengths) run their own instances,
// so the row-level cut costs the dense rows nothing
template <int DT, int WPR, int CPL, bool EXCL>
void launch_fwd_e(const FwdArgs &a, const dim3 grid, const dim3 block, bool mres, hipStream_t st) {
  const bool mask = a.mask != nullptr;
  if constexpr (DT != 0 && WPR == 2 && CPL <= 5) {  // the mask-in-registers instances
    if (mres && mask && a.vec_io) {
      hipLaunchKernelGGL((fwd_kernel<DT, WPR, CPL, true, true, EXCL, true>), grid, block, 0, st, a);
      return;
    }
  }
  if (a.vec_io) {
    if (mask) hipLaunchKernelGGL((fwd_kernel<DT, WPR, CPL, true, true, EXCL>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<DT, WPR, CPL, true, false, EXCL>), grid, block, 0, st, a);
  } else {
    if (mask) hipLaunchKernelGGL((fwd_kernel<DT, WPR, CPL, false, true, EXCL>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<DT, WPR, CPL, false, false, EXCL>), grid, block, 0, st, a);
  }
}

template <int DT, int WPR, int CPL>
hipError_t launch_fwd_t(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  const dim3 grid((unsigned)g.blocks), block(kWave * WPR * g.rpb);
  if (a.ex.causal || a.ex.key_len) launch_fwd_e<DT, WPR, CPL, true>(a, grid, block, g.mres != 0, st);
  else launch_fwd_e<DT, WPR, CPL, false>(a, grid, block, g.mres != 0, st);
  return hipGetLastError();
}

template <int DT, int WPR, int CPL>
hipError_t launch_bwd_t(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  const dim3 grid((unsigned)g.blocks), block(kWave * WPR * g.rpb);
  const bool excl = a.ex.causal || a.ex.key_len;
  if (a.vec_io) {
    if (excl) hipLaunchKernelGGL((bwd_kernel<DT, WPR, CPL, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((bwd_kernel<DT, WPR, CPL, true, false>), grid, block, 0, st, a);
  } else {
    if (excl) hipLaunchKernelGGL((bwd_kernel<DT, WPR, CPL, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((bwd_kernel<DT, WPR, CPL, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

#define JAS_CPL_CASES(FN, DT, WPR, ARGS)                     \
  switch (g.cpl) {                                           \
    case 1: return FN<DT, WPR, 1> ARGS;                      \
    case 2: return FN<DT, WPR, 2> ARGS;                      \
    case 3: return FN<DT, WPR, 3> ARGS;                      \
    case 5: return FN<DT, WPR, 5> ARGS;                      \
    case 9: return FN<DT, WPR, 9> ARGS;                      \
    default: break;                                          \
  }

template <int DT, int WPR>
hipError_t fwd_wpr(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  JAS_CPL_CASES(launch_fwd_t, DT, WPR, (a, g, st))
  if constexpr (DT == 0) {
    if (g.cpl == 17) return launch_fwd_t<DT, WPR, 17>(a, g, st);
  }
  return hipErrorInvalidValue;
}

template <int DT, int WPR>
hipError_t bwd_wpr(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  JAS_CPL_CASES(launch_bwd_t, DT, WPR, (a, g, st))
  if constexpr (DT == 0) {
    if (g.cpl == 17) return launch_bwd_t<DT, WPR, 17>(a, g, st);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t fwd_dt(const FwdArgs &a, const Geometry &g, hipStream_t st) {
  if (g.stream) {
    constexpr int c0 = DT == 0 ? kStreamCplF32[0] : kStreamCplBf16[0];
    constexpr int c1 = DT == 0 ? kStreamCplF32[1] : kStreamCplBf16[1];
    if (g.wpr == kStreamWideWaves) {  // 16-bit types only (fp32 chunks would not fit in registers)
      if constexpr (DT != 0) {
        if (g.cpl == c1) return launch_fwd_stream<DT, c1, kStreamWideWaves>(a, g, st);
      }
      return hipErrorInvalidValue;
    }
    if (g.cpl == c0) return launch_fwd_stream<DT, c0, kBlockWaves>(a, g, st);
    if (g.cpl == c1) return launch_fwd_stream<DT, c1, kBlockWaves>(a, g, st);
    return hipErrorInvalidValue;
  }
  switch (g.wpr) {
    case 1: return fwd_wpr<DT, 1>(a, g, st);
    case 2: return fwd_wpr<DT, 2>(a, g, st);
    case 4: return fwd_wpr<DT, 4>(a, g, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t bwd_dt(const BwdArgs &a, const Geometry &g, hipStream_t st) {
  if (g.stream) {
    constexpr int c0 = DT == 0 ? kStreamCplF32[0] : kStreamCplBf16[0];
    constexpr int c1 = DT == 0 ? kStreamCplF32[1] : kStreamCplBf16[1];
    if (g.wpr == kStreamWideWaves) {  // 16-bit types only (fp32 chunks would not fit in registers)
      if constexpr (DT != 0) {
        if (g.cpl == c1) return launch_bwd_stream<DT, c1, kStreamWideWaves>(a, g, st);
      }
      return hipErrorInvalidValue;
    }
    if (g.cpl == c0) return launch_bwd_stream<DT, c0, kBlockWaves>(a, g, st);
    if (g.cpl == c1) return launch_bwd_stream<DT, c1, kBlockWaves>(a, g, st);
    return hipErrorInvalidValue;
  }
  switch (g.wpr) {
    case 1: return bwd_wpr<DT, 1>(a, g, st);
    case 2: return bwd_wpr<DT, 2>(a, g, st);
    case 4: return bwd_wpr<DT, 4>(a, g, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace jas
