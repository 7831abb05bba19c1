// jas_attn.hip -- fixed-order fused attention forward on gfx950 MFMA: the QK
// product, the row softmax of jas_fwd, and the PV product in one kernel.
//
// Method: RL-Kernel PR #453, Summary (the fixed-order softmax sits between
// the QK GEMM and the AV GEMM; P is rounded once, to the tensor dtype) and
// RL-Kernel PR #240, Fixed Reduction Contract (every score and every output
// element has one writer; the head dimension and the keys are accumulated
// in a fixed order, with no split of the key range).
//
// Mapping to CDNA4.  A workgroup of 4 waves owns 64 queries of one
// (batch, head), each wave 16 of them.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_16x16x32 (bf16 or fp16): A = 16 keys x 32
// dims of K, B = 32 dims x 16 queries of Q (kept in registers for the whole
// row), so lane l holds, for query l%16, four consecutive keys of a 16-key
// block.  Keys go through the workgroup 32 at a time: K (32 keys x D) and
// the transposed V (D x 32 keys) are loaded with coalesced 16-byte loads
// into double-buffered LDS, K two steps and V one step ahead of use, and
// each step issues the next step's QK product before its own softmax work
// (a one-step software pipeline).  LDS row strides are 32 modulo 64 bytes,
// which gfx950 serves without bank conflicts for these reads.  Workgroups
// are renumbered so that one XCD works on neighbouring query blocks of one
// head (its K and V stay in that XCD's L2); with the causal flag a head's
// blocks go longest first.  In
// each 32-key step the A rows are assigned so that lane group g (= l/16)
// holds keys 8g .. 8g + 7 (the first block the first four, the second block
// the next four).  The softmax tile tree is then exact: in-lane pairs and
// quads, the two blocks in-lane, lane groups g and g^1 with
// permlane16_swap, groups {0,1} and {2,3} with permlane32_swap, then the 8
// steps of the 256-key tile in registers -- the balanced pairwise tree over
// the tile's keys in order.  The same registers, rounded to the tensor
// dtype, are the A operand of the PV product (16 queries x 32 keys, lane
// group g holding 8 consecutive keys), so P never leaves the registers; B
// is 32 keys x 16 dims of V, read from the LDS copy of the transposed V,
// which the library writes into the caller's workspace first (dims x keys,
// zero-padded to whole tiles).
//
// The softmax is done in two passes over the keys, so that P is exactly the
// row softmax of the binary32 scores (the bits jas_fwd gives on them):
// pass 1 computes each tile's (max, sum), keeps the max in LDS, and merges
// the pair into the query's running state in tile order (then the sink);
// pass 2 recomputes the scores 32 keys at a time, forms P = e * c_t, rounds
// it, and accumulates P V into fp32 registers in key order.  QK is computed
// twice, PV once.  Accumulation inside one MFMA follows the hardware's
// fixed order; every launch computes every output the same way, so results
// do not depend on batch, position or grid.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jas_kernels.h"

namespace jas {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAttnWaves = 4;  // waves per workgroup, each on its own queries

template <int DT>
__device__ __forceinline__ f32x4_t mfma32(const u32x4 a, const u32x4 b, const f32x4_t c) {
  if constexpr (DT == 1)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == 1) return pack_bf16(lo, hi);
  else return pack_f16(lo, hi);
}

__device__ __forceinline__ u32x4 bload4(const Buf &b, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)voff, (int)soff, 0);
}

// Sum over the 64 lanes' groups of 16 (lane groups g = 0..3 in order) as the
// two top levels of a balanced tree: (g0 + g1) + (g2 + g3).
__device__ __forceinline__ float groups4_sum(float v) {
  const f32x2_t p = rows16_pair(v);
  v = p[0] + p[1];
  const f32x2_t h = halves32_pair(v);
  return h[0] + h[1];
}

__device__ __forceinline__ float groups4_max(float v) {
  const f32x2_t p = rows16_pair(v);
  v = fmax2(p[0], p[1]);
  const f32x2_t h = halves32_pair(v);
  return fmax2(h[0], h[1]);
}

// The hardware hands workgroups to the 8 XCDs round-robin (workgroup i to
// XCD i % 8), and each XCD has its own L2.  Renumber so that the workgroups
// on one XCD take consecutive units, i.e. neighbouring query blocks of one
// (batch, head), whose K and V then stay in that XCD's L2.  A bijection on
// [0, G) for any G; which workgroup computes a unit never changes its bytes.
__device__ __forceinline__ int64_t xcd_unit(int64_t bid, int64_t G) {
  const int64_t x = bid % 8, per = G / 8, rem = G % 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + bid / 8;
}

// MASK: an additive mask is given; WRITE: the scores and / or P are written
// out as well (for checking), which the fast path does not carry.
template <int DT, int D, bool MASK, bool WRITE>
__global__ __launch_bounds__(kWave * kAttnWaves) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int ESZ = 2;
  constexpr int DS = D / 32;       // k-steps of the QK product
  constexpr int DB = D / 16;       // 16-dim column blocks of the output
  constexpr int SUB = 32;          // keys per staged sub-tile (one PV k-step)
  // LDS rows: a 16-byte read by each lane of 16 rows (lane groups 16 bytes
  // apart) is free of bank conflicts on gfx950 when the row stride is 32
  // modulo 64 bytes (measured; strides 16 modulo 32 bytes cost 4 extra
  // cycles per read): K rows of D + 16 elements, V^T rows of 48
  constexpr int KROW = D + 16;     // LDS row of K (elements)
  constexpr int VROW = SUB + 16;   // LDS row of V^T
  constexpr int KCH = SUB * D / 8 / (kWave * kAttnWaves);  // 16-byte chunks per thread
  constexpr int VCH = D * SUB / 8 / (kWave * kAttnWaves);
  static_assert(KCH >= 1 && VCH >= 1, "sub-tile smaller than the workgroup");
  __shared__ __align__(16) uint16_t lk[2][SUB * KROW];
  __shared__ __align__(16) uint16_t lv[2][D * VROW];
  extern __shared__ float lds_m[];  // per wave T x 16 tile maxima (sized at launch)

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15;  // the lane's query (S^T column) and A/B operand row
  const int g = lane >> 4;    // lane group: keys 8g .. 8g+7 of each 32-key step
  const int N = (int)a.N, T = a.T, Np = a.Np;
  const int Sq = (int)a.Sq;
  const int64_t qgroups = (a.Sq + 63) / 64;  // 64 queries per workgroup
  const int64_t units = a.B * a.H * qgroups;
  float *sm = lds_m + w * a.T * 16;
  const bool has_sink = a.sink != nullptr;
  constexpr bool write_all = WRITE;

  for (int64_t u = xcd_unit(blockIdx.x, gridDim.x); u < units; u += gridDim.x) {
    // causal: a head's query blocks in decreasing cost (the last block sees
    // the most keys), so the cheapest units are the last ones dispatched
    const int64_t qg = a.ex.causal ? qgroups - 1 - u % qgroups : u % qgroups, bh = u / qgroups;
    const int64_t h = bh % a.H, b = bh / a.H;
    const int64_t hk = h / (a.H / a.Hkv);
    const int q0 = (int)(qg * 64) + 16 * w;  // this wave's 16 queries
    const int q = q0 + c16;                  // this lane's query
    const bool qvalid = q < Sq;
    const int64_t row = bh * a.Sq + (qvalid ? q : Sq - 1);

    const Buf qbuf(static_cast<const char *>(a.q) + bh * a.Sq * D * ESZ, (uint32_t)(a.Sq * D * ESZ));
    const Buf kbuf(static_cast<const char *>(a.k) + (b * a.Hkv + hk) * a.N * D * ESZ,
                   (uint32_t)(a.N * D * ESZ));
    const Buf vbuf(static_cast<const char *>(a.vt) + (b * a.Hkv + hk) * (int64_t)D * Np * ESZ,
                   (uint32_t)((int64_t)D * Np * ESZ));

    // Q^T operand (B of the QK product): query q0 + c16, dims 32ds + 8g .. +7
    u32x4 qv[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qv[ds] = bload4(qbuf, (uint32_t)((c16 * D + 8 * g) * ESZ), (uint32_t)((q0 * D + ds * 32) * ESZ));

    // visible keys of the lane's query, and of the workgroup's last query
    int64_t ke = N, km = N;
    if (a.ex.causal) {
      const int64_t off = (int64_t)N - Sq + 1;
      ke = (q + off < ke) ? q + off : ke;
      const int64_t qlast = (qg * 64 + 63 < Sq) ? qg * 64 + 63 : Sq - 1;
      km = (qlast + off < km) ? qlast + off : km;
    }
    if (a.ex.key_len) {
      const int64_t l = a.ex.key_len[b];
      ke = l < ke ? l : ke;
      km = l < km ? l : km;
    }
    const int kend = (int)(ke < 0 ? 0 : ke);
    int kmax = __builtin_amdgcn_readfirstlane((int)(km < 0 ? 0 : km));
    if (write_all) kmax = N;
    const int tlive = (kmax + kTile - 1) / kTile;  // tiles holding a visible key (same in all waves)
    // keys below the workgroup's smallest cut need no select
    int64_t kn = N;
    if (a.ex.causal) {
      const int64_t off = (int64_t)N - Sq + 1;
      kn = (qg * 64 + off < kn) ? qg * 64 + off : kn;
    }
    if (a.ex.key_len) {
      const int64_t l = a.ex.key_len[b];
      kn = l < kn ? l : kn;
    }
    const int kmin = __builtin_amdgcn_readfirstlane((int)(kn < 0 ? 0 : kn));
    // the mask of (b, h) as one buffer: the lane's row at q * msq, keys at
    // +key; the buffer ends with the last row's key N - 1, so keys past N of
    // the last row read 0 (they are cut anyway)
    Buf mbuf(nullptr, 0u);
    uint32_t moff = 0;
    if constexpr (MASK) {
      mbuf = Buf(a.mask + b * a.msb + h * a.msh, (uint32_t)((((int64_t)Sq - 1) * a.msq + N) * 4));
      moff = (uint32_t)((int64_t)(qvalid ? q : Sq - 1) * a.msq * 4) + 32u * (uint32_t)g;
    }

    // ---- staging: sub-tile `it` (keys 32*it .. +31) of K, and of V^T ----
    u32x4 pk[KCH], pv[VCH];
    auto fetch_k = [&](int it) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        pk[c] = bload4(kbuf, (uint32_t)((r * D + 8 * c8) * ESZ), (uint32_t)(SUB * it * D * ESZ));
      }
    };
    // key k = 8g + 4hb + r of the sub-tile is kept at LDS row 16hb + 4g + r,
    // so the A rows of one block are 16 consecutive LDS rows
    auto put_k = [&](int buf) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        const int pr = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
        *reinterpret_cast<u32x4 *>(&lk[buf][pr * KROW + 8 * c8]) = pk[c];
      }
    };
    auto fetch_v = [&](int it) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int d = ch / (SUB / 8), k8 = ch % (SUB / 8);
        pv[c] = bload4(vbuf, (uint32_t)((d * Np + 8 * k8) * ESZ), (uint32_t)(SUB * it * ESZ));
      }
    };
    auto put_v = [&](int buf) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int d = ch / (SUB / 8), k8 = ch % (SUB / 8);
        *reinterpret_cast<u32x4 *>(&lv[buf][d * VROW + 8 * k8]) = pv[c];
      }
    };
    // S^T of sub-tile it from LDS buffer buf: blocks hb = 0, 1 (keys
    // 32it + 8(c16/4) + 4hb + c16%4 as A rows, LDS rows 16hb + c16), raw dot
    // products
    auto qk_sub = [&](int buf, f32x4_t &s0, f32x4_t &s1) {
      s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      s1 = s0;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const u32x4 k0 = *reinterpret_cast<const u32x4 *>(&lk[buf][c16 * KROW + 32 * ds + 8 * g]);
        const u32x4 k1 = *reinterpret_cast<const u32x4 *>(&lk[buf][(16 + c16) * KROW + 32 * ds + 8 * g]);
        s0 = mfma32<DT>(k0, qv[ds], s0);
        s1 = mfma32<DT>(k1, qv[ds], s1);
      }
    };
    // the mask of the lane's 8 keys 32it + 8g .. +7: two 16-byte loads, the
    // step's offset in the scalar operand (issued one step ahead of use)
    auto load_mask = [&](int it, u32x4 (&mk)[2]) {
      if constexpr (MASK) {
        mk[0] = bload4(mbuf, moff, (uint32_t)(SUB * 4 * it));
        mk[1] = bload4(mbuf, moff + 16u, (uint32_t)(SUB * 4 * it));
      }
    };
    // scaled, masked and cut scores of the lane's 8 keys 32it + 8g + 4hb + r
    auto make_x = [&](int it, const f32x4_t &s0, const f32x4_t &s1, const u32x4 (&mk)[2],
                      float (&x)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = a.scale * ((e < 4) ? s0[e] : s1[e - 4]);
        if constexpr (WRITE) {
          const int key = SUB * it + 8 * g + e;
          if (a.scores && qvalid && key < N) a.scores[row * a.N + key] = s;
        }
        x[e] = s;
        if constexpr (MASK) {
          // copy the word out first: a bit cast of a vector element in place
          // reads the vector's first element
          const uint32_t mw = mk[e >> 2][e & 3];
          x[e] = x[e] + __builtin_bit_cast(float, mw);
        }
      }
      if (SUB * it + SUB > kmin) {  // the step reaches some query's cut (uniform)
        const int nv = kend - (SUB * it + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (e < nv) ? x[e] : kNegInf;
      }
    };

    // ---- pass 1: per tile (max, sum), folded into the row state in tile order ----
    // Software pipeline, one step deep: in step `it` the wave issues the QK
    // product of step it + 1 (K sub-tile it + 1, already in LDS) and the
    // mask of step it + 1, then runs the VALU work of step it on the
    // product issued one step earlier, so the matrix cores and the VALU
    // overlap.  K sub-tile it + 2 is loaded into registers at the start of
    // step it and written to the LDS buffer of sub-tile it (read by every
    // wave in step it - 1) before the step's barrier.
    float M = kNegInf, L = 0.0f;
    f32x4_t sa[2], sb[2];  // raw S^T of a step (blocks 0 and 1), by step parity
    u32x4 mk[2][2];
    if (tlive > 0) {
      fetch_k(0);
      put_k(0);
      fetch_k(1);
      put_k(1);
      __syncthreads();
      load_mask(0, mk[0]);
      qk_sub(0, sa[0], sb[0]);
      __syncthreads();  // every wave has read sub-tile 0 before step 0 overwrites it
    }
    for (int t = 0; t < tlive; ++t) {
      float x[8][8];  // [32-key step j][key 8g + e]
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int it = 8 * t + j;
        const int cur = j & 1, nxt = cur ^ 1;  // it is 8t + j: parity of j
        fetch_k(it + 2);
        load_mask(it + 1, mk[nxt]);
        qk_sub(nxt, sa[nxt], sb[nxt]);
        make_x(it, sa[cur], sb[cur], mk[cur], x[j]);
        put_k(cur);
        __syncthreads();
      }
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 8; e += 2) mx = fmax2(mx, fmax2(x[j][e], x[j][e + 1]));
      const float m = groups4_max(mx);
      const float msafe = (m == kNegInf) ? 0.0f : m;
      float pj[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = exp_(x[j][e] - msafe);
        const float s0 = (e8[0] + e8[1]) + (e8[2] + e8[3]);
        const float s1 = (e8[4] + e8[5]) + (e8[6] + e8[7]);
        pj[j] = groups4_sum(s0 + s1);  // the step's 32 keys
      }
      const float l = ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
      if (g == 0) sm[t * 16 + c16] = m;
      // merge (m, l) into the row state
      const float Mn = fmax2(M, m);
      if (Mn == kNegInf) {
        M = kNegInf;
        L = 0.0f;
      } else {
        const float fa = (M == kNegInf) ? 0.0f : exp_(M - Mn);
        const float fb = (m == kNegInf) ? 0.0f : exp_(m - Mn);
        const float La = L * fa;
        const float lb = l * fb;
        L = La + lb;
        M = Mn;
      }
    }
    // tiles past every visible key of the workgroup hold only -inf: (-inf, 0)
    // states, which leave (M, L) as they are
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
    if (g == 0 && qvalid) {
      if (has_sink) a.p_sink[row] = (sigma == kNegInf) ? 0.0f : exp_(sigma - M) * invL;
      if (a.lse) a.lse[row] = (L == 0.0f) ? kNegInf : M + ln_(L);
    }

    // ---- pass 2: P = e * c_t rounded to the dtype, O += P V, sub-tile by sub-tile ----
    f32x4_t o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // the same pipeline: step it issues QK of step it + 1, forms P of step
    // it, accumulates P V of step it (V sub-tile it in LDS), and writes K
    // sub-tile it + 2 and V sub-tile it + 1 to LDS before its barrier
    if (tlive > 0) {
      fetch_k(0);
      put_k(0);
      fetch_k(1);
      put_k(1);
      fetch_v(0);
      put_v(0);
      __syncthreads();
      load_mask(0, mk[0]);
      qk_sub(0, sa[0], sb[0]);
      __syncthreads();
    }
    for (int t = 0; t < tlive; ++t) {
      const float mt = sm[t * 16 + c16];
      const float msafe = (mt == kNegInf) ? 0.0f : mt;
      const float ct = (mt == kNegInf) ? 0.0f : exp_(mt - M) * invL;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int it = 8 * t + j;
        const int cur = j & 1, nxt = cur ^ 1;
        fetch_k(it + 2);
        fetch_v(it + 1);
        load_mask(it + 1, mk[nxt]);
        qk_sub(nxt, sa[nxt], sb[nxt]);
        float x[8], p[8];
        make_x(it, sa[cur], sb[cur], mk[cur], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = exp_(x[e] - msafe) * ct;
        const u32x4 pa = {pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]),
                          pack2<DT>(p[6], p[7])};
        if constexpr (WRITE) {
          if (a.probs && qvalid) {
            uint16_t *prow = static_cast<uint16_t *>(a.probs) + row * a.N;
            const int key0 = SUB * it + 8 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key0 + e < N) prow[key0 + e] = (uint16_t)(pa[e >> 1] >> (16 * (e & 1)));
          }
        }
        // B operand: keys 32it + 8g .. +7 of dims 16db + c16
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 vv = *reinterpret_cast<const u32x4 *>(&lv[cur][(16 * db + c16) * VROW + 8 * g]);
          o[db] = mfma32<DT>(pa, vv, o[db]);
        }
        put_k(cur);
        put_v(nxt);
        __syncthreads();
      }
    }

    // ---- O rows q0 + 4g + r, dims 16db + c16: round once, write ----
    uint16_t *orow = static_cast<uint16_t *>(a.out) + bh * a.Sq * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qq = q0 + 4 * g + r;
      if (qq < Sq) {
#pragma unroll
        for (int db = 0; db < DB; db += 2) {
          const uint32_t w2 = pack2<DT>(o[db][r], o[db + 1][r]);
          orow[(int64_t)qq * D + 16 * db + c16] = (uint16_t)(w2 & 0xffffu);
          orow[(int64_t)qq * D + 16 * (db + 1) + c16] = (uint16_t)(w2 >> 16);
        }
      }
    }
    __syncthreads();  // LDS is reused by the workgroup's next unit
  }
}

// V [B, Hkv, N, D] -> V^T [B, Hkv, D, Np], keys N .. Np-1 zero.  One
// workgroup per (head, 64-key block): 16-byte loads of 8 dims of a key,
// scattered into an LDS tile [D][64 keys], then 16-byte stores of 8 keys
// of a dim.  The tile row is 72 elements (144 bytes) so that the 8 lanes
// writing one key's 8 dims fall in different banks.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const uint16_t *v, uint16_t *vt, int64_t heads,
                                                 int64_t N, int64_t Np) {
  constexpr int TROW = 72;
  __shared__ __align__(16) uint16_t tile[D * TROW];
  const int64_t kblocks = Np / 64;
  const int64_t hb = blockIdx.x / kblocks;
  const int64_t k0 = (blockIdx.x % kblocks) * 64;
  if (hb >= heads) return;
  const uint16_t *src = v + hb * N * D;
  uint16_t *dst = vt + hb * (int64_t)D * Np;
  constexpr int CH = 64 * D / 8 / 256;  // 16-byte chunks per thread
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = threadIdx.x + 256 * c;
    const int kk = i / (D / 8), d8 = i % (D / 8);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (k0 + kk < N) w = *reinterpret_cast<const u32x4 *>(src + (k0 + kk) * D + 8 * d8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      tile[(8 * d8 + e) * TROW + kk] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = threadIdx.x + 256 * c;
    const int d = i / 8, k8 = i % 8;
    *reinterpret_cast<u32x4 *>(dst + (int64_t)d * Np + k0 + 8 * k8) =
        *reinterpret_cast<const u32x4 *>(&tile[d * TROW + 8 * k8]);
  }
}

template <int DT, int D>
hipError_t attn_launch(const AttnArgs &a, int64_t blocks, hipStream_t st) {
  const int64_t heads = a.B * a.Hkv;
  const int64_t vblocks = heads * (a.Np / 64);
  hipLaunchKernelGGL((vt_kernel<D>), dim3((unsigned)vblocks), dim3(256), 0, st,
                     static_cast<const uint16_t *>(a.v), static_cast<uint16_t *>(a.vt), heads, a.N,
                     (int64_t)a.Np);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)blocks), block(kWave * kAttnWaves);
  const size_t dyn = (size_t)kAttnWaves * a.T * 16 * sizeof(float);
  const bool mask = a.mask != nullptr, write = a.probs != nullptr || a.scores != nullptr;
  if (mask) {
    if (write) hipLaunchKernelGGL((attn_fwd_kernel<DT, D, true, true>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<DT, D, true, false>), grid, block, dyn, st, a);
  } else {
    if (write) hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, true>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, false>), grid, block, dyn, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(int dtype, const AttnArgs &a, int64_t blocks, hipStream_t st) {
  if (dtype == 1) return a.D == 64 ? attn_launch<1, 64>(a, blocks, st) : attn_launch<1, 128>(a, blocks, st);
  return a.D == 64 ? attn_launch<2, 64>(a, blocks, st) : attn_launch<2, 128>(a, blocks, st);
}

}  // namespace jas
